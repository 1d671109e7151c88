"""Concurrent calls: several host threads, each on its own stream, call the
library at once (different entry points, variants and shapes; run alone, this
includes the racing first calls of kernels that need the large-LDS opt-in);
every result must equal the single-threaded one bit for bit."""
import threading

import pytest
import torch

from cross_correlation_amd import _lib, api
from cross_correlation_amd.inputs import ncc_case, workload

import _gpu

pytestmark = pytest.mark.gpu

ROUNDS = 5


def _jobs():
    a = ncc_case("c", 800, 200, 400, 32, 48, cut=True)
    b = ncc_case("c", 801, 150, 300, 9, 13, cut=False)
    x5 = workload("xcorr_8to16_32")
    x4 = workload("xcorr_1to64_64")
    dev = lambda arr: _gpu.to_dev(arr)
    ia, ta, ib, tb = dev(a.image), dev(a.tmpl), dev(b.image), dev(b.tmpl)
    l5, r5, l4, r4 = dev(x5.left), dev(x5.right), dev(x4.left), dev(x4.right)
    return [
        lambda: api.ncc_u8(ia, ta, width=a.width, variant=_lib.XC_NCC_MFMA),
        lambda: api.ncc_u8(ib, tb, width=b.width, variant=_lib.XC_NCC_DOT4_ILP),
        lambda: api.ncc_u8_mode(ia, ta, _lib.XC_NCC_MODE_FULL, width=a.width),
        lambda: {"out": api.xcorr_f32(l5, r5)},
        lambda: {"out": api.xcorr_f32(l4, r4)},
        lambda: api.ncc_u8_peak(ib, tb, width=b.width, outputs=("coef",)),
    ]


def test_threads_on_own_streams():
    _gpu.log("concurrency: 6 threads x own streams")
    jobs = _jobs()
    results = [[None] * ROUNDS for _ in jobs]
    errors = []
    start = threading.Barrier(len(jobs))

    def worker(j):
        try:
            s = torch.cuda.Stream()
            start.wait()
            with torch.cuda.stream(s):
                for r in range(ROUNDS):
                    results[j][r] = jobs[j]()
            s.synchronize()
        except Exception as e:  # reported below, on the main thread
            errors.append((j, repr(e)))

    threads = [threading.Thread(target=worker, args=(j,)) for j in range(len(jobs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    # single-threaded reference, on the default stream
    for j, job in enumerate(jobs):
        ref = job()
        torch.cuda.synchronize()
        for r in range(ROUNDS):
            for k in ref:
                assert torch.equal(results[j][r][k], ref[k]), (j, r, k)
