"""The library's launches under HIP graph capture: each entry point is
captured once on a capture stream, the graph replayed several times with the
program's own eager work (clearing the outputs) and synchronizations between
the replays, and every replay checked against the eager result bit for bit.
The library records no memset nodes (the best-match key is cleared by a
kernel), so a replay redoes all of its work."""
import numpy as np
import pytest
import torch

from cross_correlation_amd import _lib, api
from cross_correlation_amd.inputs import ncc_case, workload

import _gpu

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _dev_case(case):
    return _gpu.to_dev(case.image), _gpu.to_dev(case.tmpl)


def _replay_and_check(graph, outs, expect):
    for rep in range(REPLAYS):
        for t in outs:
            t.zero_()  # eager work on the default stream between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, (t, e) in enumerate(zip(outs, expect)):
            assert torch.equal(t, e), (rep, k)


@pytest.mark.parametrize("variant", [_lib.XC_NCC_DOT4_ILP, _lib.XC_NCC_MFMA])
def test_graph_ncc(variant):
    case = ncc_case("g", 700, 300, 520, 40, 64, cut=True)
    _gpu.log(f"graph ncc variant {variant}")
    img, tm = _dev_case(case)
    eager = api.ncc_u8(img, tm, width=case.width, variant=variant)
    torch.cuda.synchronize()
    out = {k: torch.empty_like(v) for k, v in eager.items()}
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        api.ncc_u8(img, tm, width=case.width, variant=variant, out=out)
    keys = sorted(out)
    _replay_and_check(g, [out[k] for k in keys], [eager[k] for k in keys])


def test_graph_ncc_peak_and_mode():
    case = workload("ncc_256x256_t16")
    _gpu.log("graph ncc_u8_peak and ncc_u8_run_mode")
    img, tm = _dev_case(case)
    eager_peak = api.ncc_u8_peak(img, tm, width=case.width, outputs=("coef",))
    eager_same = api.ncc_u8_mode(img, tm, _lib.XC_NCC_MODE_SAME, width=case.width)
    torch.cuda.synchronize()
    peak = torch.empty_like(eager_peak["peak"])
    coef = torch.empty_like(eager_peak["coef"])
    same = {k: torch.empty_like(v) for k, v in eager_same.items()}
    st, nbytes = _lib.ncc_u8_mode_workspace(case.width, case.height, case.t_width, case.t_height,
                                            _lib.XC_NCC_MODE_SAME)
    assert st == 0
    ws = torch.empty(nbytes, dtype=torch.uint8, device=_gpu.dev())
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        api.ncc_u8_peak(img, tm, width=case.width, out={"coef": coef}, peak=peak)
        api.ncc_u8_mode(img, tm, _lib.XC_NCC_MODE_SAME, width=case.width, out=same, workspace=ws)
    keys = sorted(same)
    _replay_and_check(g, [peak, coef] + [same[k] for k in keys],
                      [eager_peak["peak"], eager_peak["coef"]] + [eager_same[k] for k in keys])
    y, x, c = _lib.decode_peak(peak.cpu().numpy().tobytes())
    assert (y, x) == case.cut and c == 1.0


@pytest.mark.parametrize("name", ["xcorr_8to16_32", "xcorr_1to64_64"])
def test_graph_xcorr(name):
    c = workload(name)
    _gpu.log(f"graph xcorr {name}")
    left, right = _gpu.to_dev(c.left), _gpu.to_dev(c.right)
    eager = api.xcorr_f32(left, right)
    torch.cuda.synchronize()
    out = torch.empty_like(eager)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        api.xcorr_f32(left, right, out=out)
    _replay_and_check(g, [out], [eager])
    assert np.isfinite(out.cpu().numpy()).all()
