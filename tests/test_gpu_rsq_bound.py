"""The relative error of gfx950's fp64 reciprocal-square-root estimate
(v_rsq_f64), on which the u8 coefficient's bit-exact rounding argument rests:
the coefficient routine takes the estimate, one Newton step and a 2^-42
rounding-boundary margin, which is sound for estimates within 2^-23 (and
would still be for up to about 2^-21.3).  Measured over 10^7 values p of the
routine's domain, [1, 2^100) (p = vI * vT of two integer variances below
2^50): uniform mantissas in every binade, and the ends of every binade, where
an estimate's error tends to peak.  Reference: numpy's fp64 1/sqrt (within
one ulp, 2^-52, far below the bound tested)."""
import ctypes

import numpy as np
import pytest
import torch

from cross_correlation_amd import build

import _gpu

pytestmark = pytest.mark.gpu

BOUND = 2.0 ** -23


def _probe():
    lib = ctypes.CDLL(build.PEAK_LIB)
    lib.xc_rsq_probe.restype = ctypes.c_int
    lib.xc_rsq_probe.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
    return lib


def _domain(n_per_binade: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    e = np.repeat(np.arange(100, dtype=np.float64), n_per_binade)
    m = 1.0 + rng.random(e.size)
    ends = []
    k = np.arange(1, 2049, dtype=np.float64)
    for b in range(100):
        lo = np.ldexp(1.0 + k * 2.0 ** -52, b)        # just above 2^b
        hi = np.ldexp(2.0 - k * 2.0 ** -52, b)        # just below 2^(b+1)
        ends += [lo, hi, np.array([np.ldexp(1.0, b)])]
    p = np.concatenate([np.ldexp(m, e.astype(np.int64))] + ends)
    assert p.min() >= 1.0 and p.max() < 2.0 ** 100
    return p


def test_rsq_f64_estimate_relative_error():
    lib = _probe()
    p = _domain(100_000, 991)
    assert p.size >= 10_000_000
    _gpu.log(f"rsq probe over {p.size} values of [1, 2^100)")
    pd = torch.from_numpy(p).to(_gpu.dev())
    yd = torch.empty_like(pd)
    assert lib.xc_rsq_probe(pd.data_ptr(), yd.data_ptr(), p.size) == 0
    y = yd.cpu().numpy()
    ref = 1.0 / np.sqrt(p)
    rel = np.abs(y - ref) / ref
    worst = float(rel.max())
    _gpu.log(f"rsq max relative error {worst:.3e} = 2^{np.log2(worst):.2f} at p = {p[int(rel.argmax())]!r}")
    assert np.all(np.isfinite(y))
    assert worst <= BOUND, f"rsq estimate error {worst:.3e} exceeds 2^-23"
