"""GPU parity of the fp32 matrix-core cross-correlation (XC_XCORR_MFMA)
against the fp64 oracle.

Bar: |gpu - oracle| <= 1e-5 * sum|l*r| per output; small-integer inputs and
delta matrices exactly.  Shapes cover the three groupings at full size, tiles
cut by the output's edges, left-row ranges that do not fill the last staged
chunk, one-row and one-column-group matrices, and the shapes it refuses.
"""
import numpy as np
import pytest

import oracle
from cross_correlation_amd import _lib
from cross_correlation_amd.inputs import f32_uniform, workload

import _gpu

pytestmark = pytest.mark.gpu

A = _lib.XC_XCORR_MFMA


@pytest.mark.parametrize("name", ["xcorr_1to1_256", "xcorr_1to64_64", "xcorr_8to16_32"])
def test_xcorr_mfma_workloads_full(name):
    case = workload(name)
    _gpu.log(f"xcorr mfma {name}")
    ref, ab = oracle.xcorr_f32(case.left, case.right)
    _gpu.check_xcorr(_gpu.run_xcorr(case.left, case.right, A), ref, ab)


@pytest.mark.parametrize("shape", [
    # (n_left, n_right, rows, cols)
    (1, 1, 1, 4), (1, 1, 1, 16), (2, 3, 3, 4), (1, 1, 9, 8), (1, 1, 17, 20), (3, 2, 21, 64),
    (1, 5, 64, 60), (2, 2, 24, 40), (1, 1, 100, 28), (1, 1, 255, 12), (4, 3, 33, 100),
    (1, 1, 300, 200), (1, 1, 64, 300),
])
def test_xcorr_mfma_shapes(shape):
    nl, nr, rows, cols = shape
    rng = np.random.default_rng(rows * 131 + cols * 7 + nl + 17 * nr + 5)
    L = f32_uniform(rng, (nl, rows, cols))
    R = f32_uniform(rng, (nr, rows, cols))
    _gpu.log(f"xcorr mfma shape {shape}")
    ref, ab = oracle.xcorr_f32(L, R)
    _gpu.check_xcorr(_gpu.run_xcorr(L, R, A), ref, ab)


def test_xcorr_mfma_small_integers_and_deltas():
    rng = np.random.default_rng(2300)
    for nl, nr, rows, cols in ((2, 3, 30, 24), (1, 1, 70, 64), (3, 2, 5, 36)):
        L = rng.integers(-3, 4, size=(nl, rows, cols)).astype(np.float32)
        R = rng.integers(-3, 4, size=(nr, rows, cols)).astype(np.float32)
        _gpu.log(f"xcorr mfma small integers {nl}x{nr} of {rows}x{cols}")
        ref, _ = oracle.xcorr_f32(L, R)
        assert np.array_equal(_gpu.run_xcorr(L, R, A).astype(np.float64), ref)
    rows, cols = 40, 36
    for (a, b, c, d) in ((0, 0, rows - 1, cols - 1), (rows - 1, cols - 1, 0, 0), (7, 3, 30, 33), (20, 35, 20, 0)):
        Ld = np.zeros((1, rows, cols), np.float32)
        Rd = np.zeros((1, rows, cols), np.float32)
        Ld[0, a, b] = 1.0
        Rd[0, c, d] = 1.0
        _gpu.log(f"xcorr mfma delta L({a},{b}) R({c},{d})")
        got = _gpu.run_xcorr(Ld, Rd, A)
        expect = np.zeros((2 * rows - 1, 2 * cols - 1), np.float32)
        expect[a - c + rows - 1, b - d + cols - 1] = 1.0
        assert np.array_equal(got[0, 0], expect)


def test_xcorr_mfma_deterministic():
    case = workload("xcorr_1to64_64")
    _gpu.log("xcorr mfma determinism")
    a = _gpu.run_xcorr(case.left, case.right, A)
    b = _gpu.run_xcorr(case.left, case.right, A)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("rows,cols", [(16, 18), (8, 7), (4, 1000)])
def test_xcorr_mfma_refuses(rows, cols):
    rng = np.random.default_rng(2301)
    L = f32_uniform(rng, (1, rows, cols))
    _gpu.log(f"xcorr mfma refuses {rows}x{cols}")
    with pytest.raises(_lib.XcError) as e:
        _gpu.run_xcorr(L, L, A)
    assert e.value.status == _lib.XC_ERR_SHAPE
