"""Seeded random-shape sweeps: every NCC variant and every fp32 algorithm on
shapes drawn at random (one fixed seed per case), against the oracle to the
bars of the other parity tests (sums bit-exact, coefficient within 1e-5,
cross-correlation within 1e-5 * sum|l*r| per output).  They reach
combinations the hand-picked edge shapes do not: odd pitches, thin strips,
templates on either side of tile, word and chunk boundaries.  Variants that
do not take a shape must refuse it with XC_ERR_SHAPE."""
import numpy as np
import pytest

import oracle
from cross_correlation_amd import _lib
from cross_correlation_amd.inputs import NccCase, f32_uniform, pitch_for, u8_uniform

import _gpu

pytestmark = pytest.mark.gpu

NCC_VARIANTS = [_lib.XC_NCC_AUTO, _lib.XC_NCC_DOT4_ILP, _lib.XC_NCC_DOT4_C1, _lib.XC_NCC_SCALAR_C1,
                _lib.XC_NCC_MFMA, _lib.XC_NCC_MFMA_W4, _lib.XC_NCC_MFMA_W2, _lib.XC_NCC_DOT4_ILP_Q1,
                _lib.XC_NCC_DOT4_ILP_Q2, _lib.XC_NCC_DOT4_ILP_Q4, _lib.XC_NCC_DOT4_COLS1, _lib.XC_NCC_DOT4_COLS2,
                _lib.XC_NCC_DOT4_COLS4, _lib.XC_NCC_DOT4_COLS8, _lib.XC_NCC_MFMA32]
XCORR_ALGOS = [_lib.XC_XCORR_AUTO, _lib.XC_XCORR_OVERLAP, _lib.XC_XCORR_BLOCKDIAG, _lib.XC_XCORR_WAVE,
               _lib.XC_XCORR_SMALL, _lib.XC_XCORR_MFMA]


def _ncc_shape(seed):
    rng = np.random.default_rng(seed)
    h = int(rng.integers(1, 201))
    w = int(rng.integers(1, 301))
    th = int(rng.integers(1, h + 1))
    tw = int(rng.integers(1, min(w, 300) + 1))
    while th * tw > 20000:  # keeps the oracle to about a second
        th = max(1, th // 2)
    extra = 16 * int(rng.integers(0, 3))
    return rng, h, w, th, tw, extra


@pytest.mark.parametrize("seed", range(7000, 7024))
def test_ncc_random_shape_all_variants(seed):
    rng, h, w, th, tw, extra = _ncc_shape(seed)
    img = u8_uniform(rng, (h, w))
    cut = bool(rng.integers(0, 2))
    if cut:  # the template cut from the image: coefficient 1 there
        oy, ox = int(rng.integers(0, h - th + 1)), int(rng.integers(0, w - tw + 1))
        tmpl = np.ascontiguousarray(img[oy:oy + th, ox:ox + tw])
    else:
        tmpl = u8_uniform(rng, (th, tw))
    pitch = pitch_for(w) + extra
    buf = np.zeros((h, pitch), np.uint8)
    buf[:, :w] = img
    case = NccCase("r", buf, w, h, tmpl, None)
    ref = None
    for v in NCC_VARIANTS:
        _gpu.log(f"ncc random seed {seed}: image {h}x{w} (pitch {pitch}), template {th}x{tw}, variant {v}")
        if not _gpu.ncc_takes(v, th, tw):
            with pytest.raises(_lib.XcError) as e:
                _gpu.run_ncc(case, v)
            assert e.value.status == _lib.XC_ERR_SHAPE
            continue
        res = _gpu.run_ncc(case, v)
        ref = _gpu.check_ncc(case, res, ref)
        if cut:
            assert res["coef"][oy, ox] == np.float32(1.0) or np.all(tmpl == tmpl.flat[0])


def _small_supported(rows, cols):
    return rows <= 16 or cols <= 16


@pytest.mark.parametrize("seed", range(8000, 8020))
def test_xcorr_random_shape_all_algorithms(seed):
    rng = np.random.default_rng(seed)
    nl, nr = int(rng.integers(1, 7)), int(rng.integers(1, 7))
    rows, cols = int(rng.integers(1, 49)), int(rng.integers(1, 49))
    L = f32_uniform(rng, (nl, rows, cols))
    R = f32_uniform(rng, (nr, rows, cols))
    ref, ab = oracle.xcorr_f32(L, R)
    for algo in XCORR_ALGOS:
        _gpu.log(f"xcorr random seed {seed}: {nl}x{nr} pairs of {rows}x{cols}, algorithm {algo}")
        supported = {_lib.XC_XCORR_BLOCKDIAG: (rows + 3) // 4 >= 4,
                     _lib.XC_XCORR_SMALL: _small_supported(rows, cols),
                     _lib.XC_XCORR_MFMA: cols % 4 == 0}.get(algo, True)
        if not supported:
            with pytest.raises(_lib.XcError) as e:
                _gpu.run_xcorr(L, R, algo)
            assert e.value.status == _lib.XC_ERR_SHAPE
            continue
        _gpu.check_xcorr(_gpu.run_xcorr(L, R, algo), ref, ab)


MODE_VARIANTS = [_lib.XC_NCC_AUTO, _lib.XC_NCC_DOT4_ILP, _lib.XC_NCC_DOT4_C1, _lib.XC_NCC_MFMA,
                 _lib.XC_NCC_MFMA_W2, _lib.XC_NCC_DOT4_COLS2]


@pytest.mark.parametrize("seed", range(9000, 9012))
def test_ncc_modes_random_shape(seed):
    """Same and full output modes on random shapes (templates larger than the
    image included), through the automatic choice and one other variant drawn
    per case, against the mode oracle; canary bands around the outputs and the
    workspace."""
    from test_gpu_ncc_modes import _check, run_mode
    rng = np.random.default_rng(seed)
    h, w = int(rng.integers(1, 121)), int(rng.integers(1, 201))
    th, tw = int(rng.integers(1, 90)), int(rng.integers(1, 140))
    while th * tw > 8000:
        th = max(1, th // 2)
    img = u8_uniform(rng, (h, w))
    buf = np.zeros((h, pitch_for(w)), np.uint8)
    buf[:, :w] = img
    case = NccCase("m", buf, w, h, u8_uniform(rng, (th, tw)), None)
    other = MODE_VARIANTS[1 + int(rng.integers(0, len(MODE_VARIANTS) - 1))]
    for mode in (_lib.XC_NCC_MODE_SAME, _lib.XC_NCC_MODE_FULL):
        ref = oracle.ncc_u8_mode(case.image, case.width, case.height, case.tmpl, mode)
        for v in (_lib.XC_NCC_AUTO, other):
            if not _gpu.ncc_takes(v, th, tw):
                continue
            _gpu.log(f"ncc mode {mode} random seed {seed}: image {h}x{w}, template {th}x{tw}, variant {v}")
            _check(run_mode(case, mode, v), ref)


@pytest.mark.parametrize("seed", range(9100, 9112))
def test_ncc_peak_random_shape(seed):
    """The best match on random shapes (a cut template for most), through the
    automatic choice and one other variant per case, against the oracle's
    first maximum of its own coefficient map."""
    from test_gpu_ncc_ext import _check_peak, _run_peak
    rng, h, w, th, tw, extra = _ncc_shape(seed)
    img = u8_uniform(rng, (h, w))
    cut = None
    if rng.integers(0, 4) > 0:
        cut = (int(rng.integers(0, h - th + 1)), int(rng.integers(0, w - tw + 1)))
        tmpl = np.ascontiguousarray(img[cut[0]:cut[0] + th, cut[1]:cut[1] + tw])
    else:
        tmpl = u8_uniform(rng, (th, tw))
    buf = np.zeros((h, pitch_for(w) + extra), np.uint8)
    buf[:, :w] = img
    case = NccCase("p", buf, w, h, tmpl, cut)
    ref = oracle.ncc_u8(case.image, case.width, case.height, case.tmpl)
    other = NCC_VARIANTS[1 + int(rng.integers(0, len(NCC_VARIANTS) - 1))]
    for v in (_lib.XC_NCC_AUTO, other):
        if not _gpu.ncc_takes(v, th, tw):
            continue
        _gpu.log(f"ncc peak random seed {seed}: image {h}x{w}, template {th}x{tw}, variant {v}")
        got, maps = _run_peak(case, v, outputs=("coef",))
        _check_peak(case, got, maps["coef"], ref["coef"])
