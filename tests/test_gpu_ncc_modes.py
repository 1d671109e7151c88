"""GPU parity of the same and full output modes of the u8 normalized
correlation (ncc_u8_run_mode: the image copied into the caller's workspace
with zero borders, then a valid-mode variant on it) against the CPU oracle's
definition of the modes.  Outputs and the workspace sit inside canary bands."""
import numpy as np
import pytest
import torch

import oracle
from cross_correlation_amd import _lib, api
from cross_correlation_amd.inputs import ncc_case, workload

import _gpu

pytestmark = pytest.mark.gpu

MODES = {"same": _lib.XC_NCC_MODE_SAME, "full": _lib.XC_NCC_MODE_FULL}
VARIANTS = {"auto": _lib.XC_NCC_AUTO, "ilp": _lib.XC_NCC_DOT4_ILP, "c1": _lib.XC_NCC_DOT4_C1,
            "scalar": _lib.XC_NCC_SCALAR_C1, "mfma": _lib.XC_NCC_MFMA, "mfma_w2": _lib.XC_NCC_MFMA_W2,
            "cols2": _lib.XC_NCC_DOT4_COLS2, "cols8": _lib.XC_NCC_DOT4_COLS8}
WS_SENTINEL = 0xA5


def run_mode(case, mode, variant=_lib.XC_NCC_AUTO, ws_extra=0):
    """HIP result of one mode call; checks the canary bands of the outputs and
    of the workspace (the padding launch writes exactly the bytes it needs)."""
    th, tw = case.tmpl.shape
    oh, ow = _lib.ncc_mode_shape(case.width, case.height, tw, th, mode)
    st, nbytes = _lib.ncc_u8_mode_workspace(case.width, case.height, tw, th, mode)
    assert st == 0 and nbytes > 0
    g = _gpu.GUARD
    ws_buf = torch.full((nbytes + ws_extra + 2 * g,), WS_SENTINEL, dtype=torch.uint8, device=_gpu.dev())
    ws = ws_buf[g:g + nbytes + ws_extra]
    n = oh * ow
    bufs, out = {}, {}
    for k in ("sum_i", "sum_isq", "sum_it", "coef"):
        fill = float("nan") if k == "coef" else int(np.int32(_gpu.U32_SENTINEL.view(np.int32)))
        b = torch.full((n + 2 * g,), fill, dtype=torch.float32 if k == "coef" else torch.int32, device=_gpu.dev())
        bufs[k] = b
        out[k] = b[g:g + n].view(oh, ow)
    api.ncc_u8_mode(_gpu.to_dev(case.image), _gpu.to_dev(case.tmpl), mode, width=case.width, variant=variant,
                    out=out, workspace=ws)
    torch.cuda.synchronize()
    wsb = ws_buf.cpu().numpy()
    assert np.all(wsb[:g] == WS_SENTINEL) and np.all(wsb[g + nbytes:] == WS_SENTINEL), "workspace band overwritten"
    res = {}
    for k, b in bufs.items():
        b = b.cpu().numpy()
        if k == "coef":
            assert np.all(np.isnan(b[:g])) and np.all(np.isnan(b[-g:])), "canary band overwritten"
            v = b[g:g + n].reshape(oh, ow)
            assert not np.any(np.isnan(v)), "unwritten coefficient"
        else:
            b = b.view(np.uint32)
            assert np.all(b[:g] == _gpu.U32_SENTINEL) and np.all(b[-g:] == _gpu.U32_SENTINEL), "canary overwritten"
            v = b[g:g + n].reshape(oh, ow)
        res[k] = v
    return res


def _check(res, ref):
    for k in ("sum_i", "sum_isq", "sum_it"):
        bad = np.count_nonzero(res[k] != ref[k])
        assert bad == 0, f"{k}: {bad} mismatches"
    err = np.max(np.abs(res["coef"].astype(np.float64) - ref["coef"].astype(np.float64)))
    assert err <= 1e-5, f"coef max error {err}"


# (height, width, t_height, t_width): odd and even template sizes, widths not a
# multiple of 4, ragged tiles, a template larger than the image, one row
SHAPES = [(20, 37, 5, 7), (33, 70, 8, 12), (40, 300, 16, 16), (17, 29, 4, 6), (9, 11, 13, 15), (1, 50, 1, 9),
          (70, 260, 9, 64), (25, 90, 31, 3),
          # one image column; a 3-column image under a 40-wide template (the
          # padding copy reads only clamped words around it)
          (5, 1, 3, 1), (6, 3, 2, 40)]


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("shape", SHAPES, ids=[f"{s[0]}x{s[1]}_t{s[2]}x{s[3]}" for s in SHAPES])
def test_ncc_mode_matches_oracle(shape, mode):
    h, w, th, tw = shape
    case = ncc_case("m", 600 + th * 13 + tw, h, w, th, tw, cut=False)
    ref = oracle.ncc_u8_mode(case.image, case.width, case.height, case.tmpl, MODES[mode])
    for vname, v in VARIANTS.items():
        if (vname == "mfma" and tw > 256) or (vname == "mfma_w2" and tw > 64):
            continue
        _gpu.log(f"ncc mode {mode} {shape} variant {vname}")
        _check(run_mode(case, MODES[mode], v), ref)


def test_ncc_mode_reuses_larger_workspace():
    """Two calls in a row on one oversized workspace, the second smaller."""
    big = ncc_case("m", 620, 50, 90, 10, 14, cut=False)
    small = ncc_case("m", 621, 12, 20, 3, 5, cut=False)
    for case, mode in ((big, _lib.XC_NCC_MODE_FULL), (small, _lib.XC_NCC_MODE_SAME)):
        _gpu.log(f"ncc mode reuse {case.height}x{case.width} mode {mode}")
        ref = oracle.ncc_u8_mode(case.image, case.width, case.height, case.tmpl, mode)
        _check(run_mode(case, mode, ws_extra=4096), ref)


@pytest.mark.parametrize("mode", list(MODES))
def test_ncc_mode_1080p_sampled(mode):
    """The 1920x1080 / 64x64 workload in same and full modes: every window
    containing the cut gives coefficient 1 at the cut, and sampled windows
    (corners, borders, interior) match the oracle on the padded image."""
    case = workload("ncc_1920x1080_t64")
    th, tw = case.tmpl.shape
    _gpu.log(f"ncc mode {mode} 1920x1080 t64")
    res = run_mode(case, MODES[mode])
    oh, ow, pt, pl = oracle.ncc_mode_geometry(case.width, case.height, tw, th, MODES[mode])
    assert res["sum_i"].shape == (oh, ow)
    oy, ox = case.cut
    assert res["coef"][oy + pt, ox + pl] == np.float32(1.0)
    padded = np.zeros((oh + th - 1, ow + tw - 1), dtype=np.uint8)
    padded[pt:pt + case.height, pl:pl + case.width] = case.image[:, :case.width]
    rng = np.random.default_rng(630)
    ys = np.concatenate([[0, 0, oh - 1, oh - 1, pt, oh // 2], rng.integers(0, oh, 200)])
    xs = np.concatenate([[0, ow - 1, 0, ow - 1, pl, ow // 2], rng.integers(0, ow, 200)])
    ref = oracle.ncc_u8_points(padded, padded.shape[1], padded.shape[0], case.tmpl, ys, xs)
    for k in ("sum_i", "sum_isq", "sum_it"):
        assert np.array_equal(res[k][ys, xs], ref[k]), k
    assert np.max(np.abs(res["coef"][ys, xs].astype(np.float64) - ref["coef"])) <= 1e-5
