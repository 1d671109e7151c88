"""Helpers for the GPU parity tests: run the HIP path through the C ABI (via
the torch wrappers) and compare with the CPU oracle on the same seeded input.

Outputs are written into the middle of larger buffers pre-filled with a
sentinel; the bands around them must survive (no out-of-bounds writes) and no
sentinel may remain inside (every output written).
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from cross_correlation_amd import _lib, api

GUARD = 4096  # elements of canary band on each side
U32_SENTINEL = np.uint32(0xDEADBEEF)


# Template widths the matrix-core variants take (their LDS limits on tall
# templates are not reached by the shapes the tests use).
MFMA_MAX_T_WIDTH = {_lib.XC_NCC_MFMA: 256, _lib.XC_NCC_MFMA_W4: 256, _lib.XC_NCC_MFMA_W2: 64}


def mfma32_fits(th: int, tw: int) -> bool:
    """Whether XC_NCC_MFMA32 takes a th x tw template: t_width <= 65 and its
    tile plan (staged image rows, padded template rows, window sums) within
    160 KiB of LDS, as the library computes it."""
    if tw > 65:
        return False
    nkb = 2 if tw < 2 else (tw + 62) // 32
    s = 32 * (4 + nkb - 1) + 16
    img = -(-max((32 + th) * s, 32 * 136 * 4) // 16) * 16
    tpl = (th + 1) * (32 * nkb + 48)
    return img + tpl + 2 * 32 * 132 * 4 + 16 <= 160 * 1024


def ncc_takes(variant: int, th: int, tw: int) -> bool:
    """Whether a u8 variant takes the template shape (else XC_ERR_SHAPE)."""
    if variant == _lib.XC_NCC_MFMA32:
        return mfma32_fits(th, tw)
    return tw <= MFMA_MAX_T_WIDTH.get(variant, tw)


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def _guarded(n: int, dtype, fill):
    buf = torch.full((n + 2 * GUARD,), fill, dtype=dtype, device=dev())
    return buf, buf[GUARD:GUARD + n]


def run_ncc(case, variant=_lib.XC_NCC_AUTO, outputs=("sum_i", "sum_isq", "sum_it", "coef")):
    """HIP normalized correlation on an NccCase; returns numpy arrays (u32 / f32)."""
    oh, ow = case.out_shape
    n = oh * ow
    img = to_dev(case.image)
    tm = to_dev(case.tmpl)
    bufs, out = {}, {}
    for k in outputs:
        if k == "coef":
            b, v = _guarded(n, torch.float32, float("nan"))
        else:
            b, v = _guarded(n, torch.int32, int(np.int32(U32_SENTINEL.view(np.int32))))
        bufs[k] = b
        out[k] = v.view(oh, ow)
    api.ncc_u8(img, tm, width=case.width, variant=variant, out=out)
    torch.cuda.synchronize()
    res = {}
    for k in outputs:
        b = bufs[k].cpu().numpy()
        if k == "coef":
            assert np.all(np.isnan(b[:GUARD])) and np.all(np.isnan(b[-GUARD:])), "canary band overwritten"
            v = b[GUARD:GUARD + n].reshape(oh, ow)
            assert not np.any(np.isnan(v)), "unwritten coefficient"
        else:
            b = b.view(np.uint32)
            assert np.all(b[:GUARD] == U32_SENTINEL) and np.all(b[-GUARD:] == U32_SENTINEL), "canary band overwritten"
            v = b[GUARD:GUARD + n].reshape(oh, ow)
        res[k] = v
    return res


def check_ncc(case, res, ref=None, tol=1e-5):
    """Sums bit-exact; coefficient within tol of the oracle."""
    if ref is None:
        ref = oracle.ncc_u8(case.image, case.width, case.height, case.tmpl)
    for k in ("sum_i", "sum_isq", "sum_it"):
        if k in res:
            bad = np.count_nonzero(res[k] != ref[k])
            assert bad == 0, f"{k}: {bad} mismatches"
    if "coef" in res:
        err = np.max(np.abs(res["coef"].astype(np.float64) - ref["coef"].astype(np.float64)))
        assert err <= tol, f"coef max error {err}"
    return ref


def run_xcorr(left: np.ndarray, right: np.ndarray, algo=_lib.XC_XCORR_AUTO) -> np.ndarray:
    nl, rows, cols = left.shape
    nr = right.shape[0]
    shape = (nl, nr, 2 * rows - 1, 2 * cols - 1)
    n = int(np.prod(shape))
    buf, view = _guarded(n, torch.float32, float("nan"))
    api.xcorr_f32(to_dev(left), to_dev(right), algo=algo, out=view.view(shape))
    torch.cuda.synchronize()
    b = buf.cpu().numpy()
    assert np.all(np.isnan(b[:GUARD])) and np.all(np.isnan(b[-GUARD:])), "canary band overwritten"
    v = b[GUARD:GUARD + n].reshape(shape)
    assert not np.any(np.isnan(v)), "unwritten output"
    return v


def check_xcorr(got: np.ndarray, ref: np.ndarray, ref_abs: np.ndarray, rel=1e-5):
    """|gpu - oracle| <= rel * sum|l*r| per output (tiny absolute floor for empty-abs outputs)."""
    err = np.abs(got.astype(np.float64) - ref)
    bound = rel * ref_abs + 1e-30
    bad = np.count_nonzero(err > bound)
    worst = float(np.max(err / (ref_abs + 1e-30)))
    assert bad == 0, f"{bad} outputs over tolerance (worst err/sum|lr| = {worst:.3e})"
    return worst
