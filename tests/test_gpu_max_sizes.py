"""GPU parity at the largest sizes the library takes.

The normalized correlation runs on a 2048-column image (2304-byte pitch) with
a 4x4 template and the most output rows a 2045-column map may have: 2045 x
1,050,114 windows, 517 short of the 2^31 - 1 limit, read from an image of
2.42 GB (rows past the 2^31st byte).  The all-shift correlation runs four
pair sets whose outputs pass 2^31 elements.  The oracle cannot produce maps of
this size, so every run is checked on sampled outputs against it (the first
and last output rows or pairs whole, plus random ones) and on the device over
the whole map: every output written, the guard bands around it untouched.
"""
import numpy as np
import pytest
import torch

import oracle
from cross_correlation_amd import _lib, api
from cross_correlation_amd.inputs import f32_uniform, u8_uniform

import _gpu

pytestmark = pytest.mark.gpu

GUARD = 1 << 16                                            # elements of guard band on each side
U32_SENTINEL = int(np.uint32(0xDEADBEEF).view(np.int32))  # above any 4x4 window sum
NCC_W, NCC_PITCH, NCC_T = 2048, 2304, 4
NCC_OW = NCC_W - NCC_T + 1                                 # 2045
NCC_OH = (2**31 - 1) // NCC_OW                             # 1,050,114
NCC_H = NCC_OH + NCC_T - 1
NCC_SUMS = ("sum_i", "sum_isq", "sum_it")


def _guarded(n, dtype):
    buf = torch.empty(n + 2 * GUARD, dtype=dtype, device=_gpu.dev())
    return buf, buf[GUARD:GUARD + n]


def _check_whole(buf, fill_is):
    """Guard bands still hold the fill and no fill value remains inside."""
    assert bool(fill_is(buf[:GUARD]).all()) and bool(fill_is(buf[-GUARD:]).all()), "guard band overwritten"
    assert not bool(fill_is(buf[GUARD:-GUARD]).any()), "unwritten output"


@pytest.fixture(scope="module")
def ncc_big():
    assert NCC_OW * NCC_OH <= 2**31 - 1 < NCC_OW * (NCC_OH + 1)
    rng = np.random.default_rng(2031)
    _gpu.log(f"ncc max size: {NCC_H}x{NCC_W} image (pitch {NCC_PITCH}), generating")
    img = u8_uniform(rng, (NCC_H, NCC_PITCH))  # the bytes past the width are noise the kernels must skip
    cy, cx = NCC_OH - 1, NCC_OW - 1            # the template is cut from the last window
    tmpl = np.ascontiguousarray(img[cy:cy + NCC_T, cx:cx + NCC_T])
    n_rand = 20000
    ys = np.concatenate([np.zeros(NCC_OW, np.int64), np.full(NCC_OW, NCC_OH - 2), np.full(NCC_OW, NCC_OH - 1),
                         rng.integers(0, NCC_OH, 4000), rng.integers(0, NCC_OH, n_rand)])
    xs = np.concatenate([np.arange(NCC_OW), np.arange(NCC_OW), np.arange(NCC_OW),
                         np.full(4000, NCC_OW - 1), rng.integers(0, NCC_OW, n_rand)])
    _gpu.log(f"ncc max size: oracle at {ys.size} windows")
    ref = oracle.ncc_u8_points(img, NCC_W, NCC_H, tmpl, ys, xs)
    assert ref["coef"][3 * NCC_OW - 1] == np.float32(1.0)
    _gpu.log("ncc max size: upload and output allocation")
    d_img = torch.from_numpy(img).to(_gpu.dev())
    del img
    n = NCC_OH * NCC_OW
    bufs, views = {}, {}
    for k in NCC_SUMS + ("coef",):
        bufs[k], v = _guarded(n, torch.float32 if k == "coef" else torch.int32)
        views[k] = v.view(NCC_OH, NCC_OW)
    yield dict(img=d_img, tmpl=torch.from_numpy(tmpl).to(_gpu.dev()), ref=ref, bufs=bufs, views=views,
               idx=torch.from_numpy(ys * NCC_OW + xs).to(_gpu.dev()))
    del d_img, bufs, views
    torch.cuda.empty_cache()


def _fill_ncc(b):
    for k, buf in b["bufs"].items():
        buf.fill_(float("nan") if k == "coef" else U32_SENTINEL)


def _check_ncc_maps(b):
    torch.cuda.synchronize()
    for k, buf in b["bufs"].items():
        if k == "coef":
            _check_whole(buf, torch.isnan)
        else:
            _check_whole(buf, lambda t: t == U32_SENTINEL)
    ref, idx = b["ref"], b["idx"]
    for k in NCC_SUMS:
        got = b["views"][k].view(-1)[idx].cpu().numpy().view(np.uint32)
        bad = np.count_nonzero(got != ref[k])
        assert bad == 0, f"{k}: {bad} of {got.size} sampled windows differ"
    got = b["views"]["coef"].view(-1)[idx].cpu().numpy().astype(np.float64)
    err = np.max(np.abs(got - ref["coef"].astype(np.float64)))
    assert err <= 1e-5, f"coef max error {err}"
    assert b["views"]["coef"][NCC_OH - 1, NCC_OW - 1].item() == 1.0


@pytest.mark.parametrize("variant", [_lib.XC_NCC_AUTO, _lib.XC_NCC_DOT4_ILP, _lib.XC_NCC_DOT4_C1,
                                     _lib.XC_NCC_SCALAR_C1, _lib.XC_NCC_MFMA_W4, _lib.XC_NCC_MFMA_W2,
                                     _lib.XC_NCC_MFMA32])
def test_ncc_largest_output(ncc_big, variant):
    """2,147,483,130 windows: the 64-bit image and output offsets, the grids
    of over 65,535 row tiles, and the last rows of the image."""
    b = ncc_big
    _fill_ncc(b)
    _gpu.log(f"ncc max size {NCC_OH}x{NCC_OW} outputs, variant {variant}")
    api.ncc_u8(b["img"], b["tmpl"], width=NCC_W, variant=variant, out=b["views"])
    _check_ncc_maps(b)


def test_ncc_largest_output_peak(ncc_big):
    """The best match over the same 2,147,483,130 windows: coefficient 1 (the
    template is cut from the last window, flat index 2^31 - 518), at the first
    window in row-major order that the coefficient map gives that value."""
    b = ncc_big
    _fill_ncc(b)
    _gpu.log("ncc max size, best match with the coefficient map")
    res = api.ncc_u8_peak(b["img"], b["tmpl"], width=NCC_W, out={"coef": b["views"]["coef"]})
    torch.cuda.synchronize()
    y, x, c = _lib.decode_peak(res["peak"].cpu().numpy().tobytes())
    coef = b["views"]["coef"]
    best = coef.max()
    assert best.item() == 1.0
    hit = coef == best
    fy = int(torch.argmax(hit.any(dim=1).to(torch.uint8)).item())  # argmax takes the first of equal values
    fx = int(torch.argmax(hit[fy].to(torch.uint8)).item())
    del hit
    assert (y, x, c) == (fy, fx, 1.0)


@pytest.mark.parametrize("shape,algos", [
    # (n_left, n_right, rows, cols): 9.9 G, 8.6 G, 8.7 G and 8.7 G bytes of
    # output; the automatic choice runs the chunked block-diagonal kernel on
    # the first (also run on the fp32 matrix cores), the whole-staging one (16
    # waves, every matrix of a pair group in LDS) on the second, the
    # tiny-matrix kernel on the third and the small-matrix kernel on the last
    ((512, 300, 64, 64), (_lib.XC_XCORR_AUTO, _lib.XC_XCORR_MFMA)),
    ((512, 525, 64, 32), (_lib.XC_XCORR_AUTO,)),
    ((2048, 1100, 16, 16), (_lib.XC_XCORR_AUTO, _lib.XC_XCORR_SMALL)),
    ((8192, 5400, 4, 4), (_lib.XC_XCORR_AUTO, _lib.XC_XCORR_OVERLAP, _lib.XC_XCORR_WAVE)),
])
def test_xcorr_output_past_2_31(shape, algos):
    nl, nr, rows, cols = shape
    per_pair = (2 * rows - 1) * (2 * cols - 1)
    n = nl * nr * per_pair
    assert n > 2**31
    rng = np.random.default_rng(nl + nr + rows)
    L = f32_uniform(rng, (nl, rows, cols))
    R = f32_uniform(rng, (nr, rows, cols))
    flat = np.concatenate([np.arange(per_pair), np.arange(n - per_pair, n), rng.integers(0, n, 20000)])
    _gpu.log(f"xcorr {shape} ({n} outputs): oracle at {flat.size} outputs")
    ref, ab = oracle.xcorr_f32_points(L, R, flat)
    dL, dR = torch.from_numpy(L).to(_gpu.dev()), torch.from_numpy(R).to(_gpu.dev())
    buf, view = _guarded(n, torch.float32)
    idx = torch.from_numpy(flat).to(_gpu.dev())
    try:
        for algo in algos:
            buf.fill_(float("nan"))
            _gpu.log(f"xcorr {shape} algo {algo}")
            api.xcorr_f32(dL, dR, algo=algo, out=view.view(nl, nr, 2 * rows - 1, 2 * cols - 1))
            torch.cuda.synchronize()
            _check_whole(buf, torch.isnan)
            got = view[idx].cpu().numpy().astype(np.float64)
            err = np.abs(got - ref)
            assert np.all(err <= 1e-5 * ab + 1e-30), f"algo {algo}: max excess {np.max(err - 1e-5 * ab)}"
    finally:
        del buf, view, idx
        torch.cuda.empty_cache()
