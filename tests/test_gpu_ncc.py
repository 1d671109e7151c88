"""GPU parity of the u8 normalized correlation against the CPU oracle.

Integer sums must match bit for bit; the coefficient within 1e-5.  Each test
prints the case it runs before touching the GPU.
"""
import numpy as np
import pytest

import oracle
from cross_correlation_amd import _lib
from cross_correlation_amd.inputs import ncc_case, u8_uniform, workload, pitch_for

import _gpu

pytestmark = pytest.mark.gpu

VARIANTS = [_lib.XC_NCC_AUTO, _lib.XC_NCC_DOT4_ILP, _lib.XC_NCC_DOT4_C1, _lib.XC_NCC_SCALAR_C1, _lib.XC_NCC_MFMA,
            _lib.XC_NCC_DOT4_ILP_Q1, _lib.XC_NCC_DOT4_ILP_Q2, _lib.XC_NCC_DOT4_ILP_Q4, _lib.XC_NCC_MFMA_W4,
            _lib.XC_NCC_MFMA_W2, _lib.XC_NCC_DOT4_COLS1, _lib.XC_NCC_DOT4_COLS2, _lib.XC_NCC_DOT4_COLS4,
            _lib.XC_NCC_DOT4_COLS8, _lib.XC_NCC_MFMA32]


def _case_from(img, tmpl, name="t", pitch=None):
    from cross_correlation_amd.inputs import NccCase
    h, w = img.shape
    p = pitch_for(w) if pitch is None else pitch
    buf = np.zeros((h, p), np.uint8)
    buf[:, :w] = img
    return NccCase(name, buf, w, h, np.ascontiguousarray(tmpl), None)


@pytest.mark.parametrize("variant", VARIANTS)
def test_ncc_256_t16_cut(variant):
    case = workload("ncc_256x256_t16")
    _gpu.log(f"ncc 256x256 t16 variant={variant}")
    res = _gpu.run_ncc(case, variant)
    _gpu.check_ncc(case, res)
    oy, ox = case.cut
    assert res["coef"][oy, ox] == np.float32(1.0)


def test_ncc_1080p_t64_full():
    case = workload("ncc_1920x1080_t64")
    _gpu.log("ncc 1920x1080 t64 (auto)")
    res = _gpu.run_ncc(case)
    _gpu.check_ncc(case, res)
    oy, ox = case.cut
    assert res["coef"][oy, ox] == np.float32(1.0)


@pytest.mark.parametrize("th,tw", [(4, 4), (6, 6), (8, 8), (5, 13)])
def test_ncc_1080p_small_templates_auto(th, tw):
    """1920x1080 with small templates on the automatic path (the matrix-core
    kernel from 1M outputs, on 128-column tiles here): 3,000 sampled windows
    and the corners against the oracle, coefficient 1 at the cut, and every
    output equal to the packed-byte kernel's bit for bit."""
    case = ncc_case("s", 940 + th * tw, 1080, 1920, th, tw, cut=True)
    _gpu.log(f"ncc 1080p small template {th}x{tw} auto")
    res = _gpu.run_ncc(case)
    oh, ow = res["sum_i"].shape
    rng = np.random.default_rng(941)
    ys = np.concatenate([[0, 0, oh - 1, oh - 1], rng.integers(0, oh, 3000)])
    xs = np.concatenate([[0, ow - 1, 0, ow - 1], rng.integers(0, ow, 3000)])
    ref = oracle.ncc_u8_points(case.image, case.width, case.height, case.tmpl, ys, xs)
    for k in ("sum_i", "sum_isq", "sum_it"):
        assert np.array_equal(res[k][ys, xs], ref[k]), k
    assert np.array_equal(res["coef"][ys, xs].view(np.uint32), ref["coef"].view(np.uint32))
    assert res["coef"][case.cut] == np.float32(1.0)
    ilp = _gpu.run_ncc(case, _lib.XC_NCC_DOT4_ILP)
    for k in res:
        assert np.array_equal(res[k].view(np.uint32), ilp[k].view(np.uint32)), k


@pytest.mark.parametrize("variant", [_lib.XC_NCC_DOT4_ILP, _lib.XC_NCC_DOT4_C1, _lib.XC_NCC_SCALAR_C1, _lib.XC_NCC_MFMA,
                                     _lib.XC_NCC_DOT4_ILP_Q1, _lib.XC_NCC_DOT4_ILP_Q2, _lib.XC_NCC_DOT4_ILP_Q4,
                                     _lib.XC_NCC_MFMA_W4, _lib.XC_NCC_MFMA_W2, _lib.XC_NCC_DOT4_COLS1,
                                     _lib.XC_NCC_DOT4_COLS2, _lib.XC_NCC_DOT4_COLS4, _lib.XC_NCC_DOT4_COLS8,
                                     _lib.XC_NCC_MFMA32])
def test_ncc_1080p_variants_sampled(variant):
    """Ablation variants at full size: compare against the auto path bit for bit."""
    case = workload("ncc_1920x1080_t64")
    _gpu.log(f"ncc 1920x1080 t64 variant={variant} vs auto")
    a = _gpu.run_ncc(case)
    b = _gpu.run_ncc(case, variant)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("ox_mod", [0, 1, 2, 3])
def test_ncc_cut_template_every_byte_phase(ox_mod):
    rng = np.random.default_rng(300 + ox_mod)
    img = u8_uniform(rng, (70, 300))
    oy, ox = 21, 40 + ox_mod
    tmpl = img[oy:oy + 20, ox:ox + 32]
    case = _case_from(img, tmpl)
    _gpu.log(f"ncc cut template ox%4={ox_mod}")
    res = _gpu.run_ncc(case)
    _gpu.check_ncc(case, res)
    t = tmpl.astype(np.int64)
    assert res["coef"][oy, ox] == np.float32(1.0)
    assert int(res["sum_i"][oy, ox]) == int(t.sum())
    assert int(res["sum_it"][oy, ox]) == int((t * t).sum())


def test_ncc_delta_templates_lane_order():
    """SumIT of a one-hot template is the shifted image: every byte lane of a word."""
    rng = np.random.default_rng(310)
    img = u8_uniform(rng, (40, 270))
    for tx in range(8):
        tmpl = np.zeros((3, 8), np.uint8)
        tmpl[tx % 3, tx] = 9
        case = _case_from(img, tmpl)
        _gpu.log(f"ncc delta template tx={tx}")
        res = _gpu.run_ncc(case, outputs=("sum_it",))
        oh, ow = case.out_shape
        expect = 9 * img[tx % 3:tx % 3 + oh, tx:tx + ow].astype(np.uint32)
        assert np.array_equal(res["sum_it"], expect), tx


def test_ncc_asymmetric_template():
    rng = np.random.default_rng(311)
    img = u8_uniform(rng, (50, 333))
    j, i = np.mgrid[0:9, 0:24]
    tmpl = (1 + (i % 4) * 50 + j).astype(np.uint8)
    case = _case_from(img, tmpl)
    _gpu.log("ncc asymmetric lane template")
    _gpu.check_ncc(case, _gpu.run_ncc(case))


def test_ncc_saturated_and_constant():
    rng = np.random.default_rng(312)
    tmpl = u8_uniform(rng, (5, 12))
    for val in (255, 0, 77):
        img = np.full((30, 290), val, np.uint8)
        case = _case_from(img, tmpl)
        _gpu.log(f"ncc constant image {val}")
        res = _gpu.run_ncc(case)
        _gpu.check_ncc(case, res)
        assert np.all(res["coef"] == 0.0)
        assert np.all(res["sum_isq"] == np.uint32(val * val * tmpl.size))
    img = u8_uniform(rng, (30, 290))
    case = _case_from(img, np.full((5, 12), 200, np.uint8))
    _gpu.log("ncc constant template")
    res = _gpu.run_ncc(case)
    _gpu.check_ncc(case, res)
    assert np.all(res["coef"] == 0.0)


def test_ncc_complement():
    rng = np.random.default_rng(313)
    img = u8_uniform(rng, (64, 300))
    tmpl = u8_uniform(rng, (8, 16))
    a = _gpu.run_ncc(_case_from(img, tmpl))
    b = _gpu.run_ncc(_case_from((255 - img).astype(np.uint8), tmpl))
    _gpu.log("ncc complement image")
    n = tmpl.size
    st = int(tmpl.astype(np.int64).sum())
    assert np.array_equal(b["sum_i"].astype(np.int64), 255 * n - a["sum_i"].astype(np.int64))
    assert np.array_equal(b["sum_it"].astype(np.int64), 255 * st - a["sum_it"].astype(np.int64))
    assert np.max(np.abs(b["coef"] + a["coef"])) <= 2e-7


@pytest.mark.parametrize("shape", [
    # (height, width, t_height, t_width, pitch_extra)
    (16, 16, 16, 16, 0),      # template = image -> 1x1 output
    (17, 33, 1, 4, 0),        # one-row template, odd sizes
    (33, 257, 7, 12, 32),     # ragged column tile, pitch > width
    (100, 513, 3, 4, 0),      # 2 column tiles + ragged tail
    (5, 1000, 5, 20, 0),      # one output row; 5-word template rows (unroll 1)
    (230, 300, 200, 300, 0),  # tall template: several row chunks
    (40, 4200, 16, 4096, 0),  # 1024-word template rows: several column chunks
    (1, 64, 1, 64, 0),        # single pixel row
])
@pytest.mark.parametrize("variant", VARIANTS)
def test_ncc_edge_shapes(shape, variant):
    h, w, th, tw, extra = shape
    rng = np.random.default_rng(h * 7919 + w)
    img = u8_uniform(rng, (h, w))
    tmpl = u8_uniform(rng, (th, tw))
    case = _case_from(img, tmpl, pitch=pitch_for(w) + extra)
    _gpu.log(f"ncc edge shape {shape} variant={variant}")
    if not _gpu.ncc_takes(variant, th, tw):
        with pytest.raises(_lib.XcError) as e:
            _gpu.run_ncc(case, variant)
        assert e.value.status == _lib.XC_ERR_SHAPE
        return
    _gpu.check_ncc(case, _gpu.run_ncc(case, variant))


@pytest.mark.parametrize("shape", [
    # (height, width, t_height, t_width): template widths on both sides of the
    # 64-byte blocks, ragged 256-column and 16-row tiles, template-row chunks
    (40, 300, 16, 4),
    (31, 290, 9, 60),
    (47, 529, 17, 64),
    (33, 400, 5, 68),
    (70, 700, 33, 132),
    (29, 600, 2, 196),
    (64, 800, 16, 252),
    (20, 600, 3, 256),
    (300, 60, 290, 8),        # 290 rows: two row chunks
    (300, 300, 258, 256),     # the largest template (66,048 pixels): many chunks
    (1, 1024, 1, 128),        # one output row
    (600, 64, 100, 64),       # one output column
])
def test_ncc_mfma_shapes(shape):
    h, w, th, tw = shape
    rng = np.random.default_rng(h * 131 + w * 7 + th)
    img = u8_uniform(rng, (h, w))
    tmpl = u8_uniform(rng, (th, tw))
    case = _case_from(img, tmpl)
    _gpu.log(f"ncc mfma shape {shape}")
    _gpu.check_ncc(case, _gpu.run_ncc(case, _lib.XC_NCC_MFMA))


@pytest.mark.parametrize("shape", [
    # (height, width, t_height, t_width): 128-column tiles (two matrix-core
    # waves, one column-sum wave per field over all the words), template
    # widths 1 .. 64 on both sides of a word, ragged column and row tiles, and
    # templates taller than the rows one chunk holds (head rows kept)
    (40, 200, 16, 4),
    (31, 385, 9, 61),
    (47, 577, 17, 64),
    (33, 190, 5, 1),
    (90, 450, 29, 63),        # two row chunks
    (150, 400, 64, 64),       # three row chunks
    (140, 250, 100, 7),       # many chunks of a narrow template
    (1, 1024, 1, 64),         # one output row
    (600, 64, 100, 64),       # one output column
    (20, 129, 20, 2),         # one row, one column tile and one column over
])
@pytest.mark.parametrize("variant", [_lib.XC_NCC_MFMA_W2, _lib.XC_NCC_MFMA_W4])
def test_ncc_mfma_tile_widths(shape, variant):
    h, w, th, tw = shape
    rng = np.random.default_rng(h * 137 + w * 11 + th)
    img = u8_uniform(rng, (h, w))
    tmpl = u8_uniform(rng, (th, tw))
    case = _case_from(img, tmpl)
    _gpu.log(f"ncc mfma tile width shape {shape} variant {variant}")
    _gpu.check_ncc(case, _gpu.run_ncc(case, variant))


@pytest.mark.parametrize("shape", [
    # (height, width, t_height, t_width): 256-column tiles whose column-sum
    # waves store window sums (templates of 48 rows and more), mostly with
    # the template in several row chunks (the head rows kept for the slide),
    # widths on both sides of 64 bytes
    (140, 400, 100, 64),      # two chunks
    (170, 600, 150, 100),     # two 64-byte blocks, three chunks
    (160, 530, 120, 33),      # an odd width, two chunks
    (100, 500, 64, 128),      # the widest window-sum template, one chunk
    (230, 300, 200, 128),     # row prefixes: two chunks at one workgroup per CU
])
def test_ncc_mfma_window_sums_row_chunks(shape):
    h, w, th, tw = shape
    rng = np.random.default_rng(h * 151 + w * 13 + th)
    img = u8_uniform(rng, (h, w))
    tmpl = u8_uniform(rng, (th, tw))
    case = _case_from(img, tmpl)
    _gpu.log(f"ncc mfma window sums in row chunks {shape}")
    _gpu.check_ncc(case, _gpu.run_ncc(case, _lib.XC_NCC_MFMA_W4))


@pytest.mark.parametrize("shape", [(120, 700, 20, 40), (200, 700, 64, 64)])
@pytest.mark.parametrize("variant", [_lib.XC_NCC_MFMA_W4, _lib.XC_NCC_MFMA_W2])
def test_ncc_mfma_output_subsets(variant, shape):
    """Subsets of the outputs through the matrix-core kernels (window sums
    on 256-column tiles; on 128-column tiles row prefixes for the 20-row
    template, window sums for the 64-row one), whose column-sum waves store
    SumI and SumISq during the walk when they form window sums and whose
    epilogue writes the rest: each requested map is right, none other is
    touched (the helper's guard bands and sentinels)."""
    h, w, th, tw = shape
    case = ncc_case("t", 330 + th, h, w, th, tw, cut=True)
    ref = None
    for outs in (("coef",), ("sum_it",), ("sum_i",), ("sum_isq",), ("sum_i", "coef"), ("sum_isq", "sum_it"),
                 ("sum_i", "sum_isq", "sum_it", "coef")):
        _gpu.log(f"ncc mfma outputs {outs} variant {variant}")
        ref = _gpu.check_ncc(case, _gpu.run_ncc(case, variant, outputs=outs), ref)


def test_ncc_mfma_extreme_pixels():
    """All-255 and all-0 windows against 0/255 templates: the -128 bias and its
    exact correction at the ends of the byte range."""
    for iv, tv in ((255, 255), (0, 255), (255, 0), (0, 0)):
        img = np.full((40, 300), iv, np.uint8)
        img[::7, ::5] = 255 - iv
        tmpl = np.full((12, 64), tv, np.uint8)
        tmpl[0, 0] = 255 - tv
        case = _case_from(img, tmpl)
        for v in (_lib.XC_NCC_MFMA_W4, _lib.XC_NCC_MFMA_W2):
            _gpu.log(f"ncc mfma extremes image={iv} template={tv} variant {v}")
            _gpu.check_ncc(case, _gpu.run_ncc(case, v))


def test_ncc_output_subsets():
    case = ncc_case("t", 320, 90, 280, 9, 16, cut=True)
    ref = None
    for outs in (("coef",), ("sum_it",), ("sum_i", "coef"), ("sum_isq",)):
        _gpu.log(f"ncc outputs {outs}")
        ref = _gpu.check_ncc(case, _gpu.run_ncc(case, outputs=outs), ref)


def test_ncc_deterministic():
    case = workload("ncc_256x256_t16")
    _gpu.log("ncc repeat determinism")
    a = _gpu.run_ncc(case)
    b = _gpu.run_ncc(case)
    for k in a:
        assert np.array_equal(a[k].view(np.uint32), b[k].view(np.uint32))


def test_ncc_invalid_arguments_rejected_before_launch():
    import torch
    from cross_correlation_amd import api
    img = torch.zeros((32, 64), dtype=torch.uint8, device="cuda")
    out = torch.zeros(64, dtype=torch.int32, device="cuda")
    wide = torch.zeros((4, 66), dtype=torch.uint8, device="cuda")
    st = _lib.ncc_u8_run(img.data_ptr(), 64, 32, 64, wide.data_ptr(), 66, 4, out.data_ptr(), 0, 0, 0)
    assert st == _lib.XC_ERR_SHAPE
    tall = torch.zeros((40, 8), dtype=torch.uint8, device="cuda")
    st = _lib.ncc_u8_run(img.data_ptr(), 64, 32, 64, tall.data_ptr(), 8, 40, out.data_ptr(), 0, 0, 0)
    assert st == _lib.XC_ERR_SHAPE
    with pytest.raises(_lib.XcError) as e:
        api.ncc_u8(img[:, 1:], torch.zeros((4, 8), dtype=torch.uint8, device="cuda"))
    assert e.value.status == _lib.XC_ERR_ALIGN


@pytest.mark.parametrize("th,tw", [(257, 257), (258, 256)])
def test_ncc_largest_template_near_u32_limit(th, tw):
    """Templates at the area limit (66,049 and 66,048 pixels of 66,051) over a
    nearly saturated image: SumISq reaches 255^2 * N, just below 2^32, in every
    variant that takes the width (the matrix-core kernel up to 256 bytes)."""
    rng = np.random.default_rng(330 + tw)
    img = np.full((th + 40, tw + 60), 255, np.uint8)
    img[::9, ::7] = u8_uniform(rng, img[::9, ::7].shape)
    tmpl = u8_uniform(rng, (th, tw))
    case = _case_from(img, tmpl)
    ref = None
    variants = [_lib.XC_NCC_AUTO, _lib.XC_NCC_DOT4_ILP, _lib.XC_NCC_DOT4_C1]
    if tw <= 256:
        variants.append(_lib.XC_NCC_MFMA)
    for v in variants:
        _gpu.log(f"ncc largest template {th}x{tw} variant {v}")
        res = _gpu.run_ncc(case, v)
        ref = _gpu.check_ncc(case, res, ref)
    assert int(ref["sum_isq"].max()) > 4_200_000_000  # far above 2^31: a signed 32-bit slip would show


def test_api_rejects_mismatched_outputs():
    """The torch wrappers check caller-supplied outputs against the output
    shape before calling the library: a map one row short, a strided map, a
    wrong dtype and a short best-match record are refused, and nothing is
    written to them."""
    import torch
    from cross_correlation_amd import api
    case = workload("ncc_256x256_t16")
    _gpu.log("ncc wrappers: mismatched caller outputs")
    img, tm = _gpu.to_dev(case.image), _gpu.to_dev(case.tmpl)
    oh, ow = case.out_shape
    short = torch.full((oh - 1, ow), 7, dtype=torch.int32, device="cuda")
    wide = torch.full((oh, 2 * ow), 7, dtype=torch.int32, device="cuda")
    for bad, msg in (({"sum_i": short}, "elements"), ({"sum_it": wide[:, ::2]}, "contiguous"),
                     ({"coef": torch.empty((oh, ow), dtype=torch.float64, device="cuda")}, "dtype")):
        with pytest.raises(ValueError, match=msg):
            api.ncc_u8(img, tm, width=case.width, out=bad)
    with pytest.raises(ValueError, match="bytes"):
        api.ncc_u8_peak(img, tm, width=case.width, peak=torch.zeros(2, dtype=torch.int64, device="cuda"))
    torch.cuda.synchronize()
    assert bool((short == 7).all()) and bool((wide == 7).all())
    L = torch.zeros((2, 16, 16), device="cuda")
    with pytest.raises(ValueError, match="elements"):
        api.xcorr_f32(L, L, out=torch.empty((2, 2, 31, 30), device="cuda"))


# Output widths whose last 256-column tile is narrow: the packed-byte kernel
# may give that remainder to tail tiles of several lane groups (64 // lanes
# needed), each group taking its own band of rows, where that saves a round
# of resident workgroups.  The 3200-row outputs with 16 x 16 templates do on
# a 256-CU MI355X (600 tiles of 256 x 16, two per CU, against 500 or fewer
# with tail tiles) with 4, 44 and 128 columns left over (up to 16, 5 and 2
# groups, fewer where the taller tile would not fit in LDS); the other shapes
# keep ordinary tiles (and one-row tiles on the short image).
@pytest.mark.parametrize("out_w,out_h,t", [(516, 3200, 16), (556, 3200, 16), (640, 3200, 16), (257, 690, 9),
                                           (385, 690, 64), (300, 36, 5)])
def test_ncc_ilp_tail_tiles(out_w, out_h, t):
    case = ncc_case("tail", 77 + out_w + t, out_h + t - 1, out_w + t - 1, t, t, cut=True)
    _gpu.log(f"ncc packed-byte tail tiles: {case.height}x{case.width} t{t}x{t} (out {out_h}x{out_w})")
    res = _gpu.run_ncc(case, _lib.XC_NCC_DOT4_ILP)
    _gpu.check_ncc(case, res)
    assert res["coef"][case.cut] == np.float32(1.0)


# The one-output-per-thread dot4 kernel splits the template rows over 4 or 2
# waves per output row on grids of at most one or two workgroups per SIMD
# (256x256 with 16x16: 244 workgroups, 4 waves; 400x300 with 12x12: 511, 2),
# a template row each at least; widths that are not a multiple of 4 take the
# gathered-word form; a 700-row template comes in two row chunks.
@pytest.mark.gpu
@pytest.mark.parametrize("h,w,th,tw", [(256, 256, 16, 16), (300, 400, 12, 12), (300, 300, 10, 10),
                                       (64, 200, 3, 8), (64, 200, 2, 5), (800, 200, 700, 8), (70, 70, 65, 6)])
def test_ncc_c1_template_row_slices(h, w, th, tw):
    case = ncc_case("c1ks", 91 + h + th, h, w, th, tw, cut=True)
    _gpu.log(f"ncc dot4 c1 row slices: {h}x{w} t{th}x{tw}")
    res = _gpu.run_ncc(case, _lib.XC_NCC_DOT4_C1)
    _gpu.check_ncc(case, res)
    assert res["coef"][case.cut] == np.float32(1.0)
