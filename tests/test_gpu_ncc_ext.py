"""GPU parity for the generalizations of the u8 normalized correlation:
template widths that are not multiples of four, and the best-match search
(ncc_u8_peak), each through every kernel variant, against the CPU oracle."""
import numpy as np
import pytest

import oracle
from cross_correlation_amd import _lib
from cross_correlation_amd.inputs import ncc_case, workload

import _gpu

pytestmark = pytest.mark.gpu

VARIANTS = {
    "auto": _lib.XC_NCC_AUTO,
    "ilp": _lib.XC_NCC_DOT4_ILP,
    "c1": _lib.XC_NCC_DOT4_C1,
    "scalar": _lib.XC_NCC_SCALAR_C1,
    "mfma": _lib.XC_NCC_MFMA,
    "ilp_q1": _lib.XC_NCC_DOT4_ILP_Q1,
    "ilp_q2": _lib.XC_NCC_DOT4_ILP_Q2,
    "ilp_q4": _lib.XC_NCC_DOT4_ILP_Q4,
    "mfma_w4": _lib.XC_NCC_MFMA_W4,
    "mfma_w2": _lib.XC_NCC_MFMA_W2,
    "cols1": _lib.XC_NCC_DOT4_COLS1,
    "cols2": _lib.XC_NCC_DOT4_COLS2,
    "cols4": _lib.XC_NCC_DOT4_COLS4,
    "cols8": _lib.XC_NCC_DOT4_COLS8,
    "mfma32": _lib.XC_NCC_MFMA32,
}
# template rows the matrix-core variants take (256- and 128-column tiles)
MAX_T_WIDTH = {"mfma": 256, "mfma_w4": 256, "mfma_w2": 64}


def _variants(case):
    """Every variant that takes the case's template shape."""
    return {k: v for k, v in VARIANTS.items()
            if case.t_width <= MAX_T_WIDTH.get(k, case.t_width) and _gpu.ncc_takes(v, case.t_height, case.t_width)}


# (height, width, t_height, t_width): widths below four, odd and even
# non-multiples of four, one byte past a 64-byte block, the matrix-core limit,
# tall templates (template rows split over two waves, several row chunks)
ANY_WIDTH = [
    (20, 40, 3, 1), (20, 41, 5, 2), (33, 70, 4, 3), (40, 97, 6, 5), (17, 300, 9, 6), (50, 90, 7, 7),
    (64, 200, 11, 13), (70, 330, 16, 17), (40, 260, 8, 61), (36, 300, 5, 63), (36, 300, 5, 65),
    (30, 400, 3, 127), (30, 400, 4, 130), (24, 520, 3, 255), (24, 520, 2, 257), (200, 120, 70, 7),
    (260, 150, 250, 9),
]


@pytest.mark.parametrize("shape", ANY_WIDTH, ids=[f"{s[0]}x{s[1]}_t{s[2]}x{s[3]}" for s in ANY_WIDTH])
def test_ncc_any_template_width(shape):
    h, w, th, tw = shape
    case = ncc_case("t", 500 + th * 7 + tw, h, w, th, tw, cut=(th * tw) % 2 == 0)
    ref = None
    for name, v in _variants(case).items():
        _gpu.log(f"ncc any width {shape} variant {name}")
        ref = _gpu.check_ncc(case, _gpu.run_ncc(case, variant=v), ref)
    if case.cut is not None:
        res = _gpu.run_ncc(case, outputs=("coef",))
        assert res["coef"][case.cut] == np.float32(1.0)


# wide and tall templates on the matrix-core kernel: 3 and 4 template blocks
# of 64 bytes (one workgroup per CU, up to 160 KiB of LDS) and template rows
# in several chunks, so the column-sum waves slide from the saved head rows
WIDE_TALL = [(300, 600, 250, 256), (280, 500, 200, 193), (120, 700, 100, 130), (200, 400, 150, 250)]


@pytest.mark.parametrize("shape", WIDE_TALL, ids=[f"{s[0]}x{s[1]}_t{s[2]}x{s[3]}" for s in WIDE_TALL])
def test_ncc_mfma_wide_tall_templates(shape):
    h, w, th, tw = shape
    case = ncc_case("t", 570 + tw, h, w, th, tw, cut=True)
    ref = None
    for name in ("mfma", "ilp", "auto"):
        _gpu.log(f"ncc wide/tall {shape} variant {name}")
        ref = _gpu.check_ncc(case, _gpu.run_ncc(case, variant=VARIANTS[name]), ref)
    res = _gpu.run_ncc(case, variant=VARIANTS["mfma"], outputs=("coef",))
    assert res["coef"][case.cut] == np.float32(1.0)


def test_ncc_template_width_past_one_chunk():
    """3843 bytes: 961 packed words per row, so the packed-byte kernel's last
    template chunk holds the partial word alone."""
    case = ncc_case("t", 531, 40, 4000, 17, 3843, cut=True)
    ref = None
    for name in ("auto", "ilp"):
        _gpu.log(f"ncc 40x4000 t17x3843 variant {name}")
        ref = _gpu.check_ncc(case, _gpu.run_ncc(case, variant=VARIANTS[name]), ref)


def test_ncc_wide_template_q4_tiles():
    """Template rows of 3,604 to 4,128 bytes on the 256 x 16 tiles (four row
    waves of four rows): the template-word chunk is sized so that the tile's
    16 image rows and one template row fit in 64 KiB of LDS.  Through the
    Q = 4 ablation tile at a small size (every output against the oracle)."""
    for tw in (3604, 3700, 4128):
        case = ncc_case("t", 560 + tw % 97, 30, tw + 60, 16, tw, cut=True)
        _gpu.log(f"ncc {case.height}x{case.width} t16x{tw} variant ilp_q4")
        _gpu.check_ncc(case, _gpu.run_ncc(case, variant=VARIANTS["ilp_q4"]))


def test_ncc_wide_template_auto_full_grid():
    """A 3,700-byte template on an output of 1024 x 1024 (256 tiles of 256 x 16,
    where the automatic choice takes the packed-byte kernel's big tiles and
    splits the template rows over two waves): 3,000 sampled windows and the
    corners against the oracle, coefficient 1 at the cut."""
    tw, th = 3700, 17
    case = ncc_case("t", 571, th + 1023, tw + 1023, th, tw, cut=True)
    st, v = _lib.ncc_u8_auto_variant(case.width, case.height, tw, th)
    assert st == 0 and v == _lib.XC_NCC_DOT4_ILP
    _gpu.log(f"ncc {case.height}x{case.width} t{th}x{tw} auto (packed-byte, 256 x 16 tiles)")
    res = _gpu.run_ncc(case)
    oh, ow = case.out_shape
    rng = np.random.default_rng(572)
    ys = np.concatenate([[0, 0, oh - 1, oh - 1], rng.integers(0, oh, 3000)])
    xs = np.concatenate([[0, ow - 1, 0, ow - 1], rng.integers(0, ow, 3000)])
    ref = oracle.ncc_u8_points(case.image, case.width, case.height, case.tmpl, ys, xs)
    for k in ("sum_i", "sum_isq", "sum_it"):
        assert np.array_equal(res[k][ys, xs], ref[k]), k
    assert np.max(np.abs(res["coef"][ys, xs].astype(np.float64) - ref["coef"])) <= 1e-5
    assert res["coef"][case.cut] == np.float32(1.0)


def test_ncc_unaligned_template_base():
    """A template whose base is not 4-byte aligned (read byte by byte), at a
    width that is a multiple of four and at one that is not."""
    import torch
    from cross_correlation_amd import api
    for tw in (16, 15):
        case = ncc_case("t", 540 + tw, 60, 130, 9, tw, cut=True)
        ref = oracle.ncc_u8(case.image, case.width, case.height, case.tmpl)
        buf = torch.zeros(case.tmpl.size + 3, dtype=torch.uint8, device="cuda")
        t = buf[1:1 + case.tmpl.size].view(case.tmpl.shape)
        t.copy_(torch.from_numpy(case.tmpl))
        assert t.data_ptr() % 4 != 0
        for name, v in _variants(case).items():
            _gpu.log(f"ncc unaligned template tw={tw} variant {name}")
            got = api.ncc_u8(_gpu.to_dev(case.image), t, width=case.width, variant=v)
            torch.cuda.synchronize()
            for k in ("sum_i", "sum_isq", "sum_it"):
                assert np.array_equal(got[k].cpu().numpy().view(np.uint32), ref[k]), (tw, name, k)
            err = np.max(np.abs(got["coef"].cpu().numpy().astype(np.float64) - ref["coef"]))
            assert err <= 1e-5, (tw, name, err)


def _run_peak(case, variant, outputs=()):
    import torch
    from cross_correlation_amd import api
    res = api.ncc_u8_peak(_gpu.to_dev(case.image), _gpu.to_dev(case.tmpl), width=case.width, outputs=outputs,
                          variant=variant)
    torch.cuda.synchronize()
    y, x, c = _lib.decode_peak(res["peak"].cpu().numpy().tobytes())
    maps = {k: res[k].cpu().numpy() for k in outputs}
    return (y, x, c), maps


def _check_peak(case, got, gpu_coef, ref_coef):
    """The GPU's best match is the first maximum of its own map; against the
    oracle: the same location and value where the two maps are bit-identical,
    else a location whose oracle value is within the coefficient tolerance of
    the oracle's maximum (and the same one when that maximum is unique by a
    margin wider than the tolerance)."""
    y, x, c = got
    oy, ox, ov = oracle.ncc_peak(ref_coef)
    k = int(np.argmax(gpu_coef))
    assert (y, x) == divmod(k, gpu_coef.shape[1]) and c == gpu_coef[y, x]
    if np.array_equal(gpu_coef.view(np.uint32), ref_coef.view(np.uint32)):
        assert (y, x, c) == (oy, ox, ov)
        return
    assert abs(c - ov) <= 1e-5 and ref_coef[y, x] >= ov - 2e-5
    second = np.partition(ref_coef.ravel(), -2)[-2]
    if ov - second > 2e-5:
        assert (y, x) == (oy, ox)


PEAK_CASES = ["ncc_256x256_t16", "ncc_1920x1080_t64", "odd_97x300_t7x13", "odd_80x260_t33x61",
              "rand_90x200_t8x12"]


def _peak_case(name):
    if name.startswith("ncc_"):
        return workload(name)
    if name == "odd_97x300_t7x13":
        return ncc_case(name, 551, 97, 300, 7, 13, image_kind="gradient", cut=True)
    if name == "odd_80x260_t33x61":
        return ncc_case(name, 552, 80, 260, 33, 61, cut=True)
    return ncc_case(name, 553, 90, 200, 8, 12, cut=False)


@pytest.mark.parametrize("name", PEAK_CASES)
def test_ncc_peak_matches_oracle(name):
    case = _peak_case(name)
    ref = oracle.ncc_u8(case.image, case.width, case.height, case.tmpl)
    for vname, v in _variants(case).items():
        if name == "ncc_1920x1080_t64" and vname in ("c1", "scalar"):
            continue  # the slow ablation kernels are covered on the smaller cases
        _gpu.log(f"ncc peak {name} variant {vname}")
        got, maps = _run_peak(case, v, outputs=("coef",))
        _check_peak(case, got, maps["coef"], ref["coef"])
        if case.cut is not None:
            assert (got[0], got[1]) == case.cut and got[2] == 1.0
        # the best match alone (no map requested) is the same
        alone, _ = _run_peak(case, v)
        assert alone == got


def test_ncc_peak_ties_take_first_window():
    """A periodic image: the template matches every period with coefficient
    exactly 1; the first window in row-major order must win, in every variant."""
    rng = np.random.default_rng(560)
    tile = rng.integers(0, 256, size=(20, 24), dtype=np.uint8)
    img = np.tile(tile, (3, 5))
    for (oy, ox), (th, tw) in (((0, 0), (7, 9)), ((3, 5), (6, 10)), ((11, 17), (9, 12))):
        case = ncc_case("t", 0, 8, 8, 1, 1, cut=False)  # shell; fields replaced below
        pitch = 128
        padded = np.zeros((img.shape[0], pitch), np.uint8)
        padded[:, :img.shape[1]] = img
        case = type(case)("periodic", padded, img.shape[1], img.shape[0],
                          np.ascontiguousarray(img[oy:oy + th, ox:ox + tw]), (oy, ox))
        ref = oracle.ncc_u8(case.image, case.width, case.height, case.tmpl)
        assert oracle.ncc_peak(ref["coef"])[:2] == (oy, ox)
        assert np.count_nonzero(ref["coef"] == 1.0) > 1  # a real tie
        for vname, v in _variants(case).items():
            _gpu.log(f"ncc peak tie ({oy},{ox}) {th}x{tw} variant {vname}")
            got, maps = _run_peak(case, v, outputs=("coef",))
            assert got == (oy, ox, 1.0), (vname, got)
            _check_peak(case, got, maps["coef"], ref["coef"])


def test_ncc_peak_constant_image():
    """Every coefficient is 0 (zero variance): the first window wins."""
    case = ncc_case("t", 561, 30, 70, 5, 6, cut=False)
    case.image[:] = 77
    for vname, v in _variants(case).items():
        _gpu.log(f"ncc peak constant image variant {vname}")
        got, _ = _run_peak(case, v)
        assert got == (0, 0, 0.0), (vname, got)
