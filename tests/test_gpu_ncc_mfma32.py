"""GPU parity of the 32x32x32 matrix-core NCC variant (XC_NCC_MFMA32): the
template as the Toeplitz operand, template rows split over four waves, SumI
and SumISq from sliding column sums and row prefixes in four helper waves
(field x half of the tile's rows).

Sums bit-exact and the coefficient within 1e-5 of the oracle; at full 1080p
size every output bit-identical to the packed-byte kernel's.  Shapes cover
each template block count (1, 2, 3 blocks of 32 bytes of K), ragged 256-column
and 32-row tiles, template heights that do not split evenly over the four
matrix-core waves, and the LDS limit the variant refuses past.
"""
import numpy as np
import pytest

import oracle
from cross_correlation_amd import _lib, api
from cross_correlation_amd.inputs import ncc_case, u8_uniform, workload, pitch_for

import _gpu

pytestmark = pytest.mark.gpu

V = _lib.XC_NCC_MFMA32


def _case(img, tmpl, pitch=None):
    from cross_correlation_amd.inputs import NccCase
    h, w = img.shape
    p = pitch_for(w) if pitch is None else pitch
    buf = np.zeros((h, p), np.uint8)
    buf[:, :w] = img
    return NccCase("m32", buf, w, h, np.ascontiguousarray(tmpl), None)


def test_mfma32_256_t16_cut():
    case = workload("ncc_256x256_t16")
    _gpu.log("mfma32 256x256 t16")
    res = _gpu.run_ncc(case, V)
    _gpu.check_ncc(case, res)
    assert res["coef"][case.cut] == np.float32(1.0)


@pytest.mark.parametrize("shape", [
    # (height, width, t_height, t_width, pitch_extra)
    (40, 300, 5, 1, 0),       # one-byte rows (two K blocks)
    (64, 290, 31, 2, 16),     # two-byte rows, pitch > width
    (33, 257, 7, 12, 0),      # ragged column tile of one output
    (70, 600, 20, 33, 0),     # widest template of two K blocks
    (50, 530, 9, 34, 0),      # narrowest of three
    (100, 700, 64, 64, 0),    # the 64x64 template
    (90, 333, 13, 65, 0),     # widest the variant takes
    (16, 16, 16, 16, 0),      # template = image: one output
    (1, 64, 1, 64, 0),        # one pixel row
    (65, 1000, 3, 40, 0),     # 63 output rows: two row tiles, the second one short
    (380, 300, 350, 64, 0),   # tallest 64-wide template within the LDS plan (one workgroup per CU)
    (150, 400, 113, 64, 16),  # the first 64-wide height past two workgroups per CU
])
def test_mfma32_shapes(shape):
    h, w, th, tw, extra = shape
    rng = np.random.default_rng(h * 131 + w * 7 + th * 3 + tw)
    img = u8_uniform(rng, (h, w))
    tmpl = u8_uniform(rng, (th, tw))
    case = _case(img, tmpl, pitch=pitch_for(w) + extra)
    _gpu.log(f"mfma32 shape {shape}")
    _gpu.check_ncc(case, _gpu.run_ncc(case, V))


@pytest.mark.parametrize("ox_mod", [0, 1, 2, 3])
def test_mfma32_cut_every_byte_phase(ox_mod):
    rng = np.random.default_rng(700 + ox_mod)
    img = u8_uniform(rng, (80, 520))
    oy, ox = 33, 250 + ox_mod  # the window straddles the second and third 128-column tiles' boundary
    tmpl = img[oy:oy + 24, ox:ox + 40]
    case = _case(img, tmpl)
    _gpu.log(f"mfma32 cut template ox%4={ox_mod}")
    res = _gpu.run_ncc(case, V)
    _gpu.check_ncc(case, res)
    assert res["coef"][oy, ox] == np.float32(1.0)


def test_mfma32_delta_templates_lane_order():
    """A one-hot template's SumIT is the shifted image: every column of a
    32-byte K block and every template row of the four row quarters."""
    rng = np.random.default_rng(710)
    img = u8_uniform(rng, (60, 300))
    for tx in list(range(0, 64, 5)) + [63]:
        ty = tx % 7
        tmpl = np.zeros((7, 64), np.uint8)
        tmpl[ty, tx] = 3
        case = _case(img, tmpl)
        _gpu.log(f"mfma32 delta template ty={ty} tx={tx}")
        res = _gpu.run_ncc(case, V, outputs=("sum_it",))
        oh, ow = case.out_shape
        assert np.array_equal(res["sum_it"], 3 * img[ty:ty + oh, tx:tx + ow].astype(np.uint32)), tx


def test_mfma32_constant_image_and_template():
    rng = np.random.default_rng(711)
    tmpl = u8_uniform(rng, (9, 40))
    for val in (255, 0):
        case = _case(np.full((45, 300), val, np.uint8), tmpl)
        _gpu.log(f"mfma32 constant image {val}")
        res = _gpu.run_ncc(case, V)
        _gpu.check_ncc(case, res)
        assert np.all(res["coef"] == 0.0)
    case = _case(u8_uniform(rng, (45, 300)), np.full((9, 40), 200, np.uint8))
    _gpu.log("mfma32 constant template")
    res = _gpu.run_ncc(case, V)
    _gpu.check_ncc(case, res)
    assert np.all(res["coef"] == 0.0)


def test_mfma32_1080p_t64_matches_packed_byte():
    case = workload("ncc_1920x1080_t64")
    _gpu.log("mfma32 1920x1080 t64 vs packed-byte kernel")
    a = _gpu.run_ncc(case, V)
    b = _gpu.run_ncc(case, _lib.XC_NCC_DOT4_ILP)
    for k in a:
        assert np.array_equal(a[k].view(np.uint32), b[k].view(np.uint32)), k
    assert a["coef"][case.cut] == np.float32(1.0)


@pytest.mark.parametrize("outputs", [("coef",), ("sum_it",), ("sum_i", "sum_isq"), ("sum_isq", "coef")])
def test_mfma32_output_subsets(outputs):
    case = ncc_case("sub", 720, 120, 700, 30, 48, cut=True)
    _gpu.log(f"mfma32 outputs {outputs}")
    res = _gpu.run_ncc(case, V, outputs=outputs)
    ref = oracle.ncc_u8(case.image, case.width, case.height, case.tmpl)
    for k in outputs:
        if k == "coef":
            assert np.max(np.abs(res[k].astype(np.float64) - ref[k])) <= 1e-5
        else:
            assert np.array_equal(res[k], ref[k]), k


def test_mfma32_peak():
    case = ncc_case("pk", 721, 150, 800, 40, 56, cut=True)
    _gpu.log("mfma32 best match")
    img = _gpu.to_dev(case.image)
    tm = _gpu.to_dev(case.tmpl)
    pk = api.ncc_u8_peak(img, tm, width=case.width, variant=V)
    import torch
    torch.cuda.synchronize()
    best = _lib.decode_peak(pk["peak"].cpu().numpy().tobytes())
    ref = oracle.ncc_u8(case.image, case.width, case.height, case.tmpl)
    assert best == oracle.ncc_peak(ref["coef"])
    assert best[:2] == tuple(case.cut) and best[2] == 1.0


@pytest.mark.parametrize("th,tw", [(5, 66), (351, 64), (432, 20)])
def test_mfma32_refuses_unsupported_shapes(th, tw):
    rng = np.random.default_rng(712)
    case = _case(u8_uniform(rng, (max(th, 8) + 4, 400)), u8_uniform(rng, (th, tw)))
    _gpu.log(f"mfma32 refuses {th}x{tw}")
    with pytest.raises(_lib.XcError) as e:
        _gpu.run_ncc(case, V)
    assert e.value.status == _lib.XC_ERR_SHAPE
