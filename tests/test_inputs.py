"""Seeded input generators: determinism, ranges and structure."""
import hashlib

import numpy as np

from cross_correlation_amd import inputs


def _h(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def test_same_seed_same_bytes():
    for name in list(inputs.NCC_WORKLOADS) + list(inputs.XCORR_WORKLOADS):
        a = inputs.workload(name)
        b = inputs.workload(name)
        if hasattr(a, "image"):
            assert _h(a.image) == _h(b.image) and _h(a.tmpl) == _h(b.tmpl)
        else:
            assert _h(a.left) == _h(b.left) and _h(a.right) == _h(b.right)


def test_ncc_workloads_shapes_and_cut():
    c1 = inputs.workload("ncc_256x256_t16")
    assert c1.out_shape == (241, 241) and c1.pitch % 16 == 0
    oy, ox = c1.cut
    assert np.array_equal(c1.tmpl, c1.pixels()[oy:oy + 16, ox:ox + 16])
    c2 = inputs.workload("ncc_1920x1080_t64")
    assert (c2.height, c2.width) == (1080, 1920)
    assert c2.out_shape == (1017, 1857)
    assert c2.t_width % 4 == 0
    oy, ox = c2.cut
    assert np.array_equal(c2.tmpl, c2.pixels()[oy:oy + 64, ox:ox + 64])


def test_gradient_image_formula():
    rng = np.random.default_rng(5)
    img = inputs.gradient_image(np.random.default_rng(5), 7, 11)
    u = rng.integers(0, 256, size=(7, 11), dtype=np.uint8).astype(np.int64)
    yy, xx = np.mgrid[0:7, 0:11]
    g = (255 * (xx + yy)) // (11 + 7 - 2)
    assert np.array_equal(img.astype(np.int64), (u + g) >> 1)
    assert img.max() <= 255 and img.dtype == np.uint8


def test_f32_values_on_grid():
    a = inputs.f32_uniform(np.random.default_rng(0), (1000,))
    assert a.dtype == np.float32
    assert np.all(a >= -1.0) and np.all(a < 1.0)
    k = (a.astype(np.float64) + 1.0) * (1 << 23)
    assert np.array_equal(k, np.round(k))


def test_xcorr_workload_shapes():
    assert inputs.workload("xcorr_1to1_256").out_shape == (1, 1, 511, 511)
    assert inputs.workload("xcorr_1to64_64").out_shape == (1, 64, 127, 127)
    assert inputs.workload("xcorr_8to16_32").out_shape == (8, 16, 63, 63)
