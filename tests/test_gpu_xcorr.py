"""GPU parity of the fp32 full cross-correlation against the fp64 oracle.

Bar: |gpu - oracle| <= 1e-5 * sum|l*r| per output; small-integer inputs,
deltas and all-ones must match exactly.  Each test prints its case first.
"""
import numpy as np
import pytest

import oracle
from cross_correlation_amd import _lib
from cross_correlation_amd.inputs import f32_uniform, workload

import _gpu

pytestmark = pytest.mark.gpu

ALGOS = [_lib.XC_XCORR_AUTO, _lib.XC_XCORR_OVERLAP, _lib.XC_XCORR_BLOCKDIAG, _lib.XC_XCORR_WAVE]


@pytest.mark.parametrize("name", ["xcorr_1to1_256", "xcorr_1to64_64", "xcorr_8to16_32"])
@pytest.mark.parametrize("algo", ALGOS)
def test_xcorr_workloads_full(name, algo):
    case = workload(name)
    _gpu.log(f"xcorr {name} algo={algo}")
    ref, ab = oracle.xcorr_f32(case.left, case.right)
    got = _gpu.run_xcorr(case.left, case.right, algo)
    _gpu.check_xcorr(got, ref, ab)


@pytest.mark.parametrize("shape", [
    # (n_left, n_right, rows, cols)
    (1, 1, 13, 17),
    (1, 1, 16, 16),
    (2, 3, 37, 5),
    (3, 2, 21, 64),
    (1, 5, 64, 63),
    (5, 1, 100, 7),
    (1, 1, 255, 3),
    (1, 1, 256, 1),
    (2, 2, 24, 40),
    (3, 7, 32, 33),
    (1, 1, 1, 9),
    (1, 2, 3, 2),
    (1, 1, 257, 19),
])
@pytest.mark.parametrize("algo", [_lib.XC_XCORR_AUTO, _lib.XC_XCORR_OVERLAP, _lib.XC_XCORR_WAVE])
def test_xcorr_edge_shapes(shape, algo):
    nl, nr, rows, cols = shape
    rng = np.random.default_rng(rows * 131 + cols * 7 + nl + 17 * nr)
    L = f32_uniform(rng, (nl, rows, cols))
    R = f32_uniform(rng, (nr, rows, cols))
    _gpu.log(f"xcorr edge {shape} algo={algo}")
    ref, ab = oracle.xcorr_f32(L, R)
    _gpu.check_xcorr(_gpu.run_xcorr(L, R, algo), ref, ab)


@pytest.mark.parametrize("shape", [(1, 1, 16, 16), (2, 3, 37, 5), (1, 5, 64, 63), (3, 7, 32, 33),
                                   (1, 1, 255, 3), (1, 1, 256, 1), (2, 2, 24, 40), (4, 3, 200, 12),
                                   # too wide to stage whole: the chunked staging path (16, 8
                                   # and 4 waves per workgroup, one or two dx signs each)
                                   (2, 3, 100, 200), (1, 1, 60, 300), (1, 3, 13, 1000),
                                   (1, 1, 35, 600), (2, 3, 41, 600), (2, 3, 65, 260),
                                   # 16 diagonals whose whole staging only fits at 8 waves
                                   (3, 3, 85, 72),
                                   # whole staging would leave one wave per SIMD over several
                                   # rounds, or the rows are narrower than 32 columns: chunked
                                   (2, 3, 100, 70), (3, 5, 64, 64), (6, 6, 40, 24), (16, 16, 16, 16),
                                   # whole staging, every workgroup resident at once
                                   (32, 32, 32, 32),
                                   # whole staging of 4 x 4 blocks (rows a multiple of 4 columns
                                   # wide) with a ragged last row block, in both modes: the pair
                                   # kernel (up to 8 blocks, a diagonal's two dx signs shared by
                                   # two waves) and one wave walking both signs
                                   (8, 16, 30, 32), (5, 9, 29, 36), (1, 64, 61, 64), (2, 40, 18, 44),
                                   # more than 64 row blocks: passes of 64 blocks; 65 blocks
                                   # (the left window wraps onto itself), odd rows, 2-3 passes,
                                   # several pairs, wide rows
                                   (1, 1, 257, 19), (1, 1, 260, 40), (1, 1, 300, 17), (2, 3, 272, 9),
                                   (1, 2, 513, 6), (1, 1, 384, 64), (2, 1, 290, 33)])
def test_xcorr_blockdiag_edge_shapes(shape):
    nl, nr, rows, cols = shape
    rng = np.random.default_rng(rows * 31 + cols)
    L = f32_uniform(rng, (nl, rows, cols))
    R = f32_uniform(rng, (nr, rows, cols))
    _gpu.log(f"xcorr blockdiag edge {shape}")
    ref, ab = oracle.xcorr_f32(L, R)
    _gpu.check_xcorr(_gpu.run_xcorr(L, R, _lib.XC_XCORR_BLOCKDIAG), ref, ab)


# Shapes the pair kernel takes (up to 8 row blocks, rows of at least 32
# padded columns, every workgroup resident at once); its two waves of a
# diagonal share the walks, so the longer dx sign's sums come in two parts.
# The last two use the most LDS it takes (162,944 and 150,800 of 163,840
# bytes: staging, reduction areas and handover slots).
PAIR_SHAPES = [(4, 6, 30, 40), (3, 5, 18, 33), (1, 1, 32, 32), (2, 3, 13, 64), (1, 8, 32, 76), (1, 3, 17, 72)]


@pytest.mark.parametrize("shape", PAIR_SHAPES, ids=["x".join(map(str, s)) for s in PAIR_SHAPES])
def test_xcorr_pair_kernel_exact(shape):
    """Small integers (every partial sum an integer below 2^24, so exact in
    any order) bit for bit through the block-diagonal and automatic choices,
    and single ones at opposite corners and inside (orientation) in the last
    pair of the group."""
    nl, nr, rows, cols = shape
    rng = np.random.default_rng(rows * 7 + cols)
    L = rng.integers(-2, 3, size=(nl, rows, cols)).astype(np.float32)
    R = rng.integers(-2, 3, size=(nr, rows, cols)).astype(np.float32)
    ref, _ = oracle.xcorr_f32(L, R)
    for algo in (_lib.XC_XCORR_BLOCKDIAG, _lib.XC_XCORR_AUTO):
        _gpu.log(f"xcorr pair kernel {shape} small integers algo={algo}")
        assert np.array_equal(_gpu.run_xcorr(L, R, algo).astype(np.float64), ref)
    for (a, b, c, d) in ((0, 0, rows - 1, cols - 1), (rows - 1, cols - 1, 0, 0), (rows // 2, 1, 2, cols - 2)):
        Ld = np.zeros((nl, rows, cols), np.float32)
        Rd = np.zeros((nr, rows, cols), np.float32)
        Ld[-1, a, b] = 1.0
        Rd[-1, c, d] = 1.0
        _gpu.log(f"xcorr pair kernel {shape} delta ({a},{b}) ({c},{d})")
        expect = np.zeros((nl, nr, 2 * rows - 1, 2 * cols - 1), np.float32)
        expect[-1, -1, a - c + rows - 1, b - d + cols - 1] = 1.0
        assert np.array_equal(_gpu.run_xcorr(Ld, Rd, _lib.XC_XCORR_BLOCKDIAG), expect)


@pytest.mark.parametrize("algo", ALGOS)
def test_xcorr_small_integers_exact(algo):
    """Every partial sum is an integer below 2^24: any summation order is exact."""
    rng = np.random.default_rng(400)
    L = rng.integers(-2, 3, size=(3, 40, 28)).astype(np.float32)
    R = rng.integers(-2, 3, size=(4, 40, 28)).astype(np.float32)
    _gpu.log(f"xcorr small-integer exact algo={algo}")
    ref, _ = oracle.xcorr_f32(L, R)
    got = _gpu.run_xcorr(L, R, algo)
    assert np.array_equal(got.astype(np.float64), ref)


@pytest.mark.parametrize("algo", ALGOS)
def test_xcorr_delta_orientation(algo):
    rows, cols = 20, 28
    for (a, b, c, d) in ((0, 0, 19, 27), (19, 27, 0, 0), (3, 11, 17, 2), (5, 5, 5, 5)):
        L = np.zeros((1, rows, cols), np.float32)
        R = np.zeros((1, rows, cols), np.float32)
        L[0, a, b] = 1.0
        R[0, c, d] = 1.0
        _gpu.log(f"xcorr delta ({a},{b}) ({c},{d}) algo={algo}")
        got = _gpu.run_xcorr(L, R, algo)
        expect = np.zeros((2 * rows - 1, 2 * cols - 1), np.float32)
        expect[a - c + rows - 1, b - d + cols - 1] = 1.0
        assert np.array_equal(got[0, 0], expect)


@pytest.mark.parametrize("algo", ALGOS)
def test_xcorr_all_ones(algo):
    rows, cols = 48, 36
    _gpu.log(f"xcorr all ones algo={algo}")
    got = _gpu.run_xcorr(np.ones((1, rows, cols), np.float32), np.ones((2, rows, cols), np.float32), algo)
    dy = np.arange(2 * rows - 1) - (rows - 1)
    dx = np.arange(2 * cols - 1) - (cols - 1)
    expect = np.outer(rows - np.abs(dy), cols - np.abs(dx)).astype(np.float32)
    assert np.array_equal(got[0, 0], expect) and np.array_equal(got[0, 1], expect)


def test_xcorr_grouping_consistency():
    """Slice [l][r] of an n-to-m run equals the one-to-one run of (L_l, R_r)."""
    rng = np.random.default_rng(401)
    L = f32_uniform(rng, (3, 32, 32))
    R = f32_uniform(rng, (5, 32, 32))
    _gpu.log("xcorr grouping consistency")
    many = _gpu.run_xcorr(L, R)
    ref, ab = oracle.xcorr_f32(L, R)
    for l in range(3):
        for r in range(5):
            one = _gpu.run_xcorr(L[l:l + 1], R[r:r + 1])
            _gpu.check_xcorr(one[0, 0], ref[l, r], ab[l, r])
            _gpu.check_xcorr(many[l, r], ref[l, r], ab[l, r])


def test_xcorr_deterministic():
    case = workload("xcorr_8to16_32")
    _gpu.log("xcorr repeat determinism")
    a = _gpu.run_xcorr(case.left, case.right)
    b = _gpu.run_xcorr(case.left, case.right)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_xcorr_invalid_arguments_rejected_before_launch():
    import torch
    from cross_correlation_amd import api
    L = torch.zeros((1, 8, 8), device="cuda")
    with pytest.raises(_lib.XcError) as e:
        api.xcorr_f32(L, L, algo=7)
    assert e.value.status == _lib.XC_ERR_VARIANT
    with pytest.raises(_lib.XcError) as e:
        api.xcorr_f32(L, L, algo=_lib.XC_XCORR_BLOCKDIAG)  # 8 rows: too few for block diagonals
    assert e.value.status == _lib.XC_ERR_SHAPE
    st = _lib.xcorr_f32_run(L.data_ptr() + 4, 1, L.data_ptr(), 1, 8, 8, L.data_ptr())
    assert st == _lib.XC_ERR_ALIGN


def test_xcorr_large_one_to_one_sampled():
    """512x512 one-to-one (two passes of 64 row blocks) against the oracle at
    sampled outputs: every row and column of the output grid, plus random ones."""
    rng = np.random.default_rng(402)
    rows = cols = 512
    L = f32_uniform(rng, (1, rows, cols))
    R = f32_uniform(rng, (1, rows, cols))
    _gpu.log("xcorr 512x512 one-to-one, sampled")
    got = _gpu.run_xcorr(L, R)
    oh, ow = 2 * rows - 1, 2 * cols - 1
    ys = np.concatenate([np.arange(oh), rng.integers(0, oh, 600)])
    xs = np.concatenate([rng.integers(0, ow, oh), rng.integers(0, ow, 600)])
    ys = np.concatenate([ys, rng.integers(0, oh, ow)])
    xs = np.concatenate([xs, np.arange(ow)])
    flat = ys * ow + xs
    ref, ab = oracle.xcorr_f32_points(L, R, flat)
    g = got.reshape(-1)[flat].astype(np.float64)
    err = np.abs(g - ref)
    assert np.all(err <= 1e-5 * ab + 1e-30), f"max excess {np.max(err - 1e-5 * ab)}"


def test_xcorr_large_small_integers_exact():
    """Rows beyond 256 with small-integer inputs: exact in any summation order."""
    rng = np.random.default_rng(403)
    L = rng.integers(-2, 3, size=(2, 300, 24)).astype(np.float32)
    R = rng.integers(-2, 3, size=(1, 300, 24)).astype(np.float32)
    _gpu.log("xcorr 300-row small-integer exact")
    ref, _ = oracle.xcorr_f32(L, R)
    got = _gpu.run_xcorr(L, R, _lib.XC_XCORR_BLOCKDIAG)
    assert np.array_equal(got.astype(np.float64), ref)


def test_xcorr_large_delta_orientation():
    rows, cols = 270, 12
    for (a, b, c, d) in ((0, 0, 269, 11), (269, 11, 0, 0), (100, 3, 7, 9), (257, 0, 256, 11)):
        L = np.zeros((1, rows, cols), np.float32)
        R = np.zeros((1, rows, cols), np.float32)
        L[0, a, b] = 1.0
        R[0, c, d] = 1.0
        _gpu.log(f"xcorr 270-row delta ({a},{b}) ({c},{d})")
        got = _gpu.run_xcorr(L, R, _lib.XC_XCORR_BLOCKDIAG)
        expect = np.zeros((2 * rows - 1, 2 * cols - 1), np.float32)
        expect[a - c + rows - 1, b - d + cols - 1] = 1.0
        assert np.array_equal(got[0, 0], expect)


@pytest.mark.parametrize("shape", [
    # (n_left, n_right, rows, cols): pair groups that span several left matrices
    # (n_right below the pairs per wave), one right matrix, and n_right of 64
    # and more (the group's right index wraps at most once)
    (6, 3, 16, 16), (9, 2, 13, 20), (40, 1, 32, 8), (2, 70, 16, 16), (3, 65, 32, 32), (7, 5, 20, 4),
])
def test_xcorr_groupings(shape):
    nl, nr, rows, cols = shape
    rng = np.random.default_rng(1000 + nl * 97 + nr * 13 + rows)
    L = f32_uniform(rng, (nl, rows, cols))
    R = f32_uniform(rng, (nr, rows, cols))
    _gpu.log(f"xcorr grouping {shape}")
    ref, ab = oracle.xcorr_f32(L, R)
    _gpu.check_xcorr(_gpu.run_xcorr(L, R, _lib.XC_XCORR_BLOCKDIAG), ref, ab)


@pytest.mark.parametrize("shape", [(1, 1, 3, 200), (1, 1, 200, 3), (2, 1, 70, 65), (1, 2, 9, 64), (1, 1, 128, 1)])
def test_xcorr_wave_overlap_shapes(shape):
    """Wave-per-overlap on overlaps narrower and wider than a wave: a lane's
    next element wraps onto the next rows (64 // width of them) or stays in
    the row."""
    nl, nr, rows, cols = shape
    rng = np.random.default_rng(1700 + rows * 3 + cols)
    L = f32_uniform(rng, (nl, rows, cols))
    R = f32_uniform(rng, (nr, rows, cols))
    _gpu.log(f"xcorr wave-per-overlap {shape}")
    ref, ab = oracle.xcorr_f32(L, R)
    _gpu.check_xcorr(_gpu.run_xcorr(L, R, _lib.XC_XCORR_WAVE), ref, ab)


def test_xcorr_wave_large_sampled():
    """512x512 one-to-one through the wave-per-overlap kernel, sampled rows and
    columns of the output against the oracle, and the whole output within
    tolerance of the block-diagonal kernel's."""
    rng = np.random.default_rng(1710)
    rows = cols = 512
    L = f32_uniform(rng, (1, rows, cols))
    R = f32_uniform(rng, (1, rows, cols))
    _gpu.log("xcorr 512x512 wave-per-overlap, sampled")
    got = _gpu.run_xcorr(L, R, _lib.XC_XCORR_WAVE)
    oh, ow = 2 * rows - 1, 2 * cols - 1
    ys = np.concatenate([np.arange(oh), rng.integers(0, oh, 400)])
    xs = np.concatenate([rng.integers(0, ow, oh), rng.integers(0, ow, 400)])
    flat = ys * ow + xs
    ref, ab = oracle.xcorr_f32_points(L, R, flat)
    err = np.abs(got.reshape(-1)[flat].astype(np.float64) - ref)
    assert np.all(err <= 1e-5 * ab + 1e-30)
    bd = _gpu.run_xcorr(L, R, _lib.XC_XCORR_BLOCKDIAG)
    # both within 1e-5 * sum|lr| of the exact value: within twice that of each other
    sab = np.abs(L[0]).sum() * np.abs(R[0]).sum()
    assert np.max(np.abs(got.astype(np.float64) - bd)) <= 2e-5 * sab


# Matrices with a dimension of at most 16: rows 1 .. 12 (which the automatic
# choice gives to this kernel) with narrow and wide rows (the wide ones walk
# columns and keep the rows in registers), and narrow columns under tall rows.
SMALL_SHAPES = [(1, 1, 1, 1), (2, 3, 1, 9), (1, 2, 3, 2), (3, 5, 4, 4), (64, 64, 8, 8), (1, 512, 4, 4),
                (2, 2, 5, 7), (4, 3, 7, 13), (16, 16, 12, 12), (3, 2, 12, 16), (2, 2, 9, 17), (1, 3, 12, 100),
                (2, 1, 3, 300), (2, 2, 40, 6), (1, 2, 200, 16), (3, 3, 16, 40), (4, 4, 6, 200), (3, 1, 3, 300),
                (1, 1, 2, 1000)]


@pytest.mark.parametrize("shape", SMALL_SHAPES, ids=["x".join(map(str, s)) for s in SMALL_SHAPES])
@pytest.mark.parametrize("algo", [_lib.XC_XCORR_SMALL, _lib.XC_XCORR_AUTO])
def test_xcorr_small_matrices(shape, algo):
    nl, nr, rows, cols = shape
    if algo == _lib.XC_XCORR_AUTO and rows > 12:
        pytest.skip("the automatic choice takes the block-diagonal kernel from 13 rows")
    rng = np.random.default_rng(2000 + rows * 37 + cols * 3 + nl + nr)
    L = f32_uniform(rng, (nl, rows, cols))
    R = f32_uniform(rng, (nr, rows, cols))
    _gpu.log(f"xcorr small matrices {shape} algo={algo}")
    ref, ab = oracle.xcorr_f32(L, R)
    _gpu.check_xcorr(_gpu.run_xcorr(L, R, algo), ref, ab)


def test_xcorr_small_exact_and_orientation():
    """Small-integer inputs exactly, and delta matrices land on their shift, in
    both walking directions (rows in registers or columns in registers)."""
    rng = np.random.default_rng(2100)
    for rows, cols in ((6, 10), (10, 40), (3, 300), (200, 5)):
        L = rng.integers(-2, 3, size=(2, rows, cols)).astype(np.float32)
        R = rng.integers(-2, 3, size=(3, rows, cols)).astype(np.float32)
        _gpu.log(f"xcorr small exact {rows}x{cols}")
        ref, _ = oracle.xcorr_f32(L, R)
        assert np.array_equal(_gpu.run_xcorr(L, R, _lib.XC_XCORR_SMALL).astype(np.float64), ref)
        for (a, b, c, d) in ((0, 0, rows - 1, cols - 1), (rows - 1, cols - 1, 0, 0), (1, 3, rows - 2, 2)):
            Ld = np.zeros((1, rows, cols), np.float32)
            Rd = np.zeros((1, rows, cols), np.float32)
            Ld[0, a, b] = 1.0
            Rd[0, c, d] = 1.0
            got = _gpu.run_xcorr(Ld, Rd, _lib.XC_XCORR_SMALL)
            expect = np.zeros((2 * rows - 1, 2 * cols - 1), np.float32)
            expect[a - c + rows - 1, b - d + cols - 1] = 1.0
            assert np.array_equal(got[0, 0], expect)
    L = np.zeros((1, 20, 20), np.float32)
    with pytest.raises(_lib.XcError) as e:
        from cross_correlation_amd import api
        import torch
        api.xcorr_f32(torch.from_numpy(L).cuda(), torch.from_numpy(L).cuda(), algo=_lib.XC_XCORR_SMALL)
    assert e.value.status == _lib.XC_ERR_SHAPE


# Both dimensions at most 16 take the tiny-matrix kernel; these shapes reach
# each of its launched instances: lanes per group 1, 2, 4 or 8 with 1 to 4 row
# slots per lane, register widths 4, 8, 12 and 16, rows of whole float4s or
# not (cols below the register width).
TINY_SHAPES = [  # (rows, cols, n_left, n_right)
    (1, 16, 5, 7), (2, 8, 3, 4), (3, 4, 2, 2), (4, 4, 3, 5), (6, 16, 8, 8), (7, 13, 4, 3),
    (9, 12, 40, 30), (11, 5, 40, 30), (13, 3, 40, 30), (16, 16, 40, 30), (10, 8, 4, 4), (15, 14, 2, 3),
]


@pytest.mark.parametrize("shape", TINY_SHAPES, ids=["x".join(map(str, s)) for s in TINY_SHAPES])
def test_xcorr_tiny_instances(shape):
    rows, cols, nl, nr = shape
    rng = np.random.default_rng(2200 + rows * 17 + cols)
    L = f32_uniform(rng, (nl, rows, cols))
    R = f32_uniform(rng, (nr, rows, cols))
    _gpu.log(f"xcorr tiny {nl}x{nr} pairs of {rows}x{cols}")
    ref, ab = oracle.xcorr_f32(L, R)
    _gpu.check_xcorr(_gpu.run_xcorr(L, R, _lib.XC_XCORR_SMALL), ref, ab)
    # small integers: every product and sum exact, in any order
    Li = rng.integers(-3, 4, size=(nl, rows, cols)).astype(np.float32)
    Ri = rng.integers(-3, 4, size=(nr, rows, cols)).astype(np.float32)
    refi, _ = oracle.xcorr_f32(Li, Ri)
    assert np.array_equal(_gpu.run_xcorr(Li, Ri, _lib.XC_XCORR_SMALL).astype(np.float64), refi)
