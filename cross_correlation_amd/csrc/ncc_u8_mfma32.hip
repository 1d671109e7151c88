// ncc_u8_mfma32.hip -- u8 normalized correlation with SumIT on the 32x32x32
// i8 matrix cores, the template taken as the Toeplitz operand.
//
// Same outputs as the other u8 kernels for the computation of "The CUDA
// Handbook", ch. 15 "Image Processing: Normalized Correlation": the unsigned
// window sums SumI, SumISq, SumIT and Pearson's coefficient.  Like
// ncc_u8_mfma.hip this recasts the sum that pairs image and template bytes
// as a signed-byte matrix product (pixels and template biased by -128,
// SumIT = sum I'T' + 128 SumI + 128 SumT - 16384 N exactly, mod 2^32), but
// with the roles of the operands turned round:
//
//   * Product: for one workgroup tile of 32 output rows m and 128 output
//     columns (four 32-column tiles j), and each template row rt,
//       D_j[m][n] += sum_k A_{j+kb}[m][k] * B_kb[k][n]
//         A_a[m][k]  = I'[y0 + m + rt][x0 + 32a + k]   (image bytes as staged:
//                                                     aligned 16-byte reads)
//         B_kb[k][n] = T'[rt][32kb + k - n]           (template row rt shifted
//                                                     by the output column n;
//                                                     zero outside the row)
//     summed over kb = 0 .. NKB - 1 (NKB = ceil((t_width + 31) / 32)): the
//     window sum of output (y0 + m, x0 + 32j + n) over template row rt.  No
//     operand needs a byte shift per output column: the shift is in B, built
//     once per template row (four v_alignbyte_b32 per fragment) and used by
//     all four column tiles.  A fraction 1 - t_width / (32 NKB) of the
//     products is against the zero bytes around the template row.
//   * Template rows are split over the four matrix-core waves; their partial
//     sums are added in LDS (exact integer adds, so the order does not matter).
//   * SumI, SumISq: four helper waves (pixels or squares, for the first or
//     second 16 output rows) run beside the products.  Each keeps exact
//     column sums over the template's rows for 4 image columns per lane
//     (every image word of the tile's windows, one per lane) and slides them
//     down its 16 output rows; for each row it
//     takes the prefix along the row (in the lane, then a DPP scan across
//     lanes) and forms the window sums as differences of two prefix entries
//     read across lanes, writing SumI or SumISq to LDS.
//   * Two workgroups per CU (six waves each, at most 168 VGPRs), so each
//     SIMD holds two matrix-core waves.
//   * Epilogue: one output column per lane, so every store writes whole cache
//     lines; the coefficient with the exact formula of the other kernels
//     (ncc_coef_f32), so all kernels return the same bits.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"
#include "ncc_common.h"

namespace xc {

typedef int m32_v4i __attribute__((ext_vector_type(4)));
typedef int m32_v16i __attribute__((ext_vector_type(16)));

constexpr int M32_TY = 32;     // output rows per workgroup (the MFMA's M)
constexpr int M32_TX = 128;    // output columns per workgroup
constexpr int M32_NT = 4;      // 32-column tiles per matrix-core wave
constexpr int M32_MW = 4;      // matrix-core waves (template rows split four ways)
constexpr int M32_HW = 4;      // helper waves: field x half of the tile's rows
constexpr int M32_HROWS = M32_TY / 2;  // output rows per helper wave
constexpr int M32_THREADS = 64 * (M32_MW + M32_HW);
constexpr int M32_ACCS = 136;  // i32 per row of the merged SumIT' (the two row groups of a
                               // write sit 32 banks apart)
constexpr int M32_SRS = 132;   // u32 per row of the window sums

// 32-byte blocks of K a template row of t_width bytes needs: the output
// columns n = 0..31 of a tile read template bytes c = 32 kb + k - n, which
// must cover [0, t_width) for every n.  A one-byte row takes two blocks (the
// one-block instance needs more registers than a wave has).
__host__ __device__ constexpr int m32_nkb(int tw) { return tw < 2 ? 2 : (tw + 62) / 32; }

// LDS plan (host and device agree through it):
//   img   staged image rows (biased), M32_TY + t_height rows (one spare) of
//         s bytes; after the walk the merged SumIT' (M32_TY x M32_ACCS i32)
//   tpl   template rows (biased) with 32 zero bytes before and zeros after,
//         t_height + 1 rows of ptw bytes
//   sb    SumI and SumISq of the tile, M32_TY rows of M32_SRS each
//   tsum  SumT, SumTSq
struct M32Plan {
    int nkb, na, s, ptw, nwd;
    size_t img, tpl, sb, bytes;
};

__host__ __device__ inline M32Plan m32_plan(int tw, int th)
{
    M32Plan p;
    p.nkb = m32_nkb(tw);
    p.na = M32_NT + p.nkb - 1;       // 32-byte image blocks a tile row reads
    p.s = 32 * p.na + 16;            // 8 NA + 4 words: 16 consecutive rows start in 16 bank groups
    p.ptw = 32 * p.nkb + 48;         // covers the five words read from byte 32 NKB + 16
    p.nwd = (M32_TX + tw - 1 + 3) / 4;  // image words under the tile's windows (at most 48)
    const size_t img = (size_t)(M32_TY + th) * p.s, sit = (size_t)M32_TY * M32_ACCS * 4;
    p.img = ((img > sit ? img : sit) + 15) & ~(size_t)15;
    p.tpl = (size_t)(th + 1) * p.ptw;
    p.sb = (size_t)2 * M32_TY * M32_SRS * 4;
    p.bytes = p.img + p.tpl + p.sb + 16;
    return p;
}

// Image rows [gy0, gy0 + nrows) x 16-byte chunks [0, nchunks) from column gx0
// into LDS rows of `stride` bytes, biased to signed bytes; rows at or past
// `height` and chunks at or past `pitch` are zero pixels, so no load leaves
// the image allocation.  Loads of a batch of 8 are issued before its stores.
__device__ __forceinline__ void m32_stage_image(const uint8_t *__restrict__ image, int height, int pitch, int gy0,
                                                int gx0, int nrows, int nchunks, uint8_t *lds, int stride)
{
    constexpr int SB = 8;
    const int total = nrows * nchunks;
    for (int i0 = threadIdx.x; i0 < total; i0 += SB * M32_THREADS) {
        uint4 v[SB];
#pragma unroll
        for (int k = 0; k < SB; ++k) {
            const int i = i0 + k * M32_THREADS;
            const int r = i / nchunks;
            const int b = i - r * nchunks;
            const int gy = gy0 + r, gx = gx0 + 16 * b;
            const bool ok = i < total && gy < height && gx < pitch;
            v[k] = *reinterpret_cast<const uint4 *>(image + (ok ? (size_t)gy * pitch + gx : 0));
            if (!ok)
                v[k] = make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int k = 0; k < SB; ++k) {
            const int i = i0 + k * M32_THREADS;
            if (i < total) {
                const int r = i / nchunks;
                const int b = i - r * nchunks;
                uint4 w = v[k];
                w.x ^= 0x80808080u;
                w.y ^= 0x80808080u;
                w.z ^= 0x80808080u;
                w.w ^= 0x80808080u;
                *reinterpret_cast<uint4 *>(lds + r * stride + 16 * b) = w;
            }
        }
    }
}

// Template rows, biased, at LDS row rt: byte 32 + c holds T'[rt][c] for
// c < t_width, every other byte of the row is zero (a zero T' adds nothing to
// sum I'T').  The spare row t_height is zero too.
__device__ __forceinline__ void m32_stage_template(const uint8_t *__restrict__ tmpl, int tw, int th, uint8_t *tpl,
                                                   int ptw)
{
    const int wpr = ptw / 4, twords = (tw + 3) / 4;
    const uint32_t tm = tail_mask(tw);
    const bool wr = tmpl_word_rows(tmpl, tw);
    const int total = (th + 1) * wpr;
    constexpr int SB = 8;  // loads of a batch issued before its stores
    for (int i0 = threadIdx.x; i0 < total; i0 += SB * M32_THREADS) {
        uint32_t v[SB];
#pragma unroll
        for (int q = 0; q < SB; ++q) {
            const int i = i0 + q * M32_THREADS;
            const int r = i / wpr;
            const int k = i - r * wpr - 8;  // template word of this LDS word (32 bytes in)
            v[q] = 0u;
            if (i < total && r < th && k >= 0 && k < twords)
                v[q] = tmpl_word(tmpl, tw, wr, r, k) ^ (k == twords - 1 ? 0x80808080u & tm : 0x80808080u);
        }
#pragma unroll
        for (int q = 0; q < SB; ++q) {
            const int i = i0 + q * M32_THREADS;
            if (i < total)
                *reinterpret_cast<uint32_t *>(tpl + 4 * i) = v[q];
        }
    }
}

// The matrix-core walk of one wave over template rows [r0, r1), column tiles
// [0, tv) (FULL: all eight).  Lane (m, g) = (lane & 31, lane >> 5) reads
// image row m + rt at bytes 32a + 16g (16 bytes: K = 16g .. 16g + 15 of block
// a) and builds its B fragments from the padded template row: column n = m,
// bytes 32 kb + 16g - n .. + 15 of the row, i.e. padded bytes from
// b = 32 kb + 16g + 32 - n, five words and four byte alignments by b & 3.
// Rows go through two register sets: the next row's LDS reads are issued
// before the current row's products (the reads after the last row land in
// the spare rows).  Consecutive products go to different tiles.
template <int NKB, bool FULL>
__device__ __forceinline__ void m32_walk(const uint8_t *img, const uint8_t *tpl, int r0, int r1, int tv,
                                         m32_v16i (&acc)[M32_NT])
{
    constexpr int NA = M32_NT + NKB - 1, S = 32 * NA + 16, PTW = 32 * NKB + 48;
    if (r0 >= r1)
        return;
    const int lane = threadIdx.x & 63, m = lane & 31, g = lane >> 5;
    const int bb = 16 * g + 32 - m;  // >= 1
    const uint32_t sh = (uint32_t)bb & 3u;
    const uint8_t *ap = img + (m + r0) * S + 16 * g;
    const uint8_t *tp = tpl + r0 * PTW + (bb & ~3);
    auto load = [&](m32_v4i (&A)[NA], uint32_t (&W)[NKB][5]) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int q = 0; q < 5; ++q)
                W[kb][q] = *reinterpret_cast<const uint32_t *>(tp + 32 * kb + 4 * q);
#pragma unroll
        for (int a = 0; a < NA; ++a)
            A[a] = *reinterpret_cast<const m32_v4i *>(ap + 32 * a);
        ap += S;
        tp += PTW;
    };
    auto compute = [&](const m32_v4i (&A)[NA], const uint32_t (&W)[NKB][5]) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            m32_v4i B;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                B[q] = (int)__builtin_amdgcn_alignbyte(W[kb][q + 1], W[kb][q], sh);
#pragma unroll
            for (int j = 0; j < M32_NT; ++j)
                if (FULL || j < tv)
                    acc[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[j + kb], B, acc[j], 0, 0, 0);
        }
    };
    m32_v4i A0[NA], A1[NA];
    uint32_t W0[NKB][5], W1[NKB][5];
    load(A0, W0);
    int rt = r0;
    for (; rt + 2 <= r1; rt += 2) {
        load(A1, W1);  // row rt + 1
        compute(A0, W0);
        load(A0, W0);  // row rt + 2 (the spare row when rt + 2 == th)
        compute(A1, W1);
    }
    if (rt < r1)
        compute(A0, W0);
}

// Column sums of field F (0: pixels, 1: squared pixels) over four rows of one
// staged (biased) word u[0..3], added to c[0..3] (columns 4w .. 4w + 3): a
// 4x4 byte transpose (eight v_perm_b32) puts each column's four bytes in one
// word, then one dot4 per column.  F = 0 sums the biased bytes s = I - 128
// (signed), F = 1 the squares of the pixels themselves; wrapping u32.
template <int F>
__device__ __forceinline__ void m32_col4(const uint32_t (&u)[4], uint32_t (&c)[4])
{
    // perm(hi, lo, sel): byte i of the result is byte sel_i of hi:lo (lo in bytes 0..3)
    const uint32_t a_lo = __builtin_amdgcn_perm(u[1], u[0], 0x05010400u);
    const uint32_t a_hi = __builtin_amdgcn_perm(u[1], u[0], 0x07030602u);
    const uint32_t b_lo = __builtin_amdgcn_perm(u[3], u[2], 0x05010400u);
    const uint32_t b_hi = __builtin_amdgcn_perm(u[3], u[2], 0x07030602u);
    const uint32_t col[4] = {__builtin_amdgcn_perm(b_lo, a_lo, 0x05040100u),
                             __builtin_amdgcn_perm(b_lo, a_lo, 0x07060302u),
                             __builtin_amdgcn_perm(b_hi, a_hi, 0x05040100u),
                             __builtin_amdgcn_perm(b_hi, a_hi, 0x07060302u)};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if (F == 0) {
            c[k] = (uint32_t)__builtin_amdgcn_sdot4((int)col[k], 0x01010101, (int)c[k], false);
        } else {
            const uint32_t px = col[k] ^ 0x80808080u;
            c[k] = __builtin_amdgcn_udot4(px, px, c[k], false);
        }
    }
}

// One row of one word: c[k] += (F = 0) s_k, (F = 1) I_k^2 of the biased word u.
template <int F>
__device__ __forceinline__ void m32_col1(uint32_t u, uint32_t (&c)[4])
{
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if (F == 0) {
            c[k] = (uint32_t)__builtin_amdgcn_sdot4((int)u, (int)(1u << (8 * k)), (int)c[k], false);
        } else {
            const uint32_t px = u ^ 0x80808080u;
            c[k] = __builtin_amdgcn_udot4(px & (0xFFu << (8 * k)), px, c[k], false);
        }
    }
}

// Slide one word's column sums down one row: add row `in`, remove row `out`.
template <int F>
__device__ __forceinline__ void m32_slide1(uint32_t in, uint32_t out, uint32_t (&c)[4])
{
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if (F == 0) {
            c[k] = (uint32_t)__builtin_amdgcn_sdot4((int)in, (int)(1u << (8 * k)), (int)c[k], false);
            c[k] = (uint32_t)__builtin_amdgcn_sdot4((int)out, (int)(0xFFu << (8 * k)), (int)c[k], false);
        } else {
            const uint32_t pi = in ^ 0x80808080u, po = out ^ 0x80808080u;
            const uint32_t d = __builtin_amdgcn_udot4(po & (0xFFu << (8 * k)), po, 0u, false);
            c[k] = __builtin_amdgcn_udot4(pi & (0xFFu << (8 * k)), pi, c[k], false) - d;
        }
    }
}

// Inclusive prefix sum over the 64 lanes of a wave in DPP moves: shifts by
// 1, 2, 4 and 8 lanes within each row of 16 (lanes shifted in from outside
// the row read 0), then lane 15's total added to rows 1 and 3 and lane 31's
// to rows 2 and 3.  Every lane of the wave must take part.
__device__ __forceinline__ uint32_t m32_wave_scan(uint32_t v)
{
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, true);   // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, true);   // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, true);   // row_shr:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, true);   // row_shr:8
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);  // row_bcast:15
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return v;
}

// A helper wave: field F (0: pixels, 1: squared pixels) over the tile's 32
// output rows.  Lane l holds image word l (columns 4l .. 4l + 3 of the tile;
// lanes past the last word repeat it, which changes no prefix below them).
// The column sums of the first output row's window, then for each output
// row: the prefix along the row at the lane's four columns (a running sum in
// the lane plus an exclusive scan of the lane totals), the window sums of
// outputs x = 4l + k as the prefix at x + t_width - 1 less the one at x - 1
// (read from lanes l + d and l + d + 1, d = (t_width - 1) / 4, and l - 1),
// stored by the lanes of the 128 outputs, and the slide to the next row.
// All u32, exact (every window sum is below 2^32).
template <int F>
__device__ __forceinline__ void m32_helper(const uint8_t *img, int S, int th, int tw, int nwd, int row0, uint32_t *srow)
{
    const int lane = threadIdx.x & 63;
    const int wd = lane < nwd ? lane : nwd - 1;
    uint32_t c[4] = {0u, 0u, 0u, 0u};
    int r = 0;
#pragma unroll 2
    for (; r + 4 <= th; r += 4) {
        uint32_t u[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            u[q] = *reinterpret_cast<const uint32_t *>(img + (row0 + r + q) * S + 4 * wd);
        m32_col4<F>(u, c);
    }
    for (; r < th; ++r)
        m32_col1<F>(*reinterpret_cast<const uint32_t *>(img + (row0 + r) * S + 4 * wd), c);
    const uint32_t add = F == 0 ? 128u * (uint32_t)th : 0u;
    const int d = (tw - 1) >> 2, rr = (tw - 1) & 3;  // wave-uniform
    const int la = min(lane + d, 63), lb = min(lane + d + 1, 63), lp = max(lane - 1, 0);
    // the words leaving and entering the column sums for the next row, loaded
    // one row ahead so the LDS latency overlaps this row's scan and shuffles
    uint32_t w_in = *reinterpret_cast<const uint32_t *>(img + (row0 + th) * S + 4 * wd);
    uint32_t w_out = *reinterpret_cast<const uint32_t *>(img + row0 * S + 4 * wd);
    const int row1 = row0 + M32_HROWS;
    for (int m = row0; m < row1; ++m) {
        const uint32_t v0 = c[0] + add, v1 = c[1] + add, v2 = c[2] + add, v3 = c[3] + add;
        if (m + 1 < row1) {
            m32_slide1<F>(w_in, w_out, c);
            if (m + 2 < row1) {
                w_in = *reinterpret_cast<const uint32_t *>(img + (m + 1 + th) * S + 4 * wd);
                w_out = *reinterpret_cast<const uint32_t *>(img + (m + 1) * S + 4 * wd);
            }
        }
        const uint32_t p1 = v0 + v1, p2 = p1 + v2, t = p2 + v3;
        const uint32_t before = m32_wave_scan(t) - t;
        const uint32_t pre[4] = {before + v0, before + p1, before + p2, before + t};
        const uint32_t a[4] = {(uint32_t)__shfl((int)pre[0], la, 64), (uint32_t)__shfl((int)pre[1], la, 64),
                               (uint32_t)__shfl((int)pre[2], la, 64), (uint32_t)__shfl((int)pre[3], la, 64)};
        const uint32_t b[3] = {(uint32_t)__shfl((int)pre[0], lb, 64), (uint32_t)__shfl((int)pre[1], lb, 64),
                               (uint32_t)__shfl((int)pre[2], lb, 64)};
        // every lane takes part in the permute (a masked-off source lane reads
        // as zero), then lane 0 drops it
        const uint32_t left = (uint32_t)__shfl((int)pre[3], lp, 64);
        const uint32_t prev = lane > 0 ? left : 0u;
        // hi[k] = prefix at column 4l + k + tw - 1: component k + rr of lane
        // l + d, continuing into lane l + d + 1
        uint4 hi;
        switch (rr) {
        case 0: hi = make_uint4(a[0], a[1], a[2], a[3]); break;
        case 1: hi = make_uint4(a[1], a[2], a[3], b[0]); break;
        case 2: hi = make_uint4(a[2], a[3], b[0], b[1]); break;
        default: hi = make_uint4(a[3], b[0], b[1], b[2]); break;
        }
        if (lane < M32_TX / 4)
            *reinterpret_cast<uint4 *>(srow + m * M32_SRS + 4 * lane) =
                make_uint4(hi.x - prev, hi.y - pre[0], hi.z - pre[1], hi.w - pre[2]);
    }
}

// Workgroup roles (wave-uniform): waves 0..3 run the matrix cores over a
// quarter of the template rows each, for all 128 columns of the tile; waves
// 4..7 are the helpers (pixels for rows 0..15, squares for rows 0..15, then
// the same for rows 16..31); wave 0 also sums the template after its walk.
// Every wave stages, and every wave takes part in the epilogue.
template <int NKB>
__global__ __launch_bounds__(M32_THREADS) __attribute__((amdgpu_waves_per_eu(3)))
void ncc_u8_mfma32_kernel(NccArgs a)
{
    extern __shared__ uint4 m32_smem[];
    const M32Plan P = m32_plan(a.t_width, a.t_height);
    uint8_t *const img = reinterpret_cast<uint8_t *>(m32_smem);
    uint8_t *const tpl = img + P.img;
    uint32_t *const sb = reinterpret_cast<uint32_t *>(tpl + P.tpl);
    uint32_t *const tsum = sb + P.sb / 4;
    int32_t *const sit = reinterpret_cast<int32_t *>(img);

    const int x0 = blockIdx.x * M32_TX, y0 = blockIdx.y * M32_TY;
    const int tw = a.t_width, th = a.t_height;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    m32_stage_image(a.image, a.height, a.pitch, y0, x0, M32_TY + th, 2 * P.na, img, P.s);
    m32_stage_template(a.tmpl, tw, th, tpl, P.ptw);
    __syncthreads();

    m32_v16i acc[M32_NT];
#pragma unroll
    for (int j = 0; j < M32_NT; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v)
            acc[j][v] = 0;
    if (wave < M32_MW) {
        const int hq = (th + M32_MW - 1) / M32_MW;
        const int r0 = min(th, wave * hq), r1 = min(th, r0 + hq);
        const int tv = min(M32_NT, (a.out_w - x0 + 31) / 32);
        if (tv == M32_NT)
            m32_walk<NKB, true>(img, tpl, r0, r1, tv, acc);
        else
            m32_walk<NKB, false>(img, tpl, r0, r1, tv, acc);
        if (wave == 0) {  // the helpers are still busy when the walks end
            uint32_t ts, tq;
            template_sums(a.tmpl, tw, th, ts, tq);
            if (lane == 0) {
                tsum[0] = ts;
                tsum[1] = tq;
            }
        }
    } else {
        const int hw = wave - M32_MW, row0 = (hw >> 1) * M32_HROWS;
        if ((hw & 1) == 0)
            m32_helper<0>(img, P.s, th, tw, P.nwd, row0, sb);
        else
            m32_helper<1>(img, P.s, th, tw, P.nwd, row0, sb + M32_TY * M32_SRS);
    }
    __syncthreads();  // the image tile is free; SumI, SumISq and the template sums are in LDS

    // SumIT' of the four walks, added in LDS: lane (n, hh) of a tile holds
    // rows 8 (v >> 2) + 4 hh + (v & 3) of column n in accumulator v.
    const int n = lane & 31, hh = lane >> 5;
    if (wave == 0) {
#pragma unroll
        for (int j = 0; j < M32_NT; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                sit[(8 * (v >> 2) + 4 * hh + (v & 3)) * M32_ACCS + 32 * j + n] = acc[j][v];
    }
    __syncthreads();
    if (wave > 0 && wave < M32_MW) {
#pragma unroll
        for (int j = 0; j < M32_NT; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                atomicAdd(&sit[(8 * (v >> 2) + 4 * hh + (v & 3)) * M32_ACCS + 32 * j + n], acc[j][v]);
    }
    __syncthreads();

    const uint32_t nn = (uint32_t)(tw * th);
    const uint32_t sum_t = tsum[0], sum_tsq = tsum[1];
    const uint32_t bias = 128u * sum_t - 16384u * nn;
    // num, vI, vT are integers below 2^50, formed exactly with fp64 fused
    // multiply-adds (the same doubles as the 64-bit integer form)
    const double nd = (double)nn, std_ = (double)sum_t;
    const double vt = fma(nd, (double)sum_tsq, -(std_ * std_));
    const uint32_t *const s_i = sb, *const s_q = sb + M32_TY * M32_SRS;

    // one output column per lane, rows advancing by 3 (384 threads)
    const int x = threadIdx.x & (M32_TX - 1), gx = x0 + x;
    const size_t o0 = (size_t)y0 * a.out_w + x0;
    uint32_t *const out_i = a.sum_i ? a.sum_i + o0 : nullptr;
    uint32_t *const out_isq = a.sum_isq ? a.sum_isq + o0 : nullptr;
    uint32_t *const out_it = a.sum_it ? a.sum_it + o0 : nullptr;
    float *const out_c = a.coef ? a.coef + o0 : nullptr;
    unsigned long long best = 0ull;
    if (gx < a.out_w) {
        for (int m = threadIdx.x / M32_TX; m < M32_TY && y0 + m < a.out_h; m += M32_THREADS / M32_TX) {
            const uint32_t off = (uint32_t)m * (uint32_t)a.out_w + (uint32_t)x;
            const uint32_t si = s_i[m * M32_SRS + x], sq = s_q[m * M32_SRS + x];
            const uint32_t st = (uint32_t)sit[m * M32_ACCS + x] + 128u * si + bias;
            if (out_i) out_i[off] = si;
            if (out_isq) out_isq[off] = sq;
            if (out_it) out_it[off] = st;
            if (out_c || a.peak) {
                const double sid = (double)si;
                const double num = fma(nd, (double)st, -(sid * std_));
                const double vi = fma(nd, (double)sq, -(sid * sid));
                float cf = 0.0f;
                if (vi != 0.0 && vt != 0.0)
                    cf = ncc_coef_f32(num, vi * vt);
                if (out_c) out_c[off] = cf;
                if (a.peak) {
                    const unsigned long long k = peak_key(cf, (uint32_t)(o0 + off));
                    best = k > best ? k : best;
                }
            }
        }
    }
    if (a.peak)
        peak_commit_wg(a.peak, best, reinterpret_cast<unsigned long long *>(tpl));
}

bool ncc_mfma32_supported(const NccArgs &a)
{
    return a.t_width <= 65 && m32_plan(a.t_width, a.t_height).bytes <= 160 * 1024;
}

template <int NKB>
static hipError_t m32_launch(const NccArgs &a, hipStream_t s)
{
    static std::atomic<uint64_t> lds_allowed{0};
    const hipError_t e = allow_lds_once(&ncc_u8_mfma32_kernel<NKB>, lds_allowed);
    if (e != hipSuccess)
        return e;
    const dim3 grid((a.out_w + M32_TX - 1) / M32_TX, (a.out_h + M32_TY - 1) / M32_TY);
    hipLaunchKernelGGL((ncc_u8_mfma32_kernel<NKB>), grid, dim3(M32_THREADS), m32_plan(a.t_width, a.t_height).bytes,
                       s, a);
    return hipGetLastError();
}

hipError_t ncc_launch_mfma32(NccArgs a, hipStream_t s)
{
    if (!ncc_mfma32_supported(a))
        return hipErrorInvalidValue;
    switch (m32_nkb(a.t_width)) {
    case 2: return m32_launch<2>(a, s);
    default: return m32_launch<3>(a, s);
    }
}

} // namespace xc
