// ncc_u8_mfma.hip -- u8 normalized correlation with SumIT on the i8 matrix
// cores (v_mfma_i32_16x16x64_i8) and SumI / SumISq as exact separable box sums.
//
// Same outputs as the packed-byte kernels (ncc_u8.hip) for the computation of
// "The CUDA Handbook", ch. 15 "Image Processing: Normalized Correlation": the
// unsigned window sums SumI, SumISq, SumIT and Pearson's coefficient.  The
// page computes all three sums with DP4A; this variant recasts the one sum
// that pairs image and template bytes as a matrix product:
//
//   * Bias: I' = I - 128 and T' = T - 128 are signed bytes (an XOR with 0x80),
//     and  SumIT = sum I'T' + 128*SumI + 128*SumT - 16384*N  exactly (mod 2^32,
//     and the true value is below 2^32), so the signed i8 MFMA serves.
//   * Product: for one workgroup tile of 16 output rows n and output columns
//     x = x0 + 4m + t (m = 0..15, t = 0..3 per wave) and each image row r of
//     the tile,  D_t[m][n] += sum_k A_t[m][k] * B[k][n]  with
//       A_t[m][k] = I'[r][x0 + 4m + t + k]     (the window bytes: byte-shifted
//                                              image words, v_alignbyte_b32)
//       B[k][n]   = T'[r - n][k]               (template row r - n, zero when
//                                              that row does not exist)
//     k runs over 64-byte blocks of the template row.  Summed over r this is
//     the window sum over every template row (B is the template placed
//     Toeplitz-wise along the output rows); a fraction 15/(t_height + 15) of
//     the products is against zero rows.
//   * SumI and SumISq: while the matrix-core waves run, the column-sum waves
//     walk the tile's image words (4 columns each) down the template's rows,
//     keeping running sums per column of the biased pixels s = I - 128 and of
//     the squares (one field each; with four matrix-core waves, two waves per
//     field, one per half of the tile's outputs), four rows at a time through
//     a byte transpose and one dot4 per column: the window of output row 0.
//     Each then slides its window down the 16 output rows (add the row
//     entering, remove the row leaving; the tile's first 15 rows are kept
//     for that when the template comes in several chunks) and, as each row
//     appears, takes its prefix along the wave's words in registers (a DPP
//     scan), from which a window sum is the difference of two entries.
//   * Window sums or prefixes.  For templates up to 128 bytes wide a
//     column-sum wave takes every word its 128 outputs read (the two halves
//     of a 256-column tile overlap by the template's width), so it forms the
//     window sums itself (the prefix at x + t_width - 1 less the one at x - 1,
//     read across lanes), SumI = sum s + 128 N and SumISq = sum I^2 (the
//     squares of the unbiased pixels), keeps them in LDS for the epilogue and
//     stores them to the outputs while the matrix-core waves still walk, so
//     only SumIT and the coefficient are written at the end.  Wider templates
//     (and narrow tiles whose window sums would not take less LDS) keep the
//     row prefixes of s and s^2 over disjoint halves; the epilogue then forms
//     every sum, adding the first half's row total where a window spans both
//     halves, and SumISq = sum s^2 + 256 SumI - 16384 N.  All in wrapping
//     32-bit arithmetic, exact because every final sum is below 2^32.
//   * Tiles: 16 output rows by 256 columns (four matrix-core waves, two
//     workgroups per CU) or 128 columns (two, four workgroups per CU, for
//     templates up to 64 bytes wide); the launcher takes the narrow tiles
//     when they run the grid in fewer rounds of workgroups, or when the wide
//     ones would cover at most half of the CUs.  Narrow tiles store row
//     prefixes when the template then fits one row chunk, else window sums.
//   * The coefficient follows the packed-byte kernels' exact formula: num, vI
//     and vT are exact integers (held in fp64 here, formed with fused
//     multiply-adds), then ncc_coef_f32, so both paths return the same bits.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"
#include "ncc_common.h"

namespace xc {

typedef int mf_v4i __attribute__((ext_vector_type(4)));

constexpr int MF_TY = 16;          // output rows per workgroup (MFMA N)
constexpr int MF_MAX_NKB = 4;      // template rows up to 256 bytes
constexpr int MF_MAX_HC = 256;     // template rows per chunk

// A workgroup runs MW matrix-core waves of 64 output columns each, then its
// column-sum waves: with MW = 4 one per field and half of the image words,
// with MW = 2 (templates up to 64 bytes wide, whose 128 + t_width columns fit
// one wave's 64 lanes of words) one per field for all of them.
__host__ __device__ constexpr int mf_tx(int mw) { return 64 * mw; }
__host__ __device__ constexpr int mf_walkers(int mw) { return mw == 4 ? 4 : 2; }
__host__ __device__ constexpr int mf_threads(int mw) { return 64 * (mw + mf_walkers(mw)); }
// i32 words per output row of the SumIT staging (odd: rows start in different banks)
__host__ __device__ constexpr int mf_acc_stride(int mw) { return 64 * mw + 1; }

// LDS plan of one workgroup (host and device agree through these helpers):
//   V     2*MF_TY rows x vs u32: column sums of pixels (rows 0..15) and of
//         squares (rows 16..31), then their row prefix (per half of the words)
//   img   the staged image tile plus one spare row; after the walk, the
//         SumIT' staging of MF_TY x mf_acc_stride(MW) i32
//   tpl   template rows with zero rows around them (trows rows of tsb bytes)
//   head  the tile's first MF_TY - 1 image rows (words 0..nwd-1), kept for
//         the sliding pass when the template comes in several chunks
//   tsum  SumT and SumTSq
struct MfPlan {
    int nkb;      // 64-byte blocks per template row
    int hc;       // template rows per chunk
    int sw;       // image LDS words per row
    int tsb;      // template LDS bytes per row
    int trows;    // template LDS rows
    int nwd;      // image words covered by the column sums (16 MW .. 16 MW + 64)
    int vs;       // u32 per row of V (a multiple of 4: 16-byte stores)
    int img_words;
    int head_words;  // the first MF_TY - 1 rows' words, kept only when the template comes in several chunks
    size_t bytes;
};

// LDS row strides for MW matrix waves and NKB 64-byte template blocks
// (compile-time in the kernels, so consecutive rows are immediate offsets of
// one address)
__host__ __device__ constexpr int mf_sw(int mw, int nkb) { return 16 * mw + 16 * nkb + 4; }
// Template rows: 64-byte blocks plus 16 bytes of padding, or 32 for the
// 256-column tiles of one block, whose 16-byte B-fragment reads (lane m at row
// 15 - m) then meet no LDS bank conflicts: SQ_LDS_BANK_CONFLICT of the 1080p /
// 64x64 launch 707,584 -> 60,416 cycles (a 48-byte pad conflicts as 16 does;
// the 128-column tiles keep 16, as 32 would push a 64x64 template out of one
// row chunk of their 40 KiB)
__host__ __device__ constexpr int mf_tsb(int mw, int nkb) { return 64 * nkb + (mw == 4 && nkb == 1 ? 32 : 16); }

__host__ __device__ inline MfPlan mf_plan(int mw, int t_width, int hc, bool one_chunk, bool win)
{
    MfPlan p;
    p.nkb = (t_width + 63) / 64;
    p.hc = hc;
    p.sw = mf_sw(mw, p.nkb);
    p.tsb = mf_tsb(mw, p.nkb);
    p.trows = hc + 2 * MF_TY - 1;
    p.nwd = 16 * mw + (t_width + 2) / 4;  // words holding columns 0 .. 64 mw - 1 + t_width - 1
    // each row's prefix over the words (in two halves when MW = 4), or with
    // `win` (MW = 2) the window sums of the tile's 128 outputs themselves,
    // which take less LDS (a row is stored and read by consecutive lanes, so
    // it needs no padding)
    p.vs = win ? 64 * mw : 4 * p.nwd + 4;
    int img = (MF_TY + hc) * p.sw;  // staged rows + one spare row
    if (img < MF_TY * mf_acc_stride(mw)) img = MF_TY * mf_acc_stride(mw);
    p.img_words = img;
    p.head_words = one_chunk ? 0 : (MF_TY - 1) * p.nwd;
    p.bytes = (size_t)2 * MF_TY * p.vs * 4 + (size_t)img * 4 + (size_t)p.trows * p.tsb +
              (size_t)p.head_words * 4 + 8;
    return p;
}

// Image rows [gy0, gy0 + nrows) x words [0, 4*nchunks) from column gx0, biased
// to signed bytes; rows at or past `height` and chunks at or past `pitch` are
// zero-filled, so no load leaves the image allocation.
// Each thread takes its items in batches of 4, all loads of a batch issued
// before any of its LDS stores (one memory round trip per batch); a chunk
// outside the image loads from the image base and is zeroed afterwards.
template <int NT>
__device__ __forceinline__ void mf_stage_image(const uint8_t *__restrict__ image, int height, int pitch, int gy0,
                                               int gx0, int nrows, int nchunks, uint32_t *lds, int stride)
{
    constexpr int SB = 4;
    const int total = nrows * nchunks;
    for (int i0 = threadIdx.x; i0 < total; i0 += SB * NT) {
        uint4 v[SB];
#pragma unroll
        for (int k = 0; k < SB; ++k) {
            const int i = i0 + k * NT;
            const int r = i / nchunks;
            const int b = i - r * nchunks;
            const int gy = gy0 + r;
            const int gx = gx0 + 16 * b;
            const bool ok = i < total && gy < height && gx < pitch;
            v[k] = *reinterpret_cast<const uint4 *>(image + (ok ? (size_t)gy * pitch + gx : 0));
            if (!ok)
                v[k] = make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int k = 0; k < SB; ++k) {
            const int i = i0 + k * NT;
            if (i < total) {
                const int r = i / nchunks;
                const int b = i - r * nchunks;
                uint4 w = v[k];
                w.x ^= 0x80808080u;
                w.y ^= 0x80808080u;
                w.z ^= 0x80808080u;
                w.w ^= 0x80808080u;
                *reinterpret_cast<uint4 *>(lds + r * stride + 4 * b) = w;
            }
        }
    }
}

// Template rows [j0, j0 + hcur) biased to signed bytes at LDS rows
// [MF_TY - 1, MF_TY - 1 + hcur), with MF_TY - 1 zero rows before and MF_TY
// after (the template rows that do not exist for some output row of the tile,
// and the spare row the pipelined walk reads last) and zero bytes beyond
// t_width up to the 64-byte block (a zero byte of T' adds nothing to sum I'T').
template <int NT>
__device__ __forceinline__ void mf_stage_template(const uint8_t *__restrict__ tmpl, int t_width, int j0, int hcur,
                                                  int kw, uint8_t *tpl, int tsb, int trows)
{
    const int wpr = kw / 4;  // words per staged row
    const int twords = (t_width + 3) / 4;
    const int total = trows * wpr;
    if (tmpl_word_rows(tmpl, t_width)) {
        // whole-word rows, in batches of 4 (loads first, then the LDS stores)
        constexpr int SB = 4;
        for (int i0 = threadIdx.x; i0 < total; i0 += SB * NT) {
            uint32_t v[SB];
#pragma unroll
            for (int q = 0; q < SB; ++q) {
                const int i = i0 + q * NT;
                const int r = i / wpr;
                const int k = i - r * wpr;
                const int j = r - (MF_TY - 1);
                const bool ok = i < total && j >= 0 && j < hcur && k < twords;
                v[q] = reinterpret_cast<const uint32_t *>(tmpl)[ok ? (size_t)(j0 + j) * (t_width >> 2) + k : 0];
                v[q] = ok ? v[q] ^ 0x80808080u : 0u;
            }
#pragma unroll
            for (int q = 0; q < SB; ++q) {
                const int i = i0 + q * NT;
                if (i < total) {
                    const int r = i / wpr;
                    const int k = i - r * wpr;
                    *reinterpret_cast<uint32_t *>(tpl + r * tsb + 4 * k) = v[q];
                }
            }
        }
    } else {
        // gathered words; the partial last word is biased on its template bytes only
        const uint32_t tm = tail_mask(t_width);
        for (int i = threadIdx.x; i < total; i += blockDim.x) {
            const int r = i / wpr;
            const int k = i - r * wpr;
            const int j = r - (MF_TY - 1);
            uint32_t v = 0u;
            if (j >= 0 && j < hcur && k < twords)
                v = tmpl_word(tmpl, t_width, false, j0 + j, k) ^ (k == twords - 1 ? 0x80808080u & tm : 0x80808080u);
            *reinterpret_cast<uint32_t *>(tpl + r * tsb + 4 * k) = v;
        }
    }
}

// Column sums of field F over one staged image word (4 columns of biased
// pixels s = I - 128, signed bytes), into c[0..3]: F = 0 adds s, F = 1 adds
// s^2 (v_dot4_i32_i8), F = 2 adds I^2 (v_dot4_u32_u8 on the unbiased bytes);
// wrapping 32-bit sums.  SumI = sum s + 128 N and SumISq = sum s^2 + 256 SumI
// - 16384 N, or sum I^2 itself, exactly.
template <int F>
__device__ __forceinline__ void mf_col_add(uint32_t biased, uint32_t (&c)[4])
{
    if (F == 2) {
        const uint32_t u = biased ^ 0x80808080u;  // the pixels themselves
#pragma unroll
        for (int k = 0; k < 4; ++k)
            c[k] = __builtin_amdgcn_udot4(u & (0xFFu << (8 * k)), u, c[k], false);
        return;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k)
        c[k] = (uint32_t)__builtin_amdgcn_sdot4(
            F == 0 ? (int)biased : (int)(biased & (0xFFu << (8 * k))), F == 0 ? (int)(1u << (8 * k)) : (int)biased,
            (int)c[k], false);
}

// Column sums of field F over the same word of four consecutive rows u[0..3]:
// a 4x4 byte transpose (eight v_perm_b32) gives each column's four bytes in
// one word, which one dot4 then sums, against ones (F = 0) or against itself
// (F = 1 on the biased bytes, F = 2 on the pixels themselves).  The same
// sums as four calls of mf_col_add, in fewer instructions (12 or 16 per four
// rows instead of 16, 32 or 36).
template <int F>
__device__ __forceinline__ void mf_col_add4(const uint32_t (&u)[4], uint32_t (&c)[4])
{
    // perm(hi, lo, sel): byte i of the result is byte sel_i of hi:lo (lo in bytes 0..3)
    const uint32_t a_lo = __builtin_amdgcn_perm(u[1], u[0], 0x05010400u);  // u0.b0 u1.b0 u0.b1 u1.b1
    const uint32_t a_hi = __builtin_amdgcn_perm(u[1], u[0], 0x07030602u);  // u0.b2 u1.b2 u0.b3 u1.b3
    const uint32_t b_lo = __builtin_amdgcn_perm(u[3], u[2], 0x05010400u);
    const uint32_t b_hi = __builtin_amdgcn_perm(u[3], u[2], 0x07030602u);
    uint32_t col[4] = {__builtin_amdgcn_perm(b_lo, a_lo, 0x05040100u), __builtin_amdgcn_perm(b_lo, a_lo, 0x07060302u),
                       __builtin_amdgcn_perm(b_hi, a_hi, 0x05040100u), __builtin_amdgcn_perm(b_hi, a_hi, 0x07060302u)};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if (F == 0)
            c[k] = (uint32_t)__builtin_amdgcn_sdot4((int)col[k], 0x01010101, (int)c[k], false);
        else if (F == 1)
            c[k] = (uint32_t)__builtin_amdgcn_sdot4((int)col[k], (int)col[k], (int)c[k], false);
        else {
            const uint32_t px = col[k] ^ 0x80808080u;
            c[k] = __builtin_amdgcn_udot4(px, px, c[k], false);
        }
    }
}

// The matrix-core walk of one template-row chunk for one wave: every image
// row of the chunk's tile against the template rows it meets, NKB 64-byte
// blocks per row; rows go in pairs through two register sets, the next row's
// LDS words read while the current row's products issue (the read after the
// last row lands in the spare row each LDS area keeps).
template <int MW, int NKB>
__device__ __forceinline__ void mf_walk_chunk(const uint32_t *img, const uint8_t *tpl, int hcur, int wave,
                                              mf_v4i (&at)[4])
{
    constexpr int sw = mf_sw(MW, NKB), tsb = mf_tsb(MW, NKB);
    const int lane = threadIdx.x & 63;
    const int m = lane & 15, g = lane >> 4;
    // A: output column x0 + 64*wave + 4m + t reads image words from 16*wave + m
    // (+ 4g for its 16 bytes of the 64-byte block).  B: output row n = m meets
    // template row rr - n, staged at LDS row rr - n + MF_TY - 1.
    const uint32_t *ip = img + 16 * wave + m + 4 * g;
    const uint8_t *tp = tpl + (MF_TY - 1 - m) * tsb + 16 * g;
    const int nrows = MF_TY - 1 + hcur;

    auto load = [&](uint32_t (&w)[NKB][5], mf_v4i (&b)[NKB]) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
            for (int k = 0; k < 5; ++k)
                w[kb][k] = ip[16 * kb + k];
            b[kb] = *reinterpret_cast<const mf_v4i *>(tp + 64 * kb);
        }
        ip += sw;
        tp += tsb;
    };
    auto compute = [&](const uint32_t (&w)[NKB][5], const mf_v4i (&b)[NKB]) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            mf_v4i av[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                av[0][k] = (int)w[kb][k];
                av[1][k] = (int)shift_bytes(w[kb][k + 1], w[kb][k], 1);
                av[2][k] = (int)shift_bytes(w[kb][k + 1], w[kb][k], 2);
                av[3][k] = (int)shift_bytes(w[kb][k + 1], w[kb][k], 3);
            }
#pragma unroll
            for (int t = 0; t < 4; ++t)
                at[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[t], b[kb], at[t], 0, 0, 0);
        }
    };
    uint32_t wa[NKB][5], wb[NKB][5];
    mf_v4i ba[NKB], bb[NKB];
    load(wa, ba);
    int rr = 0;
    for (; rr + 2 <= nrows; rr += 2) {
        load(wb, bb);  // row rr + 1
        compute(wa, ba);
        load(wa, ba);  // row rr + 2 (the spare row when rr + 2 == nrows)
        compute(wb, bb);
    }
    if (rr < nrows)
        compute(wa, ba);
}

// The column walk of field F over tile rows [0, hcur) of one chunk (absolute
// rows j0 .. j0 + hcur - 1) for image word wd of this lane, into c.  With
// save_head the raw words of the first MF_TY - 1 absolute rows go to `head`
// for the sliding pass of the last chunk (only when `keep`: lanes past their
// wave's words read a clamped word and store nothing).
template <int MW, int NKB, int F>
__device__ __forceinline__ void mf_col_walk(const uint32_t *img, int hcur, int j0, bool save_head, uint32_t *head,
                                            int nwd, int wd, bool keep, uint32_t (&c)[4])
{
    constexpr int sw = mf_sw(MW, NKB);
    const uint32_t *p = img + wd;
    constexpr int U = 4;
    int rr = 0;
    for (; rr + U <= hcur; rr += U) {
        uint32_t u[U];
#pragma unroll
        for (int q = 0; q < U; ++q)
            u[q] = p[(rr + q) * sw];
        mf_col_add4<F>(u, c);
    }
    for (; rr < hcur; ++rr)
        mf_col_add<F>(p[rr * sw], c);
    if (save_head && keep)
        for (rr = 0; rr < hcur && j0 + rr < MF_TY - 1; ++rr)
            head[(j0 + rr) * nwd + wd] = p[rr * sw];
}

// Inclusive prefix sum over the 64 lanes of a wave in DPP moves: shifts by
// 1, 2, 4 and 8 lanes within each row of 16 (lanes shifted in from outside
// the row read 0), then lane 15's total added to rows 1 and 3 and lane 31's
// to rows 2 and 3.  Every lane of the wave must take part.
__device__ __forceinline__ uint32_t mf_wave_scan(uint32_t v)
{
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, true);   // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, true);   // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, true);   // row_shr:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, true);   // row_shr:8
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);  // row_bcast:15
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return v;
}

// One row of a column-sum wave's prefix: lane l holds the column sums c of
// word w0 + l, i.e. columns 4l .. 4l + 3 of the wave's half; the inclusive
// prefix along the half at those columns is the sum over the lanes before
// plus the running sum of c.  Lanes past the half (repeating its last word)
// sit above every lane they could disturb.
__device__ __forceinline__ uint4 mf_row_prefix4(const uint32_t (&c)[4])
{
    const uint32_t p1 = c[0] + c[1], p2 = p1 + c[2], t = p2 + c[3];
    const uint32_t before = mf_wave_scan(t) - t;
    return make_uint4(before + c[0], before + p1, before + p2, before + t);
}

// The sliding pass of field F for word wd after the last chunk's walk: c holds
// the column sums of absolute rows [0, th), i.e. output row 0's window.  Row
// n's window adds absolute row n + th - 1 (tile row hcur + n - 1 of the last
// chunk) and drops absolute row n - 1 (tile row n - 1 when the template came
// in one chunk, else the saved head row).  Each row's prefix along the wave's
// half (mf_row_prefix4) goes to row n of V (row stride vs) when `keep`; reads
// are unconditional and every lane takes part in the scans.
// One row of the window sums of a 128-column tile (MW = 2, one column-sum
// wave per field over all the words, so lane l's prefix `pre` covers columns
// 4l .. 4l + 3 from column 0): lane l < 32 stores the sums over columns
// [x, x + tw) for its outputs x = 4l + k, the prefix at x + tw - 1 (lanes
// l + d and l + d + 1, d = (tw - 1) / 4, read across the wave) less the
// prefix at x - 1.  Every lane takes part in the cross-lane reads.
__device__ __forceinline__ void mf_store_windows(const uint4 pre, int tw, uint32_t *row)
{
    const int lane = threadIdx.x & 63;
    const int d = (tw - 1) >> 2, r = (tw - 1) & 3;  // wave-uniform
    const int la = min(lane + d, 63), lb = min(lane + d + 1, 63);
    const uint32_t a[4] = {(uint32_t)__shfl((int)pre.x, la, 64), (uint32_t)__shfl((int)pre.y, la, 64),
                           (uint32_t)__shfl((int)pre.z, la, 64), (uint32_t)__shfl((int)pre.w, la, 64)};
    const uint32_t b[3] = {(uint32_t)__shfl((int)pre.x, lb, 64), (uint32_t)__shfl((int)pre.y, lb, 64),
                           (uint32_t)__shfl((int)pre.z, lb, 64)};
    const uint32_t prev = (uint32_t)__shfl((int)pre.w, max(lane - 1, 0), 64);
    // hi = prefix at columns 4l + k + tw - 1, k = 0..3: components k + r of
    // lane l + d, continuing into lane l + d + 1
    uint4 hi;
    switch (r) {
    case 0: hi = make_uint4(a[0], a[1], a[2], a[3]); break;
    case 1: hi = make_uint4(a[1], a[2], a[3], b[0]); break;
    case 2: hi = make_uint4(a[2], a[3], b[0], b[1]); break;
    default: hi = make_uint4(a[3], b[0], b[1], b[2]); break;
    }
    if (lane < 32)
        *reinterpret_cast<uint4 *>(row + 4 * lane) =
            make_uint4(hi.x - (lane > 0 ? prev : 0u), hi.y - pre.x, hi.z - pre.y, hi.w - pre.z);
}

template <int MW, int NKB, int F, bool WIN>
__device__ __forceinline__ void mf_slide_word(const uint32_t *img, int hcur, bool one_chunk, const uint32_t *head,
                                              int nwd, int wd, bool keep, uint32_t *V, int vs, int tw,
                                              uint32_t (&c)[4])
{
    constexpr int sw = mf_sw(MW, NKB);
    uint32_t in[MF_TY - 1], out[MF_TY - 1];
#pragma unroll
    for (int n = 1; n < MF_TY; ++n) {
        in[n - 1] = img[(hcur + n - 1) * sw + wd];
        // one address, then one read: the head rows exist only when the
        // template came in several chunks
        const uint32_t *src = one_chunk ? img + (n - 1) * sw + wd : head + (n - 1) * nwd + wd;
        out[n - 1] = *src;
    }
    uint4 pre = mf_row_prefix4(c);
    if (WIN)
        mf_store_windows(pre, tw, V);
    else if (keep)
        *reinterpret_cast<uint4 *>(V + 4 * wd) = pre;
#pragma unroll
    for (int n = 1; n < MF_TY; ++n) {
        uint32_t r[4] = {0u, 0u, 0u, 0u};
        mf_col_add<F>(in[n - 1], c);
        mf_col_add<F>(out[n - 1], r);
#pragma unroll
        for (int k = 0; k < 4; ++k)
            c[k] -= r[k];
        pre = mf_row_prefix4(c);
        if (WIN)
            mf_store_windows(pre, tw, V + n * vs);
        else if (keep)
            *reinterpret_cast<uint4 *>(V + n * vs + 4 * wd) = pre;
    }
}

// Column walk, then (after the last chunk only) the sliding pass with the row
// prefix, of field F over words [w0, w0 + cnt) by one column-sum wave.  The
// prefix runs over the wave's own columns [4*w0, 4*(w0 + cnt)), starting from
// zero.
template <int MW, int NKB, int F, bool WIN>
__device__ __forceinline__ void mf_field_chunk(const uint32_t *img, int hcur, int j0, bool last, bool one_chunk,
                                               uint32_t *head, int nwd, int w0, int cnt, uint32_t *V, int vs, int tw,
                                               uint32_t (&c)[4])
{
    const int lane = threadIdx.x & 63;
    const int wd = w0 + min(lane, cnt - 1);
    const bool keep = lane < cnt;
    mf_col_walk<MW, NKB, F>(img, hcur, j0, !one_chunk, head, nwd, wd, keep, c);
    if (last)
        mf_slide_word<MW, NKB, F, WIN>(img, hcur, one_chunk, head, nwd, wd, keep, V, vs, tw, c);
}

// Workgroup roles (wave-uniform): waves 0 .. MW - 1 run the matrix cores, 64
// output columns each; the next ones keep the column sums, one wave per field
// (pixels, squared pixels) and, with MW = 4, half of the tile's outputs (the
// first pixel wave also sums the template), so the vector work of SumI and
// SumISq runs beside the matrix products instead of inside their loop.
// Every wave takes part in the staging and in the epilogue.  With WIN the
// column-sum waves store window sums (and SumI, SumISq themselves); without,
// row prefixes over disjoint halves, each starting from zero, and the
// epilogue adds the first half's row total where a window reaches from the
// first half into the second (with one half, never).
// Wave priorities, measured on 1920x1080 with 64x64 (HIP-event medians of
// one run, us): staging 3, column-sum waves 3 and matrix-core waves 1 during
// the walk, 21.5; column-sum waves 2 or 1 and matrix-core waves 2 or 1,
// 22.9 - 23.8; column-sum waves 0, 24.4.  On a SIMD the vector instructions
// and the matrix products largely take turns (without the column-sum waves'
// work the launch took 18.4 us against 23.4), so every vector instruction in
// the walk lengthens it.
template <int MW, int NKB, bool WIN>
__global__ __launch_bounds__(mf_threads(MW)) __attribute__((amdgpu_waves_per_eu(NKB == 1 ? 4 : 1)))
void ncc_u8_mfma_kernel(NccArgs a)
{
    constexpr int NT = mf_threads(MW), TX = mf_tx(MW), NWK = mf_walkers(MW), ACC = mf_acc_stride(MW);
    extern __shared__ uint4 mf_smem[];
    static_assert(!WIN || NKB <= 2, "a column-sum wave's 64 lanes hold the words of 128 outputs");
    const MfPlan P = mf_plan(MW, a.t_width, a.hc, a.t_height <= a.hc, WIN);
    uint32_t *const V1 = reinterpret_cast<uint32_t *>(mf_smem);
    uint32_t *const V2 = V1 + MF_TY * P.vs;
    uint32_t *const img = V2 + MF_TY * P.vs;
    uint8_t *const tpl = reinterpret_cast<uint8_t *>(img + P.img_words);
    uint32_t *const head = reinterpret_cast<uint32_t *>(tpl + P.trows * P.tsb);
    uint32_t *const tsum = head + P.head_words;
    int32_t *const acc_it = reinterpret_cast<int32_t *>(img);

    const int x0 = blockIdx.x * TX, y0 = blockIdx.y * MF_TY;
    const int tw = a.t_width, th = a.t_height;
    const int twords = (tw + 3) / 4;  // packed words per template row (the last one partial when tw % 4 != 0)
    const uint32_t tm = tail_mask(tw);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bool one_chunk = th <= P.hc;
    const int half = NWK == 4 ? (P.nwd + 1) / 2 : P.nwd;  // words of the first half (<= 64)
    const int ce = 4 * half;                               // first column of the second half

    mf_v4i at[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
        at[t] = mf_v4i{0, 0, 0, 0};
    uint32_t c[4] = {0u, 0u, 0u, 0u};
    uint32_t ts = 0u, tq = 0u;

    const int nchunks16 = 4 * (MW + NKB);  // 16-byte chunks per staged image row
    for (int j0 = 0; j0 < th; j0 += P.hc) {
        const int hcur = min(P.hc, th - j0);
        const bool last = j0 + hcur == th;
        __syncthreads();  // the previous chunk's readers are done
        __builtin_amdgcn_s_setprio(3);  // staging first on a shared CU: it starts this workgroup's chain
        mf_stage_image<NT>(a.image, a.height, a.pitch, y0 + j0, x0, MF_TY - 1 + hcur, nchunks16, img, P.sw);
        mf_stage_template<NT>(a.tmpl, tw, j0, hcur, 64 * NKB, tpl, P.tsb, P.trows);
        __syncthreads();
        if (wave < MW) {
            __builtin_amdgcn_s_setprio(1);
            mf_walk_chunk<MW, NKB>(img, tpl, hcur, wave, at);
            __builtin_amdgcn_s_setprio(0);
        } else {
            // the column-sum waves issue first on their SIMD, so their sums
            // (and, with WIN, their stores) are done when the products are
            __builtin_amdgcn_s_setprio(3);
            const int h = NWK == 4 ? (wave - MW) & 1 : 0;
            const int field = NWK == 4 ? (wave - MW) >> 1 : wave - MW;
            // window sums: each wave takes every word its 128 outputs read
            // (the two halves overlap by the template's width), so its sums
            // need nothing from the other half; prefixes: disjoint halves
            const int w0 = WIN ? 32 * h : h * half;
            const int cnt = WIN ? 32 + (tw + 2) / 4 : h ? P.nwd - half : half;
            uint32_t *const vf = (field == 0 ? V1 : V2) + (WIN ? 128 * h : 0);
            if (field == 0) {
                if (h == 0) {
                    // template sums from the staged (biased) rows of this
                    // chunk; the partial last word of a row (tm != ~0) is
                    // unbiased on its template bytes only, its padding stays zero
                    for (int i = lane; i < hcur * twords; i += 64) {
                        const int r = i / twords;
                        const int k = i - r * twords;
                        const uint32_t unbias =
                            tm == 0xFFFFFFFFu || k != twords - 1 ? 0x80808080u : 0x80808080u & tm;
                        const uint32_t w =
                            *reinterpret_cast<const uint32_t *>(tpl + (MF_TY - 1 + r) * P.tsb + 4 * k) ^ unbias;
                        ts = dot4u(w, 0x01010101u, ts);
                        tq = dot4u(w, w, tq);
                    }
                }
                mf_field_chunk<MW, NKB, 0, WIN>(img, hcur, j0, last, one_chunk, head, P.nwd, w0, cnt, vf, P.vs, tw, c);
            } else {
                mf_field_chunk<MW, NKB, WIN ? 2 : 1, WIN>(img, hcur, j0, last, one_chunk, head, P.nwd, w0, cnt, vf,
                                                         P.vs, tw, c);
            }
            __builtin_amdgcn_s_setprio(0);
        }
    }
    const uint32_t nn = (uint32_t)(tw * th);
    if (WIN && wave >= MW) {
        // Window sums are final as soon as a column-sum wave has its rows:
        // it stores its 128 outputs of each row now (one per lane, from the
        // rows it wrote to V), SumI = sum s + 128 N or SumISq = sum I^2,
        // while the matrix-core waves still walk.
        const int h = NWK == 4 ? (wave - MW) & 1 : 0;
        const int field = NWK == 4 ? (wave - MW) >> 1 : wave - MW;
        uint32_t *const out = field == 0 ? a.sum_i : a.sum_isq;
        const int xh = x0 + 128 * h;
        if (out && xh < a.out_w) {
            const uint32_t *const vf = (field == 0 ? V1 : V2) + 128 * h;
            const uint32_t add = field == 0 ? 128u * nn : 0u;
            uint32_t *const ob = out + ((size_t)y0 * a.out_w + xh);  // 32-bit offsets from here
            // every LDS read first (one wait, not one per row), then the stores
            uint32_t v[MF_TY][2];
#pragma unroll
            for (int n = 0; n < MF_TY; ++n)
#pragma unroll
                for (int k = 0; k < 2; ++k)
                    v[n][k] = vf[n * P.vs + 64 * k + lane] + add;
            const int nrows = min(MF_TY, a.out_h - y0);
#pragma unroll
            for (int n = 0; n < MF_TY; ++n)
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    const int col = 64 * k + lane;
                    if (n < nrows && xh + col < a.out_w)
                        ob[(uint32_t)n * (uint32_t)a.out_w + (uint32_t)col] = v[n][k];
                }
        }
    }
    if (wave == MW) {
        ts = wave_sum_u32(ts);
        tq = wave_sum_u32(tq);
        if (lane == 0) {
            tsum[0] = ts;
            tsum[1] = tq;
        }
    }
    __syncthreads();  // every reader of the image tile is done; V, tsum written

    // SumIT' to LDS (over the image tile): lane (g, n) holds columns
    // 64*wave + 16g + 4i + t of row n.
    if (wave < MW) {
        const int n = lane & 15, g = lane >> 4;
        const int base = n * ACC + 64 * wave + 16 * g;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int t = 0; t < 4; ++t)
                acc_it[base + 4 * i + t] = at[t][i];
    }
    __syncthreads();

    const uint32_t sum_t = tsum[0], sum_tsq = tsum[1];
    const uint32_t bias = 128u * sum_t - 16384u * nn;
    // num, vI, vT are integers below 2^50 (N <= 66,051 and every sum below
    // 2^32), so fp64 fused multiply-adds form them exactly: the same doubles,
    // hence the same coefficient, as the 64-bit integer form.
    const double nd = (double)nn, std_ = (double)sum_t;
    const double vt = fma(nd, (double)sum_tsq, -(std_ * std_));

    // Each wave takes 64 consecutive columns of one output row at a time (one
    // column per lane: whole cache lines per store, no LDS bank conflicts).
    // NT is a multiple of TX, so a thread keeps its column and its terms
    // (the prefix entries it reads, whether its window needs the first
    // half's row total) while its rows advance by NT / TX.  A window needs
    // that total when it starts in the first half and ends in the second,
    // i.e. when x lies in [ce - tw + 1, ce].  Outputs are addressed from the
    // tile's first one with 32-bit offsets (n * out_w + x < 2^32).
    constexpr int RS = NT / TX;  // rows per pass
    static_assert(NT % TX == 0, "a thread keeps one column");
    const int x = threadIdx.x % TX, gx = x0 + x;
    const int hi = x + tw - 1, xl = x > 0 ? x - 1 : 0;
    const uint32_t left_keep = x > 0 ? 0xFFFFFFFFu : 0u;
    const uint32_t join_keep = (uint32_t)(x - (ce - tw + 1)) <= (uint32_t)(tw - 1) ? 0xFFFFFFFFu : 0u;
    const size_t o0 = (size_t)y0 * a.out_w + x0;
    uint32_t *const out_i = a.sum_i ? a.sum_i + o0 : nullptr;
    uint32_t *const out_isq = a.sum_isq ? a.sum_isq + o0 : nullptr;
    uint32_t *const out_it = a.sum_it ? a.sum_it + o0 : nullptr;
    float *const out_c = a.coef ? a.coef + o0 : nullptr;
    unsigned long long best = 0ull;
    if (gx < a.out_w) {
        for (int n = threadIdx.x / TX; n < MF_TY && y0 + n < a.out_h; n += RS) {
            const uint32_t off = (uint32_t)n * (uint32_t)a.out_w + (uint32_t)x;
            const uint32_t *q1 = V1 + n * P.vs;
            const uint32_t *q2 = V2 + n * P.vs;
            uint32_t si, sq;
            if (WIN) {
                // the column-sum waves stored the window sums themselves (of
                // s and of I^2), and SumI and SumISq already
                si = q1[x] + 128u * nn;
                sq = q2[x];
            } else {
                // window sums as differences of the row prefix (of s = I -
                // 128 and of s^2) at columns hi and x - 1; the entry left of
                // column 0 is read from column 0 and masked to zero
                si = q1[hi] - (q1[xl] & left_keep) + (q1[ce - 1] & join_keep) + 128u * nn;
                sq = q2[hi] - (q2[xl] & left_keep) + (q2[ce - 1] & join_keep) + 256u * si - 16384u * nn;
            }
            const uint32_t st = (uint32_t)acc_it[n * ACC + x] + 128u * si + bias;
            if (!WIN && out_i) out_i[off] = si;
            if (!WIN && out_isq) out_isq[off] = sq;
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

// Template rows per chunk: the most (up to MF_MAX_HC) whose plan fits `budget`
// bytes of LDS, 0 if none does.
static int mf_fit_hc(const NccArgs &a, size_t budget, int mw, bool win)
{
    int hc = a.t_height < MF_MAX_HC ? a.t_height : MF_MAX_HC;
    while (hc > 1 && mf_plan(mw, a.t_width, hc, hc >= a.t_height, win).bytes > budget)
        --hc;
    return mf_plan(mw, a.t_width, hc, hc >= a.t_height, win).bytes <= budget ? hc : 0;
}

// 256-column tiles: the most rows that fit two workgroups per CU (80 KiB
// each); when that leaves fewer than 32 rows (wide template rows), the most
// that fit one workgroup per CU.
static int mf_pick_hc4(const NccArgs &a, bool win)
{
    const int hc = mf_fit_hc(a, 80 * 1024, 4, win);
    if (hc >= 32 || hc == a.t_height)
        return hc;
    return mf_fit_hc(a, 160 * 1024, 4, win);
}

// Whether 256-column tiles take window sums (stored during the walk) rather
// than row prefixes: only where the walk is long enough to hide the
// column-sum waves' extra work and stores, templates of at least 48 rows
// (and at most two 64-byte blocks), and not where the prefixes need fewer
// row chunks.  A/B on 1920x1080, prefixes / window sums (us): 64x64 25.8 /
// 23.6, 16 wide x 64 tall 25.0 / 22.8, 32x64 25.6 / 23.3, 96x96 58.6 /
// 52.6 (three chunks / two), 48x48 29.4 / 29.6; but 40x40 28.6 / 29.7,
// 32x32 27.4 / 28.5, 64 wide x 16 tall 24.2 / 26.8, 8x8 22.9 / 25.6, and
// 128x128 58.8 / 70.9 (one chunk at one workgroup per CU / three).
static bool mf_win4(const NccArgs &a)
{
    if ((a.t_width + 63) / 64 > 2 || a.t_height < 48)
        return false;
    const int hw = mf_pick_hc4(a, true), hp = mf_pick_hc4(a, false);
    if (hw == 0 || hp == 0)
        return hw > 0;
    return (a.t_height + hw - 1) / hw <= (a.t_height + hp - 1) / hp;
}

// 128-column tiles: four 4-wave workgroups per CU (one wave per SIMD each),
// so a quarter of the LDS.  The column-sum waves store row prefixes when the
// template then fits one row chunk (the cheaper form for them), else window
// sums when those let it fit one, else prefixes in chunks of at least
// min(t_height, 16) rows.
constexpr size_t MF2_LDS = 160 * 1024 / 4;
struct Mf2Pick {
    int hc;
    bool win;
};
static Mf2Pick mf_pick2(const NccArgs &a)
{
    if ((a.t_width + 63) / 64 != 1)
        return {0, false};
    const int hp = mf_fit_hc(a, MF2_LDS, 2, false);
    if (hp >= a.t_height)
        return {hp, false};
    if (mf_fit_hc(a, MF2_LDS, 2, true) >= a.t_height)
        return {a.t_height, true};
    return {hp >= (a.t_height < 16 ? a.t_height : 16) ? hp : 0, false};
}

bool ncc_mfma_supported(const NccArgs &a, int mw)
{
    if (mw == 2)
        return mf_pick2(a).hc > 0;
    return (a.t_width + 63) / 64 <= MF_MAX_NKB && mf_pick_hc4(a, mf_win4(a)) > 0;
}

template <int MW, int NKB, bool WIN>
static hipError_t mf_launch(NccArgs a, hipStream_t s)
{
    // dynamic LDS above 64 KiB must be allowed explicitly
    static std::atomic<uint64_t> lds_allowed{0};
    const hipError_t e = allow_lds_once(&ncc_u8_mfma_kernel<MW, NKB, WIN>, lds_allowed);
    if (e != hipSuccess)
        return e;
    const size_t lds = mf_plan(MW, a.t_width, a.hc, a.hc >= a.t_height, WIN).bytes;
    const dim3 grid((a.out_w + mf_tx(MW) - 1) / mf_tx(MW), (a.out_h + MF_TY - 1) / MF_TY);
    hipLaunchKernelGGL((ncc_u8_mfma_kernel<MW, NKB, WIN>), grid, dim3(mf_threads(MW)), lds, s, a);
    return hipGetLastError();
}

hipError_t ncc_launch_mfma(NccArgs a, hipStream_t s, int mw)
{
    const Mf2Pick p2 = mf_pick2(a);
    if (mw == 0 && p2.hc >= a.t_height) {
        // Two 8-wave workgroups of 256-column tiles fit per CU, four 4-wave
        // ones of 128-column tiles: a grid a little over 2 wide tiles per CU
        // runs a second round of them at nearly full cost (a workgroup's
        // time is mostly its own chain of staging, walk and epilogue), where
        // the narrow tiles may all fit at once.  Take the narrow tiles (with
        // the template in one row chunk) when they need fewer rounds, or
        // when the wide ones would leave CUs idle (800x600 with 16x16: 11.2
        // us wide, 9.7 narrow; 1280x720 and 1024x768 with 16x16 within 2 %);
        // on a full grid at equal rounds the wide ones are faster.
        const int64_t cus = device_cu_count();
        const int64_t ty = (a.out_h + MF_TY - 1) / MF_TY;
        const int64_t t4 = (a.out_w + mf_tx(4) - 1) / mf_tx(4) * ty, t2 = (a.out_w + mf_tx(2) - 1) / mf_tx(2) * ty;
        const int64_t r4 = (t4 + 2 * cus - 1) / (2 * cus), r2 = (t2 + 4 * cus - 1) / (4 * cus);
        mw = r2 < r4 || t4 < cus ? 2 : 4;
    }
    if (mw == 2) {
        a.hc = p2.hc;
        return p2.win ? mf_launch<2, 1, true>(a, s) : mf_launch<2, 1, false>(a, s);
    }
    const bool win = mf_win4(a);
    a.hc = mf_pick_hc4(a, win);
    switch ((a.t_width + 63) / 64) {
    case 1: return win ? mf_launch<4, 1, true>(a, s) : mf_launch<4, 1, false>(a, s);
    case 2: return win ? mf_launch<4, 2, true>(a, s) : mf_launch<4, 2, false>(a, s);
    case 3: return mf_launch<4, 3, false>(a, s);
    default: return mf_launch<4, 4, false>(a, s);
    }
}

} // namespace xc
