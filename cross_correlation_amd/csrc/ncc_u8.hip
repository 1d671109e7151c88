// ncc_u8.hip -- gfx950 kernels for valid-mode 8-bit normalized correlation.
//
// What is computed ("The CUDA Handbook", ch. 15 "Image Processing: Normalized
// Correlation", section 15.5 "Instruction-Level Parallelism and DP4A"): for
// every window the unsigned sums SumI, SumISq and SumIT over the window's
// bytes, then Pearson's coefficient from them and the template sums.
//
// How it maps to CDNA4 (prior art on the page: DP4A over packed bytes, two
// independent output columns per thread, a funnel shift to line the image
// bytes up with the template bytes; kept, and re-shaped for wave64):
//   * v_dot4_u32_u8 (__builtin_amdgcn_udot4) replaces DP4A: one instruction
//     multiplies four unsigned byte lanes pairwise and adds them to a u32.
//     Three per packed word and output: against 0x01010101 (SumI), against
//     itself (SumISq) and against the template word (SumIT).
//   * v_alignbyte_b32 replaces the funnel shift: output column x reads bytes
//     x+4i .. x+4i+3, taken from the two aligned LDS words straddling them.
//     Lane b of a packed word is pixel offset b (little-endian) in both the
//     image word and the template word, so SumIT pairs matching pixels.
//   * Each lane owns 4 adjacent columns (one aligned word group: shift 0 is
//     free, shifts 1..3 cost one alignbyte each) and Q output rows.  The loop
//     walks image rows: every image word loaded from LDS and its three shifts
//     serve all Q rows the lane owns (template row j = image row - output
//     row), so the shifts are amortised over 12*Q dot4 per word.  The 3*4*Q
//     accumulator chains are independent, which supplies the ILP the page
//     found essential.
//   * The template row for each (image row, output row) pair is wave-uniform:
//     it is staged in LDS beside the image tile and read at a wave-uniform
//     address (a broadcast read, no bank conflicts).
//   * Tall templates split their rows over two waves that share a tile
//     (KS = 2); their partial sums meet in LDS before the epilogue, which
//     doubles the waves per SIMD without a second copy of the tile.
//   * Image tiles are staged into LDS with 16-byte loads (the page's uint4
//     versus int finding: wide coalesced copies into on-chip memory).
//   * The epilogue forms num, vI, vT exactly in 64-bit integers; the
//     coefficient (ncc_coef_f32) is the fp32 rounding of the IEEE fp64
//     quotient num / sqrt(vI * vT), bit for bit.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"
#include "ncc_common.h"
#include "xcorr.h"

namespace xc {

// One image row of one template chunk: for each template word k of the chunk
// load the next aligned image word, form the three shifted words, and for each
// output row q the row serves accumulate 3 x 4 dot4 with template row (rl - q).
// Image words and template words (at a wave-uniform address) both come from
// LDS; WC words per unrolled step.  When the chunk ends with the last word of
// a template row whose width is not a multiple of 4 (tmask != ~0), that word
// goes last, its shifted image words masked to the template's bytes (the
// template word is zero beyond them), so every sum counts exactly the
// template's pixels.
template <int Q>
__device__ __forceinline__ void ncc_word(uint32_t w1, uint32_t w0, uint32_t mask, const uint32_t *t0, int k,
                                         int tstride, int qlo, int qhi, bool full, uint32_t (&ai)[Q][4],
                                         uint32_t (&aq)[Q][4], uint32_t (&at)[Q][4])
{
    uint32_t s[4];
    s[0] = w0 & mask;
    s[1] = shift_bytes(w1, w0, 1) & mask;
    s[2] = shift_bytes(w1, w0, 2) & mask;
    s[3] = shift_bytes(w1, w0, 3) & mask;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        if (full || (q >= qlo && q <= qhi)) {
            const uint32_t t = t0[k - q * tstride];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                ai[q][c] = dot4u(s[c], 0x01010101u, ai[q][c]);
                aq[q][c] = dot4u(s[c], s[c], aq[q][c]);
                at[q][c] = dot4u(s[c], t, at[q][c]);
            }
        }
    }
}

template <int Q, int WC, bool FULL>
__device__ __forceinline__ void ncc_row(const uint32_t *rp, const uint32_t *t0, int tstride, int cw_main,
                                        uint32_t tmask, int qlo, int qhi, uint32_t (&ai)[Q][4],
                                        uint32_t (&aq)[Q][4], uint32_t (&at)[Q][4])
{
    uint32_t w0 = rp[0];
    for (int kb = 0; kb < cw_main; kb += WC) {
#pragma unroll
        for (int kk = 0; kk < WC; ++kk) {
            const int k = kb + kk;
            const uint32_t w1 = rp[k + 1];
            ncc_word<Q>(w1, w0, 0xFFFFFFFFu, t0, k, tstride, qlo, qhi, FULL, ai, aq, at);
            w0 = w1;
        }
    }
    if (tmask != 0xFFFFFFFFu)
        ncc_word<Q>(rp[cw_main + 1], w0, tmask, t0, cw_main, tstride, qlo, qhi, FULL, ai, aq, at);
}

// A row at the start or end of a template slice serves only output rows
// q in [qlo, qhi].  The (wave-uniform) test is taken once per q, outside the
// word loop; the row's words are re-read per q (only 2*(Q-1) rows per slice).
template <int Q>
__device__ __forceinline__ void ncc_row_partial(const uint32_t *rp, const uint32_t *t0, int tstride, int cw_main,
                                                uint32_t tmask, int qlo, int qhi, uint32_t (&ai)[Q][4],
                                                uint32_t (&aq)[Q][4], uint32_t (&at)[Q][4])
{
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        if (q < qlo || q > qhi)
            continue;
        const uint32_t *tq = t0 - q * tstride;
        uint32_t w0 = rp[0];
        for (int k = 0; k < cw_main; ++k) {
            const uint32_t w1 = rp[k + 1];
            const uint32_t t = tq[k];
            uint32_t s[4];
            s[0] = w0;
            s[1] = shift_bytes(w1, w0, 1);
            s[2] = shift_bytes(w1, w0, 2);
            s[3] = shift_bytes(w1, w0, 3);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                ai[q][c] = dot4u(s[c], 0x01010101u, ai[q][c]);
                aq[q][c] = dot4u(s[c], s[c], aq[q][c]);
                at[q][c] = dot4u(s[c], t, at[q][c]);
            }
            w0 = w1;
        }
        if (tmask != 0xFFFFFFFFu) {
            // the row's partial last word: only the template's bytes count
            const uint32_t w1 = rp[cw_main + 1];
            const uint32_t t = tq[cw_main];
            uint32_t s[4];
            s[0] = w0 & tmask;
            s[1] = shift_bytes(w1, w0, 1) & tmask;
            s[2] = shift_bytes(w1, w0, 2) & tmask;
            s[3] = shift_bytes(w1, w0, 3) & tmask;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                ai[q][c] = dot4u(s[c], 0x01010101u, ai[q][c]);
                aq[q][c] = dot4u(s[c], s[c], aq[q][c]);
                at[q][c] = dot4u(s[c], t, at[q][c]);
            }
        }
    }
}

// Main kernel: a workgroup covers 256 output columns x WV*Q rows with
// WV*KS waves.  Wave (rw, kh) owns output rows [rw*Q, rw*Q + Q) of the tile
// and the kh-th of KS slices of the template rows; lane l owns columns
// 4l..4l+3.  Splitting the template rows over KS waves multiplies the waves
// in flight per SIMD (the dot4 issue rate needs several) without shrinking
// the Q*4 outputs a lane's shifted words are shared by.  The KS partial sums
// are added through LDS before the epilogue.
// LDS: the image tile (WV*Q + hc - 1 rows of `lds_stride` words), then the
// template chunk (hc rows of `t_stride` words).
template <int Q, int WV, int KS, int WC, bool TAIL>
__global__ __launch_bounds__(64 * WV * KS) void ncc_u8_ilp_kernel(NccArgs a)
{
    extern __shared__ uint32_t lds[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rw = wave % WV;  // output-row group of this wave
    const int kh = wave / WV;  // template-row slice of this wave
    // Without TAIL, a 2D grid of 256 x WV*Q tiles.  With TAIL, a 1D grid:
    // workgroups [0, ncol_full * nrow_tiles) are those tiles (column tile
    // fastest), the rest tail tiles over the last column tile's remainder (at
    // most 256 / tail_g columns): lane l is column lane l % tail_nl of group
    // l / tail_nl, and the tail_g groups take tail_g consecutive bands of
    // WV*Q rows, so the lanes past the remainder's width do useful work
    // instead of idling (lanes of a last, incomplete group repeat group 0's
    // work and store nothing).
    int bx = blockIdx.x, by = blockIdx.y, G = 1, g = 0, cl = lane;
    bool active = true;
    if (TAIL) {
        const int bid = blockIdx.x;
        const int nfull = a.ncol_full * a.nrow_tiles;
        const bool tail = bid >= nfull;  // workgroup-uniform
        by = tail ? bid - nfull : bid / a.ncol_full;
        bx = tail ? a.ncol_full : bid - by * a.ncol_full;
        G = tail ? a.tail_g : 1;
        g = tail ? (int)(((uint32_t)lane * a.tail_m) >> 16) : 0;  // lane / tail_nl
        cl = tail ? lane - g * a.tail_nl : lane;                   // < tail_nl in a tail tile
        active = g < G;
        if (!active)
            g = 0;
    }
    const int x0 = bx * 256;
    const int y0 = by * (WV * Q * G);
    const int nw = (a.t_width + 3) >> 2;  // packed words per template row
    const uint32_t tm = tail_mask(a.t_width);
    const bool word_rows = tmpl_word_rows(a.tmpl, a.t_width);

    uint32_t sum_t, sum_tsq;
    template_sums(a.tmpl, a.t_width, a.t_height, sum_t, sum_tsq);

    uint32_t ai[Q][4], aq[Q][4], at[Q][4];
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
        for (int c = 0; c < 4; ++c)
            ai[q][c] = aq[q][c] = at[q][c] = 0u;

    const int stride = a.lds_stride;
    const int tstride = a.t_stride;
    const int th = WV * Q * G;  // output rows of this tile
    uint32_t *const tl = lds + (th + a.hc - 1) * stride;
    for (int jc = 0; jc < a.t_height; jc += a.hc) {
        const int hc = min(a.hc, a.t_height - jc);
        // this wave's template rows of the chunk: [j0, j1)
        const int j0 = hc * kh / KS;
        const int j1 = hc * (kh + 1) / KS;
        for (int ic = 0; ic < nw; ic += a.cw) {
            const int cw = min(a.cw, nw - ic);
            __syncthreads();
            // lane l reads words l + k and l + k + 1, k < cw: 64 + cw words per row
            stage_tile(a.image, a.height, a.pitch, y0 + jc, x0 + 4 * ic, th + hc - 1,
                       (64 + cw + 3) / 4, lds, stride);
            for (int t = threadIdx.x; t < hc * cw; t += 64 * WV * KS) {
                const int r = t / cw;
                const int c = t - r * cw;
                tl[r * tstride + c] = tmpl_word(a.tmpl, a.t_width, word_rows, jc + r, ic + c);
            }
            __syncthreads();
            // the chunk holding a row's last word ends with the masked tail word
            const uint32_t cm = ic + cw == nw ? tm : 0xFFFFFFFFu;
            const int cw_main = cw - (cm != 0xFFFFFFFFu ? 1 : 0);
            if (j1 > j0) {
                const uint32_t *wrow = lds + (g * (WV * Q) + rw * Q) * stride + cl;
                // Image rows rl (relative to the wave's first output row) meet
                // template rows j = rl - q with j in [j0, j1).  Three straight
                // loops -- ramp-up, steady (every q), ramp-down -- so the
                // accumulators never meet a branch merge inside the row loop.
                const int steady0 = j0 + Q - 1;
                for (int rl = j0; rl < min(steady0, j1 + Q - 1); ++rl)
                    ncc_row_partial<Q>(wrow + rl * stride, tl + rl * tstride, tstride, cw_main, cm,
                                       max(0, rl - j1 + 1), min(Q - 1, rl - j0), ai, aq, at);
                for (int rl = steady0; rl < j1; ++rl)
                    ncc_row<Q, WC, true>(wrow + rl * stride, tl + rl * tstride, tstride, cw_main, cm, 0, Q - 1, ai,
                                         aq, at);
                for (int rl = max(j1, steady0); rl < j1 + Q - 1; ++rl)
                    ncc_row_partial<Q>(wrow + rl * stride, tl + rl * tstride, tstride, cw_main, cm,
                                       max(0, rl - j1 + 1), min(Q - 1, rl - j0), ai, aq, at);
            }
        }
    }

    if (KS > 1) {
        // add the slices: waves kh > 0 leave their sums in LDS for wave kh = 0
        __syncthreads();
        constexpr int NACC = 3 * 4 * Q;
        uint32_t *xbuf = lds + (size_t)rw * (KS - 1) * NACC * 64;
        if (kh > 0) {
            uint32_t *mine = xbuf + (size_t)(kh - 1) * NACC * 64 + lane;
#pragma unroll
            for (int q = 0; q < Q; ++q)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    mine[((q * 4 + c) * 3 + 0) * 64] = ai[q][c];
                    mine[((q * 4 + c) * 3 + 1) * 64] = aq[q][c];
                    mine[((q * 4 + c) * 3 + 2) * 64] = at[q][c];
                }
        }
        __syncthreads();
        if (kh > 0)
            return;
        for (int o = 0; o < KS - 1; ++o) {
            const uint32_t *other = xbuf + (size_t)o * NACC * 64 + lane;
#pragma unroll
            for (int q = 0; q < Q; ++q)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    ai[q][c] += other[((q * 4 + c) * 3 + 0) * 64];
                    aq[q][c] += other[((q * 4 + c) * 3 + 1) * 64];
                    at[q][c] += other[((q * 4 + c) * 3 + 2) * 64];
                }
        }
    }

    const int64_t n = (int64_t)a.t_width * a.t_height;
    const int64_t st64 = sum_t;
    const int64_t vt = n * (int64_t)sum_tsq - st64 * st64;
    unsigned long long best = 0ull;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int y = y0 + g * (WV * Q) + rw * Q + q;
        if (y >= a.out_h || !active)
            break;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int x = x0 + 4 * cl + c;
            if (x < a.out_w)
                ncc_store(a, (size_t)y * a.out_w + x, ai[q][c], aq[q][c], at[q][c], n, st64, vt, best);
        }
    }
    if (a.peak)
        peak_commit(a.peak, best);
}

// Ablation kernels: one output per thread, a 64 x 4 tile per workgroup, the
// image tile in LDS.  DOT4 selects packed-byte dot products; otherwise the
// bytes are multiplied and added one at a time.  Each thread runs one
// dependent chain per sum, as the page's baseline kernels do.  With KS > 1
// (small grids only, the launcher's choice) KS waves share each output row,
// each taking a slice of every template chunk's rows; the slices' partial
// sums are added through LDS before the epilogue.
template <bool DOT4, bool WORD_ROWS, int KS>
__global__ __launch_bounds__(256 * KS) void ncc_u8_c1_kernel(NccArgs a)
{
    extern __shared__ uint32_t lds[];
    const int tx = threadIdx.x & 63;
    const int ty = (threadIdx.x >> 6) & 3;  // output row of the tile
    // template-row slice of this wave, wave-uniform (a scalar loop below;
    // as a lane value it made the row loop a masked vector loop, 23 % slower
    // on 1920x1080 with 64x64)
    const int ks = KS == 1 ? 0 : __builtin_amdgcn_readfirstlane(threadIdx.x >> 8);
    const int x0 = blockIdx.x * 64;
    const int y0 = blockIdx.y * 4;
    const int nw = (a.t_width + 3) >> 2;  // packed words per template row
    const uint32_t tm = tail_mask(a.t_width);

    uint32_t sum_t, sum_tsq;
    template_sums(a.tmpl, a.t_width, a.t_height, sum_t, sum_tsq);

    uint32_t si = 0, sq = 0, st = 0;
    const int stride = a.lds_stride;
    const uint32_t sh = (uint32_t)(tx & 3);
    for (int jc = 0; jc < a.t_height; jc += a.hc) {
        const int hc = min(a.hc, a.t_height - jc);
        for (int ic = 0; ic < nw; ic += a.cw) {
            const int cw = min(a.cw, nw - ic);
            __syncthreads();
            // thread tx reads words tx/4 + k and tx/4 + k + 1, k < cw: 16 + cw words per row
            stage_tile(a.image, a.height, a.pitch, y0 + jc, x0 + 4 * ic, 4 + hc - 1, (16 + cw + 3) / 4,
                       lds, stride);
            if (!WORD_ROWS) {
                // rows that are not whole words: gather the chunk's template
                // words once into LDS, after the image tile
                uint32_t *tl = lds + (4 + a.hc - 1) * stride;
                for (int t = threadIdx.x; t < hc * cw; t += blockDim.x) {
                    const int r = t / cw;
                    const int c = t - r * cw;
                    tl[r * a.t_stride + c] = tmpl_word(a.tmpl, a.t_width, false, jc + r, ic + c);
                }
            }
            __syncthreads();
            for (int j = hc * ks / KS; j < hc * (ks + 1) / KS; ++j) {
                const uint32_t *rp = lds + (ty + j) * stride + (tx >> 2);
                const uint8_t *trow = a.tmpl + (size_t)(jc + j) * a.t_width;
                auto mac = [&](uint32_t i4, uint32_t t4) {
                    if (DOT4) {
                        si = dot4u(i4, 0x01010101u, si);
                        sq = dot4u(i4, i4, sq);
                        st = dot4u(i4, t4, st);
                    } else {
#pragma unroll
                        for (int b = 0; b < 4; ++b) {
                            const uint32_t p = (i4 >> (8 * b)) & 0xFFu;
                            const uint32_t t = (t4 >> (8 * b)) & 0xFFu;
                            si += p;
                            sq += p * p;
                            st += p * t;
                        }
                    }
                };
                if (WORD_ROWS) {
                    // whole-word rows: the (wave-uniform) template words load directly
                    const uint32_t *tw = reinterpret_cast<const uint32_t *>(trow) + ic;
                    for (int k = 0; k < cw; ++k)
                        mac(shift_bytes(rp[k + 1], rp[k], sh), tw[k]);
                } else {
                    // the staged words (wave-uniform LDS reads), the row's
                    // partial last word with its image bytes masked
                    const uint32_t *tw = lds + (4 + a.hc - 1) * stride + j * a.t_stride;
                    const int cw_main = cw - (ic + cw == nw && tm != 0xFFFFFFFFu ? 1 : 0);
                    for (int k = 0; k < cw_main; ++k)
                        mac(shift_bytes(rp[k + 1], rp[k], sh), tw[k]);
                    if (cw_main < cw)
                        mac(shift_bytes(rp[cw_main + 1], rp[cw_main], sh) & tm, tw[cw_main]);
                }
            }
        }
    }
    if (KS > 1) {
        // the slices' partial sums, added through LDS by the first slice's waves
        __syncthreads();
        uint32_t *xb = lds + (size_t)(threadIdx.x & 255);
        if (ks > 0) {
            xb[((ks - 1) * 3 + 0) * 256] = si;
            xb[((ks - 1) * 3 + 1) * 256] = sq;
            xb[((ks - 1) * 3 + 2) * 256] = st;
        }
        __syncthreads();
        if (ks > 0)
            return;
#pragma unroll
        for (int o = 0; o < KS - 1; ++o) {
            si += xb[(o * 3 + 0) * 256];
            sq += xb[(o * 3 + 1) * 256];
            st += xb[(o * 3 + 2) * 256];
        }
    }
    const int y = y0 + ty;
    const int x = x0 + tx;
    unsigned long long best = 0ull;
    if (y < a.out_h && x < a.out_w) {
        const int64_t n = (int64_t)a.t_width * a.t_height;
        const int64_t st64 = sum_t;
        ncc_store(a, (size_t)y * a.out_w + x, si, sq, st, n, st64, n * (int64_t)sum_tsq - st64 * st64, best);
    }
    if (a.peak)
        peak_commit(a.peak, best);
}

// Ablation series of the page's ILP step: C adjacent output columns per lane
// and one output row, on a fixed tile of 256 x 4 outputs per workgroup
// (256 / C lanes per output row, 1024 / C threads), so that across
// C = 1, 2, 4, 8 only the number of independent accumulator chains per lane
// (3 * C) and the byte shifts a loaded image word is shared by change; the
// tile, the staging and the template reads stay the same.  Lane tx owns
// columns C*tx .. C*tx + C - 1 of the tile: they start in image word
// (C*tx) / 4 at byte (C*tx) % 4, so C = 1 takes a per-lane shift of 0..3,
// C = 2 the page's two columns (shifts s and s + 1, s = 0 or 2 from the
// lane's column parity), C = 4 one aligned word group (shifts 0..3, the first
// free) and C = 8 two word groups (three words per step).  Template words are
// staged in LDS and read at a workgroup-uniform address (a broadcast).
template <int C>
__device__ __forceinline__ void ncc_cols_word(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t sh, uint32_t t,
                                              uint32_t mask, uint32_t (&ai)[C], uint32_t (&aq)[C],
                                              uint32_t (&at)[C])
{
    uint32_t v[C];
    if (C == 1) {
        v[0] = shift_bytes(w1, w0, sh);
    } else if (C == 2) {
        v[0] = shift_bytes(w1, w0, sh);
        v[1 % C] = shift_bytes(w1, w0, sh + 1);
    } else {
#pragma unroll
        for (int g = 0; g < C / 4; ++g) {
            const uint32_t lo = g == 0 ? w0 : w1, hi = g == 0 ? w1 : w2;
            v[(4 * g) % C] = lo;
            v[(4 * g + 1) % C] = shift_bytes(hi, lo, 1);
            v[(4 * g + 2) % C] = shift_bytes(hi, lo, 2);
            v[(4 * g + 3) % C] = shift_bytes(hi, lo, 3);
        }
    }
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const uint32_t x = v[c] & mask;
        ai[c] = dot4u(x, 0x01010101u, ai[c]);
        aq[c] = dot4u(x, x, aq[c]);
        at[c] = dot4u(x, t, at[c]);
    }
}

template <int C>
__global__ __launch_bounds__(1024 / C) void ncc_u8_cols_kernel(NccArgs a)
{
    static_assert(C == 1 || C == 2 || C == 4 || C == 8, "columns per lane");
    constexpr int TX = 256 / C;  // lanes per output row of the tile
    extern __shared__ uint32_t lds[];
    const int tx = threadIdx.x % TX;
    const int ty = threadIdx.x / TX;
    const int x0 = blockIdx.x * 256;
    const int y0 = blockIdx.y * 4;
    const int nw = (a.t_width + 3) >> 2;  // packed words per template row
    const uint32_t tm = tail_mask(a.t_width);
    const bool word_rows = tmpl_word_rows(a.tmpl, a.t_width);

    uint32_t sum_t, sum_tsq;
    template_sums(a.tmpl, a.t_width, a.t_height, sum_t, sum_tsq);

    uint32_t ai[C], aq[C], at[C];
#pragma unroll
    for (int c = 0; c < C; ++c) ai[c] = aq[c] = at[c] = 0u;
    const int wbase = (C * tx) >> 2;
    const uint32_t sh = (uint32_t)((C * tx) & 3);
    const int stride = a.lds_stride;
    const int tstride = a.t_stride;
    uint32_t *const tl = lds + (4 + a.hc - 1) * stride;
    for (int jc = 0; jc < a.t_height; jc += a.hc) {
        const int hc = min(a.hc, a.t_height - jc);
        for (int ic = 0; ic < nw; ic += a.cw) {
            const int cw = min(a.cw, nw - ic);
            __syncthreads();
            // the last lane reads words up to 63 + cw: 64 + cw words per row
            stage_tile(a.image, a.height, a.pitch, y0 + jc, x0 + 4 * ic, 4 + hc - 1, (64 + cw + 3) / 4, lds,
                       stride);
            for (int t = threadIdx.x; t < hc * cw; t += 1024 / C) {
                const int r = t / cw;
                const int c = t - r * cw;
                tl[r * tstride + c] = tmpl_word(a.tmpl, a.t_width, word_rows, jc + r, ic + c);
            }
            __syncthreads();
            const uint32_t cm = ic + cw == nw ? tm : 0xFFFFFFFFu;
            const int cw_main = cw - (cm != 0xFFFFFFFFu ? 1 : 0);
            for (int j = 0; j < hc; ++j) {
                const uint32_t *rp = lds + (ty + j) * stride + wbase;
                const uint32_t *tw = tl + j * tstride;
                uint32_t w0 = rp[0], w1 = rp[1], w2 = C == 8 ? rp[2] : 0u;
                for (int k = 0; k < cw_main; ++k) {
                    const uint32_t t = tw[k];
                    uint32_t nx;
                    if (C == 8) nx = rp[k + 3];
                    else nx = rp[k + 2];
                    ncc_cols_word<C>(w0, w1, w2, sh, t, 0xFFFFFFFFu, ai, aq, at);
                    w0 = w1;
                    if (C == 8) {
                        w1 = w2;
                        w2 = nx;
                    } else {
                        w1 = nx;
                    }
                }
                if (cm != 0xFFFFFFFFu)
                    ncc_cols_word<C>(w0, w1, w2, sh, tw[cw_main], cm, ai, aq, at);
            }
        }
    }
    const int y = y0 + ty;
    const int64_t n = (int64_t)a.t_width * a.t_height;
    const int64_t st64 = sum_t;
    const int64_t vt = n * (int64_t)sum_tsq - st64 * st64;
    unsigned long long best = 0ull;
    if (y < a.out_h) {
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int x = x0 + C * tx + c;
            if (x < a.out_w)
                ncc_store(a, (size_t)y * a.out_w + x, ai[c], aq[c], at[c], n, st64, vt, best);
        }
    }
    if (a.peak)
        peak_commit(a.peak, best);
}

// Best match: clear the key before the correlation launch, decode it after.
__global__ void ncc_peak_init_kernel(xc_ncc_peak *p)
{
    p->key = 0ull;
    p->y = -1;
    p->x = -1;
    p->coef = 0.0f;
    p->reserved = 0;
}

__global__ void ncc_peak_finish_kernel(xc_ncc_peak *p, int out_w)
{
    const unsigned long long k = p->key;
    if (k == 0ull)
        return;
    const uint32_t idx = 0xFFFFFFFFu - (uint32_t)k;
    const uint32_t ord = (uint32_t)(k >> 32);
    p->y = (int32_t)(idx / (uint32_t)out_w);
    p->x = (int32_t)(idx % (uint32_t)out_w);
    p->coef = __uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
}

// ---------------------------------------------------------------------------
// Host-side launch helpers (called by the C ABI after validation).

template <int Q, int WV, int KS, int WC>
static hipError_t launch_ilp(NccArgs a, hipStream_t s)
{
    auto kern_tail = ncc_u8_ilp_kernel<Q, WV, KS, WC, true>;
    auto kern = ncc_u8_ilp_kernel<Q, WV, KS, WC, false>;
    constexpr int NT = 64 * WV * KS;
    auto lds_for = [&](int g) {  // LDS of tiles with g lane groups
        size_t l = ((size_t)(WV * Q * g + a.hc - 1) * a.lds_stride + (size_t)a.hc * a.t_stride) * 4;
        const size_t xchg = (size_t)WV * (KS - 1) * 3 * 4 * Q * 64 * 4;  // slice exchange, reuses the tile
        return l > xchg ? l : xchg;
    };
    auto tails = [&](int g) { return g > 1 ? (a.out_h + WV * Q * g - 1) / (WV * Q * g) : 0; };
    if (a.tail_g > 1) {
        // Tail tiles pay only where they take the grid to fewer rounds of
        // resident workgroups: every workgroup does the same work, so with
        // the same number of rounds the kernel takes as long, and a tail
        // tile's taller image tile makes it the last to finish (1920x1080
        // with 64x64: 512 workgroups, two per CU either way, 221 against
        // 226 us; with 16x16: 536 against 503, two rounds against one, 41
        // against 31 us).
        const int ncol = a.ncol_full + 1;
        const int64_t w1 = (int64_t)ncol * a.nrow_tiles, wg = (int64_t)a.ncol_full * a.nrow_tiles + tails(a.tail_g);
        int r1 = 0, rg = 0;
        const bool known = hipOccupancyMaxActiveBlocksPerMultiprocessor(&r1, kern, NT, lds_for(1)) == hipSuccess &&
                           hipOccupancyMaxActiveBlocksPerMultiprocessor(&rg, kern_tail, NT, lds_for(a.tail_g)) ==
                               hipSuccess &&
                           r1 > 0 && rg > 0;
        const int64_t cus = device_cu_count();
        if (!known || (wg + cus * rg - 1) / (cus * rg) >= (w1 + cus * r1 - 1) / (cus * r1)) {
            a.tail_g = 1;
            a.tail_nl = 64;
            a.tail_m = 1024;  // ceil(2^16 / 64)
            a.ncol_full = ncol;
        }
    }
    if (a.tail_g > 1) {
        const int64_t blocks = (int64_t)a.ncol_full * a.nrow_tiles + tails(a.tail_g);
        if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL(kern_tail, dim3((unsigned)blocks), dim3(NT), lds_for(a.tail_g), s, a);
    } else {
        hipLaunchKernelGGL(kern, dim3(a.ncol_full, a.nrow_tiles), dim3(NT), lds_for(1), s, a);
    }
    return hipGetLastError();
}

template <int Q, int WV, int KS>
static hipError_t dispatch_wc(const NccArgs &a, int wc, hipStream_t s)
{
    switch (wc) {
    case 4: return launch_ilp<Q, WV, KS, 4>(a, s);
    case 2: return launch_ilp<Q, WV, KS, 2>(a, s);
    default: return launch_ilp<Q, WV, KS, 1>(a, s);
    }
}

// Chooses the tile (Q rows per lane, WV row waves, KS template slices), the
// unroll WC and the chunking so that the LDS tile stays within 64 KiB.
hipError_t ncc_launch_ilp(NccArgs a, hipStream_t s, int force_q)
{
    const int nw = (a.t_width + 3) / 4;  // packed words per row, the last one partial when t_width % 4 != 0
    // Unroll of the template-word loop: the largest power of two <= 4 that
    // divides the whole words per template row (every chunk's whole words are
    // a multiple of it; a partial last word goes after them).
    const int nw_whole = a.t_width / 4;
    int wc = 4;
    while (wc > 1 && nw_whole % wc) wc >>= 1;
    // Tile shape: the big tile (256 x 16 outputs) when the image yields
    // enough of them to fill the CUs, else one-wave 256 x 1 tiles; the
    // template-row split when the template is tall enough to give each slice
    // several rows.  (A middle step, 256 x 4 tiles of two waves, was slower
    // than the 256 x 1 tiles on every image small enough to take it:
    // 640x480 with 16x16 15.3 against 10.5 us, with 8x8 9.2 against 7.1.)
    int q = 4, wv = 4;
    const long col_tiles = (a.out_w + 255) / 256;
    if (col_tiles * ((a.out_h + 15) / 16) < device_cu_count()) { q = 1; wv = 1; }
    int ks = (q == 4 && a.t_height >= 16) ? 2 : 1;
    if (force_q) {  // the ablation series: Q rows per lane, no template-row split
        q = wv = force_q;
        ks = 1;
    }
    const int lds_words = 64 * 1024 / 4;
    const int th = wv * q;
    // Chunk of template words: a multiple of 4 words (16-byte aligned chunk
    // starts), at most 960, and small enough that one template row fits
    // beside the tile's th image rows in 64 KiB:
    // th * (64 + cw) + cw <= lds_words (900 words for th = 16).
    const int unit = 4;
    int max_cw = (lds_words - 64 * th) / (th + 1) / unit * unit;
    if (max_cw > 960) max_cw = 960;
    int cw = nw;
    if (cw > max_cw) cw = max_cw;
    a.cw = cw;
    a.lds_stride = (64 + cw + 3) / 4 * 4;
    a.t_stride = (cw + 3) / 4 * 4;
    // (th + hc - 1) * stride + hc * t_stride <= lds_words
    int hc = (lds_words - (th - 1) * a.lds_stride) / (a.lds_stride + a.t_stride);
    if (hc < 1) hc = 1;
    if (hc > a.t_height) hc = a.t_height;
    a.hc = hc;
    // Tiles: the column tiles, the last one holding rem = out_w - 256 * (n - 1)
    // columns, i.e. nl = ceil(rem / 4) lanes.  When at least two groups of nl
    // lanes fit in a wave, that last column may go to tail tiles of G = 64 / nl
    // lane groups (G times the rows of a tile), as long as their taller
    // image tile still holds the same template rows per chunk in 64 KiB
    // (launch_ilp keeps them only where they save a round of workgroups).
    const int ncol = (a.out_w + 255) / 256;
    const int nl = ((a.out_w - 256 * (ncol - 1)) + 3) / 4;
    int G = 64 / nl;
    while (G >= 2 && ((G * th + hc - 1) * a.lds_stride + hc * a.t_stride > lds_words)) --G;
    a.nrow_tiles = (a.out_h + th - 1) / th;
    if (G >= 2) {
        a.tail_g = G;
        a.tail_nl = nl;
        a.tail_m = (65536u + (uint32_t)nl - 1) / (uint32_t)nl;
        a.ncol_full = ncol - 1;
    } else {
        a.tail_g = 1;
        a.tail_nl = 64;
        a.tail_m = 1024;  // ceil(2^16 / 64)
        a.ncol_full = ncol;
    }
    if (q == 4) return ks == 2 ? dispatch_wc<4, 4, 2>(a, wc, s) : dispatch_wc<4, 4, 1>(a, wc, s);
    if (q == 2) return dispatch_wc<2, 2, 1>(a, wc, s);
    return dispatch_wc<1, 1, 1>(a, wc, s);
}

hipError_t ncc_peak_init(void *peak, hipStream_t s)
{
    hipLaunchKernelGGL(ncc_peak_init_kernel, dim3(1), dim3(1), 0, s, static_cast<xc_ncc_peak *>(peak));
    return hipGetLastError();
}

hipError_t ncc_peak_finish(void *peak, int out_w, hipStream_t s)
{
    hipLaunchKernelGGL(ncc_peak_finish_kernel, dim3(1), dim3(1), 0, s, static_cast<xc_ncc_peak *>(peak), out_w);
    return hipGetLastError();
}

template <int C>
static hipError_t launch_cols(const NccArgs &a, hipStream_t s)
{
    dim3 grid((a.out_w + 255) / 256, (a.out_h + 3) / 4);
    const size_t lds = ((size_t)(4 + a.hc - 1) * a.lds_stride + (size_t)a.hc * a.t_stride) * 4;
    hipLaunchKernelGGL((ncc_u8_cols_kernel<C>), grid, dim3(1024 / C), lds, s, a);
    return hipGetLastError();
}

// The column-ILP ablation series: `cols` (1, 2, 4 or 8) output columns per
// lane on 256 x 4 tiles; template chunks of at most 512 words, the tile and
// the chunk's template words within 64 KiB of LDS.
hipError_t ncc_launch_cols(NccArgs a, int cols, hipStream_t s)
{
    const int nw = (a.t_width + 3) / 4;
    int cw = nw;
    if (cw > 512) cw = 512;
    a.cw = cw;
    a.lds_stride = (64 + cw + 3) / 4 * 4;
    a.t_stride = (cw + 3) / 4 * 4;
    // (4 + hc - 1) * lds_stride + hc * t_stride <= 16384 words (64 KiB)
    int hc = (16 * 1024 - 3 * a.lds_stride) / (a.lds_stride + a.t_stride);
    if (hc < 1) hc = 1;
    if (hc > a.t_height) hc = a.t_height;
    a.hc = hc;
    switch (cols) {
    case 1: return launch_cols<1>(a, s);
    case 2: return launch_cols<2>(a, s);
    case 4: return launch_cols<4>(a, s);
    case 8: return launch_cols<8>(a, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t ncc_launch_c1(NccArgs a, bool dot4, hipStream_t s)
{
    const int nw = (a.t_width + 3) / 4;
    int cw = nw;
    if (cw > 512) cw = 512;
    a.cw = cw;
    a.lds_stride = (16 + cw + 3) / 4 * 4;
    const bool word_rows = a.t_width % 4 == 0 && (reinterpret_cast<uintptr_t>(a.tmpl) & 3) == 0;
    // 48 KiB of LDS: the image tile, (4 + hc - 1) rows of lds_stride words,
    // then (rows that are not whole words) hc rows of cw template words
    a.t_stride = word_rows ? 0 : cw;
    int hc = (12 * 1024 - 3 * a.lds_stride) / (a.lds_stride + a.t_stride);
    if (hc < 1) hc = 1;
    if (hc > a.t_height) hc = a.t_height;
    a.hc = hc;
    dim3 grid((a.out_w + 63) / 64, (a.out_h + 3) / 4);
    size_t lds = ((size_t)(4 + hc - 1) * a.lds_stride + (size_t)hc * a.t_stride) * 4;
    // The dot4 form splits the template rows over KS = 2 or 4 waves per
    // output row when the grid would otherwise leave the SIMDs with about
    // one wave each (a long dependent chain per lane, its LDS and scalar
    // loads exposed): the most waves that stay within 4 per SIMD.
    // 256x256 with 16x16: 7.7 -> 5.3 us at KS = 4; 400x300 with 12x12:
    // 6.3 -> 5.6 at KS = 2; grids of over 1,000 workgroups (640x480 with
    // 8x8: 6.7 against 7.8 at KS = 2) keep KS = 1, and the scalar form
    // always does.
    const int64_t wgs = (int64_t)grid.x * grid.y, slots = 4 * (int64_t)device_cu_count();
    int ks = 1;
    if (dot4 && a.t_height >= 2)
        ks = wgs * 4 <= slots && a.t_height >= 4 ? 4 : wgs * 2 <= slots ? 2 : 1;
    if (ks > 1 && lds < (size_t)3 * (ks - 1) * 256 * 4)
        lds = (size_t)3 * (ks - 1) * 256 * 4;  // the slices' partial sums
    if (dot4 && word_rows) {
        if (ks == 4)
            hipLaunchKernelGGL((ncc_u8_c1_kernel<true, true, 4>), grid, dim3(1024), lds, s, a);
        else if (ks == 2)
            hipLaunchKernelGGL((ncc_u8_c1_kernel<true, true, 2>), grid, dim3(512), lds, s, a);
        else
            hipLaunchKernelGGL((ncc_u8_c1_kernel<true, true, 1>), grid, dim3(256), lds, s, a);
    } else if (dot4) {
        if (ks == 4)
            hipLaunchKernelGGL((ncc_u8_c1_kernel<true, false, 4>), grid, dim3(1024), lds, s, a);
        else if (ks == 2)
            hipLaunchKernelGGL((ncc_u8_c1_kernel<true, false, 2>), grid, dim3(512), lds, s, a);
        else
            hipLaunchKernelGGL((ncc_u8_c1_kernel<true, false, 1>), grid, dim3(256), lds, s, a);
    } else if (word_rows) {
        hipLaunchKernelGGL((ncc_u8_c1_kernel<false, true, 1>), grid, dim3(256), lds, s, a);
    } else {
        hipLaunchKernelGGL((ncc_u8_c1_kernel<false, false, 1>), grid, dim3(256), lds, s, a);
    }
    return hipGetLastError();
}

} // namespace xc
