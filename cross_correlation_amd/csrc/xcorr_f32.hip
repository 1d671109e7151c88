// xcorr_f32.hip -- gfx950 kernels for fp32 full 2D cross-correlation.
//
// What is computed (JPDC 2023 artifact README "Efficient GPU-accelerated
// Parallel Cross-correlation"): for every (left, right) pair and every shift
// (dy, dx) at which the matrices overlap, the sum of products over the
// overlap:  out[y][x] = sum_{i,j} L[i+dy][j+dx] * R[i][j],
// dy = y - (rows-1), dx = x - (cols-1).
//
// Kernels:
//
// * xcorr_overlap_kernel -- the overlap-wise baseline the page compares
//   against: one thread per output shift, no data reuse.
//
// * xcorr_wave_kernel -- the page's warp-per-overlap variant on a wave64:
//   one wave per output shift, its lanes splitting the overlap, partial sums
//   reduced across the wave in a fixed order.
//
// * xcorr_bd_whole_kernel / xcorr_bd_chunk_kernel / xcorr_bd_big_kernel --
//   the register-blocked (block-diagonal) kernel, in two staging modes for up
//   to 64 row blocks and in passes of 64 row blocks beyond.  The page's kernels give
//   each thread one or several neighbouring overlaps and cache the left rows
//   in warp-wide register buffers moved by shuffles; a thread-per-overlap
//   mapping leaves SIMT lanes idle wherever neighbouring overlaps have
//   different extents.  Here every lane of a wave runs the *same* number of
//   steps, with no idle work except a P-column border:
//     - Rows are grouped into blocks of 4.  Lane (slot s, block b) owns right
//       rows [4b, 4b+4) of pair s and pairs them with left row blocks
//       kb1 = (b + delta) mod nb and kb2 = kb1 + 1 (mod nb), where delta is
//       the wave's block diagonal.  Row pair (k, i) adds to dy = k - i, so
//       block kb1 with in-block offsets a >= e gives dy = 4*delta + (a-e) and
//       block kb2 with a < e gives dy = 4*delta + 4 + (a-e): the wave owns
//       output rows 4*delta .. 4*delta+3 completely, and lanes whose block
//       index wrapped past nb own the rows 4*delta - 4*nb .. +3 instead.  The
//       16 (a, e) row pairs cover every row pair exactly once over all
//       diagonals, so no lane ever multiplies outside the overlap in y.
//     - Columns: a lane owns P shift classes c0 .. c0+P-1; class c yields
//       dx = c and dx = c - w.  Both are one walk over the left columns u with
//       a P-wide sliding window of the right columns u - dx kept in registers
//       (the register buffer of the page, per lane instead of per warp);
//       zero-filled LDS columns make the border exact.
//     - Each step: one float4 of each of the two left blocks and one of the
//       right block from LDS, 16 x P fp32 FMAs.
//     - The per-lane partial sums of the same output are reduced across the
//       wave through LDS in a fixed order (deterministic, no atomics): the
//       split of one overlap over several lanes is the page's split-row idea.
//   Staging (columns transposed to [block][column][4 rows], so one 16-byte
//   LDS read gives a lane its 4 rows of a column):
//     - whole: when every matrix a workgroup touches fits in LDS with zero
//       column halos, it is staged once (left matrices shared by consecutive
//       pairs only once) and the waves walk both dx signs from LDS with no
//       further workgroup barrier (xcorr_bd_whole_pair_kernel, for up to 8
//       diagonals: the two signs of a diagonal on two waves that share
//       their walks evenly, with one barrier to hand partial sums over);
//     - chunk: otherwise columns pass through two LDS buffers J walk steps at
//       a time, the next chunk prefetched into registers during the FMAs.
//   The host picks waves per workgroup (16, 8 or 4 diagonals sharing one
//   staging) and whether the two dx signs go to separate workgroups, so that
//   small groupings still put enough waves on the 256 CUs; workgroup ids are
//   renumbered so each XCD (own L2) runs a contiguous range of tiles.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace xc {

// ---------------------------------------------------------------------------
// Overlap-wise baseline: one thread per output shift.

__global__ __launch_bounds__(256) void xcorr_overlap_kernel(XcorrArgs a)
{
    const int rows = a.rows, cols = a.cols;
    const int ow = 2 * cols - 1;
    const int per_pair = (2 * rows - 1) * ow;
    const int idx = blockIdx.x * 256 + threadIdx.x;
    if (idx >= per_pair)
        return;
    const int y = idx / ow;
    const int x = idx - y * ow;
    const int dy = y - (rows - 1);
    const int dx = x - (cols - 1);
    const int i0 = max(0, -dy), i1 = min(rows, rows - dy);
    const int j0 = max(0, -dx), j1 = min(cols, cols - dx);
    const int64_t npairs = (int64_t)a.n_left * a.n_right;
    const size_t mat = (size_t)rows * cols;
    for (int64_t p = blockIdx.y; p < npairs; p += gridDim.y) {
        const int l = (int)(p / a.n_right);
        const int r = (int)(p - (int64_t)l * a.n_right);
        const float *L = a.left + (size_t)l * mat;
        const float *R = a.right + (size_t)r * mat;
        float acc = 0.0f;
        for (int i = i0; i < i1; ++i) {
            const float *lr = L + (size_t)(i + dy) * cols + dx;
            const float *rr = R + (size_t)i * cols;
            for (int j = j0; j < j1; ++j)
                acc = fmaf(lr[j], rr[j], acc);
        }
        a.out[(size_t)p * per_pair + idx] = acc;
    }
}

hipError_t xcorr_launch_overlap(const XcorrArgs &a, hipStream_t s)
{
    const int per_pair = (2 * a.rows - 1) * (2 * a.cols - 1);
    const int64_t npairs = (int64_t)a.n_left * a.n_right;
    dim3 grid((per_pair + 255) / 256, (unsigned)(npairs < 65535 ? npairs : 65535));
    hipLaunchKernelGGL(xcorr_overlap_kernel, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Wave-per-overlap: one wave64 computes one output shift.  The JPDC page's
// warp-per-overlap variant gives a whole warp one overlap and reduces the
// lanes' partial sums at the end; here the 64 lanes take the overlap's
// elements in row-major order (lane l the elements l, l + 64, ...: adjacent
// lanes read adjacent columns), each adds its products in that order, and a
// butterfly of cross-lane exchanges (xor 32, 16, ..., 1) adds the 64 partial
// sums in a fixed order, so every lane ends with the same total and the
// result does not depend on scheduling.  Both matrices are read from global
// memory (the caches serve the neighbouring shifts of a workgroup).  Waves
// walk the outputs of all pairs in a grid-stride loop.

__global__ __launch_bounds__(256) void xcorr_wave_kernel(XcorrArgs a)
{
    const int lane = threadIdx.x & 63;
    const int rows = a.rows, cols = a.cols;
    const int ow = 2 * cols - 1;
    const int per_pair = (2 * rows - 1) * ow;
    const int64_t total = (int64_t)a.n_left * a.n_right * per_pair;
    const int64_t stride = (int64_t)gridDim.x * 4;
    for (int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); w < total; w += stride) {
        const int64_t pair = w / per_pair;
        const int idx = (int)(w - pair * per_pair);
        const int y = idx / ow;
        const int x = idx - y * ow;
        const int dy = y - (rows - 1);
        const int dx = x - (cols - 1);
        const int i0 = max(0, -dy), i1 = min(rows, rows - dy);
        const int j0 = max(0, -dx), j1 = min(cols, cols - dx);
        const int nw = j1 - j0;
        const int n = (i1 - i0) * nw;
        const int l = (int)(pair / a.n_right);
        const int r = (int)(pair - (int64_t)l * a.n_right);
        const float *L = a.left + (size_t)l * rows * cols;
        const float *R = a.right + (size_t)r * rows * cols;
        // element k of the overlap is (i0 + k / nw, j0 + k % nw): right
        // matrix offset ro = i * cols + j, left offset ro + shift
        const int shift = dy * cols + dx;
        const int di = 64 / nw, dj = 64 - di * nw;
        int i = i0 + lane / nw;
        int j = j0 + (lane - (lane / nw) * nw);
        float acc = 0.0f;
        for (int k = lane; k < n; k += 64) {
            const int ro = i * cols + j;
            acc = fmaf(L[ro + shift], R[ro], acc);
            i += di;
            j += dj;
            if (j >= j1) {
                j -= nw;
                ++i;
            }
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1)
            acc += __shfl_xor(acc, m, 64);
        if (lane == 0)
            a.out[(size_t)pair * per_pair + idx] = acc;
    }
}

hipError_t xcorr_launch_wave(const XcorrArgs &a, hipStream_t s)
{
    const int64_t total = (int64_t)a.n_left * a.n_right * (2 * a.rows - 1) * (2 * a.cols - 1);
    const int64_t blocks = (total + 3) / 4;
    hipLaunchKernelGGL(xcorr_wave_kernel, dim3((unsigned)(blocks < (1 << 22) ? blocks : (1 << 22))), dim3(256), 0, s,
                       a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Block-diagonal register-blocked kernel.

constexpr int BD_P = 4;  // shift classes (columns) per lane

struct BdArgs {
    XcorrArgs x;
    int nb;          // row blocks of 4 (rows padded with zero rows to 4*nb)
    int wp;          // columns padded with zero columns to a multiple of BD_P
    int S;           // pairs per wave (slots); S * nb <= 64
    int nls;         // distinct left matrices a pair group can touch (LDS slots)
    int n_groups;    // pair groups of S pairs
    int n_xtiles;    // wp / BD_P
    int n_dgroups;   // ceil(nb / waves per workgroup)
    int n_sides;     // 1: a workgroup walks both dx signs; 2: one sign each
    int wg_sides;    // 1: the pair kernel (a diagonal's two dx signs on two waves of a workgroup)
    // multipliers for division by nb and by the whole-staging row widths
    uint32_t m_nb, m_nr;  // fast_div_m(nb), small_div_m16(n_right)
    // exact division of any 32-bit value (div_m / div_exact) by n_sides,
    // n_dgroups, n_xtiles and n_right (workgroup ids, pair indices)
    uint32_t m_sides, m_dgroups, m_xtiles, m_right;
    // whole staging: items per row (cols / 4 or cols), rows per slot (4 nb)
    // and halo columns per unit
    uint32_t m_c4, m_cols, m_rpb, m_nh;
};

// floor(x / d) for any 32-bit x and d >= 1, with m = div_m(d): the high
// multiply gives floor(x / d) or one less (m = floor((2^32 - 1) / d) is at
// most d / 2^32 below 2^32 / d), and one compare corrects it.
__host__ __device__ constexpr uint32_t div_m(uint32_t d) { return 0xFFFFFFFFu / d; }
__device__ __forceinline__ uint32_t div_exact(uint32_t x, uint32_t d, uint32_t m)
{
    uint32_t q = __umulhi(x, m);
    q += (x - q * d >= d) ? 1u : 0u;
    return q;
}

// floor(x / d) as one high multiply, with m = fast_div_m(d); exact whenever
// x * d < 2^32 (m = (2^32 + e) / d with 0 < e <= d, so the product
// overshoots x / d by less than x / 2^32 < 1 / d).  d >= 2.
__host__ __device__ constexpr uint32_t fast_div_m(uint32_t d) { return 0xFFFFFFFFu / d + 1u; }
__device__ __forceinline__ int fast_div(int x, uint32_t m) { return (int)__umulhi((uint32_t)x, m); }

// floor(x / d) for 0 <= x < d + 64 (a pair offset within a group over the
// right-matrix count), with m16 = small_div_m16(d): for d >= 64 the quotient
// is 0 or 1; below that (x * m16) >> 16 with m16 = ceil(2^16 / d) overshoots
// x / d by less than x / 2^16 < 1 / d (x * d < 2^13), so it is exact.
__host__ __device__ constexpr uint32_t small_div_m16(uint32_t d) { return d >= 64 ? 0u : (65535u + d) / d; }
__device__ __forceinline__ int small_div(int x, int d, uint32_t m16)
{
    const int q_small = (int)(((uint32_t)x * m16) >> 16);
    return d >= 64 ? (x >= d ? 1 : 0) : q_small;
}

// LDS geometry of one staging buffer for J walk steps: per row block, J left
// columns and J + P - 1 right columns (the window halo), each a float4 of the
// block's 4 rows.  Strides are odd so lanes on consecutive blocks spread over
// the banks.
template <int J>
struct BdLds {
    static constexpr int NLU = J;                   // left columns used
    static constexpr int NRU = J + BD_P - 1;        // right columns used
    static constexpr int NCL = J | 1;               // left stride (float4s)
    static constexpr int NCR = (J + BD_P) | 1;      // right stride; >= NRU + 1 (pipelined read past the end)
};

// One walk step: left column u of both left blocks against the P right
// columns u + roff - p held in the ring; 16 (a, e) row pairs x P FMAs.
template <int P>
__device__ __forceinline__ void bd_step(const float4 l1, const float4 l2, const float4 (&ring)[P + 1], int m,
                                        float (&acc1)[4][P], float (&acc2)[3][P])
{
    const float la[4] = {l1.x, l1.y, l1.z, l1.w};
    const float lb[3] = {l2.x, l2.y, l2.z};
    // right LDS column m + P - 1 - p lives in ring slot (m + P - 1 - p) mod (P + 1)
    float re[P][4];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const float4 rv = ring[(m + P - 1 - p) % (P + 1)];
        re[p][0] = rv.x;
        re[p][1] = rv.y;
        re[p][2] = rv.z;
        re[p][3] = rv.w;
    }
    // Groups of 16 FMAs, one per right row e, each to 16 different
    // accumulators.  Accumulator (p, slot q = (ar - e) mod 4) -- acc1[q] for
    // ar >= e, acc2[q - 1] below -- keeps the same place in every group, so
    // its successive FMAs are exactly 16 instructions apart, across steps
    // too; a scheduling barrier per group keeps that order (left to itself
    // the compiler interleaved groups and put some 4 apart: 8x16 of 32x32
    // 9.00 -> 8.81 us, 1:64 of 64x64 31.7 -> 30.6 us, outputs identical).
#pragma unroll
    for (int e = 0; e < 4; ++e) {
#pragma unroll
        for (int p = 0; p < P; ++p) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int ar = (q + e) & 3;
                if (ar >= e)
                    acc1[ar - e][p] = fmaf(la[ar], re[p][e], acc1[ar - e][p]);
                else
                    acc2[ar - e + 3][p] = fmaf(lb[ar], re[p][e], acc2[ar - e + 3][p]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Accumulate `nsteps` walk steps (a multiple of P) of one staged chunk.
// The right-column window lives in a ring of P + 1 slots: during step m the
// free slot receives the column step m + 1 needs, so reads run one step
// ahead of the FMAs and no register moves are needed.  The loop body is P + 1
// groups of P steps (the ring's period), with an exit after every group, so
// the slot assignment at the back-edge matches the loop head.  A scheduling
// barrier per step keeps the compiler from hoisting reads further ahead.
template <int J>
__device__ __forceinline__ void bd_compute(const float4 *Lb1, const float4 *Lb2, const float4 *Rb, int nsteps,
                                           float (&acc1)[4][BD_P], float (&acc2)[3][BD_P])
{
    constexpr int P = BD_P;
    constexpr int PERIOD = P * (P + 1);
    float4 ring[P + 1];
#pragma unroll
    for (int r = 0; r < P; ++r)
        ring[r] = Rb[r];
    float4 l1 = Lb1[0], l2 = Lb2[0];
    for (int m0 = 0;; m0 += PERIOD) {
#pragma unroll
        for (int g = 0; g < P + 1; ++g) {
#pragma unroll
            for (int sp = 0; sp < P; ++sp) {
                const int mm = g * P + sp;  // step within the period (compile-time)
                const int m = m0 + mm;
                // reads for step m + 1 (the last step of a chunk reads one
                // column of padding, never used)
                const float4 n1 = Lb1[m + 1];
                const float4 n2 = Lb2[m + 1];
                ring[(mm + P) % (P + 1)] = Rb[m + P];
                bd_step<P>(l1, l2, ring, mm, acc1, acc2);
                l1 = n1;
                l2 = n2;
                __builtin_amdgcn_sched_barrier(0);
            }
            if (m0 + (g + 1) * P >= nsteps)
                return;
        }
    }
}

// ---------------------------------------------------------------------------
// Small matrices: one dimension of at most 16 (the "register" dimension, of
// size m <= M), the other any (the "loop" dimension, of size n).  A group of
// LC adjacent lanes owns one pair, one shift d along the loop dimension and
// SP = 8 consecutive shifts s along the register dimension (KC groups cover
// the 2M - 1 of them); lane lc of the group walks the lines i = i0 + lc,
// i0 + lc + LC, ... of the loop dimension where both matrices exist: at line
// i it holds line i + d of the left matrix and line i of the right one in
// registers (m values each, zero past the matrix) and adds, for each of its
// shifts, the products left[j + s] * right[j].  Each loaded value serves up
// to SP products, where the overlap-wise kernel loads two values per
// product.  Lines are rows (TR = false: the register dimension is cols) or
// columns (TR = true: it is rows).  A lane sums its lines in order, then the
// group adds its LC partial sums in a fixed butterfly of cross-lane
// exchanges, and its first min(LC, SP) lanes store the SP results
// round-robin.  LC (a power of two up to 64, chosen on the host from the
// shape alone) spreads long loops over lanes: these launches are
// latency-bound, and a short chain per lane with more waves on the chip
// finishes sooner (4x4 pairs of 6x200: 70.4 us with one lane per group,
// 10.4 with 32; 3x1 of 3x300: 49.7, 4.4 with 64).
struct SmallArgs {
    XcorrArgs x;
    int lc_log2;  // LC = 1 << lc_log2 lanes per group
};

template <int M, bool TR>
__global__ __launch_bounds__(256) void xcorr_small_kernel(SmallArgs sa)
{
    constexpr int SP = 8;                          // register-dimension shifts per group
    constexpr int KC = (2 * M - 1 + SP - 1) / SP;  // groups per (pair, d)
    const XcorrArgs &a = sa.x;
    const int rows = a.rows, cols = a.cols;
    const int m = TR ? rows : cols, n = TR ? cols : rows;
    const int nd = 2 * n - 1;
    const int lcs = sa.lc_log2, LC = 1 << lcs;
    const int64_t total = ((int64_t)a.n_left * a.n_right * nd * KC) << lcs;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= total)  // whole groups only: total is a multiple of LC, LC divides 64
        return;
    const int lc = (int)(t & (LC - 1));
    const int64_t g = t >> lcs;
    const int kc = (int)(g % KC);
    const int64_t u = g / KC;
    const int64_t pair = u / nd;
    const int d = (int)(u - pair * nd) - (n - 1);
    const int l = (int)(pair / a.n_right);
    const int r = (int)(pair - (int64_t)l * a.n_right);
    const float *L = a.left + (size_t)l * rows * cols;
    const float *R = a.right + (size_t)r * rows * cols;
    // element q of line i: (row i, col q) or (row q, col i)
    const int qs = TR ? cols : 1, is = TR ? 1 : cols;
    const int s0 = kc * SP - (M - 1);  // this group's first shift
    float acc[SP];
#pragma unroll
    for (int k = 0; k < SP; ++k)
        acc[k] = 0.0f;
    const int i0 = max(0, -d), i1 = min(n, n - d);  // lines where both exist
    for (int i = i0 + lc; i < i1; i += LC) {
        float lv[M], rv[M];
#pragma unroll
        for (int q = 0; q < M; ++q) {
            const int qq = q < m ? q : 0;  // an element that exists; zeroed below
            lv[q] = L[(size_t)(i + d) * is + (size_t)qq * qs];
            rv[q] = R[(size_t)i * is + (size_t)qq * qs];
            if (q >= m) {
                lv[q] = 0.0f;
                rv[q] = 0.0f;
            }
        }
#pragma unroll
        for (int j = 0; j < M; ++j) {
#pragma unroll
            for (int k = 0; k < SP; ++k) {
                // left element j + s0 + k (zero outside the line), picked
                // from registers by this group's chunk kc
                float lq = 0.0f;
#pragma unroll
                for (int c = 0; c < KC; ++c) {
                    const int qc = j + c * SP - (M - 1) + k;
                    if (c == kc && qc >= 0 && qc < M)
                        lq = lv[qc];
                }
                acc[k] = fmaf(lq, rv[j], acc[k]);
            }
        }
    }
    // butterfly over the group's lanes (xor 1, 2, ..., LC / 2): every lane
    // ends with the same sums, added in the same order
    for (int off = 1; off < LC; off <<= 1) {
#pragma unroll
        for (int k = 0; k < SP; ++k)
            acc[k] += __shfl_xor(acc[k], off);
    }
    const int oh = 2 * rows - 1, ow = 2 * cols - 1;
    float *const o = a.out + (size_t)pair * oh * ow;
#pragma unroll
    for (int k = 0; k < SP; ++k) {
        const int sft = s0 + k;
        if ((k & (LC - 1)) == lc && sft > -m && sft < m) {  // lanes past SP store nothing
            const int dy = TR ? sft : d, dx = TR ? d : sft;
            o[(size_t)(dy + rows - 1) * ow + (dx + cols - 1)] = acc[k];
        }
    }
}

// Tiny matrices: both dimensions at most 16 (the many-pair groupings of
// small matrices).  A group of LC = 1 << LCS adjacent lanes owns one pair and
// one row shift dy and computes the whole output row: all 2 cols - 1 column
// shifts.  Lane c of the group takes the rows i = i0 + c, i0 + c + LC, ...
// where both matrices exist (at most RM of them), loads every one of those
// rows of both matrices before any product (left row i + dy, right row i; M
// values each, zero past the matrix, 16-byte loads when rows are whole
// float4s), then adds left[j + dx] * right[j] for every j and shift dx, each
// product at a compile-time register (M^2 per row pair, none against the
// padding when cols == M).  The group's lanes add their sums in a fixed
// butterfly.  Consecutive groups are consecutive output rows (pair-major,
// then dy), so a wave's output is one contiguous span: lane c puts the shifts
// k = c, c + LC, ... of its group's row into the wave's LDS area, and the
// wave stores the span with consecutive lanes on consecutive floats.  Index
// math in 32 bits (the launcher checks the range).
struct TinyArgs {
    XcorrArgs x;
    uint32_t ngroups;  // pairs * (2 rows - 1)
};

template <int M, bool VEC>
__device__ __forceinline__ void tiny_row(const float *__restrict__ p, int cols, bool ok, float (&v)[M])
{
    if (VEC) {
#pragma unroll
        for (int q = 0; q < M / 4; ++q) {
            const float4 f = reinterpret_cast<const float4 *>(p)[q];
            v[4 * q] = ok ? f.x : 0.0f;
            v[4 * q + 1] = ok ? f.y : 0.0f;
            v[4 * q + 2] = ok ? f.z : 0.0f;
            v[4 * q + 3] = ok ? f.w : 0.0f;
        }
    } else {
#pragma unroll
        for (int q = 0; q < M; ++q) {
            const float f = p[q < cols ? q : 0];
            v[q] = ok && q < cols ? f : 0.0f;
        }
    }
}

template <int M, int LCS, int RM, bool VEC>
__global__ __launch_bounds__(256) void xcorr_tiny_kernel(TinyArgs ta)
{
    constexpr int LC = 1 << LCS, NS = 2 * M - 1, GW = 64 / LC;  // groups per wave
    __shared__ float stage[4][GW * NS];  // each wave's output rows, as stored
    const XcorrArgs &a = ta.x;
    const int rows = a.rows, cols = a.cols;
    const uint32_t t = blockIdx.x * 256u + threadIdx.x;
    const uint32_t grp = t >> LCS;
    const int lane = threadIdx.x & 63;
    const uint32_t g0 = (t - lane) >> LCS;  // the wave's first group
    if (g0 >= ta.ngroups)  // the whole wave is past the last group
        return;
    const bool live = grp < ta.ngroups;  // whole groups: LC divides 64
    const int c = (int)(t & (LC - 1));
    const uint32_t nd = 2u * rows - 1u;
    const uint32_t pair = (live ? grp : g0) / nd;  // dead lanes compute a live group's row, never stored
    const int dy = (int)((live ? grp : g0) - pair * nd) - (rows - 1);
    const uint32_t l = pair / (uint32_t)a.n_right;
    const uint32_t r = pair - l * (uint32_t)a.n_right;
    const float *L = a.left + (size_t)l * rows * cols;
    const float *R = a.right + (size_t)r * rows * cols;
    const int i0 = max(0, -dy), i1 = min(rows, rows - dy);  // rows where both exist
    float lv[RM][M], rv[RM][M];
#pragma unroll
    for (int q = 0; q < RM; ++q) {
        const int i = i0 + c + q * LC;
        const bool ok = i < i1;
        const int ii = ok ? i : i0;  // a row that exists; zeroed below
        tiny_row<M, VEC>(L + (size_t)(ii + dy) * cols, cols, ok, lv[q]);
        tiny_row<M, VEC>(R + (size_t)ii * cols, cols, ok, rv[q]);
    }
    float acc[NS];
#pragma unroll
    for (int k = 0; k < NS; ++k)
        acc[k] = 0.0f;
#pragma unroll
    for (int q = 0; q < RM; ++q)
#pragma unroll
        for (int j = 0; j < M; ++j)
#pragma unroll
            for (int k = 0; k < NS; ++k) {
                const int e = j + k - (M - 1);  // left element j + dx, dx = k - (M - 1)
                if (e >= 0 && e < M)
                    acc[k] = fmaf(lv[q][e], rv[q][j], acc[k]);
            }
#pragma unroll
    for (int off = 1; off < LC; off <<= 1)
#pragma unroll
        for (int k = 0; k < NS; ++k)
            acc[k] += __shfl_xor(acc[k], off);
    // the wave's groups are consecutive output rows, i.e. one contiguous
    // span: each group's row goes to the wave's LDS area, then the wave
    // stores the span with consecutive lanes on consecutive floats
    const int ow = 2 * cols - 1, k0 = M - cols;  // acc[k0 + x] is output column x
    float *const st = stage[threadIdx.x >> 6];
    const int gl = lane >> LCS;
#pragma unroll
    for (int k = 0; k < NS; ++k) {
        const int x = k - k0;
        if ((k & (LC - 1)) == c && x >= 0 && x < ow)
            st[gl * ow + x] = acc[k];
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): one wave's LDS requests complete in order
    __builtin_amdgcn_wave_barrier();
    const uint32_t nv = min((uint32_t)GW, ta.ngroups - g0);
    const int span = (int)nv * ow;
    float *const o = a.out + (size_t)g0 * ow;
    for (int e = lane; e < span; e += 64)
        o[e] = st[e];
}

// Template size of the register dimension for a shape (0 when neither
// dimension is at most 16) and whether lines are columns.
static int small_m(const XcorrArgs &a, bool &tr)
{
    tr = !(a.cols <= 16) && a.rows <= 16;
    const int m = tr ? a.rows : a.cols;
    if (m > 16)
        return 0;
    return m <= 4 ? 4 : m <= 8 ? 8 : m <= 12 ? 12 : 16;
}

bool xcorr_small_supported(const XcorrArgs &a)
{
    bool tr;
    return small_m(a, tr) > 0;
}

// Launch of the tiny kernel for lcs (lanes per group 1 << lcs) and rm row
// slots per lane.
template <int M, bool VEC>
static hipError_t tiny_launch_m(const TinyArgs &ta, int lcs, int rm, hipStream_t s)
{
    const uint64_t threads = (uint64_t)ta.ngroups << lcs;
    const dim3 g((unsigned)((threads + 255) / 256)), b(256);
    switch (lcs * 8 + rm) {
    case 0 * 8 + 1: hipLaunchKernelGGL((xcorr_tiny_kernel<M, 0, 1, VEC>), g, b, 0, s, ta); break;
    case 1 * 8 + 1: hipLaunchKernelGGL((xcorr_tiny_kernel<M, 1, 1, VEC>), g, b, 0, s, ta); break;
    case 1 * 8 + 2: hipLaunchKernelGGL((xcorr_tiny_kernel<M, 1, 2, VEC>), g, b, 0, s, ta); break;
    case 2 * 8 + 1: hipLaunchKernelGGL((xcorr_tiny_kernel<M, 2, 1, VEC>), g, b, 0, s, ta); break;
    case 2 * 8 + 2: hipLaunchKernelGGL((xcorr_tiny_kernel<M, 2, 2, VEC>), g, b, 0, s, ta); break;
    case 2 * 8 + 3: hipLaunchKernelGGL((xcorr_tiny_kernel<M, 2, 3, VEC>), g, b, 0, s, ta); break;
    case 3 * 8 + 2: hipLaunchKernelGGL((xcorr_tiny_kernel<M, 3, 2, VEC>), g, b, 0, s, ta); break;
    default: hipLaunchKernelGGL((xcorr_tiny_kernel<M, 2, 4, VEC>), g, b, 0, s, ta); break;
    }
    return hipGetLastError();
}

static hipError_t xcorr_launch_tiny(const XcorrArgs &a, hipStream_t s)
{
    const int rows = a.rows, cols = a.cols;
    const int M = cols <= 4 ? 4 : cols <= 8 ? 8 : cols <= 12 ? 12 : 16;
    const bool vec = cols == M;  // rows of whole float4s (bases are 16-byte aligned)
    // lanes per group: 1 for one row, 2 up to 3 rows, else 4, and 8 from 9
    // rows when four lanes per group would give fewer than 64K threads (short
    // chains on more waves); row slots per lane
    const uint64_t ngroups = (uint64_t)a.n_left * a.n_right * (2 * rows - 1);
    const int lcs = rows == 1 ? 0 : rows <= 3 ? 1 : (rows >= 9 && (ngroups << 2) < 65536) ? 3 : 2;
    const int rm = (rows + (1 << lcs) - 1) >> lcs;
    const TinyArgs ta{a, (uint32_t)ngroups};
    switch (M * 2 + (vec ? 1 : 0)) {
    case 8: return tiny_launch_m<4, false>(ta, lcs, rm, s);
    case 9: return tiny_launch_m<4, true>(ta, lcs, rm, s);
    case 16: return tiny_launch_m<8, false>(ta, lcs, rm, s);
    case 17: return tiny_launch_m<8, true>(ta, lcs, rm, s);
    case 24: return tiny_launch_m<12, false>(ta, lcs, rm, s);
    case 25: return tiny_launch_m<12, true>(ta, lcs, rm, s);
    case 32: return tiny_launch_m<16, false>(ta, lcs, rm, s);
    default: return tiny_launch_m<16, true>(ta, lcs, rm, s);
    }
}

hipError_t xcorr_launch_small(const XcorrArgs &a, hipStream_t s)
{
    // both dimensions at most 16, groups and threads within 32-bit indices:
    // the tiny kernel
    if (a.rows <= 16 && a.cols <= 16 &&
        ((uint64_t)a.n_left * a.n_right * (2 * a.rows - 1) << 3) < ((uint64_t)1 << 31))
        return xcorr_launch_tiny(a, s);
    bool tr;
    const int M = small_m(a, tr);
    const int n = tr ? a.cols : a.rows;
    const int64_t groups = (int64_t)a.n_left * a.n_right * (2 * n - 1) * ((2 * M - 1 + 7) / 8);
    // Lanes per group: double while each lane keeps at least two lines and
    // the launch stays within 2^19 threads (8 waves per SIMD); a cap of 16
    // lanes or of 2^18 threads was slower on long loops (1x2 pairs of
    // 200x16: 47.4 and 23.8 us against 24.0; 1x1 of 12x4000: 187 and 280
    // against 183)
    int lcs = 0;
    while (lcs < 6 && (2 << (lcs + 1)) <= n && (groups << (lcs + 1)) <= (int64_t)1 << 19) ++lcs;
    const int64_t blocks = ((groups << lcs) + 255) / 256;
    if (M == 0 || blocks > INT32_MAX)
        return hipErrorInvalidValue;
    const SmallArgs sa{a, lcs};
    const dim3 g((unsigned)blocks), b(256);
    switch (M * 2 + (tr ? 1 : 0)) {
    case 8: hipLaunchKernelGGL((xcorr_small_kernel<4, false>), g, b, 0, s, sa); break;
    case 9: hipLaunchKernelGGL((xcorr_small_kernel<4, true>), g, b, 0, s, sa); break;
    case 16: hipLaunchKernelGGL((xcorr_small_kernel<8, false>), g, b, 0, s, sa); break;
    case 17: hipLaunchKernelGGL((xcorr_small_kernel<8, true>), g, b, 0, s, sa); break;
    case 24: hipLaunchKernelGGL((xcorr_small_kernel<12, false>), g, b, 0, s, sa); break;
    case 25: hipLaunchKernelGGL((xcorr_small_kernel<12, true>), g, b, 0, s, sa); break;
    case 32: hipLaunchKernelGGL((xcorr_small_kernel<16, false>), g, b, 0, s, sa); break;
    default: hipLaunchKernelGGL((xcorr_small_kernel<16, true>), g, b, 0, s, sa); break;
    }
    return hipGetLastError();
}

// Workgroups are dispatched round-robin over the chip's 8 XCDs, each with
// its own L2.  Logical ids are renumbered so each XCD runs one contiguous
// range of them: neighbouring column tiles, which write parts of the same
// output cache lines and read the same matrices, then meet in one L2 instead
// of writing back partial lines from eight.  A bijection on [0, n), so
// results do not depend on it.
__device__ __forceinline__ int xcd_logical_id(int b, int n)
{
    const int q = n >> 3, r = n & 7;  // XCDs 0..r-1 run q + 1 workgroups, the others q
    const int xcd = b & 7, slot = b >> 3;
    return (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + slot;
}

// Geometry shared by both staging modes: which pairs, diagonal and column
// tile a workgroup / wave / lane works on.
struct BdWho {
    int lane, wave, grp, c0, delta, s, b, kb1, kb2, ls, bstar, side_lo, side_hi;
    int l_first, r_first;  // left and right matrix of the group's first pair
    bool wave_on;
};

template <int NW>
__device__ __forceinline__ BdWho bd_who(const BdArgs &a)
{
    BdWho w;
    w.lane = threadIdx.x & 63;
    w.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    uint32_t bid = (uint32_t)xcd_logical_id(blockIdx.x, gridDim.x);
    uint32_t q = div_exact(bid, (uint32_t)a.n_sides, a.m_sides);
    const int side = (int)(bid - q * (uint32_t)a.n_sides);
    bid = q;
    q = div_exact(bid, (uint32_t)a.n_dgroups, a.m_dgroups);
    const int dgrp = (int)(bid - q * (uint32_t)a.n_dgroups);
    bid = q;
    q = div_exact(bid, (uint32_t)a.n_xtiles, a.m_xtiles);
    const int xt = (int)(bid - q * (uint32_t)a.n_xtiles);
    w.grp = (int)q;
    w.c0 = xt * BD_P;
    w.side_lo = a.n_sides == 2 ? side : 0;
    w.side_hi = a.n_sides == 2 ? side + 1 : 2;
    w.delta = dgrp * NW + w.wave;  // this wave's block diagonal
    if (NW >= 2 && a.wg_sides) {
        // waves h and h + NW/2 share a diagonal and take the two dx signs,
        // whose walks (cols - c0 and c0 + P steps) add up to the same total
        // for every column tile
        constexpr int H = NW / 2;
        const int hs = w.wave >= H ? 1 : 0;
        w.side_lo = hs;
        w.side_hi = hs + 1;
        w.delta = dgrp * H + (w.wave - hs * H);
    }
    w.wave_on = w.delta < a.nb;
    const int nb = a.nb;
    int sl = fast_div(w.lane, a.m_nb);
    w.b = w.lane - sl * nb;
    if (sl >= a.S) sl = a.S - 1;  // spare lanes shadow the last slot; never stored
    w.s = sl;
    const int dl = w.wave_on ? w.delta : 0;
    int k1 = w.b + dl;  // b, dl < nb: at most one wrap
    k1 -= k1 >= nb ? nb : 0;
    int k2 = k1 + 1;
    k2 -= k2 >= nb ? nb : 0;
    w.kb1 = k1;
    w.kb2 = k2;
    // left-matrix slot: distinct left matrices of the group, in order.  The
    // group's first pair p0 is (l_first, r_first); pair p0 + d (d < 64) has
    // left matrix l_first + (r_first + d) / n_right.  (Pair indices are below
    // 2^31: the block-diagonal kernels take at least 13 rows, so a pair has
    // at least 625 outputs, and a call at most 2^40.)
    const uint32_t p0 = (uint32_t)w.grp * (uint32_t)a.S;
    const uint32_t np = (uint32_t)a.x.n_left * (uint32_t)a.x.n_right;
    w.l_first = (int)div_exact(p0, (uint32_t)a.x.n_right, a.m_right);
    const unsigned r_first = p0 - (uint32_t)w.l_first * (uint32_t)a.x.n_right;
    w.r_first = (int)r_first;
    const unsigned d = min((unsigned)sl, np - 1 - p0);
    w.ls = small_div((int)(r_first + d), a.x.n_right, a.m_nr);
    w.bstar = nb - dl - 1;  // the lane whose block 1 is unwrapped and block 2 wrapped
    return w;
}

// Sum of col[lo .. hi) (a wave-uniform range) in a fixed order: four
// interleaved partial sums, then ((0 + 1) + (2 + 3)).
__device__ __forceinline__ float bd_col_sum(const float *col, int lo, int hi)
{
    float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
    int b = lo;
    for (; b + 4 <= hi; b += 4) {
        a0 += col[b];
        a1 += col[b + 1];
        a2 += col[b + 2];
        a3 += col[b + 3];
    }
    for (; b < hi; ++b)
        a0 += col[b];
    return (a0 + a1) + (a2 + a3);
}

// Cross-lane reduction of one side's partial sums, in a fixed order, then the
// stores, in two parts.  bd_write_partials: each lane writes its 16 partials
// to the wave's area (row (r, p) of 65 floats, one per lane); comb = block-1
// sums plus block-2 sums when both blocks share the wrap status (every lane
// but bstar); bstar keeps its block-2 sums apart in the area's extra part.
__device__ __forceinline__ void bd_write_partials(const BdArgs &a, const BdWho &w, float *wred,
                                                  const float (&acc1)[4][BD_P], const float (&acc2)[3][BD_P])
{
    constexpr int P = BD_P;
    constexpr int RS = 65;  // row stride: lanes reading different rows hit different banks
    float *const wextra = wred + 4 * P * RS;
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float c = acc1[r][p];
            if (r >= 1 && w.b != w.bstar) c += acc2[r - 1][p];
            wred[(r * P + p) * RS + w.lane] = c;
        }
    if (w.b == w.bstar && w.lane < a.S * a.nb) {
#pragma unroll
        for (int p = 0; p < P; ++p)
#pragma unroll
            for (int r = 0; r < 3; ++r)
                wextra[(w.s * 3 + r) * P + p] = acc2[r][p];
    }
}

// bd_sum_store: the outputs of one side from the wave's partial area, once
// its writes are visible (PAIRS: two outputs per lane per pass, their LDS
// reads issued together -- the whole-staging kernels, whose reduction is a
// larger share of the launch; the chunked kernel keeps one, as the pairs
// cost it registers).  Lane (slot, r, p), p fastest (4 lanes store 16
// contiguous bytes), sums its column of block partials over two
// wave-uniform ranges: blocks [0, split) for output row 4*delta + r and,
// wrapped, [split, nb) for row 4*delta + r - 4*nb (plus the wrap lane's
// block-2 sums).
template <bool PAIRS>
__device__ __forceinline__ void bd_sum_store(const BdArgs &a, const BdWho &w, int side, const float *wred)
{
    constexpr int P = BD_P;
    constexpr int NV = 4 * P;
    constexpr int RS = 65;
    const int nb = a.nb, S = a.S;
    const int rows = a.x.rows, cols = a.x.cols, h4 = 4 * nb;
    const int oh = 2 * rows - 1, ow = 2 * cols - 1;
    const int64_t npairs = (int64_t)a.x.n_left * a.x.n_right;
    const int split = nb - w.delta;
    if constexpr (PAIRS) {
        // two outputs per lane per pass (o and o + 64), their LDS reads together
        for (int o0 = w.lane; o0 < S * NV; o0 += 128) {
            const bool has1 = o0 + 64 < S * NV;
            int sl[2], r[2], p[2];
            const float *col[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int o = h && has1 ? o0 + 64 : o0;
                sl[h] = o / NV;
                const int q = o - sl[h] * NV;
                p[h] = q % P;
                r[h] = q / P;
                col[h] = wred + (r[h] * P + p[h]) * RS + sl[h] * nb;
            }
            float un[2][4] = {}, wr[2][4] = {};
            int b = 0;
            for (; b + 4 <= split; b += 4)
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        un[h][k] += col[h][b + k];
            for (; b < split; ++b)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    un[h][0] += col[h][b];
            b = split;
            for (; b + 4 <= nb; b += 4)
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        wr[h][k] += col[h][b + k];
            for (; b < nb; ++b)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    wr[h][0] += col[h][b];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                if (h && !has1)
                    break;
                const float s_un = (un[h][0] + un[h][1]) + (un[h][2] + un[h][3]);
                float s_wr = (wr[h][0] + wr[h][1]) + (wr[h][2] + wr[h][3]);
                if (r[h] >= 1)
                    s_wr += wred[4 * P * RS + (sl[h] * 3 + (r[h] - 1)) * P + p[h]];
                const int64_t pair = (int64_t)w.grp * S + sl[h];
                const int c = w.c0 + p[h];
                const int dx = side ? c - a.wp : c;
                if (pair < npairs && dx > -cols && dx < cols) {
                    const int dy0 = 4 * w.delta + r[h], dy1 = dy0 - h4;
                    float *const outp = a.x.out + (size_t)pair * oh * ow + (dx + cols - 1);
                    if (dy0 < rows)
                        outp[(size_t)(dy0 + rows - 1) * ow] = s_un;
                    if (dy1 > -rows)
                        outp[(size_t)(dy1 + rows - 1) * ow] = s_wr;
                }
            }
        }
    } else {
        for (int o = w.lane; o < S * NV; o += 64) {
            const int sl = o / NV;
            const int q = o - sl * NV;
            const int p = q % P;
            const int r = q / P;
            const int64_t pair = (int64_t)w.grp * S + sl;
            const int c = w.c0 + p;
            const int dx = side ? c - a.wp : c;
            const float *col = wred + (r * P + p) * RS + sl * nb;
            const float s_un = bd_col_sum(col, 0, split);
            float s_wr = bd_col_sum(col, split, nb);
            if (r >= 1)
                s_wr += wred[4 * P * RS + (sl * 3 + (r - 1)) * P + p];
            if (pair < npairs && dx > -cols && dx < cols) {
                const int dy0 = 4 * w.delta + r, dy1 = dy0 - h4;
                float *const outp = a.x.out + (size_t)pair * oh * ow + (dx + cols - 1);
                if (dy0 < rows)
                    outp[(size_t)(dy0 + rows - 1) * ow] = s_un;
                if (dy1 > -rows)
                    outp[(size_t)(dy1 + rows - 1) * ow] = s_wr;
            }
        }
    }
}

// One side reduced within the wave: each wave uses only its own LDS area,
// so a wave-level barrier suffices.
template <bool PAIRS = false>
__device__ __forceinline__ void bd_reduce_store(const BdArgs &a, const BdWho &w, int side, float *wred,
                                                const float (&acc1)[4][BD_P], const float (&acc2)[3][BD_P])
{
    bd_write_partials(a, w, wred, acc1, acc2);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    bd_sum_store<PAIRS>(a, w, side, wred);
    // the next side's writes come after these reads in every lane's program
    // order and LDS serves one wave in order
    __builtin_amdgcn_wave_barrier();
}

// Whole staging: LDS columns per staged row block (P - 1 zero columns each
// side of the wp data columns, one padding column, odd for the banks).
__host__ __device__ constexpr int bd_whole_w(int wp) { return (wp + 2 * BD_P) | 1; }

// Reduction area per wave (floats).
__host__ __device__ constexpr int bd_red_floats(int S) { return 4 * BD_P * 65 + S * 3 * BD_P; }

// Four zeros in device memory: the load source of staged elements outside
// the matrix.
__device__ float bd_zero4[4] = {0.0f, 0.0f, 0.0f, 0.0f};

// The 4 rows of a row block at one column (zero outside the matrix).  Each
// row is loaded from the matrix or, outside it, from bd_zero4, so the loaded
// registers are the values themselves: nothing reads them before they are
// stored to LDS, and a chunk's loads stay in flight during the walk over the
// previous chunk instead of being waited for (and masked) up front.
__device__ __forceinline__ float4 bd_load4(const float *src, int nrow_ok, int gc, int cols, bool on)
{
    const bool ok = on && gc >= 0 && gc < cols;
    const float *z = bd_zero4;
    const float *p0 = ok && nrow_ok > 0 ? src + gc : z;
    const float *p1 = ok && nrow_ok > 1 ? src + cols + gc : z;
    const float *p2 = ok && nrow_ok > 2 ? src + 2 * cols + gc : z;
    const float *p3 = ok && nrow_ok > 3 ? src + 3 * cols + gc : z;
    return make_float4(*p0, *p1, *p2, *p3);
}

// ---- chunked staging: columns pass through LDS J walk steps at a time ----
template <int NW, int J>
__global__ __launch_bounds__(64 * NW) void xcorr_bd_chunk_kernel(BdArgs a)
{
    constexpr int P = BD_P;
    using G = BdLds<J>;
    extern __shared__ float4 smem[];
    const BdWho w = bd_who<NW>(a);
    const int nb = a.nb, S = a.S, wp = a.wp;
    const int rows = a.x.rows, cols = a.x.cols;
    const int64_t npairs = (int64_t)a.x.n_left * a.x.n_right;

    // LDS: two staging buffers, each L [S][nb][NCL] then R [S][nb][NCR].  A
    // side's reduction runs in the staging area once its last chunk is done
    // (a barrier separates it from the next side's staging).
    const int l_elems = S * nb * G::NCL;
    const int buf_elems = l_elems + S * nb * G::NCR;
    float *const red = reinterpret_cast<float *>(smem);
    float *const wred = red + w.wave * bd_red_floats(S);

    // Staging: thread t owns row block sb = t / NW (slot * nb + block, all
    // S*nb <= 64 blocks) and the columns congruent to t mod NW.  One item is
    // the 4 rows of that block at one column, stored as one float4; the NW
    // threads of a block read consecutive columns (coalesced per row).
    constexpr int LPT = (G::NLU + NW - 1) / NW;  // left items per thread
    constexpr int RPT = (G::NRU + NW - 1) / NW;  // right items per thread
    const int tid = threadIdx.x;
    const int sb = tid / NW;
    const int cres = tid - sb * NW;
    const int st_slot = sb / nb;
    const int st_row0 = 4 * (sb - st_slot * nb);
    const int64_t st_pair = (int64_t)w.grp * S + st_slot;
    const bool st_on = sb < S * nb && st_pair < npairs;
    const float *st_l = a.x.left;
    const float *st_r = a.x.right;
    if (st_on) {
        const int l = (int)(st_pair / a.x.n_right);
        const int r = (int)(st_pair - (int64_t)l * a.x.n_right);
        st_l += ((size_t)l * rows + st_row0) * cols;
        st_r += ((size_t)r * rows + st_row0) * cols;
    }
    const int nrow_ok = min(4, rows - st_row0);

    for (int side = w.side_lo; side < w.side_hi; ++side) {
        // Walk over left columns u; positive dx = c walks u in [c0, wp),
        // negative dx = c - wp walks u in [0, c0 + P).  Right column = u + roff - p.
        const int u_first = side ? 0 : w.c0;
        const int u_end = side ? w.c0 + P : wp;
        const int roff = side ? wp - w.c0 : -w.c0;
        const int nch = (u_end - u_first + J - 1) / J;

        auto load_chunk = [&](int t, float4 (&vl)[LPT], float4 (&vr)[RPT]) {
            const int ua = u_first + t * J;
#pragma unroll
            for (int k = 0; k < LPT; ++k)
                vl[k] = bd_load4(st_l, nrow_ok, ua + cres + k * NW, cols, st_on);
#pragma unroll
            for (int k = 0; k < RPT; ++k)
                vr[k] = bd_load4(st_r, nrow_ok, ua + roff - (P - 1) + cres + k * NW, cols, st_on);
        };
        auto store_chunk = [&](float4 *buf, const float4 (&vl)[LPT], const float4 (&vr)[RPT]) {
            if (sb < S * nb) {
#pragma unroll
                for (int k = 0; k < LPT; ++k)
                    if (cres + k * NW < G::NLU) buf[sb * G::NCL + cres + k * NW] = vl[k];
#pragma unroll
                for (int k = 0; k < RPT; ++k)
                    if (cres + k * NW < G::NRU) buf[l_elems + sb * G::NCR + cres + k * NW] = vr[k];
            }
        };

        float acc1[4][P], acc2[3][P];
#pragma unroll
        for (int p = 0; p < P; ++p) {
#pragma unroll
            for (int r = 0; r < 4; ++r) acc1[r][p] = 0.0f;
#pragma unroll
            for (int r = 0; r < 3; ++r) acc2[r][p] = 0.0f;
        }

        {
            float4 vl[LPT], vr[RPT];
            load_chunk(0, vl, vr);
            store_chunk(smem, vl, vr);
        }
        __syncthreads();
        for (int t = 0; t < nch; ++t) {
            float4 vl[LPT], vr[RPT];
            const bool more = t + 1 < nch;
            if (more) load_chunk(t + 1, vl, vr);
            if (w.wave_on) {
                const int ns = min(J, u_end - (u_first + t * J));
                const float4 *buf = smem + (t & 1) * buf_elems;
                bd_compute<J>(buf + (w.s * nb + w.kb1) * G::NCL, buf + (w.s * nb + w.kb2) * G::NCL,
                              buf + l_elems + (w.s * nb + w.b) * G::NCR, ns, acc1, acc2);
            }
            if (more) store_chunk(smem + ((t + 1) & 1) * buf_elems, vl, vr);
            __syncthreads();
        }
        if (w.wave_on)
            bd_reduce_store(a, w, side, wred, acc1, acc2);
        __syncthreads();  // reduction reads done before the next side stages
    }
}

// Whole staging of a pair group into LDS, layout [unit][W columns] of float4
// (a unit is a block of 4 rows; its float4 at index g + P - 1 holds the 4
// rows at source column g; zeros in the P - 1 columns before the data and
// from index cols + P - 1 to W).  Units: nls left slots x nb blocks, then S
// pair slots x nb blocks; a left slot sl holds matrix l_first + sl (present
// below n_left), a pair slot the right matrix (r_first + sl) mod n_right
// (present while the pair exists).  Rows past the matrix and empty slots
// load from four zeros in device memory, so no value is selected after its
// load.  When cols is a multiple of 4 (every row then starts 16-byte
// aligned) an item is one unit's 4 x 4 block at a column group: four 16-byte
// row loads, transposed in registers into four float4 columns, four 16-byte
// LDS stores; the workgroup's NT threads take BK items per batch, all loads
// of a batch issued before its stores (one batch covers the groupings that
// stage whole).  Otherwise an item is one element of a region row (the left
// slots' rows, then the pair slots', in one loop): region row R (of slots x
// 4 nb) is row R mod 4nb of slot R / 4nb and lands in unit R / 4, row R mod 4.
template <int NT>
__device__ __forceinline__ void bd_stage_whole(const BdArgs &a, float4 *smem, int W, const BdWho &w,
                                               int64_t npairs)
{
    constexpr int P = BD_P;
    const int nb = a.nb, cols = a.x.cols, rows = a.x.rows;
    const int64_t p0 = (int64_t)w.grp * a.S;
    const uint32_t mat_elems = (uint32_t)rows * (uint32_t)cols;
    const int n_on_l = a.x.n_left - w.l_first;
    const int n_on_r = (int)min((int64_t)a.S, npairs - p0);
    // the matrix of slot sl of a region: left slots never wrap (n_mod 2^30)
    auto matrix = [&](bool rg, int sl) {
        const uint32_t t = (uint32_t)((rg ? w.r_first : w.l_first) + sl);
        const uint32_t n_mod = rg ? (uint32_t)a.x.n_right : 0x40000000u;
        const uint32_t m_mod = rg ? a.m_right : 3u;  // div_m(2^30) = 3
        const uint32_t mi = t - div_exact(t, n_mod, m_mod) * n_mod;  // t mod n_mod
        return (rg ? a.x.right : a.x.left) + (uint64_t)mi * mat_elems;
    };
    if ((cols & 3) == 0) {  // workgroup-uniform
        constexpr int BK = 2;
        const int nc4 = cols >> 2;
        const int n_lu = a.nls * nb;
        const int total = (a.nls + a.S) * nb * nc4;
        for (int i0 = threadIdx.x; i0 < total; i0 += BK * NT) {
            float4 v[BK][4];
            int dst[BK];
#pragma unroll
            for (int k = 0; k < BK; ++k) {
                const int i = i0 + k * NT;
                const int U = fast_div(i, a.m_c4);  // unit
                const int cg = i - U * nc4;         // column group
                const bool rg = U >= n_lu;          // right region
                const int Ur = rg ? U - n_lu : U;
                const int sl = fast_div(Ur, a.m_nb);  // slot
                const int blk = Ur - sl * nb;
                const bool on = i < total && sl < (rg ? n_on_r : n_on_l);
                const float *src = matrix(rg, sl) + (uint32_t)(4 * blk * cols + 4 * cg);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const bool ok = on && 4 * blk + j < rows;
                    v[k][j] = *reinterpret_cast<const float4 *>(ok ? src + j * cols : bd_zero4);
                }
                dst[k] = i < total ? U * W + (P - 1) + 4 * cg : -1;
            }
#pragma unroll
            for (int k = 0; k < BK; ++k)
                if (dst[k] >= 0) {
                    smem[dst[k]] = make_float4(v[k][0].x, v[k][1].x, v[k][2].x, v[k][3].x);
                    smem[dst[k] + 1] = make_float4(v[k][0].y, v[k][1].y, v[k][2].y, v[k][3].y);
                    smem[dst[k] + 2] = make_float4(v[k][0].z, v[k][1].z, v[k][2].z, v[k][3].z);
                    smem[dst[k] + 3] = make_float4(v[k][0].w, v[k][1].w, v[k][2].w, v[k][3].w);
                }
        }
        // zero halos, one thread per unit: its P - 1 columns before the data
        // and the W - cols - P + 1 after it
        const float4 z4 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        const int nhr = W - cols - (P - 1);
        for (int i = threadIdx.x; i < (a.nls + a.S) * nb; i += NT) {
            float4 *const u = smem + i * W;
#pragma unroll
            for (int h = 0; h < P - 1; ++h)
                u[h] = z4;
            for (int h = 0; h < nhr; ++h)
                u[cols + P - 1 + h] = z4;
        }
        return;
    } else {
        constexpr int BK = 4;
        float *const sf = reinterpret_cast<float *>(smem);
        const int rpb = 4 * nb;
        for (int reg = 0; reg < 2; ++reg) {
            const bool rg = reg != 0;
            const int nslots = rg ? a.S : a.nls;
            const int n_on = rg ? n_on_r : n_on_l;
            const int unit0 = rg ? a.nls * nb : 0;
            const int total = nslots * rpb * cols;
            for (int i0 = threadIdx.x; i0 < total; i0 += BK * NT) {
                float v[BK];
                int dst[BK];
#pragma unroll
                for (int k = 0; k < BK; ++k) {
                    const int i = i0 + k * NT;
                    const int R = fast_div(i, a.m_cols);  // region row
                    const int c = i - R * cols;           // column
                    const int sl = fast_div(R, a.m_rpb);  // slot
                    const int rr = R - sl * rpb;          // row within the matrix
                    const bool ok = i < total && rr < rows && sl < n_on;
                    const float *src = matrix(rg, sl) + (uint32_t)(rr * cols + c);
                    v[k] = *(ok ? src : bd_zero4);
                    dst[k] = i < total ? (((unit0 + (R >> 2)) * W + (P - 1) + c) * 4 + (R & 3)) : -1;
                }
#pragma unroll
                for (int k = 0; k < BK; ++k)
                    if (dst[k] >= 0)
                        sf[dst[k]] = v[k];
            }
        }
    }
    // zero halos: columns [0, P - 1) and [cols + P - 1, W) of every unit
    const int n_units = (a.nls + a.S) * nb;
    const int nh = W - cols;
    for (int i = threadIdx.x; i < n_units * nh; i += NT) {
        const int u = fast_div(i, a.m_nh);
        const int h = i - u * nh;
        smem[u * W + (h < P - 1 ? h : cols + h)] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
}

// ---- whole staging: both matrices of every pair of the group (with zero
// column halos) are staged once; every wave then walks both dx signs straight
// from LDS, with no further workgroup barrier ----
template <int NW>
__global__ __launch_bounds__(64 * NW) void xcorr_bd_whole_kernel(BdArgs a)
{
    constexpr int P = BD_P;
    extern __shared__ float4 smem[];
    const BdWho w = bd_who<NW>(a);
    const int nb = a.nb, S = a.S, wp = a.wp;
    const int64_t npairs = (int64_t)a.x.n_left * a.x.n_right;
    // Every staged row block ("unit") is W LDS columns wide, left and right
    // alike: source column g at index g + P - 1, zero halos on both sides
    // (index wp + P - 1 is padding read by the pipelined walk).  Units: nls
    // left slots x nb blocks, then S pair slots x nb blocks.
    const int W = bd_whole_w(wp);
    const int n_lu = a.nls * nb;
    const int l_elems = n_lu * W;
    float4 *const Ls = smem;
    float4 *const Rs = smem + l_elems;
    float *const red = reinterpret_cast<float *>(smem + l_elems + S * nb * W);
    float *const wred = red + w.wave * bd_red_floats(S);

    bd_stage_whole<64 * NW>(a, smem, W, w, npairs);
    __syncthreads();
    if (!w.wave_on)
        return;
    // When a wave walks both dx signs, odd waves take them in the other
    // order, so that the waves of a SIMD do not all reach their reductions
    // (LDS round trips) at once.
    const int flip = (w.side_hi - w.side_lo == 2) ? (w.wave & 1) : 0;
    for (int sd = w.side_lo; sd < w.side_hi; ++sd) {
        const int side = sd ^ flip;
        const int u_first = side ? 0 : w.c0;
        const int u_end = side ? w.c0 + P : wp;
        const int roff = side ? wp - w.c0 : -w.c0;
        float acc1[4][P], acc2[3][P];
#pragma unroll
        for (int p = 0; p < P; ++p) {
#pragma unroll
            for (int r = 0; r < 4; ++r) acc1[r][p] = 0.0f;
#pragma unroll
            for (int r = 0; r < 3; ++r) acc2[r][p] = 0.0f;
        }
        // ring preload reads right columns u_first + roff - (P-1) .. u_first + roff,
        // i.e. indices u_first + roff .. + P - 1 (>= 0: roff >= -c0 and u_first >= c0 on side 0)
        bd_compute<16>(Ls + (w.ls * nb + w.kb1) * W + (P - 1) + u_first,
                       Ls + (w.ls * nb + w.kb2) * W + (P - 1) + u_first,
                       Rs + (w.s * nb + w.b) * W + u_first + roff, u_end - u_first, acc1, acc2);
        bd_reduce_store<true>(a, w, side, wred, acc1, acc2);
    }
}

// Whole staging with the two dx signs of a diagonal on two waves of one
// workgroup (waves h and h + NW/2, which the hardware places on the same
// SIMD: a workgroup's waves go round-robin over the CU's four, so with NW = 8
// each SIMD holds one diagonal's pair).  The signs' walks, wp - c0 and c0 + P
// steps, add up to wp + P for every column tile but are far apart at the
// edge tiles (32 and 4 steps at c0 = 0 for 32 columns), where the longer
// one would run mostly alone on its SIMD.  So the wave of the shorter sign
// also walks the last `tail` steps of the longer one, leaving each wave at
// most `half` = (wp + P) / 2 rounded up to P steps.  Both waves walk `tail`
// steps first (the longer sign's first and last), the second wave parks its
// partial sums in LDS, and a workgroup barrier (reached by every wave after
// the same number of steps, as all share the column tile) hands them over;
// then the first wave walks the rest of its share and adds them, and the
// second walks its own sign whole.  The longer sign's sums are thus formed
// in two parts added once, a fixed order.
template <int NW>
__global__ __launch_bounds__(64 * NW) void xcorr_bd_whole_pair_kernel(BdArgs a)
{
    constexpr int P = BD_P, H = NW / 2;
    static_assert(NW >= 2 && NW % 2 == 0, "waves come in pairs");
    extern __shared__ float4 smem[];
    const BdWho w = bd_who<NW>(a);  // a.wg_sides is set: side_lo is this wave's sign
    const int nb = a.nb, S = a.S, wp = a.wp;
    const int64_t npairs = (int64_t)a.x.n_left * a.x.n_right;
    const int W = bd_whole_w(wp);
    const int l_elems = a.nls * nb * W;
    float4 *const Ls = smem;
    float4 *const Rs = smem + l_elems;
    float *const red = reinterpret_cast<float *>(smem + l_elems + S * nb * W);
    float *const wred = red + w.wave * bd_red_floats(S);
    // handover area: per diagonal of the workgroup, 7 float4s of partial
    // sums per lane, lane-fastest
    const int own = w.side_lo;
    float4 *const part = reinterpret_cast<float4 *>(red + NW * bd_red_floats(S)) + (w.wave - own * H) * 7 * 64;

    bd_stage_whole<64 * NW>(a, smem, W, w, npairs);
    __syncthreads();

    const int len0 = wp - w.c0, len1 = w.c0 + P;
    const int g = len0 >= len1 ? 0 : 1;  // the longer sign
    const int lg = g ? len1 : len0;
    const int half = ((wp + P) / 2 + P - 1) / P * P;
    const int tail = lg > half ? lg - half : 0;  // uniform over the workgroup, a multiple of P
    const bool head = own == g;
    const float4 *const Lb1 = Ls + (w.ls * nb + w.kb1) * W + (P - 1);
    const float4 *const Lb2 = Ls + (w.ls * nb + w.kb2) * W + (P - 1);
    const float4 *const Rb = Rs + (w.s * nb + w.b) * W;
    float acc1[4][P], acc2[3][P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
#pragma unroll
        for (int r = 0; r < 4; ++r) acc1[r][p] = 0.0f;
#pragma unroll
        for (int r = 0; r < 3; ++r) acc2[r][p] = 0.0f;
    }
#pragma unroll 1
    for (int ph = tail > 0 ? 0 : 1; ph < 2; ++ph) {
        // phase 0: `tail` steps of the longer sign, from its start (head
        // wave) or up to its end (the other); phase 1: the rest of the head
        // wave's share, or the other wave's own sign whole
        const int side = head || ph == 0 ? g : own;
        const int u_first = side ? 0 : w.c0;
        const int roff = side ? wp - w.c0 : -w.c0;
        int u0, n;
        if (head) {
            u0 = u_first + (ph ? tail : 0);
            n = ph ? lg - 2 * tail : tail;
        } else {
            u0 = ph ? u_first : u_first + lg - tail;
            n = ph ? (side ? len1 : len0) : tail;
        }
        // ring preload reads right indices u0 + roff .. + P - 1 (>= 0: roff >= -c0, u0 >= c0 on side 0)
        if (w.wave_on && n > 0)
            bd_compute<16>(Lb1 + u0, Lb2 + u0, Rb + u0 + roff, n, acc1, acc2);
        if (ph == 0) {
            if (w.wave_on && !head) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    part[r * 64 + w.lane] = make_float4(acc1[r][0], acc1[r][1], acc1[r][2], acc1[r][3]);
#pragma unroll
                    for (int p = 0; p < P; ++p) acc1[r][p] = 0.0f;
                }
#pragma unroll
                for (int r = 0; r < 3; ++r) {
                    part[(4 + r) * 64 + w.lane] = make_float4(acc2[r][0], acc2[r][1], acc2[r][2], acc2[r][3]);
#pragma unroll
                    for (int p = 0; p < P; ++p) acc2[r][p] = 0.0f;
                }
            }
            __syncthreads();
        }
    }
    if (!w.wave_on)
        return;
    if (head && tail > 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float4 v = part[r * 64 + w.lane];
            acc1[r][0] += v.x;
            acc1[r][1] += v.y;
            acc1[r][2] += v.z;
            acc1[r][3] += v.w;
        }
#pragma unroll
        for (int r = 0; r < 3; ++r) {
            const float4 v = part[(4 + r) * 64 + w.lane];
            acc2[r][0] += v.x;
            acc2[r][1] += v.y;
            acc2[r][2] += v.z;
            acc2[r][3] += v.w;
        }
    }
    bd_reduce_store<true>(a, w, own, wred, acc1, acc2);
}

// ---- more than 64 row blocks: passes over 64-block ranges ----
// One pair per workgroup, NW consecutive diagonals per workgroup (S = 1).
// Pass q covers right blocks [64q, 64q + 64): lane b walks right block
// B = 64q + b against left blocks kb1 = (B + delta) mod nb and kb2 = kb1 + 1
// (mod nb), which lie in the window of BIG_LW blocks starting at
// (64q + delta0) mod nb (delta0 = the workgroup's first diagonal), at window
// index b + wave and b + wave + 1.  Columns stream through two LDS buffers J
// walk steps at a time.  After each side of each pass the wave reduces its
// lanes in a fixed order and stores (pass 0) or adds to (later passes) its
// output rows, which no other wave writes: the result does not depend on
// scheduling.
template <int NW>
struct BdBig {
    static constexpr int LW = 64 + NW + 1;  // left window blocks
};

__device__ __forceinline__ void bd_big_reduce_store(const BdArgs &a, int lane, int delta, int c0, int side, int64_t pair,
                                                    int q, float *wred, float *wextra,
                                                    const float (&acc1)[4][BD_P], const float (&acc2)[3][BD_P])
{
    constexpr int P = BD_P;
    constexpr int RS = 65;
    const int nb = a.nb;
    const int B = 64 * q + lane;
    const int bstar = nb - delta - 1;  // block 1 unwrapped, block 2 wrapped
    const bool star_here = bstar >= 64 * q && bstar < 64 * q + 64;
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float c = acc1[r][p];
            if (r >= 1 && B != bstar) c += acc2[r - 1][p];
            wred[(r * P + p) * RS + lane] = c;
        }
    if (B == bstar) {
#pragma unroll
        for (int p = 0; p < P; ++p)
#pragma unroll
            for (int r = 0; r < 3; ++r)
                wextra[r * P + p] = acc2[r][p];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int rows = a.x.rows, cols = a.x.cols, h4 = 4 * nb;
    const int oh = 2 * rows - 1, ow = 2 * cols - 1;
    if (lane < 8 * P) {
        const int p = lane % P;
        const int wr = (lane / P) & 1;
        const int r = lane / (2 * P);
        const int dy = 4 * delta + r - (wr ? h4 : 0);
        const int c = c0 + p;
        const int dx = side ? c - a.wp : c;
        const bool keep = dy > -rows && dy < rows && dx > -cols && dx < cols;
        // lanes of this pass that add to (r, wr): blocks [blo, bhi) shifted
        const int blo = max(wr ? nb - delta : 0, 64 * q) - 64 * q;
        const int bhi = min(wr ? nb : nb - delta, 64 * q + 64) - 64 * q;
        const float *col = wred + (r * P + p) * RS;
        float part[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) part[i] = 0.0f;
        for (int bb = blo & ~7; bb < bhi; bb += 8) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int b = bb + i;
                const float v = col[min(b, 63)];
                const int keep_b = -(int)((b >= blo) & (b < bhi));  // all ones or zero
                part[i] += __int_as_float(__float_as_int(v) & keep_b);
            }
        }
        float sum = ((part[0] + part[1]) + (part[2] + part[3])) + ((part[4] + part[5]) + (part[6] + part[7]));
        if (wr && r >= 1 && star_here)
            sum += wextra[(r - 1) * P + p];
        if (keep) {
            float *o = a.x.out + ((size_t)pair * oh + (dy + rows - 1)) * ow + (dx + cols - 1);
            *o = q == 0 ? sum : *o + sum;
        }
    }
    __builtin_amdgcn_wave_barrier();
}

template <int NW, int J>
__global__ __launch_bounds__(64 * NW) void xcorr_bd_big_kernel(BdArgs a)
{
    constexpr int P = BD_P;
    using G = BdLds<J>;
    constexpr int LW = BdBig<NW>::LW;
    extern __shared__ float4 smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int bid = xcd_logical_id(blockIdx.x, gridDim.x);
    const int side_sel = bid % a.n_sides;
    bid /= a.n_sides;
    const int dgrp = bid % a.n_dgroups;
    bid /= a.n_dgroups;
    const int xt = bid % a.n_xtiles;
    const int64_t pair = bid / a.n_xtiles;
    const int c0 = xt * P;
    const int side_lo = a.n_sides == 2 ? side_sel : 0;
    const int side_hi = a.n_sides == 2 ? side_sel + 1 : 2;
    const int nb = a.nb, wp = a.wp, rows = a.x.rows, cols = a.x.cols;
    const int delta0 = dgrp * NW;
    const int delta = delta0 + wave;
    const bool wave_on = delta < nb;
    const int npass = (nb + 63) / 64;

    const int l = (int)(pair / a.x.n_right);
    const int r = (int)(pair - (int64_t)l * a.x.n_right);
    const float *lmat = a.x.left + (size_t)l * rows * cols;
    const float *rmat = a.x.right + (size_t)r * rows * cols;

    // LDS: two staging buffers, each L [LW][NCL] then R [64][NCR]; the
    // per-wave reduction runs in the staging area once a side is done.
    constexpr int L_ELEMS = LW * G::NCL;
    constexpr int BUF = L_ELEMS + 64 * G::NCR;
    float *const wred = reinterpret_cast<float *>(smem) + wave * bd_red_floats(1);
    float *const wextra = wred + 4 * P * 65;

    // Staging items: left (window block, column) then right (block, column).
    constexpr int NL_ITEMS = LW * G::NLU;
    constexpr int N_ITEMS = NL_ITEMS + 64 * G::NRU;
    constexpr int IPT = (N_ITEMS + 64 * NW - 1) / (64 * NW);

    for (int q = 0; q < npass; ++q) {
        const int L0 = (64 * q + delta0) % nb;
        for (int side = side_lo; side < side_hi; ++side) {
            const int u_first = side ? 0 : c0;
            const int u_end = side ? c0 + P : wp;
            const int roff = side ? wp - c0 : -c0;
            const int nch = (u_end - u_first + J - 1) / J;

            auto load_chunk = [&](int t, float4 (&v)[IPT]) {
                const int ua = u_first + t * J;
#pragma unroll
                for (int k = 0; k < IPT; ++k) {
                    // left (window block, column) or right (block, column):
                    // parameters selected, one unconditional load sequence
                    const int i = threadIdx.x + k * 64 * NW;
                    const bool is_l = i < NL_ITEMS;
                    const int j = is_l ? i : i - NL_ITEMS;
                    const int blk = is_l ? j / G::NLU : j / G::NRU;
                    const int cc = j - blk * (is_l ? G::NLU : G::NRU);
                    int kb = L0 + blk;  // L0 < nb, blk < 81 < 2 nb: at most two wraps
                    kb -= kb >= nb ? nb : 0;
                    kb -= kb >= nb ? nb : 0;
                    const int rb = 64 * q + blk;
                    const bool on = is_l || (i < N_ITEMS && rb < nb);
                    const int row0 = 4 * (is_l ? kb : rb);
                    const float *src = (is_l ? lmat : rmat) + (size_t)row0 * cols;
                    const int gc = is_l ? ua + cc : ua + roff - (P - 1) + cc;
                    v[k] = bd_load4(src, min(4, rows - row0), gc, cols, on);
                }
            };
            auto store_chunk = [&](float4 *buf, const float4 (&v)[IPT]) {
#pragma unroll
                for (int k = 0; k < IPT; ++k) {
                    const int i = threadIdx.x + k * 64 * NW;
                    if (i < NL_ITEMS) {
                        const int blk = i / G::NLU, cc = i - blk * G::NLU;
                        buf[blk * G::NCL + cc] = v[k];
                    } else if (i < N_ITEMS) {
                        const int j = i - NL_ITEMS;
                        const int blk = j / G::NRU, cc = j - blk * G::NRU;
                        buf[L_ELEMS + blk * G::NCR + cc] = v[k];
                    }
                }
            };

            float acc1[4][P], acc2[3][P];
#pragma unroll
            for (int p = 0; p < P; ++p) {
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) acc1[rr][p] = 0.0f;
#pragma unroll
                for (int rr = 0; rr < 3; ++rr) acc2[rr][p] = 0.0f;
            }
            {
                float4 v[IPT];
                load_chunk(0, v);
                store_chunk(smem, v);
            }
            __syncthreads();
            for (int t = 0; t < nch; ++t) {
                float4 v[IPT];
                const bool more = t + 1 < nch;
                if (more) load_chunk(t + 1, v);
                if (wave_on) {
                    const int ns = min(J, u_end - (u_first + t * J));
                    const float4 *buf = smem + (t & 1) * BUF;
                    bd_compute<J>(buf + (lane + wave) * G::NCL, buf + (lane + wave + 1) * G::NCL,
                                  buf + L_ELEMS + lane * G::NCR, ns, acc1, acc2);
                }
                if (more) store_chunk(smem + ((t + 1) & 1) * BUF, v);
                __syncthreads();
            }
            if (wave_on)
                bd_big_reduce_store(a, lane, delta, c0, side, pair, q, wred, wextra, acc1, acc2);
            __syncthreads();  // reduction reads done before the next staging
        }
    }
}

bool xcorr_blockdiag_supported(const XcorrArgs &a)
{
    const int nb = (a.rows + 3) / 4;
    return nb >= 4;
}

constexpr size_t BD_LDS_MAX = 160 * 1024;

// Whole staging LDS: the staged units, then one partial-sum area per wave.
static size_t bd_whole_lds(const BdArgs &b, int nw, bool pairs)
{
    return (size_t)(b.nls + b.S) * b.nb * bd_whole_w(b.wp) * sizeof(float4) +
           (size_t)nw * bd_red_floats(b.S) * sizeof(float) +
           (pairs ? (size_t)(nw / 2) * 7 * 64 * sizeof(float4) : 0);  // the pair kernel's handover area
}

template <int NW, int J>
static size_t bd_chunk_lds(const BdArgs &b)
{
    using G = BdLds<J>;
    const size_t stage = 2 * (size_t)b.S * b.nb * (G::NCL + G::NCR) * sizeof(float4);
    const size_t red = (size_t)NW * bd_red_floats(b.S) * sizeof(float);
    return stage > red ? stage : red;
}

// Multipliers for the kernels' divisions by this launch's grid factors and
// staging widths (set once the launcher has fixed them).
static void bd_set_magic(BdArgs &b)
{
    b.m_sides = div_m((uint32_t)b.n_sides);
    b.m_dgroups = div_m((uint32_t)b.n_dgroups);
    b.m_xtiles = div_m((uint32_t)b.n_xtiles);
    // whole staging only (rows of at least 29 columns, so every divisor
    // below is at least 2, as fast_div needs); unused by the other kernels
    const uint32_t nc4 = (uint32_t)(b.x.cols / 4), nh = (uint32_t)(bd_whole_w(b.wp) - b.x.cols);
    b.m_c4 = nc4 >= 2 ? fast_div_m(nc4) : 0u;
    b.m_cols = b.x.cols >= 2 ? fast_div_m((uint32_t)b.x.cols) : 0u;
    b.m_nh = nh >= 2 ? fast_div_m(nh) : 0u;
    b.m_rpb = fast_div_m((uint32_t)(4 * b.nb));
}

template <int NW>
static hipError_t launch_whole(BdArgs b, hipStream_t s)
{
    // dynamic LDS above 64 KiB must be allowed explicitly
    static std::atomic<uint64_t> lds_allowed{0};
    const hipError_t e = allow_lds_once(&xcorr_bd_whole_kernel<NW>, lds_allowed);
    if (e != hipSuccess) return e;
    b.wg_sides = 0;
    b.n_dgroups = (b.nb + NW - 1) / NW;
    bd_set_magic(b);
    const int64_t blocks = (int64_t)b.n_groups * b.n_xtiles * b.n_dgroups * b.n_sides;
    if (blocks > INT32_MAX)  // the kernels number workgroups with 32-bit signed ids
        return hipErrorInvalidConfiguration;
    const size_t lds = bd_whole_lds(b, NW, false);
    hipLaunchKernelGGL((xcorr_bd_whole_kernel<NW>), dim3((unsigned)blocks), dim3(64 * NW), lds, s, b);
    return hipGetLastError();
}

// NW / 2 diagonals per workgroup, each on a pair of waves
template <int NW>
static hipError_t launch_whole_pairs(BdArgs b, hipStream_t s)
{
    static std::atomic<uint64_t> lds_allowed{0};
    const hipError_t e = allow_lds_once(&xcorr_bd_whole_pair_kernel<NW>, lds_allowed);
    if (e != hipSuccess) return e;
    b.wg_sides = 1;
    b.n_sides = 1;
    b.n_dgroups = (b.nb + NW / 2 - 1) / (NW / 2);
    bd_set_magic(b);
    const int64_t blocks = (int64_t)b.n_groups * b.n_xtiles * b.n_dgroups;
    if (blocks > INT32_MAX)
        return hipErrorInvalidConfiguration;
    const size_t lds = bd_whole_lds(b, NW, true);
    hipLaunchKernelGGL((xcorr_bd_whole_pair_kernel<NW>), dim3((unsigned)blocks), dim3(64 * NW), lds, s, b);
    return hipGetLastError();
}

template <int NW, int J>
static hipError_t launch_chunk(BdArgs b, hipStream_t s)
{
    // dynamic LDS above 64 KiB must be allowed explicitly
    static std::atomic<uint64_t> lds_allowed{0};
    const hipError_t e = allow_lds_once(&xcorr_bd_chunk_kernel<NW, J>, lds_allowed);
    if (e != hipSuccess) return e;
    b.n_dgroups = (b.nb + NW - 1) / NW;
    bd_set_magic(b);
    const int64_t blocks = (int64_t)b.n_groups * b.n_xtiles * b.n_dgroups * b.n_sides;
    if (blocks > INT32_MAX)  // the kernels number workgroups with 32-bit signed ids
        return hipErrorInvalidConfiguration;
    const size_t lds = bd_chunk_lds<NW, J>(b);
    hipLaunchKernelGGL((xcorr_bd_chunk_kernel<NW, J>), dim3((unsigned)blocks), dim3(64 * NW), lds, s, b);
    return hipGetLastError();
}

template <int NW, int J>
static size_t bd_big_lds()
{
    using G = BdLds<J>;
    const size_t stage = 2 * ((size_t)BdBig<NW>::LW * G::NCL + 64 * G::NCR) * sizeof(float4);
    const size_t red = (size_t)NW * bd_red_floats(1) * sizeof(float);
    return stage > red ? stage : red;
}

template <int NW, int J>
static hipError_t launch_big(BdArgs b, hipStream_t s)
{
    // dynamic LDS above 64 KiB must be allowed explicitly
    static std::atomic<uint64_t> lds_allowed{0};
    const hipError_t e = allow_lds_once(&xcorr_bd_big_kernel<NW, J>, lds_allowed);
    if (e != hipSuccess) return e;
    b.n_dgroups = (b.nb + NW - 1) / NW;
    const int64_t per = (int64_t)b.n_groups * b.n_xtiles * b.n_dgroups;
    b.n_sides = per >= 1024 ? 1 : 2;
    const int64_t blocks = per * b.n_sides;
    if (blocks > INT32_MAX)
        return hipErrorInvalidConfiguration;
    const size_t lds = bd_big_lds<NW, J>();
    hipLaunchKernelGGL((xcorr_bd_big_kernel<NW, J>), dim3((unsigned)blocks), dim3(64 * NW), lds, s, b);
    return hipGetLastError();
}

hipError_t xcorr_launch_blockdiag(const XcorrArgs &a, hipStream_t s)
{
    BdArgs b;
    b.x = a;
    b.nb = (a.rows + 3) / 4;
    b.wp = (a.cols + BD_P - 1) / BD_P * BD_P;
    b.m_nb = fast_div_m((uint32_t)b.nb);
    b.m_nr = small_div_m16((uint32_t)a.n_right);
    b.m_right = div_m((uint32_t)a.n_right);
    b.wg_sides = 0;

    const int64_t npairs = (int64_t)a.n_left * a.n_right;
    if (b.nb > 64) {
        // more row blocks than lanes: one pair per workgroup, passes of 64 blocks
        b.S = 1;
        b.nls = 1;
        b.n_groups = (int)npairs;
        b.n_xtiles = b.wp / BD_P;
        // 16 walk steps per chunk: half the barriers of 8 (the prefetch of
        // the next chunk overlaps the walk either way); five prologue values
        // spill, reloaded once per pass
        return launch_big<16, 16>(b, s);
    }
    b.S = 64 / b.nb;
    b.n_groups = (int)((npairs + b.S - 1) / b.S);
    b.n_xtiles = b.wp / BD_P;
    // distinct left matrices one group of S consecutive pairs can touch
    int nls = (b.S + a.n_right - 1) / a.n_right + 1;
    if (nls > b.S) nls = b.S;
    if (nls > a.n_left) nls = a.n_left;
    b.nls = nls;
    const int64_t per_side = (int64_t)b.n_groups * b.n_xtiles;
    // Waves per workgroup: the most (they share one staging) that keeps at
    // least 256 workgroups; walk the two dx signs in separate workgroups when
    // that is needed to reach 256.
    auto pick = [&](int nw) { return per_side * ((b.nb + nw - 1) / nw); };
    int nw = 4;
    if (b.nb >= 16 && pick(16) >= 256) nw = 16;
    else if (b.nb >= 8 && pick(8) >= 256) nw = 8;
    // split the two dx signs over workgroups when the grid would hold fewer
    // than 4096 waves (4 per SIMD)
    b.n_sides = pick(nw) * nw >= 4096 ? 1 : 2;
    // Whole staging keeps every matrix of a pair group in LDS, so few of its
    // workgroups fit on a CU.  Take it when those leave at least four waves
    // per SIMD or the whole grid is resident at once; otherwise stream
    // chunks, whose small LDS keeps the CUs full.  Below 32 columns the walks
    // are too short to repay staging every column before the first step (the
    // chunked kernel starts after its first J + P columns).
    const int64_t cus = device_cu_count();
    auto whole_ok = [&](int nw_, int sides, bool pairs = false) {
        if (b.wp < 32) return false;
        const size_t lds = bd_whole_lds(b, nw_, pairs);
        if (lds > BD_LDS_MAX) return false;
        const int64_t per_cu = (int64_t)(BD_LDS_MAX / lds);
        const int64_t n_wg = per_side * ((b.nb + nw_ - 1) / nw_) * sides;
        return per_cu * nw_ >= 16 || n_wg <= per_cu * cus;
    };
    // Up to 8 diagonals: 8-wave workgroups, each half walking one dx sign of
    // the same 4 diagonals, the pair of waves of a diagonal sharing its two
    // walks evenly (at most (wp + P) / 2, rounded up to P, steps each).
    if (b.nb <= 8 && whole_ok(8, 2, true))
        return launch_whole_pairs<8>(b, s);
    if (nw == 16 && whole_ok(16, b.n_sides)) return launch_whole<16>(b, s);
    if (nw >= 8 && whole_ok(8, nw == 16 ? 2 : b.n_sides)) {
        if (nw == 16) b.n_sides = 2;  // half the waves per workgroup: keep the wave count
        return launch_whole<8>(b, s);
    }
    if (nw == 4 && whole_ok(4, b.n_sides)) return launch_whole<4>(b, s);
    if (nw == 16) return launch_chunk<16, 16>(b, s);
    if (nw == 8) return launch_chunk<8, 8>(b, s);
    return launch_chunk<4, 8>(b, s);
}

} // namespace xc
