// xcorr_mfma.hip -- fp32 full 2D cross-correlation on the fp32 matrix cores
// (v_mfma_f32_16x16x4f32).
//
// The computation of the JPDC 2023 artifact README "Efficient GPU-accelerated
// Parallel Cross-correlation" (every shift at which two matrices overlap,
// for one-to-one, one-to-many and n-to-m groupings), with the same output
// convention as the other kernels of this library:
//   out[pair][dy + rows - 1][dx + cols - 1] = sum_i sum_j L[i + dy][j + dx] R[i][j].
// Writing u = i + dy (a row of the left matrix):
//   out[dy][dx] = sum_u sum_j R[u - dy][j] * L[u][j + dx],
// so for each left row u the contribution to all shifts is a matrix product:
// rows indexed by dy (R's rows, read backwards from u), columns by dx (L's
// row u, shifted by dx: Toeplitz along the columns), contracted over j.  One
// workgroup takes one 16 x 16 tile of shifts (dy0.., dx0..) of one pair:
//   D[m][n] += sum_k A[m][k] B[k][n],  A[m][k] = R[u - dy0 - m][j],
//                                      B[k][n] = L[u][j + dx0 + n],
// over the left rows u and columns j that meet some shift of the tile (the
// band of zero products outside is skipped, except at its edges).  The four
// MFMAs of a 16-column group take the K slots in a permuted order: MFMA t
// gives slot k the column j = jg + 4k + t, so lane (m, k) reads its four A
// values of the group as one aligned 16-byte LDS read and its four B values
// from four consecutive floats; every column of the group is summed once.
// Each MFMA t has its own accumulator, and each of a wave's two left rows of
// a chunk its own four (independent products back to back, eight shorter
// sums), added in a fixed order at the end.
//
// Staging: left rows in chunks of 8 (and the 23 right rows they meet with
// the tile's 16 row shifts), zero outside the matrices, double-buffered in
// LDS: the next chunk's global loads are in flight during the current
// chunk's products.  The four waves take the left rows u = q (mod 4) of each
// chunk; their partial tiles are added in LDS in a fixed order, so results do
// not depend on scheduling.  Tiles are dispatched from the centre of the
// shift range outwards (heavy tiles first), so the lighter edge tiles fill
// the compute units as the heavy ones finish.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace xc {

typedef float xm_v4f __attribute__((ext_vector_type(4)));

constexpr int XM_T = 16;        // shifts per tile side
constexpr int XM_UC = 8;        // left rows per staged chunk
constexpr int XM_RR = XM_UC + XM_T - 1;  // right rows a chunk meets
constexpr int XM_THREADS = 256; // four waves
constexpr int XM_PF = 12;       // staged float4 items per thread (the host checks the plan fits)

struct XmArgs {
    XcorrArgs x;
    int ty, tx;    // tiles along dy and dx
    int ls, rs;    // LDS floats per staged left / right row
    int nl4, nr4;  // float4 items of a chunk's left / right region
};

// Tile index of rank k from the centre c of n tiles outwards: c, c + 1,
// c - 1, c + 2, ..., then the rest of the longer side.
__device__ __forceinline__ int xm_center_out(int k, int n, int c)
{
    const int lo = c, hi = n - 1 - c, m = min(lo, hi);
    if (k <= 2 * m)
        return (k & 1) ? c + (k + 1) / 2 : c - k / 2;
    const int e = k - 2 * m;
    return hi > lo ? c + m + e : c - m - e;
}

__global__ __launch_bounds__(XM_THREADS) void xcorr_mfma_kernel(XmArgs xa)
{
    extern __shared__ xm_v4f xm_smem[];
    const XcorrArgs &a = xa.x;
    const int h = a.rows, w = a.cols;
    const int np = a.n_left * a.n_right;
    const int rank = blockIdx.x / np, pair = blockIdx.x - rank * np;
    const int ty = xm_center_out(rank / xa.tx, xa.ty, (h - 1) / XM_T);
    const int tx = xm_center_out(rank - (rank / xa.tx) * xa.tx, xa.tx, (w - 1) / XM_T);
    const int dy0 = ty * XM_T - (h - 1), dx0 = tx * XM_T - (w - 1);
    const int li = pair / a.n_right, ri = pair - li * a.n_right;
    const float *const L = a.left + (size_t)li * h * w;
    const float *const R = a.right + (size_t)ri * h * w;

    // left rows that meet some row shift of the tile, columns of R that meet
    // some column shift (16-column groups from jg0)
    const int ulo = max(0, dy0), uhi = min(h, h + dy0 + XM_T - 1);
    const int jlo = max(0, -dx0 - (XM_T - 1)), jhi = min(w, w - dx0);
    const int jg0 = jlo & ~15, ng = (jhi - jg0 + 15) >> 4;
    const int cl0 = (jg0 + dx0) & ~3;  // first staged left column (a multiple of 4, maybe negative)

    const int ls = xa.ls, rs = xa.rs;
    float *const buf0 = reinterpret_cast<float *>(xm_smem);
    const int bufsz = XM_UC * ls + XM_RR * rs;
    float *const part = buf0 + 2 * bufsz;  // four partial tiles of 256 floats

    // This thread's staging items: LDS offset, global offset at u0 = 0, the
    // row (left row, or right row + dy0 + 15 - u0... as a left-row-relative
    // index) and whether its four columns lie inside the matrix.  Columns are
    // multiples of 4 and cols % 4 == 0, so a float4 is wholly in or out.
    int it_lds[XM_PF], it_row[XM_PF];
    int64_t it_g[XM_PF];
    bool it_ok[XM_PF];
    const int nit = xa.nl4 + xa.nr4;
#pragma unroll
    for (int k = 0; k < XM_PF; ++k) {
        const int i = threadIdx.x + k * XM_THREADS;
        it_ok[k] = false;
        it_lds[k] = 0;
        it_row[k] = 0;
        it_g[k] = 0;
        if (i < xa.nl4) {
            const int row = i / (ls / 4), c4 = i - row * (ls / 4);
            const int col = cl0 + 4 * c4;
            it_lds[k] = row * ls + 4 * c4;
            it_row[k] = row;  // left row u0 + row
            it_g[k] = (int64_t)row * w + col;
            it_ok[k] = col >= 0 && col < w;
        } else if (i < nit) {
            const int i2 = i - xa.nl4;
            const int row = i2 / (rs / 4), c4 = i2 - row * (rs / 4);
            const int col = jg0 + 4 * c4;
            it_lds[k] = XM_UC * ls + row * rs + 4 * c4;
            it_row[k] = row - dy0 - (XM_T - 1);  // right row u0 + this
            it_g[k] = (int64_t)it_row[k] * w + col;
            it_ok[k] = col >= 0 && col < w;
        }
    }
    auto fetch = [&](int u0, xm_v4f (&v)[XM_PF]) {
#pragma unroll
        for (int k = 0; k < XM_PF; ++k) {
            const int i = threadIdx.x + k * XM_THREADS;
            const int row = u0 + it_row[k];
            const bool ok = i < nit && it_ok[k] && row >= 0 && row < h;
            const float *src = (i < xa.nl4) ? L : R;
            v[k] = ok ? *reinterpret_cast<const xm_v4f *>(src + it_g[k] + (int64_t)u0 * w)
                      : xm_v4f{0.f, 0.f, 0.f, 0.f};
        }
    };
    auto put = [&](float *buf, const xm_v4f (&v)[XM_PF]) {
#pragma unroll
        for (int k = 0; k < XM_PF; ++k) {
            const int i = threadIdx.x + k * XM_THREADS;
            if (i < nit)
                *reinterpret_cast<xm_v4f *>(buf + it_lds[k]) = v[k];
        }
    };

    const int lane = threadIdx.x & 63, q = threadIdx.x >> 6;
    const int mn = lane & 15, kk = lane >> 4;
    xm_v4f acc[4], acc2[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        acc[t] = xm_v4f{0.f, 0.f, 0.f, 0.f};
        acc2[t] = xm_v4f{0.f, 0.f, 0.f, 0.f};
    }

    const int nch = ulo < uhi ? (uhi - ulo + XM_UC - 1) / XM_UC : 0;
    xm_v4f pf[XM_PF];
    if (nch > 0) {
        fetch(ulo, pf);
        put(buf0, pf);
    }
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
        const int u0 = ulo + c * XM_UC;
        float *const cur = buf0 + (c & 1) * bufsz;
        const bool more = c + 1 < nch;
        if (more)
            fetch(u0 + XM_UC, pf);
        const float *const lb = cur, *const rb = cur + XM_UC * ls;
        // the wave's two left rows of the chunk (u0 + q and u0 + q + 4), each
        // into its own four accumulators; A: right row u - dy0 - m (staged
        // row ur + 15 - m), columns jg + 4kk .. +3; B: left row u, columns
        // jg + 4kk + t + dx0 + n.  Groups alternate between two register
        // sets, the next group's LDS reads issued before the current group's
        // products (reads up to two groups past the last stay inside the LDS
        // buffers and are not used).
        const int nu = min(2, max(0, (uhi - u0 - q + 3) / 4));  // rows of this wave in the chunk (wave-uniform)
        const float *ap0 = rb + (q + XM_T - 1 - mn) * rs + 4 * kk;
        const float *bp0 = lb + q * ls + (jg0 + dx0 - cl0) + 4 * kk + mn;
        const float *ap1 = ap0 + 4 * rs, *bp1 = bp0 + 4 * ls;
        auto ld = [&](const float *ap, const float *bp, int g, xm_v4f &av, float (&bv)[4]) {
            av = *reinterpret_cast<const xm_v4f *>(ap + 16 * g);
#pragma unroll
            for (int t = 0; t < 4; ++t)
                bv[t] = bp[16 * g + t];
        };
        auto mm = [&](xm_v4f (&ac)[4], const xm_v4f &av, const float (&bv)[4]) {
#pragma unroll
            for (int t = 0; t < 4; ++t)
                ac[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[t], bv[t], ac[t], 0, 0, 0);
        };
        if (nu == 2) {
            xm_v4f x0, x1, y0, y1;  // A of rows 0 and 1, groups g (x) and g + 1 (y)
            float bx0[4], bx1[4], by0[4], by1[4];
            ld(ap0, bp0, 0, x0, bx0);
            ld(ap1, bp1, 0, x1, bx1);
            int g = 0;
            for (; g + 2 <= ng; g += 2) {
                ld(ap0, bp0, g + 1, y0, by0);
                ld(ap1, bp1, g + 1, y1, by1);
                mm(acc, x0, bx0);
                mm(acc2, x1, bx1);
                ld(ap0, bp0, g + 2, x0, bx0);
                ld(ap1, bp1, g + 2, x1, bx1);
                mm(acc, y0, by0);
                mm(acc2, y1, by1);
            }
            if (g < ng) {
                mm(acc, x0, bx0);
                mm(acc2, x1, bx1);
            }
        } else if (nu == 1) {
            xm_v4f x0, y0;
            float bx0[4], by0[4];
            ld(ap0, bp0, 0, x0, bx0);
            int g = 0;
            for (; g + 2 <= ng; g += 2) {
                ld(ap0, bp0, g + 1, y0, by0);
                mm(acc, x0, bx0);
                ld(ap0, bp0, g + 2, x0, bx0);
                mm(acc, y0, by0);
            }
            if (g < ng)
                mm(acc, x0, bx0);
        }
        if (more)
            put(buf0 + ((c + 1) & 1) * bufsz, pf);  // the other buffer: last read before the previous barrier
        __syncthreads();
    }

    // the four accumulators of each wave, then the four waves, in a fixed order
    xm_v4f sum;
#pragma unroll
    for (int v = 0; v < 4; ++v)
        sum[v] = ((acc[0][v] + acc[1][v]) + (acc[2][v] + acc[3][v])) +
                 ((acc2[0][v] + acc2[1][v]) + (acc2[2][v] + acc2[3][v]));
    *reinterpret_cast<xm_v4f *>(part + q * 256 + 4 * lane) = sum;
    __syncthreads();
    if (q == 0) {
        xm_v4f tot = *reinterpret_cast<const xm_v4f *>(part + 4 * lane);
#pragma unroll
        for (int p = 1; p < 4; ++p) {
            const xm_v4f o = *reinterpret_cast<const xm_v4f *>(part + p * 256 + 4 * lane);
            tot += o;
        }
        // lane (n = lane & 15, g = lane >> 4), register v: row shift dy0 +
        // 4g + v, column shift dx0 + n
        const int oh = 2 * h - 1, ow = 2 * w - 1;
        float *const o = a.out + (size_t)pair * oh * ow;
        const int xo = tx * XM_T + mn;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int yo = ty * XM_T + 4 * kk + v;
            if (yo < oh && xo < ow)
                o[(size_t)yo * ow + xo] = tot[v];
        }
    }
}

// LDS plan and launch shape for a call, or false when the kernel does not
// take it (cols not a multiple of 4, staging beyond the per-thread items or
// the LDS, grid beyond 2^31 workgroups).
static bool xm_plan(const XcorrArgs &a, XmArgs &xa, size_t &lds)
{
    if (a.cols % 4 != 0)
        return false;
    const int ngmax = (a.cols + 30) / 16;
    xa.x = a;
    xa.ty = (2 * a.rows - 1 + XM_T - 1) / XM_T;
    xa.tx = (2 * a.cols - 1 + XM_T - 1) / XM_T;
    xa.ls = 16 * ngmax + 20;  // 16 ng + 15 columns from a start rounded down to a multiple of 4
    xa.rs = 16 * ngmax + 4;   // rows 4 (mod 16) floats apart: 16 rows' 16-byte reads meet distinct banks
    xa.nl4 = XM_UC * xa.ls / 4;
    xa.nr4 = XM_RR * xa.rs / 4;
    if (xa.nl4 + xa.nr4 > XM_PF * XM_THREADS)
        return false;
    lds = (size_t)(2 * (XM_UC * xa.ls + XM_RR * xa.rs) + 4 * 256) * sizeof(float);
    const int64_t grid = (int64_t)xa.ty * xa.tx * a.n_left * a.n_right;
    return lds <= 160 * 1024 && grid <= INT32_MAX;
}

bool xcorr_mfma_supported(const XcorrArgs &a)
{
    XmArgs xa;
    size_t lds;
    return xm_plan(a, xa, lds);
}

hipError_t xcorr_launch_mfma(const XcorrArgs &a, hipStream_t s)
{
    XmArgs xa;
    size_t lds;
    if (!xm_plan(a, xa, lds))
        return hipErrorInvalidValue;
    static std::atomic<uint64_t> lds_allowed{0};
    const hipError_t e = allow_lds_once(&xcorr_mfma_kernel, lds_allowed);
    if (e != hipSuccess)
        return e;
    const int64_t grid = (int64_t)xa.ty * xa.tx * a.n_left * a.n_right;
    hipLaunchKernelGGL(xcorr_mfma_kernel, dim3((unsigned)grid), dim3(XM_THREADS), lds, s, xa);
    return hipGetLastError();
}

} // namespace xc
