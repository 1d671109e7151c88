// ncc_common.h -- device helpers shared by the u8 normalized-correlation
// kernels (ncc_u8.hip, ncc_u8_mfma.hip): packed-byte primitives, tile staging,
// template sums and the exact epilogue.  Internal; not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace xc {

__device__ __forceinline__ uint32_t dot4u(uint32_t a, uint32_t b, uint32_t c)
{
    return __builtin_amdgcn_udot4(a, b, c, false);
}

__device__ __forceinline__ uint32_t shift_bytes(uint32_t hi, uint32_t lo, uint32_t s)
{
    // ({hi, lo} >> 8*s)[31:0]: bytes s..s+3 of the little-endian pair lo, hi.
    return __builtin_amdgcn_alignbyte(hi, lo, s);
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        v += (uint32_t)__shfl_xor((int)v, m, 64);
    return v;
}

// Copy image rows [gy0, gy0 + nrows) x 16-byte chunks [gx0, gx0 + 16*nchunks)
// into LDS (row stride `stride` words).  Rows at or past `height` and chunks
// at or past `pitch` are zero-filled, so no load leaves the image allocation.
__device__ __forceinline__ void stage_tile(const uint8_t *__restrict__ image, int height, int pitch,
                                           int gy0, int gx0, int nrows, int nchunks,
                                           uint32_t *lds, int stride)
{
    const int total = nrows * nchunks;
    for (int t = threadIdx.x; t < total; t += blockDim.x) {
        const int r = t / nchunks;
        const int b = t - r * nchunks;
        const int gy = gy0 + r;
        const int gx = gx0 + 16 * b;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (gy < height && gx < pitch)
            v = *reinterpret_cast<const uint4 *>(image + (size_t)gy * pitch + gx);
        *reinterpret_cast<uint4 *>(lds + r * stride + 4 * b) = v;
    }
}

// Packed template words: word k of template row j holds bytes 4k .. 4k+3 of
// the row (little-endian), zero beyond t_width.  Rows of a width that is a
// multiple of 4 are whole words (one load from a 4-byte aligned base);
// otherwise the word is gathered byte by byte.
__device__ __forceinline__ uint32_t tmpl_row_word(const uint8_t *__restrict__ row, int t_width, bool word_rows,
                                                  int k)
{
    if (word_rows)
        return reinterpret_cast<const uint32_t *>(row)[k];
    uint32_t w = 0u;
#pragma unroll
    for (int b = 0; b < 4; ++b)
        if (4 * k + b < t_width)
            w |= (uint32_t)row[4 * k + b] << (8 * b);
    return w;
}

__device__ __forceinline__ uint32_t tmpl_word(const uint8_t *__restrict__ tmpl, int t_width, bool word_rows, int j,
                                              int k)
{
    return tmpl_row_word(tmpl + (size_t)j * t_width, t_width, word_rows, k);
}

__device__ __forceinline__ bool tmpl_word_rows(const uint8_t *tmpl, int t_width)
{
    return (t_width & 3) == 0 && (reinterpret_cast<uintptr_t>(tmpl) & 3) == 0;
}

// Mask of the bytes of the last packed word of a template row that are
// template pixels (all four when t_width is a multiple of 4).
__host__ __device__ __forceinline__ uint32_t tail_mask(int t_width)
{
    return (t_width & 3) == 0 ? 0xFFFFFFFFu : 0xFFFFFFFFu >> (8 * (4 - (t_width & 3)));
}

// SumT and SumTSq over the whole template (every wave computes them; cheap).
__device__ __forceinline__ void template_sums(const uint8_t *__restrict__ tmpl, int t_width, int t_height,
                                              uint32_t &sum_t, uint32_t &sum_tsq)
{
    const int lane = threadIdx.x & 63;
    uint32_t a = 0, b = 0;
    if (tmpl_word_rows(tmpl, t_width)) {
        const uint32_t *tw = reinterpret_cast<const uint32_t *>(tmpl);
        const int nwords = (t_width >> 2) * t_height;
        for (int k = lane; k < nwords; k += 64) {
            const uint32_t w = tw[k];
            a = dot4u(w, 0x01010101u, a);
            b = dot4u(w, w, b);
        }
    } else {
        const int nw = (t_width + 3) >> 2;
        for (int j = 0; j < t_height; ++j)
            for (int k = lane; k < nw; k += 64) {
                const uint32_t w = tmpl_word(tmpl, t_width, false, j, k);
                a = dot4u(w, 0x01010101u, a);
                b = dot4u(w, w, b);
            }
    }
    sum_t = wave_sum_u32(a);
    sum_tsq = wave_sum_u32(b);
}

// Best-match key of one window: the coefficient's bits mapped to an unsigned
// order (negative values flipped, positive ones given the top bit) above the
// complement of the row-major output index, so the largest key is the largest
// coefficient and, among equal ones, the first window in row-major order.
// Every real key is above 0, which marks "none".
__device__ __forceinline__ unsigned long long peak_key(float coef, uint32_t idx)
{
    const uint32_t b = __float_as_uint(coef);
    const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return ((unsigned long long)ord << 32) | (0xFFFFFFFFu - idx);
}

// Largest key of the wave, then one 64-bit atomic maximum per wave (the
// maximum does not depend on the order the waves arrive in).  Every lane of
// the wave must call it.
__device__ __forceinline__ void peak_commit(unsigned long long *peak, unsigned long long v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, m, 64);
        const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), m, 64);
        const unsigned long long o = ((unsigned long long)hi << 32) | lo;
        v = o > v ? o : v;
    }
    if ((threadIdx.x & 63) == 0 && v != 0ull)
        atomicMax(peak, v);
}

// Largest key of the workgroup, then one 64-bit atomic maximum for it (one
// per workgroup instead of one per wave: the atomics on the single key
// serialize).  Every thread of the workgroup must call it.  `slots` is LDS
// for one key per wave; it may overlay any LDS the workgroup does not read
// after the call (a barrier separates the earlier reads from its writes).
__device__ __forceinline__ void peak_commit_wg(unsigned long long *peak, unsigned long long v,
                                               unsigned long long *slots)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, m, 64);
        const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), m, 64);
        const unsigned long long o = ((unsigned long long)hi << 32) | lo;
        v = o > v ? o : v;
    }
    __syncthreads();
    if ((threadIdx.x & 63) == 0)
        slots[threadIdx.x >> 6] = v;
    __syncthreads();
    if (threadIdx.x == 0) {
        const int nwaves = (int)(blockDim.x >> 6);
        for (int w = 1; w < nwaves; ++w)
            v = slots[w] > v ? slots[w] : v;
        if (v != 0ull)
            atomicMax(peak, v);
    }
}

// The coefficient num / sqrt(p), p = vI * vT (all exact integers in fp64,
// p already rounded once), rounded to fp32: bit-identical to the IEEE fp64
// square root and division followed by one rounding to fp32, at about half
// their cost.  The reciprocal square root comes from the hardware estimate
// (relative error at most 2^-23: 2^29 ulp of fp64) and one Newton step
// (quadratic convergence: relative error below 2^-45), so c = num * y is
// within |c| * 2^-44 of the IEEE quotient d (itself within |c| * 2^-52 of the
// real one).  With m = |c| * 2^-42, c - m <= d <= c + m even after rounding
// both ends to fp64, and rounding to fp32 is monotonic, so when both ends
// round to the same fp32 value d does too.  They differ only when an fp32
// rounding boundary lies within about |c| * 2^-42 of c (a few windows in a
// million); the IEEE expression is evaluated then.  c = 0 gives m = 0.
__device__ __forceinline__ float ncc_coef_f32(double num, double p)
{
    double y = __builtin_amdgcn_rsq(p);
    const double t = p * y;
    const double e = fma(-t, y, 1.0);
    y = fma(0.5 * y, e, y);
    const double c = num * y;
    const double m = fabs(c) * 0x1p-42;
    const float lo = (float)(c - m);
    if (lo == (float)(c + m))
        return lo;
    return (float)(num / sqrt(p));
}

// Exact epilogue for one window; writes whichever outputs are requested and
// folds the window into `best` when the best match is requested.
__device__ __forceinline__ void ncc_store(const NccArgs &a, size_t o, uint32_t si, uint32_t sq, uint32_t st,
                                          int64_t n, int64_t sum_t, int64_t vt, unsigned long long &best)
{
    if (a.sum_i) a.sum_i[o] = si;
    if (a.sum_isq) a.sum_isq[o] = sq;
    if (a.sum_it) a.sum_it[o] = st;
    if (a.coef || a.peak) {
        const int64_t num = n * (int64_t)st - (int64_t)si * sum_t;
        const int64_t vi = n * (int64_t)sq - (int64_t)si * (int64_t)si;
        float c = 0.0f;
        if (vi != 0 && vt != 0)
            c = ncc_coef_f32((double)num, (double)vi * (double)vt);
        if (a.coef) a.coef[o] = c;
        if (a.peak) {
            const unsigned long long k = peak_key(c, (uint32_t)o);
            best = k > best ? k : best;
        }
    }
}

} // namespace xc
