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

// SumT and SumTSq over the whole template (every wave computes them; cheap).
__device__ __forceinline__ void template_sums(const uint32_t *__restrict__ tw, int nwords,
                                              uint32_t &sum_t, uint32_t &sum_tsq)
{
    const int lane = threadIdx.x & 63;
    uint32_t a = 0, b = 0;
    for (int k = lane; k < nwords; k += 64) {
        const uint32_t w = tw[k];
        a = dot4u(w, 0x01010101u, a);
        b = dot4u(w, w, b);
    }
    sum_t = wave_sum_u32(a);
    sum_tsq = wave_sum_u32(b);
}

// Exact epilogue for one window; writes whichever outputs are requested.
__device__ __forceinline__ void ncc_store(const NccArgs &a, size_t o, uint32_t si, uint32_t sq, uint32_t st,
                                          int64_t n, int64_t sum_t, int64_t vt)
{
    if (a.sum_i) a.sum_i[o] = si;
    if (a.sum_isq) a.sum_isq[o] = sq;
    if (a.sum_it) a.sum_it[o] = st;
    if (a.coef) {
        const int64_t num = n * (int64_t)st - (int64_t)si * sum_t;
        const int64_t vi = n * (int64_t)sq - (int64_t)si * (int64_t)si;
        double c = 0.0;
        if (vi != 0 && vt != 0)
            c = (double)num / sqrt((double)vi * (double)vt);
        a.coef[o] = (float)c;
    }
}

} // namespace xc
