// ncc_pad.hip -- the zero-padded image copy behind the same and full output
// modes of the u8 normalized correlation (ncc_u8_run_mode in capi.hip): the
// valid-mode kernels then run on the copy, so outside pixels read as 0 and
// count among a window's pixels, the zero-padding convention of
// scipy.signal.correlate2d.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "kernels.h"
#include "ncc_common.h"

namespace xc {

// Zero-padded copy for the same and full output modes (see ncc_pad_image).
// A thread writes 16 bytes of one row.  Their image bytes start at column
// s = c0 - pad_left, so all four output words take the same byte shift
// (s mod 4) of five consecutive aligned image words; the five loads are
// unconditional (addresses clamped into the row) and the bytes outside the
// image, or past out_w, are cleared afterwards.
__global__ __launch_bounds__(256) void ncc_pad_kernel(const uint8_t *__restrict__ image, int width, int height,
                                                      int pitch, uint8_t *__restrict__ out, int out_w, int out_pitch,
                                                      int pad_top, int pad_left, int row0, int nrows)
{
    const int chunks = out_pitch / 16;
    const int t = blockIdx.x * 256 + threadIdx.x;  // nrows * chunks <= 2^30: see ncc_pad_image
    if (t >= nrows * chunks)
        return;
    const int rl = t / chunks;
    const int c0 = (t - rl * chunks) * 16;
    const int r = row0 + rl;
    const int sr = r - pad_top;
    const bool row_ok = sr >= 0 && sr < height;
    const uint32_t *row = reinterpret_cast<const uint32_t *>(image + (size_t)(row_ok ? sr : 0) * pitch);
    const int nwords = pitch / 4;
    const int s = c0 - pad_left;   // image column of the chunk's first byte (may be negative)
    const int sh = s & 3;          // two's complement: the remainder in 0..3
    const int w0 = (s - sh) / 4;   // exact: floor(s / 4)
    uint32_t v[5];
#pragma unroll
    for (int k = 0; k < 5; ++k) {
        const int wi = w0 + k;
        v[k] = row[wi < 0 ? 0 : (wi < nwords ? wi : nwords - 1)];
    }
    // bytes [lo, hi) of the 16 are image pixels inside the output row
    const int lo = max(0, -s);
    const int hi = row_ok ? min(16, min(width - s, out_w - c0)) : 0;
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        // keep byte b of word q when lo <= 4q + b < hi
        const int a = min(max(lo - 4 * q, 0), 4), e = min(max(hi - 4 * q, 0), 4);
        const uint32_t keep = e > a ? ((e == 4 ? 0xFFFFFFFFu : (1u << (8 * e)) - 1u) & ~((1u << (8 * a)) - 1u)) : 0u;
        w[q] = shift_bytes(v[q + 1], v[q], (uint32_t)sh) & keep;
    }
    *reinterpret_cast<uint4 *>(out + (size_t)r * out_pitch + c0) = make_uint4(w[0], w[1], w[2], w[3]);
}

hipError_t ncc_pad_image(const uint8_t *image, int width, int height, int pitch, uint8_t *out, int out_w, int out_h,
                         int out_pitch, int pad_top, int pad_left, hipStream_t s)
{
    // 32-bit thread indexing: rows go in launches of at most 2^30 threads (one
    // launch for any padded image under 16 GiB)
    const int chunks = out_pitch / 16;
    const int step = (int)std::max<int64_t>(1, ((int64_t)1 << 30) / chunks);
    for (int64_t row0 = 0; row0 < out_h; row0 += step) {
        const int nrows = (int)std::min<int64_t>(step, out_h - row0);
        const int64_t n = (int64_t)nrows * chunks;
        hipLaunchKernelGGL(ncc_pad_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, image, width, height,
                           pitch, out, out_w, out_pitch, pad_top, pad_left, (int)row0, nrows);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

} // namespace xc
