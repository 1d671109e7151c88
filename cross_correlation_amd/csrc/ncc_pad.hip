// ncc_pad.hip -- the zero-padded image copy behind the same and full output
// modes of the u8 normalized correlation (ncc_u8_run_mode in capi.hip): the
// valid-mode kernels then run on the copy, so outside pixels read as 0 and
// count among a window's pixels, the zero-padding convention of
// scipy.signal.correlate2d.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"
#include "ncc_common.h"

namespace xc {

// Zero-padded copy for the same and full output modes (see ncc_pad_image).
// A thread writes 16 bytes of one row; each 4-byte word is assembled from the
// two aligned image words holding its bytes (v_alignbyte_b32), its bytes
// outside the image (or past out_w) cleared.
__global__ __launch_bounds__(256) void ncc_pad_kernel(const uint8_t *__restrict__ image, int width, int height,
                                                      int pitch, uint8_t *__restrict__ out, int out_w, int out_h,
                                                      int out_pitch, int pad_top, int pad_left)
{
    const int chunks = out_pitch / 16;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= (int64_t)out_h * chunks)
        return;
    const int r = (int)(t / chunks);
    const int c0 = (int)(t - (int64_t)r * chunks) * 16;
    const int sr = r - pad_top;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if (sr >= 0 && sr < height) {
        const uint32_t *row = reinterpret_cast<const uint32_t *>(image + (size_t)sr * pitch);
        const int nwords = pitch / 4;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int s = c0 + 4 * q - pad_left;  // image column of the word's first byte (may be negative)
            const int sh = s & 3;                 // two's complement: the remainder in 0..3
            const int sw = (s - sh) / 4;          // exact: floor(s / 4)
            const uint32_t lo = sw >= 0 && sw < nwords ? row[sw] : 0u;
            const uint32_t hi = sw + 1 >= 0 && sw + 1 < nwords ? row[sw + 1] : 0u;
            uint32_t m = 0u;
#pragma unroll
            for (int b = 0; b < 4; ++b)
                if (s + b >= 0 && s + b < width && c0 + 4 * q + b < out_w)
                    m |= 0xFFu << (8 * b);
            w[q] = shift_bytes(hi, lo, (uint32_t)sh) & m;
        }
    }
    *reinterpret_cast<uint4 *>(out + (size_t)r * out_pitch + c0) = make_uint4(w[0], w[1], w[2], w[3]);
}

hipError_t ncc_pad_image(const uint8_t *image, int width, int height, int pitch, uint8_t *out, int out_w, int out_h,
                         int out_pitch, int pad_top, int pad_left, hipStream_t s)
{
    const int64_t n = (int64_t)out_h * (out_pitch / 16);
    hipLaunchKernelGGL(ncc_pad_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, image, width, height, pitch,
                       out, out_w, out_h, out_pitch, pad_top, pad_left);
    return hipGetLastError();
}

} // namespace xc
