// kernels.h -- internal interface between the C ABI (capi.hip) and the gfx950
// kernels of this library.  Not installed; the public interface is
// include/xcorr.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace xc {

// Allow `kernel` up to 160 KiB of dynamic LDS (gfx950's per-CU size) on the
// current device, once per device: `done` holds one bit per device id below
// 64 (higher ids make the call every time).  Thread-safe: concurrent first
// calls may both make the (idempotent) attribute call; the bit is set after
// a successful one.
template <typename K>
inline hipError_t allow_lds_once(K kernel, std::atomic<uint64_t> &done)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    const uint64_t bit = dev < 64 ? 1ull << dev : 0ull;
    if (bit && (done.load(std::memory_order_acquire) & bit))
        return hipSuccess;
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                            160 * 1024);
    if (e == hipSuccess && bit)
        done.fetch_or(bit, std::memory_order_release);
    return e;
}

// Compute units of the current device, queried once per device (256, the
// gfx950 count, if the query fails).
inline int device_cu_count()
{
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n > 0)
        return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        return 256;
    cached[dev].store(n, std::memory_order_relaxed);
    return n;
}

// Arguments of every u8 normalized-correlation kernel (validated on the host).
struct NccArgs {
    const uint8_t *image;
    int width, height, pitch;
    const uint8_t *tmpl;
    int t_width, t_height;
    uint32_t *sum_i, *sum_isq, *sum_it;
    float *coef;
    unsigned long long *peak;  // best-match key (see peak_key), or NULL
    int out_w, out_h;
    // chunking of the template, chosen by the launcher
    int hc;          // template rows per chunk
    int cw;          // template words (4 bytes) per chunk
    int lds_stride;  // LDS words per staged image row
    int t_stride;    // LDS words per staged template row
    // packed-byte (DOT4_ILP) tiles, set by its launcher: ncol_full x
    // nrow_tiles ordinary tiles, then (tail_g > 1) the last column tile's
    // narrow remainder as tail tiles whose lanes form tail_g groups of
    // tail_nl lanes, each group taking its own rows
    int ncol_full, nrow_tiles;
    int tail_g, tail_nl;
    uint32_t tail_m;  // ceil(2^16 / tail_nl): lane / tail_nl as a multiply
};

// force_q = 0: the tile picked for the shape; 1, 2 or 4: Q rows per lane
// (and as many row waves), no template-row split.
hipError_t ncc_launch_ilp(NccArgs a, hipStream_t s, int force_q = 0);
hipError_t ncc_launch_c1(NccArgs a, bool dot4, hipStream_t s);
// Column-ILP ablation: cols = 1, 2, 4 or 8 output columns per lane on
// 256 x 4 output tiles.
hipError_t ncc_launch_cols(NccArgs a, int cols, hipStream_t s);
// SumIT on the i8 matrix cores; takes template rows up to 256 bytes.
// mw: matrix-core waves per workgroup (4: 256-column tiles, 2: 128-column
// tiles, t_width <= 64 only); 0 lets the launcher pick from the grid.
hipError_t ncc_launch_mfma(NccArgs a, hipStream_t s, int mw = 0);
bool ncc_mfma_supported(const NccArgs &a, int mw = 0);
// SumIT on the 32x32x32 i8 matrix cores with the template as the Toeplitz
// operand; t_width <= 65 and a tile plan within 160 KiB of LDS.
hipError_t ncc_launch_mfma32(NccArgs a, hipStream_t s);
bool ncc_mfma32_supported(const NccArgs &a);
// Best-match search around a correlation launch: set the key to 0 before it,
// decode the key into (y, x, coefficient) after it.  `peak` points to an
// xc_ncc_peak (include/xcorr.h).
hipError_t ncc_peak_init(void *peak, hipStream_t s);
// Zero-padded copy of an image for the same and full output modes:
// out[r][c] = image[r - pad_top][c - pad_left] where that pixel exists, else
// 0, for r < out_h and c < out_pitch (out_pitch a multiple of 16).
hipError_t ncc_pad_image(const uint8_t *image, int width, int height, int pitch, uint8_t *out, int out_w, int out_h,
                         int out_pitch, int pad_top, int pad_left, hipStream_t s);
hipError_t ncc_peak_finish(void *peak, int out_w, hipStream_t s);

// Arguments of the fp32 cross-correlation kernels (validated on the host).
struct XcorrArgs {
    const float *left;
    const float *right;
    float *out;
    int n_left, n_right;
    int rows, cols;
};

hipError_t xcorr_launch_overlap(const XcorrArgs &a, hipStream_t s);
hipError_t xcorr_launch_wave(const XcorrArgs &a, hipStream_t s);
// Matrices with a dimension of at most 16 (rows or cols).
hipError_t xcorr_launch_small(const XcorrArgs &a, hipStream_t s);
bool xcorr_small_supported(const XcorrArgs &a);
hipError_t xcorr_launch_blockdiag(const XcorrArgs &a, hipStream_t s);
bool xcorr_blockdiag_supported(const XcorrArgs &a);
// fp32 matrix cores (v_mfma_f32_16x16x4f32), one 16 x 16 tile of shifts per
// workgroup; cols % 4 == 0 and a staging plan within its per-thread items
// and the LDS.
hipError_t xcorr_launch_mfma(const XcorrArgs &a, hipStream_t s);
bool xcorr_mfma_supported(const XcorrArgs &a);

} // namespace xc
