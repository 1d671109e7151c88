// capi.hip -- the library's C ABI (declared in include/xcorr.h): argument
// validation on the host, kernel selection, launch on the caller's stream and
// mapping of HIP errors to status codes.  No exception crosses this boundary.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "kernels.h"
#include "xcorr.h"

// Device scratch of ncc_u8_run_mode_noalloc: the padded image lives here
// instead of in a caller-owned workspace.  Each GPU the library runs on holds
// its own copy (XC_NCC_MODE_SCRATCH_BYTES) until the process ends; calls on
// one GPU share it, so overlapping calls on one GPU race.  Host code never
// names the array directly (on the host its name is only a stand-in for the
// symbol): it uses the device address hipGetSymbolAddress returns, kept per
// device.
static __device__ __align__(256) uint8_t scratch[XC_NCC_MODE_SCRATCH_BYTES];

namespace {

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? XC_OK : XC_ERR_HIP; }

// Host-side validation shared by both NCC entry points; fills `a` on success.
int ncc_validate(const uint8_t *image, int width, int height, int pitch_bytes, const uint8_t *tmpl,
                 int t_width, int t_height, uint32_t *sum_i, uint32_t *sum_isq, uint32_t *sum_it,
                 float *coef, bool need_map, xc::NccArgs &a)
{
    if (!image || !tmpl)
        return XC_ERR_NULL;
    if (need_map && !sum_i && !sum_isq && !sum_it && !coef)
        return XC_ERR_NULL;
    if (width <= 0 || height <= 0 || t_width <= 0 || t_height <= 0 || pitch_bytes <= 0)
        return XC_ERR_SHAPE;
    if (t_width > width || t_height > height || pitch_bytes < width)
        return XC_ERR_SHAPE;
    if ((int64_t)t_width * t_height > XC_NCC_MAX_TEMPLATE_PIXELS)
        return XC_ERR_OVERFLOW;
    const int64_t out_w = width - t_width + 1, out_h = height - t_height + 1;
    if (out_w * out_h > INT32_MAX || (int64_t)height * pitch_bytes > ((int64_t)1 << 40))
        return XC_ERR_OVERFLOW;
    if (!aligned(image, 16) || pitch_bytes % 16 != 0)
        return XC_ERR_ALIGN;
    if ((sum_i && !aligned(sum_i, 4)) || (sum_isq && !aligned(sum_isq, 4)) || (sum_it && !aligned(sum_it, 4)) ||
        (coef && !aligned(coef, 4)))
        return XC_ERR_ALIGN;
    a.image = image;
    a.width = width;
    a.height = height;
    a.pitch = pitch_bytes;
    a.tmpl = tmpl;
    a.t_width = t_width;
    a.t_height = t_height;
    a.sum_i = sum_i;
    a.sum_isq = sum_isq;
    a.sum_it = sum_it;
    a.coef = coef;
    a.peak = nullptr;
    a.out_w = (int)out_w;
    a.out_h = (int)out_h;
    a.hc = a.cw = a.lds_stride = a.t_stride = 0;
    return XC_OK;
}

// Geometry of an output mode: the output size, and the zero-padded image the
// valid-mode kernels run on (the image placed at (pad_top, pad_left)).
struct NccModeGeom {
    int out_w, out_h;        // output size
    int pw, ph, ppitch;      // padded image: width, height, pitch in bytes
    int pad_top, pad_left;   // where the image sits in it
    size_t bytes;            // workspace: ph * ppitch
};

int ncc_mode_geom(int width, int height, int t_width, int t_height, int mode, NccModeGeom &g)
{
    if (mode != XC_NCC_MODE_VALID && mode != XC_NCC_MODE_SAME && mode != XC_NCC_MODE_FULL)
        return XC_ERR_VARIANT;
    if (width <= 0 || height <= 0 || t_width <= 0 || t_height <= 0)
        return XC_ERR_SHAPE;
    if ((int64_t)t_width * t_height > XC_NCC_MAX_TEMPLATE_PIXELS)
        return XC_ERR_OVERFLOW;
    int64_t ow, oh, pl, pt;
    if (mode == XC_NCC_MODE_VALID) {
        if (t_width > width || t_height > height)
            return XC_ERR_SHAPE;
        ow = width - t_width + 1, oh = height - t_height + 1, pl = pt = 0;
    } else if (mode == XC_NCC_MODE_SAME) {
        ow = width, oh = height, pl = (t_width - 1) / 2, pt = (t_height - 1) / 2;
    } else {
        ow = (int64_t)width + t_width - 1, oh = (int64_t)height + t_height - 1, pl = t_width - 1, pt = t_height - 1;
    }
    const int64_t pw = ow + t_width - 1, ph = oh + t_height - 1, pp = (pw + 15) / 16 * 16;
    if (ow * oh > INT32_MAX || pp > INT32_MAX || ph > INT32_MAX || ph * pp > ((int64_t)1 << 40))
        return XC_ERR_OVERFLOW;
    g.out_w = (int)ow;
    g.out_h = (int)oh;
    g.pw = (int)pw;
    g.ph = (int)ph;
    g.ppitch = (int)pp;
    g.pad_top = (int)pt;
    g.pad_left = (int)pl;
    g.bytes = mode == XC_NCC_MODE_VALID ? 0 : (size_t)(ph * pp);
    return XC_OK;
}

int xcorr_validate(const float *left, int n_left, const float *right, int n_right, int rows, int cols,
                   float *out, xc::XcorrArgs &a)
{
    if (!left || !right || !out)
        return XC_ERR_NULL;
    if (n_left <= 0 || n_right <= 0 || rows <= 0 || cols <= 0)
        return XC_ERR_SHAPE;
    const int64_t per_pair = (int64_t)(2 * (int64_t)rows - 1) * (2 * (int64_t)cols - 1);
    if (per_pair > INT32_MAX || (int64_t)rows * cols > INT32_MAX)
        return XC_ERR_OVERFLOW;
    if ((int64_t)n_left * n_right > ((int64_t)1 << 40) / per_pair)
        return XC_ERR_OVERFLOW;
    if (!aligned(left, 16) || !aligned(right, 16) || !aligned(out, 4))
        return XC_ERR_ALIGN;
    a.left = left;
    a.right = right;
    a.out = out;
    a.n_left = n_left;
    a.n_right = n_right;
    a.rows = rows;
    a.cols = cols;
    return XC_OK;
}

// The kernel XC_NCC_AUTO runs for validated arguments (XC_NCC_MFMA,
// XC_NCC_DOT4_C1 or XC_NCC_DOT4_ILP), from the shapes and the current
// device's compute-unit count only.
//
// The matrix-core recast costs a nearly fixed time per output tile,
// the packed-byte kernel a time that grows with the template; the
// recast wins from 512 template pixels at any image size, from about
// 96 pixels once there are 400K outputs to spread its fixed cost
// over, and at any template size from about 1M outputs (measured on
// MI355X, packed-byte / recast time: 1920x1080 with 4x4 1.45, 8x8
// 1.59, 16x16 2.39, 32x32 5.1; 1024x1024 with 4x4 1.11, 8x8 1.31;
// 1280x720 with 4x4 0.93, 8x8 1.02, 10x10 1.37; 768x768 with 8x8
// 0.94, 10x10 1.40; 512x512 with 16x16 1.00, 24x24 1.65; 256x256 with
// 16x16 0.93, 24x24 1.55).
//
// Below that, on small images, the packed-byte kernel drops from
// 256 x 16 output tiles to one-wave 256 x 1 ones, each a long chain.
// When its 256 x 16 grid would be smaller than the chip, the
// one-output-per-thread dot4 kernel (64 x 4 tiles, many more
// workgroups) is faster for word-aligned templates of up to 64 packed
// words while its grid times the template words stays within about
// 192 per CU; failing that, the matrix cores for templates over 16
// words.  Widths that are not a multiple of 4 cost both dot4 kernels
// a masked word per row: there the one-per-thread kernel takes
// templates of up to 16 words within 96 per CU, and the matrix cores
// the rest.  Measured on MI355X, HIP-event medians in us, packed-byte
// / this rule's choice: 256x256 with 7x7 7.7 / 6.6, 8x8 5.3 / 4.2,
// 12x12 7.2 / 5.2, 16x16 7.7 / 6.7; 320x240 with 11x11 10.8 / 8.7,
// 16x16 8.2 / 7.0; 640x480 with 4x4 7.1 / 5.2, 7x7 9.3 / 8.7, 8x8
// 9.1 / 6.3, 12x12 12.3 / 8.1, 16x16 15.2 / 9.0; 800x600 with 5x5
// 10.3 / 9.4, 8x8 9.8 / 8.0; 1280x720 with 4x4 10.5 / 9.3, 7x7 15.0
// / 11.5; 400x300 with 10x10 10.2 / 9.0; 512x512 with 16x16 8.7 /
// 8.8.
//
// Since the one-per-thread kernel splits the template rows over several
// waves on small grids, it is taken first there (ahead of the matrix cores'
// template-size rule) for word-aligned templates of up to 200 words while
// its grid times the words stays within about 180 per CU (145 when the grid
// holds more workgroups than CUs, so the rows split over two waves, not
// four), where it beats the matrix cores (one-per-thread / matrix cores,
// us: 256x256 with 20x20
// 6.1 / 8.5, 24x24 7.0 / 8.7, 28x28 8.1 / 8.9; 256x192 with 24x24 6.8 /
// 8.7; 300x300 with 20x20 7.8 / 8.6; 320x240 with 20x20 7.7 / 8.6), and
// not beyond (320x240 with 24x24 9.4 / 8.7, 300x300 with 24x24 9.5 / 8.9,
// 400x400 with 20x20 11.0 /
// 8.8, 512x256 with 24x24 9.9 / 8.8, 256x256 with 40x40 12.2 / 9.9).
int ncc_auto_variant(const xc::NccArgs &a)
{
    const int64_t npix = (int64_t)a.t_width * a.t_height;
    const int64_t nout = (int64_t)a.out_w * a.out_h;
    const bool mfma_ok = xc::ncc_mfma_supported(a);
    const int64_t cus = xc::device_cu_count();
    const int64_t n_ilp = (int64_t)((a.out_w + 255) / 256) * ((a.out_h + 15) / 16);
    const int64_t words = (int64_t)((a.t_width + 3) / 4) * a.t_height;
    const int64_t n_c1 = (int64_t)((a.out_w + 63) / 64) * ((a.out_h + 3) / 4);
    const bool whole = a.t_width % 4 == 0;
    if (n_ilp < cus && whole && words <= 200 && n_c1 * words <= (n_c1 <= cus ? 180 : 145) * cus)
        return XC_NCC_DOT4_C1;
    if ((npix >= 512 || (npix >= 96 && nout >= 400000) || nout >= 1000000) && mfma_ok)
        return XC_NCC_MFMA;
    if (n_ilp < cus) {
        if (words <= (whole ? 64 : 16) && n_c1 * words <= (whole ? 192 : 96) * cus)
            return XC_NCC_DOT4_C1;
        if ((words > 16 || !whole) && mfma_ok)
            return XC_NCC_MFMA;
    }
    return XC_NCC_DOT4_ILP;
}

// Launch the chosen variant on validated arguments.
int ncc_dispatch(const xc::NccArgs &a, int variant, hipStream_t s)
{
    switch (variant) {
    case XC_NCC_AUTO:
        return ncc_dispatch(a, ncc_auto_variant(a), s);
    case XC_NCC_DOT4_ILP:
        return hip_status(xc::ncc_launch_ilp(a, s));
    case XC_NCC_DOT4_C1:
        return hip_status(xc::ncc_launch_c1(a, true, s));
    case XC_NCC_SCALAR_C1:
        return hip_status(xc::ncc_launch_c1(a, false, s));
    case XC_NCC_MFMA:
        return hip_status(xc::ncc_launch_mfma(a, s));
    case XC_NCC_DOT4_ILP_Q1:
        return hip_status(xc::ncc_launch_ilp(a, s, 1));
    case XC_NCC_DOT4_ILP_Q2:
        return hip_status(xc::ncc_launch_ilp(a, s, 2));
    case XC_NCC_DOT4_ILP_Q4:
        return hip_status(xc::ncc_launch_ilp(a, s, 4));
    case XC_NCC_MFMA_W4:
        return hip_status(xc::ncc_launch_mfma(a, s, 4));
    case XC_NCC_MFMA_W2:
        return hip_status(xc::ncc_launch_mfma(a, s, 2));
    case XC_NCC_DOT4_COLS1:
        return hip_status(xc::ncc_launch_cols(a, 1, s));
    case XC_NCC_DOT4_COLS2:
        return hip_status(xc::ncc_launch_cols(a, 2, s));
    case XC_NCC_DOT4_COLS4:
        return hip_status(xc::ncc_launch_cols(a, 4, s));
    case XC_NCC_DOT4_COLS8:
        return hip_status(xc::ncc_launch_cols(a, 8, s));
    case XC_NCC_MFMA32:
        return hip_status(xc::ncc_launch_mfma32(a, s));
    default:
        return XC_ERR_VARIANT;
    }
}

// Variant check done before anything is enqueued.
int ncc_variant_ok(const xc::NccArgs &a, int variant)
{
    if (variant < XC_NCC_AUTO || variant > XC_NCC_MFMA32)
        return XC_ERR_VARIANT;
    if (variant == XC_NCC_MFMA32 && !xc::ncc_mfma32_supported(a))
        return XC_ERR_SHAPE;
    if ((variant == XC_NCC_MFMA || variant == XC_NCC_MFMA_W4) && !xc::ncc_mfma_supported(a, 4))
        return XC_ERR_SHAPE;
    if (variant == XC_NCC_MFMA_W2 && !xc::ncc_mfma_supported(a, 2))
        return XC_ERR_SHAPE;
    return XC_OK;
}

// Same or full mode over a padded-image buffer of `padded_bytes` bytes at
// the device address `padded` (16-byte aligned, or NULL): validation, then
// the zero-padded copy and the valid-mode variant on it, both on `stream`.
// `padded` may be NULL only to ask for the validation of everything else
// (the caller reports the missing buffer).
int ncc_mode_run(const uint8_t *image, int width, int height, int pitch_bytes, const uint8_t *tmpl, int t_width,
                 int t_height, const NccModeGeom &g, uint8_t *padded, size_t padded_bytes, uint32_t *sum_i,
                 uint32_t *sum_isq, uint32_t *sum_it, float *coef, int variant, void *stream)
{
    if (!image || !tmpl || !padded)
        return XC_ERR_NULL;
    if (pitch_bytes < width || (int64_t)height * pitch_bytes > ((int64_t)1 << 40))
        return XC_ERR_SHAPE;
    if (!aligned(image, 16) || pitch_bytes % 16 != 0 || !aligned(padded, 16))
        return XC_ERR_ALIGN;
    if (padded_bytes < g.bytes)
        return XC_ERR_SHAPE;
    // the valid-mode computation on the padded image
    xc::NccArgs a;
    int st = ncc_validate(padded, g.pw, g.ph, g.ppitch, tmpl, t_width, t_height, sum_i, sum_isq, sum_it, coef, true,
                          a);
    if (st != XC_OK)
        return st;
    if ((st = ncc_variant_ok(a, variant)) != XC_OK)
        return st;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if ((st = hip_status(xc::ncc_pad_image(image, width, height, pitch_bytes, padded, g.pw, g.ph, g.ppitch, g.pad_top,
                                           g.pad_left, s))) != XC_OK)
        return st;
    return ncc_dispatch(a, variant, s);
}

// Device address of `scratch` on the current device, looked up on the first
// call on each device (ids below 64; higher ids look it up every time), or
// NULL if the lookup fails.  Thread-safe: concurrent first calls store the
// same address.
uint8_t *scratch_ptr()
{
    static std::atomic<uint8_t *> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return nullptr;
    if (dev < 64) {
        uint8_t *p = cached[dev].load(std::memory_order_acquire);
        if (p)
            return p;
    }
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
        return nullptr;
    if (dev < 64)
        cached[dev].store(static_cast<uint8_t *>(p), std::memory_order_release);
    return static_cast<uint8_t *>(p);
}

} // namespace

extern "C" {

int ncc_u8_run_variant(const uint8_t *image, int width, int height, int pitch_bytes, const uint8_t *tmpl,
                       int t_width, int t_height, uint32_t *sum_i, uint32_t *sum_isq, uint32_t *sum_it,
                       float *coef, int variant, void *stream)
{
    xc::NccArgs a;
    int st = ncc_validate(image, width, height, pitch_bytes, tmpl, t_width, t_height, sum_i, sum_isq, sum_it,
                          coef, true, a);
    if (st != XC_OK)
        return st;
    if ((st = ncc_variant_ok(a, variant)) != XC_OK)
        return st;
    return ncc_dispatch(a, variant, reinterpret_cast<hipStream_t>(stream));
}

int ncc_u8_peak(const uint8_t *image, int width, int height, int pitch_bytes, const uint8_t *tmpl, int t_width,
                int t_height, uint32_t *sum_i, uint32_t *sum_isq, uint32_t *sum_it, float *coef,
                xc_ncc_peak *peak, int variant, void *stream)
{
    if (!peak)
        return XC_ERR_NULL;
    xc::NccArgs a;
    int st = ncc_validate(image, width, height, pitch_bytes, tmpl, t_width, t_height, sum_i, sum_isq, sum_it,
                          coef, false, a);
    if (st != XC_OK)
        return st;
    if (!aligned(peak, 8))
        return XC_ERR_ALIGN;
    if ((st = ncc_variant_ok(a, variant)) != XC_OK)
        return st;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    static_assert(sizeof(peak->key) == sizeof(unsigned long long), "64-bit key");
    a.peak = reinterpret_cast<unsigned long long *>(&peak->key);
    if ((st = hip_status(xc::ncc_peak_init(peak, s))) != XC_OK)
        return st;
    if ((st = ncc_dispatch(a, variant, s)) != XC_OK)
        return st;
    return hip_status(xc::ncc_peak_finish(peak, a.out_w, s));
}

int ncc_u8_mode_workspace(int width, int height, int t_width, int t_height, int mode, size_t *bytes)
{
    if (!bytes)
        return XC_ERR_NULL;
    NccModeGeom g;
    const int st = ncc_mode_geom(width, height, t_width, t_height, mode, g);
    if (st != XC_OK)
        return st;
    *bytes = g.bytes;
    return XC_OK;
}


int ncc_u8_run_mode(const uint8_t *image, int width, int height, int pitch_bytes, const uint8_t *tmpl, int t_width,
                    int t_height, int mode, void *workspace, size_t workspace_bytes, uint32_t *sum_i,
                    uint32_t *sum_isq, uint32_t *sum_it, float *coef, int variant, void *stream)
{
    if (mode == XC_NCC_MODE_VALID)
        return ncc_u8_run_variant(image, width, height, pitch_bytes, tmpl, t_width, t_height, sum_i, sum_isq, sum_it,
                                  coef, variant, stream);
    NccModeGeom g;
    const int st = ncc_mode_geom(width, height, t_width, t_height, mode, g);
    if (st != XC_OK)
        return st;
    return ncc_mode_run(image, width, height, pitch_bytes, tmpl, t_width, t_height, g,
                        static_cast<uint8_t *>(workspace), workspace_bytes, sum_i, sum_isq, sum_it, coef, variant,
                        stream);
}

int ncc_u8_run_mode_noalloc(const uint8_t *image, int width, int height, int pitch_bytes, const uint8_t *tmpl,
                            int t_width, int t_height, int mode, uint32_t *sum_i, uint32_t *sum_isq, uint32_t *sum_it,
                            float *coef, int variant, void *stream)
{
    if (mode == XC_NCC_MODE_VALID)
        return ncc_u8_run_variant(image, width, height, pitch_bytes, tmpl, t_width, t_height, sum_i, sum_isq, sum_it,
                                  coef, variant, stream);
    NccModeGeom g;
    const int st = ncc_mode_geom(width, height, t_width, t_height, mode, g);
    if (st != XC_OK)
        return st;
    if (g.bytes > (size_t)XC_NCC_MODE_SCRATCH_BYTES)
        return XC_ERR_SCRATCH;
    uint8_t *const p = scratch_ptr();
    if (!p)
        return XC_ERR_HIP;
    return ncc_mode_run(image, width, height, pitch_bytes, tmpl, t_width, t_height, g, p,
                        (size_t)XC_NCC_MODE_SCRATCH_BYTES, sum_i, sum_isq, sum_it, coef, variant, stream);
}

int ncc_u8_run(const uint8_t *image, int width, int height, int pitch_bytes, const uint8_t *tmpl, int t_width,
               int t_height, uint32_t *sum_i, uint32_t *sum_isq, uint32_t *sum_it, float *coef, void *stream)
{
    return ncc_u8_run_variant(image, width, height, pitch_bytes, tmpl, t_width, t_height, sum_i, sum_isq, sum_it,
                              coef, XC_NCC_AUTO, stream);
}

int ncc_u8_auto_variant(int width, int height, int t_width, int t_height, int *variant)
{
    if (!variant)
        return XC_ERR_NULL;
    // the shape checks of ncc_u8_run, with stand-in addresses (never read)
    static const uint8_t probe[16] __attribute__((aligned(16))) = {};
    uint32_t sum;
    xc::NccArgs a;
    const int64_t pitch = ((int64_t)width + 15) / 16 * 16;
    if (pitch > INT32_MAX)
        return XC_ERR_OVERFLOW;
    const int st = ncc_validate(probe, width, height, (int)pitch, probe, t_width, t_height, &sum, nullptr, nullptr,
                                nullptr, true, a);
    if (st != XC_OK)
        return st;
    *variant = ncc_auto_variant(a);
    return XC_OK;
}

int xcorr_f32_run_algo(const float *left, int n_left, const float *right, int n_right, int rows, int cols,
                       float *out, int algo, void *stream)
{
    xc::XcorrArgs a;
    const int st = xcorr_validate(left, n_left, right, n_right, rows, cols, out, a);
    if (st != XC_OK)
        return st;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    switch (algo) {
    case XC_XCORR_AUTO:
        if (xc::xcorr_blockdiag_supported(a))
            return hip_status(xc::xcorr_launch_blockdiag(a, s));
        if (xc::xcorr_small_supported(a))
            return hip_status(xc::xcorr_launch_small(a, s));
        return hip_status(xc::xcorr_launch_overlap(a, s));
    case XC_XCORR_OVERLAP:
        return hip_status(xc::xcorr_launch_overlap(a, s));
    case XC_XCORR_WAVE:
        return hip_status(xc::xcorr_launch_wave(a, s));
    case XC_XCORR_SMALL:
        if (!xc::xcorr_small_supported(a))
            return XC_ERR_SHAPE;
        return hip_status(xc::xcorr_launch_small(a, s));
    case XC_XCORR_BLOCKDIAG:
        if (!xc::xcorr_blockdiag_supported(a))
            return XC_ERR_SHAPE;
        return hip_status(xc::xcorr_launch_blockdiag(a, s));
    case XC_XCORR_MFMA:
        if (!xc::xcorr_mfma_supported(a))
            return XC_ERR_SHAPE;
        return hip_status(xc::xcorr_launch_mfma(a, s));
    default:
        return XC_ERR_VARIANT;
    }
}

int xcorr_f32_run(const float *left, int n_left, const float *right, int n_right, int rows, int cols, float *out,
                  void *stream)
{
    return xcorr_f32_run_algo(left, n_left, right, n_right, rows, cols, out, XC_XCORR_AUTO, stream);
}

const char *xc_status_str(int status)
{
    switch (status) {
    case XC_OK: return "success";
    case XC_ERR_NULL: return "a required pointer is NULL, or no output was requested";
    case XC_ERR_SHAPE: return "a size is not positive, the template is larger than the image, or the shape is not supported by the chosen algorithm";
    case XC_ERR_TEMPLATE_WIDTH: return "reserved (template widths are no longer restricted)";
    case XC_ERR_OVERFLOW: return "template area over 66,051 pixels (32-bit sums could wrap) or an index range exceeded";
    case XC_ERR_ALIGN: return "a base pointer or the row pitch is not suitably aligned (16 bytes for images and matrices)";
    case XC_ERR_HIP: return "HIP launch or runtime error (or no device)";
    case XC_ERR_VARIANT: return "unknown variant or algorithm selector";
    case XC_ERR_SCRATCH: return "the call needs a larger padded image than the library's static device scratch holds (XC_NCC_MODE_SCRATCH_BYTES)";
    default: return "unknown status";
    }
}

} // extern "C"
