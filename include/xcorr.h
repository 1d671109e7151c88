/*
 * xcorr.h -- C ABI of the gfx950 (MI355X) library for direct sliding-window
 * 2D correlation.  Two forms:
 *
 *   ncc_u8_run     8-bit normalized correlation (template matching).
 *                  Defined by "The CUDA Handbook", chapter 15 "Image
 *                  Processing: Normalized Correlation", section 15.5
 *                  "Instruction-Level Parallelism and DP4A": per window the
 *                  unsigned 32-bit sums SumI (pixels), SumISq (squared pixels)
 *                  and SumIT (pixel times template pixel) over unsigned bytes,
 *                  then a correlation coefficient from those sums and the
 *                  template sums.  The page packs template rows whose width is
 *                  a multiple of four; here any width is taken (the last
 *                  packed word of a row is masked to the template's bytes).
 *
 *   xcorr_f32_run  fp32 full 2D cross-correlation over every shift at which
 *                  two matrices overlap, for one-to-one, one-to-many and
 *                  n-to-m groupings.  Defined by the JPDC 2023 artifact README
 *                  "Efficient GPU-accelerated Parallel Cross-correlation"
 *                  (overview of ccn_shuffle / warp_shuffle_impl, split-row,
 *                  grouped-overlap and the multi-matrix variants).
 *
 * Conventions shared by every entry point
 *   - Every data pointer is a DEVICE pointer (hipMalloc'd or equivalent) on
 *     the current HIP device.  `stream` is a hipStream_t passed as void*;
 *     NULL means the default stream.
 *   - The caller allocates and owns every buffer; the library allocates
 *     nothing and keeps no state between calls.  Inputs and outputs must not
 *     alias.  Calls are thread-safe.
 *   - Calls are asynchronous: work is enqueued on `stream` and the function
 *     returns.  The caller synchronizes before reading results.
 *   - Every output element is written (no pre-zeroing needed).
 *   - Results are deterministic: the same inputs give bit-identical outputs.
 *   - Arguments are validated on the host before any HIP call; on error
 *     nothing is enqueued and a negative status is returned.
 */
#ifndef XCORR_MI355X_H
#define XCORR_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define XC_OK 0
#define XC_ERR_NULL (-1)           /* a required pointer is NULL, or no output requested        */
#define XC_ERR_SHAPE (-2)          /* a size is <= 0, or the template is larger than the image */
#define XC_ERR_TEMPLATE_WIDTH (-3) /* reserved: template widths are not restricted any more     */
#define XC_ERR_OVERFLOW (-4)       /* sums could wrap 32 bits, or an index range is exceeded    */
#define XC_ERR_ALIGN (-5)          /* a base pointer or the pitch is not 16-byte aligned        */
#define XC_ERR_HIP (-6)            /* HIP launch or runtime error (including: no device)        */
#define XC_ERR_VARIANT (-7)        /* unknown variant / algorithm / output-mode selector        */
#define XC_ERR_SCRATCH (-8)        /* the call needs more than the static device scratch holds  */

/* Largest template area for which the u32 sums cannot wrap: N * 255^2 < 2^32. */
#define XC_NCC_MAX_TEMPLATE_PIXELS 66051

/*
 * ncc_u8_run -- valid-mode 8-bit normalized correlation.
 *
 * image   [height][pitch_bytes] u8, row-major; pixel (y, x) at image[y*pitch + x]
 *         for x < width.  Base and pitch_bytes must be multiples of 16.
 * tmpl    [t_height][t_width] u8, dense row-major, any alignment.
 *         Requires 0 < t_width <= width, 0 < t_height <= height and
 *         t_width * t_height <= 66,051 (any width; rows are packed into
 *         4-byte words, the last one masked to the row's bytes).
 * Outputs dense row-major [out_h][out_w], out_h = height - t_height + 1,
 *         out_w = width - t_width + 1; entry (y, x) is the window whose
 *         top-left pixel is image (y, x):
 *   sum_i   u32  SumI   = sum of the window's pixels             (may be NULL)
 *   sum_isq u32  SumISq = sum of their squares                   (may be NULL)
 *   sum_it  u32  SumIT  = sum of pixel * template pixel          (may be NULL)
 *   coef    f32  Pearson correlation of the N = t_width*t_height (pixel,
 *                template) pairs: with SumT, SumTSq the template sums,
 *                num = N*SumIT - SumI*SumT, vI = N*SumISq - SumI^2,
 *                vT = N*SumTSq - SumT^2 (exact 64-bit integers),
 *                coef = 0 if vI == 0 or vT == 0, else
 *                (float) round-to-nearest( (double)num / sqrt((double)vI*(double)vT) )
 *                                                            (may be NULL)
 *         At least one output must be non-NULL; each must be 4-byte aligned.
 * The template sums SumT and SumTSq are computed by the library on every call.
 */
int ncc_u8_run(const uint8_t *image, int width, int height, int pitch_bytes,
               const uint8_t *tmpl, int t_width, int t_height,
               uint32_t *sum_i, uint32_t *sum_isq, uint32_t *sum_it, float *coef,
               void *stream);

/*
 * ncc_u8_run_variant -- the same computation through a chosen kernel variant,
 * for ablation studies.  Every variant returns identical outputs.
 *   XC_NCC_AUTO          the library's choice (what ncc_u8_run uses).  On
 *                        images too small for the DOT4_ILP kernel's 256 x 16
 *                        output tiles to fill the GPU's compute units, first
 *                        XC_NCC_DOT4_C1 for templates whose width is a
 *                        multiple of 4, of at most 200 packed words, whose
 *                        workgroups (64 x 4 outputs) times template words are
 *                        at most 180 per compute unit (145 when there are
 *                        more workgroups than units).  Then XC_NCC_MFMA where
 *                        it takes the template and the template has at least
 *                        512 pixels, or at least 96 pixels with at least
 *                        400,000 outputs, or there are at least 1,000,000
 *                        outputs.  Then, on those small images again,
 *                        XC_NCC_DOT4_C1 for templates of at most 64 packed
 *                        words and at most 192 per unit (widths not a
 *                        multiple of 4: 16 words, 96 per unit), failing that
 *                        XC_NCC_MFMA for templates over 16 words or of a
 *                        width not a multiple of 4.  Else XC_NCC_DOT4_ILP.
 *                        ncc_u8_auto_variant reports the choice.
 *   XC_NCC_DOT4_ILP      packed-byte dot products, 4 columns x several rows per lane
 *   XC_NCC_DOT4_C1       packed-byte dot products, one output per lane
 *   XC_NCC_SCALAR_C1     byte-at-a-time multiply-adds, one output per lane
 *   XC_NCC_MFMA          SumIT as a signed-byte matrix product on the matrix
 *                        cores (pixels and template biased by -128, corrected
 *                        exactly with SumI and SumT), SumI and SumISq as
 *                        separable box sums in waves of their own (which,
 *                        for templates of 48 rows or more up to 128 bytes
 *                        wide, store those two outputs while the products
 *                        run); t_width <= 256 only, else XC_ERR_SHAPE.  A
 *                        recast of the page's computation, not its DP4A
 *                        method.
 *   XC_NCC_DOT4_ILP_Q1   the ILP series of the ablation: packed-byte dot
 *   XC_NCC_DOT4_ILP_Q2   products, 4 columns x Q = 1, 2 or 4 rows per lane,
 *   XC_NCC_DOT4_ILP_Q4   each lane walking every template row itself (no split
 *                        of the template rows over waves, which
 *                        XC_NCC_DOT4_ILP adds for templates of 16 or more rows)
 *   XC_NCC_MFMA_W4       XC_NCC_MFMA with its tile width fixed: 256 output
 *   XC_NCC_MFMA_W2       columns per workgroup (4 matrix-core waves, two
 *                        workgroups per CU) or 128 (2 matrix-core waves, four
 *                        per CU; t_width <= 64 only, else XC_ERR_SHAPE).
 *                        XC_NCC_MFMA picks the width that runs the output's
 *                        tiles in fewer rounds of workgroups, and the narrow
 *                        one where wide tiles would leave compute units idle.
 *   XC_NCC_DOT4_COLS1    the column-ILP series of the ablation (the page's
 *   XC_NCC_DOT4_COLS2    two-column step): packed-byte dot products with
 *   XC_NCC_DOT4_COLS4    C = 1, 2, 4 or 8 adjacent output columns per lane
 *   XC_NCC_DOT4_COLS8    and one output row, on the same 256 x 4 output tile
 *                        per workgroup for every C, so only the independent
 *                        accumulator chains per lane (3 * C) change.  C = 2
 *                        is the page's two columns per thread.
 *   XC_NCC_MFMA32        SumIT on the 32x32x32 signed-byte matrix cores with
 *                        the operands turned round: the image rows as they
 *                        are staged (no byte shifts) against the template
 *                        row shifted by each output column (the Toeplitz
 *                        operand), 32 x 128 outputs per workgroup, template
 *                        rows split over four waves; SumI and SumISq as
 *                        sliding column sums and row prefixes in four waves
 *                        beside them.  t_width <= 65 and templates short
 *                        enough for the tile's LDS plan (350 rows at width
 *                        64), else XC_ERR_SHAPE.
 */
#define XC_NCC_AUTO 0
#define XC_NCC_DOT4_ILP 1
#define XC_NCC_DOT4_C1 2
#define XC_NCC_SCALAR_C1 3
#define XC_NCC_MFMA 4
#define XC_NCC_DOT4_ILP_Q1 5
#define XC_NCC_DOT4_ILP_Q2 6
#define XC_NCC_DOT4_ILP_Q4 7
#define XC_NCC_MFMA_W4 8
#define XC_NCC_MFMA_W2 9
#define XC_NCC_DOT4_COLS1 10
#define XC_NCC_DOT4_COLS2 11
#define XC_NCC_DOT4_COLS4 12
#define XC_NCC_DOT4_COLS8 13
#define XC_NCC_MFMA32 14
int ncc_u8_run_variant(const uint8_t *image, int width, int height, int pitch_bytes,
                       const uint8_t *tmpl, int t_width, int t_height,
                       uint32_t *sum_i, uint32_t *sum_isq, uint32_t *sum_it, float *coef,
                       int variant, void *stream);

/*
 * ncc_u8_peak -- best match: the window with the largest coefficient.
 *
 * Computes what ncc_u8_run_variant computes (the same arguments and rules; the
 * four map outputs are optional here, all of them may be NULL) and also the
 * best match over all out_h x out_w windows:
 *   peak   DEVICE pointer to one xc_ncc_peak, 8-byte aligned, caller-owned.
 *          On completion peak->y, peak->x are the top-left pixel of the window
 *          with the largest coefficient (the coefficient ncc_u8_run returns,
 *          as an fp32 value) and peak->coef is that coefficient.  Among
 *          windows with equal coefficients the first in row-major order
 *          (smallest y * out_w + x) is returned, so the result is unique and
 *          deterministic.  peak->key is the library's working value (the
 *          packed coefficient and position) and peak->reserved is 0.
 * Three launches are enqueued on `stream` (clear the key, correlate, decode);
 * the library still allocates nothing.  Concurrent calls must not share one
 * xc_ncc_peak.  Errors as ncc_u8_run_variant, plus XC_ERR_NULL for a NULL peak
 * and XC_ERR_ALIGN for a misaligned one.
 * The pages describe the correlation only; the search is the usual last step
 * of template matching, fused into the correlation's epilogue here (each wave
 * reduces its windows, then one 64-bit atomic maximum).
 */
typedef struct {
    uint64_t key;
    int32_t y, x;
    float coef;
    int32_t reserved;
} xc_ncc_peak;
int ncc_u8_peak(const uint8_t *image, int width, int height, int pitch_bytes,
                const uint8_t *tmpl, int t_width, int t_height,
                uint32_t *sum_i, uint32_t *sum_isq, uint32_t *sum_it, float *coef,
                xc_ncc_peak *peak, int variant, void *stream);

/*
 * ncc_u8_auto_variant -- which kernel XC_NCC_AUTO (ncc_u8_run) runs for a
 * valid-mode call on these shapes, written to *variant: XC_NCC_MFMA,
 * XC_NCC_DOT4_C1 or XC_NCC_DOT4_ILP.  The choice depends only on the shapes
 * and on the current device's compute-unit count (256, the MI355X count,
 * when no device can be queried); the outputs are the same whichever kernel
 * runs.  Host-only: nothing is launched.  Errors: XC_ERR_NULL if variant is
 * NULL; XC_ERR_SHAPE or XC_ERR_OVERFLOW for shapes ncc_u8_run would reject.
 * (Same and full modes run the valid-mode choice on the padded image.)
 */
int ncc_u8_auto_variant(int width, int height, int t_width, int t_height, int *variant);

/*
 * ncc_u8_run_mode -- the 8-bit normalized correlation with a choice of output
 * domain.  The pages define only the windows inside the image (valid mode);
 * same and full modes follow the zero-padding convention of
 * scipy.signal.correlate2d: pixels outside the image are 0 and count among
 * the window's N = t_width * t_height pixels, so every output is the valid-mode
 * result on the image with zero borders.
 *   XC_NCC_MODE_VALID  out_h x out_w = (height - t_height + 1) x (width - t_width + 1);
 *                      output (y, x) is the window with top-left pixel (y, x)
 *                      (what ncc_u8_run computes; no workspace)
 *   XC_NCC_MODE_SAME   out_h x out_w = height x width; window top-left
 *                      (y - (t_height - 1) / 2, x - (t_width - 1) / 2)
 *   XC_NCC_MODE_FULL   out_h x out_w = (height + t_height - 1) x (width + t_width - 1);
 *                      window top-left (y - t_height + 1, x - t_width + 1)
 * In same and full modes the template may be larger than the image.
 *
 * ncc_u8_mode_workspace stores in *bytes the workspace a mode needs for these
 * sizes (0 for valid mode), or returns the error the shape would get.
 * ncc_u8_run_mode takes the arguments of ncc_u8_run_variant plus the mode and
 * a caller-owned DEVICE workspace of at least that many bytes, 16-byte
 * aligned (NULL allowed in valid mode): a first launch copies the image into
 * it with zero borders, the chosen variant then runs on that copy, both on
 * `stream`.  Outputs are out_h x out_w dense row-major as above, with the
 * coefficient rule of ncc_u8_run.  Errors: as ncc_u8_run_variant, plus
 * XC_ERR_VARIANT for an unknown mode, XC_ERR_NULL for a missing workspace,
 * XC_ERR_ALIGN for a misaligned one and XC_ERR_SHAPE for one too small.
 * Concurrent calls must not share a workspace.
 */
#define XC_NCC_MODE_VALID 0
#define XC_NCC_MODE_SAME 1
#define XC_NCC_MODE_FULL 2
int ncc_u8_mode_workspace(int width, int height, int t_width, int t_height, int mode, size_t *bytes);
int ncc_u8_run_mode(const uint8_t *image, int width, int height, int pitch_bytes,
                    const uint8_t *tmpl, int t_width, int t_height, int mode,
                    void *workspace, size_t workspace_bytes,
                    uint32_t *sum_i, uint32_t *sum_isq, uint32_t *sum_it, float *coef,
                    int variant, void *stream);

/*
 * ncc_u8_run_mode_noalloc -- ncc_u8_run_mode for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same arguments without the workspace, the same
 * outputs.  The zero-padded image of same and full modes goes to a static
 * device buffer of XC_NCC_MODE_SCRATCH_BYTES (16 MiB) that the library holds
 * on each GPU it runs on until the process ends; the call allocates nothing
 * (no hipMalloc, no allocating library routine).  Every call on one GPU
 * shares that GPU's buffer and leaves its contents behind (the padded copy of
 * its image; each call overwrites all of the bytes it reads), so calls that
 * overlap on one GPU -- on different streams, or from several threads without
 * ordering -- race: serialize them, e.g. on one stream.  Valid mode uses no
 * buffer.  Errors: as ncc_u8_run_mode, plus XC_ERR_SCRATCH when the padded
 * image (ncc_u8_mode_workspace's byte count) exceeds XC_NCC_MODE_SCRATCH_BYTES,
 * and XC_ERR_HIP if the buffer's device address cannot be obtained.
 */
#define XC_NCC_MODE_SCRATCH_BYTES 16777216u /* 16 MiB */
int ncc_u8_run_mode_noalloc(const uint8_t *image, int width, int height, int pitch_bytes,
                            const uint8_t *tmpl, int t_width, int t_height, int mode,
                            uint32_t *sum_i, uint32_t *sum_isq, uint32_t *sum_it, float *coef,
                            int variant, void *stream);

/*
 * xcorr_f32_run -- fp32 full 2D cross-correlation of every (left, right) pair.
 *
 * left   [n_left][rows][cols]  f32, contiguous, 16-byte aligned base.
 * right  [n_right][rows][cols] f32, contiguous, 16-byte aligned base.
 * out    [n_left][n_right][2*rows-1][2*cols-1] f32, contiguous, 4-byte aligned;
 *        pair (l, r) is slice l*n_right + r (left-major), and
 *        out[l][r][y][x] = sum over the overlap of left[l][i+dy][j+dx] * right[r][i][j]
 *        with dy = y - (rows-1), dx = x - (cols-1) (the convention of
 *        scipy.signal.correlate2d(L, R, 'full')).
 * One-to-one is n_left = n_right = 1; one-to-many is n_left = 1.
 * Requires rows, cols, n_left, n_right > 0 and each pair's output
 * (2*rows-1)*(2*cols-1) below 2^31 elements.
 * Accuracy: each output is within 1e-5 * sum|l*r| of the exact value (fp32
 * accumulation in a fixed, input-independent order).
 */
int xcorr_f32_run(const float *left, int n_left, const float *right, int n_right,
                  int rows, int cols, float *out, void *stream);

/*
 * xcorr_f32_run_algo -- the same result through a chosen algorithm.
 *   XC_XCORR_AUTO        the library's choice (what xcorr_f32_run uses)
 *   XC_XCORR_OVERLAP     one thread per output shift, no data reuse (the
 *                        overlap-wise baseline)
 *   XC_XCORR_BLOCKDIAG   register-blocked kernel: 4x4 row blocks along block
 *                        diagonals, a sliding column window per lane
 *   XC_XCORR_WAVE        one 64-lane wave per output shift: the lanes split
 *                        the overlap's elements and their partial sums are
 *                        added across the wave in a fixed order (the JPDC
 *                        README's warp-per-overlap variant, for large
 *                        overlaps; no data reuse between shifts)
 *   XC_XCORR_SMALL       matrices with rows <= 16 or cols <= 16.  When both
 *                        are: a group of 1 to 8 lanes owns one pair and one
 *                        row shift and computes the whole output row, each
 *                        lane loading its share of the rows of both matrices
 *                        before any product; a wave's output rows are stored
 *                        as one contiguous span.  Otherwise a group of 1 to
 *                        64 lanes (more for longer loops) owns one pair, one
 *                        shift along the long dimension and 8 shifts along
 *                        the short one, each lane keeping two lines (rows or
 *                        columns) in registers, each value serving up to 8
 *                        products.  Either way the group adds its partial
 *                        sums in a fixed order; XC_ERR_SHAPE for larger
 *                        matrices.  XC_XCORR_AUTO takes BLOCKDIAG from 13
 *                        rows, this below.
 *   XC_XCORR_MFMA        the fp32 matrix cores (v_mfma_f32_16x16x4f32): for
 *                        each left row u, the contribution to all shifts is a
 *                        matrix product of the right rows u - dy and the left
 *                        row u shifted by dx; one 16 x 16 tile of shifts per
 *                        workgroup, its left rows split over four waves and
 *                        added in a fixed order.  An ablation point (slower
 *                        than BLOCKDIAG on the groupings measured).
 *                        XC_ERR_SHAPE unless cols is a multiple of 4 and the
 *                        tile's staging fits (cols up to about 340).
 */
#define XC_XCORR_AUTO 0
#define XC_XCORR_OVERLAP 1
#define XC_XCORR_BLOCKDIAG 2
#define XC_XCORR_WAVE 3
#define XC_XCORR_SMALL 4
#define XC_XCORR_MFMA 5
int xcorr_f32_run_algo(const float *left, int n_left, const float *right, int n_right,
                       int rows, int cols, float *out, int algo, void *stream);

/* Human-readable text for a status code (static storage, never NULL). */
const char *xc_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* XCORR_MI355X_H */
