/*
 * oracle.c -- plain, slow, obviously correct CPU reference for direct
 * sliding-window 2D correlation.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this library.  The GPU library shares no code,
 * header or table with it, and neither one includes or links the other.
 *
 * Two forms are computed, each written out from its definition with no
 * blocking, fusion or reordering:
 *
 *  1. u8 normalized correlation (template matching).
 *     Source: "The CUDA Handbook", chapter 15 "Image Processing: Normalized
 *     Correlation", section 15.5 "Instruction-Level Parallelism and DP4A":
 *     per output window the kernel keeps the three unsigned accumulators
 *     SumI (sum of window pixels), SumISq (sum of their squares) and SumIT
 *     (sum of pixel times template pixel), over unsigned 8-bit pixels.
 *     The page does not print the coefficient; the reading used here is
 *     Pearson's correlation of the N (window, template) pixel pairs, computed
 *     exactly from those sums and the template sums SumT, SumTSq:
 *        num = N*SumIT - SumI*SumT
 *        vI  = N*SumISq - SumI^2,  vT = N*SumTSq - SumT^2      (exact int64)
 *        coef = 0 if vI == 0 or vT == 0, else
 *               (float) RNE( (double)num / sqrt((double)vI * (double)vT) ).
 *     Output domain: "valid" placements only; out[y][x] is the window whose
 *     top-left pixel is image[y][x].
 *
 *  2. fp32 full 2D cross-correlation over every shift at which the two
 *     matrices overlap.  Source: JPDC 2023 artifact README "Efficient
 *     GPU-accelerated Parallel Cross-correlation" (the overview of
 *     ccn_shuffle / warp_shuffle_impl, where each thread computes one
 *     overlap, and of the one-to-one / one-to-many / multi-matrix-both
 *     groupings).  The page does not print the formula; the reading is
 *        out[l][r][y][x] = sum over the overlap of L_l[i+dy][j+dx] * R_r[i][j]
 *     with dy = y - (rows-1), dx = x - (cols-1), which is
 *     scipy.signal.correlate2d(L, R, 'full').  Products of two fp32 values are
 *     exact in fp64 and the sum is accumulated in fp64.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_ARG (-1)
#define ORACLE_ERR_U32 (-2) /* a window sum does not fit in 32 bits */

static void set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* SumT and SumTSq: plain sums over every template pixel. */
static void template_sums(const uint8_t *tmpl, int tw, int th, uint64_t *st, uint64_t *stsq)
{
    uint64_t a = 0, b = 0;
    for (int j = 0; j < th; ++j)
        for (int i = 0; i < tw; ++i) {
            uint64_t t = tmpl[(size_t)j * tw + i];
            a += t;
            b += t * t;
        }
    *st = a;
    *stsq = b;
}

/* One window: the three sums by brute force, then Pearson's coefficient. */
static int one_window(const uint8_t *image, int pitch, const uint8_t *tmpl, int tw, int th,
                      int y, int x, uint64_t sum_t, uint64_t sum_tsq,
                      uint32_t *o_si, uint32_t *o_sq, uint32_t *o_st, float *o_coef, double *o_c64)
{
    uint64_t si = 0, sq = 0, st = 0;
    for (int j = 0; j < th; ++j) {
        const uint8_t *row = image + (size_t)(y + j) * pitch + x;
        const uint8_t *trow = tmpl + (size_t)j * tw;
        for (int i = 0; i < tw; ++i) {
            uint64_t p = row[i];
            uint64_t t = trow[i];
            si += p;
            sq += p * p;
            st += p * t;
        }
    }
    int bad = (si > 0xFFFFFFFFull) || (sq > 0xFFFFFFFFull) || (st > 0xFFFFFFFFull);
    int64_t n = (int64_t)tw * th;
    int64_t num = n * (int64_t)st - (int64_t)si * (int64_t)sum_t;
    int64_t vi = n * (int64_t)sq - (int64_t)si * (int64_t)si;
    int64_t vt = n * (int64_t)sum_tsq - (int64_t)sum_t * (int64_t)sum_t;
    double c = 0.0;
    if (vi != 0 && vt != 0)
        c = (double)num / sqrt((double)vi * (double)vt);
    if (o_si) *o_si = (uint32_t)si;
    if (o_sq) *o_sq = (uint32_t)sq;
    if (o_st) *o_st = (uint32_t)st;
    if (o_coef) *o_coef = (float)c;
    if (o_c64) *o_c64 = c;
    return bad;
}

/*
 * Output rows [y_begin, y_end) of the valid-mode result.  Every output array
 * is dense row-major with (y_end - y_begin) rows of (width - t_width + 1)
 * entries; any output pointer may be NULL.  coef64 receives the fp64 value
 * before the final rounding to fp32.
 */
int oracle_ncc_u8_rows(const uint8_t *image, int width, int height, int pitch,
                       const uint8_t *tmpl, int t_width, int t_height,
                       int y_begin, int y_end,
                       uint32_t *sum_i, uint32_t *sum_isq, uint32_t *sum_it,
                       float *coef, double *coef64, int nthreads)
{
    if (!image || !tmpl || width <= 0 || height <= 0 || t_width <= 0 || t_height <= 0 ||
        t_width > width || t_height > height || pitch < width)
        return ORACLE_ERR_ARG;
    int out_h = height - t_height + 1;
    int out_w = width - t_width + 1;
    if (y_begin < 0 || y_end > out_h || y_begin > y_end)
        return ORACLE_ERR_ARG;
    uint64_t sum_t, sum_tsq;
    template_sums(tmpl, t_width, t_height, &sum_t, &sum_tsq);
    set_threads(nthreads);
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int y = y_begin; y < y_end; ++y) {
        size_t base = (size_t)(y - y_begin) * out_w;
        for (int x = 0; x < out_w; ++x) {
            size_t o = base + x;
            bad |= one_window(image, pitch, tmpl, t_width, t_height, y, x, sum_t, sum_tsq,
                              sum_i ? sum_i + o : NULL, sum_isq ? sum_isq + o : NULL,
                              sum_it ? sum_it + o : NULL, coef ? coef + o : NULL,
                              coef64 ? coef64 + o : NULL);
        }
    }
    return bad ? ORACLE_ERR_U32 : ORACLE_OK;
}

/* Selected windows (ys[k], xs[k]), one by one; output k goes to slot k. */
int oracle_ncc_u8_points(const uint8_t *image, int width, int height, int pitch,
                         const uint8_t *tmpl, int t_width, int t_height,
                         const int32_t *ys, const int32_t *xs, int64_t n,
                         uint32_t *sum_i, uint32_t *sum_isq, uint32_t *sum_it,
                         float *coef, double *coef64, int nthreads)
{
    if (!image || !tmpl || !ys || !xs || n < 0 || t_width > width || t_height > height || pitch < width)
        return ORACLE_ERR_ARG;
    int out_h = height - t_height + 1;
    int out_w = width - t_width + 1;
    for (int64_t k = 0; k < n; ++k)
        if (ys[k] < 0 || ys[k] >= out_h || xs[k] < 0 || xs[k] >= out_w)
            return ORACLE_ERR_ARG;
    uint64_t sum_t, sum_tsq;
    template_sums(tmpl, t_width, t_height, &sum_t, &sum_tsq);
    set_threads(nthreads);
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 16) reduction(| : bad)
    for (int64_t k = 0; k < n; ++k)
        bad |= one_window(image, pitch, tmpl, t_width, t_height, ys[k], xs[k], sum_t, sum_tsq,
                          sum_i ? sum_i + k : NULL, sum_isq ? sum_isq + k : NULL,
                          sum_it ? sum_it + k : NULL, coef ? coef + k : NULL,
                          coef64 ? coef64 + k : NULL);
    return bad ? ORACLE_ERR_U32 : ORACLE_OK;
}

/*
 * Best match over a coefficient map of n entries (row-major): the index of
 * the first entry holding the largest value, and that value.  A plain scan.
 * The pages stop at the coefficient; finding its maximum is the usual last
 * step of template matching, and "first in row-major order" is the reading
 * taken for ties.
 */
int oracle_ncc_peak(const float *coef, int64_t n, int64_t *idx, float *val)
{
    if (!coef || n <= 0 || !idx || !val)
        return ORACLE_ERR_ARG;
    int64_t best = 0;
    for (int64_t k = 1; k < n; ++k)
        if (coef[k] > coef[best])
            best = k;
    *idx = best;
    *val = coef[best];
    return ORACLE_OK;
}

/* One output of one pair: the overlap sum in fp64, plus the sum of |l*r|. */
static void one_shift(const float *L, const float *R, int rows, int cols, int dy, int dx,
                      double *o_val, double *o_abs)
{
    int i0 = dy < 0 ? -dy : 0;
    int i1 = dy > 0 ? rows - dy : rows;
    int j0 = dx < 0 ? -dx : 0;
    int j1 = dx > 0 ? cols - dx : cols;
    double s = 0.0, a = 0.0;
    for (int i = i0; i < i1; ++i) {
        const float *lrow = L + (size_t)(i + dy) * cols + dx;
        const float *rrow = R + (size_t)i * cols;
        for (int j = j0; j < j1; ++j) {
            double p = (double)lrow[j] * (double)rrow[j];
            s += p;
            a += fabs(p);
        }
    }
    *o_val = s;
    if (o_abs) *o_abs = a;
}

/*
 * Every pair (l, r), every shift: out[((l*n_right + r)*(2*rows-1) + y)*(2*cols-1) + x].
 * abs_out (may be NULL) receives sum |L*R| over the same overlap.
 */
int oracle_xcorr_f32(const float *left, int n_left, const float *right, int n_right,
                     int rows, int cols, double *out, double *abs_out, int nthreads)
{
    if (!left || !right || !out || n_left <= 0 || n_right <= 0 || rows <= 0 || cols <= 0)
        return ORACLE_ERR_ARG;
    int oh = 2 * rows - 1, ow = 2 * cols - 1;
    size_t mat = (size_t)rows * cols;
    int64_t tasks = (int64_t)n_left * n_right * oh;
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < tasks; ++t) {
        int y = (int)(t % oh);
        int64_t pair = t / oh;
        int l = (int)(pair / n_right), r = (int)(pair % n_right);
        const float *L = left + (size_t)l * mat;
        const float *R = right + (size_t)r * mat;
        size_t base = ((size_t)pair * oh + y) * ow;
        for (int x = 0; x < ow; ++x)
            one_shift(L, R, rows, cols, y - (rows - 1), x - (cols - 1), out + base + x,
                      abs_out ? abs_out + base + x : NULL);
    }
    return ORACLE_OK;
}

/* Selected outputs by flat index into the [n_left][n_right][2rows-1][2cols-1] array. */
int oracle_xcorr_f32_points(const float *left, int n_left, const float *right, int n_right,
                            int rows, int cols, const int64_t *flat, int64_t n,
                            double *out, double *abs_out, int nthreads)
{
    if (!left || !right || !out || !flat || n < 0 || n_left <= 0 || n_right <= 0 || rows <= 0 || cols <= 0)
        return ORACLE_ERR_ARG;
    int64_t oh = 2 * rows - 1, ow = 2 * cols - 1;
    int64_t total = (int64_t)n_left * n_right * oh * ow;
    for (int64_t k = 0; k < n; ++k)
        if (flat[k] < 0 || flat[k] >= total)
            return ORACLE_ERR_ARG;
    size_t mat = (size_t)rows * cols;
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t k = 0; k < n; ++k) {
        int64_t f = flat[k];
        int x = (int)(f % ow);
        int y = (int)((f / ow) % oh);
        int64_t pair = f / (ow * oh);
        int l = (int)(pair / n_right), r = (int)(pair % n_right);
        one_shift(left + (size_t)l * mat, right + (size_t)r * mat, rows, cols,
                  y - (rows - 1), x - (cols - 1), out + k, abs_out ? abs_out + k : NULL);
    }
    return ORACLE_OK;
}
