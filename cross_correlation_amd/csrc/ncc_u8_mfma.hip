// ncc_u8_mfma.hip -- u8 normalized correlation with SumIT on the i8 matrix
// cores (v_mfma_i32_16x16x64_i8) and SumI / SumISq as exact separable box sums.
//
// Same outputs as the packed-byte kernels (ncc_u8.hip) for the computation of
// "The CUDA Handbook", ch. 15 "Image Processing: Normalized Correlation": the
// unsigned window sums SumI, SumISq, SumIT and Pearson's coefficient.  The
// page computes all three sums with DP4A; this variant recasts the one sum
// that pairs image and template bytes as a matrix product:
//
//   * Bias: I' = I - 128 and T' = T - 128 are signed bytes (an XOR with 0x80),
//     and  SumIT = sum I'T' + 128*SumI + 128*SumT - 16384*N  exactly (mod 2^32,
//     and the true value is below 2^32), so the signed i8 MFMA serves.
//   * Product: for one workgroup tile of 16 output rows n and output columns
//     x = x0 + 4m + t (m = 0..15, t = 0..3 per wave) and each image row r of
//     the tile,  D_t[m][n] += sum_k A_t[m][k] * B[k][n]  with
//       A_t[m][k] = I'[r][x0 + 4m + t + k]     (the window bytes: byte-shifted
//                                              image words, v_alignbyte_b32)
//       B[k][n]   = T'[r - n][k]               (template row r - n, zero when
//                                              that row does not exist)
//     k runs over 64-byte blocks of the template row.  Summed over r this is
//     the window sum over every template row (B is the template placed
//     Toeplitz-wise along the output rows); a fraction 15/(t_height + 15) of
//     the products is against zero rows.
//   * SumI and SumISq: column sums over the template height for the 16 output
//     rows (sliding down the tile, unsigned), then inclusive prefix sums along
//     each row, so a window sum is the difference of two prefix entries; all
//     unsigned 32-bit, exact because every final sum is below 2^32.
//   * The epilogue is the packed-byte kernels' exact one (64-bit integers,
//     fp64 divide and square root, one fp32 rounding).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"
#include "ncc_common.h"

namespace xc {

typedef int mf_v4i __attribute__((ext_vector_type(4)));

constexpr int MF_TY = 16;          // output rows per workgroup (MFMA N)
constexpr int MF_TX = 256;         // output columns per workgroup (4 waves x 64)
constexpr int MF_MAX_NKB = 4;      // template rows up to 256 bytes
constexpr int MF_MAX_HC = 256;     // template rows per chunk (16-bit column sums)
constexpr int MF_ACC_STRIDE = 257; // i32 words per output row of the SumIT staging

// LDS plan of one workgroup (host and device agree through these helpers).
struct MfPlan {
    int nkb;      // 64-byte blocks per template row
    int hc;       // template rows per chunk
    int sw;       // image LDS words per row
    int tsb;      // template LDS bytes per row
    int nwd;      // image words covered by the box sums
    int vs;       // u32 per row of the column-sum arrays (odd: spreads banks)
    int img_words;
    size_t bytes;
};

__host__ __device__ inline MfPlan mf_plan(int t_width, int hc)
{
    MfPlan p;
    p.nkb = (t_width + 63) / 64;
    p.hc = hc;
    p.sw = 64 + 16 * p.nkb + 4;
    p.tsb = 64 * p.nkb + 16;
    p.nwd = 64 + t_width / 4;
    p.vs = 4 * p.nwd + 1;
    int img = (MF_TY - 1 + hc) * p.sw;
    if (img < MF_TY * MF_ACC_STRIDE) img = MF_TY * MF_ACC_STRIDE;  // reused for SumIT staging
    p.img_words = img;
    p.bytes = (size_t)2 * MF_TY * p.vs * 4 + (size_t)img * 4 + (size_t)(hc + 1) * p.tsb;
    return p;
}

// Image rows [gy0, gy0 + nrows) x words [0, 4*nchunks) from column gx0, biased
// to signed bytes; rows at or past `height` and chunks at or past `pitch` are
// zero-filled, so no load leaves the image allocation.
__device__ __forceinline__ void mf_stage_image(const uint8_t *__restrict__ image, int height, int pitch, int gy0,
                                               int gx0, int nrows, int nchunks, uint32_t *lds, int stride)
{
    const int total = nrows * nchunks;
    for (int i = threadIdx.x; i < total; i += blockDim.x) {
        const int r = i / nchunks;
        const int b = i - r * nchunks;
        const int gy = gy0 + r;
        const int gx = gx0 + 16 * b;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (gy < height && gx < pitch)
            v = *reinterpret_cast<const uint4 *>(image + (size_t)gy * pitch + gx);
        v.x ^= 0x80808080u;
        v.y ^= 0x80808080u;
        v.z ^= 0x80808080u;
        v.w ^= 0x80808080u;
        *reinterpret_cast<uint4 *>(lds + r * stride + 4 * b) = v;
    }
}

// Template rows [j0, j0 + hcur) biased to signed bytes, zero beyond t_width up
// to the 64-byte block; row hcur is all zero (the rows that do not exist).
__device__ __forceinline__ void mf_stage_template(const uint8_t *__restrict__ tmpl, int t_width, int j0, int hcur,
                                                  int kw, uint8_t *tpl, int tsb)
{
    const int wpr = kw / 4;  // words per staged row
    const int twords = t_width / 4;
    const int total = (hcur + 1) * wpr;
    for (int i = threadIdx.x; i < total; i += blockDim.x) {
        const int r = i / wpr;
        const int k = i - r * wpr;
        uint32_t v = 0u;
        if (r < hcur && k < twords)
            v = reinterpret_cast<const uint32_t *>(tmpl + (size_t)(j0 + r) * t_width)[k] ^ 0x80808080u;
        *reinterpret_cast<uint32_t *>(tpl + r * tsb + 4 * k) = v;
    }
}

// Column sums of one template-row chunk, added into V1 (pixels) and V2
// (squares): V[n][c] += sum_{j in chunk} I[n + j][c] for the 16 output rows.
// Thread (part p, word wd): the chunk's rows are split into np parts; each
// part slides down the 16 output rows (add the row entering, remove the row
// leaving) with pixel sums in two 16-bit lanes per register.
__device__ __forceinline__ void mf_box_chunk(const uint32_t *img, int sw, int hcur, int nwd, uint32_t *V1,
                                             uint32_t *V2, int vs)
{
    const int np = blockDim.x / nwd;
    const int p = threadIdx.x / nwd;
    const int wd = threadIdx.x - p * nwd;
    if (p >= np)
        return;
    const int jlo = p * hcur / np, jhi = (p + 1) * hcur / np;
    if (jlo >= jhi)
        return;
    const uint32_t *col = img + wd;
    uint32_t lo = 0u, hi = 0u;     // bytes 0,2 and 1,3 of the word, 16 bits each
    uint32_t qa[4] = {0u, 0u, 0u, 0u}, qr[4] = {0u, 0u, 0u, 0u};  // squares added / removed
    auto add = [&](uint32_t w) {
        w ^= 0x80808080u;
        lo += w & 0x00FF00FFu;
        hi += (w >> 8) & 0x00FF00FFu;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            qa[k] = dot4u(w & (0xFFu << (8 * k)), w, qa[k]);
    };
    auto remove = [&](uint32_t w) {
        w ^= 0x80808080u;
        lo -= w & 0x00FF00FFu;
        hi -= (w >> 8) & 0x00FF00FFu;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            qr[k] = dot4u(w & (0xFFu << (8 * k)), w, qr[k]);
    };
    auto emit = [&](int n) {
        uint32_t *v1 = V1 + n * vs + 4 * wd;
        uint32_t *v2 = V2 + n * vs + 4 * wd;
        atomicAdd(v1 + 0, lo & 0xFFFFu);
        atomicAdd(v1 + 1, hi & 0xFFFFu);
        atomicAdd(v1 + 2, lo >> 16);
        atomicAdd(v1 + 3, hi >> 16);
#pragma unroll
        for (int k = 0; k < 4; ++k)
            atomicAdd(v2 + k, qa[k] - qr[k]);
    };
    for (int j = jlo; j < jhi; ++j)
        add(col[j * sw]);
    emit(0);
    for (int n = 1; n < MF_TY; ++n) {
        add(col[(n - 1 + jhi) * sw]);
        remove(col[(n - 1 + jlo) * sw]);
        emit(n);
    }
}

// The MFMA walk of one chunk for one wave: every image row of the chunk's tile
// against the template rows it meets, NKB 64-byte blocks per row.
template <int NKB>
__device__ __forceinline__ void mf_mfma_chunk(const uint32_t *img, int sw, const uint8_t *tpl, int tsb, int hcur,
                                              mf_v4i (&acc)[4])
{
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int m = lane & 15, g = lane >> 4;
    // A: output column x0 + 64*wave + 4m + t reads image words from 16*wave + m
    // (+ 4g for its 16 bytes of the 64-byte block); B: template row rr - n.
    const uint32_t *ibase = img + 16 * wave + m + 4 * g;
    const uint8_t *tbase = tpl + 16 * g;
    const int n = m;  // B column = output row
    const int nrows = MF_TY - 1 + hcur;
    for (int rr = 0; rr < nrows; ++rr) {
        const int jr = rr - n;
        const uint8_t *trow = tbase + (jr >= 0 && jr < hcur ? jr : hcur) * tsb;
        const uint32_t *irow = ibase + rr * sw;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            uint32_t w[5];
#pragma unroll
            for (int k = 0; k < 5; ++k)
                w[k] = irow[16 * kb + k];
            const mf_v4i b = *reinterpret_cast<const mf_v4i *>(trow + 64 * kb);
            mf_v4i a0, a1, a2, a3;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                a0[k] = (int)w[k];
                a1[k] = (int)shift_bytes(w[k + 1], w[k], 1);
                a2[k] = (int)shift_bytes(w[k + 1], w[k], 2);
                a3[k] = (int)shift_bytes(w[k + 1], w[k], 3);
            }
            acc[0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b, acc[0], 0, 0, 0);
            acc[1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b, acc[1], 0, 0, 0);
            acc[2] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a2, b, acc[2], 0, 0, 0);
            acc[3] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a3, b, acc[3], 0, 0, 0);
        }
    }
}

// In-place inclusive prefix sums along each of the 32 rows (16 of V1, 16 of
// V2) over `ncols` columns: 8 threads per row, each a contiguous segment.
__device__ __forceinline__ void mf_row_prefix(uint32_t *V, int vs, int ncols)
{
    const int row = threadIdx.x >> 3;  // 0..31
    const int seg = threadIdx.x & 7;
    const int len = (ncols + 7) / 8;
    const int c0 = seg * len, c1 = min(ncols, c0 + len);
    uint32_t *r = V + row * vs;
    uint32_t s = 0u;
    for (int c = c0; c < c1; ++c) {
        s += r[c];
        r[c] = s;
    }
    __syncthreads();
    uint32_t off = 0u;
    for (int k = 0; k < seg; ++k) {
        const int e = min(ncols, (k + 1) * len) - 1;
        if (e >= k * len)
            off += r[e];
    }
    __syncthreads();
    if (off)
        for (int c = c0; c < c1; ++c)
            r[c] += off;
}

template <int NKB>
__global__ __launch_bounds__(256) void ncc_u8_mfma_kernel(NccArgs a)
{
    extern __shared__ uint4 mf_smem[];
    const MfPlan P = mf_plan(a.t_width, a.hc);
    uint32_t *const V1 = reinterpret_cast<uint32_t *>(mf_smem);
    uint32_t *const V2 = V1 + MF_TY * P.vs;
    uint32_t *const img = V2 + MF_TY * P.vs;
    uint8_t *const tpl = reinterpret_cast<uint8_t *>(img + P.img_words);
    int32_t *const accbuf = reinterpret_cast<int32_t *>(img);

    const int x0 = blockIdx.x * MF_TX, y0 = blockIdx.y * MF_TY;
    const int tw = a.t_width, th = a.t_height;

    for (int i = threadIdx.x; i < 2 * MF_TY * P.vs; i += blockDim.x)
        V1[i] = 0u;

    mf_v4i acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
        acc[t] = mf_v4i{0, 0, 0, 0};

    const int nchunks16 = (64 + 16 * NKB) / 4;  // 16-byte chunks per staged image row
    for (int j0 = 0; j0 < th; j0 += P.hc) {
        const int hcur = min(P.hc, th - j0);
        __syncthreads();  // the previous chunk's readers are done (and V is zeroed)
        mf_stage_image(a.image, a.height, a.pitch, y0 + j0, x0, MF_TY - 1 + hcur, nchunks16, img, P.sw);
        mf_stage_template(a.tmpl, tw, j0, hcur, 64 * NKB, tpl, P.tsb);
        __syncthreads();
        mf_box_chunk(img, P.sw, hcur, P.nwd, V1, V2, P.vs);
        mf_mfma_chunk<NKB>(img, P.sw, tpl, P.tsb, hcur, acc);
    }
    __syncthreads();

    // SumIT' to LDS: lane (g, n) holds columns 64*wave + 16g + 4i + t of row n.
    {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int n = lane & 15, g = lane >> 4;
        int32_t *row = accbuf + n * MF_ACC_STRIDE + 64 * wave + 16 * g;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                row[4 * i + t] = acc[t][i];
    }
    // Window sums from prefix sums of the column sums (V1 and V2 rows are
    // contiguous, so one pass covers both).
    mf_row_prefix(V1, P.vs, 4 * P.nwd);

    uint32_t sum_t, sum_tsq;
    template_sums(reinterpret_cast<const uint32_t *>(a.tmpl), tw * th / 4, sum_t, sum_tsq);
    const int64_t nn = (int64_t)tw * th;
    const int64_t vt = nn * (int64_t)sum_tsq - (int64_t)sum_t * (int64_t)sum_t;
    const uint32_t bias = 128u * sum_t - 16384u * (uint32_t)nn;
    __syncthreads();

    const int x = threadIdx.x;
    const int gx = x0 + x;
    if (gx < a.out_w) {
        for (int n = 0; n < MF_TY; ++n) {
            const int gy = y0 + n;
            if (gy >= a.out_h)
                break;
            const uint32_t *q1 = V1 + n * P.vs;
            const uint32_t *q2 = V2 + n * P.vs;
            const uint32_t si = q1[x + tw - 1] - (x > 0 ? q1[x - 1] : 0u);
            const uint32_t sq = q2[x + tw - 1] - (x > 0 ? q2[x - 1] : 0u);
            const uint32_t st = (uint32_t)accbuf[n * MF_ACC_STRIDE + x] + 128u * si + bias;
            ncc_store(a, (size_t)gy * a.out_w + gx, si, sq, st, nn, (int64_t)sum_t, vt);
        }
    }
}

// Template rows per chunk: the most that fit two workgroups per CU (80 KiB
// each); when that leaves fewer than 32 rows (wide template rows), the most
// that fit one workgroup per CU.
static int mf_fit_hc(const NccArgs &a, size_t budget)
{
    int hc = a.t_height < MF_MAX_HC ? a.t_height : MF_MAX_HC;
    while (hc > 1 && mf_plan(a.t_width, hc).bytes > budget)
        --hc;
    return mf_plan(a.t_width, hc).bytes <= budget ? hc : 0;
}

static int mf_pick_hc(const NccArgs &a)
{
    const int hc = mf_fit_hc(a, 80 * 1024);
    if (hc >= 32 || hc == a.t_height)
        return hc;
    return mf_fit_hc(a, 160 * 1024);
}

bool ncc_mfma_supported(const NccArgs &a)
{
    return (a.t_width + 63) / 64 <= MF_MAX_NKB && mf_pick_hc(a) > 0;
}

template <int NKB>
static hipError_t mf_launch(const NccArgs &a, hipStream_t s)
{
    static bool attr = false;
    if (!attr) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&ncc_u8_mfma_kernel<NKB>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (e != hipSuccess)
            return e;
        attr = true;
    }
    const size_t lds = mf_plan(a.t_width, a.hc).bytes;
    const dim3 grid((a.out_w + MF_TX - 1) / MF_TX, (a.out_h + MF_TY - 1) / MF_TY);
    hipLaunchKernelGGL((ncc_u8_mfma_kernel<NKB>), grid, dim3(256), lds, s, a);
    return hipGetLastError();
}

hipError_t ncc_launch_mfma(NccArgs a, hipStream_t s)
{
    a.hc = mf_pick_hc(a);
    switch ((a.t_width + 63) / 64) {
    case 1: return mf_launch<1>(a, s);
    case 2: return mf_launch<2>(a, s);
    case 3: return mf_launch<3>(a, s);
    default: return mf_launch<4>(a, s);
    }
}

} // namespace xc
