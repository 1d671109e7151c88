// peak_probe.hip -- issue-rate probes for the two instructions the hot path
// is bound by, so that "fraction of peak" can be quoted against a measured
// ceiling as well as the spec sheet.  Not part of the correlation ABI; only
// the bench harness and one test (the fp64 reciprocal-square-root estimate's
// error bound, xc_rsq_probe below) load this library.
//
// Each thread runs `iters` rounds of CH independent accumulation chains of
// one instruction:
//   kind 0: v_dot4_u32_u8 (unsigned packed-byte dot product, 4 MACs)
//   kind 1: v_fmac_f32    (fp32 fused multiply-add, 2 flops)
//   kind 2: v_mfma_i32_16x16x64_i8 (16x16x64 signed-byte MACs per wave)
//   kind 3: v_mfma_i32_32x32x32_i8 (32x32x32 signed-byte MACs per wave)
//   kind 4: v_fmac_f32 with all three operands in registers: every pairing
//           of four per-lane left values with four per-lane right values
//           (all combinations of their register banks), the operand form of
//           an outer-product walk; kind 1 takes one operand as a literal and
//           the same register for another, which issues faster
// (the matrix-core kinds run 8 and 4 independent accumulators per wave).
// A launch has 64-thread workgroups, `waves_per_simd` per SIMD of every CU.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

template <int CH>
__global__ __launch_bounds__(64) void dot4_probe(uint32_t *out, int iters)
{
    uint32_t a = threadIdx.x * 77u, b = a * 2654435761u;
    uint32_t acc[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) acc[c] = c + threadIdx.x;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < CH; ++c) acc[c] = __builtin_amdgcn_udot4(a, b, acc[c], false);
        a += 0x01010101u;
    }
    uint32_t s = 0;
#pragma unroll
    for (int c = 0; c < CH; ++c) s ^= acc[c];
    out[blockIdx.x * 64 + threadIdx.x] = s;
}

template <int CH>
__global__ __launch_bounds__(64) void fma_probe(uint32_t *out, int iters)
{
    float a = (float)threadIdx.x, b = 1.0001f;
    float acc[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) acc[c] = (float)c;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < CH; ++c) acc[c] = fmaf(a, b, acc[c]);
        a += 1.0f;
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < CH; ++c) s += acc[c];
    out[blockIdx.x * 64 + threadIdx.x] = __float_as_uint(s);
}

typedef float probe_v4f __attribute__((ext_vector_type(4)));

template <int CH>
__global__ __launch_bounds__(64) void fma3_probe(uint32_t *out, int iters)
{
    probe_v4f x, y;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        x[k] = (float)(threadIdx.x + k);
        y[k] = 1.0f + (float)(threadIdx.x * 4 + k) * 0x1p-20f;
    }
    // each vector in four consecutive registers, as a 16-byte load leaves it
    asm volatile("" : "+v"(x), "+v"(y));
    float acc[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) acc[c] = (float)c;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < CH; ++c) acc[c] = fmaf(x[c & 3], y[(c >> 2) & 3], acc[c]);
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < CH; ++c) s += acc[c];
    out[blockIdx.x * 64 + threadIdx.x] = __float_as_uint(s);
}

typedef int probe_v4i __attribute__((ext_vector_type(4)));
typedef int probe_v16i __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(64) void mfma16_probe(uint32_t *out, int iters)
{
    constexpr int NA = 8;
    probe_v4i a = {(int)threadIdx.x, 3, 5, 7}, b = {11, 13, (int)threadIdx.x * 3, 17};
    probe_v4i acc[NA];
#pragma unroll
    for (int c = 0; c < NA; ++c) acc[c] = probe_v4i{c, 0, 0, 0};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < NA; ++c) acc[c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[c], 0, 0, 0);
        a[0] += 0x01010101;
    }
    int s = 0;
#pragma unroll
    for (int c = 0; c < NA; ++c) s ^= acc[c][0] ^ acc[c][1] ^ acc[c][2] ^ acc[c][3];
    out[blockIdx.x * 64 + threadIdx.x] = (uint32_t)s;
}

__global__ __launch_bounds__(64) void mfma32_probe(uint32_t *out, int iters)
{
    constexpr int NA = 4;
    probe_v4i a = {(int)threadIdx.x, 3, 5, 7}, b = {11, 13, (int)threadIdx.x * 3, 17};
    probe_v16i acc[NA];
#pragma unroll
    for (int c = 0; c < NA; ++c) {
        acc[c] = probe_v16i{};
        acc[c][0] = c;
    }
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < NA; ++c) acc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[c], 0, 0, 0);
        a[0] += 0x01010101;
    }
    int s = 0;
#pragma unroll
    for (int c = 0; c < NA; ++c)
#pragma unroll
        for (int k = 0; k < 16; ++k) s ^= acc[c][k];
    out[blockIdx.x * 64 + threadIdx.x] = (uint32_t)s;
}

// The hardware reciprocal-square-root estimate for fp64 (v_rsq_f64), the
// first step of the u8 correlation coefficient's division: y[i] = rsq(p[i]).
__global__ __launch_bounds__(256) void rsq_probe(const double *p, double *y, int n)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n)
        y[i] = __builtin_amdgcn_rsq(p[i]);
}

} // namespace

extern "C" {

// y[i] = the fp64 reciprocal-square-root estimate of p[i], i < n, for n
// doubles in device memory (p and y caller-owned, not aliased); waits for the
// result.  Returns 0, or -1 on a bad argument or a HIP error.  Lets a test
// measure the estimate's relative error, which the coefficient's rounding
// argument relies on.
int xc_rsq_probe(const double *p, double *y, int n)
{
    if (!p || !y || n <= 0)
        return -1;
    hipLaunchKernelGGL(rsq_probe, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, 0, p, y, n);
    if (hipGetLastError() != hipSuccess)
        return -1;
    return hipDeviceSynchronize() == hipSuccess ? 0 : -1;
}

// Runs the probe `reps` times after one warm-up launch; returns 0 and the mean
// milliseconds per launch in *ms, or -1 on any HIP error or unknown kind.
int xc_peak_probe(int kind, int waves_per_simd, int iters, int reps, double *ms, double *ops_per_launch)
{
    constexpr int CH = 32;
    if (kind < 0 || kind > 4 || waves_per_simd <= 0 || iters <= 0 || reps <= 0 || !ms || !ops_per_launch)
        return -1;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return -1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
    const int blocks = cus * 4 * waves_per_simd;
    uint32_t *buf = nullptr;
    if (hipMalloc(&buf, (size_t)blocks * 64 * sizeof(uint32_t)) != hipSuccess) return -1;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
        if (e0) (void)hipEventDestroy(e0);
        (void)hipFree(buf);
        return -1;
    }
    auto launch = [&]() {
        if (kind == 0)
            hipLaunchKernelGGL(dot4_probe<CH>, dim3(blocks), dim3(64), 0, 0, buf, iters);
        else if (kind == 1)
            hipLaunchKernelGGL(fma_probe<CH>, dim3(blocks), dim3(64), 0, 0, buf, iters);
        else if (kind == 4)
            hipLaunchKernelGGL(fma3_probe<CH>, dim3(blocks), dim3(64), 0, 0, buf, iters);
        else if (kind == 2)
            hipLaunchKernelGGL(mfma16_probe, dim3(blocks), dim3(64), 0, 0, buf, iters);
        else
            hipLaunchKernelGGL(mfma32_probe, dim3(blocks), dim3(64), 0, 0, buf, iters);
    };
    launch();
    int st = hipDeviceSynchronize() == hipSuccess ? 0 : -1;
    float t = 0.0f;
    if (st == 0) {
        st = hipEventRecord(e0, 0) == hipSuccess ? 0 : -1;
        for (int r = 0; r < reps; ++r) launch();
        if (st == 0 && hipEventRecord(e1, 0) != hipSuccess) st = -1;
        if (st == 0)
            st = (hipEventSynchronize(e1) == hipSuccess && hipEventElapsedTime(&t, e0, e1) == hipSuccess) ? 0 : -1;
    }
    *ms = (double)t / reps;
    // lane-operations for kinds 0, 1 and 4; int8 operations (2 per MAC) for
    // the matrix-core kinds
    if (kind <= 1 || kind == 4)
        *ops_per_launch = (double)blocks * 64 * iters * CH;
    else if (kind == 2)
        *ops_per_launch = (double)blocks * iters * 8 * (16.0 * 16 * 64) * 2;
    else
        *ops_per_launch = (double)blocks * iters * 4 * (32.0 * 32 * 32) * 2;
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (hipFree(buf) != hipSuccess) st = -1;
    return st;
}

} // extern "C"
