// probe.hip — peak-rate probes for the measurement leg (built into a separate
// library, libkda_probe.so; the forward never calls it).
//
// kda_probe_mfma: every wavefront of a full grid issues independent matrix
// instructions back to back (8 accumulator chains, so no instruction waits for
// the one before it), one kind per call:
//   kind 0: v_mfma_f32_16x16x32_bf16 (16 x 16 x 32, bf16 in, fp32 accumulate)
//   kind 1: v_mfma_f32_16x16x4_f32   (16 x 16 x 4, fp32)
// The result is the achieved dense rate in TFLOP/s (2 flops per multiply-add)
// over `iters` instructions per chain, timed with HIP events around the launch.
// The accumulators feed a conditional store so the work cannot be dropped.
#include <hip/hip_runtime.h>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kChains = 8;

__global__ __launch_bounds__(256) void mfma_bf16_kernel(int iters, float* sink)
{
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(1e-3f * (float)(threadIdx.x + i));
        b[i] = (__bf16)(2e-3f * (float)(i + 1));
    }
    f32x4 c[kChains];
#pragma unroll
    for (int j = 0; j < kChains; ++j) c[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < kChains; ++j) c[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[j], 0, 0, 0);
    }
    f32x4 s = c[0];
#pragma unroll
    for (int j = 1; j < kChains; ++j) s += c[j];
    if (s[0] == -1.2345f) sink[blockIdx.x] = s[1];
}

__global__ __launch_bounds__(256) void mfma_f32_kernel(int iters, float* sink)
{
    const float a = 1e-3f * (float)threadIdx.x, b = 2e-3f;
    f32x4 c[kChains];
#pragma unroll
    for (int j = 0; j < kChains; ++j) c[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < kChains; ++j) c[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c[j], 0, 0, 0);
    }
    f32x4 s = c[0];
#pragma unroll
    for (int j = 1; j < kChains; ++j) s += c[j];
    if (s[0] == -1.2345f) sink[blockIdx.x] = s[1];
}

}  // namespace

extern "C" {

// kind: 0 bf16 16x16x32, 1 fp32 16x16x4; waves_per_cu: wavefronts resident per
// compute unit (4 per workgroup); sink: device buffer of >= grid floats (never
// written in practice).  Writes the achieved TFLOP/s and returns 0, or returns
// a nonzero hipError_t.
int kda_probe_mfma(int kind, int iters, int waves_per_cu, float* sink, double* tflops)
{
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return (int)e;
    if (kind < 0 || kind > 1 || iters < 1 || waves_per_cu < 4 || !sink || !tflops)
        return (int)hipErrorInvalidValue;
    const unsigned grid = (unsigned)(cus * (waves_per_cu / 4));
    hipEvent_t e0, e1;
    if ((e = hipEventCreate(&e0)) != hipSuccess) return (int)e;
    if ((e = hipEventCreate(&e1)) != hipSuccess) return (int)e;
    auto launch = [&]() {
        if (kind == 0) hipLaunchKernelGGL(mfma_bf16_kernel, dim3(grid), dim3(256), 0, 0, iters, sink);
        else hipLaunchKernelGGL(mfma_f32_kernel, dim3(grid), dim3(256), 0, 0, iters, sink);
        return hipGetLastError();
    };
    float ms = 0.f;
    if ((e = launch()) == hipSuccess && (e = hipDeviceSynchronize()) == hipSuccess &&
        (e = hipEventRecord(e0, 0)) == hipSuccess && (e = launch()) == hipSuccess &&
        (e = hipEventRecord(e1, 0)) == hipSuccess && (e = hipEventSynchronize(e1)) == hipSuccess)
        e = hipEventElapsedTime(&ms, e0, e1);
    hipEventDestroy(e0);
    hipEventDestroy(e1);
    if (e != hipSuccess) return (int)e;
    const double mnk = kind == 0 ? 16.0 * 16.0 * 32.0 : 16.0 * 16.0 * 4.0;
    const double flops = 2.0 * mnk * kChains * (double)iters * 4.0 * grid;   // 4 waves per workgroup
    *tflops = flops / (ms * 1e-3) / 1e12;
    return 0;
}

}  // extern "C"
