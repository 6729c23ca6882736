// range_check.hip — the device range check behind KDA_FLAG_VALIDATE_RANGES.
// Ranges: KDA gates in [0, 1] and write strengths in [0, 1] (the layer of
// "Semidirect Fourier Delta Attention", §3, draws its per-channel decays from
// [0, 1]^d; a zero gate forgets the channel: "Kimi Delta Attention: a bounded
// case study", §12.1); CKDA gates in [-1, 1] and write strengths in [0, 2]
// ("Complex KDA", the abstract).
#include "range_check.hpp"
#include <map>
#include <mutex>

namespace kda {
namespace {

// one flag word per device, raised by any element out of range; shared by
// every checking call on that device, which the mutex below serialises
__device__ unsigned g_range_flag;

struct Bounds {
    float alo, ahi, bhi;    // alpha in [alo, ahi], beta in [0, bhi]
};

__global__ __launch_bounds__(64) void range_clear_kernel(unsigned* flag)
{
    if (threadIdx.x == 0) *flag = 0u;
}

// grid-stride pass over the three arrays; every thread that meets an element
// out of range writes 1 (all writers store the same value)
__global__ __launch_bounds__(256) void range_check_kernel(const float* __restrict__ a, size_t na,
                                                          const float* __restrict__ b, size_t nb,
                                                          const float* __restrict__ th, size_t nt,
                                                          Bounds r, unsigned* __restrict__ flag)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    const size_t i0 = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    bool bad = false;
    for (size_t i = i0; i < na; i += stride) {
        const float x = a[i];
        bad |= !(x >= r.alo && x <= r.ahi);
    }
    for (size_t i = i0; i < nb; i += stride) {
        const float x = b[i];
        bad |= !(x >= 0.f && x <= r.bhi);
    }
    for (size_t i = i0; i < nt; i += stride) bad |= !(fabsf(th[i]) <= 3.4028234663852886e38f);
    if (bad) *flag = 1u;
}

std::mutex g_mu;
std::map<int, unsigned*> g_flag_ptr;    // device -> address of g_range_flag there

}  // namespace

RangeResult check_ranges(const float* alpha, size_t na, const float* beta, size_t nb,
                         const float* theta, size_t nt, bool ckda, hipStream_t stream)
{
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cap) != hipSuccess) return RangeResult::HipError;
    if (cap != hipStreamCaptureStatusNone) return RangeResult::Capturing;

    std::lock_guard<std::mutex> guard(g_mu);
    int cur = 0, dev = 0;
    if (hipGetDevice(&cur) != hipSuccess) return RangeResult::HipError;
    if (hipStreamGetDevice(stream, &dev) != hipSuccess) return RangeResult::HipError;
    unsigned* flag = nullptr;
    const auto it = g_flag_ptr.find(dev);
    if (it != g_flag_ptr.end()) {
        flag = it->second;
    } else {
        // the symbol's address is per device: look it up with that device current
        if (dev != cur && hipSetDevice(dev) != hipSuccess) return RangeResult::HipError;
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_range_flag));
        if (dev != cur && hipSetDevice(cur) != hipSuccess) return RangeResult::HipError;
        if (e != hipSuccess || !p) return RangeResult::HipError;
        flag = static_cast<unsigned*>(p);
        g_flag_ptr[dev] = flag;
    }

    const Bounds r = ckda ? Bounds{-1.f, 1.f, 2.f} : Bounds{0.f, 1.f, 1.f};
    hipLaunchKernelGGL(range_clear_kernel, dim3(1), dim3(64), 0, stream, flag);
    if (hipGetLastError() != hipSuccess) return RangeResult::HipError;
    const size_t n = na > nb ? (na > nt ? na : nt) : (nb > nt ? nb : nt);
    if (n > 0) {
        const size_t blocks = (n + 255) / 256;
        const unsigned grid = (unsigned)(blocks < 4096 ? blocks : 4096);
        hipLaunchKernelGGL(range_check_kernel, dim3(grid), dim3(256), 0, stream, alpha, na, beta,
                           nb, theta, nt, r, flag);
        if (hipGetLastError() != hipSuccess) return RangeResult::HipError;
    }
    unsigned h = 0;
    if (hipMemcpyAsync(&h, flag, sizeof(h), hipMemcpyDeviceToHost, stream) != hipSuccess)
        return RangeResult::HipError;
    if (hipStreamSynchronize(stream) != hipSuccess) return RangeResult::HipError;
    return h ? RangeResult::OutOfRange : RangeResult::InRange;
}

}  // namespace kda
