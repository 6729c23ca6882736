// chunk_util.hip — workspace layout of the chunked forward and the T = 0 state copy.
#include <stddef.h>

#include "kda_chunk.hpp"
#include "kda_launch.hpp"

namespace kda {

thread_local LaunchTimer g_launch_timer;

namespace {

__global__ void state_copy_kernel(const float* __restrict__ src, float* __restrict__ dst, size_t n)
{
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.f;
}

// Sanitised tables of a packed batch (one workgroup of 256 threads):
//   cu_s[0] = 0, cu_s[i] = max(cu_s[i-1], clamp(cu[i], 0, total_T))
//   cs[0] = 0,  cs[i+1] = min(cs[i] + ceil((cu_s[i+1] - cu_s[i]) / C), umax)
// so the kernels index inside the inputs whatever cu holds.
__global__ __launch_bounds__(256) void varlen_table_kernel(const int* __restrict__ cu, int N,
                                                           int total_T, int C, int umax,
                                                           int* __restrict__ cu_s,
                                                           int* __restrict__ cs)
{
    __shared__ int sv[256];
    __shared__ int carry;
    const int tid = threadIdx.x;
    if (tid == 0) carry = 0;
    __syncthreads();
    for (int base = 0; base <= N; base += 256) {             // running maximum
        const int i = base + tid;
        int x = 0;
        if (i <= N && i > 0) x = min(max(cu[i], 0), total_T);
        sv[tid] = x;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            const int y = tid >= off ? sv[tid - off] : 0;
            __syncthreads();
            sv[tid] = max(sv[tid], y);
            __syncthreads();
        }
        const int m = max(sv[tid], carry);
        if (i <= N) cu_s[i] = m;
        __syncthreads();
        if (tid == 255) carry = m;
        __syncthreads();
    }
    if (tid == 0) { carry = 0; cs[0] = 0; }
    __syncthreads();
    for (int base = 0; base < N; base += 256) {              // chunk prefix
        const int i = base + tid;
        const int x = i < N ? (cu_s[i + 1] - cu_s[i] + C - 1) / C : 0;
        sv[tid] = x;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            const int y = tid >= off ? sv[tid - off] : 0;
            __syncthreads();
            sv[tid] += y;
            __syncthreads();
        }
        const int c = carry + sv[tid];
        if (i < N) cs[i + 1] = min(c, umax);
        __syncthreads();
        if (tid == 255) carry = c;
        __syncthreads();
    }
}

// streamed forward: every ready word 0, the control words 0, expect set
__global__ __launch_bounds__(256) void stream_clear_kernel(unsigned* __restrict__ ready, size_t nu,
                                                           StreamCtl* __restrict__ ctl, unsigned expect,
                                                           unsigned tiles)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < nu; i += stride) ready[i] = 0u;
    if (blockIdx.x == 0) {
        unsigned* w = reinterpret_cast<unsigned*>(ctl);
        for (unsigned i = threadIdx.x; i < sizeof(StreamCtl) / 4; i += blockDim.x)
            w[i] = i == offsetof(StreamCtl, expect) / 4 ? expect
                 : i == offsetof(StreamCtl, tiles) / 4  ? tiles : 0u;
    }
}

}  // namespace

hipError_t launch_stream_clear(unsigned* ready, size_t nu, StreamCtl* ctl, unsigned expect,
                               unsigned tiles, hipStream_t stream)
{
    const size_t blocks = (nu + 255) / 256;
    const unsigned grid = (unsigned)(blocks < 1 ? 1 : (blocks > 1024 ? 1024 : blocks));
    return launch_kernel(stream_clear_kernel, dim3(grid), dim3(256), 0, stream, ready, nu, ctl, expect,
                         tiles);
}

hipError_t launch_varlen_table(const int* cu, int N, int total_T, int C, int umax, int* cu_s,
                               int* cs, hipStream_t stream)
{
    return launch_kernel(varlen_table_kernel, dim3(1), dim3(256), 0, stream, cu, N, total_T, C,
                         umax, cu_s, cs);
}

size_t chunk_workspace_layout(const ChunkShape& s, IoType io, size_t off[kWorkspaceRegions])
{
    const size_t e = io == IoType::F32 ? 4 : 2;
    const size_t nu = (size_t)s.B * s.H * s.NC;
    const size_t C = s.C, Dk = s.Dk, Dv = s.Dv;
    const size_t sz[kWorkspaceRegions] = {nu * C * Dk * e, nu * C * Dv * e, nu * Dk * C * e,
                                          nu * C * Dk * e, nu * C * C * e,  nu * Dk * 4, nu};
    size_t o = 0;
    for (int i = 0; i < kWorkspaceRegions; ++i) {
        off[i] = o;
        o += (sz[i] + 255) & ~size_t(255);
    }
    return o;
}

hipError_t launch_state_copy(const float* S0, float* ST, size_t n, hipStream_t stream)
{
    if (n == 0) return hipSuccess;
    const unsigned grid = (unsigned)((n + 255) / 256);
    return launch_kernel(state_copy_kernel, dim3(grid), dim3(256), 0, stream, S0, ST, n);
}

}  // namespace kda
