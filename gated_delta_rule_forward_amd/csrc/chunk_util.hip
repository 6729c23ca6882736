// chunk_util.hip — workspace layout of the chunked forward and the T = 0 state copy.
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

}  // namespace

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
