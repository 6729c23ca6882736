// kda_launch.hpp — host-side launchers of the libkda kernels (internal).
// Every launcher assumes its arguments were validated by kda_api.hip and only
// enqueues work on `stream`; it returns the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

enum class IoType { F32 = 0, BF16 = 1 };

// Device regions of the chunked-forward workspace, one slab per chunk of each
// (b, h): NU = B * H * NC units.
struct ChunkWorkspace {
    void* W;     // [NU][C][Dk]  io type : Tinv diag(beta) (K * Gamma)
    float* U;    // [NU][C][Dv]  fp32    : Tinv diag(beta) V
    void* Kt;    // [NU][Dk][C]  io type : (K * rho(end, .))^T
    void* QG;    // [NU][C][Dk]  io type : Q * Gamma
    void* P;     // [NU][C][C]   io type : masked decay-weighted Q K^T (incl. diagonal)
    float* GC;   // [NU][Dk]     fp32    : decay over the whole chunk
};

struct ChunkShape {
    int B, T, H, Dk, Dv, C, NC;
};

// Bytes of each workspace region and the total (each region 256-byte aligned).
size_t chunk_workspace_layout(const ChunkShape& s, IoType io, size_t offsets[6]);

hipError_t launch_chunk_prep(IoType io, const ChunkShape& s, const void* q, const void* k,
                             const void* v, const float* alpha, const float* beta,
                             const ChunkWorkspace& ws, hipStream_t stream);

hipError_t launch_chunk_chain(IoType io, const ChunkShape& s, const ChunkWorkspace& ws,
                              const float* S0, void* out, float* ST, hipStream_t stream);

hipError_t launch_state_copy(const float* S0, float* ST, size_t n, hipStream_t stream);

hipError_t launch_decode(IoType io, int B, int H, int Dk, int Dv, const void* q,
                         const void* k, const void* v, const float* alpha,
                         const float* beta, float* state, void* out, hipStream_t stream);

hipError_t launch_gate_prep(const float* alpha, float* L, uint8_t* meta, float* gend, int B,
                            int T, int H, int Dk, int C, hipStream_t stream);

}  // namespace kda
