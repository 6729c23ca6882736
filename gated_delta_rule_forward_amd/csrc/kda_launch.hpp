// kda_launch.hpp — host-side launchers of the libkda kernels (internal).
// Every launcher assumes its arguments were validated by kda_api.hip and only
// enqueues work on `stream`; it returns the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

enum class IoType { F32 = 0, BF16 = 1 };

// Events attached to the next kernel launch of this thread (both null = none).
// Launchers pass them to hipExtLaunchKernelGGL, which stamps them with the
// kernel's own start and end, so a stage time is the kernel's duration.
struct LaunchTimer {
    hipEvent_t start = nullptr, stop = nullptr;
};
extern thread_local LaunchTimer g_launch_timer;

template <typename K, typename... Args>
inline hipError_t launch_kernel(K kernel, dim3 grid, dim3 block, uint32_t lds, hipStream_t stream,
                                Args... args)
{
    hipExtLaunchKernelGGL(kernel, grid, block, lds, stream, g_launch_timer.start,
                          g_launch_timer.stop, 0, args...);
    return hipGetLastError();
}

struct PrepArgs;
struct ChainArgs;

// Device regions of the chunked-forward workspace, one slab per chunk of each
// (b, h): NU = B * H * NC units (layout details in kda_chunk.hpp).
struct ChunkWorkspace {
    void* W;      // [NU][C][Dk]  io type
    void* U;      // [NU][C][Dv]  io type
    void* Kt;     // [NU][Dk][C]  io type
    void* QG;     // [NU][C][Dk]  io type
    void* P;      // [NU][C][C]   io type
    float* GC;    // [NU][Dk]     fp32
    uint8_t* FL;  // [NU]         exact-kernel flags
};

struct ChunkShape {
    int B, T, H, Dk, Dv, C, NC;
};

constexpr int kWorkspaceRegions = 7;

// Byte offset of each workspace region and the total (regions 256-byte aligned).
size_t chunk_workspace_layout(const ChunkShape& s, IoType io, size_t offsets[kWorkspaceRegions]);

// LDS bytes of one workgroup of the fast prep kernel (the same for any number
// of zero-segment columns: those are contracted Dk columns per pass).
size_t prep_fast_lds_bytes(IoType io, int C, int Dk);

hipError_t launch_prep_fast(IoType io, const ChunkShape& s, const PrepArgs& a, hipStream_t stream);
// streamed forward: the prep grid that claims units per XCD, the chain that
// waits on its ready words (ct column tiles per workgroup), and the clear of
// the ready and control words that precedes both
struct StreamCtl;
hipError_t launch_prep_stream(IoType io, const ChunkShape& s, const PrepArgs& a,
                              hipStream_t stream);
hipError_t launch_chain_stream(IoType io, const ChunkShape& s, const ChainArgs& a, int ct,
                               hipStream_t stream);
hipError_t launch_stream_clear(unsigned* ready, size_t nu, StreamCtl* ctl, unsigned expect,
                               unsigned tiles, hipStream_t stream);
hipError_t launch_prep_exact(IoType io, const ChunkShape& s, const PrepArgs& a, hipStream_t stream);
hipError_t launch_chain(IoType io, const ChunkShape& s, const ChainArgs& a, hipStream_t stream);
// the wide-slice chain (16 ct columns per workgroup, operands in registers);
// wide_chain_tiles: the ct to use for a shape, 0 when the kernel does not cover it
int wide_chain_tiles(IoType io, const ChunkShape& s);
hipError_t launch_chain_wide(IoType io, const ChunkShape& s, const ChainArgs& a, int ct,
                             hipStream_t stream);
hipError_t launch_segment_combine(int BH, int Dk, int Dv, int nseg, const float* S0,
                                  const float* summ, float* Sseg, hipStream_t stream);

hipError_t launch_state_copy(const float* S0, float* ST, size_t n, hipStream_t stream);
hipError_t launch_varlen_table(const int* cu, int N, int total_T, int C, int umax, int* cu_s,
                               int* cs, hipStream_t stream);

// decode from raw inputs: alpha and beta hold logits, q and k are normalised
// in the kernel (alpha = amin + arange sigmoid, beta = bmax sigmoid,
// x / (|x| + eps), q only when normq)
struct DecodePro {
    float amin, arange, bmax, eps;
    int normq;
};

hipError_t launch_decode(IoType io, int B, int H, int Dk, int Dv, const void* q,
                         const void* k, const void* v, const float* alpha,
                         const float* beta, float* state, void* out, hipStream_t stream,
                         const float* theta = nullptr, const DecodePro* pro = nullptr);

struct BwdChainArgs;
struct BwdLocalArgs;
struct ProArgs;
// the input prologue before the backward (out = false) and the raw-input
// gradients after it (out = true)
hipError_t launch_backward_prologue(bool out, IoType io, int Dk, const ProArgs& a, hipStream_t stream);
// backward stages: 0 relayout, 1 reverse chain, 2 per-chunk gradients,
// 3 small-gate dalpha (kda_chunk.hpp describes the arguments)
hipError_t launch_backward_stage(int stage, IoType io, const ChunkShape& s, const ChunkWorkspace& ws,
                                 const BwdChainArgs& ca, const BwdLocalArgs& la, hipStream_t stream);

// The backward of the phase variant (phase_bwd.hip): the inputs, the rotated
// inputs q', k' (io type) and per-channel gates alpha' (fp32) it forms, the
// plain backward's gradients of those, the outputs, the per-block tables
// [B H][NB + 1][P] (fp64: phases, then gradient sums) and the final-state
// term of d L / d phi per (b, h, p) (null without d_final_state).  Stages,
// one kernel each: 0 block sums of theta; 1 their prefix (the phases); 2 the
// rotated inputs; 3 dS'_T = R(-phi_T) dS_T (src -> dst); 4 the final-state
// term (src = dS'_T, dst = S'_T, into gT); 5 dq, dk, dalpha and the in-block
// part of dtheta; 6 the suffix of the block totals; 7 dtheta completed.
struct PhaseArgs {
    const void* q;
    const void* k;
    const float* alpha;
    const float* theta;
    void* qr;
    void* kr;
    float* ar;
    const void* dqr;
    const void* dkr;
    const float* dar;
    void* dq;
    void* dk;
    float* dalpha;
    float* dtheta;
    double* tab;
    double* tab2;
    const float* gT;
    int B, T, H, P, NB;
};
int phase_blocks(int T);   // 64-token blocks of a sequence of T tokens
hipError_t launch_phase_bwd(int stage, IoType io, const PhaseArgs& a, const float* src, float* dst,
                            float* gT, int Dv, hipStream_t stream);

hipError_t launch_gate_prep(const float* alpha, float* L, uint8_t* meta, float* gend, int B,
                            int T, int H, int Dk, int C, hipStream_t stream);

}  // namespace kda
