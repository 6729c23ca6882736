// kda_dma.hpp — direct global-to-LDS loads and the waits and barriers that
// order them (gfx950), shared by the kernels that feed an LDS operand FIFO
// from loader wavefronts.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace kda {

using lds_void = __attribute__((address_space(3))) void;

// One 16-byte-per-lane direct global-to-LDS load: lane l's 16 bytes from its
// own address land at LDS byte address dst + 16 l (dst wave-uniform, in M0).
// Written as asm so that the compiler's wait insertion does not treat every
// later LDS access as dependent on it (it would wait for all of them); the
// kernel orders these loads with explicit waits instead.  No register is
// written by the instruction.
__device__ __forceinline__ void dma16(const void* src, const unsigned char* dst)
{
    const unsigned m0 = (unsigned)(uintptr_t)(const lds_void*)dst;
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(src), "s"(m0) : "memory", "m0");
}

// copy `bytes` (a multiple of 512) contiguous global bytes into LDS;
// lane l of each 1 KB step lands at +16 l
template <int BYTES>
__device__ __forceinline__ void dma_run(const unsigned char* src, unsigned char* dst, int lane)
{
#pragma unroll
    for (int off = 0; off < BYTES; off += 1024) {
        if (off + 1024 <= BYTES || lane < 32) dma16(src + off + 16 * lane, dst + off);
    }
}

// The 1 KB runs of NB blocks of BYTES each (whole kilobytes) as one sequence
// that starts at run `rot`.  The column slices of one (b, h) read the same
// blocks at about the same time; a different start per slice spreads their
// simultaneous reads over more L2 channels (measured on the forward chain at
// B=1, H=32, T=8192, d=128: 144.5 -> 138.9 us).  One load per run whatever
// `rot`, so wait counts do not change.
template <int NB, int BYTES>
__device__ __forceinline__ void dma_runs_rot(const unsigned char* const (&src)[NB],
                                             unsigned char* const (&dst)[NB], int lane, int rot)
{
    constexpr int R = BYTES / 1024, N = NB * R;
    static_assert(BYTES % 1024 == 0, "whole kilobytes");
    const int r0 = rot % N;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        int j = i + r0;
        if (j >= N) j -= N;
        const int b = j / R, r = j - b * R;
        dma16(src[b] + r * 1024 + 16 * lane, dst[b] + r * 1024);
    }
}

// the same for two blocks of different sizes (BA, BB whole kilobytes)
template <int BA, int BB>
__device__ __forceinline__ void dma_pair_rot(const unsigned char* sa, unsigned char* da,
                                             const unsigned char* sb, unsigned char* db, int lane,
                                             int rot)
{
    static_assert(BA % 1024 == 0 && BB % 1024 == 0, "whole kilobytes");
    constexpr int NA = BA / 1024, N = NA + BB / 1024;
    const int r0 = rot % N;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        int j = i + r0;
        if (j >= N) j -= N;
        if (j < NA) dma16(sa + j * 1024 + 16 * lane, da + j * 1024);
        else dma16(sb + (j - NA) * 1024 + 16 * lane, db + (j - NA) * 1024);
    }
}

template <int N>
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// workgroup barrier for the S / Delta exchange: waits for this wave's LDS
// accesses only.  __syncthreads() would also wait for the in-flight
// direct-to-LDS loads (they count as LDS writes), draining the FIFO.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

}  // namespace kda
