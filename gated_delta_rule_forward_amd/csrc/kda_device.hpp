// kda_device.hpp — device helpers shared by the libkda kernels (gfx950 only).
//
// MFMA fragment convention used throughout (16x16 output tiles, wave64):
//   lane l = 16 * g + n  (g = l / 16 in 0..3, n = l % 16)
//   accumulator register i of lane l holds D[4g + i][n]
//   one "k16 block" contracts 16 k-indices; lane (m or n, g) supplies the four
//   consecutive k-indices 4g .. 4g+3 of its A row m / B column n.
// fp32 uses four v_mfma_f32_16x16x4_f32 per k16 block (k-index g of step i is
// 4g + i), bf16 uses one v_mfma_f32_16x16x16_bf16; both therefore consume the
// same per-lane data: 4 consecutive k of one A row and 4 consecutive k of one
// B column.  A C-layout accumulator tile (rows 4g..4g+3 of column n in lane l)
// is thus directly the B fragment of a k16 block over those 16 rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16_t;

// ---- scalar conversions ---------------------------------------------------
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
// round-to-nearest-even (the hardware conversion on gfx950)
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return (bf16_t)x; }

__device__ __forceinline__ short bf16_bits(bf16_t x) { return __builtin_bit_cast(short, x); }

// ---- four consecutive elements ----------------------------------------------
template <typename T> struct Vec4;
template <> struct Vec4<float> {
    float v[4];
    __device__ __forceinline__ static Vec4 load(const float* p) {
        const float4 x = *reinterpret_cast<const float4*>(p);
        return Vec4{{x.x, x.y, x.z, x.w}};
    }
    // non-temporal: for inputs read once (streamed past the caches)
    __device__ __forceinline__ static Vec4 load_nt(const float* p) {
        const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
        return Vec4{{x[0], x[1], x[2], x[3]}};
    }
    __device__ __forceinline__ static Vec4 from(const float* f) { return Vec4{{f[0], f[1], f[2], f[3]}}; }
    __device__ __forceinline__ static Vec4 zero() { return Vec4{{0.f, 0.f, 0.f, 0.f}}; }
    __device__ __forceinline__ float get(int i) const { return v[i]; }
    __device__ __forceinline__ float elem(int i) const { return v[i]; }
};
template <> struct Vec4<bf16_t> {
    i16x4 v;   // raw bf16 bits
    __device__ __forceinline__ static Vec4 load(const bf16_t* p) {
        return Vec4{*reinterpret_cast<const i16x4*>(p)};
    }
    __device__ __forceinline__ static Vec4 load_nt(const bf16_t* p) {
        return Vec4{__builtin_nontemporal_load(reinterpret_cast<const i16x4*>(p))};
    }
    __device__ __forceinline__ static Vec4 from(const float* f) {
        i16x4 r;
        r[0] = bf16_bits((bf16_t)f[0]); r[1] = bf16_bits((bf16_t)f[1]);
        r[2] = bf16_bits((bf16_t)f[2]); r[3] = bf16_bits((bf16_t)f[3]);
        return Vec4{r};
    }
    __device__ __forceinline__ static Vec4 zero() { return Vec4{i16x4{0, 0, 0, 0}}; }
    __device__ __forceinline__ float get(int i) const {
        return __uint_as_float((unsigned)(unsigned short)v[i] << 16);
    }
    __device__ __forceinline__ bf16_t elem(int i) const { return __builtin_bit_cast(bf16_t, (short)v[i]); }
};

// ---- one k16 block of a 16x16 MFMA tile --------------------------------------
__device__ __forceinline__ f32x4 mma_k16(const Vec4<float>& a, const Vec4<float>& b, f32x4 acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[0], b.v[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[1], b.v[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[2], b.v[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[3], b.v[3], acc, 0, 0, 0);
    return acc;
}
__device__ __forceinline__ f32x4 mma_k16(const Vec4<bf16_t>& a, const Vec4<bf16_t>& b, f32x4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.v, b.v, acc, 0, 0, 0);
}

// C = A * Bt^T over K (multiple of 16) with both operands row-major in memory
// (A[m][k] at A + m*lda + k, Bt[n][k] at Bt + n*ldb + k): the 16x16 tile whose
// top-left A row is A and top-left Bt row is Bt.
template <typename T>
__device__ __forceinline__ f32x4 tile_tn(const T* A, int lda, const T* Bt, int ldb, int K, f32x4 acc) {
    const int lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const T* pa = A + r * lda + 4 * g;
    const T* pb = Bt + r * ldb + 4 * g;
    for (int k0 = 0; k0 < K; k0 += 16)
        acc = mma_k16(Vec4<T>::load(pa + k0), Vec4<T>::load(pb + k0), acc);
    return acc;
}

// ---- DPP sum over the 16 lanes of a row (every lane receives the sum) -------
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xf, 0xf, true));
}
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_mov<0xB1>(x);    // quad_perm [1,0,3,2]
    x += dpp_mov<0x4E>(x);    // quad_perm [2,3,0,1]
    x += dpp_mov<0x141>(x);   // row_half_mirror
    x += dpp_mov<0x140>(x);   // row_mirror
    return x;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// the XCD (accelerator complex die) this wavefront runs on, from the hardware
// register XCC_ID (bits 3:0; the MI355X has 8)
__device__ __forceinline__ unsigned xcc_id()
{
    return __builtin_amdgcn_s_getreg(20 | (0 << 6) | (3 << 11)) & 7u;
}

}  // namespace kda
