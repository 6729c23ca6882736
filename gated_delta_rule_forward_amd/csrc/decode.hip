// decode.hip — single-token KDA / CKDA step on a resident fp32 state.
//
// S <- (I - beta k k^T) diag(alpha) S + beta k v^T,  o = S^T q
// ("Semidirect Fourier Delta Attention", §1 eq. (1) and §3 eq. (14), at T = 1).
// Expanded so that the state is read once and written once:
//   pred_j = sum_c (alpha_c k_c) S[c][j]      (read of the decayed state)
//   r_j    = sum_c (alpha_c q_c) S[c][j]
//   e_j    = v_j - pred_j                      (compare)
//   S[c][j] <- alpha_c S[c][j] + beta k_c e_j  (correct, in place)
//   o_j    = r_j + beta (q . k) e_j            (= S_new^T q)
// The step is bound by HBM bandwidth on the state (Dk*Dv*4 bytes read and
// written per (b, h)); the arithmetic is fp32 VALU.
//
// One 256-thread workgroup per (b, h).  Thread (rg, cg): columns 4cg..4cg+3
// (one 16-byte load per row, 32 column groups cover a 128-wide row with fully
// coalesced 512-byte rows), rows rg, rg + NRG, ... .  Partial sums meet in LDS.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace {

constexpr int kDecodeThreads = 256;

template <typename T, int DK>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, float* __restrict__ state,
    T* __restrict__ out, int Dv)
{
    constexpr int RMAX = DK / 8 > 0 ? DK / 8 : 1;   // rows per thread when Dv = 128
    __shared__ float sKa[DK], sQa[DK], sK[DK], sAl[DK], sQK[DK];
    __shared__ float sV[128], sE[128];
    __shared__ float sPk[kDecodeThreads * 4], sPq[kDecodeThreads * 4];
    __shared__ float sQKsum;

    const int bh = blockIdx.x;
    const int tid = threadIdx.x;
    const float b = beta[bh];

    if (tid < DK) {
        const float kc = to_f32(k[(size_t)bh * DK + tid]);
        const float qc = to_f32(q[(size_t)bh * DK + tid]);
        const float ac = alpha[(size_t)bh * DK + tid];
        sK[tid] = kc;
        sAl[tid] = ac;
        sKa[tid] = ac * kc;
        sQa[tid] = ac * qc;
        sQK[tid] = qc * kc;
    }
    if (tid < Dv) sV[tid] = to_f32(v[(size_t)bh * Dv + tid]);
    __syncthreads();
    if (tid < 64) {
        float s = 0.f;
        for (int c = tid; c < DK; c += 64) s += sQK[c];
        for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
        if (tid == 0) sQKsum = s;
    }

    const int ncg = Dv >> 2;               // column groups of 4
    const int nrg = kDecodeThreads / ncg;  // row groups
    const int cg = tid % ncg, rg = tid / ncg;
    const bool active = rg < nrg;          // 256 % ncg != 0 leaves a few idle threads
    float* Sbh = state + (size_t)bh * DK * Dv;

    float4 s[RMAX];
    float pk[4] = {0.f, 0.f, 0.f, 0.f}, pq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RMAX; ++i) {
        const int row = rg + i * nrg;
        if (active && row < DK) s[i] = *reinterpret_cast<const float4*>(Sbh + (size_t)row * Dv + 4 * cg);
    }
#pragma unroll
    for (int i = 0; i < RMAX; ++i) {
        const int row = rg + i * nrg;
        if (active && row < DK) {
            const float ka = sKa[row], qa = sQa[row];
            pk[0] += ka * s[i].x; pk[1] += ka * s[i].y; pk[2] += ka * s[i].z; pk[3] += ka * s[i].w;
            pq[0] += qa * s[i].x; pq[1] += qa * s[i].y; pq[2] += qa * s[i].z; pq[3] += qa * s[i].w;
        }
    }
    if (active) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            sPk[rg * Dv + 4 * cg + j] = pk[j];
            sPq[rg * Dv + 4 * cg + j] = pq[j];
        }
    }
    __syncthreads();
    if (tid < Dv) {
        float pred = 0.f, r = 0.f;
        for (int g = 0; g < nrg; ++g) {
            pred += sPk[g * Dv + tid];
            r += sPq[g * Dv + tid];
        }
        const float e = sV[tid] - pred;
        sE[tid] = e;
        out[(size_t)bh * Dv + tid] = from_f32<T>(r + b * sQKsum * e);
    }
    __syncthreads();
    const float e0 = sE[4 * cg], e1 = sE[4 * cg + 1], e2 = sE[4 * cg + 2], e3 = sE[4 * cg + 3];
#pragma unroll
    for (int i = 0; i < RMAX; ++i) {
        const int row = rg + i * nrg;
        if (active && row < DK) {
            const float a = sAl[row], bk = b * sK[row];
            float4 o;
            o.x = a * s[i].x + bk * e0;
            o.y = a * s[i].y + bk * e1;
            o.z = a * s[i].z + bk * e2;
            o.w = a * s[i].w + bk * e3;
            *reinterpret_cast<float4*>(Sbh + (size_t)row * Dv + 4 * cg) = o;
        }
    }
}

template <typename T>
hipError_t launch_decode_t(int B, int H, int Dk, int Dv, const void* q, const void* k,
                           const void* v, const float* alpha, const float* beta, float* state,
                           void* out, hipStream_t stream)
{
    const dim3 grid((unsigned)(B * H)), block(kDecodeThreads);
    const T* qq = static_cast<const T*>(q);
    const T* kk = static_cast<const T*>(k);
    const T* vv = static_cast<const T*>(v);
    T* oo = static_cast<T*>(out);
    switch (Dk) {
    case 16: return launch_kernel(decode_kernel<T, 16>, grid, block, 0, stream, qq, kk, vv, alpha, beta, state, oo, Dv);
    case 32: return launch_kernel(decode_kernel<T, 32>, grid, block, 0, stream, qq, kk, vv, alpha, beta, state, oo, Dv);
    case 64: return launch_kernel(decode_kernel<T, 64>, grid, block, 0, stream, qq, kk, vv, alpha, beta, state, oo, Dv);
    case 128: return launch_kernel(decode_kernel<T, 128>, grid, block, 0, stream, qq, kk, vv, alpha, beta, state, oo, Dv);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode(IoType io, int B, int H, int Dk, int Dv, const void* q, const void* k,
                         const void* v, const float* alpha, const float* beta, float* state,
                         void* out, hipStream_t stream)
{
    if (io == IoType::F32)
        return launch_decode_t<float>(B, H, Dk, Dv, q, k, v, alpha, beta, state, out, stream);
    return launch_decode_t<bf16_t>(B, H, Dk, Dv, q, k, v, alpha, beta, state, out, stream);
}

}  // namespace kda
