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
//
// PH (phase variant, "Semidirect Fourier Delta Attention" eq. (13)): the decay
// is the 2x2 block Lambda_p = alpha_p R(theta_p) on rows 2p, 2p+1, so the reads
// use Lambda^T k and Lambda^T q, and a thread owns whole row pairs (rows
// 2(rg + j NRG) and the next) to apply Lambda to its own registers.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace {

constexpr int kDecodeThreads = 256;

template <typename T, int DK, bool PH>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ theta,
    const float* __restrict__ beta, float* __restrict__ state, T* __restrict__ out, int Dv)
{
    constexpr int RMAX = DK / 8 > 0 ? DK / 8 : 1;   // rows per thread when Dv = 128
    static_assert(!PH || RMAX % 2 == 0, "row pairs");
    __shared__ float sKa[DK], sQa[DK], sK[DK], sAl[DK], sQK[DK];
    __shared__ float sLc[DK / 2], sLs[DK / 2];      // (PH) alpha cos, alpha sin per pair
    __shared__ float sV[128], sE[128];
    __shared__ float sPk[kDecodeThreads * 4], sPq[kDecodeThreads * 4];
    __shared__ float sQKsum;

    const int bh = blockIdx.x;
    const int tid = threadIdx.x;
    const float b = beta[bh];

    if (tid < DK) {
        const float kc = to_f32(k[(size_t)bh * DK + tid]);
        const float qc = to_f32(q[(size_t)bh * DK + tid]);
        sK[tid] = kc;
        sQK[tid] = qc * kc;
        if constexpr (PH) {
            const int p = tid >> 1;
            float sn, cs;
            __sincosf(theta[(size_t)bh * (DK / 2) + p], &sn, &cs);
            const float ap = alpha[(size_t)bh * (DK / 2) + p];
            const float lc = ap * cs, ls = ap * sn;
            const float ko = to_f32(k[(size_t)bh * DK + (tid ^ 1)]);
            const float qo = to_f32(q[(size_t)bh * DK + (tid ^ 1)]);
            // (Lambda^T x)_{2p} = lc x_{2p} + ls x_{2p+1}, (..)_{2p+1} = lc x_{2p+1} - ls x_{2p}
            const float sg = (tid & 1) ? -1.f : 1.f;
            sKa[tid] = lc * kc + sg * ls * ko;
            sQa[tid] = lc * qc + sg * ls * qo;
            if ((tid & 1) == 0) { sLc[p] = lc; sLs[p] = ls; }
        } else {
            const float ac = alpha[(size_t)bh * DK + tid];
            sAl[tid] = ac;
            sKa[tid] = ac * kc;
            sQa[tid] = ac * qc;
        }
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
    auto row_of = [&](int i) { return PH ? 2 * (rg + (i >> 1) * nrg) + (i & 1) : rg + i * nrg; };
#pragma unroll
    for (int i = 0; i < RMAX; ++i) {
        const int row = row_of(i);
        if (active && row < DK) s[i] = *reinterpret_cast<const float4*>(Sbh + (size_t)row * Dv + 4 * cg);
    }
#pragma unroll
    for (int i = 0; i < RMAX; ++i) {
        const int row = row_of(i);
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
    if constexpr (PH) {
        // rows (2p, 2p+1) sit in s[i], s[i + 1]: Lambda S, then the correction
#pragma unroll
        for (int i = 0; i < RMAX; i += 2) {
            const int row = row_of(i);
            if (active && row < DK) {
                const float lc = sLc[row >> 1], ls = sLs[row >> 1];
                const float b0 = b * sK[row], b1 = b * sK[row + 1];
                const float4 x = s[i], y = s[i + 1];
                float4 o0, o1;
                o0.x = lc * x.x - ls * y.x + b0 * e0; o1.x = ls * x.x + lc * y.x + b1 * e0;
                o0.y = lc * x.y - ls * y.y + b0 * e1; o1.y = ls * x.y + lc * y.y + b1 * e1;
                o0.z = lc * x.z - ls * y.z + b0 * e2; o1.z = ls * x.z + lc * y.z + b1 * e2;
                o0.w = lc * x.w - ls * y.w + b0 * e3; o1.w = ls * x.w + lc * y.w + b1 * e3;
                *reinterpret_cast<float4*>(Sbh + (size_t)row * Dv + 4 * cg) = o0;
                *reinterpret_cast<float4*>(Sbh + (size_t)(row + 1) * Dv + 4 * cg) = o1;
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < RMAX; ++i) {
            const int row = row_of(i);
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
}

template <typename T, bool PH>
hipError_t launch_decode_t(int B, int H, int Dk, int Dv, const void* q, const void* k,
                           const void* v, const float* alpha, const float* theta,
                           const float* beta, float* state, void* out, hipStream_t stream)
{
    const dim3 grid((unsigned)(B * H)), block(kDecodeThreads);
    const T* qq = static_cast<const T*>(q);
    const T* kk = static_cast<const T*>(k);
    const T* vv = static_cast<const T*>(v);
    T* oo = static_cast<T*>(out);
    switch (Dk) {
    case 16: return launch_kernel(decode_kernel<T, 16, PH>, grid, block, 0, stream, qq, kk, vv, alpha, theta, beta, state, oo, Dv);
    case 32: return launch_kernel(decode_kernel<T, 32, PH>, grid, block, 0, stream, qq, kk, vv, alpha, theta, beta, state, oo, Dv);
    case 64: return launch_kernel(decode_kernel<T, 64, PH>, grid, block, 0, stream, qq, kk, vv, alpha, theta, beta, state, oo, Dv);
    case 128: return launch_kernel(decode_kernel<T, 128, PH>, grid, block, 0, stream, qq, kk, vv, alpha, theta, beta, state, oo, Dv);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode(IoType io, int B, int H, int Dk, int Dv, const void* q, const void* k,
                         const void* v, const float* alpha, const float* beta, float* state,
                         void* out, hipStream_t stream, const float* theta)
{
    if (theta) {
        if (io == IoType::F32)
            return launch_decode_t<float, true>(B, H, Dk, Dv, q, k, v, alpha, theta, beta, state, out, stream);
        return launch_decode_t<bf16_t, true>(B, H, Dk, Dv, q, k, v, alpha, theta, beta, state, out, stream);
    }
    if (io == IoType::F32)
        return launch_decode_t<float, false>(B, H, Dk, Dv, q, k, v, alpha, nullptr, beta, state, out, stream);
    return launch_decode_t<bf16_t, false>(B, H, Dk, Dv, q, k, v, alpha, nullptr, beta, state, out, stream);
}

}  // namespace kda
