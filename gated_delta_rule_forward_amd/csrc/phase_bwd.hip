// phase_bwd.hip — the backward of the phase variant ("Semidirect Fourier Delta
// Attention" §3 eq. (13): the decay of channel pair p is the block
// alpha_p R(theta_p) on state rows 2p, 2p+1) by reduction to the plain
// backward.
//
// With phi_t = theta_1 + ... + theta_t per pair (the running phase of one
// sequence), the rotated state S'_t = R(-phi_t) S_t obeys the plain recurrence
// with q'_t = R(-phi_t) q_t, k'_t = R(-phi_t) k_t and the pair's decay alpha_p
// on both of its channels: rotations are orthogonal, so they pass through
// k k^T and the read-out S^T q, and a 2x2 rotation commutes with the scalar
// alpha_p.  The final state is S_T = R(phi_T) S'_T and S'_0 = S_0.  Hence the
// gradients: the plain backward on (q', k', alpha') with dS'_T = R(-phi_T) dS_T
// gives dv, dbeta, dS0 as they are; dq_t = R(phi_t) dq'_t, dk_t likewise;
// dalpha_p is the sum of the pair's two channel gradients; and, J being the
// rotation by a right angle (d R(phi) / d phi = J R(phi)),
//   d L / d phi_t = <dq'_t, -J q'_t> + <dk'_t, -J k'_t>   (+ <dS'_T, J S'_T> at t = T),
//   dtheta_s = sum over t >= s of d L / d phi_t.
//
// Kernels (one thread per channel pair of a 64-token block of one sequence,
// pairs of consecutive threads adjacent in memory):
//   block_sum   theta summed over the block (fp64)
//   scan        exclusive prefix over the blocks of each (b, h, p), reduced
//               mod 2 pi (phases), or inclusive suffix (gradient sums)
//   rotate_in   q', k' (io type) and alpha' per channel (fp32)
//   state_rot   dS'_T = R(-phi_T) dS_T
//   final_dphi  <dS'_T, J S'_T> per (b, h, p) (one wavefront each)
//   rotate_out  dq, dk, dalpha, and minus the in-block prefix of d L / d phi
//               (dtheta before the suffix), with the block totals
//   add_suffix  dtheta += the inclusive suffix of the block totals
// The phase of a token is formed in fp64 from the fp64 block prefix and
// reduced to [0, 2 pi) before the fp32 sine and cosine, so long sequences keep
// the rotation angles exact to fp32 rounding.
#include <hip/hip_runtime.h>

#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace {

constexpr int kPhaseBlock = 64;
constexpr double kTwoPi = 6.283185307179586476925286766559;

__device__ __forceinline__ void phase_cos_sin(double phi, float& c, float& s)
{
    const double r = phi - kTwoPi * floor(phi / kTwoPi);
    sincosf((float)r, &s, &c);
}

struct PairIdx {
    int bh, n, p;
    bool ok;
};

__device__ __forceinline__ PairIdx pair_index(const PhaseArgs& a)
{
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t per_bh = (size_t)a.NB * a.P;
    PairIdx r;
    r.ok = i < (size_t)a.B * a.H * per_bh;
    const size_t j = r.ok ? i : 0;
    r.bh = (int)(j / per_bh);
    r.n = (int)((j % per_bh) / a.P);
    r.p = (int)(j % a.P);
    return r;
}

// token row (b T + t) H + h of sequence bh
__device__ __forceinline__ size_t token_row(const PhaseArgs& a, int bh, int t)
{
    const int b = bh / a.H, h = bh % a.H;
    return ((size_t)b * a.T + t) * a.H + h;
}

__device__ __forceinline__ size_t tab_index(const PhaseArgs& a, int bh, int n, int p)
{
    return ((size_t)bh * (a.NB + 1) + n) * a.P + p;
}

__global__ __launch_bounds__(256) void block_sum_kernel(PhaseArgs a)
{
    const PairIdx x = pair_index(a);
    if (!x.ok) return;
    const int t0 = x.n * kPhaseBlock, t1 = min(t0 + kPhaseBlock, a.T);
    double s = 0.0;
    for (int t = t0; t < t1; ++t) s += (double)a.theta[token_row(a, x.bh, t) * a.P + x.p];
    a.tab[tab_index(a, x.bh, x.n, x.p)] = s;
}

// one thread per (b, h, p): phases (suffix == 0) become the exclusive prefix
// of the block sums mod 2 pi, with the total phase at index NB; gradient sums
// (suffix == 1) become the inclusive suffix
__global__ __launch_bounds__(256) void scan_kernel(double* tab, int nbh, int NB, int P, int suffix)
{
    const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
    if (i >= nbh * P) return;
    double* col = tab + (size_t)(i / P) * (NB + 1) * P + i % P;
    double acc = 0.0;
    if (!suffix) {
        for (int n = 0; n < NB; ++n) {
            const double v = col[(size_t)n * P];
            col[(size_t)n * P] = acc;
            acc += v;
            acc -= kTwoPi * floor(acc / kTwoPi);
        }
        col[(size_t)NB * P] = acc;
    } else {
        for (int n = NB - 1; n >= 0; --n) {
            acc += col[(size_t)n * P];
            col[(size_t)n * P] = acc;
        }
    }
}

template <typename T>
__global__ __launch_bounds__(256) void rotate_in_kernel(PhaseArgs a)
{
    const PairIdx x = pair_index(a);
    if (!x.ok) return;
    const int DK = 2 * a.P;
    const int t0 = x.n * kPhaseBlock, t1 = min(t0 + kPhaseBlock, a.T);
    double phi = a.tab[tab_index(a, x.bh, x.n, x.p)];
    const T* q = static_cast<const T*>(a.q);
    const T* k = static_cast<const T*>(a.k);
    T* qr = static_cast<T*>(a.qr);
    T* kr = static_cast<T*>(a.kr);
    for (int t = t0; t < t1; ++t) {
        const size_t row = token_row(a, x.bh, t);
        const size_t e = row * DK + 2 * x.p, g = row * a.P + x.p;
        phi += (double)a.theta[g];
        float c, s;
        phase_cos_sin(phi, c, s);
        const float q0 = to_f32(q[e]), q1 = to_f32(q[e + 1]);
        const float k0 = to_f32(k[e]), k1 = to_f32(k[e + 1]);
        // R(-phi) = [[c, s], [-s, c]]
        qr[e] = from_f32<T>(c * q0 + s * q1);
        qr[e + 1] = from_f32<T>(c * q1 - s * q0);
        kr[e] = from_f32<T>(c * k0 + s * k1);
        kr[e + 1] = from_f32<T>(c * k1 - s * k0);
        const float al = a.alpha[g];
        *reinterpret_cast<float2*>(a.ar + e) = make_float2(al, al);
    }
}

// dS'_T = R(-phi_T) dS_T on every row pair; one thread per (b, h, p, column)
__global__ __launch_bounds__(256) void state_rot_kernel(PhaseArgs a, const float* src, float* dst,
                                                        int Dv)
{
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t n = (size_t)a.B * a.H * a.P * Dv;
    if (i >= n) return;
    const int j = (int)(i % Dv);
    const int p = (int)((i / Dv) % a.P);
    const int bh = (int)(i / ((size_t)Dv * a.P));
    float c, s;
    phase_cos_sin(a.tab[tab_index(a, bh, a.NB, p)], c, s);
    const size_t r0 = ((size_t)bh * 2 * a.P + 2 * p) * Dv + j;
    const float x = src[r0], y = src[r0 + Dv];
    dst[r0] = c * x + s * y;
    dst[r0 + Dv] = c * y - s * x;
}

// <dS'_T, J S'_T> of one (b, h, p): sum over the columns of
// dS'[2p+1] S'[2p] - dS'[2p] S'[2p+1]; one wavefront per (b, h, p)
__global__ __launch_bounds__(256) void final_dphi_kernel(PhaseArgs a, const float* dst,
                                                         const float* st, float* gT, int Dv)
{
    const int w = (int)((blockIdx.x * blockDim.x + threadIdx.x) / 64), lane = threadIdx.x % 64;
    if (w >= a.B * a.H * a.P) return;
    const int bh = w / a.P, p = w % a.P;
    const size_t r0 = ((size_t)bh * 2 * a.P + 2 * p) * Dv;
    float acc = 0.f;
    for (int j = lane; j < Dv; j += 64)
        acc += dst[r0 + Dv + j] * st[r0 + j] - dst[r0 + j] * st[r0 + Dv + j];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
    if (lane == 0) gT[w] = acc;
}

template <typename T>
__global__ __launch_bounds__(256) void rotate_out_kernel(PhaseArgs a)
{
    const PairIdx x = pair_index(a);
    if (!x.ok) return;
    const int DK = 2 * a.P;
    const int t0 = x.n * kPhaseBlock, t1 = min(t0 + kPhaseBlock, a.T);
    double phi = a.tab[tab_index(a, x.bh, x.n, x.p)];
    const T* qr = static_cast<const T*>(a.qr);
    const T* kr = static_cast<const T*>(a.kr);
    const T* dqr = static_cast<const T*>(a.dqr);
    const T* dkr = static_cast<const T*>(a.dkr);
    T* dq = static_cast<T*>(a.dq);
    T* dk = static_cast<T*>(a.dk);
    const float gT = (a.gT && t1 == a.T) ? a.gT[(size_t)x.bh * a.P + x.p] : 0.f;
    float pre = 0.f;   // d L / d phi summed over the block's tokens before t
    for (int t = t0; t < t1; ++t) {
        const size_t row = token_row(a, x.bh, t);
        const size_t e = row * DK + 2 * x.p, g = row * a.P + x.p;
        phi += (double)a.theta[g];
        float c, s;
        phase_cos_sin(phi, c, s);
        const float dq0 = to_f32(dqr[e]), dq1 = to_f32(dqr[e + 1]);
        const float dk0 = to_f32(dkr[e]), dk1 = to_f32(dkr[e + 1]);
        const float q0 = to_f32(qr[e]), q1 = to_f32(qr[e + 1]);
        const float k0 = to_f32(kr[e]), k1 = to_f32(kr[e + 1]);
        // R(phi) = [[c, -s], [s, c]]
        dq[e] = from_f32<T>(c * dq0 - s * dq1);
        dq[e + 1] = from_f32<T>(s * dq0 + c * dq1);
        dk[e] = from_f32<T>(c * dk0 - s * dk1);
        dk[e + 1] = from_f32<T>(s * dk0 + c * dk1);
        const float2 da = *reinterpret_cast<const float2*>(a.dar + e);
        a.dalpha[g] = da.x + da.y;
        float gphi = (dq0 * q1 - dq1 * q0) + (dk0 * k1 - dk1 * k0);
        if (t == a.T - 1) gphi += gT;
        a.dtheta[g] = -pre;
        pre += gphi;
    }
    a.tab2[tab_index(a, x.bh, x.n, x.p)] = (double)pre;
}

// dtheta_t = (sum of d L / d phi over the block's tokens from t on and over
// every later block) = suffix(n) - (the block's sum before t)
__global__ __launch_bounds__(256) void add_suffix_kernel(PhaseArgs a)
{
    const PairIdx x = pair_index(a);
    if (!x.ok) return;
    const int t0 = x.n * kPhaseBlock, t1 = min(t0 + kPhaseBlock, a.T);
    const float suf = (float)a.tab2[tab_index(a, x.bh, x.n, x.p)];
    for (int t = t0; t < t1; ++t) {
        float* d = a.dtheta + token_row(a, x.bh, t) * a.P + x.p;
        *d = suf + *d;
    }
}

unsigned blocks_for(size_t threads) { return (unsigned)((threads + 255) / 256); }

}  // namespace

int phase_blocks(int T) { return (T + kPhaseBlock - 1) / kPhaseBlock; }

hipError_t launch_phase_bwd(int stage, IoType io, const PhaseArgs& a, const float* src, float* dst,
                            float* gT, int Dv, hipStream_t stream)
{
    const unsigned gp = blocks_for((size_t)a.B * a.H * a.NB * a.P);
    const int nbh = a.B * a.H;
    const unsigned gs = blocks_for((size_t)nbh * a.P);
    const bool f32 = io == IoType::F32;
    switch (stage) {
    case 0: return launch_kernel(block_sum_kernel, dim3(gp), dim3(256), 0, stream, a);
    case 1: return launch_kernel(scan_kernel, dim3(gs), dim3(256), 0, stream, a.tab, nbh, a.NB, a.P, 0);
    case 2:
        return f32 ? launch_kernel(rotate_in_kernel<float>, dim3(gp), dim3(256), 0, stream, a)
                   : launch_kernel(rotate_in_kernel<bf16_t>, dim3(gp), dim3(256), 0, stream, a);
    case 3:
        return launch_kernel(state_rot_kernel, dim3(blocks_for((size_t)nbh * a.P * Dv)), dim3(256),
                             0, stream, a, src, dst, Dv);
    case 4:
        return launch_kernel(final_dphi_kernel, dim3(blocks_for((size_t)nbh * a.P * 64)),
                             dim3(256), 0, stream, a, src, static_cast<const float*>(dst), gT, Dv);
    case 5:
        return f32 ? launch_kernel(rotate_out_kernel<float>, dim3(gp), dim3(256), 0, stream, a)
                   : launch_kernel(rotate_out_kernel<bf16_t>, dim3(gp), dim3(256), 0, stream, a);
    case 6: return launch_kernel(scan_kernel, dim3(gs), dim3(256), 0, stream, a.tab2, nbh, a.NB, a.P, 1);
    case 7: return launch_kernel(add_suffix_kernel, dim3(gp), dim3(256), 0, stream, a);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace kda
