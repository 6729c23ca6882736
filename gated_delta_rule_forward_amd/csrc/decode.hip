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
// Columns of S update independently (pred_j, r_j and e_j use column j only),
// so one workgroup owns NCOL columns of one (b, h), all Dk rows: thread
// (row group rg, column quad cq) holds RPT consecutive rows x 4 columns in
// registers from the read to the write (16-byte accesses; NCOL / 4
// consecutive lanes cover one row's NCOL columns).  The sums over rows go
// through lane shuffles within a wavefront, then LDS across wavefronts.
// Each thread holds one row pair, so a workgroup has NCOL * Dk / 8 threads
// (1024 at 64 columns and Dk = 128: 32 KB of state); slices of 64 columns
// (256-byte row segments) keep more of HBM busy than one workgroup per (b, h)
// (launch_decode_cols gives the measurements).  The state is read and written
// with non-temporal accesses (it is touched once per step and does not fit
// the caches).  The column slices of one (b, h) are numbered onto one XCD
// (consecutive workgroups go to consecutive XCDs).
//
// PRO (input parameterisation, same page §3 eqs. (15), (17), (18)): alpha and
// beta arrive as logits and q, k raw; the loads apply alpha = amin + arange
// sigmoid(gate), beta = bmax sigmoid(logit) and k / (|k| + eps) (q likewise
// when normq), with the norms summed over the Dk channels across the
// workgroup and the normalised q, k rounded to the io type once, as in the
// chunked forward.
//
// PH (phase variant, "Semidirect Fourier Delta Attention" eq. (13)): the decay
// is the 2x2 block Lambda_p = alpha_p R(theta_p) on rows 2p, 2p+1, so the reads
// use Lambda^T k and Lambda^T q, and each thread's rows come in pairs
// (RPT even) so that it applies Lambda to its own registers.
#include "kda_chunk.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace {

constexpr int kDecodeXcds = 8;

// threads of a workgroup with NCOL columns: one row pair per thread, at most 1024
constexpr int decode_threads(int DK, int NCOL)
{
    return NCOL * DK / 8 > 1024 ? 1024 : (NCOL * DK / 8 < 64 ? 64 : NCOL * DK / 8);
}

template <int DK, int NCOL, int NTHR>
struct DecodeGeom {
    static constexpr int NCQ = NCOL / 4;                                    // column quads
    static constexpr int NRG = (NTHR / NCQ) < DK / 2 ? NTHR / NCQ : DK / 2;
    static constexpr int RPT = DK / NRG;                                    // rows per thread (even)
    static constexpr int ACTIVE = NRG * NCQ;                                // threads holding state
    static constexpr int WAVES = (ACTIVE + 63) / 64;
    static_assert(RPT % 2 == 0 && RPT * NRG == DK, "row pairs");
};

template <typename T, int DK, int NCOL, int NTHR, bool PH, bool PRO>
__global__ __launch_bounds__(NTHR) void decode_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ theta,
    const float* __restrict__ beta, float* __restrict__ state, T* __restrict__ out, int BH, int Dv,
    DecodePro pro)
{
    static_assert(!(PH && PRO), "the parameterisation and the phase variant are not combined");
    using G = DecodeGeom<DK, NCOL, NTHR>;
    constexpr int NCQ = G::NCQ, RPT = G::RPT;
    __shared__ float sKa[DK], sQa[DK], sK[DK], sAl[DK];
    __shared__ float sLc[DK / 2], sLs[DK / 2];      // (PH) alpha cos, alpha sin per pair
    __shared__ float sPk[G::WAVES][NCOL], sPq[G::WAVES][NCOL], sE[NCOL];
    __shared__ float sQKw[NTHR / 64];

    // workgroup -> (b h, column slice): the NS slices of one (b, h) share g % 8
    const int NS = Dv / NCOL;
    const int g = blockIdx.x, xcd = g % kDecodeXcds, jx = g / kDecodeXcds;
    const int slice = jx % NS, bh = (jx / NS) * kDecodeXcds + xcd;
    if (bh >= BH) return;
    const int c0 = slice * NCOL;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float b = PRO ? pro.bmax * sigmoid_f32(beta[bh]) : beta[bh];

    float qk = 0.f;
    float kc = tid < DK ? to_f32(k[(size_t)bh * DK + tid]) : 0.f;
    float qc = tid < DK ? to_f32(q[(size_t)bh * DK + tid]) : 0.f;
    if constexpr (PRO) {
        // |k| and |q| over the Dk channels: per wavefront, then across them
        __shared__ float sNrm[NTHR / 64][2];
        float kk = kc * kc, qq = qc * qc;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            kk += __shfl_xor(kk, off);
            qq += __shfl_xor(qq, off);
        }
        if (lane == 0) { sNrm[wave][0] = kk; sNrm[wave][1] = qq; }
        __syncthreads();
        kk = 0.f;
        qq = 0.f;
#pragma unroll
        for (int w = 0; w < (DK + 63) / 64; ++w) { kk += sNrm[w][0]; qq += sNrm[w][1]; }
        const float nk = __builtin_sqrtf(kk) + pro.eps, nq = __builtin_sqrtf(qq) + pro.eps;
        kc = to_f32(from_f32<T>(kc * (nk > 0.f ? 1.f / nk : 0.f)));
        if (pro.normq) qc = to_f32(from_f32<T>(qc * (nq > 0.f ? 1.f / nq : 0.f)));
    }
    if (tid < DK) {
        sK[tid] = kc;
        qk = qc * kc;
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
            const float ac = PRO ? pro.amin + pro.arange * sigmoid_f32(alpha[(size_t)bh * DK + tid])
                                 : alpha[(size_t)bh * DK + tid];
            sAl[tid] = ac;
            sKa[tid] = ac * kc;
            sQa[tid] = ac * qc;
        }
    }
    // q . k over the Dk channels: per wavefront, then across them after the barrier
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) qk += __shfl_xor(qk, off);
    if (lane == 0) sQKw[wave] = qk;

    const int cq = tid % NCQ, rg = tid / NCQ;
    const bool active = tid < G::ACTIVE;
    float* Sc = state + (size_t)bh * DK * Dv + c0 + 4 * cq;     // column quad cq of the slice
    f32x4 s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int row = rg * RPT + i;
        s[i] = active ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Sc + (size_t)row * Dv))
                      : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    __syncthreads();
    f32x4 pk = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
    if (active) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int row = rg * RPT + i;
            pk += sKa[row] * s[i];
            pq += sQa[row] * s[i];
        }
    }
    // sum over the row groups of this wavefront (lanes NCQ apart)
#pragma unroll
    for (int off = NCQ; off < 64; off <<= 1) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            pk[j] += __shfl_xor(pk[j], off);
            pq[j] += __shfl_xor(pq[j], off);
        }
    }
    if (lane < NCQ && wave < G::WAVES) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            sPk[wave][4 * lane + j] = pk[j];
            sPq[wave][4 * lane + j] = pq[j];
        }
    }
    __syncthreads();
    if (tid < NCOL) {
        float pred = 0.f, r = 0.f, qks = 0.f;
#pragma unroll
        for (int w = 0; w < G::WAVES; ++w) { pred += sPk[w][tid]; r += sPq[w][tid]; }
#pragma unroll
        for (int w = 0; w < (DK + 63) / 64; ++w) qks += sQKw[w];
        const float e = to_f32(v[(size_t)bh * Dv + c0 + tid]) - pred;
        sE[tid] = e;
        out[(size_t)bh * Dv + c0 + tid] = from_f32<T>(r + b * qks * e);
    }
    __syncthreads();
    if (!active) return;
    const f32x4 e4 = {sE[4 * cq], sE[4 * cq + 1], sE[4 * cq + 2], sE[4 * cq + 3]};
    if constexpr (PH) {
        // rows (2p, 2p+1) sit in s[i], s[i + 1]: Lambda S, then the correction
#pragma unroll
        for (int i = 0; i < RPT; i += 2) {
            const int row = rg * RPT + i;
            const float lc = sLc[row >> 1], ls = sLs[row >> 1];
            const f32x4 o0 = lc * s[i] - ls * s[i + 1] + (b * sK[row]) * e4;
            const f32x4 o1 = ls * s[i] + lc * s[i + 1] + (b * sK[row + 1]) * e4;
            __builtin_nontemporal_store(o0, reinterpret_cast<f32x4*>(Sc + (size_t)row * Dv));
            __builtin_nontemporal_store(o1, reinterpret_cast<f32x4*>(Sc + (size_t)(row + 1) * Dv));
        }
    } else {
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int row = rg * RPT + i;
            const f32x4 o = sAl[row] * s[i] + (b * sK[row]) * e4;
            __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(Sc + (size_t)row * Dv));
        }
    }
}

template <typename T, bool PH, bool PRO, int NCOL>
hipError_t launch_decode_t(int B, int H, int Dk, int Dv, const void* q, const void* k,
                           const void* v, const float* alpha, const float* theta,
                           const float* beta, float* state, void* out, hipStream_t stream,
                           const DecodePro& pro)
{
    const int BH = B * H;
    // (b h) rounded up to whole XCD rounds, times the column slices
    const unsigned nblk = (unsigned)(((BH + kDecodeXcds - 1) / kDecodeXcds) * kDecodeXcds * (Dv / NCOL));
    const dim3 grid(nblk);
    const T* qq = static_cast<const T*>(q);
    const T* kk = static_cast<const T*>(k);
    const T* vv = static_cast<const T*>(v);
    T* oo = static_cast<T*>(out);
    switch (Dk) {
    case 16: return launch_kernel(decode_kernel<T, 16, NCOL, decode_threads(16, NCOL), PH, PRO>, grid,
                                   dim3(decode_threads(16, NCOL)), 0, stream, qq, kk, vv, alpha, theta, beta, state, oo, BH, Dv, pro);
    case 32: return launch_kernel(decode_kernel<T, 32, NCOL, decode_threads(32, NCOL), PH, PRO>, grid,
                                   dim3(decode_threads(32, NCOL)), 0, stream, qq, kk, vv, alpha, theta, beta, state, oo, BH, Dv, pro);
    case 64: return launch_kernel(decode_kernel<T, 64, NCOL, decode_threads(64, NCOL), PH, PRO>, grid,
                                   dim3(decode_threads(64, NCOL)), 0, stream, qq, kk, vv, alpha, theta, beta, state, oo, BH, Dv, pro);
    case 128: return launch_kernel(decode_kernel<T, 128, NCOL, decode_threads(128, NCOL), PH, PRO>, grid,
                                   dim3(decode_threads(128, NCOL)), 0, stream, qq, kk, vv, alpha, theta, beta, state, oo, BH, Dv, pro);
    default: return hipErrorInvalidValue;
    }
}

template <typename T, bool PH, bool PRO>
hipError_t launch_decode_cols(int B, int H, int Dk, int Dv, const void* q, const void* k,
                              const void* v, const float* alpha, const float* theta,
                              const float* beta, float* state, void* out, hipStream_t stream,
                              const DecodePro& pro)
{
    // 64 columns (256-byte row segments) where Dv allows, else 32, else 16.
    // Measured (B=256, H=32, d=128, in-place fp32 state, 1.086 GB per step):
    // 212 us with one workgroup per (b, h); 175 us at 64 columns / 1024
    // threads, 181 us at 32 / 256, 185 us at 128 / 1024, 217 us at 16 / 256
    // (half-line row segments), 429 us at 8 / 128.
    if (Dv % 64 == 0)
        return launch_decode_t<T, PH, PRO, 64>(B, H, Dk, Dv, q, k, v, alpha, theta, beta, state, out, stream, pro);
    if (Dv % 32 == 0)
        return launch_decode_t<T, PH, PRO, 32>(B, H, Dk, Dv, q, k, v, alpha, theta, beta, state, out, stream, pro);
    return launch_decode_t<T, PH, PRO, 16>(B, H, Dk, Dv, q, k, v, alpha, theta, beta, state, out, stream, pro);
}

}  // namespace

hipError_t launch_decode(IoType io, int B, int H, int Dk, int Dv, const void* q, const void* k,
                         const void* v, const float* alpha, const float* beta, float* state,
                         void* out, hipStream_t stream, const float* theta, const DecodePro* pro)
{
    const DecodePro none{};
    if (pro) {
        if (theta) return hipErrorInvalidValue;
        if (io == IoType::F32)
            return launch_decode_cols<float, false, true>(B, H, Dk, Dv, q, k, v, alpha, nullptr, beta, state, out, stream, *pro);
        return launch_decode_cols<bf16_t, false, true>(B, H, Dk, Dv, q, k, v, alpha, nullptr, beta, state, out, stream, *pro);
    }
    if (theta) {
        if (io == IoType::F32)
            return launch_decode_cols<float, true, false>(B, H, Dk, Dv, q, k, v, alpha, theta, beta, state, out, stream, none);
        return launch_decode_cols<bf16_t, true, false>(B, H, Dk, Dv, q, k, v, alpha, theta, beta, state, out, stream, none);
    }
    if (io == IoType::F32)
        return launch_decode_cols<float, false, false>(B, H, Dk, Dv, q, k, v, alpha, nullptr, beta, state, out, stream, none);
    return launch_decode_cols<bf16_t, false, false>(B, H, Dk, Dv, q, k, v, alpha, nullptr, beta, state, out, stream, none);
}

}  // namespace kda
