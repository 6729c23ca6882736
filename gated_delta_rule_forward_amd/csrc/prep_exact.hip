// prep_exact.hip — exact per-chunk WY factors for chunks the fast kernel
// flags (a half span of the log decay too wide for the midpoint factorisation,
// or more zero gates than extra columns).  Same outputs as prep_fast.hip, but
// every decay ratio is a running product of gates that starts at a reference
// token, so |factor| <= 1 everywhere and zero or negative gates are carried
// exactly, at the cost of per-pair VALU work on the 16x16 diagonal blocks:
//  - off-diagonal 16x16 blocks of A and P (rows in block a, columns before
//    it): rho(r,i) = rho(r,e) rho(e,i) with e the last token before block a,
//    one MFMA product of (K or Q) * rho(.,e) with K * rho(e,.);
//  - diagonal 16x16 blocks: per pair, a running product over the block;
//  - Tinv = (I + A)^{-1} by forward substitution (one wavefront, lane j owns
//    column j).
// A grid of at most 256 workgroups (one per CU) covers all chunks: each
// workgroup reads the flags of its chunks (blockIdx.x, blockIdx.x + gridDim.x,
// ...) together, lists the flagged ones in LDS and then works through that
// list, so a launch with nothing flagged costs one round of flag loads.
#include "kda_chunk.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace {

constexpr int kPrepThreads = 256;

template <typename T, int C, int DK>
struct PrepLds {
    static constexpr int NB = C / 16;                      // 16-token blocks per chunk
    static constexpr int DVMAX = 128;
    static constexpr int KG_ROWS = 16 * NB * (NB - 1) / 2;  // sum over a of 16a
    // fp32 with Dk = 128: the off-diagonal factor tables are built and
    // contracted for half the channels at a time (CH passes of DKH channels),
    // and beta K * Gamma (X) is written over the staged Q (each channel's
    // column once its own tables are built), so the whole layout fits 160 KB
    static constexpr bool BIG = sizeof(T) == 4 && DK == 128;
    static constexpr int CH = BIG ? 2 : 1;
    static constexpr int DKH = DK / CH;
    static constexpr size_t al16(size_t x) { return (x + 15) & ~size_t(15); }
    static constexpr size_t K = 0;                                   // T[C][DK]
    static constexpr size_t Q = al16(K + sizeof(T) * C * DK);        // T[C][DK]
    static constexpr size_t A = al16(Q + sizeof(T) * C * DK);        // float[C][C]
    static constexpr size_t BETA = al16(A + 4 * C * C);              // float[C]
    static constexpr size_t X = BIG ? Q : al16(BETA + 4 * C);        // T[C][DK]
    static constexpr size_t TI = BIG ? al16(BETA + 4 * C) : al16(X + sizeof(T) * C * DK);   // T[C][C]
    static constexpr size_t UNI = al16(TI + sizeof(T) * C * C);      // union
    // union members
    static constexpr size_t SZ_AL = 4 * C * DK;                                    // float[C][DK]
    static constexpr size_t KF = 0;                                                // T[NB-1][16][DKH]
    static constexpr size_t QF = al16(KF + sizeof(T) * 16 * (NB > 1 ? NB - 1 : 0) * DKH);
    static constexpr size_t KG = al16(QF + sizeof(T) * 16 * (NB > 1 ? NB - 1 : 0) * DKH);
    static constexpr size_t SZ_FAC = al16(KG + sizeof(T) * KG_ROWS * DKH);
    static constexpr size_t SZ_Y = sizeof(T) * C * DVMAX;                          // T[C][DVMAX]
    static constexpr size_t SZ_UNI =
        SZ_AL > SZ_FAC ? (SZ_AL > SZ_Y ? SZ_AL : SZ_Y) : (SZ_FAC > SZ_Y ? SZ_FAC : SZ_Y);
    static constexpr size_t TOTAL = al16(UNI + SZ_UNI);
    static_assert(TOTAL <= 160 * 1024, "LDS of one workgroup");
};


// C = A * B with A row-major [m][k] (vector loads) and B row-major [k][n]
// (four scalar loads per k16 block), K a multiple of 16.
template <typename T>
__device__ __forceinline__ f32x4 tile_nn(const T* A, int lda, const T* B, int ldb, int K, f32x4 acc) {
    const int lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const T* pa = A + r * lda + 4 * g;
    const T* pb = B + (4 * g) * ldb + r;
    for (int k0 = 0; k0 < K; k0 += 16) {
        float bf[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) bf[j] = to_f32(pb[(k0 + j) * ldb]);
        acc = mma_k16(Vec4<T>::load(pa + k0), Vec4<T>::from(bf), acc);
    }
    return acc;
}

template <typename T, int C, int DK>
__global__ __launch_bounds__(kPrepThreads) void prep_exact_kernel(PrepArgs args, int NU)
{
    constexpr int KB = KBlock<T, C, DK>::value;
    using L = PrepLds<T, C, DK>;
    constexpr int NB = L::NB;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    T* sK = reinterpret_cast<T*>(lds + L::K);
    T* sQ = reinterpret_cast<T*>(lds + L::Q);
    float* sA = reinterpret_cast<float*>(lds + L::A);
    float* sBeta = reinterpret_cast<float*>(lds + L::BETA);
    T* sX = reinterpret_cast<T*>(lds + L::X);
    T* sTi = reinterpret_cast<T*>(lds + L::TI);
    unsigned char* uni = lds + L::UNI;
    float* sAl = reinterpret_cast<float*>(uni);
    T* sKF = reinterpret_cast<T*>(uni + L::KF);
    T* sQF = reinterpret_cast<T*>(uni + L::QF);
    T* sKG = reinterpret_cast<T*>(uni + L::KG);
    T* sY = reinterpret_cast<T*>(uni);

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, ln = lane & 15, lg = lane >> 4;
    const int T_ = args.T, H = args.H, Dv = args.Dv, NC = args.NC;
    __shared__ int sList[kPrepThreads];
    __shared__ int sCount;
    const int nper = (NU - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
    for (int base = 0; base < nper; base += kPrepThreads) {
    if (tid == 0) sCount = 0;
    __syncthreads();
    if (base + tid < nper) {
        const int u = part_unit((int)blockIdx.x + (base + tid) * (int)gridDim.x,
                                args.pc0, args.pcn, NC);
        if (args.FL[u] != 0) sList[atomicAdd(&sCount, 1)] = u;
    }
    __syncthreads();
    const int nlist = sCount;
    for (int li = 0; li < nlist; ++li) {
    const int unit = sList[li];
    const UnitPos up = locate_unit(unit, H, T_, NC, C, args.cu, args.cs, args.N);
    const int h = up.h, nvalid = up.nvalid, row0 = up.row0;

    const T* __restrict__ gq = static_cast<const T*>(args.q);
    const T* __restrict__ gk = static_cast<const T*>(args.k);
    const T* __restrict__ gv = static_cast<const T*>(args.v);
    T* __restrict__ Wg = static_cast<T*>(args.W) + (size_t)unit * C * DK;
    T* __restrict__ Ug = static_cast<T*>(args.U) + (size_t)unit * C * Dv;
    T* __restrict__ Ktg = static_cast<T*>(args.Kt) + (size_t)unit * DK * C;
    T* __restrict__ QGg = static_cast<T*>(args.QG) + (size_t)unit * C * DK;
    T* __restrict__ Pg = static_cast<T*>(args.P) + (size_t)unit * C * C;
    float* __restrict__ GCg = args.GC + (size_t)unit * DK;

    // ---- phase 1: stage k, q, alpha, beta of the chunk (tail rows: k = q = 0,
    //      alpha = 1, beta = 0, which makes them exact no-ops) -------------------
    {
        constexpr int VPR = DK * (int)sizeof(T) / 16;        // 16-byte vectors per row
        for (int idx = tid; idx < C * VPR; idx += kPrepThreads) {
            const int r = idx / VPR, vi = idx % VPR;
            uint4 kv = {0u, 0u, 0u, 0u}, qv = {0u, 0u, 0u, 0u};
            if (r < nvalid) {
                const size_t g = (((size_t)row0 + r) * H + h) * DK;
                kv = reinterpret_cast<const uint4*>(gk + g)[vi];
                qv = reinterpret_cast<const uint4*>(gq + g)[vi];
            }
            reinterpret_cast<uint4*>(sK + r * DK)[vi] = kv;
            reinterpret_cast<uint4*>(sQ + r * DK)[vi] = qv;
        }
        constexpr int VPA = DK / 4;
        for (int idx = tid; idx < C * VPA; idx += kPrepThreads) {
            const int r = idx / VPA, vi = idx % VPA;
            float4 av = make_float4(1.f, 1.f, 1.f, 1.f);
            if (r < nvalid) {
                if (args.theta) {        // phase variant: one gate per channel pair
                    const float2 a2 = reinterpret_cast<const float2*>(
                        args.alpha + (((size_t)row0 + r) * H + h) * (DK / 2))[vi];
                    av = make_float4(a2.x, a2.x, a2.y, a2.y);
                } else {
                    av = reinterpret_cast<const float4*>(args.alpha + (((size_t)row0 + r) * H + h) * DK)[vi];
                }
            }
            reinterpret_cast<float4*>(sAl + r * DK)[vi] = av;
        }
        for (int r = tid; r < C; r += kPrepThreads)
            sBeta[r] = r < nvalid ? args.beta[((size_t)row0 + r) * H + h] : 0.f;
    }
    __syncthreads();
    __shared__ float sPhEnd[64];       // (phase variant) summed phase of each pair
    if (args.theta) {
        // rotate k_r, q_r of every pair by -phi_r (phi_r: the pair's phases
        // summed over tokens 0..r of the chunk), so that the decay-weighted
        // products below are the plain ones of the rotated vectors; Ktil and
        // Gamma_{C-1} are rotated back by phi_{C-1} when they are stored
        for (int p = tid; p < DK / 2; p += kPrepThreads) {
            float ph = 0.f;
            for (int r = 0; r < nvalid; ++r) {
                ph += args.theta[(((size_t)row0 + r) * H + h) * (DK / 2) + p];
                float sn, cs;
                __sincosf(ph, &sn, &cs);
                T* kr = sK + r * DK + 2 * p;
                T* qr = sQ + r * DK + 2 * p;
                const float k0 = to_f32(kr[0]), k1 = to_f32(kr[1]), q0 = to_f32(qr[0]), q1 = to_f32(qr[1]);
                kr[0] = from_f32<T>(cs * k0 + sn * k1);
                kr[1] = from_f32<T>(cs * k1 - sn * k0);
                qr[0] = from_f32<T>(cs * q0 + sn * q1);
                qr[1] = from_f32<T>(cs * q1 - sn * q0);
            }
            sPhEnd[p] = ph;
        }
        __syncthreads();
    }
    if (args.pro) {
        // raw inputs: gate range eq. (15), beta eq. (17), unit-norm keys (and
        // queries) eq. (18) ("Semidirect Fourier Delta Attention" §3), on the
        // valid rows only (tail rows stay no-ops)
        for (int idx = tid; idx < nvalid * DK; idx += kPrepThreads)
            sAl[idx] = args.amin + args.arange * sigmoid_f32(sAl[idx]);
        for (int r = tid; r < nvalid; r += kPrepThreads) sBeta[r] = args.bmax * sigmoid_f32(sBeta[r]);
        for (int r = wave; r < nvalid; r += kPrepThreads / 64) {
            for (int m = 0; m < (args.normq ? 2 : 1); ++m) {
                T* row = (m == 0 ? sK : sQ) + r * DK;
                float ss = 0.f;
                for (int c = lane; c < DK; c += 64) ss += to_f32(row[c]) * to_f32(row[c]);
#pragma unroll
                for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
                const float nrm = __builtin_sqrtf(ss) + args.eps;
                const float inv = nrm > 0.f ? 1.f / nrm : 0.f;
                for (int c = lane; c < DK; c += 64) row[c] = from_f32<T>(to_f32(row[c]) * inv);
            }
        }
        __syncthreads();
    }

    // ---- phase 2: diagonal 16x16 blocks of A and P, one running product per
    //      (column i, channel): thread (i = tid/16, channel group tid%16) ----------
    {
        constexpr int CPG = DK / 16;
        const int di = tid >> 4, cg = tid & 15, ch0 = cg * CPG;
        for (int blk = 0; blk < NB; ++blk) {
            const int s = blk * 16;
            float p[CPG];
#pragma unroll
            for (int x = 0; x < CPG; ++x) p[x] = to_f32(sK[(s + di) * DK + ch0 + x]);
            float aout = 0.f, pout = 0.f;
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                const int r = s + rr;
                if (rr > di) {
#pragma unroll
                    for (int x = 0; x < CPG; ++x) p[x] *= sAl[r * DK + ch0 + x];
                }
                float da = 0.f, dq = 0.f;
#pragma unroll
                for (int x = 0; x < CPG; ++x) {
                    da += to_f32(sK[r * DK + ch0 + x]) * p[x];
                    dq += to_f32(sQ[r * DK + ch0 + x]) * p[x];
                }
                da = row16_sum(da);
                dq = row16_sum(dq);
                if (rr == cg) { aout = da; pout = dq; }
            }
            // lane cg owns entry (row s+cg, column s+di)
            if (cg > di) sA[(s + cg) * C + s + di] = sBeta[s + cg] * aout;
            Pg[frag_off<KB>(s + cg, s + di, C)] = from_f32<T>(cg >= di ? pout : 0.f);
        }
    }

    // ---- phase 3: per-channel decay factors from reference tokens ------------
    float a[C];
    if (tid < DK) {
#pragma unroll
        for (int r = 0; r < C; ++r) a[r] = sAl[r * DK + tid];
    }
    __syncthreads();   // sAl is dead from here on (the union is reused)
    if (tid < DK) {
        const int c = tid;
        // Gamma_r = rho(r, -1): Q*Gamma (global) and diag(beta) K*Gamma (LDS;
        // written in the table pass below when X shares Q's space)
        float gm = 1.f;
#pragma unroll
        for (int r = 0; r < C; ++r) {
            gm *= a[r];
            const float kr = to_f32(sK[r * DK + c]), qr = to_f32(sQ[r * DK + c]);
            QGg[frag_off<KB>(r, c, DK)] = from_f32<T>(qr * gm);
            if constexpr (!L::BIG) sX[r * DK + c] = from_f32<T>(sBeta[r] * kr * gm);
        }
        // Ktil_i = k_i rho(C-1, i), stored transposed (row c), 16-byte stores
        float kt[C];
        float e = 1.f;
#pragma unroll
        for (int i = C - 1; i >= 0; --i) {
            kt[i] = to_f32(sK[i * DK + c]) * e;
            e *= a[i];
        }
        if (args.theta) {
            // rotate back by phi_{C-1}: channel c pairs with lane c ^ 1
            float sn, cs;
            __sincosf(sPhEnd[c >> 1], &sn, &cs);
            const float sg = (c & 1) ? 1.f : -1.f;    // even: c x0 - s x1, odd: s x0 + c x1
#pragma unroll
            for (int i = 0; i < C; ++i) {
                const float other = __shfl_xor(kt[i], 1);
                kt[i] = cs * kt[i] + sg * sn * other;
            }
            const float go = __shfl_xor(gm, 1);
            gm = (c & 1) ? sn * go : cs * gm;           // (|G| cos, |G| sin); |G| equal in a pair
        }
        GCg[c] = gm;
#pragma unroll
        for (int i = 0; i < C; ++i) Ktg[frag_off<KB>(c, i, C)] = from_f32<T>(kt[i]);
    }

    // ---- phase 3b / 4: off-diagonal blocks of A and P, CH channel passes -------
    // pass hh: the channels [hh DKH, (hh + 1) DKH) write their factor tables
    // (off-diagonal block a: rows r in block a scaled by rho(r, e_a), columns
    // i < 16a by rho(e_a, i), e_a = 16a - 1), then every wave adds the pass's
    // contraction to its tiles' accumulators
    constexpr int NTILE = NB * (NB - 1);             // (a, b < a, A or P) tiles
    constexpr int TPW = NTILE > 0 ? (NTILE + 3) / 4 : 1;
    f32x4 acc4[TPW];
#pragma unroll
    for (int j = 0; j < TPW; ++j) acc4[j] = zero4();
#pragma unroll
    for (int hh = 0; hh < L::CH; ++hh) {
        __syncthreads();   // (hh = 0: sAl dead; hh > 0: the previous tables read)
        if (tid >= hh * L::DKH && tid < (hh + 1) * L::DKH) {
            const int c = tid, cc = c - hh * L::DKH;
#pragma unroll
            for (int ab = 1; ab < NB; ++ab) {
                float f = 1.f;
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) {
                    const int r = 16 * ab + rr;
                    f *= a[r];
                    sKF[((ab - 1) * 16 + rr) * L::DKH + cc] = from_f32<T>(to_f32(sK[r * DK + c]) * f);
                    sQF[((ab - 1) * 16 + rr) * L::DKH + cc] = from_f32<T>(to_f32(sQ[r * DK + c]) * f);
                }
                T* kg = sKG + 16 * (ab * (ab - 1) / 2) * L::DKH;
                float gg = 1.f;
#pragma unroll
                for (int i = 16 * ab - 1; i >= 0; --i) {
                    kg[i * L::DKH + cc] = from_f32<T>(to_f32(sK[i * DK + c]) * gg);
                    gg *= a[i];
                }
            }
            if constexpr (L::BIG) {
                // this channel's Q column is no longer read: X takes its place
                float gx = 1.f;
#pragma unroll
                for (int r = 0; r < C; ++r) {
                    gx *= a[r];
                    sX[r * DK + c] = from_f32<T>(sBeta[r] * to_f32(sK[r * DK + c]) * gx);
                }
            }
        }
        __syncthreads();
        int tile = 0;
#pragma unroll
        for (int ab = 1; ab < NB; ++ab) {
            const T* kg = sKG + 16 * (ab * (ab - 1) / 2) * L::DKH;
#pragma unroll
            for (int bb = 0; bb < ab; ++bb) {
#pragma unroll
                for (int kind = 0; kind < 2; ++kind, ++tile) {
                    if ((tile & 3) != wave) continue;
                    const T* op = (kind == 0 ? sKF : sQF) + (ab - 1) * 16 * L::DKH;
                    acc4[tile >> 2] = tile_tn(op, L::DKH, kg + 16 * bb * L::DKH, L::DKH, L::DKH,
                                              acc4[tile >> 2]);
                }
            }
        }
    }
    {
        int tile = 0;
#pragma unroll
        for (int ab = 1; ab < NB; ++ab) {
#pragma unroll
            for (int bb = 0; bb < ab; ++bb) {
#pragma unroll
                for (int kind = 0; kind < 2; ++kind, ++tile) {
                    if ((tile & 3) != wave) continue;
                    const f32x4 acc = acc4[tile >> 2];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = 16 * ab + 4 * lg + i, col = 16 * bb + ln;
                        if (kind == 0) sA[r * C + col] = sBeta[r] * acc[i];
                        else Pg[frag_off<KB>(r, col, C)] = from_f32<T>(acc[i]);
                    }
                }
            }
        }
        // P above its block diagonal is zero
        for (int idx = tid; idx < C * C; idx += kPrepThreads) {
            const int r = idx / C, col = idx % C;
            if ((col >> 4) > (r >> 4)) Pg[frag_off<KB>(r, col, C)] = from_f32<T>(0.f);
        }
    }
    __syncthreads();

    // ---- phase 5: Tinv = (I + A)^{-1} by forward substitution (wave 0, lane j
    //      owns column j); the other waves stage diag(beta) V ------------------
    if (wave == 0) {
        const int j = lane;
        if (j < C) {
            float t[C];
#pragma unroll
            for (int r = 0; r < C; ++r) {
                float s = (r == j) ? 1.f : 0.f;
#pragma unroll
                for (int i = 0; i < r; ++i) s -= sA[r * C + i] * t[i];
                t[r] = s;
            }
#pragma unroll
            for (int r = 0; r < C; ++r) sTi[r * C + j] = from_f32<T>(t[r]);
            if (args.Tm) {
                float* tg = args.Tm + (size_t)unit * C * C;
#pragma unroll
                for (int r = 0; r < C; ++r) tg[r * C + j] = t[r];
            }
        }
    } else {
        const int VPR = Dv / 4;    // groups of 4 elements
        for (int idx = tid - 64; idx < C * VPR; idx += kPrepThreads - 64) {
            const int r = idx / VPR, c4 = (idx % VPR) * 4;
            float y[4] = {0.f, 0.f, 0.f, 0.f};
            if (r < nvalid) {
                const T* src = gv + (((size_t)row0 + r) * H + h) * Dv + c4;
                const float bt = sBeta[r];
#pragma unroll
                for (int x = 0; x < 4; ++x) y[x] = bt * to_f32(src[x]);
            }
            *reinterpret_cast<Vec4<T>*>(sY + r * Dv + c4) = Vec4<T>::from(y);
        }
    }
    __syncthreads();

    // ---- phase 6: W = Tinv X, U = Tinv Y (MFMA) --------------------------------
    {
        constexpr int NM = C / 16, NW = DK / 16;
        const int NU = Dv / 16;
        const int ntiles = NM * (NW + NU);
        for (int tile = wave; tile < ntiles; tile += 4) {
            const int mt = tile % NM, ct = tile / NM;
            if (ct < NW) {
                const f32x4 acc = tile_nn(sTi + 16 * mt * C, C, sX + 16 * ct, DK, C, zero4());
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    Wg[frag_off<KB>(16 * mt + 4 * lg + i, 16 * ct + ln, DK)] = from_f32<T>(acc[i]);
            } else {
                const int ut = ct - NW;
                const f32x4 acc = tile_nn(sTi + 16 * mt * C, C, sY + 16 * ut, Dv, C, zero4());
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    Ug[u_off(16 * mt + 4 * lg + i, 16 * ut + ln, Dv)] = from_f32<T>(acc[i]);
            }
        }
    }
    __syncthreads();   // LDS is reused by the next flagged unit
    }
    }
}


template <typename T, int C, int DK>
hipError_t launch_exact_t(const ChunkShape& s, const PrepArgs& a, hipStream_t stream)
{
    using L = PrepLds<T, C, DK>;
    auto kern = prep_exact_kernel<T, C, DK>;
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)L::TOTAL);
    if (e != hipSuccess) return e;
    const int nu = (int)((size_t)s.B * s.H * (a.pcn > 0 ? a.pcn : s.NC));
    const int grid = nu < 256 ? nu : 256;   // one workgroup per CU (LDS-bound)
    return launch_kernel(kern, dim3(grid), dim3(kPrepThreads), (uint32_t)L::TOTAL, stream, a, nu);
}

template <typename T, int C>
hipError_t dispatch_dk(const ChunkShape& s, const PrepArgs& a, hipStream_t st)
{
    switch (s.Dk) {
    case 16: return launch_exact_t<T, C, 16>(s, a, st);
    case 32: return launch_exact_t<T, C, 32>(s, a, st);
    case 64: return launch_exact_t<T, C, 64>(s, a, st);
    case 128: return launch_exact_t<T, C, 128>(s, a, st);
    default: return hipErrorInvalidValue;
    }
}

template <typename T>
hipError_t dispatch_c(const ChunkShape& s, const PrepArgs& a, hipStream_t st)
{
    switch (s.C) {
    case 16: return dispatch_dk<T, 16>(s, a, st);
    case 32: return dispatch_dk<T, 32>(s, a, st);
    case 64: return dispatch_dk<T, 64>(s, a, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_prep_exact(IoType io, const ChunkShape& s, const PrepArgs& a, hipStream_t stream)
{
    if (io == IoType::F32) return dispatch_c<float>(s, a, stream);
    return dispatch_c<bf16_t>(s, a, stream);
}

}  // namespace kda
