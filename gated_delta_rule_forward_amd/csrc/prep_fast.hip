// prep_fast.hip — per-chunk WY factors (the parallel part of the chunkwise
// forward), all chunks of all (b, h) at once, one 256-thread workgroup each.
//
// Within a chunk of C tokens (S = state entering the chunk), with
// rho(r,i) = prod_{j=i+1..r} alpha_j per channel and Gamma_r = rho(r,-1):
//   A[r,i] = beta_r sum_c k_rc k_ic rho(r,i)_c   (i < r)     Tinv = (I + A)^{-1}
//   W = Tinv diag(beta)(K * Gamma)   U = Tinv diag(beta) V
//   P[r,i] = sum_c q_rc k_ic rho(r,i)_c          (i <= r)
//   QG = Q * Gamma,  Ktil_i = k_i * rho(C-1, i),  GC = Gamma_{C-1}
// (chunkwise execution and its exactness: "Kimi Delta Attention: a bounded
// case study", Exercise 2; the compact WY form via a triangular solve:
// "Semidirect Fourier Delta Attention", §1 and §2.2.)
//
// Gate summary first (the chunk-local log-magnitude / sign / zero form, per
// channel): L_r = sum_{j<=r, alpha_j != 0} log2|alpha_j|, parity_r, and the
// zero count seg_r = #{j <= r : alpha_j == 0}.  Then for i <= r
//   rho(r,i) = [seg_r == seg_i] (-1)^(parity_r + parity_i) 2^(L_r - L_i).
// A and P need every pair, so each channel is factored through its midpoint
// M = L_{C-1} / 2:  2^(L_r - L_i) = 2^(L_r - M) 2^(M - L_i), and each zero-free
// segment of a channel becomes its own contraction column ("virtual channel":
// segment 0 stays in column c, later segments get extra columns), so pairs
// across a zero gate meet only zeros and stay exactly zero.  A and P are then
// one MFMA product each over Dk + (#zeros) columns, contracted Dk columns at a
// time: the Dk main columns first, then the extra columns in passes of Dk
// that reuse the same operand region, so the LDS size does not depend on the
// zero count.  A chunk whose half span max|L_r - M| exceeds 96 (factors could
// leave the normal range) or whose zero count exceeds the allowed extra
// columns is flagged for the exact kernel (prep_exact.hip) instead.
//
// Tinv is a blocked inverse over 16x16 diagonal blocks (fp32 MFMA):
//   T_aa = (I + A_aa)^{-1} by forward substitution,
//   T_ab = -T_aa sum_{j=b..a-1} A_aj T_jb   (a > b, by block distance).
//
// Outputs go out fragment-major (kda_chunk.hpp): P and W are produced as
// transposed tiles (P^T = Y X_P^T, W^T = X_W^T Tinv^T), whose C-layout
// accumulators are exactly the A fragments the chain kernel consumes, so each
// lane stores one contiguous 16-byte fragment.  Q*Gamma and (without zero
// segments) Ktil are read back from the LDS operands (q F, k G) and scaled per
// channel, one whole fragment per lane store; with zero segments the thread
// that owns (channel quad, tokens) writes its Ktil fragment slots directly.
//
// LDS is one region reused phase by phase (gate summary, A/P operands, A and
// Tinv, X_W^T and (beta V)^T), about 52 KB for bf16 C = 64, Dk = 128 without
// extra columns, so three workgroups share a CU.
#include "kda_chunk.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace {

constexpr int kThreads = 256;

// Store of a workspace block written as whole fragments (P, W: 1 KB per
// wavefront; U: 512 B), non-temporal in the NT kernel variant (PrepArgs ntst:
// many chains stream the workspace; a compile-time choice, since a run-time
// branch between two equal stores is merged into one plain store).  Measured at H=32, T=8192, d=128
// (256 chains): prep 140 -> 144 us but chain 158 -> 145 us; with 16 chains
// (H=2, T=65536) the chain was 4-10 % slower, so few chains keep ordinary
// stores.  Never for the 8-byte Q*Gamma / Ktil pieces: those rely on write
// combining in L2 (prep 140 -> 398 us as non-temporal stores).
typedef unsigned nt_u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned nt_u32x2 __attribute__((ext_vector_type(2)));
template <bool NT, typename V>
__device__ __forceinline__ void store_ws(void* p, const V& v)
{
    static_assert(sizeof(V) == 16 || sizeof(V) == 8, "16 or 8 bytes");
    if constexpr (!NT)
        *reinterpret_cast<V*>(p) = v;
    else if constexpr (sizeof(V) == 16)
        __builtin_nontemporal_store(__builtin_bit_cast(nt_u32x4, v), reinterpret_cast<nt_u32x4*>(p));
    else
        __builtin_nontemporal_store(__builtin_bit_cast(nt_u32x2, v), reinterpret_cast<nt_u32x2*>(p));
}
constexpr float kHalfSpanMax = 96.f;
constexpr float kMinPart = 0x1p-120f;   // smallest product of one token range's gates

template <typename T, int C, int DK>
struct FastGeom {
    static constexpr int KB = KBlock<T, C, DK>::value;
    static constexpr int NV = KB / 4;                         // fragment slots per lane
    static constexpr int TPB = KB / 16;                       // 16-wide tiles per k block
    static constexpr int NQ = DK / 4;                         // channel quads
    static constexpr int PARTS = (kThreads / NQ) < C ? (kThreads / NQ) : C;   // token ranges
    static constexpr int TOK = C / PARTS;                     // tokens per thread
    static constexpr int ACTIVE = NQ * PARTS;                 // threads that own elements
    static constexpr int PADE = 16 / (int)sizeof(T);          // 16-byte row pad
    static constexpr int LDF = C + 4;                         // row stride of fp32 A / Tinv
    static constexpr int NB = C / 16;
    static constexpr int DVMAX = 128;
    static constexpr int XTS = C + PADE;                      // row stride of X_W^T, (beta V)^T
    static constexpr int TV = 16 / (int)sizeof(T);            // tokens per 16-byte run of a V^T row
    // V items: (column quad, run of TV tokens); at most VIT per thread
    static constexpr int VIT = ((DVMAX / 4) * (C / TV) + kThreads - 1) / kThreads;
};

template <typename T, int C, int DK>
struct FastLayout {
    static constexpr int KS = DK + FastGeom<T, C, DK>::PADE;   // operand row stride (elements)
    size_t scr, total;
    // one region reused phase by phase (offsets from 0):
    //   gate summary: partL, partPZ [PARTS][DK] fp32 / int
    //   A / P:        XA, XP, Y [C][KS] io type (one contraction pass of DK columns)
    //   Tinv:         A, Tinv [C][LDF] fp32
    //   W / U:        X_W^T [DK][XTS], (beta V)^T [DVMAX][XTS] io type
    __host__ __device__ FastLayout() {
        using G = FastGeom<T, C, DK>;
        const size_t e = sizeof(T);
        const size_t r1 = (size_t)2 * G::PARTS * DK * 4 + (size_t)G::PARTS * (DK / 2) * 4;
        const size_t r2 = 3 * (size_t)C * KS * e;
        const size_t r3 = (size_t)2 * C * G::LDF * 4;
        const size_t r4 = (size_t)(DK + G::DVMAX) * G::XTS * e;
        size_t r = r1 > r2 ? r1 : r2;
        r = r > r3 ? r : r3;
        r = r > r4 ? r : r4;
        scr = (r + 15) & ~size_t(15);
        // base [DK] (phase variant without zero segments: cos, sin of each
        // pair's chunk phase), misc [8], beta [C], stot E [DK]
        total = scr + (DK + 8 + C + DK) * 4;
        total = (total + 15) & ~size_t(15);
    }
};

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float flog2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float frcp(float x) { return __builtin_amdgcn_rcpf(x); }

// ZS: the chunk may hold zero gates, placed in extra contraction columns (the
// launch passes ZS = true exactly when extra columns are allotted); without
// them a zero gate makes a part product vanish and flags the chunk.
// PRO: the inputs are raw (gate and beta logits, unnormalised q and k) and go
// through the parameterisation first.
// PH: phase variant: channels 2p, 2p+1 decay by alpha_p R(theta_p) (gates and
// phases per pair).  With phi_r the summed phase of the chunk's tokens up to
// r, rho(r, i) = |rho| R(phi_r - phi_i), so rotating every k_r and q_r by
// -phi_r turns every decay-weighted product into the real one of the plain
// kernel on the rotated vectors; Ktil is rotated back by phi_{C-1} and
// Gamma_{C-1} is stored as (|Gamma| cos phi_{C-1}, |Gamma| sin phi_{C-1}).
// One unit (one chunk of one (b, h)) by the whole workgroup.  Every thread
// returns from it at the same point.
template <typename T, int C, int DK, bool ZS, bool PRO, bool PH, bool NT>
__device__ __forceinline__ bool prep_fast_unit(const PrepArgs& args, const int unit)
{
    using G = FastGeom<T, C, DK>;
    using F = Frag<T, G::KB>;
    constexpr int KB = G::KB, NV = G::NV, TPB = G::TPB, PARTS = G::PARTS, TOK = G::TOK;
    constexpr int NB = G::NB, LDF = G::LDF, XTS = G::XTS, TV = G::TV;
    constexpr int NKD = DK / KB, NKC = C / KB;
    const int Dv = args.Dv;
    const FastLayout<T, C, DK> LY;
    constexpr int KS = FastLayout<T, C, DK>::KS;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    float* partL = reinterpret_cast<float*>(lds);                           // gate summary
    int* partPZ = reinterpret_cast<int*>(partL + PARTS * DK);               // nz << 1 | parity
    float* partPh = partL + 2 * PARTS * DK;                                 // (PH) [PARTS][DK/2]
    T* XA = reinterpret_cast<T*>(lds);                                      // A / P operands
    T* XP = XA + C * KS;
    T* Y = XP + C * KS;
    float* sA = reinterpret_cast<float*>(lds);                              // Tinv phase
    float* sT = sA + C * LDF;
    T* sXWt = reinterpret_cast<T*>(lds);                                    // X_W^T [DK][XTS]
    T* sVt = sXWt + DK * XTS;                                               // (beta V)^T [Dv][XTS]
    int* sBase = reinterpret_cast<int*>(lds + LY.scr);
    int* misc = sBase + DK;
    float* sBeta = reinterpret_cast<float*>(misc + 8);
    float* sRE = sBeta + C;            // per channel: the chunk product's sign times E = 2^M (> 0)
    float* sRot = reinterpret_cast<float*>(sBase);   // (phase, no zero segments) cos, sin per pair

    int tid_ = threadIdx.x;
    // (opaque per unit: in the persistent grid this keeps the compiler from
    // hoisting every per-thread index out of the unit loop and holding it live
    // across the whole body, which spills)
    asm volatile("" : "+v"(tid_));
    const int tid = tid_;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, ln = lane & 15, lg = lane >> 4;
    const bool own = tid < G::ACTIVE;
    const int q4 = tid % G::NQ, part = own ? tid / G::NQ : PARTS - 1;
    const int c0 = 4 * q4;                                    // my channels c0 .. c0+3
    const int T_ = args.T, H = args.H, NC = args.NC;
    const UnitPos up = locate_unit(unit, H, T_, NC, C, args.cu, args.cs, args.N);
    if (!up.valid) {                  // past the last sequence of a packed batch
        if (tid == 0) args.FL[unit] = 0;
        return false;
    }
    const int h = up.h, nvalid = up.nvalid;

    const size_t tok0 = (size_t)up.row0 * H + h;          // first token of the unit, head h
    const T* gq = static_cast<const T*>(args.q) + tok0 * DK;
    const T* gk = static_cast<const T*>(args.k) + tok0 * DK;
    const float* ga = args.alpha + tok0 * DK;
    const T* gv = static_cast<const T*>(args.v) + tok0 * Dv;
    const float* gb = args.beta + tok0;
    const int rs = H * DK, rsv = H * Dv;                    // token strides
    T* Wg = static_cast<T*>(args.W) + (size_t)unit * C * DK;
    T* Ug = static_cast<T*>(args.U) + (size_t)unit * C * Dv;
    T* Ktg = static_cast<T*>(args.Kt) + (size_t)unit * DK * C;
    T* QGg = static_cast<T*>(args.QG) + (size_t)unit * C * DK;
    T* Pg = static_cast<T*>(args.P) + (size_t)unit * C * C;

    // ---- loads: my 4 channels over my TOK tokens (k, q kept in io precision) ----
    // (rows past the end re-read the last valid row and become no-op tokens;
    // the inputs are read once, so the loads are non-temporal)
    float al[TOK][4], bt[TOK];
    float th[TOK][2];                  // (PH) the phases of my two channel pairs
    Vec4<T> kv[TOK], qv[TOK];
#pragma unroll
    for (int j = 0; j < TOK; ++j) {
        const int r = min(part * TOK + j, nvalid - 1);
        if constexpr (PH) {
            const float2 a2 = *reinterpret_cast<const float2*>(args.alpha + (tok0 + (size_t)r * H) * (DK / 2) + c0 / 2);
            const float2 t2 = *reinterpret_cast<const float2*>(args.theta + (tok0 + (size_t)r * H) * (DK / 2) + c0 / 2);
            al[j][0] = al[j][1] = a2.x;
            al[j][2] = al[j][3] = a2.y;
            th[j][0] = t2.x;
            th[j][1] = t2.y;
        } else {
            const f32x4 a4 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(ga + r * rs + c0));
            al[j][0] = a4[0]; al[j][1] = a4[1]; al[j][2] = a4[2]; al[j][3] = a4[3];
        }
        kv[j] = Vec4<T>::load_nt(gk + r * rs + c0);
        qv[j] = Vec4<T>::load_nt(gq + r * rs + c0);
        bt[j] = gb[r * H];
    }
    if constexpr (PRO) {
        // eq. (15) gate range, eq. (17) beta, eq. (18) unit-norm keys (and queries)
#pragma unroll
        for (int j = 0; j < TOK; ++j) {
#pragma unroll
            for (int x = 0; x < 4; ++x) al[j][x] = args.amin + args.arange * sigmoid_f32(al[j][x]);
            bt[j] = args.bmax * sigmoid_f32(bt[j]);
            kv[j] = l2_normalised<T, G::NQ>(kv[j], args.eps);
            if (args.normq) qv[j] = l2_normalised<T, G::NQ>(qv[j], args.eps);
        }
    }
#pragma unroll
    for (int j = 0; j < TOK; ++j) {
        if (part * TOK + j >= nvalid) {
            bt[j] = 0.f;
            kv[j] = Vec4<T>::zero();
            qv[j] = Vec4<T>::zero();
            if constexpr (PH) { th[j][0] = 0.f; th[j][1] = 0.f; }
#pragma unroll
            for (int x = 0; x < 4; ++x) al[j][x] = 1.f;
        }
    }

    // ---- gate summary in product form: per channel, the running product of the
    //      (nonzero) gates over my tokens, signs included, and the zero count;
    //      the part totals enter a log2 magnitude / parity / zero-count summary
    //      combined across token ranges through LDS -------------------------------
    float pr[TOK][4];
    unsigned zc[TOK];                  // (ZS) byte x: zeros of channel c0 + x so far in my range
    float cur[4] = {1.f, 1.f, 1.f, 1.f};
    bool badp = false;
    {
        int zn[4] = {0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < TOK; ++j) {
            zc[j] = 0;
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const float a = al[j][x];
                if constexpr (ZS) {
                    const bool z = a == 0.f;
                    cur[x] *= z ? 1.f : a;
                    zn[x] += z ? 1 : 0;
                    zc[j] |= (unsigned)zn[x] << (8 * x);
                } else {
                    cur[x] *= a;
                }
                pr[j][x] = cur[x];
            }
        }
        float lp[4];
        int pz[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const float m = fabsf(cur[x]);
            // the magnitude must stay a normal float no larger than one (NaN fails too)
            badp = badp || !(m >= kMinPart && m <= 1.f);
            lp[x] = flog2(m);
            pz[x] = (zn[x] << 1) | (cur[x] < 0.f ? 1 : 0);
        }
        if constexpr (PH) {
            // running phase sums of my two pairs over my tokens
#pragma unroll
            for (int j = 1; j < TOK; ++j) { th[j][0] += th[j - 1][0]; th[j][1] += th[j - 1][1]; }
            if (own)
                *reinterpret_cast<float2*>(partPh + part * (DK / 2) + c0 / 2) =
                    make_float2(th[TOK - 1][0], th[TOK - 1][1]);
        }
        if (own) {
            *reinterpret_cast<float4*>(partL + part * DK + c0) = make_float4(lp[0], lp[1], lp[2], lp[3]);
            *reinterpret_cast<int4*>(partPZ + part * DK + c0) = make_int4(pz[0], pz[1], pz[2], pz[3]);
            if (q4 == 0) {
#pragma unroll
                for (int j = 0; j < TOK; ++j) sBeta[part * TOK + j] = bt[j];
            }
        }
    }
    __syncthreads();
    float offL[4] = {0.f, 0.f, 0.f, 0.f}, totL[4] = {0.f, 0.f, 0.f, 0.f};
    int offPZ[4] = {0, 0, 0, 0}, totPZ[4] = {0, 0, 0, 0};   // (zero count) << 1 | parity
#pragma unroll 8
    for (int p = 0; p < PARTS; ++p) {
        const float4 l = *reinterpret_cast<const float4*>(partL + p * DK + c0);
        const int4 z = *reinterpret_cast<const int4*>(partPZ + p * DK + c0);
        const float lv[4] = {l.x, l.y, l.z, l.w};
        const int zv[4] = {z.x, z.y, z.z, z.w};
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            if (p < part) { offL[x] += lv[x]; offPZ[x] = (((offPZ[x] >> 1) + (zv[x] >> 1)) << 1) | ((offPZ[x] ^ zv[x]) & 1); }
            totL[x] += lv[x];
            totPZ[x] = (((totPZ[x] >> 1) + (zv[x] >> 1)) << 1) | ((totPZ[x] ^ zv[x]) & 1);
        }
    }
    float offPh[2] = {0.f, 0.f}, totPh[2] = {0.f, 0.f};     // (PH) phases before my range, in the chunk
    if constexpr (PH) {
        for (int p = 0; p < PARTS; ++p) {
            const float2 t2 = *reinterpret_cast<const float2*>(partPh + p * (DK / 2) + c0 / 2);
            if (p < part) { offPh[0] += t2.x; offPh[1] += t2.y; }
            totPh[0] += t2.x;
            totPh[1] += t2.y;
        }
    }
    int Ztot = 0;
    bool bad = badp;
    if constexpr (ZS) {
        if (own && part == 0) {
#pragma unroll
            for (int x = 0; x < 4; ++x) sBase[c0 + x] = totPZ[x] >> 1;
        }
        __syncthreads();
        // exclusive prefix of the per-channel zero counts -> first extra column of a channel
        if (wave == 0) {
            int carry = 0;
            for (int cc = 0; cc < DK; cc += 64) {
                const int v = (cc + lane < DK) ? sBase[cc + lane] : 0;
                int incl = v;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const int y = __shfl_up(incl, off, 64);
                    if (lane >= off) incl += y;
                }
                if (cc + lane < DK) sBase[cc + lane] = carry + incl - v;
                carry += __shfl(incl, 63, 64);
            }
            if (lane == 0) misc[0] = carry;
        }
        __syncthreads();
        Ztot = __builtin_amdgcn_readfirstlane(misc[0]);
        bad = Ztot > args.zx;
    }
    // midpoint M = L_total / 2;  F_r = F0 pr_r and G_r = G0 / pr_r, where F0, G0
    // carry the sign and magnitude of the earlier token ranges
    float M[4], E[4], F0[4], G0[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        M[x] = 0.5f * totL[x];
        bad = bad || (-M[x] > kHalfSpanMax) || !(M[x] <= 0.f);
        E[x] = fexp2(M[x]);
        const float so = (offPZ[x] & 1) ? -1.f : 1.f;
        F0[x] = so * fexp2(offL[x] - M[x]);
        G0[x] = so * fexp2(M[x] - offL[x]);
    }
    // (the workgroup-wide answer, made provably uniform for the compiler, so
    // that every branch around a barrier here is a uniform one)
    if (__builtin_amdgcn_readfirstlane((int)__syncthreads_or(bad && own))) {
        if (tid == 0) args.FL[unit] = 1;
        return true;
    }
    if (tid == 0) args.FL[unit] = 0;

    if constexpr (PH) {
        // k_r, q_r <- R(-phi_r) k_r, R(-phi_r) q_r per channel pair
#pragma unroll
        for (int j = 0; j < TOK; ++j) {
            float kf[4], qf[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) { kf[x] = kv[j].get(x); qf[x] = qv[j].get(x); }
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
                float sn, cs;
                __sincosf(offPh[pp] + th[j][pp], &sn, &cs);
                const float k0 = kf[2 * pp], k1 = kf[2 * pp + 1], q0 = qf[2 * pp], q1 = qf[2 * pp + 1];
                kf[2 * pp] = cs * k0 + sn * k1;
                kf[2 * pp + 1] = cs * k1 - sn * k0;
                qf[2 * pp] = cs * q0 + sn * q1;
                qf[2 * pp + 1] = cs * q1 - sn * q0;
            }
            kv[j] = Vec4<T>::from(kf);
            qv[j] = Vec4<T>::from(qf);
        }
    }

    // ---- factored operands (LDS) ------------------------------------------------
    // (Q*Gamma, and Ktil of the channels without a zero gate in the chunk, are
    // written from the LDS operands after the build, one whole fragment per
    // lane store: Q*Gamma = (q F) E and Ktil^T = (k G) stot E per channel, then
    // turned by the chunk phase.  Ktil of a channel with zero gates, and every
    // Ktil of the phase variant with zero segments, goes out directly here.)
    constexpr bool KT_LDS = !(ZS && PH);
    // A operand beta k F, P operand q F, shared operand k G of token j, channel x
    auto factors = [&](int j, int x, float& fa, float& fp, float& fy) {
        const float kx = kv[j].get(x);
        const float Fv = F0[x] * pr[j][x];
        fa = bt[j] * kx * Fv;
        fp = qv[j].get(x) * Fv;
        fy = kx * (G0[x] * frcp(pr[j][x]));
    };
    Vec4<T> xw[TOK];
    float kt[TOK][4];
#pragma unroll
    for (int j = 0; j < TOK; ++j) {
        const int r = part * TOK + j;
        float fa[4], fp[4], fy[4], fw[4];
        int segs[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            factors(j, x, fa[x], fp[x], fy[x]);
            // Gamma_r = F_r E in the first zero segment; rho(C-1, r) = stot E G_r
            // in the last one (stot: sign of the whole chunk's product)
            const float stot = (totPZ[x] & 1) ? -1.f : 1.f;
            float ge = E[x], re = stot * E[x];
            int seg = 0;
            if constexpr (ZS) {
                seg = (offPZ[x] >> 1) + (int)((zc[j] >> (8 * x)) & 0xffu);
                ge = seg == 0 ? ge : 0.f;
                re = seg == (totPZ[x] >> 1) ? re : 0.f;
            }
            fw[x] = fa[x] * ge;
            kt[j][x] = fy[x] * re;
            segs[x] = seg;
        }
        xw[j] = Vec4<T>::from(fw);
        if (own) {
            // main columns hold zero segment 0 only; later segments wait for
            // their extra-column pass
            if constexpr (ZS) {
#pragma unroll
                for (int x = 0; x < 4; ++x)
                    if (segs[x] != 0) { fa[x] = 0.f; fp[x] = 0.f; fy[x] = 0.f; }
            }
            *reinterpret_cast<Vec4<T>*>(XA + r * KS + c0) = Vec4<T>::from(fa);
            *reinterpret_cast<Vec4<T>*>(XP + r * KS + c0) = Vec4<T>::from(fp);
            *reinterpret_cast<Vec4<T>*>(Y + r * KS + c0) = Vec4<T>::from(fy);
        }
    }
    if (own) {
        float ce[2] = {1.f, 1.f}, se[2] = {0.f, 0.f};     // (PH) cos, sin of phi_{C-1}
        if constexpr (PH) {
            // Ktil_i = |rho(C-1, i)| R(phi_{C-1}) R(-phi_i) k_i: rotate back
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) __sincosf(totPh[pp], &se[pp], &ce[pp]);
            if (KT_LDS && part == 0) {
#pragma unroll
                for (int pp = 0; pp < 2; ++pp) {
                    sRot[c0 + 2 * pp] = ce[pp];
                    sRot[c0 + 2 * pp + 1] = se[pp];
                }
            }
#pragma unroll
            for (int j = 0; j < TOK; ++j)
#pragma unroll
                for (int pp = 0; pp < 2; ++pp) {
                    const float x0 = kt[j][2 * pp], x1 = kt[j][2 * pp + 1];
                    kt[j][2 * pp] = ce[pp] * x0 - se[pp] * x1;
                    kt[j][2 * pp + 1] = se[pp] * x0 + ce[pp] * x1;
                }
        }
        // Ktil: A operand with rows = channels, k = tokens; 4 consecutive tokens
        // starting at a multiple of 4 are 4 consecutive slots of one fragment
        if constexpr (!KT_LDS || ZS) {
            bool direct[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) direct[x] = !KT_LDS || (totPZ[x] >> 1) != 0;
            if constexpr (TOK % 4 == 0) {
#pragma unroll
                for (int j0 = 0; j0 < TOK; j0 += 4)
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        const float f4[4] = {kt[j0][x], kt[j0 + 1][x], kt[j0 + 2][x], kt[j0 + 3][x]};
                        if (direct[x])
                            *reinterpret_cast<Vec4<T>*>(Ktg + frag_off<KB>(c0 + x, part * TOK + j0, C)) =
                                Vec4<T>::from(f4);
                    }
            } else {
#pragma unroll
                for (int j = 0; j < TOK; ++j)
#pragma unroll
                    for (int x = 0; x < 4; ++x)
                        if (direct[x]) Ktg[frag_off<KB>(c0 + x, part * TOK + j, C)] = from_f32<T>(kt[j][x]);
            }
        }
        if (part == 0) {
            // (written here, past the build's register peak)
            *reinterpret_cast<float4*>(sRE + c0) =
                make_float4((totPZ[0] & 1) ? -E[0] : E[0], (totPZ[1] & 1) ? -E[1] : E[1],
                            (totPZ[2] & 1) ? -E[2] : E[2], (totPZ[3] & 1) ? -E[3] : E[3]);
            float g4[4];
#pragma unroll
            for (int x = 0; x < 4; ++x)
                g4[x] = (totPZ[x] >> 1) == 0 ? ((totPZ[x] & 1) ? -1.f : 1.f) * E[x] * E[x] : 0.f;
            if constexpr (PH) {
                // Gamma_{C-1} of pair p as (|Gamma| cos phi, |Gamma| sin phi)
#pragma unroll
                for (int pp = 0; pp < 2; ++pp) {
                    const float gm = g4[2 * pp];
                    g4[2 * pp] = gm * ce[pp];
                    g4[2 * pp + 1] = gm * se[pp];
                }
            }
            *reinterpret_cast<float4*>(args.GC + (size_t)unit * DK + c0) = make_float4(g4[0], g4[1], g4[2], g4[3]);
        }
    }
    __syncthreads();
    // Q*Gamma (rows = tokens, k = channels) and Ktil (rows = channels, k =
    // tokens) from the main operand columns in LDS, before the V loads and the
    // contraction, while few registers are live: lane (m, g) of fragment
    // (tile, k block s) holds row m's columns kcol(s, g, j), j = 0 .. NV-1, in
    // the workspace's slot order.  (With zero segments the main columns hold
    // segment 0 only: that is all of Q*Gamma, and all of Ktil for a channel
    // without zeros; the other channels' Ktil went out directly.)
    {
        auto kcol = [&](int s, int j) {
            if constexpr (KB == 32) return 32 * s + 16 * (j >> 2) + 4 * lg + (j & 3);
            else return 16 * s + 4 * lg + j;
        };
        if (wave < NB) {
            const T* xrow = XP + (16 * wave + ln) * KS;
#pragma unroll
            for (int s = 0; s < NKD; ++s) {
                float f[NV];
#pragma unroll
                for (int h4 = 0; h4 < NV / 4; ++h4) {       // runs of 4 consecutive columns
                    const int c = kcol(s, 4 * h4);
                    const Vec4<T> xv = Vec4<T>::load(xrow + c);
                    const float4 ev = *reinterpret_cast<const float4*>(sRE + c);
                    f[4 * h4 + 0] = xv.get(0) * fabsf(ev.x);
                    f[4 * h4 + 1] = xv.get(1) * fabsf(ev.y);
                    f[4 * h4 + 2] = xv.get(2) * fabsf(ev.z);
                    f[4 * h4 + 3] = xv.get(3) * fabsf(ev.w);
                }
                store_ws<NT>(QGg + ((size_t)(wave * NKD + s) * 64 + lane) * NV, F::from(f));
            }
        }
        if constexpr (KT_LDS) {
            constexpr int NKT = (DK / 16) * NKC;            // Ktil fragments
            for (int fi = wave; fi < NKT; fi += kThreads / 64) {
                const int ct = fi / NKC, s = fi % NKC;
                const int c = 16 * ct + ln;
                const float re = sRE[c];
                if constexpr (ZS) {
                    if ((c + 1 < DK ? sBase[c + 1] : Ztot) != sBase[c]) continue;   // zeros: direct
                }
                float f[NV];
                if constexpr (PH) {
                    // rows 2p, 2p+1 turn by the pair's chunk phase (same gate, same re)
                    const int c2 = c & ~1;
                    const float cs = sRot[c2], sn = sRot[c2 + 1];
#pragma unroll
                    for (int j = 0; j < NV; ++j) {
                        const float y0 = to_f32(Y[kcol(s, j) * KS + c2]);
                        const float y1 = to_f32(Y[kcol(s, j) * KS + c2 + 1]);
                        f[j] = re * ((c & 1) ? sn * y0 + cs * y1 : cs * y0 - sn * y1);
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < NV; ++j) f[j] = to_f32(Y[kcol(s, j) * KS + c]) * re;
                }
                store_ws<NT>(Ktg + ((size_t)(ct * NKC + s) * 64 + lane) * NV, F::from(f));
            }
        }
    }
    // V tile loads: in flight during the A / P tiles and Tinv
    // item (column quad vq, token run tg): 4 columns x TV tokens, stored later
    // as 4 rows of (beta V)^T; rows past the end re-read the last valid row
    const int nvq = Dv / 4, nvit = nvq * (C / TV);
    Vec4<T> vreg[G::VIT][TV];
#pragma unroll
    for (int x = 0; x < G::VIT; ++x) {
        const int it = min(tid + x * kThreads, nvit - 1);
        const int vq = it % nvq, tg = it / nvq;
#pragma unroll
        for (int z = 0; z < TV; ++z)
            vreg[x][z] = Vec4<T>::load_nt(gv + min(tg * TV + z, nvalid - 1) * rsv + 4 * vq);
    }

    // ---- A (strictly lower, LDS) and P^T tiles (global, fragment-major) --------
    // wave w takes row tile ta = w: over the contraction it keeps the row's
    // (beta K * F) and (Q * F) fragments and streams (K * G) of tiles tb <= ta
    // (NB <= 4: each wavefront has at most one row tile; its A tiles stay in
    // registers until the operands are dead and the region becomes A, Tinv)
    static_assert(NB <= 4, "one row tile per wavefront");
    const int ta = wave;
    f32x4 accA[NB], accP[NB];
#pragma unroll
    for (int tb = 0; tb < NB; ++tb) { accA[tb] = zero4(); accP[tb] = zero4(); }
    // one pass: the first kw columns of the operand region
    auto contract = [&](int kw) {
        if (ta < NB) {
            for (int k0 = 0; k0 < kw; k0 += KB) {
                const F xa = frag_row<T, KB>(XA + (16 * ta + ln) * KS, k0);
                const F xp = frag_row<T, KB>(XP + (16 * ta + ln) * KS, k0);
#pragma unroll
                for (int tb = 0; tb < NB; ++tb) {
                    if (tb <= ta) {
                        const F y = frag_row<T, KB>(Y + (16 * tb + ln) * KS, k0);
                        accA[tb] = mma(xa, y, accA[tb]);    // A[16ta + 4g + i][16tb + n]
                        accP[tb] = mma(y, xp, accP[tb]);    // P[16ta + n][16tb + 4g + i]
                    }
                }
            }
        }
    };
    contract(DK);
    if constexpr (ZS) {
        // extra columns e = 0 .. Ztot-1, DK per pass: (channel c, segment s >= 1)
        // is column e = sBase[c] + s - 1
        for (int e0 = 0; e0 < Ztot; e0 += DK) {
            __syncthreads();                              // previous pass read
            constexpr int RV = DK * (int)sizeof(T) / 16;  // 16-byte runs per operand row
            for (int idx = tid; idx < 3 * C * RV; idx += kThreads) {
                const int row = idx / RV, run = idx % RV;
                *reinterpret_cast<uint4*>(XA + row * KS + run * (16 / (int)sizeof(T))) =
                    make_uint4(0u, 0u, 0u, 0u);
            }
            __syncthreads();
            if (own) {
#pragma unroll
                for (int j = 0; j < TOK; ++j) {
                    const int r = part * TOK + j;
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        const int seg = (offPZ[x] >> 1) + (int)((zc[j] >> (8 * x)) & 0xffu);
                        const int col = sBase[c0 + x] + seg - 1 - e0;
                        if (seg > 0 && col >= 0 && col < DK) {
                            float fa, fp, fy;
                            factors(j, x, fa, fp, fy);
                            XA[r * KS + col] = from_f32<T>(fa);
                            XP[r * KS + col] = from_f32<T>(fp);
                            Y[r * KS + col] = from_f32<T>(fy);
                        }
                    }
                }
            }
            __syncthreads();
            contract(min(DK, ((Ztot - e0 + KB - 1) / KB) * KB));
        }
    }
    if (ta < NB) {
#pragma unroll
        for (int s = 0; s < NKC; ++s) {
            float f[NV];
#pragma unroll
            for (int u = 0; u < TPB; ++u) {
                const int tb = s * TPB + u;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    f[4 * u + i] = (tb <= ta && 16 * tb + 4 * lg + i <= 16 * ta + ln) ? accP[tb][i] : 0.f;
            }
            store_ws<NT>(Pg + ((size_t)(ta * NKC + s) * 64 + lane) * NV, F::from(f));
        }
    }
    __syncthreads();   // operands dead: the region now holds A and Tinv
    if (ta < NB) {
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) {
            if (tb <= ta) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * ta + 4 * lg + i, col = 16 * tb + ln;
                    sA[r * LDF + col] = col < r ? accA[tb][i] : 0.f;
                }
            }
        }
    }
    for (int idx = tid; idx < C * C; idx += kThreads) {       // upper blocks of Tinv
        const int r = idx / C, col = idx % C;
        if ((col >> 4) > (r >> 4)) sT[r * LDF + col] = 0.f;
    }
    __syncthreads();

    // ---- Tinv diagonal blocks ---------------------------------------------------
    // forward substitution on the 16x16 diagonal blocks: wave 0, lane 16a + j
    // owns column j of block a
    if (wave == 0 && (lane >> 4) < NB) {
        const int a = lane >> 4, j = lane & 15;
        float t[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float s = (r == j) ? 1.f : 0.f;
#pragma unroll
            for (int i = 0; i < r; ++i) s -= sA[(16 * a + r) * LDF + 16 * a + i] * t[i];
            t[r] = s;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sT[(16 * a + r) * LDF + 16 * a + j] = t[r];
    }
    __syncthreads();
    // ---- Tinv off-diagonal blocks by block distance (fp32 MFMA) ----------------
    for (int d = 1; d < NB; ++d) {
        for (int idx = wave; idx < NB - d; idx += 4) {
            const int a = idx + d, bb = idx;
            f32x4 inner = zero4();
            for (int jb = bb; jb < a; ++jb) {
                // A_{a,jb} (row-major in sA) times T_{jb,bb} (row-major [k][n] in sT)
                const Frag<float, 16> fa =
                    Frag<float, 16>::load(sA + (16 * a + ln) * LDF + 16 * jb + 4 * lg);
                float fb[4];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) fb[jj] = sT[(16 * jb + 4 * lg + jj) * LDF + 16 * bb + ln];
                inner = mma(fa, Frag<float, 16>::from(fb), inner);
            }
            const float fi[4] = {inner[0], inner[1], inner[2], inner[3]};
            const Frag<float, 16> taa =
                Frag<float, 16>::load(sT + (16 * a + ln) * LDF + 16 * a + 4 * lg);
            const f32x4 tab = mma(taa, Frag<float, 16>::from(fi), zero4());
#pragma unroll
            for (int i = 0; i < 4; ++i) sT[(16 * a + 4 * lg + i) * LDF + 16 * bb + ln] = -tab[i];
        }
        __syncthreads();
    }
    if (args.Tm) {
        float* tg = args.Tm + (size_t)unit * C * C;
        for (int idx = tid; idx < C * C; idx += kThreads) tg[idx] = sT[(idx / C) * LDF + idx % C];
    }

    // ---- W = Tinv X_W and U = Tinv (diag(beta) V): wave w takes token tile
    //      mt = w; its Tinv rows serve as the A operand of U and the B operand
    //      of W^T (same per-lane data).  Tinv[16mt + i][k] = 0 for k beyond
    //      the tile, so k blocks past it are skipped.
    {
        constexpr int NM = C / 16;
        const int NUt = Dv / 16;
        const int mt = wave;
        F tf[NKC];
        if (mt < NM) {
#pragma unroll
            for (int kb = 0; kb < NKC; ++kb)
                tf[kb] = frag_row_cvt<T, KB>(sT + (16 * mt + ln) * LDF, kb * KB);
        }
        __syncthreads();   // A and Tinv dead: the region now holds X_W^T, (beta V)^T
        // ---- stage X_W^T and (diag(beta) V)^T ------------------------------------
        // X_W^T row c holds this thread's TOK tokens of channel c contiguously
        if (own) {
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                T* dst = sXWt + (c0 + x) * XTS + part * TOK;
                if constexpr (TOK * sizeof(T) == 16) {
                    T v[TOK];
#pragma unroll
                    for (int j = 0; j < TOK; ++j) v[j] = xw[j].elem(x);
                    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(v);
                } else {
#pragma unroll
                    for (int j = 0; j < TOK; ++j) dst[j] = xw[j].elem(x);
                }
            }
        }
#pragma unroll
        for (int x = 0; x < G::VIT; ++x) {
            const int it = tid + x * kThreads;
            if (it < nvit) {
                const int vq = it % nvq, tg = it / nvq;
#pragma unroll
                for (int y = 0; y < 4; ++y) {
                    T v[TV];
#pragma unroll
                    for (int z = 0; z < TV; ++z) v[z] = from_f32<T>(sBeta[tg * TV + z] * vreg[x][z].get(y));
                    *reinterpret_cast<uint4*>(sVt + (4 * vq + y) * XTS + tg * TV) = *reinterpret_cast<const uint4*>(v);
                }
            }
        }
        __syncthreads();
        if (mt < NM) {
            const int nkb = (16 * (mt + 1) + KB - 1) / KB;
#pragma unroll
            for (int s = 0; s < NKD; ++s) {
                float f[NV];
#pragma unroll
                for (int u = 0; u < TPB; ++u) {
                    const int ct = s * TPB + u;
                    // W^T[16ct + 4g + i][16mt + n] = sum_k X_W^T[16ct + .][k] Tinv[16mt + n][k]
                    f32x4 acc = zero4();
#pragma unroll
                    for (int kb = 0; kb < NKC; ++kb)
                        if (kb < nkb)
                            acc = mma(frag_row<T, KB>(sXWt + (16 * ct + ln) * XTS, kb * KB), tf[kb], acc);
#pragma unroll
                    for (int i = 0; i < 4; ++i) f[4 * u + i] = acc[i];
                }
                store_ws<NT>(Wg + ((size_t)(mt * NKD + s) * 64 + lane) * NV, F::from(f));
            }
            for (int nt = 0; nt < NUt; ++nt) {
                f32x4 acc = zero4();
#pragma unroll
                for (int kb = 0; kb < NKC; ++kb)
                    if (kb < nkb) acc = mma(tf[kb], frag_row<T, KB>(sVt + (16 * nt + ln) * XTS, kb * KB), acc);
                {
                    const float u4[4] = {acc[0], acc[1], acc[2], acc[3]};
                    store_ws<NT>(Ug + ((size_t)(mt * NUt + nt) * 64 + lane) * 4, Vec4<T>::from(u4));
                }
            }
        }
    }
    return false;
}

template <typename T, int C, int DK, bool ZS, bool PRO, bool PH, bool NT = false>
__global__ __launch_bounds__(kThreads, (sizeof(T) == 4 && DK == 128) ? 1 : 2) void prep_fast_kernel(PrepArgs args)
{
    // a launch over every unit takes them chunk by chunk, all (b, h) of a
    // chunk index together: the workgroups running at one time then read
    // whole token rows of q, k, v and alpha (every head of those tokens),
    // 146 -> 139 us at B=1, H=32, T=8192 against (b, h) by (b, h)
    int v = (int)blockIdx.x;
    if (args.pcn == 0) {
        const int bhn = (int)gridDim.x / args.NC;
        v = (v % bhn) * args.NC + v / bhn;
    }
    prep_fast_unit<T, C, DK, ZS, PRO, PH, NT>(args, part_unit(v, args.pc0, args.pcn, args.NC));
}

// Streamed forward (dense batches): one unit per workgroup, but not the unit
// of its index: each workgroup claims the next unit of the heads on its own
// XCD (b H + h = xcd + 8 j, read from the hardware) from that XCD's counter,
// in chunk-major order, so the chain workgroups of the same XCD read the unit
// from the L2 they share, and chunk n of every head comes before chunk n + 1
// of any.  After the unit, every wave waits for its stores, then the unit's
// ready word is set (1: the factors are in the
// workspace; 2: the unit needs the exact kernel, which runs after this grid).
// The grid holds 8 x (the most units any XCD has) workgroups; those that find
// no unit left exit.
template <typename T, int C, int DK, bool ZS, bool NT>
__global__ __launch_bounds__(kThreads, (sizeof(T) == 4 && DK == 128) ? 1 : 2) void prep_stream_kernel(PrepArgs args)
{
    __shared__ int sUnit;
    const int xcd = (int)xcc_id();
    const int BH = args.nbh, NC = args.NC;
    const int hx = (BH - xcd + 7) / 8;               // heads of this XCD
    const int total = hx > 0 ? hx * NC : 0;
    if (threadIdx.x == 0) {
        const int u = total > 0 ? (int)atomicAdd(&args.sctl->prep_next[xcd], 1u) : 0;
        sUnit = u < total ? (xcd + 8 * (u % hx)) * NC + u / hx : -1;
    }
    __syncthreads();
    const int unit = __builtin_amdgcn_readfirstlane(sUnit);
    if (unit < 0) return;
    // lead limit: chunk n waits until the chain of its (b, h) has taken chunk
    // n - lead (ready word 3), so the units between prep and chain stay in
    // the caches; bounded, given up at once when a chain workgroup has given
    // up (its marks stop), and only a matter of speed
    if (args.lead > 0 && unit % args.NC >= args.lead) {
        if (threadIdx.x == 0) {
            const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
            for (unsigned n = 0; n < kLeadWaitPolls; ++n) {
                if (__hip_atomic_load(&args.ready[unit - args.lead], __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT) == 3u ||
                    __hip_atomic_load(&args.sctl->abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ||
                    __builtin_amdgcn_s_memrealtime() - t0 > kLeadWaitTicks)
                    break;
                __builtin_amdgcn_s_sleep(8);
            }
        }
        __syncthreads();
    }
    const bool flagged = prep_fast_unit<T, C, DK, ZS, false, false, NT>(args, unit);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0)
        __hip_atomic_store(&args.ready[unit], flagged ? 2u : 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T, int C, int DK>
hipError_t launch_fast_t(const ChunkShape& s, const PrepArgs& a, hipStream_t stream)
{
    const FastLayout<T, C, DK> LY;
    // (the input parameterisation and the phase variant are not combined; the
    // non-temporal workspace stores exist for the plain variants)
    auto kern = a.theta ? (a.zx > 0 ? prep_fast_kernel<T, C, DK, true, false, true>
                                    : prep_fast_kernel<T, C, DK, false, false, true>)
              : a.zx > 0 ? (a.pro ? prep_fast_kernel<T, C, DK, true, true, false>
                                  : a.ntst ? prep_fast_kernel<T, C, DK, true, false, false, true>
                                           : prep_fast_kernel<T, C, DK, true, false, false>)
                         : (a.pro ? prep_fast_kernel<T, C, DK, false, true, false>
                                  : a.ntst ? prep_fast_kernel<T, C, DK, false, false, false, true>
                                           : prep_fast_kernel<T, C, DK, false, false, false>);
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)LY.total);
    if (e != hipSuccess) return e;
    const unsigned nunits = (unsigned)((size_t)s.B * s.H * (a.pcn > 0 ? a.pcn : s.NC));
    return launch_kernel(kern, dim3(nunits), dim3(kThreads), (uint32_t)LY.total, stream, a);
}

template <typename T, int C, int DK>
size_t fast_lds_t() { return FastLayout<T, C, DK>().total; }

template <typename T, int C, int DK>
hipError_t launch_stream_t(const PrepArgs& a, hipStream_t stream)
{
    const FastLayout<T, C, DK> LY;
    auto kern = a.zx > 0 ? prep_stream_kernel<T, C, DK, true, false>
                         : prep_stream_kernel<T, C, DK, false, false>;
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)LY.total);
    if (e != hipSuccess) return e;
    constexpr int kXcd = 8;                              // XCDs of the MI355X
    const unsigned grid = (unsigned)(kXcd * ((a.nbh + kXcd - 1) / kXcd) * a.NC);
    return launch_kernel(kern, dim3(grid), dim3(kThreads), (uint32_t)LY.total, stream, a);
}

template <typename T, int C>
hipError_t dispatch_dk(const ChunkShape& s, const PrepArgs& a, hipStream_t st)
{
    switch (s.Dk) {
    case 16: return launch_fast_t<T, C, 16>(s, a, st);
    case 32: return launch_fast_t<T, C, 32>(s, a, st);
    case 64: return launch_fast_t<T, C, 64>(s, a, st);
    case 128: return launch_fast_t<T, C, 128>(s, a, st);
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

template <typename T, int C>
size_t lds_dk(int Dk)
{
    switch (Dk) {
    case 16: return fast_lds_t<T, C, 16>();
    case 32: return fast_lds_t<T, C, 32>();
    case 64: return fast_lds_t<T, C, 64>();
    default: return fast_lds_t<T, C, 128>();
    }
}

}  // namespace

size_t prep_fast_lds_bytes(IoType io, int C, int Dk)
{
    if (io == IoType::F32) {
        return C == 16 ? lds_dk<float, 16>(Dk) : C == 32 ? lds_dk<float, 32>(Dk)
                                                          : lds_dk<float, 64>(Dk);
    }
    return C == 16 ? lds_dk<bf16_t, 16>(Dk) : C == 32 ? lds_dk<bf16_t, 32>(Dk)
                                                       : lds_dk<bf16_t, 64>(Dk);
}

hipError_t launch_prep_stream(IoType io, const ChunkShape& s, const PrepArgs& a,
                              hipStream_t stream)
{
    if (io != IoType::BF16 || s.C != 64) return hipErrorInvalidValue;
    if (s.Dk == 128) return launch_stream_t<bf16_t, 64, 128>(a, stream);
    if (s.Dk == 64) return launch_stream_t<bf16_t, 64, 64>(a, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_prep_fast(IoType io, const ChunkShape& s, const PrepArgs& a, hipStream_t stream)
{
    if (io == IoType::F32) return dispatch_c<float>(s, a, stream);
    return dispatch_c<bf16_t>(s, a, stream);
}

}  // namespace kda
