// bwd.hip — the chunkwise backward: gradients of L = sum_t <o_t, dO_t> +
// <S_T, dST> with respect to q, k, v, alpha, beta and S0, for the recurrence
// of "Semidirect Fourier Delta Attention" §1 eq. (1) read out by §3 eq. (14).
//
// Per chunk (C tokens, S the state entering it, dSn the loss gradient of the
// state leaving it through later chunks and dST), differentiating the
// chunkwise forward  Delta = U - W S,  O = (Q * Gamma) S + P Delta,
// S_next = diag(Gamma_{C-1}) S + Ktil^T Delta  gives the reverse chain
//   X  = P^T dO + Ktil dSn                          (gradient of Delta)
//   dS = diag(Gamma_{C-1}) dSn + (Q * Gamma)^T dO - W^T X
// (columns of dS are independent, as the forward's columns of S are), and
// per chunk, with y = Tinv^T X (y_r = G_r^T k_r, G_r the gradient of the
// state after token r), B1 = dO Delta^T, B3 = Y Delta^T, F1 = dO S^T,
// F2 = Y S^T, F3 = Delta dSn^T and the decay-weighted sums
//   LQ1_r = sum_{i<r} B1[r,i] rho(r,i) k_i     LK3_r = sum_{i<r} B3[r,i] rho(r,i) k_i
//   UQ1_r = sum_{j>r} B1[j,r] rho(j,r) q_j     UK2_r = sum_{j>r} beta_j B3[j,r] rho(j,r) k_j
// (rho(r,i) = prod_{l=i+1..r} alpha_l per channel):
//   dv = diag(beta) y
//   dq = Gamma F1 + LQ1 + diag(B1) k
//   dk = rho(C-1,.) F3 + UQ1 + diag(B1) q - UK2 - beta (Gamma F2 + LK3)
//   dbeta_r = v_r.y_r - (k_r Gamma_r).F2_r - k_r.LK3_r
//   alpha_r dalpha_r = Gamma_{C-1} sigma + sum_{i<r} (Ktil F3)_i
//                      + sum_{j>=r} [Gamma (q F1 - beta k F2) + q LQ1 - beta k LK3
//                                    - k (UQ1 - UK2)]_j,   sigma_c = <dSn[c], S[c]>
// the last term read off the reverse-mode derivative of the gates through
// every product rho that contains alpha_r.  Where |alpha_r| < 2^-6 (zero
// gates included) the quotient is replaced by the direct form
//   dalpha_r[c] = <H_r[c,:], S_{r-1}[c,:]>,  H_r = G_r - k_r dv_r^T,
// from a per-channel sweep over the chunk (bwd_tiny_kernel).
//
// Kernels, after the forward's prep (which also stores Tinv) and its chain
// (which also stores the fp32 chunk states and Delta):
//   relayout_kernel    W, Q*Gamma, Ktil^T, P -> W^T, (Q*Gamma)^T, Ktil, P^T in
//                      the fragment-major A-operand layout, in place
//   bwd_chain_fifo_kernel  the reverse chain, one workgroup per (b, h, 16 columns)
//                      (operands through an LDS FIFO fed by loader wavefronts)
//   bwd_local_kernel   every chunk's gradients, one workgroup per chunk
//   bwd_tiny_kernel    the direct dalpha of small gates, flagged chunks only
// Packed batches locate chunks and sequences through the forward's tables.
// With raw inputs, prologue_in_kernel forms the transformed inputs first and
// prologue_out_kernel maps the gradients back (eqs. (15), (17), (18)).
#include <type_traits>

#include "kda_chunk.hpp"
#include "kda_dma.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace {

constexpr int kBwdThreads = 256;
constexpr int kXcds = 8;
constexpr float kTinyGate = 0x1p-6f;

// ---- relayout ---------------------------------------------------------------
// (row, column) of the element at offset o of an A-operand matrix with K
// columns (the inverse of frag_off)
template <int KB>
__device__ __forceinline__ void frag_pos(int o, int K, int& r, int& k)
{
    constexpr int NV = KB / 4;
    const int j = o % NV, x = o / NV;
    const int lane = x & 63, blk = x >> 6;
    const int nkb = K / KB;
    const int g = lane >> 4;
    int kk;
    if constexpr (KB == 32) kk = 16 * (j >> 2) + 4 * g + (j & 3);
    else kk = 4 * g + j;
    r = 16 * (blk / nkb) + (lane & 15);
    k = (blk % nkb) * KB + kk;
}

template <typename T, int C, int DK>
struct RelayoutLds {
    static constexpr size_t W = 0, Q = W + (size_t)C * DK, K = Q + (size_t)C * DK, P = K + (size_t)C * DK;
    static constexpr size_t BYTES = (P + (size_t)C * C) * sizeof(T);
};

// copy NV consecutive elements (one lane's fragment slots, NV * sizeof(T)
// bytes: 8 or 16, aligned to that size)
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

template <typename T, int NV>
struct FragVec {
    static constexpr int BYTES = NV * (int)sizeof(T);
    using V = typename std::conditional<BYTES == 16, uint4, uint2>::type;
    using NV_t = typename std::conditional<BYTES == 16, u32x4_t, u32x2_t>::type;
    __attribute__((aligned(16))) T e[NV];
    // non-temporal: each fragment is read once and written once
    __device__ __forceinline__ void load(const T* p) {
        *reinterpret_cast<NV_t*>(e) = __builtin_nontemporal_load(reinterpret_cast<const NV_t*>(p));
    }
    __device__ __forceinline__ void store(T* p) const {
        __builtin_nontemporal_store(*reinterpret_cast<const NV_t*>(e), reinterpret_cast<NV_t*>(p));
    }
};

template <typename T, int C, int DK>
__global__ __launch_bounds__(kBwdThreads) void relayout_kernel(T* __restrict__ W, T* __restrict__ QG,
                                                               T* __restrict__ Kt, T* __restrict__ P)
{
    constexpr int KB = KBlock<T, C, DK>::value, NV = KB / 4;
    using L = RelayoutLds<T, C, DK>;
    using FV = FragVec<T, NV>;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    T* s = reinterpret_cast<T*>(lds);
    const size_t unit = blockIdx.x;
    T* gW = W + unit * C * DK;
    T* gQ = QG + unit * C * DK;
    T* gK = Kt + unit * DK * C;
    T* gP = P + unit * C * C;
    const int tid = threadIdx.x;
    int r, k;
    // read: one lane fragment (NV slots) per step, scattered to row-major LDS
    for (int f = tid; f < C * DK / NV; f += kBwdThreads) {
        FV w, q, kt;
        w.load(gW + f * NV);
        q.load(gQ + f * NV);
        kt.load(gK + f * NV);
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            frag_pos<KB>(f * NV + j, DK, r, k);        // W, Q*Gamma: [C][DK]
            s[L::W + r * DK + k] = w.e[j];
            s[L::Q + r * DK + k] = q.e[j];
            frag_pos<KB>(f * NV + j, C, r, k);         // Ktil^T: [DK][C]
            s[L::K + r * C + k] = kt.e[j];
        }
    }
    for (int f = tid; f < C * C / NV; f += kBwdThreads) {
        FV p;
        p.load(gP + f * NV);
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            frag_pos<KB>(f * NV + j, C, r, k);
            s[L::P + r * C + k] = p.e[j];
        }
    }
    __syncthreads();
    // write the transposes, one lane fragment per step
    for (int f = tid; f < C * DK / NV; f += kBwdThreads) {
        FV w, q, kt;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            frag_pos<KB>(f * NV + j, C, r, k);         // W^T, (Q*Gamma)^T: rows DK, K = C
            w.e[j] = s[L::W + k * DK + r];
            q.e[j] = s[L::Q + k * DK + r];
            frag_pos<KB>(f * NV + j, DK, r, k);        // Ktil: rows C, K = DK
            kt.e[j] = s[L::K + k * C + r];
        }
        w.store(gW + f * NV);
        q.store(gQ + f * NV);
        kt.store(gK + f * NV);
    }
    for (int f = tid; f < C * C / NV; f += kBwdThreads) {
        FV p;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            frag_pos<KB>(f * NV + j, C, r, k);
            p.e[j] = s[L::P + k * C + r];
        }
        p.store(gP + f * NV);
    }
}

// ---- reverse chain ----------------------------------------------------------
template <typename T, int C, int DK>
struct RevGeom {
    static constexpr int KB = KBlock<T, C, DK>::value;
    static constexpr int NV = KB / 4;
    static constexpr int NT = DK / 16, NM = C / 16, NKD = DK / KB, NKC = C / KB;
    static constexpr int SPW = (NT + 3) / 4;
};

// One workgroup per (b, h, 16-column slice), chunks in reverse: X = P^T dO +
// Ktil dS for token tile w, then dS <- diag(Gamma_{C-1}) dS + (Q*Gamma)^T dO
// - W^T X for the state tiles w, w + 4, ..; dS and -X are exchanged through
// LDS as MFMA B fragments (two barriers per chunk), dO of the column slice is
// staged transposed, and dSn and X go out through LDS as 16-byte stores.
// Operands take the forward chain's route: four compute wavefronts and four
// loader wavefronts.  Loader 4 + w moves compute wave w's operands of the chunk two
// steps ahead into a two-stage FIFO with direct global-to-LDS loads (the P^T
// and Ktil fragments of its token tile before the step's first barrier, the
// (Q*Gamma)^T and W^T fragments and Gamma_C rows of its state tiles after it,
// then L2 prefetches of the chunk five steps ahead into a sink); it waits for
// the next chunk before the first barrier, and the compute wave moves that
// chunk into registers before the second.  Every loader issues the same
// loads each step, so its explicit wait counts are exact.
template <typename T, int C, int DK>
struct RevFifo {
    using G = RevGeom<T, C, DK>;
    static constexpr int FB = 64 * G::NV * (int)sizeof(T);      // one 64-lane fragment
    static constexpr int OPT = 0;                               // P^T, token tile     [NKC]
    static constexpr int OKT = OPT + G::NKC * FB;               // Ktil, token tile    [NKD]
    static constexpr int OQT = OKT + G::NKD * FB;               // (Q*Gamma)^T, state tiles [SPW][NKC]
    static constexpr int OWT = OQT + G::SPW * G::NKC * FB;      // W^T, state tiles    [SPW][NKC]
    static constexpr int OG = OWT + G::SPW * G::NKC * FB;       // Gamma_C rows        [SPW][4][16 B]
    static constexpr int STAGE = OG + G::SPW * 64;
    static constexpr size_t SINK = 2 * 4 * (size_t)STAGE;
    static constexpr size_t BYTES = SINK + 1024;
    static constexpr int runs(int bytes) { return (bytes + 1023) / 1024; }
    static constexpr int NA = runs(G::NKC * FB) + runs(G::NKD * FB);         // loads before barrier 1
    static constexpr int NDMA = NA + 2 * G::SPW * runs(G::NKC * FB) + 1;
    static constexpr int KPF = 2;                                             // L2 prefetch loads
    static constexpr size_t STATIC = (size_t)(G::NKD + G::NKC) * 64 * G::NV * sizeof(T) +
                                     2 * 16 * (size_t)C * sizeof(T) + (size_t)(DK + C) * 16 * 4;
    static_assert(NDMA + KPF <= 63, "vmcnt holds at most 63 outstanding loads");
    static_assert(BYTES + STATIC <= 160 * 1024, "LDS of one workgroup");
};

constexpr int kRevThreads = 512;                 // four compute + four loader wavefronts

template <typename T, int C, int DK>
__global__ __launch_bounds__(kRevThreads) void bwd_chain_fifo_kernel(BwdChainArgs a)
{
    using G = RevGeom<T, C, DK>;
    using L = RevFifo<T, C, DK>;
    using F = Frag<T, G::KB>;
    __shared__ F sSf[G::NKD * 64];      // dS as B fragments, k = channels
    __shared__ F sXf[G::NKC * 64];      // -X as B fragments, k = tokens
    __shared__ __attribute__((aligned(16))) T sDOt[2][16][C];
    __shared__ __attribute__((aligned(16))) float sOut[(DK + C) * 16];
    extern __shared__ __attribute__((aligned(16))) unsigned char fifo[];

    const int Dv = a.Dv, H = a.H, NS = Dv / 16;
    const int gid = blockIdx.x, xcd = gid % kXcds, jx = gid / kXcds;
    const int bh = (jx / NS) * kXcds + xcd, slice = jx % NS;
    if (bh >= a.B * H) return;
    const int h = bh % H;
    const int tid = threadIdx.x, lane = tid & 63, ln = lane & 15, lg = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int cw = wave & 3;                       // the compute wave a loader serves
    const int col = slice * 16 + ln;
    const T* dO = static_cast<const T*>(a.dO);
    const int drow = tid >> 2, dcol = 4 * (tid & 3);
    const SeqPos sp = locate_seq(bh, H, a.T, a.NC, a.cu, a.cs);
    const int NCs = sp.nc;
    if (NCs == 0) {
        // an empty sequence of a packed batch: dS0 = dST
        if (a.dS0 && wave < 4) {
#pragma unroll
            for (int u = 0; u < G::SPW; ++u) {
                const int t = wave + 4 * u;
                if (t < G::NT) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const size_t e = ((size_t)bh * DK + 16 * t + 4 * lg + i) * Dv + col;
                        a.dS0[e] = a.dST ? a.dST[e] : 0.f;
                    }
                }
            }
        }
        return;
    }
    // the chunk of step i (steps run the chunks backwards), clamped so that the
    // loads past the first chunk repeat it
    auto chunk_of = [&](int i) { return max(NCs - 1 - i, 0); };
    auto stg = [&](int i) { return fifo + (size_t)((i & 1) * 4 + cw) * L::STAGE; };

    if (wave >= 4) {
        // ---- loader wavefront ---------------------------------------------------
        // each column slice issues its runs of the shared blocks from another
        // starting run (dma_runs_rot)
        auto issue_a = [&](unsigned char* st, size_t unit) {
            const int mt = cw < G::NM ? cw : G::NM - 1;
            const unsigned char* pt = static_cast<const unsigned char*>(a.PT) +
                                      (unit * C * C + (size_t)mt * G::NKC * 64 * G::NV) * sizeof(T);
            const unsigned char* kt = static_cast<const unsigned char*>(a.Ktil) +
                                      (unit * C * DK + (size_t)mt * G::NKD * 64 * G::NV) * sizeof(T);
            if constexpr ((G::NKC * L::FB) % 1024 == 0 && (G::NKD * L::FB) % 1024 == 0) {
                dma_pair_rot<G::NKC * L::FB, G::NKD * L::FB>(pt, st + L::OPT, kt, st + L::OKT, lane, slice);
            } else {
                dma_run<G::NKC * L::FB>(pt, st + L::OPT, lane);
                dma_run<G::NKD * L::FB>(kt, st + L::OKT, lane);
            }
        };
        auto issue_b = [&](unsigned char* st, size_t unit) {
            const unsigned char* bs[2 * G::SPW];
            unsigned char* bd[2 * G::SPW];
#pragma unroll
            for (int u = 0; u < G::SPW; ++u) {
                const int t = min(cw + 4 * u, G::NT - 1);
                const size_t off = (unit * DK * C + (size_t)t * G::NKC * 64 * G::NV) * sizeof(T);
                bs[2 * u] = static_cast<const unsigned char*>(a.QGT) + off;
                bd[2 * u] = st + L::OQT + u * G::NKC * L::FB;
                bs[2 * u + 1] = static_cast<const unsigned char*>(a.WT) + off;
                bd[2 * u + 1] = st + L::OWT + u * G::NKC * L::FB;
            }
            if constexpr ((G::NKC * L::FB) % 1024 == 0) {
                dma_runs_rot<2 * G::SPW, G::NKC * L::FB>(bs, bd, lane, slice);
            } else {
#pragma unroll
                for (int x = 0; x < 2 * G::SPW; ++x) dma_run<G::NKC * L::FB>(bs[x], bd[x], lane);
            }
            // Gamma_C: lane j < 4 SPW fetches rows 16t + 4(j % 4) .. +3 of state
            // tile u = j / 4; they land at OG + 16 j
            if (lane < 4 * G::SPW) {
                const int t = min(cw + 4 * (lane >> 2), G::NT - 1);
                dma16(a.GC + unit * DK + 16 * t + 4 * (lane & 3), st + L::OG);
            }
        };
        // L2 prefetch: 1 KB pieces of a chunk's P^T, Ktil, (Q*Gamma)^T, W^T; the
        // column slices of one (b, h) share an XCD, so each takes every NS-th
        // piece, its four loaders every fourth of those
        constexpr int NPIECE = (C * C + 3 * C * DK) * (int)sizeof(T) / 1024;
        const int per_wg = (NPIECE + NS - 1) / NS;
        unsigned char* sink = fifo + L::SINK;
        auto prefetch = [&](size_t unit) {
#pragma unroll
            for (int i = 0; i < L::KPF; ++i) {
                const int q = cw + 4 * i;
                int p = slice + NS * q;
                if (q >= per_wg || p >= NPIECE) p = slice % NPIECE;
                int off = p * 1024;
                const unsigned char* base;
                if (off < C * C * (int)sizeof(T)) {
                    base = static_cast<const unsigned char*>(a.PT) + unit * C * C * sizeof(T);
                } else {
                    off -= C * C * (int)sizeof(T);
                    const int blk = C * DK * (int)sizeof(T);
                    const void* arr = off < blk ? a.Ktil : (off < 2 * blk ? a.QGT : a.WT);
                    off %= blk;
                    base = static_cast<const unsigned char*>(arr) + unit * C * DK * sizeof(T);
                }
                dma16(base + off + 16 * lane, sink);
            }
        };
        issue_a(stg(0), sp.ubase + chunk_of(0));
        issue_b(stg(0), sp.ubase + chunk_of(0));
        issue_a(stg(1), sp.ubase + chunk_of(1));
        issue_b(stg(1), sp.ubase + chunk_of(1));
        prefetch(sp.ubase + chunk_of(2));
        wait_vm<L::NDMA + L::KPF>();                  // step 0's chunk landed
        lds_barrier();                                // B0: compute reads it
        lds_barrier();                                // B1: stage 0 free
        for (int i = 0; i < NCs; ++i) {
            // step i + 2's chunk into the stage step i's chunk left; loads
            // issued after step i + 1's chunk: the previous prefetch and part A
            issue_a(stg(i), sp.ubase + chunk_of(i + 2));
            wait_vm<L::NA + L::KPF>();                // step i + 1's chunk landed
            lds_barrier();                            // barrier 1 of step i
            issue_b(stg(i), sp.ubase + chunk_of(i + 2));
            prefetch(sp.ubase + chunk_of(i + 5));
            lds_barrier();                            // barrier 2 of step i
        }
        wait_vm<0>();   // no load may land in LDS after the workgroup ends
        return;
    }

    // ---- compute wavefront ----------------------------------------------------------
    f32x4 dS[G::SPW];
#pragma unroll
    for (int u = 0; u < G::SPW; ++u) {
        const int t = wave + 4 * u;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            dS[u][i] = (a.dST && t < G::NT) ? a.dST[((size_t)bh * DK + 16 * t + 4 * lg + i) * Dv + col] : 0.f;
        if (t < G::NT) put_tile<T, G::KB>(sSf, t, lane, dS[u]);
    }
    struct Ops {
        F pt[G::NKC], kt[G::NKD], qt[G::SPW][G::NKC], wt[G::SPW][G::NKC];
        f32x4 gc[G::SPW];
    };
    auto read_ops = [&](Ops& o, const unsigned char* st) {
        const F* pt = reinterpret_cast<const F*>(st + L::OPT);
        const F* kt = reinterpret_cast<const F*>(st + L::OKT);
#pragma unroll
        for (int s = 0; s < G::NKC; ++s) o.pt[s] = pt[s * 64 + lane];
#pragma unroll
        for (int s = 0; s < G::NKD; ++s) o.kt[s] = kt[s * 64 + lane];
#pragma unroll
        for (int u = 0; u < G::SPW; ++u) {
            const F* qt = reinterpret_cast<const F*>(st + L::OQT + u * G::NKC * L::FB);
            const F* wt = reinterpret_cast<const F*>(st + L::OWT + u * G::NKC * L::FB);
#pragma unroll
            for (int s = 0; s < G::NKC; ++s) {
                o.qt[u][s] = qt[s * 64 + lane];
                o.wt[u][s] = wt[s * 64 + lane];
            }
            o.gc[u] = *reinterpret_cast<const f32x4*>(st + L::OG + 16 * (4 * u + lg));
        }
    };
    // this thread's dO piece of chunk m (rows past the end, and threads past
    // the chunk, read the sequence's last row; they are zeroed when staged)
    auto load_do = [&](int m) {
        const int row = min(m * C + min(drow, C - 1), sp.len - 1);
        return Vec4<T>::load(dO + (((size_t)sp.row0 + row) * H + h) * Dv + slice * 16 + dcol);
    };
    auto stage_do = [&](const Vec4<T>& dv, int n) {
        if (drow < C) {
            const bool ok = n * C + drow < sp.len;
#pragma unroll
            for (int x = 0; x < 4; ++x) sDOt[n & 1][dcol + x][drow] = ok ? dv.elem(x) : from_f32<T>(0.f);
        }
    };
    auto do_frags = [&](F* dof, int n) {
#pragma unroll
        for (int s = 0; s < G::NKC; ++s) {
            const T* base = &sDOt[n & 1][ln][s * G::KB + 4 * lg];
            if constexpr (G::KB == 32) {
                const Vec4<T> lo = Vec4<T>::load(base), hi = Vec4<T>::load(base + 16);
                float f[8];
#pragma unroll
                for (int x = 0; x < 4; ++x) { f[x] = lo.get(x); f[4 + x] = hi.get(x); }
                dof[s] = F::from(f);
            } else {
                const Vec4<T> q4 = Vec4<T>::load(base);
                float f[4];
#pragma unroll
                for (int x = 0; x < 4; ++x) f[x] = q4.get(x);
                dof[s] = F::from(f);
            }
        }
    };

    stage_do(load_do(NCs - 1), NCs - 1);
    Vec4<T> dnext = load_do(max(NCs - 2, 0));        // dO of the next step's chunk
    Ops cur;
    lds_barrier();                                    // B0: step 0's chunk is in stage 0
    read_ops(cur, stg(0));
    lds_barrier();                                    // B1: stage 0 may be refilled
    for (int i = 0; i < NCs; ++i) {
        const int n = NCs - 1 - i;
        const size_t unit = sp.ubase + n;
        // the gradient of the state leaving chunk n (rows 0 .. DK-1 of sOut)
#pragma unroll
        for (int u = 0; u < G::SPW; ++u) {
            const int t = wave + 4 * u;
            if (t < G::NT) {
#pragma unroll
                for (int x = 0; x < 4; ++x) sOut[(16 * t + 4 * lg + x) * 16 + ln] = dS[u][x];
            }
        }
        F sf[G::NKD], dof[G::NKC];
#pragma unroll
        for (int s = 0; s < G::NKD; ++s) sf[s] = sSf[s * 64 + lane];
        do_frags(dof, n);
        // X for token tile `wave`
        if (G::NM == 4 || wave < G::NM) {
            f32x4 acc = zero4();
#pragma unroll
            for (int s = 0; s < G::NKC; ++s) acc = mma(cur.pt[s], dof[s], acc);
#pragma unroll
            for (int s = 0; s < G::NKD; ++s) acc = mma(cur.kt[s], sf[s], acc);
            f32x4 neg;
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                sOut[(DK + 16 * wave + 4 * lg + x) * 16 + ln] = acc[x];
                neg[x] = -acc[x];
            }
            put_tile<T, G::KB>(sXf, wave, lane, neg);
        }
        lds_barrier();                                // barrier 1
        // dSn [DK][16] and X [C][16] of this column slice to memory (written by
        // the loader waves instead, between the barriers: no faster)
        for (int e = tid; e < (DK + C) * 4; e += 256) {
            const int r = e >> 2, c4 = 4 * (e & 3);
            const float4 v = *reinterpret_cast<const float4*>(&sOut[r * 16 + c4]);
            float* dst = r < DK ? a.DSN + (unit * DK + r) * Dv + slice * 16 + c4
                                : a.XB + (unit * C + r - DK) * Dv + slice * 16 + c4;
            *reinterpret_cast<float4*>(dst) = v;
        }
        F xf[G::NKC];
#pragma unroll
        for (int s = 0; s < G::NKC; ++s) xf[s] = sXf[s * 64 + lane];
        // dS <- diag(Gamma_{C-1}) dS + (Q*Gamma)^T dO - W^T X for this wave's state tiles
#pragma unroll
        for (int u = 0; u < G::SPW; ++u) {
            const int t = wave + 4 * u;
            if (G::NT % 4 == 0 || t < G::NT) {
                f32x4 acc;
#pragma unroll
                for (int x = 0; x < 4; ++x) acc[x] = cur.gc[u][x] * dS[u][x];
#pragma unroll
                for (int s = 0; s < G::NKC; ++s) acc = mma(cur.qt[u][s], dof[s], acc);
#pragma unroll
                for (int s = 0; s < G::NKC; ++s) acc = mma(cur.wt[u][s], xf[s], acc);
                dS[u] = acc;
                put_tile<T, G::KB>(sSf, t, lane, acc);
            }
        }
        if (n >= 1) {
            stage_do(dnext, n - 1);
            dnext = load_do(max(n - 2, 0));
        }
        // the next step's operands (its loader waited for them before barrier 1)
        read_ops(cur, stg(i + 1));
        lds_barrier();                                // barrier 2
    }
    if (a.dS0) {
#pragma unroll
        for (int u = 0; u < G::SPW; ++u) {
            const int t = wave + 4 * u;
            if (t < G::NT) {
#pragma unroll
                for (int x = 0; x < 4; ++x)
                    a.dS0[((size_t)bh * DK + 16 * t + 4 * lg + x) * Dv + col] = dS[u][x];
            }
        }
    }
}

// ---- per-chunk gradients ----------------------------------------------------
// One workgroup of 8 wavefronts per chunk.  Wave w owns the channel tiles
// ct = w, w + 8, ..; its lane (n, g) owns, for each such tile, the rows
// 16 mt + 4 g + m (every token tile mt, m = 0..3) of channel 16 ct + n: the
// C-layout of the F1 / F2 / F3 accumulator tiles, so every per-(row, channel)
// quantity stays in that lane, and the 64 rows of one channel sit in the four
// lanes n, n + 16, n + 32, n + 48 of one wavefront (the prefix and suffix
// sums of dalpha are shuffles among them).
constexpr int kLocalThreads = 512;
constexpr int kLocalWaves = kLocalThreads / 64;

template <typename T, int C, int DK>
struct LocalGeom {
    static constexpr int NM = C / 16, NCT = DK / 16, CTW = (NCT + kLocalWaves - 1) / kLocalWaves;
    static constexpr int DVMAX = sizeof(T) == 4 ? 64 : 128;
    static constexpr int LDV = DVMAX + 4;      // row stride of the [C][Dv] fp32 arrays
    static constexpr int LDT = C + 4;          // row stride of the [C][C] fp32 arrays
    static constexpr size_t al16(size_t x) { return (x + 15) & ~size_t(15); }
    // R0: Tinv (y phase), then B1, B3
    // (after the final phase's reads of B1 and B3, the region holds dalpha
    // [C][DKA] fp32 for the coalesced write-out)
    static constexpr int DKA = DK + 4;
    static constexpr size_t DAB = 4 * (size_t)C * DKA;
    static constexpr size_t B1 = 0, B3 = B1 + 4 * (size_t)C * LDT,
                            R0 = al16(B3 + 4 * (size_t)C * LDT > DAB ? B3 + 4 * (size_t)C * LDT : DAB);
    static constexpr size_t TI = 0;
    // R1, GEMM phase: dO, Delta, Y
    static constexpr size_t DO = R0, DL = DO + 4 * (size_t)C * LDV, YY = DL + 4 * (size_t)C * LDV;
    static constexpr size_t R1A = YY + 4 * (size_t)C * LDV;
    // R1, weight phase: alpha (fp32), k, q (io type), one decayed operand
    // (fp32 [NDR][DKP]: k, q or beta k decayed to the 16-token block edges)
    // and the per-channel block-edge products GB (Gamma_{16 b - 1}) and GE
    // (rho(C - 1, 16 b + 15)), [NM][DK] each
    // (row strides padded by 16 bytes: the final phase's lanes read one
    // channel from rows 4 apart, which would otherwise share banks)
    static constexpr int NDR = 8 * NM * (NM - 1), DKP = DK + 4;
    static constexpr int DKT = DK + 16 / (int)sizeof(T);
    static constexpr size_t AL = R0, KK = AL + 4 * (size_t)C * DKA, QQ = al16(KK + sizeof(T) * C * DKT);
    // DEC: the decayed operands, then (final phase) dq and dk [C][DKT] io type
    static constexpr size_t DECB = 4 * (size_t)NDR * DKP, DQB = 2 * sizeof(T) * (size_t)C * DKT;
    static constexpr size_t DEC = al16(QQ + sizeof(T) * C * DKT), GB = DEC + al16(DECB > DQB ? DECB : DQB);
    static constexpr size_t GE = GB + 4 * (size_t)NM * DK;
    static constexpr size_t R1B = GE + 4 * (size_t)NM * DK;
    // small arrays
    static constexpr size_t R1 = R1A > R1B ? R1A : R1B;
    static constexpr size_t BETA = R1, DB = BETA + 4 * C, DBW = DB + 4 * C;
    static constexpr size_t DBV = DBW + 4 * (size_t)kLocalWaves * C;
    static constexpr size_t BYTES = DBV + 4 * (size_t)kLocalWaves * C;
    static_assert(BYTES <= 160 * 1024, "LDS");
    static_assert(CTW == 1, "one channel tile per wavefront");
    static_assert((NM - 1) * DK <= kLocalThreads, "one thread per (channel, block)");
};

template <typename T, int C, int DK>
__global__ __launch_bounds__(kLocalThreads) void bwd_local_kernel(BwdLocalArgs a)
{
    using G = LocalGeom<T, C, DK>;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    float* sT = reinterpret_cast<float*>(lds + G::TI);
    float* sB1 = reinterpret_cast<float*>(lds + G::B1);
    float* sB3 = reinterpret_cast<float*>(lds + G::B3);
    float* sDO = reinterpret_cast<float*>(lds + G::DO);
    float* sDL = reinterpret_cast<float*>(lds + G::DL);
    float* sY = reinterpret_cast<float*>(lds + G::YY);
    float* sAl = reinterpret_cast<float*>(lds + G::AL);
    T* sK = reinterpret_cast<T*>(lds + G::KK);
    T* sQ = reinterpret_cast<T*>(lds + G::QQ);
    float* sDec = reinterpret_cast<float*>(lds + G::DEC);
    float* sGB = reinterpret_cast<float*>(lds + G::GB);
    float* sGE = reinterpret_cast<float*>(lds + G::GE);
    float* sBeta = reinterpret_cast<float*>(lds + G::BETA);
    float* sDBw = reinterpret_cast<float*>(lds + G::DBW);     // [waves][C]
    float* sDBv = reinterpret_cast<float*>(lds + G::DBV);     // [waves][C]: v . y partials
    constexpr int LDV = G::LDV, LDT = G::LDT, NM = G::NM, NW = kLocalWaves, NTH = kLocalThreads;
    constexpr int DKA = G::DKA, DKT = G::DKT;

    const int Dv = a.Dv, H = a.H, NVT = Dv / 16;
    // dense batches: chunk index by chunk index, every (b, h) of one chunk
    // index on consecutive workgroups, so the workgroups in flight read whole
    // token rows of q, k, v, dO and alpha
    size_t unit = blockIdx.x;
    if (!a.cu) {
        const int bhn = (int)gridDim.x / a.NC;
        unit = (size_t)((int)blockIdx.x % bhn) * a.NC + (int)blockIdx.x / bhn;
    }
    const UnitPos up = locate_unit((int)unit, H, a.T, a.NC, C, a.cu, a.cs, a.N);
    if (!up.valid) {                  // past the last sequence of a packed batch
        if (threadIdx.x == 0) a.FLB[unit] = 0;
        return;
    }
    const int h = up.h;
    const int nvalid = up.nvalid;
    const size_t row0 = (size_t)up.row0;                        // first token row
    const int tid = threadIdx.x, lane = tid & 63, ln = lane & 15, lg = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    auto tok = [&](int r) { return (row0 + r) * H + h; };       // token index of local row r

    // ---- load (every loop has a compile-time trip count, so the loads of a
    //      thread are issued together) ---------------------------------------------
    // (every load of this phase is issued before its results are used: the
    // addresses are clamped instead of guarded, and the gate test has no
    // short-circuit, so no load waits for another)
    constexpr int NA0 = (C * DK / 4 + NTH - 1) / NTH;
    float4 al0[NA0];
#pragma unroll
    for (int x = 0; x < NA0; ++x) {
        const int idx = min(tid + NTH * x, C * DK / 4 - 1);
        const int r = min(idx / (DK / 4), nvalid - 1), c4 = 4 * (idx % (DK / 4));
        al0[x] = *reinterpret_cast<const float4*>(a.alpha + tok(r) * DK + c4);
    }
    const float bt0 = a.beta[tok(min(tid, nvalid - 1))];
    constexpr int NTL = (C * C / 4 + NTH - 1) / NTH;
    float4 t40[NTL];
#pragma unroll
    for (int x = 0; x < NTL; ++x)
        t40[x] = *reinterpret_cast<const float4*>(a.Tm + unit * C * C + 4 * min(tid + NTH * x, C * C / 4 - 1));
    const T* dO = static_cast<const T*>(a.dO);
    // dO, Delta, and X (into the Y buffer; y replaces it below)
    constexpr int NL = (C * G::DVMAX / 4 + NTH - 1) / NTH;
    const int DV4 = Dv / 4;
    Vec4<T> ro[NL];
    float4 rd[NL], rx[NL];
#pragma unroll
    for (int x = 0; x < NL; ++x) {
        const int idx = min(tid + NTH * x, C * DV4 - 1);
        const int r = idx / DV4, c4 = 4 * (idx % DV4), rv = min(r, nvalid - 1);
        ro[x] = Vec4<T>::load(dO + tok(rv) * Dv + c4);
        rd[x] = *reinterpret_cast<const float4*>(a.DL + (unit * C + rv) * Dv + c4);
        rx[x] = *reinterpret_cast<const float4*>(a.XB + (unit * C + r) * Dv + c4);
    }
    bool tiny = false;
#pragma unroll
    for (int x = 0; x < NA0; ++x) {
        const int idx = tid + NTH * x;
        const float4 al = al0[x];
        const float m = fminf(fminf(fabsf(al.x), fabsf(al.y)), fminf(fabsf(al.z), fabsf(al.w)));
        tiny = tiny | (idx < C * DK / 4 && idx / (DK / 4) < nvalid && m < kTinyGate);
    }
    if (tid < C) {
        sBeta[tid] = tid < nvalid ? bt0 : 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) sDBv[w * C + tid] = 0.f;
    }
#pragma unroll
    for (int x = 0; x < NTL; ++x) {
        const int idx = tid + NTH * x;
        if (idx < C * C / 4)
            *reinterpret_cast<float4*>(sT + (4 * idx / C) * LDT + (4 * idx) % C) = t40[x];
    }
#pragma unroll
    for (int x = 0; x < NL; ++x) {
        const int idx = tid + NTH * x;
        if (idx < C * DV4) {
            const int r = idx / DV4, c4 = 4 * (idx % DV4);
            const float w = r < nvalid ? 1.f : 0.f;          // rows past the end: zero
            const float4 dd = rd[x];
            *reinterpret_cast<float4*>(sDO + r * LDV + c4) =
                make_float4(w * ro[x].get(0), w * ro[x].get(1), w * ro[x].get(2), w * ro[x].get(3));
            *reinterpret_cast<float4*>(sDL + r * LDV + c4) = make_float4(w * dd.x, w * dd.y, w * dd.z, w * dd.w);
            *reinterpret_cast<float4*>(sY + r * LDV + c4) = rx[x];
        }
    }
    // loads of later phases issued now, so that their latency overlaps the
    // y and B products: v of this wave's y tiles, S and dSn of its channel tiles
    T* dv = static_cast<T*>(a.dv);
    const T* vg = static_cast<const T*>(a.v);
    constexpr int MAXJ = (NM * (G::DVMAX / 16) + NW - 1) / NW;
    constexpr int NKV = G::DVMAX / 16;
    float vv[MAXJ][4];
#pragma unroll
    for (int jj = 0; jj < MAXJ; ++jj) {
        const int job = min(wave + NW * jj, NM * NVT - 1);
        const int mt = job / NVT, vt = job % NVT;
#pragma unroll
        for (int i = 0; i < 4; ++i)        // rows past the end read the last row (weight 0 below)
            vv[jj][i] = to_f32(vg[tok(min(16 * mt + 4 * lg + i, nvalid - 1)) * Dv + 16 * vt + ln]);
    }
    Vec4<float> pS[G::CTW][NKV], pN[G::CTW][NKV];
#pragma unroll
    for (int cw = 0; cw < G::CTW; ++cw) {
        const int ct = min(wave + NW * cw, G::NCT - 1);
        const float* ps = a.CS32 + (unit * DK + 16 * ct + ln) * Dv + 4 * lg;
        const float* pn = a.DSN + (unit * DK + 16 * ct + ln) * Dv + 4 * lg;
#pragma unroll
        for (int s2 = 0; s2 < NKV; ++s2) {
            const int so = 16 * min(s2, NVT - 1);
            pS[cw][s2] = Vec4<float>::load(ps + so);
            pN[cw][s2] = Vec4<float>::load(pn + so);
        }
    }
    const int any_tiny = __syncthreads_or(tiny);

    // ---- y = Tinv^T X, dv = diag(beta) y, and v . y -----------------------------------
    f32x4 yt[MAXJ];
#pragma unroll
    for (int jj = 0; jj < MAXJ; ++jj) {
        const int job = wave + NW * jj;
        yt[jj] = zero4();
        if (job < NM * NVT) {
            const int mt = job / NVT, vt = job % NVT;
#pragma unroll
            for (int s2 = 0; s2 < NM; ++s2) {        // Tinv[k][m] = 0 for k < m
                if (s2 < mt) continue;
                float fa[4], fb[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int kk = 16 * s2 + 4 * lg + j;
                    fa[j] = sT[kk * LDT + 16 * mt + ln];
                    fb[j] = sY[kk * LDV + 16 * vt + ln];
                }
                yt[jj] = mma_k16(Vec4<float>::from(fa), Vec4<float>::from(fb), yt[jj]);
            }
        }
    }
    __syncthreads();     // every read of X is done: y takes its place
#pragma unroll
    for (int jj = 0; jj < MAXJ; ++jj) {
        const int job = wave + NW * jj;
        if (job < NM * NVT) {
            const int mt = job / NVT, vt = job % NVT;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * mt + 4 * lg + i, c = 16 * vt + ln;
                const float yv = yt[jj][i];
                sY[r * LDV + c] = yv;
                const float vy = row16_sum(r < nvalid ? vv[jj][i] * yv : 0.f);
                if (ln == 0) sDBv[wave * C + r] += vy;
            }
        }
    }
    __syncthreads();
    // dv = diag(beta) y, written as whole 16-byte row pieces
    {
        constexpr int VQ = 16 / (int)sizeof(T);
        const int NQV = Dv / VQ;
        for (int idx = tid; idx < C * NQV; idx += NTH) {
            const int r = idx / NQV, cq = VQ * (idx % NQV);
            if (r < nvalid) {
                const float br = sBeta[r];
                __attribute__((aligned(16))) T o[VQ];
#pragma unroll
                for (int x = 0; x < VQ; ++x) o[x] = from_f32<T>(br * sY[r * LDV + cq + x]);
                *reinterpret_cast<uint4*>(dv + tok(r) * Dv + cq) = *reinterpret_cast<const uint4*>(o);
            }
        }
    }

    // ---- B1 = dO Delta^T (i <= r), B3 = Y Delta^T (i < r): lower tiles --------------
    // (each strictly lower element also goes to its mirror place, which nothing
    // else uses: the final phase reads B[r0 .. r0 + 3][i] as one 16-byte row
    // piece B^T[i][r0 .. r0 + 3])
    {
        constexpr int NP = NM * (NM + 1) / 2;
        for (int job = wave; job < 2 * NP; job += NW) {
            const int which = job / NP;
            int p = job % NP, mt = 0;
            while (p > mt) { p -= mt + 1; ++mt; }
            const int it = p;                          // it <= mt
            const float* src = which == 0 ? sDO : sY;
            const f32x4 acc = tile_tn<float>(src + 16 * mt * LDV, LDV, sDL + 16 * it * LDV, LDV, Dv, zero4());
            float* dst = which == 0 ? sB1 : sB3;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * mt + 4 * lg + i, ic = 16 * it + ln;
                if (ic < r) {
                    dst[r * LDT + ic] = acc[i];
                    dst[ic * LDT + r] = acc[i];
                } else if (ic == r) {
                    dst[r * LDT + r] = which == 0 ? acc[i] : 0.f;
                }
            }
        }
    }

    // ---- F1 = dO S^T, F2 = Y S^T, F3 = Delta dSn^T; sigma = rowdot(dSn, S) ----------
    // the weight phase's gates, keys and queries, loaded now (rows past the end
    // read the last row and are replaced by alpha = 1, k = q = 0 when stored)
    const T* kg = static_cast<const T*>(a.k);
    const T* qg = static_cast<const T*>(a.q);
    constexpr int NA = (C * DK / 4 + NTH - 1) / NTH;
    float4 wal[NA];
    Vec4<T> wk4[NA], wq4[NA];
#pragma unroll
    for (int x = 0; x < NA; ++x) {
        const int idx = min(tid + NTH * x, C * DK / 4 - 1);
        const int r = min(idx / (DK / 4), nvalid - 1), c4 = 4 * (idx % (DK / 4));
        wal[x] = *reinterpret_cast<const float4*>(a.alpha + tok(r) * DK + c4);
        wk4[x] = Vec4<T>::load(kg + tok(r) * DK + c4);
        wq4[x] = Vec4<T>::load(qg + tok(r) * DK + c4);
    }
    f32x4 F1[G::CTW][NM], F2[G::CTW][NM], F3[G::CTW][NM];
    float sigv[G::CTW];
#pragma unroll
    for (int cw = 0; cw < G::CTW; ++cw) {
        const int ct = wave + NW * cw;
        sigv[cw] = 0.f;
#pragma unroll
        for (int mt = 0; mt < NM; ++mt) F1[cw][mt] = F2[cw][mt] = F3[cw][mt] = zero4();
        if (ct < G::NCT) {
            float sig = 0.f;
            // bf16 inputs: the products run as bf16 MFMAs (operands rounded
            // from fp32, fp32 accumulation), fp32 inputs stay in fp32
            using V = Vec4<T>;
#pragma unroll
            for (int s = 0; s < G::DVMAX / 16; ++s) {
                if (s >= NVT) break;
                const Vec4<float> fS = pS[cw][s];
                const Vec4<float> fN = pN[cw][s];
#pragma unroll
                for (int j = 0; j < 4; ++j) sig += fS.v[j] * fN.v[j];
                const V bS = V::from(fS.v), bN = V::from(fN.v);
#pragma unroll
                for (int mt = 0; mt < NM; ++mt) {
                    const int off = (16 * mt + ln) * LDV + 16 * s + 4 * lg;
                    F1[cw][mt] = mma_k16(V::from(Vec4<float>::load(sDO + off).v), bS, F1[cw][mt]);
                    F2[cw][mt] = mma_k16(V::from(Vec4<float>::load(sY + off).v), bS, F2[cw][mt]);
                    F3[cw][mt] = mma_k16(V::from(Vec4<float>::load(sDL + off).v), bN, F3[cw][mt]);
                }
            }
            sig += __shfl_xor(sig, 16);
            sig += __shfl_xor(sig, 32);
            sigv[cw] = sig;
        }
    }
    // the small-gate kernel needs y: it replaces X in place (every read of X is done)
    if (any_tiny) {
        for (int idx = tid; idx < C * Dv; idx += NTH)
            a.XB[unit * C * Dv + idx] = sY[(idx / Dv) * LDV + idx % Dv];
    }
    __syncthreads();

    // ---- weight phase: alpha, k, q ----------------------------------------------------
    {
#pragma unroll
        for (int x = 0; x < NA; ++x) {
            const int idx = tid + NTH * x;
            if (idx >= C * DK / 4) break;
            const int r = idx / (DK / 4), c4 = 4 * (idx % (DK / 4));
            const bool ok = r < nvalid;
            *reinterpret_cast<float4*>(sAl + r * DKA + c4) = ok ? wal[x] : make_float4(1.f, 1.f, 1.f, 1.f);
            *reinterpret_cast<Vec4<T>*>(sK + r * DKT + c4) = ok ? wk4[x] : Vec4<T>::zero();
            *reinterpret_cast<Vec4<T>*>(sQ + r * DKT + c4) = ok ? wq4[x] : Vec4<T>::zero();
        }
    }
    __syncthreads();

    // ---- the off-diagonal parts of the decay-weighted sums, per 16-token block
    // b (rows 16 b .. 16 b + 15), as fp32 MFMA products: with e = 16 b - 1,
    //   sum_{i <= e} B[r,i] rho(r,i) k_i = rho(r, e) sum_i B[r,i] (k_i rho(e, i))
    // and with e' = 16 b + 15,
    //   sum_{j > e'} B[j,r] rho(j,r) x_j = rho(e', r) sum_j B[j,r] (x_j rho(j, e'))
    // (x = q with B1, x = beta k with B3).  The decayed operands are exact
    // running products of the gates (|factor| <= 1), built per channel.
    constexpr int DKP = G::DKP;
    auto offL = [](int b) { return 8 * b * (b - 1); };                 // rows of blocks before b
    auto offU = [](int b) { return 16 * (b * (NM - 1) - b * (b - 1) / 2); };
    f32x4 mL1[NM], mL3[NM], mU1[NM], mU2[NM];
#pragma unroll
    for (int b = 0; b < NM; ++b) mL1[b] = mL3[b] = mU1[b] = mU2[b] = zero4();
    const int ctw = wave;                       // this wave's channel tile (DK <= 128: one)
    // k decayed forward to each block edge; Gamma at the block edges
    // (each 16-token piece of the channel is read into registers before any
    // of its results is written, so the reads are issued together)
    // (one thread per (channel, block b): a channel's chains run side by side)
    if (tid < DK) {
        sGB[tid] = 1.f;
        sGE[(NM - 1) * DK + tid] = 1.f;
    }
    if (tid < (NM - 1) * DK) {
        const int c = tid % DK, b = 1 + tid / DK;
        float w = 1.f;
        for (int blk = b - 1; blk >= 0; --blk) {
            float av[16], kv[16];
#pragma unroll
            for (int x = 0; x < 16; ++x) {
                av[x] = sAl[(16 * blk + x) * DKA + c];
                kv[x] = to_f32(sK[(16 * blk + x) * DKT + c]);
            }
#pragma unroll
            for (int x = 15; x >= 0; --x) {
                sDec[(offL(b) + 16 * blk + x) * DKP + c] = kv[x] * w;
                w *= av[x];
            }
        }
        sGB[b * DK + c] = w;
    }
    __syncthreads();
    if (ctw < G::NCT) {
#pragma unroll
        for (int b = 1; b < NM; ++b) {
#pragma unroll
            for (int k0 = 0; k0 < 16 * b; k0 += 4) {
                const float bb = sDec[(offL(b) + k0 + lg) * DKP + 16 * ctw + ln];
                mL1[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(sB1[(16 * b + ln) * LDT + k0 + lg], bb, mL1[b], 0, 0, 0);
                mL3[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(sB3[(16 * b + ln) * LDT + k0 + lg], bb, mL3[b], 0, 0, 0);
            }
        }
    }
    __syncthreads();
    // q decayed backward to each block's end; rho(C - 1, block end)
    if (tid < (NM - 1) * DK) {
        const int c = tid % DK, b = tid / DK;
        float w = 1.f;
        for (int blk = b + 1; blk < NM; ++blk) {
            float av[16], qv[16];
#pragma unroll
            for (int x = 0; x < 16; ++x) {
                av[x] = sAl[(16 * blk + x) * DKA + c];
                qv[x] = to_f32(sQ[(16 * blk + x) * DKT + c]);
            }
#pragma unroll
            for (int x = 0; x < 16; ++x) {
                w *= av[x];
                sDec[(offU(b) + 16 * (blk - b - 1) + x) * DKP + c] = qv[x] * w;
            }
        }
        sGE[b * DK + c] = w;
    }
    __syncthreads();
    if (ctw < G::NCT) {
#pragma unroll
        for (int b = 0; b + 1 < NM; ++b) {
#pragma unroll
            for (int k0 = 16 * b + 16; k0 < C; k0 += 4) {
                const float bb = sDec[(offU(b) + k0 - 16 * b - 16 + lg) * DKP + 16 * ctw + ln];
                mU1[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(sB1[(k0 + lg) * LDT + 16 * b + ln], bb, mU1[b], 0, 0, 0);
            }
        }
    }
    __syncthreads();
    // beta k decayed backward to each block's end
    if (tid < (NM - 1) * DK) {
        const int c = tid % DK, b = tid / DK;
        float w = 1.f;
        for (int blk = b + 1; blk < NM; ++blk) {
            float av[16], kv[16];
#pragma unroll
            for (int x = 0; x < 16; ++x) {
                av[x] = sAl[(16 * blk + x) * DKA + c];
                kv[x] = sBeta[16 * blk + x] * to_f32(sK[(16 * blk + x) * DKT + c]);
            }
#pragma unroll
            for (int x = 0; x < 16; ++x) {
                w *= av[x];
                sDec[(offU(b) + 16 * (blk - b - 1) + x) * DKP + c] = kv[x] * w;
            }
        }
    }
    __syncthreads();
    if (ctw < G::NCT) {
#pragma unroll
        for (int b = 0; b + 1 < NM; ++b) {
#pragma unroll
            for (int k0 = 16 * b + 16; k0 < C; k0 += 4) {
                const float bb = sDec[(offU(b) + k0 - 16 * b - 16 + lg) * DKP + 16 * ctw + ln];
                mU2[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(sB3[(k0 + lg) * LDT + 16 * b + ln], bb, mU2[b], 0, 0, 0);
            }
        }
    }

    __syncthreads();   // the decayed operands are read: their region takes dq, dk
    float dbp[NM][4];
#pragma unroll
    for (int mt = 0; mt < NM; ++mt)
#pragma unroll
        for (int m = 0; m < 4; ++m) dbp[mt][m] = 0.f;
    T* dqg = static_cast<T*>(a.dq);
    T* dkg = static_cast<T*>(a.dk);
    // dq, dk and dalpha are staged in LDS (dq, dk where the decayed operands
    // were; dalpha where B1, B3 were, once every wave has read them) and
    // written out at the end as whole 16-byte row pieces
    T* sDQ = reinterpret_cast<T*>(lds + G::DEC);
    T* sDK = sDQ + C * DKT;
    float* sDA = reinterpret_cast<float*>(lds + G::B1);
    {
        constexpr int cw = 0;                  // (one channel tile per wavefront)
        const int ct = wave;
        const bool act = ct < G::NCT;
        const int c = 16 * (act ? ct : G::NCT - 1) + ln;
        auto al = [&](int t) { return sAl[t * DKA + c]; };
        auto kf = [&](int t) { return to_f32(sK[t * DKT + c]); };
        auto qf = [&](int t) { return to_f32(sQ[t * DKT + c]); };
        float Za[NM][4], Zb[NM][4];
        float gcl = 1.f;                   // Gamma of the lane's last row (row C - 1 in lanes lg = 3)
        if (act) {
#pragma unroll
            for (int mt = 0; mt < NM; ++mt) {
                const int r0 = 16 * mt + 4 * lg, r3 = r0 + 3;
                // L sums inside block mt (16 mt <= i < r0) with w = rho(r0, i), then
                // the block product (rho(r0, 16 mt - 1) = w alpha_{16 mt}) and
                // rho(r0 + m, r0); Gamma_{r0+m} = GB rho(r0, 16 mt - 1) rho(r0 + m, r0)
                float lq[4] = {0.f, 0.f, 0.f, 0.f}, lk[4] = {0.f, 0.f, 0.f, 0.f};
                float fL[4] = {1.f, 1.f, 1.f, 1.f}, wL = 1.f;
                {
                    for (int i = r0 - 1; i >= 16 * mt; --i) {
                        wL *= al(i + 1);
                        const float wk = wL * kf(i);
                        const float4 b1 = *reinterpret_cast<const float4*>(sB1 + i * LDT + r0);   // B1[r0 + m][i]
                        const float4 b3 = *reinterpret_cast<const float4*>(sB3 + i * LDT + r0);
                        lq[0] += b1.x * wk; lq[1] += b1.y * wk; lq[2] += b1.z * wk; lq[3] += b1.w * wk;
                        lk[0] += b3.x * wk; lk[1] += b3.y * wk; lk[2] += b3.z * wk; lk[3] += b3.w * wk;
                    }
                    const float pe = wL * al(16 * mt);          // rho(r0, 16 mt - 1)
                    wL = pe;
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        lq[m] += pe * mL1[mt][m];
                        lk[m] += pe * mL3[mt][m];
                    }
                    float f = 1.f;
#pragma unroll
                    for (int m = 1; m < 4; ++m) {
                        f *= al(r0 + m);
                        fL[m] = f;
                        lq[m] *= f;
                        lk[m] *= f;
                        // pairs inside the group: r0 <= i < r0 + m
                        float wi = 1.f;
#pragma unroll
                        for (int d = 1; d <= m; ++d) {
                            const int i = r0 + m - d;
                            wi *= al(i + 1);
                            const float wk = wi * kf(i);
                            lq[m] += sB1[i * LDT + r0 + m] * wk;
                            lk[m] += sB3[i * LDT + r0 + m] * wk;
                        }
                    }
                }
                // U sums inside block mt (r3 < j <= 16 mt + 15) with w = rho(j, r3),
                // then the block product (w = rho(16 mt + 15, r3)) and rho(r3, r0 + m);
                // rho(C - 1, r0 + m) = GE w rho(r3, r0 + m)
                float uq[4] = {0.f, 0.f, 0.f, 0.f}, uk[4] = {0.f, 0.f, 0.f, 0.f};
                float hU[4] = {1.f, 1.f, 1.f, 1.f}, wU = 1.f;
                {
                    for (int j = r3 + 1; j <= 16 * mt + 15; ++j) {
                        wU *= al(j);
                        const float wq = wU * qf(j), wk = wU * sBeta[j] * kf(j);
                        const float4 b1 = *reinterpret_cast<const float4*>(sB1 + j * LDT + r0);
                        const float4 b3 = *reinterpret_cast<const float4*>(sB3 + j * LDT + r0);
                        uq[0] += b1.x * wq; uq[1] += b1.y * wq; uq[2] += b1.z * wq; uq[3] += b1.w * wq;
                        uk[0] += b3.x * wk; uk[1] += b3.y * wk; uk[2] += b3.z * wk; uk[3] += b3.w * wk;
                    }
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        uq[m] += wU * mU1[mt][m];
                        uk[m] += wU * mU2[mt][m];
                    }
                    float f = 1.f;
#pragma unroll
                    for (int m = 2; m >= 0; --m) {
                        f *= al(r0 + m + 1);
                        hU[m] = f;
                        uq[m] *= f;
                        uk[m] *= f;
                        // pairs inside the group: r0 + m < j <= r3
                        float wj = 1.f;
#pragma unroll
                        for (int j = r0 + m + 1; j <= r3; ++j) {
                            wj *= al(j);
                            uq[m] += sB1[j * LDT + r0 + m] * wj * qf(j);
                            uk[m] += sB3[j * LDT + r0 + m] * wj * sBeta[j] * kf(j);
                        }
                    }
                }
                const float gbm = sGB[mt * DK + c], gem = sGE[mt * DK + c];
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int r = r0 + m;
                    const float kr = kf(r), qr = qf(r), br = sBeta[r];
                    const float b1d = sB1[r * LDT + r];
                    const float g = gbm * wL * fL[m], ge = gem * wU * hU[m];
                    const float f1 = F1[cw][mt][m], f2 = F2[cw][mt][m], f3 = F3[cw][mt][m];
                    const float dqv = g * f1 + lq[m] + b1d * kr;
                    const float dkv = ge * f3 + uq[m] + b1d * qr - uk[m] - br * (g * f2 + lk[m]);
                    dbp[mt][m] -= kr * (g * f2 + lk[m]);
                    Za[mt][m] = ge * kr * f3;
                    Zb[mt][m] = g * (qr * f1 - br * kr * f2) + qr * lq[m] - br * kr * lk[m] - kr * (uq[m] - uk[m]);
                    if (m == 3) gcl = g;
                    sDQ[r * DKT + c] = from_f32<T>(dqv);
                    sDK[r * DKT + c] = from_f32<T>(dkv);
                }
            }
        }
        __syncthreads();   // every read of B1 and B3 is done: the region takes dalpha
        if (act) {
            // alpha_r dalpha_r = Gamma_{C-1} sigma + (sum of Za over rows before r)
            // + (sum of Zb over rows from r on); the channel's rows are the lanes
            // ln + 16 j, j = 0..3 (row 16 mt + 4 j + m).  Za is replaced by its
            // exclusive prefix, then the suffix of Zb completes dalpha.
            const float gcs = __shfl(gcl, ln + 48) * sigv[cw];
            float run = 0.f;
#pragma unroll
            for (int mt = 0; mt < NM; ++mt) {
                const float sa = (Za[mt][0] + Za[mt][1]) + (Za[mt][2] + Za[mt][3]);
                float tot = 0.f, before = 0.f;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float x = __shfl(sa, ln + 16 * j);
                    tot += x;
                    before += j < lg ? x : 0.f;
                }
                float in = run + before;
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const float z = Za[mt][m];
                    Za[mt][m] = in;
                    in += z;
                }
                run += tot;
            }
            run = 0.f;
#pragma unroll
            for (int mt = NM - 1; mt >= 0; --mt) {
                const float sb = (Zb[mt][0] + Zb[mt][1]) + (Zb[mt][2] + Zb[mt][3]);
                float tot = 0.f, after = 0.f;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float x = __shfl(sb, ln + 16 * j);
                    tot += x;
                    after += j > lg ? x : 0.f;
                }
                float in = run + after;
#pragma unroll
                for (int m = 3; m >= 0; --m) {
                    in += Zb[mt][m];
                    const int r = 16 * mt + 4 * lg + m;
                    const float av = al(r);
                    const float z = gcs + Za[mt][m] + in;
                    sDA[r * DKA + c] = fabsf(av) >= kTinyGate ? z / av : 0.f;
                }
                run += tot;
            }
        }
    }
    // dbeta: sum over the lane's channels, then over the 16 lanes of a row
    // group; each wave covers every row once, and the waves' sums are added in
    // a fixed order below (the result does not depend on scheduling)
#pragma unroll
    for (int mt = 0; mt < NM; ++mt)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const float sacc = row16_sum(dbp[mt][m]);
            if (ln == 0) sDBw[wave * C + 16 * mt + 4 * lg + m] = sacc;
        }
    __syncthreads();
    {
        constexpr int VQ = 16 / (int)sizeof(T);        // io elements per 16-byte piece
        for (int idx = tid; idx < C * (DK / VQ); idx += NTH) {
            const int r = idx / (DK / VQ), cq = VQ * (idx % (DK / VQ));
            if (r < nvalid) {
                *reinterpret_cast<uint4*>(dqg + tok(r) * DK + cq) = *reinterpret_cast<const uint4*>(sDQ + r * DKT + cq);
                *reinterpret_cast<uint4*>(dkg + tok(r) * DK + cq) = *reinterpret_cast<const uint4*>(sDK + r * DKT + cq);
            }
        }
        for (int idx = tid; idx < C * (DK / 4); idx += NTH) {
            const int r = idx / (DK / 4), cq = 4 * (idx % (DK / 4));
            if (r < nvalid)
                *reinterpret_cast<float4*>(a.dalpha + tok(r) * DK + cq) = *reinterpret_cast<const float4*>(sDA + r * DKA + cq);
        }
    }
    if (tid < nvalid) {
        float sv = 0.f, sw = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            sv += sDBv[w * C + tid];
            sw += sDBw[w * C + tid];
        }
        a.dbeta[tok(tid)] = sv + sw;
    }
    if (tid == 0) a.FLB[unit] = any_tiny ? 1 : 0;
}

// ---- direct dalpha of small gates ---------------------------------------------
template <typename T, int C, int DK>
struct TinyLds {
    static constexpr int DVMAX = sizeof(T) == 4 ? 64 : 128;
    static constexpr size_t DL = 0, DO = DL + 4 * (size_t)C * DVMAX, E = DO + 4 * (size_t)C * DVMAX;
    static constexpr size_t LIST = E + 4 * (size_t)C * DVMAX, CNT = LIST + 4 * (size_t)C * DK;
    static constexpr size_t BYTES = CNT + 16;
};

template <typename T, int C, int DK>
__global__ __launch_bounds__(kBwdThreads) void bwd_tiny_kernel(BwdLocalArgs a)
{
    using L = TinyLds<T, C, DK>;
    static_assert(C <= 64, "one token per lane");
    const size_t unit = blockIdx.x;
    if (!a.FLB[unit]) return;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    float* sDL = reinterpret_cast<float*>(lds + L::DL);
    float* sDO = reinterpret_cast<float*>(lds + L::DO);
    float* sE = reinterpret_cast<float*>(lds + L::E);
    int* sList = reinterpret_cast<int*>(lds + L::LIST);
    int* sCnt = reinterpret_cast<int*>(lds + L::CNT);
    const int Dv = a.Dv, H = a.H;
    const UnitPos up = locate_unit((int)unit, H, a.T, a.NC, C, a.cu, a.cs, a.N);
    if (!up.valid) return;
    const int h = up.h;
    const int nvalid = up.nvalid;
    const size_t row0 = (size_t)up.row0;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    auto tok = [&](int r) { return (row0 + r) * H + h; };
    const T* dO = static_cast<const T*>(a.dO);
    const T* kg = static_cast<const T*>(a.k);
    const T* qg = static_cast<const T*>(a.q);

    if (tid == 0) *sCnt = 0;
    {
        // Delta, dO and dv = beta y of the chunk, and the gates: every load is
        // issued before any result is used (clamped addresses, no guards)
        constexpr int NL = (C * L::DVMAX / 4 + kBwdThreads - 1) / kBwdThreads;
        constexpr int NA = (C * DK / 4 + kBwdThreads - 1) / kBwdThreads;
        const int DV4 = Dv / 4, nl = nvalid * DV4, na = nvalid * (DK / 4);
        float4 rd[NL], ry[NL], ral[NA];
        Vec4<T> ro[NL];
        float rb[NL];
#pragma unroll
        for (int x = 0; x < NL; ++x) {
            const int idx = min(tid + kBwdThreads * x, nl - 1);
            const int r = idx / DV4, c4 = 4 * (idx % DV4);
            rd[x] = *reinterpret_cast<const float4*>(a.DL + (unit * C + r) * Dv + c4);
            ro[x] = Vec4<T>::load(dO + tok(r) * Dv + c4);
            ry[x] = *reinterpret_cast<const float4*>(a.XB + (unit * C + r) * Dv + c4);
            rb[x] = a.beta[tok(r)];
        }
#pragma unroll
        for (int x = 0; x < NA; ++x) {
            const int idx = min(tid + kBwdThreads * x, na - 1);
            const int r = idx / (DK / 4), c4 = 4 * (idx % (DK / 4));
            ral[x] = *reinterpret_cast<const float4*>(a.alpha + tok(r) * DK + c4);
        }
#pragma unroll
        for (int x = 0; x < NL; ++x) {
            const int idx = tid + kBwdThreads * x;
            if (idx < nl) {
                const int r = idx / DV4, c4 = 4 * (idx % DV4);
                const float bt = rb[x];
                const float4 y = ry[x];
                *reinterpret_cast<float4*>(sDL + r * Dv + c4) = rd[x];
                *reinterpret_cast<float4*>(sDO + r * Dv + c4) =
                    make_float4(ro[x].get(0), ro[x].get(1), ro[x].get(2), ro[x].get(3));
                *reinterpret_cast<float4*>(sE + r * Dv + c4) = make_float4(bt * y.x, bt * y.y, bt * y.z, bt * y.w);
            }
        }
        __syncthreads();   // (the count is zero before any thread adds to it)
#pragma unroll
        for (int x = 0; x < NA; ++x) {
            const int idx = tid + kBwdThreads * x;
            if (idx < na) {
                const int r = idx / (DK / 4), c4 = 4 * (idx % (DK / 4));
                const float v4[4] = {ral[x].x, ral[x].y, ral[x].z, ral[x].w};
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (fabsf(v4[j]) < kTinyGate) sList[atomicAdd(sCnt, 1)] = r * DK + c4 + j;
            }
        }
    }
    __syncthreads();
    const int cnt = *sCnt;
    constexpr int JPL = L::DVMAX / 64;           // columns per lane (at most)
    for (int e = wave; e < cnt; e += 4) {
        const int r = sList[e] / DK, c = sList[e] % DK;
        // the channel's gates, keys and queries, token t in lane t, broadcast
        // to the whole wavefront by readlane in the sweeps
        float at = 1.f, kt = 0.f, qt = 0.f;
        if (lane < nvalid) {
            at = a.alpha[tok(lane) * DK + c];
            kt = to_f32(kg[tok(lane) * DK + c]);
            qt = to_f32(qg[tok(lane) * DK + c]);
        }
        auto bc = [](float x, int t) {
            return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), t));
        };
        // S_{r-1}[c, :] forward from the chunk start
        float s[JPL], hh[JPL], g[JPL];
#pragma unroll
        for (int x = 0; x < JPL; ++x) {
            const int j = lane + 64 * x;
            s[x] = j < Dv ? a.CS32[(unit * DK + c) * Dv + j] : 0.f;
        }
        for (int t = 0; t < r; ++t) {
            const float a_t = bc(at, t), k_t = bc(kt, t);
#pragma unroll
            for (int x = 0; x < JPL; ++x) {
                const int j = lane + 64 * x;
                if (j < Dv) s[x] = a_t * s[x] + k_t * sDL[t * Dv + j];
            }
        }
        // H_r[c, :] backward from the chunk end: G_{last} = dSn + q dO, then
        // H_t = G_t - k_t dv_t,  G_{t-1} = alpha_t H_t + q_{t-1} dO_{t-1}
        const int tl = nvalid - 1;
        const float ql = bc(qt, tl);
#pragma unroll
        for (int x = 0; x < JPL; ++x) {
            const int j = lane + 64 * x;
            g[x] = j < Dv ? a.DSN[(unit * DK + c) * Dv + j] + ql * sDO[tl * Dv + j] : 0.f;
        }
        for (int t = tl; t >= r; --t) {
            const float k_t = bc(kt, t);
#pragma unroll
            for (int x = 0; x < JPL; ++x) {
                const int j = lane + 64 * x;
                hh[x] = j < Dv ? g[x] - k_t * sE[t * Dv + j] : 0.f;
            }
            if (t > r) {
                const float a_t = bc(at, t), q_p = bc(qt, t - 1);
#pragma unroll
                for (int x = 0; x < JPL; ++x) {
                    const int j = lane + 64 * x;
                    g[x] = j < Dv ? a_t * hh[x] + q_p * sDO[(t - 1) * Dv + j] : 0.f;
                }
            }
        }
        float d = 0.f;
#pragma unroll
        for (int x = 0; x < JPL; ++x) d += hh[x] * s[x];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) d += __shfl_xor(d, o);
        if (lane == 0) a.dalpha[tok(r) * DK + c] = d;
    }
}

// ---- the input prologue around the backward ("Semidirect Fourier Delta
// Attention" §3, eqs. (15), (17), (18)) --------------------------------------
// One token of one head per NQ = DK / 4 consecutive lanes, four channels per
// lane (the same grouping and fp32 arithmetic as the prep kernels' prologue).
template <typename T, int DK>
__global__ __launch_bounds__(256) void prologue_in_kernel(ProArgs a)
{
    constexpr int NQ = DK / 4, TPB = 256 / NQ;
    const size_t tokn = (size_t)blockIdx.x * TPB + threadIdx.x / NQ;
    const int c0 = 4 * (threadIdx.x % NQ);
    const bool ok = tokn < a.ntok;
    const size_t t = ok ? tokn : a.ntok - 1;          // idle lanes repeat the last token
    const size_t e = t * DK + c0;
    Vec4<T> k = Vec4<T>::load(static_cast<const T*>(a.k_raw) + e);
    Vec4<T> q = Vec4<T>::load(static_cast<const T*>(a.q_raw) + e);
    k = l2_normalised<T, NQ>(k, a.eps);
    if (a.normq) q = l2_normalised<T, NQ>(q, a.eps);
    const float4 g = *reinterpret_cast<const float4*>(a.gate + e);
    if (ok) {
        *reinterpret_cast<Vec4<T>*>(static_cast<T*>(a.kh) + e) = k;
        *reinterpret_cast<Vec4<T>*>(static_cast<T*>(a.qh) + e) = q;
        *reinterpret_cast<float4*>(a.al + e) =
            make_float4(a.amin + a.arange * sigmoid_f32(g.x), a.amin + a.arange * sigmoid_f32(g.y),
                        a.amin + a.arange * sigmoid_f32(g.z), a.amin + a.arange * sigmoid_f32(g.w));
        if (c0 == 0) a.be[t] = a.bmax * sigmoid_f32(a.blogit[t]);
    }
}

// gradients of the raw inputs from those of the transformed ones:
//   d gate = d alpha (amax - amin) s (1 - s),  d beta_logit = d beta bmax s (1 - s)
//   d x_raw = d x / (n + eps) - x_raw <x_raw, d x> / (n (n + eps)^2),  n = |x_raw|
// (x = k, and q when normalised; the second term absent for n = 0, zero
// when n + eps = 0).  d gate and d beta_logit are updated in place.
template <typename T, int DK>
__global__ __launch_bounds__(256) void prologue_out_kernel(ProArgs a)
{
    constexpr int NQ = DK / 4, TPB = 256 / NQ;
    const size_t tokn = (size_t)blockIdx.x * TPB + threadIdx.x / NQ;
    const int c0 = 4 * (threadIdx.x % NQ);
    const bool ok = tokn < a.ntok;
    const size_t t = ok ? tokn : a.ntok - 1;
    const size_t e = t * DK + c0;
    auto raw_grad = [&](const void* rawp, const void* gp, void* outp, bool norm) {
        const Vec4<T> x = Vec4<T>::load(static_cast<const T*>(rawp) + e);
        const Vec4<T> g = Vec4<T>::load(static_cast<const T*>(gp) + e);
        float f[4];
        if (!norm) {
#pragma unroll
            for (int i = 0; i < 4; ++i) f[i] = g.get(i);
        } else {
            float ss = 0.f, dot = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ss += x.get(i) * x.get(i);
                dot += x.get(i) * g.get(i);
            }
            const float n = __builtin_sqrtf(quad_group_sum<NQ>(ss));
            dot = quad_group_sum<NQ>(dot);
            const float den = n + a.eps;
            const float inv = den > 0.f ? 1.f / den : 0.f;
            const float c2 = (den > 0.f && n > 0.f) ? dot / (n * den * den) : 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) f[i] = g.get(i) * inv - x.get(i) * c2;
        }
        if (ok) *reinterpret_cast<Vec4<T>*>(static_cast<T*>(outp) + e) = Vec4<T>::from(f);
    };
    raw_grad(a.k_raw, a.dkh, a.dk_raw, true);
    raw_grad(a.q_raw, a.dqh, a.dq_raw, a.normq != 0);
    if (ok) {
        const float4 g = *reinterpret_cast<const float4*>(a.gate + e);
        float4 d = *reinterpret_cast<const float4*>(a.dgate + e);
        auto ds = [&](float x) { const float s = sigmoid_f32(x); return a.arange * s * (1.f - s); };
        d.x *= ds(g.x); d.y *= ds(g.y); d.z *= ds(g.z); d.w *= ds(g.w);
        *reinterpret_cast<float4*>(a.dgate + e) = d;
        if (c0 == 0) {
            const float s = sigmoid_f32(a.blogit[t]);
            a.dblogit[t] *= a.bmax * s * (1.f - s);
        }
    }
}

template <typename T, int DK>
hipError_t launch_pro_t(bool out, const ProArgs& a, hipStream_t stream)
{
    constexpr int TPB = 256 / (DK / 4);
    const unsigned grid = (unsigned)((a.ntok + TPB - 1) / TPB);
    if (out) return launch_kernel(prologue_out_kernel<T, DK>, dim3(grid), dim3(256), 0, stream, a);
    return launch_kernel(prologue_in_kernel<T, DK>, dim3(grid), dim3(256), 0, stream, a);
}

template <typename T>
hipError_t launch_pro_dk(bool out, int Dk, const ProArgs& a, hipStream_t stream)
{
    switch (Dk) {
    case 32: return launch_pro_t<T, 32>(out, a, stream);
    case 64: return launch_pro_t<T, 64>(out, a, stream);
    case 128: return launch_pro_t<T, 128>(out, a, stream);
    default: return hipErrorInvalidValue;
    }
}

// ---- launchers ------------------------------------------------------------------
template <typename K>
hipError_t set_lds(K kern, size_t bytes)
{
    return hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <typename T, int C, int DK>
hipError_t launch_bwd_t(int stage, const ChunkShape& s, const ChunkWorkspace& ws,
                        const BwdChainArgs& ca, const BwdLocalArgs& la, hipStream_t stream)
{
    const unsigned nu = (unsigned)((size_t)s.B * s.H * s.NC);
    switch (stage) {
    case 0: {
        using L = RelayoutLds<T, C, DK>;
        auto kern = relayout_kernel<T, C, DK>;
        const hipError_t e = set_lds(kern, L::BYTES);
        if (e != hipSuccess) return e;
        return launch_kernel(kern, dim3(nu), dim3(kBwdThreads), (uint32_t)L::BYTES, stream,
                             static_cast<T*>(ws.W), static_cast<T*>(ws.QG), static_cast<T*>(ws.Kt),
                             static_cast<T*>(ws.P));
    }
    case 1: {
        const int bh = s.B * s.H;
        const unsigned grid = (unsigned)(kXcds * (s.Dv / 16) * ((bh + kXcds - 1) / kXcds));
        using L = RevFifo<T, C, DK>;
        auto kern = bwd_chain_fifo_kernel<T, C, DK>;
        const hipError_t e = set_lds(kern, L::BYTES);
        if (e != hipSuccess) return e;
        return launch_kernel(kern, dim3(grid), dim3(kRevThreads), (uint32_t)L::BYTES, stream, ca);
    }
    case 2: {
        using G = LocalGeom<T, C, DK>;
        auto kern = bwd_local_kernel<T, C, DK>;
        const hipError_t e = set_lds(kern, G::BYTES);
        if (e != hipSuccess) return e;
        return launch_kernel(kern, dim3(nu), dim3(kLocalThreads), (uint32_t)G::BYTES, stream, la);
    }
    case 3: {
        using L = TinyLds<T, C, DK>;
        auto kern = bwd_tiny_kernel<T, C, DK>;
        const hipError_t e = set_lds(kern, L::BYTES);
        if (e != hipSuccess) return e;
        return launch_kernel(kern, dim3(nu), dim3(kBwdThreads), (uint32_t)L::BYTES, stream, la);
    }
    default: return hipErrorInvalidValue;
    }
}

template <typename T, int C>
hipError_t bwd_dk(int stage, const ChunkShape& s, const ChunkWorkspace& ws, const BwdChainArgs& ca,
                  const BwdLocalArgs& la, hipStream_t st)
{
    switch (s.Dk) {
    case 32: return launch_bwd_t<T, C, 32>(stage, s, ws, ca, la, st);
    case 64: return launch_bwd_t<T, C, 64>(stage, s, ws, ca, la, st);
    case 128:
        if constexpr (sizeof(T) == 2) return launch_bwd_t<T, C, 128>(stage, s, ws, ca, la, st);
        else return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
    }
}

template <typename T>
hipError_t bwd_c(int stage, const ChunkShape& s, const ChunkWorkspace& ws, const BwdChainArgs& ca,
                 const BwdLocalArgs& la, hipStream_t st)
{
    switch (s.C) {
    case 32: return bwd_dk<T, 32>(stage, s, ws, ca, la, st);
    case 64: return bwd_dk<T, 64>(stage, s, ws, ca, la, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_backward_prologue(bool out, IoType io, int Dk, const ProArgs& a, hipStream_t stream)
{
    if (a.ntok == 0) return hipSuccess;
    if (io == IoType::F32) return launch_pro_dk<float>(out, Dk, a, stream);
    return launch_pro_dk<bf16_t>(out, Dk, a, stream);
}

hipError_t launch_backward_stage(int stage, IoType io, const ChunkShape& s, const ChunkWorkspace& ws,
                                 const BwdChainArgs& ca, const BwdLocalArgs& la, hipStream_t stream)
{
    if (io == IoType::F32) return bwd_c<float>(stage, s, ws, ca, la, stream);
    return bwd_c<bf16_t>(stage, s, ws, ca, la, stream);
}

}  // namespace kda
