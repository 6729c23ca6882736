// chain_wide.hip — the sequential part of the chunkwise forward (state carried
// from chunk to chunk, "Kimi Delta Attention: a bounded case study", Exercise 2;
// "Semidirect Fourier Delta Attention", §1 contribution 4 and §2.2) with each
// chunk's outputs (same page, §3 eq. (14)):
//   Delta  = U - W S
//   O      = (Q * Gamma) S + P Delta
//   S_next = diag(Gamma_{C-1}) S + Ktil^T Delta
// for workgroups that own 16 CT columns of one (b, h) (columns of S evolve
// independently: §2.2 eq. (9)).  Every (b, h) needs all of a chunk's W, Q*Gamma,
// P and Ktil whatever the slice width, so wider slices take in fewer bytes per
// column; the operands are loaded straight into registers (no LDS staging),
// which measured faster per compute unit than direct-to-LDS loads.
//
// Workgroup = 8 wavefronts, chunk of 64 tokens (4 token tiles):
//   D wave m (0..3): token tile m of Delta (all CT column tiles); loads W and U
//                    rows of that tile;
//   O wave m (4..7): token tile m - 4 of O; loads Q*Gamma and P rows;
//   wave t (0..Dk/16 - 1): state row tile t (all column tiles); loads Ktil rows
//                    and Gamma_{C-1} of that tile.
// Each fragment of a chunk's operands is loaded by exactly one wave.  S and
// Delta are exchanged through LDS as MFMA B fragments; two barriers per chunk:
//   top:  D waves form Delta(n) from S(n) and write it; O waves finish O(n-1)
//         (P Delta(n-1)), store it, and form (Q*Gamma) S(n);
//   B1:   every wave reads Delta(n) and updates its state rows to S(n+1);
//   B2:   S(n+1) visible.
// Operands of chunk n + NS - 1 are loaded at the top of chunk n into the
// register set chunk n - 1 used (NS sets in turn, the loop unrolled by NS so
// every set keeps fixed registers); the compiler's own wait counts order them.
//
// Workgroups are numbered so that the column slices of one (b, h) run on one
// XCD (consecutive workgroup ids go to consecutive XCDs) and share its L2 for
// the chunk operands.
#include <type_traits>

#include "kda_chunk.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace {

constexpr int kWideWaves = 8;
constexpr int kWideThreads = 64 * kWideWaves;
constexpr int kXcds = 8;

template <typename T, int C, int DK, int CT>
struct WideGeom {
    static constexpr int KB = KBlock<T, C, DK>::value;
    static constexpr int NV = KB / 4;            // elements per lane of one fragment
    static constexpr int FE = 64 * NV;           // elements of one 64-lane fragment block
    static constexpr int NT = DK / 16;           // state row tiles
    static constexpr int NM = C / 16;            // token tiles
    static constexpr int NKD = DK / KB;          // k blocks over channels
    static constexpr int NKC = C / KB;           // k blocks over tokens
    static_assert(2 * NM == kWideWaves, "one D wave and one O wave per token tile");
    static_assert(NT <= kWideWaves, "at most one state row tile per wave");
    using F = Frag<T, KB>;
    // whether the waves of a role own a state row tile: D waves always (tile
    // t = wave < NM <= NT), O waves when Dk / 16 covers all eight waves
    template <bool ROLE_D> static constexpr bool has_t() { return ROLE_D || NT == kWideWaves; }
    // LDS: B fragments of S [CT][NKD][64] and of Delta [CT][NKC][64]
    static constexpr size_t SF = 0;
    static constexpr size_t DF = SF + (size_t)CT * NKD * 64 * sizeof(F);
    static constexpr size_t LDS = DF + (size_t)CT * NKC * 64 * sizeof(F);
};

// one chunk's operands of one wavefront; D waves (ROLE_D) and O waves keep
// different sets, and each role runs its own copy of the chunk loop, so the
// register allocator never holds both roles' operands at once
template <typename T, int C, int DK, int CT, bool ROLE_D>
struct WideOps {
    using G = WideGeom<T, C, DK, CT>;
    typename G::F a[G::NKD];                    // D: W rows of its token tile; O: Q * Gamma rows
    typename G::F p[ROLE_D ? 1 : G::NKC];       // O: P rows of its token tile
    Vec4<T> u[ROLE_D ? CT : 1];                 // D: U tiles of its token tile, one per column tile
    typename G::F kt[G::NKC];                   // Ktil rows of the wave's state row tile
    f32x4 gc;                                   // Gamma_{C-1} of the four rows this lane holds there
};

template <typename T, int C, int DK, int CT, bool ROLE_D>
__device__ __forceinline__ void load_ops(WideOps<T, C, DK, CT, ROLE_D>& o, const ChainArgs& a,
                                         size_t unit, int mt, int t, int ucol, int lane, int lg)
{
    using G = WideGeom<T, C, DK, CT>;
    using F = typename G::F;
    const T* A = static_cast<const T*>(ROLE_D ? a.W : a.QG) + unit * C * DK +
                 (size_t)mt * G::NKD * G::FE + lane * G::NV;
#pragma unroll
    for (int s = 0; s < G::NKD; ++s) o.a[s] = F::load(A + s * G::FE);
    if constexpr (ROLE_D) {
        // U tile (mt, column tile ucol + c): C layout, 4 elements per lane
        const T* U = static_cast<const T*>(a.U) + unit * C * a.Dv +
                     ((size_t)mt * (a.Dv / 16) + ucol) * 256 + lane * 4;
#pragma unroll
        for (int c = 0; c < CT; ++c) o.u[c] = Vec4<T>::load(U + c * 256);
    } else {
        const T* P = static_cast<const T*>(a.P) + unit * C * C + (size_t)mt * G::NKC * G::FE +
                     lane * G::NV;
#pragma unroll
        for (int s = 0; s < G::NKC; ++s) o.p[s] = F::load(P + s * G::FE);
    }
    if constexpr (WideGeom<T, C, DK, CT>::template has_t<ROLE_D>()) {
        const T* K = static_cast<const T*>(a.Kt) + unit * DK * C + (size_t)t * G::NKC * G::FE +
                     lane * G::NV;
#pragma unroll
        for (int s = 0; s < G::NKC; ++s) o.kt[s] = F::load(K + s * G::FE);
        o.gc = *reinterpret_cast<const f32x4*>(a.GC + unit * DK + 16 * t + 4 * lg);
    }
}

// workgroup barrier for the S / Delta exchange: waits for this wave's LDS
// accesses only (global loads in flight stay in flight)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// what both roles of a workgroup share
struct WideCtx {
    int bh, h, NC, T_, nc_seq, c0;
    size_t u0, row0;
    int mt, t, ucol, col, lane, lg;
};

// the chunk loop of one role (D waves: ROLE_D; O waves: !ROLE_D).  Both roles
// pass the same barriers in the same order.  Every chunk step issues the same
// loads and stores whatever the data (operands past the last chunk re-read the
// last one; only the last chunk's output store is masked), so the compiler's
// wait counts are exact and chunk n + NSETS - 1 stays in flight during chunk n.
// CS: also write the state entering every chunk.
// STREAM: the operands are written by the prep kernel running at the same
// time; before the loads of a chunk, wave NM (the first O wave) has seen its
// ready word (polled during the previous step, answered through barrier B2 in
// *status).  Returns false when the workgroup gave up (nothing more is
// written; the call's fallback chain redoes the work).
template <typename T, int C, int DK, int CT, int NSETS, bool ROLE_D, bool CS, bool STREAM>
__device__ __forceinline__ bool wide_role(const ChainArgs& a, const WideCtx& x, f32x4 (&S)[CT],
                                          typename WideGeom<T, C, DK, CT>::F* Sf,
                                          typename WideGeom<T, C, DK, CT>::F* Df, int* status)
{
    using G = WideGeom<T, C, DK, CT>;
    using F = typename G::F;
    using Ops = WideOps<T, C, DK, CT, ROLE_D>;
    constexpr bool has_t = G::template has_t<ROLE_D>();
    const int NC = x.NC, lane = x.lane, lg = x.lg, mt = x.mt, t = x.t;
    const int Dv = a.Dv;

    const bool poller = STREAM && !ROLE_D && mt == 0;     // wave NM
    if constexpr (STREAM) {
        if (poller) {
            // the units of the first NSETS steps' loads: NSETS - 1 here, one
            // more in step 0 (step n waits for the unit step n + 1 loads)
            bool ok = true;
            for (int j = 0; j < NSETS && ok; ++j) {
                const size_t u = x.u0 + min(j, NC - 1);
                ok = stream_wait_ready(a.ready, a.sctl, u, __hip_atomic_load(&a.ready[u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
            }
            *status = ok ? 0 : 1;                     // (every lane, the same word)
        }
        lds_barrier();
        if (__builtin_amdgcn_readfirstlane(*status)) return false;
    }
    Ops ops[NSETS];
#pragma unroll
    for (int j = 0; j + 1 < NSETS; ++j)
        load_ops<T, C, DK, CT, ROLE_D>(ops[j], a, x.u0 + min(j, NC - 1), mt, t, x.ucol, lane, lg);
    lds_barrier();                                    // the initial state is in Sf

    T* out = static_cast<T*>(a.out);
    const size_t ostride = (size_t)a.H * Dv;          // one token
    T* obase = out + ((x.row0 + (size_t)x.c0 * C + 16 * mt + 4 * lg) * a.H + x.h) * Dv + x.col;
    f32x4 oacc[CT];                                   // O wave: O(n) accumulating
    F pdf[ROLE_D ? 1 : CT][G::NKC];                   // O wave: Delta(n) fragments kept for O(n)

    // O wave: O(n) += P Delta(n), then the store; FULL: every row of the chunk
    // lies inside the sequence (all chunks but the last), else rows past the
    // sequence end are skipped
    auto finish_o = [&](const Ops& on, int n, auto full) {
        if constexpr (!ROLE_D) {
#pragma unroll
            for (int c = 0; c < CT; ++c) {
#pragma unroll
                for (int s = 0; s < G::NKC; ++s) oacc[c] = mma(on.p[s], pdf[c][s], oacc[c]);
            }
            T* o = obase + (size_t)n * C * ostride;
            const int r0 = n * C + 16 * mt + 4 * lg;
#pragma unroll
            for (int c = 0; c < CT; ++c) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (decltype(full)::value || r0 + i < x.T_) o[i * ostride + 16 * c] = from_f32<T>(oacc[c][i]);
            }
        }
    };

    auto step = [&](Ops& cur, Ops& prv, int n) -> bool {
        // (streamed) the ready word of the unit the next step loads
        const size_t unext = x.u0 + min(n + NSETS, NC - 1);
        unsigned rnext = 1u;
        if constexpr (STREAM) {
            if (poller) rnext = __hip_atomic_load(&a.ready[unext], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if constexpr (CS && has_t) {
            // the state entering chunk n (this wave's tiles, rounded to T)
            T* cs = static_cast<T*>(a.CS) + ((size_t)x.bh * x.nc_seq + x.c0 + n) * DK * Dv + x.col;
#pragma unroll
            for (int c = 0; c < CT; ++c)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    cs[(size_t)(16 * t + 4 * lg + i) * Dv + 16 * c] = from_f32<T>(S[c][i]);
        }
        if constexpr (!ROLE_D) {
            if (n > 0) finish_o(prv, n - 1, std::true_type{});
        }
        load_ops<T, C, DK, CT, ROLE_D>(prv, a, x.u0 + min(n + NSETS - 1, NC - 1), mt, t, x.ucol, lane, lg);
        {
            F sf[CT][G::NKD];
#pragma unroll
            for (int c = 0; c < CT; ++c)
#pragma unroll
                for (int s = 0; s < G::NKD; ++s) sf[c][s] = Sf[(c * G::NKD + s) * 64 + lane];
            if constexpr (ROLE_D) {
                // Delta(n) = U - W S(n), this wave's token tile, every column tile
#pragma unroll
                for (int c = 0; c < CT; ++c) {
                    f32x4 acc = zero4();
#pragma unroll
                    for (int s = 0; s < G::NKD; ++s) acc = mma(cur.a[s], sf[c][s], acc);
                    f32x4 dl;
#pragma unroll
                    for (int i = 0; i < 4; ++i) dl[i] = cur.u[c].get(i) - acc[i];
                    put_tile<T, G::KB>(Df + c * G::NKC * 64, mt, lane, dl);
                }
            } else {
                // (Q * Gamma) S(n), this wave's token tile
#pragma unroll
                for (int c = 0; c < CT; ++c) {
                    oacc[c] = zero4();
#pragma unroll
                    for (int s = 0; s < G::NKD; ++s) oacc[c] = mma(cur.a[s], sf[c][s], oacc[c]);
                }
            }
        }
        lds_barrier();                                // B1: Delta(n) visible
        F df[CT][G::NKC];
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
            for (int s = 0; s < G::NKC; ++s) df[c][s] = Df[(c * G::NKC + s) * 64 + lane];
        if constexpr (has_t) {
            // S(n+1) = diag(Gamma_{C-1}) S(n) + Ktil^T Delta(n), this wave's row tile
#pragma unroll
            for (int c = 0; c < CT; ++c) {
                f32x4 acc;
                if (a.ph) {
                    // phase variant: rows 2p, 2p+1 turn by Gamma's 2x2 block
                    // (g0 = |G| cos, g1 = |G| sin)
#pragma unroll
                    for (int i = 0; i < 4; i += 2) {
                        const float g0 = cur.gc[i], g1 = cur.gc[i + 1];
                        acc[i] = g0 * S[c][i] - g1 * S[c][i + 1];
                        acc[i + 1] = g1 * S[c][i] + g0 * S[c][i + 1];
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[i] = cur.gc[i] * S[c][i];
                }
#pragma unroll
                for (int s = 0; s < G::NKC; ++s) acc = mma(cur.kt[s], df[c][s], acc);
                S[c] = acc;
                put_tile<T, G::KB>(Sf + c * G::NKD * 64, t, lane, acc);
            }
        }
        if constexpr (!ROLE_D) {
#pragma unroll
            for (int c = 0; c < CT; ++c)
#pragma unroll
                for (int s = 0; s < G::NKC; ++s) pdf[c][s] = df[c][s];
        }
        if constexpr (STREAM) {
            if (poller) {
                const bool ok = stream_wait_ready(a.ready, a.sctl, unext, rnext);
                *status = ok ? 0 : 1;
            }
        }
        lds_barrier();                                // B2: S(n+1) visible
        if constexpr (STREAM) {
            if (__builtin_amdgcn_readfirstlane(*status)) {
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                return false;
            }
        }
        return true;
    };

    // the loop unrolled by NSETS (every register set keeps fixed registers);
    // the only way out is after a whole step, so every path into the next
    // step has issued the same memory operations
    int n = 0;
    for (;;) {
        if (!step(ops[0], ops[NSETS - 1], n)) return false;
        if (++n >= NC) { finish_o(ops[0], n - 1, std::false_type{}); break; }
        if (!step(ops[1], ops[0], n)) return false;
        if (++n >= NC) { finish_o(ops[1], n - 1, std::false_type{}); break; }
        if constexpr (NSETS == 3) {
            if (!step(ops[2], ops[1], n)) return false;
            if (++n >= NC) { finish_o(ops[2], n - 1, std::false_type{}); break; }
        }
    }
    return true;
}

template <typename T, int C, int DK, int CT, int NSETS, bool STREAM>
__global__ __launch_bounds__(kWideThreads) void chain_wide_kernel(ChainArgs a)
{
    using G = WideGeom<T, C, DK, CT>;
    using F = typename G::F;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    F* Sf = reinterpret_cast<F*>(lds + G::SF);     // [CT][NKD][64]
    F* Df = reinterpret_cast<F*>(lds + G::DF);     // [CT][NKC][64]
    __shared__ int sStatus;

    // the fallback launch of a streamed call runs only when the streamed chain
    // gave up or left a (b, h) out
    if (a.gate && !(a.gate->abort || a.gate->chains_done < a.gate->expect)) return;
    const int Dv = a.Dv, H = a.H;
    const int NSL = Dv / (16 * CT);                 // column slices per (b, h)
    int bh, slice;
    if constexpr (STREAM) {
        // a (b, h, column slice) of the heads on this workgroup's own XCD
        // (b H + h = xcd + 8 j), so the units it reads were written there
        if (threadIdx.x == 0) {
            const int xcd = (int)xcc_id();
            const int k = (int)atomicAdd(&a.sctl->chain_next[xcd], 1u);
            const int bhx = xcd + kXcds * (k / NSL);
            sStatus = bhx < a.B * H ? bhx * NSL + k % NSL : -1;
        }
        __syncthreads();
        const int role = __builtin_amdgcn_readfirstlane(sStatus);
        __syncthreads();
        if (role < 0) return;
        bh = role / NSL;
        slice = role % NSL;
    } else {
        const int g = blockIdx.x, xcd = g % kXcds, jx = g / kXcds;
        bh = (jx / NSL) * kXcds + xcd;
        slice = jx % NSL;
        if (bh >= a.B * H) return;
    }
    const SeqPos sp = locate_seq(bh, H, a.T, a.NC, a.cu, a.cs);
    WideCtx x;
    x.bh = bh;
    x.h = bh % H;
    x.c0 = a.pcn > 0 ? a.pc0 : 0;
    x.NC = a.pcn > 0 ? min(a.pcn, sp.nc - x.c0) : sp.nc;
    x.T_ = sp.len - x.c0 * C;                       // tokens from the first chunk of the range
    x.nc_seq = sp.nc;
    x.u0 = sp.ubase + x.c0;
    x.row0 = (size_t)sp.row0;
    const int tid = threadIdx.x;
    x.lane = tid & 63;
    x.lg = x.lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool dwave = wave < G::NM;
    x.mt = dwave ? wave : wave - G::NM;             // token tile of a D or O wave
    const bool has_t = wave < G::NT;                // owns state row tile t = wave
    x.t = wave;
    x.ucol = slice * CT;                            // first column tile of the slice
    x.col = 16 * x.ucol + (x.lane & 15);            // this lane's column in tile 0
    const int t = x.t, lg = x.lg, col = x.col;

    const float* sinit = a.S0 ? a.S0 + (size_t)bh * DK * Dv : nullptr;
    f32x4 S[CT];
    if (has_t) {
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                S[c][i] = sinit ? sinit[(size_t)(16 * t + 4 * lg + i) * Dv + col + 16 * c] : 0.f;
    }
    if (x.NC > 0) {
        if (has_t) {
#pragma unroll
            for (int c = 0; c < CT; ++c) put_tile<T, G::KB>(Sf + c * G::NKD * 64, t, x.lane, S[c]);
        }
        bool done;
        if constexpr (STREAM) {
            done = dwave ? wide_role<T, C, DK, CT, NSETS, true, false, true>(a, x, S, Sf, Df, &sStatus)
                         : wide_role<T, C, DK, CT, NSETS, false, false, true>(a, x, S, Sf, Df, &sStatus);
        } else if (a.CS) {
            done = dwave ? wide_role<T, C, DK, CT, NSETS, true, true, false>(a, x, S, Sf, Df, &sStatus)
                         : wide_role<T, C, DK, CT, NSETS, false, true, false>(a, x, S, Sf, Df, &sStatus);
        } else {
            done = dwave ? wide_role<T, C, DK, CT, NSETS, true, false, false>(a, x, S, Sf, Df, &sStatus)
                         : wide_role<T, C, DK, CT, NSETS, false, false, false>(a, x, S, Sf, Df, &sStatus);
        }
        if (!done) return;                          // (streamed: gave up)
    }
    // (an empty sequence of a packed batch passes its state through)
    if (a.ST && has_t) {
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a.ST[((size_t)bh * DK + 16 * t + 4 * lg + i) * Dv + col + 16 * c] = S[c][i];
    }
    if constexpr (STREAM) {
        if (threadIdx.x == 0) atomicAdd(&a.sctl->chains_done, 1u);
    }
}

template <typename T, int C, int DK, int CT, int NSETS, bool STREAM = false>
hipError_t launch_wide_t(const ChunkShape& s, const ChainArgs& a, hipStream_t stream)
{
    using G = WideGeom<T, C, DK, CT>;
    auto kern = chain_wide_kernel<T, C, DK, CT, NSETS, STREAM>;
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)G::LDS);
    if (e != hipSuccess) return e;
    const int NSL = s.Dv / (16 * CT);
    const int bh = s.B * s.H;
    const unsigned grid = (unsigned)(kXcds * NSL * ((bh + kXcds - 1) / kXcds));
    return launch_kernel(kern, dim3(grid), dim3(kWideThreads), (uint32_t)G::LDS, stream, a);
}

}  // namespace

// Column tiles per workgroup of the wide chain for this shape, or 0 when the
// 16-column chain of chain.hip should run instead.  Covered: chunk 64, Dk 128
// or 64, one column tile (16 columns) per workgroup.  Always used for fp32
// with Dk = 128 (whose operands do not fit the 16-column kernel's LDS
// staging), otherwise chosen only when the
// (b, h, 16-column) chains number at most 64: there it measured faster
// (B=1, H=2, T=65536, d=128, bf16: 0.75 ms against 0.96 ms; 0.72 against
// 0.92 us per chunk step at H=8), while with 128 or 256 chains both kernels
// are bound by fetching the chunk operands (1.16 against 1.13-1.26 us per
// step at H=32, T=8192; 1.56 against 1.43 ms in the parts path at H=16,
// T=65536) and the LDS-staged kernel keeps its deeper prefetch.  Two column
// tiles per workgroup (half the workgroups fetching the operands) measured
// slower still (1.38 us per step at H=32).
int wide_chain_tiles(IoType io, const ChunkShape& s)
{
    if (s.C != 64 || (s.Dk != 128 && s.Dk != 64)) return 0;
    if (io == IoType::F32 && s.Dk == 128) return 1;      // the only chain for this form
    if ((long long)s.B * s.H * (s.Dv / 16) > 64) return 0;
    return 1;
}

hipError_t launch_chain_wide(IoType io, const ChunkShape& s, const ChainArgs& a, int ct,
                             hipStream_t stream)
{
    (void)ct;
    if (io == IoType::BF16) {
        if (s.Dk == 128) return launch_wide_t<bf16_t, 64, 128, 1, 3>(s, a, stream);
        return launch_wide_t<bf16_t, 64, 64, 1, 3>(s, a, stream);
    }
    if (s.Dk == 128) return launch_wide_t<float, 64, 128, 1, 2>(s, a, stream);
    return launch_wide_t<float, 64, 64, 1, 3>(s, a, stream);
}

// The chain of the streamed forward: ct column tiles per workgroup, waiting on
// the ready words of the prep kernel that runs beside it.
hipError_t launch_chain_stream(IoType io, const ChunkShape& s, const ChainArgs& a, int ct,
                               hipStream_t stream)
{
    if (io != IoType::BF16 || s.C != 64) return hipErrorInvalidValue;
    if (s.Dk == 128) {
        if (ct == 4) return launch_wide_t<bf16_t, 64, 128, 4, 2, true>(s, a, stream);
        if (ct == 2) return launch_wide_t<bf16_t, 64, 128, 2, 3, true>(s, a, stream);
        return launch_wide_t<bf16_t, 64, 128, 1, 3, true>(s, a, stream);
    }
    if (s.Dk == 64) {
        if (ct == 2) return launch_wide_t<bf16_t, 64, 64, 2, 3, true>(s, a, stream);
        return launch_wide_t<bf16_t, 64, 64, 1, 3, true>(s, a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace kda
