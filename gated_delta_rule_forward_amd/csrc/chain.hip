// chain.hip — the sequential part of the chunkwise forward: the state carried
// from chunk to chunk ("Kimi Delta Attention: a bounded case study", Exercise
// 2; "Semidirect Fourier Delta Attention", contribution 4: the chunk's affine
// write summary) plus each chunk's outputs (eq. (14)):
//   Delta  = U - W S                      (the deltas the chunk's tokens write)
//   O      = (Q * Gamma) S + P Delta
//   S_next = diag(Gamma_{C-1}) S + Ktil^T Delta
// Columns of S evolve independently (the transition acts on rows, the write
// beta k v^T is separable by column: §2.2 eq. (9)), so one workgroup owns 16
// columns of one (b, h) and needs no communication with any other.
//
// Workgroup = 4 wavefronts.  Wave w computes token tile w of Delta and O and
// state row tiles w, w+4, ...; the state and Delta are exchanged through LDS
// already in MFMA B-fragment form (one 8- or 16-byte slot per lane).  Two
// barriers per chunk.  The fp32 state slice stays in registers for the whole
// sequence.
//
// Operands reach the wavefronts through a two-stage LDS FIFO per wavefront,
// filled with direct global-to-LDS loads (no registers held while in flight):
// the prep kernels store every operand fragment-major, so one wavefront's
// fragment of one MFMA is one contiguous block that a single 16-byte-per-lane
// load copies verbatim.  At the start of chunk c the wave waits for chunk c's
// stage, moves its fragments into registers and refills the same stage with
// chunk c+2, so chunk c+1's loads are in flight for a whole step and chunk
// c+2's for most of one.  The loads are not visible to the compiler's wait
// counting, so the waits are explicit: every step issues exactly NDMA loads,
// hence "at most NDMA outstanding" means the older stage has landed.
//
// Workgroups are numbered so that the column slices of one (b, h) land on the
// same XCD (consecutive workgroup ids go to consecutive XCDs) and share that
// XCD's L2 for the chunk operands.
#include "kda_chunk.hpp"
#include "kda_dma.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace {

constexpr int kChainWaves = 4;                        // compute wavefronts
constexpr int kChainThreads = 64 * 2 * kChainWaves;   // + one loader wavefront each
constexpr int kXcds = 8;

template <typename T, int C, int DK>
struct ChainGeom {
    static constexpr int KB = KBlock<T, C, DK>::value;
    static constexpr int NT = DK / 16;           // state row tiles
    static constexpr int NM = C / 16;            // token tiles
    static constexpr int NKD = DK / KB;          // k blocks over channels
    static constexpr int NKC = C / KB;           // k blocks over tokens
    static constexpr int SPW = (NT + 3) / 4;     // state tiles per wave
    static constexpr int TPB = KB / 16;          // tiles per k block
    static constexpr int FB = 64 * (KB / 4) * (int)sizeof(T);   // bytes of one 64-lane fragment
    // one wavefront's share of a chunk's operands in an LDS stage (byte offsets)
    static constexpr int OW = 0;                      // W, its token tile      [NKD]
    static constexpr int OQ = OW + NKD * FB;          // Q * Gamma              [NKD]
    static constexpr int OP = OQ + NKD * FB;          // P                      [NKC]
    static constexpr int OU = OP + NKC * FB;          // U tile (64 x 16 B)
    static constexpr int UB = 64 * 4 * (int)sizeof(T);     // bytes of one U tile
    static constexpr int OK = OU + 1024;              // Ktil, its state tiles  [SPW][NKC]
    static constexpr int OG = OK + SPW * NKC * FB;    // Gamma_C rows of its state tiles [SPW][4][16 B]
    static constexpr int STAGE = OG + SPW * 64;
    static constexpr int runs(int bytes) { return (bytes + 1023) / 1024; }
    // 16-byte-per-lane direct-to-LDS loads one wavefront issues per chunk
    static constexpr int NDMA = 2 * runs(NKD * FB) + runs(NKC * FB) + runs(UB) + SPW * runs(NKC * FB) + 1;
    static constexpr size_t LDS = 2 * 4 * (size_t)STAGE;     // two stages, four waves
    // plus the S and Delta exchange fragments and a 1 KB sink for L2 prefetches
    static constexpr size_t XCH = LDS;
    static constexpr size_t SINK = XCH + (size_t)(NKD + NKC) * 64 * (KB / 4) * sizeof(T);
    static constexpr size_t LDS_TOTAL = SINK + 1024;
    // L2 prefetch: 1 KB pieces of a chunk's blocks shared by the column slices
    // (W, Q * Gamma, Ktil, P; only when whole kilobytes), plus each slice's U
    // tiles; KPF prefetch loads per loader wavefront and step (one: with the
    // rotated run order of the operand loads, two or three were slower)
    static constexpr int PW = C * DK * (int)sizeof(T) / 1024, PP = C * C * (int)sizeof(T) / 1024;
    static constexpr bool PREFETCH =
        (C * DK * (int)sizeof(T)) % 1024 == 0 && (C * C * (int)sizeof(T)) % 1024 == 0;
    static constexpr int PTOT = 3 * PW + PP;
    static constexpr int KPF = PREFETCH ? 1 : 0;
    static_assert(NDMA <= 63, "vmcnt holds at most 63 outstanding loads");
    // P (token tile mt's rows) is zero in the k blocks past its diagonal
    // block: with one 1 KB run per k block those runs are not loaded, and the
    // fragments are set to zero instead (the same MFMA products)
    static constexpr bool PSKIP = FB == 1024;
    __device__ static constexpr int nkp(int mt) {
        return PSKIP ? ((16 * (mt + 1) + KB - 1) / KB < NKC ? (16 * (mt + 1) + KB - 1) / KB : NKC) : NKC;
    }
};


// enqueue one chunk's operands for this wavefront into its stage region, in
// three parts spread over a step (PART 0: W, Q*Gamma; 1: P, U; 2: Ktil,
// Gamma_C) so the load pipe drains while the wave computes.  Waves without a
// token tile or state tile load the last one instead, so every wavefront
// issues exactly NDMA loads per chunk.
template <typename T, int C, int DK, int PART>
__device__ __forceinline__ void issue_chunk(unsigned char* st, const ChainArgs& a, size_t unit,
                                            int wave, int lane, int slice)
{
    using G = ChainGeom<T, C, DK>;
    const int mt = wave < G::NM ? wave : G::NM - 1;
    const int Dv = a.Dv;
    if constexpr (PART == 0) {
        const size_t off = (unit * C * DK + (size_t)mt * G::NKD * 64 * (G::KB / 4)) * sizeof(T);
        if constexpr ((G::NKD * G::FB) % 1024 == 0) {
            const unsigned char* const s2[2] = {static_cast<const unsigned char*>(a.W) + off,
                                                static_cast<const unsigned char*>(a.QG) + off};
            unsigned char* const d2[2] = {st + G::OW, st + G::OQ};
            dma_runs_rot<2, G::NKD * G::FB>(s2, d2, lane, slice);
        } else {
            dma_run<G::NKD * G::FB>(static_cast<const unsigned char*>(a.W) + off, st + G::OW, lane);
            dma_run<G::NKD * G::FB>(static_cast<const unsigned char*>(a.QG) + off, st + G::OQ, lane);
        }
    } else if constexpr (PART == 1) {
        const unsigned char* P = static_cast<const unsigned char*>(a.P) +
                                 (unit * C * C + (size_t)mt * G::NKC * 64 * (G::KB / 4)) * sizeof(T);
        const unsigned char* U = reinterpret_cast<const unsigned char*>(
            static_cast<const T*>(a.U) + unit * C * Dv + (size_t)(mt * (Dv / 16) + slice) * 64 * 4);
        if constexpr (G::PSKIP) {
            // the k blocks up to the diagonal block, from another run per slice
            const int np = G::nkp(mt), r0 = slice % np;
#pragma unroll
            for (int i = 0; i < G::NKC; ++i) {
                if (i < np) {
                    int j = i + r0;
                    if (j >= np) j -= np;
                    dma16(P + j * 1024 + 16 * lane, st + G::OP + j * 1024);
                }
            }
        } else if constexpr ((G::NKC * G::FB) % 1024 == 0) {
            const unsigned char* const s1[1] = {P};
            unsigned char* const d1[1] = {st + G::OP};
            dma_runs_rot<1, G::NKC * G::FB>(s1, d1, lane, slice);
        } else {
            dma_run<G::NKC * G::FB>(P, st + G::OP, lane);
        }
        dma_run<G::UB>(U, st + G::OU, lane);
    } else {
        const unsigned char* ks[G::SPW];
        unsigned char* kd[G::SPW];
#pragma unroll
        for (int u = 0; u < G::SPW; ++u) {
            const int t = (wave + 4 * u) < G::NT ? wave + 4 * u : G::NT - 1;
            ks[u] = static_cast<const unsigned char*>(a.Kt) +
                    (unit * DK * C + (size_t)t * G::NKC * 64 * (G::KB / 4)) * sizeof(T);
            kd[u] = st + G::OK + u * G::NKC * G::FB;
        }
        if constexpr ((G::NKC * G::FB) % 1024 == 0) {
            dma_runs_rot<G::SPW, G::NKC * G::FB>(ks, kd, lane, slice);
        } else {
#pragma unroll
            for (int u = 0; u < G::SPW; ++u) dma_run<G::NKC * G::FB>(ks[u], kd[u], lane);
        }
        // Gamma_C: lane j < 4 SPW fetches rows 16t + 4(j % 4) .. +3 of state tile
        // u = j / 4; they land at OG + 16 j
        if (lane < 4 * G::SPW) {
            const int u = lane >> 2;
            const int t = (wave + 4 * u) < G::NT ? wave + 4 * u : G::NT - 1;
            dma16(a.GC + unit * DK + 16 * t + 4 * (lane & 3), st + G::OG);
        }
    }
}

template <typename T, int C, int DK>
__device__ __forceinline__ void issue_all(unsigned char* st, const ChainArgs& a, size_t unit,
                                          int wave, int lane, int slice)
{
    issue_chunk<T, C, DK, 0>(st, a, unit, wave, lane, slice);
    issue_chunk<T, C, DK, 1>(st, a, unit, wave, lane, slice);
    issue_chunk<T, C, DK, 2>(st, a, unit, wave, lane, slice);
}

// KPF L2 prefetch loads of one chunk by loader `cw` of column slice `slice`
// (of NS): the slice's pieces are every NS-th kilobyte of the shared blocks and
// its own U tiles; the four loaders of a workgroup take every fourth piece.
// The data lands in an LDS sink; the point is the L2 fill.  The column slices
// of one (b, h) run on one XCD, so together they prefetch the whole chunk.
template <typename T, int C, int DK>
__device__ __forceinline__ void prefetch_chunk(const ChainArgs& a, size_t unit, int slice, int NS,
                                               int cw, int lane, unsigned char* sink)
{
    using G = ChainGeom<T, C, DK>;
    const int ps = (G::PTOT - slice + NS - 1) / NS;   // shared pieces of this slice
    const int npw = ps + G::NM;
    const size_t blk = (size_t)C * DK * sizeof(T);
#pragma unroll
    for (int i = 0; i < G::KPF; ++i) {
        const int k = min(cw + kChainWaves * i, npw - 1);
        const unsigned char* src;
        if (k < ps) {
            const int p = slice + NS * k;
            if (p < G::PW) src = static_cast<const unsigned char*>(a.W) + unit * blk + (size_t)p * 1024;
            else if (p < 2 * G::PW)
                src = static_cast<const unsigned char*>(a.QG) + unit * blk + (size_t)(p - G::PW) * 1024;
            else if (p < 3 * G::PW)
                src = static_cast<const unsigned char*>(a.Kt) + unit * blk + (size_t)(p - 2 * G::PW) * 1024;
            else
                src = static_cast<const unsigned char*>(a.P) + unit * C * C * sizeof(T) +
                      (size_t)(p - 3 * G::PW) * 1024;
        } else {
            src = reinterpret_cast<const unsigned char*>(
                static_cast<const T*>(a.U) + unit * C * a.Dv + (size_t)((k - ps) * NS + slice) * 64 * 4);
        }
        // (a U tile may be 512 bytes: lanes past it re-read its start)
        dma16(src + 16 * (k < ps ? lane : lane % (G::UB / 16)), sink);
    }
}

// one chunk's operands of one wavefront, in registers
template <typename T, int C, int DK>
struct ChainOps {
    using G = ChainGeom<T, C, DK>;
    using F = Frag<T, G::KB>;
    F w[G::NKD], qg[G::NKD], p[G::NKC], kt[G::SPW][G::NKC];
    f32x4 u, gc[G::SPW];
};

template <typename T, int C, int DK>
__device__ __forceinline__ void read_ops(ChainOps<T, C, DK>& o, const unsigned char* st, int lane, int lg, int np)
{
    using G = ChainGeom<T, C, DK>;
    using F = Frag<T, G::KB>;
#pragma unroll
    for (int s = 0; s < G::NKD; ++s) {
        o.w[s] = *reinterpret_cast<const F*>(st + G::OW + s * G::FB + lane * sizeof(F));
        o.qg[s] = *reinterpret_cast<const F*>(st + G::OQ + s * G::FB + lane * sizeof(F));
    }
#pragma unroll
    for (int s = 0; s < G::NKC; ++s)
    {
        const float zf[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        o.p[s] = s < np ? *reinterpret_cast<const F*>(st + G::OP + s * G::FB + lane * sizeof(F)) : F::from(zf);
    }
    {
        const Vec4<T> u4 = *reinterpret_cast<const Vec4<T>*>(st + G::OU + lane * 4 * sizeof(T));
        o.u = f32x4{u4.get(0), u4.get(1), u4.get(2), u4.get(3)};
    }
#pragma unroll
    for (int u = 0; u < G::SPW; ++u) {
#pragma unroll
        for (int s = 0; s < G::NKC; ++s)
            o.kt[u][s] = *reinterpret_cast<const F*>(st + G::OK + (u * G::NKC + s) * G::FB + lane * sizeof(F));
        o.gc[u] = *reinterpret_cast<const f32x4*>(st + G::OG + (u * 4 + lg) * 16);
    }
}

template <typename T, int C, int DK>
__global__ __launch_bounds__(kChainThreads) void chain_kernel(ChainArgs a)
{
    using G = ChainGeom<T, C, DK>;
    using F = Frag<T, G::KB>;
    extern __shared__ __attribute__((aligned(16))) unsigned char stages[];
    F* sSf = reinterpret_cast<F*>(stages + G::XCH);
    F* sDf = sSf + G::NKD * 64;

    // the fallback launch of a streamed call runs only when the streamed chain
    // gave up or left a (b, h) out
    if (a.gate && !(a.gate->abort || a.gate->chains_done < a.gate->expect)) return;
    const int Dv = a.Dv, H = a.H;
    const int NS = Dv / 16;
    const bool summary = a.summ != nullptr;
    const int nseg = a.nseg > 1 ? a.nseg : 1;
    const int NSX = summary ? DK / 16 + NS : NS;           // column slices per chain
    const int g = blockIdx.x, xcd = g % kXcds, jx = g / kXcds;
    const int vb = (jx / NSX) * kXcds + xcd, xslice = jx % NSX;
    if (vb >= a.B * H * nseg) return;
    const int bh = vb / nseg, sg = vb % nseg;
    if (summary && sg == nseg - 1) return;        // the last segment's map is never used
    const int h = bh % H;
    // summary pass: slices below DK / 16 carry the homogeneous part (columns of
    // the identity, U taken as zero), the others the particular part
    const bool xpart = summary && xslice < DK / 16;
    const int slice = summary ? (xpart ? 0 : xslice - DK / 16) : xslice;   // U / column slice
    // this (sequence, head): chunk count, first token row, length, first unit;
    // a segment is chunks [c0, c0 + NC) of it
    const SeqPos sp = locate_seq(bh, H, a.T, a.NC, a.cu, a.cs);
    const int c0 = nseg > 1 ? sg * a.seg : (a.pcn > 0 ? a.pc0 : 0);
    const int NC = nseg > 1 ? min(a.seg, sp.nc - c0) : (a.pcn > 0 ? min(a.pcn, sp.nc - c0) : sp.nc);
    const int T_ = sp.len - c0 * C;
    const int tid = threadIdx.x, lane = tid & 63, ln = lane & 15, lg = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = slice * 16 + ln;

    // Operand FIFO.  Chunk c is loaded into stage c & 1 by the loader
    // wavefronts (wave 4 + w fills compute wave w's region) during step c - 2
    // (part 0 before its barrier 1, the rest after it) and moved into
    // registers by the compute wavefronts at the end of step c - 1, between
    // the step's two barriers: the loader waits for chunk c before barrier 1
    // of step c - 1, and stage c & 1 is free again after barrier 2 of step
    // c - 1.  Past the last chunk the last one is re-read, so every step
    // issues the same NDMA loads per loader.
    const size_t u0 = sp.ubase + c0;
    const int last = NC - 1;
    if (NC == 0) {
        // an empty sequence of a packed batch: the state passes through
        if (a.ST && wave < kChainWaves) {
#pragma unroll
            for (int u = 0; u < G::SPW; ++u) {
                const int t = wave + 4 * u;
                if (t < G::NT) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const size_t e = ((size_t)bh * DK + 16 * t + 4 * lg + i) * Dv + col;
                        a.ST[e] = a.S0 ? a.S0[e] : 0.f;
                    }
                }
            }
        }
        return;
    }
    const int cw = wave & (kChainWaves - 1);     // the compute wave a loader serves
    auto stg = [&](int c) { return stages + (size_t)((c & 1) * kChainWaves + cw) * G::STAGE; };
    if (wave >= kChainWaves) {
        // chunk c is also prefetched into L2 at step c - 5 (KPF loads per
        // loader and step)
        unsigned char* sink = stages + G::SINK;
        issue_all<T, C, DK>(stg(0), a, u0, cw, lane, slice);
        prefetch_chunk<T, C, DK>(a, u0 + min(2, last), slice, NS, cw, lane, sink);
        prefetch_chunk<T, C, DK>(a, u0 + min(3, last), slice, NS, cw, lane, sink);
        issue_all<T, C, DK>(stg(1), a, u0 + min(1, last), cw, lane, slice);
        prefetch_chunk<T, C, DK>(a, u0 + min(4, last), slice, NS, cw, lane, sink);
        // chunk 0 landed: its loads are followed by chunk 1's and three prefetches
        switch (G::NKC - G::nkp(cw < G::NM ? cw : G::NM - 1)) {
        case 0: wait_vm<G::NDMA + 3 * G::KPF>(); break;
        case 1: wait_vm<G::NDMA - 1 + 3 * G::KPF>(); break;
        case 2: wait_vm<G::NDMA - 2 + 3 * G::KPF>(); break;
        default: wait_vm<G::NDMA - 3 + 3 * G::KPF>(); break;
        }
        lds_barrier();                               // B0: compute reads chunk 0
        lds_barrier();                               // B1: stage 0 free
        constexpr int N0 = 2 * G::runs(G::NKD * G::FB);   // loads of part 0
        for (int nc = 0; nc < NC; ++nc) {
            // part 0 of chunk nc + 2 before barrier 1 and the rest after it:
            // issuing blocks while the load pipe is full, so the compute
            // wavefronts must not wait at barrier 1 for all of it.  Loads
            // issued after chunk nc + 1: the previous step's prefetch and part 0.
            issue_chunk<T, C, DK, 0>(stg(nc), a, u0 + min(nc + 2, last), cw, lane, slice);
            wait_vm<N0 + G::KPF>();                  // chunk nc + 1 landed
            lds_barrier();
            issue_chunk<T, C, DK, 1>(stg(nc), a, u0 + min(nc + 2, last), cw, lane, slice);
            issue_chunk<T, C, DK, 2>(stg(nc), a, u0 + min(nc + 2, last), cw, lane, slice);
            prefetch_chunk<T, C, DK>(a, u0 + min(nc + 5, last), slice, NS, cw, lane, sink);
            lds_barrier();
        }
        wait_vm<0>();   // no load may land in LDS after the workgroup ends
        return;
    }

    f32x4 S[G::SPW];
    // initial state: S0 (or the segment's start state), the identity columns of
    // a homogeneous summary slice, or zero
    const float* sinit = summary ? nullptr
                       : (sg > 0 ? a.Sseg + (size_t)(bh * nseg + sg) * DK * Dv : (a.S0 ? a.S0 + (size_t)bh * DK * Dv : nullptr));
#pragma unroll
    for (int u = 0; u < G::SPW; ++u) {
        const int t = wave + 4 * u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * t + 4 * lg + i;
            S[u][i] = xpart ? (row == 16 * xslice + ln ? 1.f : 0.f)
                            : ((sinit && t < G::NT) ? sinit[(size_t)row * Dv + col] : 0.f);
        }
        if (t < G::NT) put_tile<T, G::KB>(sSf, t, lane, S[u]);
    }

    ChainOps<T, C, DK> cur;
    const int npw = G::nkp(wave < G::NM ? wave : G::NM - 1);   // nonzero P k blocks
    lds_barrier();                                   // B0: chunk 0 is in stage 0
    read_ops<T, C, DK>(cur, stg(0), lane, lg, npw);
    lds_barrier();                                   // B1: stage 0 may be refilled

    T* out = static_cast<T*>(a.out);
    const size_t ostride = (size_t)H * Dv;                      // one token
    T* obase = out + (((size_t)sp.row0 + (size_t)c0 * C + 16 * wave + 4 * lg) * H + h) * Dv + col;
    // outputs of chunk n: O = (Q * Gamma) S_n + P Delta_n (off the state's
    // critical path, so computed during the next chunk's first phase)
    F pqg[G::NKD], pp[G::NKC], psf[G::NKD], pdf[G::NKC];
    auto emit = [&](int n) {
        if (a.out && (G::NM == 4 || wave < G::NM)) {
            f32x4 acc = zero4();
#pragma unroll
            for (int s = 0; s < G::NKD; ++s) acc = mma(pqg[s], psf[s], acc);
#pragma unroll
            for (int s = 0; s < G::NKC; ++s) acc = mma(pp[s], pdf[s], acc);
            T* o = obase + (size_t)n * C * ostride;
            if (n * C + C <= T_) {
#pragma unroll
                for (int i = 0; i < 4; ++i) o[i * ostride] = from_f32<T>(acc[i]);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (n * C + 16 * wave + 4 * lg + i < T_) o[i * ostride] = from_f32<T>(acc[i]);
            }
        }
    };

    for (int nc = 0; nc < NC; ++nc) {
        if (a.CS) {
            // the state entering chunk nc (this wave's tiles, rounded to T)
            T* cs = static_cast<T*>(a.CS) + ((size_t)bh * sp.nc + c0 + nc) * DK * Dv + col;
#pragma unroll
            for (int u = 0; u < G::SPW; ++u) {
                const int t = wave + 4 * u;
                if (t < G::NT) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) cs[(size_t)(16 * t + 4 * lg + i) * Dv] = from_f32<T>(S[u][i]);
                }
            }
        }
        if (a.CS32) {
            // the same state in fp32, by unit
            float* cs = a.CS32 + (u0 + nc) * DK * Dv + col;
#pragma unroll
            for (int u = 0; u < G::SPW; ++u) {
                const int t = wave + 4 * u;
                if (t < G::NT) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) cs[(size_t)(16 * t + 4 * lg + i) * Dv] = S[u][i];
                }
            }
        }
        F sf[G::NKD];
#pragma unroll
        for (int s = 0; s < G::NKD; ++s) sf[s] = sSf[s * 64 + lane];
        if (nc > 0) emit(nc - 1);

        // Delta = U - W S for this wave's token tile
        if (G::NM == 4 || wave < G::NM) {
            f32x4 acc = zero4();
#pragma unroll
            for (int s = 0; s < G::NKD; ++s) acc = mma(cur.w[s], sf[s], acc);
            f32x4 dl;
#pragma unroll
            for (int i = 0; i < 4; ++i) dl[i] = (xpart ? 0.f : cur.u[i]) - acc[i];
            put_tile<T, G::KB>(sDf, wave, lane, dl);
            if (a.DL) {
                float* d = a.DL + ((u0 + nc) * C + 16 * wave + 4 * lg) * Dv + col;
#pragma unroll
                for (int i = 0; i < 4; ++i) d[(size_t)i * Dv] = dl[i];
            }
        }
        lds_barrier();
        F df[G::NKC];
#pragma unroll
        for (int s = 0; s < G::NKC; ++s) df[s] = sDf[s * 64 + lane];
        // S_next = diag(Gamma_C) S + Ktil^T Delta for this wave's state tiles
#pragma unroll
        for (int u = 0; u < G::SPW; ++u) {
            const int t = wave + 4 * u;
            if (G::NT % 4 == 0 || t < G::NT) {
                f32x4 acc;
                if (a.ph) {
                    // phase variant: rows 2p, 2p+1 turn by Gamma's 2x2 block
                    // (g0 = |G| cos, g1 = |G| sin)
#pragma unroll
                    for (int i = 0; i < 4; i += 2) {
                        const float g0 = cur.gc[u][i], g1 = cur.gc[u][i + 1];
                        acc[i] = g0 * S[u][i] - g1 * S[u][i + 1];
                        acc[i + 1] = g1 * S[u][i] + g0 * S[u][i + 1];
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[i] = cur.gc[u][i] * S[u][i];
                }
#pragma unroll
                for (int s = 0; s < G::NKC; ++s) acc = mma(cur.kt[u][s], df[s], acc);
                S[u] = acc;
                put_tile<T, G::KB>(sSf, t, lane, acc);
            }
        }
#pragma unroll
        for (int s = 0; s < G::NKD; ++s) { pqg[s] = cur.qg[s]; psf[s] = sf[s]; }
#pragma unroll
        for (int s = 0; s < G::NKC; ++s) { pp[s] = cur.p[s]; pdf[s] = df[s]; }
        // next chunk's operands (its loader waited for them before barrier 1)
        read_ops<T, C, DK>(cur, stg(nc + 1), lane, lg, npw);
        lds_barrier();
    }
    emit(NC - 1);

    if (summary) {
        // this slice's columns of [X_g | Y_g]
        float* dst = a.summ + (size_t)(bh * nseg + sg) * DK * (DK + Dv) + 16 * xslice + ln;
#pragma unroll
        for (int u = 0; u < G::SPW; ++u) {
            const int t = wave + 4 * u;
            if (t < G::NT) {
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[(size_t)(16 * t + 4 * lg + i) * (DK + Dv)] = S[u][i];
            }
        }
    } else if (a.ST && sg == nseg - 1) {
#pragma unroll
        for (int u = 0; u < G::SPW; ++u) {
            const int t = wave + 4 * u;
            if (t < G::NT) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    a.ST[((size_t)bh * DK + 16 * t + 4 * lg + i) * Dv + col] = S[u][i];
            }
        }
    }
}

// Segment start states: S_0 = S0 (or zero), S_{g+1} = X_g S_g + Y_g in fp32
// ("Semidirect Fourier Delta Attention", §2.2 eq. (10): affine maps compose).
// One workgroup per (b, h, 16-column slice).  The slice of S_g stays in LDS,
// transposed, as the B operand of fp32 MFMA tiles (16 x 16 x 4); wavefront w
// takes row tiles w, w + 4, .. of X_g S_g, reading X_g straight from memory as
// the A operand (each element once per step) and starting from Y_g.
template <int DK>
__global__ __launch_bounds__(256) void segment_combine_kernel(const float* __restrict__ S0,
                                                              const float* __restrict__ summ,
                                                              float* __restrict__ Sseg, int BH,
                                                              int nseg, int Dv)
{
    constexpr int LD = DK + 4;
    __shared__ __attribute__((aligned(16))) float sT[16 * LD];     // S_g^T: [column][row]
    const int NS = Dv / 16;
    const int bh = blockIdx.x / NS, slice = blockIdx.x % NS;
    if (bh >= BH) return;
    const int tid = threadIdx.x, lane = tid & 63, ln = lane & 15, lg = lane >> 4;
    const int wave = tid >> 6;
    for (int idx = tid; idx < DK * 16; idx += 256) {
        const int r = idx / 16, j = idx % 16;
        sT[j * LD + r] = S0 ? S0[((size_t)bh * DK + r) * Dv + slice * 16 + j] : 0.f;
    }
    __syncthreads();
    constexpr int NT = DK / 16, TPW = (NT + 3) / 4;     // row tiles, per wavefront
    constexpr int NK = DK / 16;                          // k16 blocks
    // the operands of map gi: X_g rows of this wavefront's tiles (A fragments)
    // and Y_g's tile entries; the next map's are loaded during this product
    Vec4<float> xa[TPW][NK];
    f32x4 ya[TPW];
    auto load_ops = [&](int gi) {
        const float* xg = summ + (size_t)(bh * nseg + gi) * DK * (DK + Dv);
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            const int mt = min(wave + 4 * u, NT - 1);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                ya[u][i] = xg[(size_t)(16 * mt + 4 * lg + i) * (DK + Dv) + DK + slice * 16 + ln];
            const float* xr = xg + (size_t)(16 * mt + ln) * (DK + Dv) + 4 * lg;
#pragma unroll
            for (int kb = 0; kb < NK; ++kb) xa[u][kb] = Vec4<float>::load(xr + 16 * kb);
        }
    };
    if (nseg > 1) load_ops(0);
    for (int gi = 0; gi + 1 < nseg; ++gi) {
        f32x4 acc[TPW];
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            acc[u] = ya[u];
#pragma unroll
            for (int kb = 0; kb < NK; ++kb)
                acc[u] = mma_k16(xa[u][kb], Vec4<float>::load(sT + ln * LD + 16 * kb + 4 * lg), acc[u]);
        }
        if (gi + 2 < nseg) load_ops(gi + 1);
        __syncthreads();
        float* dst = Sseg + (size_t)(bh * nseg + gi + 1) * DK * Dv + slice * 16 + ln;
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            const int mt = wave + 4 * u;
            if (mt < NT) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * mt + 4 * lg + i;
                    sT[ln * LD + r] = acc[u][i];
                    dst[(size_t)r * Dv] = acc[u][i];
                }
            }
        }
        __syncthreads();
    }
}

template <int DK>
hipError_t launch_combine_t(int BH, int Dv, int nseg, const float* S0, const float* summ,
                            float* Sseg, hipStream_t stream)
{
    return launch_kernel(segment_combine_kernel<DK>, dim3((unsigned)(BH * (Dv / 16))), dim3(256),
                         0, stream, S0, summ, Sseg, BH, nseg, Dv);
}

template <typename T, int C, int DK>
hipError_t launch_chain_t(const ChunkShape& s, const ChainArgs& a, hipStream_t stream)
{
    using G = ChainGeom<T, C, DK>;
    auto kern = chain_kernel<T, C, DK>;
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)G::LDS_TOTAL);
    if (e != hipSuccess) return e;
    const int NS = a.summ ? DK / 16 + s.Dv / 16 : s.Dv / 16;
    const int bh = s.B * s.H * (a.nseg > 1 ? a.nseg : 1);
    const unsigned grid = (unsigned)(kXcds * NS * ((bh + kXcds - 1) / kXcds));
    return launch_kernel(kern, dim3(grid), dim3(kChainThreads), (uint32_t)G::LDS_TOTAL, stream, a);
}

template <typename T, int C>
hipError_t dispatch_dk(const ChunkShape& s, const ChainArgs& a, hipStream_t st)
{
    switch (s.Dk) {
    case 16: return launch_chain_t<T, C, 16>(s, a, st);
    case 32: return launch_chain_t<T, C, 32>(s, a, st);
    case 64: return launch_chain_t<T, C, 64>(s, a, st);
    case 128:
        if constexpr (sizeof(T) == 2) return launch_chain_t<T, C, 128>(s, a, st);
        else return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
    }
}

template <typename T>
hipError_t dispatch_c(const ChunkShape& s, const ChainArgs& a, hipStream_t st)
{
    switch (s.C) {
    case 16: return dispatch_dk<T, 16>(s, a, st);
    case 32: return dispatch_dk<T, 32>(s, a, st);
    case 64: return dispatch_dk<T, 64>(s, a, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_segment_combine(int BH, int Dk, int Dv, int nseg, const float* S0,
                                  const float* summ, float* Sseg, hipStream_t stream)
{
    switch (Dk) {
    case 16: return launch_combine_t<16>(BH, Dv, nseg, S0, summ, Sseg, stream);
    case 32: return launch_combine_t<32>(BH, Dv, nseg, S0, summ, Sseg, stream);
    case 64: return launch_combine_t<64>(BH, Dv, nseg, S0, summ, Sseg, stream);
    case 128: return launch_combine_t<128>(BH, Dv, nseg, S0, summ, Sseg, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_chain(IoType io, const ChunkShape& s, const ChainArgs& a, hipStream_t stream)
{
    if (io == IoType::F32) return dispatch_c<float>(s, a, stream);
    return dispatch_c<bf16_t>(s, a, stream);
}

}  // namespace kda
