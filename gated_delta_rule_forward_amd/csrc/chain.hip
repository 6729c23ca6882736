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
// sequence.  Operand fragments of chunks c+1 and c+2 are in flight while
// chunk c computes; the prep kernels store them fragment-major, so each
// wavefront's fragment of one MFMA is one contiguous 1 KB block.  Workgroups are numbered so that the column slices
// of one (b, h) land on the same XCD (consecutive workgroup ids go to
// consecutive XCDs) and share that XCD's L2 for the chunk operands.
#include "kda_chunk.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace {

constexpr int kChainThreads = 256;
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
};

template <typename T, int C, int DK>
struct ChainOps {
    using G = ChainGeom<T, C, DK>;
    using F = Frag<T, G::KB>;
    F w[G::NKD], qg[G::NKD], p[G::NKC];
    float u[4];
    F kt[G::SPW][G::NKC];
    float gc[G::SPW][4];
};

template <typename T, int C, int DK>
__device__ __forceinline__ void load_ops(ChainOps<T, C, DK>& o, const ChainArgs& a, size_t unit,
                                         int wave, int lane, int lg, int slice)
{
    using G = ChainGeom<T, C, DK>;
    using F = Frag<T, G::KB>;
    constexpr int NV = F::NV;
    const int Dv = a.Dv;
    if (G::NM == 4 || wave < G::NM) {
        const T* W = static_cast<const T*>(a.W) + unit * C * DK + (size_t)wave * G::NKD * 64 * NV;
        const T* QG = static_cast<const T*>(a.QG) + unit * C * DK + (size_t)wave * G::NKD * 64 * NV;
        const T* P = static_cast<const T*>(a.P) + unit * C * C + (size_t)wave * G::NKC * 64 * NV;
#pragma unroll
        for (int s = 0; s < G::NKD; ++s) {
            o.w[s] = F::load(W + (s * 64 + lane) * NV);
            o.qg[s] = F::load(QG + (s * 64 + lane) * NV);
        }
#pragma unroll
        for (int s = 0; s < G::NKC; ++s) o.p[s] = F::load(P + (s * 64 + lane) * NV);
        const float4 u = *reinterpret_cast<const float4*>(
            a.U + unit * C * Dv + ((size_t)(wave * (Dv / 16) + slice) * 64 + lane) * 4);
        o.u[0] = u.x; o.u[1] = u.y; o.u[2] = u.z; o.u[3] = u.w;
    }
#pragma unroll
    for (int u = 0; u < G::SPW; ++u) {
        const int t = wave + 4 * u;
        if (G::NT % 4 == 0 || t < G::NT) {
            const T* Kt = static_cast<const T*>(a.Kt) + unit * DK * C + (size_t)t * G::NKC * 64 * NV;
#pragma unroll
            for (int s = 0; s < G::NKC; ++s) o.kt[u][s] = F::load(Kt + (s * 64 + lane) * NV);
            const float4 g = *reinterpret_cast<const float4*>(a.GC + unit * DK + 16 * t + 4 * lg);
            o.gc[u][0] = g.x; o.gc[u][1] = g.y; o.gc[u][2] = g.z; o.gc[u][3] = g.w;
        }
    }
}

// write a C-layout tile (4 values per lane) into slot base (tile % TPB) * 4 of
// the lane's fragment of k block tile / TPB
template <typename T, int KB>
__device__ __forceinline__ void put_tile(Frag<T, KB>* frags, int tile, int lane, const f32x4& v)
{
    constexpr int TPB = KB / 16;
    T* p = reinterpret_cast<T*>(&frags[(tile / TPB) * 64 + lane]) + 4 * (tile % TPB);
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = from_f32<T>(v[i]);
}

template <typename T, int C, int DK>
__global__ __launch_bounds__(kChainThreads) void chain_kernel(ChainArgs a)
{
    using G = ChainGeom<T, C, DK>;
    using F = Frag<T, G::KB>;
    __shared__ F sSf[G::NKD * 64];
    __shared__ F sDf[G::NKC * 64];

    const int Dv = a.Dv, H = a.H, T_ = a.T, NC = a.NC;
    const int NS = Dv / 16;
    const int g = blockIdx.x, xcd = g % kXcds, jx = g / kXcds;
    const int bh = (jx / NS) * kXcds + xcd, slice = jx % NS;
    if (bh >= a.B * H) return;
    const int b = bh / H, h = bh % H;
    const int tid = threadIdx.x, lane = tid & 63, ln = lane & 15, lg = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = slice * 16 + ln;

    f32x4 S[G::SPW];
#pragma unroll
    for (int u = 0; u < G::SPW; ++u) {
        const int t = wave + 4 * u;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            S[u][i] = (a.S0 && t < G::NT) ? a.S0[((size_t)bh * DK + 16 * t + 4 * lg + i) * Dv + col] : 0.f;
        if (t < G::NT) put_tile<T, G::KB>(sSf, t, lane, S[u]);
    }
    __syncthreads();

    T* out = static_cast<T*>(a.out);
    const size_t ostride = (size_t)H * Dv;                      // one token
    T* obase = out + (((size_t)b * T_ + 16 * wave + 4 * lg) * H + h) * Dv + col;

    auto step = [&](const ChainOps<T, C, DK>& cur, int nc) {
        F sf[G::NKD];
#pragma unroll
        for (int s = 0; s < G::NKD; ++s) sf[s] = sSf[s * 64 + lane];
        if (G::NM == 4 || wave < G::NM) {
            f32x4 acc = zero4();
#pragma unroll
            for (int s = 0; s < G::NKD; ++s) acc = mma(cur.w[s], sf[s], acc);
            f32x4 dl;
#pragma unroll
            for (int i = 0; i < 4; ++i) dl[i] = cur.u[i] - acc[i];
            put_tile<T, G::KB>(sDf, wave, lane, dl);
        }
        __syncthreads();
        F df[G::NKC];
#pragma unroll
        for (int s = 0; s < G::NKC; ++s) df[s] = sDf[s * 64 + lane];
        if (G::NM == 4 || wave < G::NM) {
            f32x4 acc = zero4();
#pragma unroll
            for (int s = 0; s < G::NKD; ++s) acc = mma(cur.qg[s], sf[s], acc);
#pragma unroll
            for (int s = 0; s < G::NKC; ++s) acc = mma(cur.p[s], df[s], acc);
            T* o = obase + (size_t)nc * C * ostride;
            if (nc * C + C <= T_) {
#pragma unroll
                for (int i = 0; i < 4; ++i) o[i * ostride] = from_f32<T>(acc[i]);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (nc * C + 16 * wave + 4 * lg + i < T_) o[i * ostride] = from_f32<T>(acc[i]);
            }
        }
#pragma unroll
        for (int u = 0; u < G::SPW; ++u) {
            const int t = wave + 4 * u;
            if (G::NT % 4 == 0 || t < G::NT) {
                f32x4 acc;
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] = cur.gc[u][i] * S[u][i];
#pragma unroll
                for (int s = 0; s < G::NKC; ++s) acc = mma(cur.kt[u][s], df[s], acc);
                S[u] = acc;
                put_tile<T, G::KB>(sSf, t, lane, acc);
            }
        }
        __syncthreads();
    };

    // operand ring: chunk nc uses ops[nc % 3]; the loads of chunks nc+1 and
    // nc+2 are in flight while chunk nc computes.  Past the last chunk the
    // ring re-reads the last chunk instead of skipping the loads: every path
    // through the loop then issues the same loads, so the compiler's wait
    // counts stay exact and the waits only cover the chunk being used.
    ChainOps<T, C, DK> ops[3];
    const size_t u0 = (size_t)bh * NC;
    const int last = NC - 1;
    load_ops(ops[0], a, u0, wave, lane, lg, slice);
    load_ops(ops[1], a, u0 + min(1, last), wave, lane, lg, slice);
    for (int nc = 0; nc < NC; nc += 3) {
        load_ops(ops[2], a, u0 + min(nc + 2, last), wave, lane, lg, slice);
        step(ops[0], nc);
        if (nc + 1 >= NC) break;
        load_ops(ops[0], a, u0 + min(nc + 3, last), wave, lane, lg, slice);
        step(ops[1], nc + 1);
        if (nc + 2 >= NC) break;
        load_ops(ops[1], a, u0 + min(nc + 4, last), wave, lane, lg, slice);
        step(ops[2], nc + 2);
    }

    if (a.ST) {
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

template <typename T, int C, int DK>
hipError_t launch_chain_t(const ChunkShape& s, const ChainArgs& a, hipStream_t stream)
{
    const int NS = s.Dv / 16;
    const int bh = s.B * s.H;
    const unsigned grid = (unsigned)(kXcds * NS * ((bh + kXcds - 1) / kXcds));
    return launch_kernel(chain_kernel<T, C, DK>, dim3(grid), dim3(kChainThreads), 0, stream, a);
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

hipError_t launch_chain(IoType io, const ChunkShape& s, const ChainArgs& a, hipStream_t stream)
{
    if (io == IoType::F32) return dispatch_c<float>(s, a, stream);
    return dispatch_c<bf16_t>(s, a, stream);
}

}  // namespace kda
