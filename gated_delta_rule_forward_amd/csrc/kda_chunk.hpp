// kda_chunk.hpp — definitions shared by the chunked-forward kernels (internal).
//
// Workspace layout (per unit = one chunk of one (b, h); NU units).  The chain
// kernel feeds W, QG, P and Kt to MFMA as A operands against B operands taken
// straight from C-layout accumulators, so they are stored fragment-major: an
// A-operand matrix with R rows and K columns is [R/16][K/KB][64 lanes][KB/4],
// each (16-row tile, k block) being the 64 per-lane fragments of one MFMA, one
// contiguous block (see frag_off).  U is stored as the C-layout accumulator
// tiles the chain adds it to.
//   W  [NU] A-operand, rows = tokens (C),   k = channels (Dk)   io type
//   QG [NU] A-operand, rows = tokens (C),   k = channels (Dk)   io type
//   P  [NU] A-operand, rows = tokens (C),   k = tokens (C)      io type
//   Kt [NU] A-operand, rows = channels (Dk), k = tokens (C)     io type
//   U  [NU][C/16][Dv/16][64 lanes][4]  io type (lane 16g+n, element i holds
//                                      row 4g+i, column n of the tile)
//   GC [NU][Dk]      fp32
//   FL [NU]          uint8: 1 = the unit needs the exact fallback kernel
//
// Fragment slots.  With k32 blocks (bf16, 16x16x32) lane (m, g) = 16g + m of
// block s holds, in slot j = 0..7, column 32s + 16(j/4) + 4g + (j%4) of row m:
// the slots pair with the B fragment built from two C-layout tiles (rows 4g..
// 4g+3 of tiles 2s and 2s+1).  k16 blocks (bf16 16x16x16, fp32 4 x 16x16x4)
// use column 16s + 4g + j.
#pragma once

#include "kda_device.hpp"

namespace kda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

// k-block width used for a (dtype, chunk, Dk) instance: bf16 contracts 32 at a
// time when both contraction lengths allow it, else 16; fp32 always 16.
template <typename T, int C, int DK>
struct KBlock {
    static constexpr int value = (sizeof(T) == 2 && C >= 32 && DK >= 32) ? 32 : 16;
};

// Offset of element (row r, column k) of an A-operand matrix with K columns
// in the fragment-major layout described above.
template <int KB>
__host__ __device__ __forceinline__ int frag_off(int r, int k, int K) {
    constexpr int NV = KB / 4;
    const int kk = k % KB;
    int g, j;
    if constexpr (KB == 32) { g = (kk & 15) >> 2; j = 4 * (kk >> 4) + (kk & 3); }
    else { g = kk >> 2; j = kk & 3; }
    return (((r >> 4) * (K / KB) + k / KB) * 64 + 16 * g + (r & 15)) * NV + j;
}
// Offset of element (row r, column c) of U (C-layout tiles, Dv columns).
__host__ __device__ __forceinline__ int u_off(int r, int c, int Dv) {
    return (((r >> 4) * (Dv >> 4) + (c >> 4)) * 64 + 16 * ((r & 15) >> 2) + (c & 15)) * 4 + (r & 3);
}

// ---- k-block fragments -------------------------------------------------------
// one lane's share of a k block: KB/4 consecutive k of one A row / B column
template <typename T, int KB> struct Frag;
template <> struct Frag<bf16_t, 32> {
    static constexpr int NV = 8;
    i16x8 v;
    __device__ __forceinline__ static Frag load(const bf16_t* p) {   // 16-byte aligned
        return Frag{*reinterpret_cast<const i16x8*>(p)};
    }
    __device__ __forceinline__ static Frag from(const float* f) {
        i16x8 r;
#pragma unroll
        for (int j = 0; j < 8; ++j) r[j] = bf16_bits((bf16_t)f[j]);
        return Frag{r};
    }
};
template <> struct Frag<bf16_t, 16> {
    static constexpr int NV = 4;
    i16x4 v;
    __device__ __forceinline__ static Frag load(const bf16_t* p) {   // 8-byte aligned
        return Frag{*reinterpret_cast<const i16x4*>(p)};
    }
    __device__ __forceinline__ static Frag from(const float* f) {
        i16x4 r;
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = bf16_bits((bf16_t)f[j]);
        return Frag{r};
    }
};
template <> struct Frag<float, 16> {
    static constexpr int NV = 4;
    float v[4];
    __device__ __forceinline__ static Frag load(const float* p) {     // 16-byte aligned
        const float4 x = *reinterpret_cast<const float4*>(p);
        return Frag{{x.x, x.y, x.z, x.w}};
    }
    __device__ __forceinline__ static Frag from(const float* f) { return Frag{{f[0], f[1], f[2], f[3]}}; }
};

__device__ __forceinline__ f32x4 mma(const Frag<bf16_t, 32>& a, const Frag<bf16_t, 32>& b, f32x4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a.v),
                                                   __builtin_bit_cast(bf16x8, b.v), acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const Frag<bf16_t, 16>& a, const Frag<bf16_t, 16>& b, f32x4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const Frag<float, 16>& a, const Frag<float, 16>& b, f32x4 acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[0], b.v[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[1], b.v[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[2], b.v[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[3], b.v[3], acc, 0, 0, 0);
    return acc;
}

// write a C-layout tile (4 values per lane) into slot base (tile % TPB) * 4 of
// the lane's fragment of k block tile / TPB (B fragments kept in LDS)
template <typename T, int KB>
__device__ __forceinline__ void put_tile(Frag<T, KB>* frags, int tile, int lane, const f32x4& v)
{
    constexpr int TPB = KB / 16;
    T* p = reinterpret_cast<T*>(&frags[(tile / TPB) * 64 + lane]) + 4 * (tile % TPB);
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = from_f32<T>(v[i]);
}

// B fragment of k block s built from C-layout accumulator tiles (rows 4g+i of
// column n in lane l = 16g + n): a k32 block spans tiles 2s and 2s+1 (slot j =
// tile 2s + j/4, register j%4), a k16 block is tile s.
template <typename T, int KB>
__device__ __forceinline__ Frag<T, KB> frag_from_tiles(const f32x4* tiles, int s) {
    if constexpr (KB == 32) {
        const float f[8] = {tiles[2 * s][0], tiles[2 * s][1], tiles[2 * s][2], tiles[2 * s][3],
                            tiles[2 * s + 1][0], tiles[2 * s + 1][1], tiles[2 * s + 1][2],
                            tiles[2 * s + 1][3]};
        return Frag<T, KB>::from(f);
    } else {
        const float f[4] = {tiles[s][0], tiles[s][1], tiles[s][2], tiles[s][3]};
        return Frag<T, KB>::from(f);
    }
}

// A (or Bt) fragment of one row, k block starting at k0, from a row-major
// matrix in natural k order: lane group g takes k0 + (KB/4) g .. + KB/4 - 1,
// which is the hardware's own k order for both operands.
template <typename T, int KB>
__device__ __forceinline__ Frag<T, KB> frag_row(const T* row, int k0) {
    const int g = (threadIdx.x & 63) >> 4;
    return Frag<T, KB>::load(row + k0 + Frag<T, KB>::NV * g);
}
// same from an fp32 row, converted to T
template <typename T, int KB>
__device__ __forceinline__ Frag<T, KB> frag_row_cvt(const float* row, int k0) {
    const int g = (threadIdx.x & 63) >> 4;
    constexpr int NV = Frag<T, KB>::NV;
    float f[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) f[j] = row[k0 + NV * g + j];
    return Frag<T, KB>::from(f);
}

// 16x16 tile of A * Bt^T, both row-major with k contiguous (natural k order);
// row r of the tile is A + r*lda, column n is Bt + n*ldb.
template <typename T, int KB>
__device__ __forceinline__ f32x4 tile_tn_nat(const T* A, int lda, const T* Bt, int ldb, int K) {
    const int r = threadIdx.x & 15;
    f32x4 acc = zero4();
    for (int k0 = 0; k0 < K; k0 += KB)
        acc = mma(frag_row<T, KB>(A + r * lda, k0), frag_row<T, KB>(Bt + r * ldb, k0), acc);
    return acc;
}

// Streamed forward: the prep and chain kernels run at the same time and hand
// each unit over through the L2 of the XCD both run on; these control words
// and a ready word per unit live in the workspace (cleared by the call).
// (each group of words that workgroups poll or update often sits on a
// 128-byte cache line of its own)
struct StreamCtl {
    unsigned prep_next[8];     // next unit index per XCD (prep workgroups)
    unsigned pad0[24];
    unsigned chain_next[8];    // next (head, column slice) index per XCD (chain workgroups)
    unsigned chains_done;      // chain workgroups that ran their sequence to the end
    unsigned expect;           // chain workgroups the call needs
    unsigned tiles;            // column tiles per chain workgroup (a record of the call's choice)
    unsigned pad1[21];
    unsigned abort;            // a chain workgroup met a unit of the exact kernel or gave up waiting
    unsigned pad2[31];
};
static_assert(sizeof(StreamCtl) == 384, "three 128-byte lines");

struct PrepArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* alpha;
    const float* beta;
    void* W;
    void* U;
    void* Kt;
    void* QG;
    void* P;
    float* GC;
    uint8_t* FL;
    int T, H, Dv, NC;
    int zx;   // most zero gates per chunk the fast prep kernel takes (each one
              // adds a contraction column; 0: a chunk with a zero gate is flagged)
    // input parameterisation ("Semidirect Fourier Delta Attention" §3, eqs.
    // (15), (17), (18)); when pro != 0, alpha holds gate logits, beta holds
    // beta logits and q, k are raw:  alpha = amin + arange * sigmoid(gate),
    // beta = bmax * sigmoid(logit), k = k / (|k| + eps), q likewise if normq
    int pro;
    float amin, arange, bmax, eps;
    int normq;
    // packed (variable-length) batches: cu [N + 1] token offsets and cs [N + 1]
    // chunk offsets of the N sequences (sanitised copies), or null for dense
    const int* cu;
    const int* cs;
    int N;
    // phase variant ("Semidirect Fourier Delta Attention" eq. (13)): theta
    // [..., Dk/2] per channel pair and alpha then also per pair; null = KDA
    const float* theta;
    // backward support: Tinv = (I + A)^{-1} of every unit, fp32 [NU][C][C]
    // row-major (zero above the diagonal), or null
    float* Tm;
    // dense batches: pcn > 0 restricts a launch to chunks [pc0, pc0 + pcn) of
    // every (b, h) (launch index v -> unit part_unit(v, ...)); 0: all units
    int pc0, pcn;
    // nonzero: the fast prep kernel writes the whole-fragment workspace blocks
    // (P, W, U) with non-temporal stores (worth it when many chains stream the
    // workspace; plain inputs only, not the prologue or phase variants)
    int ntst;
    // streamed forward: B H, the ready word of every unit and the control words
    int nbh;
    unsigned* ready;
    StreamCtl* sctl;
    // streamed forward: a unit of chunk n >= lead first waits (a bounded,
    // advisory wait) until the chain of its (b, h) has taken chunk n - lead;
    // 0: no wait
    int lead;
};

// unit of launch index v when a launch covers chunks [pc0, pc0 + pcn) of every
// (b, h) of a dense batch with NC chunks per (b, h); pcn = 0: v itself
__host__ __device__ __forceinline__ int part_unit(int v, int pc0, int pcn, int NC)
{
    return pcn > 0 ? (v / pcn) * NC + pc0 + v % pcn : v;
}

// sum over the NQ consecutive lanes of a group (every lane receives the sum)
template <int NQ>
__device__ __forceinline__ float quad_group_sum(float x)
{
#pragma unroll
    for (int off = NQ / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, NQ);
    return x;
}

// x / (|x|_2 + eps) for one token whose Dk channels are spread as quads over NQ
// consecutive lanes (a zero vector stays zero)
template <typename T, int NQ>
__device__ __forceinline__ Vec4<T> l2_normalised(const Vec4<T>& v, float eps)
{
    float f[4], ss = 0.f;
#pragma unroll
    for (int x = 0; x < 4; ++x) { f[x] = v.get(x); ss += f[x] * f[x]; }
    const float nrm = __builtin_sqrtf(quad_group_sum<NQ>(ss)) + eps;
    const float inv = nrm > 0.f ? 1.f / nrm : 0.f;
#pragma unroll
    for (int x = 0; x < 4; ++x) f[x] *= inv;
    return Vec4<T>::from(f);
}

// logistic function in fp32 (exp2 of the scaled argument; saturates to 0 / 1)
__device__ __forceinline__ float sigmoid_f32(float x)
{
    return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-x * 1.4426950408889634f));
}

struct ChainArgs {
    const void* W;
    const void* U;
    const void* Kt;
    const void* QG;
    const void* P;
    const float* GC;
    const float* S0;
    void* out;
    float* ST;
    void* CS;          // chunk-start states [B,H,NC,Dk,Dv] in the io type, or null
    int B, T, H, Dv, NC;
    const int* cu;     // packed batches (B = number of sequences): see PrepArgs
    const int* cs;
    int ph;            // GC holds (magnitude cos, magnitude sin) per channel pair
    // sequence segments (dense batches): nseg segments of seg chunks per (b, h).
    // summ != null: summary pass, segment g's affine map S -> X_g S + Y_g into
    // summ [B H][nseg][Dk][Dk + Dv] (column slices 0 .. Dk/16 - 1 carry X from
    // the identity with U = 0, the rest carry Y from zero), no outputs.
    // Otherwise with nseg > 1: segment g starts from Sseg [B H][nseg][Dk][Dv]
    // (g = 0: S0) and only the last segment writes ST.
    int seg, nseg;
    float* summ;
    const float* Sseg;
    // backward support (dense batches): the fp32 state entering every chunk,
    // CS32 [NU][Dk][Dv], and every chunk's deltas Delta, DL [NU][C][Dv]
    // (rows past the sequence end hold zeros); either may be null.  out may
    // be null when only these are wanted.
    float* CS32;
    float* DL;
    // dense batches without segments: pcn > 0 runs chunks [pc0, pc0 + pcn) of
    // every (b, h) only, from S0 (the state entering chunk pc0) to ST (the
    // state leaving the range; may be S0: each workgroup reads its slice of S0
    // before it writes that slice of ST)
    int pc0, pcn;
    // streamed forward: the ready words (the chain marks each unit it takes)
    // and control words the chain waits on (streamed kernel), or (gate) the
    // control words that decide whether this launch runs at all: only when
    // the streamed chain gave up or did not cover every (b, h)
    unsigned* ready;
    StreamCtl* sctl;
    const StreamCtl* gate;
};

// Streamed forward: how long a chain wavefront waits for one unit before it
// gives up (s_memrealtime ticks, 100 MHz: 10 ms, far beyond the time the prep
// grid takes per chunk index), and a cap on the polls of one wait that ends it
// whatever the clock reads (about 0.2 us per poll); the call then recomputes
// the chain after the prep grid has finished, so giving up costs time, never
// correctness.  (The usual cause: the two streams share a hardware queue, so
// the prep grid cannot start before the chain ends.)
constexpr unsigned long long kStreamWaitTicks = 1000000ull;
constexpr unsigned kStreamWaitPolls = 1u << 18;
// The prep's lead wait (advisory: past its bound the unit goes ahead): 1 ms,
// and a poll cap likewise
constexpr unsigned long long kLeadWaitTicks = 100000ull;
constexpr unsigned kLeadWaitPolls = 1u << 15;

// Wait until unit u's ready word reads 1 (its factors are in the workspace,
// written from this XCD).  Gives up, raising the abort word, when the unit
// needs the exact kernel (2), when another workgroup gave up, or when the
// bound expires.  `first` is a value of the ready word read earlier.  Every
// lane of the wavefront takes part and gets the same answer.
__device__ inline bool stream_wait_ready(unsigned* ready, StreamCtl* ctl, size_t u,
                                         unsigned first)
{
    // ready: 1, or 3 once a chain workgroup of the (b, h) has taken the unit
    // (the prep's lead limit reads that mark); 2: the exact kernel's unit
    if (first == 3u) return true;
    if (first == 1u) {
        __hip_atomic_store(&ready[u], 3u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return true;
    }
    unsigned r = first;
    const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
    for (unsigned n = 0;; ++n) {
        if (r == 2u ||
            ((n & 15) == 15 && __hip_atomic_load(&ctl->abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) ||
            __builtin_amdgcn_s_memrealtime() - t0 > kStreamWaitTicks || n >= kStreamWaitPolls)
            break;
        __builtin_amdgcn_s_sleep(2);
        r = __hip_atomic_load(&ready[u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (r == 3u) return true;
        if (r == 1u) {
            __hip_atomic_store(&ready[u], 3u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return true;
        }
    }
    __hip_atomic_store(&ctl->abort, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return false;
}

// Backward (dense batches).  The reverse chain reads the forward's operands
// after relayout_kernel turned them into W^T, (Q * Gamma)^T, Ktil and P^T
// (fragment-major A operands: rows channels / tokens / tokens, k tokens /
// channels / tokens) and writes, per unit, the gradient of the state leaving
// the chunk (DSN [NU][Dk][Dv] fp32) and X = P^T dO + Ktil dSn (XB [NU][C][Dv]
// fp32); dS0 [B,H,Dk,Dv] may be null, dST (may be null = zero) seeds it.
struct BwdChainArgs {
    const void* Ktil;
    const void* PT;
    const void* QGT;
    const void* WT;
    const float* GC;
    const void* dO;
    const float* dST;
    float* dS0;
    float* DSN;
    float* XB;
    int B, T, H, Dv, NC;
    const int* cu;     // packed batches (B = number of sequences): see PrepArgs
    const int* cs;
};
// The per-chunk gradient kernels: inputs, Tinv (Tm), the fp32 chunk states
// (CS32), Delta (DL), DSN and XB (replaced by y in flagged units); outputs
// dq, dk, dv (io type), dalpha, dbeta (fp32) and FLB [NU] (1 = the unit has a
// gate with |alpha| < 2^-6, whose dalpha the small-gate kernel writes).
struct BwdLocalArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* alpha;
    const float* beta;
    const void* dO;
    const float* Tm;
    const float* CS32;
    const float* DL;
    const float* DSN;
    float* XB;
    void* dq;
    void* dk;
    void* dv;
    float* dalpha;
    float* dbeta;
    uint8_t* FLB;
    int T, H, Dv, NC;
    const int* cu;     // packed batches: see PrepArgs (null for dense)
    const int* cs;
    int N;
};

// The input prologue around the backward: raw q, k (io type), gate and beta
// logits (fp32) -> qh, kh (io type), al, be (fp32), and afterwards the raw
// gradients dq_raw, dk_raw (io type) from dqh, dkh, with dgate / dblogit
// (holding d alpha / d beta on entry) turned into the logits' gradients.
struct ProArgs {
    const void* q_raw;
    const void* k_raw;
    const float* gate;
    const float* blogit;
    void* qh;
    void* kh;
    float* al;
    float* be;
    const void* dqh;
    const void* dkh;
    void* dq_raw;
    void* dk_raw;
    float* dgate;
    float* dblogit;
    size_t ntok;
    float amin, arange, bmax, eps;
    int normq;
};

// Where one unit (one chunk of one sequence and head) lives.  Dense batches:
// unit = (b H + h) NC + n, tokens from row b T + n C.  Packed batches:
// sequence i owns units [cs[i] H, cs[i+1] H) ordered (head, chunk), tokens
// from row cu[i] + n C; the same numbering as the dense one when every
// sequence has the same length.  Units past the last sequence are invalid.
struct UnitPos { int bh, h, n, row0, nvalid; bool valid; };
__device__ __forceinline__ UnitPos locate_unit(int unit, int H, int T, int NC, int C,
                                               const int* cu, const int* cs, int N)
{
    UnitPos p;
    if (!cu) {
        p.n = unit % NC;
        p.bh = unit / NC;
        p.h = p.bh % H;
        p.row0 = (p.bh / H) * T + p.n * C;
        p.nvalid = min(C, T - p.n * C);
        p.valid = true;
        return p;
    }
    p.valid = unit < cs[N] * H;
    int lo = 0, hi = N;               // cs[lo] H <= unit < cs[hi] H
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (cs[mid] * H <= unit) lo = mid; else hi = mid;
    }
    const int nci = max(cs[lo + 1] - cs[lo], 1);
    const int rem = unit - cs[lo] * H;
    p.h = min(rem / nci, H - 1);
    p.n = rem % nci;
    p.bh = lo * H + p.h;
    p.row0 = cu[lo] + p.n * C;
    p.nvalid = min(C, cu[lo + 1] - cu[lo] - p.n * C);
    p.valid = p.valid && p.nvalid > 0;
    return p;
}

// One (sequence, head) chain: its chunk count, first token row, length and
// first unit.
struct SeqPos { int nc, row0, len; size_t ubase; };
__device__ __forceinline__ SeqPos locate_seq(int bh, int H, int T, int NC, const int* cu,
                                             const int* cs)
{
    SeqPos p;
    if (!cu) {
        p.nc = NC;
        p.row0 = (bh / H) * T;
        p.len = T;
        p.ubase = (size_t)bh * NC;
        return p;
    }
    const int i = bh / H, h = bh % H;
    p.nc = cs[i + 1] - cs[i];
    p.row0 = cu[i];
    p.len = cu[i + 1] - cu[i];
    p.ubase = (size_t)cs[i] * H + (size_t)h * p.nc;
    return p;
}

}  // namespace kda
