// kda_api.hip — the C ABI declared in include/kda.h.
//
// Every entry point validates all of its arguments before making any HIP call,
// then only enqueues kernels on the caller's stream (no allocation, no
// synchronisation).  Per-kernel HIP events are recorded only when the caller
// passes KDA_FLAG_STAGE_EVENTS.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <stdint.h>
#include <string.h>

#include <map>
#include <vector>
#include <algorithm>
#include <mutex>

#include "../../include/kda.h"
#include "kda_chunk.hpp"
#include "kda_launch.hpp"
#include "range_check.hpp"

namespace {

using kda::ChunkShape;
using kda::ChunkWorkspace;
using kda::IoType;

constexpr unsigned kKnownFlags = KDA_FLAG_VALIDATE_RANGES | KDA_FLAG_STAGE_EVENTS |
                                  KDA_FLAG_NO_SEGMENTS | KDA_FLAG_SINGLE_STREAM | KDA_FLAG_STREAMED;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
bool aligned16(const void* p) { return aligned(p, 16); }

bool dk_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool dv_ok(int d) { return d >= 16 && d <= 128 && d % 16 == 0; }
bool chunk_ok(int c) { return c == 16 || c == 32 || c == 64; }

size_t elem_size(kda_dtype_t t) { return t == KDA_DTYPE_F32 ? 4 : 2; }

// Extra zero-segment columns the fast prep kernel may take per chunk: none in
// KDA mode (a zero gate is in range but rare there; a chunk that holds one goes
// to the exact kernel), 4 Dk in CKDA mode (contracted Dk per pass, so at most four
// extra passes); a chunk with more zero gates goes to the exact kernel.
int fast_zero_columns(int mode, int Dk) { return mode == KDA_MODE_CKDA ? 4 * Dk : 0; }

// Non-temporal stores of the prep kernel's whole-fragment workspace blocks:
// with at least 128 (b, h, 16-column) chains streaming the workspace the chain
// runs faster (256 chains at H=32, T=8192: 0.322 -> 0.314 ms per forward);
// with 16 chains (H=2, T=65536) it ran 4-10 % slower.
int workspace_nt(long long chains) { return chains >= 128 ? 1 : 0; }

// [p, p + n) and [q, q + m) intersect (n, m in bytes; empty ranges never do)
bool overlaps(const void* p, size_t n, const void* q, size_t m)
{
    if (!p || !q || n == 0 || m == 0) return false;
    const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
    return a < b + m && b < a + n;
}

// ---- per-kernel events (opt-in) ---------------------------------------------
// Stage i owns events 2i and 2i+1, attached to its kernel launch: the elapsed
// time between them is that kernel's own duration.
constexpr int kMaxParts = 8;
constexpr int kMaxStages = 3 * kMaxParts;
struct StageEvents {
    std::mutex mu;
    hipEvent_t ev[2 * kMaxStages] = {};
    const char* names[kMaxStages] = {};
    int count = 0;
    bool created = false;
};
StageEvents g_stage;

hipError_t stage_begin()
{
    if (!g_stage.created) {
        for (int i = 0; i < 2 * kMaxStages; ++i) {
            const hipError_t e = hipEventCreate(&g_stage.ev[i]);
            if (e != hipSuccess) return e;
        }
        g_stage.created = true;
    }
    g_stage.count = 0;
    return hipSuccess;
}

struct Recorder {
    bool on;
    hipStream_t stream;
    hipError_t mark(const char* name_of_next)   // the next launch is stage `name`
    {
        if (!on) return hipSuccess;
        if (g_stage.count >= kMaxStages) return hipErrorInvalidValue;
        g_stage.names[g_stage.count] = name_of_next;
        kda::g_launch_timer = {g_stage.ev[2 * g_stage.count], g_stage.ev[2 * g_stage.count + 1]};
        return hipSuccess;
    }
    hipError_t done()   // that launch has been enqueued
    {
        if (!on) return hipSuccess;
        kda::g_launch_timer = {};
        g_stage.count += 1;
        return hipSuccess;
    }
    ~Recorder() { if (on) kda::g_launch_timer = {}; }
};

// The chain of a forward: the wide-slice kernel (chain_wide.hip) where it
// covers the shape and the call (outputs wanted; no summary pass, segment
// starts or backward side outputs), else the 16-column kernel (chain.hip).
hipError_t launch_forward_chain(IoType io, const ChunkShape& sh, const kda::ChainArgs& a,
                                hipStream_t s)
{
    const int ct = kda::wide_chain_tiles(io, sh);
    if (ct > 0 && a.out && !a.summ && a.nseg <= 1 && !a.CS32 && !a.DL)
        return kda::launch_chain_wide(io, sh, a, ct, s);
    return kda::launch_chain(io, sh, a, s);
}

// fields shared by the forward and its workspace query
kda_status_t check_forward_shape(int B, int T, int H, int Dk, int Dv, int chunk,
                                 kda_dtype_t dtype)
{
    if (B < 1 || H < 1 || T < 0) return KDA_ERR_BAD_SHAPE;
    if (dtype != KDA_DTYPE_F32 && dtype != KDA_DTYPE_BF16) return KDA_ERR_UNSUPPORTED;
    if (!dk_ok(Dk) || !dv_ok(Dv) || !chunk_ok(chunk)) return KDA_ERR_UNSUPPORTED;
    // fp32 with Dk = 128: the chain is the register-operand kernel, chunk 64 only
    if (dtype == KDA_DTYPE_F32 && Dk == 128 && chunk != 64) return KDA_ERR_UNSUPPORTED;
    const long long NC = ((long long)T + chunk - 1) / chunk;
    const long long units = (long long)B * H * NC;
    if (units > 0x7fffffffLL || (long long)B * H * (Dv / 16) > 0x7fffffffLL)
        return KDA_ERR_BAD_SHAPE;
    const long long tok = (long long)B * T * H;
    if (tok * (Dk > Dv ? Dk : Dv) > (1LL << 46)) return KDA_ERR_BAD_SHAPE;
    return KDA_OK;
}

ChunkShape make_shape(int B, int T, int H, int Dk, int Dv, int chunk)
{
    return ChunkShape{B, T, H, Dk, Dv, chunk, (T + chunk - 1) / chunk};
}

// Sequence segments for a dense forward whose chains leave most of the GPU
// idle: with few (b, h, column slice) chains and many chunks, each (b, h) is
// cut into nseg segments that run side by side (a summary pass computes each
// segment's affine map, a short fp32 pass chains the segment start states,
// then every segment runs the normal chain from its own start).  nseg <= 1:
// no segments.  The summary pass must fit one round of workgroups.
struct Segments { int nseg, seg; };
Segments segments_for(int B, int H, int Dk, int Dv, int NC, kda_dtype_t dtype)
{
    // (the summary pass runs on the 16-column chain, which has no fp32 Dk = 128 form)
    if (dtype == KDA_DTYPE_F32 && Dk == 128) return {1, NC};
    const long long chains = (long long)B * H * (Dv / 16);
    if (chains > 64 || NC < 128) return {1, NC};
    const long long per = (long long)B * H * ((Dk + Dv) / 16);   // summary workgroups per segment
    long long g = 256 / per;
    if (g > NC / 32) g = NC / 32;
    if (g < 2) return {1, NC};
    const int seg = (int)((NC + g - 1) / g);
    return {(NC + seg - 1) / seg, seg};
}

static_assert(KDA_SIDE_EVENTS == 1 + kMaxParts, "one event for the call's start, one per part");

// Prep / chain overlap for a dense forward whose chains leave half the GPU or
// more idle: the chunks of every (b, h) are cut into `parts` consecutive
// ranges of `len` chunks, and the prep kernels of range p + 1 run on a second
// stream, on the idle compute units, while the chain runs range p.  Measured
// (B=1, H=16, T=65536, d=128, CKDA bf16: 128 chains, 1024 chunks): 2.09 ms in
// one pass, 1.87 ms in 8 parts.  With 256 chains (H=32, T=8192) the prep
// slows the chain more than it saves (0.340 -> 0.375 ms in 2 parts), and
// short chunk axes lose to the extra launches.  parts <= 1: one prep pass,
// then one chain pass.
struct Parts { int parts, len; };
Parts parts_for(int B, int H, int Dk, int Dv, int NC)
{
    (void)Dk;
    const long long chains = (long long)B * H * (Dv / 16);
    if (chains > 128 || NC < 256) return {1, NC};
    const int len = (NC + kMaxParts - 1) / kMaxParts;
    return {(NC + len - 1) / len, len};
}

// Streamed forward: the prep's lead limit.  Left alone, the prep grid runs
// far ahead of the chain on long sequences, and the factors of the chunks in
// between (72.5 KB per unit at bf16, Dk = Dv = 128) no longer fit the
// caches by the time the chain reads them; the limit keeps about 64 MiB of
// units between the two, a quarter of the MI355X's 256 MB last-level cache
// (at H = 16, T = 65536: 56 chunks, 1.80 -> 1.66 ms per call; 8 chunks starve
// the chain, 2.6 ms).
constexpr size_t kStreamLeadBytes = (size_t)64 << 20;
static int stream_lead(long long bhn, int Dk, int Dv, int chunk, size_t e)
{
    const size_t unit = (size_t)chunk * (3 * (size_t)Dk + Dv + chunk) * e + (size_t)Dk * 4;
    const size_t l = kStreamLeadBytes / ((size_t)bhn * unit);
    return (int)(l < 16 ? 16 : (l > (1u << 20) ? (1u << 20) : l));
}

// Streamed forward (kda_chunk_forward_side with KDA_FLAG_STREAMED): the chunk
// factors are formed by a prep grid on the side stream while the chain
// consumes them on the caller's stream, unit by unit, through the L2 of the
// XCD both run on.  Covered: bf16, chunk 64, Dk 128 or 64, at least 8 (b, h)
// (every XCD holds heads, so every XCD's prep workgroups have units to form),
// and a chain width that leaves half the compute units to the prep grid.
int stream_tiles(int B, int H, int Dk, int Dv);
bool stream_shape(int B, int H, int Dk, int Dv, int chunk, kda_dtype_t dtype)
{
    return dtype == KDA_DTYPE_BF16 && chunk == 64 && (Dk == 128 || Dk == 64) &&
           (long long)B * H >= 8 && stream_tiles(B, H, Dk, Dv) > 0;
}
// Column tiles per workgroup of the streamed chain (the wide kernel; each
// workgroup holds a whole compute unit).  Allowed: the widths that keep the
// chain within 128 workgroups (stream_tiles: the fewest such, 0 when none:
// the call then takes the two-pass form).  Chosen (stream_pick_tiles): the
// allowed width whose estimated call is shortest, the call being about the
// longer of the chain (NC steps of 1.3, 1.6 or 2.9 us at 1, 2 or 4 tiles
// beside the prep grid) and the prep grid on the compute units the chain
// leaves (8.6 us of one compute unit per unit, 11.2 with zero-segment
// columns: the prep's time on the whole GPU at H=32, T=8192 and at H=16,
// T=65536 CKDA; with the earlier 9.4 / 13.4 the long-context call took two
// tiles, 1.60 ms, against 1.51 at one).  Measured (bf16, d = 128; ms per call, two-pass against
// streamed at 1 / 2 / 4 tiles): H=32, T=8192: 0.327 against gives up (the
// chain fills every compute unit) / 0.318 / 0.395; H=16, T=8192: 0.237
// against 0.187 / 0.225 / 0.289; H=16, T=65536 (CKDA): 1.84 in parts
// against 1.79 / 1.675 / 2.41; H=24, T=8192: 0.272 against - / 0.230 /
// 0.290; B=2, H=32, T=8192: 0.606 against - / - / 0.58.
int stream_tiles(int B, int H, int Dk, int Dv)
{
    const long long chains = (long long)B * H * (Dv / 16);
    const int maxt = Dk == 128 ? 4 : 2;
    for (int ct = 1; ct <= maxt; ct *= 2)
        if (Dv % (16 * ct) == 0 && chains / ct <= 128) return ct;
    return 0;
}
int stream_pick_tiles(int B, int H, int Dk, int Dv, int NC, bool zero_cols, int ncu)
{
    const long long chains = (long long)B * H * (Dv / 16);
    const double units = (double)B * H * NC, unit_cu_us = zero_cols ? 11.2 : 8.6;
    const int maxt = Dk == 128 ? 4 : 2;
    int best = stream_tiles(B, H, Dk, Dv);
    double best_t = 1e30;
    for (int ct = best; ct >= 1 && ct <= maxt; ct *= 2) {
        if (Dv % (16 * ct) != 0 || chains / ct > 128) continue;
        const double wgs = (double)(chains / ct);
        const double chain = NC * (ct == 1 ? 1.3 : ct == 2 ? 1.6 : 2.9);
        const double prep = units * unit_cu_us / std::max(1.0, ncu - wgs);
        const double t = std::max(chain, prep);
        if (t < best_t) { best_t = t; best = ct; }
    }
    return best;
}

// workspace of a dense forward: the per-unit regions, then (with segments)
// the segment maps [B H][nseg][Dk][Dk + Dv] and start states [B H][nseg][Dk][Dv],
// then (with parts) the state between parts [B H][Dk][Dv] fp32
size_t dense_layout(int B, int T, int H, int Dk, int Dv, int chunk, IoType io,
                    size_t off[kda::kWorkspaceRegions], size_t* summ_off, size_t* sseg_off,
                    size_t* spart_off = nullptr, size_t* ready_off = nullptr,
                    size_t* sctl_off = nullptr)
{
    const ChunkShape sh = make_shape(B, T, H, Dk, Dv, chunk);
    size_t n = kda::chunk_workspace_layout(sh, io, off);
    const Segments sgm = segments_for(B, H, Dk, Dv, sh.NC, io == IoType::F32 ? KDA_DTYPE_F32 : KDA_DTYPE_BF16);
    *summ_off = *sseg_off = 0;
    if (sgm.nseg > 1) {
        const size_t bhs = (size_t)B * H * sgm.nseg;
        *summ_off = n;
        n += (bhs * Dk * (Dk + Dv) * 4 + 255) & ~size_t(255);
        *sseg_off = n;
        n += (bhs * Dk * Dv * 4 + 255) & ~size_t(255);
    }
    if (spart_off) *spart_off = 0;
    if (parts_for(B, H, Dk, Dv, sh.NC).parts > 1) {
        if (spart_off) *spart_off = n;
        n += ((size_t)B * H * Dk * Dv * 4 + 255) & ~size_t(255);
    }
    // (streamed forward) a ready word per unit, then the control words
    if (ready_off) *ready_off = 0;
    if (sctl_off) *sctl_off = 0;
    if (stream_shape(B, H, Dk, Dv, chunk, io == IoType::F32 ? KDA_DTYPE_F32 : KDA_DTYPE_BF16)) {
        if (ready_off) *ready_off = n;
        n += ((size_t)B * H * sh.NC * 4 + 255) & ~size_t(255);
        if (sctl_off) *sctl_off = n;
        n += sizeof(kda::StreamCtl);
    }
    return n;
}

// prologue parameters inside the mode's ranges (KDA: gates in [0, 1], beta in
// [0, 1]; CKDA: gates in [-1, 1], beta in [0, 2]), finite, eps >= 0
bool prologue_ok(const kda_prologue_t& p, kda_mode_t mode)
{
    const float lo = mode == KDA_MODE_CKDA ? -1.f : 0.f, bhi = mode == KDA_MODE_CKDA ? 2.f : 1.f;
    return p.alpha_min >= lo && p.alpha_min <= p.alpha_max && p.alpha_max <= 1.f &&
           p.beta_max >= 0.f && p.beta_max <= bhi && p.eps >= 0.f && p.eps < 1e30f &&
           (p.normalize_q == 0 || p.normalize_q == 1);
}

// KDA_FLAG_VALIDATE_RANGES: the device range check (synchronises the stream),
// run once the arguments are validated and before any work is enqueued
kda_status_t validate_ranges(unsigned flags, kda_mode_t mode, const float* alpha, size_t na,
                             const float* beta, size_t nb, const float* theta, size_t nt,
                             hipStream_t s)
{
    if (!(flags & KDA_FLAG_VALIDATE_RANGES)) return KDA_OK;
    switch (kda::check_ranges(alpha, na, beta, nb, theta, nt, mode == KDA_MODE_CKDA, s)) {
    case kda::RangeResult::InRange: return KDA_OK;
    case kda::RangeResult::OutOfRange: return KDA_ERR_RANGE;
    case kda::RangeResult::Capturing: return KDA_ERR_UNSUPPORTED;
    default: return KDA_ERR_HIP;
    }
}

// the chunked forward; chunk_states (may be null) receives the state entering
// every chunk; pro (may be null) makes alpha / beta logits and q, k raw
kda_status_t chunk_forward(const void* q, const void* k, const void* v, const float* alpha,
                           const float* beta, const float* initial_state, void* out,
                           float* final_state, void* chunk_states, const kda_prologue_t* pro,
                           int B, int T, int H, int Dk, int Dv, int chunk, kda_dtype_t dtype,
                           kda_mode_t mode, unsigned flags, void* workspace,
                           size_t workspace_bytes, void* stream, const float* theta = nullptr,
                           const kda_side_t* side = nullptr)
{
    kda_status_t st = check_forward_shape(B, T, H, Dk, Dv, chunk, dtype);
    if (st != KDA_OK) return st;
    if (mode != KDA_MODE_KDA && mode != KDA_MODE_CKDA) return KDA_ERR_UNSUPPORTED;
    if (flags & ~kKnownFlags) return KDA_ERR_UNSUPPORTED;
    if (T > 0 && (!q || !k || !v || !alpha || !beta || !out)) return KDA_ERR_NULL_POINTER;
    if (pro && !prologue_ok(*pro, mode)) return KDA_ERR_UNSUPPORTED;
    if (pro && theta) return KDA_ERR_UNSUPPORTED;
    if (side) {
        if (!side->stream) return KDA_ERR_NULL_POINTER;
        for (int i = 0; i < KDA_SIDE_EVENTS; ++i)
            if (!side->events[i]) return KDA_ERR_NULL_POINTER;
    }

    const size_t e = elem_size(dtype);
    const size_t ntok = (size_t)B * T * H;
    const size_t na = theta ? (size_t)Dk / 2 : (size_t)Dk;     // gates per token
    const size_t nstate = (size_t)B * H * Dk * Dv * 4;
    size_t ws_need = 0;
    kda_chunk_forward_workspace_size(B, T, H, Dk, Dv, chunk, dtype, &ws_need);
    if (T > 0 && !workspace) return KDA_ERR_NULL_POINTER;
    if (workspace_bytes < ws_need) return KDA_ERR_WORKSPACE_TOO_SMALL;

    // q, k, alpha and the workspace are read with 16-byte vector loads; the rest
    // element by element
    const void* vec[] = {q, k, theta ? nullptr : alpha, workspace};
    for (const void* p : vec)
        if (p && !aligned16(p)) return KDA_ERR_MISALIGNED;
    // (phase variant: alpha and theta are read as pairs of floats)
    const void* elt[] = {v, out, beta, initial_state, final_state, chunk_states,
                         theta ? alpha : nullptr, theta};
    const uintptr_t ea[] = {e, e, 4, 4, 4, e, 8, 8};
    for (int i = 0; i < 8; ++i)
        if (elt[i] && !aligned(elt[i], ea[i])) return KDA_ERR_MISALIGNED;

    // aliasing: out, workspace and chunk_states overlap nothing; final_state
    // may equal initial_state exactly but overlap nothing else
    const size_t ncs = chunk_states ? (size_t)B * H * ((T + chunk - 1) / chunk) * Dk * Dv * e : 0;
    struct R { const void* p; size_t n; } in[] = {
        {q, ntok * Dk * e}, {k, ntok * Dk * e}, {v, ntok * Dv * e},
        {alpha, ntok * na * 4}, {beta, ntok * 4}, {initial_state, initial_state ? nstate : 0},
        {theta, theta ? ntok * na * 4 : 0}};
    const R outs[] = {{out, ntok * Dv * e}, {workspace, ws_need}, {chunk_states, ncs}};
    for (const R& o : outs)
        for (const R& i : in)
            if (overlaps(o.p, o.n, i.p, i.n)) return KDA_ERR_ALIAS;
    for (int x = 0; x < 3; ++x)
        for (int y = x + 1; y < 3; ++y)
            if (overlaps(outs[x].p, outs[x].n, outs[y].p, outs[y].n)) return KDA_ERR_ALIAS;
    if (final_state) {
        const R fs{final_state, nstate};
        for (const R& i : in) {
            if (i.p == initial_state && final_state == initial_state) continue;
            if (overlaps(fs.p, fs.n, i.p, i.n)) return KDA_ERR_ALIAS;
        }
        for (const R& o : outs)
            if (overlaps(fs.p, fs.n, o.p, o.n)) return KDA_ERR_ALIAS;
    }

    // ---- validated: enqueue ------------------------------------------------------
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!pro && T > 0) {    // (with a prologue the ranges hold by construction)
        st = validate_ranges(flags, mode, alpha, ntok * na, beta, ntok, theta,
                             theta ? ntok * na : 0, s);
        if (st != KDA_OK) return st;
    }
    std::unique_lock<std::mutex> lock(g_stage.mu, std::defer_lock);
    Recorder rec{(flags & KDA_FLAG_STAGE_EVENTS) != 0, s};
    if (rec.on) {
        lock.lock();
        if (stage_begin() != hipSuccess) return KDA_ERR_HIP;
    }
    if (T == 0) {
        if (!final_state || final_state == initial_state) return KDA_OK;
        if (rec.mark("state_copy") != hipSuccess) return KDA_ERR_HIP;
        if (kda::launch_state_copy(initial_state, final_state, nstate / 4, s) != hipSuccess)
            return KDA_ERR_HIP;
        return rec.done() == hipSuccess ? KDA_OK : KDA_ERR_HIP;
    }

    const ChunkShape sh = make_shape(B, T, H, Dk, Dv, chunk);
    const IoType io = dtype == KDA_DTYPE_F32 ? IoType::F32 : IoType::BF16;
    size_t off[kda::kWorkspaceRegions];
    kda::chunk_workspace_layout(sh, io, off);
    unsigned char* w = static_cast<unsigned char*>(workspace);
    const ChunkWorkspace ws{w + off[0], w + off[1], w + off[2],
                            w + off[3], w + off[4], reinterpret_cast<float*>(w + off[5]),
                            w + off[6]};
    const int zx = fast_zero_columns(mode, Dk);
    kda::PrepArgs pa{q, k, v, alpha, beta, ws.W, ws.U, ws.Kt, ws.QG, ws.P, ws.GC, ws.FL,
                           T, H, Dv, sh.NC, zx,
                           pro ? 1 : 0,
                           pro ? pro->alpha_min : 0.f,
                           pro ? pro->alpha_max - pro->alpha_min : 0.f,
                           pro ? pro->beta_max : 0.f,
                           pro ? pro->eps : 0.f,
                           pro ? pro->normalize_q : 0,
                           nullptr, nullptr, 0, theta};
    pa.ntst = workspace_nt((long long)B * H * (Dv / 16));
    const Segments sgm = (flags & KDA_FLAG_NO_SEGMENTS) ? Segments{1, sh.NC}
                                                          : segments_for(B, H, Dk, Dv, sh.NC, dtype);
    const Parts prt = (!side || sgm.nseg > 1 || (flags & KDA_FLAG_SINGLE_STREAM))
                          ? Parts{1, sh.NC} : parts_for(B, H, Dk, Dv, sh.NC);
    size_t so = 0, ss = 0, sp = 0;
    if (sgm.nseg > 1 || prt.parts > 1) {
        size_t off2[kda::kWorkspaceRegions];
        dense_layout(B, T, H, Dk, Dv, chunk, io, off2, &so, &ss, &sp);
    }
    float* summ = sgm.nseg > 1 ? reinterpret_cast<float*>(w + so) : nullptr;
    float* sseg = sgm.nseg > 1 ? reinterpret_cast<float*>(w + ss) : nullptr;
    const kda::ChainArgs ca{ws.W, ws.U, ws.Kt, ws.QG, ws.P, ws.GC, initial_state, out,
                            final_state, chunk_states, B, T, H, Dv, sh.NC, nullptr, nullptr,
                            theta ? 1 : 0, sgm.seg, sgm.nseg, nullptr, sseg};

    // the caller's second stream takes part in the call only when it belongs to
    // the same device as `stream` (else the call keeps to `stream`)
    // (streamed: not from the null stream, which waits for the work of every
    // blocking stream, a side stream made by kda_side_stream_create included)
    const bool streamed = side && s && (flags & KDA_FLAG_STREAMED) &&
                          !(flags & KDA_FLAG_SINGLE_STREAM) && !pro && !theta &&
                          !chunk_states && !(final_state && final_state == initial_state) &&
                          sgm.nseg == 1 && stream_shape(B, H, Dk, Dv, chunk, dtype);
    bool use_side = prt.parts > 1 || streamed;
    hipDevice_t d0 = 0;
    if (use_side) {
        hipDevice_t d1 = 0;
        if (s) {
            if (hipStreamGetDevice(s, &d0) != hipSuccess) return KDA_ERR_HIP;
        } else {
            int cur = 0;
            if (hipGetDevice(&cur) != hipSuccess) return KDA_ERR_HIP;
            d0 = cur;
        }
        if (hipStreamGetDevice(static_cast<hipStream_t>(side->stream), &d1) != hipSuccess)
            return KDA_ERR_HIP;
        use_side = d0 == d1;
    }
    if (use_side && streamed) {
        // prep grid on the side stream and the chain on `stream` at the same
        // time; then, on `stream`, the exact kernel for flagged units and a
        // fallback chain that runs only if the streamed one gave up
        hipStream_t ss = static_cast<hipStream_t>(side->stream);
        hipEvent_t ev0 = static_cast<hipEvent_t>(side->events[0]);
        hipEvent_t ev1 = static_cast<hipEvent_t>(side->events[1]);
        size_t offs[kda::kWorkspaceRegions], a0, a1, a2, roff = 0, coff = 0;
        dense_layout(B, T, H, Dk, Dv, chunk, io, offs, &a0, &a1, &a2, &roff, &coff);
        unsigned* ready = reinterpret_cast<unsigned*>(w + roff);
        kda::StreamCtl* ctl = reinterpret_cast<kda::StreamCtl*>(w + coff);
        int ncu = 0;
        if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, d0) != hipSuccess)
            return KDA_ERR_HIP;
        const int ct = stream_pick_tiles(B, H, Dk, Dv, sh.NC, zx > 0, ncu);   // (>= 1: stream_shape)
        const long long bhn = (long long)B * H;
        const int nsl = Dv / (16 * ct);
        kda::PrepArgs ps = pa;
        ps.ntst = 0;
        ps.nbh = (int)bhn;
        ps.ready = ready;
        ps.sctl = ctl;
        ps.lead = stream_lead(bhn, Dk, Dv, chunk, 2);
        kda::ChainArgs cst = ca;
        cst.ready = ready;
        cst.sctl = ctl;
        if (rec.mark("stream_clear") != hipSuccess) return KDA_ERR_HIP;
        if (kda::launch_stream_clear(ready, (size_t)bhn * sh.NC, ctl, (unsigned)(bhn * nsl),
                                     (unsigned)ct, s) !=
            hipSuccess)
            return KDA_ERR_HIP;
        if (rec.done() != hipSuccess) return KDA_ERR_HIP;
        if (hipEventRecord(ev0, s) != hipSuccess) return KDA_ERR_HIP;
        if (rec.mark("chain_stream") != hipSuccess) return KDA_ERR_HIP;
        if (kda::launch_chain_stream(io, sh, cst, ct, s) != hipSuccess) return KDA_ERR_HIP;
        if (rec.done() != hipSuccess) return KDA_ERR_HIP;
        if (hipStreamWaitEvent(ss, ev0, 0) != hipSuccess) return KDA_ERR_HIP;
        if (rec.mark("prep_stream") != hipSuccess) return KDA_ERR_HIP;
        if (kda::launch_prep_stream(io, sh, ps, ss) != hipSuccess) return KDA_ERR_HIP;
        if (rec.done() != hipSuccess) return KDA_ERR_HIP;
        if (hipEventRecord(ev1, ss) != hipSuccess) return KDA_ERR_HIP;
        if (hipStreamWaitEvent(s, ev1, 0) != hipSuccess) return KDA_ERR_HIP;
        if (rec.mark("prep_exact") != hipSuccess) return KDA_ERR_HIP;
        if (kda::launch_prep_exact(io, sh, pa, s) != hipSuccess) return KDA_ERR_HIP;
        if (rec.done() != hipSuccess) return KDA_ERR_HIP;
        kda::ChainArgs cf = ca;
        cf.gate = ctl;
        if (rec.mark("chain") != hipSuccess) return KDA_ERR_HIP;
        if (launch_forward_chain(io, sh, cf, s) != hipSuccess) return KDA_ERR_HIP;
        if (rec.done() != hipSuccess) return KDA_ERR_HIP;
        return KDA_OK;
    }
    if (use_side) {
        // prep of every part on the side stream, chain of part p on the
        // caller's stream after the prep of part p; the state between parts
        // lives in the workspace (each chain workgroup reads its slice before
        // writing it back)
        hipStream_t ss = static_cast<hipStream_t>(side->stream);
        hipEvent_t ev[KDA_SIDE_EVENTS];
        for (int i = 0; i < KDA_SIDE_EVENTS; ++i) ev[i] = static_cast<hipEvent_t>(side->events[i]);
        float* spart = reinterpret_cast<float*>(w + sp);
        if (hipEventRecord(ev[0], s) != hipSuccess) return KDA_ERR_HIP;
        if (hipStreamWaitEvent(ss, ev[0], 0) != hipSuccess) return KDA_ERR_HIP;
        for (int p = 0; p < prt.parts; ++p) {
            kda::PrepArgs pp = pa;
            pp.pc0 = p * prt.len;
            pp.pcn = std::min(prt.len, sh.NC - pp.pc0);
            if (rec.mark("prep_fast") != hipSuccess) return KDA_ERR_HIP;
            if (kda::launch_prep_fast(io, sh, pp, ss) != hipSuccess) return KDA_ERR_HIP;
            if (rec.done() != hipSuccess) return KDA_ERR_HIP;
            if (rec.mark("prep_exact") != hipSuccess) return KDA_ERR_HIP;
            if (kda::launch_prep_exact(io, sh, pp, ss) != hipSuccess) return KDA_ERR_HIP;
            if (rec.done() != hipSuccess) return KDA_ERR_HIP;
            if (hipEventRecord(ev[p + 1], ss) != hipSuccess) return KDA_ERR_HIP;
        }
        for (int p = 0; p < prt.parts; ++p) {
            kda::ChainArgs cp = ca;
            cp.pc0 = p * prt.len;
            cp.pcn = std::min(prt.len, sh.NC - cp.pc0);
            cp.S0 = p == 0 ? initial_state : spart;
            cp.ST = p == prt.parts - 1 ? final_state : spart;
            if (hipStreamWaitEvent(s, ev[p + 1], 0) != hipSuccess) return KDA_ERR_HIP;
            if (rec.mark("chain") != hipSuccess) return KDA_ERR_HIP;
            if (launch_forward_chain(io, sh, cp, s) != hipSuccess) return KDA_ERR_HIP;
            if (rec.done() != hipSuccess) return KDA_ERR_HIP;
        }
        return KDA_OK;
    }

    if (rec.mark("prep_fast") != hipSuccess) return KDA_ERR_HIP;
    if (kda::launch_prep_fast(io, sh, pa, s) != hipSuccess) return KDA_ERR_HIP;
    if (rec.done() != hipSuccess) return KDA_ERR_HIP;
    if (rec.mark("prep_exact") != hipSuccess) return KDA_ERR_HIP;
    if (kda::launch_prep_exact(io, sh, pa, s) != hipSuccess) return KDA_ERR_HIP;
    if (rec.done() != hipSuccess) return KDA_ERR_HIP;
    if (sgm.nseg > 1) {
        // segment maps, then the segment start states, then every segment
        kda::ChainArgs cs = ca;
        cs.S0 = nullptr;
        cs.out = nullptr;
        cs.ST = nullptr;
        cs.CS = nullptr;
        cs.summ = summ;
        if (rec.mark("chain_summary") != hipSuccess) return KDA_ERR_HIP;
        if (kda::launch_chain(io, sh, cs, s) != hipSuccess) return KDA_ERR_HIP;
        if (rec.done() != hipSuccess) return KDA_ERR_HIP;
        if (rec.mark("segment_combine") != hipSuccess) return KDA_ERR_HIP;
        if (kda::launch_segment_combine(B * H, Dk, Dv, sgm.nseg, initial_state, summ, sseg, s) !=
            hipSuccess)
            return KDA_ERR_HIP;
        if (rec.done() != hipSuccess) return KDA_ERR_HIP;
    }
    if (rec.mark("chain") != hipSuccess) return KDA_ERR_HIP;
    if (launch_forward_chain(io, sh, ca, s) != hipSuccess) return KDA_ERR_HIP;
    if (rec.done() != hipSuccess) return KDA_ERR_HIP;
    return KDA_OK;
}

// packed batches: an upper bound of the chunk count (each sequence adds at most
// one partial chunk), the shape the prep kernels and the workspace use
// (B = 1, NC = that bound), and the tables after the per-unit regions
long long varlen_max_chunks(int N, int total_T, int chunk)
{
    return ((long long)total_T + chunk - 1) / chunk + N;
}

kda_status_t check_varlen_shape(int N, int total_T, int H, int Dk, int Dv, int chunk,
                                kda_dtype_t dtype)
{
    if (N < 1 || N > (1 << 24) || total_T < 0 || H < 1) return KDA_ERR_BAD_SHAPE;
    const kda_status_t st = check_forward_shape(1, total_T, H, Dk, Dv, chunk, dtype);
    if (st != KDA_OK) return st;
    const long long umax = varlen_max_chunks(N, total_T, chunk);
    if (umax * H > 0x7fffffffLL || (long long)N * H * (Dv / 16) > 0x7fffffffLL) return KDA_ERR_BAD_SHAPE;
    return KDA_OK;
}

size_t varlen_layout(int N, int total_T, int H, int Dk, int Dv, int chunk, IoType io,
                     size_t off[kda::kWorkspaceRegions], size_t* table_off)
{
    const int umax = (int)varlen_max_chunks(N, total_T, chunk);
    const size_t units = kda::chunk_workspace_layout(ChunkShape{1, total_T, H, Dk, Dv, chunk, umax},
                                                     io, off);
    *table_off = units;
    return units + ((2 * ((size_t)N + 1) * sizeof(int) + 255) & ~size_t(255));
}

// one token per (b, h); theta (may be null) selects the phase variant, whose
// alpha and theta hold one value per channel pair
kda_status_t decode_step(const void* q, const void* k, const void* v, const float* alpha,
                         const float* theta, const float* beta, float* state, void* out, int B,
                         int H, int Dk, int Dv, kda_dtype_t dtype, kda_mode_t mode,
                         unsigned flags, void* stream, const kda_prologue_t* pro = nullptr)
{
    if (B < 1 || H < 1) return KDA_ERR_BAD_SHAPE;
    if (dtype != KDA_DTYPE_F32 && dtype != KDA_DTYPE_BF16) return KDA_ERR_UNSUPPORTED;
    if (!dk_ok(Dk) || !dv_ok(Dv)) return KDA_ERR_UNSUPPORTED;
    if (mode != KDA_MODE_KDA && mode != KDA_MODE_CKDA) return KDA_ERR_UNSUPPORTED;
    if (flags & ~kKnownFlags) return KDA_ERR_UNSUPPORTED;
    if ((long long)B * H > 0x7fffffffLL) return KDA_ERR_BAD_SHAPE;
    if (!q || !k || !v || !alpha || !beta || !state || !out) return KDA_ERR_NULL_POINTER;
    if (pro && !prologue_ok(*pro, mode)) return KDA_ERR_UNSUPPORTED;
    const size_t e = elem_size(dtype), nbh = (size_t)B * H;
    // the state is streamed with 16-byte vectors; everything else element-wise
    if (!aligned16(state)) return KDA_ERR_MISALIGNED;
    const size_t na = theta ? (size_t)Dk / 2 : (size_t)Dk;
    const void* elt[] = {q, k, v, out, alpha, beta, theta};
    const uintptr_t ea[] = {e, e, e, e, 4, 4, 4};
    for (int i = 0; i < 7; ++i)
        if (elt[i] && !aligned(elt[i], ea[i])) return KDA_ERR_MISALIGNED;
    struct R { const void* p; size_t n; } in[] = {
        {q, nbh * Dk * e}, {k, nbh * Dk * e}, {v, nbh * Dv * e}, {alpha, nbh * na * 4},
        {beta, nbh * 4}, {theta, theta ? nbh * na * 4 : 0}};
    const R st{state, nbh * Dk * Dv * 4}, o{out, nbh * Dv * e};
    for (const R& i : in)
        if (overlaps(st.p, st.n, i.p, i.n) || overlaps(o.p, o.n, i.p, i.n)) return KDA_ERR_ALIAS;
    if (overlaps(st.p, st.n, o.p, o.n)) return KDA_ERR_ALIAS;

    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!pro) {
        const kda_status_t vr = validate_ranges(flags, mode, alpha, nbh * na, beta, nbh, theta,
                                                theta ? nbh * na : 0, s);
        if (vr != KDA_OK) return vr;
    }
    std::unique_lock<std::mutex> lock(g_stage.mu, std::defer_lock);
    Recorder rec{(flags & KDA_FLAG_STAGE_EVENTS) != 0, s};
    if (rec.on) {
        lock.lock();
        if (stage_begin() != hipSuccess) return KDA_ERR_HIP;
    }
    if (rec.mark("decode") != hipSuccess) return KDA_ERR_HIP;
    kda::DecodePro dp{};
    if (pro)
        dp = kda::DecodePro{pro->alpha_min, pro->alpha_max - pro->alpha_min, pro->beta_max, pro->eps,
                            pro->normalize_q};
    if (kda::launch_decode(dtype == KDA_DTYPE_F32 ? IoType::F32 : IoType::BF16, B, H, Dk, Dv, q, k,
                           v, alpha, beta, state, out, s, theta, pro ? &dp : nullptr) != hipSuccess)
        return KDA_ERR_HIP;
    return rec.done() == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

// ---- backward ----------------------------------------------------------------
// workspace: the forward's per-unit regions, then Tinv [NU][C][C], the fp32
// chunk states [NU][Dk][Dv], Delta [NU][C][Dv], the state gradients
// [NU][Dk][Dv], X / y [NU][C][Dv] (all fp32) and the small-gate flags [NU]
constexpr int kBwdRegions = 6;
size_t backward_layout_sh(const ChunkShape& sh, IoType io, size_t off[kda::kWorkspaceRegions],
                          size_t boff[kBwdRegions])
{
    const size_t chunk = sh.C, Dk = sh.Dk, Dv = sh.Dv;
    size_t n = kda::chunk_workspace_layout(sh, io, off);
    const size_t nu = (size_t)sh.B * sh.H * sh.NC;
    const size_t sz[kBwdRegions] = {nu * chunk * chunk * 4, nu * Dk * Dv * 4, nu * chunk * Dv * 4,
                                    nu * Dk * Dv * 4, nu * chunk * Dv * 4, nu};
    for (int i = 0; i < kBwdRegions; ++i) {
        boff[i] = n;
        n += (sz[i] + 255) & ~size_t(255);
    }
    return n;
}

size_t backward_layout(int B, int T, int H, int Dk, int Dv, int chunk, IoType io,
                       size_t off[kda::kWorkspaceRegions], size_t boff[kBwdRegions])
{
    return backward_layout_sh(make_shape(B, T, H, Dk, Dv, chunk), io, off, boff);
}

// packed batches: the per-unit regions for the chunk-count bound, then the
// sanitised tables (cu_s, cs: 2 (N + 1) ints)
size_t backward_varlen_layout(int N, int total_T, int H, int Dk, int Dv, int chunk, IoType io,
                              size_t off[kda::kWorkspaceRegions], size_t boff[kBwdRegions],
                              size_t* table_off)
{
    const int umax = (int)varlen_max_chunks(N, total_T, chunk);
    const size_t n = backward_layout_sh(ChunkShape{1, total_T, H, Dk, Dv, chunk, umax}, io, off, boff);
    *table_off = n;
    return n + ((2 * ((size_t)N + 1) * sizeof(int) + 255) & ~size_t(255));
}

// which part of the backward's work a call enqueues: all of it; the forward
// pass that leaves its saved state in the workspace (with the forward's
// outputs); or the gradient pass from such a workspace
enum class BwdPart { ALL, SAVE, FROM_SAVED };

kda_status_t backward_enqueue(const void* q, const void* k, const void* v, const float* alpha,
                              const float* beta, const float* initial_state, const void* d_out,
                              const float* d_final_state, void* dq, void* dk, void* dv,
                              float* d_alpha, float* d_beta, float* d_initial_state, int B, int T,
                              int H, int Dk, int Dv, int chunk, kda_dtype_t dtype, kda_mode_t mode,
                              void* workspace, Recorder& rec, hipStream_t s,
                              const int* cu_seqlens = nullptr, BwdPart part = BwdPart::ALL,
                              void* out = nullptr, float* final_state = nullptr);

kda_status_t check_backward_shape(int B, int T, int H, int Dk, int Dv, int chunk,
                                  kda_dtype_t dtype)
{
    const kda_status_t st = check_forward_shape(B, T, H, Dk, Dv, chunk, dtype);
    if (st != KDA_OK) return st;
    if (chunk != 32 && chunk != 64) return KDA_ERR_UNSUPPORTED;
    if (Dk != 32 && Dk != 64 && Dk != 128) return KDA_ERR_UNSUPPORTED;
    if (dtype == KDA_DTYPE_F32 && (Dk > 64 || Dv > 64)) return KDA_ERR_UNSUPPORTED;
    return KDA_OK;
}

// The backward, or one part of it (BwdPart): argument checks, then the enqueue.
// SAVE takes no gradient arguments and writes out / final_state; FROM_SAVED
// takes no initial_state (the saved chunk states hold it).
kda_status_t chunk_backward_part(const void* q, const void* k, const void* v, const float* alpha,
                                 const float* beta, const float* initial_state, const void* d_out,
                                 const float* d_final_state, void* dq, void* dk, void* dv,
                                 float* d_alpha, float* d_beta, float* d_initial_state, int B,
                                 int T, int H, int Dk, int Dv, int chunk, kda_dtype_t dtype,
                                 kda_mode_t mode, unsigned flags, void* workspace,
                                 size_t workspace_bytes, void* stream, BwdPart part,
                                 void* out = nullptr, float* final_state = nullptr)
{
    kda_status_t st = check_backward_shape(B, T, H, Dk, Dv, chunk, dtype);
    if (st != KDA_OK) return st;
    if (mode != KDA_MODE_KDA && mode != KDA_MODE_CKDA) return KDA_ERR_UNSUPPORTED;
    if (flags & ~KDA_FLAG_STAGE_EVENTS) return KDA_ERR_UNSUPPORTED;
    const bool grads = part != BwdPart::SAVE;
    if (T > 0 && (!q || !k || !v || !alpha || !beta))
        return KDA_ERR_NULL_POINTER;
    if (T > 0 && grads && (!d_out || !dq || !dk || !dv || !d_alpha || !d_beta))
        return KDA_ERR_NULL_POINTER;
    if (T > 0 && !grads && !out) return KDA_ERR_NULL_POINTER;
    size_t ws_need = 0;
    kda_chunk_backward_workspace_size(B, T, H, Dk, Dv, chunk, dtype, &ws_need);
    if (T > 0 && !workspace) return KDA_ERR_NULL_POINTER;
    if (workspace_bytes < ws_need) return KDA_ERR_WORKSPACE_TOO_SMALL;

    const size_t e = elem_size(dtype);
    const size_t ntok = (size_t)B * T * H;
    const size_t nstate = (size_t)B * H * Dk * Dv * 4;
    const void* vec[] = {q, k, d_out, alpha, workspace};
    for (const void* p : vec)
        if (p && !aligned16(p)) return KDA_ERR_MISALIGNED;
    const void* elt[] = {v, beta, initial_state, d_final_state, dq, dk, dv, d_alpha, d_beta,
                         d_initial_state, out, final_state};
    const uintptr_t ea[] = {e, 4, 4, 4, e, e, e, 4, 4, 4, e, 4};
    for (int i = 0; i < 12; ++i)
        if (elt[i] && !aligned(elt[i], ea[i])) return KDA_ERR_MISALIGNED;
    struct R { const void* p; size_t n; };
    const R in[] = {{q, ntok * Dk * e}, {k, ntok * Dk * e}, {v, ntok * Dv * e},
                    {alpha, ntok * Dk * 4}, {beta, ntok * 4},
                    {initial_state, initial_state ? nstate : 0}, {d_out, d_out ? ntok * Dv * e : 0},
                    {d_final_state, d_final_state ? nstate : 0}};
    const R outs[] = {{dq, dq ? ntok * Dk * e : 0}, {dk, dk ? ntok * Dk * e : 0},
                      {dv, dv ? ntok * Dv * e : 0}, {d_alpha, d_alpha ? ntok * Dk * 4 : 0},
                      {d_beta, d_beta ? ntok * 4 : 0},
                      {d_initial_state, d_initial_state ? nstate : 0}, {workspace, ws_need},
                      {out, out ? ntok * Dv * e : 0}, {final_state, final_state ? nstate : 0}};
    constexpr int NO = sizeof(outs) / sizeof(outs[0]);
    for (const R& o : outs)
        for (const R& i : in)
            if (overlaps(o.p, o.n, i.p, i.n)) return KDA_ERR_ALIAS;
    for (int x = 0; x < NO; ++x)
        for (int y = x + 1; y < NO; ++y)
            if (overlaps(outs[x].p, outs[x].n, outs[y].p, outs[y].n)) return KDA_ERR_ALIAS;

    hipStream_t s = static_cast<hipStream_t>(stream);
    std::unique_lock<std::mutex> lock(g_stage.mu, std::defer_lock);
    Recorder rec{(flags & KDA_FLAG_STAGE_EVENTS) != 0, s};
    if (rec.on) {
        lock.lock();
        if (stage_begin() != hipSuccess) return KDA_ERR_HIP;
    }
    return backward_enqueue(q, k, v, alpha, beta, part == BwdPart::FROM_SAVED ? nullptr : initial_state,
                            d_out, d_final_state, dq, dk, dv, d_alpha, d_beta, d_initial_state, B,
                            T, H, Dk, Dv, chunk, dtype, mode, workspace, rec, s, nullptr, part, out,
                            final_state);
}

kda_status_t chunk_backward(const void* q, const void* k, const void* v, const float* alpha,
                            const float* beta, const float* initial_state, const void* d_out,
                            const float* d_final_state, void* dq, void* dk, void* dv,
                            float* d_alpha, float* d_beta, float* d_initial_state, int B, int T,
                            int H, int Dk, int Dv, int chunk, kda_dtype_t dtype, kda_mode_t mode,
                            unsigned flags, void* workspace, size_t workspace_bytes, void* stream)
{
    return chunk_backward_part(q, k, v, alpha, beta, initial_state, d_out, d_final_state, dq, dk,
                               dv, d_alpha, d_beta, d_initial_state, B, T, H, Dk, Dv, chunk, dtype,
                               mode, flags, workspace, workspace_bytes, stream, BwdPart::ALL);
}

// the backward's launches (arguments validated by the caller, stage events
// through rec); with cu_seqlens (device, B + 1 offsets) the batch is packed:
// B sequences over T tokens in total
kda_status_t backward_enqueue(const void* q, const void* k, const void* v, const float* alpha,
                              const float* beta, const float* initial_state, const void* d_out,
                              const float* d_final_state, void* dq, void* dk, void* dv,
                              float* d_alpha, float* d_beta, float* d_initial_state, int B, int T,
                              int H, int Dk, int Dv, int chunk, kda_dtype_t dtype, kda_mode_t mode,
                              void* workspace, Recorder& rec, hipStream_t s, const int* cu_seqlens,
                              BwdPart part, void* out, float* final_state)
{
    const size_t nstate = (size_t)B * H * Dk * Dv * 4;
    if (T == 0 && part == BwdPart::SAVE) {
        // no tokens: the final state is the initial one
        if (!final_state) return KDA_OK;
        if (rec.mark("state_copy") != hipSuccess) return KDA_ERR_HIP;
        if (kda::launch_state_copy(initial_state, final_state, nstate / 4, s) != hipSuccess)
            return KDA_ERR_HIP;
        return rec.done() == hipSuccess ? KDA_OK : KDA_ERR_HIP;
    }
    if (T == 0) {
        // no tokens: the loss is <S0, dST>, so dS0 = dST
        if (!d_initial_state) return KDA_OK;
        if (rec.mark("state_copy") != hipSuccess) return KDA_ERR_HIP;
        if (d_final_state) {
            if (kda::launch_state_copy(d_final_state, d_initial_state, nstate / 4, s) != hipSuccess)
                return KDA_ERR_HIP;
        } else if (kda::launch_state_copy(nullptr, d_initial_state, nstate / 4, s) != hipSuccess) {
            return KDA_ERR_HIP;
        }
        return rec.done() == hipSuccess ? KDA_OK : KDA_ERR_HIP;
    }

    const IoType io = dtype == KDA_DTYPE_F32 ? IoType::F32 : IoType::BF16;
    size_t off[kda::kWorkspaceRegions], boff[kBwdRegions];
    unsigned char* w = static_cast<unsigned char*>(workspace);
    // dense: units and chains from (B, T); packed: all units of the chunk-count
    // bound (shp) and B x H chains (shc), located through the tables
    ChunkShape shp = make_shape(B, T, H, Dk, Dv, chunk), shc = shp;
    int* cu_s = nullptr;
    int* cs = nullptr;
    if (cu_seqlens) {
        size_t toff = 0;
        backward_varlen_layout(B, T, H, Dk, Dv, chunk, io, off, boff, &toff);
        const int umax = (int)varlen_max_chunks(B, T, chunk);
        shp = ChunkShape{1, T, H, Dk, Dv, chunk, umax};
        shc = ChunkShape{B, T, H, Dk, Dv, chunk, umax};
        cu_s = reinterpret_cast<int*>(w + toff);
        cs = cu_s + (B + 1);
        if (rec.mark("varlen_table") != hipSuccess) return KDA_ERR_HIP;
        if (kda::launch_varlen_table(cu_seqlens, B, T, chunk, umax, cu_s, cs, s) != hipSuccess)
            return KDA_ERR_HIP;
        if (rec.done() != hipSuccess) return KDA_ERR_HIP;
    } else {
        backward_layout(B, T, H, Dk, Dv, chunk, io, off, boff);
    }
    const ChunkShape& sh = shp;
    const ChunkWorkspace ws{w + off[0], w + off[1], w + off[2],
                            w + off[3], w + off[4], reinterpret_cast<float*>(w + off[5]),
                            w + off[6]};
    float* Tm = reinterpret_cast<float*>(w + boff[0]);
    float* CS32 = reinterpret_cast<float*>(w + boff[1]);
    float* DL = reinterpret_cast<float*>(w + boff[2]);
    float* DSN = reinterpret_cast<float*>(w + boff[3]);
    float* XB = reinterpret_cast<float*>(w + boff[4]);
    uint8_t* FLB = w + boff[5];
    const int zx = fast_zero_columns(mode, Dk);
    kda::PrepArgs pa{q, k, v, alpha, beta, ws.W, ws.U, ws.Kt, ws.QG, ws.P, ws.GC, ws.FL,
                     T, H, Dv, sh.NC, zx, 0, 0.f, 0.f, 0.f, 0.f, 0,
                     cu_s, cs, cu_seqlens ? B : 0, nullptr};
    pa.ntst = workspace_nt((long long)B * H * (Dv / 16));
    pa.Tm = Tm;
    kda::ChainArgs ca{ws.W, ws.U, ws.Kt, ws.QG, ws.P, ws.GC, initial_state, nullptr,
                      nullptr, nullptr, B, T, H, Dv, sh.NC, cu_s, cs,
                      0, sh.NC, 1, nullptr, nullptr};
    ca.CS32 = CS32;
    ca.DL = DL;
    // the chain's final state (S_T of the saving forward, or of the rotated
    // recurrence for the phase variant's backward)
    ca.ST = final_state;
    if (part == BwdPart::SAVE) ca.out = out;
    const kda::BwdChainArgs ra{ws.Kt, ws.P, ws.QG, ws.W, ws.GC, d_out, d_final_state,
                               d_initial_state, DSN, XB, B, T, H, Dv, sh.NC, cu_s, cs};
    const kda::BwdLocalArgs la{q, k, v, alpha, beta, d_out, Tm, CS32, DL, DSN, XB,
                               dq, dk, dv, d_alpha, d_beta, FLB, T, H, Dv, sh.NC,
                               cu_s, cs, cu_seqlens ? B : 0};

    if (part != BwdPart::FROM_SAVED) {
        if (rec.mark("prep_fast") != hipSuccess) return KDA_ERR_HIP;
        if (kda::launch_prep_fast(io, sh, pa, s) != hipSuccess) return KDA_ERR_HIP;
        if (rec.done() != hipSuccess) return KDA_ERR_HIP;
        if (rec.mark("prep_exact") != hipSuccess) return KDA_ERR_HIP;
        if (kda::launch_prep_exact(io, sh, pa, s) != hipSuccess) return KDA_ERR_HIP;
        if (rec.done() != hipSuccess) return KDA_ERR_HIP;
        if (rec.mark("chain_states") != hipSuccess) return KDA_ERR_HIP;
        if (kda::launch_chain(io, shc, ca, s) != hipSuccess) return KDA_ERR_HIP;
        if (rec.done() != hipSuccess) return KDA_ERR_HIP;
    }
    if (part == BwdPart::SAVE) return KDA_OK;
    static const char* const names[4] = {"relayout", "chain_reverse", "chunk_grads", "small_gates"};
    for (int stage = 0; stage < 4; ++stage) {
        if (rec.mark(names[stage]) != hipSuccess) return KDA_ERR_HIP;
        if (kda::launch_backward_stage(stage, io, stage == 1 ? shc : shp, ws, ra, la, s) != hipSuccess)
            return KDA_ERR_HIP;
        if (rec.done() != hipSuccess) return KDA_ERR_HIP;
    }
    return KDA_OK;
}

// the backward from raw inputs: workspace = the backward's, then the
// transformed inputs q^, k^ (io type), alpha, beta (fp32) and the gradients
// dq^, dk^ (io type) of the transformed q, k
size_t backward_prologue_layout(int B, int T, int H, int Dk, int Dv, int chunk, IoType io,
                                size_t xo[6])
{
    size_t off[kda::kWorkspaceRegions], boff[kBwdRegions];
    size_t n = backward_layout(B, T, H, Dk, Dv, chunk, io, off, boff);
    const size_t ntok = (size_t)B * T * H, e = io == IoType::F32 ? 4 : 2;
    const size_t sz[6] = {ntok * Dk * e, ntok * Dk * e, ntok * Dk * 4, ntok * 4, ntok * Dk * e,
                          ntok * Dk * e};
    for (int i = 0; i < 6; ++i) {
        xo[i] = n;
        n += (sz[i] + 255) & ~size_t(255);
    }
    return n;
}

// the same six regions after a packed batch's backward workspace
size_t backward_varlen_prologue_layout(int N, int total_T, int H, int Dk, int Dv, int chunk,
                                       IoType io, size_t xo[6])
{
    size_t off[kda::kWorkspaceRegions], boff[kBwdRegions], toff = 0;
    size_t n = backward_varlen_layout(N, total_T, H, Dk, Dv, chunk, io, off, boff, &toff);
    const size_t ntok = (size_t)total_T * H, e = io == IoType::F32 ? 4 : 2;
    const size_t sz[6] = {ntok * Dk * e, ntok * Dk * e, ntok * Dk * 4, ntok * 4, ntok * Dk * e,
                          ntok * Dk * e};
    for (int i = 0; i < 6; ++i) {
        xo[i] = n;
        n += (sz[i] + 255) & ~size_t(255);
    }
    return n;
}

// raw-input backward of a dense batch, or of a packed batch when cu_seqlens
// is given (then B is ignored, N sequences share the T = total_T rows and the
// states are per sequence)
kda_status_t chunk_backward_prologue(const void* q_raw, const void* k_raw, const void* v,
                                     const float* gate, const float* beta_logit,
                                     const float* initial_state, const void* d_out,
                                     const float* d_final_state, const kda_prologue_t* pro,
                                     void* dq_raw, void* dk_raw, void* dv, float* d_gate,
                                     float* d_beta_logit, float* d_initial_state, int B, int T,
                                     int H, int Dk, int Dv, int chunk, kda_dtype_t dtype,
                                     kda_mode_t mode, unsigned flags, void* workspace,
                                     size_t workspace_bytes, void* stream,
                                     const int* cu_seqlens = nullptr, int N = 0)
{
    const bool packed = cu_seqlens != nullptr;
    kda_status_t st = packed ? check_varlen_shape(N, T, H, Dk, Dv, chunk, dtype) : KDA_OK;
    if (st != KDA_OK) return st;
    if (packed) B = 1;
    st = check_backward_shape(B, T, H, Dk, Dv, chunk, dtype);
    if (st != KDA_OK) return st;
    if (mode != KDA_MODE_KDA && mode != KDA_MODE_CKDA) return KDA_ERR_UNSUPPORTED;
    if (flags & ~KDA_FLAG_STAGE_EVENTS) return KDA_ERR_UNSUPPORTED;
    if (!pro) return KDA_ERR_NULL_POINTER;
    if (!prologue_ok(*pro, mode)) return KDA_ERR_UNSUPPORTED;
    if (T > 0 && (!q_raw || !k_raw || !v || !gate || !beta_logit || !d_out || !dq_raw || !dk_raw ||
                  !dv || !d_gate || !d_beta_logit))
        return KDA_ERR_NULL_POINTER;
    const IoType io = dtype == KDA_DTYPE_F32 ? IoType::F32 : IoType::BF16;
    size_t xo[6];
    const size_t ws_need = T == 0 ? 0
                         : packed ? backward_varlen_prologue_layout(N, T, H, Dk, Dv, chunk, io, xo)
                                  : backward_prologue_layout(B, T, H, Dk, Dv, chunk, io, xo);
    if (T > 0 && !workspace) return KDA_ERR_NULL_POINTER;
    if (workspace_bytes < ws_need) return KDA_ERR_WORKSPACE_TOO_SMALL;

    const size_t e = elem_size(dtype);
    const size_t ntok = (size_t)B * T * H;
    const size_t nstate = (size_t)(packed ? N : B) * H * Dk * Dv * 4;
    if (packed && !aligned(cu_seqlens, 4)) return KDA_ERR_MISALIGNED;
    const void* vec[] = {q_raw, k_raw, d_out, gate, workspace, dq_raw, dk_raw, d_gate};
    for (const void* p : vec)
        if (p && !aligned16(p)) return KDA_ERR_MISALIGNED;
    const void* elt[] = {v, beta_logit, initial_state, d_final_state, dv, d_beta_logit,
                         d_initial_state};
    const uintptr_t ea[] = {e, 4, 4, 4, e, 4, 4};
    for (int i = 0; i < 7; ++i)
        if (elt[i] && !aligned(elt[i], ea[i])) return KDA_ERR_MISALIGNED;
    struct R { const void* p; size_t n; };
    const R in[] = {{q_raw, ntok * Dk * e}, {k_raw, ntok * Dk * e}, {v, ntok * Dv * e},
                    {gate, ntok * Dk * 4}, {beta_logit, ntok * 4},
                    {initial_state, initial_state ? nstate : 0}, {d_out, ntok * Dv * e},
                    {d_final_state, d_final_state ? nstate : 0},
                    {cu_seqlens, packed ? ((size_t)N + 1) * 4 : 0}};
    const R outs[] = {{dq_raw, ntok * Dk * e}, {dk_raw, ntok * Dk * e}, {dv, ntok * Dv * e},
                      {d_gate, ntok * Dk * 4}, {d_beta_logit, ntok * 4},
                      {d_initial_state, d_initial_state ? nstate : 0}, {workspace, ws_need}};
    constexpr int NO = sizeof(outs) / sizeof(outs[0]);
    for (const R& o : outs)
        for (const R& i : in)
            if (overlaps(o.p, o.n, i.p, i.n)) return KDA_ERR_ALIAS;
    for (int x = 0; x < NO; ++x)
        for (int y = x + 1; y < NO; ++y)
            if (overlaps(outs[x].p, outs[x].n, outs[y].p, outs[y].n)) return KDA_ERR_ALIAS;

    hipStream_t s = static_cast<hipStream_t>(stream);
    std::unique_lock<std::mutex> lock(g_stage.mu, std::defer_lock);
    Recorder rec{(flags & KDA_FLAG_STAGE_EVENTS) != 0, s};
    if (rec.on) {
        lock.lock();
        if (stage_begin() != hipSuccess) return KDA_ERR_HIP;
    }
    const int Bs = packed ? N : B;      // batch entries of the states
    if (T == 0)
        return backward_enqueue(nullptr, nullptr, nullptr, nullptr, nullptr, initial_state, nullptr,
                                d_final_state, nullptr, nullptr, nullptr, nullptr, nullptr,
                                d_initial_state, Bs, T, H, Dk, Dv, chunk, dtype, mode, workspace,
                                rec, s);
    unsigned char* w = static_cast<unsigned char*>(workspace);
    void* qh = w + xo[0];
    void* kh = w + xo[1];
    float* al = reinterpret_cast<float*>(w + xo[2]);
    float* be = reinterpret_cast<float*>(w + xo[3]);
    void* dqh = w + xo[4];
    void* dkh = w + xo[5];
    const kda::ProArgs pa{q_raw, k_raw, gate, beta_logit, qh, kh, al, be, dqh, dkh, dq_raw, dk_raw,
                          d_gate, d_beta_logit, ntok, pro->alpha_min,
                          pro->alpha_max - pro->alpha_min, pro->beta_max, pro->eps,
                          pro->normalize_q};
    if (rec.mark("prologue_in") != hipSuccess) return KDA_ERR_HIP;
    if (kda::launch_backward_prologue(false, io, Dk, pa, s) != hipSuccess) return KDA_ERR_HIP;
    if (rec.done() != hipSuccess) return KDA_ERR_HIP;
    st = backward_enqueue(qh, kh, v, al, be, initial_state, d_out, d_final_state, dqh, dkh, dv,
                          d_gate, d_beta_logit, d_initial_state, Bs, T, H, Dk, Dv, chunk, dtype,
                          mode, workspace, rec, s, cu_seqlens);
    if (st != KDA_OK) return st;
    if (rec.mark("prologue_out") != hipSuccess) return KDA_ERR_HIP;
    if (kda::launch_backward_prologue(true, io, Dk, pa, s) != hipSuccess) return KDA_ERR_HIP;
    return rec.done() == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

// the backward of a packed batch (kda_chunk_backward_varlen)
kda_status_t chunk_backward_varlen(const void* q, const void* k, const void* v, const float* alpha,
                                   const float* beta, const int* cu_seqlens, int N,
                                   const float* initial_state, const void* d_out,
                                   const float* d_final_state, void* dq, void* dk, void* dv,
                                   float* d_alpha, float* d_beta, float* d_initial_state,
                                   int total_T, int H, int Dk, int Dv, int chunk,
                                   kda_dtype_t dtype, kda_mode_t mode, unsigned flags,
                                   void* workspace, size_t workspace_bytes, void* stream)
{
    kda_status_t st = check_varlen_shape(N, total_T, H, Dk, Dv, chunk, dtype);
    if (st != KDA_OK) return st;
    st = check_backward_shape(1, total_T, H, Dk, Dv, chunk, dtype);
    if (st != KDA_OK) return st;
    if (mode != KDA_MODE_KDA && mode != KDA_MODE_CKDA) return KDA_ERR_UNSUPPORTED;
    if (flags & ~KDA_FLAG_STAGE_EVENTS) return KDA_ERR_UNSUPPORTED;
    if (!cu_seqlens) return KDA_ERR_NULL_POINTER;
    if (total_T > 0 && (!q || !k || !v || !alpha || !beta || !d_out || !dq || !dk || !dv ||
                        !d_alpha || !d_beta))
        return KDA_ERR_NULL_POINTER;
    const IoType io = dtype == KDA_DTYPE_F32 ? IoType::F32 : IoType::BF16;
    size_t off[kda::kWorkspaceRegions], boff[kBwdRegions], toff = 0;
    const size_t ws_need =
        total_T == 0 ? 0 : backward_varlen_layout(N, total_T, H, Dk, Dv, chunk, io, off, boff, &toff);
    if (total_T > 0 && !workspace) return KDA_ERR_NULL_POINTER;
    if (workspace_bytes < ws_need) return KDA_ERR_WORKSPACE_TOO_SMALL;

    const size_t e = elem_size(dtype);
    const size_t ntok = (size_t)total_T * H;
    const size_t nstate = (size_t)N * H * Dk * Dv * 4;
    const void* vec[] = {q, k, d_out, alpha, workspace};
    for (const void* p : vec)
        if (p && !aligned16(p)) return KDA_ERR_MISALIGNED;
    const void* elt[] = {v, beta, initial_state, d_final_state, dq, dk, dv, d_alpha, d_beta,
                         d_initial_state, cu_seqlens};
    const uintptr_t ea[] = {e, 4, 4, 4, e, e, e, 4, 4, 4, 4};
    for (int i = 0; i < 11; ++i)
        if (elt[i] && !aligned(elt[i], ea[i])) return KDA_ERR_MISALIGNED;
    struct R { const void* p; size_t n; };
    const R in[] = {{q, ntok * Dk * e}, {k, ntok * Dk * e}, {v, ntok * Dv * e},
                    {alpha, ntok * Dk * 4}, {beta, ntok * 4},
                    {initial_state, initial_state ? nstate : 0}, {d_out, ntok * Dv * e},
                    {d_final_state, d_final_state ? nstate : 0},
                    {cu_seqlens, ((size_t)N + 1) * 4}};
    const R outs[] = {{dq, ntok * Dk * e}, {dk, ntok * Dk * e}, {dv, ntok * Dv * e},
                      {d_alpha, ntok * Dk * 4}, {d_beta, ntok * 4},
                      {d_initial_state, d_initial_state ? nstate : 0}, {workspace, ws_need}};
    constexpr int NO = sizeof(outs) / sizeof(outs[0]);
    for (const R& o : outs)
        for (const R& i : in)
            if (overlaps(o.p, o.n, i.p, i.n)) return KDA_ERR_ALIAS;
    for (int x = 0; x < NO; ++x)
        for (int y = x + 1; y < NO; ++y)
            if (overlaps(outs[x].p, outs[x].n, outs[y].p, outs[y].n)) return KDA_ERR_ALIAS;

    hipStream_t s = static_cast<hipStream_t>(stream);
    std::unique_lock<std::mutex> lock(g_stage.mu, std::defer_lock);
    Recorder rec{(flags & KDA_FLAG_STAGE_EVENTS) != 0, s};
    if (rec.on) {
        lock.lock();
        if (stage_begin() != hipSuccess) return KDA_ERR_HIP;
    }
    return backward_enqueue(q, k, v, alpha, beta, initial_state, d_out, d_final_state, dq, dk, dv,
                            d_alpha, d_beta, d_initial_state, N, total_T, H, Dk, Dv, chunk, dtype,
                            mode, workspace, rec, s, total_T > 0 ? cu_seqlens : nullptr);
}

// the backward of the phase variant: workspace = the backward's, then the
// rotated q', k' (io type), the per-channel gates alpha' (fp32), the plain
// backward's dq', dk' (io type) and dalpha' (fp32), the two per-block tables
// (fp64), dS'_T and S'_T (fp32) and the final-state term of d L / d phi
size_t backward_phase_layout(int B, int T, int H, int Dk, int Dv, int chunk, IoType io,
                             size_t xo[11])
{
    size_t off[kda::kWorkspaceRegions], boff[kBwdRegions];
    size_t n = backward_layout(B, T, H, Dk, Dv, chunk, io, off, boff);
    const size_t ntok = (size_t)B * T * H, e = io == IoType::F32 ? 4 : 2;
    const size_t tab = (size_t)B * H * (kda::phase_blocks(T) + 1) * (Dk / 2) * 8;
    const size_t st = (size_t)B * H * Dk * Dv * 4;
    const size_t sz[11] = {ntok * Dk * e, ntok * Dk * e, ntok * Dk * 4, ntok * Dk * e,
                           ntok * Dk * e, ntok * Dk * 4, tab, tab, st, st,
                           (size_t)B * H * (Dk / 2) * 4};
    for (int i = 0; i < 11; ++i) {
        xo[i] = n;
        n += (sz[i] + 255) & ~size_t(255);
    }
    return n;
}

// kda_chunk_backward_phase: the phase variant's backward as the plain backward
// of the rotated recurrence (phase_bwd.hip states the reduction)
kda_status_t chunk_backward_phase(const void* q, const void* k, const void* v, const float* alpha,
                                  const float* theta, const float* beta,
                                  const float* initial_state, const void* d_out,
                                  const float* d_final_state, void* dq, void* dk, void* dv,
                                  float* d_alpha, float* d_theta, float* d_beta,
                                  float* d_initial_state, int B, int T, int H, int Dk, int Dv,
                                  int chunk, kda_dtype_t dtype, kda_mode_t mode, unsigned flags,
                                  void* workspace, size_t workspace_bytes, void* stream)
{
    kda_status_t st = check_backward_shape(B, T, H, Dk, Dv, chunk, dtype);
    if (st != KDA_OK) return st;
    if (mode != KDA_MODE_KDA && mode != KDA_MODE_CKDA) return KDA_ERR_UNSUPPORTED;
    if (flags & ~KDA_FLAG_STAGE_EVENTS) return KDA_ERR_UNSUPPORTED;
    if (T > 0 && (!q || !k || !v || !alpha || !theta || !beta || !d_out || !dq || !dk || !dv ||
                  !d_alpha || !d_theta || !d_beta))
        return KDA_ERR_NULL_POINTER;
    const IoType io = dtype == KDA_DTYPE_F32 ? IoType::F32 : IoType::BF16;
    size_t xo[11];
    const size_t ws_need = T == 0 ? 0 : backward_phase_layout(B, T, H, Dk, Dv, chunk, io, xo);
    if (T > 0 && !workspace) return KDA_ERR_NULL_POINTER;
    if (workspace_bytes < ws_need) return KDA_ERR_WORKSPACE_TOO_SMALL;

    const size_t e = elem_size(dtype);
    const size_t ntok = (size_t)B * T * H, np = (size_t)Dk / 2;
    const size_t nstate = (size_t)B * H * Dk * Dv * 4;
    const void* vec[] = {q, k, d_out, workspace};
    for (const void* p : vec)
        if (p && !aligned16(p)) return KDA_ERR_MISALIGNED;
    const void* elt[] = {v, alpha, theta, beta, initial_state, d_final_state, dq, dk, dv,
                         d_alpha, d_theta, d_beta, d_initial_state};
    const uintptr_t ea[] = {e, 4, 4, 4, 4, 4, e, e, e, 4, 4, 4, 4};
    for (int i = 0; i < 13; ++i)
        if (elt[i] && !aligned(elt[i], ea[i])) return KDA_ERR_MISALIGNED;
    struct R { const void* p; size_t n; };
    const R in[] = {{q, ntok * Dk * e}, {k, ntok * Dk * e}, {v, ntok * Dv * e},
                    {alpha, ntok * np * 4}, {theta, ntok * np * 4}, {beta, ntok * 4},
                    {initial_state, initial_state ? nstate : 0}, {d_out, ntok * Dv * e},
                    {d_final_state, d_final_state ? nstate : 0}};
    const R outs[] = {{dq, ntok * Dk * e}, {dk, ntok * Dk * e}, {dv, ntok * Dv * e},
                      {d_alpha, ntok * np * 4}, {d_theta, ntok * np * 4}, {d_beta, ntok * 4},
                      {d_initial_state, d_initial_state ? nstate : 0}, {workspace, ws_need}};
    constexpr int NO = sizeof(outs) / sizeof(outs[0]);
    for (const R& o : outs)
        for (const R& i : in)
            if (overlaps(o.p, o.n, i.p, i.n)) return KDA_ERR_ALIAS;
    for (int x = 0; x < NO; ++x)
        for (int y = x + 1; y < NO; ++y)
            if (overlaps(outs[x].p, outs[x].n, outs[y].p, outs[y].n)) return KDA_ERR_ALIAS;

    hipStream_t s = static_cast<hipStream_t>(stream);
    std::unique_lock<std::mutex> lock(g_stage.mu, std::defer_lock);
    Recorder rec{(flags & KDA_FLAG_STAGE_EVENTS) != 0, s};
    if (rec.on) {
        lock.lock();
        if (stage_begin() != hipSuccess) return KDA_ERR_HIP;
    }
    if (T == 0)
        return backward_enqueue(nullptr, nullptr, nullptr, nullptr, nullptr, initial_state, nullptr,
                                d_final_state, nullptr, nullptr, nullptr, nullptr, nullptr,
                                d_initial_state, B, T, H, Dk, Dv, chunk, dtype, mode, workspace,
                                rec, s);
    unsigned char* w = static_cast<unsigned char*>(workspace);
    float* ar = reinterpret_cast<float*>(w + xo[2]);
    float* dar = reinterpret_cast<float*>(w + xo[5]);
    float* dstr = reinterpret_cast<float*>(w + xo[8]);
    float* str = reinterpret_cast<float*>(w + xo[9]);
    float* gT = reinterpret_cast<float*>(w + xo[10]);
    const kda::PhaseArgs pa{q, k, alpha, theta, w + xo[0], w + xo[1], ar, w + xo[3], w + xo[4],
                            dar, dq, dk, d_alpha, d_theta,
                            reinterpret_cast<double*>(w + xo[6]),
                            reinterpret_cast<double*>(w + xo[7]), d_final_state ? gT : nullptr,
                            B, T, H, Dk / 2, kda::phase_blocks(T)};
    auto stage = [&](int i, const char* name, const float* src, float* dst) -> bool {
        return rec.mark(name) == hipSuccess &&
               kda::launch_phase_bwd(i, io, pa, src, dst, gT, Dv, s) == hipSuccess &&
               rec.done() == hipSuccess;
    };
    if (!stage(0, "phase_sums", nullptr, nullptr) || !stage(1, "phase_scan", nullptr, nullptr) ||
        !stage(2, "phase_in", nullptr, nullptr))
        return KDA_ERR_HIP;
    if (d_final_state && !stage(3, "phase_state", d_final_state, dstr)) return KDA_ERR_HIP;
    st = backward_enqueue(w + xo[0], w + xo[1], v, ar, beta, initial_state, d_out,
                          d_final_state ? dstr : nullptr, w + xo[3], w + xo[4], dv, dar, d_beta,
                          d_initial_state, B, T, H, Dk, Dv, chunk, dtype, mode, workspace, rec, s,
                          nullptr, BwdPart::ALL, nullptr, d_final_state ? str : nullptr);
    if (st != KDA_OK) return st;
    if (d_final_state && !stage(4, "phase_final", dstr, str)) return KDA_ERR_HIP;
    if (!stage(5, "phase_out", nullptr, nullptr) || !stage(6, "phase_suffix", nullptr, nullptr) ||
        !stage(7, "phase_dtheta", nullptr, nullptr))
        return KDA_ERR_HIP;
    return KDA_OK;
}

// ---- scratch of kda_chunk_forward_noalloc -------------------------------------
// A fixed array per device in place of the caller's workspace, for callers that
// cannot allocate.  The runtime sets it aside when the library's code object is
// loaded on a device, and it stays until the process ends.  On the host the
// name `scratch` is only a stand-in for the symbol, not a device address: the
// address is taken per device with hipGetSymbolAddress, once, with that device
// current, and only that address is ever handed to kernels.  The forward writes
// every workspace byte it reads later in the same call (the per-unit factors,
// flags and, with segments, the maps and start states), so nothing is cleared
// between calls.
static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// the address of `scratch` on `dev`, looked up on first use with dev current
hipError_t scratch_address(int dev, void** out)
{
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> guard(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = 0;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        const hipError_t eg = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur && (e = hipSetDevice(cur)) != hipSuccess) return e;
        if (eg != hipSuccess) return eg;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

const char* kda_status_string(int s)
{
    switch (s) {
    case KDA_OK: return "ok";
    case KDA_ERR_NULL_POINTER: return "a required pointer is NULL";
    case KDA_ERR_BAD_SHAPE: return "a size is out of range or overflows";
    case KDA_ERR_UNSUPPORTED: return "unsupported shape, dtype, mode or flag";
    case KDA_ERR_MISALIGNED: return "a pointer breaks the alignment rule";
    case KDA_ERR_WORKSPACE_TOO_SMALL: return "workspace smaller than kda_chunk_forward_workspace_size";
    case KDA_ERR_ALIAS: return "an output overlaps an input";
    case KDA_ERR_HIP: return "a HIP runtime call or kernel launch failed";
    case KDA_ERR_RANGE: return "an input lies outside the mode's ranges";
    case KDA_ERR_SCRATCH_LIMIT:
        return "the shape's workspace exceeds the built-in scratch of kda_chunk_forward_noalloc";
    default: return "unknown status";
    }
}

kda_status_t kda_chunk_forward_workspace_size(int B, int T, int H, int Dk, int Dv, int chunk,
                                              kda_dtype_t dtype, size_t* bytes)
{
    if (!bytes) return KDA_ERR_NULL_POINTER;
    const kda_status_t st = check_forward_shape(B, T, H, Dk, Dv, chunk, dtype);
    if (st != KDA_OK) return st;
    size_t off[kda::kWorkspaceRegions], so, ss;
    *bytes = T == 0 ? 0
                    : dense_layout(B, T, H, Dk, Dv, chunk,
                                   dtype == KDA_DTYPE_F32 ? IoType::F32 : IoType::BF16, off, &so, &ss);
    return KDA_OK;
}

kda_status_t kda_chunk_forward(const void* q, const void* k, const void* v, const float* alpha,
                               const float* beta, const float* initial_state, void* out,
                               float* final_state, int B, int T, int H, int Dk, int Dv, int chunk,
                               kda_dtype_t dtype, kda_mode_t mode, unsigned flags, void* workspace,
                               size_t workspace_bytes, void* stream)
{
    return chunk_forward(q, k, v, alpha, beta, initial_state, out, final_state, nullptr, nullptr,
                         B, T, H, Dk, Dv, chunk, dtype, mode, flags, workspace, workspace_bytes,
                         stream);
}

kda_status_t kda_chunk_forward_side(const void* q, const void* k, const void* v,
                                    const float* alpha, const float* beta,
                                    const float* initial_state, void* out, float* final_state,
                                    int B, int T, int H, int Dk, int Dv, int chunk,
                                    kda_dtype_t dtype, kda_mode_t mode, unsigned flags,
                                    void* workspace, size_t workspace_bytes, void* stream,
                                    const kda_side_t* side)
{
    return chunk_forward(q, k, v, alpha, beta, initial_state, out, final_state, nullptr, nullptr,
                         B, T, H, Dk, Dv, chunk, dtype, mode, flags, workspace, workspace_bytes,
                         stream, nullptr, side);
}

kda_status_t kda_side_stream_create(kda_side_t* side)
{
    if (!side) return KDA_ERR_NULL_POINTER;
    memset(side, 0, sizeof(*side));
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        return KDA_ERR_HIP;
    // every compute unit in the mask: the mask only buys the queue of its own
    std::vector<uint32_t> mask((size_t)(cus + 31) / 32, 0u);
    for (int i = 0; i < cus; ++i) mask[(size_t)i / 32] |= 1u << (i % 32);
    hipStream_t st = nullptr;
    if (hipExtStreamCreateWithCUMask(&st, (uint32_t)mask.size(), mask.data()) != hipSuccess)
        return KDA_ERR_HIP;
    side->stream = st;
    // (the events only order work on this device: a device-scope release is
    // enough, and it spares the system-scope cache write-back at each record)
    for (int i = 0; i < KDA_SIDE_EVENTS; ++i) {
        hipEvent_t e = nullptr;
        if (hipEventCreateWithFlags(&e, hipEventDisableTiming | hipEventReleaseToDevice) != hipSuccess) {
            kda_side_stream_destroy(side);
            return KDA_ERR_HIP;
        }
        side->events[i] = e;
    }
    return KDA_OK;
}

kda_status_t kda_side_stream_destroy(kda_side_t* side)
{
    if (!side) return KDA_ERR_NULL_POINTER;
    bool ok = true;
    if (side->stream) ok = hipStreamSynchronize(static_cast<hipStream_t>(side->stream)) == hipSuccess && ok;
    for (int i = 0; i < KDA_SIDE_EVENTS; ++i)
        if (side->events[i]) ok = hipEventDestroy(static_cast<hipEvent_t>(side->events[i])) == hipSuccess && ok;
    if (side->stream) ok = hipStreamDestroy(static_cast<hipStream_t>(side->stream)) == hipSuccess && ok;
    memset(side, 0, sizeof(*side));
    return ok ? KDA_OK : KDA_ERR_HIP;
}

kda_status_t kda_chunk_forward_noalloc(const void* q, const void* k, const void* v,
                                       const float* alpha, const float* beta,
                                       const float* initial_state, void* out, float* final_state,
                                       int B, int T, int H, int Dk, int Dv, int chunk,
                                       kda_dtype_t dtype, kda_mode_t mode, unsigned flags,
                                       void* stream)
{
    // every check that needs no HIP call first (shape, flags, the scratch limit)
    const kda_status_t st = check_forward_shape(B, T, H, Dk, Dv, chunk, dtype);
    if (st != KDA_OK) return st;
    if (flags & (KDA_FLAG_STAGE_EVENTS | KDA_FLAG_VALIDATE_RANGES)) return KDA_ERR_UNSUPPORTED;
    if (flags & ~kKnownFlags) return KDA_ERR_UNSUPPORTED;
    size_t need = 0;
    kda_chunk_forward_workspace_size(B, T, H, Dk, Dv, chunk, dtype, &need);
    if (need > (size_t)KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_SCRATCH_LIMIT;
    if (T == 0 || need == 0)
        return chunk_forward(q, k, v, alpha, beta, initial_state, out, final_state, nullptr,
                             nullptr, B, T, H, Dk, Dv, chunk, dtype, mode,
                             flags | KDA_FLAG_SINGLE_STREAM, nullptr, 0, stream);
    // the scratch of the device `stream` belongs to
    int dev = 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev)) != hipSuccess) return KDA_ERR_HIP;
    void* ws = nullptr;
    if (scratch_address(dev, &ws) != hipSuccess) return KDA_ERR_HIP;
    return chunk_forward(q, k, v, alpha, beta, initial_state, out, final_state, nullptr, nullptr,
                         B, T, H, Dk, Dv, chunk, dtype, mode, flags | KDA_FLAG_SINGLE_STREAM, ws,
                         (size_t)KDA_NOALLOC_SCRATCH_BYTES, stream);
}

kda_status_t kda_chunk_forward_prologue(const void* q_raw, const void* k_raw, const void* v,
                                        const float* gate, const float* beta_logit,
                                        const kda_prologue_t* prologue,
                                        const float* initial_state, void* out, float* final_state,
                                        int B, int T, int H, int Dk, int Dv, int chunk,
                                        kda_dtype_t dtype, kda_mode_t mode, unsigned flags,
                                        void* workspace, size_t workspace_bytes, void* stream)
{
    if (!prologue) return KDA_ERR_NULL_POINTER;
    return chunk_forward(q_raw, k_raw, v, gate, beta_logit, initial_state, out, final_state,
                         nullptr, prologue, B, T, H, Dk, Dv, chunk, dtype, mode, flags, workspace,
                         workspace_bytes, stream);
}

kda_status_t kda_chunk_forward_states(const void* q, const void* k, const void* v,
                                      const float* alpha, const float* beta,
                                      const float* initial_state, void* out, float* final_state,
                                      void* chunk_states, int B, int T, int H, int Dk, int Dv,
                                      int chunk, kda_dtype_t dtype, kda_mode_t mode,
                                      unsigned flags, void* workspace, size_t workspace_bytes,
                                      void* stream)
{
    if (T > 0 && !chunk_states) return KDA_ERR_NULL_POINTER;
    return chunk_forward(q, k, v, alpha, beta, initial_state, out, final_state, chunk_states,
                         nullptr, B, T, H, Dk, Dv, chunk, dtype, mode, flags, workspace,
                         workspace_bytes, stream);
}

kda_status_t kda_chunk_forward_phase(const void* q, const void* k, const void* v,
                                     const float* alpha, const float* theta, const float* beta,
                                     const float* initial_state, void* out, float* final_state,
                                     int B, int T, int H, int Dk, int Dv, int chunk,
                                     kda_dtype_t dtype, kda_mode_t mode, unsigned flags,
                                     void* workspace, size_t workspace_bytes, void* stream)
{
    if (T > 0 && !theta) return KDA_ERR_NULL_POINTER;
    if (T == 0) theta = nullptr;
    return chunk_forward(q, k, v, alpha, beta, initial_state, out, final_state, nullptr, nullptr,
                         B, T, H, Dk, Dv, chunk, dtype, mode, flags, workspace, workspace_bytes,
                         stream, theta);
}

kda_status_t kda_chunk_forward_varlen_workspace_size(int N, int total_T, int H, int Dk, int Dv,
                                                     int chunk, kda_dtype_t dtype, size_t* bytes)
{
    if (!bytes) return KDA_ERR_NULL_POINTER;
    const kda_status_t st = check_varlen_shape(N, total_T, H, Dk, Dv, chunk, dtype);
    if (st != KDA_OK) return st;
    size_t off[kda::kWorkspaceRegions], toff;
    *bytes = varlen_layout(N, total_T, H, Dk, Dv, chunk,
                           dtype == KDA_DTYPE_F32 ? IoType::F32 : IoType::BF16, off, &toff);
    return KDA_OK;
}

kda_status_t kda_chunk_forward_varlen(const void* q, const void* k, const void* v,
                                      const float* alpha, const float* beta,
                                      const kda_prologue_t* prologue, const int* cu_seqlens,
                                      int N, const float* initial_state, void* out,
                                      float* final_state, int total_T, int H, int Dk, int Dv,
                                      int chunk, kda_dtype_t dtype, kda_mode_t mode,
                                      unsigned flags, void* workspace, size_t workspace_bytes,
                                      void* stream)
{
    kda_status_t st = check_varlen_shape(N, total_T, H, Dk, Dv, chunk, dtype);
    if (st != KDA_OK) return st;
    if (mode != KDA_MODE_KDA && mode != KDA_MODE_CKDA) return KDA_ERR_UNSUPPORTED;
    if (flags & ~kKnownFlags) return KDA_ERR_UNSUPPORTED;
    if (prologue && !prologue_ok(*prologue, mode)) return KDA_ERR_UNSUPPORTED;
    if (!cu_seqlens || !workspace || !out) return KDA_ERR_NULL_POINTER;
    if (total_T > 0 && (!q || !k || !v || !alpha || !beta)) return KDA_ERR_NULL_POINTER;

    const IoType io = dtype == KDA_DTYPE_F32 ? IoType::F32 : IoType::BF16;
    const size_t e = elem_size(dtype);
    const size_t ntok = (size_t)total_T * H;
    const size_t nstate = (size_t)N * H * Dk * Dv * 4;
    size_t off[kda::kWorkspaceRegions], toff;
    const size_t ws_need = varlen_layout(N, total_T, H, Dk, Dv, chunk, io, off, &toff);
    if (workspace_bytes < ws_need) return KDA_ERR_WORKSPACE_TOO_SMALL;

    const void* vec[] = {q, k, alpha, workspace};
    for (const void* p : vec)
        if (p && !aligned16(p)) return KDA_ERR_MISALIGNED;
    const void* elt[] = {v, out, beta, initial_state, final_state, cu_seqlens};
    const uintptr_t ea[] = {e, e, 4, 4, 4, 4};
    for (int i = 0; i < 6; ++i)
        if (elt[i] && !aligned(elt[i], ea[i])) return KDA_ERR_MISALIGNED;

    struct R { const void* p; size_t n; } in[] = {
        {q, ntok * Dk * e}, {k, ntok * Dk * e}, {v, ntok * Dv * e},
        {alpha, ntok * Dk * 4}, {beta, ntok * 4}, {initial_state, initial_state ? nstate : 0},
        {cu_seqlens, ((size_t)N + 1) * 4}};
    const R outs[] = {{out, ntok * Dv * e}, {workspace, ws_need}};
    for (const R& o : outs)
        for (const R& i : in)
            if (overlaps(o.p, o.n, i.p, i.n)) return KDA_ERR_ALIAS;
    if (overlaps(out, ntok * Dv * e, workspace, ws_need)) return KDA_ERR_ALIAS;
    if (final_state) {
        const R fs{final_state, nstate};
        for (const R& i : in) {
            if (i.p == initial_state && final_state == initial_state) continue;
            if (overlaps(fs.p, fs.n, i.p, i.n)) return KDA_ERR_ALIAS;
        }
        for (const R& o : outs)
            if (overlaps(fs.p, fs.n, o.p, o.n)) return KDA_ERR_ALIAS;
    }

    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!prologue && total_T > 0) {
        st = validate_ranges(flags, mode, alpha, ntok * Dk, beta, ntok, nullptr, 0, s);
        if (st != KDA_OK) return st;
    }
    std::unique_lock<std::mutex> lock(g_stage.mu, std::defer_lock);
    Recorder rec{(flags & KDA_FLAG_STAGE_EVENTS) != 0, s};
    if (rec.on) {
        lock.lock();
        if (stage_begin() != hipSuccess) return KDA_ERR_HIP;
    }
    const int umax = (int)varlen_max_chunks(N, total_T, chunk);
    unsigned char* w = static_cast<unsigned char*>(workspace);
    int* cu_s = reinterpret_cast<int*>(w + toff);
    int* cs = cu_s + (N + 1);
    if (rec.mark("varlen_table") != hipSuccess) return KDA_ERR_HIP;
    if (kda::launch_varlen_table(cu_seqlens, N, total_T, chunk, umax, cu_s, cs, s) != hipSuccess)
        return KDA_ERR_HIP;
    if (rec.done() != hipSuccess) return KDA_ERR_HIP;

    const ChunkShape shp{1, total_T, H, Dk, Dv, chunk, umax};      // prep: all units
    const ChunkShape shc{N, total_T, H, Dk, Dv, chunk, umax};      // chain: N x H chains
    const ChunkWorkspace ws{w + off[0], w + off[1], w + off[2],
                            w + off[3], w + off[4], reinterpret_cast<float*>(w + off[5]),
                            w + off[6]};
    const int zx = fast_zero_columns(mode, Dk);
    kda::PrepArgs pa{q, k, v, alpha, beta, ws.W, ws.U, ws.Kt, ws.QG, ws.P, ws.GC, ws.FL,
                           total_T, H, Dv, umax, zx,
                           prologue ? 1 : 0,
                           prologue ? prologue->alpha_min : 0.f,
                           prologue ? prologue->alpha_max - prologue->alpha_min : 0.f,
                           prologue ? prologue->beta_max : 0.f,
                           prologue ? prologue->eps : 0.f,
                           prologue ? prologue->normalize_q : 0,
                           cu_s, cs, N, nullptr};
    pa.ntst = workspace_nt((long long)N * H * (Dv / 16));
    const kda::ChainArgs ca{ws.W, ws.U, ws.Kt, ws.QG, ws.P, ws.GC, initial_state, out,
                            final_state, nullptr, N, total_T, H, Dv, umax, cu_s, cs, 0,
                            0, 1, nullptr, nullptr};
    if (rec.mark("prep_fast") != hipSuccess) return KDA_ERR_HIP;
    if (kda::launch_prep_fast(io, shp, pa, s) != hipSuccess) return KDA_ERR_HIP;
    if (rec.done() != hipSuccess) return KDA_ERR_HIP;
    if (rec.mark("prep_exact") != hipSuccess) return KDA_ERR_HIP;
    if (kda::launch_prep_exact(io, shp, pa, s) != hipSuccess) return KDA_ERR_HIP;
    if (rec.done() != hipSuccess) return KDA_ERR_HIP;
    if (rec.mark("chain") != hipSuccess) return KDA_ERR_HIP;
    if (launch_forward_chain(io, shc, ca, s) != hipSuccess) return KDA_ERR_HIP;
    if (rec.done() != hipSuccess) return KDA_ERR_HIP;
    return KDA_OK;
}

kda_status_t kda_decode_step(const void* q, const void* k, const void* v, const float* alpha,
                             const float* beta, float* state, void* out, int B, int H, int Dk,
                             int Dv, kda_dtype_t dtype, kda_mode_t mode, unsigned flags,
                             void* stream)
{
    return decode_step(q, k, v, alpha, nullptr, beta, state, out, B, H, Dk, Dv, dtype, mode, flags,
                       stream);
}

kda_status_t kda_decode_step_phase(const void* q, const void* k, const void* v,
                                   const float* alpha, const float* theta, const float* beta,
                                   float* state, void* out, int B, int H, int Dk, int Dv,
                                   kda_dtype_t dtype, kda_mode_t mode, unsigned flags,
                                   void* stream)
{
    if (!theta) return KDA_ERR_NULL_POINTER;
    return decode_step(q, k, v, alpha, theta, beta, state, out, B, H, Dk, Dv, dtype, mode, flags,
                       stream);
}

kda_status_t kda_decode_step_prologue(const void* q_raw, const void* k_raw, const void* v,
                                      const float* gate, const float* beta_logit,
                                      const kda_prologue_t* prologue, float* state, void* out,
                                      int B, int H, int Dk, int Dv, kda_dtype_t dtype,
                                      kda_mode_t mode, unsigned flags, void* stream)
{
    if (!prologue) return KDA_ERR_NULL_POINTER;
    return decode_step(q_raw, k_raw, v, gate, nullptr, beta_logit, state, out, B, H, Dk, Dv, dtype,
                       mode, flags, stream, prologue);
}

kda_status_t kda_gate_prep(const float* alpha, float* L, unsigned char* meta, float* gend, int B,
                           int T, int H, int Dk, int chunk, void* stream)
{
    if (B < 1 || H < 1 || T < 0) return KDA_ERR_BAD_SHAPE;
    if (!dk_ok(Dk) || !chunk_ok(chunk)) return KDA_ERR_UNSUPPORTED;
    const long long NC = ((long long)T + chunk - 1) / chunk;
    if ((long long)B * H * NC > 0x7fffffffLL) return KDA_ERR_BAD_SHAPE;
    if (T == 0) return KDA_OK;
    if (!alpha || !L || !meta || !gend) return KDA_ERR_NULL_POINTER;
    if (!aligned16(alpha) || !aligned16(L) || !aligned16(gend) || !aligned(meta, 4))
        return KDA_ERR_MISALIGNED;
    const size_t nel = (size_t)B * H * NC * chunk * Dk;
    const size_t na = (size_t)B * T * H * Dk * 4;
    struct R { const void* p; size_t n; } rs[] = {
        {alpha, na}, {L, nel * 4}, {meta, nel}, {gend, (size_t)B * H * NC * Dk * 4}};
    for (int i = 0; i < 4; ++i)
        for (int j = i + 1; j < 4; ++j)
            if (overlaps(rs[i].p, rs[i].n, rs[j].p, rs[j].n)) return KDA_ERR_ALIAS;
    if (kda::launch_gate_prep(alpha, L, meta, gend, B, T, H, Dk, chunk,
                              static_cast<hipStream_t>(stream)) != hipSuccess)
        return KDA_ERR_HIP;
    return KDA_OK;
}

kda_status_t kda_chunk_backward_workspace_size(int B, int T, int H, int Dk, int Dv, int chunk,
                                               kda_dtype_t dtype, size_t* bytes)
{
    if (!bytes) return KDA_ERR_NULL_POINTER;
    const kda_status_t st = check_backward_shape(B, T, H, Dk, Dv, chunk, dtype);
    if (st != KDA_OK) return st;
    size_t off[kda::kWorkspaceRegions], boff[kBwdRegions];
    *bytes = T == 0 ? 0
                    : backward_layout(B, T, H, Dk, Dv, chunk,
                                      dtype == KDA_DTYPE_F32 ? IoType::F32 : IoType::BF16, off, boff);
    return KDA_OK;
}

kda_status_t kda_chunk_backward_phase_workspace_size(int B, int T, int H, int Dk, int Dv, int chunk,
                                                     kda_dtype_t dtype, size_t* bytes)
{
    if (!bytes) return KDA_ERR_NULL_POINTER;
    const kda_status_t st = check_backward_shape(B, T, H, Dk, Dv, chunk, dtype);
    if (st != KDA_OK) return st;
    size_t xo[11];
    *bytes = T == 0 ? 0
                    : backward_phase_layout(B, T, H, Dk, Dv, chunk,
                                            dtype == KDA_DTYPE_F32 ? IoType::F32 : IoType::BF16, xo);
    return KDA_OK;
}

kda_status_t kda_chunk_backward_phase(const void* q, const void* k, const void* v,
                                      const float* alpha, const float* theta, const float* beta,
                                      const float* initial_state, const void* d_out,
                                      const float* d_final_state, void* dq, void* dk, void* dv,
                                      float* d_alpha, float* d_theta, float* d_beta,
                                      float* d_initial_state, int B, int T, int H, int Dk, int Dv,
                                      int chunk, kda_dtype_t dtype, kda_mode_t mode,
                                      unsigned flags, void* workspace, size_t workspace_bytes,
                                      void* stream)
{
    return chunk_backward_phase(q, k, v, alpha, theta, beta, initial_state, d_out, d_final_state,
                                dq, dk, dv, d_alpha, d_theta, d_beta, d_initial_state, B, T, H, Dk,
                                Dv, chunk, dtype, mode, flags, workspace, workspace_bytes, stream);
}

kda_status_t kda_chunk_backward(const void* q, const void* k, const void* v, const float* alpha,
                                const float* beta, const float* initial_state, const void* d_out,
                                const float* d_final_state, void* dq, void* dk, void* dv,
                                float* d_alpha, float* d_beta, float* d_initial_state, int B,
                                int T, int H, int Dk, int Dv, int chunk, kda_dtype_t dtype,
                                kda_mode_t mode, unsigned flags, void* workspace,
                                size_t workspace_bytes, void* stream)
{
    return chunk_backward(q, k, v, alpha, beta, initial_state, d_out, d_final_state, dq, dk, dv,
                          d_alpha, d_beta, d_initial_state, B, T, H, Dk, Dv, chunk, dtype, mode,
                          flags, workspace, workspace_bytes, stream);
}

kda_status_t kda_chunk_forward_save(const void* q, const void* k, const void* v,
                                    const float* alpha, const float* beta,
                                    const float* initial_state, void* out, float* final_state,
                                    int B, int T, int H, int Dk, int Dv, int chunk,
                                    kda_dtype_t dtype, kda_mode_t mode, unsigned flags,
                                    void* saved, size_t saved_bytes, void* stream)
{
    return chunk_backward_part(q, k, v, alpha, beta, initial_state, nullptr, nullptr, nullptr,
                               nullptr, nullptr, nullptr, nullptr, nullptr, B, T, H, Dk, Dv, chunk,
                               dtype, mode, flags, saved, saved_bytes, stream, BwdPart::SAVE, out,
                               final_state);
}

kda_status_t kda_chunk_backward_saved(const void* q, const void* k, const void* v,
                                      const float* alpha, const float* beta, const void* d_out,
                                      const float* d_final_state, void* dq, void* dk, void* dv,
                                      float* d_alpha, float* d_beta, float* d_initial_state,
                                      int B, int T, int H, int Dk, int Dv, int chunk,
                                      kda_dtype_t dtype, kda_mode_t mode, unsigned flags,
                                      void* saved, size_t saved_bytes, void* stream)
{
    return chunk_backward_part(q, k, v, alpha, beta, nullptr, d_out, d_final_state, dq, dk, dv,
                               d_alpha, d_beta, d_initial_state, B, T, H, Dk, Dv, chunk, dtype,
                               mode, flags, saved, saved_bytes, stream, BwdPart::FROM_SAVED);
}

kda_status_t kda_chunk_backward_prologue_workspace_size(int B, int T, int H, int Dk, int Dv,
                                                        int chunk, kda_dtype_t dtype, size_t* bytes)
{
    if (!bytes) return KDA_ERR_NULL_POINTER;
    const kda_status_t st = check_backward_shape(B, T, H, Dk, Dv, chunk, dtype);
    if (st != KDA_OK) return st;
    size_t xo[6];
    *bytes = T == 0 ? 0
                    : backward_prologue_layout(B, T, H, Dk, Dv, chunk,
                                               dtype == KDA_DTYPE_F32 ? IoType::F32 : IoType::BF16, xo);
    return KDA_OK;
}

kda_status_t kda_chunk_backward_varlen_prologue_workspace_size(int N, int total_T, int H, int Dk,
                                                               int Dv, int chunk,
                                                               kda_dtype_t dtype, size_t* bytes)
{
    if (!bytes) return KDA_ERR_NULL_POINTER;
    kda_status_t st = check_varlen_shape(N, total_T, H, Dk, Dv, chunk, dtype);
    if (st != KDA_OK) return st;
    st = check_backward_shape(1, total_T, H, Dk, Dv, chunk, dtype);
    if (st != KDA_OK) return st;
    size_t xo[6];
    *bytes = total_T == 0 ? 0
                          : backward_varlen_prologue_layout(N, total_T, H, Dk, Dv, chunk,
                                                            dtype == KDA_DTYPE_F32 ? IoType::F32
                                                                                   : IoType::BF16,
                                                            xo);
    return KDA_OK;
}

kda_status_t kda_chunk_backward_varlen_prologue(
    const void* q_raw, const void* k_raw, const void* v, const float* gate,
    const float* beta_logit, const int* cu_seqlens, int N, const float* initial_state,
    const void* d_out, const float* d_final_state, const kda_prologue_t* prologue, void* dq_raw,
    void* dk_raw, void* dv, float* d_gate, float* d_beta_logit, float* d_initial_state,
    int total_T, int H, int Dk, int Dv, int chunk, kda_dtype_t dtype, kda_mode_t mode,
    unsigned flags, void* workspace, size_t workspace_bytes, void* stream)
{
    if (!cu_seqlens) return KDA_ERR_NULL_POINTER;
    return chunk_backward_prologue(q_raw, k_raw, v, gate, beta_logit, initial_state, d_out,
                                   d_final_state, prologue, dq_raw, dk_raw, dv, d_gate, d_beta_logit,
                                   d_initial_state, 1, total_T, H, Dk, Dv, chunk, dtype, mode, flags,
                                   workspace, workspace_bytes, stream, cu_seqlens, N);
}

kda_status_t kda_chunk_backward_prologue(const void* q_raw, const void* k_raw, const void* v,
                                         const float* gate, const float* beta_logit,
                                         const float* initial_state, const void* d_out,
                                         const float* d_final_state, const kda_prologue_t* prologue,
                                         void* dq_raw, void* dk_raw, void* dv, float* d_gate,
                                         float* d_beta_logit, float* d_initial_state, int B, int T,
                                         int H, int Dk, int Dv, int chunk, kda_dtype_t dtype,
                                         kda_mode_t mode, unsigned flags, void* workspace,
                                         size_t workspace_bytes, void* stream)
{
    return chunk_backward_prologue(q_raw, k_raw, v, gate, beta_logit, initial_state, d_out,
                                   d_final_state, prologue, dq_raw, dk_raw, dv, d_gate, d_beta_logit,
                                   d_initial_state, B, T, H, Dk, Dv, chunk, dtype, mode, flags,
                                   workspace, workspace_bytes, stream);
}

kda_status_t kda_chunk_backward_varlen_workspace_size(int N, int total_T, int H, int Dk, int Dv,
                                                      int chunk, kda_dtype_t dtype, size_t* bytes)
{
    if (!bytes) return KDA_ERR_NULL_POINTER;
    kda_status_t st = check_varlen_shape(N, total_T, H, Dk, Dv, chunk, dtype);
    if (st != KDA_OK) return st;
    st = check_backward_shape(1, total_T, H, Dk, Dv, chunk, dtype);
    if (st != KDA_OK) return st;
    size_t off[kda::kWorkspaceRegions], boff[kBwdRegions], toff;
    *bytes = total_T == 0 ? 0
                          : backward_varlen_layout(N, total_T, H, Dk, Dv, chunk,
                                                   dtype == KDA_DTYPE_F32 ? IoType::F32 : IoType::BF16,
                                                   off, boff, &toff);
    return KDA_OK;
}

kda_status_t kda_chunk_backward_varlen(const void* q, const void* k, const void* v,
                                       const float* alpha, const float* beta,
                                       const int* cu_seqlens, int N, const float* initial_state,
                                       const void* d_out, const float* d_final_state, void* dq,
                                       void* dk, void* dv, float* d_alpha, float* d_beta,
                                       float* d_initial_state, int total_T, int H, int Dk, int Dv,
                                       int chunk, kda_dtype_t dtype, kda_mode_t mode,
                                       unsigned flags, void* workspace, size_t workspace_bytes,
                                       void* stream)
{
    return chunk_backward_varlen(q, k, v, alpha, beta, cu_seqlens, N, initial_state, d_out,
                                 d_final_state, dq, dk, dv, d_alpha, d_beta, d_initial_state,
                                 total_T, H, Dk, Dv, chunk, dtype, mode, flags, workspace,
                                 workspace_bytes, stream);
}

kda_status_t kda_last_stage_times(float* ms, const char** names, int max, int* count)
{
    if (!count || (max > 0 && !ms)) return KDA_ERR_NULL_POINTER;
    std::lock_guard<std::mutex> lock(g_stage.mu);
    *count = g_stage.count;
    if (!g_stage.created || g_stage.count == 0) return KDA_OK;
    if (hipEventSynchronize(g_stage.ev[2 * g_stage.count - 1]) != hipSuccess) return KDA_ERR_HIP;
    for (int i = 0; i < g_stage.count && i < max; ++i) {
        float t = 0.f;
        if (hipEventElapsedTime(&t, g_stage.ev[2 * i], g_stage.ev[2 * i + 1]) != hipSuccess)
            return KDA_ERR_HIP;
        ms[i] = t;
        if (names) names[i] = g_stage.names[i];
    }
    return KDA_OK;
}

}  // extern "C"
