// gate_prep.hip — chunk-local gate summary in log-magnitude / sign / zero form.
//
// Per (b, h, chunk n, channel c), a scan over the chunk's tokens r:
//   L_r    = sum_{j<=r, alpha_j != 0} log2|alpha_j|      (fp32)
//   parity = #{j <= r : alpha_j < 0} mod 2
//   zpos   = 1 + last j <= r with alpha_j == 0 (0 if none)
// so every decay ratio inside the chunk is exact in sign and zero:
//   prod_{j=i+1..r} alpha_j = [zpos_r <= i+1] (-1)^(parity_r - parity_i) 2^(L_r - L_i)
// (per-channel decay: "Kimi Delta Attention: a bounded case study", Chapter 12
// §12.1; the CKDA gate range with exact -1 and 0 entries: "Complex KDA", the
// abstract).  A plain log-space cumulative sum of log(alpha) would turn a zero
// gate into -inf and a negative one into NaN; the separate parity bit and
// last-zero index keep both exact.
//
// Thread = (chunk, channel quad): 16-byte gate reads (the quads of one
// chunk's token row are contiguous), a 16-byte L store and one 4-byte meta
// store per token, four independent scans per thread; 1024 / Dk chunks share
// a 256-thread workgroup.  The loads of 8 tokens are issued before their
// scan steps, and every access is non-temporal (each byte is touched once).
// HBM-bound: 4 bytes read and 5 bytes written per element, plus Dk*4 bytes of
// chunk decay per chunk.  The scan order per channel is the token order.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace {

constexpr int kGateThreads = 256;
constexpr int kGateBatch = 8;          // tokens whose loads are issued together

template <int DK>
__global__ __launch_bounds__(kGateThreads) void gate_prep_kernel(const float* __restrict__ alpha,
                                                                 float* __restrict__ L,
                                                                 uint8_t* __restrict__ meta,
                                                                 float* __restrict__ gend, int T,
                                                                 int H, int C, int NC, int units)
{
    constexpr int NQ = DK / 4;                    // channel quads: threads per chunk
    constexpr int CPW = kGateThreads / NQ;        // chunks per workgroup
    const int q4 = threadIdx.x % NQ;
    const int unit = blockIdx.x * CPW + threadIdx.x / NQ;
    if (unit >= units) return;
    const int n = unit % NC;
    const int bh = unit / NC;
    const int b = bh / H, h = bh % H;
    const int t0 = n * C;
    const size_t obase = (size_t)unit * C * DK + 4 * q4;
    const float* ap = alpha + (((size_t)b * T + t0) * H + h) * DK + 4 * q4;
    const size_t tstride = (size_t)H * DK;

    f32x4 lsum = {0.f, 0.f, 0.f, 0.f}, prod = {1.f, 1.f, 1.f, 1.f};
    int parity[4] = {0, 0, 0, 0}, zpos[4] = {0, 0, 0, 0};
    for (int r0 = 0; r0 < C; r0 += kGateBatch) {
        f32x4 a[kGateBatch];
#pragma unroll
        for (int j = 0; j < kGateBatch; ++j) {
            const int r = r0 + j;
            a[j] = t0 + r < T ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(ap + r * tstride))
                              : f32x4{1.f, 1.f, 1.f, 1.f};
        }
#pragma unroll
        for (int j = 0; j < kGateBatch; ++j) {
            const int r = r0 + j;
            f32x4 Lr = {0.f, 0.f, 0.f, 0.f};
            unsigned m = 0;
            if (t0 + r < T) {
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const float v = a[j][x];
                    if (v == 0.f) zpos[x] = r + 1;
                    else lsum[x] += log2f(fabsf(v));
                    parity[x] ^= (v < 0.f) ? 1 : 0;
                    prod[x] *= v;
                    Lr[x] = lsum[x];
                    m |= (unsigned)((zpos[x] << 1) | parity[x]) << (8 * x);
                }
            }
            __builtin_nontemporal_store(Lr, reinterpret_cast<f32x4*>(L + obase + (size_t)r * DK));
            __builtin_nontemporal_store(m, reinterpret_cast<unsigned*>(meta + obase + (size_t)r * DK));
        }
    }
    __builtin_nontemporal_store(prod, reinterpret_cast<f32x4*>(gend + (size_t)unit * DK + 4 * q4));
}

}  // namespace

hipError_t launch_gate_prep(const float* alpha, float* L, uint8_t* meta, float* gend, int B,
                            int T, int H, int Dk, int C, hipStream_t stream)
{
    const int NC = (T + C - 1) / C;
    const int units = B * H * NC;
    const int cpw = kGateThreads / (Dk / 4);
    const dim3 grid((unsigned)((units + cpw - 1) / cpw)), block(kGateThreads);
    switch (Dk) {
    case 16: return launch_kernel(gate_prep_kernel<16>, grid, block, 0, stream, alpha, L, meta, gend, T, H, C, NC, units);
    case 32: return launch_kernel(gate_prep_kernel<32>, grid, block, 0, stream, alpha, L, meta, gend, T, H, C, NC, units);
    case 64: return launch_kernel(gate_prep_kernel<64>, grid, block, 0, stream, alpha, L, meta, gend, T, H, C, NC, units);
    case 128: return launch_kernel(gate_prep_kernel<128>, grid, block, 0, stream, alpha, L, meta, gend, T, H, C, NC, units);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace kda
