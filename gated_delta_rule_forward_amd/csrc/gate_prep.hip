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
// One workgroup per (b, h, chunk), one thread per channel: the 4-byte gate
// reads of a token are contiguous across the workgroup (Dk*4 bytes per row)
// and so are the L / meta writes.  HBM-bound: 4 bytes read and 5 bytes written
// per element, plus Dk*4 bytes of chunk decay per chunk.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace {

__global__ __launch_bounds__(128) void gate_prep_kernel(const float* __restrict__ alpha,
                                                        float* __restrict__ L,
                                                        uint8_t* __restrict__ meta,
                                                        float* __restrict__ gend, int T, int H,
                                                        int Dk, int C, int NC)
{
    const int c = threadIdx.x;
    if (c >= Dk) return;
    const int unit = blockIdx.x;
    const int n = unit % NC;
    const int bh = unit / NC;
    const int b = bh / H, h = bh % H;
    const int t0 = n * C;
    const size_t obase = (size_t)unit * C * Dk;

    float lsum = 0.f, prod = 1.f;
    int parity = 0, zpos = 0;
    for (int r = 0; r < C; ++r) {
        const int t = t0 + r;
        float Lr = 0.f;
        uint8_t m = 0;
        if (t < T) {
            const float a = alpha[(((size_t)b * T + t) * H + h) * Dk + c];
            if (a == 0.f) zpos = r + 1;
            else lsum += log2f(fabsf(a));
            parity ^= (a < 0.f) ? 1 : 0;
            prod *= a;
            Lr = lsum;
            m = (uint8_t)((zpos << 1) | parity);
        }
        L[obase + (size_t)r * Dk + c] = Lr;
        meta[obase + (size_t)r * Dk + c] = m;
    }
    gend[(size_t)unit * Dk + c] = prod;
}

}  // namespace

hipError_t launch_gate_prep(const float* alpha, float* L, uint8_t* meta, float* gend, int B,
                            int T, int H, int Dk, int C, hipStream_t stream)
{
    const int NC = (T + C - 1) / C;
    const dim3 grid((unsigned)((size_t)B * H * NC)), block(128);
    return launch_kernel(gate_prep_kernel, grid, block, 0, stream, alpha, L, meta, gend, T, H, Dk,
                         C, NC);
}

}  // namespace kda
