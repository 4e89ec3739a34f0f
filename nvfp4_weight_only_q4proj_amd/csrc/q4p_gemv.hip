// q4p_gemv.hip — decode / speculative-verify projection, 1 <= M <= 16.
//
// Shape of the problem: at M = 1..16 every weight byte is used by at most 16
// multiply-adds, so the kernel is bound by streaming the packed weight from
// HBM once (0.5625 bytes per weight).  Design:
//
//  * One workgroup per 16-row tile of W; its S waves split the k-tiles of
//    that row tile evenly (split-K inside the workgroup), so short-N shapes
//    still put enough waves on the chip.  Partial sums are combined through
//    LDS in a fixed order: results are bitwise deterministic.
//  * Each wave streams one 1 KB code tile + one 128 B scale tile per k-tile
//    with 128-bit loads, PF k-tiles ahead in registers.
//  * Per 16-element scale block the wave issues one 16x16x16 bf16 MFMA:
//    A = 16 activation rows (rows >= M are zero), B = the 16 weight rows'
//    unscaled e2m1 values (exact in bf16).  The MFMA returns the block's
//    partial sums p[m][n] = sum_{k in block} x[m][k] q[n][k]; the lane then
//    accumulates acc += s[n][block] * p with one fma per live output row.
//    This keeps the per-weight vector work at one conversion per two codes;
//    folding the e4m3 scale into the operand would cost two more multiplies
//    because the hardware fp4 conversion honours only the scale's exponent.
//  * g is applied once per output after the reduction, in fp32.
#include "q4p_device.h"
#include "q4p_launch.h"

namespace q4p {

namespace {

constexpr int kMaxSplit = 8;       // waves per workgroup
constexpr int kPrefetch = 4;       // k-tiles in flight per wave

// Accumulate one k-tile.  R = number of accumulator rows per lane that hold
// live outputs (min(M, 4)); rows beyond it only ever see zero activations.
template <int R>
__device__ __forceinline__ void gemv_tile(const uint4 &cw, const uint2 &sw, const uint2 (&xw)[8],
                                          floatx4_t &acc)
{
    const uint32_t words[4] = {cw.x, cw.y, cw.z, cw.w};
    const floatx4_t zero = {0.f, 0.f, 0.f, 0.f};
    floatx4_t p[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) {
        const uint32_t w = words[b >> 1];
        uint32_t lo, hi;
        if (b & 1) {
            lo = fp4x2_to_bf16x2<2>(w);
            hi = fp4x2_to_bf16x2<3>(w);
        } else {
            lo = fp4x2_to_bf16x2<0>(w);
            hi = fp4x2_to_bf16x2<1>(w);
        }
        const uint2 bq = make_uint2(lo, hi);
        const short4_t a = __builtin_bit_cast(short4_t, xw[b]);
        const short4_t bb = __builtin_bit_cast(short4_t, bq);
        p[b] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, bb, zero, 0, 0, 0);
    }
#pragma unroll
    for (int b = 0; b < 8; ++b) {
        float s;
        const uint32_t sv = (b < 4) ? sw.x : sw.y;
        switch (b & 3) {
        case 0: s = e4m3_to_f32<0>(sv); break;
        case 1: s = e4m3_to_f32<1>(sv); break;
        case 2: s = e4m3_to_f32<2>(sv); break;
        default: s = e4m3_to_f32<3>(sv); break;
        }
#pragma unroll
        for (int i = 0; i < R; ++i)
            acc[i] = __builtin_fmaf(s, p[b][i], acc[i]);
    }
}

template <int R>
__global__ void __launch_bounds__(64 * kMaxSplit)
gemv_kernel(const uint4 *__restrict__ pcodes, const uint2 *__restrict__ pscales, float g,
            const uint16_t *__restrict__ x, float *__restrict__ y, int M, int N, int K, int KT,
            int S)
{
    const int t = blockIdx.x;
    const int w = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int r = lane & 15;       // weight row within the tile / activation row
    const int gq = lane >> 4;      // k-group within each scale block
    const int c0 = (int)(((int64_t)KT * w) / S);
    const int c1 = (int)(((int64_t)KT * (w + 1)) / S);

    const uint4 *pc = pcodes + (int64_t)t * KT * 64 + lane;
    const uint2 *ps = pscales + (int64_t)t * KT * 16 + r;
    const bool xrow = r < M;
    const uint16_t *xr = x + (int64_t)(xrow ? r : 0) * K + 4 * gq;

    uint4 cw[kPrefetch];
    uint2 sw[kPrefetch];
    uint2 xw[kPrefetch][8];

    auto load = [&](int slot, int c) {
        cw[slot] = load_stream16(pc + (int64_t)c * 64);
        sw[slot] = ps[(int64_t)c * 16];
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const int k = c * kTileK + 16 * b;          // + 4*gq folded into xr
            xw[slot][b] = (xrow && k + 4 * gq < K)
                              ? *reinterpret_cast<const uint2 *>(xr + k)
                              : make_uint2(0u, 0u);
        }
    };

#pragma unroll
    for (int u = 0; u < kPrefetch; ++u)
        if (c0 + u < c1)
            load(u, c0 + u);

    floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int c = c0; c < c1; c += kPrefetch) {
#pragma unroll
        for (int u = 0; u < kPrefetch; ++u) {
            if (c + u < c1) {
                gemv_tile<R>(cw[u], sw[u], xw[u], acc);
                if (c + u + kPrefetch < c1)
                    load(u, c + u + kPrefetch);
            }
        }
    }

    if (S > 1) {
        __shared__ floatx4_t red[kMaxSplit][64];
        red[w][lane] = acc;
        __syncthreads();
        if (w == 0) {
            acc = red[0][lane];
            for (int v = 1; v < S; ++v)
                acc += red[v][lane];
        }
    }
    if (w == 0) {
        // lane (r, gq) holds outputs y[4*gq + i][16*t + r], i = 0..3
        const int n = 16 * t + r;
        if (n < N) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 4 * gq + i;
                if (m < M)
                    y[(int64_t)m * N + n] = g * acc[i];
            }
        }
    }
}

// k-splits per row tile: enough waves to cover the chip several times over,
// at least 4 k-tiles per wave, at most kMaxSplit waves per workgroup.
int choose_split(int64_t NT, int64_t KT)
{
    const int64_t target_waves = 4096;
    int64_t s = (target_waves + NT - 1) / NT;
    if (s > KT / 4)
        s = KT / 4;
    if (s > kMaxSplit)
        s = kMaxSplit;
    if (s < 1)
        s = 1;
    return (int)s;
}

}  // namespace

hipError_t launch_gemv(const uint8_t *packed_codes, const uint8_t *packed_scales, float g,
                       const uint16_t *x, float *y, int64_t M, int64_t N, int64_t K,
                       hipStream_t stream)
{
    const int64_t NT = n_tiles(N);
    const int64_t KT = k_tiles(K);
    const int S = choose_split(NT, KT);
    const dim3 grid((unsigned)NT), block(64 * S);
    const uint4 *pc = reinterpret_cast<const uint4 *>(packed_codes);
    const uint2 *ps = reinterpret_cast<const uint2 *>(packed_scales);
    const int m = (int)M, n = (int)N, k = (int)K, kt = (int)KT;
    switch (M < 4 ? M : 4) {
    case 1: hipLaunchKernelGGL(gemv_kernel<1>, grid, block, 0, stream, pc, ps, g, x, y, m, n, k, kt, S); break;
    case 2: hipLaunchKernelGGL(gemv_kernel<2>, grid, block, 0, stream, pc, ps, g, x, y, m, n, k, kt, S); break;
    case 3: hipLaunchKernelGGL(gemv_kernel<3>, grid, block, 0, stream, pc, ps, g, x, y, m, n, k, kt, S); break;
    default: hipLaunchKernelGGL(gemv_kernel<4>, grid, block, 0, stream, pc, ps, g, x, y, m, n, k, kt, S); break;
    }
    return hipGetLastError();
}

}  // namespace q4p
