// q4p_quant.hip — NVFP4 quantizer: bf16 W [N][K] -> canonical e2m1 codes,
// e4m3 block scales and the fp32 global scale.
//
// The FlashRT "Qwen3.6 NVFP4 usage" page converts a checkpoint to NVFP4 at
// load time (its MTP checkpoint entry: FP8 -> BF16 -> NVFP4).  Two-level
// recipe, every rounding decision one IEEE fp32 operation in this order:
//     amax = max |w|,   g = amax / 2688   (g = 1 when amax == 0)
//   per 16-element block:
//     t = (amax_b / 6) / g,   s = e4m3 nearest to t (ties to even, <= 448)
//     unit = e4m3(s) * g,     inv = 1 / unit
//   per element:
//     r = |w| * inv,   code = e2m1 magnitude nearest to r (ties to the even
//     code, <= 6; NaN -> 0), bit 3 = sign of w; all codes 0 when unit == 0.
//
// Two launches, both bound by HBM: (1) a grid-stride max of |w| into one slot
// per workgroup; (2) every workgroup of the quantize launch first reduces
// those slots itself (a few KB, L2-resident), so all of them derive the same
// g with no further synchronisation and no scratch state survives the call.
// A thread owns one 16-element block: 32 B in, 8 B of codes and 1 scale out,
// consecutive lanes on consecutive blocks (contiguous wave segments).
//
// Element rounding uses gfx950's fp32 -> fp4 conversion with scale 1.0 on
// w * inv (sign kept): checked on the device against the nearest-even rule
// above for every non-NaN fp32 input (ties, saturation at 6, infinities,
// negative zero -> code 8 all agree).  It returns a nonzero code for NaN, and
// w * inv is NaN only for w = 0 with inv = inf (unit below 2^-128), so such
// blocks take the threshold form instead.  This cuts the loop from ~24 VALU
// per element to ~3, which is what kept the pass below the HBM rate.
#include "q4p_device.h"
#include "q4p_launch.h"

namespace q4p {

namespace {

constexpr int kQuantThreads = 256;
constexpr int kAmaxGroups = 1024;        // slots of the |w| max
constexpr int kQuantGroups = 4096;       // grid-stride quantize launch

// max of the eight |bf16| in v as bit patterns (non-negative bf16 compare as
// integers)
__device__ __forceinline__ uint32_t absmax8(uint4 v)
{
    uint32_t m = 0;
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo = w[i] & 0x7FFFu, hi = (w[i] >> 16) & 0x7FFFu;
        m = max(m, max(lo, hi));
    }
    return m;
}

__device__ __forceinline__ uint32_t wave_max(uint32_t m)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
    return m;
}

// max over the workgroup (kQuantThreads threads); every thread gets it
__device__ __forceinline__ uint32_t group_max(uint32_t m, uint32_t *red)
{
    m = wave_max(m);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0)
        red[wave] = m;
    __syncthreads();
    m = red[0];
#pragma unroll
    for (int i = 1; i < kQuantThreads / 64; ++i)
        m = max(m, red[i]);
    return m;
}

__global__ void __launch_bounds__(kQuantThreads)
quant_amax_kernel(const uint4 *__restrict__ w, int64_t n16, uint32_t *__restrict__ slots)
{
    __shared__ uint32_t red[kQuantThreads / 64];
    uint32_t m = 0;
    const int64_t stride = (int64_t)gridDim.x * kQuantThreads;
    for (int64_t i = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x; i < n16; i += stride)
        m = max(m, absmax8(w[i]));
    m = group_max(m, red);
    if (threadIdx.x == 0)
        slots[blockIdx.x] = m;
}

// e4m3 code nearest to t (0 <= t, finite), ties to the even code, values
// above 448 saturating to 448 (0x7E)
__device__ __forceinline__ uint32_t e4m3_nearest(float t)
{
    if (t > 448.0f)
        return 0x7Eu;
    if (t < 0.015625f)                                   // below 2^-6: step 2^-9
        return (uint32_t)__builtin_rintf(t * 512.0f);   // 0..8 (8 = 2^-6 = 0x08)
    const uint32_t b = __builtin_bit_cast(uint32_t, t);
    uint32_t e = (b >> 23) - 120u;                       // biased e4m3 exponent 1..15
    uint32_t keep = (b >> 20) & 7u;
    const uint32_t rest = b & 0xFFFFFu;
    if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u)))
        ++keep;
    if (keep == 8u) {
        keep = 0;
        ++e;
    }
    const uint32_t c = (e << 3) | keep;
    return c > 0x7Eu ? 0x7Eu : c;
}

// e2m1 magnitude code nearest to r (ties to the even code, above 6 -> 6,
// NaN -> 0): the number of decision points r has passed
__device__ __forceinline__ uint32_t e2m1_nearest(float r)
{
    return (uint32_t)(r > 0.25f) + (uint32_t)(r >= 0.75f) + (uint32_t)(r > 1.25f) +
           (uint32_t)(r >= 1.75f) + (uint32_t)(r > 2.5f) + (uint32_t)(r >= 3.5f) +
           (uint32_t)(r > 5.0f);
}

// two fp32 -> two e2m1 codes (a low nibble, b high) in byte SEL of old, the
// other bytes kept
template <int SEL>
__device__ __forceinline__ uint32_t fp4_pair(uint32_t old, float a, float b)
{
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, SEL);
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __builtin_bit_cast(float, v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __builtin_bit_cast(float, v & 0xFFFF0000u); }

__global__ void __launch_bounds__(kQuantThreads)
quant_kernel(const uint4 *__restrict__ w, int64_t nblk, const uint32_t *__restrict__ slots,
             int nslots, uint2 *__restrict__ codes, uint8_t *__restrict__ scales,
             float *__restrict__ gout)
{
    __shared__ uint32_t red[kQuantThreads / 64];
    uint32_t m = 0;
    for (int i = threadIdx.x; i < nslots; i += kQuantThreads)
        m = max(m, slots[i]);
    m = group_max(m, red);
    const float amax = __builtin_bit_cast(float, m << 16);
    const float g = amax == 0.0f ? 1.0f : amax / 2688.0f;
    if (blockIdx.x == 0 && threadIdx.x == 0)
        *gout = g;

    const int64_t stride = (int64_t)gridDim.x * kQuantThreads;
    for (int64_t b = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x; b < nblk; b += stride) {
        const uint4 v0 = w[2 * b], v1 = w[2 * b + 1];
        const uint32_t wd[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        const float amax_b = bf16_lo(max(absmax8(v0), absmax8(v1)));
        const float t = (amax_b / 6.0f) / g;
        const uint32_t s = e4m3_nearest(t);
        const float unit = e4m3_to_f32<0>(s) * g;
        const float inv = 1.0f / unit;
        uint32_t out[2] = {0u, 0u};
        if (unit != 0.0f && inv != __builtin_inff()) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                // elements 2i, 2i+1 -> byte i: low nibble 2i, high nibble 2i+1
                const float a = bf16_lo(wd[i]) * inv, b2 = bf16_hi(wd[i]) * inv;
                switch (i & 3) {
                case 0: out[i >> 2] = fp4_pair<0>(out[i >> 2], a, b2); break;
                case 1: out[i >> 2] = fp4_pair<1>(out[i >> 2], a, b2); break;
                case 2: out[i >> 2] = fp4_pair<2>(out[i >> 2], a, b2); break;
                default: out[i >> 2] = fp4_pair<3>(out[i >> 2], a, b2); break;
                }
            }
        } else if (unit != 0.0f) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                // elements 2i (low half) and 2i+1 (high half) -> one byte
                const uint32_t qlo = e2m1_nearest(__builtin_fabsf(bf16_lo(wd[i])) * inv) |
                                     ((wd[i] >> 12) & 8u);
                const uint32_t qhi = e2m1_nearest(__builtin_fabsf(bf16_hi(wd[i])) * inv) |
                                     ((wd[i] >> 28) & 8u);
                out[i >> 2] |= (qlo | (qhi << 4)) << (8 * (i & 3));
            }
        }
        codes[b] = make_uint2(out[0], out[1]);
        scales[b] = (uint8_t)s;
    }
}

}  // namespace

size_t quant_workspace_bytes() { return (size_t)kAmaxGroups * sizeof(uint32_t); }

hipError_t launch_quantize(const uint16_t *w, int64_t N, int64_t K, uint8_t *codes,
                           uint8_t *scales, float *global_scale, void *workspace,
                           hipStream_t stream)
{
    const int64_t total = N * K;                 // elements, a multiple of 16
    const int64_t n16 = total / 8;               // 16-byte chunks
    const int64_t nblk = total / 16;             // scale blocks
    int64_t ga = (n16 + kQuantThreads - 1) / kQuantThreads;
    if (ga > kAmaxGroups)
        ga = kAmaxGroups;
    int64_t gq = (nblk + kQuantThreads - 1) / kQuantThreads;
    if (gq > kQuantGroups)
        gq = kQuantGroups;
    uint32_t *slots = static_cast<uint32_t *>(workspace);
    hipLaunchKernelGGL(quant_amax_kernel, dim3((unsigned)ga), dim3(kQuantThreads), 0, stream,
                       reinterpret_cast<const uint4 *>(w), n16, slots);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(quant_kernel, dim3((unsigned)gq), dim3(kQuantThreads), 0, stream,
                       reinterpret_cast<const uint4 *>(w), nblk, slots, (int)ga,
                       reinterpret_cast<uint2 *>(codes), scales, global_scale);
    return hipGetLastError();
}

}  // namespace q4p
