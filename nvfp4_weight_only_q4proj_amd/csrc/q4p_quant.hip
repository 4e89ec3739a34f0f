// q4p_quant.hip — NVFP4 quantizer: bf16 W [N][K] -> canonical e2m1 codes,
// e4m3 block scales and the fp32 global scale.
//
// The FlashRT "Qwen3.6 NVFP4 usage" page converts a checkpoint to NVFP4 at
// load time (its MTP checkpoint entry: FP8 -> BF16 -> NVFP4).  Two-level
// recipe:
//     amax = max |w|,   g = fp32(amax / 2688)   (g = 1 when amax == 0)
//   per 16-element block, amax_b = max |w| over the block:
//     s    = the e4m3 code (0..0x7E) whose value is nearest to the exact
//            quotient amax_b / (6 g), ties to the even code
//   per element:
//     code = the e2m1 magnitude (0..7) nearest to the exact quotient
//            |w| / (e4m3(s) g), ties to the even code; bit 3 = sign of w;
//            all codes 0 when s == 0.
//
// The decisions are exact, not those of an fp32 evaluation of the quotients:
//  * scale: an fp32 estimate of the quotient (amax_b times a per-thread
//    1/(6g)) gives a code at most one away from the nearest; the two
//    midpoints around it are then compared with amax_b exactly.  A midpoint times 6 has at most 7 significant bits and g
//    24, so fma(6 mu, g, -amax_b) is the exact difference rounded once, and
//    its sign (zero included) is the exact comparison.
//  * codes: each element is converted twice, with 1/(e4m3(s) g) (the
//    hardware reciprocal, within 1 ulp) raised and lowered by 2^-19 (far more
//    than the few ulps the estimate w * inv can be off by), by
//    gfx950's fp32 -> fp4 conversion (nearest even, verified on the device
//    for every fp32 input).  The exact quotient lies strictly between the two
//    estimates and the rounding is monotone, so where both give the same
//    code for an element, that is the exact one.  Where they differ (an
//    element within ~2^-19 of a midpoint: about 0.2 % of the elements of
//    ordinary weights, as g = amax / 2688 and bf16 weights put many
//    quotients within 2^-23 of a midpoint) they are neighbours c, c + 1, and
//    one comparison with the midpoint between them decides: the midpoint
//    times e4m3(s) is exact in fp32 (at most 7 bits), and fma(mid * s, g,
//    -|w|) is again the exact difference rounded once.
//  * tiny tensors: when g < 2^-100 (or a block's e4m3(s) g < 2^-100) the
//    differences could fall below the smallest fp32 subnormal and round to
//    zero; both sides of every comparison are then multiplied by 2^64
//    (exact) and every element of the block is decided by comparisons with
//    all seven midpoints.
//
// Two launches, both bound by HBM: (1) a grid-stride max of |w| into one slot
// per workgroup; (2) every workgroup of the quantize launch first reduces
// those slots itself (a few KB, L2-resident), so all of them derive the same
// g with no further synchronisation and no scratch state survives the call.
// A thread owns one 16-element block: 32 B in, 8 B of codes and 1 scale out,
// consecutive lanes on consecutive blocks (contiguous wave segments).  The
// max pass reads with non-temporal loads, four in flight per thread; the
// quantize pass walks the blocks from the end backwards and reads through
// the caches, so the part of the tensor the last-level cache still holds
// from the max pass is read first (3-4 % less time than forward passes with
// plain loads on the 0.36 and 2.5 GB weights).
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

// 16 bytes of the weight for the max pass: a non-temporal load
__device__ __forceinline__ uint4 nt_load(const uint4 *p)
{
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
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
    int64_t i = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x;
    // four non-temporal loads in flight per thread, then the remainder one
    // at a time
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const uint4 v0 = nt_load(w + i), v1 = nt_load(w + i + stride), v2 = nt_load(w + i + 2 * stride),
                    v3 = nt_load(w + i + 3 * stride);
        m = max(max(m, absmax8(v0)), max(absmax8(v1), max(absmax8(v2), absmax8(v3))));
    }
    for (; i < n16; i += stride)
        m = max(m, absmax8(nt_load(w + i)));
    m = group_max(m, red);
    if (threadIdx.x == 0)
        slots[blockIdx.x] = m;
}

// e4m3 code nearest to t (0 <= t, finite, normal or zero), ties to the even
// code, values above 448 saturating to 448 (0x7E): the estimate that the
// exact comparisons below correct by at most one code
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

__device__ __forceinline__ float e4m3_value(uint32_t c) { return e4m3_to_f32<0>(c); }

// a / d has passed the midpoint lim / d (d > 0) between codes `upper` - 1 and
// `upper`: a > lim, or a == lim with `upper` even.  diff = lim - a, rounded
// once from the exact value (an fma), so its sign is exact.
__device__ __forceinline__ bool passed(float diff, uint32_t upper)
{
    return diff < 0.0f || (diff == 0.0f && !(upper & 1u));
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

// the eight element pairs of a block (words wd) -> codes, converting w * inv
template <typename T>
__device__ __forceinline__ void fp4_block(const uint32_t (&wd)[8], float inv, T (&out)[2])
{
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
}

// exact e2m1 magnitude code of |w| * 2^E / (v_s * g * 2^E): seven
// comparisons with the midpoints (each mu * v_s exact in fp32)
__device__ __forceinline__ uint32_t e2m1_exact(float aw, float vs, float gs)
{
    const float mu[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < 7; ++j)
        c += passed(__builtin_fmaf(mu[j] * vs, gs, -aw), (uint32_t)j + 1u) ? 1u : 0u;
    return c;
}

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
    // comparisons of tiny tensors run on values scaled by 2^64 (exact)
    const bool tiny = g < 0x1p-100f;
    const float gs = tiny ? g * 0x1p64f : g;
    const float escale = tiny ? 0x1p64f : 1.0f;
    // the scale estimate amax_b / (6 g) as a product (a few ulps from the
    // quotient, well inside the one-code margin the exact tests correct)
    const float r6gs = 1.0f / (6.0f * gs);

    const int64_t stride = (int64_t)gridDim.x * kQuantThreads;
    // blocks from the end of the tensor backwards (the first pass read it
    // forwards, so its tail is the part most likely still cached)
    for (int64_t bi = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x; bi < nblk; bi += stride) {
        const int64_t b = nblk - 1 - bi;
        const uint4 v0 = w[2 * b], v1 = w[2 * b + 1];
        const uint32_t wd[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        const float as = bf16_lo(max(absmax8(v0), absmax8(v1))) * escale;
        // scale: the estimate, then the exact test of the midpoints around it
        uint32_t s = e4m3_nearest(as * r6gs);
        if (s < 0x7Eu && passed(__builtin_fmaf(3.0f * (e4m3_value(s) + e4m3_value(s + 1)), gs, -as),
                                s + 1))
            ++s;
        else if (s > 0u && !passed(__builtin_fmaf(3.0f * (e4m3_value(s - 1) + e4m3_value(s)), gs,
                                                  -as),
                                   s))
            --s;
        const float vs = e4m3_value(s);
        uint32_t out[2] = {0u, 0u};
        const float unit = vs * g;
        if (s != 0u && !tiny && unit >= 0x1p-100f) {
            // the hardware reciprocal (1 ulp): with the roundings of unit and
            // of w * inv the estimate stays within 3 ulps, far inside 2^-19
            const float inv = __builtin_amdgcn_rcpf(unit);
            uint32_t hi[2] = {0u, 0u};
            fp4_block(wd, inv * (1.0f + 0x1p-19f), hi);
            fp4_block(wd, inv * (1.0f - 0x1p-19f), out);
            // elements whose two estimates differ lie within ~2^-19 of the
            // midpoint between magnitudes c (out) and c + 1 (hi): decide each
            // by one exact comparison with that midpoint
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint32_t d = hi[h] ^ out[h];
                while (d != 0u) {
                    const uint32_t sh = (uint32_t)__builtin_ctz(d) & ~3u;   // nibble of the element
                    const uint32_t e = sh >> 2;                             // element 8h + e
                    const uint32_t q = e >> 1;
                    const uint32_t word = q == 0 ? wd[4 * h] : q == 1 ? wd[4 * h + 1]
                                        : q == 2 ? wd[4 * h + 2] : wd[4 * h + 3];
                    const float aw = __builtin_fabsf((e & 1u) ? bf16_hi(word) : bf16_lo(word));
                    const uint32_t nib = (out[h] >> sh) & 15u;
                    const uint32_t c = nib & 7u;
                    // the two magnitudes c, c + 1 decoded as one byte
                    const floatx2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(
                        c | ((c + 1u) << 4), 1.0f, 0);
                    const float mu = 0.5f * (v2[0] + v2[1]);
                    const uint32_t cx =
                        c + (passed(__builtin_fmaf(mu * vs, g, -aw), c + 1u) ? 1u : 0u);
                    out[h] = (out[h] & ~(15u << sh)) | (((nib & 8u) | cx) << sh);
                    d &= ~(15u << sh);
                }
            }
        } else if (s != 0u) {
            // tiny scales: every element by the exact comparisons
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t qlo =
                    e2m1_exact(__builtin_fabsf(bf16_lo(wd[i])) * escale, vs, gs) |
                    ((wd[i] >> 12) & 8u);
                const uint32_t qhi =
                    e2m1_exact(__builtin_fabsf(bf16_hi(wd[i])) * escale, vs, gs) |
                    ((wd[i] >> 28) & 8u);
                const uint32_t byte = (qlo | (qhi << 4)) << (8 * (i & 3));
                out[i >> 2] = (i & 3) ? (out[i >> 2] | byte) : byte;
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
