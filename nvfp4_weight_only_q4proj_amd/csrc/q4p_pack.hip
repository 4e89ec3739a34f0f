// q4p_pack.hip — the one-time weight swizzle (q4proj_pack) and its inverse.
//
// A pure byte permutation between the canonical layout (codes [N][K/2],
// scales [N][K/16]) and the tiled layout described in q4p_device.h.  One
// thread moves one (tile, row) pair: 64 canonical code bytes (one row of a
// 16 x 128 tile) become four 16-byte lane slots, and 8 scale bytes move as is.
//
// The fused gate/up pack reads two canonical [F][K] weights (a checkpoint's
// separate gate and up projections) and writes the packed layout of the
// [2F][K] weight whose rows alternate 8 gate rows and the matching 8 up rows:
// row 16t + r of the fused weight is gate row 8t + r for r < 8 and up row
// 8t + r - 8 otherwise.
#include "q4p_device.h"
#include "q4p_launch.h"

namespace q4p {

namespace {

// Canonical code bytes of row n, k-tile c: bytes [64c, 64c+64) of the row.
__device__ __forceinline__ void load_row_codes(const uint8_t *codes, int64_t N, int64_t K,
                                               int64_t n, int64_t c, uint16_t u[32])
{
    const int64_t row_bytes = K / 2;
    const int64_t b0 = 64 * c;
    if (n < N && b0 + 64 <= row_bytes) {
        // row start n*K/2 and b0 are multiples of 8 (K % 16 == 0)
        const uint2 *src = reinterpret_cast<const uint2 *>(codes + n * row_bytes + b0);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint2 v = src[i];
            u[4 * i + 0] = (uint16_t)(v.x & 0xFFFFu);
            u[4 * i + 1] = (uint16_t)(v.x >> 16);
            u[4 * i + 2] = (uint16_t)(v.y & 0xFFFFu);
            u[4 * i + 3] = (uint16_t)(v.y >> 16);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            int64_t b = b0 + 2 * i;   // row_bytes is even: a pair is all in or all out
            u[i] = (n < N && b < row_bytes)
                       ? (uint16_t)(codes[n * row_bytes + b] | (codes[n * row_bytes + b + 1] << 8))
                       : (uint16_t)0;
        }
    }
}

// FUSE: rows of the fused gate/up weight from (codes, scales) = gate and
// (codes2, scales2) = up, each with N rows; otherwise one weight of N rows.
template <bool FUSE>
__global__ void __launch_bounds__(256)
pack_kernel(const uint8_t *__restrict__ codes, const uint8_t *__restrict__ scales,
            const uint8_t *__restrict__ codes2, const uint8_t *__restrict__ scales2, int64_t N,
            int64_t K, int64_t KT, int64_t total, uint8_t *__restrict__ pcodes,
            uint8_t *__restrict__ pscales)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= total)
        return;
    const int r = (int)(idx & 15);
    const int64_t tc = idx >> 4;               // tile index t*KT + c
    const int64_t t = tc / KT, c = tc % KT;
    // source weight and row of packed row 16t + r
    const uint8_t *src_codes = codes, *src_scales = scales;
    int64_t n = 16 * t + r;
    if (FUSE) {
        if (r >= 8) {
            src_codes = codes2;
            src_scales = scales2;
        }
        n = 8 * t + (r & 7);
    }

    uint16_t u[32];                            // u[4b + g]: block b, k-group g
    load_row_codes(src_codes, N, K, n, c, u);
    uint4 *dst = reinterpret_cast<uint4 *>(pcodes + tc * kTileCodeBytes);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        uint4 o;
        o.x = (uint32_t)u[4 * 0 + g] | ((uint32_t)u[4 * 1 + g] << 16);
        o.y = (uint32_t)u[4 * 2 + g] | ((uint32_t)u[4 * 3 + g] << 16);
        o.z = (uint32_t)u[4 * 4 + g] | ((uint32_t)u[4 * 5 + g] << 16);
        o.w = (uint32_t)u[4 * 6 + g] | ((uint32_t)u[4 * 7 + g] << 16);
        dst[16 * g + r] = o;
    }

    const int64_t row_blocks = K / 16;
    uint32_t s[2] = {0u, 0u};
#pragma unroll
    for (int b = 0; b < 8; ++b) {
        const int64_t kb = 8 * c + b;
        uint32_t v = (n < N && kb < row_blocks) ? src_scales[n * row_blocks + kb] : 0u;
        s[b >> 2] |= v << (8 * (b & 3));
    }
    uint2 so;
    so.x = s[0];
    so.y = s[1];
    *reinterpret_cast<uint2 *>(pscales + tc * kTileScaleBytes + 8 * r) = so;
}

__global__ void __launch_bounds__(256)
unpack_kernel(const uint8_t *__restrict__ pcodes, const uint8_t *__restrict__ pscales, int64_t N,
              int64_t K, int64_t KT, int64_t total, uint8_t *__restrict__ codes,
              uint8_t *__restrict__ scales)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= total)
        return;
    const int r = (int)(idx & 15);
    const int64_t tc = idx >> 4;
    const int64_t t = tc / KT, c = tc % KT;
    const int64_t n = 16 * t + r;
    if (n >= N)
        return;

    const uint4 *src = reinterpret_cast<const uint4 *>(pcodes + tc * kTileCodeBytes);
    uint16_t u[32];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        uint4 v = src[16 * g + r];
        u[4 * 0 + g] = (uint16_t)(v.x & 0xFFFFu);
        u[4 * 1 + g] = (uint16_t)(v.x >> 16);
        u[4 * 2 + g] = (uint16_t)(v.y & 0xFFFFu);
        u[4 * 3 + g] = (uint16_t)(v.y >> 16);
        u[4 * 4 + g] = (uint16_t)(v.z & 0xFFFFu);
        u[4 * 5 + g] = (uint16_t)(v.z >> 16);
        u[4 * 6 + g] = (uint16_t)(v.w & 0xFFFFu);
        u[4 * 7 + g] = (uint16_t)(v.w >> 16);
    }
    const int64_t row_bytes = K / 2;
    const int64_t b0 = 64 * c;
    if (b0 + 64 <= row_bytes) {
        uint2 *dst = reinterpret_cast<uint2 *>(codes + n * row_bytes + b0);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint2 v;
            v.x = (uint32_t)u[4 * i + 0] | ((uint32_t)u[4 * i + 1] << 16);
            v.y = (uint32_t)u[4 * i + 2] | ((uint32_t)u[4 * i + 3] << 16);
            dst[i] = v;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            int64_t b = b0 + 2 * i;
            if (b < row_bytes) {
                codes[n * row_bytes + b] = (uint8_t)(u[i] & 0xFFu);
                codes[n * row_bytes + b + 1] = (uint8_t)(u[i] >> 8);
            }
        }
    }

    const int64_t row_blocks = K / 16;
    const uint8_t *ps = pscales + tc * kTileScaleBytes + 8 * r;
#pragma unroll
    for (int b = 0; b < 8; ++b) {
        const int64_t kb = 8 * c + b;
        if (kb < row_blocks)
            scales[n * row_blocks + kb] = ps[b];
    }
}

}  // namespace

hipError_t launch_pack(const uint8_t *codes, const uint8_t *scales, int64_t N, int64_t K,
                       uint8_t *packed_codes, uint8_t *packed_scales, hipStream_t stream)
{
    const int64_t KT = k_tiles(K);
    const int64_t total = n_tiles(N) * KT * 16;
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(pack_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, codes,
                       scales, codes, scales, N, K, KT, total, packed_codes, packed_scales);
    return hipGetLastError();
}

hipError_t launch_pack_gate_up(const uint8_t *gate_codes, const uint8_t *gate_scales,
                               const uint8_t *up_codes, const uint8_t *up_scales, int64_t F,
                               int64_t K, uint8_t *packed_codes, uint8_t *packed_scales,
                               hipStream_t stream)
{
    const int64_t KT = k_tiles(K);
    const int64_t total = n_tiles(2 * F) * KT * 16;
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(pack_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, gate_codes,
                       gate_scales, up_codes, up_scales, F, K, KT, total, packed_codes,
                       packed_scales);
    return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t *packed_codes, const uint8_t *packed_scales, int64_t N,
                         int64_t K, uint8_t *codes, uint8_t *scales, hipStream_t stream)
{
    const int64_t KT = k_tiles(K);
    const int64_t total = n_tiles(N) * KT * 16;
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(unpack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, packed_codes,
                       packed_scales, N, K, KT, total, codes, scales);
    return hipGetLastError();
}

}  // namespace q4p
