// q4p_device.h — packed weight layout and per-lane fragment decoders for gfx950.
//
// Packed layout (the one-time weight swizzle; the FlashRT "Qwen3.6 NVFP4
// usage" page does an NVFP4 swizzle at construction, redesigned here for
// 64-wide wavefronts and CDNA4 matrix cores):
//
//   The N x K weight is cut into tiles of 16 rows x 128 k (eight 16-element
//   scale blocks).  Tiles are stored row-tile major, k-tile minor:
//       tile (t, c) = rows 16t..16t+15, k 128c..128c+127,  index t*KT + c.
//   Code tile: 1024 bytes = 64 lanes x 16 bytes.  Lane l = 16*g + r holds row
//   r and, for each block b = 0..7, the four codes k = 128c + 16b + 4g + {0..3}
//   in bytes 2b (codes 4g, 4g+1) and 2b+1 (codes 4g+2, 4g+3), low nibble first
//   exactly as in the canonical layout.  One 128-bit load per lane fetches a
//   1 KB contiguous wave-wide segment.
//   Scale tile: 128 bytes = 16 rows x 8 blocks, byte 8r + b = e4m3 scale of
//   row 16t + r, block 8c + b.
//   Padding rows (n >= N) and columns (k >= K) hold code 0 and scale 0.
//
// With this layout lane (r, g) of a wave owns, for every scale block, the four
// k-values that a 16x16x16 bf16 MFMA assigns to k-group g of column r.  The
// GEMV uses that directly (one MFMA per block, scale applied to the partial
// sum); the GEMM feeds two blocks per 16x16x32 MFMA with the scale folded
// into the bf16 operand.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q4p_layout.h"

namespace q4p {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float floatx2_t __attribute__((ext_vector_type(2)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// 16-byte load of data that is read exactly once (packed weights): marked
// non-temporal so it does not displace the activations from the caches.
__device__ __forceinline__ uint4 load_stream16(const uint4 *p)
{
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Two e2m1 codes (byte SEL of w, low nibble first) -> two bf16, unscaled.
// The hardware conversion multiplies by 2^exponent(scale) only; with 1.0 it is
// the exact e2m1 value.
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t w)
{
    bf16x2_t v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, SEL);
    return __builtin_bit_cast(uint32_t, v);
}

// Two e2m1 codes (byte SEL of w) times the decoded block scale s -> two bf16.
// q*s has at most 6 significant bits and lies in [2^-10, 2688] (or is 0, or
// NaN for a NaN scale), so the product and the bf16 rounding are exact.
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_scaled_to_bf16x2(uint32_t w, float s)
{
    floatx2_t f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
    bf16x2_t v = {(__bf16)(f[0] * s), (__bf16)(f[1] * s)};
    return __builtin_bit_cast(uint32_t, v);
}

// OCP e4m3 ("fn") byte SEL of w -> fp32.  gfx950's fp8 conversion decodes
// the OCP variant (bias 7, S.1111.111 = NaN), not the FNUZ one of gfx942.
template <int SEL>
__device__ __forceinline__ float e4m3_to_f32(uint32_t w)
{
    return __builtin_amdgcn_cvt_f32_fp8((int)w, SEL);
}

// silu(gate) * up in fp32, rounded to bf16 (nearest even): the epilogue of
// the fused gate/up projection
__device__ __forceinline__ uint16_t silu_mul_bf16(float gate, float up)
{
    const float h = gate / (1.0f + expf(-gate)) * up;
    return __builtin_bit_cast(uint16_t, (__bf16)h);
}

// lane r <- lane r ^ 8 within each 16-lane row (a row rotate by 8).  In a
// fused gate/up tile lane r < 8 holds a gate output and lane r + 8 the
// matching up output.  Every lane of the row must be active.
__device__ __forceinline__ float swap8(float v)
{
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));
}

}  // namespace q4p
