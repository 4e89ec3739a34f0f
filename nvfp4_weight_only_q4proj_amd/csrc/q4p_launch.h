// q4p_launch.h — kernel launchers behind the C ABI (internal).
// Arguments are validated by the caller (q4p_api.cpp); launchers only size the
// grid, enqueue on `stream` and return hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4p {

hipError_t launch_pack(const uint8_t *codes, const uint8_t *scales, int64_t N, int64_t K,
                       uint8_t *packed_codes, uint8_t *packed_scales, hipStream_t stream);

// The fused gate/up weight's packed layout from two canonical [F][K]
// weights (F % 8 == 0): rows alternate 8 gate rows and 8 up rows.
hipError_t launch_pack_gate_up(const uint8_t *gate_codes, const uint8_t *gate_scales,
                               const uint8_t *up_codes, const uint8_t *up_scales, int64_t F,
                               int64_t K, uint8_t *packed_codes, uint8_t *packed_scales,
                               hipStream_t stream);

hipError_t launch_unpack(const uint8_t *packed_codes, const uint8_t *packed_scales, int64_t N,
                         int64_t K, uint8_t *codes, uint8_t *scales, hipStream_t stream);

// Device scratch q4proj_gemv needs (zero-filled before first use; each call
// leaves it zero-filled again).
size_t gemv_workspace_bytes(int64_t M, int64_t N, int64_t K);

hipError_t launch_gemv(const uint8_t *packed_codes, const uint8_t *packed_scales, float g,
                       const uint16_t *x, float *y, int64_t M, int64_t N, int64_t K,
                       void *workspace, hipStream_t stream);

// launch_gemv with the library's per-device scratch array as the workspace
// (no allocation); shapes whose workspace exceeds gemv_noalloc_max_bytes()
// must be refused by the caller.
size_t gemv_noalloc_max_bytes();
hipError_t launch_gemv_noalloc(const uint8_t *packed_codes, const uint8_t *packed_scales,
                               float g, const uint16_t *x, float *y, int64_t M, int64_t N,
                               int64_t K, hipStream_t stream);

// Fused gate/up projection + silu(gate)*up (weight of 2F rows, gate and up
// rows alternating in blocks of 8), for the shapes the stream-K GEMV serves,
// F % 8 == 0.
bool gemv_silu_mul_supported(int64_t M, int64_t F, int64_t K);
size_t gemv_silu_mul_workspace_bytes(int64_t M, int64_t F, int64_t K);

hipError_t launch_gemv_silu_mul(const uint8_t *packed_codes, const uint8_t *packed_scales,
                                float g, const uint16_t *x, uint16_t *h, int64_t M, int64_t F,
                                int64_t K, void *workspace, hipStream_t stream);

// Projection with a fused greedy-argmax epilogue (1 <= M <= 16, the shapes
// the stream-K GEMV serves); y may be null.  Workspace: zero-filled before
// first use, left zero-filled.
bool gemv_argmax_supported(int64_t M, int64_t N, int64_t K);
size_t gemv_argmax_workspace_bytes(int64_t M, int64_t N, int64_t K);

hipError_t launch_gemv_argmax(const uint8_t *packed_codes, const uint8_t *packed_scales, float g,
                              const uint16_t *x, float *y, float *best_val, int64_t *best_idx,
                              int64_t M, int64_t N, int64_t K, void *workspace,
                              hipStream_t stream);

// GEMM workspace: the fp16 copy of the activations and the per-row output
// multipliers (no initial contents; left holding them).  A null workspace
// runs the bf16 operand path.
size_t gemm_workspace_bytes(int64_t M, int64_t K);

hipError_t launch_gemm(const uint8_t *packed_codes, const uint8_t *packed_scales, float g,
                       const uint16_t *x, float *y, int64_t M, int64_t N, int64_t K,
                       void *workspace, hipStream_t stream);

// The fused gate/up projection + silu(gate)*up for any M (F % 8 == 0).
hipError_t launch_gemm_silu_mul(const uint8_t *packed_codes, const uint8_t *packed_scales,
                                float g, const uint16_t *x, uint16_t *h, int64_t M, int64_t F,
                                int64_t K, void *workspace, hipStream_t stream);

// NVFP4 quantizer: bf16 W [N][K] -> canonical codes, scales, global scale
// (device float).  workspace: quant_workspace_bytes(), no initial contents.
size_t quant_workspace_bytes();

hipError_t launch_quantize(const uint16_t *w, int64_t N, int64_t K, uint8_t *codes,
                           uint8_t *scales, float *global_scale, void *workspace,
                           hipStream_t stream);

}  // namespace q4p
