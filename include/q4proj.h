/*
 * q4proj.h — NVFP4 weight-only linear projection on AMD MI355X (gfx950).
 *
 *     y[m][n] = sum_k x[m][k] * W[n][k],    W[n][k] = e2m1(q[n][k]) * e4m3(s[n][k/16]) * g
 *
 * The operation is the projection behind the batch-one NVFP4 runners described
 * on the Qwen3x-Orin README (section "Functional evaluation quick start": the
 * SM87 projection backend with 512-row prefill chunks) and on the FlashRT
 * "Qwen3.6 NVFP4 usage" page (speculative decoding section: verify runs K+1
 * rows at once, 1 <= K <= 15; plain decode section: one row per step).  The
 * weight format is the compressed-tensors NVFP4 checkpoint named in that
 * page's constructor-argument table: e2m1 codes two per byte, one fp8-e4m3
 * scale per 16 consecutive k, one fp32 per-tensor global scale g.
 *
 * Element formats.  e2m1 per the OCP Microscaling Formats v1.0 FP4 element
 * (values 0, .5, 1, 1.5, 2, 3, 4, 6 and their negatives); e4m3 per the OCP
 * 8-bit floating point spec, "fn" variant (bias 7, max 448, S.1111.111 = NaN,
 * no infinities).  A NaN block scale makes every output of its row NaN.
 *
 * Canonical (caller) layouts, all row-major and densely packed:
 *     codes   uint8   [N][K/2]   element 2j in bits 3:0, element 2j+1 in bits 7:4
 *     scales  uint8   [N][K/16]  e4m3 bit patterns
 *     x       uint16  [M][K]     bf16 bit patterns
 *     y       float   [M][N]
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers owned by the caller; the library neither
 *     allocates nor frees memory, keeps no state between calls except a cached
 *     device check, and is reentrant.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Calls
 *     enqueue work on it and return without synchronising.
 *   - Arguments are validated on the host before anything is launched; on any
 *     error nothing is enqueued and a status code is returned.
 *   - Outputs must not alias inputs.
 *   - The weight is packed once (q4proj_pack, the one-time weight swizzle done
 *     at construction on the FlashRT page); every projection reads the packed
 *     form, and gemv and gemm read the same packed buffers.
 */
#ifndef Q4PROJ_H
#define Q4PROJ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    Q4P_OK = 0,
    Q4P_EINVAL = 1,       /* null pointer, non-positive size, K % 16 != 0, misalignment */
    Q4P_EUNSUPPORTED = 2, /* valid arguments outside an entry point's range (gemv M > 16) */
    Q4P_EDEVICE = 3,      /* current device is not gfx950, or no device */
    Q4P_EWORKSPACE = 4,   /* workspace smaller than q4proj_workspace_bytes() */
    Q4P_EHIP = 5          /* the HIP runtime reported an error at launch */
} q4proj_status;

/* Largest M accepted by q4proj_gemv: the verify shape K+1 with K <= 15. */
#define Q4PROJ_GEMV_MAX_M 16

/*
 * Sizes of the packed buffers for an N x K weight (0 if N <= 0, K <= 0 or
 * K % 16 != 0).  The packed layout pads N up to a multiple of 16 and K up to a
 * multiple of 128 with zero codes and zero scales:
 *     packed codes  = ceil(N/16) * ceil(K/128) * 1024 bytes  (>= N*K/2)
 *     packed scales = ceil(N/16) * ceil(K/128) * 128 bytes   (>= N*K/16)
 * The layout itself is private to the library; only q4proj_unpack reads it
 * back out.
 */
size_t q4proj_packed_codes_bytes(int64_t N, int64_t K);
size_t q4proj_packed_scales_bytes(int64_t N, int64_t K);

/*
 * Device scratch q4proj_gemv needs for (M, N, K), 1 <= M <= 16 (valid N, K):
 *     8 * (65536 + (KS - 1) * M * N) bytes,
 * where KS (1, 2, 4 or 8) is the number of ranges K is cut into.  One
 * range's activations, M * ceil(K/128) * 256 / KS bytes, must fit in the
 * 147,392 bytes of on-chip memory a workgroup stages them in; among the
 * counts that fit, the library picks the one its cost estimate (staging per
 * workgroup against joins through the workspace) rates fastest: KS = 1 for
 * every M = 1 shape up to K = 65536, KS = 4 for M = 7 at K = 17408.
 * 0 otherwise (the GEMM's optional workspace is q4proj_gemm_workspace_bytes).
 * The gemv workspace holds one 64-bit exchange word per output of the row
 * tiles that two workgroups share, and per output and join of the K ranges'
 * partial results.  Ownership and state:
 *   - owned by the caller, 8-byte aligned, not overlapping any other argument;
 *   - zero-filled by the caller before its first use; every call that
 *     completes leaves it zero-filled again, so it is reused as is;
 *   - calls that may run at the same time (different streams) need separate
 *     workspaces: two kernels swapping words in one workspace corrupt each
 *     other's sums (silently) and can leave words set;
 *   - a call that returns an error status enqueued nothing and left the
 *     workspace as it was; only a kernel that did not run to completion (a
 *     device fault, a killed process) can leave words set, after which the
 *     workspace must be zero-filled again before it is reused.
 */
size_t q4proj_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * q4proj_pack — the one-time weight swizzle.
 * In:  codes [N][K/2] and scales [N][K/16] in the canonical layout above.
 * Out: packed_codes (q4proj_packed_codes_bytes(N,K) bytes) and packed_scales
 *      (q4proj_packed_scales_bytes(N,K) bytes), laid out for 128-bit,
 *      wave-contiguous loads by the projection kernels.  Padding is written
 *      with zeros.  A pure byte permutation: no value is decoded or changed.
 * Errors: EINVAL (null pointer, N <= 0, K <= 0, K % 16 != 0, in-place call),
 *         EDEVICE, EHIP.
 */
q4proj_status q4proj_pack(const uint8_t *codes, const uint8_t *scales, int64_t N,
                          int64_t K, uint8_t *packed_codes, uint8_t *packed_scales,
                          void *stream);

/*
 * q4proj_unpack — exact inverse of q4proj_pack (padding is dropped).
 * Errors: as q4proj_pack.
 */
q4proj_status q4proj_unpack(const uint8_t *packed_codes, const uint8_t *packed_scales,
                            int64_t N, int64_t K, uint8_t *codes, uint8_t *scales,
                            void *stream);

/*
 * q4proj_gemv — decode and speculative-verify projection, 1 <= M <= 16.
 *     y[M][N] (fp32) = x[M][K] (bf16) . dequant(W)^T, fp32 accumulation.
 * Streams the packed weight once.  Each 16-element block's partial sum is
 * formed from the unscaled e2m1 values and multiplied by its e4m3 scale; g is
 * applied once per output after accumulation.  Deterministic: the same inputs
 * give the same bits on every call.
 * x must be 16-byte aligned (K % 16 == 0 keeps every row aligned).
 * workspace: q4proj_workspace_bytes(M, N, K) bytes, zero-filled before first
 * use (see above); NULL only when that size is 0.
 * Errors: EINVAL (null pointer, M/N/K <= 0, K % 16 != 0, misaligned x or
 *         workspace, workspace overlapping an argument),
 *         EUNSUPPORTED (M > 16), EWORKSPACE (workspace_bytes too small),
 *         EDEVICE, EHIP.
 */
q4proj_status q4proj_gemv(const uint8_t *packed_codes, const uint8_t *packed_scales,
                          float global_scale, const uint16_t *x, float *y, int64_t M,
                          int64_t N, int64_t K, void *workspace, size_t workspace_bytes,
                          void *stream);

/*
 * Optional device scratch of q4proj_gemm and q4proj_gemm_silu_mul for M rows
 * of K activations (N does not matter; 0 for invalid arguments):
 *     roundup256(2 * M * K) + roundup256(4 * M) bytes.
 * With it the call first stages the activations there as fp16 (each row
 * scaled by a power of two so that the copy is exact, plus one output
 * multiplier per row) and runs fp16 matrix-core instructions, which need a
 * third of the weight-decoding work of the bf16 ones; rows that fp16 cannot
 * hold exactly (a row spanning more than 29 binades of nonzero magnitudes,
 * or a global scale whose row multiplier would leave the normal range) keep
 * bf16 for their 128-row block.  Every product is exact either way and the
 * sums run in the same order, so the results equal those without a
 * workspace bit for bit (barring fp32 overflow or underflow of the unscaled
 * sums).  Ownership: the caller's, 16-byte aligned, overlapping no other
 * argument; no contents are required on entry and the call leaves its
 * scratch there, so it must not share memory with a gemv, silu or argmax
 * workspace (those must stay zero-filled).  Calls that may overlap in time
 * (different streams) need separate workspaces.
 */
size_t q4proj_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * q4proj_gemm — prefill-chunk projection, any M >= 1 (sized for M = 512).
 * Same arguments and result definition as q4proj_gemv.  Dequantises weight
 * tiles exactly (q*s has at most 6 significant bits) and runs matrix-core
 * instructions with fp32 accumulation; g is applied once per output after
 * accumulation.  Deterministic.
 * workspace: NULL (workspace_bytes ignored): bf16 operands; or at least
 * q4proj_gemm_workspace_bytes(M, N, K) bytes as described there: fp16
 * operands, the same results, faster.
 * Errors: EINVAL (as q4proj_gemv; also a misaligned or overlapping
 *         workspace), EWORKSPACE (a workspace smaller than required),
 *         EDEVICE, EHIP.
 */
q4proj_status q4proj_gemm(const uint8_t *packed_codes, const uint8_t *packed_scales,
                          float global_scale, const uint16_t *x, float *y, int64_t M,
                          int64_t N, int64_t K, void *workspace, size_t workspace_bytes,
                          void *stream);

/*
 * q4proj_gemv_noalloc — q4proj_gemv for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same projection, arguments and result as
 * q4proj_gemv, without the workspace.  The exchange words live in a device
 * array inside the library instead: 8 MiB per GPU, allocated when the
 * library's code is loaded on that GPU and held until the process ends;
 * the call itself allocates and frees nothing.
 * Limit: shapes whose q4proj_workspace_bytes(M, N, K) exceeds 8 MiB return
 * EWORKSPACE before any launch (e.g. M >= 13 on a 248320 x 5120 lm-head);
 * every M = 1 shape the stream-K GEMV serves fits.
 * State: all calls on one GPU share that GPU's array.  It is zero-filled on
 * the first call on each GPU (by a kernel on that call's stream) and every
 * completed call leaves it zero-filled, so calls issued one after another
 * need nothing more.  Calls that may overlap on one GPU (different streams
 * without ordering between them) race on the array and corrupt each other's
 * results: serialise them, or use q4proj_gemv with separate workspaces.
 * Errors: as q4proj_gemv, with EWORKSPACE for shapes beyond the limit.
 */
q4proj_status q4proj_gemv_noalloc(const uint8_t *packed_codes, const uint8_t *packed_scales,
                                  float global_scale, const uint16_t *x, float *y, int64_t M,
                                  int64_t N, int64_t K, void *stream);

/*
 * Device scratch q4proj_gemv_silu_mul needs for (M, F, K):
 *     8 * (65536 + (KS - 1) * M * F) bytes,
 * with KS the number of K ranges as for q4proj_gemv (the joins carry a gate
 * and an up value in one word, so each join needs M * F words).  0 when the
 * entry point does not serve the shape: M outside 1..16, F <= 0 or
 * F % 8 != 0, invalid K, or K so long that even eight ranges' activations
 * exceed 128 KiB (M * ceil(ceil(K/128) / 8) * 256 > 131072, e.g. K > 32768 at
 * M = 16).  Ownership and state as for q4proj_workspace_bytes; the two entry
 * points may share one workspace (of the larger size) on one stream.
 */
size_t q4proj_silu_mul_workspace_bytes(int64_t M, int64_t F, int64_t K);

/*
 * q4proj_gemv_silu_mul — the MLP gate and up projections fused into one
 * NVFP4 GEMV with the SiLU-times-up epilogue, 1 <= M <= 16.  The FlashRT
 * "Qwen3.6 NVFP4 usage" page runs gate/up as one fused NVFP4 projection when
 * the two weights' global scales are equal, followed by a fused silu(gate)*up
 * (its environment-variable table); here the epilogue writes bf16.
 *     gate[m][f] = sum_k x[m][k] * dequant(W)[16(f/8) + f%8][k]
 *     up[m][f]   = sum_k x[m][k] * dequant(W)[16(f/8) + 8 + f%8][k]
 *     h[m][f]    = bf16( silu(gate) * up ),  silu(z) = z / (1 + exp(-z))
 * gate and up are fp32 sums as in q4proj_gemv, each scaled by the one global
 * scale g; silu and the product are evaluated in fp32 and rounded to bf16
 * (nearest even).
 * W is the fused [2F][K] weight, packed with q4proj_pack(N = 2F, K): its rows
 * alternate blocks of 8 gate rows and 8 up rows (gate rows 8p..8p+7 at
 * 16p..16p+7, up rows 8p..8p+7 at 16p+8..16p+15), so every 16-row tile of
 * the packed layout holds both halves of its 8 outputs.  F % 8 == 0.
 *     x  uint16 [M][K] bf16 bit patterns, 16-byte aligned
 *     h  uint16 [M][F] bf16 bit patterns (output), 2-byte aligned
 * workspace: q4proj_silu_mul_workspace_bytes(M, F, K) bytes, zero-filled
 * before first use, left zero-filled by every completed call.
 * Deterministic: the same inputs give the same bits on every call.
 * Errors: EINVAL (null pointer, M/F/K <= 0, F % 8 != 0, K % 16 != 0,
 *         misaligned x, h or workspace, h or workspace overlapping an input),
 *         EUNSUPPORTED (M > 16, or K too long as above), EWORKSPACE,
 *         EDEVICE, EHIP.
 */
q4proj_status q4proj_gemv_silu_mul(const uint8_t *packed_codes, const uint8_t *packed_scales,
                                   float global_scale, const uint16_t *x, uint16_t *h,
                                   int64_t M, int64_t F, int64_t K, void *workspace,
                                   size_t workspace_bytes, void *stream);

/*
 * q4proj_pack_gate_up — the packed fused gate/up weight built from a
 * checkpoint's separate gate and up NVFP4 weights.  The FlashRT "Qwen3.6
 * NVFP4 usage" page (environment-variable table) fuses the MLP gate and up
 * projections into one NVFP4 projection when the two weights' global scales
 * are equal; this call is that fusion at load time.
 * In:  gate_codes, up_codes  uint8 [F][K/2] canonical codes, 8-byte aligned
 *      gate_scales, up_scales uint8 [F][K/16] canonical e4m3 scales
 *      gate_global_scale, up_global_scale: the two weights' global scales,
 *      which must be equal bit for bit (the fused projections take one g);
 *      F % 8 == 0.
 * Out: packed_codes (q4proj_packed_codes_bytes(2F, K) bytes, 16-byte aligned)
 *      and packed_scales (q4proj_packed_scales_bytes(2F, K) bytes): the same
 *      bytes q4proj_pack writes for the [2F][K] weight whose rows alternate
 *      8 gate rows and the matching 8 up rows (the layout q4proj_gemv_silu_mul
 *      and q4proj_gemm_silu_mul read).  A pure byte permutation.
 * Errors: EINVAL (null pointer, F <= 0, F % 8 != 0, K <= 0, K % 16 != 0,
 *         unequal or NaN global scales, misaligned buffers, an output
 *         overlapping an input or the other output), EDEVICE, EHIP.
 */
q4proj_status q4proj_pack_gate_up(const uint8_t *gate_codes, const uint8_t *gate_scales,
                                  const uint8_t *up_codes, const uint8_t *up_scales,
                                  float gate_global_scale, float up_global_scale, int64_t F,
                                  int64_t K, uint8_t *packed_codes, uint8_t *packed_scales,
                                  void *stream);

/*
 * q4proj_gemm_silu_mul — the same fused gate/up projection and epilogue as
 * q4proj_gemv_silu_mul for any M >= 1 (sized for the M = 512 prefill chunk):
 * the bf16 matrix-core projection of q4proj_gemm over the fused [2F][K]
 * weight, h[M][F] = bf16(silu(g*gate) * (g*up)) written in place of y.
 * Same layouts and result definition as q4proj_gemv_silu_mul.  workspace:
 * as q4proj_gemm's, q4proj_gemm_workspace_bytes(M, 2F, K) bytes or NULL.
 * Deterministic.
 * Errors: EINVAL (null pointer, M/F/K <= 0, F % 8 != 0, K % 16 != 0,
 *         misaligned x, h or workspace, h or workspace overlapping an
 *         input), EWORKSPACE (a workspace smaller than required), EDEVICE,
 *         EHIP.
 */
q4proj_status q4proj_gemm_silu_mul(const uint8_t *packed_codes, const uint8_t *packed_scales,
                                   float global_scale, const uint16_t *x, uint16_t *h,
                                   int64_t M, int64_t F, int64_t K, void *workspace,
                                   size_t workspace_bytes, void *stream);

/*
 * Device scratch q4proj_gemv_argmax needs for (M, N, K): the q4proj_gemv
 * workspace of the same shape plus 8 * (M + 1) bytes (one 64-bit key per row
 * and a completion counter); 0 when the entry point does not serve the shape
 * (as q4proj_gemv_silu_mul: M outside 1..16, invalid N/K, or K past the
 * eight-range limit).  Zero-filled by the caller before first use, left
 * zero-filled by every completed call; one per stream.
 */
size_t q4proj_argmax_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * q4proj_gemv_argmax — the lm-head GEMV with a fused greedy argmax,
 * 1 <= M <= 16.  The FlashRT "Qwen3.6 NVFP4 usage" page decodes greedily
 * only (speculative-decode section: the public path is greedy, a
 * deterministic argmax sequence) and picks each token as the argmax of the
 * logits row (its per-step forward example); verify takes the argmax of each
 * of its K+1 rows.
 *     logits[m][n] = y[m][n] as q4proj_gemv computes it (fp32)
 *     max_idx[m]   = the first n with the largest logits[m][n]; NaN counts
 *                    as larger than every number and -0 equals +0
 *     max_val[m]   = logits[m][max_idx[m]]   (bit for bit, a NaN as the
 *                    canonical quiet NaN)
 * y may be NULL: then the logits are not written at all.  The decision is
 * taken on the fp32 logits the kernel computes; deterministic.
 *     max_val float [M], max_idx int64 [M]: device memory, 4- and 8-byte
 *     aligned.
 * Errors: EINVAL (null pointer other than y, M/N/K <= 0, K % 16 != 0,
 *         misalignment, outputs overlapping inputs or each other, workspace
 *         overlapping any argument), EUNSUPPORTED (M > 16, or K too long),
 *         EWORKSPACE, EDEVICE, EHIP.
 */
q4proj_status q4proj_gemv_argmax(const uint8_t *packed_codes, const uint8_t *packed_scales,
                                 float global_scale, const uint16_t *x, float *y,
                                 float *max_val, int64_t *max_idx, int64_t M, int64_t N,
                                 int64_t K, void *workspace, size_t workspace_bytes,
                                 void *stream);

/*
 * Device scratch q4proj_quantize needs: 4096 bytes for every valid (N, K),
 * 0 otherwise.  No initial contents are required and none are kept between
 * calls; calls that may run at the same time need separate workspaces.
 */
size_t q4proj_quantize_workspace_bytes(int64_t N, int64_t K);

/*
 * q4proj_quantize — the load-time NVFP4 conversion of a bf16 weight (the
 * FlashRT "Qwen3.6 NVFP4 usage" page converts its MTP checkpoint FP8 ->
 * BF16 -> NVFP4 when the runner is constructed), producing the canonical
 * codes and scales that q4proj_pack takes, and the global scale.
 * In:  w       uint16 [N][K] bf16 bit patterns, finite, 16-byte aligned.
 * Out: codes   uint8 [N][K/2] (element 2j in the low nibble), 8-byte aligned
 *      scales  uint8 [N][K/16] e4m3
 *      global_scale  one float in DEVICE memory (copy it to the host once to
 *      pass it by value to the projections).
 * Two-level recipe, every rounding decision exact:
 *      amax = max |w|;  g = fp32(amax / 2688) (6 * 448; g = 1 when amax == 0)
 *      per 16-element block (amax_b = its max |w|): s = the e4m3 code
 *      (0..0x7E) whose value is nearest to the exact quotient
 *      amax_b / (6 g), ties to the even code (beyond 448: 448);
 *      per element: the e2m1 magnitude nearest to the exact quotient
 *      |w| / (e4m3(s) g), ties to the even code (beyond 6: 6); the code's
 *      sign bit is w's sign bit; a block with s == 0 gets all-zero codes.
 * Deterministic.  The result for non-finite w is unspecified (no fault).
 * Errors: EINVAL (null pointer, N/K <= 0, K % 16 != 0, misaligned w or
 *         codes, overlapping buffers), EWORKSPACE, EDEVICE, EHIP.
 */
q4proj_status q4proj_quantize(const uint16_t *w, int64_t N, int64_t K, uint8_t *codes,
                              uint8_t *scales, float *global_scale, void *workspace,
                              size_t workspace_bytes, void *stream);

/* Human-readable name of a status code (static storage, never NULL). */
const char *q4proj_status_string(q4proj_status s);

/* Last HIP error string recorded by a Q4P_EHIP return on this thread. */
const char *q4proj_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* Q4PROJ_H */
