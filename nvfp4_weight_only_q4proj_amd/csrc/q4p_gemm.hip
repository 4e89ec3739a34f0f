// q4p_gemm.hip — prefill-chunk projection (sized for M = 512), any M >= 1.
//
// At M = 512 each weight is used 512 times: the work is a dense bf16
// contraction and belongs on the matrix cores.  Design:
//
//  * Workgroup = 8 waves, two per SIMD, covering kBM = 128 activation rows
//    and T weight-row tiles of 16 (BN = 16*T).  T is chosen so the grid has
//    about one workgroup per CU (256), e.g. T = 17 for N = 17408 and T = 14
//    for N = 14336 at M = 512: 256 equal workgroups, no tail wave.
//  * Waves w and w+4 (one SIMD) own the same outputs and split every k-tile:
//    wave w takes its first two 32-wide k-steps, wave w+4 the last two.  At
//    the end each hands the other, through LDS, the half of its partial sums
//    that the other finishes (four of the eight 16-row blocks of every tile),
//    so both waves of a SIMD share the epilogue.
//  * Each wave pair owns Q = T/4 whole weight tiles (all 128 rows) plus a
//    share of the RT = T%4 remaining tiles: half of one tile (64 rows) when
//    RT = 2, a quarter (32 rows) of each otherwise, so all waves do the same
//    number of MFMAs whatever T is.  A wave walks the eight 16-row blocks of
//    activations starting with its rows of the remaining tiles (block i ^ rb
//    for i = 0..7), so those MFMAs reuse the activation operands it reads
//    anyway.
//  * Operands reach LDS without passing through registers: per k-tile (128 k)
//    the 128 activation rows and the workgroup's T packed code tiles and
//    scale tiles are fetched with 16-byte buffer loads straight into one of
//    three LDS stages.  Offsets past the end of a buffer read as zero, which
//    covers rows past M, tiles past N and activations past K (lanes whose
//    chunk lies past K are pointed there), so the k-loop holds no LDS stores
//    of its own: the compiler then tracks the stage loads per LDS array and
//    never drains loads of a stage it is not reading.  Every wave issues the
//    same branch-free loads (a load with nothing to fetch writes zeros into a
//    spare 1 KB), with the k-tile advance in the scalar offset.
//  * MFMA k-order: in 16x16x32 step d, lane (r, gq) supplies k = 32d + 8gq
//    + 0..7, i.e. one 16-byte chunk of an activation row (one ds_read_b128).
//    Chunks are XOR-swizzled by row within LDS so the rows one read touches
//    fall in different banks.  The matching eight weight codes are halves of
//    two code slots of the packed tile (one byte permute); they share one
//    e4m3 scale.  The code slots are XOR-swizzled within the weight stage
//    too (code_pos), so the slots one read touches fall in different banks.
//  * Software pipeline: a wave's operands for its second k-step are
//    dequantised between the MFMAs of its first; one workgroup barrier per
//    k-tile sits between the two steps (past it, stage c+1 has landed
//    everywhere and stage c-1 is free); during the second step the loads of
//    k-tile c+2 go out and the next k-tile's code words are read and its
//    first step dequantised.  The matrix core never waits for a wave's own
//    dequantisation, only for issue slots: on gfx950 VALU work beside the
//    MFMAs of the same SIMD costs about half its cycles on top of theirs, so
//    the VALU count per MFMA is what the loop is written to keep low
//    (per-step base addresses plus immediate offsets, no per-load address
//    arithmetic).
//  * Dequantisation to bf16 with the e4m3 scale folded in is exact: q*s has
//    at most 6 significant bits.  fp32 accumulation in the MFMA; y = g * acc
//    stored once.
//  * fp16 operands when the caller gives a workspace: a staging kernel first
//    copies every activation row to fp16 scaled by a power of two chosen so
//    that the copy is exact, with g times the inverse power as the row's
//    output multiplier.  The weights then dequantise to fp16 with one packed
//    multiply per pair (4 conversions + 4 multiplies per 8 codes instead of
//    4 + 8 + 4 for bf16, which has no packed arithmetic on gfx950), and the
//    fp16 MFMAs sum the same exact products in the same order, so y is the
//    same bit for bit.  A block holding a row that fp16 cannot carry exactly
//    runs the bf16 loop; the choice is made once per workgroup from the row
//    multipliers, before the activation loads go out.
//  * SILU variant (fused gate/up weight, 8 gate rows and the matching 8 up
//    rows per 16-row tile): the lanes r and r + 8 that hold a gate/up pair
//    swap values by a row rotate and write h = bf16(silu(g*gate) * (g*up))
//    instead of y; lanes r < 8 take rows 4gq, 4gq+1 of each block and lanes
//    r >= 8 rows 4gq+2, 4gq+3, so every lane evaluates two epilogues.
#include <type_traits>

#include "q4p_device.h"
#include "q4p_launch.h"

namespace q4p {

namespace {

constexpr int kBM = 128;                       // activation rows per workgroup
constexpr int kMaxT = 17;                      // weight tiles per workgroup
constexpr int kXStageBytes = kBM * 256;        // one k-tile of activations
// weight stage: the packed code and scale tiles of up to kMaxT tiles, rounded
// up to whole 1 KB loads, plus 1 KB that loads with nothing to fetch write
// their zeros into (so every wave issues the same loads, without branches)
constexpr int kWDataBytes = (kMaxT * (kTileCodeBytes + kTileScaleBytes) + 1023) / 1024 * 1024;
constexpr int kWStageBytes = kWDataBytes + 1024;
// A buffer offset at or past a buffer's size reads as zero; this one marks
// rows and tiles outside the problem (it stays past every buffer after the
// per-stage advance, since one launch addresses less than 1 GiB per buffer).
constexpr uint32_t kOutside = 0x80000000u;
constexpr int64_t kMaxLaunchBytes = int64_t(1) << 30;

// Raw buffer resource over `bytes` bytes at p (gfx9 dword 3 for untyped
// 32-bit-element access; offsets are checked against `bytes`).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (int)bytes, 0x00020000);
}

// 16 bytes per lane from rsrc at voffset + soffset into LDS at lds + 16*lane.
// Lanes are marked outside the buffer through voffset alone; soffset carries
// the k-tile advance and never leads a lane past the buffer on its own.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rsrc, uint8_t *lds, uint32_t voffset,
                                           uint32_t soffset)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsrc, (__attribute__((address_space(3))) void *)lds, 16, voffset, soffset, 0, 0);
}

// Eight e2m1 codes (one dword, low nibble first) times one decoded scale.
__device__ __forceinline__ bf16x8_t dequant8(uint32_t wd, float s)
{
    uint4 v;
    v.x = fp4x2_scaled_to_bf16x2<0>(wd, s);
    v.y = fp4x2_scaled_to_bf16x2<1>(wd, s);
    v.z = fp4x2_scaled_to_bf16x2<2>(wd, s);
    v.w = fp4x2_scaled_to_bf16x2<3>(wd, s);
    return __builtin_bit_cast(bf16x8_t, v);
}

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

// The same eight products as fp16: each e2m1 pair converts exactly to fp16
// and one packed fp16 multiply applies the scale, exactly (q*s has at most 6
// significant bits and lies in [2^-10, 2688], inside fp16's normal range).
__device__ __forceinline__ f16x8_t dequant8h(uint32_t wd, _Float16 s)
{
    const f16x2_t s2 = {s, s};
    const f16x2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd, 1.0f, 0) * s2;
    const f16x2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd, 1.0f, 1) * s2;
    const f16x2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd, 1.0f, 2) * s2;
    const f16x2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd, 1.0f, 3) * s2;
    return (f16x8_t){v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
}

// OCP e4m3 byte SEL of w -> fp16 (exact: every e4m3 value is an fp16 value)
template <int SEL>
__device__ __forceinline__ _Float16 e4m3_to_f16(uint32_t w)
{
    return __builtin_amdgcn_cvt_scalef32_f16_fp8((f16x2_t){0, 0}, (int)w, 1.0f, SEL, false)[0];
}

// Position of code slot s (16 bytes) of a packed tile in a weight stage.
// A k-step's read takes 8 bytes of slots 32h + r and 32h + r + 16 (r < 16,
// h = 0, 1) in one ds_read2_b64, so without a swizzle the slots r, r + 8,
// r + 32 and r + 40 of one half-wave share LDS banks.  XORing bit 3 into bit
// 0 and bit 5 into bit 1 spreads them over different banks and leaves bit 4
// alone, so the second slot stays 256 bytes after the first; the map is its
// own inverse, so the stage loads fetch slot code_pos(p) into position p.
__device__ __forceinline__ int code_pos(int s)
{
    return s ^ ((s >> 3) & 1) ^ (((s >> 5) & 1) << 1);
}

// gfx9 s_waitcnt immediates: vmcnt(0) (expcnt and lgkmcnt left alone) and
// lgkmcnt(0)
constexpr int kWaitVm0 = 0x0f70;
constexpr int kWaitLgkm0 = 0xc07f;

template <int Q, int RT, bool SILU>
__global__ void __launch_bounds__(512)
gemm_kernel(const uint8_t *__restrict__ pcodes, const uint8_t *__restrict__ pscales, float g,
            const uint16_t *__restrict__ x, const uint16_t *__restrict__ xh,
            const float *__restrict__ rowmul, void *__restrict__ out, int M, int N, int64_t ldy,
            int K, int KT, int NT, int buf_out)
{
    constexpr int TT = 4 * Q + RT;                         // tiles per workgroup (== T)
    constexpr int RB = RT == 2 ? 1 : RT;                   // remaining-tile operands per wave
    constexpr int RR = RT == 2 ? 4 : 2;                    // 16-row blocks per such operand
    // weight chunks (16 bytes) per stage: 64 per code tile + 8 per scale tile,
    // spread over whole 64-lane loads, the same number for every wave
    constexpr int kWChunks = 72 * TT;
    constexpr int kWLoadsPerWave = (kWChunks + 511) / 512;

    __shared__ __attribute__((aligned(16))) uint8_t sx0[kXStageBytes];
    __shared__ __attribute__((aligned(16))) uint8_t sx1[kXStageBytes];
    __shared__ __attribute__((aligned(16))) uint8_t sx2[kXStageBytes];
    __shared__ __attribute__((aligned(16))) uint8_t sw0[kWStageBytes];
    __shared__ __attribute__((aligned(16))) uint8_t sw1[kWStageBytes];
    __shared__ __attribute__((aligned(16))) uint8_t sw2[kWStageBytes];
    // per-row output multipliers of the fp16 run (rowmul of the block's rows)
    __shared__ __attribute__((aligned(16))) float srow[kBM];

    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int w = wave & 3;                                // tile group
    const int kh = wave >> 2;                              // k-half: steps 2kh, 2kh+1
    const int lane = threadIdx.x & 63;
    const int r = lane & 15;
    const int gq = lane >> 4;
    const int m0 = blockIdx.y * kBM;
    const int tile0 = blockIdx.x * TT;
    // first 16-row block of this wave's share of the remaining tiles; the
    // wave visits row blocks rb, rb+1, ... (mod 8)
    const int rb = RT == 0 ? 0 : RT == 2 ? 4 * (w & 1) : 2 * w;

    // buffer sizes (a load past the last k-tile gets size 0: all zeros)
    const uint32_t xbytes = (uint32_t)((int64_t)M * K * 2);
    const uint32_t cbytes = (uint32_t)((int64_t)NT * KT * kTileCodeBytes);
    const uint32_t sbytes = (uint32_t)((int64_t)NT * KT * kTileScaleBytes);

    // ---- stage loads: per-lane byte offsets of k-tile 0 ----------------------
    // Activations: wave v, load i fills LDS bytes 1024*(4v+i) .. +1023, i.e.
    // rows 16v + 4i + l/16; lane l fills position l%16 of its row, which holds
    // chunk (l%16) ^ (row%16) (eight bf16, k = 8*chunk + 0..7).
    // k-tile c is at xoff + 256c; the last k-tile of a ragged K uses xlast,
    // which points chunks past K outside the buffer as well.
    const bool ragged = (K & 127) != 0;
    uint32_t xoff[4], xlast[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = m0 + 16 * wave + 4 * i + (lane >> 4);
        const int chunk = (lane & 15) ^ ((4 * i + (lane >> 4)) & 15);
        xoff[i] = row < M ? (uint32_t)(((int64_t)row * K + 8 * chunk) * 2) : kOutside;
        xlast[i] = row < M && 128 * (KT - 1) + 8 * chunk < K
                       ? xoff[i] + 256u * (uint32_t)(KT - 1) : kOutside;
    }
    // Weights: chunk e = 64*(8q + v) + lane for wave v's q-th load; e < 64*TT:
    // code tile e/64, slot e%64; else scale tile (e-64TT)/8, part (e-64TT)%8.
    // LDS offset e*16 either way (codes then scales).  A load is all codes or
    // all scales (64*TT is a multiple of 64).  Lanes past the last chunk read
    // past the buffer end (zeros into the stage's rounding); a load with no
    // chunk at all writes into the spare 1 KB.
    uint32_t woff[kWLoadsPerWave];
    int wlds[kWLoadsPerWave];
#pragma unroll
    for (int q = 0; q < kWLoadsPerWave; ++q) {
        const int e = 64 * (8 * q + wave) + lane;
        const bool code = 8 * q + wave < TT;
        const int j = code ? e >> 6 : (e - 64 * TT) >> 3;
        // the lane filling stage position p of a code tile fetches slot
        // code_pos(p), so slot s lands at position code_pos(s)
        const int part = code ? code_pos(e & 63) : ((e - 64 * TT) & 7);
        const int t = tile0 + j;
        const int64_t tb = code ? kTileCodeBytes : kTileScaleBytes;
        woff[q] = t < NT && e < kWChunks ? (uint32_t)((int64_t)t * KT * tb + part * 16) : kOutside;
        wlds[q] = 64 * (8 * q + wave) < kWChunks ? 1024 * (8 * q + wave) : kWDataBytes;
    }

    // One stage load n (0..3 activations, then weights) of k-tile c.  A load
    // that is not live (past the last k-tile) gets a buffer of size 0 and
    // only writes zeros into a free stage.
    constexpr int kLoads = 4 + kWLoadsPerWave;
    auto issue_load = [&](int n, int c, bool live, uint8_t *sx, uint8_t *sw, const uint16_t *xa) __attribute__((always_inline)) {
        if (n < 4) {
            const int i = n < 4 ? n : 0;
            const bool last = ragged && c == KT - 1;
            load_lds16(make_rsrc(xa, live ? xbytes : 0u), sx + 1024 * (4 * wave + n),
                       last ? xlast[i] : xoff[i], last ? 0u : 256u * (uint32_t)c);
        } else {
            const int q = n - 4 < kWLoadsPerWave ? n - 4 : 0;
            const bool code = 8 * q + wave < TT;
            const uint8_t *base = code ? pcodes : pscales;
            const uint32_t bytes = live ? (code ? cbytes : sbytes) : 0u;
            // the k-tile advance is wave-uniform; pinning it to a scalar register
            // keeps the compiler from computing it per lane and wrapping the load
            // in a loop over distinct values
            const uint32_t adv = (uint32_t)__builtin_amdgcn_readfirstlane(
                (int)((code ? (uint32_t)kTileCodeBytes : (uint32_t)kTileScaleBytes) * (uint32_t)c));
            load_lds16(make_rsrc(base, bytes), sw + wlds[q], woff[q], adv);
        }
    };
    // the weight loads (n >= 4) and the activation loads (n < 4) of a stage
    auto issue_wstage = [&](int c, bool live, uint8_t *sw) __attribute__((always_inline)) {
#pragma unroll
        for (int n = 4; n < kLoads; ++n)
            issue_load(n, c, live, nullptr, sw, nullptr);
    };
    auto issue_xstage = [&](int c, bool live, uint8_t *sx, const uint16_t *xa) __attribute__((always_inline)) {
#pragma unroll
        for (int n = 0; n < 4; ++n)
            issue_load(n, c, live, sx, nullptr, xa);
    };

    // code slots (r, 2h) and (r, 2h+1) hold this lane's k-values; the byte
    // permute picks block 2d + gq/2 of each
    const int h = gq & 1;
    const uint32_t sel = (gq >> 1) ? 0x07060302u : 0x05040100u;
    const int code_lane = code_pos(32 * h + r) * 16 + kh * 8;
    const int scale_lane = r * 8 + kh * 4;
    const int a_lane = r * 256;
    // The wave visits row blocks i ^ rb, i = 0..7 (rb is even, a multiple of
    // 4 when RT = 2): the activation operand of row block i ^ rb at step
    // base ab is at ab + ((i ^ rb) << 12), i.e. a few per-step base
    // addresses plus constant offsets.
    auto row_bases = [&](const uint8_t *ab, const uint8_t **rbase) __attribute__((always_inline)) {
        if (RT == 0) {
            rbase[0] = ab;
        } else if (RT == 2) {
            rbase[0] = ab + (rb << 12);                    // i = 0..3: rows rb + i
            rbase[1] = ab + ((4 - rb) << 12);              // i = 4..7: rows (4 - rb) + i - 4
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)                    // i = 2k, 2k+1: rows (2k ^ rb) + i % 2
                rbase[k] = ab + (((2 * k) ^ rb) << 12);
        }
    };

    // ---- software-pipelined k-loop --------------------------------------------
    // NB operands per k-step: the Q whole tiles, then the wave's remaining
    // tiles.  Raw code words and scales of one k-tile for this wave (pW, qW,
    // sW).
    constexpr int NB = Q + RB;
    uint2 pW[NB], qW[NB];
    uint32_t sW[NB];

    // this wave's code bytes (blocks 4kh..4kh+3 of two slots) and scales of
    // tile j of one landed stage; the scale of block 4kh + 2dd + gq/2 moved
    // to byte 2dd
    auto read_tile = [&](const uint8_t *sw, int j) __attribute__((always_inline)) {
        const int jt = j < Q ? w * Q + j : (RT == 2 ? 4 * Q + (w >> 1) : 4 * Q + (j - Q));
        const uint8_t *cb = sw + jt * kTileCodeBytes + code_lane;
        pW[j] = *reinterpret_cast<const uint2 *>(cb);
        qW[j] = *reinterpret_cast<const uint2 *>(cb + 256);
        sW[j] = *reinterpret_cast<const uint32_t *>(
                    sw + TT * kTileCodeBytes + jt * kTileScaleBytes + scale_lane) >> (8 * (gq >> 1));
    };

    // The k-loop and epilogue on one operand type.  F16: fp16 activations xa
    // (each row scaled by a power of two, see gemm_xprep_kernel) times fp16
    // weights; otherwise the bf16 activations xa times bf16 weights.  The
    // products are exact either way and the MFMAs accumulate them in the same
    // order.  The weight loads of stages 0 and 1 are already in flight.
    auto run = [&](auto f16_tag, const uint16_t *xa) __attribute__((always_inline)) {
        constexpr bool F16 = decltype(f16_tag)::value;
        using op_t = typename std::conditional<F16, f16x8_t, bf16x8_t>::type;
        // ---- accumulators -------------------------------------------------------
        // accF[j][i]: whole tile w*Q + j, row block i ^ rb.
        // accR[j][i]: remaining tile, row block rb + i.
        floatx4_t accF[Q > 0 ? Q : 1][8];
        floatx4_t accR[RB > 0 ? RB : 1][RR];
#pragma unroll
        for (int j = 0; j < Q; ++j)
#pragma unroll
            for (int i = 0; i < 8; ++i)
                accF[j][i] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < RB; ++j)
#pragma unroll
            for (int i = 0; i < RR; ++i)
                accR[j][i] = floatx4_t{0.f, 0.f, 0.f, 0.f};

        // the dequantised operands of the wave's two k-steps
        op_t b0[NB], b1[NB];
        auto row_operand = [&](const uint8_t *const *rbase, int i) __attribute__((always_inline)) {
            const uint8_t *pa = RT == 0 ? rbase[0] + (i << 12)
                              : RT == 2 ? rbase[i >> 2] + ((i & 3) << 12)
                                        : rbase[i >> 1] + ((i & 1) << 12);
            return *reinterpret_cast<const op_t *>(pa);
        };
        // operand of tile j for the wave's k-step dd from the raw words
        auto dequant_tile = [&](int j, int dd) __attribute__((always_inline)) {
            const uint32_t wd = __builtin_amdgcn_perm(dd ? qW[j].y : qW[j].x, dd ? pW[j].y : pW[j].x, sel);
            if constexpr (F16)
                return dequant8h(wd, dd ? e4m3_to_f16<2>(sW[j]) : e4m3_to_f16<0>(sW[j]));
            else
                return dequant8(wd, dd ? e4m3_to_f32<2>(sW[j]) : e4m3_to_f32<0>(sW[j]));
        };
        auto mma = [&](op_t a, op_t bb, floatx4_t acc) __attribute__((always_inline)) {
            if constexpr (F16)
                return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bb, acc, 0, 0, 0);
            else
                return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bb, acc, 0, 0, 0);
        };
        // the MFMAs of the wave's k-step dd on the activations of stage sx with
        // operands b; fill(i) is independent work placed after row block i
        auto mfma_step = [&](int dd, const uint8_t *sx, const op_t *b, auto fill) __attribute__((always_inline)) {
            const int d = 2 * kh + dd;
            const uint8_t *rbase[4];
            row_bases(sx + a_lane + (((4 * d + gq) ^ r) << 4), rbase);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const op_t a = row_operand(rbase, i);
#pragma unroll
                for (int j = 0; j < Q; ++j)
                    accF[j][i] = mma(a, b[j], accF[j][i]);
                if (i < RR) {
#pragma unroll
                    for (int j = 0; j < RB; ++j)
                        accR[j][i < RR ? i : 0] = mma(a, b[Q + j], accR[j][i < RR ? i : 0]);
                }
                fill(i);
            }
        };

        // One k-tile c.  Phase 1: the MFMAs of the first k-step, with the second
        // step's operands dequantised in between.  Then a barrier: stage c+1 has
        // landed everywhere and every wave is done with stage c-1.  Phase 2: the
        // MFMAs of the second k-step, with the stage loads of k-tile c+2 (into the
        // stage of c-1) and the reading and dequantising of k-tile c+1's first
        // step in between.  So no wave ever waits for its own dequantisation, and
        // each stage has about one k-tile to land.
        auto ktile = [&](int c, const uint8_t *sxc, const uint8_t *swn, uint8_t *sxl, uint8_t *swl) __attribute__((always_inline)) {
            mfma_step(0, sxc, b0, [&](int i) __attribute__((always_inline)) {
                if (i < NB)
                    b1[i < NB ? i : 0] = dequant_tile(i < NB ? i : 0, 1);
            });
            __builtin_amdgcn_s_waitcnt(kWaitVm0);
            __builtin_amdgcn_s_waitcnt(kWaitLgkm0);                 // lgkmcnt(0)
            __builtin_amdgcn_s_barrier();
            const bool live = c + 2 < KT;
            mfma_step(1, sxc, b1, [&](int i) __attribute__((always_inline)) {
                if (i < kLoads)
                    issue_load(i, c + 2, live, sxl, swl, xa);
                // tile i's words are read two row blocks before they are used
                if (i < NB)
                    read_tile(swn, i < NB ? i : 0);
                if (i >= 2 && i - 2 < NB)
                    b0[i >= 2 && i - 2 < NB ? i - 2 : 0] = dequant_tile(i >= 2 && i - 2 < NB ? i - 2 : 0, 0);
            });
            static_assert(NB <= 6, "every tile is dequantised inside the row loop");
        };

        // the activations of stages 0 and 1 (skipped past the last k-tile);
        // afterwards every k-tile issues the loads of the k-tile two ahead.
        // Stage 1's activation loads (the last 4 issued) may still be in
        // flight; the first k-tile's barrier waits for them.
        issue_xstage(0, true, sx0, xa);
        issue_xstage(1, KT > 1, sx1, xa);
        __builtin_amdgcn_s_waitcnt(0x0f70 | 4);
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        __builtin_amdgcn_s_barrier();
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            read_tile(sw0, j);
            b0[j] = dequant_tile(j, 0);
        }
        for (int c = 0; c < KT; c += 3) {
            ktile(c, sx0, sw1, sx2, sw2);
            if (c + 1 < KT)
                ktile(c + 1, sx1, sw2, sx0, sw0);
            if (c + 2 < KT)
                ktile(c + 2, sx2, sw0, sx1, sw1);
        }

        // ---- add the k-halves ------------------------------------------------------
        // Wave kh finishes row-block positions 4kh..4kh+3 of its whole tiles and
        // the kh-th half of its remaining-tile blocks.  Both waves of a pair hand
        // the partner the half it finishes, all through LDS at once: fragment f
        // (64 lanes x 16 bytes) of wave v sits in its own slot of the now free
        // stage buffers, so one barrier separates the writes from the reads, and
        // both waves of a SIMD then share the epilogue.
        constexpr int HR = RR / 2;                                 // remaining blocks kept per wave
        constexpr int kKeep = 4 * Q + RB * HR;                     // fragments kept (and handed over)
        static_assert(kKeep <= 8 || 2 * (kKeep - 8 < 8 ? kKeep - 8 : 8) * 1024 <= kWStageBytes,
                      "fragments 8..15 of waves 4..7: two waves per weight stage");
        static_assert(kKeep <= 16 || (kKeep <= 18 && 8 * 2048 <= kWStageBytes),
                      "fragments 16, 17: the third weight stage");
        static_assert(3 * (kXStageBytes + kWStageBytes) + kBM * 4 <= 160 * 1024, "LDS of one CU");
        floatx4_t keep[kKeep > 0 ? kKeep : 1];
        {
            // every wave is past its last LDS read of the stages (the last
            // compute ended with them) and its trailing zero-writing loads have
            // landed, so the stage buffers are free
            __builtin_amdgcn_s_waitcnt(kWaitVm0);
            __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
            __builtin_amdgcn_s_barrier();
            auto slot = [&](int v, int f) __attribute__((always_inline)) {
                uint8_t *base;
                if (f < 8)
                    base = (v < 4 ? sx0 : sx1) + (v & 3) * 8192 + f * 1024;
                else if (f < 16)
                    base = v < 4 ? sx2 + v * 8192 + (f - 8) * 1024
                                 : (v < 6 ? sw0 : sw1) + (v & 1) * (kKeep - 8 < 8 ? kKeep - 8 : 8) * 1024 + (f - 8) * 1024;
                else
                    base = sw2 + v * 2048 + (f - 16) * 1024;
                return reinterpret_cast<floatx4_t *>(base) + lane;
            };
            const bool upper = kh != 0;
#pragma unroll
            for (int j = 0; j < Q; ++j)
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    const floatx4_t lo = accF[j][ii], hi = accF[j][ii + 4];
                    *slot(wave, 4 * j + ii) = upper ? lo : hi;
                    keep[4 * j + ii] = upper ? hi : lo;
                }
#pragma unroll
            for (int j = 0; j < RB; ++j)
#pragma unroll
                for (int ii = 0; ii < HR; ++ii) {
                    const floatx4_t lo = accR[j][ii], hi = accR[j][ii + HR];
                    *slot(wave, 4 * Q + HR * j + ii) = upper ? lo : hi;
                    keep[4 * Q + HR * j + ii] = upper ? hi : lo;
                }
            __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
            __builtin_amdgcn_s_barrier();
#pragma unroll
            for (int f = 0; f < kKeep; ++f)
                keep[f] += *slot(wave ^ 4, f);
        }
        // fragment f of keep: tile and 16-row block (wave-uniform)
        auto frag_tile = [&](int f) __attribute__((always_inline)) {
            return f < 4 * Q ? tile0 + w * Q + f / 4
                             : tile0 + (RT == 2 ? 4 * Q + (w >> 1) : 4 * Q + (f - 4 * Q) / (HR > 0 ? HR : 1));
        };
        auto frag_block = [&](int f) __attribute__((always_inline)) {
            return f < 4 * Q ? (4 * kh + f % 4) ^ rb : rb + HR * kh + (f - 4 * Q) % (HR > 0 ? HR : 1);
        };
        // output multipliers of rows 4gq..4gq+3 of 16-row block blk: g, or after
        // an fp16 run g * 2^c of each row (which undoes the row's scaling exactly)
        auto row_mul = [&](int blk) __attribute__((always_inline)) {
            if constexpr (F16)
                return *reinterpret_cast<const floatx4_t *>(srow + 16 * blk + 4 * gq);
            else
                return floatx4_t{g, g, g, g};
        };

        // ---- epilogue: lane (r, gq) holds rows 4*gq + i of each 16-row block ----
        if (SILU) {
            const bool hi = r >= 8;
            if (buf_out) {
                // bf16 h through buffer stores as y below (2 bytes per output, rows
                // past M dropped at the buffer's end)
                const uint32_t hstride = (uint32_t)ldy * 2u;        // bytes per row of h
                const __amdgpu_buffer_rsrc_t hrs = make_rsrc(out, (uint32_t)M * hstride);
                // lanes r < 8 write rows 4gq, 4gq+1 of a block, lanes r >= 8 rows
                // 4gq+2, 4gq+3; output f = 8t + r%8
                const uint32_t lane_row = (uint32_t)(4 * gq + (hi ? 2 : 0)) * hstride;
#pragma unroll
                for (int f = 0; f < kKeep; ++f) {
                    const int t = frag_tile(f);
                    if (t < NT) {
                        const floatx4_t v = keep[f];
                        const float v0 = v[0], v1 = v[1], v2 = v[2], v3 = v[3];
                        const float s0 = swap8(v0), s1 = swap8(v1), s2 = swap8(v2), s3 = swap8(v3);
                        const float ga = hi ? s2 : v0, ua = hi ? v2 : s0;
                        const float gb = hi ? s3 : v1, ub = hi ? v3 : s1;
                        const floatx4_t gv = row_mul(frag_block(f));
                        const float gma = hi ? gv[2] : gv[0], gmb = hi ? gv[3] : gv[1];
                        const uint32_t fo = 8u * (uint32_t)t + (uint32_t)(r & 7);
                        const uint32_t row = (uint32_t)__builtin_amdgcn_readfirstlane(
                            (int)((uint32_t)(m0 + 16 * frag_block(f)) * hstride));
                        const uint32_t off = lane_row + fo * 2u + row;
                        __builtin_amdgcn_raw_buffer_store_b16(silu_mul_bf16(gma * ga, gma * ua), hrs, (int)off, 0, 0);
                        __builtin_amdgcn_raw_buffer_store_b16(silu_mul_bf16(gmb * gb, gmb * ub), hrs,
                                                              (int)(off + hstride), 0, 0);
                    }
                }
            } else {
                // outputs past 2 GiB of 32-bit offsets: plain stores, rows tested
                uint16_t *h = static_cast<uint16_t *>(out);
#pragma unroll
                for (int f = 0; f < kKeep; ++f) {
                    const int t = frag_tile(f);
                    if (t < NT) {
                        const floatx4_t v = keep[f];
                        const float v0 = v[0], v1 = v[1], v2 = v[2], v3 = v[3];
                        const float s0 = swap8(v0), s1 = swap8(v1), s2 = swap8(v2), s3 = swap8(v3);
                        const float ga = hi ? s2 : v0, ua = hi ? v2 : s0;
                        const float gb = hi ? s3 : v1, ub = hi ? v3 : s1;
                        const floatx4_t gv = row_mul(frag_block(f));
                        const float gma = hi ? gv[2] : gv[0], gmb = hi ? gv[3] : gv[1];
                        const int m = m0 + 16 * frag_block(f) + 4 * gq + (hi ? 2 : 0);
                        const int64_t fo = 8 * (int64_t)t + (r & 7);
                        if (m < M)
                            h[(int64_t)m * ldy + fo] = silu_mul_bf16(gma * ga, gma * ua);
                        if (m + 1 < M)
                            h[(int64_t)(m + 1) * ldy + fo] = silu_mul_bf16(gmb * gb, gmb * ub);
                    }
                }
            }
            return;
        }
        if (buf_out) {
            // y through buffer stores: the row part of each offset is wave-uniform
            // and the lane part fixed, so a store costs one add.  Rows past M lie
            // past the end of the buffer (buf_out: the launch's rows plus one block
            // stay under 2 GiB of y) and are dropped by the hardware instead of
            // being tested per store.
            const uint32_t rstride = (uint32_t)ldy * 4u;            // bytes per row of y
            const __amdgpu_buffer_rsrc_t yrs = make_rsrc(out, (uint32_t)M * rstride);
            const uint32_t lane_row = (uint32_t)(4 * gq) * rstride;
#pragma unroll
            for (int f = 0; f < kKeep; ++f) {
                const int t = frag_tile(f);
                const int n = t * 16 + r;
                if (t < NT && n < N) {
                    const int mb = m0 + 16 * frag_block(f);
                    const floatx4_t gv = row_mul(frag_block(f));
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t row = (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(mb + e) * rstride));
                        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, gv[e] * keep[f][e]), yrs,
                                                              (int)(lane_row + (uint32_t)n * 4u + row), 0, 0);
                    }
                }
            }
            return;
        }
        // outputs past 2 GiB of 32-bit offsets: plain stores, rows tested
        float *y = static_cast<float *>(out);
#pragma unroll
        for (int f = 0; f < kKeep; ++f) {
            const int t = frag_tile(f);
            const int n = t * 16 + r;
            if (t < NT && n < N) {
                const int mb = m0 + 16 * frag_block(f) + 4 * gq;
                const floatx4_t gv = row_mul(frag_block(f));
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int m = mb + e;
                    if (m < M)
                        y[(int64_t)m * ldy + n] = gv[e] * keep[f][e];
                }
            }
        }
    };

    // The block's 128 row multipliers, two per lane (rows past M read zero),
    // then the weight loads of stages 0 and 1, which do not depend on the
    // operand type.  The multipliers return first: fp16 operands when the
    // activations were staged (xh) and none of the block's rows is marked
    // inexact (NaN), else bf16.  Every wave holds the same 128 multipliers,
    // so the decision is the workgroup's.
    float rm0 = 0.f, rm1 = 0.f;
    if (xh != nullptr) {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(rowmul, (uint32_t)M * 4u);
        rm0 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                           rs, (int)((uint32_t)(m0 + lane) * 4u), 0, 0));
        rm1 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                           rs, (int)((uint32_t)(m0 + 64 + lane) * 4u), 0, 0));
    }
    issue_wstage(0, true, sw0);
    issue_wstage(1, KT > 1, sw1);
    static_assert(kLoads < 16, "vmcnt immediate");
    const bool f16 = xh != nullptr &&
                     __builtin_amdgcn_ballot_w64(__builtin_isnan(rm0) || __builtin_isnan(rm1)) == 0;
    if (f16) {
        // the epilogue's copy (read after the k-loop's barriers)
        if (wave == 0) {
            srow[lane] = rm0;
            srow[64 + lane] = rm1;
        }
        run(std::true_type{}, xh);
    } else {
        run(std::false_type{}, x);
    }
}

// ---- fp16 staging of the activations ----------------------------------------
// Row m of x (K bf16 values) is written to xh as fp16 values scaled by 2^-c,
// with c = E - 15 for E the largest exponent (floor(log2|v|)) among the row's
// nonzero values: every value of the row then lies below 2^16 and converts
// exactly as long as the smallest nonzero one stays at or above fp16's
// smallest normal 2^-14, i.e. when the row spans at most 29 binades (bf16
// carries 8 significant bits, fp16 11).  rowmul[m] = g * 2^c, the factor
// that turns the row's fp32 sums back into g times the unscaled sums
// exactly; it is NaN when the row would not convert exactly, holds an
// infinity or a NaN, or g * 2^c is not a normal float (or g is not finite),
// and the GEMM then runs the bf16 loop for that row's block.
// One 256-thread workgroup (four waves) per row; K % 8 == 0.
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

// floor(log2 v) of the nonzero finite bf16 magnitude with bit pattern a
__device__ __forceinline__ int bf16_exponent(uint32_t a)
{
    const uint32_t e = a >> 7;
    return e ? (int)e - 127 : (31 - __builtin_clz(a & 0x7fu)) - 133;
}

// max (MAX) or min over each 16-lane row of the wave by DPP butterflies
// (lane ^ 1, lane ^ 2, then the half-row and row mirrors), then over the
// four rows by readlane: a wave-uniform result
template <bool MAX>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v)
{
    auto step = [&](uint32_t t) { v = MAX ? (t > v ? t : v) : (t < v ? t : v); };
    step((uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));    // quad_perm 1,0,3,2
    step((uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));    // quad_perm 2,3,0,1
    step((uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false));   // row_half_mirror
    step((uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false));   // row_mirror
    uint32_t r = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
#pragma unroll
    for (int l = 16; l < 64; l += 16) {
        const uint32_t t = (uint32_t)__builtin_amdgcn_readlane((int)v, l);
        r = MAX ? (t > r ? t : r) : (t < r ? t : r);
    }
    return r;
}

__global__ void __launch_bounds__(256)
gemm_xprep_kernel(const uint16_t *__restrict__ x, int64_t M, int64_t K, float g,
                  uint16_t *__restrict__ xh, float *__restrict__ rowmul)
{
    // 16-byte chunks (8 values) of the row: thread t takes chunks t, t + 256,
    // ...; the first kHeld of them stay in registers between the two passes
    // (rows up to K = 8192), the rest are read again.  Buffer accesses past
    // the row read zero / are dropped.
    constexpr int kHeld = 4;
    __shared__ uint32_t part[8];
    const int64_t m = blockIdx.x;
    const uint32_t t = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane((int)(t >> 6));
    const uint32_t row_bytes = (uint32_t)(K * 2);
    const __amdgpu_buffer_rsrc_t xs = make_rsrc(x + m * K, row_bytes);
    const __amdgpu_buffer_rsrc_t hs = make_rsrc(xh + m * K, row_bytes);
    auto load = [&](uint32_t chunk) __attribute__((always_inline)) {
        return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(xs, (int)(chunk * 16u), 0, 0));
    };
    // largest magnitude and smallest nonzero magnitude as bf16 bit patterns
    // (ordered like the values): packed 16-bit max of |v| and min of |v| - 1
    // (zero wraps to 0xffff)
    u16x2_t amax = {0, 0}, amin1 = {0xffff, 0xffff};
    auto scan = [&](const u32x4_t &v) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u16x2_t a = __builtin_bit_cast(u16x2_t, v[i] & 0x7fff7fffu);
            amax = __builtin_elementwise_max(amax, a);
            amin1 = __builtin_elementwise_min(amin1, a - (u16x2_t){1, 1});
        }
    };
    const uint32_t nchunks = (uint32_t)(K / 8);
    u32x4_t held[kHeld];
#pragma unroll
    for (int i = 0; i < kHeld; ++i)
        held[i] = load(t + 256u * i);
#pragma unroll
    for (int i = 0; i < kHeld; ++i)
        scan(held[i]);
    for (uint32_t ch = t + 256u * kHeld; ch < nchunks; ch += 256u)
        scan(load(ch));
    // the four waves' results through LDS
    const uint32_t wmax = wave_reduce_u32<true>(amax[0] > amax[1] ? amax[0] : amax[1]);
    const uint32_t wmin = wave_reduce_u32<false>(amin1[0] < amin1[1] ? amin1[0] : amin1[1]);
    if ((t & 63) == 0) {
        part[wave] = wmax;
        part[4 + wave] = wmin;
    }
    __syncthreads();
    uint32_t hi_bits = part[0], lo_bits1 = part[4];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
        hi_bits = part[w] > hi_bits ? part[w] : hi_bits;
        lo_bits1 = part[4 + w] < lo_bits1 ? part[4 + w] : lo_bits1;
    }
    const bool nonfinite = hi_bits >= 0x7f80u;
    const bool zero_row = hi_bits == 0;
    const int c = zero_row || nonfinite ? 0 : bf16_exponent(hi_bits) - 15;
    const bool exact = zero_row || (!nonfinite && bf16_exponent(lo_bits1 + 1) - c >= -14);
    auto convert_store = [&](const u32x4_t &v, uint32_t chunk) __attribute__((always_inline)) {
        u32x4_t o;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float f0 = __builtin_bit_cast(float, v[i] << 16);
            const float f1 = __builtin_bit_cast(float, v[i] & 0xffff0000u);
            const f16x2_t hh = {(_Float16)__builtin_ldexpf(f0, -c), (_Float16)__builtin_ldexpf(f1, -c)};
            o[i] = __builtin_bit_cast(uint32_t, hh);
        }
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, o), hs, (int)(chunk * 16u), 0, 0);
    };
    // rows that take the bf16 loop need no fp16 copy
    if (exact) {
#pragma unroll
        for (int i = 0; i < kHeld; ++i)
            convert_store(held[i], t + 256u * i);
        for (uint32_t ch = t + 256u * kHeld; ch < nchunks; ch += 256u)
            convert_store(load(ch), ch);
    }
    if (t == 0) {
        const float gm = __builtin_ldexpf(g, c);
        const float agm = __builtin_fabsf(gm);
        const bool mul_ok = g == 0.0f || (agm >= 1.17549435e-38f && agm <= 3.40282347e+38f);
        rowmul[m] = exact && mul_ok ? gm : __builtin_nanf("");
    }
}

typedef void (*gemm_fn)(const uint8_t *, const uint8_t *, float, const uint16_t *, const uint16_t *,
                        const float *, void *, int, int, int64_t, int, int, int, int);

#define Q4P_GEMM_ENTRY(T) gemm_kernel<(T) / 4, (T) % 4, false>
const gemm_fn kGemmTable[kMaxT + 1] = {
    nullptr,             Q4P_GEMM_ENTRY(1),  Q4P_GEMM_ENTRY(2),  Q4P_GEMM_ENTRY(3),
    Q4P_GEMM_ENTRY(4),   Q4P_GEMM_ENTRY(5),  Q4P_GEMM_ENTRY(6),  Q4P_GEMM_ENTRY(7),
    Q4P_GEMM_ENTRY(8),   Q4P_GEMM_ENTRY(9),  Q4P_GEMM_ENTRY(10), Q4P_GEMM_ENTRY(11),
    Q4P_GEMM_ENTRY(12),  Q4P_GEMM_ENTRY(13), Q4P_GEMM_ENTRY(14), Q4P_GEMM_ENTRY(15),
    Q4P_GEMM_ENTRY(16),  Q4P_GEMM_ENTRY(17),
};
#undef Q4P_GEMM_ENTRY

#define Q4P_GEMM_ENTRY(T) gemm_kernel<(T) / 4, (T) % 4, true>
const gemm_fn kGemmSiluTable[kMaxT + 1] = {
    nullptr,             Q4P_GEMM_ENTRY(1),  Q4P_GEMM_ENTRY(2),  Q4P_GEMM_ENTRY(3),
    Q4P_GEMM_ENTRY(4),   Q4P_GEMM_ENTRY(5),  Q4P_GEMM_ENTRY(6),  Q4P_GEMM_ENTRY(7),
    Q4P_GEMM_ENTRY(8),   Q4P_GEMM_ENTRY(9),  Q4P_GEMM_ENTRY(10), Q4P_GEMM_ENTRY(11),
    Q4P_GEMM_ENTRY(12),  Q4P_GEMM_ENTRY(13), Q4P_GEMM_ENTRY(14), Q4P_GEMM_ENTRY(15),
    Q4P_GEMM_ENTRY(16),  Q4P_GEMM_ENTRY(17),
};
#undef Q4P_GEMM_ENTRY

int64_t align256(int64_t n) { return (n + 255) / 256 * 256; }

// out: fp32 y[M][N], or with silu bf16 h[M][N/2] (N = 2F, fused gate/up).
// workspace (or null: bf16 operands throughout): gemm_workspace_bytes(M, K)
// bytes, 16-byte aligned: the fp16 activations, then the row multipliers.
hipError_t launch_gemm_any(const uint8_t *packed_codes, const uint8_t *packed_scales, float g,
                           const uint16_t *x, void *out, int64_t M, int64_t N, int64_t K,
                           bool silu, void *workspace, hipStream_t stream)
{
    const int64_t NT = n_tiles(N);
    const int64_t KT = k_tiles(K);
    uint16_t *xh = nullptr;
    float *rowmul = nullptr;
    if (workspace) {
        xh = static_cast<uint16_t *>(workspace);
        rowmul = reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) + align256(M * K * 2));
        hipLaunchKernelGGL(gemm_xprep_kernel, dim3((unsigned)M), dim3(256), 0, stream, x,
                           M, K, g, xh, rowmul);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    // Buffer offsets are 32-bit: one launch covers at most 1 GiB of
    // activations and of packed codes; larger problems run as several
    // launches over row and tile ranges (y keeps its row stride N).
    int64_t rows_per_launch = kMaxLaunchBytes / (K * 2);
    rows_per_launch = rows_per_launch / kBM * kBM;
    if (rows_per_launch > int64_t(65535) * kBM)
        rows_per_launch = int64_t(65535) * kBM;
    const int64_t tiles_per_launch = kMaxLaunchBytes / (KT * kTileCodeBytes);
    if (rows_per_launch < 1 || tiles_per_launch < 1)
        return hipErrorInvalidValue;                     // K beyond what one tile row allows
    for (int64_t mb = 0; mb < M; mb += rows_per_launch) {
        const int64_t Mc = M - mb < rows_per_launch ? M - mb : rows_per_launch;
        const int64_t MB = (Mc + kBM - 1) / kBM;
        for (int64_t tb = 0; tb < NT; tb += tiles_per_launch) {
            const int64_t NTc = NT - tb < tiles_per_launch ? NT - tb : tiles_per_launch;
            const int64_t Nc = N - 16 * tb < 16 * NTc ? N - 16 * tb : 16 * NTc;
            // tiles per workgroup: about one workgroup per CU over the grid
            int64_t T = (NTc * MB + 255) / 256;
            if (T < 1)
                T = 1;
            if (T > kMaxT)
                T = kMaxT;
            const int64_t NB = (NTc + T - 1) / T;
            const dim3 grid((unsigned)NB, (unsigned)MB), block(512);
            // output columns of this chunk: 16 per tile (8 with silu)
            void *o = silu ? static_cast<void *>(static_cast<uint16_t *>(out) + mb * (N / 2) + 8 * tb)
                           : static_cast<void *>(static_cast<float *>(out) + mb * N + 16 * tb);
            // outputs through buffer stores (32-bit offsets from o) while the
            // launch's rows plus one block of rows stay under 2 GiB
            const int64_t row_bytes = silu ? N : N * 4;     // N/2 bf16 or N fp32
            const int buf_out = (Mc + kBM) * row_bytes <= (int64_t(1) << 31) ? 1 : 0;
            hipLaunchKernelGGL(silu ? kGemmSiluTable[T] : kGemmTable[T], grid, block, 0, stream,
                               packed_codes + tb * KT * kTileCodeBytes,
                               packed_scales + tb * KT * kTileScaleBytes, g, x + mb * K,
                               xh ? xh + mb * K : nullptr, rowmul ? rowmul + mb : nullptr, o,
                               (int)Mc, (int)Nc, silu ? N / 2 : N, (int)K, (int)KT, (int)NTc,
                               buf_out);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess)
                return e;
        }
    }
    return hipSuccess;
}

}  // namespace

size_t gemm_workspace_bytes(int64_t M, int64_t K)
{
    return (size_t)(align256(M * K * 2) + align256(M * 4));
}

hipError_t launch_gemm(const uint8_t *packed_codes, const uint8_t *packed_scales, float g,
                       const uint16_t *x, float *y, int64_t M, int64_t N, int64_t K,
                       void *workspace, hipStream_t stream)
{
    return launch_gemm_any(packed_codes, packed_scales, g, x, y, M, N, K, false, workspace, stream);
}

hipError_t launch_gemm_silu_mul(const uint8_t *packed_codes, const uint8_t *packed_scales,
                                float g, const uint16_t *x, uint16_t *h, int64_t M, int64_t F,
                                int64_t K, void *workspace, hipStream_t stream)
{
    return launch_gemm_any(packed_codes, packed_scales, g, x, h, M, 2 * F, K, true, workspace,
                           stream);
}

}  // namespace q4p
