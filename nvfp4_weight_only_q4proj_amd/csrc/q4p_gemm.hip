// q4p_gemm.hip — prefill-chunk projection (sized for M = 512), any M >= 1.
//
// At M = 512 each weight is used 512 times: the work is a dense bf16
// contraction and belongs on the matrix cores.  Design:
//
//  * Workgroup = 8 waves, two per SIMD, covering kBM = 128 activation rows
//    and T weight-row tiles of 16 (BN = 16*T).  T is chosen so the grid has
//    about one workgroup per CU (256), e.g. T = 17 for N = 17408 and T = 14
//    for N = 14336 at M = 512: 256 equal workgroups, no tail wave.
//  * Waves w and w+4 own the same outputs and split every k-tile: wave w
//    takes its first two 32-wide k-steps, wave w+4 the last two, and the two
//    partial sums are added through LDS at the end.  Two waves per SIMD let
//    one wave's dequantisation and LDS waits overlap the other's MFMAs.
//  * Each wave pair owns Q = T/4 whole weight tiles (all 128 rows) plus a
//    quarter (32 rows) of each of the RT = T%4 remaining tiles, so all waves
//    do exactly the same number of MFMAs whatever T is.
//  * Operands reach LDS without passing through registers: per k-tile (128 k)
//    the 128 activation rows and the workgroup's T packed code tiles and
//    scale tiles are fetched with 16-byte direct-to-LDS loads into one of
//    three stages, two k-tiles ahead of the MFMAs.  Workgroup barriers are
//    bare s_barrier with an explicit wait for the stage being consumed (a
//    full barrier would also drain the loads of the stages in flight).
//  * Activation rows are stored in LDS with the 16-byte chunks of each row
//    XOR-swizzled by the row index, so that the sixteen rows an A-operand read
//    touches fall in sixteen different bank groups.  A lane's eight bf16 for
//    one 16x16x32 MFMA are two 8-byte pieces (k = 4g..4g+3 of two adjacent
//    scale blocks), matching the k-values its weight code word holds.
//  * Weights: each wave reads its tiles' 16-byte code slots and 8-byte scale
//    rows from LDS and dequantises them to bf16 with the e4m3 scale folded in
//    (exact: q*s has <= 6 significant bits).  One 32-bit code word = two
//    scale blocks x 4 codes = one MFMA operand.
//  * fp32 accumulation in the MFMA; y = g * acc stored once.
#include "q4p_device.h"
#include "q4p_launch.h"

namespace q4p {

namespace {

constexpr int kBM = 128;                       // activation rows per workgroup
constexpr int kMaxT = 17;                      // weight tiles per workgroup
constexpr int kXStageBytes = kBM * 256;        // one k-tile of activations
constexpr int kWStageBytes = kMaxT * (kTileCodeBytes + kTileScaleBytes);

// One 16x16x32 MFMA operand from code word `wd` (blocks 2d and 2d+1 of the
// lane's row) with their decoded scales s0, s1.
__device__ __forceinline__ bf16x8_t dequant_operand(uint32_t wd, float s0, float s1)
{
    uint4 v;
    v.x = fp4x2_scaled_to_bf16x2<0>(wd, s0);
    v.y = fp4x2_scaled_to_bf16x2<1>(wd, s0);
    v.z = fp4x2_scaled_to_bf16x2<2>(wd, s1);
    v.w = fp4x2_scaled_to_bf16x2<3>(wd, s1);
    return __builtin_bit_cast(bf16x8_t, v);
}

template <int D>
__device__ __forceinline__ bf16x8_t weight_operand(const uint4 &c, const uint2 &s)
{
    const uint32_t wd = D == 0 ? c.x : D == 1 ? c.y : D == 2 ? c.z : c.w;
    const uint32_t sv = D < 2 ? s.x : s.y;
    float s0, s1;
    if (D & 1) {
        s0 = e4m3_to_f32<2>(sv);
        s1 = e4m3_to_f32<3>(sv);
    } else {
        s0 = e4m3_to_f32<0>(sv);
        s1 = e4m3_to_f32<1>(sv);
    }
    return dequant_operand(wd, s0, s1);
}

// Operand of the first (DD = 0) or second (DD = 1) of a wave's two k-steps,
// from its two code words and the scale dword of their four blocks.
template <int DD>
__device__ __forceinline__ bf16x8_t weight_operand_half(const uint2 &c, uint32_t sv)
{
    const uint32_t wd = DD == 0 ? c.x : c.y;
    float s0, s1;
    if (DD == 1) {
        s0 = e4m3_to_f32<2>(sv);
        s1 = e4m3_to_f32<3>(sv);
    } else {
        s0 = e4m3_to_f32<0>(sv);
        s1 = e4m3_to_f32<1>(sv);
    }
    return dequant_operand(wd, s0, s1);
}

// gfx9 s_waitcnt immediate: wait until at most n vector-memory operations of
// this wave are outstanding (expcnt and lgkmcnt left alone)
__device__ __forceinline__ void wait_vm(int n)
{
    switch (n) {
#define Q4P_VM(k) \
    case k: __builtin_amdgcn_s_waitcnt(0x0f70 | ((k) & 15) | (((k) >> 4) << 14)); break;
        Q4P_VM(0) Q4P_VM(1) Q4P_VM(2) Q4P_VM(3) Q4P_VM(4) Q4P_VM(5) Q4P_VM(6) Q4P_VM(7)
        Q4P_VM(8) Q4P_VM(9) Q4P_VM(10) Q4P_VM(11) Q4P_VM(12) Q4P_VM(13) Q4P_VM(14) Q4P_VM(15)
        Q4P_VM(16) Q4P_VM(17) Q4P_VM(18) Q4P_VM(19) Q4P_VM(20)
#undef Q4P_VM
    default: __builtin_amdgcn_s_waitcnt(0x0f70); break;
    }
}

template <int Q, int RT>
__global__ void __launch_bounds__(512)
gemm_kernel(const uint4 *__restrict__ pcodes, const uint2 *__restrict__ pscales, float g,
            const uint16_t *__restrict__ x, float *__restrict__ y, int M, int N, int K, int KT,
            int NT, int T)
{
    constexpr int TT = 4 * Q + RT;                         // tiles per workgroup (== T)
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

    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int w = wave & 3;                                // tile group
    const int kh = wave >> 2;                              // k-half: steps 2kh, 2kh+1
    const int lane = threadIdx.x & 63;
    const int r = lane & 15;
    const int gq = lane >> 4;
    const int m0 = blockIdx.y * kBM;
    const int tile0 = blockIdx.x * TT;
    (void)T;

    // ---- direct-to-LDS stage loads ---------------------------------------
    // Activations: wave v, load i covers LDS slots 64*(4v+i) .. +63, i.e.
    // rows 4*(4v+i) .. +3; lane l -> row 4*(4v+i) + l/16, slot position
    // l%16, which holds chunk (l%16) ^ (row%16) of the row (8 bf16 each).
    // Rows past M read row M-1 (outputs never stored); chunks past K read the
    // row start and are zeroed after landing (ragged last k-tile only).
    // (addresses are recomputed per stage from a few values: holding them all
    // would cost registers the accumulators need)
    const int xrow0 = m0 + 16 * wave + (lane >> 4);        // row of load i: xrow0 + 4i
    // Weights: chunk e = 64*(8q + v) + lane for wave v's q-th weight load;
    // e < 64*TT: code tile e/64, slot e%64; else scale tile (e-64TT)/8, part
    // (e-64TT)%8.  LDS offset e*16 either way (codes then scales).
    // loads this wave issues per stage (a weight load with no live lane is
    // skipped): the wait for a stage leaves exactly the next stage's in flight
    int loads_per_stage = 4;
#pragma unroll
    for (int q = 0; q < kWLoadsPerWave; ++q)
        loads_per_stage += 64 * (8 * q + wave) < kWChunks ? 1 : 0;
    const uint8_t *pc8 = reinterpret_cast<const uint8_t *>(pcodes);
    const uint8_t *ps8 = reinterpret_cast<const uint8_t *>(pscales);

    auto issue_stage = [&](int c, uint8_t *sx, uint8_t *sw) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int grow = xrow0 + 4 * i;
            grow = grow < M ? grow : M - 1;
            const int chunk = (lane & 15) ^ ((4 * i + (lane >> 4)) & 15);
            const int k = 128 * c + 8 * chunk;
            const uint16_t *src = x + (int64_t)grow * K + (k < K ? k : 0);
            __builtin_amdgcn_global_load_lds(src, sx + 1024 * (4 * wave + i), 16, 0, 0);
        }
#pragma unroll
        for (int q = 0; q < kWLoadsPerWave; ++q) {
            const int e = 64 * (8 * q + wave) + lane;
            if (e < kWChunks) {
                const bool code = e < 64 * TT;
                const int j = code ? e >> 6 : (e - 64 * TT) >> 3;
                const int part = code ? (e & 63) : ((e - 64 * TT) & 7);
                int t = tile0 + j;
                t = t < NT ? t : NT - 1;                    // past NT: outputs never stored
                const int64_t tc = (int64_t)t * KT + c;
                const uint8_t *src = code ? pc8 + tc * kTileCodeBytes + part * 16
                                          : ps8 + tc * kTileScaleBytes + part * 16;
                __builtin_amdgcn_global_load_lds(src, sw + 1024 * (8 * q + wave), 16, 0, 0);
            }
        }
    };

    // ---- accumulators -------------------------------------------------------
    floatx4_t accF[Q > 0 ? Q : 1][8];
    floatx4_t accR[RT > 0 ? RT : 1][2];
#pragma unroll
    for (int j = 0; j < Q; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i)
            accF[j][i] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < RT; ++j)
#pragma unroll
        for (int i = 0; i < 2; ++i)
            accR[j][i] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    const bool ragged = (K & 127) != 0;

    // ---- one k-tile from a landed stage -------------------------------------
    auto compute = [&](int c, uint8_t *sx, const uint8_t *sw, uint8_t *sxn, uint8_t *swn) {
        // wait for this stage (the next one may still be in flight), then
        // make every wave's loads of it visible; this wave's LDS reads of the
        // stage that is overwritten next are complete (lgkmcnt(0))
        if (c + 1 < KT)
            wait_vm(loads_per_stage);
        else
            wait_vm(0);
        __builtin_amdgcn_s_waitcnt(0xc07f);                 // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        if (c + 2 < KT)
            issue_stage(c + 2, sxn, swn);                   // into the stage consumed at c-1
        if (ragged && c == KT - 1) {
            // zero the activation chunks past K of the last k-tile
            for (int s = (int)threadIdx.x; s < kBM * 16; s += 512) {
                const int row = s >> 4, chunk = (s & 15) ^ (row & 15);
                if (128 * c + 8 * chunk >= K)
                    *reinterpret_cast<uint4 *>(sx + 16 * s) = make_uint4(0u, 0u, 0u, 0u);
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);
            __builtin_amdgcn_s_barrier();
        }

        // this wave's code words and scales for its two k-steps: code words
        // 2kh, 2kh+1 of the lane's slot, scales of blocks 4kh..4kh+3
        uint2 cF[Q > 0 ? Q : 1], cR[RT > 0 ? RT : 1];
        uint32_t sF[Q > 0 ? Q : 1], sR[RT > 0 ? RT : 1];
#pragma unroll
        for (int j = 0; j < Q; ++j) {
            const int jt = w * Q + j;
            cF[j] = *reinterpret_cast<const uint2 *>(sw + jt * kTileCodeBytes + lane * 16 + kh * 8);
            sF[j] = *reinterpret_cast<const uint32_t *>(sw + TT * kTileCodeBytes + jt * kTileScaleBytes + r * 8 + kh * 4);
        }
#pragma unroll
        for (int j = 0; j < RT; ++j) {
            const int jt = 4 * Q + j;
            cR[j] = *reinterpret_cast<const uint2 *>(sw + jt * kTileCodeBytes + lane * 16 + kh * 8);
            sR[j] = *reinterpret_cast<const uint32_t *>(sw + TT * kTileCodeBytes + jt * kTileScaleBytes + r * 8 + kh * 4);
        }

        // A operand of row tile mt, k-step d: rows 16mt + r, the two 8-byte
        // pieces k = 32d + 4gq + {0..3} and 32d + 16 + 4gq + {0..3}
        auto read_a = [&](int d, int rowt) {
            const int row = 16 * rowt + r;
            const int c0 = 4 * d + (gq >> 1);
            const uint8_t *base = sx + row * 256 + (gq & 1) * 8;
            const uint2 lo = *reinterpret_cast<const uint2 *>(base + ((c0 ^ r) << 4));
            const uint2 hi = *reinterpret_cast<const uint2 *>(base + (((c0 + 2) ^ r) << 4));
            return __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
        };

#pragma unroll
        for (int dd = 0; dd < 2; ++dd) {
            const int d = 2 * kh + dd;
            // B operands of every tile for this step, then one A operand at a
            // time (fewer live registers than holding all eight A operands)
            bf16x8_t bF[Q > 0 ? Q : 1], bR[RT > 0 ? RT : 1];
#pragma unroll
            for (int j = 0; j < Q; ++j)
                bF[j] = dd == 0 ? weight_operand_half<0>(cF[j], sF[j]) : weight_operand_half<1>(cF[j], sF[j]);
#pragma unroll
            for (int j = 0; j < RT; ++j)
                bR[j] = dd == 0 ? weight_operand_half<0>(cR[j], sR[j]) : weight_operand_half<1>(cR[j], sR[j]);
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) {
                const bf16x8_t a = read_a(d, mt);
#pragma unroll
                for (int j = 0; j < Q; ++j)
                    accF[j][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bF[j], accF[j][mt], 0, 0, 0);
            }
            // this wave's rows of the remaining tiles (A operands re-read
            // from LDS: indexing by the wave number would need scratch)
            if (RT > 0) {
                const bf16x8_t ar0 = read_a(d, 2 * w), ar1 = read_a(d, 2 * w + 1);
#pragma unroll
                for (int j = 0; j < RT; ++j) {
                    accR[j][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ar0, bR[j], accR[j][0], 0, 0, 0);
                    accR[j][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ar1, bR[j], accR[j][1], 0, 0, 0);
                }
            }
        }
    };

    // ---- pipeline: stages 0, 1 in flight, then one k-tile per step ----------
    issue_stage(0, sx0, sw0);
    if (KT > 1)
        issue_stage(1, sx1, sw1);
    for (int c = 0; c < KT; c += 3) {
        compute(c, sx0, sw0, sx2, sw2);
        if (c + 1 < KT)
            compute(c + 1, sx1, sw1, sx0, sw0);
        if (c + 2 < KT)
            compute(c + 2, sx2, sw2, sx1, sw1);
    }

    // ---- add the k-halves: waves 4..7 hand their sums to waves 0..3 --------
    {
        // every wave is past its last LDS read of the stages (the last
        // compute ended with them), so the stage buffers are free
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_s_barrier();
        constexpr int kAcc = 8 * Q + 2 * RT;                 // floatx4 per lane
        // one slot per wave pair: three activation stages and one weight
        // stage, each holding kPass fragments of 64 lanes x 16 bytes
        constexpr int kPass = kWStageBytes / (64 * 16);
        floatx4_t *red = reinterpret_cast<floatx4_t *>(w < 2 ? (w == 0 ? sx0 : sx1) : (w == 2 ? sx2 : sw0));
        static_assert(kWStageBytes <= kXStageBytes, "pass size bounded by the smaller stage");
#pragma unroll
        for (int p0 = 0; p0 < kAcc; p0 += kPass) {
            if (kh == 1) {
#pragma unroll
                for (int f = p0; f < kAcc && f < p0 + kPass; ++f)
                    red[(f - p0) * 64 + lane] = f < 8 * Q ? accF[f >> 3][f & 7] : accR[(f - 8 * Q) >> 1][(f - 8 * Q) & 1];
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);
            __builtin_amdgcn_s_barrier();
            if (kh == 0) {
#pragma unroll
                for (int f = p0; f < kAcc && f < p0 + kPass; ++f) {
                    if (f < 8 * Q)
                        accF[f >> 3][f & 7] += red[(f - p0) * 64 + lane];
                    else
                        accR[(f - 8 * Q) >> 1][(f - 8 * Q) & 1] += red[(f - p0) * 64 + lane];
                }
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);
            __builtin_amdgcn_s_barrier();
        }
        if (kh == 1)
            return;
    }

    // ---- epilogue: lane (r, gq) holds rows 4*gq + i of each 16-row M tile ----
#pragma unroll
    for (int j = 0; j < Q; ++j) {
        const int t = tile0 + w * Q + j;
        const int n = t * 16 + r;
        if (t < NT && n < N) {
#pragma unroll
            for (int mt = 0; mt < 8; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int m = m0 + 16 * mt + 4 * gq + i;
                    if (m < M)
                        y[(int64_t)m * N + n] = g * accF[j][mt][i];
                }
        }
    }
#pragma unroll
    for (int j = 0; j < RT; ++j) {
        const int t = tile0 + 4 * Q + j;
        const int n = t * 16 + r;
        if (t < NT && n < N) {
#pragma unroll
            for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int m = m0 + 16 * (2 * w + i2) + 4 * gq + i;
                    if (m < M)
                        y[(int64_t)m * N + n] = g * accR[j][i2][i];
                }
        }
    }
}

typedef void (*gemm_fn)(const uint4 *, const uint2 *, float, const uint16_t *, float *, int, int,
                        int, int, int, int);

#define Q4P_GEMM_ENTRY(T) gemm_kernel<(T) / 4, (T) % 4>
const gemm_fn kGemmTable[kMaxT + 1] = {
    nullptr,             Q4P_GEMM_ENTRY(1),  Q4P_GEMM_ENTRY(2),  Q4P_GEMM_ENTRY(3),
    Q4P_GEMM_ENTRY(4),   Q4P_GEMM_ENTRY(5),  Q4P_GEMM_ENTRY(6),  Q4P_GEMM_ENTRY(7),
    Q4P_GEMM_ENTRY(8),   Q4P_GEMM_ENTRY(9),  Q4P_GEMM_ENTRY(10), Q4P_GEMM_ENTRY(11),
    Q4P_GEMM_ENTRY(12),  Q4P_GEMM_ENTRY(13), Q4P_GEMM_ENTRY(14), Q4P_GEMM_ENTRY(15),
    Q4P_GEMM_ENTRY(16),  Q4P_GEMM_ENTRY(17),
};
#undef Q4P_GEMM_ENTRY

}  // namespace

hipError_t launch_gemm(const uint8_t *packed_codes, const uint8_t *packed_scales, float g,
                       const uint16_t *x, float *y, int64_t M, int64_t N, int64_t K,
                       hipStream_t stream)
{
    const int64_t NT = n_tiles(N);
    const int64_t KT = k_tiles(K);
    const int64_t MB = (M + kBM - 1) / kBM;
    // tiles per workgroup: about one workgroup per CU over the whole grid
    int64_t T = (NT * MB + 255) / 256;
    if (T < 1)
        T = 1;
    if (T > kMaxT)
        T = kMaxT;
    const int64_t NB = (NT + T - 1) / T;
    const dim3 grid((unsigned)NB, (unsigned)MB), block(512);
    hipLaunchKernelGGL(kGemmTable[T], grid, block, 0, stream,
                       reinterpret_cast<const uint4 *>(packed_codes),
                       reinterpret_cast<const uint2 *>(packed_scales), g, x, y, (int)M, (int)N,
                       (int)K, (int)KT, (int)NT, (int)T);
    return hipGetLastError();
}

}  // namespace q4p
