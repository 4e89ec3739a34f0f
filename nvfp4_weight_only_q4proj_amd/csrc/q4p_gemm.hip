// q4p_gemm.hip — prefill-chunk projection (sized for M = 512), any M >= 1.
//
// At M = 512 each weight is used 512 times: the work is a dense bf16
// contraction and belongs on the matrix cores.  Design:
//
//  * Workgroup = 4 waves, one per SIMD, covering kBM = 128 activation rows
//    and T weight-row tiles of 16 (BN = 16*T).  T is chosen so the grid has
//    about one workgroup per CU (256), e.g. T = 17 for N = 17408 and T = 14
//    for N = 14336 at M = 512: 256 equal workgroups, no tail wave.
//  * Each wave owns Q = T/4 whole weight tiles (all 128 rows) plus a quarter
//    (32 rows) of each of the RT = T%4 remaining tiles, so the four waves do
//    exactly the same number of MFMAs whatever T is.
//  * Activations: each k-tile (128 k) of the 128 rows is staged in LDS,
//    double-buffered, in a permuted order so that one 16-byte LDS read
//    returns the 8 bf16 a lane feeds to one 16x16x32 MFMA; rows are padded to
//    272 bytes to spread consecutive rows over the banks.
//  * Weights: each wave streams its tiles' 16-byte code slots and 8-byte scale
//    rows straight into registers one k-tile ahead, and dequantises them to
//    bf16 with the e4m3 scale folded in (exact: q*s has <= 6 significant
//    bits).  One 32-bit code word = two scale blocks x 4 codes = one MFMA
//    operand, so the dequantised tile is reused by every activation row tile
//    of the wave without touching LDS.
//  * fp32 accumulation in the MFMA; y = g * acc stored once.
#include "q4p_device.h"
#include "q4p_launch.h"

namespace q4p {

namespace {

constexpr int kBM = 128;          // activation rows per workgroup
constexpr int kXPitch = 272;      // LDS bytes per staged activation row (256 + 16)
constexpr int kMaxT = 19;         // weight tiles per workgroup (Q <= 4)

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

template <int Q, int RT>
__global__ void __launch_bounds__(256)
gemm_kernel(const uint4 *__restrict__ pcodes, const uint2 *__restrict__ pscales, float g,
            const uint16_t *__restrict__ x, float *__restrict__ y, int M, int N, int K, int KT,
            int NT, int T)
{
    __shared__ __attribute__((aligned(16))) uint8_t xs[2][kBM * kXPitch];

    const int w = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int r = lane & 15;
    const int gq = lane >> 4;
    const int m0 = blockIdx.y * kBM;
    const int tile0 = blockIdx.x * T;

    // weight tiles of this wave
    int tf[Q > 0 ? Q : 1];
    int tr[RT > 0 ? RT : 1];
#pragma unroll
    for (int j = 0; j < Q; ++j)
        tf[j] = tile0 + w * Q + j;
#pragma unroll
    for (int j = 0; j < RT; ++j)
        tr[j] = tile0 + 4 * Q + j;

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

    // ---- activation staging: thread -> (row srow + 16p, 8 k at 8*su) ----
    const int su = threadIdx.x & 15;
    const int srow = threadIdx.x >> 4;
    uint4 xst[8];
    auto load_x = [&](int c) {
        const int k = c * kTileK + 8 * su;
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            const int row = m0 + 16 * p + srow;
            xst[p] = (row < M && k < K)
                         ? *reinterpret_cast<const uint4 *>(x + (int64_t)row * K + k)
                         : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    // element 8*su + e of a k-tile goes to operand slot (d, g', h, i) with
    // d = su/4, h = (su/2)&1, g' = 2*(su&1) + e/4, i = e&3
    const int sd = su >> 2, sh = (su >> 1) & 1, sg = 2 * (su & 1);
    const int posA = (((sd * 4 + sg) * 8) + sh * 4) * 2;
    const int posB = (((sd * 4 + sg + 1) * 8) + sh * 4) * 2;
    auto store_x = [&](int buf) {
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            uint8_t *base = &xs[buf][(16 * p + srow) * kXPitch];
            *reinterpret_cast<uint2 *>(base + posA) = make_uint2(xst[p].x, xst[p].y);
            *reinterpret_cast<uint2 *>(base + posB) = make_uint2(xst[p].z, xst[p].w);
        }
    };

    // ---- weight streaming ----
    uint4 cF[Q > 0 ? Q : 1], nF[Q > 0 ? Q : 1];
    uint2 sF[Q > 0 ? Q : 1], nsF[Q > 0 ? Q : 1];
    uint4 cR[RT > 0 ? RT : 1], nR[RT > 0 ? RT : 1];
    uint2 sR[RT > 0 ? RT : 1], nsR[RT > 0 ? RT : 1];
    auto load_w = [&](int c, uint4 *dc, uint2 *ds, uint4 *dcr, uint2 *dsr) {
#pragma unroll
        for (int j = 0; j < Q; ++j) {
            if (tf[j] < NT) {
                const int64_t tc = (int64_t)tf[j] * KT + c;
                dc[j] = load_stream16(pcodes + tc * 64 + lane);
                ds[j] = pscales[tc * 16 + r];
            }
        }
#pragma unroll
        for (int j = 0; j < RT; ++j) {
            if (tr[j] < NT) {
                const int64_t tc = (int64_t)tr[j] * KT + c;
                dcr[j] = load_stream16(pcodes + tc * 64 + lane);
                dsr[j] = pscales[tc * 16 + r];
            }
        }
    };

    load_x(0);
    load_w(0, cF, sF, cR, sR);
    store_x(0);
    __syncthreads();

    for (int c = 0; c < KT; ++c) {
        const int buf = c & 1;
        const bool more = c + 1 < KT;
        if (more) {
            load_x(c + 1);
            load_w(c + 1, nF, nsF, nR, nsR);
        }
        const uint8_t *xb = xs[buf];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const int off = (d * 4 + gq) * 16;
            bf16x8_t a[8];
#pragma unroll
            for (int mt = 0; mt < 8; ++mt)
                a[mt] = __builtin_bit_cast(
                    bf16x8_t, *reinterpret_cast<const uint4 *>(xb + (16 * mt + r) * kXPitch + off));
#pragma unroll
            for (int j = 0; j < Q; ++j) {
                if (tf[j] < NT) {
                    bf16x8_t b;
                    switch (d) {
                    case 0: b = weight_operand<0>(cF[j], sF[j]); break;
                    case 1: b = weight_operand<1>(cF[j], sF[j]); break;
                    case 2: b = weight_operand<2>(cF[j], sF[j]); break;
                    default: b = weight_operand<3>(cF[j], sF[j]); break;
                    }
#pragma unroll
                    for (int mt = 0; mt < 8; ++mt)
                        accF[j][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mt], b, accF[j][mt], 0, 0, 0);
                }
            }
#pragma unroll
            for (int j = 0; j < RT; ++j) {
                if (tr[j] < NT) {
                    bf16x8_t b;
                    switch (d) {
                    case 0: b = weight_operand<0>(cR[j], sR[j]); break;
                    case 1: b = weight_operand<1>(cR[j], sR[j]); break;
                    case 2: b = weight_operand<2>(cR[j], sR[j]); break;
                    default: b = weight_operand<3>(cR[j], sR[j]); break;
                    }
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        const bf16x8_t ar = __builtin_bit_cast(
                            bf16x8_t, *reinterpret_cast<const uint4 *>(
                                          xb + (16 * (2 * w + i) + r) * kXPitch + off));
                        accR[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ar, b, accR[j][i], 0, 0, 0);
                    }
                }
            }
        }
        if (more) {
            store_x(buf ^ 1);
#pragma unroll
            for (int j = 0; j < Q; ++j) {
                cF[j] = nF[j];
                sF[j] = nsF[j];
            }
#pragma unroll
            for (int j = 0; j < RT; ++j) {
                cR[j] = nR[j];
                sR[j] = nsR[j];
            }
        }
        __syncthreads();
    }

    // ---- epilogue: lane (r, gq) holds rows 4*gq + i of each 16-row M tile ----
#pragma unroll
    for (int j = 0; j < Q; ++j) {
        const int n = tf[j] * 16 + r;
        if (tf[j] < NT && n < N) {
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
        const int n = tr[j] * 16 + r;
        if (tr[j] < NT && n < N) {
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
    Q4P_GEMM_ENTRY(16),  Q4P_GEMM_ENTRY(17), Q4P_GEMM_ENTRY(18), Q4P_GEMM_ENTRY(19),
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
    const dim3 grid((unsigned)NB, (unsigned)MB), block(256);
    hipLaunchKernelGGL(kGemmTable[T], grid, block, 0, stream,
                       reinterpret_cast<const uint4 *>(packed_codes),
                       reinterpret_cast<const uint2 *>(packed_scales), g, x, y, (int)M, (int)N,
                       (int)K, (int)KT, (int)NT, (int)T);
    return hipGetLastError();
}

}  // namespace q4p
