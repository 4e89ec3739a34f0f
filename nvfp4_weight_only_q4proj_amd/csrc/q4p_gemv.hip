// q4p_gemv.hip — decode / speculative-verify projection, 1 <= M <= 16.
//
// At M = 1..16 every weight byte feeds at most 16 multiply-adds, so the
// kernel is bound by streaming the packed weight from HBM once (0.5625 bytes
// per weight).  Two kernels share the per-block arithmetic (gemv_half):
//
//  * gemv_sk_kernel, the stream-K kernel further down: every CU streams an
//    equal contiguous range of the k-tiles of all row tiles.  It serves every
//    shape whose activations of at most 8 K ranges fit in LDS and whose
//    packed codes stay below 4 GiB: all the decode, verify and lm-head shapes.
//  * gemv_kernel, the split kernel described next, for the remaining shapes
//    (M*K beyond the LDS budget, or codes of 4 GiB and more).
//
// Split kernel:
//
//  * A workgroup owns TB 16-row tiles of W; S waves per tile split its
//    k-tiles into contiguous ranges (split-K inside the workgroup), and the
//    partial sums are added through LDS in a fixed order, so results are
//    bitwise deterministic.  The host picks (TB, S) from the occupancy API so
//    that, where possible, every workgroup is resident at once: no tail round.
//  * Each wave keeps PF k-tiles in flight in a register ring: the 1 KB code
//    tile (16 B per lane) and the 128 B scale tile (8 B per lane); every
//    wave-wide weight load is a contiguous 1 KB segment.
//  * Per 16-element scale block the wave issues one 16x16x16 bf16 MFMA:
//    A = activation rows (lane row r, k-group g holds 4 values), B = the 16
//    weight rows' unscaled e2m1 values (exact in bf16).  The MFMA returns the
//    block's partial sums p[m][n] = sum_{k in block} x[m][k] q[n][k]; the lane
//    accumulates acc += s[n][block] * p with one fma per live output row.
//    Folding the e4m3 scale into the operand instead would cost two more
//    multiplies per code pair, because gfx950's fp4 conversion honours only
//    the exponent of its scale operand.
//  * Activations, when M*K fits (decode, lm-head): each wave copies the
//    activations of its own k-range into LDS once, permuted so that a lane's
//    32 values of a k-tile are 64 contiguous bytes (two 16-byte LDS reads per
//    half tile); no workgroup barrier stands between a wave and its first
//    tile.  Lanes whose A row is >= M read a zero strip.
//  * Activations otherwise (larger M*K, e.g. verify with K = 17408): the
//    pieces ride in the register ring with the weights.  A rows >= M only
//    produce discarded output rows, so for small M one register pair holds
//    the pieces of BPP blocks (lane m + M*t holds block t's piece of row m)
//    and a DPP row shift by M*t moves block t's pieces into lanes 0..M-1
//    just before its MFMA.  M <= 2 needs one pair per k-tile, M <= 4 two,
//    M <= 8 four, larger M eight (no shifts).
//  * g is applied once per output after the reduction, in fp32.
#include <mutex>
#include <vector>

#include "q4p_device.h"
#include "q4p_launch.h"

// Exchange words of q4proj_gemv_noalloc: a device array inside the library
// (one copy per GPU, held until the process ends) in place of the caller's
// workspace.  Host code never uses this name as an address: it asks the
// runtime for each device's address once and passes that to the kernels.
static constexpr size_t kScratchBytes = 8u << 20;
static __device__ __align__(256) unsigned long long scratch[kScratchBytes / 8];

namespace q4p {

namespace {

constexpr int kMaxWaves = 16;          // waves per workgroup
constexpr int kZeroBytes = 64;         // zero strip for activation rows >= M
constexpr int kXLdsMaxBytes = 40 * 1024;
constexpr int kXStage = 8;             // staged activation groups per lane

// Compile-time shape for M (MT = M for M <= 8, MT = 0 for 9 <= M <= 16).
template <int MT, bool XLDS>
struct Shape {
    static constexpr int kPairs = XLDS ? 0 : MT == 0 ? 8 : MT <= 2 ? 1 : MT <= 4 ? 2 : 4;
    static constexpr int kBpp = XLDS ? 1 : 8 / kPairs;          // blocks per pair
    static constexpr int kRows = MT == 0 ? 4 : (MT < 4 ? MT : 4);   // live acc rows
    static constexpr int kPrefetch = XLDS ? 6 : kPairs <= 1 ? 6 : kPairs <= 2 ? 5 : kPairs <= 4 ? 4 : 3;
    static constexpr int kRing = kPairs > 0 ? kPairs : 1;
};

// row shift within each 16-lane DPP row: lane i <- lane i + SH
template <int SH>
__device__ __forceinline__ uint2 shift_rows(uint2 v)
{
    if (SH == 0)
        return v;
    return make_uint2((uint32_t)__builtin_amdgcn_mov_dpp((int)v.x, 0x100 | SH, 0xF, 0xF, false),
                      (uint32_t)__builtin_amdgcn_mov_dpp((int)v.y, 0x100 | SH, 0xF, 0xF, false));
}

// runtime-valued shift that folds to one of the immediates once the caller's
// loops are unrolled
__device__ __forceinline__ uint2 shift_rows_n(uint2 v, int sh)
{
    switch (sh) {
    case 1: return shift_rows<1>(v);
    case 2: return shift_rows<2>(v);
    case 3: return shift_rows<3>(v);
    case 4: return shift_rows<4>(v);
    case 5: return shift_rows<5>(v);
    case 6: return shift_rows<6>(v);
    case 7: return shift_rows<7>(v);
    case 8: return shift_rows<8>(v);
    case 9: return shift_rows<9>(v);
    case 10: return shift_rows<10>(v);
    case 11: return shift_rows<11>(v);
    case 12: return shift_rows<12>(v);
    case 13: return shift_rows<13>(v);
    case 14: return shift_rows<14>(v);
    case 15: return shift_rows<15>(v);
    default: return v;
    }
}

// Accumulate half a k-tile (scale blocks 4H..4H+3); xa(b) gives block b's
// A operand.  Working in halves keeps the live MFMA results small.
template <int ROWS, int H, typename XA>
__device__ __forceinline__ void gemv_half(const uint4 &cw, const uint2 &sw, XA &&xa, floatx4_t &acc)
{
    const uint32_t w0 = H ? cw.z : cw.x;
    const uint32_t w1 = H ? cw.w : cw.y;
    const uint32_t sv = H ? sw.y : sw.x;
    const floatx4_t zero = {0.f, 0.f, 0.f, 0.f};
    floatx4_t p[4];
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
        const uint32_t w = (bb < 2) ? w0 : w1;
        uint32_t lo, hi;
        if (bb & 1) {
            lo = fp4x2_to_bf16x2<2>(w);
            hi = fp4x2_to_bf16x2<3>(w);
        } else {
            lo = fp4x2_to_bf16x2<0>(w);
            hi = fp4x2_to_bf16x2<1>(w);
        }
        const short4_t a = __builtin_bit_cast(short4_t, xa(4 * H + bb));
        const short4_t bq = __builtin_bit_cast(short4_t, make_uint2(lo, hi));
        p[bb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, bq, zero, 0, 0, 0);
    }
    // the block scales, two per conversion (OCP e4m3 on gfx950)
    const floatx2_t s01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)sv, false);
    const floatx2_t s23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)sv, true);
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
        const float s = bb == 0 ? s01[0] : bb == 1 ? s01[1] : bb == 2 ? s23[0] : s23[1];
#pragma unroll
        for (int i = 0; i < ROWS; ++i)
            acc[i] = __builtin_fmaf(s, p[bb][i], acc[i]);
    }
}

template <int MT, bool XLDS>
__global__ void __launch_bounds__(64 * kMaxWaves)
gemv_kernel(const uint4 *__restrict__ pcodes, const uint2 *__restrict__ pscales, float g,
            const uint16_t *__restrict__ x, float *__restrict__ y, int M, int N, int K, int KT,
            int NT, int TB, int S)
{
    using X = Shape<MT, XLDS>;
    constexpr int PF = X::kPrefetch;
    constexpr int PAIRS = X::kPairs;
    constexpr int BPP = X::kBpp;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63;
    const int r = lane & 15;          // weight row in the tile / A-operand row
    const int gq = lane >> 4;         // k-group within each scale block
    const int tb = wave / S;
    const int ks = wave - tb * S;
    const int t = blockIdx.x * TB + tb;
    const bool live = t < NT;
    const int c0 = (int)(((int64_t)KT * ks) / S);
    const int c1 = (int)(((int64_t)KT * (ks + 1)) / S);
    const int n = live ? c1 - c0 : 0;
    const int last = n > 0 ? n - 1 : 0;

    const int xbytes = XLDS ? M * KT * 256 : 0;
    uint8_t *xl = smem;
    uint8_t *zstrip = smem + xbytes;
    floatx4_t *red = reinterpret_cast<floatx4_t *>(smem + xbytes + (XLDS ? kZeroBytes : 0));

    const uint4 *pc = pcodes + ((int64_t)(live ? t : 0) * KT + c0) * 64 + lane;
    const uint2 *ps = pscales + ((int64_t)(live ? t : 0) * KT + c0) * 16 + r;

    // ---- activation pieces riding in the ring (!XLDS) ----
    // This lane's piece in pair j of k-tile c: row xm, block j*BPP + xt,
    // k = 128c + 16(j*BPP + xt) + 4gq.  Lanes past the packed pieces repeat
    // the last one (their A rows are discarded).
    const int mm = MT == 0 ? 16 : MT;
    int xm = MT == 0 ? r : r % mm;
    int xt = MT == 0 ? 0 : r / mm;
    if (xt > BPP - 1)
        xt = BPP - 1;
    if (xm > M - 1)
        xm = M - 1;
    const int xk = 16 * xt + 4 * gq;
    const uint16_t *xrowg = x + (int64_t)xm * K;

    // 1. issue this wave's activation staging loads.  With split-K (S > 1)
    //    each wave stages exactly the k-tiles it will read, so no workgroup
    //    barrier stands between a wave and its first tile; with several row
    //    tiles per workgroup (TB > 1) the waves share one copy of all K,
    //    staged in TB parts behind a barrier.
    const int sc0 = TB > 1 ? (int)(((int64_t)KT * tb) / TB) : c0;
    const int sn = TB > 1 ? (int)(((int64_t)KT * (tb + 1)) / TB) - sc0 : n;
    const int gpr = sn * 32;                   // 8-byte groups per activation row
    const int wn = gpr * M;                    // groups staged by this wave
    // group lane + 64*j of this wave is (row, q): walk rows without dividing
    int srow[kXStage], sq[kXStage];
    if (XLDS) {
        int row = 0, q = lane;
#pragma unroll
        for (int j = 0; j < kXStage; ++j) {
            while (q >= gpr && row < M) {
                q -= gpr;
                ++row;
            }
            srow[j] = row;
            sq[j] = q;
            q += 64;
        }
    }
    uint2 xv[kXStage];
    if (XLDS) {
#pragma unroll
        for (int j = 0; j < kXStage; ++j) {
            const int k = 128 * sc0 + 4 * sq[j];
            xv[j] = make_uint2(0u, 0u);
            if (srow[j] < M && k < K)
                xv[j] = *reinterpret_cast<const uint2 *>(x + (int64_t)srow[j] * K + k);
        }
    }

    // ---- weight ring (+ activation pieces when !XLDS) ----
    uint4 cw[PF];
    uint2 sw[PF];
    uint2 xq[PF][X::kRing];
    // Reloads past the end of the range re-read the wave's last tile: the
    // load stays unconditional (a conditional reload makes each ring slot a
    // phi, resolved with copies that wait for every load in flight) and it
    // hits lines this wave is fetching anyway.
    auto load = [&](int u, int idx) {
        const int j = idx < n ? idx : last;
        cw[u] = load_stream16(pc + (int64_t)j * 64);
        sw[u] = ps[(int64_t)j * 16];
        if (!XLDS) {
            const int kc = 128 * (c0 + j) + xk;
#pragma unroll
            for (int q = 0; q < PAIRS; ++q) {
                const int k = kc + 16 * BPP * q;
                xq[u][q] = *reinterpret_cast<const uint2 *>(xrowg + (k < K ? k : 0));
            }
        }
    };
    // prologue in slot order: the loop-entry state is merged into the loop's
    // wait counts, so a reordered prologue would make every iteration wait
    // for all loads in flight
#pragma unroll
    for (int u = 0; u < PF; ++u) {
        load(u, u);
        __builtin_amdgcn_sched_barrier(0);
    }

    // 3. write the activations to LDS, permuted so that lane (r, gq) finds its
    //    32 values of k-tile c at xl + ((r*KT + c)*4 + gq)*64
    if (XLDS) {
        auto put = [&](int row, int q, uint2 v) {
            const int c = sc0 + (q >> 5), qq = q & 31;
            *reinterpret_cast<uint2 *>(xl + ((row * KT + c) * 4 + (qq & 3)) * 64 + (qq >> 2) * 8) = v;
        };
#pragma unroll
        for (int j = 0; j < kXStage; ++j)
            if (srow[j] < M)
                put(srow[j], sq[j], xv[j]);
        // groups beyond kXStage per lane (long k-ranges or many rows)
        if (wn > 64 * kXStage) {
            int row = srow[kXStage - 1], q = sq[kXStage - 1] + 64;
            for (;;) {
                while (q >= gpr && row < M) {
                    q -= gpr;
                    ++row;
                }
                if (row >= M)
                    break;
                const int k = 128 * sc0 + 4 * q;
                put(row, q, k < K ? *reinterpret_cast<const uint2 *>(x + (int64_t)row * K + k)
                                  : make_uint2(0u, 0u));
                q += 64;
            }
        }
        if (lane < kZeroBytes / 4)
            reinterpret_cast<uint32_t *>(zstrip)[lane] = 0u;   // same zeros from every wave
        if (TB > 1) {
            __syncthreads();
        } else {
            // the wave reads back only its own writes: wait for them to land
            __builtin_amdgcn_s_waitcnt(0xc07f);                  // lgkmcnt(0)
            __builtin_amdgcn_wave_barrier();
        }
    }

    const uint8_t *xls = (r < M) ? xl + (r * KT * 4 + gq) * 64 : zstrip;
    const int xstep = (r < M) ? 256 : 0;

    floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
    auto tile = [&](int u, int idx) {
        const int c = c0 + idx;
        if (XLDS) {
            const uint4 *src = reinterpret_cast<const uint4 *>(xls + c * xstep);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint2 xf[4];
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const uint4 v = src[2 * h + j];
                    xf[2 * j] = make_uint2(v.x, v.y);
                    xf[2 * j + 1] = make_uint2(v.z, v.w);
                }
                auto xa = [&](int b) { return xf[b & 3]; };
                if (h == 0)
                    gemv_half<X::kRows, 0>(cw[u], sw[u], xa, acc);
                else
                    gemv_half<X::kRows, 1>(cw[u], sw[u], xa, acc);
            }
        } else {
            uint2 xv[X::kRing];
#pragma unroll
            for (int q = 0; q < PAIRS; ++q)
                xv[q] = xq[u][q];
            if (128 * c + 128 > K) {
                // k-tile padding past K (K % 128 != 0): zero those activations
#pragma unroll
                for (int q = 0; q < PAIRS; ++q)
                    if (128 * c + xk + 16 * BPP * q >= K)
                        xv[q] = make_uint2(0u, 0u);
            }
            auto xa = [&](int b) { return shift_rows_n(xv[b / BPP], MT == 0 ? 0 : MT * (b % BPP)); };
            gemv_half<X::kRows, 0>(cw[u], sw[u], xa, acc);
            gemv_half<X::kRows, 1>(cw[u], sw[u], xa, acc);
        }
        // pin this tile's fma chain here; otherwise chains are sunk past
        // later tiles' MFMAs, which then all stay live
        asm volatile("" : "+v"(acc));
        __builtin_amdgcn_sched_barrier(0);
    };

    for (int i = 0; i < n; i += PF) {
#pragma unroll
        for (int u = 0; u < PF; ++u) {
            if (i + u < n)
                tile(u, i + u);
            load(u, i + u + PF);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    if (S > 1) {
        red[wave * 64 + lane] = acc;
        __syncthreads();
        if (ks == 0) {
            acc = red[(tb * S) * 64 + lane];
            for (int v = 1; v < S; ++v)
                acc += red[(tb * S + v) * 64 + lane];
        }
    }
    if (ks == 0 && live) {
        // lane (r, gq) holds outputs y[4*gq + i][16*t + r], i = 0..3
        const int col = 16 * t + r;
        if (col < N) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int m = 4 * gq + j;
                if (m < M)
                    y[(int64_t)m * N + col] = g * acc[j];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Stream-K variant, used whenever the activations of at most 8 K ranges fit
// in LDS and the packed codes stay below 4 GiB (32-bit buffer offsets).
//
// The k-tiles of all row tiles, in packed-memory order (row tile t, k-tile c
// at unit t*KT + c), are dealt out in equal contiguous ranges: G workgroups,
// one per CU (each asks for more than half the CU's LDS, so no two share a
// CU), then WPG waves per workgroup.  Every CU streams the same number of
// bytes.  With 8 waves per CU and 4 tiles in flight per wave the chip keeps
// about 9 MB of requests queued, where HBM delivers best: deeper queues from
// every wave at once, or fewer waves with deeper rings, measured slower.
//
// A wave flushes its accumulator at each row-tile boundary.  A row tile that
// lies wholly inside one wave is stored directly.  Partial row tiles go to
// LDS; after the stream the lowest contributing wave of the workgroup adds
// the parts in wave order.  A row tile that also continues in the
// neighbouring workgroup (ranges are at least KT units, so at most two
// workgroups share one) is finished through a 64-bit exchange per output:
// each side swaps (flag, partial) into a workspace word; the side that finds
// the flag set adds the two partials -- fp32 addition of two values is
// commutative, so the result does not depend on which side comes second --
// stores y and clears the word for the next call.  No fences, no waiting.
//
// K may be cut into KS ranges (a power of two), each streamed as above by
// its own G/KS workgroups, which then stage only their range's activations.
// The KS partial results of an output are joined along a fixed binary tree of
// the same two-party exchanges (ranges 2i and 2i+1 first, then pairs of
// pairs, ...): each join adds two values, so the total does not depend on
// arrival order either.  The tree's words follow the boundary words in the
// workspace, one per output and join.  When a lane holds two or more rows of
// a column (M > 4) it exchanges two rows per word, with the NaN-keyed pair
// encoding below, both between workgroups and up the tree, so the side that
// completes one row completes its partner row too.  KS trades staging (every
// workgroup reads its range's activations into LDS) against joining; the
// launcher picks the count with the least measured cost (sk_ranges).
//
// Every wave starts at once and the launch ends with the last finish, so the
// scalar work before a wave's first loads and after its last unit adds to
// every launch: the host precomputes the unit split and a reciprocal for
// the staging map, and the finish finds its partner waves without dividing.

constexpr int kSkMaxGroups = 256;
constexpr int kSkMaxWaves = 8;
constexpr int kSkPrefetch = 4;
// ring depth for M <= 4 with one K range when a wave streams few units (the
// 4B-model decode shapes, ~6 units per wave): three in flight were 1-2.5 %
// faster there, and slower on the 50 MB shapes (21 units per wave)
constexpr int kSkPrefetchShort = 3;
constexpr int kSkShortUnits = 10;
// activations of a range in LDS: all of a CU's 160 KB beside the zero strip
// and the partial sums of 8 waves (2 x 1 KB each)
constexpr int kSkXMaxBytes = 160 * 1024 - kZeroBytes - kSkMaxWaves * 2 * 64 * 16;
constexpr int kSkLdsFloor = 96 * 1024;
// 16-byte activation loads per lane issued together before the ring (the
// rest follow one at a time): 8 when M <= 4, 16 above, where the activations
// of a range take up to 16 loads per lane; more staging slots at M <= 4 only
// delayed the first weight loads (a 4 % slower decode GEMV at M = 1)
constexpr int sk_stage(int rows) { return rows >= 2 ? 16 : 8; }

constexpr int kSkMaxRanges = 8;               // K ranges joined by the exchange tree
constexpr int64_t kSkBoundaryWords = (int64_t)kSkMaxGroups * 64 * 4;

struct SkArgs {
    int M, N, K, KT, NT, G, WPG;
    int KS, KTR;                               // K ranges, k-tiles per range (last may be shorter)
    float g;
    float *best_val;                           // argmax epilogue: per-row result
    int64_t *best_idx;
    // Division-free set-up, filled by the host: workgroups per K range; per
    // range kind (0: KTR k-tiles, 1: the shorter last range) the units per
    // workgroup (base, remainder) and the per-wave split (base, remainder)
    // of a workgroup range of `base` and of `base + 1` units; and
    // ceil(2^32 / (16 * k-tiles)), so that umulhi(i, xrcp) = i / (16 * k-tiles)
    // for the staging group indices i (i * 16 * k-tiles < 2^32).
    int GR;
    int split[2][6];
    uint32_t xrcp[2];
};

// Epilogues of the stream-K kernel
constexpr int kEpiY = 0;                       // y = g * acc (fp32)
constexpr int kEpiSilu = 1;                    // fused gate/up: h = bf16(silu(gate) * up)
constexpr int kEpiArgmax = 2;                  // y optional; per-row max value and index

// Argmax key of value v at column col: an order-preserving map of v in the
// high half (NaN above every number, -0 equal to +0) and ~col in the low half,
// so the largest key is the largest value at its lowest column -- the first
// maximum, NaN counting as the largest, as a greedy argmax over the logits
// reads it.  Max over keys is exact and order-independent.
__device__ __forceinline__ unsigned long long argmax_key(float v, int col)
{
    const uint32_t b = __builtin_bit_cast(uint32_t, v);
    uint32_t o;
    if ((b & 0x7FFFFFFFu) > 0x7F800000u)
        o = 0xFFFFFFFFu;
    else if ((b & 0x7FFFFFFFu) == 0u)
        o = 0x80000000u;
    else
        o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return ((unsigned long long)o << 32) | (0xFFFFFFFFu - (uint32_t)col);
}

__device__ __forceinline__ float argmax_key_value(unsigned long long k)
{
    const uint32_t o = (uint32_t)(k >> 32);
    if (o == 0xFFFFFFFFu)
        return __builtin_nanf("");
    return __builtin_bit_cast(float, (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// A gate/up pair of partial sums in one 64-bit exchange word.  Both fields
// are XORed with a NaN pattern that no stored value has (a NaN is stored as
// the one canonical quiet NaN), so a word holding a pair is never zero and
// zero still means empty.
constexpr uint32_t kPairKey = 0x7FC00001u;

__device__ __forceinline__ uint32_t pair_field(float v)
{
    const uint32_t b = __builtin_bit_cast(uint32_t, v);
    return ((b & 0x7FFFFFFFu) > 0x7F800000u ? 0x7FC00000u : b) ^ kPairKey;
}

__device__ __forceinline__ unsigned long long pair_word(float gate, float up)
{
    return ((unsigned long long)pair_field(up) << 32) | pair_field(gate);
}

__device__ __forceinline__ float pair_gate(unsigned long long w)
{
    return __builtin_bit_cast(float, (uint32_t)w ^ kPairKey);
}

__device__ __forceinline__ float pair_up(unsigned long long w)
{
    return __builtin_bit_cast(float, (uint32_t)(w >> 32) ^ kPairKey);
}

// SILU: the weight is a fused gate/up projection of 2F rows in which 8 gate
// rows and the matching 8 up rows alternate, so row tile t holds the gate
// rows (lanes r < 8) and the up rows (lanes r >= 8) of outputs f = 8t..8t+7.
// Wherever a tile's values complete, a row rotate hands lane r + 8's value
// to lane r; exchanges between workgroups and K ranges then carry (gate, up)
// in one word from lane r, and the side that completes a pair applies the
// epilogue.  out is bf16 h[M][F] instead of fp32 y[M][N].
//
// ARGMAX: y is stored only when out is not null; every completed output also
// updates its lane's running best key per row (argmax_key).  After the finish
// the workgroup reduces its keys (16 lanes, then the waves through LDS) and
// adds them to one 64-bit atomic max per row in the workspace, waits for
// those atomics to return, and counts itself done on a counter word; the
// workgroup that brings the count to G reads and clears the row keys with
// atomic exchanges, clears the counter and writes each row's value and
// index.  The row keys and the counter are touched only by device-scope
// atomics, which are performed where all XCDs see them, and an atomic that
// has returned has been performed: so no cache write-back or invalidation
// is needed (an agent-scope fence here costs an L2 write-back per workgroup
// while others are still streaming).
template <int ROWS, int PF, bool KR, int EPI>
__global__ void __launch_bounds__(64 * kSkMaxWaves)
gemv_sk_kernel(const uint4 *__restrict__ pcodes, const uint2 *__restrict__ pscales,
               const uint16_t *__restrict__ x, void *__restrict__ out,
               unsigned long long *__restrict__ xch, SkArgs a)
{
    constexpr bool SILU = EPI == kEpiSilu;
    constexpr bool ARGMAX = EPI == kEpiArgmax;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63;
    const int r = lane & 15;
    const int gq = lane >> 4;
    // Output rows of a lane: the MFMA gives lane (r, gq) the rows 4gq..4gq+3
    // of A.  With ROWS = ceil(M/4) activation row m is placed at A row
    // 4*(m/ROWS) + m%ROWS, so a lane's live rows are its first ROWS slots,
    // ROWS*gq + j, and the per-block scale costs ROWS fmas per lane instead
    // of four (ROWS = 4, M > 12: A row i is row i).
    auto out_row = [](int q, int j) { return ROWS * q + j; };
    const int G = a.G, WPG = a.WPG, KTG = a.KT, M = a.M, K = a.K;

    // workgroup b takes the b-th range.  (Giving consecutive ranges to the
    // workgroups of one XCD, so that exchange partners share an L2, measured
    // 1-2.5% slower: the exchange words are device-scope atomics either way,
    // and spreading each XCD's stream over the whole matrix serves HBM
    // better.)
    const int LG = blockIdx.x;
    // K range of this workgroup: k-tiles c0 .. c0 + KT - 1, streamed by the
    // GR workgroups of that range; below, units, KT and L are range-local.
    // Every instruction before the first loads adds to the launch, so the
    // divisions of this set-up come precomputed from the host (a.split).
    const int GR = a.GR;
    const int kr = KR ? LG / GR : 0;
    const int L = LG - kr * GR;
    const int c0 = kr * a.KTR;
    const int KT = KTG - c0 < a.KTR ? KTG - c0 : a.KTR;
    const int kind = KR && KT != a.KTR ? 1 : 0;
    // balanced split: the first `urem` groups (and, inside a group, the first
    // `wr` waves) take one unit more
    const int ubase = kind ? a.split[1][0] : a.split[0][0];
    const int urem = kind ? a.split[1][1] : a.split[0][1];
    const bool more = L < urem;
    const int UW0 = L * ubase + (more ? L : urem);
    const int UWn = ubase + (more ? 1 : 0);
    const int UW1 = UW0 + UWn;
    const int wb = kind ? (more ? a.split[1][4] : a.split[1][2]) : (more ? a.split[0][4] : a.split[0][2]);
    const int wr = kind ? (more ? a.split[1][5] : a.split[1][3]) : (more ? a.split[0][5] : a.split[0][3]);
    auto wave_start = [&](int v) { return UW0 + v * wb + (v < wr ? v : wr); };
    const int u0 = wave_start(wave), u1 = wave_start(wave + 1);
    const int n = u1 - u0;
    const int ulast = n > 0 ? u1 - 1 : 0;

    const int xbytes = M * KT * 256;
    uint8_t *xl = smem;
    uint8_t *zstrip = smem + xbytes;
    floatx4_t *part = reinterpret_cast<floatx4_t *>(smem + xbytes + kZeroBytes);

    // 1. activation staging loads (rows < M, the k-tiles of this range)
    constexpr int kSkStage = sk_stage(ROWS);
    const int nthr = 64 * WPG;
    const int gpr = KT * 16;                   // 16-byte groups per activation row
    const int kbase = c0 * 128;
    const int ngroups = M * gpr;
    // group tid + i*nthr is (row srow[i], group sq[i] of that row); rows past
    // M are marked M
    uint4 xs[kSkStage];
    int srow[kSkStage], sq[kSkStage];
    {
        const uint32_t xrcp = kind ? a.xrcp[1] : a.xrcp[0];
#pragma unroll
        for (int i = 0; i < kSkStage; ++i) {
            const uint32_t gi = threadIdx.x + (uint32_t)(i * nthr);
            const int row = (int)__umulhi(gi, xrcp);
            srow[i] = row < M ? row : M;
            sq[i] = (int)gi - row * gpr;
        }
    }
#pragma unroll
    for (int i = 0; i < kSkStage; ++i) {
        xs[i] = make_uint4(0u, 0u, 0u, 0u);
        const int k = kbase + sq[i] * 8;
        if (srow[i] < M && k < K)
            xs[i] = *reinterpret_cast<const uint4 *>(x + (int64_t)srow[i] * K + k);
    }

    // 2. weight ring prologue, in slot order.
    //    One K range: the wave's units are contiguous in the packed buffers,
    //    so each wave gets descriptors sized to its own units; a load past its
    //    last unit falls outside and returns zeros without a memory access,
    //    and the ring needs no per-load bookkeeping (position p reads code
    //    offset 1024p and scale offset 128p).
    //    K ranges: a unit's packed index is t*KTG + c0 + c for (row tile t,
    //    range-local k-tile c), walked incrementally, with loads past the
    //    wave's last unit on a descriptor of size 0.
    const uint32_t cbytes = (uint32_t)((int64_t)a.NT * KTG * 1024);
    const uint32_t sbytes = (uint32_t)((int64_t)a.NT * KTG * 128);
    uint4 cw[PF];
    uint2 sw[PF];
    const auto rc_w = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint4 *>(pcodes + (int64_t)(KR ? 0 : u0) * 64), 0, (int)(KR ? 0u : (uint32_t)n * 1024u), 0x00020000);
    const auto rs_w = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint2 *>(pscales + (int64_t)(KR ? 0 : u0) * 16), 0, (int)(KR ? 0u : (uint32_t)n * 128u), 0x00020000);
    auto load_pos = [&](int s, int pos) {
        const u32x4_t c = __builtin_amdgcn_raw_buffer_load_b128(rc_w, lane * 16, pos * 1024, 2 /* non-temporal */);
        cw[s] = make_uint4(c.x, c.y, c.z, c.w);
        const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(rs_w, r * 8, pos * 128, 0);
        sw[s] = make_uint2(v.x, v.y);
    };
    int ld_q = 0;                              // loads issued by this wave
    int ld_u = u0, ld_t = KR && n > 0 ? u0 / KT : 0, ld_c = KR && n > 0 ? u0 - ld_t * KT : 0;
    auto load = [&](int s) {
        const uint32_t j = (uint32_t)(ld_t * KTG + c0 + ld_c);
        const bool live = ld_q < n;
        ++ld_q;
        const u32x4_t c = __builtin_amdgcn_raw_buffer_load_b128(
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4 *>(pcodes), 0, (int)(live ? cbytes : 0u), 0x00020000),
            lane * 16, j * 1024u, 2 /* non-temporal */);
        cw[s] = make_uint4(c.x, c.y, c.z, c.w);
        const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint2 *>(pscales), 0, (int)(live ? sbytes : 0u), 0x00020000),
            r * 8, j * 128u, 0);
        sw[s] = make_uint2(v.x, v.y);
        if (ld_u < ulast) {
            ++ld_u;
            if (++ld_c == KT) {
                ld_c = 0;
                ++ld_t;
            }
        }
    };
#pragma unroll
    for (int s = 0; s < PF; ++s) {
        if (KR)
            load(s);
        else
            load_pos(s, s);
        __builtin_amdgcn_sched_barrier(0);
    }

    // 3. activations to LDS: lane (r, gq) finds its 32 values of k-tile c at
    //    xl + ((r*KT + c)*4 + gq)*64
    auto put = [&](int m, int q, uint4 v) {
        const int c = q >> 4, j = q & 15;
        uint8_t *base = xl + ((m * KT + c) * 4 + ((2 * j) & 3)) * 64 + (j >> 1) * 8;
        *reinterpret_cast<uint2 *>(base) = make_uint2(v.x, v.y);
        *reinterpret_cast<uint2 *>(base + 64) = make_uint2(v.z, v.w);
    };
#pragma unroll
    for (int i = 0; i < kSkStage; ++i)
        if (srow[i] < M)
            put(srow[i], sq[i], xs[i]);
    if (ngroups > kSkStage * nthr) {
        int row = srow[kSkStage - 1], q = sq[kSkStage - 1] + nthr;
        for (;;) {
            while (q >= gpr && row < M) {
                q -= gpr;
                ++row;
            }
            if (row >= M)
                break;
            const int k = kbase + q * 8;
            put(row, q, k < K ? *reinterpret_cast<const uint4 *>(x + (int64_t)row * K + k)
                              : make_uint4(0u, 0u, 0u, 0u));
            q += nthr;
        }
    }
    if (threadIdx.x < kZeroBytes / 4)
        reinterpret_cast<uint32_t *>(zstrip)[threadIdx.x] = 0u;
    __syncthreads();

    // 4. stream this wave's units
    const int xr = ROWS * (r >> 2) + (r & 3);                  // activation row of A row r
    const bool xlive = (r & 3) < ROWS && xr < M;
    const uint8_t *xls = xlive ? xl + (xr * KT * 4 + gq) * 64 : zstrip;
    const int xstep = xlive ? 256 : 0;
    const float g = a.g;
    const int N = a.N;
    const int tfirst = n > 0 ? u0 / KT : 0;
    const int cfirst = n > 0 ? u0 - tfirst * KT : 0;
    int t = tfirst, c = cfirst;

    float *y = static_cast<float *>(out);
    uint16_t *hout = static_cast<uint16_t *>(out);
    const int F = N >> 1;

    // This range's complete value v of output (m, col) (col < N): joined with
    // the other ranges' values along the tree -- at each level the side that
    // finds its partner's value adds the two, clears the word and goes on --
    // and stored by the last join (at once when there is one range).
    unsigned long long bestk[4] = {0ull, 0ull, 0ull, 0ull};   // ARGMAX: per row slot j
    auto join = [&](int m, int col, float v, int j) {
        for (int span = 1; span < (KR ? a.KS : 1); span *= 2) {
            const int set = (a.KS - a.KS / span) + kr / (2 * span);
            unsigned long long *wd = xch + kSkBoundaryWords + ((int64_t)set * M + m) * N + col;
            const unsigned long long mine =
                (1ull << 32) | (unsigned long long)__builtin_bit_cast(uint32_t, v);
            const unsigned long long old =
                __hip_atomic_exchange(wd, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (!(old >> 32))
                return;                                 // the partner side goes on
            v = __builtin_bit_cast(float, (uint32_t)old) + v;
            __hip_atomic_store(wd, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        const float gv = g * v;
        if (!ARGMAX || y != nullptr)
            y[(int64_t)m * N + col] = gv;
        if (ARGMAX) {
            const unsigned long long k = argmax_key(gv, col);
            bestk[j] = k > bestk[j] ? k : bestk[j];
        }
    };
    // Two rows m, m + 1 of output column col held by one lane (ROWS >= 2):
    // the same tree with both values in one word (pair_word, never zero), so
    // each join level costs one exchange per two outputs.  The word of row
    // m is used; row m + 1's stays zero.  Row m + 1 may lie past M (its value
    // is then never stored).
    auto join2 = [&](int m, int col, float v0, float v1, int j) {
        for (int span = 1; span < (KR ? a.KS : 1); span *= 2) {
            const int set = (a.KS - a.KS / span) + kr / (2 * span);
            unsigned long long *wd = xch + kSkBoundaryWords + ((int64_t)set * M + m) * N + col;
            const unsigned long long old = __hip_atomic_exchange(
                wd, pair_word(v0, v1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (old == 0ull)
                return;                                 // the partner side goes on
            v0 = pair_gate(old) + v0;
            v1 = pair_up(old) + v1;
            __hip_atomic_store(wd, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        const float g0 = g * v0, g1 = g * v1;
        if (!ARGMAX || y != nullptr) {
            y[(int64_t)m * N + col] = g0;
            if (m + 1 < M)
                y[(int64_t)(m + 1) * N + col] = g1;
        }
        if (ARGMAX) {
            const unsigned long long k0 = argmax_key(g0, col);
            bestk[j] = k0 > bestk[j] ? k0 : bestk[j];
            if (m + 1 < M) {
                const unsigned long long k1 = argmax_key(g1, col);
                bestk[j + 1] = k1 > bestk[j + 1] ? k1 : bestk[j + 1];
            }
        }
    };
    // SILU: the same for this range's complete gate and up values of output
    // (m, f), one word per pair; the last join applies the epilogue
    auto join_pair = [&](int m, int f, float vg, float vu) {
        for (int span = 1; span < (KR ? a.KS : 1); span *= 2) {
            const int set = (a.KS - a.KS / span) + kr / (2 * span);
            unsigned long long *wd = xch + kSkBoundaryWords + ((int64_t)set * M + m) * F + f;
            const unsigned long long old = __hip_atomic_exchange(
                wd, pair_word(vg, vu), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (old == 0ull)
                return;
            vg = pair_gate(old) + vg;
            vu = pair_up(old) + vu;
            __hip_atomic_store(wd, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        hout[(int64_t)m * F + f] = silu_mul_bf16(g * vg, g * vu);
    };
    // Row tile tt complete in this range: lane (r, gq) holds rows 4gq + j of
    // output column 16tt + r.  Called with the whole wave active (the row
    // rotate reads every lane).
    auto store_y = [&](int tt, const floatx4_t &v) {
        if (SILU) {
            const int f = 8 * tt + r;
#pragma unroll
            for (int j = 0; j < ROWS; ++j) {
                const int m = out_row(gq, j);
                // copy the element out first: clang mis-lowers a bit_cast whose
                // operand is a vector element (it reads element 0)
                const float vg = v[j];
                const float vu = swap8(vg);
                if (r < 8 && m < M)
                    join_pair(m, f, vg, vu);
            }
            return;
        }
        const int col = 16 * tt + r;
        if (col < N) {
#pragma unroll
            for (int j = 0; j < ROWS; j += 2) {
                const int m = out_row(gq, j);
                const float vj = v[j];
                if (j + 1 < ROWS) {
                    const float vk = v[j + 1];
                    if (m < M)
                        join2(m, col, vj, vk, j);
                } else if (m < M) {
                    join(m, col, vj, j);
                }
            }
        }
    };

    floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
    auto tile_x = [&](int s, const uint8_t *xp) {
        const uint4 *src = reinterpret_cast<const uint4 *>(xp);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            uint2 xf[4];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const uint4 v = src[2 * h + j];
                xf[2 * j] = make_uint2(v.x, v.y);
                xf[2 * j + 1] = make_uint2(v.z, v.w);
            }
            auto xa = [&](int bb) { return xf[bb & 3]; };
            if (h == 0)
                gemv_half<ROWS, 0>(cw[s], sw[s], xa, acc);
            else
                gemv_half<ROWS, 1>(cw[s], sw[s], xa, acc);
        }
        asm volatile("" : "+v"(acc));
        __builtin_amdgcn_sched_barrier(0);
    };

    if (KR) {
        for (int i = 0; i < n; i += PF) {
#pragma unroll
            for (int s = 0; s < PF; ++s) {
                if (i + s < n) {
                    tile_x(s, xls + c * xstep);
                    ++c;
                    if (c == KT || i + s == n - 1) {
                        const int cstart = (t == tfirst) ? cfirst : 0;
                        if (cstart == 0 && c == KT)
                            store_y(t, acc);                           // whole row tile
                        else
                            part[(wave * 2 + (t == tfirst ? 0 : 1)) * 64 + lane] = acc;
                        acc = floatx4_t{0.f, 0.f, 0.f, 0.f};
                        if (c == KT) {
                            c = 0;
                            ++t;
                        }
                    }
                }
                load(s);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    } else {
        // countdown to the next row-tile boundary (or the wave's end)
        int to_flush = KT - cfirst < n ? KT - cfirst : n;
        const uint8_t *xp = xls + cfirst * xstep;
        auto unit = [&](int s, int pos) {
            tile_x(s, xp);
            xp += xstep;
            if (--to_flush == 0) {
                // row tile t done here: whole in this wave, or a part
                if ((t != tfirst || cfirst == 0) && (t + 1) * KT <= u1)
                    store_y(t, acc);
                else
                    part[(wave * 2 + (t == tfirst ? 0 : 1)) * 64 + lane] = acc;
                acc = floatx4_t{0.f, 0.f, 0.f, 0.f};
                ++t;
                to_flush = n - pos - 1 < KT ? n - pos - 1 : KT;
                xp = xls;
            }
        };
        int i = 0;
        for (; i + PF <= n; i += PF) {
#pragma unroll
            for (int s = 0; s < PF; ++s) {
                unit(s, i + s);
                load_pos(s, i + s + PF);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int s = 0; s < PF; ++s)
            if (i + s < n)
                unit(s, i + s);
    }

    // 5. finish the row tiles split between waves or workgroups
    __syncthreads();
    // the stream leaves t one past the wave's last row tile, or on it when
    // (K ranges) that tile's last unit was not this wave's
    const int tlast = n == 0 ? 0 : KR && c != 0 ? t : t - 1;
    for (int side = 0; side < (n > 0 ? 2 : 0); ++side) {
        const int tau = side == 0 ? tfirst : tlast;
        if (side == 1 && tlast == tfirst)
            break;
        const int ta = tau * KT, tb = ta + KT;
        const int a0 = ta > UW0 ? ta : UW0, a1 = tb < UW1 ? tb : UW1;
        const bool cross = ta < UW0 || tb > UW1;
        // this wave holds the tile's first units in the workgroup when the
        // tile starts inside its range, and all of them when the tile also
        // ends inside it (stored already, unless it crosses into a neighbour)
        if (a0 < u0 || (a1 <= u1 && !cross))
            continue;
        // the later waves whose ranges start inside the tile hold the rest,
        // each as the partial of its first tile; summed in wave order
        floatx4_t sum = part[(wave * 2 + side) * 64 + lane];
        for (int v = wave + 1; v < WPG && wave_start(v) < a1; ++v)
            sum += part[v * 2 * 64 + lane];
        if (!cross) {
            store_y(tau, sum);
            continue;
        }
        // boundary between groups bnd, bnd + 1 of this range
        const int bnd = kr * GR + (ta < UW0 ? L - 1 : L);
        unsigned long long *slot = xch + ((int64_t)bnd * 64 + lane) * 4;
        if (SILU) {
#pragma unroll
            for (int j = 0; j < ROWS; ++j) {
                const int m = out_row(gq, j);
                const float sg = sum[j];
                const float su = swap8(sg);
                if (r < 8 && m < M) {
                    const unsigned long long old = __hip_atomic_exchange(
                        slot + j, pair_word(sg, su), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    if (old != 0ull) {
                        __hip_atomic_store(slot + j, 0ull, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                        join_pair(m, 8 * tau + r, pair_gate(old) + sg, pair_up(old) + su);
                    }
                }
            }
            continue;
        }
        const int col = 16 * tau + r;
#pragma unroll
        for (int j = 0; j < ROWS; j += 2) {
            const int m = out_row(gq, j);
            if (m < M) {
                // copy the elements out first: clang mis-lowers a bit_cast whose
                // operand is a vector element (it reads element 0)
                const float sj = sum[j];
                if (j + 1 < ROWS) {
                    // rows m, m + 1 in one word (slot j; slot j + 1 unused)
                    const float sk = sum[j + 1];
                    const unsigned long long old = __hip_atomic_exchange(
                        slot + j, pair_word(sj, sk), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    if (old != 0ull) {
                        __hip_atomic_store(slot + j, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        if (col < N)
                            join2(m, col, pair_gate(old) + sj, pair_up(old) + sk, j);
                    }
                    continue;
                }
                const unsigned long long mine =
                    (1ull << 32) | (unsigned long long)__builtin_bit_cast(uint32_t, sj);
                const unsigned long long old = __hip_atomic_exchange(
                    slot + j, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (old >> 32) {
                    const float other = __builtin_bit_cast(float, (uint32_t)old);
                    __hip_atomic_store(slot + j, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    if (col < N)
                        join(m, col, other + sj, j);
                }
            }
        }
    }

    if (ARGMAX) {
        // part[] is free once every wave is past the finish
        unsigned long long *red = reinterpret_cast<unsigned long long *>(part);
        unsigned long long *keys = xch + kSkBoundaryWords + (int64_t)(a.KS - 1) * M * N;
        unsigned long long *counter = keys + M;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < ROWS; ++j) {
            unsigned long long k = bestk[j];
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) {
                const unsigned long long o = __shfl_xor(k, off, 64);
                k = o > k ? o : k;
            }
            if (r == 0)
                red[wave * 16 + out_row(gq, j)] = k;
        }
        __syncthreads();
        if ((int)threadIdx.x < M) {
            unsigned long long k = red[threadIdx.x];
            for (int v = 1; v < WPG; ++v) {
                const unsigned long long o = red[v * 16 + threadIdx.x];
                k = o > k ? o : k;
            }
            const unsigned long long prev = __hip_atomic_fetch_max(
                keys + threadIdx.x, k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            asm volatile("" ::"v"(prev) : "memory");       // the max has returned
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            const unsigned long long done = __hip_atomic_fetch_add(
                counter, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            red[0] = done == (unsigned long long)(G - 1) ? 1ull : 0ull;
        }
        __syncthreads();
        if (red[0] != 0ull) {
            if ((int)threadIdx.x < M) {
                const unsigned long long k = __hip_atomic_exchange(
                    keys + threadIdx.x, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                a.best_val[threadIdx.x] = argmax_key_value(k);
                a.best_idx[threadIdx.x] = (int64_t)(0xFFFFFFFFu - (uint32_t)k);
            }
            if (threadIdx.x == 0)
                __hip_atomic_store(counter, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

typedef void (*gemv_fn)(const uint4 *, const uint2 *, float, const uint16_t *, float *, int, int,
                        int, int, int, int, int);

template <bool XLDS>
gemv_fn pick_kernel_x(int64_t M)
{
    switch (M) {
    case 1: return gemv_kernel<1, XLDS>;
    case 2: return gemv_kernel<2, XLDS>;
    case 3: return gemv_kernel<3, XLDS>;
    case 4: return gemv_kernel<4, XLDS>;
    case 5: return gemv_kernel<5, XLDS>;
    case 6: return gemv_kernel<6, XLDS>;
    case 7: return gemv_kernel<7, XLDS>;
    case 8: return gemv_kernel<8, XLDS>;
    default: return gemv_kernel<0, XLDS>;
    }
}

gemv_fn pick_kernel(int64_t M, bool xlds)
{
    return xlds ? pick_kernel_x<true>(M) : pick_kernel_x<false>(M);
}

struct Plan {
    gemv_fn fn;
    int TB, S;
    size_t lds;
    int64_t blocks;
};

int device_cus()
{
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    if (cus[dev] == 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            v <= 0)
            v = 256;
        cus[dev] = v;
    }
    return cus[dev];
}

// Launch shape: among (TB, S) with TB = 1 for S > 1 (at least 2 k-tiles per
// wave), the one with the most waves whose workgroups are all resident at
// once (one round, no tail); if none fits in one round, one wave per tile
// (TB = 4 tiles per workgroup, sharing one staged copy of the activations).
Plan make_plan(int64_t M, int64_t N, int64_t K)
{
    const int64_t NT = n_tiles(N), KT = k_tiles(K);
    const int64_t xbytes = M * KT * 256;
    const bool xlds = xbytes <= kXLdsMaxBytes;
    const size_t xl = xlds ? (size_t)xbytes + kZeroBytes : 0;
    gemv_fn fn = pick_kernel(M, xlds);
    const int cus = device_cus();
    Plan best = {fn, 4, 1, xl, (NT + 3) / 4};
    int64_t best_waves = 0;
    auto consider = [&](int TB, int S) {
        const size_t lds = xl + (S > 1 ? (size_t)TB * S * 1024 : 0);
        int occ = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, reinterpret_cast<const void *>(fn),
                                                         64 * TB * S, lds) != hipSuccess)
            return;
        const int64_t blocks = (NT + TB - 1) / TB;
        if (occ <= 0 || blocks > (int64_t)cus * occ)
            return;
        const int64_t waves = blocks * TB * S;
        if (waves > best_waves) {
            best_waves = waves;
            best = {fn, TB, S, lds, blocks};
        }
    };
    for (int S = 2; S <= kMaxWaves; ++S)
        if (KT / S >= 2)
            consider(1, S);
    for (int TB : {1, 2, 4})
        consider(TB, 1);
    return best;
}

struct CachedPlan {
    int dev;
    int64_t M, N, K;
    Plan plan;
};

// Plans depend only on (device, M, N, K); a decode loop reuses a handful.
Plan cached_plan(int64_t M, int64_t N, int64_t K)
{
    static std::mutex mu;
    static std::vector<CachedPlan> cache;
    int dev = 0;
    (void)hipGetDevice(&dev);
    std::lock_guard<std::mutex> lock(mu);
    for (const CachedPlan &c : cache)
        if (c.dev == dev && c.M == M && c.N == N && c.K == K)
            return c.plan;
    const Plan p = make_plan(M, N, K);
    if (cache.size() >= 256)
        cache.clear();
    cache.push_back({dev, M, N, K, p});
    return p;
}

typedef void (*gemv_sk_fn)(const uint4 *, const uint2 *, const uint16_t *, void *,
                           unsigned long long *, SkArgs);

template <bool KR, int EPI>
gemv_sk_fn pick_sk_kernel_k(int64_t M)
{
    // ceil(M/4) live rows per lane (rows placed that many per group of four)
    return M <= 4 ? gemv_sk_kernel<1, kSkPrefetch, KR, EPI>
         : M <= 8 ? gemv_sk_kernel<2, kSkPrefetch, KR, EPI>
         : M <= 12 ? gemv_sk_kernel<3, kSkPrefetch, KR, EPI>
                   : gemv_sk_kernel<4, kSkPrefetch, KR, EPI>;
}

template <int EPI>
gemv_sk_fn pick_sk_kernel_e(int64_t M, bool ranges, bool short_waves)
{
    if (!ranges && M <= 4 && short_waves)
        return gemv_sk_kernel<1, kSkPrefetchShort, false, EPI>;
    return ranges ? pick_sk_kernel_k<true, EPI>(M) : pick_sk_kernel_k<false, EPI>(M);
}

// short_waves: every wave streams at most kSkShortUnits units
gemv_sk_fn pick_sk_kernel(int64_t M, bool ranges, int epi, bool short_waves)
{
    switch (epi) {
    case kEpiSilu: return pick_sk_kernel_e<kEpiSilu>(M, ranges, short_waves);
    case kEpiArgmax: return pick_sk_kernel_e<kEpiArgmax>(M, ranges, short_waves);
    default: return pick_sk_kernel_e<kEpiY>(M, ranges, short_waves);
    }
}

// Exchange words one join level touches per output column: a lane holds
// rows ROWS*gq + j (j < ROWS) of a column and joins them two to a word when
// ROWS >= 2 (one per row when ROWS = 1); the fused gate/up epilogue joins
// (gate, up) pairs, one word per output f.
int64_t sk_join_words_per_col(int64_t M, bool silu)
{
    if (silu)
        return M;
    const int64_t rows = (M + 3) / 4;                   // ROWS
    int64_t w = 0;
    for (int64_t gq = 0; gq < 4; ++gq)
        for (int64_t j = 0; j < rows; j += rows >= 2 ? 2 : 1)
            w += rows * gq + j < M ? 1 : 0;
    return w;
}

// K ranges for the stream-K kernel (a power of two, 0 when none fits).  One
// range stages the activations of all of K in every workgroup; more ranges
// stage less each but join their partial sums through the workspace.  The
// count with the least estimated cost is used, from timings of the verify
// shapes on MI355X: staging about 22 ns per KB per workgroup, joining about
// 14 ns per 1000 exchange words, and about 0.6 us per level of the join
// tree.  Columns: N outputs (F for the fused gate/up epilogue).
constexpr double kSkStageUsPerKB = 0.0224;
constexpr double kSkJoinUsPerKWord = 0.0137;
constexpr double kSkLevelUs = 0.6;

int64_t sk_ranges(int64_t M, int64_t N, int64_t K, bool silu)
{
    const int64_t KT = k_tiles(K);
    const int64_t cols = silu ? N / 2 : N;
    const int64_t wpc = sk_join_words_per_col(M, silu);
    int64_t best = 0;
    double best_cost = 0.0;
    int level = 0;
    for (int64_t KS = 1; KS <= kSkMaxRanges; KS *= 2, ++level) {
        const int64_t KTR = (KT + KS - 1) / KS;
        if (KT - (KS - 1) * KTR < 1)
            break;                                      // a range without k-tiles
        const int64_t xbytes = M * KTR * 256;
        if (xbytes > kSkXMaxBytes)
            continue;
        const double cost = kSkStageUsPerKB * (double)xbytes / 1024.0 +
                            kSkJoinUsPerKWord * (double)((KS - 1) * wpc * cols) / 1000.0 +
                            kSkLevelUs * level;
        if (best == 0 || cost < best_cost) {
            best = KS;
            best_cost = cost;
        }
    }
    return best;
}

// The stream-K kernel serves a shape when some K range count fits its
// activations in LDS, and the packed codes stay below 4 GiB (32-bit buffer
// offsets: fewer than 2^22 units of 1 KB).
bool sk_usable(int64_t M, int64_t N, int64_t K, bool silu)
{
    return sk_ranges(M, N, K, silu) > 0 && n_tiles(N) * k_tiles(K) < ((int64_t)1 << 22);
}

struct SkPlan {
    gemv_sk_fn fn;
    SkArgs args;
    size_t lds;
};

// One workgroup per CU (at most kSkMaxGroups), but no more workgroups than
// row tiles, so that every workgroup's range covers at least KT units and a
// row tile is shared by at most two workgroups.
SkPlan make_sk_plan(int64_t M, int64_t N, int64_t K, int epi)
{
    const int64_t KT = k_tiles(K), NT = n_tiles(N);
    const int64_t KS = sk_ranges(M, N, K, epi == kEpiSilu);
    const int64_t KTR = (KT + KS - 1) / KS;
    int64_t GR = device_cus() / KS;                     // workgroups per K range
    if (GR > kSkMaxGroups / KS)
        GR = kSkMaxGroups / KS;
    if (GR > NT)
        GR = NT;
    if (GR < 1)
        GR = 1;
    const int64_t ULAST = NT * (KT - (KS - 1) * KTR);   // units of the shortest range
    int64_t WPG = kSkMaxWaves;
    if (WPG > ULAST / GR)
        WPG = ULAST / GR;
    SkPlan p;
    // units of the busiest wave: ceil(ceil(units of the range / GR) / WPG)
    const int64_t UR = NT * KTR;
    const int64_t wave_units = ((UR + GR - 1) / GR + WPG - 1) / WPG;
    p.fn = pick_sk_kernel(M, KS > 1, epi, wave_units <= kSkShortUnits);
    p.args = SkArgs{(int)M, (int)N, (int)K, (int)KT, (int)NT, (int)(GR * KS), (int)WPG, (int)KS,
                    (int)KTR, 0.f, nullptr, nullptr};
    p.args.GR = (int)GR;
    for (int kind = 0; kind < 2; ++kind) {
        // sk_ranges leaves no range without k-tiles: the last has 1..KTR
        const int64_t KTx = kind == 0 ? KTR : KT - (KS - 1) * KTR;
        const int64_t U = NT * KTx, ub = U / GR;
        int *sp = p.args.split[kind];
        sp[0] = (int)ub;
        sp[1] = (int)(U % GR);
        sp[2] = (int)(ub / WPG);
        sp[3] = (int)(ub % WPG);
        sp[4] = (int)((ub + 1) / WPG);
        sp[5] = (int)((ub + 1) % WPG);
        // exact for every staging group index i: umulhi(i, ceil(2^32 / d))
        // is i / d while i * d < 2^32, and i < 16 slots * 512 threads while
        // d = 16 * KTx is bounded by the range's activations fitting in LDS
        static_assert((uint64_t)16 * 64 * kSkMaxWaves * 16 * (kSkXMaxBytes / 256) < (uint64_t(1) << 32),
                      "staging reciprocal out of its exact range");
        const uint64_t gpr = 16 * (uint64_t)KTx;
        p.args.xrcp[kind] = (uint32_t)(((uint64_t(1) << 32) + gpr - 1) / gpr);
    }
    size_t lds = (size_t)(M * KTR * 256) + kZeroBytes + (size_t)WPG * 2 * 64 * sizeof(floatx4_t);
    if (lds < (size_t)kSkLdsFloor)
        lds = kSkLdsFloor;
    p.lds = lds;
    return p;
}

struct CachedSkPlan {
    int dev;
    int64_t M, N, K;
    int epi;
    SkPlan plan;
};

SkPlan cached_sk_plan(int64_t M, int64_t N, int64_t K, int epi)
{
    static std::mutex mu;
    static std::vector<CachedSkPlan> cache;
    int dev = 0;
    (void)hipGetDevice(&dev);
    std::lock_guard<std::mutex> lock(mu);
    for (const CachedSkPlan &c : cache)
        if (c.dev == dev && c.M == M && c.N == N && c.K == K && c.epi == epi)
            return c.plan;
    const SkPlan p = make_sk_plan(M, N, K, epi);
    if (cache.size() >= 256)
        cache.clear();
    cache.push_back({dev, M, N, K, epi, p});
    return p;
}

}  // namespace

size_t gemv_workspace_bytes(int64_t M, int64_t N, int64_t K)
{
    if (M < 1 || M > 16 || N < 1 || K < 1)
        return 0;
    const int64_t KS = sk_usable(M, N, K, false) ? sk_ranges(M, N, K, false) : 1;
    return (size_t)(kSkBoundaryWords + (KS - 1) * M * N) * sizeof(unsigned long long);
}

bool gemv_silu_mul_supported(int64_t M, int64_t F, int64_t K)
{
    return M >= 1 && M <= 16 && F >= 8 && F % 8 == 0 && K >= 1 && sk_usable(M, 2 * F, K, true);
}

size_t gemv_silu_mul_workspace_bytes(int64_t M, int64_t F, int64_t K)
{
    if (!gemv_silu_mul_supported(M, F, K))
        return 0;
    const int64_t KS = sk_ranges(M, 2 * F, K, true);
    return (size_t)(kSkBoundaryWords + (KS - 1) * M * F) * sizeof(unsigned long long);
}

hipError_t launch_gemv(const uint8_t *packed_codes, const uint8_t *packed_scales, float g,
                       const uint16_t *x, float *y, int64_t M, int64_t N, int64_t K,
                       void *workspace, hipStream_t stream)
{
    const int64_t KT = k_tiles(K), NT = n_tiles(N);
    if (sk_usable(M, N, K, false)) {
        const SkPlan p = cached_sk_plan(M, N, K, kEpiY);
        SkArgs args = p.args;
        args.g = g;
        hipLaunchKernelGGL(p.fn, dim3((unsigned)args.G), dim3(64 * args.WPG), p.lds, stream,
                           reinterpret_cast<const uint4 *>(packed_codes),
                           reinterpret_cast<const uint2 *>(packed_scales), x, y,
                           static_cast<unsigned long long *>(workspace), args);
        return hipGetLastError();
    }
    const Plan p = cached_plan(M, N, K);
    hipLaunchKernelGGL(p.fn, dim3((unsigned)p.blocks), dim3(64 * p.TB * p.S), p.lds, stream,
                       reinterpret_cast<const uint4 *>(packed_codes),
                       reinterpret_cast<const uint2 *>(packed_scales), g, x, y, (int)M, (int)N,
                       (int)K, (int)KT, (int)NT, p.TB, p.S);
    return hipGetLastError();
}

hipError_t launch_gemv_silu_mul(const uint8_t *packed_codes, const uint8_t *packed_scales,
                                float g, const uint16_t *x, uint16_t *h, int64_t M, int64_t F,
                                int64_t K, void *workspace, hipStream_t stream)
{
    if (!gemv_silu_mul_supported(M, F, K))
        return hipErrorInvalidValue;
    const SkPlan p = cached_sk_plan(M, 2 * F, K, kEpiSilu);
    SkArgs args = p.args;
    args.g = g;
    hipLaunchKernelGGL(p.fn, dim3((unsigned)args.G), dim3(64 * args.WPG), p.lds, stream,
                       reinterpret_cast<const uint4 *>(packed_codes),
                       reinterpret_cast<const uint2 *>(packed_scales), x, h,
                       static_cast<unsigned long long *>(workspace), args);
    return hipGetLastError();
}

bool gemv_argmax_supported(int64_t M, int64_t N, int64_t K)
{
    return M >= 1 && M <= 16 && N >= 1 && K >= 1 && sk_usable(M, N, K, false);
}

size_t gemv_argmax_workspace_bytes(int64_t M, int64_t N, int64_t K)
{
    if (!gemv_argmax_supported(M, N, K))
        return 0;
    // the GEMV's exchange words, then one key per row and the counter
    return gemv_workspace_bytes(M, N, K) + (size_t)(M + 1) * sizeof(unsigned long long);
}

hipError_t launch_gemv_argmax(const uint8_t *packed_codes, const uint8_t *packed_scales, float g,
                              const uint16_t *x, float *y, float *best_val, int64_t *best_idx,
                              int64_t M, int64_t N, int64_t K, void *workspace,
                              hipStream_t stream)
{
    if (!gemv_argmax_supported(M, N, K))
        return hipErrorInvalidValue;
    const SkPlan p = cached_sk_plan(M, N, K, kEpiArgmax);
    SkArgs args = p.args;
    args.g = g;
    args.best_val = best_val;
    args.best_idx = best_idx;
    hipLaunchKernelGGL(p.fn, dim3((unsigned)args.G), dim3(64 * args.WPG), p.lds, stream,
                       reinterpret_cast<const uint4 *>(packed_codes),
                       reinterpret_cast<const uint2 *>(packed_scales), x, y,
                       static_cast<unsigned long long *>(workspace), args);
    return hipGetLastError();
}

namespace {

__global__ void __launch_bounds__(256) scratch_clear_kernel(unsigned long long *p, size_t words)
{
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < words; i += (size_t)gridDim.x * 256)
        p[i] = 0ull;
}

// Per-device address of the scratch array (the runtime's address for the
// device that is current), looked up once per device; the array is cleared
// on the first call on each device, on that call's stream.
struct ScratchSlot {
    unsigned long long *ptr;
    bool cleared;
};

}  // namespace

size_t gemv_noalloc_max_bytes() { return kScratchBytes; }

hipError_t launch_gemv_noalloc(const uint8_t *packed_codes, const uint8_t *packed_scales,
                               float g, const uint16_t *x, float *y, int64_t M, int64_t N,
                               int64_t K, hipStream_t stream)
{
    static std::mutex mu;
    static ScratchSlot slots[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= 64)
        return hipErrorInvalidDevice;
    unsigned long long *ptr = nullptr;
    {
        std::lock_guard<std::mutex> lock(mu);
        ScratchSlot &sl = slots[dev];
        if (sl.ptr == nullptr) {
            void *p = nullptr;
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess)
                return e;
            sl.ptr = static_cast<unsigned long long *>(p);
        }
        if (!sl.cleared) {
            hipLaunchKernelGGL(scratch_clear_kernel, dim3(256), dim3(256), 0, stream, sl.ptr,
                               kScratchBytes / 8);
            e = hipGetLastError();
            if (e != hipSuccess)
                return e;
            sl.cleared = true;
        }
        ptr = sl.ptr;
    }
    return launch_gemv(packed_codes, packed_scales, g, x, y, M, N, K, ptr, stream);
}

}  // namespace q4p
