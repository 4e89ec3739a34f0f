/* Drives the library's host front (q4p_api.cpp, the argument validation and
 * dispatch of include/q4proj.h) in a CPU build under AddressSanitizer and
 * UndefinedBehaviorSanitizer, with the HIP runtime and the kernel launchers
 * replaced by recording stand-ins (stubs.cpp).  Every rejected call must
 * return its status without reaching a launcher; every accepted call must
 * reach the right launcher with its arguments unchanged.  Buffers are
 * addresses only: the front never dereferences them, and the stand-ins do
 * not either.  Exit status 0 when every check holds.  Test infrastructure
 * only. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "q4proj.h"
#include "stub_control.h"

static int g_checks, g_failed;

#define CHECK(cond, ...)                                                  \
    do {                                                                  \
        ++g_checks;                                                       \
        if (!(cond)) {                                                    \
            ++g_failed;                                                   \
            fprintf(stderr, "hostcheck: line %d: ", __LINE__);            \
            fprintf(stderr, __VA_ARGS__);                                 \
            fputc('\n', stderr);                                          \
        }                                                                 \
    } while (0)

/* disjoint 64 GiB regions of the address space, never dereferenced */
#define REGION(i) ((uintptr_t)0x100000000000ull + ((uintptr_t)(i) << 36))
#define U8(i, off) ((uint8_t *)(REGION(i) + (off)))
#define U16(i, off) ((uint16_t *)(REGION(i) + (off)))
#define F32(i, off) ((float *)(REGION(i) + (off)))
#define I64(i, off) ((int64_t *)(REGION(i) + (off)))
#define VP(i, off) ((void *)(REGION(i) + (off)))

enum { PC = 0, PS = 1, X = 2, Y = 3, WS = 4, C = 5, S = 6, C2 = 7, S2 = 8, V = 9, IDX = 10 };

static void *const STREAM = (void *)(uintptr_t)0x5150;

/* a rejected call: status `want`, no launch */
#define REJECT(call, want, what)                                                   \
    do {                                                                           \
        const int before = stub_last()->count;                                     \
        const q4proj_status got = (call);                                          \
        CHECK(got == (want), "%s: status %d, want %d", what, (int)got, (int)(want)); \
        CHECK(stub_last()->count == before, "%s: reached a launcher", what);       \
    } while (0)

/* an accepted call: Q4P_OK and one launch of `name` */
#define ACCEPT(call, name_, what)                                                  \
    do {                                                                           \
        const int before = stub_last()->count;                                     \
        const q4proj_status got = (call);                                          \
        CHECK(got == Q4P_OK, "%s: status %d, want Q4P_OK", what, (int)got);        \
        CHECK(stub_last()->count == before + 1, "%s: %d launches", what,           \
              stub_last()->count - before);                                        \
        CHECK(strcmp(stub_last()->name, name_) == 0, "%s: launched %s", what,      \
              stub_last()->name);                                                  \
        CHECK(stub_last()->stream == STREAM, "%s: stream not passed through", what); \
    } while (0)

static void gemv_checks(void)
{
    const int64_t M = 1, N = 17408, K = 5120;
    const float g = 0.75f;
    /* first call on device 0 reads its properties once; later calls hit the cache */
    ACCEPT(q4proj_gemv(U8(PC, 0), U8(PS, 0), g, U16(X, 0), F32(Y, 0), M, N, K, VP(WS, 0), 4096,
                       STREAM),
           "gemv", "gemv valid");
    const stub_launch *l = stub_last();
    CHECK(l->M == M && l->N == N && l->K == K && l->g == g && l->workspace == VP(WS, 0) &&
              l->in0 == U8(PC, 0) && l->in1 == U8(PS, 0) && l->out == F32(Y, 0),
          "gemv: arguments changed on the way to the launcher");
    CHECK(stub_props_calls() == 1, "device properties read %d times", stub_props_calls());
    ACCEPT(q4proj_gemv(U8(PC, 0), U8(PS, 0), g, U16(X, 0), F32(Y, 0), 16, N, K, VP(WS, 0), 4096,
                       STREAM),
           "gemv", "gemv M=16");
    CHECK(stub_props_calls() == 1, "device check not cached (%d reads)", stub_props_calls());

    REJECT(q4proj_gemv(NULL, U8(PS, 0), g, U16(X, 0), F32(Y, 0), M, N, K, VP(WS, 0), 4096, STREAM),
           Q4P_EINVAL, "gemv null codes");
    REJECT(q4proj_gemv(U8(PC, 0), U8(PS, 0), g, NULL, F32(Y, 0), M, N, K, VP(WS, 0), 4096, STREAM),
           Q4P_EINVAL, "gemv null x");
    REJECT(q4proj_gemv(U8(PC, 8), U8(PS, 0), g, U16(X, 0), F32(Y, 0), M, N, K, VP(WS, 0), 4096,
                       STREAM),
           Q4P_EINVAL, "gemv codes misaligned");
    REJECT(q4proj_gemv(U8(PC, 0), U8(PS, 4), g, U16(X, 0), F32(Y, 0), M, N, K, VP(WS, 0), 4096,
                       STREAM),
           Q4P_EINVAL, "gemv scales misaligned");
    REJECT(q4proj_gemv(U8(PC, 0), U8(PS, 0), g, U16(X, 8), F32(Y, 0), M, N, K, VP(WS, 0), 4096,
                       STREAM),
           Q4P_EINVAL, "gemv x misaligned");
    REJECT(q4proj_gemv(U8(PC, 0), U8(PS, 0), g, U16(X, 0), F32(Y, 2), M, N, K, VP(WS, 0), 4096,
                       STREAM),
           Q4P_EINVAL, "gemv y misaligned");
    const int64_t bad[][3] = {{1, N, 5121}, {1, N, 0}, {1, 0, K}, {0, N, K}, {-1, N, K},
                              {1, ((int64_t)1 << 30) + 1, K}, {1, N, ((int64_t)1 << 24) + 16},
                              {INT64_MAX, N, K}, {1, INT64_MAX, K}, {1, N, INT64_MIN},
                              {INT64_MIN, INT64_MIN, INT64_MIN}, {1, -16, K}, {1, N, -16}};
    for (size_t i = 0; i < sizeof bad / sizeof bad[0]; ++i)
        REJECT(q4proj_gemv(U8(PC, 0), U8(PS, 0), g, U16(X, 0), F32(Y, 0), bad[i][0], bad[i][1],
                           bad[i][2], VP(WS, 0), 4096, STREAM),
               Q4P_EINVAL, "gemv bad size");
    REJECT(q4proj_gemv(U8(PC, 0), U8(PS, 0), g, U16(X, 0), F32(Y, 0), 17, N, K, VP(WS, 0), 4096,
                       STREAM),
           Q4P_EUNSUPPORTED, "gemv M=17");
    REJECT(q4proj_gemv(U8(PC, 0), U8(PS, 0), g, U16(X, 0), F32(Y, 0), M, N, K, VP(WS, 0), 4095,
                       STREAM),
           Q4P_EWORKSPACE, "gemv workspace short");
    REJECT(q4proj_gemv(U8(PC, 0), U8(PS, 0), g, U16(X, 0), F32(Y, 0), M, N, K, NULL, 4096, STREAM),
           Q4P_EINVAL, "gemv null workspace");
    REJECT(q4proj_gemv(U8(PC, 0), U8(PS, 0), g, U16(X, 0), F32(Y, 0), M, N, K, VP(WS, 4), 4096,
                       STREAM),
           Q4P_EINVAL, "gemv workspace misaligned");
    REJECT(q4proj_gemv(U8(PC, 0), U8(PS, 0), g, U16(X, 0), F32(Y, 0), M, N, K,
                       VP(Y, 64), 4096, STREAM),
           Q4P_EINVAL, "gemv workspace overlaps y");
    REJECT(q4proj_gemv(U8(PC, 0), U8(PS, 0), g, U16(X, 0), F32(X, 16), M, N, K, VP(WS, 0), 4096,
                       STREAM),
           Q4P_EINVAL, "gemv y overlaps x");
    REJECT(q4proj_gemv(U8(PC, 0), U8(PS, 0), g, U16(X, 0), (float *)U8(PC, 1024), M, N, K,
                       VP(WS, 0), 4096, STREAM),
           Q4P_EINVAL, "gemv y overlaps codes");
    /* y just past the end of x: no overlap */
    ACCEPT(q4proj_gemv(U8(PC, 0), U8(PS, 0), g, U16(X, 0), F32(X, (uint64_t)M * K * 2), M, N, K,
                       VP(WS, 0), 4096, STREAM),
           "gemv", "gemv y adjacent to x");

    /* launch errors become Q4P_EHIP with the runtime's message */
    stub_set_launch_error(719);
    const q4proj_status st = q4proj_gemv(U8(PC, 0), U8(PS, 0), g, U16(X, 0), F32(Y, 0), M, N, K,
                                         VP(WS, 0), 4096, STREAM);
    CHECK(st == Q4P_EHIP, "launch error: status %d", (int)st);
    CHECK(strcmp(q4proj_last_hip_error(), "hipErrorLaunchFailure") == 0, "last error '%s'",
          q4proj_last_hip_error());
    stub_set_launch_error(0);

    /* noalloc: the scratch array's size bounds the workspace */
    ACCEPT(q4proj_gemv_noalloc(U8(PC, 0), U8(PS, 0), g, U16(X, 0), F32(Y, 0), M, N, K, STREAM),
           "gemv_noalloc", "noalloc valid");
    stub_set_sizes(4096, 8192, 12288, 256, 4095, 1, 1);
    REJECT(q4proj_gemv_noalloc(U8(PC, 0), U8(PS, 0), g, U16(X, 0), F32(Y, 0), M, N, K, STREAM),
           Q4P_EWORKSPACE, "noalloc beyond the scratch array");
    stub_set_sizes(4096, 8192, 12288, 256, 1 << 20, 1, 1);
    REJECT(q4proj_gemv_noalloc(U8(PC, 0), U8(PS, 0), g, U16(X, 0), F32(Y, 0), 17, N, K, STREAM),
           Q4P_EUNSUPPORTED, "noalloc M=17");
    REJECT(q4proj_gemv_noalloc(U8(PC, 0), U8(PS, 0), g, U16(X, 0), NULL, M, N, K, STREAM),
           Q4P_EINVAL, "noalloc null y");
}

static void device_checks(void)
{
    const int64_t M = 1, N = 4096, K = 2560;
    stub_set_device(1, 0);
    stub_set_arch(1, "gfx942");
    REJECT(q4proj_gemv(U8(PC, 0), U8(PS, 0), 1.f, U16(X, 0), F32(Y, 0), M, N, K, VP(WS, 0), 4096,
                       STREAM),
           Q4P_EDEVICE, "gfx942 device");
    REJECT(q4proj_gemm(U8(PC, 0), U8(PS, 0), 1.f, U16(X, 0), F32(Y, 0), M, N, K, NULL, 0, STREAM),
           Q4P_EDEVICE, "gemm on gfx942");
    stub_set_device(2, 0);
    stub_set_arch(2, "gfx950:sramecc+:xnack-");
    ACCEPT(q4proj_gemm(U8(PC, 0), U8(PS, 0), 1.f, U16(X, 0), F32(Y, 0), M, N, K, NULL, 0, STREAM),
           "gemm", "gemm on a second gfx950");
    stub_set_device(0, 100);
    REJECT(q4proj_gemm(U8(PC, 0), U8(PS, 0), 1.f, U16(X, 0), F32(Y, 0), M, N, K, NULL, 0, STREAM),
           Q4P_EDEVICE, "no device");
    stub_set_device(70, 0);                      /* past the cache: checked every call */
    REJECT(q4proj_gemm(U8(PC, 0), U8(PS, 0), 1.f, U16(X, 0), F32(Y, 0), M, N, K, NULL, 0, STREAM),
           Q4P_EDEVICE, "device ordinal 70");
    stub_set_device(0, 0);
}

static void gemm_checks(void)
{
    const int64_t N = 14336, K = 5120;
    ACCEPT(q4proj_gemm(U8(PC, 0), U8(PS, 0), 2.f, U16(X, 0), F32(Y, 0), 512, N, K, NULL, 0, STREAM),
           "gemm", "gemm M=512");
    CHECK(stub_last()->M == 512 && stub_last()->N == N && stub_last()->K == K, "gemm sizes");
    REJECT(q4proj_gemm(U8(PC, 0), U8(PS, 0), 2.f, U16(X, 0), F32(Y, 0), ((int64_t)1 << 24) + 1, N,
                       K, NULL, 0, STREAM),
           Q4P_EINVAL, "gemm M past 2^24");
    REJECT(q4proj_gemm(U8(PC, 0), U8(PS, 0), 2.f, U16(X, 0), F32(Y, 0), (int64_t)1 << 24,
                       (int64_t)1 << 17, 16, NULL, 0, STREAM),
           Q4P_EINVAL, "gemm M*N past 2^40");
    REJECT(q4proj_gemm(U8(PC, 0), U8(PS, 0), 2.f, U16(X, 0), F32(X, 64), 512, N, K, NULL, 0,
                       STREAM),
           Q4P_EINVAL, "gemm y overlaps x");
    CHECK(stub_last()->workspace == NULL, "gemm without a workspace: NULL passed on");

    /* the optional fp16-staging workspace: 2MK and 4M bytes, each rounded up to 256 */
    const size_t need = q4proj_gemm_workspace_bytes(512, N, K);
    CHECK(need == 5242880u + 2048u, "gemm workspace size %zu", need);
    CHECK(q4proj_gemm_workspace_bytes(3, N, 16) == 256u + 256u, "gemm workspace rounding");
    CHECK(q4proj_gemm_workspace_bytes(0, N, K) == 0 && q4proj_gemm_workspace_bytes(1, N, 1041) == 0 &&
              q4proj_gemm_workspace_bytes(((int64_t)1 << 24) + 1, N, K) == 0 &&
              q4proj_gemm_workspace_bytes(1, 0, K) == 0,
          "gemm workspace size of invalid arguments");
    ACCEPT(q4proj_gemm(U8(PC, 0), U8(PS, 0), 2.f, U16(X, 0), F32(Y, 0), 512, N, K, VP(WS, 0), need,
                       STREAM),
           "gemm", "gemm with a workspace");
    CHECK(stub_last()->workspace == VP(WS, 0), "gemm workspace not passed on");
    ACCEPT(q4proj_gemm(U8(PC, 0), U8(PS, 0), 2.f, U16(X, 0), F32(Y, 0), 512, N, K, NULL, 12345,
                       STREAM),
           "gemm", "gemm: workspace_bytes ignored without a workspace");
    REJECT(q4proj_gemm(U8(PC, 0), U8(PS, 0), 2.f, U16(X, 0), F32(Y, 0), 512, N, K, VP(WS, 0),
                       need - 1, STREAM),
           Q4P_EWORKSPACE, "gemm workspace one byte short");
    REJECT(q4proj_gemm(U8(PC, 0), U8(PS, 0), 2.f, U16(X, 0), F32(Y, 0), 512, N, K, VP(WS, 8), need,
                       STREAM),
           Q4P_EINVAL, "gemm workspace misaligned");
    REJECT(q4proj_gemm(U8(PC, 0), U8(PS, 0), 2.f, U16(X, 0), F32(Y, 0), 512, N, K, VP(X, 4096),
                       need, STREAM),
           Q4P_EINVAL, "gemm workspace overlaps x");
    REJECT(q4proj_gemm(U8(PC, 0), U8(PS, 0), 2.f, U16(X, 0), F32(Y, 0), 512, N, K, VP(Y, 0), need,
                       STREAM),
           Q4P_EINVAL, "gemm workspace overlaps y");
    REJECT(q4proj_gemm(U8(PC, 0), U8(PS, 0), 2.f, U16(X, 0), F32(Y, 0), 512, N, K, VP(PC, 1024),
                       need, STREAM),
           Q4P_EINVAL, "gemm workspace overlaps the packed codes");
    REJECT(q4proj_gemm(U8(PC, 0), U8(PS, 0), 2.f, U16(X, 0), F32(Y, 0), 512, N, K, VP(PS, 0), need,
                       STREAM),
           Q4P_EINVAL, "gemm workspace overlaps the packed scales");
}

static void pack_checks(void)
{
    const int64_t N = 300, K = 1040;
    ACCEPT(q4proj_pack(U8(C, 0), U8(S, 0), N, K, U8(PC, 0), U8(PS, 0), STREAM), "pack", "pack");
    REJECT(q4proj_pack(U8(C, 4), U8(S, 0), N, K, U8(PC, 0), U8(PS, 0), STREAM), Q4P_EINVAL,
           "pack codes misaligned");
    REJECT(q4proj_pack(U8(C, 0), U8(S, 0), N, 1041, U8(PC, 0), U8(PS, 0), STREAM), Q4P_EINVAL,
           "pack K % 16");
    REJECT(q4proj_pack(U8(C, 0), U8(S, 0), N, K, U8(C, 4096), U8(PS, 0), STREAM), Q4P_EINVAL,
           "pack output overlaps codes");
    REJECT(q4proj_pack(U8(C, 0), U8(S, 0), N, K, U8(PC, 0), U8(PC, 1024), STREAM), Q4P_EINVAL,
           "pack outputs overlap");
    ACCEPT(q4proj_unpack(U8(PC, 0), U8(PS, 0), N, K, U8(C, 0), U8(S, 0), STREAM), "unpack",
           "unpack");
    REJECT(q4proj_unpack(U8(PC, 0), U8(PS, 0), N, K, U8(C, 0), U8(C, 64), STREAM), Q4P_EINVAL,
           "unpack codes overlap scales");

    const int64_t F = 8704;
    ACCEPT(q4proj_pack_gate_up(U8(C, 0), U8(S, 0), U8(C2, 0), U8(S2, 0), 0.5f, 0.5f, F, 5120,
                               U8(PC, 0), U8(PS, 0), STREAM),
           "pack_gate_up", "pack_gate_up");
    CHECK(stub_last()->N == F, "pack_gate_up F");
    const int64_t badF[] = {0, 4, 12, -8, INT64_MIN, (int64_t)1 << 62, INT64_MAX - 7,
                            ((int64_t)1 << 29) + 8};
    for (size_t i = 0; i < sizeof badF / sizeof badF[0]; ++i)
        REJECT(q4proj_pack_gate_up(U8(C, 0), U8(S, 0), U8(C2, 0), U8(S2, 0), 0.5f, 0.5f, badF[i],
                                   5120, U8(PC, 0), U8(PS, 0), STREAM),
               Q4P_EINVAL, "pack_gate_up bad F");
    REJECT(q4proj_pack_gate_up(U8(C, 0), U8(S, 0), U8(C2, 0), U8(S2, 0), 0.5f, 1.0f, F, 5120,
                               U8(PC, 0), U8(PS, 0), STREAM),
           Q4P_EINVAL, "pack_gate_up unequal global scales");
    REJECT(q4proj_pack_gate_up(U8(C, 0), U8(S, 0), U8(C2, 0), U8(S2, 0), NAN, NAN, F, 5120,
                               U8(PC, 0), U8(PS, 0), STREAM),
           Q4P_EINVAL, "pack_gate_up NaN global scales");
    REJECT(q4proj_pack_gate_up(U8(C, 0), U8(S, 0), U8(C2, 0), U8(S2, 0), 0.0f, -0.0f, F, 5120,
                               U8(PC, 0), U8(PS, 0), STREAM),
           Q4P_EINVAL, "pack_gate_up +0 vs -0");
    REJECT(q4proj_pack_gate_up(U8(C, 0), U8(S, 0), U8(C, 256), U8(S2, 0), 0.5f, 0.5f, F, 5120,
                               U8(PC, 0), U8(C, 0), STREAM),
           Q4P_EINVAL, "pack_gate_up output overlaps an input");
}

static void silu_argmax_quant_checks(void)
{
    const int64_t F = 8704, K = 5120, N = 248320;
    ACCEPT(q4proj_gemv_silu_mul(U8(PC, 0), U8(PS, 0), 1.f, U16(X, 0), U16(Y, 0), 1, F, K,
                                VP(WS, 0), 8192, STREAM),
           "gemv_silu_mul", "gemv_silu_mul");
    REJECT(q4proj_gemv_silu_mul(U8(PC, 0), U8(PS, 0), 1.f, U16(X, 0), U16(Y, 0), 1, 12, K,
                                VP(WS, 0), 8192, STREAM),
           Q4P_EINVAL, "silu F % 8");
    REJECT(q4proj_gemv_silu_mul(U8(PC, 0), U8(PS, 0), 1.f, U16(X, 0), U16(Y, 0), 1,
                                (int64_t)1 << 62, K, VP(WS, 0), 8192, STREAM),
           Q4P_EINVAL, "silu F = 2^62");
    REJECT(q4proj_gemv_silu_mul(U8(PC, 0), U8(PS, 0), 1.f, U16(X, 0), U16(Y, 0), 17, F, K,
                                VP(WS, 0), 8192, STREAM),
           Q4P_EUNSUPPORTED, "silu M=17");
    REJECT(q4proj_gemv_silu_mul(U8(PC, 0), U8(PS, 0), 1.f, U16(X, 0), U16(Y, 0), 1, F, K,
                                VP(WS, 0), 8191, STREAM),
           Q4P_EWORKSPACE, "silu workspace short");
    REJECT(q4proj_gemv_silu_mul(U8(PC, 0), U8(PS, 0), 1.f, U16(X, 0), U16(X, 2), 1, F, K,
                                VP(WS, 0), 8192, STREAM),
           Q4P_EINVAL, "silu h overlaps x");
    stub_set_sizes(4096, 8192, 12288, 256, 1 << 20, 0, 1);
    REJECT(q4proj_gemv_silu_mul(U8(PC, 0), U8(PS, 0), 1.f, U16(X, 0), U16(Y, 0), 1, F, K,
                                VP(WS, 0), 8192, STREAM),
           Q4P_EUNSUPPORTED, "silu shape the GEMV does not serve");
    stub_set_sizes(4096, 8192, 12288, 256, 1 << 20, 1, 1);
    ACCEPT(q4proj_gemm_silu_mul(U8(PC, 0), U8(PS, 0), 1.f, U16(X, 0), U16(Y, 0), 512, F, K, NULL, 0,
                                STREAM),
           "gemm_silu_mul", "gemm_silu_mul");
    {
        const size_t need = q4proj_gemm_workspace_bytes(512, 2 * F, K);
        ACCEPT(q4proj_gemm_silu_mul(U8(PC, 0), U8(PS, 0), 1.f, U16(X, 0), U16(Y, 0), 512, F, K,
                                    VP(WS, 0), need, STREAM),
               "gemm_silu_mul", "gemm_silu_mul with a workspace");
        CHECK(stub_last()->workspace == VP(WS, 0), "gemm_silu_mul workspace not passed on");
        REJECT(q4proj_gemm_silu_mul(U8(PC, 0), U8(PS, 0), 1.f, U16(X, 0), U16(Y, 0), 512, F, K,
                                    VP(WS, 0), need - 256, STREAM),
               Q4P_EWORKSPACE, "gemm_silu_mul workspace short");
        REJECT(q4proj_gemm_silu_mul(U8(PC, 0), U8(PS, 0), 1.f, U16(X, 0), U16(Y, 0), 512, F, K,
                                    VP(Y, 64), need, STREAM),
               Q4P_EINVAL, "gemm_silu_mul workspace overlaps h");
        REJECT(q4proj_gemm_silu_mul(U8(PC, 0), U8(PS, 0), 1.f, U16(X, 0), U16(Y, 0), 512, F, K,
                                    VP(WS, 4), need, STREAM),
               Q4P_EINVAL, "gemm_silu_mul workspace misaligned");
    }

    ACCEPT(q4proj_gemv_argmax(U8(PC, 0), U8(PS, 0), 1.f, U16(X, 0), NULL, F32(V, 0), I64(IDX, 0), 1,
                              N, K, VP(WS, 0), 12288, STREAM),
           "gemv_argmax", "argmax without logits");
    ACCEPT(q4proj_gemv_argmax(U8(PC, 0), U8(PS, 0), 1.f, U16(X, 0), F32(Y, 0), F32(V, 0),
                              I64(IDX, 0), 7, N, K, VP(WS, 0), 12288, STREAM),
           "gemv_argmax", "argmax with logits");
    REJECT(q4proj_gemv_argmax(U8(PC, 0), U8(PS, 0), 1.f, U16(X, 0), NULL, F32(V, 2), I64(IDX, 0), 1,
                              N, K, VP(WS, 0), 12288, STREAM),
           Q4P_EINVAL, "argmax value misaligned");
    REJECT(q4proj_gemv_argmax(U8(PC, 0), U8(PS, 0), 1.f, U16(X, 0), NULL, F32(V, 0), I64(IDX, 4), 1,
                              N, K, VP(WS, 0), 12288, STREAM),
           Q4P_EINVAL, "argmax index misaligned");
    REJECT(q4proj_gemv_argmax(U8(PC, 0), U8(PS, 0), 1.f, U16(X, 0), NULL, F32(V, 0), I64(V, 0), 1, N,
                              K, VP(WS, 0), 12288, STREAM),
           Q4P_EINVAL, "argmax value overlaps index");
    REJECT(q4proj_gemv_argmax(U8(PC, 0), U8(PS, 0), 1.f, U16(X, 0), F32(V, 0), F32(V, 0),
                              I64(IDX, 0), 1, N, K, VP(WS, 0), 12288, STREAM),
           Q4P_EINVAL, "argmax logits overlap value");
    REJECT(q4proj_gemv_argmax(U8(PC, 0), U8(PS, 0), 1.f, U16(X, 0), NULL, F32(V, 0), I64(IDX, 0), 17,
                              N, K, VP(WS, 0), 12288, STREAM),
           Q4P_EUNSUPPORTED, "argmax M=17");
    REJECT(q4proj_gemv_argmax(U8(PC, 0), U8(PS, 0), 1.f, U16(X, 0), NULL, F32(V, 0), I64(IDX, 0), 1,
                              N, K, VP(WS, 0), 12287, STREAM),
           Q4P_EWORKSPACE, "argmax workspace short");
    REJECT(q4proj_gemv_argmax(U8(PC, 0), U8(PS, 0), 1.f, U16(X, 0), NULL, F32(V, 0), I64(IDX, 0), 1,
                              N, K, VP(V, 0), 12288, STREAM),
           Q4P_EINVAL, "argmax workspace overlaps value");

    ACCEPT(q4proj_quantize(U16(X, 0), 34816, K, U8(C, 0), U8(S, 0), F32(V, 0), VP(WS, 0), 256,
                           STREAM),
           "quantize", "quantize");
    REJECT(q4proj_quantize(U16(X, 0), 34816, K, U8(X, 1024), U8(S, 0), F32(V, 0), VP(WS, 0), 256,
                           STREAM),
           Q4P_EINVAL, "quantize codes overlap w");
    REJECT(q4proj_quantize(U16(X, 0), 34816, K, U8(C, 0), U8(S, 0), F32(V, 2), VP(WS, 0), 256,
                           STREAM),
           Q4P_EINVAL, "quantize global scale misaligned");
    REJECT(q4proj_quantize(U16(X, 0), 34816, K, U8(C, 0), U8(S, 0), F32(V, 0), VP(WS, 0), 255,
                           STREAM),
           Q4P_EWORKSPACE, "quantize workspace short");
}

static void size_checks(void)
{
    CHECK(q4proj_packed_codes_bytes(17, 144) == 4 * 1024, "codes bytes of 17 x 144");
    CHECK(q4proj_packed_scales_bytes(17, 144) == 4 * 128, "scales bytes of 17 x 144");
    CHECK(q4proj_packed_codes_bytes(17408, 5120) == (size_t)1088 * 40 * 1024, "codes bytes");
    CHECK(q4proj_packed_codes_bytes(0, 16) == 0 && q4proj_packed_codes_bytes(16, 8) == 0 &&
              q4proj_packed_codes_bytes(INT64_MAX, INT64_MAX) == 0 &&
              q4proj_packed_scales_bytes(-16, 16) == 0,
          "sizes of invalid shapes");
    CHECK(q4proj_workspace_bytes(1, 17408, 5120) == 4096, "workspace bytes");
    CHECK(q4proj_workspace_bytes(0, 17408, 5120) == 0 && q4proj_workspace_bytes(17, 17408, 5120) == 0,
          "workspace bytes outside the GEMV range");
    CHECK(q4proj_silu_mul_workspace_bytes(1, 12, 5120) == 0 &&
              q4proj_silu_mul_workspace_bytes(1, (int64_t)1 << 62, 5120) == 0 &&
              q4proj_silu_mul_workspace_bytes(1, 8704, 5120) == 8192,
          "silu workspace bytes");
    CHECK(q4proj_argmax_workspace_bytes(17, 248320, 5120) == 0 &&
              q4proj_argmax_workspace_bytes(1, 248320, 5120) == 12288,
          "argmax workspace bytes");
    CHECK(q4proj_quantize_workspace_bytes(-1, 16) == 0 && q4proj_quantize_workspace_bytes(16, 16) == 256,
          "quantize workspace bytes");
    const q4proj_status all[] = {Q4P_OK, Q4P_EINVAL, Q4P_EUNSUPPORTED, Q4P_EDEVICE,
                                 Q4P_EWORKSPACE, Q4P_EHIP};
    const char *names[] = {"Q4P_OK", "Q4P_EINVAL", "Q4P_EUNSUPPORTED", "Q4P_EDEVICE",
                           "Q4P_EWORKSPACE", "Q4P_EHIP"};
    for (int i = 0; i < 6; ++i) {
        const char *s = q4proj_status_string(all[i]);
        CHECK(s && strncmp(s, names[i], strlen(names[i])) == 0, "status string %d: %s", i, s);
    }
    CHECK(strcmp(q4proj_status_string((q4proj_status)99), "unknown q4proj_status") == 0,
          "unknown status string");
}

int main(void)
{
    stub_reset();
    stub_set_arch(0, "gfx950:sramecc+:xnack-");
    stub_set_device(0, 0);
    gemv_checks();
    device_checks();
    gemm_checks();
    pack_checks();
    silu_argmax_quant_checks();
    size_checks();
    printf("hostcheck: %d checks, %d failed\n", g_checks, g_failed);
    return g_failed == 0 ? 0 : 1;
}
