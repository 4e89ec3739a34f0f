/*
 * A plain C consumer of the q4proj C ABI (include/q4proj.h): no Python, no
 * torch.  It allocates device memory with the HIP runtime, packs a seeded
 * NVFP4 weight, runs q4proj_gemv (M = 3) and q4proj_gemm (M = 40) on a
 * stream of its own, unpacks the weight again, and checks every output
 * against the CPU oracle (oracle/oracle.c, fp64) with the projection's
 * tolerance |y - y_ref| <= 2e-3 * sum_k |x_k w_k|.  It also checks that
 * invalid calls are rejected with the documented status before anything is
 * launched.  Test infrastructure: built by tests/c_abi/build.py into a shared
 * library whose one entry point tests/test_gpu_c_abi.py calls (in-process:
 * the test process must not start another program once it uses the GPU).
 *
 * abi_consumer_run() returns 0 when every check passes, 1 otherwise (the
 * failing check is printed).
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "q4proj.h"

/* the seeded input generators (synth/synth.c) */
void syn_uniform_codes(uint64_t seed, uint64_t stream, int64_t byte0, int64_t count, uint8_t *out);
void syn_abs_normal_e4m3(uint64_t seed, uint64_t stream, double sd, double offset, int64_t i0,
                         int64_t count, uint8_t *out);
void syn_normal_bf16(uint64_t seed, uint64_t stream, double stddev, int64_t i0, int64_t count,
                     uint16_t *out);
/* the oracle (oracle/oracle.c) */
int orc_proj(int64_t M, int64_t N, int64_t K, const uint8_t *codes, const uint8_t *scales,
             double g, const uint16_t *x, double *y, double *S, int nthreads);
int64_t orc_check(int64_t count, const double *yref, const double *S, const float *ygpu,
                  double rtol, double *max_ratio);

#define CHECK(cond, ...)                                                   \
    do {                                                                   \
        if (!(cond)) {                                                     \
            fprintf(stderr, "FAILED: " __VA_ARGS__);                       \
            fprintf(stderr, "\n");                                         \
            fflush(stderr);                                                \
            return 1;                                                      \
        }                                                                  \
    } while (0)

#define HIP(call) CHECK((call) == hipSuccess, "%s", #call)

static void *dev_alloc(size_t n)
{
    void *p = NULL;
    return hipMalloc(&p, n) == hipSuccess ? p : NULL;
}

int abi_consumer_run(void)
{
    const int64_t N = 300, K = 1040, MV = 3, MG = 40;
    const float g = 0.75f;
    const size_t ncodes = (size_t)(N * K / 2), nscales = (size_t)(N * K / 16);

    uint8_t *codes = malloc(ncodes), *scales = malloc(nscales);
    uint8_t *codes2 = malloc(ncodes), *scales2 = malloc(nscales);
    uint16_t *x = malloc((size_t)(MG * K) * 2);
    float *y = malloc((size_t)(MG * N) * 4);
    double *yref = malloc((size_t)(MG * N) * 8), *S = malloc((size_t)(MG * N) * 8);
    CHECK(codes && scales && codes2 && scales2 && x && y && yref && S, "host allocation");
    syn_uniform_codes(21, 1, 0, (int64_t)ncodes, codes);
    syn_abs_normal_e4m3(21, 2, 0.5, 0.01, 0, (int64_t)nscales, scales);
    syn_normal_bf16(21, 3, 1.0, 0, MG * K, x);

    hipStream_t stream;
    HIP(hipStreamCreate(&stream));
    const size_t pcb = q4proj_packed_codes_bytes(N, K), psb = q4proj_packed_scales_bytes(N, K);
    const size_t wsb = q4proj_workspace_bytes(MV, N, K);
    CHECK(pcb >= ncodes && psb >= nscales && wsb > 0, "size queries");
    uint8_t *d_codes = dev_alloc(ncodes), *d_scales = dev_alloc(nscales);
    uint8_t *d_pc = dev_alloc(pcb), *d_ps = dev_alloc(psb);
    uint16_t *d_x = dev_alloc((size_t)(MG * K) * 2);
    float *d_y = dev_alloc((size_t)(MG * N) * 4);
    void *d_ws = dev_alloc(wsb);
    CHECK(d_codes && d_scales && d_pc && d_ps && d_x && d_y && d_ws, "device allocation");
    HIP(hipMemcpy(d_codes, codes, ncodes, hipMemcpyHostToDevice));
    HIP(hipMemcpy(d_scales, scales, nscales, hipMemcpyHostToDevice));
    HIP(hipMemcpy(d_x, x, (size_t)(MG * K) * 2, hipMemcpyHostToDevice));
    HIP(hipMemset(d_ws, 0, wsb));   /* zero-filled once; every call leaves it so */

    q4proj_status st = q4proj_pack(d_codes, d_scales, N, K, d_pc, d_ps, stream);
    CHECK(st == Q4P_OK, "q4proj_pack: %s", q4proj_status_string(st));

    /* rejected before any launch */
    st = q4proj_gemv(d_pc, d_ps, g, d_x, d_y, 17, N, K, d_ws, wsb, stream);
    CHECK(st == Q4P_EUNSUPPORTED, "gemv M = 17 gave %d", (int)st);
    st = q4proj_gemv(d_pc, d_ps, g, d_x, NULL, MV, N, K, d_ws, wsb, stream);
    CHECK(st == Q4P_EINVAL, "gemv y = NULL gave %d", (int)st);
    st = q4proj_gemv(d_pc, d_ps, g, d_x, d_y, MV, N, K + 8, d_ws, wsb, stream);
    CHECK(st == Q4P_EINVAL, "gemv K %% 16 != 0 gave %d", (int)st);
    st = q4proj_gemv(d_pc, d_ps, g, d_x, d_y, MV, N, K, d_ws, wsb - 1, stream);
    CHECK(st == Q4P_EWORKSPACE, "gemv short workspace gave %d", (int)st);
    CHECK(q4proj_status_string(Q4P_EHIP) != NULL, "status string");

    CHECK(orc_proj(MG, N, K, codes, scales, (double)g, x, yref, S, 4) == 0, "oracle");
    const struct { const char *name; int64_t M; } runs[2] = {{"q4proj_gemv", MV}, {"q4proj_gemm", MG}};
    for (int i = 0; i < 2; ++i) {
        const int64_t M = runs[i].M;
        HIP(hipMemsetAsync(d_y, 0xFF, (size_t)(M * N) * 4, stream));    /* NaN fill */
        st = i == 0 ? q4proj_gemv(d_pc, d_ps, g, d_x, d_y, M, N, K, d_ws, wsb, stream)
                    : q4proj_gemm(d_pc, d_ps, g, d_x, d_y, M, N, K, NULL, 0, stream);
        CHECK(st == Q4P_OK, "%s: %s", runs[i].name, q4proj_status_string(st));
        HIP(hipStreamSynchronize(stream));
        HIP(hipMemcpy(y, d_y, (size_t)(M * N) * 4, hipMemcpyDeviceToHost));
        double worst = 0.0;
        /* the oracle's rows 0..M-1 are the first M*N entries */
        const int64_t bad = orc_check(M * N, yref, S, y, 2e-3, &worst);
        CHECK(bad == 0, "%s: %lld of %lld outputs outside tolerance", runs[i].name,
              (long long)bad, (long long)(M * N));
        printf("%s M=%lld N=%lld K=%lld ok, max |y-y_ref|/S = %.3g\n", runs[i].name,
               (long long)M, (long long)N, (long long)K, worst);
    }

    st = q4proj_unpack(d_pc, d_ps, N, K, d_codes, d_scales, stream);
    CHECK(st == Q4P_OK, "q4proj_unpack: %s", q4proj_status_string(st));
    HIP(hipStreamSynchronize(stream));
    HIP(hipMemcpy(codes2, d_codes, ncodes, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(scales2, d_scales, nscales, hipMemcpyDeviceToHost));
    CHECK(memcmp(codes, codes2, ncodes) == 0 && memcmp(scales, scales2, nscales) == 0,
          "pack/unpack round trip");
    printf("pack/unpack round trip ok\n");

    hipFree(d_codes); hipFree(d_scales); hipFree(d_pc); hipFree(d_ps);
    hipFree(d_x); hipFree(d_y); hipFree(d_ws);
    HIP(hipStreamDestroy(stream));
    free(codes); free(scales); free(codes2); free(scales2); free(x); free(y); free(yref); free(S);
    printf("c abi consumer: all checks passed\n");
    fflush(stdout);
    return 0;
}
