/*
 * A plain C consumer of the q4proj C ABI (include/q4proj.h): no Python, no
 * torch.  It allocates device memory with the HIP runtime, packs a seeded
 * NVFP4 weight, runs q4proj_gemv (M = 3) and q4proj_gemm (M = 40, without
 * and with its fp16 staging workspace, bit for bit alike) on a stream of its
 * own, unpacks the weight again, and checks every output
 * against the CPU oracle (oracle/oracle.c, fp64) with the projection's
 * tolerance |y - y_ref| <= 2e-3 * sum_k |x_k w_k|.  It then builds a fused
 * gate/up weight from two separate weights (q4proj_pack_gate_up) and runs
 * q4proj_gemv_silu_mul and q4proj_gemm_silu_mul on it, runs the greedy
 * argmax (q4proj_gemv_argmax) and the NVFP4 quantizer (q4proj_quantize),
 * each against the oracle (bit for bit for the quantizer).  It also checks that
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
void orc_silu_mul(int64_t count, const double *gate, const double *up, double *h);
void orc_silu_mul_bound(int64_t count, const double *gate, const double *up, const double *Sg,
                        const double *Su, double rtol, double *bound);
int64_t orc_check_bf16(int64_t count, const double *href, const double *bound,
                       const uint16_t *hgpu, double *max_ratio);
int64_t orc_argmax_check(int64_t M, int64_t N, const double *yref, const double *S, double rtol,
                         const int64_t *idx, const float *val);
float orc_quant_global_scale(int64_t count, const uint16_t *w);
void orc_quantize(int64_t N, int64_t K, const uint16_t *w, float g, uint8_t *codes,
                  uint8_t *scales);

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
    /* the GEMMs' optional staging workspace: fp16 operands, the same results */
    const size_t gwsb = q4proj_gemm_workspace_bytes(MG, N, K);
    CHECK(gwsb == (size_t)(MG * K * 2 + 255) / 256 * 256 + (size_t)(MG * 4 + 255) / 256 * 256,
          "gemm workspace size %zu", gwsb);
    void *d_gws = dev_alloc(gwsb);
    CHECK(d_gws != NULL, "device allocation (gemm workspace)");
    st = q4proj_gemm(d_pc, d_ps, g, d_x, d_y, MG, N, K, d_gws, gwsb - 1, stream);
    CHECK(st == Q4P_EWORKSPACE, "gemm short workspace gave %d", (int)st);
    st = q4proj_gemm(d_pc, d_ps, g, d_x, d_y, MG, N, K, d_x, gwsb, stream);
    CHECK(st == Q4P_EINVAL, "gemm workspace overlapping x gave %d", (int)st);
    float *ybf = malloc((size_t)(MG * N) * 4);
    CHECK(ybf != NULL, "host allocation");
    const struct { const char *name; int64_t M; } runs[3] = {
        {"q4proj_gemv", MV}, {"q4proj_gemm", MG}, {"q4proj_gemm (staged fp16)", MG}};
    for (int i = 0; i < 3; ++i) {
        const int64_t M = runs[i].M;
        HIP(hipMemsetAsync(d_y, 0xFF, (size_t)(M * N) * 4, stream));    /* NaN fill */
        st = i == 0   ? q4proj_gemv(d_pc, d_ps, g, d_x, d_y, M, N, K, d_ws, wsb, stream)
             : i == 1 ? q4proj_gemm(d_pc, d_ps, g, d_x, d_y, M, N, K, NULL, 0, stream)
                      : q4proj_gemm(d_pc, d_ps, g, d_x, d_y, M, N, K, d_gws, gwsb, stream);
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
        if (i == 1)
            memcpy(ybf, y, (size_t)(M * N) * 4);
        if (i == 2)
            CHECK(memcmp(ybf, y, (size_t)(M * N) * 4) == 0, "staged gemm differs from bf16 gemm");
    }
    free(ybf);
    hipFree(d_gws);

    st = q4proj_unpack(d_pc, d_ps, N, K, d_codes, d_scales, stream);
    CHECK(st == Q4P_OK, "q4proj_unpack: %s", q4proj_status_string(st));
    HIP(hipStreamSynchronize(stream));
    HIP(hipMemcpy(codes2, d_codes, ncodes, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(scales2, d_scales, nscales, hipMemcpyDeviceToHost));
    CHECK(memcmp(codes, codes2, ncodes) == 0 && memcmp(scales, scales2, nscales) == 0,
          "pack/unpack round trip");
    printf("pack/unpack round trip ok\n");

    /* greedy argmax over the logits of rows 0..MV-1, no logits written */
    {
        const size_t awb = q4proj_argmax_workspace_bytes(MV, N, K);
        void *d_aws = dev_alloc(awb);
        float *d_val = dev_alloc(MV * sizeof(float));
        int64_t *d_idx = dev_alloc(MV * sizeof(int64_t));
        CHECK(awb > 0 && d_aws && d_val && d_idx, "argmax allocation");
        HIP(hipMemset(d_aws, 0, awb));
        st = q4proj_gemv_argmax(d_pc, d_ps, g, d_x, NULL, d_val, d_idx, MV, N, K, d_aws, awb,
                                stream);
        CHECK(st == Q4P_OK, "q4proj_gemv_argmax: %s", q4proj_status_string(st));
        HIP(hipStreamSynchronize(stream));
        float val[16];
        int64_t idx[16];
        HIP(hipMemcpy(val, d_val, MV * sizeof(float), hipMemcpyDeviceToHost));
        HIP(hipMemcpy(idx, d_idx, MV * sizeof(int64_t), hipMemcpyDeviceToHost));
        CHECK(orc_argmax_check(MV, N, yref, S, 2e-3, idx, val) == 0, "argmax rows");
        printf("q4proj_gemv_argmax M=%lld N=%lld K=%lld ok\n", (long long)MV, (long long)N,
               (long long)K);
        hipFree(d_aws); hipFree(d_val); hipFree(d_idx);
    }

    /* fused gate/up from two separate weights (one global scale) + silu * up */
    {
        const int64_t F = 152, FK = 1040;
        const size_t fc = (size_t)(F * FK / 2), fs = (size_t)(F * FK / 16);
        uint8_t *gc = malloc(fc), *gs = malloc(fs), *uc = malloc(fc), *us = malloc(fs);
        double *ga = malloc((size_t)(MG * F) * 8), *gS = malloc((size_t)(MG * F) * 8);
        double *ua = malloc((size_t)(MG * F) * 8), *uS = malloc((size_t)(MG * F) * 8);
        double *href = malloc((size_t)(MG * F) * 8), *hb = malloc((size_t)(MG * F) * 8);
        uint16_t *h = malloc((size_t)(MG * F) * 2);
        CHECK(gc && gs && uc && us && ga && gS && ua && uS && href && hb && h, "host allocation");
        syn_uniform_codes(22, 1, 0, (int64_t)fc, gc);
        syn_abs_normal_e4m3(22, 2, 0.5, 0.01, 0, (int64_t)fs, gs);
        syn_uniform_codes(22, 3, 0, (int64_t)fc, uc);
        syn_abs_normal_e4m3(22, 4, 0.5, 0.01, 0, (int64_t)fs, us);
        const size_t fpcb = q4proj_packed_codes_bytes(2 * F, FK);
        const size_t fpsb = q4proj_packed_scales_bytes(2 * F, FK);
        const size_t fwsb = q4proj_silu_mul_workspace_bytes(MV, F, FK);
        uint8_t *d_gc = dev_alloc(fc), *d_gs = dev_alloc(fs), *d_uc = dev_alloc(fc), *d_us = dev_alloc(fs);
        uint8_t *d_fpc = dev_alloc(fpcb), *d_fps = dev_alloc(fpsb);
        uint16_t *d_h = dev_alloc((size_t)(MG * F) * 2);
        void *d_fws = dev_alloc(fwsb);
        CHECK(d_gc && d_gs && d_uc && d_us && d_fpc && d_fps && d_h && d_fws && fwsb > 0,
              "device allocation");
        HIP(hipMemcpy(d_gc, gc, fc, hipMemcpyHostToDevice));
        HIP(hipMemcpy(d_gs, gs, fs, hipMemcpyHostToDevice));
        HIP(hipMemcpy(d_uc, uc, fc, hipMemcpyHostToDevice));
        HIP(hipMemcpy(d_us, us, fs, hipMemcpyHostToDevice));
        HIP(hipMemset(d_fws, 0, fwsb));
        st = q4proj_pack_gate_up(d_gc, d_gs, d_uc, d_us, g, 0.5f, F, FK, d_fpc, d_fps, stream);
        CHECK(st == Q4P_EINVAL, "pack_gate_up with unequal global scales gave %d", (int)st);
        st = q4proj_pack_gate_up(d_gc, d_gs, d_uc, d_us, g, g, F, FK, d_fpc, d_fps, stream);
        CHECK(st == Q4P_OK, "q4proj_pack_gate_up: %s", q4proj_status_string(st));
        CHECK(orc_proj(MG, F, FK, gc, gs, (double)g, x, ga, gS, 4) == 0, "oracle gate");
        CHECK(orc_proj(MG, F, FK, uc, us, (double)g, x, ua, uS, 4) == 0, "oracle up");
        orc_silu_mul(MG * F, ga, ua, href);
        orc_silu_mul_bound(MG * F, ga, ua, gS, uS, 2e-3, hb);
        for (int i = 0; i < 2; ++i) {
            const int64_t M = i == 0 ? MV : MG;
            HIP(hipMemsetAsync(d_h, 0xFF, (size_t)(M * F) * 2, stream));
            st = i == 0 ? q4proj_gemv_silu_mul(d_fpc, d_fps, g, d_x, d_h, M, F, FK, d_fws, fwsb, stream)
                        : q4proj_gemm_silu_mul(d_fpc, d_fps, g, d_x, d_h, M, F, FK, NULL, 0, stream);
            CHECK(st == Q4P_OK, "silu_mul %d: %s", i, q4proj_status_string(st));
            HIP(hipStreamSynchronize(stream));
            HIP(hipMemcpy(h, d_h, (size_t)(M * F) * 2, hipMemcpyDeviceToHost));
            double worst = 0.0;
            const int64_t bad = orc_check_bf16(M * F, href, hb, h, &worst);
            CHECK(bad == 0, "%s: %lld outputs outside the allowance",
                  i == 0 ? "q4proj_gemv_silu_mul" : "q4proj_gemm_silu_mul", (long long)bad);
            printf("%s M=%lld F=%lld K=%lld ok\n",
                   i == 0 ? "q4proj_gemv_silu_mul" : "q4proj_gemm_silu_mul", (long long)M,
                   (long long)F, (long long)FK);
        }
        hipFree(d_gc); hipFree(d_gs); hipFree(d_uc); hipFree(d_us); hipFree(d_fpc); hipFree(d_fps);
        hipFree(d_h); hipFree(d_fws);
        free(gc); free(gs); free(uc); free(us); free(ga); free(gS); free(ua); free(uS);
        free(href); free(hb); free(h);
    }

    /* NVFP4 quantizer, bit for bit */
    {
        const int64_t QN = 96, QK = 1040;
        const size_t qn = (size_t)(QN * QK);
        uint16_t *w = malloc(qn * 2);
        uint8_t *qc = malloc(qn / 2), *qs = malloc(qn / 16), *rc = malloc(qn / 2), *rs = malloc(qn / 16);
        CHECK(w && qc && qs && rc && rs, "host allocation");
        syn_normal_bf16(23, 1, 0.02, 0, (int64_t)qn, w);
        const size_t qwb = q4proj_quantize_workspace_bytes(QN, QK);
        uint16_t *d_w = dev_alloc(qn * 2);
        uint8_t *d_qc = dev_alloc(qn / 2), *d_qs = dev_alloc(qn / 16);
        float *d_g = dev_alloc(sizeof(float));
        void *d_qws = dev_alloc(qwb);
        CHECK(d_w && d_qc && d_qs && d_g && d_qws, "device allocation");
        HIP(hipMemcpy(d_w, w, qn * 2, hipMemcpyHostToDevice));
        st = q4proj_quantize(d_w, QN, QK, d_qc, d_qs, d_g, d_qws, qwb, stream);
        CHECK(st == Q4P_OK, "q4proj_quantize: %s", q4proj_status_string(st));
        HIP(hipStreamSynchronize(stream));
        float gq = 0.0f;
        HIP(hipMemcpy(&gq, d_g, sizeof(float), hipMemcpyDeviceToHost));
        HIP(hipMemcpy(qc, d_qc, qn / 2, hipMemcpyDeviceToHost));
        HIP(hipMemcpy(qs, d_qs, qn / 16, hipMemcpyDeviceToHost));
        const float gr = orc_quant_global_scale((int64_t)qn, w);
        orc_quantize(QN, QK, w, gr, rc, rs);
        CHECK(memcmp(&gq, &gr, sizeof(float)) == 0, "quantize: global scale");
        CHECK(memcmp(qc, rc, qn / 2) == 0 && memcmp(qs, rs, qn / 16) == 0, "quantize: codes/scales");
        printf("q4proj_quantize N=%lld K=%lld bit-exact\n", (long long)QN, (long long)QK);
        hipFree(d_w); hipFree(d_qc); hipFree(d_qs); hipFree(d_g); hipFree(d_qws);
        free(w); free(qc); free(qs); free(rc); free(rs);
    }

    hipFree(d_codes); hipFree(d_scales); hipFree(d_pc); hipFree(d_ps);
    hipFree(d_x); hipFree(d_y); hipFree(d_ws);
    HIP(hipStreamDestroy(stream));
    free(codes); free(scales); free(codes2); free(scales2); free(x); free(y); free(yref); free(S);
    printf("c abi consumer: all checks passed\n");
    fflush(stdout);
    return 0;
}
