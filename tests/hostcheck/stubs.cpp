// CPU stand-ins for the HIP runtime calls and the kernel launchers behind
// the library's host front (q4p_api.cpp), for its CPU build under ASan and
// UBSan: every launcher records its arguments and returns the error the
// driver set; no buffer is ever dereferenced.  Test infrastructure only.
#include <hip/hip_runtime.h>

#include <cstring>

#include "q4p_launch.h"
#include "stub_control.h"

namespace {

int g_device = 0, g_device_rc = 0, g_launch_error = 0, g_props_calls = 0;
char g_arch[64][64];
size_t g_gemv_ws = 4096, g_silu_ws = 8192, g_argmax_ws = 12288, g_quant_ws = 256,
       g_noalloc_max = 1 << 20;
int g_silu_ok = 1, g_argmax_ok = 1;
stub_launch g_last;

hipError_t record(const char *name, int64_t M, int64_t N, int64_t K, const void *in0,
                  const void *in1, void *out, void *ws, hipStream_t stream, float g)
{
    g_last.count += 1;
    std::strncpy(g_last.name, name, sizeof g_last.name - 1);
    g_last.name[sizeof g_last.name - 1] = '\0';
    g_last.M = M;
    g_last.N = N;
    g_last.K = K;
    g_last.in0 = in0;
    g_last.in1 = in1;
    g_last.out = out;
    g_last.workspace = ws;
    g_last.stream = static_cast<void *>(stream);
    g_last.g = g;
    return static_cast<hipError_t>(g_launch_error);
}

}  // namespace

extern "C" {

void stub_reset(void)
{
    std::memset(&g_last, 0, sizeof g_last);
    g_launch_error = 0;
    g_props_calls = 0;
}

void stub_set_device(int device, int rc)
{
    g_device = device;
    g_device_rc = rc;
}

void stub_set_arch(int device, const char *arch)
{
    if (device >= 0 && device < 64) {
        std::strncpy(g_arch[device], arch, sizeof g_arch[device] - 1);
        g_arch[device][sizeof g_arch[device] - 1] = '\0';
    }
}

void stub_set_launch_error(int error) { g_launch_error = error; }

void stub_set_sizes(size_t gemv_ws, size_t silu_ws, size_t argmax_ws, size_t quant_ws,
                    size_t noalloc_max, int silu_supported, int argmax_supported)
{
    g_gemv_ws = gemv_ws;
    g_silu_ws = silu_ws;
    g_argmax_ws = argmax_ws;
    g_quant_ws = quant_ws;
    g_noalloc_max = noalloc_max;
    g_silu_ok = silu_supported;
    g_argmax_ok = argmax_supported;
}

int stub_props_calls(void) { return g_props_calls; }

const stub_launch *stub_last(void) { return &g_last; }

hipError_t hipGetDevice(int *device)
{
    if (g_device_rc != 0)
        return static_cast<hipError_t>(g_device_rc);
    *device = g_device;
    return hipSuccess;
}

hipError_t hipGetDeviceProperties(hipDeviceProp_t *prop, int device)
{
    g_props_calls += 1;
    if (device < 0 || device >= 64)
        return hipErrorInvalidValue;
    std::memset(prop, 0, sizeof *prop);
    std::strncpy(prop->gcnArchName, g_arch[device], sizeof prop->gcnArchName - 1);
    return hipSuccess;
}

const char *hipGetErrorString(hipError_t error)
{
    switch (error) {
    case hipSuccess: return "hipSuccess";
    case hipErrorInvalidValue: return "hipErrorInvalidValue";
    case hipErrorNoDevice: return "hipErrorNoDevice";
    case hipErrorLaunchFailure: return "hipErrorLaunchFailure";
    }
    return "stub: unknown error";
}

}  // extern "C"

namespace q4p {

hipError_t launch_pack(const uint8_t *codes, const uint8_t *scales, int64_t N, int64_t K,
                       uint8_t *packed_codes, uint8_t *packed_scales, hipStream_t stream)
{
    (void)packed_scales;
    return record("pack", 0, N, K, codes, scales, packed_codes, nullptr, stream, 0.f);
}

hipError_t launch_pack_gate_up(const uint8_t *gate_codes, const uint8_t *gate_scales,
                               const uint8_t *up_codes, const uint8_t *up_scales, int64_t F,
                               int64_t K, uint8_t *packed_codes, uint8_t *packed_scales,
                               hipStream_t stream)
{
    (void)up_codes;
    (void)up_scales;
    (void)packed_scales;
    return record("pack_gate_up", 0, F, K, gate_codes, gate_scales, packed_codes, nullptr,
                  stream, 0.f);
}

hipError_t launch_unpack(const uint8_t *packed_codes, const uint8_t *packed_scales, int64_t N,
                         int64_t K, uint8_t *codes, uint8_t *scales, hipStream_t stream)
{
    (void)scales;
    return record("unpack", 0, N, K, packed_codes, packed_scales, codes, nullptr, stream, 0.f);
}

size_t gemv_workspace_bytes(int64_t, int64_t, int64_t) { return g_gemv_ws; }

hipError_t launch_gemv(const uint8_t *packed_codes, const uint8_t *packed_scales, float g,
                       const uint16_t *x, float *y, int64_t M, int64_t N, int64_t K,
                       void *workspace, hipStream_t stream)
{
    (void)x;
    return record("gemv", M, N, K, packed_codes, packed_scales, y, workspace, stream, g);
}

size_t gemv_noalloc_max_bytes() { return g_noalloc_max; }

hipError_t launch_gemv_noalloc(const uint8_t *packed_codes, const uint8_t *packed_scales,
                               float g, const uint16_t *x, float *y, int64_t M, int64_t N,
                               int64_t K, hipStream_t stream)
{
    (void)x;
    return record("gemv_noalloc", M, N, K, packed_codes, packed_scales, y, nullptr, stream, g);
}

bool gemv_silu_mul_supported(int64_t, int64_t, int64_t) { return g_silu_ok != 0; }

size_t gemv_silu_mul_workspace_bytes(int64_t, int64_t, int64_t)
{
    return g_silu_ok ? g_silu_ws : 0;
}

hipError_t launch_gemv_silu_mul(const uint8_t *packed_codes, const uint8_t *packed_scales,
                                float g, const uint16_t *x, uint16_t *h, int64_t M, int64_t F,
                                int64_t K, void *workspace, hipStream_t stream)
{
    (void)x;
    return record("gemv_silu_mul", M, F, K, packed_codes, packed_scales, h, workspace, stream, g);
}

bool gemv_argmax_supported(int64_t, int64_t, int64_t) { return g_argmax_ok != 0; }

size_t gemv_argmax_workspace_bytes(int64_t, int64_t, int64_t)
{
    return g_argmax_ok ? g_argmax_ws : 0;
}

hipError_t launch_gemv_argmax(const uint8_t *packed_codes, const uint8_t *packed_scales, float g,
                              const uint16_t *x, float *y, float *best_val, int64_t *best_idx,
                              int64_t M, int64_t N, int64_t K, void *workspace,
                              hipStream_t stream)
{
    (void)x;
    (void)y;
    (void)best_idx;
    return record("gemv_argmax", M, N, K, packed_codes, packed_scales, best_val, workspace,
                  stream, g);
}

// the documented size: the fp16 activations and the row multipliers, each
// rounded up to 256 bytes
size_t gemm_workspace_bytes(int64_t M, int64_t K)
{
    return (size_t)((M * K * 2 + 255) / 256 * 256 + (M * 4 + 255) / 256 * 256);
}

hipError_t launch_gemm(const uint8_t *packed_codes, const uint8_t *packed_scales, float g,
                       const uint16_t *x, float *y, int64_t M, int64_t N, int64_t K,
                       void *workspace, hipStream_t stream)
{
    (void)x;
    return record("gemm", M, N, K, packed_codes, packed_scales, y, workspace, stream, g);
}

hipError_t launch_gemm_silu_mul(const uint8_t *packed_codes, const uint8_t *packed_scales,
                                float g, const uint16_t *x, uint16_t *h, int64_t M, int64_t F,
                                int64_t K, void *workspace, hipStream_t stream)
{
    (void)x;
    return record("gemm_silu_mul", M, F, K, packed_codes, packed_scales, h, workspace, stream, g);
}

size_t quant_workspace_bytes() { return g_quant_ws; }

hipError_t launch_quantize(const uint16_t *w, int64_t N, int64_t K, uint8_t *codes,
                           uint8_t *scales, float *global_scale, void *workspace,
                           hipStream_t stream)
{
    (void)scales;
    return record("quantize", 0, N, K, w, global_scale, codes, workspace, stream, 0.f);
}

}  // namespace q4p
