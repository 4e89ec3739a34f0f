// q4p_api.cpp — the C ABI of include/q4proj.h: argument validation, the
// gfx950 device check, and dispatch to the kernel launchers.
//
// Every argument check runs on the host before any HIP call, so a rejected
// call enqueues nothing and touches no device.  The device check runs next
// and is cached per device ordinal.
#include "q4proj.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <initializer_list>

#include "q4p_launch.h"
#include "q4p_layout.h"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_device_ok[kMaxDevices];   // 0 unknown, 1 gfx950, -1 other

thread_local char g_last_hip_error[256] = "";

q4proj_status record_hip(hipError_t e)
{
    if (e == hipSuccess)
        return Q4P_OK;
    const char *s = hipGetErrorString(e);
    std::strncpy(g_last_hip_error, s ? s : "unknown HIP error", sizeof g_last_hip_error - 1);
    g_last_hip_error[sizeof g_last_hip_error - 1] = '\0';
    return Q4P_EHIP;
}

// The library carries gfx950 code objects only and refuses every other device
// instead of falling back to another path.
q4proj_status check_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return Q4P_EDEVICE;
    if (dev < kMaxDevices) {
        int known = g_device_ok[dev].load(std::memory_order_relaxed);
        if (known != 0)
            return known > 0 ? Q4P_OK : Q4P_EDEVICE;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
        return Q4P_EDEVICE;
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < kMaxDevices)
        g_device_ok[dev].store(ok ? 1 : -1, std::memory_order_relaxed);
    return ok ? Q4P_OK : Q4P_EDEVICE;
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool shape_ok(int64_t N, int64_t K)
{
    // sizes the kernels index with 32-bit ints
    return N > 0 && K > 0 && K % 16 == 0 && N <= (int64_t)1 << 30 && K <= (int64_t)1 << 24;
}

bool overlap(const void *a, size_t na, const void *b, size_t nb)
{
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

q4proj_status check_projection(const uint8_t *pc, const uint8_t *ps, const uint16_t *x,
                               const float *y, int64_t M, int64_t N, int64_t K,
                               size_t workspace_bytes, size_t workspace_need)
{
    if (!pc || !ps || !x || !y)
        return Q4P_EINVAL;
    if (M <= 0 || !shape_ok(N, K) || M > (int64_t)1 << 24)
        return Q4P_EINVAL;
    if ((uint64_t)M * (uint64_t)N > ((uint64_t)1 << 40))
        return Q4P_EINVAL;
    if (!aligned(pc, 16) || !aligned(ps, 8) || !aligned(x, 16) || !aligned(y, 4))
        return Q4P_EINVAL;
    const size_t ybytes = (size_t)M * (size_t)N * sizeof(float);
    if (overlap(y, ybytes, x, (size_t)M * (size_t)K * 2) ||
        overlap(y, ybytes, pc, q4proj_packed_codes_bytes(N, K)) ||
        overlap(y, ybytes, ps, q4proj_packed_scales_bytes(N, K)))
        return Q4P_EINVAL;
    if (workspace_bytes < workspace_need)
        return Q4P_EWORKSPACE;
    return Q4P_OK;
}

// Arguments of the fused gate/up entry points (h: bf16 [M][F]).
q4proj_status check_silu_mul(const uint8_t *pc, const uint8_t *ps, const uint16_t *x,
                             const uint16_t *h, int64_t M, int64_t F, int64_t K)
{
    if (!pc || !ps || !x || !h)
        return Q4P_EINVAL;
    if (M <= 0 || M > (int64_t)1 << 24 || F <= 0 || F % 8 != 0 || F > ((int64_t)1 << 29) ||
        !shape_ok(2 * F, K))
        return Q4P_EINVAL;
    if ((uint64_t)M * (uint64_t)F > ((uint64_t)1 << 40))
        return Q4P_EINVAL;
    if (!aligned(pc, 16) || !aligned(ps, 8) || !aligned(x, 16) || !aligned(h, 2))
        return Q4P_EINVAL;
    const size_t hbytes = (size_t)M * (size_t)F * 2, xbytes = (size_t)M * (size_t)K * 2;
    if (overlap(h, hbytes, x, xbytes) || overlap(h, hbytes, pc, q4proj_packed_codes_bytes(2 * F, K)) ||
        overlap(h, hbytes, ps, q4proj_packed_scales_bytes(2 * F, K)))
        return Q4P_EINVAL;
    return Q4P_OK;
}

struct Span {
    const void *p;
    size_t n;
};

// The optional GEMM workspace: none (NULL) is fine; one that is given must
// be 16-byte aligned, hold q4proj_gemm_workspace_bytes(M, N, K) bytes and
// overlap no other argument.
q4proj_status check_gemm_workspace(const void *ws, size_t ws_bytes, int64_t M, int64_t N,
                                   int64_t K, std::initializer_list<Span> args)
{
    if (!ws)
        return Q4P_OK;
    const size_t need = q4p::gemm_workspace_bytes(M, K);
    (void)N;
    if (ws_bytes < need)
        return Q4P_EWORKSPACE;
    if (!aligned(ws, 16))
        return Q4P_EINVAL;
    for (const Span &a : args)
        if (overlap(ws, need, a.p, a.n))
            return Q4P_EINVAL;
    return Q4P_OK;
}

}  // namespace

extern "C" {

size_t q4proj_packed_codes_bytes(int64_t N, int64_t K)
{
    if (!shape_ok(N, K))
        return 0;
    return (size_t)(q4p::n_tiles(N) * q4p::k_tiles(K)) * q4p::kTileCodeBytes;
}

size_t q4proj_packed_scales_bytes(int64_t N, int64_t K)
{
    if (!shape_ok(N, K))
        return 0;
    return (size_t)(q4p::n_tiles(N) * q4p::k_tiles(K)) * q4p::kTileScaleBytes;
}

size_t q4proj_workspace_bytes(int64_t M, int64_t N, int64_t K)
{
    if (M <= 0 || M > Q4PROJ_GEMV_MAX_M || !shape_ok(N, K))
        return 0;
    return q4p::gemv_workspace_bytes(M, N, K);
}

q4proj_status q4proj_pack(const uint8_t *codes, const uint8_t *scales, int64_t N, int64_t K,
                          uint8_t *packed_codes, uint8_t *packed_scales, void *stream)
{
    if (!codes || !scales || !packed_codes || !packed_scales || !shape_ok(N, K))
        return Q4P_EINVAL;
    if (!aligned(codes, 8) || !aligned(packed_codes, 16) || !aligned(packed_scales, 8))
        return Q4P_EINVAL;
    const size_t pcb = q4proj_packed_codes_bytes(N, K), psb = q4proj_packed_scales_bytes(N, K);
    const size_t cb = (size_t)N * (size_t)(K / 2), sb = (size_t)N * (size_t)(K / 16);
    if (overlap(packed_codes, pcb, codes, cb) || overlap(packed_codes, pcb, scales, sb) ||
        overlap(packed_scales, psb, codes, cb) || overlap(packed_scales, psb, scales, sb) ||
        overlap(packed_codes, pcb, packed_scales, psb))
        return Q4P_EINVAL;
    q4proj_status st = check_device();
    if (st != Q4P_OK)
        return st;
    return record_hip(q4p::launch_pack(codes, scales, N, K, packed_codes, packed_scales,
                                       static_cast<hipStream_t>(stream)));
}

q4proj_status q4proj_pack_gate_up(const uint8_t *gate_codes, const uint8_t *gate_scales,
                                  const uint8_t *up_codes, const uint8_t *up_scales,
                                  float gate_global_scale, float up_global_scale, int64_t F,
                                  int64_t K, uint8_t *packed_codes, uint8_t *packed_scales,
                                  void *stream)
{
    if (!gate_codes || !gate_scales || !up_codes || !up_scales || !packed_codes || !packed_scales)
        return Q4P_EINVAL;
    // F is bounded before 2F is formed (no signed overflow for any F)
    if (F < 8 || F % 8 != 0 || F > ((int64_t)1 << 29) || !shape_ok(2 * F, K))
        return Q4P_EINVAL;
    // one global scale multiplies the fused projection: both halves need the
    // same one (bit for bit; a NaN never equals itself)
    if (!(gate_global_scale == up_global_scale) ||
        std::memcmp(&gate_global_scale, &up_global_scale, sizeof(float)) != 0)
        return Q4P_EINVAL;
    if (!aligned(gate_codes, 8) || !aligned(up_codes, 8) || !aligned(packed_codes, 16) ||
        !aligned(packed_scales, 8))
        return Q4P_EINVAL;
    const size_t pcb = q4proj_packed_codes_bytes(2 * F, K);
    const size_t psb = q4proj_packed_scales_bytes(2 * F, K);
    const size_t cb = (size_t)F * (size_t)(K / 2), sb = (size_t)F * (size_t)(K / 16);
    const void *in[4] = {gate_codes, gate_scales, up_codes, up_scales};
    const size_t inb[4] = {cb, sb, cb, sb};
    for (int i = 0; i < 4; ++i)
        if (overlap(packed_codes, pcb, in[i], inb[i]) || overlap(packed_scales, psb, in[i], inb[i]))
            return Q4P_EINVAL;
    if (overlap(packed_codes, pcb, packed_scales, psb))
        return Q4P_EINVAL;
    q4proj_status st = check_device();
    if (st != Q4P_OK)
        return st;
    return record_hip(q4p::launch_pack_gate_up(gate_codes, gate_scales, up_codes, up_scales, F, K,
                                               packed_codes, packed_scales,
                                               static_cast<hipStream_t>(stream)));
}

q4proj_status q4proj_unpack(const uint8_t *packed_codes, const uint8_t *packed_scales, int64_t N,
                            int64_t K, uint8_t *codes, uint8_t *scales, void *stream)
{
    if (!codes || !scales || !packed_codes || !packed_scales || !shape_ok(N, K))
        return Q4P_EINVAL;
    if (!aligned(codes, 8) || !aligned(packed_codes, 16) || !aligned(packed_scales, 8))
        return Q4P_EINVAL;
    const size_t pcb = q4proj_packed_codes_bytes(N, K), psb = q4proj_packed_scales_bytes(N, K);
    const size_t cb = (size_t)N * (size_t)(K / 2), sb = (size_t)N * (size_t)(K / 16);
    if (overlap(packed_codes, pcb, codes, cb) || overlap(packed_codes, pcb, scales, sb) ||
        overlap(packed_scales, psb, codes, cb) || overlap(packed_scales, psb, scales, sb) ||
        overlap(codes, cb, scales, sb))
        return Q4P_EINVAL;
    q4proj_status st = check_device();
    if (st != Q4P_OK)
        return st;
    return record_hip(q4p::launch_unpack(packed_codes, packed_scales, N, K, codes, scales,
                                         static_cast<hipStream_t>(stream)));
}

q4proj_status q4proj_gemv(const uint8_t *packed_codes, const uint8_t *packed_scales,
                          float global_scale, const uint16_t *x, float *y, int64_t M, int64_t N,
                          int64_t K, void *workspace, size_t workspace_bytes, void *stream)
{
    const size_t need = q4proj_workspace_bytes(M, N, K);
    q4proj_status st = check_projection(packed_codes, packed_scales, x, y, M, N, K,
                                        workspace_bytes, need);
    if (st != Q4P_OK)
        return st;
    if (M > Q4PROJ_GEMV_MAX_M)
        return Q4P_EUNSUPPORTED;
    if (need > 0 && (!workspace || !aligned(workspace, 8)))
        return Q4P_EINVAL;
    if (need > 0 && (overlap(workspace, need, y, (size_t)M * (size_t)N * sizeof(float)) ||
                     overlap(workspace, need, x, (size_t)M * (size_t)K * 2) ||
                     overlap(workspace, need, packed_codes, q4proj_packed_codes_bytes(N, K)) ||
                     overlap(workspace, need, packed_scales, q4proj_packed_scales_bytes(N, K))))
        return Q4P_EINVAL;
    st = check_device();
    if (st != Q4P_OK)
        return st;
    return record_hip(q4p::launch_gemv(packed_codes, packed_scales, global_scale, x, y, M, N, K,
                                       workspace, static_cast<hipStream_t>(stream)));
}

q4proj_status q4proj_gemv_noalloc(const uint8_t *packed_codes, const uint8_t *packed_scales,
                                  float global_scale, const uint16_t *x, float *y, int64_t M,
                                  int64_t N, int64_t K, void *stream)
{
    // the library's scratch array stands in for the workspace: a shape whose
    // exchange words do not fit is refused (EWORKSPACE) before any launch
    const size_t need = q4proj_workspace_bytes(M, N, K);
    q4proj_status st = check_projection(packed_codes, packed_scales, x, y, M, N, K,
                                        q4p::gemv_noalloc_max_bytes(), need);
    if (st != Q4P_OK)
        return st;
    if (M > Q4PROJ_GEMV_MAX_M)
        return Q4P_EUNSUPPORTED;
    st = check_device();
    if (st != Q4P_OK)
        return st;
    return record_hip(q4p::launch_gemv_noalloc(packed_codes, packed_scales, global_scale, x, y, M,
                                               N, K, static_cast<hipStream_t>(stream)));
}

size_t q4proj_silu_mul_workspace_bytes(int64_t M, int64_t F, int64_t K)
{
    if (M <= 0 || M > Q4PROJ_GEMV_MAX_M || F <= 0 || F % 8 != 0 || F > ((int64_t)1 << 29) ||
        !shape_ok(2 * F, K))
        return 0;
    return q4p::gemv_silu_mul_workspace_bytes(M, F, K);
}

q4proj_status q4proj_gemv_silu_mul(const uint8_t *packed_codes, const uint8_t *packed_scales,
                                   float global_scale, const uint16_t *x, uint16_t *h, int64_t M,
                                   int64_t F, int64_t K, void *workspace, size_t workspace_bytes,
                                   void *stream)
{
    q4proj_status st = check_silu_mul(packed_codes, packed_scales, x, h, M, F, K);
    if (st != Q4P_OK)
        return st;
    const int64_t N = 2 * F;
    const size_t hbytes = (size_t)M * (size_t)F * 2, xbytes = (size_t)M * (size_t)K * 2;
    const size_t pcb = q4proj_packed_codes_bytes(N, K), psb = q4proj_packed_scales_bytes(N, K);
    if (M > Q4PROJ_GEMV_MAX_M)
        return Q4P_EUNSUPPORTED;
    const size_t need = q4proj_silu_mul_workspace_bytes(M, F, K);
    if (need == 0)
        return Q4P_EUNSUPPORTED;
    if (workspace_bytes < need)
        return Q4P_EWORKSPACE;
    if (!workspace || !aligned(workspace, 8))
        return Q4P_EINVAL;
    if (overlap(workspace, need, h, hbytes) || overlap(workspace, need, x, xbytes) ||
        overlap(workspace, need, packed_codes, pcb) || overlap(workspace, need, packed_scales, psb))
        return Q4P_EINVAL;
    st = check_device();
    if (st != Q4P_OK)
        return st;
    return record_hip(q4p::launch_gemv_silu_mul(packed_codes, packed_scales, global_scale, x, h,
                                                M, F, K, workspace,
                                                static_cast<hipStream_t>(stream)));
}

q4proj_status q4proj_gemm_silu_mul(const uint8_t *packed_codes, const uint8_t *packed_scales,
                                   float global_scale, const uint16_t *x, uint16_t *h, int64_t M,
                                   int64_t F, int64_t K, void *workspace, size_t workspace_bytes,
                                   void *stream)
{
    q4proj_status st = check_silu_mul(packed_codes, packed_scales, x, h, M, F, K);
    if (st != Q4P_OK)
        return st;
    const int64_t N = 2 * F;
    st = check_gemm_workspace(workspace, workspace_bytes, M, N, K,
                              {{x, (size_t)M * (size_t)K * 2}, {h, (size_t)M * (size_t)F * 2},
                               {packed_codes, q4proj_packed_codes_bytes(N, K)},
                               {packed_scales, q4proj_packed_scales_bytes(N, K)}});
    if (st != Q4P_OK)
        return st;
    st = check_device();
    if (st != Q4P_OK)
        return st;
    return record_hip(q4p::launch_gemm_silu_mul(packed_codes, packed_scales, global_scale, x, h,
                                                M, F, K, workspace,
                                                static_cast<hipStream_t>(stream)));
}

size_t q4proj_argmax_workspace_bytes(int64_t M, int64_t N, int64_t K)
{
    if (M <= 0 || M > Q4PROJ_GEMV_MAX_M || !shape_ok(N, K))
        return 0;
    return q4p::gemv_argmax_workspace_bytes(M, N, K);
}

q4proj_status q4proj_gemv_argmax(const uint8_t *packed_codes, const uint8_t *packed_scales,
                                 float global_scale, const uint16_t *x, float *y,
                                 float *max_val, int64_t *max_idx, int64_t M, int64_t N,
                                 int64_t K, void *workspace, size_t workspace_bytes,
                                 void *stream)
{
    if (!packed_codes || !packed_scales || !x || !max_val || !max_idx)
        return Q4P_EINVAL;
    if (M <= 0 || M > (int64_t)1 << 24 || !shape_ok(N, K))
        return Q4P_EINVAL;
    if ((uint64_t)M * (uint64_t)N > ((uint64_t)1 << 40))
        return Q4P_EINVAL;
    if (!aligned(packed_codes, 16) || !aligned(packed_scales, 8) || !aligned(x, 16) ||
        (y && !aligned(y, 4)) || !aligned(max_val, 4) || !aligned(max_idx, 8))
        return Q4P_EINVAL;
    const size_t xb = (size_t)M * (size_t)K * 2, yb = (size_t)M * (size_t)N * 4;
    const size_t vb = (size_t)M * 4, ib = (size_t)M * 8;
    const size_t pcb = q4proj_packed_codes_bytes(N, K), psb = q4proj_packed_scales_bytes(N, K);
    const void *outs[3] = {y, max_val, max_idx};
    const size_t outb[3] = {yb, vb, ib};
    for (int i = 0; i < 3; ++i) {
        if (!outs[i])
            continue;
        if (overlap(outs[i], outb[i], x, xb) || overlap(outs[i], outb[i], packed_codes, pcb) ||
            overlap(outs[i], outb[i], packed_scales, psb))
            return Q4P_EINVAL;
        for (int j = i + 1; j < 3; ++j)
            if (outs[j] && overlap(outs[i], outb[i], outs[j], outb[j]))
                return Q4P_EINVAL;
    }
    if (M > Q4PROJ_GEMV_MAX_M)
        return Q4P_EUNSUPPORTED;
    const size_t need = q4proj_argmax_workspace_bytes(M, N, K);
    if (need == 0)
        return Q4P_EUNSUPPORTED;
    if (workspace_bytes < need)
        return Q4P_EWORKSPACE;
    if (!workspace || !aligned(workspace, 8))
        return Q4P_EINVAL;
    if (overlap(workspace, need, x, xb) || overlap(workspace, need, packed_codes, pcb) ||
        overlap(workspace, need, packed_scales, psb))
        return Q4P_EINVAL;
    for (int i = 0; i < 3; ++i)
        if (outs[i] && overlap(workspace, need, outs[i], outb[i]))
            return Q4P_EINVAL;
    q4proj_status st = check_device();
    if (st != Q4P_OK)
        return st;
    return record_hip(q4p::launch_gemv_argmax(packed_codes, packed_scales, global_scale, x, y,
                                              max_val, max_idx, M, N, K, workspace,
                                              static_cast<hipStream_t>(stream)));
}

size_t q4proj_quantize_workspace_bytes(int64_t N, int64_t K)
{
    return shape_ok(N, K) ? q4p::quant_workspace_bytes() : 0;
}

q4proj_status q4proj_quantize(const uint16_t *w, int64_t N, int64_t K, uint8_t *codes,
                              uint8_t *scales, float *global_scale, void *workspace,
                              size_t workspace_bytes, void *stream)
{
    if (!w || !codes || !scales || !global_scale || !shape_ok(N, K))
        return Q4P_EINVAL;
    if (!aligned(w, 16) || !aligned(codes, 8) || !aligned(global_scale, 4))
        return Q4P_EINVAL;
    const size_t wb = (size_t)N * (size_t)K * 2, cb = (size_t)N * (size_t)(K / 2),
                 sb = (size_t)N * (size_t)(K / 16);
    if (overlap(codes, cb, w, wb) || overlap(scales, sb, w, wb) || overlap(codes, cb, scales, sb) ||
        overlap(global_scale, 4, w, wb) || overlap(global_scale, 4, codes, cb) ||
        overlap(global_scale, 4, scales, sb))
        return Q4P_EINVAL;
    const size_t need = q4proj_quantize_workspace_bytes(N, K);
    if (workspace_bytes < need)
        return Q4P_EWORKSPACE;
    if (!workspace || !aligned(workspace, 4))
        return Q4P_EINVAL;
    if (overlap(workspace, need, w, wb) || overlap(workspace, need, codes, cb) ||
        overlap(workspace, need, scales, sb) || overlap(workspace, need, global_scale, 4))
        return Q4P_EINVAL;
    q4proj_status st = check_device();
    if (st != Q4P_OK)
        return st;
    return record_hip(q4p::launch_quantize(w, N, K, codes, scales, global_scale, workspace,
                                           static_cast<hipStream_t>(stream)));
}

size_t q4proj_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K)
{
    if (M <= 0 || M > (int64_t)1 << 24 || !shape_ok(N, K))
        return 0;
    return q4p::gemm_workspace_bytes(M, K);
}

q4proj_status q4proj_gemm(const uint8_t *packed_codes, const uint8_t *packed_scales,
                          float global_scale, const uint16_t *x, float *y, int64_t M, int64_t N,
                          int64_t K, void *workspace, size_t workspace_bytes, void *stream)
{
    q4proj_status st = check_projection(packed_codes, packed_scales, x, y, M, N, K,
                                        workspace_bytes, 0);
    if (st != Q4P_OK)
        return st;
    st = check_gemm_workspace(workspace, workspace_bytes, M, N, K,
                              {{x, (size_t)M * (size_t)K * 2},
                               {y, (size_t)M * (size_t)N * sizeof(float)},
                               {packed_codes, q4proj_packed_codes_bytes(N, K)},
                               {packed_scales, q4proj_packed_scales_bytes(N, K)}});
    if (st != Q4P_OK)
        return st;
    st = check_device();
    if (st != Q4P_OK)
        return st;
    return record_hip(q4p::launch_gemm(packed_codes, packed_scales, global_scale, x, y, M, N, K,
                                       workspace, static_cast<hipStream_t>(stream)));
}

const char *q4proj_status_string(q4proj_status s)
{
    switch (s) {
    case Q4P_OK: return "Q4P_OK";
    case Q4P_EINVAL: return "Q4P_EINVAL: invalid argument";
    case Q4P_EUNSUPPORTED: return "Q4P_EUNSUPPORTED: arguments outside this entry point's range";
    case Q4P_EDEVICE: return "Q4P_EDEVICE: current device is not gfx950";
    case Q4P_EWORKSPACE: return "Q4P_EWORKSPACE: workspace too small";
    case Q4P_EHIP: return "Q4P_EHIP: HIP runtime error";
    }
    return "unknown q4proj_status";
}

const char *q4proj_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
