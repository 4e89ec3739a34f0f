/* Control of the CPU stand-ins behind the host front's CPU build (see
 * stubs.cpp): the current device and its architecture, the error the next
 * launch returns, the sizes the sizing functions report, and a record of the
 * last launch.  Test infrastructure only. */
#pragma once

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct stub_launch {
    int count;                /* launches since stub_reset() */
    char name[32];            /* launcher of the last launch, e.g. "gemv" */
    int64_t M, N, K;          /* its sizes (N: F for the gate/up entries) */
    const void *in0, *in1;    /* its first two buffer arguments */
    void *out, *workspace;    /* its output and workspace (or NULL) */
    void *stream;             /* the stream it was given */
    float g;                  /* its global scale (0 where none) */
} stub_launch;

void stub_reset(void);
/* hipGetDevice reports `device` (rc != 0: fails with that error) */
void stub_set_device(int device, int rc);
/* hipGetDeviceProperties reports this architecture for `device` */
void stub_set_arch(int device, const char *arch);
/* the next launches return this HIP error (0: success) */
void stub_set_launch_error(int error);
/* values of the library's sizing functions */
void stub_set_sizes(size_t gemv_ws, size_t silu_ws, size_t argmax_ws, size_t quant_ws,
                    size_t noalloc_max, int silu_supported, int argmax_supported);
/* number of hipGetDeviceProperties calls since stub_reset() */
int stub_props_calls(void);
const stub_launch *stub_last(void);

#ifdef __cplusplus
}
#endif
