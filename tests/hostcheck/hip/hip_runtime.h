// Stand-in for <hip/hip_runtime.h> in the CPU build of the library's host
// front (nvfp4_weight_only_q4proj_amd/csrc/q4p_api.cpp) under AddressSanitizer
// and UndefinedBehaviorSanitizer: the types and the three runtime calls that
// file makes.  stubs.cpp implements them and the kernel launchers, recording
// each launch instead of touching a GPU.  Test infrastructure only; never
// part of the library build.
#pragma once

#include <stddef.h>
#include <stdint.h>

typedef enum hipError_t {
    hipSuccess = 0,
    hipErrorInvalidValue = 1,
    hipErrorNoDevice = 100,
    hipErrorLaunchFailure = 719,
} hipError_t;

typedef struct ihipStream_t *hipStream_t;

typedef struct hipDeviceProp_t {
    char name[256];
    char gcnArchName[256];
} hipDeviceProp_t;

#ifdef __cplusplus
extern "C" {
#endif
hipError_t hipGetDevice(int *device);
hipError_t hipGetDeviceProperties(hipDeviceProp_t *prop, int device);
const char *hipGetErrorString(hipError_t error);
#ifdef __cplusplus
}
#endif
