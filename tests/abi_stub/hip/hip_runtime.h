/* Minimal stand-in for <hip/hip_runtime.h>, used only to build the C ABI's host code
 * (argument checks, workspace layouts, tile and grid arithmetic) for the CPU under
 * AddressSanitizer and UndefinedBehaviorSanitizer. The HIP calls that host code makes
 * are declared here and defined by the test driver; no kernel is built. */
#pragma once
#include <stddef.h>
#include <stdint.h>

typedef int hipError_t;
enum { hipSuccess = 0, hipErrorInvalidValue = 1 };
typedef struct ihipStream_t *hipStream_t;
typedef struct ihipEvent_t *hipEvent_t;

#define __device__
#define __align__(n) __attribute__((aligned(n)))
#define HIP_SYMBOL(s) ((const void *)&(s))

hipError_t hipGetDevice(int *device);
hipError_t hipGetSymbolAddress(void **devPtr, const void *symbol);
hipError_t hipEventRecord(hipEvent_t event, hipStream_t stream);
