// Host-only stand-in for the few HIP runtime declarations that the attention
// library's C ABI layer (csrc/api.cpp) uses, for its sanitizer build on the
// CPU: "device" memory is host memory and copies are memcpy.  Definitions are
// in tests/host_abi_driver.cpp.
#pragma once
#include <cstddef>

typedef enum hipError_t { hipSuccess = 0, hipErrorInvalidValue = 1, hipErrorLaunchFailure = 719 } hipError_t;
typedef struct ihipStream_t* hipStream_t;
typedef enum hipMemcpyKind {
  hipMemcpyHostToHost = 0,
  hipMemcpyHostToDevice = 1,
  hipMemcpyDeviceToHost = 2,
  hipMemcpyDeviceToDevice = 3,
  hipMemcpyDefault = 4
} hipMemcpyKind;

typedef enum hipDeviceAttribute_t { hipDeviceAttributeMultiprocessorCount = 63 } hipDeviceAttribute_t;

hipError_t hipGetDevice(int* device);
hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t attr, int device);
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t bytes, hipMemcpyKind kind, hipStream_t stream);
hipError_t hipStreamSynchronize(hipStream_t stream);
const char* hipGetErrorString(hipError_t e);
