// Host-only stand-in for <hip/hip_runtime_api.h>, used when the C ABI
// (api.cpp) is compiled by g++ for the sanitizer build: the entry points need
// only the status and stream types of the runtime.
#pragma once
typedef enum hipError_t { hipSuccess = 0, hipErrorInvalidValue = 1 } hipError_t;
typedef struct ihipStream_t *hipStream_t;
