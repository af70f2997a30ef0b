// Host-only stand-in for <hip/hip_runtime.h>, used when the scheduler header
// and the C ABI are compiled by g++ for the sanitizer build: the scheduler
// needs only the function qualifiers, which mean nothing on the host, and the
// C ABI the runtime's status and stream types.
#pragma once
#define __host__
#define __device__
#include "hip_runtime_api.h"
