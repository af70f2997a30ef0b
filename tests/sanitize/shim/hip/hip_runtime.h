// Host-only stand-in for <hip/hip_runtime.h>, used when the scheduler header
// is compiled by g++ for the sanitizer build: the scheduler needs only the
// function qualifiers, which mean nothing on the host.
#pragma once
#define __host__
#define __device__
