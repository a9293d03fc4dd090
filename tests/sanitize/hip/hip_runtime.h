/* Host-only stand-in for <hip/hip_runtime.h>, used by the sanitizer build of the ABI layer's
 * argument checks (tests/test_sanitizers.py).  The ABI layer needs only these three names from
 * the HIP runtime; the kernel launchers it calls are replaced by launch_stubs.cpp. */
#pragma once
typedef int hipError_t;
typedef struct ihipStream_t* hipStream_t;
enum { hipSuccess = 0, hipErrorInvalidValue = 1 };
