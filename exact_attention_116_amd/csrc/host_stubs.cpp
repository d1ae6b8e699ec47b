// Host-only stand-ins for the HIP runtime calls and the kernel launchers that
// the C-ABI layer (fa_api.cpp) makes, for a CPU build of that layer under
// AddressSanitizer (no GPU, no device code).  Allocations are host memory;
// launchers do nothing and succeed.  hipMalloc and hipFree report each call
// on stderr so that a test can see the library-owned workspace released when
// the library is unloaded.  Never part of libfa.so.
#include <hip/hip_runtime_api.h>

#include <cstdio>
#include <cstdlib>

#include "fa_internal.h"

extern "C" {

hipError_t hipGetDevice(int* device) {
  *device = 0;
  return hipSuccess;
}

hipError_t hipSetDevice(int device) { return device == 0 ? hipSuccess : hipErrorInvalidDevice; }

hipError_t hipMalloc(void** ptr, size_t size) {
  *ptr = std::malloc(size);
  std::fprintf(stderr, "stub hipMalloc %zu -> %p\n", size, *ptr);
  return *ptr ? hipSuccess : hipErrorOutOfMemory;
}

hipError_t hipFree(void* ptr) {
  std::fprintf(stderr, "stub hipFree %p\n", ptr);
  std::free(ptr);
  return hipSuccess;
}

hipError_t hipDeviceSynchronize(void) { return hipSuccess; }

const char* hipGetErrorString(hipError_t) { return "stub HIP error"; }

}  // extern "C"

namespace fa {

hipError_t launch_fwd_bf16(const FwdArgs&) { return hipSuccess; }
hipError_t launch_fwd_fp8(const FwdArgs&) { return hipSuccess; }
hipError_t launch_fp8_quant(const QuantArgs&) { return hipSuccess; }
hipError_t launch_bwd(const BwdArgs&) { return hipSuccess; }
hipError_t launch_decode(const DecodeArgs&) { return hipSuccess; }
hipError_t launch_decode_gqa(const DecodeArgs&) { return hipSuccess; }
hipError_t launch_decode_combine(const DecodeArgs&) { return hipSuccess; }

hipError_t decode_scratch(void** ptr) {
  static unsigned char host_scratch[256];   // never written: the launchers are stubs
  *ptr = host_scratch;
  return hipSuccess;
}

}  // namespace fa
