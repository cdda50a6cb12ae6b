// Host-only stand-ins for the device side of libpkv.so, so that the C-ABI
// layer (pkv_api.cpp: argument validation, workspace sizing, dispatch) can be
// built with g++ under AddressSanitizer / UndefinedBehaviorSanitizer and
// driven by the CPU ABI tests.  Test infrastructure only: every launcher
// reports that no device is present, as the real library does on a machine
// without a GPU, and nothing here is part of the product library.
#include <hip/hip_runtime_api.h>

#include "pkv_internal.h"

extern "C" const char* hipGetErrorString(hipError_t) { return "no device (host-only test build)"; }

namespace pkv {
int device_cu_count() { return -1; }
hipError_t static_scratch(void** ptr) {
  *ptr = nullptr;
  return hipErrorNoDevice;
}
hipError_t launch_alloc_pages(const PageArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_release_pages(const PageArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_append(const AppendArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_append_chunk(const AppendChunkArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_prefill(const PrefillArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_append_quant(const AppendQuantArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_gather(const GatherArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_read_probe(const void*, size_t, uint32_t*, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decode(const DecodeArgs&, hipStream_t) { return hipErrorNoDevice; }
}  // namespace pkv
