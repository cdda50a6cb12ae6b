// Streaming-read probe for gfx950: a measurement aid beside the decode
// kernels (the first page, TensorRT-LLM concept page, "key performance
// parameters", ties decode throughput to memory bandwidth; this kernel gives
// the rate a plain read of the same kind reaches on the device).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_internal.h"
#include "pkv_device.h"

namespace pkv {

// ---------------------------------------------------------------------------
// Read probe: every byte of a buffer once, as 16-byte nontemporal loads (the
// access the decode's K/V stream uses), with nothing else to do, to measure
// the streaming-read rate the decode is compared with.  Like the decode, each
// wave streams one contiguous share of the buffer, 1 KB per load instruction
// and 8 loads in flight per lane.  The loaded words are folded into one value,
// stored only if it equals a constant no real data is expected to give, so
// the loads are not dropped and almost nothing is written.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void read_probe_kernel(const uint8_t* __restrict__ buf, size_t n16,
                                                         uint32_t* __restrict__ out) {
  constexpr int U = 8;
  const int lane = threadIdx.x & 63;
  const size_t nw = (size_t)gridDim.x * 4;
  const size_t w = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const size_t per = ((n16 + nw - 1) / nw + 63) & ~(size_t)63;   // whole 1 KB rows per wave
  const size_t v0 = w * per, v1 = min(v0 + per, n16);
  uint32_t acc = 0;
  size_t v = v0;
  for (; v + 64 * U <= v1; v += 64 * U) {
    u32x4_t x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = ld16_stream(buf + 16 * (v + 64 * u + lane));
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= x[u][0] ^ x[u][1] ^ x[u][2] ^ x[u][3];
  }
  for (v += lane; v < v1; v += 64) {
    const u32x4_t x = ld16_stream(buf + 16 * v);
    acc ^= x[0] ^ x[1] ^ x[2] ^ x[3];
  }
  if (acc == 0x9E3779B9u) out[0] = acc;
}

hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* out, hipStream_t s) {
  const int cus = device_cu_count();
  if (cus <= 0) return hipErrorInvalidDevice;
  if (bytes < 16) return hipSuccess;
  // 8 waves per compute unit; the last wave's share is cut at the end
  hipLaunchKernelGGL(read_probe_kernel, dim3(2 * cus), dim3(256), 0, s, static_cast<const uint8_t*>(buf),
                     bytes / 16, out);
  return hipGetLastError();
}

}  // namespace pkv
