// Bandwidth reference for the measurements: a plain streaming read of a device
// buffer, with no arithmetic beyond an XOR that keeps the loads alive.  Timing
// it over a large buffer gives the HBM read rate the chip attains in practice;
// timing it over the bytes of one expert-FFN launch gives the rate a single
// launch of that size can reach.  Holds no arithmetic of the MoE layer.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;  // 16-byte loads in flight per thread per pass

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4* __restrict__ p, int64_t n16,
                                                                uint32_t* sink) {
  const int64_t pass = (int64_t)gridDim.x * kThreads * kUnroll;
  uint32_t acc = 0;
  for (int64_t base = (int64_t)blockIdx.x * kThreads * kUnroll + threadIdx.x; base < n16; base += pass) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + (int64_t)u * kThreads;
      v[u] = i < n16 ? p[i] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  // a store that practically never happens; the loads cannot be dropped
  if (acc == 0x9E3779B9u && threadIdx.x == 0) sink[blockIdx.x & 1023] = acc;
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16) from the 16-byte aligned device buffer `p`
// with `grid` workgroups (0: one workgroup per 32 KiB, at most 8192).  `sink`
// is a device buffer of 1024 uint32 that is written only in the improbable
// case that the XOR of the data equals a fixed constant.  With start/stop
// events (may be null) the launch is bracketed by hipExtLaunchKernel events.
// Returns 0, -1 for bad arguments, -2 for a HIP launch error.
int synth_stream_read(const void* p, size_t bytes, int grid, uint32_t* sink, void* stream, void* start,
                      void* stop) {
  if (!p || !sink || bytes % 16 || ((uintptr_t)p & 15u) || grid < 0) return -1;
  if (bytes == 0) return 0;
  const int64_t n16 = (int64_t)(bytes / 16);
  if (grid == 0) {
    const int64_t g = (n16 + kThreads * kUnroll - 1) / (kThreads * kUnroll);
    grid = (int)(g > 8192 ? 8192 : g);
  }
  hipExtLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream,
                        (hipEvent_t)start, (hipEvent_t)stop, 0, reinterpret_cast<const uint4*>(p), n16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"
