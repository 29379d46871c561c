// Measurement helpers (not part of the LoopVQ ABI): a plain device-to-device
// copy and a plain streaming read, both with 16-byte accesses per lane, built
// into libloopvq_calib.so.  The benchmark times them to give the HBM stream
// rates of this device, and the hardware byte counters (FETCH_SIZE,
// WRITE_SIZE) read on them give the scale that turns the counters of the
// LoopVQ kernels into bytes.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace loopvq_calib {

__global__ __launch_bounds__(256) void calib_copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                         uint64_t n16) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

__global__ __launch_bounds__(256) void calib_read_kernel(const uint4* __restrict__ src, uint64_t n16,
                                                         uint32_t* __restrict__ sink) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // one word per thread keeps the loads live; the sink holds gridDim.x * 256 words
  sink[(uint64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

int grid_for(uint64_t n16) {
  const uint64_t want = (n16 + 255) / 256;
  return (int)(want < 8192 ? (want ? want : 1) : 8192);
}

}  // namespace loopvq_calib

using namespace loopvq_calib;

extern "C" {

// Copies `bytes` (a multiple of 16; both pointers 16-byte aligned) from src to
// dst on `stream`.  Returns 0, or -1 for bad arguments, -3 for a launch error.
int loopvq_calib_copy(const void* src, void* dst, uint64_t bytes, void* stream) {
  if (!src || !dst || bytes % 16 || reinterpret_cast<uintptr_t>(src) % 16 || reinterpret_cast<uintptr_t>(dst) % 16)
    return -1;
  const uint64_t n16 = bytes / 16;
  hipLaunchKernelGGL(calib_copy_kernel, dim3(grid_for(n16)), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(src), static_cast<uint4*>(dst), n16);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

// Number of uint32 words the sink of loopvq_calib_read must hold for `bytes`.
uint64_t loopvq_calib_read_sink_words(uint64_t bytes) { return (uint64_t)grid_for(bytes / 16) * 256; }

// Reads `bytes` (a multiple of 16, src 16-byte aligned) and writes one word
// per thread to sink.  Returns 0, -1 for bad arguments, -3 for a launch error.
int loopvq_calib_read(const void* src, uint64_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink || bytes % 16 || reinterpret_cast<uintptr_t>(src) % 16) return -1;
  const uint64_t n16 = bytes / 16;
  hipLaunchKernelGGL(calib_read_kernel, dim3(grid_for(n16)), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(src), n16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // extern "C"
