// bench_kernels.hip -- measurement ceilings for the benchmark harness
// (declared in include/q4k_bench.h): an empty kernel (launch floor) and a
// plain streaming read and copy over caller buffers (achievable HBM rate,
// and the calibration of the HBM byte counters).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q4k_bench.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ void empty_kernel() {}

// One wave that waits until `ticks` periods of the constant-rate real-time
// counter have passed.  The wait is bounded by an iteration count as well,
// so the kernel ends even if the counter were not advancing.
__global__ void delay_kernel(uint64_t ticks) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (uint32_t i = 0; i < (1u << 22); ++i) {
    if (__builtin_amdgcn_s_memrealtime() - t0 >= ticks) break;
    __builtin_amdgcn_s_sleep(4);
  }
}

// Reads n16 16-byte words with grid-stride non-temporal loads and writes one
// word per workgroup so the reads cannot be elided.
__global__ __launch_bounds__(256) void stream_read_kernel(
    const u32x4 *__restrict__ src, int64_t n16, uint32_t *__restrict__ sink) {
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  __shared__ uint32_t red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int k = 0; k < 256; ++k) t ^= red[k];
    sink[blockIdx.x] = t;
  }
}

__global__ __launch_bounds__(256) void copy_kernel(const uint4 *__restrict__ src,
                                                   uint4 *__restrict__ dst,
                                                   int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    dst[i] = src[i];
}

}  // namespace

extern "C" {

int q4k_bench_empty(void *stream) {
  hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int q4k_bench_delay(int64_t ns, void *stream) {
  if (ns < 0 || ns > 100000000) return -1;
  // the real-time counter runs at 100 MHz on this part: 10 ns per tick
  hipLaunchKernelGGL(delay_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream,
                     (uint64_t)(ns / 10));
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int q4k_bench_stream_read(const void *src, int64_t nbytes, uint32_t *sink,
                          int64_t sink_words, void *stream) {
  if (nbytes <= 0 || nbytes % 16 != 0 || sink_words <= 0) return -1;
  if (!src || !sink) return -2;
  if (((uintptr_t)src & 15u) != 0) return -3;
  const int64_t n16 = nbytes / 16;
  int64_t grid = (n16 + 255) / 256;
  if (grid > sink_words) grid = sink_words;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(256), 0,
                     (hipStream_t)stream, (const u32x4 *)src, n16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int q4k_bench_copy(const void *src, void *dst, int64_t nbytes, void *stream) {
  if (nbytes <= 0 || nbytes % 16 != 0) return -1;
  if (!src || !dst) return -2;
  if (((uintptr_t)src & 15u) != 0 || ((uintptr_t)dst & 15u) != 0) return -3;
  const int64_t n16 = nbytes / 16;
  int64_t grid = (n16 + 255) / 256;
  if (grid > 65536) grid = 65536;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)grid), dim3(256), 0,
                     (hipStream_t)stream, (const uint4 *)src, (uint4 *)dst, n16);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
