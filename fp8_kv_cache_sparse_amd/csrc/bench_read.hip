// Streaming-read reference for the benchmark (not part of the decode path; built into its
// own library, libsmqa_bench.so).  It measures what a plain read of a large buffer reaches
// on the device at hand, so the score stage's bandwidth can be set against a ceiling that
// was measured the same way (cold caches, HIP events) instead of only against the data
// sheet's peak.
//
// Each thread reads 16-byte words with non-temporal loads, `depth` independent loads per
// iteration at a stride of one grid, and folds them into one word it stores at the end (so
// no load can be dropped).  The host picks the grid (workgroups of 256 threads) and depth.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef unsigned v4u __attribute__((ext_vector_type(4)));

template <int DEPTH>
__global__ __launch_bounds__(256) void stream_read_kernel(const v4u* __restrict__ p, int64_t n16,
                                                          unsigned* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  unsigned acc = 0u;
  for (; i + (DEPTH - 1) * stride < n16; i += DEPTH * stride) {
    v4u v[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) v[d] = __builtin_nontemporal_load(p + i + d * stride);
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) acc ^= v[d].x ^ v[d].y ^ v[d].z ^ v[d].w;
  }
  for (; i < n16; i += stride) {
    const v4u v = __builtin_nontemporal_load(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

}  // namespace

// Read `bytes` (a multiple of 16) from device memory at `src` with `grid` workgroups of 256
// threads and `depth` loads in flight per thread (1, 2, 4, 8 or 16); `out` takes grid * 256
// words.  Returns 0, or -1 for an unsupported argument, or the HIP error of the launch.
extern "C" int smqa_bench_stream_read(const void* src, int64_t bytes, void* out, int32_t grid,
                                      int32_t depth, void* stream) {
  if (src == nullptr || out == nullptr || bytes <= 0 || bytes % 16 != 0 || grid <= 0) return -1;
  const int64_t n16 = bytes / 16;
  const hipStream_t s = (hipStream_t)stream;
  const v4u* p = (const v4u*)src;
  unsigned* o = (unsigned*)out;
  switch (depth) {
    case 1: hipLaunchKernelGGL(stream_read_kernel<1>, dim3(grid), dim3(256), 0, s, p, n16, o); break;
    case 2: hipLaunchKernelGGL(stream_read_kernel<2>, dim3(grid), dim3(256), 0, s, p, n16, o); break;
    case 4: hipLaunchKernelGGL(stream_read_kernel<4>, dim3(grid), dim3(256), 0, s, p, n16, o); break;
    case 8: hipLaunchKernelGGL(stream_read_kernel<8>, dim3(grid), dim3(256), 0, s, p, n16, o); break;
    case 16: hipLaunchKernelGGL(stream_read_kernel<16>, dim3(grid), dim3(256), 0, s, p, n16, o); break;
    default: return -1;
  }
  return (int)hipGetLastError();
}
