// Indexer logits on the FP8 matrix cores, for measuring their summation error (benchmark
// library only; the decode path scores on bf16 MFMA).  The pages' indexer scores FP8 keys
// against FP8 queries (vLLM blog, section "Kernels", sparse MQA logits); this kernel takes the
// E4M3 bytes of both as stored and forms logits[h][j] = sum_d q[h][d] * k[j][d] over Di = 128
// dims on one of two gfx950 instruction forms:
//   form 0: v_mfma_scale_f32_16x16x128_f8f6f4 with unit scales (E8M0 127), one instruction
//           per 16 heads x 16 positions covering all 128 dims;
//   form 1: v_mfma_f32_16x16x32_fp8_fp8, four instructions accumulating 32 dims each.
// Every product of two E4M3 values is exact in fp32; what differs from an exact dot product
// is how the instruction adds them.  Lane (g, n) of a wave supplies, for head row n of A and
// position column n of B, the same 32 dims in both operands (form 0: dims 32 g .. 32 g + 31;
// form 1, instruction s: dims 32 s + 8 g .. + 7), so every product pairs the right q and k
// bytes whatever order the instruction assigns to them.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

template <int FORM>
__global__ __launch_bounds__(64) void fp8_logits_kernel(const uint8_t* __restrict__ q, const uint8_t* __restrict__ k,
                                                        int32_t N, float* __restrict__ out) {
  const int lane = threadIdx.x, g = lane >> 4, n = lane & 15;
  const int pt = blockIdx.x, ht = blockIdx.y;
  const uint8_t* qr = q + (int64_t)(16 * ht + n) * 128;
  const uint8_t* kr = k + (int64_t)(16 * pt + n) * 128;
  v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
  if constexpr (FORM == 0) {
    const v4u a0 = *(const v4u*)(qr + 32 * g), a1 = *(const v4u*)(qr + 32 * g + 16);
    const v4u b0 = *(const v4u*)(kr + 32 * g), b1 = *(const v4u*)(kr + 32 * g + 16);
    const v8i a = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
    const v8i b = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 0, 0, 127, 0, 127);
  } else {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const long a = *(const long*)(qr + 32 * s + 8 * g);
      const long b = *(const long*)(kr + 32 * s + 8 * g);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, acc, 0, 0, 0);
    }
  }
  // C layout: lane (g, n) holds rows 4 g .. 4 g + 3 (heads) of column n (position)
#pragma unroll
  for (int r = 0; r < 4; ++r) out[(int64_t)(16 * ht + 4 * g + r) * N + 16 * pt + n] = acc[r];
}

}  // namespace

// logits [H][N] fp32 from q_e4m3 [H][128] and k_e4m3 [N][128] (E4M3 bytes, device memory) on
// the FP8 matrix cores in `form` (0 or 1, above).  H and N must be positive multiples of 16.
// Returns 0, -1 for an unsupported argument, or the HIP error of the launch.
extern "C" int smqa_bench_fp8_mfma_logits(const void* q_e4m3, const void* k_e4m3, int32_t H, int32_t N,
                                          float* logits, int32_t form, void* stream) {
  if (!q_e4m3 || !k_e4m3 || !logits || H <= 0 || N <= 0 || H % 16 || N % 16 || (form != 0 && form != 1))
    return -1;
  const hipStream_t s = (hipStream_t)stream;
  const dim3 grid(N / 16, H / 16);
  const uint8_t* q = (const uint8_t*)q_e4m3;
  const uint8_t* k = (const uint8_t*)k_e4m3;
  if (form == 0)
    hipLaunchKernelGGL(fp8_logits_kernel<0>, grid, dim3(64), 0, s, q, k, N, logits);
  else
    hipLaunchKernelGGL(fp8_logits_kernel<1>, grid, dim3(64), 0, s, q, k, N, logits);
  return (int)hipGetLastError();
}
