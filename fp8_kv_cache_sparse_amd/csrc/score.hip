// Indexer scoring on gfx950 (vLLM blog "DeepSeek-V4.1-Flash sur vLLM", section
// "Kernels", paragraph "Logits MQA creux": one score per context position, or per
// candidate position for the late indexer layers).
//
//   S[t, j] = sum_h w[t,h] * max(0, kappa_j * <qI[t,h], kI[j]>)
//
// The [heads x Di] x [Di x positions] contraction runs on bf16 MFMA 16x16x32 with
// fp32 accumulation: E4M3 -> bf16 is exact (v_cvt_scalef32_pk_bf16_fp8), so every
// product is exact and only the fp32 sums round.  (gfx950's FP8 MFMA forms add the
// products of one instruction with about 2^-17 of sum|q_d k_d| of error, too coarse
// for scores that must hold 1e-4 relative accuracy when heads nearly cancel.)
// Heads sit on the M dimension so each lane ends with 4 heads of one position; the
// ReLU-weighted head reduction is done in registers plus two cross-lane exchanges.
//
// Work split: a workgroup owns a block of positions of one sequence (dense mode)
// or of one query's candidate list, keeps those keys in registers (converted once),
// and loops over the queries of that sequence, so keys are read from HBM once per
// sequence even when many queries share it (bounded replay).  Each lane loads
// Di/4 contiguous key bytes per position (16-byte loads).
#include "common.h"

namespace smqa {

constexpr int kScoreThreads = 256;

// 8 E4M3 bytes (two dwords, byte i = element i) -> 8 exact bf16 values.
__device__ __forceinline__ v8bf fp8x8_to_bf16(unsigned w0, unsigned w1) {
  v4u u;
  u.x = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false));
  u.y = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true));
  u.z = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false));
  u.w = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true));
  return __builtin_bit_cast(v8bf, u);
}
constexpr int kQRow = 144;   // LDS bytes per head row (128 + 16 pad: conflict-free b128 reads)

template <int MT, int TPW, bool CAND>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(ScoreArgs a) {
  __shared__ __align__(16) uint8_t q_lds[16 * MT * kQRow];
  __shared__ float w_lds[16 * MT];
  __shared__ int s_pmax;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, g = lane >> 4, n = lane & 15;
  constexpr int kPosPerWave = 16 * TPW;
  constexpr int kPosPerWG = 4 * kPosPerWave;
  const int Di = a.Di, Hi = a.Hi;

  int b, t0, t1;
  if (CAND) {
    t0 = blockIdx.y;
    t1 = t0 + 1;
    b = seq_of_query(a.q_start, a.B, t0);
  } else {
    b = blockIdx.y;
    t0 = a.q_start[b];
    t1 = a.q_start[b + 1];
  }
  const int64_t base = a.seq_start[b];
  const int len = (int)(a.seq_start[b + 1] - base);
  const int col0 = blockIdx.x * kPosPerWG;
  if (CAND) {
    if (col0 >= a.n_cand) return;
  } else {
    if (col0 >= len || t0 >= t1) return;
    if (tid == 0) s_pmax = -1;
    __syncthreads();
    int pm = -1;
    for (int t = t0 + tid; t < t1; t += kScoreThreads) pm = max(pm, a.q_pos[t]);
    if (pm >= 0) atomicMax(&s_pmax, pm);
    __syncthreads();
    if (col0 > s_pmax) return;
  }

  // ---- this wave's keys (B operands), loaded and converted to bf16 once ----
  // Lane (g, n) holds position n of the tile and key bytes [g*Di/4, (g+1)*Di/4);
  // K-step s uses bytes g*Di/4 + 8s .. +8.  q uses the same byte->k assignment, so
  // the sum over k is the full dot product.
  constexpr int NKS_MAX = 4;
  const int nks = Di / 32;
  v8bf kb[TPW][NKS_MAX];
  float kap[TPW];
  int kpos[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int col = col0 + wave * kPosPerWave + 16 * i + n;
    int pos;
    bool ok;
    if (CAND) {
      ok = col < a.n_cand;
      pos = ok ? a.cand[(int64_t)t0 * a.n_cand + col] : -1;
      ok = ok && pos >= 0 && pos < len;
    } else {
      pos = col;
      ok = col < len;
    }
    kpos[i] = ok ? pos : -1;
    v4u lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
    if (ok) {
      const uint8_t* row = a.k_fp8 + (base + pos) * Di + g * (Di / 4);
      lo = *(const v4u*)row;
      if (Di == 128) hi = *(const v4u*)(row + 16);
    }
    const unsigned wds[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
    for (int s2 = 0; s2 < NKS_MAX; ++s2) kb[i][s2] = fp8x8_to_bf16(wds[2 * s2], wds[2 * s2 + 1]);
    kap[i] = (ok && a.k_scale) ? a.k_scale[base + pos] : 1.0f;
  }

  for (int t = t0; t < t1; ++t) {
    const int p = a.q_pos[t];
    if (!CAND && p < col0) continue;
    __syncthreads();
    // stage q[t] (heads padded to 16*MT with zeros) and w[t]
    {
      const int pieces_per_row = Di / 16;
      const int total = 16 * MT * pieces_per_row;
      for (int pc = tid; pc < total; pc += kScoreThreads) {
        const int h = pc / pieces_per_row, c = pc % pieces_per_row;
        v4u v = {0u, 0u, 0u, 0u};
        if (h < Hi) v = *(const v4u*)(a.q_fp8 + ((int64_t)t * Hi + h) * Di + 16 * c);
        *(v4u*)(q_lds + h * kQRow + 16 * c) = v;
      }
      if (tid < 16 * MT) w_lds[tid] = tid < Hi ? a.w[(int64_t)t * Hi + tid] : 0.0f;
    }
    __syncthreads();
    // heads outer, positions inner: one 16-head slice of q is live at a time; the keys
    // were converted once per block.  kappa > 0 commutes with the ReLU, so it scales the
    // head sum instead of every term.
    float sum[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) sum[i] = 0.0f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      v8bf qa[NKS_MAX];
      float wr[4];
      {
        const uint8_t* src = q_lds + (16 * mt + n) * kQRow + g * (Di / 4);
        const v4u lo = *(const v4u*)src;
        v4u hi = {0u, 0u, 0u, 0u};
        if (Di == 128) hi = *(const v4u*)(src + 16);
        const unsigned wds[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
        for (int s2 = 0; s2 < NKS_MAX; ++s2) qa[s2] = fp8x8_to_bf16(wds[2 * s2], wds[2 * s2 + 1]);
#pragma unroll
        for (int r = 0; r < 4; ++r) wr[r] = w_lds[16 * mt + 4 * g + r];
      }
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        const int colbase = col0 + wave * kPosPerWave + 16 * i;
        if (!CAND && colbase > p) break;
        v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s2 = 0; s2 < NKS_MAX; ++s2)
          if (s2 < nks) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s2], kb[i][s2], acc, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) sum[i] += wr[r] * fmaxf(acc[r], 0.0f);
      }
    }
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int colbase = col0 + wave * kPosPerWave + 16 * i;
      if (!CAND && colbase > p) break;
      float sm = sum[i];
      sm += __shfl_xor(sm, 16);
      sm += __shfl_xor(sm, 32);
      sm *= kap[i];
      if (g == 0) {
        const int col = colbase + n;
        if (CAND) {
          if (col < a.n_cand) {
            const bool valid = kpos[i] >= 0 && kpos[i] <= p;
            a.scores[(int64_t)t * a.ld + col] = valid ? sm : -__builtin_inff();
          }
        } else if (col <= p && col < len) {
          a.scores[(int64_t)t * a.ld + col] = sm;
        }
      }
    }
  }
}

template <int MT, int TPW, bool CAND>
static hipError_t launch_score_t(const ScoreArgs& a, hipStream_t s) {
  constexpr int per_wg = 4 * 16 * TPW;
  dim3 grid;
  if (CAND) grid = dim3((a.n_cand + per_wg - 1) / per_wg, a.T);
  else grid = dim3((a.max_ctx + per_wg - 1) / per_wg, a.B);
  if (grid.x == 0 || grid.y == 0) return hipSuccess;
  hipLaunchKernelGGL((score_kernel<MT, TPW, CAND>), grid, dim3(kScoreThreads), 0, s, a);
  return hipGetLastError();
}

template <int MT>
static hipError_t launch_score_mt(const ScoreArgs& a, hipStream_t s) {
  // Small problems use 64 positions per workgroup to spread over more CUs.
  const int64_t cols = a.cand ? (int64_t)a.n_cand * a.T : (int64_t)a.max_ctx * a.B;
  const bool small = cols / 256 < 1024;
  if (a.cand) return small ? launch_score_t<MT, 1, true>(a, s) : launch_score_t<MT, 4, true>(a, s);
  return small ? launch_score_t<MT, 1, false>(a, s) : launch_score_t<MT, 4, false>(a, s);
}

hipError_t launch_score(const ScoreArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (a.Hi <= 16) return launch_score_mt<1>(a, s);
  if (a.Hi <= 32) return launch_score_mt<2>(a, s);
  if (a.Hi <= 64) return launch_score_mt<4>(a, s);
  return launch_score_mt<8>(a, s);
}

}  // namespace smqa
