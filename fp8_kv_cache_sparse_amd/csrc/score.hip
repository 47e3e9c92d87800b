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
// max(x, 0) as one integer max: non-negative floats order like their bit patterns, and
// every negative float (and -0) is a negative int32.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

constexpr int kQRow = 272;   // LDS bytes per head row of bf16 q (256 + 16 pad: conflict-free b128 reads)

// Raw keys of one block of positions for one lane: TPW tiles x DI/4 bytes.
template <int TPW, int DI>
struct RawKeys {
  v4u lo[TPW], hi[TPW];
  float kap[TPW];
  int pos[TPW];   // position (CAND: from the list), -1 when the column is empty or invalid
};

template <int MT, int TPW, int DI, bool CAND>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(ScoreArgs a) {
  __shared__ __align__(16) uint8_t q_lds[16 * MT * kQRow];
  __shared__ float w_lds[16 * MT];
  __shared__ int s_pmax;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, g = lane >> 4, n = lane & 15;
  constexpr int kPosPerWave = 16 * TPW;
  constexpr int kPosPerWG = 4 * kPosPerWave;
  constexpr int NKS = DI / 32;
  const int Hi = a.Hi;

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
  const int ncols = CAND ? a.n_cand : len;
  int nblk = (ncols + kPosPerWG - 1) / kPosPerWG;
  int blk = blockIdx.x;
  if (blk >= nblk || t0 >= t1) return;
  if (len == 0) {                                  // candidate mode only: nothing is visible
    for (int c = blk * kPosPerWG + tid; c < a.n_cand; c += gridDim.x * kPosPerWG)
      a.scores[(int64_t)t0 * a.ld + c] = -__builtin_inff();
    return;
  }

  // Keys of block `bk` straight into registers: lane (g, n) holds position n of each tile
  // and key bytes [g*DI/4, (g+1)*DI/4); MFMA K-step s uses bytes g*DI/4 + 8s .. +8, and q
  // uses the same byte -> k assignment, so the k-sum is the full dot product.  Addresses
  // of empty columns are clamped to the sequence's first row, so every load is issued.
  auto load_keys = [&](int bk, RawKeys<TPW, DI>& r) {
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int col = bk * kPosPerWG + wave * kPosPerWave + 16 * i + n;
      int pos = col;
      bool ok = col < ncols;
      if (CAND) {
        pos = ok ? a.cand[(int64_t)t0 * a.n_cand + col] : -1;
        ok = ok && pos >= 0 && pos < len;
      }
      const int64_t rowi = base + (ok ? pos : 0);
      const uint8_t* row = a.k_fp8 + rowi * DI + g * (DI / 4);
      r.lo[i] = *(const v4u*)row;
      if (DI == 128) r.hi[i] = *(const v4u*)(row + 16);
      r.kap[i] = a.k_scale ? a.k_scale[rowi] : 1.0f;
      r.pos[i] = ok ? pos : -1;
    }
  };

  RawKeys<TPW, DI> raw;
  load_keys(blk, raw);

  // largest query position of the sequence: blocks past it are never scored (dense)
  int pmax = 0x7FFFFFFF;
  if (!CAND) {
    if (tid == 0) s_pmax = -1;
    __syncthreads();
    int pm = -1;
    for (int t = t0 + tid; t < t1; t += kScoreThreads) pm = max(pm, a.q_pos[t]);
    if (pm >= 0) atomicMax(&s_pmax, pm);
    __syncthreads();
    pmax = s_pmax;
    nblk = min(nblk, pmax / kPosPerWG + 1);
  }

  // q of query t staged in LDS as bf16 (E4M3 -> bf16 exact), converted once per query
  auto stage_q = [&](int t) {
    const int pieces_per_row = DI / 16;
    const int total = 16 * MT * pieces_per_row;
    for (int pc = tid; pc < total; pc += kScoreThreads) {
      const int h = pc / pieces_per_row, c = pc % pieces_per_row;
      v4u v = {0u, 0u, 0u, 0u};
      if (h < Hi) v = *(const v4u*)(a.q_fp8 + ((int64_t)t * Hi + h) * DI + 16 * c);
      uint8_t* dst = q_lds + h * kQRow + 32 * c;
      *(v8bf*)dst = fp8x8_to_bf16(v.x, v.y);
      *(v8bf*)(dst + 16) = fp8x8_to_bf16(v.z, v.w);
    }
    if (tid < 16 * MT) w_lds[tid] = tid < Hi ? a.w[(int64_t)t * Hi + tid] : 0.0f;
  };
  // One query per sequence (decode): q, w and the position are loaded once, so the block
  // loop issues no load besides the key prefetch and never waits for it early.
  const bool single = t1 - t0 == 1;
  const int p0 = __builtin_amdgcn_readfirstlane(a.q_pos[t0]);
  if (single) {
    stage_q(t0);
    __syncthreads();
  }

  // The next block's keys load while this block is scored.
  auto score_block = [&](RawKeys<TPW, DI>& rk) {
    // convert this block's keys (exact E4M3 -> bf16), then reuse rk for block + G
    v8bf kb[TPW][NKS];
    float kap[TPW];
    int kpos[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const unsigned wds[8] = {rk.lo[i].x, rk.lo[i].y, rk.lo[i].z, rk.lo[i].w,
                               rk.hi[i].x, rk.hi[i].y, rk.hi[i].z, rk.hi[i].w};
#pragma unroll
      for (int s2 = 0; s2 < NKS; ++s2) kb[i][s2] = fp8x8_to_bf16(wds[2 * s2], wds[2 * s2 + 1]);
      kap[i] = rk.kap[i];
      kpos[i] = rk.pos[i];
    }
    const int col0 = blk * kPosPerWG;
    if (blk + (int)gridDim.x < nblk) load_keys(blk + gridDim.x, rk);

      for (int t = t0; t < t1; ++t) {
        const int p = single ? p0 : __builtin_amdgcn_readfirstlane(a.q_pos[t]);
        if (!CAND && p < col0) continue;
        if (!single) {
          __syncthreads();
          stage_q(t);
          __syncthreads();
        }
        // heads outer, positions inner: one 16-head slice of q is live at a time; the TPW
        // accumulator chains are interleaved so consecutive MFMAs are independent.  kappa > 0
        // commutes with the ReLU, so it scales the head sum instead of every term.
        float sum[TPW];
#pragma unroll
        for (int i = 0; i < TPW; ++i) sum[i] = 0.0f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          v8bf qa[NKS];
          float wr[4];
          {
            const uint8_t* src = q_lds + (16 * mt + n) * kQRow + 2 * g * (DI / 4);
#pragma unroll
            for (int s2 = 0; s2 < NKS; ++s2) qa[s2] = *(const v8bf*)(src + 16 * s2);
#pragma unroll
            for (int r = 0; r < 4; ++r) wr[r] = w_lds[16 * mt + 4 * g + r];
          }
          v4f acc[TPW];
#pragma unroll
          for (int i = 0; i < TPW; ++i) acc[i] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int s2 = 0; s2 < NKS; ++s2)
#pragma unroll
            for (int i = 0; i < TPW; ++i)
              acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s2], kb[i][s2], acc[i], 0, 0, 0);
#pragma unroll
          for (int i = 0; i < TPW; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) sum[i] += wr[r] * relu(acc[i][r]);
        }
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
          const int colbase = col0 + wave * kPosPerWave + 16 * i;
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
  };

  for (; blk < nblk; blk += gridDim.x) score_block(raw);
}

// Workgroups of this kernel that fit on the device at once (cached per instantiation).
template <class K>
static int resident_workgroups(K kernel) {
  static int cached = 0;
  if (cached == 0) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kScoreThreads, 0) != hipSuccess ||
        cus <= 0 || per_cu <= 0)
      return 512;
    cached = cus * per_cu;
  }
  return cached;
}

template <int MT, int TPW, int DI, bool CAND>
static hipError_t launch_score_t(const ScoreArgs& a, hipStream_t s, bool persistent) {
  constexpr int per_wg = 4 * 16 * TPW;
  const int rows = CAND ? a.T : a.B;
  const int nblk = ((CAND ? a.n_cand : a.max_ctx) + per_wg - 1) / per_wg;
  // persistent: exactly the workgroups that are resident at once, each looping over
  // blocks with the next block's keys in flight; otherwise one block per workgroup
  int gx = nblk;
  if (persistent) {
    const int res = resident_workgroups(score_kernel<MT, TPW, DI, CAND>);
    gx = std::min(nblk, std::max(1, res / std::max(rows, 1)));
  }
  if (gx == 0 || rows == 0) return hipSuccess;
  hipLaunchKernelGGL((score_kernel<MT, TPW, DI, CAND>), dim3(gx, rows), dim3(kScoreThreads), 0, s, a);
  return hipGetLastError();
}

template <int MT, int DI>
static hipError_t launch_score_mt(const ScoreArgs& a, hipStream_t s) {
  // Small problems use 64 positions per workgroup to spread over more CUs.
  const int64_t cols = a.cand ? (int64_t)a.n_cand * a.T : (int64_t)a.max_ctx * a.B;
  const bool small = cols / 256 < 1024;
  if (a.cand) return small ? launch_score_t<MT, 1, DI, true>(a, s, false) : launch_score_t<MT, 4, DI, true>(a, s, true);
  // Several queries per sequence make a block compute-bound (q is restaged per query), so
  // every block gets its own workgroup; one query per sequence streams keys persistently.
  const bool one_query_per_seq = a.T == a.B;
  return small ? launch_score_t<MT, 1, DI, false>(a, s, false)
               : launch_score_t<MT, 4, DI, false>(a, s, one_query_per_seq);
}

template <int DI>
static hipError_t launch_score_di(const ScoreArgs& a, hipStream_t s) {
  if (a.Hi <= 16) return launch_score_mt<1, DI>(a, s);
  if (a.Hi <= 32) return launch_score_mt<2, DI>(a, s);
  if (a.Hi <= 64) return launch_score_mt<4, DI>(a, s);
  return launch_score_mt<8, DI>(a, s);
}

hipError_t launch_score(const ScoreArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  return a.Di == 128 ? launch_score_di<128>(a, s) : launch_score_di<64>(a, s);
}

}  // namespace smqa
