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
// and loops over the queries of that sequence (or over one of a few equal parts of them,
// when that fills the resident workgroup slots better), so keys are read from HBM once
// per sequence, or once per part, even when many queries share it (bounded replay).
// Each lane loads Di/4 contiguous key bytes per position (16-byte loads).
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

// -inf into columns [from, a.ld) of query t's score row, spread over the workgroups along x.
__device__ __forceinline__ void fill_tail(const ScoreArgs& a, int t, int from, int wg, int nwg) {
  for (int64_t c = from + (int64_t)wg * kScoreThreads + threadIdx.x; c < a.ld; c += (int64_t)nwg * kScoreThreads)
    a.scores[(int64_t)t * a.ld + c] = -__builtin_inff();
}
__device__ __forceinline__ void fill_tail(const ScoreArgs& a, int t, int from) {
  fill_tail(a, t, from, blockIdx.x, gridDim.x);
}

constexpr int kQRow = 272;   // LDS bytes per head row of bf16 q (256 + 16 pad: conflict-free b128 reads)

// Raw keys of one block of positions for one lane: TPW tiles x DI/4 bytes.
template <int TPW, int DI>
struct RawKeys {
  v4u lo[TPW], hi[TPW];
  float kap[TPW];
  int pos[TPW];   // position (CAND: from the list), -1 when the column is empty or invalid
};

// F8: the contraction on the FP8 matrix cores (v_mfma_scale_f32_16x16x128_f8f6f4, unit
// scales; DI = 128): q and the keys enter as the stored E4M3 bytes, one instruction per
// 16 heads x 16 positions covering all 128 dims, instead of four bf16 ones after an exact
// conversion.  Lane (g, n) already holds key bytes [32 g, 32 g + 32) of position n, which is
// its operand for that instruction; q's bytes go in the same order, so every product pairs
// the right dims.  The instruction adds its 128 exact products with an error of up to ~2^-15
// of their absolute sum (measured on gfx950); the bf16 form adds them in fp32.
template <int MT, int TPW, int DI, bool CAND, bool F8 = false>
__global__ __launch_bounds__(kScoreThreads, 2) void score_kernel(ScoreArgs a) {
  static_assert(!F8 || DI == 128, "the FP8 form covers 128 dims per instruction");
  // two q buffers: query t is scored from one while query t+1 is written to the other (bf16
  // rows, or the raw E4M3 bytes in the first half of each row for F8)
  __shared__ __align__(16) uint8_t q_lds[2][16 * MT * kQRow];
  __shared__ float w_lds[2][16 * MT];
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
    // dense: the sequence's queries, or the blockIdx.z-th of gridDim.z equal parts of them
    b = blockIdx.y;
    const int q0 = a.q_start[b], q1 = a.q_start[b + 1];
    const int per = (q1 - q0 + (int)gridDim.z - 1) / (int)gridDim.z;
    t0 = min(q0 + per * (int)blockIdx.z, q1);
    t1 = min(t0 + per, q1);
  }
  const int64_t base = a.seq_start[b];
  const int len = (int)(a.seq_start[b + 1] - base);
  const int ncols = CAND ? a.n_cand : len;
#ifdef SMQA_DEBUG
  if (blockIdx.x == 0) {
    dbg_flag(a.dbg, threadIdx.x == 0 && (len < 0 || t1 < t0), kDbgLayout);
    for (int t = t0 + (int)threadIdx.x; t < t1; t += kScoreThreads) dbg_flag(a.dbg, a.q_pos[t] < 0, kDbgLayout);
  }
#endif
  if (a.fill_tail) {
    if (CAND) fill_tail(a, t0, a.n_cand);
    else
      for (int t = t0; t < t1; ++t) fill_tail(a, t, max(min(a.q_pos[t], len - 1) + 1, 0));
  }
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
#ifdef SMQA_DEBUG
        dbg_flag(a.dbg, ok && col + 1 < a.n_cand && a.cand[(int64_t)t0 * a.n_cand + col + 1] <= pos, kDbgCand);
#endif
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

  // q of query t staged in LDS as bf16 (E4M3 -> bf16 exact), converted once per query:
  // fetch_q reads it into registers (16 bytes of E4M3 per piece), put_q converts and
  // stores it into one of the two buffers
  constexpr int kQPieces = 16 * MT * (DI / 16);
  constexpr int kQPer = (kQPieces + kScoreThreads - 1) / kScoreThreads;
  struct QRegs {
    v4u v[kQPer];
    float w;
  };
  auto fetch_q = [&](int t, QRegs& r) {
#pragma unroll
    for (int u = 0; u < kQPer; ++u) {
      const int pc = tid + kScoreThreads * u;
      const int h = pc / (DI / 16), c = pc % (DI / 16);
      r.v[u] = v4u{0u, 0u, 0u, 0u};
      if (pc < kQPieces && h < Hi) r.v[u] = *(const v4u*)(a.q_fp8 + ((int64_t)t * Hi + h) * DI + 16 * c);
    }
    r.w = tid < 16 * MT && tid < Hi ? a.w[(int64_t)t * Hi + tid] : 0.0f;
  };
  auto put_q = [&](int buf, const QRegs& r) {
#pragma unroll
    for (int u = 0; u < kQPer; ++u) {
      const int pc = tid + kScoreThreads * u;
      const int h = pc / (DI / 16), c = pc % (DI / 16);
      if (pc < kQPieces) {
        if constexpr (F8) {
          *(v4u*)(q_lds[buf] + h * kQRow + 16 * c) = r.v[u];
        } else {
          uint8_t* dst = q_lds[buf] + h * kQRow + 32 * c;
          *(v8bf*)dst = fp8x8_to_bf16(r.v[u].x, r.v[u].y);
          *(v8bf*)(dst + 16) = fp8x8_to_bf16(r.v[u].z, r.v[u].w);
        }
      }
    }
    if (tid < 16 * MT) w_lds[buf][tid] = r.w;
  };
  auto stage_q = [&](int t, int buf) {
    QRegs r;
    fetch_q(t, r);
    put_q(buf, r);
  };
  // One query per sequence (decode): q, w and the position are loaded once, in the same
  // round trip as the first block's keys, so the block loop issues no load besides the key
  // prefetch and never waits for it early.
  const bool single = t1 - t0 == 1;
  const int p0 = __builtin_amdgcn_readfirstlane(a.q_pos[t0]);
  QRegs q0;
  if (single) fetch_q(t0, q0);

  // largest query position of the sequence: blocks past it are never scored (dense)
  int pmax = 0x7FFFFFFF;
  if (!CAND) {
    if (single) {
      pmax = p0;
    } else {
      if (tid == 0) s_pmax = -1;
      __syncthreads();
      int pm = -1;
      for (int t = t0 + tid; t < t1; t += kScoreThreads) pm = max(pm, a.q_pos[t]);
      if (pm >= 0) atomicMax(&s_pmax, pm);
      __syncthreads();
      pmax = s_pmax;
    }
    nblk = min(nblk, pmax / kPosPerWG + 1);
  }
  if (single) {
    put_q(0, q0);
    __syncthreads();
  }

  // The next block's keys load while this block is scored.
  auto score_block = [&](RawKeys<TPW, DI>& rk) {
    // convert this block's keys (exact E4M3 -> bf16), then reuse rk for block + G
    v8bf kb[F8 ? 1 : TPW][F8 ? 1 : NKS];
    v8i k8[F8 ? TPW : 1];
    float kap[TPW];
    int kpos[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const unsigned wds[8] = {rk.lo[i].x, rk.lo[i].y, rk.lo[i].z, rk.lo[i].w,
                               rk.hi[i].x, rk.hi[i].y, rk.hi[i].z, rk.hi[i].w};
      if constexpr (F8) {
        k8[i] = v8i{(int)wds[0], (int)wds[1], (int)wds[2], (int)wds[3],
                    (int)wds[4], (int)wds[5], (int)wds[6], (int)wds[7]};
      } else {
#pragma unroll
        for (int s2 = 0; s2 < NKS; ++s2) kb[i][s2] = fp8x8_to_bf16(wds[2 * s2], wds[2 * s2 + 1]);
      }
      kap[i] = rk.kap[i];
      kpos[i] = rk.pos[i];
    }
    const int col0 = blk * kPosPerWG;
    if (blk + (int)gridDim.x < nblk) load_keys(blk + gridDim.x, rk);

      // several queries: q of query t+1 is read while query t is scored and written to the
      // other buffer after it, one barrier per query
      if (!single) {
        __syncthreads();                       // the previous block's last q is no longer read
        stage_q(t0, 0);
        __syncthreads();
      }
      for (int t = t0; t < t1; ++t) {
        const int buf = single ? 0 : (t - t0) & 1;
        QRegs nq;
        if (!single && t + 1 < t1) fetch_q(t + 1, nq);
        const int p = single ? p0 : __builtin_amdgcn_readfirstlane(a.q_pos[t]);
        if (CAND || p >= col0) {
        // heads outer, positions inner: one 16-head slice of q is live at a time; the TPW
        // accumulator chains are interleaved so consecutive MFMAs are independent.  kappa > 0
        // commutes with the ReLU, so it scales the head sum instead of every term.
        float sum[TPW];
#pragma unroll
        for (int i = 0; i < TPW; ++i) sum[i] = 0.0f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          float wr[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) wr[r] = w_lds[buf][16 * mt + 4 * g + r];
          v4f acc[TPW];
#pragma unroll
          for (int i = 0; i < TPW; ++i) acc[i] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
          if constexpr (F8) {
            const uint8_t* src = q_lds[buf] + (16 * mt + n) * kQRow + 32 * g;
            const v4u q0 = *(const v4u*)src, q1 = *(const v4u*)(src + 16);
            const v8i qa = {(int)q0.x, (int)q0.y, (int)q0.z, (int)q0.w, (int)q1.x, (int)q1.y, (int)q1.z, (int)q1.w};
#pragma unroll
            for (int i = 0; i < TPW; ++i)
              acc[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa, k8[i], acc[i], 0, 0, 0, 127, 0, 127);
          } else {
            v8bf qa[NKS];
            const uint8_t* src = q_lds[buf] + (16 * mt + n) * kQRow + 2 * g * (DI / 4);
#pragma unroll
            for (int s2 = 0; s2 < NKS; ++s2) qa[s2] = *(const v8bf*)(src + 16 * s2);
#pragma unroll
            for (int s2 = 0; s2 < NKS; ++s2)
#pragma unroll
              for (int i = 0; i < TPW; ++i)
                acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s2], kb[i][s2], acc[i], 0, 0, 0);
          }
#pragma unroll
          for (int i = 0; i < TPW; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) sum[i] += wr[r] * relu(acc[i][r]);
        }
        if constexpr (TPW == 4) {
          // reduce-scatter over the lane groups g (two permlane32 swaps, one permlane16
          // swap): lane (g, n) ends with the head sum of tile g, position n, so the wave's
          // 64 scores go out in one coalesced store
          const auto x02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(sum[0]), __float_as_uint(sum[2]), false, false);
          const auto x13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(sum[1]), __float_as_uint(sum[3]), false, false);
          const float u = __uint_as_float(x02[0]) + __uint_as_float(x02[1]);
          const float v = __uint_as_float(x13[0]) + __uint_as_float(x13[1]);
          const auto y = __builtin_amdgcn_permlane16_swap(__float_as_uint(u), __float_as_uint(v), false, false);
          const float tot = __uint_as_float(y[0]) + __uint_as_float(y[1]);
          const float kg = g == 0 ? kap[0] : g == 1 ? kap[1] : g == 2 ? kap[2] : kap[3];
          const float sm = tot * kg;
          const int col = col0 + wave * kPosPerWave + lane;
          if (CAND) {
            const int kp = g == 0 ? kpos[0] : g == 1 ? kpos[1] : g == 2 ? kpos[2] : kpos[3];
            if (col < a.n_cand) a.scores[(int64_t)t * a.ld + col] = kp >= 0 && kp <= p ? sm : -__builtin_inff();
          } else if (col <= p && col < len) {
            a.scores[(int64_t)t * a.ld + col] = sm;
          }
        } else {
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
        }
        if (!single && t + 1 < t1) {
          put_q(buf ^ 1, nq);
          __syncthreads();
        }
      }
  };

  for (; blk < nblk; blk += gridDim.x) score_block(raw);
}

// Buffer resource over [base, base + bytes): loads past the end return zeros without a
// memory access and stores past it are dropped, so the streaming loop below issues every
// load and store unconditionally (no branch, hence no conservative wait at a join).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t range_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// Dense scoring when each query streams its sequence's keys once (decode: one query per
// sequence).  Same contraction as score_kernel; the difference is how HBM is kept busy:
//  * q (bf16) and the head weights stay in registers for the whole stream;
//  * each wave owns a two-block ring of raw keys, and a tile's registers are refilled with
//    the tile two blocks ahead as soon as they are converted, so about two blocks of
//    loads per wave are always in flight;
//  * bounds come from the buffer resources (positions >= min(len, p + 1) read as zero
//    and are never stored);
//  * the four 16-position tiles of a block are reduced over the lane groups with one
//    reduce-scatter (two permlane32 swaps, one permlane16 swap), after which lane l holds
//    position 64 * wave + l, so kappa is one load and the block's scores one store;
//  * HIST: each score's top-k order key also goes into an LDS histogram of its top 12
//    bits (one LDS atomic per lane per block), whose nonzero bins are added to the
//    query's global histogram when the stream ends, so the top-k needs no pass of its own
//    to find the first digit.
// Lane (g, n) of tile i holds key bytes [16g, 16g + 16) and [64 + 16g, 64 + 16g + 16) of
// position 16i + n; q uses the same byte -> k assignment.
template <int MT, int DI, bool HIST>
__global__ __launch_bounds__(kScoreThreads) void score_stream_kernel(ScoreArgs a) {
  __shared__ __align__(16) uint8_t q_lds[16 * MT * kQRow];
  __shared__ float w_lds[16 * MT];
  __shared__ unsigned khist[HIST ? kTopkBins : 1];
  __shared__ int s_scan[kScoreThreads / 64];
  __shared__ int64_t s_own[4];
  constexpr int TPW = 4, NKS = DI / 32, NH = DI / 64;
  constexpr int kPosPerWG = 4 * 16 * TPW;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, n = lane & 15;
  // The workgroups of the 1D grid are dealt to the sequences in proportion to their work (at
  // least one each), so rows of different lengths finish together: with work_i = the blocks
  // of min(len_i, max_ctx) times the queries of sequence i, P_i its exclusive prefix and N the
  // total, sequence i owns workgroups [F_i, F_{i+1}), F_i = i + floor(P_i (G - B) / N) and
  // F_B = G, and a workgroup strides over its sequence's blocks with the sequence's count.
  // The thread that finds the owner passes the sequence's bounds on, so the mapping adds a
  // block scan and no round trip to memory.  Thread tid takes sequences tid * spt .. + spt - 1.
  int b, wl, Gb, t0, t1, len;
  int64_t base;
  {
    const int B = a.B, Gt = gridDim.x, w = blockIdx.x;
    const int spt = (B + kScoreThreads - 1) / kScoreThreads;
    auto work = [&](int i, int64_t& sb, int& ln, int& q0, int& q1) {
      sb = a.seq_start[i];
      ln = (int)(a.seq_start[i + 1] - sb);
      q0 = a.q_start[i];
      q1 = a.q_start[i + 1];
      return ((max(min(ln, a.max_ctx), 0) + kPosPerWG - 1) / kPosPerWG) * max(q1 - q0, 0);
    };
    int mine = 0;
    for (int j = 0; j < spt; ++j) {
      const int i = tid * spt + j;
      int64_t sb;
      int ln, q0, q1;
      if (i < B) mine += work(i, sb, ln, q0, q1);
    }
    const int incl = wave_inclusive_sum(mine);
    if (lane == 63) s_scan[wave] = incl;
    __syncthreads();
    int P = incl - mine, N = 0;
#pragma unroll
    for (int i = 0; i < kScoreThreads / 64; ++i) {
      P += i < wave ? s_scan[i] : 0;
      N += s_scan[i];
    }
    const int64_t spare = Gt - B;
    for (int j = 0; j < spt; ++j) {
      const int i = tid * spt + j;
      if (i < B) {
        int64_t sb;
        int ln, q0, q1;
        const int wk = work(i, sb, ln, q0, q1);
        const int f0 = i + (N > 0 ? (int)((int64_t)P * spare / N) : 0);
        const int f1 = i + 1 == B ? Gt : i + 1 + (N > 0 ? (int)((int64_t)(P + wk) * spare / N) : 0);
        if (f0 <= w && w < f1) {
          s_own[0] = ((int64_t)i << 32) | (unsigned)(w - f0);
          s_own[1] = ((int64_t)(f1 - f0) << 32) | (unsigned)ln;
          s_own[2] = ((int64_t)q0 << 32) | (unsigned)q1;
          s_own[3] = sb;
        }
        P += wk;
      }
    }
    __syncthreads();
    b = (int)(s_own[0] >> 32);
    wl = (int)(unsigned)s_own[0];
    Gb = (int)(s_own[1] >> 32);
    len = (int)(unsigned)s_own[1];
    t0 = (int)(s_own[2] >> 32);
    t1 = (int)(unsigned)s_own[2];
    base = s_own[3];
    // (uniform by construction; readfirstlane lets the compiler build the buffer resources
    // from them in scalar registers)
    b = __builtin_amdgcn_readfirstlane(b);
    wl = __builtin_amdgcn_readfirstlane(wl);
    Gb = __builtin_amdgcn_readfirstlane(Gb);
    t0 = __builtin_amdgcn_readfirstlane(t0);
    t1 = __builtin_amdgcn_readfirstlane(t1);
    len = __builtin_amdgcn_readfirstlane(len);
    base = (int64_t)(((uint64_t)(unsigned)__builtin_amdgcn_readfirstlane((int)(base >> 32)) << 32) |
                     (uint64_t)(unsigned)__builtin_amdgcn_readfirstlane((int)base));
  }
  const int G = Gb;
  const bool has_scale = a.k_scale != nullptr;

  struct Slot {
    v4u k[TPW][NH];
    float kap;
  };

  for (int t = t0; t < t1; ++t) {
    const int p = __builtin_amdgcn_readfirstlane(a.q_pos[t]);
#ifdef SMQA_DEBUG
    dbg_flag(a.dbg, wl == 0 && threadIdx.x == 0 && (p < 0 || len < 0 || t1 < t0), kDbgLayout);
#endif
    // (readfirstlane: keeps the compiler from treating the buffer resources built from it
    // as divergent, which would wrap every load in a waterfall loop)
    // clamped at 0: a negative position (outside the stated range) scores nothing and never
    // moves the -inf fill before the row
    const int nvalid = __builtin_amdgcn_readfirstlane(max(min(min(len, p + 1), a.max_ctx), 0));
    const int nblk = (nvalid + kPosPerWG - 1) / kPosPerWG;
    if (HIST && wl == 0 && tid == 0) a.qcols[(int64_t)t * a.qcols_stride] = nvalid;
    if (a.fill_tail) fill_tail(a, t, nvalid, wl, Gb);
    if (wl >= nblk) continue;

    v8bf qa[MT][NKS];
    float wr[MT][4];

    const __amdgpu_buffer_rsrc_t kr = range_rsrc(a.k_fp8 + base * DI, nvalid * DI);
    const __amdgpu_buffer_rsrc_t sr = range_rsrc(has_scale ? (const void*)(a.k_scale + base) : (const void*)a.k_fp8,
                                                 has_scale ? nvalid * 4 : 0);
    const __amdgpu_buffer_rsrc_t orr = range_rsrc(a.scores + (int64_t)t * a.ld, nvalid * 4);
    const int koff = (wave * 64 + n) * DI + 16 * g;
    const int poff = (wave * 64 + lane) * 4;

    auto load_tile = [&](Slot& s, int bk, int i) {
#pragma unroll
      for (int h = 0; h < NH; ++h)
        s.k[i][h] = __builtin_amdgcn_raw_buffer_load_b128(kr, (bk * kPosPerWG + 16 * i) * DI + koff + 64 * h, 0, 0);
    };
    auto load_kap = [&](Slot& s, int bk) {
      s.kap = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(sr, bk * kPosPerWG * 4 + poff, 0, 0));
    };
    // Score block bk from s, refilling s with block nbk tile by tile.
    auto run = [&](Slot& s, int bk, int nbk) {
      float part[TPW];
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        v8bf kb[NKS];
#pragma unroll
        for (int h = 0; h < NH; ++h) {
          kb[2 * h] = fp8x8_to_bf16(s.k[i][h].x, s.k[i][h].y);
          kb[2 * h + 1] = fp8x8_to_bf16(s.k[i][h].z, s.k[i][h].w);
        }
        load_tile(s, nbk, i);
        v4f acc[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s2 = 0; s2 < NKS; ++s2)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[mt][s2], kb[s2], acc[mt], 0, 0, 0);
        float sm = 0.0f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) sm += wr[mt][r] * relu(acc[mt][r]);
        part[i] = sm;
      }
      // reduce-scatter over the lane groups g: lane (g, n) ends with tile g's head sum
      const auto x02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]), __float_as_uint(part[2]), false, false);
      const auto x13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[1]), __float_as_uint(part[3]), false, false);
      const float u = __uint_as_float(x02[0]) + __uint_as_float(x02[1]);
      const float v = __uint_as_float(x13[0]) + __uint_as_float(x13[1]);
      const auto y = __builtin_amdgcn_permlane16_swap(__float_as_uint(u), __float_as_uint(v), false, false);
      const float tot = __uint_as_float(y[0]) + __uint_as_float(y[1]);
      const float kap = has_scale ? s.kap : 1.0f;
      load_kap(s, nbk);
      const float sc = tot * kap;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sc), orr, bk * kPosPerWG * 4 + poff, 0, 0);
      if (HIST) {   // positions past the row count in bin 0, which the top-k ignores
        const unsigned key = bk * kPosPerWG + wave * 64 + lane < nvalid ? score_key(sc) : 0u;
        atomicAdd(&khist[key >> 20], 1u);
      }
    };

    // Issue order matters: the loop consumes tiles in this order and waits on the count of
    // loads issued after each one, so the scheduler may not reorder the prologue's loads.
    int blk = wl;
    Slot r0, r1;
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      load_tile(r0, blk, i);
      __builtin_amdgcn_sched_barrier(0);
    }
    load_kap(r0, blk);
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      load_tile(r1, blk + G, i);
    }
    load_kap(r1, blk + G);
    __builtin_amdgcn_sched_barrier(0);
    // q and the head weights are requested after the first two blocks' keys, so that both
    // arrive in one round trip to memory
    constexpr int kQPieces = 16 * MT * (DI / 16);     // 16-byte pieces of the q slice
    constexpr int kQPer = (kQPieces + kScoreThreads - 1) / kScoreThreads;
    v4u qv[kQPer];
#pragma unroll
    for (int u = 0; u < kQPer; ++u) {
      const int pc = tid + u * kScoreThreads, h = pc / (DI / 16), c = pc % (DI / 16);
      qv[u] = v4u{0u, 0u, 0u, 0u};
      if (pc < kQPieces && h < a.Hi) qv[u] = *(const v4u*)(a.q_fp8 + ((int64_t)t * a.Hi + h) * DI + 16 * c);
    }
    const float wv = tid < 16 * MT && tid < a.Hi ? a.w[(int64_t)t * a.Hi + tid] : 0.0f;
    __syncthreads();   // the previous query's q and histogram are no longer read
    if (HIST)
      for (int i = tid; i < kTopkBins; i += kScoreThreads) khist[i] = 0u;
#pragma unroll
    for (int u = 0; u < kQPer; ++u) {
      const int pc = tid + u * kScoreThreads, h = pc / (DI / 16), c = pc % (DI / 16);
      if (pc < kQPieces) {
        uint8_t* dst = q_lds + h * kQRow + 32 * c;
        *(v8bf*)dst = fp8x8_to_bf16(qv[u].x, qv[u].y);
        *(v8bf*)(dst + 16) = fp8x8_to_bf16(qv[u].z, qv[u].w);
      }
    }
    if (tid < 16 * MT) w_lds[tid] = wv;
    __syncthreads();
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int s2 = 0; s2 < NKS; ++s2)
        qa[mt][s2] = *(const v8bf*)(q_lds + (16 * mt + n) * kQRow + 2 * (64 * (s2 >> 1) + 16 * g + 8 * (s2 & 1)));
#pragma unroll
      for (int r = 0; r < 4; ++r) wr[mt][r] = w_lds[16 * mt + 4 * g + r];
    }
    for (; blk < nblk; blk += 2 * G) {
      run(r0, blk, blk + 2 * G);
      __builtin_amdgcn_sched_barrier(0);   // no conversion of r1 hoisted into r0's half
      run(r1, blk + G, blk + 3 * G);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (HIST) {
      __syncthreads();
      unsigned* gh = a.hist + (int64_t)t * kTopkBins;
      for (int i = tid; i < kTopkBins; i += kScoreThreads) {
        const unsigned c = khist[i];
        if (i > 0 && c) atomicAdd(&gh[i], c);
      }
    }
  }
}

// Workgroups of this kernel that fit on the current device at once (cached per
// instantiation and device).
template <class K>
static int resident_workgroups(K kernel) {
  static PerDevice cache;
  const int dev = current_device();
  if (dev < kMaxDevices) {
    if (const int c = cache.v[dev].load(std::memory_order_acquire)) return c;
  }
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kScoreThreads, 0) != hipSuccess ||
      cus <= 0 || per_cu <= 0)
    return 512;
  if (dev < kMaxDevices) cache.v[dev].store(cus * per_cu, std::memory_order_release);
  return cus * per_cu;
}

// Parts to split each sequence's queries into (dense mode, several queries per sequence),
// so that the blocks x sequences x parts workgroups fill whole rounds of the `slots`
// workgroups resident at once: the count that maximises the filled share of the last
// round, less 1.5% per extra part (each part reloads its block's keys and restages q), at
// most 8 parts and no more than the queries per sequence.  One block per workgroup is a
// coarse unit: eight sessions of 100K positions make 3,128 workgroups, 6.1 rounds of the 512
// that the occupancy query reports resident at once, so the last round is a ninth full;
// three parts (the last of 19 rounds 0.97 full) score the same bits 4-6% faster.
static int query_parts(int64_t wgs, int T, int B, int slots) {
  const int qmax = std::max(1, std::min(8, (T + B - 1) / std::max(B, 1)));
  int best = 1;
  double best_v = -1.0;
  for (int qs = 1; qs <= qmax; ++qs) {
    const int64_t w = wgs * qs;
    const int64_t rounds = (w + slots - 1) / slots;
    const double v = (double)w / (double)(rounds * slots) - 0.015 * (qs - 1);
    if (v > best_v + 1e-9) {
      best_v = v;
      best = qs;
    }
  }
  return best;
}

template <int MT, int TPW, int DI, bool CAND, bool F8 = false>
static hipError_t launch_score_t(const ScoreArgs& a, hipStream_t s, bool persistent) {
  constexpr int per_wg = 4 * 16 * TPW;
  const int rows = CAND ? a.T : a.B;
  const int nblk = ((CAND ? a.n_cand : a.max_ctx) + per_wg - 1) / per_wg;
  // persistent: exactly the workgroups that are resident at once, each looping over
  // blocks with the next block's keys in flight; otherwise one block per workgroup, and
  // with several queries per sequence the queries split into parts along z
  int gx = nblk, gz = 1;
  if (persistent) {
    const int res = resident_workgroups(score_kernel<MT, TPW, DI, CAND, F8>);
    gx = std::min(nblk, std::max(1, res / std::max(rows, 1)));
  } else if (!CAND && a.T > a.B) {
    gz = query_parts((int64_t)nblk * rows, a.T, a.B, resident_workgroups(score_kernel<MT, TPW, DI, CAND, F8>));
  }
  if (gx == 0 || rows == 0) return hipSuccess;
  hipLaunchKernelGGL((score_kernel<MT, TPW, DI, CAND, F8>), dim3(gx, rows, gz), dim3(kScoreThreads), 0, s, a);
  return hipGetLastError();
}

// Problems of fewer than 1024 blocks of 256 positions use 64 positions per workgroup to
// spread over more CUs.
static bool small_problem(const ScoreArgs& a) {
  const int64_t cols = a.cand ? (int64_t)a.n_cand * a.T : (int64_t)a.max_ctx * a.B;
  return cols / 256 < 1024;
}

// Whether the streaming kernel applies, and its grid width (workgroups per sequence):
// resident workgroups shared over the sequences, at most kMaxStreamGrid, so that every block
// the key ring touches (up to 4 grid strides past the row) has a 32-bit buffer offset.
constexpr int kMaxStreamGrid = 2048;

static bool stream_applies(const ScoreArgs& a) {
  if (a.T == 0 || a.cand || a.T != a.B || a.Hi > 64 || small_problem(a)) return false;
  const int per_wg = 4 * 16 * 4;
  const int64_t nblk = (a.max_ctx + per_wg - 1) / per_wg;
  return (nblk + 4 * (int64_t)kMaxStreamGrid) * per_wg * a.Di < ((int64_t)1 << 31);
}

static int stream_grid(const ScoreArgs& a, int resident) {
  const int per_wg = 4 * 16 * 4;
  const int nblk = (a.max_ctx + per_wg - 1) / per_wg;
  return std::min(std::min(nblk, kMaxStreamGrid), std::max(1, resident / std::max(a.B, 1)));
}

bool score_streams(const ScoreArgs& a) { return stream_applies(a); }

// The FP8 matrix-core form (DI = 128): score_kernel for every shape, with the launch
// choices of the bf16 form (the streaming kernel, whose decode rows are bound by HBM, has no
// FP8 form).
template <int MT>
static hipError_t launch_score_f8(const ScoreArgs& a, hipStream_t s) {
  const bool small = small_problem(a);
  if (a.cand) return small ? launch_score_t<MT, 1, 128, true, true>(a, s, false)
                           : launch_score_t<MT, 4, 128, true, true>(a, s, true);
  if (small) return launch_score_t<MT, 1, 128, false, true>(a, s, false);
  return launch_score_t<MT, 4, 128, false, true>(a, s, a.T == a.B);
}

template <int MT, int DI>
static hipError_t launch_score_mt(const ScoreArgs& a, hipStream_t s) {
  if constexpr (DI == 128) {
    if (a.fp8mma) return launch_score_f8<MT>(a, s);
  }
  const bool small = small_problem(a);
  if (a.cand) return small ? launch_score_t<MT, 1, DI, true>(a, s, false) : launch_score_t<MT, 4, DI, true>(a, s, true);
  // Several queries per sequence make a block compute-bound (q is restaged per query), so
  // every block gets its own workgroup; one query per sequence streams keys persistently.
  const bool one_query_per_seq = a.T == a.B;
  if (small) return launch_score_t<MT, 1, DI, false>(a, s, false);
  if (stream_applies(a)) {
    constexpr int M = MT <= 4 ? MT : 4;
    if (a.hist) {
      const int gx = stream_grid(a, resident_workgroups(score_stream_kernel<M, DI, true>));
      hipLaunchKernelGGL((score_stream_kernel<M, DI, true>), dim3(gx * a.B), dim3(kScoreThreads), 0, s, a);
    } else {
      const int gx = stream_grid(a, resident_workgroups(score_stream_kernel<M, DI, false>));
      hipLaunchKernelGGL((score_stream_kernel<M, DI, false>), dim3(gx * a.B), dim3(kScoreThreads), 0, s, a);
    }
    return hipGetLastError();
  }
  return launch_score_t<MT, 4, DI, false>(a, s, one_query_per_seq);
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
