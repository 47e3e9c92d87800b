// Sparse multi-query attention over selected FP4 latent rows plus FP8 window rows
// (vLLM blog "DeepSeek-V4.1-Flash sur vLLM": section "Kernels", MegaAttention reading
// the compressed FP4 KV; section "SWA bounded replay", the FP8 window of the last 128
// positions and its clip at the replay start; section "Performances agentiques", one
// KV latent shared by every head).
//
// Workgroup = (query t, group of 16*MT heads, contiguous range of 32-row tiles).
// Tiles 0..ceil(k/32)-1 hold the selected global rows, the remaining ones the window
// rows.  Per tile:
//   stage    global rows: E2M1 codes + E8M0 bytes are gathered into LDS with 16-byte
//            loads (window rows are read straight from global memory, L2-resident);
//   Q.K^T    bf16 MFMA 16x16x32; every wave owns <= 2 slices of 128 dims of the
//            contraction and keeps its slice of q in registers; FP4 -> bf16 via
//            v_cvt_scalef32_pk_bf16_fp4 (exact); partial logits reduced through LDS;
//   softmax  online, base-2, fp32; rho / sigma folded into the logit and into P;
//   P.V      fp16 MFMA 16x16x32; every wave owns <= 2 slices of 128 output dims.  The
//            B operand needs 8 rows of one column per lane: each lane converts a 4-byte
//            word (8 dims) of 8 rows and transposes in registers with v_perm_b32, which
//            makes one lane feed 8 MFMAs whose output columns are dims 8n+j.
// Several tile ranges per (query, head group) are merged with their log-sum-exp in a
// second kernel.
#include "common.h"

namespace smqa {

constexpr int kAttThreads = 512;
constexpr int kRows = 32;

template <class T>
__device__ __forceinline__ unsigned bits_of(T x) {
  static_assert(sizeof(T) == 4, "packed pair expected");
  return __builtin_bit_cast(unsigned, x);
}

template <int MT>
struct AttSmem {
  static constexpr int kHG = 16 * MT;
  int valid[kRows];
  float rscale[kRows];
  int64_t roff[kRows];
  float m[kHG], l[kHG], alpha[kHG];
  int any_valid;
  int rescale;
  __attribute__((aligned(16))) _Float16 P[kHG][40];     // 80-byte rows: conflict-free b128 reads
  float red[8][kHG][kRows];
  __attribute__((aligned(16))) uint8_t e8[kRows][64];
};

template <int MT, int NS>
__global__ __launch_bounds__(kAttThreads) void attend_kernel(AttendArgs a, int S, int ngroups, int total) {
  constexpr int kHG = 16 * MT;
  __shared__ AttSmem<MT> sm;
  extern __shared__ __attribute__((aligned(16))) uint8_t raw[];   // 32 rows of E2M1 codes

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, g = lane >> 4, n = lane & 15;

  // XCD-aware order: consecutive logical blocks (same query) land on one XCD.
  const int nb = gridDim.x;
  const int bid = blockIdx.x;
  const int logical = (bid & 7) * (nb >> 3) + (bid >> 3);
  if (logical >= total) return;
  const int split = logical % S;
  const int grp = (logical / S) % ngroups;
  const int t = logical / (S * ngroups);

  const int D = a.D, W = a.W, k = a.k, Hq = a.Hq;
  const int NSS = D / 128;                 // 128-dim slices
  const int RS = D / 2 + 16;               // LDS row stride of the code tile
  const int b = seq_of_query(a.q_start, a.B, t);
  const int64_t base = a.seq_start[b];
  const int p = a.q_pos[t];
  int lo_win = max(p - W + 1, 0);
  if (a.swa_clip) lo_win = max(lo_win, a.swa_clip[t]);
  const int pos0 = a.swa_pos0[b];
  const int ng = (k + kRows - 1) / kRows;
  const int ntiles = ng + (W + kRows - 1) / kRows;
  const int tb = (int)((int64_t)split * ntiles / S);
  const int te = (int)((int64_t)(split + 1) * ntiles / S);
  const int h0 = grp * kHG;
  const float lscale = a.sm_scale * kLog2e;

  // q slices for Q.K^T (A operands): dims 128*ss + 32*g + 8*i .. +8, head h0 + 16*mt + n
  v8bf qa[NS][4][MT];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int ss = wave + 8 * s;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint16_t* qrow = a.q + ((int64_t)t * Hq + h0 + 16 * mt + n) * D;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v4u v = {0u, 0u, 0u, 0u};
        if (ss < NSS) v = *(const v4u*)(qrow + 128 * ss + 32 * g + 8 * i);
        qa[s][i][mt] = __builtin_bit_cast(v8bf, v);
      }
    }
  }

  v4f o[NS][8][MT];
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) o[s][j][mt] = v4f{0.f, 0.f, 0.f, 0.f};

  if (tid < kHG) {
    sm.m[tid] = -__builtin_inff();
    sm.l[tid] = 0.0f;
  }
  if (tid == 0) sm.rescale = 0;

  for (int tile = tb; tile < te; ++tile) {
    const bool is_swa = tile >= ng;
    __syncthreads();
    if (tid == 0) sm.any_valid = 0;
    __syncthreads();
    if (tid < kRows) {
      bool valid;
      int64_t roff;
      float sc;
      if (!is_swa) {
        const int x = tile * kRows + tid;
        const int j = x < k ? a.idx[(int64_t)t * k + x] : -1;
        valid = j >= 0;
        roff = valid ? base + j : -1;
        sc = valid ? (a.kv_rowscale ? a.kv_rowscale[roff] : 1.0f) : 0.0f;
      } else {
        const int u = (tile - ng) * kRows + tid;
        const int pos = pos0 + u;
        valid = u < W && pos >= lo_win && pos <= p;
        roff = u < W ? (int64_t)b * W + u : -1;
        sc = (u < W && a.swa_scale) ? a.swa_scale[(int64_t)b * W + u] : 1.0f;
      }
      sm.valid[tid] = valid;
      sm.roff[tid] = roff;
      sm.rscale[tid] = sc;
      if (valid) atomicOr(&sm.any_valid, 1);
    }
    __syncthreads();
    if (!sm.any_valid) continue;

    if (!is_swa) {
      const int ppr = D / 32;              // 16-byte pieces per row
      for (int pc = tid; pc < kRows * ppr; pc += kAttThreads) {
        const int r = pc / ppr, c = pc - r * ppr;
        const int64_t ro = sm.roff[r];
        v4u v = {0u, 0u, 0u, 0u};
        if (ro >= 0) v = *(const v4u*)(a.kv_codes + ro * (D / 2) + 16 * c);
        *(v4u*)(raw + r * RS + 64 * (r >> 3) + 16 * c) = v;
      }
      const int epr = D / 128;             // E8M0 dwords per row
      for (int pc = tid; pc < kRows * epr; pc += kAttThreads) {
        const int r = pc / epr, c = pc - r * epr;
        const int64_t ro = sm.roff[r];
        unsigned v = 0x7F7F7F7Fu;
        if (ro >= 0) v = *(const unsigned*)(a.kv_e8m0 + ro * (D / 32) + 4 * c);
        *(unsigned*)(&sm.e8[r][4 * c]) = v;
      }
      __syncthreads();
    }

    // ---------------- Q.K^T partial over this wave's dim slices
    v4f sacc[MT][2];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) sacc[mt][0] = sacc[mt][1] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int ss = wave + 8 * s;
      if (ss < NSS) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int r = 16 * nt + n;
          v8bf kb[4];
          if (!is_swa) {
            const v4u c = *(const v4u*)(raw + r * RS + 64 * (r >> 3) + 64 * ss + 16 * g);
            const float scl = e8m0_to_float(sm.e8[r][4 * ss + g]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const unsigned wd = c[i];
              v4u u4;
              u4.x = bits_of(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, scl, 0));
              u4.y = bits_of(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, scl, 1));
              u4.z = bits_of(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, scl, 2));
              u4.w = bits_of(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, scl, 3));
              kb[i] = __builtin_bit_cast(v8bf, u4);
            }
          } else {
            const int64_t ro = sm.roff[r];
            v4u c0 = {0u, 0u, 0u, 0u}, c1 = {0u, 0u, 0u, 0u};
            if (ro >= 0) {
              const uint8_t* src = a.swa + ro * D + 128 * ss + 32 * g;
              c0 = *(const v4u*)src;
              c1 = *(const v4u*)(src + 16);
            }
            const unsigned wds[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              v4u u4;
              u4.x = bits_of(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wds[2 * i], 1.0f, false));
              u4.y = bits_of(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wds[2 * i], 1.0f, true));
              u4.z = bits_of(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wds[2 * i + 1], 1.0f, false));
              u4.w = bits_of(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wds[2 * i + 1], 1.0f, true));
              kb[i] = __builtin_bit_cast(v8bf, u4);
            }
          }
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
              sacc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s][i][mt], kb[i], sacc[mt][nt], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.red[wave][16 * mt + 4 * g + r][16 * nt + n] = sacc[mt][nt][r];
    __syncthreads();

    // ---------------- online softmax (base 2)
    {
      constexpr int TPH = 32 / MT;          // threads per head
      const int h = tid / TPH;
      const int x0 = (tid % TPH) * MT;
      float sv[MT];
      float tmax = -__builtin_inff();
#pragma unroll
      for (int e = 0; e < MT; ++e) {
        const int x = x0 + e;
        float acc = 0.0f;
#pragma unroll
        for (int w8 = 0; w8 < 8; ++w8) acc += sm.red[w8][h][x];
        sv[e] = sm.valid[x] ? acc * lscale * sm.rscale[x] : -__builtin_inff();
        tmax = fmaxf(tmax, sv[e]);
      }
#pragma unroll
      for (int o2 = 1; o2 < TPH; o2 <<= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, o2));
      const float m_old = sm.m[h];
      const float m_new = fmaxf(m_old, tmax);
      const bool none = m_new == -__builtin_inff();
      const float alpha = none ? 1.0f : exp2f(m_old - m_new);
      float psum = 0.0f;
#pragma unroll
      for (int e = 0; e < MT; ++e) {
        const int x = x0 + e;
        const float pe = (none || !sm.valid[x]) ? 0.0f : exp2f(sv[e] - m_new);
        psum += pe;
        sm.P[h][x] = (_Float16)(pe * sm.rscale[x]);
      }
#pragma unroll
      for (int o2 = 1; o2 < TPH; o2 <<= 1) psum += __shfl_xor(psum, o2);
      __syncthreads();   // every thread has read m/l before they are updated
      if (tid % TPH == 0) {
        sm.m[h] = m_new;
        sm.l[h] = sm.l[h] * alpha + psum;
        sm.alpha[h] = alpha;
        if (alpha != 1.0f) sm.rescale = 1;
      }
    }
    __syncthreads();

    // ---------------- P.V into this wave's output dim slices
    if (sm.rescale) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        float al[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) al[r] = sm.alpha[16 * mt + 4 * g + r];
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
          for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) o[s][j][mt][r] *= al[r];
      }
    }
    v8h pa[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) pa[mt] = *(const v8h*)(&sm.P[16 * mt + n][8 * g]);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int c = wave + 8 * s;
      if (c < NSS) {
        const int d0 = 128 * c + 8 * n;
        unsigned wd[8][2];
        float scl[8];
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
          const int row = 8 * g + rr;
          if (!is_swa) {
            wd[rr][0] = *(const unsigned*)(raw + row * RS + 64 * (row >> 3) + (d0 >> 1));
            scl[rr] = e8m0_to_float(sm.e8[row][d0 >> 5]);
          } else {
            const int64_t ro = sm.roff[row];
            v2u v = {0u, 0u};
            if (ro >= 0) v = *(const v2u*)(a.swa + ro * D + d0);
            wd[rr][0] = v.x;
            wd[rr][1] = v.y;
          }
        }
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          unsigned cv[8];
#pragma unroll
          for (int rr = 0; rr < 8; ++rr) {
            if (!is_swa) {
              switch (bb) {
                case 0: cv[rr] = bits_of(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd[rr][0], scl[rr], 0)); break;
                case 1: cv[rr] = bits_of(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd[rr][0], scl[rr], 1)); break;
                case 2: cv[rr] = bits_of(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd[rr][0], scl[rr], 2)); break;
                default: cv[rr] = bits_of(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd[rr][0], scl[rr], 3)); break;
              }
            } else {
              const unsigned src = wd[rr][bb >> 1];
              cv[rr] = (bb & 1) ? bits_of(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(src, 1.0f, true))
                                : bits_of(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(src, 1.0f, false));
            }
          }
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const unsigned sel = hh ? 0x07060302u : 0x05040100u;
            v4u bv;
            bv.x = __builtin_amdgcn_perm(cv[1], cv[0], sel);
            bv.y = __builtin_amdgcn_perm(cv[3], cv[2], sel);
            bv.z = __builtin_amdgcn_perm(cv[5], cv[4], sel);
            bv.w = __builtin_amdgcn_perm(cv[7], cv[6], sel);
            const v8h bj = __builtin_bit_cast(v8h, bv);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
              o[s][2 * bb + hh][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[mt], bj, o[s][2 * bb + hh][mt], 0, 0, 0);
          }
        }
      }
    }
    __syncthreads();
    if (tid == 0) sm.rescale = 0;
  }
  __syncthreads();

  // ---------------- epilogue
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int hl = 16 * mt + 4 * g + r;
      const int hg = h0 + hl;
      const float l = sm.l[hl];
      const float inv = (S == 1) ? (l > 0.0f ? 1.0f / l : 0.0f) : 1.0f;
      float* dst = (S == 1) ? a.out + ((int64_t)t * Hq + hg) * D
                            : (float*)a.ws + (((int64_t)split * a.T + t) * Hq + hg) * D;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int c = wave + 8 * s;
        if (c < NSS) {
          const int d0 = 128 * c + 8 * n;
          v4f lo = {o[s][0][mt][r] * inv, o[s][1][mt][r] * inv, o[s][2][mt][r] * inv, o[s][3][mt][r] * inv};
          v4f hi = {o[s][4][mt][r] * inv, o[s][5][mt][r] * inv, o[s][6][mt][r] * inv, o[s][7][mt][r] * inv};
          *(v4f*)(dst + d0) = lo;
          *(v4f*)(dst + d0 + 4) = hi;
        }
      }
    }
  }
  if (tid < kHG) {
    const int hg = h0 + tid;
    const float m = sm.m[tid], l = sm.l[tid];
    if (S == 1) {
      if (a.lse) a.lse[(int64_t)t * Hq + hg] = l > 0.0f ? (m + log2f(l)) * kLn2 : -__builtin_inff();
    } else {
      float* ml = (float*)a.ws + (size_t)S * a.T * Hq * D;
      const int64_t i = ((int64_t)split * a.T + t) * Hq + hg;
      ml[2 * i] = m;
      ml[2 * i + 1] = l;
    }
  }
}

__global__ __launch_bounds__(256) void attend_merge_kernel(AttendArgs a, int S) {
  const int th = blockIdx.x;
  const int t = th / a.Hq, h = th % a.Hq;
  const int D = a.D;
  const float* opart = (const float*)a.ws;
  const float* ml = opart + (size_t)S * a.T * a.Hq * D;
  float M = -__builtin_inff();
  for (int s = 0; s < S; ++s) M = fmaxf(M, ml[2 * (((int64_t)s * a.T + t) * a.Hq + h)]);
  float L = 0.0f;
  float wts[32];
  for (int s = 0; s < S; ++s) {
    const int64_t i = ((int64_t)s * a.T + t) * a.Hq + h;
    const float ms = ml[2 * i], ls = ml[2 * i + 1];
    const float wv = (M == -__builtin_inff() || ls == 0.0f) ? 0.0f : exp2f(ms - M);
    wts[s] = wv;
    L += wv * ls;
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  float* dst = a.out + ((int64_t)t * a.Hq + h) * D;
  for (int d = threadIdx.x; d < D; d += 256) {
    float acc = 0.0f;
    for (int s = 0; s < S; ++s) acc += wts[s] * opart[(((int64_t)s * a.T + t) * a.Hq + h) * D + d];
    dst[d] = acc * inv;
  }
  if (threadIdx.x == 0 && a.lse) a.lse[(int64_t)t * a.Hq + h] = L > 0.0f ? (M + log2f(L)) * kLn2 : -__builtin_inff();
}

// 32 heads per workgroup when the q slices and output accumulators fit the register
// file without spilling (D <= 1024); 16 heads otherwise.
static int head_tiles(int Hq, int D) { return (Hq % 32 == 0 && D <= 1024) ? 2 : 1; }

int attend_splits(int32_t T, int32_t k, int32_t W, int32_t Hq, int32_t D) {
  const int MT = head_tiles(Hq, D);
  const int ngroups = Hq / (16 * MT);
  const int ntiles = (k + kRows - 1) / kRows + (W + kRows - 1) / kRows;
  const int64_t base = (int64_t)T * ngroups;
  if (base <= 0) return 1;
  int S = 1;
  if (base < 512) S = (int)((512 + base - 1) / base);
  S = std::min(S, std::max(1, ntiles / 2));
  S = std::min(S, 32);
  return std::max(S, 1);
}

size_t attend_workspace_bytes(int32_t T, int32_t k, int32_t W, int32_t Hq, int32_t D) {
  const int S = attend_splits(T, k, W, Hq, D);
  if (S == 1) return 0;
  return (size_t)S * T * Hq * D * 4 + (size_t)S * T * Hq * 8;
}

template <int MT, int NS>
static hipError_t launch_attend_t(const AttendArgs& a, hipStream_t s) {
  const int S = attend_splits(a.T, a.k, a.W, a.Hq, a.D);
  const int ngroups = a.Hq / (16 * MT);
  const int total = a.T * ngroups * S;
  const int nb = (total + 7) / 8 * 8;
  const size_t raw_bytes = (size_t)kRows * (a.D / 2 + 16) + 4 * 64;
  hipLaunchKernelGGL((attend_kernel<MT, NS>), dim3(nb), dim3(kAttThreads), raw_bytes, s, a, S, ngroups, total);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S == 1) return e;
  hipLaunchKernelGGL(attend_merge_kernel, dim3(a.T * a.Hq), dim3(256), 0, s, a, S);
  return hipGetLastError();
}

hipError_t launch_attend(const AttendArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const int mt = head_tiles(a.Hq, a.D);
  if (a.D <= 1024) return mt == 2 ? launch_attend_t<2, 1>(a, s) : launch_attend_t<1, 1>(a, s);
  return launch_attend_t<1, 2>(a, s);
}

}  // namespace smqa
