// Sparse multi-query attention over selected FP4 latent rows plus FP8 window rows
// (vLLM blog "DeepSeek-V4.1-Flash sur vLLM": section "Kernels", MegaAttention reading
// the compressed FP4 KV; section "SWA bounded replay", the FP8 window of the last 128
// positions and its clip at the replay start; section "Performances agentiques", one
// KV latent shared by every head).
//
// A query's tiles are ceil(k/32) tiles of 32 selected global rows followed by the
// 16-row tiles of window rows that overlap its visible window (fully clipped window
// rows are never touched).  A workgroup (8 waves) owns (query, head group, contiguous
// range of tiles); every tile goes through the same pipeline: gathered into registers
// two tiles ahead with 16-byte loads, committed to one of two LDS buffers, Q.K^T on
// bf16 MFMA 16x16x32 (E2M1 / E4M3 -> bf16 exact through v_cvt_scalef32_pk_bf16_*),
// online softmax in base 2 (fp32; rho / sigma folded into the logit and into P), P.V on
// fp16 MFMA 16x16x32; P.V of tile i and Q.K^T of tile i+1 share one barrier interval.
// Several tile ranges per (query, head group) are merged by log-sum-exp in a second
// kernel.  Two kernels implement this:
//
//   lat  16 heads per workgroup (32 when D <= 1024): twice the workgroups per query, for
//        calls with few queries, where latency and filling the CUs matter.  Waves own
//        128-dim slices of the contraction: Q.K^T slices {w, w+8}, P.V slices
//        {(w+3)%8, (w+3)%8+8}, which balances the combined phase when D/128 is not a
//        multiple of 8; q slice staged in LDS.
//   thr  32 heads per workgroup, for calls with many queries (throughput): every
//        dequantised value feeds twice the heads.  Wave w owns latent dims
//        [w*D/8, (w+1)*D/8) for both products: partial logits over its dims for all heads
//        (q held in registers), summed over the 8 waves through LDS, and the P.V outputs
//        of its dims (each lane converts one byte -- two dims -- of 8 rows and pairs the
//        halves with v_perm_b32 into the even-dim and odd-dim MFMA operands).
//
// In both, the P.V B operand needs 8 rows of one column per lane, built by converting
// per row and transposing in registers with v_perm_b32.
#include "common.h"

namespace smqa {

constexpr int kGRows = 32;   // rows per tile of selected global rows
constexpr int kWRows = 16;   // rows per tile of window rows

template <class T>
__device__ __forceinline__ unsigned bits_of(T x) {
  static_assert(sizeof(T) == 4, "packed pair expected");
  return __builtin_bit_cast(unsigned, x);
}

// Dynamic LDS of the attention kernels (tile buffers, positions, row and window scales).
extern __shared__ __attribute__((aligned(16))) uint8_t att_dyn[];

// ================================================================ 16-head kernel
namespace lat {

constexpr int kAttThreads = 512;

template <int MT>
struct AttSmem {
  static constexpr int kHG = 16 * MT;
  int valid[2][kGRows];
  float rscale[2][kGRows];
  float m[kHG], l[kHG], alpha[kHG];
  __attribute__((aligned(16))) _Float16 P[kHG][40];     // 80-byte rows: conflict-free b128 reads
  float red[8][kHG][kGRows];
  __attribute__((aligned(16))) uint8_t e8[2][kGRows][64];
};

// Per-workgroup constants of one query / head group / tile range.
struct AttCtx {
  int D, W, k, NSS, RS4, RS8, QS, BUF;
  int ng, wt0, tb, te, gx0;
  int b, p, lo_win, pos0, jmax;
  int64_t base;
  float lscale;
};

__device__ __forceinline__ v8bf cvt8_fp4_bf16(unsigned wd, float scl) {
  v4u u;
  u.x = bits_of(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, scl, 0));
  u.y = bits_of(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, scl, 1));
  u.z = bits_of(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, scl, 2));
  u.w = bits_of(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, scl, 3));
  return __builtin_bit_cast(v8bf, u);
}

__device__ __forceinline__ v8bf cvt8_fp8_bf16(unsigned w0, unsigned w1) {
  v4u u;
  u.x = bits_of(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false));
  u.y = bits_of(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true));
  u.z = bits_of(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false));
  u.w = bits_of(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true));
  return __builtin_bit_cast(v8bf, u);
}

// Partial logits of this wave's Q.K^T slices for one tile, written to red[wave].
template <int MT, int NS, bool FP8>
__device__ __forceinline__ void qk_tile(const AttCtx& c, AttSmem<MT>& sm, const uint8_t* buf, int slot,
                                        const uint8_t* qs, int wave, int g, int n) {
  asm volatile("" : "+v"(g), "+v"(n));
  v4f sacc[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) sacc[mt][0] = sacc[mt][1] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int ss = wave + 8 * s;
    if (ss < c.NSS) {
      // A operands: q of head 16*mt + n, dims 128*ss + 32*g + 8*i .. +8
      v8bf qa[4][MT];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          qa[i][mt] = *(const v8bf*)(qs + (16 * mt + n) * c.QS + 2 * (128 * ss + 32 * g + 8 * i));
      if (!FP8) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int r = 16 * nt + n;
          const v4u cw = *(const v4u*)(buf + r * c.RS4 + 64 * (r >> 3) + 64 * ss + 16 * g);
          const float scl = e8m0_to_float(sm.e8[slot][r][4 * ss + g]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const v8bf kb = cvt8_fp4_bf16(cw[i], scl);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
              sacc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[i][mt], kb, sacc[mt][nt], 0, 0, 0);
          }
        }
      } else {
        const uint8_t* src = buf + n * c.RS8 + 128 * ss + 32 * g;
        const v4u c0 = *(const v4u*)src;
        const v4u c1 = *(const v4u*)(src + 16);
        const unsigned wds[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const v8bf kb = cvt8_fp8_bf16(wds[2 * i], wds[2 * i + 1]);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            sacc[mt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[i][mt], kb, sacc[mt][0], 0, 0, 0);
        }
      }
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.red[wave][16 * mt + 4 * g + r][16 * nt + n] = sacc[mt][nt][r];
}

// Online softmax update for one tile (base 2): P = exp2(l - m_new) * row scale (fp16).
template <int MT>
__device__ __forceinline__ void softmax_tile(const AttCtx& c, AttSmem<MT>& sm, int slot, int tid) {
  constexpr int TPH = 32 / MT;             // threads per head, all in one wave
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
    sv[e] = sm.valid[slot][x] ? acc * c.lscale * sm.rscale[slot][x] : -__builtin_inff();
    tmax = fmaxf(tmax, sv[e]);
  }
#pragma unroll
  for (int o2 = 1; o2 < TPH; o2 <<= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, o2));
  const float m_old = sm.m[h];             // read by every lane of the head before lane 0 writes
  const float m_new = fmaxf(m_old, tmax);
  const bool none = m_new == -__builtin_inff();
  const float alpha = none ? 1.0f : exp2f(m_old - m_new);
  float psum = 0.0f;
#pragma unroll
  for (int e = 0; e < MT; ++e) {
    const int x = x0 + e;
    const float pe = (none || !sm.valid[slot][x]) ? 0.0f : exp2f(sv[e] - m_new);
    psum += pe;
    sm.P[h][x] = (_Float16)(pe * sm.rscale[slot][x]);
  }
#pragma unroll
  for (int o2 = 1; o2 < TPH; o2 <<= 1) psum += __shfl_xor(psum, o2);
  if (tid % TPH == 0) {
    sm.m[h] = m_new;
    sm.l[h] = sm.l[h] * alpha + psum;
    sm.alpha[h] = alpha;
  }
}

// P.V of one tile into this wave's output slices.
template <int MT, int NS, bool FP8>
__device__ __forceinline__ void pv_tile(const AttCtx& c, const AttSmem<MT>& sm, const uint8_t* buf, int slot,
                                        v4f (&o)[NS][8][MT], int wave, int g, int n) {
  asm volatile("" : "+v"(g), "+v"(n));
  // rescale by alpha when the running max moved for any head of this wave's outputs
  float al[MT][4];
  bool moved = false;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      al[mt][r] = sm.alpha[16 * mt + 4 * g + r];
      moved |= al[mt][r] != 1.0f;
    }
  if (__ballot(moved)) {
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) o[s][j][mt][r] *= al[mt][r];
  }
  v8h pa[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) pa[mt] = *(const v8h*)(&sm.P[16 * mt + n][8 * g]);
  const int cw0 = (wave + 3) & 7;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int cc = cw0 + 8 * s;
    if (cc < c.NSS) {
      const int d0 = 128 * cc + 8 * n;
      unsigned wd[8][2];
      float scl[8];
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        const int row = 8 * g + rr;
        if (!FP8) {
          wd[rr][0] = *(const unsigned*)(buf + row * c.RS4 + 64 * (row >> 3) + (d0 >> 1));
          wd[rr][1] = 0u;
          scl[rr] = e8m0_to_float(sm.e8[slot][row][d0 >> 5]);
        } else {
          v2u v = {0u, 0u};
          if (row < kWRows) v = *(const v2u*)(buf + row * c.RS8 + d0);
          wd[rr][0] = v.x;
          wd[rr][1] = v.y;
          scl[rr] = 1.0f;
        }
      }
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        unsigned cv[8];
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
          if (!FP8) {
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
}

template <int MT, int NS>
__global__ __launch_bounds__(kAttThreads) void attend_kernel(AttendArgs a, int S, int ngroups, int total) {
  constexpr int kHG = 16 * MT;
  __shared__ AttSmem<MT> sm;
  uint8_t* dyn = att_dyn;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, g = lane >> 4, n = lane & 15;
  (void)lane;

  // XCD-aware order: workgroups are dealt to the 8 XCDs round-robin, so logical block
  // (bid & 7) * (nb / 8) + (bid >> 3) puts runs of consecutive logical blocks on one XCD.
  // Head groups vary fastest: the workgroups that gather the same rows (one query, one
  // tile range, every head group) share that XCD's L2.
  const int nb = gridDim.x;
  const int bid = blockIdx.x;
  const int logical = (bid & 7) * (nb >> 3) + (bid >> 3);
  if (logical >= total) return;
  const int grp = logical % ngroups;
  const int split = (logical / ngroups) % S;
  const int t = logical / (S * ngroups);

  AttCtx c;
  c.D = a.D;
  c.W = a.W;
  c.k = a.k;
  c.NSS = c.D / 128;
  c.RS4 = c.D / 2 + 16;
  c.RS8 = c.D + 16;
  c.QS = 2 * c.D + 16;
  c.BUF = (max(kGRows * c.RS4 + 4 * 64, kWRows * c.RS8) + 15) & ~15;
  c.b = seq_of_query(a.q_start, a.B, t);
  c.base = a.seq_start[c.b];
  c.p = a.q_pos[t];
  c.jmax = min(c.p, (int)(a.seq_start[c.b + 1] - c.base) - 1);
  c.lo_win = max(c.p - c.W + 1, 0);
  if (a.swa_clip) c.lo_win = max(c.lo_win, a.swa_clip[t]);
  c.pos0 = a.swa_pos0[c.b];
  c.lscale = a.sm_scale * kLog2e;
  c.ng = (c.k + kGRows - 1) / kGRows;
  // window tiles overlapping the visible slots [u_lo, u_hi]
  const int u_lo = max(c.lo_win - c.pos0, 0);
  const int u_hi = min(c.p - c.pos0, c.W - 1);
  c.wt0 = u_lo / kWRows;
  const int nwt = u_lo <= u_hi ? u_hi / kWRows - c.wt0 + 1 : 0;
  const int ntiles = c.ng + nwt;
  c.tb = (int)((int64_t)split * ntiles / S);
  c.te = (int)((int64_t)(split + 1) * ntiles / S);
  const int h0 = grp * kHG;

  uint8_t* bufs = dyn;                             // two tile buffers
  uint8_t* qs = dyn + 2 * c.BUF;                   // q slice [kHG][QS]
  int* sidx = (int*)(qs + kHG * c.QS);
  c.gx0 = min(c.tb, c.ng) * kGRows;
  const int gx1 = min(min(c.te, c.ng) * kGRows, c.k);
  const int nsel = gx1 > c.gx0 ? gx1 - c.gx0 : 0;
  float* srho = (float*)(sidx + nsel);
  float* ssig = srho + nsel;

  auto row_pos = [&](int tile, int r) -> int {     // selected position of global row r, or -1
    const int x = tile * kGRows + r;
    return x < c.k ? sidx[x - c.gx0] : -1;
  };

  // Gather layout: a global tile is 32 FP4 rows of D/32 16-byte pieces, thread tid moving
  // pieces (tid & 15) + 16u of row tid >> 4 and E8M0 word tid & 15 of that row; a window
  // tile is 16 FP8 rows of D/16 pieces, thread tid moving pieces (tid & 31) + 32u of row
  // tid >> 5.  Each load instruction of a wave reads 256-byte runs of 4 (2) rows.
  // One code path for both tile kinds: addresses are selected, never branched on, so no
  // control-flow join sits between a load and its use (a join after a load makes the
  // compiler wait for every outstanding load, the prefetch included).
  auto positions = [&](int tile) -> int {          // position of this thread's global row
    int tid = threadIdx.x;                         // opaque: address math stays in the loop
    asm volatile("" : "+v"(tid));
    return tile < c.ng ? row_pos(tile, tid >> 4) : -1;
  };
  v4u pf[4];
  unsigned pf_e8;
  auto loads = [&](int tile, int j) {
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const bool glob = tile < c.ng;
    const int r = glob ? tid >> 4 : tid >> 5;
    const int q = glob ? tid & 15 : tid & 31;
    const int step = glob ? 16 : 32;
    const int ppr = glob ? c.D / 32 : c.D / 16;
    const int uu = kWRows * (c.wt0 + tile - c.ng) + r;
    const uint8_t* gsrc = a.kv_codes + (c.base + j) * (c.D / 2);
    const uint8_t* wsrc = a.swa + ((int64_t)c.b * c.W + uu) * c.D;
    const uint8_t* src = glob ? gsrc : wsrc;
    const bool row_ok = glob ? j >= 0 : uu < c.W;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int piece = q + step * u;
      v4u v = {0u, 0u, 0u, 0u};
      if (row_ok && piece < ppr) v = *(const v4u*)(src + 16 * piece);
      pf[u] = v;
    }
    unsigned e = 0x7F7F7F7Fu;
    if (glob && j >= 0 && (tid & 15) < c.D / 128)
      e = *(const unsigned*)(a.kv_e8m0 + (c.base + j) * (c.D / 32) + 4 * (tid & 15));
    pf_e8 = e;
  };
  auto prefetch = [&](int tile) { loads(tile, positions(tile)); };

  // ---- prologue.  Every load of step (1) is unconditional (clamped addresses), so the
  // compiler can count them exactly and keep the q slice in flight while it waits for
  // the positions; (2) the first tile's rows and the split's row scales follow.
  const int tb = c.tb, te = c.te;
  {
    const int per_row = c.D / 8;
    const int nq = kHG * per_row;                  // <= 4096 16-byte pieces
    const int32_t* ip = a.idx + (int64_t)t * c.k;
    const int x0 = c.gx0 + tid;
    const int j0 = ip[min(x0, c.k - 1)];
    v4u qv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int pc = min(tid + kAttThreads * u, nq - 1);
      const int h = pc / per_row, cc = pc - h * per_row;
      qv[u] = *(const v4u*)(a.q + ((int64_t)t * a.Hq + h0 + h) * c.D + 8 * cc);
    }
    // positions outside the query's rows are skipped like -1 (flagged in debug builds)
    if (x0 < gx1) {
      dbg_flag(a.dbg, j0 != -1 && !takes_part(j0, c.jmax), kDbgPosition);
      sidx[x0 - c.gx0] = takes_part(j0, c.jmax) ? j0 : -1;
    }
    for (int x = x0 + kAttThreads; x < gx1; x += kAttThreads) {
      const int j = ip[x];
      dbg_flag(a.dbg, j != -1 && !takes_part(j, c.jmax), kDbgPosition);
      sidx[x - c.gx0] = takes_part(j, c.jmax) ? j : -1;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int pc = tid + kAttThreads * u;
      const int h = pc / per_row, cc = pc - h * per_row;
      if (pc < nq) *(v4u*)(qs + h * c.QS + 16 * cc) = qv[u];
    }
    for (int u = tid; u < c.W; u += kAttThreads)
      ssig[u] = a.swa_scale ? a.swa_scale[(int64_t)c.b * c.W + u] : 1.0f;
    if (tid < kHG) {
      sm.m[tid] = -__builtin_inff();
      sm.l[tid] = 0.0f;
      sm.alpha[tid] = 1.0f;
    }
  }
  __syncthreads();
  if (tb < te) prefetch(tb);
  for (int x = c.gx0 + tid; x < gx1; x += kAttThreads) {
    const int j = sidx[x - c.gx0];
    srho[x - c.gx0] = (j >= 0 && a.kv_rowscale) ? a.kv_rowscale[c.base + j] : 1.0f;
  }
  __syncthreads();


  auto commit = [&](int tile, int slot) {
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    uint8_t* buf = bufs + slot * c.BUF;
    if (tile < c.ng) {
      const int r = tid >> 4, q = tid & 15;
      uint8_t* dst = buf + r * c.RS4 + 64 * (r >> 3);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (q + 16 * u < c.D / 32) *(v4u*)(dst + 16 * (q + 16 * u)) = pf[u];
      if (q < c.D / 128) *(unsigned*)(&sm.e8[slot][r][4 * q]) = pf_e8;
      if (tid < kGRows) {
        const int j = row_pos(tile, tid);
        sm.valid[slot][tid] = j >= 0;
        sm.rscale[slot][tid] = j >= 0 ? srho[tile * kGRows + tid - c.gx0] : 0.0f;
      }
    } else {
      const int r = tid >> 5, q = tid & 31;
      uint8_t* dst = buf + r * c.RS8;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (q + 32 * u < c.D / 16) *(v4u*)(dst + 16 * (q + 32 * u)) = pf[u];
      if (tid < kGRows) {
        const int uu = kWRows * (c.wt0 + tile - c.ng) + tid;
        const int pos = c.pos0 + uu;
        const bool in_buf = tid < kWRows && uu < c.W;
        sm.valid[slot][tid] = in_buf && pos >= c.lo_win && pos <= c.p;
        sm.rscale[slot][tid] = in_buf ? ssig[uu] : 0.0f;
      }
    }
  };

  // Q.K^T / P.V of tile `tile` held in LDS slot `slot`; one uniform branch on its kind.
  auto qk = [&](int tile, int slot) {
    if (tile < c.ng) qk_tile<MT, NS, false>(c, sm, bufs + slot * c.BUF, slot, qs, wave, g, n);
    else qk_tile<MT, NS, true>(c, sm, bufs + slot * c.BUF, slot, qs, wave, g, n);
  };

  v4f o[NS][8][MT];
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) o[s][j][mt] = v4f{0.f, 0.f, 0.f, 0.f};

  // ---- pipeline fill: tile tb committed and scored, tile tb+1 in flight
  if (tb < te) {
    commit(tb, 0);
    if (tb + 1 < te) prefetch(tb + 1);
  }
  __syncthreads();
  if (tb < te) qk(tb, 0);
  __syncthreads();
  if (tb < te) softmax_tile<MT>(c, sm, 0, tid);

  for (int i = tb; i < te; ++i) {
    const int cur = (i - tb) & 1, nxt = cur ^ 1;
    if (i + 1 < te) {
      commit(i + 1, nxt);
      if (i + 2 < te) prefetch(i + 2);
    }
    __syncthreads();                               // P(i), tile i+1 and its row flags published
    if (i < c.ng) pv_tile<MT, NS, false>(c, sm, bufs + cur * c.BUF, cur, o, wave, g, n);
    else pv_tile<MT, NS, true>(c, sm, bufs + cur * c.BUF, cur, o, wave, g, n);
    if (i + 1 < te) qk(i + 1, nxt);
    __syncthreads();                               // partial logits of tile i+1 published
    if (i + 1 < te) softmax_tile<MT>(c, sm, nxt, tid);
  }
  __syncthreads();

  // ---- epilogue
  const int cw0 = (wave + 3) & 7;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int hl = 16 * mt + 4 * g + r;
      const int hg = h0 + hl;
      const float l = sm.l[hl];
      const float inv = (S == 1) ? (l > 0.0f ? 1.0f / l : 0.0f) : 1.0f;
      float* dst = (S == 1) ? a.out + ((int64_t)t * a.Hq + hg) * c.D
                            : (float*)a.ws + (((int64_t)split * a.T + t) * a.Hq + hg) * c.D;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int cc = cw0 + 8 * s;
        if (cc < c.NSS) {
          const int d0 = 128 * cc + 8 * n;
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
      if (a.lse) a.lse[(int64_t)t * a.Hq + hg] = l > 0.0f ? (m + log2f(l)) * kLn2 : -__builtin_inff();
    } else {
      float* ml = (float*)a.ws + (size_t)S * a.T * a.Hq * c.D;
      const int64_t ii = ((int64_t)split * a.T + t) * a.Hq + hg;
      ml[2 * ii] = m;
      ml[2 * ii + 1] = l;
    }
  }
}

}  // namespace lat

// ================================================================ 32-head kernel
namespace thr {

constexpr int kAttThreads = 512;

template <class T>
__device__ __forceinline__ T lds_ld(int off) { return *(const T*)(att_dyn + off); }

template <int MT>
struct AttSmem {
  static constexpr int kHG = 16 * MT;
  int valid[2][kGRows];
  float rscale[2][kGRows];
  float m[kHG], l[kHG], alpha[kHG];
  __attribute__((aligned(16))) _Float16 P[kHG][40];     // 80-byte rows: conflict-free b128 reads
  float red[8][kHG][kGRows];                            // per-wave partial logits
};

// Tile-buffer geometry for latent width D (compile time, so LDS offsets are immediates).
// FP4 tile: row r of codes at r*RS4 + 64*(r >> 3) (RS4 = D/2 + 16; the extra 64 bytes
// every 8 rows keep the 8-row-apart P.V reads on distinct banks), then at SCO the block
// scales as floats, row r at r*SCS (SCS = D/32 + 1, odd).  FP8 tile: row r at r*RS8
// (RS8 = D + 16).  Wave w owns dims [w*DW, (w+1)*DW), NCH chunks of 32 (the last one
// half used when DW % 32 == 16).
template <int D>
struct Geo {
  static constexpr int DW = D / 8;
  static constexpr int NCH = (DW + 31) / 32;
  static constexpr int RS4 = D / 2 + 16;
  static constexpr int RS8 = D + 16;
  static constexpr int SCS = D / 32 + 1;
  static constexpr int SCO = (kGRows * RS4 + 4 * 64 + 15) & ~15;
  static constexpr int BUF4 = SCO + kGRows * SCS * 4;
  static constexpr int BUF8 = kWRows * RS8;
  static constexpr int BUF = ((BUF4 > BUF8 ? BUF4 : BUF8) + 15) & ~15;
  static __device__ __forceinline__ int fp4_row_off(int r) { return r * RS4 + 64 * (r >> 3); }
};

// Per-workgroup constants of one query / head group / tile range.
struct AttCtx {
  int W, k;
  int ng, wt0, tb, te, gx0;
  int b, p, lo_win, pos0, jmax;
  int64_t base;
  float lscale;
};

// ---------------------------------------------------------------- Q.K^T of one tile
// Partial logits over this wave's dims for all heads, written to red[wave].
// One code path for both tile kinds: only the B-operand build branches (uniformly), so
// the accumulators are never duplicated across two paths.
template <int MT, int D>
__device__ __forceinline__ void qk_tile(AttSmem<MT>& sm, int buf, bool fp8, const v8bf (&qa)[Geo<D>::NCH][MT],
                                        int wave, int g, int n) {
  using G = Geo<D>;
  constexpr int NCH = G::NCH;
  asm volatile("" : "+v"(g), "+v"(n));
  constexpr int NT = 2;                            // 16-row column tiles (a window tile has one)
  v4f sacc[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) sacc[mt][0] = sacc[mt][1] = v4f{0.f, 0.f, 0.f, 0.f};
  const int dw0 = wave * G::DW;
#pragma unroll
  for (int s = 0; s < NCH; ++s) {
    const int d0 = 32 * s + 8 * g;                 // this lane's 8 dims, relative to dw0
    const bool in = d0 < G::DW;                    // a half K-step when DW % 32 == 16
    const int dd = min(dw0 + d0, D - 8);           // clamped: out-of-slice lanes read in bounds
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int r = 16 * nt + n;
      v8bf kb;
      if (!fp8) {
        unsigned wd = lds_ld<unsigned>(buf + G::fp4_row_off(r) + (dd >> 1));
        float scl = lds_ld<float>(buf + G::SCO + 4 * (r * G::SCS + (dd >> 5)));
        wd = in ? wd : 0u;
        scl = in ? scl : 1.0f;
        v4u u;
        u.x = bits_of(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, scl, 0));
        u.y = bits_of(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, scl, 1));
        u.z = bits_of(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, scl, 2));
        u.w = bits_of(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, scl, 3));
        kb = __builtin_bit_cast(v8bf, u);
      } else {
        v2u w2 = lds_ld<v2u>(buf + (r & 15) * G::RS8 + dd);
        w2.x = (in && nt == 0) ? w2.x : 0u;
        w2.y = (in && nt == 0) ? w2.y : 0u;
        v4u u;
        u.x = bits_of(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w2.x, 1.0f, false));
        u.y = bits_of(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w2.x, 1.0f, true));
        u.z = bits_of(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w2.y, 1.0f, false));
        u.w = bits_of(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w2.y, 1.0f, true));
        kb = __builtin_bit_cast(v8bf, u);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        sacc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s][mt], kb, sacc[mt][nt], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);             // bound the registers held by read-ahead
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.red[wave][16 * mt + 4 * g + r][16 * nt + n] = sacc[mt][nt][r];
}

// ---------------------------------------------------------------- softmax of one tile
// Online softmax update (base 2): P = exp2(l - m_new) * row scale (fp16).
template <int MT>
__device__ __forceinline__ void softmax_tile(const AttCtx& c, AttSmem<MT>& sm, int slot, int tid) {
  constexpr int TPH = 32 / MT;             // threads per head, all in one wave
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
    sv[e] = sm.valid[slot][x] ? acc * c.lscale * sm.rscale[slot][x] : -__builtin_inff();
    tmax = fmaxf(tmax, sv[e]);
  }
#pragma unroll
  for (int o2 = 1; o2 < TPH; o2 <<= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, o2));
  const float m_old = sm.m[h];             // read by every lane of the head before lane 0 writes
  const float m_new = fmaxf(m_old, tmax);
  const bool none = m_new == -__builtin_inff();
  const float alpha = none ? 1.0f : exp2f(m_old - m_new);
  float psum = 0.0f;
#pragma unroll
  for (int e = 0; e < MT; ++e) {
    const int x = x0 + e;
    const float pe = (none || !sm.valid[slot][x]) ? 0.0f : exp2f(sv[e] - m_new);
    psum += pe;
    sm.P[h][x] = (_Float16)(pe * sm.rscale[slot][x]);
  }
#pragma unroll
  for (int o2 = 1; o2 < TPH; o2 <<= 1) psum += __shfl_xor(psum, o2);
  if (tid % TPH == 0) {
    sm.m[h] = m_new;
    sm.l[h] = sm.l[h] * alpha + psum;
    sm.alpha[h] = alpha;
  }
}

// ---------------------------------------------------------------- P.V of one tile
// o[ch][j][mt] holds heads 16*mt + 4g + r and dim dw0 + 32*ch + 2n + j.
template <int MT, int D>
__device__ __forceinline__ void pv_tile(const AttSmem<MT>& sm, int buf, bool fp8, v4f (&o)[Geo<D>::NCH][2][MT],
                                        int wave, int g, int n) {
  using G = Geo<D>;
  constexpr int NCH = G::NCH;
  asm volatile("" : "+v"(g), "+v"(n));
  // rescale by alpha when the running max moved for any head of this wave's outputs
  float al[MT][4];
  bool moved = false;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      al[mt][r] = sm.alpha[16 * mt + 4 * g + r];
      moved |= al[mt][r] != 1.0f;
    }
  if (__ballot(moved)) {
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) o[ch][j][mt][r] *= al[mt][r];
  }
  v8h pa[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) pa[mt] = *(const v8h*)(&sm.P[16 * mt + n][8 * g]);
  const int dw0 = wave * G::DW;
  // FP8 window tiles have 16 rows: lanes of row groups 2, 3 (rows 16..31) feed zeros
  const bool rows_ok = !fp8 || g < 2;
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
    const int dl = 32 * ch + 2 * n;                // this lane's dim pair, relative to dw0
    const bool ok = rows_ok && dl < G::DW;         // a half chunk when DW % 32 == 16
    const int dd = min(dw0 + dl, D - 2);           // clamped: out-of-slice lanes read in bounds
    unsigned cv[8];
    if (!fp8) {
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        const int row = 8 * g + rr;
        unsigned byte = lds_ld<uint8_t>(buf + G::fp4_row_off(row) + (dd >> 1));
        float scl = lds_ld<float>(buf + G::SCO + 4 * (row * G::SCS + (dd >> 5)));
        byte = ok ? byte : 0u;
        scl = ok ? scl : 1.0f;
        cv[rr] = bits_of(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(byte, scl, 0));
      }
    } else {
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        const int row = 8 * (g & 1) + rr;
        unsigned pair = lds_ld<unsigned short>(buf + row * G::RS8 + dd);
        pair = ok ? pair : 0u;
        cv[rr] = bits_of(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(pair, 1.0f, false));
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const unsigned sel = j ? 0x07060302u : 0x05040100u;
      v4u bv;
      bv.x = __builtin_amdgcn_perm(cv[1], cv[0], sel);
      bv.y = __builtin_amdgcn_perm(cv[3], cv[2], sel);
      bv.z = __builtin_amdgcn_perm(cv[5], cv[4], sel);
      bv.w = __builtin_amdgcn_perm(cv[7], cv[6], sel);
      const v8h bj = __builtin_bit_cast(v8h, bv);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        o[ch][j][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[mt], bj, o[ch][j][mt], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);             // bound the registers held by read-ahead
  }
}

// ---------------------------------------------------------------- the kernel
template <int MT, int D>
__global__ __launch_bounds__(kAttThreads) void attend_kernel(AttendArgs a, int S, int ngroups, int total) {
  constexpr int kHG = 16 * MT;
  using G = Geo<D>;
  constexpr int NCH = G::NCH;
  __shared__ AttSmem<MT> sm;
  uint8_t* dyn = att_dyn;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, g = lane >> 4, n = lane & 15;
  (void)lane;

  // XCD-aware order: workgroups are dealt to the 8 XCDs round-robin, so logical block
  // (bid & 7) * (nb / 8) + (bid >> 3) puts runs of consecutive logical blocks on one XCD.
  // Head groups vary fastest: the workgroups that gather the same rows (one query, one
  // tile range, every head group) share that XCD's L2.
  const int nb = gridDim.x;
  const int bid = blockIdx.x;
  const int logical = (bid & 7) * (nb >> 3) + (bid >> 3);
  if (logical >= total) return;
  const int grp = logical % ngroups;
  const int split = (logical / ngroups) % S;
  const int t = logical / (S * ngroups);

  AttCtx c;
  c.W = a.W;
  c.k = a.k;
  c.b = seq_of_query(a.q_start, a.B, t);
  c.base = a.seq_start[c.b];
  c.p = a.q_pos[t];
  c.jmax = min(c.p, (int)(a.seq_start[c.b + 1] - c.base) - 1);
  c.lo_win = max(c.p - c.W + 1, 0);
  if (a.swa_clip) c.lo_win = max(c.lo_win, a.swa_clip[t]);
  c.pos0 = a.swa_pos0[c.b];
  c.lscale = a.sm_scale * kLog2e;
  c.ng = (c.k + kGRows - 1) / kGRows;
  // window tiles overlapping the visible slots [u_lo, u_hi]
  const int u_lo = max(c.lo_win - c.pos0, 0);
  const int u_hi = min(c.p - c.pos0, c.W - 1);
  c.wt0 = u_lo / kWRows;
  const int nwt = u_lo <= u_hi ? u_hi / kWRows - c.wt0 + 1 : 0;
  const int ntiles = c.ng + nwt;
  c.tb = (int)((int64_t)split * ntiles / S);
  c.te = (int)((int64_t)(split + 1) * ntiles / S);
  const int h0 = grp * kHG;

  uint8_t* bufs = dyn;                             // two tile buffers
  int* sidx = (int*)(dyn + 2 * G::BUF);
  c.gx0 = min(c.tb, c.ng) * kGRows;
  const int gx1 = min(min(c.te, c.ng) * kGRows, c.k);
  const int nsel = gx1 > c.gx0 ? gx1 - c.gx0 : 0;
  float* srho = (float*)(sidx + nsel);
  float* ssig = srho + nsel;

  auto row_pos = [&](int tile, int r) -> int {     // selected position of global row r, or -1
    const int x = tile * kGRows + r;
    return x < c.k ? sidx[x - c.gx0] : -1;
  };

  // Gather layout: a global tile is 32 FP4 rows of D/32 16-byte pieces, thread tid moving
  // pieces (tid & 15) + 16u of row tid >> 4 and E8M0 word tid & 15 of that row; a window
  // tile is 16 FP8 rows of D/16 pieces, thread tid moving pieces (tid & 31) + 32u of row
  // tid >> 5.  Each load instruction of a wave reads 256-byte runs of 4 (2) rows.
  // One code path for both tile kinds: addresses are selected, never branched on, so no
  // control-flow join sits between a load and its use (a join after a load makes the
  // compiler wait for every outstanding load, the prefetch included).
  auto positions = [&](int tile) -> int {          // position of this thread's global row
    int tid = threadIdx.x;                         // opaque: address math stays in the loop
    asm volatile("" : "+v"(tid));
    return tile < c.ng ? row_pos(tile, tid >> 4) : -1;
  };
  v4u pf[4];
  unsigned pf_e8;
  auto loads = [&](int tile, int j) {
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const bool glob = tile < c.ng;
    const int r = glob ? tid >> 4 : tid >> 5;
    const int q = glob ? tid & 15 : tid & 31;
    const int step = glob ? 16 : 32;
    const int ppr = glob ? D / 32 : D / 16;
    const int uu = kWRows * (c.wt0 + tile - c.ng) + r;
    const uint8_t* gsrc = a.kv_codes + (c.base + j) * (D / 2);
    const uint8_t* wsrc = a.swa + ((int64_t)c.b * c.W + uu) * D;
    const uint8_t* src = glob ? gsrc : wsrc;
    const bool row_ok = glob ? j >= 0 : uu < c.W;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int piece = q + step * u;
      v4u v = {0u, 0u, 0u, 0u};
      if (row_ok && piece < ppr) v = *(const v4u*)(src + 16 * piece);
      pf[u] = v;
    }
    unsigned e = 0x7F7F7F7Fu;
    if (glob && j >= 0 && (tid & 15) < D / 128)
      e = *(const unsigned*)(a.kv_e8m0 + (c.base + j) * (D / 32) + 4 * (tid & 15));
    pf_e8 = e;
  };
  auto prefetch = [&](int tile) { loads(tile, positions(tile)); };

  // ---- prologue: q of this wave's dims into registers (A operands), this split's
  // positions, first tile in flight, row and window scales.
  const int tb = c.tb, te = c.te;
  v8bf qa[NCH][MT];
  {
    const int dw0 = wave * G::DW;
#pragma unroll
    for (int s = 0; s < NCH; ++s)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int d0 = 32 * s + 8 * g;
        const int dd = min(dw0 + d0, D - 8);     // clamped: the half step's upper lanes are unused
        v4u v = *(const v4u*)(a.q + ((int64_t)t * a.Hq + h0 + 16 * mt + n) * D + dd);
        if (d0 >= G::DW) v = v4u{0u, 0u, 0u, 0u};
        qa[s][mt] = __builtin_bit_cast(v8bf, v);
      }
    const int32_t* ip = a.idx + (int64_t)t * c.k;
    // positions outside the query's rows are skipped like -1 (flagged in debug builds)
    for (int x = c.gx0 + tid; x < gx1; x += kAttThreads) {
      const int j = ip[x];
      dbg_flag(a.dbg, j != -1 && !takes_part(j, c.jmax), kDbgPosition);
      sidx[x - c.gx0] = takes_part(j, c.jmax) ? j : -1;
    }
    for (int u = tid; u < c.W; u += kAttThreads)
      ssig[u] = a.swa_scale ? a.swa_scale[(int64_t)c.b * c.W + u] : 1.0f;
    if (tid < kHG) {
      sm.m[tid] = -__builtin_inff();
      sm.l[tid] = 0.0f;
      sm.alpha[tid] = 1.0f;
    }
  }
  __syncthreads();
  if (tb < te) prefetch(tb);
  for (int x = c.gx0 + tid; x < gx1; x += kAttThreads) {
    const int j = sidx[x - c.gx0];
    srho[x - c.gx0] = (j >= 0 && a.kv_rowscale) ? a.kv_rowscale[c.base + j] : 1.0f;
  }
  __syncthreads();

  auto commit = [&](int tile, int slot) {
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    uint8_t* buf = bufs + slot * G::BUF;
    if (tile < c.ng) {
      const int r = tid >> 4, q = tid & 15;
      uint8_t* dst = buf + G::fp4_row_off(r);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (q + 16 * u < D / 32) *(v4u*)(dst + 16 * (q + 16 * u)) = pf[u];
      if (q < D / 128) {
        float* sc = (float*)(buf + G::SCO) + r * G::SCS + 4 * q;
#pragma unroll
        for (int e = 0; e < 4; ++e) sc[e] = e8m0_to_float((pf_e8 >> (8 * e)) & 0xFFu);
      }
      if (tid < kGRows) {
        const int j = row_pos(tile, tid);
        sm.valid[slot][tid] = j >= 0;
        sm.rscale[slot][tid] = j >= 0 ? srho[tile * kGRows + tid - c.gx0] : 0.0f;
      }
    } else {
      const int r = tid >> 5, q = tid & 31;
      uint8_t* dst = buf + r * G::RS8;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (q + 32 * u < D / 16) *(v4u*)(dst + 16 * (q + 32 * u)) = pf[u];
      if (tid < kGRows) {
        const int uu = kWRows * (c.wt0 + tile - c.ng) + tid;
        const int pos = c.pos0 + uu;
        const bool in_buf = tid < kWRows && uu < c.W;
        sm.valid[slot][tid] = in_buf && pos >= c.lo_win && pos <= c.p;
        sm.rscale[slot][tid] = in_buf ? ssig[uu] : 0.0f;
      }
    }
  };

  auto qk = [&](int tile, int slot) { qk_tile<MT, D>(sm, slot * G::BUF, tile >= c.ng, qa, wave, g, n); };

  v4f o[NCH][2][MT];
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) o[ch][j][mt] = v4f{0.f, 0.f, 0.f, 0.f};

  // ---- pipeline fill: tile tb committed and scored, tile tb+1 in flight
  if (tb < te) {
    commit(tb, 0);
    if (tb + 1 < te) prefetch(tb + 1);
  }
  __syncthreads();
  if (tb < te) qk(tb, 0);
  __syncthreads();
  if (tb < te) softmax_tile<MT>(c, sm, 0, tid);

  for (int i = tb; i < te; ++i) {
    const int cur = (i - tb) & 1, nxt = cur ^ 1;
    if (i + 1 < te) {
      commit(i + 1, nxt);
      if (i + 2 < te) prefetch(i + 2);
    }
    __syncthreads();                               // P(i), tile i+1 and its row flags published
    pv_tile<MT, D>(sm, cur * G::BUF, i >= c.ng, o, wave, g, n);
    if (i + 1 < te) qk(i + 1, nxt);
    __syncthreads();                               // partial logits of tile i+1 published
    if (i + 1 < te) softmax_tile<MT>(c, sm, nxt, tid);
  }
  __syncthreads();

  // ---- epilogue: this wave's dims of every head
  const int dw0 = wave * G::DW;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int hl = 16 * mt + 4 * g + r;
      const int hg = h0 + hl;
      const float l = sm.l[hl];
      const float inv = (S == 1) ? (l > 0.0f ? 1.0f / l : 0.0f) : 1.0f;
      float* dst = (S == 1) ? a.out + ((int64_t)t * a.Hq + hg) * D
                            : (float*)a.ws + (((int64_t)split * a.T + t) * a.Hq + hg) * D;
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
        const int dl = 32 * ch + 2 * n;
        if (dl < G::DW) {
          float2 v = make_float2(o[ch][0][mt][r] * inv, o[ch][1][mt][r] * inv);
          *(float2*)(dst + dw0 + dl) = v;
        }
      }
    }
  }
  if (tid < kHG) {
    const int hg = h0 + tid;
    const float m = sm.m[tid], l = sm.l[tid];
    if (S == 1) {
      if (a.lse) a.lse[(int64_t)t * a.Hq + hg] = l > 0.0f ? (m + log2f(l)) * kLn2 : -__builtin_inff();
    } else {
      float* ml = (float*)a.ws + (size_t)S * a.T * a.Hq * D;
      const int64_t ii = ((int64_t)split * a.T + t) * a.Hq + hg;
      ml[2 * ii] = m;
      ml[2 * ii + 1] = l;
    }
  }
}

}  // namespace thr

// ================================================================ merge and dispatch
// out[t,h,d] = sum_s 2^(m_s - M) O_s[d] / sum_s 2^(m_s - M) l_s ; four consecutive output
// dims per thread with 16-byte loads and stores (the boundary requires a 256-byte aligned
// workspace and a 16-byte aligned output; D is a multiple of 128).  Every thread issues its
// S partial loads before the weights are known, so the merge costs one round trip to
// memory (SMAX >= S partials per output, at most 64; the instantiations 16, 24, 32, 64
// cover the split counts the planner makes with few repeated loads: k = 2048 with up to
// five queries takes 24).
template <int SMAX>
__global__ __launch_bounds__(128) void attend_merge_kernel(AttendArgs a, int S) {
  __shared__ float wts[64];
  __shared__ float sL, sM;
  const int th = blockIdx.y;
  const int t = th / a.Hq, h = th % a.Hq;
  const int D = a.D;
  const float* opart = (const float*)a.ws;
  const float* ml = opart + (size_t)S * a.T * a.Hq * D;
  const size_t sstride = (size_t)a.T * a.Hq * D;
  const int d = 4 * (blockIdx.x * 128 + threadIdx.x);
  // every slot loads a valid partial (slots past S repeat the last one, whose weight is 0),
  // so the loads carry no branches and all of them are in flight before the first wait
  v4f v[SMAX];
  {
    const float* src = opart + ((int64_t)t * a.Hq + h) * D + (d < D ? d : 0);
#pragma unroll
    for (int s = 0; s < SMAX; ++s) v[s] = *(const v4f*)(src + min(s, S - 1) * sstride);
  }
  if (threadIdx.x < 64) {
    const int s = threadIdx.x;
    float ms = -__builtin_inff(), ls = 0.0f;
    if (s < S) {
      const int64_t i = ((int64_t)s * a.T + t) * a.Hq + h;
      ms = ml[2 * i];
      ls = ml[2 * i + 1];
    }
    float M = ms;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) M = fmaxf(M, __shfl_xor(M, o));
    const float wv = (M == -__builtin_inff() || ls == 0.0f) ? 0.0f : exp2f(ms - M);
    float L = wv * ls;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) L += __shfl_xor(L, o);
    wts[s] = wv;
    if (s == 0) {
      sL = L;
      sM = M;
    }
  }
  __syncthreads();
  const float L = sL;
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  if (d < D) {
    v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < SMAX; ++s) acc += wts[s] * v[s];   // wts[s] = 0 for s >= S
    *(v4f*)(a.out + ((int64_t)t * a.Hq + h) * D + d) = acc * inv;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0 && a.lse)
    a.lse[(int64_t)t * a.Hq + h] = L > 0.0f ? (sM + log2f(L)) * kLn2 : -__builtin_inff();
}

// MegaAttention's epilogue (blog §Kernels: inverse RoPE on the output and FP8 conversion,
// written for the output projection): one workgroup per (query, head) merges the S split
// partials by log-sum-exp (4 dims per thread), rotates the pairs of the last
// 2 * rope_pairs dims back by the query's angle in fp32, takes the row's amax and writes
// E4M3 codes of x * (448 / amax) (fp32, round to nearest even) with the scale amax / 448.
template <int SMAX>
__global__ __launch_bounds__(512) void attend_fused_epilogue_kernel(AttendArgs a, int S) {
  __shared__ float wts[64];
  __shared__ float sL, sM;
  __shared__ float wmax[8];
  const int th = blockIdx.x;
  const int t = th / a.Hq, h = th % a.Hq;
  const int D = a.D;
  const float* opart = (const float*)a.ws;
  const float* ml = opart + (size_t)S * a.T * a.Hq * D;
  const size_t sstride = (size_t)a.T * a.Hq * D;
  const int d = 4 * threadIdx.x;
  const bool act = d < D;
  v4f v[SMAX];
  {
    // branch-free loads as in attend_merge_kernel (slots past S repeat the last partial)
    const float* src = opart + ((int64_t)t * a.Hq + h) * D + (act ? d : 0);
#pragma unroll
    for (int s = 0; s < SMAX; ++s) v[s] = *(const v4f*)(src + min(s, S - 1) * sstride);
  }
  if (threadIdx.x < 64) {
    const int s = threadIdx.x;
    float ms = -__builtin_inff(), ls = 0.0f;
    if (s < S) {
      const int64_t i = ((int64_t)s * a.T + t) * a.Hq + h;
      ms = ml[2 * i];
      ls = ml[2 * i + 1];
    }
    float M = ms;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) M = fmaxf(M, __shfl_xor(M, o));
    const float wv = (M == -__builtin_inff() || ls == 0.0f) ? 0.0f : exp2f(ms - M);
    float L = wv * ls;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) L += __shfl_xor(L, o);
    wts[s] = wv;
    if (s == 0) {
      sL = L;
      sM = M;
    }
  }
  __syncthreads();
  const float L = sL;
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int s = 0; s < SMAX; ++s) acc += wts[s] * v[s];     // wts[s] = 0 for s >= S
  acc *= inv;
  const int r0 = D - 2 * a.rope_pairs;
  if (act && a.rope_pairs > 0 && d >= r0) {
    const int64_t pj = (int64_t)t * a.rope_pairs + (d - r0) / 2;
    const float c0 = a.rope_cos[pj], s0 = a.rope_sin[pj], c1 = a.rope_cos[pj + 1], s1 = a.rope_sin[pj + 1];
    const float x0 = acc[0], x1 = acc[1], x2 = acc[2], x3 = acc[3];
    acc[0] = __builtin_fmaf(x0, c0, x1 * s0);
    acc[1] = __builtin_fmaf(-x0, s0, x1 * c0);
    acc[2] = __builtin_fmaf(x2, c1, x3 * s1);
    acc[3] = __builtin_fmaf(-x2, s1, x3 * c1);
  }
  // the row's amax: lanes, then the 8 waves through LDS
  float mx = act ? fmaxf(fmaxf(fabsf(acc[0]), fabsf(acc[1])), fmaxf(fabsf(acc[2]), fabsf(acc[3]))) : 0.0f;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = mx;
  __syncthreads();
  float amax = wmax[0];
#pragma unroll
  for (int w = 1; w < 8; ++w) amax = fmaxf(amax, wmax[w]);
  const float scale = amax / 448.0f;
  const float rq = amax > 0.0f ? 448.0f / amax : 0.0f;
  const int64_t row = (int64_t)t * a.Hq + h;
  if (act) {
    unsigned codes = 0u;
    if (amax > 0.0f) {
      const float y0 = acc[0] * rq, y1 = acc[1] * rq, y2 = acc[2] * rq, y3 = acc[3] * rq;
      codes = (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
      codes = (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, (int)codes, true);
    }
    *(unsigned*)(a.out_fp8 + row * D + d) = codes;
    if (a.out) *(v4f*)(a.out + row * D + d) = acc;
  }
  if (threadIdx.x == 0) {
    a.out_scale[row] = scale;
    if (a.lse) a.lse[row] = L > 0.0f ? (sM + log2f(L)) * kLn2 : -__builtin_inff();
  }
}

static int max_tiles(int32_t k, int32_t W) {
  return (k + kGRows - 1) / kGRows + (W + kWRows - 1) / kWRows + 1;
}

// Which kernel serves a call, with how many heads per workgroup and tile-range splits.
// The 32-head kernel needs Hq % 32 == 0 and D <= 1792 (its registers), and is chosen
// when at least 64 (query, 32-head group) pairs exist; otherwise the 16-head kernel
// (32 heads when D <= 1024) gives twice the workgroups per query.
struct AttPlan {
  bool wide;
  int MT, ngroups, S;
  int lds;                 // bytes per workgroup, static + dynamic
};

int sd_lds_bytes(int32_t D);   // attend_sd.hip: the dimension-split kernel's (fixed) LDS

// LDS of one workgroup (static + dynamic) for a plan with S splits.  The positions of a
// workgroup's tile range are staged whole, so the dynamic part shrinks as S grows.
static size_t plan_lds(const AttPlan& p, int32_t k, int32_t W, int32_t D, int S) {
  const size_t split_tiles = (size_t)(max_tiles(k, W) + S - 1) / S + 1;
  if (p.wide && D <= 1664) return (size_t)sd_lds_bytes(D);
  if (p.wide) {                                  // thr, D = 1792
    return 2 * (size_t)thr::Geo<1792>::BUF + split_tiles * kGRows * 8 + (size_t)W * 4 +
           sizeof(thr::AttSmem<2>);
  }
  const size_t buf = (std::max<size_t>((size_t)kGRows * (D / 2 + 16) + 4 * 64, (size_t)kWRows * (D + 16)) +
                      15) & ~(size_t)15;
  const size_t stat = p.MT == 2 ? sizeof(lat::AttSmem<2>) : sizeof(lat::AttSmem<1>);
  return 2 * buf + (size_t)16 * p.MT * (2 * D + 16) + split_tiles * kGRows * 8 + (size_t)W * 4 + stat;
}

constexpr int kMaxSplits = 64;                   // the merge kernels take up to 64 partials

static AttPlan attend_plan(int32_t T, int32_t k, int32_t W, int32_t Hq, int32_t D) {
  AttPlan p;
  // the dimension-split kernel for every query count it supports; the 16-head-group
  // kernels for the rest (the 32-head tile kernel only once there are enough workgroups)
  p.wide = Hq % 32 == 0 && (D <= 1664 || (D <= 1792 && (int64_t)T * (Hq / 32) >= 64));
  p.MT = p.wide ? 2 : ((Hq % 32 == 0 && D <= 1024) ? 2 : 1);
  p.ngroups = Hq / (16 * p.MT);
  const int ntiles = max_tiles(k, W);
  const int64_t base = (int64_t)T * p.ngroups;
  // about one workgroup per CU (a workgroup fills most of a CU's LDS), at least 3 tiles
  // per split so the prefetch pipeline has work to overlap its start-up cost, and at
  // most 32 partials per output
  int S = 1;
  if (base > 0 && base < 256) S = (int)((256 + base - 1) / base);
  S = std::min(S, std::max(1, ntiles / 3));
  S = std::max(std::min(S, 32), 1);
  // then as many more splits as it takes for a workgroup's LDS to fit the CU's
  while (S < kMaxSplits && plan_lds(p, k, W, D, S) > (size_t)kLdsBytes) ++S;
  p.lds = (int)plan_lds(p, k, W, D, S);
  p.S = p.lds <= kLdsBytes ? S : 0;
  return p;
}

int attend_splits(int32_t T, int32_t k, int32_t W, int32_t Hq, int32_t D, int32_t* lds) {
  const AttPlan p = attend_plan(T, k, W, Hq, D);
  if (lds) *lds = p.lds;
  return p.S;
}

// Whether decode_step may take the selection in the attention kernel (kKvMXS): the
// dimension-split kernel at D = 1664, every split of at most four tiles (so a workgroup's
// positions fit its ring; the kernel cuts ranges of ceil(nominal / S) tiles at most).
bool attend_select_fits(int32_t T, int32_t k, int32_t W, int32_t Hq, int32_t D) {
  const AttPlan p = attend_plan(T, k, W, Hq, D);
  if (p.S == 0 || !p.wide || D != 1664) return false;
  const int nominal = (k + kGRows - 1) / kGRows + (W + kWRows - 1) / kWRows;
  return (nominal + p.S - 1) / p.S <= 4;
}

size_t attend_workspace_bytes(int32_t T, int32_t k, int32_t W, int32_t Hq, int32_t D) {
  const int S = attend_splits(T, k, W, Hq, D);
  if (S <= 1) return 0;
  return (size_t)S * T * Hq * D * 4 + (size_t)S * T * Hq * 8;
}

hipError_t launch_attend_merge(const AttendArgs& a, int S, hipStream_t s) {
  if (S == 1) return hipSuccess;
  const dim3 grid((a.D / 4 + 127) / 128, a.T * a.Hq);
  if (S <= 16) hipLaunchKernelGGL(attend_merge_kernel<16>, grid, dim3(128), 0, s, a, S);
  else if (S <= 24) hipLaunchKernelGGL(attend_merge_kernel<24>, grid, dim3(128), 0, s, a, S);
  else if (S <= 32) hipLaunchKernelGGL(attend_merge_kernel<32>, grid, dim3(128), 0, s, a, S);
  else hipLaunchKernelGGL(attend_merge_kernel<64>, grid, dim3(128), 0, s, a, S);
  return hipGetLastError();
}

template <int MT, int NS>
static hipError_t launch_lat(const AttendArgs& a, const AttPlan& p, hipStream_t s) {
  const int total = a.T * p.ngroups * p.S;
  const int nb = (total + 7) / 8 * 8;
  const int split_tiles = (max_tiles(a.k, a.W) + p.S - 1) / p.S + 1;
  const size_t buf = (std::max<size_t>((size_t)kGRows * (a.D / 2 + 16) + 4 * 64,
                                       (size_t)kWRows * (a.D + 16)) + 15) & ~(size_t)15;
  const size_t dyn = 2 * buf + (size_t)16 * MT * (2 * a.D + 16) + (size_t)split_tiles * kGRows * 8 +
                     (size_t)a.W * 4;
  static PerDevice attr;
  hipError_t e = allow_dynamic_lds(lat::attend_kernel<MT, NS>, kLdsBytes - (int)sizeof(lat::AttSmem<MT>), attr);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((lat::attend_kernel<MT, NS>), dim3(nb), dim3(lat::kAttThreads), dyn, s, a, p.S,
                     p.ngroups, total);
  e = hipGetLastError();
  return e != hipSuccess ? e : launch_attend_merge(a, p.S, s);
}

template <int D>
static hipError_t launch_thr(const AttendArgs& a, const AttPlan& p, hipStream_t s) {
  if constexpr (thr::Geo<D>::NCH > 7) {           // never planned: would spill
    return hipErrorInvalidValue;
  } else {
    const int total = a.T * p.ngroups * p.S;
    const int nb = (total + 7) / 8 * 8;
    const int split_tiles = (max_tiles(a.k, a.W) + p.S - 1) / p.S + 1;
    const size_t dyn = 2 * (size_t)thr::Geo<D>::BUF + (size_t)split_tiles * kGRows * 8 + (size_t)a.W * 4;
    static PerDevice attr;
    hipError_t e = allow_dynamic_lds(thr::attend_kernel<2, D>, kLdsBytes - (int)sizeof(thr::AttSmem<2>), attr);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((thr::attend_kernel<2, D>), dim3(nb), dim3(thr::kAttThreads), dyn, s, a, p.S,
                       p.ngroups, total);
    e = hipGetLastError();
    return e != hipSuccess ? e : launch_attend_merge(a, p.S, s);
  }
}

hipError_t launch_attend_sd(const AttendArgs& a, int S, hipStream_t s);

// One split quantises in the attention kernel itself: the partials, and so the workspace,
// are those of the plain call.
size_t attend_fused_workspace_bytes(int32_t T, int32_t k, int32_t W, int32_t Hq, int32_t D) {
  return attend_workspace_bytes(T, k, W, Hq, D);
}

// The fused form: the dimension-split kernel (MX cache, Hq % 32 == 0, D <= 1664, checked by
// the caller) with the query RoPE; with one split its epilogue writes the FP8 output, with
// several the partials go to the workspace (no plain merge) and the epilogue kernel runs.
hipError_t launch_attend_fused(const AttendArgs& a0, hipStream_t s) {
  if (a0.T == 0) return hipSuccess;
  const AttPlan p = attend_plan(a0.T, a0.k, a0.W, a0.Hq, a0.D);
  if (p.S == 0 || !p.wide || a0.D > 1664 || a0.kv_fmt != kKvMX || !a0.out_fp8 || !a0.out_scale) return hipErrorInvalidValue;
  AttendArgs a = a0;
  // one split: the attention kernel's own epilogue rotates back and quantises; several:
  // partials, then the epilogue kernel
  a.kv_fmt = p.S > 1 ? kKvMXR : kKvMXF;
  hipError_t e = launch_attend_sd(a, p.S, s);
  if (e != hipSuccess || p.S == 1) return e;
  const dim3 grid(a.T * a.Hq);
  if (p.S <= 16) hipLaunchKernelGGL(attend_fused_epilogue_kernel<16>, grid, dim3(512), 0, s, a, p.S);
  else if (p.S <= 24) hipLaunchKernelGGL(attend_fused_epilogue_kernel<24>, grid, dim3(512), 0, s, a, p.S);
  else if (p.S <= 32) hipLaunchKernelGGL(attend_fused_epilogue_kernel<32>, grid, dim3(512), 0, s, a, p.S);
  else hipLaunchKernelGGL(attend_fused_epilogue_kernel<64>, grid, dim3(512), 0, s, a, p.S);
  return hipGetLastError();
}

// FP8 and NVFP4 global caches: only the dimension-split kernel reads them (Hq % 32 == 0,
// D <= 1664, checked by the caller); the split count and workspace are those of the MX call.
hipError_t launch_attend_fmt(const AttendArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const AttPlan p = attend_plan(a.T, a.k, a.W, a.Hq, a.D);
  if (p.S == 0 || !p.wide || a.D > 1664 || (a.kv_fmt != kKvFP8 && a.kv_fmt != kKvNV && a.kv_fmt != kKvMXN))
    return hipErrorInvalidValue;
  return launch_attend_sd(a, p.S, s);
}

hipError_t launch_attend(const AttendArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const AttPlan p = attend_plan(a.T, a.k, a.W, a.Hq, a.D);
  if (p.S == 0) return hipErrorInvalidValue;
  if (!p.wide) {
    if (a.D <= 1024) return p.MT == 2 ? launch_lat<2, 1>(a, p, s) : launch_lat<1, 1>(a, p, s);
    return launch_lat<1, 2>(a, p, s);
  }
  if (a.D <= 1664) return launch_attend_sd(a, p.S, s);
  if (a.D == 1792) return launch_thr<1792>(a, p, s);   // the plan takes no other width here
  return hipErrorInvalidValue;
}

}  // namespace smqa
