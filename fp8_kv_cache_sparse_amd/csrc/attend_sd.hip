// Sparse multi-query attention, split over the latent dimension inside a workgroup
// (vLLM blog "DeepSeek-V4.1-Flash sur vLLM": section "Kernels", MegaAttention reading the
// compressed FP4 KV; section "SWA bounded replay", the FP8 window of the last 128
// positions and its clip at the replay start; section "Performances agentiques", one KV
// latent shared by every head, so K = V = the latent row).
//
// A workgroup (8 waves, one per 2 SIMD slots) owns one query, 32 heads and a contiguous
// range of tiles: ceil(k/32) tiles of 32 selected FP4 rows, then the 16-row tiles of FP8
// window rows that overlap the query's visible window.  Wave w owns a contiguous run of
// 32-dim latent blocks (the E8M0 block size) for both products, so every dequantised
// value feeds 32 heads of MFMA work and no wave converts a value another wave needs.
//
//   gather   global_load_lds_dwordx4 straight into one of four LDS tile buffers (rows
//            padded so both read patterns below are bank-conflict free), issued by all 8
//            waves (waves 0-3 before their products, waves 4-7 after them); the raw E8M0
//            bytes and the row scales land beside them.  Tile i+2 is in flight while tile
//            i is scored and tile i-1 is accumulated; a workgroup with at most four tiles
//            (short contexts split over many workgroups) gathers all of them at once, so
//            it waits for memory once instead of once per tile.
//   q        staged through the idle tile buffers with coalesced direct-to-LDS loads, in
//            the same round trip as the positions of the first tiles, then read into the
//            MFMA operand registers.
//   Q.K^T    v_mfma_f32_32x32x16_bf16, heads x rows: each lane reads 8 dims of one row
//            (ds_read_b32 for E2M1, ds_read_b64 for E4M3) and converts them exactly to
//            bf16 with the block's E8M0 scale (v_cvt_scalef32_pk_bf16_*); q stays in
//            registers.  Each wave's partial logits over its blocks go to LDS.
//   softmax  every wave sums the 8 partials of 4 heads, applies tau * log2(e) and the row
//            scale and updates the exact running max (so the largest P of a head is exactly
//            1 in fp16); the accumulators of a group of 8 heads are rescaled only when one
//            of their maxima moved.
//   P.V      v_mfma_f32_32x32x16_f16, heads x dims: the B operand (8 rows of one dim per
//            lane) comes straight from the row-major tile through the LDS transpose reads
//            ds_read_b64_tr_b4 (E2M1: 16 rows of one dim per lane) and ds_read_b64_tr_b8
//            (E4M3), is converted to fp16 with scale 1 and multiplied by the rows' block
//            scales (v_pk_mul_f16: the scale is exact in fp16 for -24 <= e - 127 <= 15, the
//            product for -23 <= e - 127 <= 13); P carries the row scale rho (or sigma).
//
// Two more global-cache formats take the same pipeline.  FP8 rows (E4M3 with a row scale,
// the format the FP4 cache replaced) come in 16-row tiles that take the window tiles'
// products.  NVFP4 (E2M1 with an E4M3 scale per 16 elements and a tensor scale; CocoLoop
// digest, section "Les particularités du modèle lui-même") keeps the 32-row E2M1 tiles; its
// scale dwords land block-major ([dword][row]) so that Q.K^T reads one byte per lane and
// P.V the 16 rows of a transpose read from 64 contiguous bytes, paired by v_perm.  Both
// products multiply fp16 codes (converted with scale 1) by the fp16 block scale, exactly;
// the scaled conversions are meant for power-of-two (E8M0) scales and are not trusted with
// an E4M3 one.  Q.K^T then runs on fp16 MFMA, q converted to fp16 once.
//
// Several tile ranges of one (query, head group) leave unnormalised partials that
// attend_merge_kernel combines by log-sum-exp.
//
// kMXS (decode_step on dense rows of at most kSelCols columns, D = 1664): instead of reading
// the positions of its tiles, every workgroup of a query loads the query's scores and
// computes the whole top-k itself (the selection topk_select makes, bit for bit) before its
// first gather; the first workgroup of the query writes the selection out.  The step then has
// no top-k launch, and q is staged into LDS while the selection runs.
#include <type_traits>

#include "common.h"

namespace smqa {

hipError_t launch_attend_merge(const AttendArgs& a, int S, hipStream_t s);

namespace sd {

// fp64 -> bf16 bits, rounded once to the nearest bf16 (ties to even).  A normal bf16 keeps 8
// significant bits, i.e. drops the low 45 of the fp64 significand: an integer
// round-half-even at bit 45 (a carry moves into the exponent, as it should).  Below 2^-126
// the bf16 grid is the subnormal one, spacing 2^-133.  The result is exact in fp32.
__device__ __forceinline__ unsigned bf16_rne(double y) {
  if (__builtin_fabs(y) < 0x1p-126) y = __builtin_rint(y * 0x1p133) * 0x1p-133;
  unsigned long long u = (unsigned long long)__double_as_longlong(y);
  u = (u + 0x0FFFFFFFFFFFull + ((u >> 45) & 1ull)) & ~0x1FFFFFFFFFFFull;
  return __float_as_uint((float)__longlong_as_double((long long)u)) >> 16;
}


typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

constexpr int kThreads = 512;
constexpr int kRows = 32;     // selected global rows per tile
constexpr int kWRows = 16;    // window rows per tile
constexpr int kNBuf = 4;      // tile buffers in LDS: tiles i-1 (P.V), i (Q.K^T), i+1, i+2 in flight

constexpr int align16(int x) { return (x + 15) & ~15; }

// Global cache formats: MX FP4 (E2M1, E8M0 per 32, fp32 row scale), FP8 rows (E4M3, row
// scale) and NVFP4 (E2M1, E4M3 per 16, row scale, fp32 tensor scale).
// MegaAttention's fused form over the MX format has two instantiations of its own (so the
// plain kernel keeps its registers and neither ends in a branch between two epilogues):
// kMXF, query RoPE and the FP8 epilogue in the kernel (one split), and kMXR, query RoPE
// with split partials for attend_fused_epilogue_kernel.
// kMXN: the MX format with Q.K^T on the scaled matrix cores (v_mfma_scale_f32_32x32x64_
// f8f6f4): the query is quantised to MXFP8 in the prologue, the gathered E2M1 codes and their
// E8M0 bytes are the B operand and its scale as they sit in LDS, window rows are E4M3 with
// scale 2^0; P.V is the MX one.
constexpr int kMX = kKvMX, kFP8 = kKvFP8, kNV = kKvNV, kMXF = kKvMXF, kMXR = kKvMXR, kMXN = kKvMXN;
constexpr int kMXS = kKvMXS;
constexpr bool mx_like(int F) { return F == kMX || F == kMXF || F == kMXR || F == kMXN || F == kMXS; }

// LDS geometry for latent width D and global format F (compile time, so every offset is an
// immediate).
template <int D, int F>
struct Geo {
  static constexpr int NB = D / 32;                 // 32-dim blocks
  static constexpr int BPW = NB / 8;                // blocks of every wave
  static constexpr int EXTRA = NB % 8;              // waves 0..EXTRA-1 own one more (0 or 4)
  static constexpr int NBW = BPW + (EXTRA ? 1 : 0); // most blocks of one wave
  static constexpr int RS4 = D / 2 + 16;            // E2M1 row stride (16 * odd dwords / 4)
  static constexpr int RS8 = D + 16;                // E4M3 row stride
  static constexpr int E8S = D / 32;                // raw E8M0 bytes per row (MX)
  static constexpr int NQ = D / 64;                 // dwords of E4M3 block scales per row (NV)
  // one tile buffer: codes | block scales | row scales [4 loader waves][8]; the block scales
  // are the raw E8M0 bytes [32 rows][E8S] (MX) or the E4M3 scale dwords [NQ][32 rows] (NV,
  // block-major, so the 16 rows of one transpose read are 64 contiguous bytes)
  static constexpr int CODES = kRows * RS4;
  static constexpr int E8 = CODES;
  static constexpr int RHO = align16(E8 + (F == kNV ? NQ * kRows * 4 : kRows * E8S));
  static constexpr int BUF = align16(RHO + kRows * 4);
  // shared areas after the buffers
  static constexpr int RING = kNBuf * BUF;                      // positions [4][32]
  static constexpr int SCHN = mx_like(F) ? NB * 16 : 16;       // u32 per slot: MX f16 scale pairs
  static constexpr int SCH = RING + kNBuf * kRows * 4;          // [2][SCHN]: scale pairs / row masks
  static constexpr int RED = SCH + 2 * SCHN * 4;                // [8 waves][32 heads][32 rows] f32
  static constexpr int PS = RED + 8 * 32 * kRows * 4;           // P [32 heads][40] f16
  static constexpr int RI = PS + 32 * 40 * 2;                   // logit scale[32], P scale[32]
  static constexpr int MR = RI + 2 * 32 * 4;                    // mref[32] alpha[32] lsum[32]
  static constexpr int LDS = MR + 3 * 32 * 4;
  // global loads a loader wave issues per tile (fixed, so vmcnt can wait for the older tile)
  static constexpr int PIECES8 = D / 16;                        // 16-byte pieces of an E4M3 row
  static constexpr int NSC = F == kNV ? (D / 128 + 7) / 8 : 1;  // block-scale loads per wave
  static constexpr int NLOAD4 = kRows / 8 + NSC + 1;            // 4 code rows, block scales, rho
  static constexpr int NLOAD8 = (kWRows / 8) * (PIECES8 > 64 ? 2 : 1) + 1;  // 2 rows, sigma
  static_assert(kWRows * RS8 <= CODES, "a window tile must fit a buffer");
  static_assert(EXTRA == 0 || EXTRA == 4, "D must be a multiple of 128");
  static_assert(LDS <= 160 * 1024, "LDS budget");
  static_assert(32 * D <= kNBuf * BUF, "the fused epilogue stages 32 rows of FP8 codes in the tile buffers");
};

struct Ctx {
  int k, W;
  int ng, wt0, tb, te, gx1;
  int b, p, lo_win, pos0, jmax;
  int64_t base;
  float lscale;
};

template <class T>
__device__ __forceinline__ T lds(const uint8_t* p) { return *(const T*)p; }

__device__ __forceinline__ v8bf cvt8_fp4_bf16(unsigned wd, float scl) {
  v4u u;
  u.x = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, scl, 0));
  u.y = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, scl, 1));
  u.z = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, scl, 2));
  u.w = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, scl, 3));
  return __builtin_bit_cast(v8bf, u);
}

__device__ __forceinline__ v8bf cvt8_fp8_bf16(v2u w) {
  v4u u;
  u.x = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, false));
  u.y = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, true));
  u.z = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, false));
  u.w = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, true));
  return __builtin_bit_cast(v8bf, u);
}

// E2M1 nibble pair `sel` of wd (two consecutive rows after a transpose read), exact fp16.
__device__ __forceinline__ v2h fp4x2_f16(unsigned wd, int sel) {
  switch (sel) {
    case 0: return __builtin_bit_cast(v2h, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd, 1.0f, 0));
    case 1: return __builtin_bit_cast(v2h, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd, 1.0f, 1));
    case 2: return __builtin_bit_cast(v2h, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd, 1.0f, 2));
    default: return __builtin_bit_cast(v2h, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd, 1.0f, 3));
  }
}

// s_waitcnt with only the vector-memory counter bounded (gfx9 encoding: vmcnt in bits 3:0,
// expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// An opaque copy of a per-lane value: re-deriving lane offsets inside each stage keeps the
// compiler from hoisting dozens of loop-invariant addresses into registers.
__device__ __forceinline__ int opq(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
// Reduction over each 16-lane row: quad swaps, half-row mirror, row mirror (DPP).
template <bool MAX>
__device__ __forceinline__ float row_reduce(float v) {
  auto op = [](float x, float y) { return MAX ? fmaxf(x, y) : x + y; };
  v = op(v, dpp_f<0xB1>(v));                      // quad_perm [1,0,3,2]
  v = op(v, dpp_f<0x4E>(v));                      // quad_perm [2,3,0,1]
  v = op(v, dpp_f<0x141>(v));                     // row_half_mirror
  v = op(v, dpp_f<0x140>(v));                     // row_mirror
  return v;
}

// One tile of global loads straight into LDS (global_load_lds: each lane's bytes land at
// the wave-uniform LDS address M0 + lane * size).  Written as inline assembly so that the
// compiler does not treat every later LDS read as possibly aliasing an in-flight load (it
// would wait for all of them, the prefetch included); the kernel bounds the vector-memory
// counter itself before the barrier that publishes a tile.  Every wave issues a fixed
// number of these per tile kind; rows that take no part read a harmless in-bounds dummy
// (the query's own q row) instead of being skipped.
__device__ __forceinline__ void gload16(const void* src, unsigned m0) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(m0) : "memory");
}
__device__ __forceinline__ void gload4(const void* src, unsigned m0) {
  asm volatile("global_load_lds_dword %0, off" ::"v"(src), "{m0}"(m0) : "memory");
}

// The per-query values: q_pos[t], swa_clip[t] and the sequence of query t (the largest b
// with q_start[b] <= t) with its seq_start (both ends) and swa_pos0 entries, by a 64-way
// search: each lane reads one sample of the arrays, so for B <= 64 everything arrives in a
// single round trip to memory.
struct SeqInfo {
  int b;
  int64_t base;
  int len;
  int pos0;
  int p;
  int clip;
};
__device__ __forceinline__ SeqInfo locate_seq(const AttendArgs& a, int t, int lane) {
  int lo = 0, hi = a.B;
  const int extra = lane == 0 ? a.q_pos[t] : (lane == 1 && a.swa_clip ? a.swa_clip[t] : 0);
  for (;;) {
    const int step = (hi - lo + 63) / 64;
    const int idx = lo + lane * step;
    const bool in = idx < hi;
    const int qs = in ? a.q_start[idx] : 0;
    const int64_t ss = in ? a.seq_start[idx] : 0;
    const int64_t se = in ? a.seq_start[idx + 1] : 0;
    const int p0 = in ? a.swa_pos0[idx] : 0;
    asm volatile("" ::"v"(qs), "v"(ss), "v"(se), "v"(p0), "v"(extra));   // one wait for all five loads
    const int L = max(__builtin_popcountll(__builtin_amdgcn_ballot_w64(in && qs <= t)) - 1, 0);
    if (step == 1) {
      SeqInfo r;
      r.b = lo + L;
      const uint64_t u = (uint64_t)ss;
      r.base = (int64_t)(((uint64_t)(unsigned)__builtin_amdgcn_readlane((int)(u >> 32), L) << 32) |
                         (unsigned)__builtin_amdgcn_readlane((int)u, L));
      const uint64_t ue = (uint64_t)se;
      const int64_t end = (int64_t)(((uint64_t)(unsigned)__builtin_amdgcn_readlane((int)(ue >> 32), L) << 32) |
                                    (unsigned)__builtin_amdgcn_readlane((int)ue, L));
      r.len = (int)(end - r.base);
      r.pos0 = __builtin_amdgcn_readlane(p0, L);
      r.p = __builtin_amdgcn_readlane(extra, 0);
      r.clip = __builtin_amdgcn_readlane(extra, 1);
      return r;
    }
    lo += L * step;
    hi = min(lo + step, hi);
  }
}

// F = kFP8: the global cache holds E4M3 rows with a row scale (the FP8 cache the FP4 format
// replaced); its tiles are then 16 gathered rows that take the window tiles' products.
// F = kNV: E2M1 with an E4M3 scale per 16 elements (a.kv_e8m0 points at them) and the
// tensor scale a.kv_gscale; the tiles are those of the MX format.
template <int D, int F>
__global__ __launch_bounds__(kThreads) void attend_kernel(AttendArgs a, int S, int ngroups, int total) {
  using G = Geo<D, F>;
  constexpr bool G8 = F == kFP8, NV = F == kNV;
  // kMXS: the workgroup takes the query's selection from its scores itself (below) instead of
  // reading positions; every range then holds at most kNBuf tiles (checked by the caller)
  constexpr bool SEL = F == kMXS;
  constexpr int GR = G8 ? kWRows : kRows;         // global rows per tile
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  // Per-lane roles (re-derived from an opaque lane id inside each stage):
  //   r32 = lane & 31, kh = lane >> 5    MFMA 32x32 operand lane: column / k-half
  //   i16 = lane & 15, hh = lane >> 4 & 1 transpose-read lane, dim half of a block
#define SMQA_LANE_ROLES                                                                   \
  const int ln_ = opq(lane);                                                              \
  const int r32 = ln_ & 31, kh = ln_ >> 5, i16 = ln_ & 15, hh = (ln_ >> 4) & 1;          \
  (void)r32; (void)kh; (void)i16; (void)hh;

  // XCD-aware order: workgroups are dealt to the 8 XCDs round-robin, so logical block
  // (bid & 7) * (nb / 8) + (bid >> 3) keeps runs of consecutive logical blocks on one XCD;
  // the head groups of one query (same rows) are consecutive and share that XCD's L2.
  const int nb = gridDim.x;
  const int bid = blockIdx.x;
  const int logical = (bid & 7) * (nb >> 3) + (bid >> 3);
  if (logical >= total) return;
  const int grp = __builtin_amdgcn_readfirstlane(logical % ngroups);
  const int split = __builtin_amdgcn_readfirstlane((logical / ngroups) % S);
  const int t = __builtin_amdgcn_readfirstlane(logical / (S * ngroups));
  const int h0 = grp * 32;

  // Tile ranges are cut from the largest possible tile count (every window tile of the
  // ring), so a split's global tiles, and the positions of its first ones, are known
  // before any per-query value has been read; the window part of a range is clipped to
  // the query's visible window once those values arrive.
  Ctx c;
  c.k = a.k;
  c.W = a.W;
  c.lscale = a.sm_scale * kLog2e;
  c.ng = (c.k + GR - 1) / GR;
  const int nominal = c.ng + (c.W + kWRows - 1) / kWRows;
  c.tb = (int)((int64_t)split * nominal / S);
  c.te = (int)((int64_t)(split + 1) * nominal / S);
  c.gx1 = min(min(c.te, c.ng) * GR, c.k);          // global rows of this split end here

  float* mref = (float*)(smem + G::MR);
  float* malpha = mref + 32;
  float* mlsum = mref + 64;
  float* rl = (float*)(smem + G::RI);
  float* rp = rl + 32;
  const uint8_t* dummy = (const uint8_t*)(a.q + (int64_t)t * a.Hq * D);
  // LDS byte address of a location in the dynamic array (the M0 operand of the loads): the
  // dynamic array starts right after the kernel's static LDS
  auto lds_addr = [&](const uint8_t* p) __attribute__((always_inline)) -> unsigned {
    return __builtin_amdgcn_readfirstlane(__builtin_amdgcn_groupstaticsize() + (unsigned)(p - smem));
  };

  // wave w's blocks [b0, b0 + BPW + (w < EXTRA))
  const int b0 = wave * G::BPW + min(wave, G::EXTRA);
  // the query's sequence in the latent cache (set by the prologue)
  const uint8_t* codes_base = nullptr;
  const uint8_t* e8_base = nullptr;
  const float* rho_base = nullptr;

  // ---- loads of one tile: positions (into the ring) and rows (into a buffer).  Every wave
  // loads rows 8u + wave of the tile, so the loads of a tile are spread over all 8 waves.
  auto load_pos = [&](int tile, int rslot) __attribute__((always_inline)) {       // wave 0, lanes 0..GR-1
    const int ln = opq(lane);
    const int x = tile * GR + (ln & 31);
    const void* src = x < c.gx1 ? (const void*)(a.idx + (int64_t)t * c.k + x) : (const void*)dummy;
    if (ln < GR) gload4(src, lds_addr(smem + G::RING + rslot * kRows * 4));
  };
  auto issue = [&](int tile, int slot, int rslot) __attribute__((always_inline)) {
    const int ln = opq(lane);
    uint8_t* B = smem + slot * G::BUF;
    if (tile < c.ng) {
      if constexpr (G8) {
        // FP8 global tile: rows 8u + wave, u = 0..1, gathered by position; the row scales
        // of rows 8u + wave, u = lane < 2 -> RHO[wave][u]
        const int* pos = (const int*)(smem + G::RING) + rslot * kRows;
        const int xt = tile * kWRows;
        const int pall = pos[ln & 15];
        const int rr = 8 * (ln & 1) + wave;
        const int pr = pos[rr];
#pragma unroll
        for (int u = 0; u < kWRows / 8; ++u) {
          const int r = 8 * u + wave;
          const int j = __builtin_amdgcn_readlane(pall, r);
          const bool ok = (xt + r < c.gx1) & takes_part(j, c.jmax);
          const uint8_t* src = ok ? codes_base + (int64_t)j * D : dummy;
          if (ln < (G::PIECES8 < 64 ? G::PIECES8 : 64)) gload16(src + 16 * ln, lds_addr(B + r * G::RS8));
          if constexpr (G::PIECES8 > 64) {
            if (ln < G::PIECES8 - 64) gload16(src + 1024 + 16 * ln, lds_addr(B + r * G::RS8 + 1024));
          }
        }
        const bool ok = a.kv_rowscale && xt + rr < c.gx1 && takes_part(pr, c.jmax);
        const void* src = ok ? (const void*)(rho_base + pr) : (const void*)dummy;
        if (ln < 2) gload4(src, lds_addr(B + G::RHO + 16 * wave));
      } else {
        constexpr int per_row = D / 128;              // E8M0 dwords per row
        const int* pos = (const int*)(smem + G::RING) + rslot * kRows;
        const int xt = tile * kRows;
        // every position this wave needs, read before one wait: all 32 (for the code rows),
        // the rows of its E8M0 load, the rows of its rho lanes
        const int pall = pos[ln & 31];
        const int re = 4 * wave + ln / per_row;
        const int pe = pos[re & 31];
        const int rr = 8 * (ln & 3) + wave;
        const int pr = pos[rr];
        // code rows 8u + wave, u = 0..3.  Lane r (r < 32) forms row r's source address once
        // (the dummy row when the row takes no part), so a row's load costs two readlanes
        // instead of a scalar bounds check and 64-bit multiply per row.
        {
          const bool okl = (xt + (ln & 31) < c.gx1) & takes_part(pall, c.jmax);
          const uint64_t al = (uint64_t)(okl ? codes_base + (int64_t)pall * (D / 2) : dummy);
          const unsigned alo = (unsigned)al, ahi = (unsigned)(al >> 32);
#pragma unroll
          for (int u = 0; u < kRows / 8; ++u) {
            const int r = 8 * u + wave;
            // (readlane returns int: both halves widen through unsigned, so the low word is
            // not sign-extended into the high one)
            const uint64_t ar = ((uint64_t)(unsigned)__builtin_amdgcn_readlane(ahi, r) << 32) |
                                (uint64_t)(unsigned)__builtin_amdgcn_readlane(alo, r);
            if (ln < D / 32) gload16((const uint8_t*)ar + 16 * ln, lds_addr(B + r * G::RS4));
          }
        }
        if constexpr (NV) {
          // E4M3 scale dwords q = 2m + lane / 32 of row lane % 32 -> table[q][row]: D/128
          // loads of 64 lanes per tile, dealt round the waves (the surplus repeat a load
          // another wave makes: same bytes to the same place)
          const int row = ln & 31;
          const bool ok = (xt + row < c.gx1) & takes_part(pall, c.jmax);
#pragma unroll
          for (int u = 0; u < G::NSC; ++u) {
            const int m = (wave + 8 * u) % (D / 128);
            const int q = 2 * m + (ln >> 5);
            const uint8_t* src = ok ? e8_base + (int64_t)pall * (D / 16) + 4 * q : dummy;
            gload4(src, lds_addr(B + G::E8 + 2 * m * kRows * 4));
          }
        } else {  // raw E8M0: rows 4 wave .. +4, contiguous
          const int dd = ln % per_row;
          const bool ok = xt + re < c.gx1 && takes_part(pe, c.jmax);
          const uint8_t* s0 = ok ? e8_base + (int64_t)pe * (D / 32) : dummy;
          if (ln < 4 * per_row) gload4(s0 + 4 * dd, lds_addr(B + G::E8 + 4 * wave * G::E8S));
        }
        {  // rho of rows 8u + wave, u = lane < 4 -> RHO[wave][u]
          const bool ok = a.kv_rowscale && xt + rr < c.gx1 && takes_part(pr, c.jmax);
          const void* src = ok ? (const void*)(rho_base + pr) : (const void*)dummy;
          if (ln < 4) gload4(src, lds_addr(B + G::RHO + 16 * wave));
        }
      }
    } else {
      // window tile: rows 8u + wave, u = 0..1; D/16 pieces of 16 bytes per row (two loads
      // when > 64)
      const int wt = c.wt0 + tile - c.ng;
#pragma unroll
      for (int u = 0; u < kWRows / 8; ++u) {
        const int r = 8 * u + wave;
        const int uu = kWRows * wt + r;
        const uint8_t* src = uu < c.W ? a.swa + ((int64_t)c.b * c.W + uu) * D : dummy;
        if (ln < (G::PIECES8 < 64 ? G::PIECES8 : 64)) gload16(src + 16 * ln, lds_addr(B + r * G::RS8));
        if constexpr (G::PIECES8 > 64) {
          if (ln < G::PIECES8 - 64) gload16(src + 1024 + 16 * ln, lds_addr(B + r * G::RS8 + 1024));
        }
      }
      {  // sigma of rows 8u + wave, u = lane < 2 -> RHO[wave][u]
        const int uu = kWRows * wt + 8 * (ln & 1) + wave;
        const bool ok = a.swa_scale && uu < c.W;
        const void* src = ok ? (const void*)(a.swa_scale + (int64_t)c.b * c.W + uu) : (const void*)dummy;
        if (ln < 2) gload4(src, lds_addr(B + G::RHO + 16 * wave));
      }
    }
  };

  // ---- prologue: positions of the first three tiles, q and the per-query values (one
  // round trip), then the rows of the first two tiles
  if (!SEL && wave == 0) {
    for (int u = 0; u < kNBuf; ++u)
      if (c.tb + u < c.te && c.tb + u < c.ng) load_pos(c.tb + u, u);
  }
  constexpr int NP = (G::NBW + 1) / 2;
  v8i qf[NP];
  int qsc[NP];
  v8bf qa[G::NBW][2];
  // q of the 32 heads: staged in LDS by coalesced loads (rows QS bytes apart: 16 mod 256, so
  // the per-lane 16-byte reads below hit 16 distinct bank quads per 16 lanes), except for the
  // fused RoPE forms, whose rotation tables are read beside q straight from global memory.
  // qget: the 8 bf16 from element e of head h0 + r32's dims 16 kh ..
  constexpr bool QLDS = !(F == kMXF || F == kMXR);
  constexpr int QS = 2 * D + 16;
  static_assert(32 * QS <= kNBuf * G::BUF, "q is staged in the idle tile buffers");
  auto qget = [&](int r32, int kh, int e) __attribute__((always_inline)) -> v4u {
    if constexpr (QLDS) return lds<v4u>(smem + r32 * QS + 32 * kh + 2 * e);
    else return *(const v4u*)(a.q + ((int64_t)t * a.Hq + h0 + r32) * D + 16 * kh + e);
  };
  auto build_q = [&]() __attribute__((always_inline)) {
    // kMXN: the query as the fp8 A operand of the scaled MFMA, one register octet per pair of
    // this wave's blocks (K-block 0 = b0 + 2j, K-block 1 = b0 + 2j + 1).  Lane (r32, kh) holds
    // dims 32 bA + 16 kh .. +16 of head h0 + r32 in bytes 0..15 and 32 bB + 16 kh .. +16 in
    // bytes 16..31, and supplies the E8M0 scale of K-block kh (the instruction takes K-block
    // b's scale from lane r32 + 32 b).  OCP MXFP8: E = floor(log2 amax) - 8 + 127 per 32-dim
    // block (clamped at 0; 0 for a zero block), elements E4M3(x / 2^(E-127)), nearest even,
    // saturated at 448.  A block's 32 values are split over lanes l and l ^ 32.
    if constexpr (F == kMXN) {
      SMQA_LANE_ROLES
      const int nbw = G::BPW + (wave < G::EXTRA ? 1 : 0);
  #pragma unroll
      for (int j = 0; j < NP; ++j) {
        v4u raw[2][2];
        int ex[2];
  #pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const bool ok = 2 * j + hb < nbw;
          const int e0 = 32 * (b0 + 2 * j + hb);
          raw[hb][0] = ok ? qget(r32, kh, e0) : v4u{0u, 0u, 0u, 0u};
          raw[hb][1] = ok ? qget(r32, kh, e0 + 8) : v4u{0u, 0u, 0u, 0u};
          unsigned m = 0u;                             // |x| as bf16 magnitude bits
  #pragma unroll
          for (int pc = 0; pc < 2; ++pc)
  #pragma unroll
            for (int e = 0; e < 4; ++e) m = max(m, max(raw[hb][pc][e] & 0x7FFFu, (raw[hb][pc][e] >> 16) & 0x7FFFu));
          m = max(m, (unsigned)__shfl_xor((int)m, 32));
          // floor(log2 amax) + 127 is the bf16 exponent field (normal amax); subnormal or zero
          // blocks give E = 0
          ex[hb] = max((int)(m >> 7) - 8, 0);
        }
        qsc[j] = kh ? ex[1] : ex[0];
  #pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const float mul = e8m0_to_float(254 - ex[hb]);   // 2^(127 - E), exact scaling
  #pragma unroll
          for (int dd = 0; dd < 4; ++dd) {
            const unsigned w0 = raw[hb][dd >> 1][2 * (dd & 1)], w1 = raw[hb][dd >> 1][2 * (dd & 1) + 1];
            auto q8 = [&](unsigned bits) {
              return __builtin_amdgcn_fmed3f(__uint_as_float(bits) * mul, -448.0f, 448.0f);
            };
            int wd = __builtin_amdgcn_cvt_pk_fp8_f32(q8(w0 << 16), q8(w0 & 0xFFFF0000u), 0, false);
            wd = __builtin_amdgcn_cvt_pk_fp8_f32(q8(w1 << 16), q8(w1 & 0xFFFF0000u), wd, true);
            qf[j][4 * hb + dd] = wd;
          }
        }
      }
    }
    // A operands of Q.K^T: head h0 + r32, dims 32 b + 16 kh + 8 cc .. +8 of block b = b0 + i
    if constexpr (F != kMXN) {
      SMQA_LANE_ROLES
  #pragma unroll
      for (int i = 0; i < G::NBW; ++i)
  #pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          v4u v = {0u, 0u, 0u, 0u};
          if (i < G::BPW || wave < G::EXTRA) v = qget(r32, kh, 32 * (b0 + i) + 8 * cc);
          if constexpr (F == kMXF || F == kMXR) {
            // fused query RoPE (blog §Kernels, MegaAttention): the pairs (2j, 2j+1) of the last
            // 2 * rope_pairs dims rotate by query t's angle, rounded once to bf16 (RNE).  In
            // fp64 the products of a bf16 and an fp32 value are exact, so each output is the
            // exact rotation rounded once to fp64 and then once to bf16.
            const int r0 = D - 2 * a.rope_pairs;
            const int d0 = 32 * (b0 + i) + 16 * kh + 8 * cc;
            if (a.rope_pairs > 0 && d0 >= r0 && (i < G::BPW || wave < G::EXTRA)) {
              const int64_t pj = (int64_t)t * a.rope_pairs + (d0 - r0) / 2;
              const v4f cs = *(const v4f*)(a.rope_cos + pj);
              const v4f sn = *(const v4f*)(a.rope_sin + pj);
  #pragma unroll
              for (int j = 0; j < 4; ++j) {
                const double x0 = __uint_as_float(v[j] << 16), x1 = __uint_as_float(v[j] & 0xFFFF0000u);
                const double c = cs[j], sj = sn[j];
                const double y0 = __builtin_fma(x0, c, -(x1 * sj));
                const double y1 = __builtin_fma(x0, sj, x1 * c);
                v[j] = bf16_rne(y0) | (bf16_rne(y1) << 16);
              }
            }
          }
          if constexpr (NV) {
            // NVFP4 scores in fp16: bf16 -> fp16 is exact for 2^-14 <= |q| <= 65504
            v8h h;
  #pragma unroll
            for (int j = 0; j < 4; ++j) {
              h[2 * j] = (_Float16)__uint_as_float(v[j] << 16);
              h[2 * j + 1] = (_Float16)__uint_as_float(v[j] & 0xFFFF0000u);
            }
            qa[i][cc] = __builtin_bit_cast(v8bf, h);
          } else {
            qa[i][cc] = __builtin_bit_cast(v8bf, v);
          }
        }
    }
  };
  auto stage_q = [&]() __attribute__((always_inline)) {
    // rows 8 rr + wave, 16-byte piece pc = 64 jj + lane of each (the tail instruction of a
    // row runs on fewer lanes)
    constexpr int QP = D / 8;
    const uint8_t* qsrc = (const uint8_t*)(a.q + ((int64_t)t * a.Hq + h0) * D);
    const int ln = opq(lane);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int r = 8 * rr + wave;
#pragma unroll
      for (int jj = 0; jj < (QP + 63) / 64; ++jj) {
        const int pc = 64 * jj + ln;
        if (pc < QP) gload16(qsrc + (int64_t)r * 2 * D + 16 * pc, lds_addr(smem + r * QS + 1024 * jj));
      }
    }
  };
  // kMXS stages q after its scores and the sequence lookup have arrived, so the select starts
  // on them while q is still in flight (the q copies land where the select does not work)
  if constexpr (QLDS) {
    if constexpr (!SEL) stage_q();
  } else {
    build_q();
  }
  // kMXS: the query's scores, columns tid + 512 u, requested first (q follows the sequence
  // lookup)
  constexpr int kSPer = kSelCols / kThreads;
  float sv[SEL ? kSPer : 1];
  if constexpr (SEL) {
    const float* srow = a.sel_scores + (int64_t)t * a.sel_ld;
#pragma unroll
    for (int u = 0; u < kSPer; ++u) {
      const int col = tid + kThreads * u;
      sv[u] = col < a.sel_max_ctx ? srow[col] : -__builtin_inff();
    }
  }
  {
    const SeqInfo si = locate_seq(a, t, lane);
    c.b = si.b;
    c.base = si.base;
    codes_base = a.kv_codes + si.base * (G8 ? D : D / 2);
    e8_base = G8 ? nullptr : a.kv_e8m0 + si.base * (NV ? D / 16 : D / 32);
    rho_base = a.kv_rowscale ? a.kv_rowscale + si.base : nullptr;
    c.pos0 = si.pos0;
    c.p = si.p;
    c.jmax = min(si.p, si.len - 1);
    c.lo_win = max(max(c.p - c.W + 1, 0), si.clip);
  }
  if constexpr (SEL && QLDS) stage_q();
  if (tid < 32) {
    mref[tid] = -__builtin_inff();
    malpha[tid] = 1.0f;
  }
  {
    const int u_lo = max(c.lo_win - c.pos0, 0);
    const int u_hi = min(c.p - c.pos0, c.W - 1);
    c.wt0 = u_lo / kWRows;
    const int nwt = u_lo <= u_hi ? u_hi / kWRows - c.wt0 + 1 : 0;
    c.te = min(c.te, c.ng + nwt);
    c.tb = min(c.tb, c.te);
  }
  const int tb = c.tb, te = c.te;
  // a range of at most kNBuf tiles is gathered at once (one memory latency for all of it),
  // a longer one two tiles ahead of the products
  const bool pre = te - tb <= kNBuf;
  if constexpr (!SEL) __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if constexpr (SEL) {
    // The query's top-k as topk_select takes it (the k largest scores of columns 0 ..
    // min(p, len - 1), ties to the lower column, -1 past the valid columns), computed by every
    // workgroup of the query: 11-bit radix digits after the bits every valid key shares, then
    // one block scan of packed (ties, greater) counts gives each thread the output offsets of
    // its 16 consecutive columns.  The positions of this range's tiles go to the ring; the
    // first workgroup of the query also writes the selection out.  LDS: keys in the logits
    // area, the histogram past the staged q, counters in the P area (all idle until the
    // first tile).
    static_assert(kSelCols * 4 <= 8 * 32 * kRows * 4, "the keys fit the logits area");
    static_assert(32 * QS + 2048 * 4 <= kNBuf * G::BUF, "the histogram fits past the staged q");
    unsigned* keys = (unsigned*)(smem + G::RED);
    unsigned* hist = (unsigned*)(smem + 32 * QS);
    int* scr = (int*)(smem + G::PS);                 // partials [3][8], scan [8], sh [4]
    int* scan = scr + 24;
    int* sh = scr + 32;
    int* ring = (int*)(smem + G::RING);
    const int ncols = max(0, min(c.jmax + 1, a.sel_max_ctx));
#pragma unroll
    for (int u = 0; u < kSPer; ++u) {
      const int col = tid + kThreads * u;
      keys[col] = col < ncols ? score_key(sv[u]) : 0u;
    }
    for (int i = tid; i < 2048; i += kThreads) hist[i] = 0u;
    if (tid < kNBuf * kRows) ring[tid] = -1;
    __syncthreads();
    unsigned key[kSPer];
#pragma unroll
    for (int u = 0; u < kSPer; u += 4) {
      const v4u k4 = *(const v4u*)(keys + kSPer * tid + u);
      key[u] = k4.x;
      key[u + 1] = k4.y;
      key[u + 2] = k4.z;
      key[u + 3] = k4.w;
    }
    const int c0 = kSPer * tid;
    // valid count and the min / max valid key (min as the max of ~key)
    int cnt = 0;
    unsigned nlo = 0u, hi = 0u;
#pragma unroll
    for (int u = 0; u < kSPer; ++u) {
      cnt += key[u] != 0u;
      nlo = key[u] ? max(nlo, ~key[u]) : nlo;
      hi = max(hi, key[u]);
    }
    cnt = wave_inclusive_sum(cnt);
    nlo = wave_inclusive_max(nlo);
    hi = wave_inclusive_max(hi);
    if (lane == 63) {
      scr[wave] = cnt;
      scr[8 + wave] = (int)nlo;
      scr[16 + wave] = (int)hi;
    }
    __syncthreads();
    int nvalid = 0;
    nlo = 0u;
    hi = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      nvalid += scr[i];
      nlo = max(nlo, (unsigned)scr[8 + i]);
      hi = max(hi, (unsigned)scr[16 + i]);
    }
    const unsigned lo = ~nlo;
    unsigned tau = 1u;                               // every valid key is >= 1
    int tie_need = kSelCols;
    if (nvalid > a.k) {
      int nbits = lo == hi ? 32 : __clz((int)(lo ^ hi));
      unsigned prefix = nbits == 32 ? lo : (nbits == 0 ? 0u : (lo >> (32 - nbits)) << (32 - nbits));
      int need = a.k;
      bool whole_bin = false;
      while (nbits < 32) {
        const int dbits = min(11, 32 - nbits);
        const int shift = 32 - nbits - dbits;
        const unsigned dmask = (1u << dbits) - 1u;
#pragma unroll
        for (int u = 0; u < kSPer; ++u) {
          const bool match = key[u] != 0u && (nbits == 0 || (key[u] >> (32 - nbits)) == (prefix >> (32 - nbits)));
          if (match) atomicAdd(&hist[(key[u] >> shift) & dmask], 1u);
        }
        __syncthreads();
        // thread i holds bins 2047 - 4i .. 2044 - 4i (counting down with the thread index, so
        // a prefix sum counts the keys above)
        int hb[4], local = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          hb[j] = (int)hist[2047 - 4 * tid - j];
          local += hb[j];
        }
        const int incl = wave_inclusive_sum(local);
        if (lane == 63) scan[wave] = incl;
        if (tid == 0) sh[0] = -1;
        __syncthreads();
        int cum = incl - local;
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (i < wave) cum += scan[i];
        if (cum < need && need <= cum + local) {
          int cc = cum;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (cc < need && need <= cc + hb[j]) {
              sh[0] = 2047 - 4 * tid - j;
              sh[1] = cc;
              sh[2] = hb[j];
            }
            cc += hb[j];
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) hist[4 * tid + j] = 0u;   // every bin was read before the barrier
        __syncthreads();
        const int d = sh[0];
        if (d < 0) break;                            // cannot happen: nvalid > k
        need -= sh[1];
        const int inbin = sh[2];
        prefix |= (unsigned)d << shift;
        nbits += dbits;
        if (inbin == need) {                         // the whole bin is taken
          whole_bin = true;
          break;
        }
      }
      tau = max(prefix, 1u);                         // a bin's lower bound may be the invalid key 0
      if (!whole_bin) tie_need = need;               // tau fully resolved: `need` of its ties
    }
    int ngt = 0, nties = 0;
#pragma unroll
    for (int u = 0; u < kSPer; ++u) {
      ngt += key[u] > tau;
      nties += key[u] == tau;
    }
    const int x = (nties << 16) | ngt;               // both counts fit 16 bits
    const int xi = wave_inclusive_sum(x);
    if (lane == 63) scan[wave] = xi;
    __syncthreads();
    int pre_x = xi - x, total = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int si = scan[i];
      pre_x += i < wave ? si : 0;
      total += si;
    }
    int tie_rank = pre_x >> 16;
    int off = (pre_x & 0xFFFF) + min(tie_rank, tie_need);
    const int nsel = (total & 0xFFFF) + min(total >> 16, tie_need);
    const bool writer = split == 0 && grp == 0;
    int32_t* dst = a.sel_idx + (int64_t)t * a.k;
    const int r0 = kRows * tb, r1 = kRows * min(te, c.ng);
#pragma unroll
    for (int u = 0; u < kSPer; ++u) {
      bool sel = key[u] > tau;
      if (key[u] == tau) sel = tie_rank++ < tie_need;
      if (sel) {
        if (off < a.k) {
          if (writer) dst[off] = c0 + u;
          if (off >= r0 && off < r1) ring[off - r0] = c0 + u;
        }
        ++off;
      }
    }
    if (writer)
      for (int i = nsel + tid; i < a.k; i += kThreads) dst[i] = -1;
    __syncthreads();
  }
  if constexpr (QLDS) {
    if constexpr (SEL) {
      __builtin_amdgcn_s_waitcnt(0);               // this wave's q copies landed
      __syncthreads();
    }
    build_q();
    __syncthreads();                               // q read: the tile buffers are free
  }
  for (int u = 0; u < (pre ? te - tb : min(te - tb, 2)); ++u) issue(tb + u, u, u);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // ---- Q.K^T of one tile (FP4 = global rows, else window rows): this wave's partial
  // logits [32 heads][32 rows] to LDS.  Lane (r32, kh) of MFMA cc supplies dims
  // 32 b + 16 kh + 8 cc .. +8 of row r32 (one 8-byte read covers both cc for E2M1).
  auto qk = [&](auto FP4, int slot) __attribute__((always_inline)) {
    SMQA_LANE_ROLES
    const uint8_t* B = smem + slot * G::BUF;
    v16f acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
    if constexpr (F == kMXN) {
      const int nbw = G::BPW + (wave < G::EXTRA ? 1 : 0);
      if constexpr (decltype(FP4)::value) {
        // B = K^T in E2M1 as stored: lane (r32, kh) holds the 32 codes of row r32 in K-block
        // kh (block b0 + 2j + kh, 16 bytes) and that block's E8M0 byte is its scale.  A half
        // past this wave's blocks reads in-bounds LDS and is replaced by zeros.
        const uint8_t* rowp = B + r32 * G::RS4 + 16 * b0;
        const uint8_t* e8p = B + G::E8 + r32 * G::E8S + b0;
#pragma unroll
        for (int j = 0; j < NP; ++j) {
          if (2 * j < nbw) {
            const int blk = 2 * j + kh;
            const bool ok = blk < nbw;
            const v4u w = lds<v4u>(rowp + 16 * blk);
            const int sb = ok ? (int)lds<uint8_t>(e8p + blk) : 127;
            const v8i bv = {ok ? (int)w.x : 0, ok ? (int)w.y : 0, ok ? (int)w.z : 0, ok ? (int)w.w : 0, 0, 0, 0, 0};
            acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qf[j], bv, acc, 0, 4, 0, qsc[j], 0, sb);
          }
        }
      } else {
        // B = window rows in E4M3 (scale 2^0): lane (r32, kh) holds dims 32 bA + 16 kh .. +16
        // in bytes 0..15 and 32 bB + 16 kh .. +16 in bytes 16..31 of row r32 & 15
        const uint8_t* rowp = B + (r32 & 15) * G::RS8 + 16 * kh + 32 * b0;
#pragma unroll
        for (int j = 0; j < NP; ++j) {
          if (2 * j < nbw) {
            const v4u w0 = lds<v4u>(rowp + 64 * j);
            v4u w1 = {0u, 0u, 0u, 0u};
            if (2 * j + 1 < nbw) w1 = lds<v4u>(rowp + 64 * j + 32);
            const v8i bv = {(int)w0.x, (int)w0.y, (int)w0.z, (int)w0.w, (int)w1.x, (int)w1.y, (int)w1.z, (int)w1.w};
            acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qf[j], bv, acc, 0, 0, 0, qsc[j], 0, 127);
          }
        }
      }
    } else if constexpr (decltype(FP4)::value) {
      const uint8_t* rowp = B + r32 * G::RS4 + 8 * kh + 16 * b0;
      const uint8_t* e8p = B + G::E8 + r32 * G::E8S + b0;
      const uint8_t* nvp = B + G::E8 + r32 * 4 + kh;
#pragma unroll
      for (int i = 0; i < G::NBW; ++i) {
        if (i < G::BPW || wave < G::EXTRA) {
          const v2u wd = lds<v2u>(rowp + 16 * i);
          if constexpr (NV) {
            // the E4M3 scale of 16-block 2 (b0 + i) + kh: byte 2 ((b0 + i) & 1) + kh of dword
            // (b0 + i) / 2 of the row.  The codes go to fp16 with scale 1 and are multiplied
            // by the fp16 scale (exact), against q in fp16.
            const int bb = b0 + i;
            const unsigned byte = lds<uint8_t>(nvp + (bb >> 1) * (kRows * 4) + 2 * (bb & 1));
            const v2h s2 = __builtin_bit_cast(v2h, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(byte * 0x101u, 1.0f, false));
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
              const unsigned w = cc ? wd.y : wd.x;
              const v4u bw = {__builtin_bit_cast(unsigned, fp4x2_f16(w, 0) * s2),
                              __builtin_bit_cast(unsigned, fp4x2_f16(w, 1) * s2),
                              __builtin_bit_cast(unsigned, fp4x2_f16(w, 2) * s2),
                              __builtin_bit_cast(unsigned, fp4x2_f16(w, 3) * s2)};
              acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, qa[i][cc]),
                                                           __builtin_bit_cast(v8h, bw), acc, 0, 0, 0);
            }
          } else {
            // E8M0 e -> 2^(e-127) as the float e << 23 (e = 0, below 4e-38 in magnitude, gives 0)
            const float scl = __uint_as_float((unsigned)lds<uint8_t>(e8p + i) << 23);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[i][0], cvt8_fp4_bf16(wd.x, scl), acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[i][1], cvt8_fp4_bf16(wd.y, scl), acc, 0, 0, 0);
          }
        }
      }
    } else {
      const uint8_t* rowp = B + (r32 & 15) * G::RS8 + 16 * kh + 32 * b0;
#pragma unroll
      for (int i = 0; i < G::NBW; ++i) {
        if (i < G::BPW || wave < G::EXTRA) {
          const v4u wd = lds<v4u>(rowp + 32 * i);
          if constexpr (NV) {                    // q is held in fp16 here (E4M3 is exact in fp16)
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
              const unsigned w0 = cc ? wd.z : wd.x, w1 = cc ? wd.w : wd.y;
              const v4u bw = {__builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false)),
                              __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true)),
                              __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false)),
                              __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true))};
              acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, qa[i][cc]),
                                                           __builtin_bit_cast(v8h, bw), acc, 0, 0, 0);
            }
          } else {
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[i][0], cvt8_fp8_bf16(v2u{wd.x, wd.y}), acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[i][1], cvt8_fp8_bf16(v2u{wd.z, wd.w}), acc, 0, 0, 0);
          }
        }
      }
    }
    // acc[4 q4 + e] is the logit of head 8 q4 + 4 kh + e, row r32 -> red[wave][head][row]
    float* red = (float*)(smem + G::RED) + wave * 32 * kRows + r32;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
      for (int e = 0; e < 4; ++e) red[(8 * q4 + 4 * kh + e) * kRows] = acc[4 * q4 + e];
  };

  // ---- per-tile row data, computed while the tile is scored: the logit multiplier
  // tau * log2(e) * (rho or sigma), 0 for rows that take no part, the P multiplier (rho
  // or sigma), and the V-operand block scales as fp16 pairs (rows 2pp, 2pp+1; zero for
  // rows that take no part) or, for a window tile, 16-bit row masks in pairs.
  auto convert = [&](auto KIND, int tile, int slot, int rslot, int sslot) __attribute__((always_inline)) {
    constexpr int kind = decltype(KIND)::value;    // 1 E2M1 global, 2 window, 3 E4M3 global
    const int ct = opq(tid);                       // waves 0..3: 0..255
    const int ln = ct & 63;
    const uint8_t* B = smem + slot * G::BUF;
    unsigned* sch = (unsigned*)(smem + G::SCH) + sslot * G::SCHN;
    if constexpr (kind == 1) {
      const int* pos = (const int*)(smem + G::RING) + rslot * kRows;
      // rows that take part, as a bit mask (every loader wave computes it)
      const int pl = pos[ln & 31];
      const bool in_range = ln < kRows && tile * kRows + ln < c.gx1;
      const unsigned vmask = (unsigned)__builtin_amdgcn_ballot_w64(in_range && takes_part(pl, c.jmax));
      dbg_flag(a.dbg, ct < 64 && in_range && pl != -1 && !takes_part(pl, c.jmax), kDbgPosition);
      // blocks 4 bq .. 4 bq + 3 of rows 2 pp, 2 pp + 1 (one dword of raw E8M0 per row)
      const int pp = ct & 15, bq = ct >> 4;
      if constexpr (NV) {
        // rows that take no part get zero block scales, so that their (dummy) codes give
        // exact zeros in P.V; the products read the table only after the next barrier
        if (vmask != 0xFFFFFFFFu) {
          unsigned* tbl = (unsigned*)(B + G::E8);
          for (int e = ct; e < G::NQ * kRows; e += 256)
            if (!((vmask >> (e & 31)) & 1u)) tbl[e] = 0u;
        }
      } else if (bq < G::NB / 4) {
        const unsigned w0 = lds<unsigned>(B + G::E8 + (2 * pp) * G::E8S + 4 * bq);
        const unsigned w1 = lds<unsigned>(B + G::E8 + (2 * pp + 1) * G::E8S + 4 * bq);
        const bool v0 = (vmask >> (2 * pp)) & 1u, v1 = (vmask >> (2 * pp + 1)) & 1u;
#ifdef SMQA_DEBUG
        bool bad = false;
        for (int j = 0; j < 4; ++j)
          bad |= (v0 && !e8m0_fp16_exact((w0 >> (8 * j)) & 0xFFu)) || (v1 && !e8m0_fp16_exact((w1 >> (8 * j)) & 0xFFu));
        dbg_flag(a.dbg, bad, kDbgE8m0);
#endif
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // E8M0 e -> 2^(e-127) as the float e << 23 (e = 0 gives 0); exact in fp16 for
          // -24 <= e - 127 <= 15
          const float f0 = v0 ? __uint_as_float(((w0 >> (8 * j)) & 0xFFu) << 23) : 0.0f;
          const float f1 = v1 ? __uint_as_float(((w1 >> (8 * j)) & 0xFFu) << 23) : 0.0f;
          sch[(4 * bq + j) * 16 + pp] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pkrtz(f0, f1));
        }
      }
      if (ct < kRows) {
        const bool v = (vmask >> ct) & 1u;
        const float m = a.kv_rowscale ? ((const float*)(B + G::RHO))[4 * (ct & 7) + (ct >> 3)] : 1.0f;
        // the NVFP4 tensor scale g: the logits take rho * g; P takes rho * g * K with K the
        // power of two that puts g * K in [1, 2), and the epilogue 1 / K (P * rho * g alone
        // would fall into fp16 subnormals for the usual g ~ amax / 2688)
        rl[ct] = v ? (NV ? c.lscale * m * a.kv_gscale : c.lscale * m) : 0.0f;
        rp[ct] = v ? (NV ? m * (a.kv_gscale * a.kv_pscale) : m) : 0.0f;
      }
    } else if (ct < kRows) {
      bool v;
      if constexpr (kind == 3) {
        const int pl = ((const int*)(smem + G::RING) + rslot * kRows)[ct & 15];
        const bool in_range = ct < kWRows && tile * kWRows + ct < c.gx1;
        v = in_range && takes_part(pl, c.jmax);
        dbg_flag(a.dbg, in_range && pl != -1 && !v, kDbgPosition);
      } else {
        const int uu = kWRows * (c.wt0 + tile - c.ng) + ct;
        const int pos = c.pos0 + uu;
        v = ct < kWRows && uu < c.W && pos >= c.lo_win && pos <= c.p;
      }
      const unsigned vb = (unsigned)__builtin_amdgcn_ballot_w64(v);   // rows 0..15 of wave 0
      const bool scaled = kind == 3 ? a.kv_rowscale != nullptr : a.swa_scale != nullptr;
      const float m = scaled ? ((const float*)(B + G::RHO))[4 * (ct & 7) + ((ct & 15) >> 3)] : 1.0f;
      rl[ct] = v ? c.lscale * m : 0.0f;
      rp[ct] = v ? (NV ? m * a.kv_pscale : m) : 0.0f;    // NVFP4: window P carries K too
      if (ct < kWRows / 2) {
        const unsigned pr = (vb >> (2 * ct)) & 3u;
        sch[ct] = ((pr & 1u) ? 0x0000FFFFu : 0u) | ((pr & 2u) ? 0xFFFF0000u : 0u);
      }
    }
  };

  // ---- softmax of one tile: wave w owns heads 4w .. 4w+3; lane l takes head
  // 4w + l / 16 and rows 2 (l % 16), +1, so a head's max is a 16-lane reduction
  float lpart = 0.0f;                              // this lane's share of the head's row sum
  auto softmax = [&]() __attribute__((always_inline)) {
    const int ln_ = opq(lane);
    const int sh = 4 * wave + (ln_ >> 4), srow = 2 * (ln_ & 15);
    const float* red = (const float*)(smem + G::RED) + sh * kRows + srow;
    const float2 lsr = *(const float2*)(rl + srow);
    const float2 psr = *(const float2*)(rp + srow);
    const float mo = mref[sh];
    // the 8 waves' partial logits, read before any is added (one LDS round trip)
    float2 v[8];
#pragma unroll
    for (int w8 = 0; w8 < 8; ++w8) v[w8] = *(const float2*)(red + w8 * 32 * kRows);
    __builtin_amdgcn_sched_barrier(0);
    float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
    for (int w8 = 0; w8 < 8; ++w8) {
      s0 += v[w8].x;
      s1 += v[w8].y;
    }
    const bool ok0 = lsr.x != 0.0f, ok1 = lsr.y != 0.0f;
    s0 = ok0 ? s0 * lsr.x : -__builtin_inff();
    s1 = ok1 ? s1 * lsr.y : -__builtin_inff();
    const float tmax = row_reduce<true>(fmaxf(s0, s1));
    const float mn = fmaxf(mo, tmax);
    const float al = mn == mo ? 1.0f : __builtin_amdgcn_exp2f(mo - mn);
    const float p0 = ok0 ? __builtin_amdgcn_exp2f(s0 - mn) : 0.0f;
    const float p1 = ok1 ? __builtin_amdgcn_exp2f(s1 - mn) : 0.0f;
    lpart = lpart * al + (p0 + p1);
    *(v2h*)((_Float16*)(smem + G::PS) + sh * 40 + srow) = v2h{(_Float16)(p0 * psr.x), (_Float16)(p1 * psr.y)};
    if ((ln_ & 15) == 0) {
      mref[sh] = mn;
      malpha[sh] = al;
    }
  };

  // ---- P.V of one tile into the output accumulators
  v16f o[G::NBW];
#pragma unroll
  for (int i = 0; i < G::NBW; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[i][e] = 0.0f;

  auto pv = [&](auto FP4, int slot, int sslot) __attribute__((always_inline)) {
    SMQA_LANE_ROLES
    const uint8_t* B = smem + slot * G::BUF;
    const unsigned* sch = (const unsigned*)(smem + G::SCH) + sslot * G::SCHN;
    // rescale when the running max of a group of 8 heads (4 per k-half) moved: one
    // uniform branch per group, so only groups whose max moved pay for the multiplies
    v4f alq[4];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) alq[q4] = *(const v4f*)(malpha + 8 * q4 + 4 * kh);
    __builtin_amdgcn_sched_barrier(0);             // the four reads in one LDS round trip
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const v4f al = alq[q4];
      const bool moved = al.x != 1.0f || al.y != 1.0f || al.z != 1.0f || al.w != 1.0f;
      if (__builtin_amdgcn_ballot_w64(moved)) {
#pragma unroll
        for (int i = 0; i < G::NBW; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) o[i][4 * q4 + e] *= al[e];
      }
    }
    const _Float16* P = (const _Float16*)(smem + G::PS);
    if constexpr (decltype(FP4)::value) {
      // k-slot 8 kh + j of MFMA s <-> row 16 kh + 8 s + j
      const v8h pa0 = *(const v8h*)(P + r32 * 40 + 16 * kh);
      const v8h pa1 = *(const v8h*)(P + r32 * 40 + 16 * kh + 8);
      const uint8_t* tp = B + (16 * kh + i16) * G::RS4 + 8 * hh + 16 * b0;
      const unsigned* sp = sch + 16 * b0 + 8 * kh;
      const uint8_t* nvp = B + G::E8 + 16 * kh * 4;
#pragma unroll
      for (int i = 0; i < G::NBW; ++i) {
        if (i < G::BPW || wave < G::EXTRA) {
          const v2i raw = __builtin_amdgcn_ds_read_tr4_b64_v2i32(
              (__attribute__((address_space(3))) v2i*)(tp + 16 * i));
          if constexpr (NV) {
            // the scales of 16-block 2 (b0 + i) + hh for rows 16 kh + 8 s + 0..7 (MFMA s):
            // byte e = 2 ((b0 + i) & 1) + hh of 8 consecutive table dwords, paired by rows
            // (v_perm) and converted exactly to fp16; one half at a time, since hoisting
            // more scale reads would run out of registers
            const int bb = b0 + i;
            const uint8_t* tq = nvp + (bb >> 1) * (kRows * 4);
            const unsigned e = 2 * (bb & 1) + hh;
            const unsigned sel = 0x0C0C0000u | ((4u + e) << 8) | e;
#pragma unroll
            for (int hs = 0; hs < 2; ++hs) {
              const v4u d0 = lds<v4u>(tq + 32 * hs), d1 = lds<v4u>(tq + 32 * hs + 16);
              const unsigned d[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
              unsigned wv[4];
#pragma unroll
              for (int kk = 0; kk < 4; ++kk) {
                const unsigned scp = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(
                                                                      __builtin_amdgcn_perm(d[2 * kk + 1], d[2 * kk], sel),
                                                                      1.0f, false));
                const v2h f = fp4x2_f16((unsigned)raw[hs], kk) * __builtin_bit_cast(v2h, scp);
                wv[kk] = __builtin_bit_cast(unsigned, f);
              }
              o[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(hs ? pa1 : pa0,
                                                           __builtin_bit_cast(v8h, v4u{wv[0], wv[1], wv[2], wv[3]}),
                                                           o[i], 0, 0, 0);
              __builtin_amdgcn_sched_barrier(0);
            }
          } else {
            const v4u s0 = *(const v4u*)(sp + 16 * i);
            const v4u s1 = *(const v4u*)(sp + 16 * i + 4);
            const unsigned sc[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
            unsigned wv[8];
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
              const v2h f = fp4x2_f16((unsigned)raw[kk >> 2], kk & 3) * __builtin_bit_cast(v2h, sc[kk]);
              wv[kk] = __builtin_bit_cast(unsigned, f);
            }
            o[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(pa0, __builtin_bit_cast(v8h, v4u{wv[0], wv[1], wv[2], wv[3]}),
                                                         o[i], 0, 0, 0);
            o[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(pa1, __builtin_bit_cast(v8h, v4u{wv[4], wv[5], wv[6], wv[7]}),
                                                         o[i], 0, 0, 0);
          }
        }
      }
    } else {
      // k-slot 8 kh + j <-> window row 8 kh + j
      const v8h pa = *(const v8h*)(P + r32 * 40 + 8 * kh);
      const v4u mk = *(const v4u*)(sch + 4 * kh);
      const uint8_t* tp = B + (8 * kh + (i16 >> 1)) * G::RS8 + 16 * hh + 8 * (i16 & 1) + 32 * b0;
#pragma unroll
      for (int i = 0; i < G::NBW; ++i) {
        if (i < G::BPW || wave < G::EXTRA) {
          const v2i raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (__attribute__((address_space(3))) v2i*)(tp + 32 * i));
          v4u bw;
          bw.x = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)raw.x, 1.0f, false)) & mk.x;
          bw.y = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)raw.x, 1.0f, true)) & mk.y;
          bw.z = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)raw.y, 1.0f, false)) & mk.z;
          bw.w = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)raw.y, 1.0f, true)) & mk.w;
          o[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(pa, __builtin_bit_cast(v8h, bw), o[i], 0, 0, 0);
        }
      }
    }
  };

  // ---- pipeline.  Iteration i: gather tile i+2 (and the positions of tile i+3) unless the
  // prologue gathered every tile, P.V of tile i-1, Q.K^T of tile i, build the row data of
  // tile i; barrier; softmax of tile i and wait for tile i+1; barrier.  Tiles are global (E2M1) rows first, then window (E4M3)
  // rows, so the iterations run as separate loops per pair of kinds and no inner loop
  // branches on the kind.
  using KN = std::integral_constant<int, 0>;      // no tile
  using KG = std::integral_constant<int, G8 ? 3 : 1>;   // global tile (E2M1, or E4M3 when G8)
  using KW = std::integral_constant<int, 2>;      // window E4M3 tile
  auto body = [&](auto PVK, auto QKK, int i) __attribute__((always_inline)) {
    constexpr int pvk = decltype(PVK)::value, qkk = decltype(QKK)::value;
    const int n = i - tb;
    const bool more = !pre && i + 2 < te;
    const bool more_g = i + 2 < c.ng;
    // the prologue loaded the positions of the first kNBuf tiles
    if (!SEL && wave == 0 && n >= 1 && i + 3 < te && i + 3 < c.ng) load_pos(i + 3, (n + 3) & 3);
    // waves 0..3 issue the loads of tile i+2 before their products, waves 4..7 after them,
    // so half the waves queue for the vector-memory path while the other half run MFMAs
    if (more && wave < 4) issue(i + 2, (n + 2) & 3, (n + 2) & 3);
    if constexpr (pvk != 0) pv(std::integral_constant<bool, pvk == 1>{}, (n - 1) & 3, (n - 1) & 1);
    if constexpr (qkk != 0) qk(std::integral_constant<bool, qkk == 1>{}, n & 3);
    if (more && wave >= 4) issue(i + 2, (n + 2) & 3, (n + 2) & 3);
    // waves 0..3 build the row data of tile i after their products, in time they would
    // otherwise spend waiting at the barrier for waves 4..7 (per-phase cycle counters)
    if constexpr (qkk != 0) {
      if (wave < 4) convert(QKK, i, n & 3, n & 3, n & 1);
    }
    __syncthreads();                               // partial logits and row data of tile i
    if constexpr (qkk != 0) softmax();
    // tile i+1 (and the positions of tile i+3) landed; tile i+2 may still be in flight
    if (!more) __builtin_amdgcn_s_waitcnt(0);
    else if (!G8 && more_g) wait_vmcnt<G::NLOAD4>();
    else wait_vmcnt<G::NLOAD8>();
    __syncthreads();                               // P(i), tile i+1 published
  };
  if (tb < te) {
    const int ng = c.ng;
    int i = tb;
    if (i < ng) body(KN{}, KG{}, i);
    else body(KN{}, KW{}, i);
    for (++i; i < te && i < ng; ++i) body(KG{}, KG{}, i);
    if (i < te && i == ng) body(KG{}, KW{}, i++);
    for (; i < te; ++i) body(KW{}, KW{}, i);
    if (te - 1 < ng) body(KG{}, KN{}, te);
    else body(KW{}, KN{}, te);
  }

  // ---- epilogue: row sums, outputs of this wave's blocks, LSE / partial state
  SMQA_LANE_ROLES
  {
    const float l = row_reduce<false>(lpart);
    if (i16 == 0) mlsum[4 * wave + (lane >> 4)] = l;
  }
  __syncthreads();
  // one split writes the normalised output itself, unless the fused epilogue takes partials
  const bool direct = F == kMXR ? false : S == 1;
  float inv[16];
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float l = mlsum[8 * q4 + 4 * kh + e];
      inv[4 * q4 + e] = (direct ? (l > 0.0f ? 1.0f / l : 0.0f) : 1.0f) * (NV ? 1.0f / a.kv_pscale : 1.0f);
    }
  if constexpr (F == kMXF) {
    {
      // MegaAttention's epilogue in place (one split; blog §Kernels): the normalised outputs
      // are rotated back on the rotary pairs (the partner dim is the neighbouring lane, so a
      // DPP pair swap), then each head's amax over all 8 waves' dims gives the scale of its
      // E4M3 codes.  The same fp32 formulas as attend_fused_epilogue_kernel.
      const int r0 = D - 2 * a.rope_pairs;
#pragma unroll
      for (int i = 0; i < G::NBW; ++i) {
        if (i < G::BPW || wave < G::EXTRA) {
          const int d = 32 * (b0 + i) + r32;
          const bool rot = a.rope_pairs > 0 && d >= r0;
          float c = 1.0f, sn = 0.0f;
          if (rot) {
            const int64_t pj = (int64_t)t * a.rope_pairs + (d - r0) / 2;
            c = a.rope_cos[pj];
            sn = a.rope_sin[pj];
          }
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const float x = o[i][j] * inv[j];
            const float xp = dpp_f<0xB1>(x);                  // the other dim of the pair
            o[i][j] = !rot ? x : ((r32 & 1) ? __builtin_fmaf(-xp, sn, x * c) : __builtin_fmaf(x, c, xp * sn));
          }
        }
        __builtin_amdgcn_sched_barrier(0);             // one block at a time (registers)
      }
      // per head: amax over this lane's blocks, the 32 lanes of its k-half (two DPP rows)
      // and the 8 waves (LDS)
      float* amx = (float*)(smem + G::RED);             // [8 waves][32 heads], then scales [32]
      float* hsc = amx + 8 * 32;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < G::NBW; ++i)
          if (i < G::BPW || wave < G::EXTRA) m = fmaxf(m, fabsf(o[i][j]));
        m = row_reduce<true>(m);
        m = fmaxf(m, __shfl_xor(m, 16));
        if (r32 == 0) amx[wave * 32 + 8 * (j >> 2) + 4 * kh + (j & 3)] = m;
      }
      __syncthreads();
      if (tid < 32) {
        float m = amx[tid];
#pragma unroll
        for (int w = 1; w < 8; ++w) m = fmaxf(m, amx[w * 32 + tid]);
        hsc[tid] = m > 0.0f ? 448.0f / m : 0.0f;        // the quantisation multiplier
        a.out_scale[(int64_t)t * a.Hq + h0 + tid] = m / 448.0f;
      }
      __syncthreads();
      v4f rq[4];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) rq[q4] = *(const v4f*)(hsc + 8 * q4 + 4 * kh);
      // codes staged in the (idle) tile buffers as [32 heads][D] bytes, then stored 16 bytes
      // a lane
      uint8_t* stage = smem;
      float* df = a.out ? a.out + ((int64_t)t * a.Hq + h0) * D : nullptr;
#pragma unroll
      for (int i = 0; i < G::NBW; ++i) {
        if (i < G::BPW || wave < G::EXTRA) {
          const int d = 32 * (b0 + i) + r32;
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int hl = 8 * q4 + 4 * kh + e;
              const float y = o[i][4 * q4 + e];
              const float r = rq[q4][e];
              const unsigned code = r > 0.0f ? (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(y * r, 0.0f, 0, false) & 0xFFu : 0u;
              stage[hl * D + d] = (uint8_t)code;
              if (df) df[(int64_t)hl * D + d] = y;
            }
        }
      }
      __syncthreads();
      uint8_t* d8 = a.out_fp8 + ((int64_t)t * a.Hq + h0) * D;   // 32 consecutive rows of D bytes
      for (int x = tid; x < 32 * D / 16; x += kThreads) *(v4u*)(d8 + 16 * x) = *(const v4u*)(stage + 16 * x);
    }
  } else {
    float* dst = direct ? a.out + ((int64_t)t * a.Hq + h0) * D
                        : (float*)a.ws + (((int64_t)split * a.T + t) * a.Hq + h0) * D;
#pragma unroll
    for (int i = 0; i < G::NBW; ++i) {
      if (i < G::BPW || wave < G::EXTRA) {
        const int d = 32 * (b0 + i) + r32;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int hl = 8 * q4 + 4 * kh + e;
            dst[(int64_t)hl * D + d] = o[i][4 * q4 + e] * inv[4 * q4 + e];
          }
      }
    }
  }
  if (tid < 32) {
    const int hg = h0 + tid;
    const float m = mref[tid], l = mlsum[tid];
    if (direct) {
      if (a.lse) a.lse[(int64_t)t * a.Hq + hg] = l > 0.0f ? (m + log2f(l)) * kLn2 : -__builtin_inff();
    } else {
      float* ml = (float*)a.ws + (size_t)S * a.T * a.Hq * D;
      const int64_t ii = ((int64_t)split * a.T + t) * a.Hq + hg;
      ml[2 * ii] = m;
      ml[2 * ii + 1] = l;
    }
  }
}

template <int D, int F>
hipError_t launch(const AttendArgs& a, int S, hipStream_t s) {
  using G = Geo<D, F>;
  const int ngroups = a.Hq / 32;
  const int total = a.T * ngroups * S;
  const int nb = (total + 7) / 8 * 8;
  static_assert(G::LDS <= kLdsBytes, "the tile ring and softmax state must fit one CU's LDS");
  static PerDevice attr;
  if (hipError_t e = allow_dynamic_lds(attend_kernel<D, F>, G::LDS, attr); e != hipSuccess) return e;
  hipLaunchKernelGGL((attend_kernel<D, F>), dim3(nb), dim3(kThreads), G::LDS, s, a, S, ngroups, total);
  hipError_t e = hipGetLastError();
  // the fused form merges in its own epilogue (kernel)
  return e != hipSuccess ? e : ((F == kMXF || F == kMXR) ? hipSuccess : launch_attend_merge(a, S, s));
}

// kMXS (decode_step's selection in the attention kernel) exists at D = 1664 only
template <int D>
hipError_t launch_sel(const AttendArgs& a, int S, hipStream_t s) {
  if constexpr (D == 1664) return launch<D, kMXS>(a, S, s);
  else return hipErrorInvalidValue;
}

}  // namespace sd

int sd_lds_bytes(int32_t D) {
  switch (D) {
#define SMQA_SD_LDS(d) \
  case d:             \
    return sd::Geo<d, sd::kMX>::LDS;
    SMQA_SD_LDS(128) SMQA_SD_LDS(256) SMQA_SD_LDS(384) SMQA_SD_LDS(512)
    SMQA_SD_LDS(640) SMQA_SD_LDS(768) SMQA_SD_LDS(896) SMQA_SD_LDS(1024)
    SMQA_SD_LDS(1152) SMQA_SD_LDS(1280) SMQA_SD_LDS(1408) SMQA_SD_LDS(1536)
    SMQA_SD_LDS(1664)
#undef SMQA_SD_LDS
    default: return 0;
  }
}

// Dimension-split attention for Hq % 32 == 0 and D <= 1664 (the register budget of 8
// waves holding 32 heads of outputs and q, and four tile buffers in LDS), over the FP4
// global cache in the format a.kv_fmt (MX FP4, FP8 rows, NVFP4); returns
// hipErrorInvalidValue otherwise.
hipError_t launch_attend_sd(const AttendArgs& a, int S, hipStream_t s) {
  switch (a.D) {
#define SMQA_SD_D(d)                                              \
  case d:                                                         \
    return a.kv_fmt == sd::kMXS   ? sd::launch_sel<d>(a, S, s)        \
           : a.kv_fmt == sd::kFP8 ? sd::launch<d, sd::kFP8>(a, S, s)  \
           : a.kv_fmt == sd::kNV  ? sd::launch<d, sd::kNV>(a, S, s)   \
           : a.kv_fmt == sd::kMXN ? sd::launch<d, sd::kMXN>(a, S, s)  \
           : a.kv_fmt == sd::kMXF ? sd::launch<d, sd::kMXF>(a, S, s)  \
           : a.kv_fmt == sd::kMXR ? sd::launch<d, sd::kMXR>(a, S, s)  \
                                  : sd::launch<d, sd::kMX>(a, S, s);
    SMQA_SD_D(128) SMQA_SD_D(256) SMQA_SD_D(384) SMQA_SD_D(512)
    SMQA_SD_D(640) SMQA_SD_D(768) SMQA_SD_D(896) SMQA_SD_D(1024)
    SMQA_SD_D(1152) SMQA_SD_D(1280) SMQA_SD_D(1408) SMQA_SD_D(1536)
    SMQA_SD_D(1664)
#undef SMQA_SD_D
    default: return hipErrorInvalidValue;
  }
}

}  // namespace smqa
