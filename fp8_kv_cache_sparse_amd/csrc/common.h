// Internal device/host helpers shared by the gfx950 kernels of libsmqa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "smqa.h"

namespace smqa {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// E8M0 exponent byte -> the float 2^(e-127) (e = 0 gives the subnormal 2^-127).
__device__ __forceinline__ float e8m0_to_float(unsigned e) {
  return e ? __uint_as_float(e << 23) : __uint_as_float(0x00400000u);
}

// Order-preserving map float -> uint32 (larger float -> larger key).
// -inf (a masked score) and NaN map to 0, which marks "not in the scored set";
// every finite score maps to a key >= 0x00800000.
__device__ __forceinline__ unsigned score_key(float s) {
  unsigned u = __float_as_uint(s);
  if (s == -__builtin_inff() || s != s) return 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inverse of score_key on the keys of finite scores (>= 0x00800000).
__device__ __forceinline__ float key_score(unsigned key) {
  return __uint_as_float((key & 0x80000000u) ? (key ^ 0x80000000u) : ~key);
}

// Inclusive prefix sum over a wave with DPP row shifts and row broadcasts: within each
// row of 16 lanes by shifts of 1, 2, 4, 8 (lanes shifted in from outside the row read
// 0), then the total of row 0 into row 1 and of row 2 into row 3, then the total of
// rows 0-1 into rows 2-3.
__device__ __forceinline__ int wave_inclusive_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return v;
}

// Inclusive running maximum over a wave (unsigned; 0 is the identity), same DPP pattern.
__device__ __forceinline__ unsigned wave_inclusive_max(unsigned v) {
  v = max(v, (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, true));
  v = max(v, (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, true));
  v = max(v, (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, true));
  v = max(v, (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, true));
  v = max(v, (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false));
  v = max(v, (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false));
  return v;
}

// Largest b with q_start[b] <= t (queries are grouped by sequence).
__device__ __forceinline__ int seq_of_query(const int32_t* q_start, int B, int t) {
  int lo = 0, hi = B;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (q_start[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

// ---------------------------------------------------------------- host-side caches

// A value computed once per device by host code (a kernel attribute set, an occupancy
// query).  Thread safe: racing callers may both compute it, which is harmless because the
// computation is idempotent; 0 means "not yet".  Devices past kMaxDevices are not cached.
constexpr int kMaxDevices = 64;
struct PerDevice {
  std::atomic<int> v[kMaxDevices];
};

inline int current_device() {
  int d = 0;
  return hipGetDevice(&d) == hipSuccess ? d : 0;
}

// Raise `kernel`'s dynamic-LDS limit to `bytes` once per device.
template <class K>
inline hipError_t allow_dynamic_lds(K kernel, int bytes, PerDevice& done) {
  const int dev = current_device();
  if (dev < kMaxDevices && done.v[dev].load(std::memory_order_acquire)) return hipSuccess;
  hipError_t e = hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && dev < kMaxDevices) done.v[dev].store(1, std::memory_order_release);
  return e;
}

constexpr int kLdsBytes = 160 * 1024;   // LDS of one gfx950 compute unit

// ---------------------------------------------------------------- launchers
// (defined in score.hip / topk.hip / attend.hip; arguments already validated)

struct ScoreArgs {
  const int64_t* seq_start;
  const int32_t* q_start;
  const int32_t* q_pos;
  int32_t B, T, max_ctx;
  const uint8_t* q_fp8;
  const float* w;
  const uint8_t* k_fp8;
  const float* k_scale;
  const int32_t* cand;
  int32_t n_cand;
  int32_t Hi, Di;
  float* scores;
  int64_t ld;
  // Optional (streaming kernel only): [T][kTopkBins] counts of the top 12 key bits of every
  // scored position (score_key(s) >> 20), added with device atomics to a zeroed array, and
  // each query's number of scored columns, stored at qcols[t * qcols_stride].
  unsigned* hist;
  int32_t* qcols;
  int32_t qcols_stride;
  // Write -inf into the columns no score goes to: dense, [min(p_t, len_b - 1) + 1, ld);
  // candidate mode, [n_cand, ld) (the public call; decode_step's internal rows skip it).
  bool fill_tail;
  // Contract on the FP8 matrix cores instead of bf16 ones (Di = 128; sparse_mqa_score_fp8mma)
  bool fp8mma;
  // SMQA_DEBUG builds: the device word the kernels OR kDbg* bits into; null otherwise
  unsigned* dbg;
};
hipError_t launch_score(const ScoreArgs& a, hipStream_t s);
// True when launch_score takes the streaming kernel, the one that can fill ScoreArgs::hist.
bool score_streams(const ScoreArgs& a);

constexpr int kTopkBins = 4096;   // top-k first digit: the top 12 bits of the order key

struct TopkArgs {
  const int64_t* seq_start;
  const int32_t* q_start;
  const int32_t* q_pos;
  int32_t B, T, max_ctx;
  const float* scores;
  int64_t ld;
  const int32_t* cand;
  int32_t n_cand;
  int32_t k;
  int32_t* idx;
  void* ws;
  float* val;           // optional [T][k]: the score of each selected position, -inf for padding
};
size_t topk_workspace_bytes(int32_t T, int32_t max_ctx, int32_t k);
hipError_t launch_topk(const TopkArgs& a, hipStream_t s);
// Split form for a producer that builds the first-digit histogram itself: prepare zeroes the
// workspace state and returns the [T][kTopkBins] histogram to fill (nullptr when the rows are
// short and the single-kernel path needs none); finish runs the rest of the selection.
struct TopkFill {
  unsigned* hist;       // [T][kTopkBins], zeroed
  int32_t* qcols;       // scored columns of query t at qcols[t * qcols_stride]
  int32_t qcols_stride;
};
hipError_t launch_topk_prepare(const TopkArgs& a, hipStream_t s, TopkFill* fill);
hipError_t launch_topk_from_hist(const TopkArgs& a, hipStream_t s);

// Global cache formats of AttendArgs::kv_fmt.  kKvMX: kv_codes E2M1, kv_e8m0 E8M0 per 32.
// kKvFP8: kv_codes E4M3 rows [N][D], kv_e8m0 unused.  kKvNV: kv_codes E2M1, kv_e8m0 E4M3 per
// 16, tensor scale kv_gscale.  kKvMXF / kKvMXR: the MX format with MegaAttention's fused query
// RoPE and FP8 epilogue, in the attention kernel (one split) / through split partials (set by
// launch_attend_fused only).
// kKvMXN: the MX format with Q.K^T on the scaled matrix cores, the query quantised to
// MXFP8 in the kernel and the E2M1 rows and their E8M0 bytes consumed as stored.
// kKvMXS: the MX format, the selection computed in the attention kernel from the query's
// scores (decode_step on rows of at most kSelCols columns; set by decode_step only).
enum KvFmt : int32_t { kKvMX = 0, kKvFP8 = 1, kKvNV = 2, kKvMXF = 3, kKvMXR = 4, kKvMXN = 5, kKvMXS = 6 };
constexpr int kSelCols = 8192;   // the longest row kKvMXS selects from (512 threads x 16)

struct AttendArgs {
  const int64_t* seq_start;
  const int32_t* q_start;
  const int32_t* q_pos;
  int32_t B, T;
  const uint16_t* q;
  const uint8_t* kv_codes;
  const uint8_t* kv_e8m0;
  const float* kv_rowscale;
  const int32_t* idx;
  int32_t k;
  const uint8_t* swa;
  const float* swa_scale;
  const int32_t* swa_pos0;
  const int32_t* swa_clip;
  int32_t W, Hq, D;
  float sm_scale;
  float* out;
  float* lse;
  void* ws;
  int32_t kv_fmt;             // KvFmt
  float kv_gscale;
  float kv_pscale;            // NVFP4: the power of two K with kv_gscale * K in [1, 2)
  // fused epilogue (kKvMXF / kKvMXR): the last 2 * rope_pairs latent dims of q are rotated by
  // (rope_cos, rope_sin)[t] before the products; out_fp8 / out_scale receive the quantised,
  // inversely rotated output
  const float* rope_cos;
  const float* rope_sin;
  int32_t rope_pairs;
  uint8_t* out_fp8;
  float* out_scale;
  // SMQA_DEBUG builds: the device word the kernels OR kDbg* bits into; null otherwise
  unsigned* dbg;
  // kKvMXS: the scores [T][sel_ld] the selection is taken from (columns < sel_max_ctx read),
  // and the selection's output [T][k] (idx above is not read)
  const float* sel_scores;
  int32_t sel_ld;
  int32_t sel_max_ctx;
  int32_t* sel_idx;
};

// A selected position j takes part iff 0 <= j <= jmax = min(p_t, len_b - 1); -1 pads the
// selection, and any other value is skipped the same way (so a bad index never leads to a
// gather outside the query's rows).  SMQA_DEBUG builds report such values (kDbgPosition).
__host__ __device__ inline bool takes_part(int j, int jmax) { return j >= 0 && j <= jmax; }
// E8M0 exponents whose 32 values P.V holds exactly in fp16 (-23 <= e - 127 <= 13), and 0
// (scale 2^-127: the block's values are far below fp16's range and count as zeros).
// SMQA_DEBUG builds report any other exponent of a row that takes part (kDbgE8m0).
__host__ __device__ inline bool e8m0_fp16_exact(unsigned e) { return e == 0u || (e >= 104u && e <= 140u); }
constexpr unsigned kDbgPosition = 1u;
constexpr unsigned kDbgE8m0 = 2u;
constexpr unsigned kDbgLayout = 4u;     // seq_start or q_start decreasing, or a negative q_pos
constexpr unsigned kDbgCand = 8u;       // a candidate list not strictly ascending
// OR `bit` into the debug word when `cond` holds (a vector atomic; compiled out of release
// builds, where `w` is null anyway).
__device__ __forceinline__ void dbg_flag(unsigned* w, bool cond, unsigned bit) {
#ifdef SMQA_DEBUG
  if (w != nullptr && cond) __hip_atomic_fetch_or(w, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#else
  (void)w;
  (void)cond;
  (void)bit;
#endif
}
// Tile-range splits per (query, head group) of a call of this shape, or 0 when no split
// count fits the workgroup's LDS (the call is unsupported); lds receives the bytes per
// workgroup (static + dynamic) of the chosen plan.
int attend_splits(int32_t T, int32_t k, int32_t W, int32_t Hq, int32_t D, int32_t* lds = nullptr);
size_t attend_workspace_bytes(int32_t T, int32_t k, int32_t W, int32_t Hq, int32_t D);
bool attend_select_fits(int32_t T, int32_t k, int32_t W, int32_t Hq, int32_t D);
hipError_t launch_attend(const AttendArgs& a, hipStream_t s);
hipError_t launch_attend_fmt(const AttendArgs& a, hipStream_t s);   // kKvFP8, kKvNV, kKvMXN
size_t attend_fused_workspace_bytes(int32_t T, int32_t k, int32_t W, int32_t Hq, int32_t D);
hipError_t launch_attend_fused(const AttendArgs& a, hipStream_t s);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace smqa
