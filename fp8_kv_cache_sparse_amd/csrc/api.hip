// C-ABI entry points of libsmqa: host-side validation, workspace carving and
// launches on the caller's stream.  Every check runs before the first HIP call,
// so argument errors are reported without touching a device.
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "common.h"

// Device-resident workspace of decode_step_noalloc, for callers that cannot allocate.  Every
// GPU the library runs on holds its own copy until the process ends.  In host code this
// name is only a stand-in for the symbol: its device address comes from hipGetSymbolAddress.
static __device__ __align__(256) uint8_t scratch[SMQA_NOALLOC_SCRATCH_BYTES];

#ifdef SMQA_DEBUG
// SMQA_DEBUG builds: the word the attention kernels OR their kDbg* findings into (one per
// GPU; read and cleared by smqa_debug_flags).  Its device address comes from
// hipGetSymbolAddress, like scratch's.
static __device__ unsigned debug_word;
#endif

namespace {

// Device address of a file-scope __device__ symbol on the current device, looked up once per
// device and kept in `ptrs`; nullptr with the HIP error in *err when the lookup fails.
template <class Sym>
void* symbol_ptr(const Sym& sym, std::atomic<void*>* ptrs, hipError_t* err) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *err = e;
    return nullptr;
  }
  if (dev < smqa::kMaxDevices) {
    if (void* p = ptrs[dev].load(std::memory_order_acquire)) return p;
  }
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, sym);
  if (e != hipSuccess || !p) {
    *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
    return nullptr;
  }
  if (dev < smqa::kMaxDevices) ptrs[dev].store(p, std::memory_order_release);
  return p;
}

// The debug word's device address on the current device (SMQA_DEBUG builds); null in
// release builds, whose kernels never touch it.
hipError_t debug_word_ptr(unsigned** out) {
#ifdef SMQA_DEBUG
  static std::atomic<void*> ptrs[smqa::kMaxDevices];
  hipError_t e = hipSuccess;
  *out = (unsigned*)symbol_ptr(HIP_SYMBOL(debug_word), ptrs, &e);
  return *out ? hipSuccess : e;
#else
  *out = nullptr;
  return hipSuccess;
#endif
}

// SMQA_DEBUG builds point the attention kernels at the debug word; release builds leave
// AttendArgs::dbg null.
hipError_t attach_debug(smqa::AttendArgs& a) { return debug_word_ptr(&a.dbg); }

}  // namespace

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(SMQA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

#define REQUIRE_PTR(p)                                               \
  do {                                                               \
    if (!(p)) return fail(SMQA_ERR_NULL, "%s is NULL", #p);          \
  } while (0)
#define REQUIRE_ALIGN(p, a)                                                          \
  do {                                                                               \
    if ((p) && !aligned((p), (a)))                                                   \
      return fail(SMQA_ERR_ALIGN, "%s must be %d-byte aligned", #p, (int)(a));       \
  } while (0)

int check_layout(const smqa_layout* L) {
  if (!L) return fail(SMQA_ERR_NULL, "layout is NULL");
  if (L->num_seqs < 1) return fail(SMQA_ERR_SHAPE, "num_seqs = %d must be >= 1", L->num_seqs);
  if (L->num_q < 0) return fail(SMQA_ERR_SHAPE, "num_q = %d must be >= 0", L->num_q);
  if (!L->seq_start) return fail(SMQA_ERR_NULL, "layout.seq_start is NULL");
  if (!L->q_start) return fail(SMQA_ERR_NULL, "layout.q_start is NULL");
  if (L->num_q > 0 && !L->q_pos) return fail(SMQA_ERR_NULL, "layout.q_pos is NULL");
  if (!aligned(L->seq_start, 8)) return fail(SMQA_ERR_ALIGN, "layout.seq_start must be 8-byte aligned");
  if (!aligned(L->q_start, 4) || !aligned(L->q_pos, 4))
    return fail(SMQA_ERR_ALIGN, "layout.q_start / q_pos must be 4-byte aligned");
  if (L->num_q > 0 && L->max_ctx < 1) return fail(SMQA_ERR_SHAPE, "max_ctx = %d must be >= 1", L->max_ctx);
  return SMQA_OK;
}

int check_score(const smqa_layout* L, const uint8_t* q_fp8, const float* w, const uint8_t* k_fp8,
                const float* k_scale, const int32_t* cand, int32_t n_cand, int32_t Hi, int32_t Di,
                const float* scores, int64_t ld, bool need_scores) {
  REQUIRE_PTR(q_fp8);
  REQUIRE_PTR(w);
  REQUIRE_PTR(k_fp8);
  if (need_scores) REQUIRE_PTR(scores);
  if (Di != 64 && Di != 128) return fail(SMQA_ERR_UNSUPPORTED, "Di = %d: supported 64, 128", Di);
  if (Hi < 1 || Hi > 128) return fail(SMQA_ERR_UNSUPPORTED, "Hi = %d: supported 1..128", Hi);
  if (cand) {
    if (n_cand < 1) return fail(SMQA_ERR_SHAPE, "n_cand = %d must be >= 1 with a candidate list", n_cand);
    if (ld < n_cand) return fail(SMQA_ERR_SHAPE, "ld_scores = %lld < n_cand = %d", (long long)ld, n_cand);
  } else if (ld < L->max_ctx) {
    return fail(SMQA_ERR_SHAPE, "ld_scores = %lld < max_ctx = %d", (long long)ld, L->max_ctx);
  }
  REQUIRE_ALIGN(q_fp8, 16);
  REQUIRE_ALIGN(k_fp8, 16);
  REQUIRE_ALIGN(w, 4);
  REQUIRE_ALIGN(k_scale, 4);
  REQUIRE_ALIGN(cand, 4);
  REQUIRE_ALIGN(scores, 4);
  return SMQA_OK;
}

int check_topk(const smqa_layout* L, const float* scores, int64_t ld, const int32_t* cand,
               int32_t n_cand, int32_t k, const int32_t* idx, const float* val) {
  REQUIRE_PTR(scores);
  REQUIRE_PTR(idx);
  if (k < 1 || k > 4096) return fail(SMQA_ERR_UNSUPPORTED, "k = %d: supported 1..4096", k);
  if (cand) {
    if (n_cand < 1) return fail(SMQA_ERR_SHAPE, "n_cand = %d must be >= 1 with a candidate list", n_cand);
    if (ld < n_cand) return fail(SMQA_ERR_SHAPE, "ld_scores = %lld < n_cand = %d", (long long)ld, n_cand);
  } else if (ld < L->max_ctx) {
    return fail(SMQA_ERR_SHAPE, "ld_scores = %lld < max_ctx = %d", (long long)ld, L->max_ctx);
  }
  REQUIRE_ALIGN(scores, 4);
  REQUIRE_ALIGN(cand, 4);
  REQUIRE_ALIGN(idx, 4);
  REQUIRE_ALIGN(val, 4);
  return SMQA_OK;
}

int check_attend(const uint16_t* q, const uint8_t* kv_codes, const uint8_t* kv_e8m0,
                 const float* kv_rowscale, const int32_t* idx, int32_t k, const uint8_t* swa,
                 const float* swa_scale, const int32_t* swa_pos0, const int32_t* swa_clip, int32_t W,
                 int32_t Hq, int32_t D, float sm_scale, const float* out, const float* lse,
                 bool need_idx) {
  REQUIRE_PTR(q);
  REQUIRE_PTR(kv_codes);
  REQUIRE_PTR(kv_e8m0);
  if (need_idx) REQUIRE_PTR(idx);
  REQUIRE_PTR(swa);
  REQUIRE_PTR(swa_pos0);
  REQUIRE_PTR(out);
  if (D % 128 != 0 || D < 128 || D > 2048)
    return fail(SMQA_ERR_UNSUPPORTED, "D = %d: supported multiples of 128 in 128..2048", D);
  if (Hq % 16 != 0 || Hq < 16 || Hq > 128)
    return fail(SMQA_ERR_UNSUPPORTED, "Hq = %d: supported multiples of 16 in 16..128", Hq);
  if (W < 1 || W > 128) return fail(SMQA_ERR_UNSUPPORTED, "W = %d: supported 1..128", W);
  if (k < 1 || k > 4096) return fail(SMQA_ERR_UNSUPPORTED, "k = %d: supported 1..4096", k);
  if (!(sm_scale == sm_scale)) return fail(SMQA_ERR_SHAPE, "sm_scale is NaN");
  REQUIRE_ALIGN(q, 16);
  REQUIRE_ALIGN(kv_codes, 16);
  REQUIRE_ALIGN(kv_e8m0, 4);
  REQUIRE_ALIGN(kv_rowscale, 4);
  REQUIRE_ALIGN(idx, 4);
  REQUIRE_ALIGN(swa, 16);
  REQUIRE_ALIGN(swa_scale, 4);
  REQUIRE_ALIGN(swa_pos0, 4);
  REQUIRE_ALIGN(swa_clip, 4);
  REQUIRE_ALIGN(out, 16);
  REQUIRE_ALIGN(lse, 4);
  return SMQA_OK;
}

// The extra arguments of the fused form (MegaAttention's query RoPE and FP8 output).
int check_fused(const float* rope_cos, const float* rope_sin, int32_t rope_pairs, int32_t Hq,
                int32_t D, const uint8_t* out_fp8, const float* out_scale) {
  REQUIRE_PTR(out_fp8);
  REQUIRE_PTR(out_scale);
  REQUIRE_ALIGN(out_fp8, 16);
  REQUIRE_ALIGN(out_scale, 4);
  if (Hq % 32 != 0 || D > 1664)
    return fail(SMQA_ERR_UNSUPPORTED, "fused attention: Hq = %d, D = %d; supported Hq %% 32 == 0, D <= 1664",
                Hq, D);
  if (rope_pairs < 0 || rope_pairs % 4 != 0 || 2 * rope_pairs > D)
    return fail(SMQA_ERR_UNSUPPORTED, "rope_pairs = %d: supported multiples of 4 with 2 * rope_pairs <= D",
                rope_pairs);
  if (rope_pairs > 0) {
    REQUIRE_PTR(rope_cos);
    REQUIRE_PTR(rope_sin);
    REQUIRE_ALIGN(rope_cos, 16);
    REQUIRE_ALIGN(rope_sin, 16);
  }
  return SMQA_OK;
}

// The attention plan of a call: some shapes the limits accept need more LDS per workgroup
// than a CU has at every split count (wide latents with large k over 16-head groups).
int check_plan(const smqa_layout* L, int32_t k, int32_t W, int32_t Hq, int32_t D) {
  int32_t lds = 0;
  if (smqa::attend_splits(L->num_q, k, W, Hq, D, &lds) == 0)
    return fail(SMQA_ERR_UNSUPPORTED,
                "attention with T = %d, k = %d, W = %d, Hq = %d, D = %d needs %d bytes of LDS per "
                "workgroup at every split count (%d available)",
                L->num_q, k, W, Hq, D, lds, smqa::kLdsBytes);
  return SMQA_OK;
}

int check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return SMQA_OK;
  if (!ws) return fail(SMQA_ERR_WORKSPACE, "workspace is NULL but %zu bytes are required", need);
  if (!aligned(ws, 256)) return fail(SMQA_ERR_ALIGN, "workspace must be 256-byte aligned");
  if (have < need) return fail(SMQA_ERR_WORKSPACE, "workspace has %zu bytes, %zu required", have, need);
  return SMQA_OK;
}

int32_t score_cols(const smqa_layout* L, int32_t n_cand, bool cand) { return cand ? n_cand : L->max_ctx; }

struct DecodeWs {
  size_t scores_off, idx_off, topk_off, attend_off, total;
};

DecodeWs decode_ws_layout(const smqa_layout* L, int32_t k, int32_t ncols, int32_t W, int32_t Hq, int32_t D) {
  DecodeWs d;
  const size_t T = (size_t)L->num_q;
  size_t off = 0;
  d.scores_off = off;
  off += smqa::align_up(T * (size_t)ncols * 4, 256);
  d.idx_off = off;
  off += smqa::align_up(T * (size_t)k * 4, 256);
  d.topk_off = off;
  off += smqa::align_up(smqa::topk_workspace_bytes(L->num_q, ncols, k), 256);
  d.attend_off = off;
  off += smqa::align_up(smqa::attend_workspace_bytes(L->num_q, k, W, Hq, D), 256);
  d.total = off;
  return d;
}

}  // namespace

namespace {

// sparse_mqa_score and its FP8 matrix-core form (Di = 128 only).
int score_entry(const smqa_layout* L, const uint8_t* q_fp8, const float* w, const uint8_t* k_fp8,
                const float* k_scale, const int32_t* cand, int32_t n_cand, int32_t Hi, int32_t Di,
                float* scores, int64_t ld_scores, void* stream, bool fp8mma) {
  g_err.clear();
  int st = check_layout(L);
  if (st) return st;
  if (L->num_q == 0) return SMQA_OK;
  st = check_score(L, q_fp8, w, k_fp8, k_scale, cand, n_cand, Hi, Di, scores, ld_scores, true);
  if (st) return st;
  if (fp8mma && Di != 128)
    return fail(SMQA_ERR_UNSUPPORTED, "sparse_mqa_score_fp8mma: Di = %d (the FP8 form needs Di = 128)", Di);
  smqa::ScoreArgs a{L->seq_start, L->q_start, L->q_pos, L->num_seqs, L->num_q, L->max_ctx,
                    q_fp8, w, k_fp8, k_scale, cand, cand ? n_cand : 0, Hi, Di, scores, ld_scores,
                    nullptr, nullptr, 0, true, fp8mma};
  if (hipError_t e = debug_word_ptr(&a.dbg); e != hipSuccess) return hip_fail(e, "debug word lookup");
  hipError_t e = smqa::launch_score(a, (hipStream_t)stream);
  return e == hipSuccess ? SMQA_OK : hip_fail(e, fp8mma ? "sparse_mqa_score_fp8mma launch" : "sparse_mqa_score launch");
}

}  // namespace

extern "C" {

const char* smqa_last_error(void) { return g_err.c_str(); }

const char* smqa_version(void) { return "smqa 0.1.0 gfx950"; }

int smqa_debug_flags(uint32_t* flags, int32_t clear) {
  g_err.clear();
  if (!flags) return fail(SMQA_ERR_NULL, "flags is NULL");
  *flags = 0u;
#ifdef SMQA_DEBUG
  static std::atomic<void*> ptrs[smqa::kMaxDevices];
  hipError_t e = hipSuccess;
  void* p = symbol_ptr(HIP_SYMBOL(debug_word), ptrs, &e);
  if (!p) return hip_fail(e, "debug word lookup");
  if ((e = hipDeviceSynchronize()) != hipSuccess) return hip_fail(e, "smqa_debug_flags synchronise");
  unsigned v = 0u;
  if ((e = hipMemcpy(&v, p, sizeof v, hipMemcpyDeviceToHost)) != hipSuccess) return hip_fail(e, "smqa_debug_flags read");
  if (clear) {
    const unsigned zero = 0u;
    if ((e = hipMemcpy(p, &zero, sizeof zero, hipMemcpyHostToDevice)) != hipSuccess)
      return hip_fail(e, "smqa_debug_flags clear");
  }
  *flags = v;
  return SMQA_OK;
#else
  (void)clear;
  return fail(SMQA_ERR_UNSUPPORTED, "smqa_debug_flags: not an SMQA_DEBUG build");
#endif
}

size_t smqa_topk_workspace_size(const smqa_layout* L, int32_t k, int32_t n_cand) {
  if (check_layout(L) != SMQA_OK) return 0;
  return smqa::topk_workspace_bytes(L->num_q, n_cand > 0 ? n_cand : L->max_ctx, k);
}

size_t smqa_attend_workspace_size(const smqa_layout* L, int32_t k, int32_t W, int32_t Hq, int32_t D) {
  g_err.clear();
  if (check_layout(L) != SMQA_OK || check_plan(L, k, W, Hq, D) != SMQA_OK) return 0;
  return smqa::attend_workspace_bytes(L->num_q, k, W, Hq, D);
}

int smqa_attend_plan(const smqa_layout* L, int32_t k, int32_t W, int32_t Hq, int32_t D, int32_t* splits,
                     int32_t* lds_bytes) {
  g_err.clear();
  int st = check_layout(L);
  if (st) return st;
  if (D % 128 != 0 || D < 128 || D > 2048 || Hq % 16 != 0 || Hq < 16 || Hq > 128 || W < 1 || W > 128 ||
      k < 1 || k > 4096)
    return fail(SMQA_ERR_UNSUPPORTED, "attention shape outside the limits (k = %d, W = %d, Hq = %d, D = %d)",
                k, W, Hq, D);
  int32_t lds = 0;
  const int32_t S = smqa::attend_splits(L->num_q, k, W, Hq, D, &lds);
  if (splits) *splits = S;
  if (lds_bytes) *lds_bytes = lds;
  return check_plan(L, k, W, Hq, D);
}

size_t smqa_attend_fused_workspace_size(const smqa_layout* L, int32_t k, int32_t W, int32_t Hq,
                                        int32_t D) {
  g_err.clear();
  if (check_layout(L) != SMQA_OK || check_plan(L, k, W, Hq, D) != SMQA_OK) return 0;
  return smqa::attend_fused_workspace_bytes(L->num_q, k, W, Hq, D);
}

size_t smqa_decode_step_workspace_size(const smqa_layout* L, int32_t k, int32_t n_cand, int32_t W,
                                       int32_t Hq, int32_t D) {
  g_err.clear();
  if (check_layout(L) != SMQA_OK || check_plan(L, k, W, Hq, D) != SMQA_OK) return 0;
  return decode_ws_layout(L, k, n_cand > 0 ? n_cand : L->max_ctx, W, Hq, D).total;
}

int sparse_mqa_score(const smqa_layout* L, const uint8_t* q_fp8, const float* w, const uint8_t* k_fp8,
                     const float* k_scale, const int32_t* cand, int32_t n_cand, int32_t Hi, int32_t Di,
                     float* scores, int64_t ld_scores, void* stream) {
  return score_entry(L, q_fp8, w, k_fp8, k_scale, cand, n_cand, Hi, Di, scores, ld_scores, stream, false);
}

int sparse_mqa_score_fp8mma(const smqa_layout* L, const uint8_t* q_fp8, const float* w, const uint8_t* k_fp8,
                            const float* k_scale, const int32_t* cand, int32_t n_cand, int32_t Hi, int32_t Di,
                            float* scores, int64_t ld_scores, void* stream) {
  return score_entry(L, q_fp8, w, k_fp8, k_scale, cand, n_cand, Hi, Di, scores, ld_scores, stream, true);
}

int topk_select(const smqa_layout* L, const float* scores, int64_t ld_scores, const int32_t* cand,
                int32_t n_cand, int32_t k, int32_t* idx_out, float* val_out, void* workspace,
                size_t workspace_bytes, void* stream) {
  g_err.clear();
  int st = check_layout(L);
  if (st) return st;
  if (L->num_q == 0) return SMQA_OK;
  st = check_topk(L, scores, ld_scores, cand, n_cand, k, idx_out, val_out);
  if (st) return st;
  const int32_t cols = score_cols(L, n_cand, cand != nullptr);
  st = check_ws(workspace, workspace_bytes, smqa::topk_workspace_bytes(L->num_q, cols, k));
  if (st) return st;
  smqa::TopkArgs a{L->seq_start, L->q_start, L->q_pos, L->num_seqs, L->num_q, cols,
                   scores, ld_scores, cand, cand ? n_cand : 0, k, idx_out, workspace, val_out};
  hipError_t e = smqa::launch_topk(a, (hipStream_t)stream);
  return e == hipSuccess ? SMQA_OK : hip_fail(e, "topk_select launch");
}

int sparse_mqa_attend(const smqa_layout* L, const uint16_t* q_bf16, const uint8_t* kv_codes,
                      const uint8_t* kv_e8m0, const float* kv_rowscale, const int32_t* idx, int32_t k,
                      const uint8_t* swa_fp8, const float* swa_scale, const int32_t* swa_pos0,
                      const int32_t* swa_clip, int32_t W, int32_t Hq, int32_t D, float sm_scale,
                      float* out, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  int st = check_layout(L);
  if (st) return st;
  if (L->num_q == 0) return SMQA_OK;
  st = check_attend(q_bf16, kv_codes, kv_e8m0, kv_rowscale, idx, k, swa_fp8, swa_scale, swa_pos0,
                    swa_clip, W, Hq, D, sm_scale, out, lse, true);
  if (st) return st;
  st = check_plan(L, k, W, Hq, D);
  if (st) return st;
  st = check_ws(workspace, workspace_bytes, smqa::attend_workspace_bytes(L->num_q, k, W, Hq, D));
  if (st) return st;
  smqa::AttendArgs a{L->seq_start, L->q_start, L->q_pos, L->num_seqs, L->num_q, q_bf16, kv_codes,
                     kv_e8m0, kv_rowscale, idx, k, swa_fp8, swa_scale, swa_pos0, swa_clip, W, Hq, D,
                     sm_scale, out, lse, workspace};
  if (hipError_t e = attach_debug(a); e != hipSuccess) return hip_fail(e, "debug word lookup");
  hipError_t e = smqa::launch_attend(a, (hipStream_t)stream);
  return e == hipSuccess ? SMQA_OK : hip_fail(e, "sparse_mqa_attend launch");
}

int sparse_mqa_attend_fp8kv(const smqa_layout* L, const uint16_t* q_bf16, const uint8_t* kv_fp8,
                            const float* kv_rowscale, const int32_t* idx, int32_t k,
                            const uint8_t* swa_fp8, const float* swa_scale, const int32_t* swa_pos0,
                            const int32_t* swa_clip, int32_t W, int32_t Hq, int32_t D,
                            float sm_scale, float* out, float* lse, void* workspace,
                            size_t workspace_bytes, void* stream) {
  g_err.clear();
  int st = check_layout(L);
  if (st) return st;
  if (L->num_q == 0) return SMQA_OK;
  // kv_fp8 stands in for kv_codes and kv_e8m0 in the shared checks
  st = check_attend(q_bf16, kv_fp8, kv_fp8, kv_rowscale, idx, k, swa_fp8, swa_scale, swa_pos0,
                    swa_clip, W, Hq, D, sm_scale, out, lse, true);
  if (st) return st;
  st = check_plan(L, k, W, Hq, D);
  if (st) return st;
  if (Hq % 32 != 0 || D > 1664)
    return fail(SMQA_ERR_UNSUPPORTED, "FP8 global cache: Hq = %d, D = %d; supported Hq %% 32 == 0, D <= 1664",
                Hq, D);
  st = check_ws(workspace, workspace_bytes, smqa::attend_workspace_bytes(L->num_q, k, W, Hq, D));
  if (st) return st;
  smqa::AttendArgs a{L->seq_start, L->q_start, L->q_pos, L->num_seqs, L->num_q, q_bf16, kv_fp8,
                     nullptr, kv_rowscale, idx, k, swa_fp8, swa_scale, swa_pos0, swa_clip, W, Hq, D,
                     sm_scale, out, lse, workspace, smqa::kKvFP8, 1.0f};
  if (hipError_t e = attach_debug(a); e != hipSuccess) return hip_fail(e, "debug word lookup");
  hipError_t e = smqa::launch_attend_fmt(a, (hipStream_t)stream);
  return e == hipSuccess ? SMQA_OK : hip_fail(e, "sparse_mqa_attend_fp8kv launch");
}

int sparse_mqa_attend_nvfp4(const smqa_layout* L, const uint16_t* q_bf16, const uint8_t* kv_codes,
                            const uint8_t* kv_scales, const float* kv_rowscale, float kv_global_scale,
                            const int32_t* idx, int32_t k, const uint8_t* swa_fp8,
                            const float* swa_scale, const int32_t* swa_pos0, const int32_t* swa_clip,
                            int32_t W, int32_t Hq, int32_t D, float sm_scale, float* out, float* lse,
                            void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  int st = check_layout(L);
  if (st) return st;
  if (L->num_q == 0) return SMQA_OK;
  st = check_attend(q_bf16, kv_codes, kv_scales, kv_rowscale, idx, k, swa_fp8, swa_scale, swa_pos0,
                    swa_clip, W, Hq, D, sm_scale, out, lse, true);
  if (st) return st;
  st = check_plan(L, k, W, Hq, D);
  if (st) return st;
  if (Hq % 32 != 0 || D > 1664)
    return fail(SMQA_ERR_UNSUPPORTED, "NVFP4 global cache: Hq = %d, D = %d; supported Hq %% 32 == 0, D <= 1664",
                Hq, D);
  if (!(kv_global_scale >= 1e-30f && kv_global_scale <= 1e30f))
    return fail(SMQA_ERR_SHAPE, "kv_global_scale must lie in [1e-30, 1e30]");
  int ex = 0;
  std::frexp(kv_global_scale, &ex);              // g = f * 2^ex, f in [0.5, 1)
  const float K = std::ldexp(1.0f, 1 - ex);      // g * K = 2 f in [1, 2)
  st = check_ws(workspace, workspace_bytes, smqa::attend_workspace_bytes(L->num_q, k, W, Hq, D));
  if (st) return st;
  smqa::AttendArgs a{L->seq_start, L->q_start, L->q_pos, L->num_seqs, L->num_q, q_bf16, kv_codes,
                     kv_scales, kv_rowscale, idx, k, swa_fp8, swa_scale, swa_pos0, swa_clip, W, Hq, D,
                     sm_scale, out, lse, workspace, smqa::kKvNV, kv_global_scale, K};
  if (hipError_t e = attach_debug(a); e != hipSuccess) return hip_fail(e, "debug word lookup");
  hipError_t e = smqa::launch_attend_fmt(a, (hipStream_t)stream);
  return e == hipSuccess ? SMQA_OK : hip_fail(e, "sparse_mqa_attend_nvfp4 launch");
}

int sparse_mqa_attend_mxfp8q(const smqa_layout* L, const uint16_t* q_bf16, const uint8_t* kv_codes,
                             const uint8_t* kv_e8m0, const float* kv_rowscale, const int32_t* idx,
                             int32_t k, const uint8_t* swa_fp8, const float* swa_scale,
                             const int32_t* swa_pos0, const int32_t* swa_clip, int32_t W, int32_t Hq,
                             int32_t D, float sm_scale, float* out, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream) {
  g_err.clear();
  int st = check_layout(L);
  if (st) return st;
  if (L->num_q == 0) return SMQA_OK;
  st = check_attend(q_bf16, kv_codes, kv_e8m0, kv_rowscale, idx, k, swa_fp8, swa_scale, swa_pos0,
                    swa_clip, W, Hq, D, sm_scale, out, lse, true);
  if (st) return st;
  st = check_plan(L, k, W, Hq, D);
  if (st) return st;
  if (Hq % 32 != 0 || D > 1664)
    return fail(SMQA_ERR_UNSUPPORTED, "MXFP8-query attention: Hq = %d, D = %d; supported Hq %% 32 == 0, D <= 1664",
                Hq, D);
  st = check_ws(workspace, workspace_bytes, smqa::attend_workspace_bytes(L->num_q, k, W, Hq, D));
  if (st) return st;
  smqa::AttendArgs a{L->seq_start, L->q_start, L->q_pos, L->num_seqs, L->num_q, q_bf16, kv_codes,
                     kv_e8m0, kv_rowscale, idx, k, swa_fp8, swa_scale, swa_pos0, swa_clip, W, Hq, D,
                     sm_scale, out, lse, workspace, smqa::kKvMXN, 1.0f, 1.0f};
  if (hipError_t e = attach_debug(a); e != hipSuccess) return hip_fail(e, "debug word lookup");
  hipError_t e = smqa::launch_attend_fmt(a, (hipStream_t)stream);
  return e == hipSuccess ? SMQA_OK : hip_fail(e, "sparse_mqa_attend_mxfp8q launch");
}

int sparse_mqa_attend_fused(const smqa_layout* L, const uint16_t* q_bf16, const float* rope_cos,
                            const float* rope_sin, int32_t rope_pairs, const uint8_t* kv_codes,
                            const uint8_t* kv_e8m0, const float* kv_rowscale, const int32_t* idx,
                            int32_t k, const uint8_t* swa_fp8, const float* swa_scale,
                            const int32_t* swa_pos0, const int32_t* swa_clip, int32_t W, int32_t Hq,
                            int32_t D, float sm_scale, uint8_t* out_fp8, float* out_scale, float* out,
                            float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  int st = check_layout(L);
  if (st) return st;
  if (L->num_q == 0) return SMQA_OK;
  // out is optional here: out_fp8 stands in for it in the shared checks
  st = check_attend(q_bf16, kv_codes, kv_e8m0, kv_rowscale, idx, k, swa_fp8, swa_scale, swa_pos0,
                    swa_clip, W, Hq, D, sm_scale, out ? out : (const float*)out_fp8, lse, true);
  if (st) return st;
  st = check_plan(L, k, W, Hq, D);
  if (st) return st;
  st = check_fused(rope_cos, rope_sin, rope_pairs, Hq, D, out_fp8, out_scale);
  if (st) return st;
  st = check_ws(workspace, workspace_bytes, smqa::attend_fused_workspace_bytes(L->num_q, k, W, Hq, D));
  if (st) return st;
  smqa::AttendArgs a{L->seq_start, L->q_start, L->q_pos, L->num_seqs, L->num_q, q_bf16, kv_codes,
                     kv_e8m0, kv_rowscale, idx, k, swa_fp8, swa_scale, swa_pos0, swa_clip, W, Hq, D,
                     sm_scale, out, lse, workspace, smqa::kKvMX, 1.0f, 1.0f,
                     rope_pairs > 0 ? rope_cos : nullptr, rope_pairs > 0 ? rope_sin : nullptr, rope_pairs,
                     out_fp8, out_scale};
  if (hipError_t e = attach_debug(a); e != hipSuccess) return hip_fail(e, "debug word lookup");
  hipError_t e = smqa::launch_attend_fused(a, (hipStream_t)stream);
  return e == hipSuccess ? SMQA_OK : hip_fail(e, "sparse_mqa_attend_fused launch");
}

}  // extern "C"

namespace {

// Device address of `scratch` on the current device, looked up once per device (the first
// call on it) and kept; nullptr with the HIP error in *err when the lookup fails.
void* scratch_ptr(hipError_t* err) {
  static std::atomic<void*> ptrs[smqa::kMaxDevices];
  return symbol_ptr(HIP_SYMBOL(scratch), ptrs, err);
}

}  // namespace

namespace {

// The fused form's extra outputs of a decode step (NULL: the plain step).
struct FusedOut {
  const float* rope_cos;
  const float* rope_sin;
  int32_t rope_pairs;
  uint8_t* out_fp8;
  float* out_scale;
};

int decode_step_impl(const smqa_layout* L, const uint8_t* q_fp8, const float* w, const uint8_t* k_fp8,
                     const float* k_scale, const int32_t* cand, int32_t n_cand, int32_t Hi, int32_t Di,
                     const uint16_t* q_bf16, const uint8_t* kv_codes, const uint8_t* kv_e8m0,
                     const float* kv_rowscale, const uint8_t* swa_fp8, const float* swa_scale,
                     const int32_t* swa_pos0, const int32_t* swa_clip, int32_t W, int32_t Hq, int32_t D,
                     float sm_scale, int32_t k, float* out, float* lse, int32_t* idx_out, void* workspace,
                     size_t workspace_bytes, void* stream, const FusedOut* fz, bool use_scratch = false) {
  g_err.clear();
  int st = check_layout(L);
  if (st) return st;
  if (L->num_q == 0) return SMQA_OK;
  const int32_t cols = score_cols(L, n_cand, cand != nullptr);
  // the score matrix lives in the workspace with ld = cols
  st = check_score(L, q_fp8, w, k_fp8, k_scale, cand, n_cand, Hi, Di, nullptr, cols, false);
  if (st) return st;
  if (k < 1 || k > 4096) return fail(SMQA_ERR_UNSUPPORTED, "k = %d: supported 1..4096", k);
  // the fused form's fp32 output is optional: out_fp8 stands in for it in the shared checks
  const float* out_chk = (fz && !out) ? (const float*)fz->out_fp8 : out;
  st = check_attend(q_bf16, kv_codes, kv_e8m0, kv_rowscale, idx_out, k, swa_fp8, swa_scale, swa_pos0,
                    swa_clip, W, Hq, D, sm_scale, out_chk, lse, false);
  if (st) return st;
  st = check_plan(L, k, W, Hq, D);
  if (st) return st;
  if (fz) {
    st = check_fused(fz->rope_cos, fz->rope_sin, fz->rope_pairs, Hq, D, fz->out_fp8, fz->out_scale);
    if (st) return st;
  }
  const DecodeWs d = decode_ws_layout(L, k, cols, W, Hq, D);
  if (use_scratch) {
    // every argument is checked: only now is the device touched, for the scratch address
    if (d.total > (size_t)SMQA_NOALLOC_SCRATCH_BYTES)
      return fail(SMQA_ERR_WORKSPACE,
                  "decode_step_noalloc: this batch needs %zu bytes of workspace, more than the %zu-byte "
                  "device scratch buffer; call decode_step with a workspace instead",
                  d.total, (size_t)SMQA_NOALLOC_SCRATCH_BYTES);
    hipError_t e = hipSuccess;
    workspace = scratch_ptr(&e);
    if (!workspace) return hip_fail(e, "decode_step_noalloc: scratch buffer address");
    workspace_bytes = SMQA_NOALLOC_SCRATCH_BYTES;
  }
  st = check_ws(workspace, workspace_bytes, d.total);
  if (st) return st;
  char* ws = (char*)workspace;
  float* scores = (float*)(ws + d.scores_off);
  int32_t* idx = idx_out ? idx_out : (int32_t*)(ws + d.idx_off);
  hipStream_t s = (hipStream_t)stream;
  smqa::ScoreArgs sa{L->seq_start, L->q_start, L->q_pos, L->num_seqs, L->num_q, L->max_ctx,
                     q_fp8, w, k_fp8, k_scale, cand, cand ? n_cand : 0, Hi, Di, scores, cols,
                     nullptr, nullptr, 0};
  smqa::TopkArgs ta{L->seq_start, L->q_start, L->q_pos, L->num_seqs, L->num_q, cols,
                    scores, cols, cand, cand ? n_cand : 0, k, idx, ws + d.topk_off};
  // the debug word (SMQA_DEBUG builds) is looked up before anything is launched
  smqa::AttendArgs dbg_probe{};
  if (hipError_t e = attach_debug(dbg_probe); e != hipSuccess) return hip_fail(e, "debug word lookup");
  sa.dbg = dbg_probe.dbg;
  // When the streaming score kernel runs, it also builds the top-k's first-digit histogram.
  hipError_t e = hipSuccess;
  if (smqa::score_streams(sa)) {
    smqa::TopkFill fill{nullptr, nullptr, 0};
    e = smqa::launch_topk_prepare(ta, s, &fill);
    if (e != hipSuccess) return hip_fail(e, "decode_step topk launch");
    sa.hist = fill.hist;
    sa.qcols = fill.qcols;
    sa.qcols_stride = fill.qcols_stride;
  }
  e = smqa::launch_score(sa, s);
  if (e != hipSuccess) return hip_fail(e, "decode_step score launch");
  // Dense rows of at most kSelCols columns at D = 1664: every attention workgroup takes the
  // query's selection from the scores itself (same selection as topk_select), so the step has
  // no top-k launch and the workgroups start on q while the select runs.
  const bool sel_in_attend = !fz && !cand && L->max_ctx <= smqa::kSelCols &&
                             smqa::attend_select_fits(L->num_q, k, W, Hq, D);
  if (!sel_in_attend) {
    e = sa.hist ? smqa::launch_topk_from_hist(ta, s) : smqa::launch_topk(ta, s);
    if (e != hipSuccess) return hip_fail(e, "decode_step topk launch");
  }
  smqa::AttendArgs aa{L->seq_start, L->q_start, L->q_pos, L->num_seqs, L->num_q, q_bf16, kv_codes,
                      kv_e8m0, kv_rowscale, idx, k, swa_fp8, swa_scale, swa_pos0, swa_clip, W, Hq, D,
                      sm_scale, out, lse, ws + d.attend_off};
  aa.dbg = dbg_probe.dbg;
  if (sel_in_attend) {
    aa.kv_fmt = smqa::kKvMXS;
    aa.sel_scores = scores;
    aa.sel_ld = cols;
    aa.sel_max_ctx = L->max_ctx;
    aa.sel_idx = idx;
  }
  if (fz) {
    aa.rope_pairs = fz->rope_pairs;
    aa.rope_cos = fz->rope_pairs > 0 ? fz->rope_cos : nullptr;
    aa.rope_sin = fz->rope_pairs > 0 ? fz->rope_sin : nullptr;
    aa.out_fp8 = fz->out_fp8;
    aa.out_scale = fz->out_scale;
    e = smqa::launch_attend_fused(aa, s);
  } else {
    e = smqa::launch_attend(aa, s);
  }
  if (e != hipSuccess) return hip_fail(e, "decode_step attend launch");
  return SMQA_OK;
}

}  // namespace

extern "C" {

int decode_step(const smqa_layout* L, const uint8_t* q_fp8, const float* w, const uint8_t* k_fp8,
                const float* k_scale, const int32_t* cand, int32_t n_cand, int32_t Hi, int32_t Di,
                const uint16_t* q_bf16, const uint8_t* kv_codes, const uint8_t* kv_e8m0,
                const float* kv_rowscale, const uint8_t* swa_fp8, const float* swa_scale,
                const int32_t* swa_pos0, const int32_t* swa_clip, int32_t W, int32_t Hq, int32_t D,
                float sm_scale, int32_t k, float* out, float* lse, int32_t* idx_out, void* workspace,
                size_t workspace_bytes, void* stream) {
  return decode_step_impl(L, q_fp8, w, k_fp8, k_scale, cand, n_cand, Hi, Di, q_bf16, kv_codes, kv_e8m0,
                          kv_rowscale, swa_fp8, swa_scale, swa_pos0, swa_clip, W, Hq, D, sm_scale, k, out,
                          lse, idx_out, workspace, workspace_bytes, stream, nullptr);
}

int decode_step_noalloc(const smqa_layout* L, const uint8_t* q_fp8, const float* w, const uint8_t* k_fp8,
                        const float* k_scale, const int32_t* cand, int32_t n_cand, int32_t Hi, int32_t Di,
                        const uint16_t* q_bf16, const uint8_t* kv_codes, const uint8_t* kv_e8m0,
                        const float* kv_rowscale, const uint8_t* swa_fp8, const float* swa_scale,
                        const int32_t* swa_pos0, const int32_t* swa_clip, int32_t W, int32_t Hq,
                        int32_t D, float sm_scale, int32_t k, float* out, float* lse, int32_t* idx_out,
                        void* stream) {
  return decode_step_impl(L, q_fp8, w, k_fp8, k_scale, cand, n_cand, Hi, Di, q_bf16, kv_codes, kv_e8m0,
                          kv_rowscale, swa_fp8, swa_scale, swa_pos0, swa_clip, W, Hq, D, sm_scale, k, out,
                          lse, idx_out, nullptr, 0, stream, nullptr, true);
}

int decode_step_fused(const smqa_layout* L, const uint8_t* q_fp8, const float* w, const uint8_t* k_fp8,
                      const float* k_scale, const int32_t* cand, int32_t n_cand, int32_t Hi, int32_t Di,
                      const uint16_t* q_bf16, const float* rope_cos, const float* rope_sin,
                      int32_t rope_pairs, const uint8_t* kv_codes, const uint8_t* kv_e8m0,
                      const float* kv_rowscale, const uint8_t* swa_fp8, const float* swa_scale,
                      const int32_t* swa_pos0, const int32_t* swa_clip, int32_t W, int32_t Hq, int32_t D,
                      float sm_scale, int32_t k, uint8_t* out_fp8, float* out_scale, float* out, float* lse,
                      int32_t* idx_out, void* workspace, size_t workspace_bytes, void* stream) {
  const FusedOut fz{rope_cos, rope_sin, rope_pairs, out_fp8, out_scale};
  return decode_step_impl(L, q_fp8, w, k_fp8, k_scale, cand, n_cand, Hi, Di, q_bf16, kv_codes, kv_e8m0,
                          kv_rowscale, swa_fp8, swa_scale, swa_pos0, swa_clip, W, Hq, D, sm_scale, k, out,
                          lse, idx_out, workspace, workspace_bytes, stream, &fz);
}

}  // extern "C"
