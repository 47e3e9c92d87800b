/*
 * smqa.h — sparse multi-query attention decode path for AMD MI355X (gfx950).
 *
 * The operation (vLLM blog "DeepSeek-V4.1-Flash sur vLLM : 5x de débit
 * agentique dès le jour 0", sections "SWA bounded replay" and "Kernels";
 * CocoLoop digest, section "Les particularités du modèle lui-même"):
 * a decoder layer reads two caches — a compressed global latent KV, shared by
 * all heads and all layers, stored in FP4 at about 890 bytes per token, and an
 * uncompressed FP8 sliding window over the last 128 positions.  Per query
 * token it
 *   1. scores context positions with a multi-head FP8 indexer
 *      (sparse_mqa_score; blog §Kernels, "Logits MQA creux"),
 *   2. keeps the top-k positions (topk_select; blog §TL;DR and §Kernels,
 *      the DeepSelect top-k step),
 *   3. attends over the selected FP4 latent rows plus the visible FP8 window
 *      rows with one softmax (sparse_mqa_attend; blog §Kernels,
 *      "MegaAttention avec KV compressé NVFP4"),
 * and decode_step runs 1-3 in one call.  Bounded replay (blog §"Côté
 * encodeur") re-runs the last 128 tokens of a prefix hit of length H with
 * the window clipped at s = H - 128: pass per-query positions and swa_clip.
 *
 * Conventions for every entry point
 * ---------------------------------
 * - Array pointers are DEVICE pointers owned by the caller.  The library
 *   never allocates, frees or synchronises; it enqueues kernels on `stream`
 *   (a hipStream_t; NULL = the null stream) and returns.  Inputs must stay
 *   valid until the stream reaches the work.  Outputs are overwritten.
 * - Arguments are validated on the host before any HIP call.  On a
 *   validation error nothing is launched, outputs are untouched and the call
 *   returns a negative smqa_status; smqa_last_error() then describes it.
 *   Values stored inside device arrays (positions, offsets, indices) are not
 *   validated and must satisfy the stated ranges.
 * - A failed launch returns SMQA_ERR_HIP.  Device faults surface at the
 *   caller's next synchronisation.
 * - Re-entrant and thread safe: the library's only state is a thread-local
 *   error string and per-device caches of kernel attributes, filled once
 *   with atomic flags.  Concurrent calls on different streams with
 *   different workspaces are safe.
 *
 * Storage formats
 * ---------------
 * - FP8: OCP E4M3FN bytes (bias 7, max 448, 0x7F/0xFF NaN).
 * - FP4: OCP MX E2M1 nibbles, element 2i in the low nibble of byte i, one
 *   E8M0 exponent byte per 32 elements (scale 2^(e-127)), optional fp32 row
 *   scale rho.  At D = 1664 a row is 832 + 52 + 4 = 888 bytes.
 * - bf16 queries: raw bfloat16 bits.
 * Inputs must be finite (no NaN codes).  The attention path stores decoded
 * latent values in fp16 for the P*V product; this is exact when every E8M0
 * exponent e of a nonzero block satisfies -23 <= e - 127 <= 13.
 */
#ifndef SMQA_H
#define SMQA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SMQA_OK = 0,
  SMQA_ERR_NULL = -1,         /* a required pointer is NULL                          */
  SMQA_ERR_SHAPE = -2,        /* inconsistent sizes (negative, ld too small, ...)    */
  SMQA_ERR_ALIGN = -3,        /* a pointer violates its alignment requirement        */
  SMQA_ERR_UNSUPPORTED = -4,  /* a size outside the supported limits (see below)     */
  SMQA_ERR_WORKSPACE = -5,    /* workspace NULL or smaller than the size query says  */
  SMQA_ERR_HIP = -6           /* a HIP launch failed                                 */
} smqa_status;

/*
 * Ragged batch layout, shared by every call.
 *   Sequence b owns cache rows [seq_start[b], seq_start[b+1]) of the global
 *   latent and indexer-key arrays; its position j is row seq_start[b] + j.
 *   Queries are grouped by sequence: the queries of b are
 *   t in [q_start[b], q_start[b+1]) (decode: one per sequence).
 *   q_pos[t] is the absolute position p_t of query t; it bounds everything the
 *   query sees (causal, inclusive): scored positions j <= p_t, window rows at
 *   positions <= p_t.
 *   max_ctx (host) is an upper bound on the number of score columns of any
 *   query: max_t(p_t) + 1 in dense mode, n_cand in candidate mode.
 * Device arrays: seq_start int64 [B+1] (non-decreasing, seq_start[0] = 0),
 * q_start int32 [B+1] (non-decreasing, q_start[B] = num_q), q_pos int32 [T]
 * with 0 <= p_t.
 */
typedef struct {
  int32_t num_seqs;           /* B >= 1                                     */
  const int64_t* seq_start;   /* device int64 [B+1]                         */
  int32_t num_q;              /* T >= 0                                     */
  const int32_t* q_start;     /* device int32 [B+1]                         */
  const int32_t* q_pos;       /* device int32 [T]                           */
  int32_t max_ctx;            /* host bound on score columns per query      */
} smqa_layout;

/*
 * Limits (SMQA_ERR_UNSUPPORTED beyond them):
 *   indexer  Di in {64, 128}; 1 <= Hi <= 128
 *   attention D % 128 == 0, 128 <= D <= 2048; Hq % 16 == 0, 16 <= Hq <= 128;
 *             1 <= W <= 128
 *   top-k    1 <= k <= 4096
 * Alignment: q_fp8, k_fp8, kv_codes, swa_fp8, q_bf16, out: 16 bytes;
 *            workspace: 256 bytes; every other pointer: 4 bytes.
 */

/*
 * sparse_mqa_score — indexer scoring (blog §Kernels, "Logits MQA creux": one
 * score per context position; late indexer layers score only a fixed set of
 * 16K candidate positions, so their cost does not grow with the context).
 *
 *   S[t, j] = sum_{h < Hi} w[t,h] * max(0, kappa_j * sum_{d < Di} qI[t,h,d] * kI[row(j), d])
 *
 * Dense mode (cand == NULL): for every query t and every position
 *   0 <= j <= min(p_t, len_b - 1), scores[t * ld_scores + j] = S[t, j];
 *   the columns past that bound, up to ld_scores, receive -INFINITY.
 * Candidate mode (cand != NULL): cand[t * n_cand + i] (i < n_cand) are
 *   positions of query t's sequence, strictly ascending per query;
 *   scores[t * ld_scores + i] = S[t, cand[t,i]], or -INFINITY when the
 *   candidate is past p_t or past the sequence; columns n_cand .. ld_scores-1
 *   receive -INFINITY.
 * Every entry of the [T][ld_scores] array is written.
 * q_fp8   uint8  [T][Hi][Di]  E4M3 indexer queries
 * w       float  [T][Hi]      head weights (any sign)
 * k_fp8   uint8  [N][Di]      E4M3 indexer keys, N = seq_start[B]
 * k_scale float  [N] or NULL  per-key scale kappa (> 0; NULL = 1)
 * scores  float  [T][ld_scores], ld_scores >= max_ctx (dense) / >= n_cand
 * Arithmetic: FP8 x FP8 products are exact; sums are fp32.
 */
int sparse_mqa_score(const smqa_layout* L,
                     const uint8_t* q_fp8, const float* w,
                     const uint8_t* k_fp8, const float* k_scale,
                     const int32_t* cand, int32_t n_cand,
                     int32_t Hi, int32_t Di,
                     float* scores, int64_t ld_scores,
                     void* stream);

/*
 * sparse_mqa_score_fp8mma — sparse_mqa_score with the contraction on the FP8
 * matrix cores (blog §Kernels: the indexer's logits are computed in FP8).  Same
 * arguments, outputs and errors, plus SMQA_ERR_UNSUPPORTED unless Di == 128.
 * The E4M3 bytes of q and k enter v_mfma_scale_f32_16x16x128_f8f6f4 as stored
 * (unit scales), one instruction per 16 heads x 16 positions x 128 dims.
 * Arithmetic: the products are exact, but the instruction adds the 128 of one
 * logit with an error of up to about 2^-15 of their absolute sum (measured on
 * gfx950); the head sum, ReLU and kappa are fp32 as in sparse_mqa_score.  So a
 * score S carries an error up to about 2^-15 * sum_h |w_h| * sum_d |q_hd k_d|
 * (times kappa): relative to S this stays below 1e-4 when the head weights are
 * non-negative and the logits do not nearly cancel, not for every input.
 * sparse_mqa_score (exact products, fp32 sums) is the reference form;
 * decode_step uses it.
 */
int sparse_mqa_score_fp8mma(const smqa_layout* L,
                            const uint8_t* q_fp8, const float* w,
                            const uint8_t* k_fp8, const float* k_scale,
                            const int32_t* cand, int32_t n_cand,
                            int32_t Hi, int32_t Di,
                            float* scores, int64_t ld_scores,
                            void* stream);

/*
 * topk_select — the k best positions per query (blog §TL;DR: DeepSelect, a
 * top-k library for DeepSeek Sparse Attention; §Kernels: the indexer's top-k
 * over the scored positions).
 *
 * Order: score descending, ties to the lower position.  The scored set of
 * query t is columns 0..min(p_t, len_b - 1) (dense) or the columns whose
 * score is not -INFINITY (candidate mode; positions are cand[t, col]).
 * idx_out[t * k + i] receives the selected positions in ascending order;
 * when the set has m < k entries, slots m..k-1 hold -1.  val_out (float
 * [T][k], or NULL) receives the score of each selected position, bit for bit
 * the input entry, and -INFINITY in the padding slots.  Bitwise
 * deterministic.  scores is read only.
 * workspace: smqa_topk_workspace_size() bytes, 256-byte aligned, contents
 * need not be initialised; it is clobbered.
 */
int topk_select(const smqa_layout* L,
                const float* scores, int64_t ld_scores,
                const int32_t* cand, int32_t n_cand,
                int32_t k, int32_t* idx_out, float* val_out,
                void* workspace, size_t workspace_bytes,
                void* stream);

/*
 * sparse_mqa_attend — multi-query attention of Hq heads over one shared
 * latent (blog §"Performances agentiques": the KV latent is shared by all
 * heads; §Kernels, MegaAttention: sparse attention reading the FP4 KV) over
 *   the selected global rows   V[j] = e2m1 * 2^(E-127) * rho_j, j in idx[t] (j >= 0),
 *   plus the window rows       X[u] = e4m3 * sigma_u at positions
 *                              max(p_t - W + 1, s_t, 0) <= swa_pos0[b] + u <= p_t
 * (blog §"SWA bounded replay": FP8 window of the last 128 positions; clipped
 * at the replay start s = H - 128).  The latent row is both key and value.
 * One softmax over the union, per head h:
 *   l_x = sm_scale * <q[t,h], row_x>;  out[t,h] = sum_x softmax(l)_x row_x;
 *   lse[t,h] = log(sum_x exp(l_x))   (natural log; -INFINITY and out = 0
 *   when the query sees no row).
 * q_bf16      uint16 [T][Hq][D]     bf16 bits
 * kv_codes    uint8  [N][D/2]       E2M1 pairs
 * kv_e8m0     uint8  [N][D/32]      block exponents
 * kv_rowscale float  [N] or NULL    rho (NULL = 1)
 * idx         int32  [T][k]         positions within the query's sequence,
 *                                   0 <= j <= p_t and j < len_b, or -1 (skipped)
 * swa_fp8     uint8  [B][W][D]      window rows; row u has position swa_pos0[b] + u
 * swa_scale   float  [B][W] or NULL sigma (NULL = 1)
 * swa_pos0    int32  [B]
 * swa_clip    int32  [T] or NULL    s_t (NULL = no clip)
 * out         float  [T][Hq][D]     lse float [T][Hq] or NULL
 * workspace: smqa_attend_workspace_size() bytes (may be 0 -> workspace may be NULL).
 * Arithmetic: q.row on bf16 MFMA with fp32 sums; softmax in fp32; P*V on fp16
 * MFMA (P rounded to fp16 once) with fp32 sums; rho and sigma applied in fp32.
 */
int sparse_mqa_attend(const smqa_layout* L,
                      const uint16_t* q_bf16,
                      const uint8_t* kv_codes, const uint8_t* kv_e8m0, const float* kv_rowscale,
                      const int32_t* idx, int32_t k,
                      const uint8_t* swa_fp8, const float* swa_scale,
                      const int32_t* swa_pos0, const int32_t* swa_clip,
                      int32_t W, int32_t Hq, int32_t D, float sm_scale,
                      float* out, float* lse,
                      void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * sparse_mqa_attend_fp8kv — sparse_mqa_attend over an FP8 global cache, the
 * format the FP4 cache replaced (CocoLoop digest, section "Les
 * particularités du modèle lui-même": the NVFP4 global KV is about 45%
 * smaller than the FP8 one; blog §Kernels).  A baseline for measuring what
 * the FP4 format saves; the selected global rows are
 *   V[j] = e4m3 * rho_j,  j in idx[t] (j >= 0)
 * and everything else (window, clip, softmax, outputs, workspace size from
 * smqa_attend_workspace_size, errors) is as in sparse_mqa_attend.
 * kv_fp8      uint8  [N][D]         E4M3 latent rows, 16-byte aligned
 * kv_rowscale float  [N] or NULL    rho (> 0; NULL = 1)
 * Limits: those of sparse_mqa_attend plus Hq % 32 == 0 and D <= 1664.
 * Arithmetic as in sparse_mqa_attend (E4M3 values are exact in bf16 and fp16).
 */
int sparse_mqa_attend_fp8kv(const smqa_layout* L,
                            const uint16_t* q_bf16,
                            const uint8_t* kv_fp8, const float* kv_rowscale,
                            const int32_t* idx, int32_t k,
                            const uint8_t* swa_fp8, const float* swa_scale,
                            const int32_t* swa_pos0, const int32_t* swa_clip,
                            int32_t W, int32_t Hq, int32_t D, float sm_scale,
                            float* out, float* lse,
                            void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * sparse_mqa_attend_nvfp4 — sparse_mqa_attend over a global cache in the
 * NVFP4 layout (blog §Kernels, MegaAttention reading the NVFP4 KV; CocoLoop
 * digest, section "Les particularités du modèle lui-même": the global KV is
 * stored in NVFP4): E2M1 elements with one E4M3 scale per 16 elements and one
 * fp32 scale per tensor.  The selected global rows are
 *   V[j, d] = e2m1 * e4m3(S[j, d/16]) * rho_j * g,  j in idx[t] (j >= 0)
 * and everything else (window, clip, softmax, outputs, workspace size from
 * smqa_attend_workspace_size, errors) is as in sparse_mqa_attend.
 * kv_codes        uint8 [N][D/2]   E2M1 pairs (element 2i in the low nibble), 16-byte aligned
 * kv_scales       uint8 [N][D/16]  E4M3 block scales, 4-byte aligned
 * kv_rowscale     float [N] or NULL  optional extra row scale rho (> 0; NULL = 1)
 * kv_global_scale g, the tensor scale, in [1e-30, 1e30] (else SMQA_ERR_SHAPE);
 *                 the window scales must satisfy sigma_u <= 32768 * g (P carries
 *                 sigma times a power of two near 1/g in fp16)
 * Limits: those of sparse_mqa_attend plus Hq % 32 == 0 and D <= 1664.
 * Arithmetic as in sparse_mqa_attend except that q.row runs on fp16 MFMA:
 * q is converted to fp16 once (exact for 2^-14 <= |q| <= 65504; |q| must
 * stay below 65504), e2m1 * e4m3 is exact in fp16; rho * g multiplies the
 * logits in fp32.
 */
int sparse_mqa_attend_nvfp4(const smqa_layout* L,
                            const uint16_t* q_bf16,
                            const uint8_t* kv_codes, const uint8_t* kv_scales,
                            const float* kv_rowscale, float kv_global_scale,
                            const int32_t* idx, int32_t k,
                            const uint8_t* swa_fp8, const float* swa_scale,
                            const int32_t* swa_pos0, const int32_t* swa_clip,
                            int32_t W, int32_t Hq, int32_t D, float sm_scale,
                            float* out, float* lse,
                            void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * sparse_mqa_attend_mxfp8q — sparse_mqa_attend with Q.K^T on gfx950's scaled matrix
 * cores (v_mfma_scale_f32_32x32x64_f8f6f4), which read the gathered E2M1 rows and their
 * E8M0 block exponents as stored (blog §Kernels: MegaAttention reads the NVFP4 KV
 * natively).  Their other operand is 8-bit, so the query is quantised to OCP MXFP8 first:
 * per (query, head) and 32-dim block, E = floor(log2 amax) - 8 + 127 (clamped at 0; 0 for
 * a zero block) and elements E4M3(q / 2^(E-127)), nearest even, saturating at 448.  Both
 * branches' logits use that quantised query (window rows enter as E4M3 with scale 2^0);
 * the softmax, P*V (exact fp16 values, as in sparse_mqa_attend) and the outputs are those
 * of sparse_mqa_attend, as are the arguments, layout, workspace
 * (smqa_attend_workspace_size) and errors.
 * Limits: those of sparse_mqa_attend plus Hq % 32 == 0 and D <= 1664.
 * Arithmetic: the products of the MXFP8 query and the E2M1 / E4M3 rows are exact; each
 * instruction sums its 64 products with an internal error of about 1e-5 of their
 * absolute sum before the fp32 accumulation.
 */
int sparse_mqa_attend_mxfp8q(const smqa_layout* L,
                             const uint16_t* q_bf16,
                             const uint8_t* kv_codes, const uint8_t* kv_e8m0, const float* kv_rowscale,
                             const int32_t* idx, int32_t k,
                             const uint8_t* swa_fp8, const float* swa_scale,
                             const int32_t* swa_pos0, const int32_t* swa_clip,
                             int32_t W, int32_t Hq, int32_t D, float sm_scale,
                             float* out, float* lse,
                             void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * sparse_mqa_attend_fused — MegaAttention's fused form (blog §Kernels,
 * "MegaAttention avec KV compressé NVFP4": query RoPE, the sparse attention,
 * inverse RoPE on the output and FP8 conversion in one pass, written for the
 * output projection) over the FP4 (MX) cache of sparse_mqa_attend:
 *   q'      = q with the pairs (2i, 2i+1) of its last 2R dims (R = rope_pairs)
 *             rotated by query t's angle: (a, b) -> (a c - b s, a s + b c),
 *             c = rope_cos[t][i], s = rope_sin[t][i], rounded once to bf16
 *             (nearest even) for the products.  The rotation is evaluated in
 *             fp64, where the products are exact, so q' is the bf16 nearest to
 *             the rotation (one bf16 unit of q' moves a flat-softmax output by
 *             about 1e-3 of its magnitude, so the rounding is not left loose).
 *   O       = sparse_mqa_attend(q', ...)
 *   O'      = O with the same pairs rotated back: (a, b) -> (a c + b s, -a s + b c)
 *   out_scale[t,h] = max_d |O'[t,h,d]| / 448,
 *   out_fp8[t,h,d] = E4M3(O'[t,h,d] * 448 / amax), nearest even (an all-zero
 *             row gives scale 0 and zero codes).  Evaluated in fp32 as
 *             O' * (448 / amax): one division per row, one product per element,
 *             so a value within 2^-22 relative of a rounding midpoint may take
 *             the neighbouring code.
 * so out_fp8 * out_scale approximates O' within E4M3's 2^-4 relative step.
 * rope_cos, rope_sin float [T][R], 16-byte aligned (may be NULL when R = 0);
 *             the angles of each query's position (frequencies, scaling and the
 *             position itself are the caller's)
 * rope_pairs  R: a multiple of 4 with 2R <= D (0 = no rotation)
 * out_fp8     uint8 [T][Hq][D], 16-byte aligned;  out_scale float [T][Hq]
 * out         float [T][Hq][D] or NULL: O' in fp32 (optional)
 * lse         float [T][Hq] or NULL (of the rotated query's logits)
 * workspace:  smqa_attend_fused_workspace_size() bytes (the split partials;
 *             0 when one split suffices, as for sparse_mqa_attend).
 * Limits: those of sparse_mqa_attend plus Hq % 32 == 0 and D <= 1664; other
 * arguments as in sparse_mqa_attend.
 */
int sparse_mqa_attend_fused(const smqa_layout* L,
                            const uint16_t* q_bf16,
                            const float* rope_cos, const float* rope_sin, int32_t rope_pairs,
                            const uint8_t* kv_codes, const uint8_t* kv_e8m0, const float* kv_rowscale,
                            const int32_t* idx, int32_t k,
                            const uint8_t* swa_fp8, const float* swa_scale,
                            const int32_t* swa_pos0, const int32_t* swa_clip,
                            int32_t W, int32_t Hq, int32_t D, float sm_scale,
                            uint8_t* out_fp8, float* out_scale, float* out, float* lse,
                            void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * decode_step — sparse_mqa_score -> topk_select -> sparse_mqa_attend in one
 * call on one stream, with the scores and the selection kept in the
 * workspace (blog §Kernels: fusing the steps removes memory round trips and
 * launches between them).  Arguments mean what they mean in the three calls;
 * idx_out (int32 [T][k]) optionally receives the selection.  Works for any
 * layout: decode (one query per sequence at p = len - 1) and bounded-replay
 * chunks (several queries per sequence with swa_clip).  On dense rows of at
 * most 8192 columns with D = 1664 the attention kernel takes the selection
 * from the scores itself (no separate top-k launch); the selection, the
 * output and the LSE are those of the three separate calls, bit for bit.
 */
int decode_step(const smqa_layout* L,
                const uint8_t* q_fp8, const float* w,
                const uint8_t* k_fp8, const float* k_scale,
                const int32_t* cand, int32_t n_cand,
                int32_t Hi, int32_t Di,
                const uint16_t* q_bf16,
                const uint8_t* kv_codes, const uint8_t* kv_e8m0, const float* kv_rowscale,
                const uint8_t* swa_fp8, const float* swa_scale,
                const int32_t* swa_pos0, const int32_t* swa_clip,
                int32_t W, int32_t Hq, int32_t D, float sm_scale,
                int32_t k,
                float* out, float* lse, int32_t* idx_out,
                void* workspace, size_t workspace_bytes,
                void* stream);

/*
 * decode_step_noalloc — decode_step for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation, arguments, outputs and errors, without the
 * workspace arguments.  The workspace is a device array inside the library,
 * SMQA_NOALLOC_SCRATCH_BYTES bytes per GPU, held from the library's first use on
 * that GPU until the process ends; its address is looked up on the first call on
 * each device.  The call allocates nothing and frees nothing.
 * - A batch whose decode_step workspace (smqa_decode_step_workspace_size) exceeds
 *   SMQA_NOALLOC_SCRATCH_BYTES returns SMQA_ERR_WORKSPACE before any HIP call
 *   (96 MiB covers decode batches up to 4 x 512K positions or 32 x 64K; a
 *   1024-query replay chunk does not fit: use decode_step).
 * - Every call on one GPU shares that GPU's array, which keeps the last call's
 *   contents; the step clears what must start at zero itself.  Calls that
 *   overlap on one GPU (different streams, or threads) race on the array and must
 *   be serialised by the caller.
 */
#define SMQA_NOALLOC_SCRATCH_BYTES (96u << 20)
int decode_step_noalloc(const smqa_layout* L,
                        const uint8_t* q_fp8, const float* w,
                        const uint8_t* k_fp8, const float* k_scale,
                        const int32_t* cand, int32_t n_cand,
                        int32_t Hi, int32_t Di,
                        const uint16_t* q_bf16,
                        const uint8_t* kv_codes, const uint8_t* kv_e8m0, const float* kv_rowscale,
                        const uint8_t* swa_fp8, const float* swa_scale,
                        const int32_t* swa_pos0, const int32_t* swa_clip,
                        int32_t W, int32_t Hq, int32_t D, float sm_scale,
                        int32_t k,
                        float* out, float* lse, int32_t* idx_out,
                        void* stream);

/*
 * decode_step_fused — decode_step with MegaAttention's fused form as its
 * attention (sparse_mqa_attend_fused: query RoPE by rope_cos / rope_sin on the
 * last 2 * rope_pairs dims, inverse RoPE and FP8 output): the output
 * projection's input comes out of one call.  Arguments mean what they mean in
 * decode_step and sparse_mqa_attend_fused (out, the fp32 output, is optional;
 * out_fp8 and out_scale are required); the workspace is
 * smqa_decode_step_workspace_size() bytes; the limits are those of both.
 */
int decode_step_fused(const smqa_layout* L,
                      const uint8_t* q_fp8, const float* w,
                      const uint8_t* k_fp8, const float* k_scale,
                      const int32_t* cand, int32_t n_cand,
                      int32_t Hi, int32_t Di,
                      const uint16_t* q_bf16,
                      const float* rope_cos, const float* rope_sin, int32_t rope_pairs,
                      const uint8_t* kv_codes, const uint8_t* kv_e8m0, const float* kv_rowscale,
                      const uint8_t* swa_fp8, const float* swa_scale,
                      const int32_t* swa_pos0, const int32_t* swa_clip,
                      int32_t W, int32_t Hq, int32_t D, float sm_scale,
                      int32_t k,
                      uint8_t* out_fp8, float* out_scale, float* out, float* lse, int32_t* idx_out,
                      void* workspace, size_t workspace_bytes,
                      void* stream);

/* Workspace sizes in bytes (host-only arithmetic, no HIP call).  A NULL or
 * inconsistent layout, or an attention shape smqa_attend_plan rejects, returns 0 and
 * sets smqa_last_error(). */
size_t smqa_topk_workspace_size(const smqa_layout* L, int32_t k, int32_t n_cand);
size_t smqa_attend_workspace_size(const smqa_layout* L, int32_t k, int32_t W,
                                  int32_t Hq, int32_t D);
size_t smqa_attend_fused_workspace_size(const smqa_layout* L, int32_t k, int32_t W,
                                        int32_t Hq, int32_t D);
size_t smqa_decode_step_workspace_size(const smqa_layout* L, int32_t k, int32_t n_cand,
                                       int32_t W, int32_t Hq, int32_t D);

/* How the attention calls run a batch of this shape (host-only arithmetic, no HIP
 * call): *splits receives the number of tile ranges each (query, head group) is cut into
 * (their partial results are merged by log-sum-exp; 1 = no partials, no workspace) and
 * *lds_bytes the LDS one workgroup uses (static + dynamic) at that split count; either
 * pointer may be NULL.  Returns SMQA_OK, SMQA_ERR_UNSUPPORTED for a shape outside the
 * limits or one whose workgroup needs more than a compute unit's 160 KiB of LDS at every
 * split count (every attention call and workspace query rejects such a shape the same
 * way), or the layout's error. */
int smqa_attend_plan(const smqa_layout* L, int32_t k, int32_t W, int32_t Hq, int32_t D,
                     int32_t* splits, int32_t* lds_bytes);

/* Thread-local description of the last non-OK return on this thread ("" if none). */
const char* smqa_last_error(void);

/* Library version string. */
const char* smqa_version(void);

/* ---------------------------------------------------------------------------
 * Range checks of the values stored inside device arrays (debug builds).
 *
 * Every build treats a selected position j outside [0, min(p_t, len_b - 1)] as
 * skipped, like the padding value -1, so a bad index never makes an attention
 * kernel read outside the query's rows; a negative q_pos scores nothing (its row
 * is all -INFINITY) and a decreasing seq_start reads as an empty sequence.  A library built with SMQA_DEBUG
 * defined (fp8_kv_cache_sparse_amd/libsmqa_debug.so, from the same sources)
 * also reports what it met, in one word per GPU that the attention kernels OR
 * bits into:
 *   SMQA_DEBUG_POSITION  a selected position outside that range other than -1
 *                        (sparse_mqa_attend*, decode_step*)
 *   SMQA_DEBUG_E8M0      an E8M0 exponent e of a row that takes part, outside
 *                        the range P*V holds exactly in fp16 (-23 <= e - 127
 *                        <= 13) and not 0 (MX global caches)
 *   SMQA_DEBUG_LAYOUT    seq_start or q_start decreasing, or a negative q_pos
 *                        (sparse_mqa_score*, decode_step*)
 *   SMQA_DEBUG_CAND      a candidate list that is not strictly ascending
 *                        (sparse_mqa_score*, decode_step* in candidate mode)
 * smqa_debug_flags waits for the current device to finish its work
 * (hipDeviceSynchronize), stores the word in *flags and clears it when clear
 * is nonzero.  It returns SMQA_OK in a debug build and SMQA_ERR_UNSUPPORTED
 * (with *flags = 0) in a release build, SMQA_ERR_NULL for flags == NULL and
 * SMQA_ERR_HIP when a HIP call fails.  Kernels never trap on these findings;
 * outputs are computed with the offending positions skipped.
 * ------------------------------------------------------------------------- */
#define SMQA_DEBUG_POSITION 1u
#define SMQA_DEBUG_E8M0 2u
#define SMQA_DEBUG_LAYOUT 4u
#define SMQA_DEBUG_CAND 8u
int smqa_debug_flags(uint32_t* flags, int32_t clear);

#ifdef __cplusplus
}
#endif
#endif /* SMQA_H */
