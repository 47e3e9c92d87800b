"""Reference (fp64) definitions of the three steps and of the fused decode step.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Layout conventions shared with the GPU library's boundary (the arrays are the
same bytes; the code is not shared):

* sequence b owns cache rows [seq_start[b], seq_start[b+1]); its position j
  is row seq_start[b] + j;
* queries are grouped by sequence: queries of b are t in [q_start[b], q_start[b+1]);
* q_pos[t] = p_t, the query's absolute position (the causal bound, inclusive);
* the window buffer of sequence b holds W rows; row u has position swa_pos0[b] + u;
* swa_clip[t] = s_t, the replay clip start (None: no clip).

Readings where the pages are silent (each restated where it is used):
  R1  indexer form S = sum_h w_h * max(0, kappa_j <q_h, k_j>)   [parity unpinned vs the pages]
  R2  top-k order: score descending, ties to the lower position; output sorted
      ascending by position, padded with -1
  R3  K = V = the decoded latent row (multi-query attention over one latent
      shared by all heads)                                      [parity unpinned vs the pages]
  R4  one softmax over the union of selected global rows and visible window
      rows; a position in both sets contributes twice (two representations)
  R5  the window of query t is positions [max(p_t - W + 1, s_t, 0), p_t]
      that exist in the buffer; rows before the clip s_t are excluded
  R6  an empty row set gives O = 0 and LSE = -inf
  R14 the FP8 global cache (the baseline format) is E4M3 rows with one fp32
      scale per row
  R15 NVFP4 = E2M1 with one E4M3 scale per 16 elements and one fp32 tensor
      scale (the pages name the format only)
  R16 fused RoPE: the last 2R latent dims rotate in consecutive pairs by
      per-query angles the caller gives as cos / sin; the rotated query is
      rounded once to bf16 (nearest even) before the products
  R17 FP8 output: per (query, head) row, scale = amax / 448 and codes =
      E4M3(x * 448 / amax), nearest even, saturating at 448 (an all-zero row:
      scale 0, codes 0)
  R18 attention on scaled matrix cores (NEXT row f4): the query is quantised
      to OCP MXFP8 (32-dim blocks, E8M0 = floor(log2 amax) - 8 + 127 clamped
      to [0, 254], E4M3 elements nearest even, saturating) for the logits of
      both branches; P * V keeps the exact values
"""
from __future__ import annotations

import numpy as np

from . import codecs


def _q_seq(q_start: np.ndarray) -> np.ndarray:
    q_start = np.asarray(q_start, dtype=np.int64)
    counts = np.diff(q_start)
    return np.repeat(np.arange(len(counts)), counts)


def scored_positions(t, q_pos, seq_len, cand=None):
    """J_t: the positions query t scores, with the column each score is stored in.

    Dense mode: J_t = {0..p_t}, column = position.  Candidate mode (blog
    §Kernels, "Logits MQA creux": late indexer layers take their top-k from a
    fixed set of 16K candidate positions): J_t = {cand[t,i] : cand[t,i] <= p_t,
    0 <= cand[t,i] < seq_len}, column = i.
    """
    p = int(q_pos[t])
    if cand is None:
        pos = np.arange(0, min(p, seq_len - 1) + 1, dtype=np.int64)
        return pos, pos.copy()
    c = np.asarray(cand[t], dtype=np.int64)
    keep = (c >= 0) & (c <= p) & (c < seq_len)
    cols = np.nonzero(keep)[0]
    return c[cols], cols


def score(qI, w, kI, kscale, seq_start, q_start, q_pos, cand=None, ld=None):
    """Indexer scores S[t, col] (float64, -inf where nothing is scored).

    Blog §Kernels ("Logits MQA creux"): the indexer produces one score per
    context position, from which top-k positions are taken; the sparse variant
    scores only the candidate set.  Reading R1 gives the per-position value:
    S[t,j] = sum_h w[t,h] * max(0, kappa_j * sum_d qI[t,h,d] * kI[row(j),d]).
    """
    qI = np.asarray(qI)
    T = qI.shape[0]
    seq_start = np.asarray(seq_start, dtype=np.int64)
    qs = _q_seq(q_start)
    if ld is None:
        ld = np.asarray(cand).shape[1] if cand is not None else int(np.max(q_pos)) + 1
    S = np.full((T, ld), -np.inf, dtype=np.float64)
    for t in range(T):
        b = qs[t]
        base = seq_start[b]
        n = int(seq_start[b + 1] - base)
        pos, cols = scored_positions(t, q_pos, n, cand)
        if pos.size == 0:
            continue
        rows = base + pos
        Q = codecs.e4m3(qI[t])                       # [Hi, Di]
        K = codecs.e4m3(np.asarray(kI)[rows])        # [n, Di]
        dots = K @ Q.T                               # [n, Hi]
        if kscale is not None:
            dots = dots * np.asarray(kscale, dtype=np.float64)[rows][:, None]
        S[t, cols] = np.maximum(dots, 0.0) @ np.asarray(w[t], dtype=np.float64)
    return S


def topk(S, k, cand=None):
    """Top-k positions per query (reading R2), int64 [T, k], ascending, -1 padded.

    Entries equal to -inf are not in J_t and are never selected.  With a
    candidate list the returned values are positions cand[t, col].
    """
    S = np.asarray(S, dtype=np.float64)
    T, L = S.shape
    out = np.full((T, k), -1, dtype=np.int64)
    for t in range(T):
        cols = np.nonzero(S[t] != -np.inf)[0]
        pos = cols if cand is None else np.asarray(cand[t], dtype=np.int64)[cols]
        order = np.lexsort((pos, -S[t, cols]))       # primary: -score, secondary: position
        take = np.sort(pos[order[:k]])
        out[t, :take.size] = take
    return out


def window_positions(t, b, q_pos, swa_pos0, swa_clip, W):
    """Buffer slots u (and positions) visible to query t (reading R5)."""
    p = int(q_pos[t])
    lo = max(p - W + 1, 0)
    if swa_clip is not None:
        lo = max(lo, int(swa_clip[t]))
    pos = int(swa_pos0[b]) + np.arange(W, dtype=np.int64)
    u = np.nonzero((pos >= lo) & (pos <= p))[0]
    return u, pos[u]


def _attend_union(q, global_of, idx, swa, swa_scale, swa_pos0, swa_clip, seq_start, q_start,
                  q_pos, W, sm_scale, q_values=None):
    """One softmax per (query, head) over the selected global rows plus the visible window
    rows; global_of(cache_rows) decodes the selected rows of the global cache.  q_values, when
    given, replaces the decoded bf16 query (float64 [T, Hq, D])."""
    qv = codecs.bf16(q) if q_values is None else np.asarray(q_values, dtype=np.float64)
    T, Hq, D = qv.shape
    seq_start = np.asarray(seq_start, dtype=np.int64)
    qs = _q_seq(q_start)
    idx = np.asarray(idx, dtype=np.int64)
    O = np.zeros((T, Hq, D), dtype=np.float64)
    LSE = np.full((T, Hq), -np.inf, dtype=np.float64)
    for t in range(T):
        b = qs[t]
        sel = idx[t][idx[t] >= 0]
        Vg = global_of(seq_start[b] + sel)
        u, _ = window_positions(t, b, q_pos, swa_pos0, swa_clip, W)
        Xw = codecs.window_rows(np.asarray(swa)[b][u],
                                None if swa_scale is None else np.asarray(swa_scale)[b][u])
        R = np.concatenate([Vg.reshape(-1, D), Xw.reshape(-1, D)], axis=0)
        if R.shape[0] == 0:
            continue
        L = sm_scale * (qv[t] @ R.T)                 # [Hq, nrows]
        m = L.max(axis=1, keepdims=True)
        e = np.exp(L - m)
        Z = e.sum(axis=1, keepdims=True)
        O[t] = (e @ R) / Z
        LSE[t] = (m + np.log(Z))[:, 0]
    return O, LSE


def attend(q, kv_codes, kv_e8m0, kv_rowscale, idx, swa, swa_scale, swa_pos0, swa_clip,
           seq_start, q_start, q_pos, W, sm_scale):
    """Sparse MQA attention over selected global rows plus the visible window rows.

    Blog §Kernels (MegaAttention with NVFP4 KV): sparse attention reading the
    FP4 compressed KV; blog §"SWA bounded replay": a global KV shared across
    layers in FP4 and an uncompressed FP8 window of the last 128 positions;
    blog §"Performances agentiques": the KV latent is shared by all heads.
    For each query t and head h (readings R3, R4, R6):
        rows  = {V[j] : j in idx[t], j >= 0} + {X[u] : u visible (R5)}
        l_x   = sm_scale * <q[t,h], row_x>
        O     = sum_x exp(l_x - m) row_x / sum_x exp(l_x - m),   m = max_x l_x
        LSE   = m + ln(sum_x exp(l_x - m))
    q is bf16 bits (uint16 [T, Hq, D]); returns float64 O [T, Hq, D], LSE [T, Hq].
    """
    codes, e8 = np.asarray(kv_codes), np.asarray(kv_e8m0)
    rs = None if kv_rowscale is None else np.asarray(kv_rowscale)

    def global_of(rows):
        return codecs.global_rows(codes[rows], e8[rows], None if rs is None else rs[rows])
    return _attend_union(q, global_of, idx, swa, swa_scale, swa_pos0, swa_clip, seq_start,
                         q_start, q_pos, W, sm_scale)


def attend_fp8kv(q, kv_fp8, kv_rowscale, idx, swa, swa_scale, swa_pos0, swa_clip,
                 seq_start, q_start, q_pos, W, sm_scale):
    """The same attention over an FP8 global cache (the format the FP4 cache replaces).

    CocoLoop digest §"Les particularités du modèle lui-même" and blog §Kernels:
    the NVFP4 global KV is about 45% smaller than the FP8 cache used before it.
    Reading R14: that FP8 cache holds each latent row as D E4M3 bytes times one
    fp32 row scale rho_j (the window's format), V[j, d] = e4m3(byte) * rho_j;
    everything else is `attend`.  kv_fp8 uint8 [N, D], kv_rowscale float32 [N]
    or None (rho = 1).
    """
    codes = np.asarray(kv_fp8)
    rs = None if kv_rowscale is None else np.asarray(kv_rowscale)

    def global_of(rows):
        return codecs.window_rows(codes[rows], None if rs is None else rs[rows])
    return _attend_union(q, global_of, idx, swa, swa_scale, swa_pos0, swa_clip, seq_start,
                         q_start, q_pos, W, sm_scale)


def attend_nvfp4(q, kv_codes, kv_scales, kv_rowscale, kv_global_scale, idx, swa, swa_scale,
                 swa_pos0, swa_clip, seq_start, q_start, q_pos, W, sm_scale):
    """The same attention over a global cache in the NVFP4 layout.

    Blog §Kernels and CocoLoop digest §"Les particularités du modèle lui-même" name the
    global KV format NVFP4: E2M1 elements, one E4M3 scale per 16 consecutive elements and
    one fp32 scale g per tensor (reading R15), V[j, d] = e2m1 * e4m3(S[j, d // 16]) * rho_j * g
    with the optional fp32 row scale rho of the MX layout kept; everything else is `attend`.
    kv_codes uint8 [N, D/2], kv_scales uint8 [N, D/16], kv_rowscale float32 [N] or None.
    """
    codes, sc = np.asarray(kv_codes), np.asarray(kv_scales)
    rs = None if kv_rowscale is None else np.asarray(kv_rowscale)

    def global_of(rows):
        return codecs.nvfp4_rows(codes[rows], sc[rows], None if rs is None else rs[rows],
                                 kv_global_scale)
    return _attend_union(q, global_of, idx, swa, swa_scale, swa_pos0, swa_clip, seq_start,
                         q_start, q_pos, W, sm_scale)


def attend_mxfp8q(q, kv_codes, kv_e8m0, kv_rowscale, idx, swa, swa_scale, swa_pos0, swa_clip,
                  seq_start, q_start, q_pos, W, sm_scale):
    """`attend` with the query quantised to MXFP8 (reading R18), the numerics of attention on
    scaled matrix cores that read the FP4 rows and their E8M0 scales as stored (blog
    §Kernels: MegaAttention reads the NVFP4 KV natively): every (query, head) row of q is
    cut into 32-dim blocks, each with a shared E8M0 exponent and E4M3 elements
    (`codecs.mxfp8_quantize`), and the decoded values replace q in both branches' logits;
    the rows, the softmax and O are those of `attend`.  Returns (O, LSE) as `attend` does."""
    codes, E = codecs.mxfp8_quantize(codecs.bf16(q))
    qhat = codecs.mxfp8_decode(codes, E)
    c, e8 = np.asarray(kv_codes), np.asarray(kv_e8m0)
    rs = None if kv_rowscale is None else np.asarray(kv_rowscale)

    def global_of(rows):
        return codecs.global_rows(c[rows], e8[rows], None if rs is None else rs[rows])
    return _attend_union(q, global_of, idx, swa, swa_scale, swa_pos0, swa_clip, seq_start,
                         q_start, q_pos, W, sm_scale, q_values=qhat)


def rope_rotate(x, rope_cos, rope_sin, inverse=False):
    """Rotate the last 2 * R entries of x[t, h, :] in consecutive pairs (2i, 2i+1) by the
    angle of query t (cos / sin float32 [T, R]; reading R16): forward
    (a, b) -> (a c - b s, a s + b c), inverse by the opposite angle
    (a, b) -> (a c + b s, -a s + b c).  float64 result."""
    x = np.array(x, dtype=np.float64)
    c = np.asarray(rope_cos, dtype=np.float64)[:, None, :]
    s = np.asarray(rope_sin, dtype=np.float64)[:, None, :]
    R = c.shape[-1]
    if R == 0:
        return x
    D = x.shape[-1]
    a = x[..., D - 2 * R::2].copy()
    b = x[..., D - 2 * R + 1::2].copy()
    if inverse:
        s = -s
    x[..., D - 2 * R::2] = a * c - b * s
    x[..., D - 2 * R + 1::2] = a * s + b * c
    return x


def rope_query(q, rope_cos, rope_sin):
    """The rotated query as the attention's bf16 operand (reading R16): the pairs of the last
    2R dims rotated in float64 by `rope_rotate`, then rounded once to bf16 (nearest even).
    q uint16 bf16 bits [T, Hq, D] -> uint16 bits."""
    if np.asarray(rope_cos).shape[-1] == 0:
        return np.asarray(q).copy()
    return codecs.bf16_round(rope_rotate(codecs.bf16(q), rope_cos, rope_sin))


def fp8_quantize(x):
    """Per row (last axis): scale = amax / 448, the factor that maps the codes back, and
    codes = E4M3(x * 448 / amax), nearest even, saturating at 448 (reading R17), evaluated in
    float64; an all-zero row gives scale 0 and zero codes.  Returns (codes uint8, scale
    float64)."""
    x = np.asarray(x, dtype=np.float64)
    amax = np.abs(x).max(axis=-1)
    scale = amax / 448.0
    safe = np.where(amax > 0, amax, 1.0)
    codes = codecs.e4m3_encode(x * 448.0 / safe[..., None])
    codes = np.where((amax > 0)[..., None], codes, np.uint8(0)).astype(np.uint8)
    return codes, scale


def attend_fused(q, rope_cos, rope_sin, kv_codes, kv_e8m0, kv_rowscale, idx, swa, swa_scale,
                 swa_pos0, swa_clip, seq_start, q_start, q_pos, W, sm_scale):
    """MegaAttention's fused form (blog §Kernels, #56935): query RoPE, the sparse attention,
    inverse RoPE on the output and FP8 conversion of the result for the output projection.

    q is the unrotated bf16 query; its last 2R dims are rotated by query t's angles and the
    result is rounded to bf16 (`rope_query`, reading R16); O is then `attend`'s output,
    rotated back by the same angles, and quantised per (t, h) row by `fp8_quantize`
    (reading R17), everything in float64.
    Returns (O_rot float64 [T, Hq, D], LSE [T, Hq], codes uint8 [T, Hq, D], scale [T, Hq]).
    """
    qr = rope_query(q, rope_cos, rope_sin)
    O, LSE = attend(qr, kv_codes, kv_e8m0, kv_rowscale, idx, swa, swa_scale, swa_pos0, swa_clip,
                    seq_start, q_start, q_pos, W, sm_scale)
    Oi = rope_rotate(O, rope_cos, rope_sin, inverse=True)
    codes, scale = fp8_quantize(Oi)
    return Oi, LSE, codes, scale


def decode_step(wl_np: dict, k=None, cand=None):
    """score -> topk -> attend on one batch (dict of numpy arrays, keys as in synth.Workload)."""
    a = wl_np
    k = a["k"] if k is None else k
    S = score(a["qI"], a["w"], a["kI"], a.get("kscale"), a["seq_start"], a["q_start"],
              a["q_pos"], cand=cand)
    idx = topk(S, k, cand=cand)
    O, LSE = attend(a["q"], a["kv_codes"], a["kv_e8m0"], a.get("kv_rowscale"), idx, a["swa"],
                    a.get("swa_scale"), a["swa_pos0"], a.get("swa_clip"), a["seq_start"],
                    a["q_start"], a["q_pos"], a["W"], a["sm_scale"])
    return S, idx, O, LSE
