"""Shared test helpers: workload -> numpy views for the oracle, brute-force drivers, comparators."""
from __future__ import annotations

import math

import numpy as np
import torch

from oracle import brute


def np_inputs(wl) -> dict:
    """synth.Workload (any device) -> dict of numpy arrays in the oracle's argument names."""
    w = wl.cpu()
    a = {}
    for name in ("seq_start", "q_start", "q_pos", "qI", "w", "kI", "kscale", "kv_codes",
                 "kv_e8m0", "kv_rowscale", "swa", "swa_scale", "swa_pos0", "swa_clip", "cand",
                 "kv_fp8", "kv_fp8_scale", "kv_nv_codes", "kv_nv_scales"):
        v = getattr(w, name)
        a[name] = None if v is None else v.numpy()
    a["q"] = w.q.view(torch.int16).numpy().view(np.uint16)
    for name in ("k", "W", "sm_scale", "Hi", "Di", "Hq", "D", "T", "B", "max_ctx", "kv_nv_global"):
        a[name] = getattr(w, name)
    return a


def q_seq_of(a) -> list:
    qs = []
    for b in range(len(a["q_start"]) - 1):
        qs += [b] * int(a["q_start"][b + 1] - a["q_start"][b])
    return qs


def brute_scores(a, cand=None) -> list:
    """Per query: dict {column: score} from the scalar definition."""
    out = []
    qs = q_seq_of(a)
    for t in range(a["T"]):
        b = qs[t]
        base = int(a["seq_start"][b])
        n = int(a["seq_start"][b + 1]) - base
        p = int(a["q_pos"][t])
        cols = {}
        if cand is None:
            items = [(j, j) for j in range(0, min(p, n - 1) + 1)]
        else:
            items = [(i, int(c)) for i, c in enumerate(cand[t]) if 0 <= c <= p and c < n]
        for col, j in items:
            kap = None if a["kscale"] is None else a["kscale"][base + j]
            cols[col] = brute.score_one(a["qI"][t], a["w"][t], a["kI"][base + j], kap)
        out.append(cols)
    return out


def brute_attend(a, idx, fp8kv=False, nvfp4=False) -> tuple:
    """Scalar-loop attention; fp8kv takes the global rows from kv_fp8 / kv_fp8_scale, nvfp4
    from kv_nv_codes / kv_nv_scales / kv_nv_global (with the row scale kv_rowscale)."""
    qs = q_seq_of(a)
    T, Hq, D = a["q"].shape
    O = np.zeros((T, Hq, D))
    L = np.full((T, Hq), -np.inf)
    W = a["W"]
    for t in range(T):
        b = qs[t]
        base = int(a["seq_start"][b])
        rows = []
        for j in idx[t]:
            if j < 0:
                continue
            r = base + int(j)
            if fp8kv:
                rho = None if a["kv_fp8_scale"] is None else a["kv_fp8_scale"][r]
                rows.append(brute.window_row(a["kv_fp8"][r], rho))
                continue
            rho = None if a["kv_rowscale"] is None else a["kv_rowscale"][r]
            if nvfp4:
                rows.append(brute.nvfp4_row(a["kv_nv_codes"][r], a["kv_nv_scales"][r], rho,
                                            a["kv_nv_global"]))
                continue
            rows.append(brute.global_row(a["kv_codes"][r], a["kv_e8m0"][r], rho))
        p = int(a["q_pos"][t])
        lo = max(p - W + 1, 0)
        if a["swa_clip"] is not None:
            lo = max(lo, int(a["swa_clip"][t]))
        for u in range(W):
            pos = int(a["swa_pos0"][b]) + u
            if lo <= pos <= p:
                sig = None if a["swa_scale"] is None else a["swa_scale"][b][u]
                rows.append(brute.window_row(a["swa"][b][u], sig))
        for h in range(Hq):
            o, lse = brute.attend_one(a["q"][t][h], rows, a["sm_scale"])
            O[t, h] = o
            L[t, h] = lse
    return O, L


def topk_set_ok(S_ref, cand_pos, k, got, rel_gap=1e-5):
    """Check a GPU top-k result against oracle scores (set semantics, near-tie band).

    S_ref: float64 [L] oracle scores (-inf = not scored); cand_pos: positions of the
    columns (or None for dense); got: int array [k] (ascending, -1 padded).
    Returns (ok, message).  Outside a 1e-5-relative gap at the k-th score the set
    must equal the oracle's exactly; inside it, every strictly-better position must
    be present and every chosen one must lie within the band.
    """
    cols = np.nonzero(S_ref != -np.inf)[0]
    pos = cols if cand_pos is None else np.asarray(cand_pos)[cols]
    sc = S_ref[cols]
    nvalid = cols.size
    m = min(k, nvalid)
    got = np.asarray(got)
    if not np.all(got[m:] == -1):
        return False, "padding mismatch"
    g = got[:m]
    if np.any(g < 0) or len(set(g.tolist())) != m:
        return False, "invalid or duplicate positions"
    if not np.all(np.diff(g) > 0):
        return False, "not ascending"
    order = np.lexsort((pos, -sc))
    ref = np.sort(pos[order[:m]])
    if m == nvalid or np.array_equal(ref, g):
        return (np.array_equal(ref, g), "full set mismatch")
    sk = sc[order[m - 1]]
    sk1 = sc[order[m]]
    band = rel_gap * abs(sk)
    if sk - sk1 >= band and sk != sk1:
        return False, f"set mismatch with clear gap ({sk} vs {sk1})"
    score_of = dict(zip(pos.tolist(), sc.tolist()))
    must = set(pos[sc > sk + band].tolist())
    allowed = set(pos[sc >= sk - band].tolist())
    gs = set(g.tolist())
    if not must <= gs:
        return False, "missing a strictly better position"
    if not gs <= allowed:
        return False, "chose a position outside the near-tie band"
    # exact ties are decided by position: among equal scores the lower position wins
    for p_ in gs:
        s_ = score_of[p_]
        better_lower = [q for q in pos[(sc == s_)].tolist() if q < p_ and q not in gs]
        if better_lower:
            return False, "tie-break by position violated"
    return True, "near-tie band"


def close_attention(O_gpu, O_ref, lse_gpu=None, lse_ref=None, atol=2e-3, rtol=1e-3, lse_tol=1e-4,
                    lse_rtol=1e-6):
    """Per (t, h): max|dO| <= atol and max|dO| <= rtol * max|O_ref|;
    |dLSE| <= lse_tol + lse_rtol * |LSE_ref| (fp32 logits carry ~2^-24 relative error, which
    dominates the absolute bar only once |LSE| reaches ~1e3)."""
    d = np.abs(np.asarray(O_gpu, dtype=np.float64) - O_ref).max(axis=-1)
    scale = np.abs(O_ref).max(axis=-1)
    ok = (d <= atol) & (d <= rtol * scale + 1e-30)
    msg = f"max|dO|={d.max():.3e}, worst ratio={(d / np.maximum(scale, 1e-30)).max():.3e}"
    if lse_gpu is not None:
        dl = np.abs(np.asarray(lse_gpu, dtype=np.float64) - lse_ref)
        both_inf = np.isinf(lse_ref) & (np.asarray(lse_gpu) == lse_ref)
        dl = np.where(both_inf, 0.0, dl)
        ok &= dl <= lse_tol + lse_rtol * np.where(np.isinf(lse_ref), 0.0, np.abs(lse_ref))
        msg += f", max|dLSE|={dl.max():.3e}"
    return bool(ok.all()), msg


def close_scores(S_gpu, S_ref, rtol=1e-4, floor=1e-7):
    """|S_gpu - S_ref| <= rtol*|S_ref| + floor*max|S_ref| on scored entries; -inf must match."""
    S_gpu = np.asarray(S_gpu, dtype=np.float64)
    inf = S_ref == -np.inf
    if not np.array_equal(S_gpu[inf], S_ref[inf]):
        return False, "masked entries differ"
    fin = ~inf
    if not fin.any():
        return True, "empty"
    tol = rtol * np.abs(S_ref[fin]) + floor * np.abs(S_ref[fin]).max()
    err = np.abs(S_gpu[fin] - S_ref[fin])
    return bool((err <= tol).all()), f"max err {err.max():.3e}, worst ratio {(err / tol).max():.3f}"


def _e4m3_half_step(y):
    """Half the spacing of the E4M3 grid at magnitude |y| <= 448: 2^(E-4) in the binade
    [2^E, 2^(E+1)) (3 mantissa bits), 2^-10 on the subnormal grid below 2^-6."""
    _, e = np.frexp(np.maximum(np.abs(y), 2.0 ** -6))       # |y| in [2^(e-1), 2^e)
    return np.ldexp(1.0, e.astype(np.int64) - 5)


def fp8_output_ok(codes_gpu, scale_gpu, O_ref, err):
    """The fused attention's FP8 output against the oracle's own float64 O' (reading R17:
    scale = amax / 448, codes = E4M3(x * 448 / amax), nearest even).

    err[t, h] bounds max_d |x_gpu - x_ref| of the output the GPU quantised (the attention
    tolerance, or the error measured on its fp32 output).  Then |amax_gpu - amax_ref| <= err
    too, and the GPU's pre-rounding value y_gpu = x_gpu * 448 / amax_gpu (plus its fp32
    rounding, < 2^-21 relative) lies within
        delta = 448 * err * (amax + |x|) / (amax * (amax - err)) + 2^-21 |y|
    of the oracle's y = x_ref * 448 / amax_ref.  So every code must lie between
    E4M3(y - delta) and E4M3(y + delta): equal to the oracle's code except where y sits within
    delta of a rounding midpoint, where the neighbouring code is allowed as well.  Also
    |scale_gpu - scale_ref| <= err / 448 (+ one fp32 rounding) and the dequantised output
    codes * scale stays within half an E4M3 step (plus delta) of O' and err.
    Returns (ok, message)."""
    from oracle import codecs
    O_ref = np.asarray(O_ref, dtype=np.float64)
    c = np.asarray(codes_gpu, dtype=np.uint8)
    sg = np.asarray(scale_gpu, dtype=np.float64)
    err = np.broadcast_to(np.asarray(err, dtype=np.float64), O_ref.shape[:-1])
    amax = np.abs(O_ref).max(axis=-1)
    scale_ref = amax / 448.0
    ds = np.abs(sg - scale_ref)
    ok_s = ds <= err / 448.0 + 2.0 ** -23 * scale_ref
    live = amax > err                                 # rows whose amax the bound pins
    safe = np.where(live, amax, 1.0)[..., None]
    e3 = err[..., None]
    y = O_ref * 448.0 / safe
    delta = 448.0 * e3 * (safe + np.abs(O_ref)) / (safe * (safe - np.where(live[..., None], e3, 0.0)))
    delta = delta + 2.0 ** -21 * np.abs(y)
    lo = codecs.e4m3(codecs.e4m3_encode(y - delta))
    hi = codecs.e4m3(codecs.e4m3_encode(y + delta))
    v = codecs.e4m3(c)
    ok_c = np.where(live[..., None], (v >= lo) & (v <= hi), True)
    # a row the bound cannot pin (amax <= err): its codes only have to dequantise near O'
    deq = v * sg[..., None]
    bound = (_e4m3_half_step(np.abs(y) + delta) + delta) * scale_ref[..., None] * (1 + 2.0 ** -20) + e3
    ok_d = np.abs(deq - O_ref) <= bound + 1e-30
    ok = bool(ok_s.all() and ok_c.all() and ok_d.all())
    exact = codecs.e4m3_encode(y)
    n_amb = int((live[..., None] & (lo != hi)).sum())
    n_diff = int((live[..., None] & (codecs.e4m3(exact) != v)).sum())
    msg = (f"scale max|d|={ds.max():.3e}, codes outside band={int((~ok_c).sum())}, "
           f"dequant outside bound={int((~ok_d).sum())}, codes != oracle's={n_diff} "
           f"(ambiguous {n_amb} of {v.size})")
    return ok, msg


def fp8_output_checks(codes_gpu, scale_gpu, O_ref, out_gpu=None, atol=2e-3, rtol=1e-3):
    """fp8_output_ok with err = the attention tolerance (the contract), then, when the GPU's
    fp32 output is available, with err = its measured error (tight), and the oracle's
    quantiser applied to that fp32 output with err = 0 (only the kernel's fp32 rounding)."""
    O_ref = np.asarray(O_ref, dtype=np.float64)
    amax = np.abs(O_ref).max(axis=-1)
    ok, msg = fp8_output_ok(codes_gpu, scale_gpu, O_ref, np.minimum(atol, rtol * amax))
    assert ok, f"against O' with the tolerance band: {msg}"
    if out_gpu is None:
        return msg
    x = np.asarray(out_gpu, dtype=np.float64)
    meas = np.abs(x - O_ref).max(axis=-1) * (1 + 1e-6) + 1e-12 * amax
    ok, msg2 = fp8_output_ok(codes_gpu, scale_gpu, O_ref, meas)
    assert ok, f"against O' with the measured-error band: {msg2}"
    ok, msg3 = fp8_output_ok(codes_gpu, scale_gpu, x, np.zeros_like(amax))
    assert ok, f"against the quantiser on the GPU's own fp32 output: {msg3}"
    return msg2


def fsum(xs):
    return math.fsum(xs)


# ------------------------------------------------------------------ GPU call wrappers

def announce(msg: str):
    """Name the case on stdout before GPU work (flushed, so a fault still shows it)."""
    print(f"[gpu-case] {msg}", flush=True)


def gpu_batch(smqa, wl):
    return smqa.Batch(wl.seq_start, wl.q_start, wl.q_pos, wl.max_ctx)


def gpu_score(smqa, wl):
    return smqa.sparse_mqa_score(gpu_batch(smqa, wl), wl.qI, wl.w, wl.kI, wl.kscale, wl.cand)


def gpu_topk(smqa, wl, scores, k=None):
    return smqa.topk_select(gpu_batch(smqa, wl), scores, wl.k if k is None else k, cand=wl.cand)


def gpu_attend(smqa, wl, idx):
    return smqa.sparse_mqa_attend(gpu_batch(smqa, wl), wl.q, wl.kv_codes, wl.kv_e8m0,
                                  wl.kv_rowscale, idx, wl.swa, wl.swa_scale, wl.swa_pos0,
                                  wl.swa_clip, wl.sm_scale)


def gpu_attend_fp8kv(smqa, wl, idx):
    return smqa.sparse_mqa_attend_fp8kv(gpu_batch(smqa, wl), wl.q, wl.kv_fp8, wl.kv_fp8_scale, idx,
                                        wl.swa, wl.swa_scale, wl.swa_pos0, wl.swa_clip, wl.sm_scale)


def gpu_attend_nvfp4(smqa, wl, idx):
    return smqa.sparse_mqa_attend_nvfp4(gpu_batch(smqa, wl), wl.q, wl.kv_nv_codes, wl.kv_nv_scales,
                                        wl.kv_rowscale, wl.kv_nv_global, idx, wl.swa, wl.swa_scale,
                                        wl.swa_pos0, wl.swa_clip, wl.sm_scale)


def gpu_attend_fused(smqa, wl, idx, rope_cos, rope_sin, want_out=True):
    return smqa.sparse_mqa_attend_fused(gpu_batch(smqa, wl), wl.q, rope_cos, rope_sin, wl.kv_codes,
                                        wl.kv_e8m0, wl.kv_rowscale, idx, wl.swa, wl.swa_scale,
                                        wl.swa_pos0, wl.swa_clip, wl.sm_scale, want_out=want_out)


def gpu_decode(smqa, wl, k=None):
    return smqa.decode_step(gpu_batch(smqa, wl), wl.qI, wl.w, wl.kI, wl.kscale, wl.cand, wl.q,
                            wl.kv_codes, wl.kv_e8m0, wl.kv_rowscale, wl.swa, wl.swa_scale,
                            wl.swa_pos0, wl.swa_clip, wl.k if k is None else k, wl.sm_scale)


def oracle_scores_for(a, ts, cand=None):
    """Oracle scores of the queries ts only (same columns as the full call)."""
    ld = a["max_ctx"]
    return np.stack([_score_one_query(a, t, cand, ld) for t in ts])


def _score_one_query(a, t, cand, ld):
    from oracle import ref
    b = q_seq_of(a)[t]
    base = int(a["seq_start"][b])
    n = int(a["seq_start"][b + 1]) - base
    seq = np.array([0, n], dtype=np.int64)
    kI = a["kI"][base:base + n]
    ks = None if a["kscale"] is None else a["kscale"][base:base + n]
    return ref.score(a["qI"][t:t + 1], a["w"][t:t + 1], kI, ks, seq, np.array([0, 1]),
                     a["q_pos"][t:t + 1], cand=None if cand is None else cand[t:t + 1], ld=ld)[0]


def oracle_attend_for(a, ts, idx_rows):
    """Oracle attention of queries ts with the given selections (rows of idx)."""
    from oracle import ref
    qs = q_seq_of(a)
    O, L = [], []
    for i, t in enumerate(ts):
        b = qs[t]
        base = int(a["seq_start"][b])
        n = int(a["seq_start"][b + 1]) - base
        o, l = ref.attend(a["q"][t:t + 1], a["kv_codes"][base:base + n], a["kv_e8m0"][base:base + n],
                          None if a["kv_rowscale"] is None else a["kv_rowscale"][base:base + n],
                          np.asarray(idx_rows[i])[None], a["swa"][b:b + 1],
                          None if a["swa_scale"] is None else a["swa_scale"][b:b + 1],
                          a["swa_pos0"][b:b + 1],
                          None if a["swa_clip"] is None else a["swa_clip"][t:t + 1],
                          np.array([0, n]), np.array([0, 1]), a["q_pos"][t:t + 1], a["W"],
                          a["sm_scale"])
        O.append(o[0])
        L.append(l[0])
    return np.stack(O), np.stack(L)
