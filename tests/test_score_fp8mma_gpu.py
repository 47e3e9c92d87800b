"""FP8 matrix-core scoring (sparse_mqa_score_fp8mma) against the fp64 oracle.

The products of two E4M3 values are exact; the instruction adds a logit's 128 products with
an error of up to ~2^-15 of their absolute sum (measured on gfx950: 3.1e-5 at most over the
decode_8k and decode_512k inputs, 8e-7 at the median).  Every score is checked against the
bound that error implies, which holds for any inputs (head weights of either sign, logits
that nearly cancel):

    |S_gpu - S| <= kappa * sum_h |w_h| * (2^-14 * A_h + 1e-5 * |L_h|) + 1e-7 * max|S|

with L_h the exact logit, A_h = sum_d |q_hd * k_d| (2^-14: twice the largest measured
ratio) and 1e-5 |L_h| for the fp32 head sum; -inf columns must match exactly.  On the
benchmark's inputs (head weights U(0,1), so the ReLU'd terms never cancel) the scores also
meet the reference form's 1e-4 relative bar and give the oracle's top-k set.
"""
import numpy as np
import pytest
import torch

import synth
from helpers import announce, close_scores, gpu_batch, gpu_topk, np_inputs, q_seq_of, topk_set_ok
from oracle import codecs, ref

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _fp8_scores(lib, wl):
    return lib.sparse_mqa_score_fp8mma(gpu_batch(lib, wl), wl.qI, wl.w, wl.kI, wl.kscale, wl.cand)


def _bound_ok(a, t, S_gpu, S_ref):
    """The per-score bound above for query t's row (dense or candidate columns)."""
    b = q_seq_of(a)[t]
    base = int(a["seq_start"][b])
    n = int(a["seq_start"][b + 1]) - base
    p = int(a["q_pos"][t])
    if a["cand"] is not None:
        pos = a["cand"][t].astype(np.int64)
        cols = np.nonzero((pos >= 0) & (pos <= p) & (pos < n))[0]
        pos = pos[cols]
    else:
        cols = np.arange(min(p, n - 1) + 1)
        pos = cols
    fin = S_ref != -np.inf
    if not np.array_equal(np.asarray(S_gpu) == -np.inf, ~fin):
        return False, "-inf columns differ"
    Q = codecs.e4m3(a["qI"][t]).astype(np.float64)                  # [Hi][Di]
    K = codecs.e4m3(a["kI"][base + pos]).astype(np.float64)         # [m][Di]
    L = Q @ K.T
    A = np.abs(Q) @ np.abs(K).T
    wabs = np.abs(a["w"][t].astype(np.float64))
    kap = np.ones(pos.size) if a["kscale"] is None else a["kscale"][base + pos].astype(np.float64)
    smax = np.abs(S_ref[fin]).max() if fin.any() else 0.0
    bound = kap * (2.0 ** -14 * (wabs @ A) + 1e-5 * (wabs @ np.abs(L))) + 1e-7 * smax
    err = np.abs(np.asarray(S_gpu, dtype=np.float64)[cols] - S_ref[cols])
    worst = (err / np.maximum(bound, 1e-300)).max() if cols.size else 0.0
    return bool(np.all(err <= bound)), f"worst error / bound = {worst:.3f}"


@pytest.mark.parametrize("name,kw,n_cand", [
    ("decode_8k", {}, None),                                              # short rows
    ("decode_8k", dict(B=1, lengths=300000), None),                       # one query, long row
    ("replay_h100k", dict(B=2, lengths=140000, replay=(140000, 8)), None),  # many queries, kappa
    ("decode_8k", dict(B=2, lengths=(20000, 40000)), 16384),             # candidate lists
    ("decode_8k", dict(B=16, lengths=(20000, 40000)), 16384),            # long candidate grid
])
def test_score_fp8mma_within_the_instruction_bound(lib, name, kw, n_cand):
    wl = synth.generate(name, seed=0, device=DEV, n_cand=n_cand, **kw)
    if name == "replay_h100k":
        wl = synth.with_scales(wl)
    if n_cand is not None:
        wl.q_pos[0] -= 777                   # some candidates lie past the query
    announce(f"score fp8mma {name} {kw} n_cand={n_cand} T={wl.T}")
    S = _fp8_scores(lib, wl)
    torch.cuda.synchronize()
    a = np_inputs(wl)
    S_ref = ref.score(a["qI"], a["w"], a["kI"], a["kscale"], a["seq_start"], a["q_start"], a["q_pos"],
                      cand=a["cand"], ld=S.shape[1])
    S_gpu = S.cpu().numpy()
    for t in range(wl.T):
        ok, msg = _bound_ok(a, t, S_gpu[t], S_ref[t])
        assert ok, f"query {t}: {msg}"
        # benchmark inputs (non-negative head weights): the reference form's bar holds too
        ok, msg = close_scores(S_gpu[t], S_ref[t])
        assert ok, f"query {t} (1e-4 bar): {msg}"


def test_score_fp8mma_topk_matches_the_oracle(lib):
    """decode_8k: the top-2048 of the FP8-form scores is the oracle's set."""
    wl = synth.generate("decode_8k", seed=0, device=DEV)
    announce("score fp8mma decode_8k top-k")
    S = _fp8_scores(lib, wl)
    idx = gpu_topk(lib, wl, S)
    idx = idx[0] if isinstance(idx, tuple) else idx
    torch.cuda.synchronize()
    a = np_inputs(wl)
    S_ref = ref.score(a["qI"], a["w"], a["kI"], a["kscale"], a["seq_start"], a["q_start"], a["q_pos"])
    ok, msg = topk_set_ok(S_ref[0], None, wl.k, idx.cpu().numpy()[0])
    assert ok, msg


def test_score_fp8mma_mixed_sign_weights_stay_within_the_bound(lib):
    """Head weights of both signs let the head sum cancel, where a relative bar can fail; the
    instruction bound still holds for every score."""
    wl = synth.generate("decode_8k", seed=5, device=DEV, lengths=6000)
    g = torch.Generator(device=DEV)
    g.manual_seed(123)
    wl.w.copy_(torch.randn(wl.w.shape, generator=g, device=DEV, dtype=torch.float32))
    announce("score fp8mma decode_8k mixed-sign weights")
    S = _fp8_scores(lib, wl)
    torch.cuda.synchronize()
    a = np_inputs(wl)
    S_ref = ref.score(a["qI"], a["w"], a["kI"], a["kscale"], a["seq_start"], a["q_start"], a["q_pos"],
                      ld=S.shape[1])
    ok, msg = _bound_ok(a, 0, S.cpu().numpy()[0], S_ref[0])
    assert ok, msg


@pytest.mark.parametrize("form", [0, 1], ids=["scale_16x16x128_f8f6f4", "16x16x32_fp8_fp8"])
def test_fp8_instruction_summation_error(lib, form):
    """The measurement behind the bound above: decode_8k's 64 x 8192 indexer logits from the
    benchmark library's FP8-instruction kernel against exact fp64 dot products.  Products of
    E4M3 values are exact, so any difference is the instruction's summation; it is nonzero
    (the sum is not exact in fp32) and below 2^-14 of the absolute sum of the products."""
    import ctypes
    import os
    path = os.path.join(os.path.dirname(lib.__file__), "libsmqa_bench.so")
    blib = ctypes.CDLL(path)
    fn = blib.smqa_bench_fp8_mfma_logits
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                   ctypes.c_int32, ctypes.c_void_p]
    wl = synth.generate("decode_8k", seed=0, device=DEV)
    announce(f"fp8 instruction error form {form}")
    qI = wl.qI[0].contiguous()
    kI = wl.kI.contiguous()
    H, N = qI.shape[0], kI.shape[0]
    assert qI.shape[1] == 128 and H % 16 == 0 and N % 16 == 0
    out = torch.empty((H, N), dtype=torch.float32, device=DEV)
    assert fn(qI.data_ptr(), kI.data_ptr(), H, N, out.data_ptr(), form, None) == 0
    torch.cuda.synchronize()
    Q = codecs.e4m3(qI.cpu().numpy()).astype(np.float64)
    K = codecs.e4m3(kI.cpu().numpy()).astype(np.float64)
    L = Q @ K.T
    A = np.abs(Q) @ np.abs(K).T
    nz = A > 0
    ratio = np.abs(out.cpu().numpy().astype(np.float64) - L)[nz] / A[nz]
    assert ratio.max() > 0.0
    assert ratio.max() <= 2.0 ** -14, f"max error / sum|qk| = {ratio.max():.3e}"
