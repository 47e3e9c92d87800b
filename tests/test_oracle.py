"""Pins for the fp64 oracle (CPU only).

Each test checks the oracle against something other than itself: the scalar
loop versions (oracle.brute, own decoders, exact summation), exact integer
arithmetic, hand-worked fixtures (tests/golden), torch's scaled-dot-product
attention in float64, and invariants of the definitions (permutations,
linearity, window clipping).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import synth
from oracle import brute, codecs, ref
from helpers import brute_attend, brute_scores, np_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

TINY = dict(Hi=3, Di=8, k=6, Hq=2, D=64, W=8, rowscale=True)


def tiny(seed=0, **kw):
    p = dict(TINY)
    p.update(kw)
    return synth.generate("tiny", seed=seed, **p)


# ----------------------------------------------------------------- score

def test_score_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "hand_score_topk.json")))
    qI = np.array([g["qI"]], dtype=np.uint8)
    w = np.array([g["w"]], dtype=np.float32)
    kI = np.array(g["kI"], dtype=np.uint8)
    seq = np.array([0, 4]); qst = np.array([0, 1]); qpos = np.array([3])
    S = ref.score(qI, w, kI, None, seq, qst, qpos)
    assert S[0].tolist() == g["S"]
    S2 = ref.score(qI, w, kI, np.array(g["kappa"], dtype=np.float32), seq, qst, qpos)
    assert S2[0].tolist() == g["S_kappa"]
    assert ref.topk(S, 2)[0].tolist() == g["top2"]
    assert ref.topk(S, 3)[0].tolist() == g["top3"]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_score_matches_brute(seed):
    wl = synth.with_scales(tiny(seed, B=2, lengths=(20, 37)), seed=seed)
    a = np_inputs(wl)
    S = ref.score(a["qI"], a["w"], a["kI"], a["kscale"], a["seq_start"], a["q_start"], a["q_pos"])
    bs = brute_scores(a)
    for t in range(a["T"]):
        scored = np.nonzero(S[t] != -np.inf)[0]
        assert sorted(bs[t]) == scored.tolist()
        for c, v in bs[t].items():
            assert abs(S[t, c] - v) <= 1e-12 * max(1.0, abs(v))


def test_score_candidates_match_brute():
    wl = tiny(4, B=2, lengths=(20, 60), n_cand=40)
    a = np_inputs(wl)
    S = ref.score(a["qI"], a["w"], a["kI"], None, a["seq_start"], a["q_start"], a["q_pos"],
                  cand=a["cand"])
    bs = brute_scores(a, cand=a["cand"])
    for t in range(a["T"]):
        for c in range(S.shape[1]):
            if c in bs[t]:
                assert abs(S[t, c] - bs[t][c]) <= 1e-12 * max(1.0, abs(bs[t][c]))
            else:
                assert S[t, c] == -np.inf
    # the shorter sequence's padding entries (past the query) are masked
    assert np.isinf(S).any()


def test_score_integer_inputs_exact():
    # integer-valued E4M3 inputs and power-of-two weights: exact integer arithmetic
    rng = np.random.default_rng(0)
    ints = np.arange(-4, 5)
    codes = synth.encode_e4m3(torch.tensor(ints, dtype=torch.float32)).numpy()
    lut = dict(zip(codes.tolist(), ints.tolist()))
    Hi, Di, n = 4, 16, 50
    qI = rng.choice(codes, size=(1, Hi, Di)).astype(np.uint8)
    kI = rng.choice(codes, size=(n, Di)).astype(np.uint8)
    w = np.array([[0.5, 2.0, 0.25, 1.0]], dtype=np.float32)
    S = ref.score(qI, w, kI, None, np.array([0, n]), np.array([0, 1]), np.array([n - 1]))
    for j in range(n):
        tot = 0
        for h in range(Hi):
            dot = sum(lut[int(qI[0, h, d])] * lut[int(kI[j, d])] for d in range(Di))
            tot += float(w[0, h]) * max(0, dot)
        assert S[0, j] == tot


def test_score_one_hot_weight_and_negative_dots():
    wl = tiny(5)
    a = np_inputs(wl)
    Hi = a["Hi"]
    for h in range(Hi):
        w = np.zeros_like(a["w"]); w[0, h] = 1.0
        S = ref.score(a["qI"], w, a["kI"], None, a["seq_start"], a["q_start"], a["q_pos"])
        Q = codecs.e4m3(a["qI"][0, h]); K = codecs.e4m3(a["kI"])
        n = int(a["q_pos"][0]) + 1
        assert np.array_equal(S[0, :n], np.maximum(K[:n] @ Q, 0.0))
    # keys pointing against every head's query give exactly zero
    qI = np.tile(synth.encode_e4m3(torch.ones(1, 1, 8)).numpy(), (1, 3, 1))
    kI = synth.encode_e4m3(-torch.rand(10, 8) - 0.1).numpy()
    S = ref.score(qI, np.ones((1, 3), np.float32), kI, None, np.array([0, 10]), np.array([0, 1]),
                  np.array([9]))
    assert np.all(S[0] == 0.0)


def test_score_head_permutation_and_kappa_linearity():
    wl = tiny(6, Hi=5)
    a = np_inputs(wl)
    args = (a["seq_start"], a["q_start"], a["q_pos"])
    S = ref.score(a["qI"], a["w"], a["kI"], None, *args)
    perm = np.array([3, 0, 4, 1, 2])
    Sp = ref.score(a["qI"][:, perm], a["w"][:, perm], a["kI"], None, *args)
    assert np.allclose(S, Sp, rtol=1e-13, atol=0)
    kap = np.full(a["kI"].shape[0], 2.5, dtype=np.float32)
    Sk = ref.score(a["qI"], a["w"], a["kI"], kap, *args)
    assert np.allclose(Sk, 2.5 * S, rtol=1e-13, atol=0)


# ----------------------------------------------------------------- top-k

@pytest.mark.parametrize("seed", [0, 1])
def test_topk_matches_brute(seed):
    rng = np.random.default_rng(seed)
    S = rng.standard_normal((3, 40))
    S[1, 30:] = -np.inf
    S[2, ::3] = S[2, 1]                 # exact ties
    for k in (1, 5, 13, 40, 45):
        got = ref.topk(S, k)
        for t in range(3):
            sc = {j: S[t, j] for j in range(40) if S[t, j] != -np.inf}
            exp = brute.topk_positions(sc, k)
            assert got[t, :len(exp)].tolist() == exp
            assert np.all(got[t, len(exp):] == -1)


def test_topk_constant_scores_take_lowest_positions():
    S = np.zeros((1, 100))
    assert ref.topk(S, 7)[0].tolist() == list(range(7))


def test_topk_candidates_return_positions():
    S = np.array([[0.1, 0.9, 0.5, -np.inf]])
    cand = np.array([[10, 3, 7, 99]])
    assert ref.topk(S, 2, cand=cand)[0].tolist() == [3, 7]
    assert ref.topk(S, 5, cand=cand)[0].tolist() == [3, 7, 10, -1, -1]


def test_topk_agrees_with_argpartition_away_from_ties():
    rng = np.random.default_rng(7)
    S = rng.standard_normal((4, 5000))
    got = ref.topk(S, 100)
    for t in range(4):
        part = np.sort(np.argpartition(-S[t], 100)[:100])
        assert np.array_equal(got[t], part)


# ----------------------------------------------------------------- attend

def _attend(a, idx, **over):
    b = dict(a)
    b.update(over)
    return ref.attend(b["q"], b["kv_codes"], b["kv_e8m0"], b["kv_rowscale"], idx, b["swa"],
                      b["swa_scale"], b["swa_pos0"], b["swa_clip"], b["seq_start"], b["q_start"],
                      b["q_pos"], b["W"], b["sm_scale"])


@pytest.mark.parametrize("seed,clip", [(0, False), (1, True)])
def test_attend_matches_brute(seed, clip):
    wl = synth.with_scales(tiny(seed, B=2, lengths=(20, 37)), seed=seed)
    a = np_inputs(wl)
    if clip:
        a["swa_clip"] = (a["q_pos"] - 3).astype(np.int32)
    S = ref.score(a["qI"], a["w"], a["kI"], a["kscale"], a["seq_start"], a["q_start"], a["q_pos"])
    idx = ref.topk(S, a["k"])
    O, L = _attend(a, idx)
    Ob, Lb = brute_attend(a, idx)
    assert np.allclose(O, Ob, rtol=1e-12, atol=1e-14)
    assert np.allclose(L, Lb, rtol=1e-12, atol=1e-14)


def test_attend_select_all_equals_dense_sdpa():
    """k >= n: the sparse attention is dense attention over every row plus the window."""
    wl = tiny(8, lengths=33, k=64, W=8)
    a = np_inputs(wl)
    n = 33
    idx = np.arange(64)[None, :].copy(); idx[0, n:] = -1
    O, L = _attend(a, idx)
    rows = codecs.global_rows(a["kv_codes"][:n], a["kv_e8m0"][:n], a["kv_rowscale"][:n])
    win = codecs.window_rows(a["swa"][0][a["W"] - 8:], None)      # window = last 8 positions
    R = torch.tensor(np.concatenate([rows, win]), dtype=torch.float64)
    q = torch.tensor(codecs.bf16(a["q"]), dtype=torch.float64)          # [1, Hq, D]
    Hq = q.shape[1]
    kv = R[None, None].expand(1, Hq, -1, -1)
    o = torch.nn.functional.scaled_dot_product_attention(q[:, :, None, :], kv, kv,
                                                         scale=a["sm_scale"])[:, :, 0]
    lse = torch.logsumexp(a["sm_scale"] * (q[0] @ R.T), dim=-1)
    assert np.allclose(O, o.numpy(), rtol=1e-12, atol=1e-14)
    assert np.allclose(L[0], lse.numpy(), rtol=1e-12, atol=1e-14)


def test_attend_single_row_and_identical_rows():
    wl = tiny(9, lengths=40, W=8)
    a = np_inputs(wl)
    # one global row, window clipped to nothing: O = row, LSE = tau <q,row>
    idx = np.full((1, 6), -1); idx[0, 0] = 17
    clip = np.array([10_000], dtype=np.int32)
    O, L = _attend(a, idx, swa_clip=clip)
    row = codecs.global_rows(a["kv_codes"][17:18], a["kv_e8m0"][17:18], a["kv_rowscale"][17:18])[0]
    q = codecs.bf16(a["q"][0])
    assert np.allclose(O[0], np.broadcast_to(row, O[0].shape), rtol=1e-14, atol=0)
    assert np.allclose(L[0], a["sm_scale"] * (q @ row), rtol=1e-13, atol=1e-15)
    # all rows decode to the same vector -> O is that vector for any logits
    b = dict(a)
    b["kv_codes"] = np.tile(a["kv_codes"][17:18], (a["kv_codes"].shape[0], 1))
    b["kv_e8m0"] = np.tile(a["kv_e8m0"][17:18], (a["kv_e8m0"].shape[0], 1))
    b["kv_rowscale"] = np.full_like(a["kv_rowscale"], a["kv_rowscale"][17])
    idx = np.arange(6)[None] * 3
    O, _ = _attend(b, idx, swa_clip=clip)
    assert np.allclose(O[0], np.broadcast_to(row, O[0].shape), rtol=1e-13, atol=1e-15)


def test_attend_weights_sum_to_one():
    # every row decodes to all-ones (E2M1 0x22 = [1, 1], E8M0 127; E4M3 0x38 = 1) -> O == 1
    wl = tiny(10, lengths=40, W=8)
    a = np_inputs(wl)
    a["kv_codes"][:] = 0x22
    a["kv_e8m0"][:] = 127
    a["kv_rowscale"][:] = 1.0
    a["swa"][:] = 0x38
    idx = np.arange(6)[None] * 5
    O, _ = _attend(a, idx)
    assert np.allclose(O, 1.0, rtol=0, atol=1e-13)


def test_attend_permutation_invariance_and_lse_merge():
    wl = tiny(11, lengths=60, k=12, W=8)
    a = np_inputs(wl)
    S = ref.score(a["qI"], a["w"], a["kI"], None, a["seq_start"], a["q_start"], a["q_pos"])
    idx = ref.topk(S, 12)
    O, L = _attend(a, idx)
    perm = idx[:, np.random.default_rng(0).permutation(12)]
    Op, Lp = _attend(a, perm)
    assert np.allclose(O, Op, rtol=1e-12, atol=1e-14) and np.allclose(L, Lp, rtol=1e-13)
    # split the selected rows in two disjoint halves (no window on either side) and merge by LSE
    none = np.array([10_000], dtype=np.int32)
    h1 = idx.copy(); h1[:, 6:] = -1
    h2 = idx.copy(); h2[:, :6] = -1
    O1, L1 = _attend(a, h1, swa_clip=none)
    O2, L2 = _attend(a, h2, swa_clip=none)
    Oa, La = _attend(a, idx, swa_clip=none)
    M = np.maximum(L1, L2)
    e1, e2 = np.exp(L1 - M), np.exp(L2 - M)
    Om = (e1[..., None] * O1 + e2[..., None] * O2) / (e1 + e2)[..., None]
    assert np.allclose(Om, Oa, rtol=1e-12, atol=1e-14)
    assert np.allclose(M + np.log(e1 + e2), La, rtol=1e-13)


def test_attend_empty_set():
    wl = tiny(12, lengths=40, W=8)
    a = np_inputs(wl)
    O, L = _attend(a, np.full((1, 6), -1), swa_clip=np.array([10_000], dtype=np.int32))
    assert np.all(O == 0) and np.all(L == -np.inf)


# ----------------------------------------------------------------- attend over an FP8 cache

def _attend8(a, idx, **over):
    b = dict(a)
    b.update(over)
    return ref.attend_fp8kv(b["q"], b["kv_fp8"], b["kv_fp8_scale"], idx, b["swa"], b["swa_scale"],
                            b["swa_pos0"], b["swa_clip"], b["seq_start"], b["q_start"], b["q_pos"],
                            b["W"], b["sm_scale"])


@pytest.mark.parametrize("seed,clip", [(0, False), (1, True)])
def test_attend_fp8kv_matches_brute(seed, clip):
    wl = synth.with_fp8_kv(synth.with_scales(tiny(seed, B=2, lengths=(20, 37)), seed=seed), seed=seed)
    a = np_inputs(wl)
    if clip:
        a["swa_clip"] = (a["q_pos"] - 3).astype(np.int32)
    rng = np.random.default_rng(seed)
    idx = np.full((a["T"], a["k"]), -1, dtype=np.int64)
    for t, b in enumerate([0, 1]):
        n = int(a["seq_start"][b + 1] - a["seq_start"][b])
        m = min(a["k"] - 1, n)
        idx[t, :m] = np.sort(rng.choice(min(n, int(a["q_pos"][t]) + 1), size=m, replace=False))
    O, L = _attend8(a, idx)
    Ob, Lb = brute_attend(a, idx, fp8kv=True)
    assert np.allclose(O, Ob, rtol=1e-12, atol=1e-14)
    assert np.allclose(L, Lb, rtol=1e-12, atol=1e-14)
    a = np_inputs(synth.with_fp8_kv(wl, seed=seed, rowscale=False))     # rho = 1
    if clip:
        a["swa_clip"] = (a["q_pos"] - 3).astype(np.int32)
    assert a["kv_fp8_scale"] is None
    O, L = _attend8(a, idx)
    Ob, Lb = brute_attend(a, idx, fp8kv=True)
    assert np.allclose(O, Ob, rtol=1e-12, atol=1e-14)


def test_attend_fp8kv_of_an_exact_reencoding_equals_fp4():
    """Every FP4 row value e2m1 * 2^(E-127) here is an E4M3 value: the FP8 cache holding the
    same values (row scale rho unchanged) must give the FP4 cache's attention exactly."""
    wl = synth.with_scales(tiny(3, B=2, lengths=(30, 45)), seed=3)
    a = np_inputs(wl)
    vals = codecs.global_rows(a["kv_codes"], a["kv_e8m0"], None)
    e4 = synth.encode_e4m3(torch.tensor(vals, dtype=torch.float32)).numpy()
    assert np.array_equal(codecs.e4m3(e4), vals)     # the re-encoding is exact
    S = ref.score(a["qI"], a["w"], a["kI"], a["kscale"], a["seq_start"], a["q_start"], a["q_pos"])
    idx = ref.topk(S, a["k"])
    O4, L4 = _attend(a, idx)
    O8, L8 = _attend8(a, idx, kv_fp8=e4, kv_fp8_scale=a["kv_rowscale"])
    assert np.array_equal(O4, O8) and np.array_equal(L4, L8)


def _attend_nv(a, idx, **over):
    b = dict(a)
    b.update(over)
    return ref.attend_nvfp4(b["q"], b["kv_nv_codes"], b["kv_nv_scales"], b["kv_rowscale"],
                            b["kv_nv_global"], idx, b["swa"], b["swa_scale"], b["swa_pos0"],
                            b["swa_clip"], b["seq_start"], b["q_start"], b["q_pos"], b["W"],
                            b["sm_scale"])


@pytest.mark.parametrize("seed,clip,rowscale", [(0, False, True), (1, True, False)])
def test_attend_nvfp4_matches_brute(seed, clip, rowscale):
    wl = synth.with_nvfp4_kv(synth.with_scales(tiny(seed, B=2, lengths=(20, 37), rowscale=rowscale),
                                               seed=seed), seed=seed, g=0.75)
    a = np_inputs(wl)
    if clip:
        a["swa_clip"] = (a["q_pos"] - 3).astype(np.int32)
    S = ref.score(a["qI"], a["w"], a["kI"], a["kscale"], a["seq_start"], a["q_start"], a["q_pos"])
    idx = ref.topk(S, a["k"])
    O, L = _attend_nv(a, idx)
    Ob, Lb = brute_attend(a, idx, nvfp4=True)
    assert np.allclose(O, Ob, rtol=1e-12, atol=1e-14)
    assert np.allclose(L, Lb, rtol=1e-12, atol=1e-14)


def test_attend_nvfp4_of_an_exact_reencoding_equals_mx():
    """The MX layout's power-of-two block scales 2^(E-127) are E4M3 values here: the same E2M1
    codes with those scales written per 16 elements (tensor scale 1) must give the MX
    layout's attention exactly."""
    wl = synth.with_scales(tiny(4, B=2, lengths=(30, 45)), seed=4)
    a = np_inputs(wl)
    pw = codecs.e8m0(a["kv_e8m0"])                                  # [N, D/32]
    e4 = synth.encode_e4m3(torch.tensor(np.repeat(pw, 2, axis=1), dtype=torch.float32)).numpy()
    assert np.array_equal(codecs.e4m3(e4), np.repeat(pw, 2, axis=1))   # exact re-encoding
    S = ref.score(a["qI"], a["w"], a["kI"], a["kscale"], a["seq_start"], a["q_start"], a["q_pos"])
    idx = ref.topk(S, a["k"])
    Om, Lm = _attend(a, idx)
    On, Ln = _attend_nv(a, idx, kv_nv_codes=a["kv_codes"], kv_nv_scales=e4, kv_nv_global=1.0)
    assert np.array_equal(Om, On) and np.array_equal(Lm, Ln)


def test_nvfp4_tensor_scale_is_linear_in_the_rows():
    """Scaling g by 2 doubles every decoded global row (checked on the decoder) and, with the
    row-free window empty, leaves the attention weights those of the logits doubled."""
    wl = synth.with_nvfp4_kv(tiny(5, lengths=40), seed=5, g=0.5)
    a = np_inputs(wl)
    r1 = codecs.nvfp4_rows(a["kv_nv_codes"][:8], a["kv_nv_scales"][:8], None, 0.5)
    r2 = codecs.nvfp4_rows(a["kv_nv_codes"][:8], a["kv_nv_scales"][:8], None, 1.0)
    assert np.array_equal(2 * r1, r2)
    idx = np.arange(a["k"])[None, :] % 40
    idx = np.sort(np.unique(idx))[None, :a["k"]]
    clip = np.array([10_000], dtype=np.int32)                       # no window row
    O1, _ = _attend_nv(a, idx, swa_clip=clip, kv_nv_global=0.5)
    O2, _ = _attend_nv(a, idx, swa_clip=clip, kv_nv_global=1.0, sm_scale=a["sm_scale"] / 2)
    assert np.allclose(2 * O1, O2, rtol=1e-12, atol=1e-14)


# ----------------------------------------------------------------- fused RoPE / FP8 epilogue

def _angles(T, R, seed=0):
    th = np.random.default_rng(seed).uniform(-np.pi, np.pi, (T, R))
    return np.cos(th).astype(np.float32), np.sin(th).astype(np.float32)


def test_rope_closed_forms():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, 3, 16))
    one, zero = np.ones((2, 4), np.float32), np.zeros((2, 4), np.float32)
    assert np.array_equal(ref.rope_rotate(x, one, zero), x)             # angle 0
    y = ref.rope_rotate(x, zero, one)                                    # 90 degrees
    assert np.array_equal(y[..., :8], x[..., :8])                        # only the last 2R dims
    assert np.array_equal(y[..., 8::2], -x[..., 9::2]) and np.array_equal(y[..., 9::2], x[..., 8::2])
    c, s_ = _angles(2, 4)
    z = ref.rope_rotate(x, c, s_)
    back = ref.rope_rotate(z, c, s_, inverse=True)
    # float32 cos / sin satisfy c^2 + s^2 = 1 only to ~1e-7: the inverse undoes the rotation
    # up to that factor, and a rotation scales each pair's squared norm by exactly it
    k = (c.astype(np.float64) ** 2 + s_.astype(np.float64) ** 2)[:, None, :]
    assert np.allclose(back[..., :8], x[..., :8], rtol=0, atol=0)
    assert np.allclose(back[..., 8::2], x[..., 8::2] * k, rtol=1e-13, atol=1e-15)
    assert np.allclose(back[..., 9::2], x[..., 9::2] * k, rtol=1e-13, atol=1e-15)
    n0 = x[..., 8::2] ** 2 + x[..., 9::2] ** 2
    n1 = z[..., 8::2] ** 2 + z[..., 9::2] ** 2
    assert np.allclose(n1, n0 * k, rtol=1e-13)


def _bf16_nearest_exact(x: Fraction) -> int:
    """Brute force: the bfloat16 bit pattern nearest to the exact rational x (ties to the even
    pattern), searched among the neighbours of x's float32 rounding with exact distances."""
    import struct
    f = struct.unpack("<I", struct.pack("<f", float(x)))[0] >> 16
    best = None
    for bits in (f - 1, f, f + 1):
        bits &= 0xFFFF
        v = brute.bf16_scalar(bits)
        if not math.isfinite(v):
            continue
        key = (abs(Fraction(v) - x), bits & 1)
        if best is None or key < best[0]:
            best = (key, bits)
    return best[1]


def test_rope_query_is_the_exact_rotation_rounded_once():
    """Every rotated dim equals the exact rational rotation a c - b s / a s + b c of the bf16
    query by the float32 angles, rounded once to the nearest bf16 (brute force with exact
    fractions); the other dims are untouched; angle 0 gives the query itself and 90 degrees
    the exact swap."""
    wl = tiny(9, lengths=40)
    a = np_inputs(wl)
    R, D = 8, a["D"]
    c, s_ = _angles(a["T"], R, seed=9)
    got = ref.rope_query(a["q"], c, s_)
    assert np.array_equal(got[..., :D - 2 * R], a["q"][..., :D - 2 * R])
    for t in range(a["T"]):
        for h in range(0, a["Hq"], 5):
            for i in range(R):
                qa = Fraction(brute.bf16_scalar(a["q"][t, h, D - 2 * R + 2 * i]))
                qb = Fraction(brute.bf16_scalar(a["q"][t, h, D - 2 * R + 2 * i + 1]))
                ci, si = Fraction(float(c[t, i])), Fraction(float(s_[t, i]))
                assert got[t, h, D - 2 * R + 2 * i] == _bf16_nearest_exact(qa * ci - qb * si)
                assert got[t, h, D - 2 * R + 2 * i + 1] == _bf16_nearest_exact(qa * si + qb * ci)
    one, zero = np.ones_like(c), np.zeros_like(s_)
    assert np.array_equal(ref.rope_query(a["q"], one, zero), a["q"])
    sw = ref.rope_query(a["q"], zero, one)
    assert np.array_equal(codecs.bf16(sw[..., D - 16::2]), -codecs.bf16(a["q"][..., D - 15::2]))
    assert np.array_equal(sw[..., D - 15::2], a["q"][..., D - 16::2])


def test_fp8_quantize_closed_forms():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((3, 5, 64)).astype(np.float32)
    x[1, 2] = 0.0
    codes, scale = ref.fp8_quantize(x)
    assert scale[1, 2] == 0 and not codes[1, 2].any()
    am = np.abs(x).argmax(axis=-1)
    for i in range(3):
        for j in range(5):
            if (i, j) != (1, 2):
                assert codes[i, j, am[i, j]] & 0x7F == 0x7E                  # the amax maps to 448
    deq = codecs.e4m3(codes) * scale[..., None]
    # E4M3 keeps 3 mantissa bits: normal values within 2^-4 relative, subnormals within
    # half their spacing 2^-9 * scale
    assert np.all(np.abs(deq - x) <= np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * scale[..., None]) + 1e-30)
    # amax = 448 makes the scale 1 and the codes the plain E4M3 rounding: exact values stay,
    # midpoints go to the even code (1.0625 -> 1.0 = 0x38, 1.1875 -> 1.25 = 0x3A), negative
    # values keep their sign, the subnormal midpoint 2^-10 goes to zero
    row = np.array([448.0, 1.0625, 1.1875, -3.25, 2.0 ** -10, -(2.0 ** -9) * 3, 447.0, 0.0])
    codes, scale = ref.fp8_quantize(row)
    assert scale == 1.0
    assert codes.tolist() == [0x7E, 0x38, 0x3A, 0xC5, 0x00, 0x83, 0x7E, 0x00]
    # scaling the row by a power of two scales the scale and keeps the codes
    c2, s2 = ref.fp8_quantize(row * 2.0 ** -20)
    assert np.array_equal(c2, codes) and s2 == 2.0 ** -20
    # a row that is not a power of two: x * 448 / amax in exact arithmetic (1/3 of the amax
    # maps to 149.33.., between the codes 144 (0x71) and 160 -> 144; -1.5 maps to -224 = 0xF6)
    c3, s3 = ref.fp8_quantize(np.array([3.0, 1.0, -1.5]))
    assert s3 == 3.0 / 448.0 and c3.tolist() == [0x7E, 0x71, 0xF6]


def test_fp8_output_comparator_catches_planted_mistakes():
    """The fused output's comparator: the oracle's own codes pass with a zero error band; a
    code moved by one step away from a midpoint, a wrong scale, or codes of a different row
    fail; with a measured error band a code at an ambiguous midpoint may take either
    neighbour but no other."""
    from helpers import fp8_output_ok
    rng = np.random.default_rng(4)
    O = rng.standard_normal((2, 3, 96))
    codes, scale = ref.fp8_quantize(O)
    zero = np.zeros(O.shape[:-1])
    assert fp8_output_ok(codes, scale, O, zero)[0]
    bad = codes.copy()
    y = O * 448.0 / np.abs(O).max(axis=-1, keepdims=True)
    far = np.argmax((np.abs(y[0, 0]) > 20) & (np.abs(y[0, 0]) < 200))
    bad[0, 0, far] = bad[0, 0, far] + 1                      # next magnitude: one step off
    assert not fp8_output_ok(bad, scale, O, zero)[0]
    assert not fp8_output_ok(codes, scale * 1.01, O, zero)[0]
    assert not fp8_output_ok(codes[:, ::-1], scale, O, zero)[0]
    # put one element exactly on a midpoint: 1.0625 * amax / 448 -> either 0x38 or 0x39
    # passes once the band is nonzero, 0x3A does not
    O2 = O.copy()
    amax = np.abs(O2[1, 2]).max()
    O2[1, 2, 5] = 1.0625 * amax / 448.0
    c2, s2 = ref.fp8_quantize(O2)
    eps = np.full(O.shape[:-1], 1e-9)
    for code, want in ((0x38, True), (0x39, True), (0x3A, False)):
        c = c2.copy()
        c[1, 2, 5] = code
        assert fp8_output_ok(c, s2, O2, eps)[0] is want, code


def test_attend_fused_without_rope_is_attend_then_quantise():
    wl = synth.with_scales(tiny(6, B=2, lengths=(30, 45)), seed=6)
    a = np_inputs(wl)
    S = ref.score(a["qI"], a["w"], a["kI"], a["kscale"], a["seq_start"], a["q_start"], a["q_pos"])
    idx = ref.topk(S, a["k"])
    O, L = _attend(a, idx)
    z = np.zeros((a["T"], 0), np.float32)
    Of, Lf, codes, scale = ref.attend_fused(a["q"], z, z, a["kv_codes"], a["kv_e8m0"], a["kv_rowscale"],
                                            idx, a["swa"], a["swa_scale"], a["swa_pos0"], a["swa_clip"],
                                            a["seq_start"], a["q_start"], a["q_pos"], a["W"], a["sm_scale"])
    assert np.array_equal(Of, O) and np.array_equal(Lf, L)
    c2, s2 = ref.fp8_quantize(O)
    assert np.array_equal(codes, c2) and np.array_equal(scale, s2)


def test_attend_fused_rope_only_touches_the_rope_dims():
    """Rows whose last 2R dims are zero: the query's rotation cannot change any logit, so the
    output equals plain attention, and its (zero) rotary part stays zero after the inverse."""
    wl = synth.with_scales(tiny(7, B=2, lengths=(30, 45)), seed=7)
    a = np_inputs(wl)
    R, D = 8, a["D"]
    a["kv_codes"] = a["kv_codes"].copy()
    a["kv_codes"][:, (D - 2 * R) // 2:] = 0
    a["swa"] = a["swa"].copy()
    a["swa"][..., D - 2 * R:] = 0
    S = ref.score(a["qI"], a["w"], a["kI"], a["kscale"], a["seq_start"], a["q_start"], a["q_pos"])
    idx = ref.topk(S, a["k"])
    O, L = _attend(a, idx)
    c, s_ = _angles(a["T"], R, seed=3)
    Of, Lf, _, _ = ref.attend_fused(a["q"], c, s_, a["kv_codes"], a["kv_e8m0"], a["kv_rowscale"], idx,
                                    a["swa"], a["swa_scale"], a["swa_pos0"], a["swa_clip"],
                                    a["seq_start"], a["q_start"], a["q_pos"], a["W"], a["sm_scale"])
    assert np.array_equal(Of, O) and np.array_equal(Lf, L)
    assert not Of[..., D - 2 * R:].any()


def test_attend_fused_single_row_returns_the_unrotated_row():
    """One selected row and no window row: O is that row, so the output is the row rotated
    back by the query's angle (closed form), whatever q is."""
    wl = tiny(8, lengths=40, W=8)
    a = np_inputs(wl)
    R, D = 4, a["D"]
    idx = np.full((1, a["k"]), -1)
    idx[0, 0] = 17
    c, s_ = _angles(1, R, seed=4)
    Of, _, _, _ = ref.attend_fused(a["q"], c, s_, a["kv_codes"], a["kv_e8m0"], a["kv_rowscale"], idx,
                                   a["swa"], None, a["swa_pos0"], np.array([10_000], np.int32),
                                   a["seq_start"], a["q_start"], a["q_pos"], a["W"], a["sm_scale"])
    row = codecs.global_rows(a["kv_codes"][17:18], a["kv_e8m0"][17:18], a["kv_rowscale"][17:18])[0]
    exp = row.copy()
    cc, ss = c[0].astype(np.float64), s_[0].astype(np.float64)
    e, o = row[D - 2 * R::2], row[D - 2 * R + 1::2]
    exp[D - 2 * R::2] = e * cc + o * ss
    exp[D - 2 * R + 1::2] = -e * ss + o * cc
    assert np.allclose(Of[0], exp[None, :], rtol=1e-13, atol=1e-15)


# ----------------------------------------------------------------- window clipping

def _replay(H=50, nq=6, W=8, seed=13):
    return np_inputs(tiny(seed, lengths=H, W=W, replay=(H, nq)))


def test_clip_at_replay_start_leaves_one_window_row():
    a = _replay()
    s = int(a["swa_clip"][0])
    for t in range(a["T"]):
        u, pos = ref.window_positions(t, 0, a["q_pos"], a["swa_pos0"], a["swa_clip"], a["W"])
        assert pos.min() == s and pos.max() == a["q_pos"][t]
        assert len(u) == a["q_pos"][t] - s + 1
    assert a["q_pos"][0] == s
    u, _ = ref.window_positions(0, 0, a["q_pos"], a["swa_pos0"], a["swa_clip"], a["W"])
    assert len(u) == 1


def test_clip_excludes_rows_before_s_exactly():
    # rows of the window before s never contribute: poison them with NaN codes
    a = _replay()
    idx = np.tile(np.arange(6)[None] * 4, (a["T"], 1))
    O, L = _attend(a, idx)
    s = int(a["swa_clip"][0])
    b = dict(a)
    b["swa"] = a["swa"].copy()
    n_before = s - int(a["swa_pos0"][0])
    b["swa"][0, :n_before] = 0x7F                 # E4M3 NaN
    Ob, Lb = _attend(b, idx)
    assert np.array_equal(O, Ob) and np.array_equal(L, Lb)
    # ... while without a clip they do contribute (the NaN shows up)
    On, _ = _attend(b, idx, swa_clip=None)
    assert np.isnan(On).any()


def test_loose_clip_equals_no_clip_and_w1_is_self_row():
    a = np_inputs(tiny(14, lengths=40, W=8))
    idx = np.arange(6)[None] * 2
    O0, L0 = _attend(a, idx)
    loose = (a["q_pos"] - a["W"] + 1 - 5).astype(np.int32)
    O1, L1 = _attend(a, idx, swa_clip=loose)
    assert np.array_equal(O0, O1) and np.array_equal(L0, L1)
    u, pos = ref.window_positions(0, 0, a["q_pos"], a["swa_pos0"], None, 1)
    assert pos.tolist() == [int(a["q_pos"][0])] or len(pos) == 0


# ----------------------------------------------------------------- decode step

def test_decode_step_is_composition():
    wl = synth.with_scales(tiny(15, B=2, lengths=(25, 41)))
    a = np_inputs(wl)
    S, idx, O, L = ref.decode_step(a)
    S2 = ref.score(a["qI"], a["w"], a["kI"], a["kscale"], a["seq_start"], a["q_start"], a["q_pos"])
    idx2 = ref.topk(S2, a["k"])
    O2, L2 = _attend(a, idx2)
    assert np.array_equal(S, S2) and np.array_equal(idx, idx2)
    assert np.array_equal(O, O2) and np.array_equal(L, L2)


def test_window_membership_hand_cases():
    # buffer rows u=0..3 hold positions 10..13; W = 4
    q_pos = np.array([14, 13, 11, 9]); pos0 = np.array([10])
    u, pos = ref.window_positions(0, 0, q_pos, pos0, None, 4)
    assert pos.tolist() == [11, 12, 13]           # window [11, 14]; position 14 is not in the buffer
    u, pos = ref.window_positions(1, 0, q_pos, pos0, None, 4)
    assert pos.tolist() == [10, 11, 12, 13]       # window [10, 13]
    u, pos = ref.window_positions(2, 0, q_pos, pos0, None, 4)
    assert pos.tolist() == [10, 11]               # causal: nothing after the query
    u, pos = ref.window_positions(3, 0, q_pos, pos0, None, 4)
    assert pos.tolist() == []                     # query before the buffer
    clip = np.array([12, 12, 12, 12])
    u, pos = ref.window_positions(1, 0, q_pos, pos0, clip, 4)
    assert pos.tolist() == [12, 13] and u.tolist() == [2, 3]
    u, pos = ref.window_positions(1, 0, q_pos, np.array([13]), None, 1)
    assert pos.tolist() == [13]                   # W = 1: the query's own row only


# ---------------------------------------------------------------- MXFP8 query (reading R18)

def _e4m3_nearest_brute(y: Fraction) -> int:
    """Nearest finite E4M3 code to the exact value y (ties to the even code, saturating at
    448), by exact comparison against every non-negative code."""
    mag = min(abs(y), Fraction(448))
    best = None
    for code in range(0x7F):
        v = Fraction(brute.e4m3_scalar(code))
        key = (abs(v - mag), code & 1)
        if best is None or key < best[0]:
            best = (key, code)
    return best[1] | 0x80 if y < 0 else best[1]


def test_mxfp8_quantize_matches_a_scalar_brute_force():
    """Blocks of bf16-valued numbers over a wide range of magnitudes: the shared exponent is
    floor(log2 amax) - 8 + 127 and every element the nearest E4M3 code of x / 2^(E-127),
    computed with exact fractions."""
    rng = np.random.default_rng(21)
    x = codecs.bf16(codecs.bf16_round(rng.standard_normal((6, 64)) * 2.0 ** rng.integers(-20, 20, (6, 1))))
    codes, E = codecs.mxfp8_quantize(x)
    for r in range(x.shape[0]):
        for blk in range(2):
            vals = x[r, 32 * blk:32 * blk + 32]
            amax = max(abs(float(v)) for v in vals)
            e_ref = math.frexp(amax)[1] - 1 - 8 + 127
            assert E[r, blk] == e_ref
            for i, v in enumerate(vals):
                y = Fraction(float(v)) / Fraction(2) ** (e_ref - 127)
                want = _e4m3_nearest_brute(y)
                got = int(codes[r, 32 * blk + i])
                assert got == want


def test_mxfp8_quantize_closed_forms():
    # amax 448: scale 1, codes as E4M3 (midpoint 1.0625 -> 1.0); a block whose amax is a power
    # of two 2^k: E = k + 119 and the amax maps to 256 (0x78); 1.9375 * 2^k maps to 496 and
    # saturates at 448 (0x7E); an all-zero block gets exponent 0 and zero codes
    z = [0.0] * 28
    x = np.array([[448.0, 1.0625, -3.0, 0.0] + z,
                  [2.0 ** -5, 2.0 ** -13, -(2.0 ** -6), 0.0] + z,
                  [1.9375 * 8, 1.0, 0.0, 0.0] + z,
                  [0.0] * 32])
    codes, E = codecs.mxfp8_quantize(x)
    assert E[:, 0].tolist() == [127, 114, 122, 0]
    assert codes[0, :3].tolist() == [0x7E, 0x38, 0xC4]
    assert codes[1, :3].tolist() == [0x78, 0x38, 0xF0]
    assert codes[2, :2].tolist() == [0x7E, 0x60]
    assert not codes[3].any()
    deq = codecs.mxfp8_decode(codes, E)
    assert deq[0, 0] == 448.0 and deq[1, 0] == 2.0 ** -5 and deq[2, 0] == 448 * 2.0 ** -5


def _mxfp8_grid_query(shape, seed):
    """bf16 bits of a query whose 32-dim blocks lie on the MXFP8 grid exactly: E4M3 values
    with a block amax in [256, 448] (so E8M0 = 127), times a power of two per block."""
    rng = np.random.default_rng(seed)
    T, H, D = shape
    c = rng.integers(0, 0x7F, (T, H, D)).astype(np.uint8) | (rng.integers(0, 2, (T, H, D)) << 7).astype(np.uint8)
    c[..., ::32] = 0x7C                                   # one element of every block at 384
    v = codecs.e4m3(c) * np.repeat(2.0 ** rng.integers(-12, 4, (T, H, D // 32)), 32, axis=-1)
    return codecs.bf16_round(v)


def test_attend_mxfp8q_is_attend_when_q_is_on_the_grid():
    wl = tiny(22, B=2, lengths=(40, 70))
    a = np_inputs(wl)
    a["q"] = _mxfp8_grid_query(a["q"].shape, 22)
    codes, E = codecs.mxfp8_quantize(codecs.bf16(a["q"]))
    assert np.array_equal(codecs.mxfp8_decode(codes, E), codecs.bf16(a["q"]))
    S = ref.score(a["qI"], a["w"], a["kI"], a["kscale"], a["seq_start"], a["q_start"], a["q_pos"])
    idx = ref.topk(S, a["k"])
    O, L = _attend(a, idx)
    O8, L8 = ref.attend_mxfp8q(a["q"], a["kv_codes"], a["kv_e8m0"], a["kv_rowscale"], idx, a["swa"],
                               a["swa_scale"], a["swa_pos0"], a["swa_clip"], a["seq_start"], a["q_start"],
                               a["q_pos"], a["W"], a["sm_scale"])
    assert np.array_equal(O8, O) and np.array_equal(L8, L)


@pytest.mark.parametrize("seed", [0, 1])
def test_attend_mxfp8q_matches_brute_on_the_quantised_query(seed):
    """The variant against the scalar-loop attention fed the quantised query: the decoded
    MXFP8 values have at most 4 significant bits, so they are exact bf16 values."""
    wl = synth.with_scales(tiny(30 + seed, B=2, lengths=(20, 33), Hq=2, D=64, k=8, W=6), seed=seed)
    a = np_inputs(wl)
    S = ref.score(a["qI"], a["w"], a["kI"], a["kscale"], a["seq_start"], a["q_start"], a["q_pos"])
    idx = ref.topk(S, a["k"])
    O8, L8 = ref.attend_mxfp8q(a["q"], a["kv_codes"], a["kv_e8m0"], a["kv_rowscale"], idx, a["swa"],
                               a["swa_scale"], a["swa_pos0"], a["swa_clip"], a["seq_start"], a["q_start"],
                               a["q_pos"], a["W"], a["sm_scale"])
    codes, E = codecs.mxfp8_quantize(codecs.bf16(a["q"]))
    qhat = codecs.mxfp8_decode(codes, E)
    a2 = dict(a)
    a2["q"] = codecs.bf16_round(qhat)
    assert np.array_equal(codecs.bf16(a2["q"]), qhat)
    Ob, Lb = brute_attend(a2, idx)
    assert np.allclose(O8, Ob, rtol=1e-12, atol=1e-14) and np.allclose(L8, Lb, rtol=1e-12, atol=1e-14)
    # and the quantisation really changed the query
    assert not np.array_equal(qhat, codecs.bf16(a["q"]))
