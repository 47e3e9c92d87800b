"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Comparators: scores within 1e-4 relative (floor 1e-7 of the row max) and
bit-exact on integer-valued inputs; top-k sets exact outside a 1e-5-relative
gap at the k-th score, and inside it every strictly-better position present
and every chosen one within the band; attention per (query, head) within
max|dO| <= 2e-3 and <= 1e-3 * max|O|, |dLSE| <= 1e-4, with the oracle run on the
GPU's own selection.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import ref
from helpers import (announce, close_attention, close_scores, fp8_output_checks, gpu_attend,
                     gpu_attend_fp8kv, gpu_attend_fused, gpu_attend_nvfp4, gpu_decode, gpu_score,
                     gpu_topk, np_inputs, oracle_attend_for, oracle_scores_for, q_seq_of, topk_set_ok)

pytestmark = pytest.mark.gpu

DEV = "cuda"


def gen(name, seed=0, **kw):
    announce(f"generate {name} seed={seed} {kw}")
    return synth.generate(name, seed=seed, device=DEV, **kw)


def sync():
    torch.cuda.synchronize()


# ------------------------------------------------------------------ score

@pytest.mark.parametrize("name,kw", [
    ("tiny", {}),
    ("decode_8k", {}),
    ("decode_8k", dict(B=3, lengths=(3000, 9000), Hi=40)),            # ragged, Hi not a multiple of 16
    ("replay_h100k", dict(B=2, lengths=3000, replay=(3000, 40))),     # many queries per sequence
])
def test_score_dense(lib, name, kw):
    wl = synth.with_scales(gen(name, **kw)) if name == "replay_h100k" else gen(name, **kw)
    announce(f"score {name} T={wl.T} N={wl.N}")
    S = gpu_score(lib, wl)
    sync()
    a = np_inputs(wl)
    S_ref = ref.score(a["qI"], a["w"], a["kI"], a["kscale"], a["seq_start"], a["q_start"], a["q_pos"],
                      ld=wl.max_ctx)
    S_gpu = S.cpu().numpy().astype(np.float64)
    for t in range(wl.T):
        ok, msg = close_scores(S_gpu[t], S_ref[t])
        assert ok, f"query {t}: {msg}"


# Long single-query-per-sequence rows take the streaming kernel (keys read once, two
# blocks in flight per wave): every head-slice count it is built for, both key widths,
# with and without key scales, ragged lengths that end mid-block.
@pytest.mark.parametrize("Hi,Di,scaled", [(64, 128, True), (20, 64, False), (16, 128, False),
                                          (48, 64, True)])
def test_score_dense_streaming(lib, Hi, Di, scaled):
    wl = gen("decode_8k", B=2, lengths=(131001, 160000), Hi=Hi, Di=Di)
    if scaled:
        wl = synth.with_scales(wl)
    announce(f"score streaming Hi={Hi} Di={Di} lengths={wl.seq_start.tolist()}")
    S = gpu_score(lib, wl)
    sync()
    a = np_inputs(wl)
    S_ref = ref.score(a["qI"], a["w"], a["kI"], a["kscale"], a["seq_start"], a["q_start"], a["q_pos"],
                      ld=wl.max_ctx)
    S_gpu = S.cpu().numpy().astype(np.float64)
    for t in range(wl.T):
        ok, msg = close_scores(S_gpu[t], S_ref[t])
        assert ok, f"query {t}: {msg}"


def test_score_dense_streaming_lengths_an_order_of_magnitude_apart(lib):
    """The streaming kernel deals its workgroups to the sequences in proportion to their
    lengths: five rows between 17K and 300K positions, every score against the oracle."""
    wl = gen("decode_8k", B=5, lengths=(17000, 300000))
    announce(f"score streaming lengths {wl.seq_start.tolist()}")
    S = gpu_score(lib, wl)
    sync()
    a = np_inputs(wl)
    S_ref = ref.score(a["qI"], a["w"], a["kI"], a["kscale"], a["seq_start"], a["q_start"], a["q_pos"],
                      ld=wl.max_ctx)
    S_gpu = S.cpu().numpy().astype(np.float64)
    for t in range(wl.T):
        ok, msg = close_scores(S_gpu[t], S_ref[t])
        assert ok, f"query {t}: {msg}"


def test_score_dense_streaming_uneven_queries(lib):
    """As many queries as sequences, but two on one sequence (one mid-sequence) and none on
    the other: the streaming kernel re-streams the keys per query and scores only j <= p."""
    import dataclasses
    wl = gen("decode_8k", B=2, lengths=150000)
    n0 = int(wl.seq_start[1])
    q_start = torch.tensor([0, 2, 2], dtype=torch.int32, device=DEV)
    q_pos = torch.tensor([n0 - 1, 70001], dtype=torch.int32, device=DEV)
    wl = dataclasses.replace(wl, q_start=q_start, q_pos=q_pos, max_ctx=n0)
    announce("score streaming uneven queries")
    S = gpu_score(lib, wl)
    sync()
    a = np_inputs(wl)
    S_ref = ref.score(a["qI"], a["w"], a["kI"], a["kscale"], a["seq_start"], a["q_start"], a["q_pos"],
                      ld=wl.max_ctx)
    S_gpu = S.cpu().numpy().astype(np.float64)
    assert np.isfinite(S_gpu[1, :70002]).all()
    for t in range(wl.T):
        ok, msg = close_scores(S_gpu[t], S_ref[t])
        assert ok, f"query {t}: {msg}"


# Several queries per sequence: the block kernel splits each sequence's queries into up to
# eight equal parts (grid z) to fill the resident workgroup slots.  Uneven query counts (one
# sequence without queries, parts of one query, empty trailing parts) and queries in the
# middle of their rows, on the 64- and the 256-position block widths.
@pytest.mark.parametrize("lengths,qps", [(3000, 8), (140000, 6)])
def test_score_dense_query_parts_uneven(lib, lengths, qps):
    import dataclasses
    wl = gen("replay_h100k", B=3, lengths=lengths, replay=(lengths, qps))
    T = wl.T
    n = int(wl.seq_start[1])
    q_start = torch.tensor([0, qps - 1, qps - 1, T], dtype=torch.int32, device=DEV)
    q_pos = wl.q_pos.clone()
    q_pos[1] = n // 2                        # mid-row queries in the first and last sequence
    q_pos[T - 3] = n // 3
    q_pos[T - 1] = 5
    wl = dataclasses.replace(wl, q_start=q_start, q_pos=q_pos)
    announce(f"score query parts lengths={lengths} q_start={q_start.tolist()}")
    S = gpu_score(lib, wl)
    sync()
    a = np_inputs(wl)
    S_ref = ref.score(a["qI"], a["w"], a["kI"], a["kscale"], a["seq_start"], a["q_start"], a["q_pos"],
                      ld=wl.max_ctx)
    S_gpu = S.cpu().numpy().astype(np.float64)
    for t in range(T):
        ok, msg = close_scores(S_gpu[t], S_ref[t])
        assert ok, f"query {t}: {msg}"


def test_score_integer_inputs_bit_exact(lib):
    announce("score integer-valued inputs")
    g = torch.Generator(device=DEV).manual_seed(5)
    ints = torch.randint(-4, 5, (1, 64, 128), generator=g, device=DEV).float()
    keys = torch.randint(-4, 5, (5000, 128), generator=g, device=DEV).float()
    wl = gen("decode_8k", lengths=5000)
    wl.qI = synth.encode_e4m3(ints)
    wl.kI = synth.encode_e4m3(keys)
    wl.w = (2.0 ** torch.randint(-3, 3, (1, 64), generator=g, device=DEV).float()).contiguous()
    S = gpu_score(lib, wl)
    sync()
    a = np_inputs(wl)
    S_ref = ref.score(a["qI"], a["w"], a["kI"], None, a["seq_start"], a["q_start"], a["q_pos"])
    assert np.array_equal(S.cpu().numpy()[0, :5000].astype(np.float64), S_ref[0, :5000])


def test_score_candidates(lib):
    wl = gen("decode_8k", B=2, lengths=(20000, 40000), n_cand=16384)
    wl.q_pos[0] -= 777                       # some candidates lie past the query
    announce(f"score candidates lengths={wl.meta['lengths']}")
    S = gpu_score(lib, wl)
    sync()
    a = np_inputs(wl)
    S_ref = ref.score(a["qI"], a["w"], a["kI"], None, a["seq_start"], a["q_start"], a["q_pos"],
                      cand=a["cand"])
    for t in range(wl.T):
        ok, msg = close_scores(S.cpu().numpy()[t], S_ref[t])
        assert ok, f"query {t}: {msg}"
    assert np.isinf(S_ref).any()


@pytest.mark.parametrize("name,kw,n_cand", [
    ("decode_8k", dict(B=3, lengths=(3000, 9000)), None),               # short rows
    ("decode_8k", dict(B=2, lengths=(131001, 140000)), None),           # the streaming kernel
    ("replay_h100k", dict(B=2, lengths=3000, replay=(3000, 40)), None),  # many queries per sequence
    ("decode_8k", dict(B=2, lengths=(20000, 40000)), 4000),             # candidate lists
])
def test_score_writes_every_column(lib, name, kw, n_cand):
    """Every entry of the [T][ld] score array is written: the columns past each query's
    position (and past its sequence), and past the candidate list, up to an ld wider than
    needed, hold -inf; the rest are the scores."""
    wl = gen(name, n_cand=n_cand, **kw)
    if n_cand is None and wl.T > 1:
        wl.q_pos[1] -= 500                                  # a query well inside its sequence
    ld = (wl.max_ctx if n_cand is None else n_cand) + 77
    S = torch.full((wl.T, ld), 7.0, dtype=torch.float32, device=DEV)
    announce(f"score every column {name} T={wl.T} ld={ld} cand={n_cand}")
    lib.sparse_mqa_score(lib.Batch(wl.seq_start, wl.q_start, wl.q_pos, wl.max_ctx), wl.qI, wl.w, wl.kI,
                         wl.kscale, wl.cand, scores=S)
    sync()
    a = np_inputs(wl)
    S_ref = ref.score(a["qI"], a["w"], a["kI"], a["kscale"], a["seq_start"], a["q_start"], a["q_pos"],
                      cand=a["cand"], ld=ld)
    S_gpu = S.cpu().numpy().astype(np.float64)
    assert not (S_gpu == 7.0).any()
    for t in range(wl.T):
        ok, msg = close_scores(S_gpu[t], S_ref[t])
        assert ok, f"query {t}: {msg}"


# ------------------------------------------------------------------ top-k

def _topk_case(lib, S_host, k, cand=None, q_pos=None):
    T, n = S_host.shape
    seq_start = torch.tensor([0, 1 << 30], dtype=torch.int64, device=DEV)   # one long sequence
    q_start = torch.tensor([0, T], dtype=torch.int32, device=DEV)
    if q_pos is None:
        q_pos = np.full(T, n - 1)
    qp = torch.tensor(q_pos, dtype=torch.int32, device=DEV)
    max_ctx = n if cand is None else cand.shape[1]
    L = lib.Batch(seq_start, q_start, qp, int(max_ctx) if cand is not None else int(q_pos.max()) + 1)
    S_dev = torch.tensor(S_host, dtype=torch.float32, device=DEV)
    cd = None if cand is None else torch.tensor(cand, dtype=torch.int32, device=DEV)
    idx, val = lib.topk_select(L, S_dev, k, cand=cd, want_val=True)
    idx, val = idx.cpu().numpy(), val.cpu().numpy()
    # without val_out the selection is the same
    assert np.array_equal(lib.topk_select(L, S_dev, k, cand=cd).cpu().numpy(), idx)
    for t in range(T):
        # val_out: the selected entries' scores, bit for bit, -inf in the padding
        sel = idx[t] >= 0
        cols = idx[t][sel] if cand is None else np.searchsorted(cand[t], idx[t][sel])
        assert np.array_equal(val[t][sel].view(np.uint32),
                              S_host[t].astype(np.float32)[cols].view(np.uint32))
        assert np.all(val[t][~sel] == -np.inf)
        S_ref = S_host[t].astype(np.float32).astype(np.float64)
        if cand is None:
            S_ref = S_ref.copy()
            S_ref[q_pos[t] + 1:] = -np.inf
        ok, msg = topk_set_ok(S_ref, None if cand is None else cand[t], k, idx[t])
        assert ok, f"query {t}: {msg}"
        # exact where there is no near tie
        exp = ref.topk(S_ref[None], k, cand=None if cand is None else cand[t:t + 1])[0]
        if msg != "near-tie band":
            assert np.array_equal(exp, idx[t])
    return idx


# (rows past 524,288 columns read their selection out in two rounds of 16,384 bitmap words)
@pytest.mark.parametrize("n,k", [(8192, 2048), (4096, 256), (16384, 4096), (100_000, 2048),
                                 (524_288, 2048), (30_000, 7), (1_000_000, 4096)])
def test_topk_random(lib, n, k):
    announce(f"topk random n={n} k={k}")
    rng = np.random.default_rng(n + k)
    S = rng.standard_normal((3, n)).astype(np.float32) * 10 + 50
    _topk_case(lib, S, k, q_pos=np.array([n - 1, n // 2, n - 3]))


def test_topk_many_chunks_two_per_workgroup(lib):
    """Calls of at least 4,096 chunks of 4,096 columns take the collect kernel with two chunks
    per workgroup: an odd chunk count (the last workgroup's second chunk lies past the
    bitmap), rows ending mid-chunk, just past one chunk and shorter than k, a row whose
    threshold bin overflows the candidate list (every score equal), and one with a tie
    crowd at the k-th place."""
    n, T, k = 346_000, 49, 2048                      # 85 chunks x 49 queries
    rng = np.random.default_rng(5)
    S = (rng.standard_normal((T, n)) * 10 + 50).astype(np.float32)
    S[3] = 7.0                                       # one bin holds the whole row
    S[4, : 2 * k] = 120.0                            # 4,096 ties across the k-th place
    q_pos = np.full(T, n - 1)
    q_pos[1] = n // 2 + 3
    q_pos[2] = 4097
    q_pos[5] = 100
    q_pos[6] = 8191
    idx = _topk_case(lib, S, k, q_pos=q_pos)
    assert idx[3].tolist() == list(range(k))
    assert idx[4].tolist() == list(range(k))
    assert np.all(idx[5, 101:] == -1) and idx[5, :101].tolist() == list(range(101))


@pytest.mark.parametrize("n", [5000, 60_000])
def test_topk_ties_take_lowest_positions(lib, n):
    announce(f"topk constant scores n={n}")
    S = np.zeros((2, n), dtype=np.float32)
    S[1, ::2] = 1.0                                    # half the entries tie at the top
    idx = _topk_case(lib, S, 2048)
    assert idx[0].tolist() == list(range(2048))
    assert idx[1].tolist() == list(range(0, 4096, 2))


def test_topk_fewer_valid_than_k(lib):
    announce("topk fewer than k")
    rng = np.random.default_rng(1)
    S = rng.standard_normal((2, 40000)).astype(np.float32)
    idx = _topk_case(lib, S, 2048, q_pos=np.array([999, 30000]))
    assert np.all(idx[0, 1000:] == -1) and idx[0, :1000].tolist() == list(range(1000))


def test_topk_candidates_with_masked_entries(lib):
    announce("topk candidates")
    rng = np.random.default_rng(2)
    n_cand = 20000
    cand = np.stack([np.sort(rng.choice(200000, n_cand, replace=False)) for _ in range(2)])
    S = rng.standard_normal((2, n_cand)).astype(np.float32)
    S[0, 15000:] = -np.inf
    _topk_case(lib, S, 2048, cand=cand.astype(np.int32))


# ------------------------------------------------------------------ attention

def _attend_check(lib, wl, idx_np=None):
    a = np_inputs(wl)
    if idx_np is None:
        S = ref.score(a["qI"], a["w"], a["kI"], a["kscale"], a["seq_start"], a["q_start"], a["q_pos"])
        idx_np = ref.topk(S, wl.k)
    idx = torch.tensor(idx_np, dtype=torch.int32, device=DEV)
    announce(f"attend {wl.name} T={wl.T} Hq={wl.Hq} D={wl.D} k={wl.k}")
    out, lse = gpu_attend(lib, wl, idx)
    sync()
    a["swa_clip"] = None if wl.swa_clip is None else wl.swa_clip.cpu().numpy()
    O, L = ref.attend(a["q"], a["kv_codes"], a["kv_e8m0"], a["kv_rowscale"], idx_np, a["swa"],
                      a["swa_scale"], a["swa_pos0"], a["swa_clip"], a["seq_start"], a["q_start"],
                      a["q_pos"], a["W"], a["sm_scale"])
    ok, msg = close_attention(out.cpu().numpy(), O, lse.cpu().numpy(), L)
    assert ok, msg
    return out, lse


@pytest.mark.parametrize("name,kw", [
    ("tiny", {}),
    ("decode_8k", dict(lengths=6000)),
    ("decode_8k", dict(B=2, lengths=3000, Hq=32, D=1024, k=500)),       # 32-head workgroups
    ("decode_8k", dict(B=3, lengths=(300, 2000), k=1000, W=100)),       # partial tiles, W % 32 != 0
    ("replay_h100k", dict(B=2, lengths=4000, replay=(4000, 128))),       # clipped window
])
def test_attend(lib, name, kw):
    _attend_check(lib, gen(name, **kw))


# Every attention kernel and latent width class: the dimension-split kernel with one block per
# wave pair (D = 128: waves 4..7 own no block), an even split (D = 512) and an uneven one
# (D = 640); the 16-head kernel for few queries at D = 1792 and for head counts that are not
# a multiple of 32; the 32-head tile kernel at D = 1792 with 64 (query, head group) pairs;
# and the widest latent the boundary accepts (D = 2048), also at a size whose LDS decides
# the split count.
@pytest.mark.parametrize("name,kw", [
    ("decode_8k", dict(B=2, lengths=1500, Hq=32, D=128, k=256)),
    ("decode_8k", dict(B=2, lengths=1500, Hq=64, D=512, k=256)),
    ("decode_8k", dict(B=2, lengths=(700, 1500), Hq=32, D=640, k=300)),
    ("decode_8k", dict(B=1, lengths=1500, Hq=64, D=1792, k=256)),
    ("decode_8k", dict(B=2, lengths=1500, Hq=48, D=768, k=256)),
    ("decode_8k", dict(B=2, lengths=1500, Hq=32, D=2048, k=256)),
    ("replay_h100k", dict(B=1, lengths=2000, replay=(2000, 32), Hq=64, D=1792, k=256)),
    # 64 queries at the widest latent with k = 2048: one split would need ~175 KB of LDS per
    # workgroup, so the plan takes more splits until a workgroup fits the CU's 160 KiB
    ("decode_8k", dict(B=64, lengths=2100, Hq=64, D=2048, k=2048)),
])
def test_attend_widths_and_head_counts(lib, name, kw):
    _attend_check(lib, gen(name, **kw))


def test_attend_empty_and_window_only_rows(lib):
    """No selected global rows at all (every index -1): query 0 also sees no window row (its
    clip lies past its position), so its output is 0 and its LSE -inf; the others attend to
    their window rows only."""
    wl = gen("replay_h100k", B=1, lengths=2000, replay=(2000, 4))
    clip = wl.swa_clip.clone()
    clip[0] = wl.q_pos[0] + 1
    import dataclasses
    wl = dataclasses.replace(wl, swa_clip=clip)
    idx = np.full((wl.T, wl.k), -1, dtype=np.int32)
    out, lse = _attend_check(lib, wl, idx)
    assert torch.all(out[0] == 0) and torch.all(torch.isneginf(lse[0]))
    assert torch.all(torch.isfinite(lse[1:]))


def test_attend_with_scales_and_padding(lib):
    wl = synth.with_scales(gen("decode_8k", B=2, lengths=(1500, 2500), k=2048))
    a = np_inputs(wl)
    S = ref.score(a["qI"], a["w"], a["kI"], a["kscale"], a["seq_start"], a["q_start"], a["q_pos"])
    idx = ref.topk(S, wl.k)
    assert (idx == -1).any()                          # fewer valid positions than k
    _attend_check(lib, wl, idx)


def test_attend_peaked_rows_respect_the_clip(lib):
    """One dominant row decides O: a dominant window row just before the clip must be excluded
    and one at the clip start included."""
    wl = gen("replay_h100k", B=1, lengths=3000, replay=(3000, 128))
    s = int(wl.swa_clip[0])
    W = wl.W
    pos0 = int(wl.swa_pos0[0])
    # make window row at position s-1 (excluded) and s (included) huge along q of query 0
    q0 = wl.q[0].float()
    direction = torch.sign(q0[0]).to(torch.float32)
    big = synth.encode_e4m3(direction * 448.0)
    u_excl, u_incl = s - 1 - pos0, s - pos0
    if u_excl >= 0:
        wl.swa[0, u_excl] = big
    wl.swa[0, u_incl] = synth.encode_e4m3(direction * 300.0)
    out, _ = _attend_check(lib, wl)
    row_incl = wl.swa[0, u_incl].view(torch.float8_e4m3fn).float()
    # head 0 of query 0 is dominated by the included row
    assert torch.allclose(out[0, 0], row_incl, rtol=1e-2, atol=1e-2)


def _dominant_fp4_row(q_head, mag_code=0x7):
    """E2M1 codes of a latent row whose every element is +-6 (code 0x7 / 0xF) with the sign of
    q_head: its logit tau * 6 * sum|q| dominates every random row's."""
    neg = (q_head < 0).to(torch.uint8)
    nib = mag_code | (neg << 3)
    return (nib[0::2] | (nib[1::2] << 4)).to(torch.uint8)


def test_decode_step_dominant_rows_at_the_topk_boundary(lib):
    """Through decode_step: the oracle's k-th best position gets a latent row that dominates
    head 0's softmax, and the (k+1)-th best an even stronger one (1.5x the row scale).  The
    selection keeps the k-th and drops the (k+1)-th, so head 0's output is the k-th row; a
    boundary off by one would make it the other row (a 50% change)."""
    wl = gen("decode_8k", lengths=6000)
    a = np_inputs(wl)
    S = oracle_scores_for(a, [0])[0]
    order = np.lexsort((np.arange(S.size), -S))
    pk, pk1 = int(order[wl.k - 1]), int(order[wl.k])
    assert S[pk] - S[pk1] > 2e-5 * abs(S[pk])            # outside the 1e-5 band: the set is unique
    q0 = wl.q[0, 0].float()
    for pos, rho in ((pk, 1.0), (pk1, 1.5)):
        wl.kv_codes[pos] = _dominant_fp4_row(q0)
        wl.kv_e8m0[pos] = 127
        wl.kv_rowscale[pos] = rho
    out, lse, idx = _decode_check(lib, wl)
    sel = set(idx[0].cpu().numpy().tolist())
    assert pk in sel and pk1 not in sel
    row = 6.0 * torch.sign(q0)
    assert torch.allclose(out[0, 0], row, rtol=0, atol=1e-3)


def test_decode_step_position_in_both_branches_counts_twice(lib):
    """Reading R4 through decode_step: a window position that top-k also selects contributes
    its global row and its window row as two entries of one softmax.  Both rows are made
    dominant with logits within ~1e-3 of each other and differ in one dim d* (where |q| is
    smallest), +6 in one and -6 in the other: counted twice, head 0's output there is ~0;
    counted once it would be +-6."""
    wl = gen("decode_8k", lengths=6000)
    n = 6000
    P = n - 5                                             # inside the window [n-128, n-1]
    u = P - int(wl.swa_pos0[0])
    # make P's indexer score the largest: its key follows the weighted head sum of q
    qI = wl.qI[0].view(torch.float8_e4m3fn).float()       # [Hi, Di]
    dirn = torch.sign((wl.w[0][:, None] * qI).sum(0))
    wl.kI[P] = synth.encode_e4m3(dirn * 8.0)
    q0 = wl.q[0, 0].float()
    dstar = int(torch.argmin(q0.abs()))
    sgn = torch.sign(q0)
    sgn[sgn == 0] = 1.0
    wl.kv_codes[P] = _dominant_fp4_row(sgn)
    wl.kv_e8m0[P] = 127
    wl.kv_rowscale[P] = 1.0
    w_row = 6.0 * sgn
    w_row[dstar] = -w_row[dstar]
    wl.swa[0, u] = synth.encode_e4m3(w_row)
    out, lse, idx = _decode_check(lib, wl)
    assert P in set(idx[0].cpu().numpy().tolist())
    assert abs(float(out[0, 0, dstar])) < 0.1             # both copies: (+6 - 6) / 2
    others = torch.ones(wl.D, dtype=torch.bool, device=out.device)
    others[dstar] = False
    assert torch.allclose(out[0, 0][others], (6.0 * sgn)[others], rtol=0, atol=1e-2)


# ------------------------------------------------------------------ attend over an FP8 cache

def _attend8_check(lib, wl, idx_np=None):
    a = np_inputs(wl)
    if idx_np is None:
        S = ref.score(a["qI"], a["w"], a["kI"], a["kscale"], a["seq_start"], a["q_start"], a["q_pos"])
        idx_np = ref.topk(S, wl.k)
    idx = torch.tensor(idx_np, dtype=torch.int32, device=DEV)
    announce(f"attend_fp8kv {wl.name} T={wl.T} Hq={wl.Hq} D={wl.D} k={wl.k}")
    out, lse = gpu_attend_fp8kv(lib, wl, idx)
    sync()
    O, L = ref.attend_fp8kv(a["q"], a["kv_fp8"], a["kv_fp8_scale"], idx_np, a["swa"],
                            a["swa_scale"], a["swa_pos0"], a["swa_clip"], a["seq_start"],
                            a["q_start"], a["q_pos"], a["W"], a["sm_scale"])
    ok, msg = close_attention(out.cpu().numpy(), O, lse.cpu().numpy(), L)
    assert ok, msg
    return out, lse


# 16-row global tiles: k = 2048 (whole tiles), k = 1000 and 300 (a partial last tile), the
# dimension-split widths of one, an even and an uneven block share per wave, the clipped
# replay window, row scales on both caches and none.
@pytest.mark.parametrize("name,kw,scales", [
    ("decode_8k", dict(lengths=6000), True),
    ("decode_8k", dict(B=3, lengths=(300, 2000), k=1000, W=100), False),
    ("decode_8k", dict(B=2, lengths=1500, Hq=32, D=128, k=256), True),
    ("decode_8k", dict(B=2, lengths=1500, Hq=64, D=512, k=256), False),
    ("decode_8k", dict(B=2, lengths=(700, 1500), Hq=32, D=640, k=300), True),
    ("replay_h100k", dict(B=2, lengths=4000, replay=(4000, 128)), True),
])
def test_attend_fp8kv(lib, name, kw, scales):
    wl = synth.with_fp8_kv(gen(name, **kw), rowscale=scales)
    if scales:
        wl = synth.with_scales(wl)
    _attend8_check(lib, wl)


def test_attend_fp8kv_window_only_and_padding(lib):
    """Every index -1 (window rows only; query 0 sees none), then a selection padded with -1."""
    import dataclasses
    wl = synth.with_fp8_kv(gen("replay_h100k", B=1, lengths=2000, replay=(2000, 4)))
    clip = wl.swa_clip.clone()
    clip[0] = wl.q_pos[0] + 1
    wl = dataclasses.replace(wl, swa_clip=clip)
    out, lse = _attend8_check(lib, wl, np.full((wl.T, wl.k), -1, dtype=np.int32))
    assert torch.all(out[0] == 0) and torch.all(torch.isneginf(lse[0]))
    wl = synth.with_fp8_kv(gen("decode_8k", B=2, lengths=(1500, 2500), k=2048))
    a = np_inputs(wl)
    S = ref.score(a["qI"], a["w"], a["kI"], a["kscale"], a["seq_start"], a["q_start"], a["q_pos"])
    idx = ref.topk(S, wl.k)
    assert (idx == -1).any()
    _attend8_check(lib, wl, idx)


# ------------------------------------------------------------------ attend over an NVFP4 cache

def _attend_nv_check(lib, wl, idx_np=None):
    a = np_inputs(wl)
    if idx_np is None:
        S = ref.score(a["qI"], a["w"], a["kI"], a["kscale"], a["seq_start"], a["q_start"], a["q_pos"])
        idx_np = ref.topk(S, wl.k)
    idx = torch.tensor(idx_np, dtype=torch.int32, device=DEV)
    announce(f"attend_nvfp4 {wl.name} T={wl.T} Hq={wl.Hq} D={wl.D} k={wl.k}")
    out, lse = gpu_attend_nvfp4(lib, wl, idx)
    sync()
    O, L = ref.attend_nvfp4(a["q"], a["kv_nv_codes"], a["kv_nv_scales"], a["kv_rowscale"],
                            a["kv_nv_global"], idx_np, a["swa"], a["swa_scale"], a["swa_pos0"],
                            a["swa_clip"], a["seq_start"], a["q_start"], a["q_pos"], a["W"],
                            a["sm_scale"])
    ok, msg = close_attention(out.cpu().numpy(), O, lse.cpu().numpy(), L)
    assert ok, msg
    return out, lse


# MX-sized 32-row tiles with E4M3 block scales per 16: whole and partial tiles, one, an even
# and an uneven block share per wave (D = 128 / 512 / 640: 1, 4 and 13 scale loads per tile),
# the clipped replay window, with and without the extra row scale.
@pytest.mark.parametrize("name,kw", [
    ("decode_8k", dict(lengths=6000)),
    ("decode_8k", dict(B=3, lengths=(300, 2000), k=1000, W=100, rowscale=False)),
    ("decode_8k", dict(B=2, lengths=1500, Hq=32, D=128, k=256)),
    ("decode_8k", dict(B=2, lengths=1500, Hq=64, D=512, k=256, rowscale=False)),
    ("decode_8k", dict(B=2, lengths=(700, 1500), Hq=32, D=640, k=300)),
    ("replay_h100k", dict(B=2, lengths=4000, replay=(4000, 128))),
])
def test_attend_nvfp4(lib, name, kw):
    _attend_nv_check(lib, synth.with_scales(synth.with_nvfp4_kv(gen(name, **kw))))


def test_attend_nvfp4_window_only_and_padding(lib):
    """Every index -1 (window rows only; query 0 sees none), then a selection padded with -1
    (the padded rows' dummy scales must not reach the output)."""
    import dataclasses
    wl = synth.with_nvfp4_kv(gen("replay_h100k", B=1, lengths=2000, replay=(2000, 4)))
    clip = wl.swa_clip.clone()
    clip[0] = wl.q_pos[0] + 1
    wl = dataclasses.replace(wl, swa_clip=clip)
    out, lse = _attend_nv_check(lib, wl, np.full((wl.T, wl.k), -1, dtype=np.int32))
    assert torch.all(out[0] == 0) and torch.all(torch.isneginf(lse[0]))
    wl = synth.with_nvfp4_kv(gen("decode_8k", B=2, lengths=(1500, 2500), k=2048), g=0.01)
    a = np_inputs(wl)
    S = ref.score(a["qI"], a["w"], a["kI"], a["kscale"], a["seq_start"], a["q_start"], a["q_pos"])
    idx = ref.topk(S, wl.k)
    assert (idx == -1).any()
    _attend_nv_check(lib, wl, idx)


# ------------------------------------------------------------------ scaled matrix cores, MXFP8 query

def _attend_mx8q_check(lib, wl, idx_np=None):
    a = np_inputs(wl)
    if idx_np is None:
        S = ref.score(a["qI"], a["w"], a["kI"], a["kscale"], a["seq_start"], a["q_start"], a["q_pos"])
        idx_np = ref.topk(S, wl.k)
    idx = torch.tensor(idx_np, dtype=torch.int32, device=DEV)
    announce(f"attend_mxfp8q {wl.name} T={wl.T} Hq={wl.Hq} D={wl.D} k={wl.k}")
    out, lse = lib.sparse_mqa_attend_mxfp8q(lib.Batch(wl.seq_start, wl.q_start, wl.q_pos, wl.max_ctx), wl.q,
                                            wl.kv_codes, wl.kv_e8m0, wl.kv_rowscale, idx, wl.swa, wl.swa_scale,
                                            wl.swa_pos0, wl.swa_clip, wl.sm_scale)
    sync()
    args = (a["kv_codes"], a["kv_e8m0"], a["kv_rowscale"], idx_np, a["swa"], a["swa_scale"], a["swa_pos0"],
            a["swa_clip"], a["seq_start"], a["q_start"], a["q_pos"], a["W"], a["sm_scale"])
    O, L = ref.attend_mxfp8q(a["q"], *args)
    ok, msg = close_attention(out.cpu().numpy(), O, lse.cpu().numpy(), L)
    assert ok, msg
    return out, lse, O, ref.attend(a["q"], *args)[0]


# Whole and partial tiles, several splits (decode) and one (replay), an odd number of 32-dim
# blocks per wave (D = 640: 3 and 2; D = 128: one block on waves 0..3, none on 4..7), the
# clipped replay window, with and without row scales.
@pytest.mark.parametrize("name,kw,scales", [
    ("decode_8k", dict(lengths=6000), True),
    ("decode_8k", dict(B=3, lengths=(300, 2000), k=1000, W=100, rowscale=False), False),
    ("decode_8k", dict(B=2, lengths=1500, Hq=32, D=128, k=256), True),
    ("decode_8k", dict(B=2, lengths=1500, Hq=64, D=512, k=256), False),
    ("decode_8k", dict(B=2, lengths=(700, 1500), Hq=32, D=640, k=300), True),
    ("replay_h100k", dict(B=2, lengths=4000, replay=(4000, 128)), True),
])
def test_attend_mxfp8q(lib, name, kw, scales):
    wl = gen(name, **kw)
    if scales:
        wl = synth.with_scales(wl)
    out, _, O8, O = _attend_mx8q_check(lib, wl)
    # the variant is not the plain attention: quantising q moves O well past the bar
    assert np.abs(O8 - O).max() > 1e-3


def test_attend_mxfp8q_window_only_and_padding(lib):
    """Every index -1 (window rows only; query 0 sees none), then a selection padded with -1."""
    import dataclasses
    wl = gen("replay_h100k", B=1, lengths=2000, replay=(2000, 4))
    clip = wl.swa_clip.clone()
    clip[0] = wl.q_pos[0] + 1
    wl = dataclasses.replace(wl, swa_clip=clip)
    out, lse, _, _ = _attend_mx8q_check(lib, wl, np.full((wl.T, wl.k), -1, dtype=np.int32))
    assert torch.all(out[0] == 0) and torch.all(torch.isneginf(lse[0]))
    wl = gen("decode_8k", B=2, lengths=(1500, 2500), k=2048)
    a = np_inputs(wl)
    S = ref.score(a["qI"], a["w"], a["kI"], a["kscale"], a["seq_start"], a["q_start"], a["q_pos"])
    idx = ref.topk(S, wl.k)
    assert (idx == -1).any()
    _attend_mx8q_check(lib, wl, idx)


# ------------------------------------------------------------------ fused RoPE / FP8 epilogue

def _angles(T, R, seed):
    g = torch.Generator().manual_seed(seed)
    th = (torch.rand((T, R), generator=g, dtype=torch.float64) * 2 - 1) * 3.14159
    return th.cos().float().to(DEV), th.sin().float().to(DEV)


# The rotary part of DeepSeek-style latents (64 dims) and a short one, on whole and partial
# tiles, one and several splits, the clipped replay window.  The FP8 codes and scales are
# checked against the oracle's own O' (equal codes except where the oracle's pre-rounding
# value lies within the error band of an E4M3 rounding midpoint), and the oracle's quantiser
# applied to the GPU's own fp32 output must reproduce them up to the kernel's fp32 rounding.
@pytest.mark.parametrize("name,kw,R", [
    ("decode_8k", dict(lengths=6000), 32),
    ("decode_8k", dict(B=3, lengths=(300, 2000), k=1000, W=100), 32),
    ("decode_8k", dict(B=2, lengths=1500, Hq=32, D=128, k=256), 4),
    ("decode_8k", dict(B=2, lengths=(700, 1500), Hq=32, D=640, k=300), 0),
    ("replay_h100k", dict(B=2, lengths=4000, replay=(4000, 128)), 32),
    ("decode_8k", dict(B=2, lengths=(900, 1800), Hq=96, D=512, k=300), 256),   # every dim rotary
    ("replay_h100k", dict(B=1, lengths=2500, replay=(2500, 128), Hq=96, D=512, k=500), 64),
])
def test_attend_fused(lib, name, kw, R):
    wl = synth.with_scales(gen(name, **kw))
    a = np_inputs(wl)
    S = ref.score(a["qI"], a["w"], a["kI"], a["kscale"], a["seq_start"], a["q_start"], a["q_pos"])
    idx_np = ref.topk(S, wl.k)
    idx = torch.tensor(idx_np, dtype=torch.int32, device=DEV)
    c, s_ = _angles(wl.T, R, seed=R + wl.T)
    announce(f"attend_fused {wl.name} T={wl.T} Hq={wl.Hq} D={wl.D} k={wl.k} R={R}")
    o8, osc, out, lse = gpu_attend_fused(lib, wl, idx, c if R else None, s_ if R else None)
    sync()
    Oi, L, _, _ = ref.attend_fused(a["q"], c.cpu().numpy(), s_.cpu().numpy(), a["kv_codes"], a["kv_e8m0"],
                                   a["kv_rowscale"], idx_np, a["swa"], a["swa_scale"], a["swa_pos0"],
                                   a["swa_clip"], a["seq_start"], a["q_start"], a["q_pos"], a["W"],
                                   a["sm_scale"])
    ok, msg = close_attention(out.cpu().numpy(), Oi, lse.cpu().numpy(), L)
    assert ok, msg
    print(fp8_output_checks(o8.cpu().numpy(), osc.cpu().numpy(), Oi, out.cpu().numpy()))
    # without the fp32 output the codes are the same
    o8b, oscb, outb, _ = gpu_attend_fused(lib, wl, idx, c if R else None, s_ if R else None, want_out=False)
    sync()
    assert outb is None and torch.equal(o8b, o8) and torch.equal(oscb, osc)


def test_attend_fused_zero_rows_and_window_only(lib):
    """A query that sees no row gives an all-zero output: scale 0 and zero codes; the others
    attend to their window rows only (every index -1)."""
    import dataclasses
    wl = gen("replay_h100k", B=1, lengths=2000, replay=(2000, 4))
    clip = wl.swa_clip.clone()
    clip[0] = wl.q_pos[0] + 1
    wl = dataclasses.replace(wl, swa_clip=clip)
    a = np_inputs(wl)
    idx_np = np.full((wl.T, wl.k), -1, dtype=np.int32)
    idx = torch.tensor(idx_np, device=DEV)
    c, s_ = _angles(wl.T, 32, seed=5)
    announce(f"attend_fused zero rows T={wl.T}")
    o8, osc, out, lse = gpu_attend_fused(lib, wl, idx, c, s_)
    sync()
    assert torch.all(o8[0] == 0) and torch.all(osc[0] == 0) and torch.all(out[0] == 0)
    Oi, L, _, _ = ref.attend_fused(a["q"], c.cpu().numpy(), s_.cpu().numpy(), a["kv_codes"], a["kv_e8m0"],
                                   a["kv_rowscale"], idx_np, a["swa"], a["swa_scale"], a["swa_pos0"],
                                   a["swa_clip"], a["seq_start"], a["q_start"], a["q_pos"], a["W"],
                                   a["sm_scale"])
    ok, msg = close_attention(out.cpu().numpy(), Oi, lse.cpu().numpy(), L)
    assert ok, msg
    fp8_output_checks(o8.cpu().numpy(), osc.cpu().numpy(), Oi, out.cpu().numpy())


def test_attend_nvfp4_small_tensor_scale(lib):
    """g = 2^-12 puts the block scales near the top of E4M3 (~100-400) and the window P
    multiplier sigma * K near 4096: both within the documented range."""
    wl = synth.with_nvfp4_kv(gen("decode_8k", B=2, lengths=(3000, 5000), k=1024), g=2.0 ** -12)
    assert int(wl.kv_nv_scales.max()) <= 0x7E
    _attend_nv_check(lib, synth.with_scales(wl))


# ------------------------------------------------------------------ decode step

def _decode_check(lib, wl, ts=None):
    announce(f"decode_step {wl.name} T={wl.T} N={wl.N} cand={wl.cand is not None}")
    out, lse, idx = gpu_decode(lib, wl)
    sync()
    a = np_inputs(wl)
    ts = list(range(wl.T)) if ts is None else ts
    cand = a["cand"]
    S_ref = oracle_scores_for(a, ts, cand)
    idx_g = idx.cpu().numpy()
    for i, t in enumerate(ts):
        ok, msg = topk_set_ok(S_ref[i], None if cand is None else cand[t], wl.k, idx_g[t])
        assert ok, f"query {t}: {msg}"
    O, L = oracle_attend_for(a, ts, idx_g[ts])
    ok, msg = close_attention(out.cpu().numpy()[ts], O, lse.cpu().numpy()[ts], L)
    assert ok, msg
    return out, lse, idx


@pytest.mark.parametrize("name,kw", [
    ("tiny", {}),
    ("decode_8k", {}),
    ("ragged_b32", dict(B=4, lengths=(16384, 30000))),
    ("replay_h100k", dict(B=2, lengths=5000, replay=(5000, 128))),
    ("decode_512k", dict(B=2, lengths=70000)),
])
def test_decode_step(lib, name, kw):
    _decode_check(lib, gen(name, **kw))


# Long single-query rows: the streaming score kernel also builds the top-k's first-digit
# histogram, and the top-k skips its own histogram pass.
# decode_step with MegaAttention's fused attention: several splits (one decode query) and
# one split (a 128-query replay chunk, quantised inside the attention kernel).
@pytest.mark.parametrize("name,kw", [
    ("decode_8k", dict(lengths=6000)),
    ("replay_h100k", dict(B=1, lengths=3000, replay=(3000, 128))),
])
def test_decode_step_fused(lib, name, kw):
    wl = gen(name, **kw)
    c, s_ = _angles(wl.T, 32, seed=wl.T)
    L = lib.Batch(wl.seq_start, wl.q_start, wl.q_pos, wl.max_ctx)
    announce(f"decode_step_fused {wl.name} T={wl.T}")
    o8, osc, out, lse, idx = lib.decode_step_fused(L, wl.qI, wl.w, wl.kI, wl.kscale, wl.cand, wl.q, c, s_,
                                                   wl.kv_codes, wl.kv_e8m0, wl.kv_rowscale, wl.swa,
                                                   wl.swa_scale, wl.swa_pos0, wl.swa_clip, wl.k, wl.sm_scale)
    _, _, idx_plain = gpu_decode(lib, wl)
    sync()
    assert torch.equal(idx, idx_plain)                 # the same selection as the plain step
    a = np_inputs(wl)
    idx_g = idx.cpu().numpy()
    S_ref = oracle_scores_for(a, [0], a["cand"])
    ok, msg = topk_set_ok(S_ref[0], None, wl.k, idx_g[0])
    assert ok, msg
    Oi, Lr, _, _ = ref.attend_fused(a["q"], c.cpu().numpy(), s_.cpu().numpy(), a["kv_codes"], a["kv_e8m0"],
                                    a["kv_rowscale"], idx_g, a["swa"], a["swa_scale"], a["swa_pos0"],
                                    a["swa_clip"], a["seq_start"], a["q_start"], a["q_pos"], a["W"],
                                    a["sm_scale"])
    ok, msg = close_attention(out.cpu().numpy(), Oi, lse.cpu().numpy(), Lr)
    assert ok, msg
    fp8_output_checks(o8.cpu().numpy(), osc.cpu().numpy(), Oi, out.cpu().numpy())


def _with_queries(wl, q_start, q_pos):
    import dataclasses
    qs = torch.tensor(q_start, dtype=torch.int32, device=DEV)
    qp = torch.tensor(q_pos, dtype=torch.int32, device=DEV)
    T = len(q_pos)
    assert T == wl.T, "the helper keeps the per-query tensors, so T must not change"
    return dataclasses.replace(wl, q_start=qs, q_pos=qp, max_ctx=int(max(q_pos)) + 1)


def test_decode_step_streaming_histogram(lib):
    _decode_check(lib, gen("decode_512k", B=2, lengths=(140000, 160000)))


def test_decode_step_streaming_unequal_lengths(lib):
    _decode_check(lib, gen("decode_512k", B=4, lengths=(20000, 250000)))


def test_decode_step_streaming_short_query(lib):
    """One query sees fewer positions than k (everything scored is selected)."""
    wl = gen("decode_512k", B=2, lengths=150000)
    _decode_check(lib, _with_queries(wl, [0, 1, 2], [149999, 1500]))


def test_decode_step_streaming_two_queries_one_sequence(lib):
    wl = gen("decode_512k", B=2, lengths=150000)
    _decode_check(lib, _with_queries(wl, [0, 2, 2], [149999, 90001]))


def test_decode_step_candidates(lib):
    _decode_check(lib, gen("decode_512k", B=2, lengths=60000, n_cand=16384))


# full sizes, in the configuration the benchmark times; sampled queries where the oracle is slow
@pytest.mark.parametrize("name,ts", [
    ("decode_8k", None),
    ("decode_512k", None),
    ("ragged_b32", [0, 7, 31]),
    ("replay_h100k", [0, 1, 127, 128, 700, 1023]),
])
def test_decode_step_full_size(lib, name, ts):
    _decode_check(lib, gen(name), ts)


# run to run, bit for bit: the split merge sums partials in a fixed order and the top-k
# histogram's atomics only add integers
@pytest.mark.parametrize("name,kw", [
    ("ragged_b32", dict(B=3, lengths=(20000, 40000))),
    ("decode_512k", {}),                                      # full size: histogram atomics
    ("replay_h100k", dict(B=2, lengths=20000, replay=(20000, 128))),
])
def test_decode_step_deterministic(lib, name, kw):
    wl = gen(name, **kw)
    announce(f"decode_step determinism {name}")
    o1, l1, i1 = gpu_decode(lib, wl)
    o2, l2, i2 = gpu_decode(lib, wl)
    sync()
    assert torch.equal(i1, i2) and torch.equal(o1, o2) and torch.equal(l1, l2)


# full-size scores in the configurations the benchmark times: every query at 512K, sampled
# queries of the ragged batch and of the replay chunk (the oracle's cost)
@pytest.mark.parametrize("name,ts", [
    ("decode_512k", None),
    ("ragged_b32", [0, 13, 31]),
    ("replay_h100k", [0, 127, 128, 700, 1023]),
])
def test_score_full_size(lib, name, ts):
    wl = gen(name)
    announce(f"score full size {name} T={wl.T}")
    S = gpu_score(lib, wl)
    sync()
    a = np_inputs(wl)
    ts = list(range(wl.T)) if ts is None else ts
    S_ref = oracle_scores_for(a, ts)
    S_gpu = S.cpu().numpy()
    for i, t in enumerate(ts):
        ok, msg = close_scores(S_gpu[t], S_ref[i])
        assert ok, f"query {t}: {msg}"


# decode_step inside a captured HIP graph (no allocation, memset or host synchronisation in
# the call): every replay, with unrelated eager work between replays, must reproduce the
# eager call bit for bit.
@pytest.mark.parametrize("name,kw", [
    ("decode_8k", {}),                                        # short rows, split attention
    ("decode_512k", dict(B=2, lengths=70000)),                # long rows: zeroing, histogram
    ("replay_h100k", dict(B=1, lengths=5000, replay=(5000, 64))),
])
def test_decode_step_graph_replay(lib, name, kw):
    wl = gen(name, **kw)
    announce(f"decode_step graph replay {name}")
    L = lib.Batch(wl.seq_start, wl.q_start, wl.q_pos, wl.max_ctx)
    n_cand = 0 if wl.cand is None else wl.cand.shape[1]
    out = torch.empty((wl.T, wl.Hq, wl.D), dtype=torch.float32, device=DEV)
    lse = torch.empty((wl.T, wl.Hq), dtype=torch.float32, device=DEV)
    idx = torch.empty((wl.T, wl.k), dtype=torch.int32, device=DEV)
    ws = torch.empty(lib.decode_step_workspace_size(L, wl.k, n_cand, wl.W, wl.Hq, wl.D) + 256,
                     dtype=torch.uint8, device=DEV)
    args = (L, wl.qI, wl.w, wl.kI, wl.kscale, wl.cand, wl.q, wl.kv_codes, wl.kv_e8m0, wl.kv_rowscale,
            wl.swa, wl.swa_scale, wl.swa_pos0, wl.swa_clip, wl.k, wl.sm_scale)
    step = lambda: lib.decode_step(*args, out=out, lse=lse, idx=idx, workspace=ws)
    step()
    sync()
    ref_out, ref_lse, ref_idx = out.clone(), lse.clone(), idx.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    sync()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    sync()
    noise = torch.randn(1 << 20, device=DEV)
    for r in range(3):
        out.zero_(); lse.zero_(); idx.zero_(); ws.zero_()
        noise.mul_(1.0001)                                   # eager work between replays
        sync()
        g.replay()
        sync()
        assert torch.equal(idx, ref_idx), f"replay {r}: idx"
        assert torch.equal(out, ref_out), f"replay {r}: out"
        assert torch.equal(lse, ref_lse), f"replay {r}: lse"


@pytest.mark.parametrize("name,kw", [
    ("decode_8k", dict(lengths=5000)),                                    # several splits
    ("replay_h100k", dict(B=1, lengths=3000, replay=(3000, 128))),        # one split
])
def test_decode_step_fused_graph_replay(lib, name, kw):
    """The fused decode step captured into a HIP graph: three replays, with eager work and a
    cleared workspace and outputs between them, each equal to the eager call bit for bit."""
    wl = gen(name, **kw)
    announce(f"decode_step_fused graph replay {name}")
    L = lib.Batch(wl.seq_start, wl.q_start, wl.q_pos, wl.max_ctx)
    c, s_ = _angles(wl.T, 32, seed=11)
    o8 = torch.empty((wl.T, wl.Hq, wl.D), dtype=torch.uint8, device=DEV)
    osc = torch.empty((wl.T, wl.Hq), dtype=torch.float32, device=DEV)
    lse = torch.empty((wl.T, wl.Hq), dtype=torch.float32, device=DEV)
    idx = torch.empty((wl.T, wl.k), dtype=torch.int32, device=DEV)
    ws = torch.empty(lib.decode_step_workspace_size(L, wl.k, 0, wl.W, wl.Hq, wl.D) + 256,
                     dtype=torch.uint8, device=DEV)
    step = lambda: lib.decode_step_fused(L, wl.qI, wl.w, wl.kI, wl.kscale, None, wl.q, c, s_, wl.kv_codes,
                                         wl.kv_e8m0, wl.kv_rowscale, wl.swa, wl.swa_scale, wl.swa_pos0,
                                         wl.swa_clip, wl.k, wl.sm_scale, out_fp8=o8, out_scale=osc,
                                         lse=lse, idx=idx, want_out=False, workspace=ws)
    step()
    sync()
    ref8, refs, refl, refi = o8.clone(), osc.clone(), lse.clone(), idx.clone()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        step()
    torch.cuda.current_stream().wait_stream(st)
    sync()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    sync()
    noise = torch.randn(1 << 20, device=DEV)
    for r in range(3):
        o8.zero_(); osc.zero_(); lse.zero_(); idx.zero_(); ws.zero_()
        noise.mul_(1.0001)
        sync()
        g.replay()
        sync()
        assert torch.equal(idx, refi), f"replay {r}: idx"
        assert torch.equal(o8, ref8) and torch.equal(osc, refs), f"replay {r}: fp8 output"
        assert torch.equal(lse, refl), f"replay {r}: lse"
