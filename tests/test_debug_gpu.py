"""Selected positions outside a query's rows, in the release and the SMQA_DEBUG library.

Every build skips a selected position outside [0, min(p_t, len_b - 1)] exactly as it skips
the padding value -1: the output must equal, bit for bit, the output of the same selection
with those entries replaced by -1.  The debug library (libsmqa_debug.so, same sources built
with SMQA_DEBUG) must also report them through smqa_debug_flags, report an E8M0 exponent
outside the range P.V holds exactly in fp16, report nothing for clean inputs, and compute
the same bits as the release library.

Every planted position stays inside the allocated cache (another session's rows, or rows
after the query inside its own session), so even a kernel that ignored the check would
read memory it owns.
"""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from helpers import announce, gpu_attend

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _bits(x):
    return x.contiguous().view(torch.int32)


def _selection(wl, k, seed):
    """k distinct positions per query in [0, p_t] (sorted), from a seeded generator."""
    rng = np.random.default_rng(seed)
    q_start = wl.q_start.cpu().numpy()
    q_pos = wl.q_pos.cpu().numpy()
    idx = np.full((wl.T, k), -1, dtype=np.int32)
    for b in range(wl.B):
        for t in range(q_start[b], q_start[b + 1]):
            p = int(q_pos[t])
            idx[t] = np.sort(rng.choice(p + 1, size=k, replace=False))
    return idx


def _plant_bad_positions(wl, idx):
    """Replace the last two entries of every query with positions outside its rows: in session
    0 one past the session's end (session 1's first rows) and the one after the query; in
    session 1 negative ones other than -1 (session 0's last rows) or the one after the query
    when that is still inside the session.  Returns (bad, clean) selections."""
    seq = wl.seq_start.cpu().numpy()
    q_start = wl.q_start.cpu().numpy()
    q_pos = wl.q_pos.cpu().numpy()
    assert wl.B == 2 and seq[2] - seq[1] > 8 and seq[1] > 8
    bad = idx.copy()
    clean = idx.copy()
    for b in range(2):
        n = int(seq[b + 1] - seq[b])
        for t in range(q_start[b], q_start[b + 1]):
            p = int(q_pos[t])
            if b == 0:
                # past the query; p + 1 <= n stays inside the cache (session 1 follows)
                bad[t, -2:] = (n + 3, p + 1)
            else:
                # the last session's rows end the cache: positions after the query only when
                # the session has one, else a second negative value
                bad[t, -2:] = (-5, p + 1 if p + 1 < n else -7)
            clean[t, -2:] = -1
    return bad, clean


CASES = [
    pytest.param(dict(Hq=64, D=512), 8, id="dimension-split-D512"),
    pytest.param(dict(Hq=16, D=512), 8, id="16-head-D512"),
    pytest.param(dict(Hq=64, D=1792), 4, id="16-head-D1792-few-pairs"),
    pytest.param(dict(Hq=64, D=1792), 16, id="32-head-D1792"),
]


@pytest.mark.parametrize("kw,qps", CASES)
def test_out_of_range_positions_are_skipped_and_reported(lib, kw, qps):
    k = 96
    announce(f"debug positions {kw} queries/session={qps}")
    wl = synth.generate("replay_h100k", seed=3, device=DEV, B=2, lengths=4000, replay=(4000, qps),
                        k=k, **kw)
    bad, clean = _plant_bad_positions(wl, _selection(wl, k, seed=11))
    ib = torch.tensor(bad, device=DEV)
    ic = torch.tensor(clean, device=DEV)
    out_c, lse_c = gpu_attend(lib, wl, ic)
    out_b, lse_b = gpu_attend(lib, wl, ib)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out_b), _bits(out_c)) and torch.equal(_bits(lse_b), _bits(lse_c))
    with lib.debug_build():
        lib.debug_flags(clear=True)
        dout_c, dlse_c = gpu_attend(lib, wl, ic)
        assert lib.debug_flags() == 0
        dout_b, dlse_b = gpu_attend(lib, wl, ib)
        assert lib.debug_flags() == lib.SMQA_DEBUG_POSITION
    assert torch.equal(_bits(dout_c), _bits(out_c)) and torch.equal(_bits(dlse_c), _bits(lse_c))
    assert torch.equal(_bits(dout_b), _bits(out_b)) and torch.equal(_bits(dlse_b), _bits(lse_b))


def test_e8m0_outside_the_fp16_range_is_reported(lib):
    """One block exponent of a selected row set to 150 (2^23: beyond fp16's range once scaled):
    the debug library reports it, and computes what the release library computes."""
    k = 96
    announce("debug e8m0 range")
    wl = synth.generate("replay_h100k", seed=3, device=DEV, B=2, lengths=4000, replay=(4000, 8),
                        k=k, Hq=64, D=512)
    idx = torch.tensor(_selection(wl, k, seed=12), device=DEV)
    row = int(wl.seq_start[0].item()) + int(idx[0, 5].item())
    e8 = wl.kv_e8m0.clone()
    e8[row, 3] = 150
    wl_bad = dataclasses.replace(wl, kv_e8m0=e8)
    out_r, lse_r = gpu_attend(lib, wl_bad, idx)
    torch.cuda.synchronize()
    with lib.debug_build():
        lib.debug_flags(clear=True)
        gpu_attend(lib, wl, idx)
        assert lib.debug_flags() == 0
        out_d, lse_d = gpu_attend(lib, wl_bad, idx)
        assert lib.debug_flags() == lib.SMQA_DEBUG_E8M0
    assert torch.equal(_bits(out_d), _bits(out_r)) and torch.equal(_bits(lse_d), _bits(lse_r))


def test_decode_step_in_the_debug_library_reports_nothing(lib):
    """A whole decode step on valid inputs leaves the debug word clear and matches the release
    library bit for bit (the checks only read)."""
    from helpers import gpu_decode
    announce("debug decode_step decode_8k lengths=6000")
    wl = synth.generate("decode_8k", seed=4, device=DEV, lengths=6000)
    out_r, lse_r, idx_r = gpu_decode(lib, wl)
    torch.cuda.synchronize()
    with lib.debug_build():
        lib.debug_flags(clear=True)
        out_d, lse_d, idx_d = gpu_decode(lib, wl)
        assert lib.debug_flags() == 0
    assert torch.equal(idx_d, idx_r)
    assert torch.equal(_bits(out_d), _bits(out_r)) and torch.equal(_bits(lse_d), _bits(lse_r))


@pytest.mark.parametrize("kw", [
    pytest.param(dict(B=2, lengths=3000), id="short-rows"),
    pytest.param(dict(B=2, lengths=300000), id="streaming-rows"),
])
def test_negative_query_position_scores_nothing(lib, kw):
    """A negative q_pos (outside the stated range) leaves its row all -inf and every other
    row as in a clean call, in both libraries; the debug library reports it as a layout
    finding.  The bad query is the second, so even a fill that started before its row would
    land in the first row (inside the buffer), where the comparison sees it."""
    from helpers import gpu_score
    announce(f"debug negative q_pos {kw}")
    wl = synth.generate("decode_8k", seed=6, device=DEV, **kw)
    S_clean = gpu_score(lib, wl).clone()
    wl.q_pos[1] = -5
    S = gpu_score(lib, wl)
    torch.cuda.synchronize()
    assert torch.equal(S[0], S_clean[0])
    assert bool(torch.all(S[1] == -float("inf")))
    with lib.debug_build():
        lib.debug_flags(clear=True)
        S_d = gpu_score(lib, wl)
        assert lib.debug_flags() == lib.SMQA_DEBUG_LAYOUT
    assert torch.equal(_bits(S_d), _bits(S))


def test_unordered_candidates_are_reported(lib):
    """Two swapped entries of one candidate list: the debug library reports it and, like the
    release library, scores each column at the position it names."""
    from helpers import gpu_score
    announce("debug candidate order")
    wl = synth.generate("decode_8k", seed=7, device=DEV, B=2, lengths=(20000, 40000), n_cand=4096)
    with lib.debug_build():
        lib.debug_flags(clear=True)
        gpu_score(lib, wl)
        assert lib.debug_flags() == 0
    c = wl.cand[0, 10].clone()
    wl.cand[0, 10] = wl.cand[0, 11]
    wl.cand[0, 11] = c
    S = gpu_score(lib, wl)
    torch.cuda.synchronize()
    with lib.debug_build():
        lib.debug_flags(clear=True)
        S_d = gpu_score(lib, wl)
        assert lib.debug_flags() == lib.SMQA_DEBUG_CAND
    assert torch.equal(_bits(S_d), _bits(S))
