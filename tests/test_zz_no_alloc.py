"""decode_step_noalloc (the library's device scratch buffer as workspace) against
decode_step with a caller workspace: two calls in a row, the second on a smaller batch,
each bit for bit equal to decode_step on the same inputs (same kernels, same plan), and
the first also within the oracle's bar."""
import numpy as np
import pytest
import torch

import synth
from helpers import announce, close_attention, gpu_decode, np_inputs, oracle_attend_for, \
    oracle_scores_for, topk_set_ok

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _noalloc(lib, wl):
    L = lib.Batch(wl.seq_start, wl.q_start, wl.q_pos, wl.max_ctx)
    out = torch.empty((wl.T, wl.Hq, wl.D), dtype=torch.float32, device=DEV)
    lse = torch.empty((wl.T, wl.Hq), dtype=torch.float32, device=DEV)
    idx = torch.empty((wl.T, wl.k), dtype=torch.int32, device=DEV)
    lib.decode_step_noalloc(L, wl.qI, wl.w, wl.kI, wl.kscale, wl.cand, wl.q, wl.kv_codes, wl.kv_e8m0,
                            wl.kv_rowscale, wl.swa, wl.swa_scale, wl.swa_pos0, wl.swa_clip, wl.k,
                            wl.sm_scale, out, lse, idx)
    return out, lse, idx


@pytest.mark.parametrize("first,second", [
    (("decode_512k", dict(B=2, lengths=70000)), ("decode_8k", dict(lengths=6000))),
    (("ragged_b32", dict(B=6, lengths=(16384, 40000))), ("tiny", {})),
])
def test_decode_step_noalloc_matches_decode_step(lib, first, second):
    for r, (name, kw) in enumerate((first, second)):
        wl = synth.generate(name, seed=r, device=DEV, **kw)
        announce(f"decode_step_noalloc call {r}: {name} T={wl.T} N={wl.N}")
        out, lse, idx = _noalloc(lib, wl)
        ref_out, ref_lse, ref_idx = gpu_decode(lib, wl)
        torch.cuda.synchronize()
        assert torch.equal(idx, ref_idx), f"call {r}: idx"
        assert torch.equal(out, ref_out), f"call {r}: out"
        assert torch.equal(lse, ref_lse), f"call {r}: lse"
        if r == 0:
            a = np_inputs(wl)
            ts = [0, wl.T - 1]
            S_ref = oracle_scores_for(a, ts)
            idx_g = idx.cpu().numpy()
            for i, t in enumerate(ts):
                ok, msg = topk_set_ok(S_ref[i], None, wl.k, idx_g[t])
                assert ok, f"query {t}: {msg}"
            O, L = oracle_attend_for(a, ts, idx_g[ts])
            ok, msg = close_attention(out.cpu().numpy()[ts], O, lse.cpu().numpy()[ts], L)
            assert ok, msg


def test_decode_step_noalloc_rejects_an_oversized_batch(lib):
    wl = synth.generate("replay_h100k", seed=0, device=DEV, B=3, lengths=80000, replay=(80000, 128))
    L = lib.Batch(wl.seq_start, wl.q_start, wl.q_pos, wl.max_ctx)
    assert lib.decode_step_workspace_size(L, wl.k, 0, wl.W, wl.Hq, wl.D) > (96 << 20)
    out = torch.empty((wl.T, wl.Hq, wl.D), dtype=torch.float32, device=DEV)
    lse = torch.empty((wl.T, wl.Hq), dtype=torch.float32, device=DEV)
    with pytest.raises(lib.SmqaError, match="scratch"):
        lib.decode_step_noalloc(L, wl.qI, wl.w, wl.kI, wl.kscale, wl.cand, wl.q, wl.kv_codes, wl.kv_e8m0,
                                wl.kv_rowscale, wl.swa, wl.swa_scale, wl.swa_pos0, wl.swa_clip, wl.k,
                                wl.sm_scale, out, lse)
