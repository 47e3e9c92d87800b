"""decode_step on dense short rows at D = 1664 takes the selection inside the attention kernel
(every workgroup of a query selects from the query's scores); it must give exactly what the
separate calls give: sparse_mqa_score, then topk_select on those scores, then
sparse_mqa_attend on that selection, bit for bit in the selection, the output and the LSE.
The cases cover ties across the k-th place (all scores equal), rows with fewer valid columns
than k (-1 padding), several queries of different lengths and a query position before the
end of its row."""
import pytest
import torch

import synth
from helpers import announce, gpu_attend, gpu_decode, gpu_score, gpu_topk

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _bits(x):
    return x.contiguous().view(torch.int32)


def _composed(lib, wl):
    S = gpu_score(lib, wl)
    r = gpu_topk(lib, wl, S)
    idx = r[0] if isinstance(r, tuple) else r
    out, lse = gpu_attend(lib, wl, idx)
    return out, lse, idx


CASES = [
    pytest.param(dict(), None, id="decode_8k"),
    pytest.param(dict(B=3, lengths=(100, 3000, 8192)), None, id="three-rows-one-shorter-than-k"),
    pytest.param(dict(B=2, lengths=(6000, 7000)), "ties", id="all-scores-equal"),
    pytest.param(dict(B=2, lengths=(8000, 8192)), "early", id="query-before-the-row-end"),
]


@pytest.mark.parametrize("kw,mode", CASES)
def test_decode_step_selection_in_attention_equals_the_separate_calls(lib, kw, mode):
    wl = synth.generate("decode_8k", seed=9, device=DEV, **kw)
    if mode == "ties":
        wl.qI.zero_()                      # every logit 0: every score 0, a tie across the k-th place
    if mode == "early":
        wl.q_pos[0] = 5000                 # positions 5001.. of the first row are not scored
    announce(f"decode_step selection in attention {kw} {mode}")
    out_c, lse_c, idx_c = _composed(lib, wl)
    out_d, lse_d, idx_d = gpu_decode(lib, wl)
    torch.cuda.synchronize()
    assert torch.equal(idx_d, idx_c)
    assert torch.equal(_bits(out_d), _bits(out_c))
    assert torch.equal(_bits(lse_d), _bits(lse_c))
    if mode == "ties":                     # ties go to the lowest columns
        n0 = int(wl.seq_start[1] - wl.seq_start[0])
        assert torch.equal(idx_d[0].cpu(), torch.arange(min(wl.k, n0), dtype=torch.int32))
    if mode == "early":
        sel = idx_d[0][idx_d[0] >= 0]
        assert int(sel.max()) <= 5000
