"""Host-side pieces of bench.py (CPU only): the one-GPU contract and the algorithmic work
that the roofline figures divide by the measured time."""
import os
import subprocess
import sys

import numpy as np

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stdout + r.stderr


def test_work_closed_forms_for_decode():
    """Decode (one query per sequence at p = len - 1, no clip): J = sum of the lengths, each
    query selects min(len, k) rows and sees min(len, W) window rows."""
    wl = synth.generate("tiny", seed=0, B=3, lengths=(100, 700), k=256, W=128)
    J, w = bench.work(wl)
    lengths = np.array(wl.meta["lengths"])             # drawn from [100, 700]
    assert np.array_equal(wl.q_pos.numpy(), lengths - 1)
    assert J == lengths.sum()
    sel = np.minimum(lengths, wl.k)
    vis = np.minimum(lengths, wl.W)
    assert w["attend"]["flops"] == 4 * wl.Hq * wl.D * int((sel + vis).sum())
    assert w["score"]["flops"] == 2 * wl.Hi * wl.Di * J
    assert w["topk"]["bytes"] == 4 * J + 4 * wl.T * wl.k
    row = wl.D // 2 + wl.D // 32 + (4 if wl.kv_rowscale is not None else 0)
    assert w["attend"]["bytes"] == (int(sel.sum()) * (row + 4) + wl.B * wl.W * wl.D
                                    + wl.T * wl.Hq * (wl.D * 2 + wl.D * 4 + 4))


def test_work_counts_the_clipped_replay_window():
    """A replay chunk at p = H - n + i with the window clipped at s = H - n: query i sees
    i + 1 window rows and scores p + 1 positions."""
    H, n = 500, 16
    wl = synth.generate("tiny", seed=1, B=1, lengths=H, k=64, W=128, replay=(H, n))
    J, w = bench.work(wl)
    p = np.arange(H - n, H)
    assert J == int((p + 1).sum())
    vis = np.arange(1, n + 1)
    sel = np.minimum(p + 1, wl.k)
    assert w["attend"]["flops"] == 4 * wl.Hq * wl.D * int((sel + vis).sum())
