#!/usr/bin/env python3
"""Benchmark of the sparse-MQA decode step on one MI355X.

One step = one decode_step call over the whole batch: indexer scoring of every
context position, top-k selection and sparse MQA attention over the selected FP4
latent rows plus the FP8 window (the three stages of the method, in one call).
Inputs are the seeded synthetic workloads of ``synth``, resident in HBM when
timing starts.

Timing protocol (every figure is per call, on the stream the library launches on):
  * cold: before each rep a kernel reads 512 MiB (twice the 256 MB Infinity Cache, far
    more than the L2s) outside the timed region, then HIP events bracket the call;
    median, p10 and p90 over the reps;
  * warm (labelled as such): a captured HIP graph of 10 consecutive steps replayed
    back to back, the GPU-side steady state of a captured decode loop.
The headline line is the decode_8k workload (batch 1 at 8K context): ``value`` is
context positions scored per second over the median cold step (the whole hot path),
``ms_per_step`` that median.  The same protocol runs per stage (score, top-k,
attention), for candidate-mode scoring (16,384 candidates per query, the pages'
late-indexer comparison) and for the other workloads (``--also``).  ``cpu_baseline``
times the fp64 CPU oracle on the same bytes.

    python bench.py [--steps K] [--warmup W] [--workload decode_8k]
                    [--also decode_512k,ragged_b32,replay_h100k]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "context tokens scored/s and decode-attention us/step at 8K and 512K ctx, 1 GPU"
UNIT = "context tokens scored/s"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"fp8": 5000.0, "bf16": 2500.0}
FLUSH_BYTES = 512 << 20
# cold reps per workload: at least 50 for the small batches, 20 for the large ones
MIN_REPS = {"tiny": 50, "decode_8k": 50, "ragged_b32": 50, "decode_512k": 20, "replay_h100k": 20}
N_CAND = 16384


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_8k")
    ap.add_argument("--also", default="decode_512k,ragged_b32,replay_h100k",
                    help="comma list of extra workloads ('' = none)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--stage-only", default="", help="run only this stage entry point (profiling)")
    ap.add_argument("--flush", default="read", choices=("read", "write"),
                    help="cold-cache flush before each rep: read or write 512 MiB")
    return ap.parse_args()


# ---------------------------------------------------------------- algorithmic work per stage

def work(wl, n_cand=None):
    """Algorithmic bytes / flops of each stage for one step (what the method must move/compute)."""
    import numpy as np
    lengths = np.array(wl.meta["lengths"], dtype=np.int64)
    q_seq = np.array(wl.meta["q_seq"], dtype=np.int64)
    q_pos = wl.q_pos.cpu().numpy().astype(np.int64)
    scored = np.minimum(q_pos, lengths[q_seq] - 1) + 1
    J = int(scored.sum())
    keys_read = int(np.minimum(lengths, np.array([scored[q_seq == b].max() if (q_seq == b).any() else 0
                                                   for b in range(wl.B)])).sum())
    T, k, Hq, D, W, Hi, Di = wl.T, wl.k, wl.Hq, wl.D, wl.W, wl.Hi, wl.Di
    row_b = D // 2 + D // 32 + (4 if wl.kv_rowscale is not None else 0)
    # visible window rows per query
    lo = np.maximum(q_pos - W + 1, 0)
    if wl.swa_clip is not None:
        lo = np.maximum(lo, wl.swa_clip.cpu().numpy())
    pos0 = wl.swa_pos0.cpu().numpy()[q_seq]
    vis = np.clip(np.minimum(q_pos, pos0 + W - 1) - np.maximum(lo, pos0) + 1, 0, W)
    sel = np.minimum(scored, k)
    out = {
        "score": dict(bytes=keys_read * Di + J * 4, flops=2 * Hi * Di * J, mfma="bf16"),
        "topk": dict(bytes=J * 4 + T * k * 4, flops=0, mfma=None),
        "attend": dict(bytes=int(sel.sum()) * (row_b + 4) + wl.B * W * D + T * Hq * (D * 2 + D * 4 + 4),
                       flops=int(4 * Hq * D * (sel + vis).sum()), mfma="bf16"),
    }
    if n_cand:
        # candidate mode: each query reads its candidate list and those keys, writes n_cand scores
        out["score_cand"] = dict(bytes=T * n_cand * (4 + Di + 4), flops=2 * Hi * Di * T * n_cand, mfma="bf16")
    return J, out


# kernels behind each stage's entry point (what rocprofv3 lists for it)
STAGE_KERNELS = {
    "score": "score_kernel | score_stream_kernel (one query per sequence, long rows)",
    "score_cand": "score_kernel (candidate lists)",
    "topk": "topk_small_kernel (rows <= 16384) | topk_zero/hist/collect/finish_kernel",
    "attend": "sd::attend_kernel (dimension split; lat::/thr:: for other head counts and widths) "
              "+ attend_merge_kernel (split partials)",
}
TRAFFIC_MD = os.path.join(ROOT, "profiles", "pmc_traffic.md")
SOURCES = {"score": ["score.hip"], "score_cand": ["score.hip"], "topk": ["topk.hip"],
           "attend": ["attend.hip", "attend_sd.hip"]}


def source_digest(stage):
    import hashlib
    h = hashlib.sha256()
    for f in SOURCES[stage] + ["common.h"]:
        with open(os.path.join(ROOT, "fp8_kv_cache_sparse_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(stage, workload):
    """HBM bytes per call of `stage` from the committed rocprofv3 --pmc summary (FETCH_SIZE and
    WRITE_SIZE, scaled by the copy-kernel calibration), or None when no summary exists or the
    stage's source has changed since the counters were taken."""
    if not os.path.exists(TRAFFIC_MD):
        return None
    for line in open(TRAFFIC_MD):
        if not line.startswith("traffic:"):
            continue
        rec = json.loads(line[len("traffic:"):])
        if rec.get("stage") == stage and rec.get("workload") == workload:
            if rec.get("source_digest") != source_digest(stage):
                return None
            return rec["hbm_bytes_per_call"]
    return None


def roofline(stage, w, seconds, workload=None):
    """Roofline record of one stage: achieved = algorithmic work per call / measured time per
    call, against the MFMA peak when the stage's algorithmic flop/byte exceeds the ridge of
    its MFMA type, else against HBM."""
    ai = w["flops"] / max(w["bytes"], 1)
    traffic = measured_traffic(stage, workload) if workload else None
    if w["mfma"] and ai > MFMA_PEAK_TFLOPS[w["mfma"]] * 1e12 / (HBM_PEAK_GBS * 1e9):
        ach = w["flops"] / seconds / 1e12
        peak = MFMA_PEAK_TFLOPS[w["mfma"]]
        return {"kernel": f"{stage}: {STAGE_KERNELS[stage]}", "bound": "mfma", "achieved": round(ach, 3),
                "peak": peak, "unit": "TFLOP/s", "frac": round(ach / peak, 4), "traffic": traffic,
                "algorithmic_flops": w["flops"], "algorithmic_bytes": w["bytes"]}
    ach = w["bytes"] / seconds / 1e9
    return {"kernel": f"{stage}: {STAGE_KERNELS[stage]}", "bound": "hbm", "achieved": round(ach, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic,
            "algorithmic_bytes": w["bytes"], "algorithmic_flops": w["flops"]}


def stats(us):
    """median / p10 / p90 / mean of per-rep times in microseconds."""
    import numpy as np
    a = np.asarray(us, dtype=np.float64)
    return {"median": round(float(np.median(a)), 2), "p10": round(float(np.percentile(a, 10)), 2),
            "p90": round(float(np.percentile(a, 90)), 2), "mean": round(float(a.mean()), 2), "reps": int(a.size)}


# ---------------------------------------------------------------- GPU measurement

class Timer:
    """Per-call HIP-event timing on torch's current stream (the stream every entry point of
    the binding launches on), cold or warm.  Cold: before each rep a kernel reads (default)
    or writes a 512 MiB buffer.  Reading evicts the call's data from the L2s and the 256 MB
    Infinity Cache and leaves only clean lines; a writing flush leaves up to 256 MB of
    dirty lines that are written back while the next timed call runs, which charges that
    call for the flush's own traffic."""

    def __init__(self, dev, mode="read"):
        import torch
        self.torch = torch
        self.mode = mode
        self.flush_buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)

    def flush(self):
        if self.mode == "write":
            self.flush_buf.fill_(1.0)
        else:
            self.flush_buf.sum()

    def cold(self, fn, reps, warmup=2):
        torch = self.torch
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for e0, e1 in ev:
            self.flush()
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        return [e0.elapsed_time(e1) * 1e3 for e0, e1 in ev]

    def warm_graph(self, fn, steps=10, reps=5):
        """Mean per-call time of a captured graph of `steps` back-to-back calls (warm)."""
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for _ in range(steps):
                fn()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (reps * steps), g


# launch shapes tried for the streaming-read reference: (workgroups of 256 threads, 16-byte
# loads in flight per thread); about 32 KB in flight per CU reads fastest on MI355X
STREAM_READ_SHAPES = ((256, 8), (512, 4), (1024, 2), (1024, 1), (2048, 1))


def hbm_reference(timer, dev, sizes=()):
    """What plain streaming kernels reach on this machine (cold, GB/s): a 1 GiB device-to-device
    copy (bytes read + written), a 1 GiB read by torch's sum, and the same 1 GiB read by the
    streaming-read reference kernel (libsmqa_bench.so) at its best launch shape.  The same
    kernel also reads each byte count in `sizes` (an HBM-bound stage's algorithmic bytes), at
    the best of its launch shapes for that count, so the stage can be set against a plain
    read of exactly its bytes (launch ramp and tail included)."""
    import ctypes
    import torch
    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    cp = stats(timer.cold(lambda: dst.copy_(src), 10))["median"]
    rd = stats(timer.cold(lambda: src.sum(), 10))["median"]
    res = {"copy_GBs": round(2 * (1 << 30) / (cp * 1e-6) / 1e9, 1),
           "read_GBs": round((1 << 30) / (rd * 1e-6) / 1e9, 1)}
    lib_path = os.path.join(ROOT, "fp8_kv_cache_sparse_amd", "libsmqa_bench.so")
    if os.path.exists(lib_path):
        lib = ctypes.CDLL(lib_path)
        fn = lib.smqa_bench_stream_read
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                       ctypes.c_void_p]
        out = torch.empty(max(g for g, _ in STREAM_READ_SHAPES) * 256, dtype=torch.int32, device=dev)
        stream = torch.cuda.current_stream().cuda_stream

        def best_read(nbytes):
            best = None
            for grid, depth in STREAM_READ_SHAPES:
                def call():
                    if fn(src.data_ptr(), nbytes, out.data_ptr(), grid, depth, stream) != 0:
                        raise RuntimeError("smqa_bench_stream_read failed")
                us = stats(timer.cold(call, 10))["median"]
                gbs = nbytes / (us * 1e-6) / 1e9
                if best is None or gbs > best[0]:
                    best = (gbs, grid, depth, us)
            return best

        best = best_read(1 << 30)
        res["stream_read_GBs"] = round(best[0], 1)
        res["stream_read_shape"] = {"workgroups": best[1], "loads_in_flight_per_thread": best[2]}
        same = {}
        for nbytes in sorted({min(int(n) // 16 * 16, 1 << 30) for n in sizes if n >= 16}):
            b = best_read(nbytes)
            same[str(nbytes)] = {"us": round(b[3], 2), "GBs": round(b[0], 1),
                                 "shape": {"workgroups": b[1], "loads_in_flight_per_thread": b[2]}}
        if same:
            res["stream_read_same_bytes"] = same
    del src, dst
    return res


def measure(name, steps, warmup, timer, primary=False, stage_only=""):
    import torch
    import synth
    import fp8_kv_cache_sparse_amd as smqa

    reps = steps if primary else max(steps, MIN_REPS.get(name, 20))
    reps_stage = max(steps, MIN_REPS.get(name, 20))
    wl = synth.generate(name, seed=0, device="cuda")
    J, w = work(wl, N_CAND if wl.cand is None and wl.swa_clip is None else None)
    L = smqa.Batch(wl.seq_start, wl.q_start, wl.q_pos, wl.max_ctx)
    dev = wl.q.device
    out = torch.empty((wl.T, wl.Hq, wl.D), dtype=torch.float32, device=dev)
    lse = torch.empty((wl.T, wl.Hq), dtype=torch.float32, device=dev)
    idx = torch.empty((wl.T, wl.k), dtype=torch.int32, device=dev)
    ws = torch.empty(smqa.decode_step_workspace_size(L, wl.k, 0, wl.W, wl.Hq, wl.D) + 256,
                     dtype=torch.uint8, device=dev)
    args = (L, wl.qI, wl.w, wl.kI, wl.kscale, wl.cand, wl.q, wl.kv_codes, wl.kv_e8m0, wl.kv_rowscale,
            wl.swa, wl.swa_scale, wl.swa_pos0, wl.swa_clip, wl.k, wl.sm_scale)

    def step():
        smqa.decode_step(*args, out=out, lse=lse, idx=idx, workspace=ws)

    scores = torch.empty((wl.T, max(wl.max_ctx, 1)), dtype=torch.float32, device=dev)
    idx2 = torch.empty_like(idx)
    out2, lse2 = torch.empty_like(out), torch.empty_like(lse)
    ws2 = torch.empty_like(ws)

    def st_score():
        smqa.sparse_mqa_score(L, wl.qI, wl.w, wl.kI, wl.kscale, wl.cand, scores=scores)

    def st_topk():
        smqa.topk_select(L, scores, wl.k, cand=wl.cand, idx=idx2, workspace=ws2)

    def st_attend():
        smqa.sparse_mqa_attend(L, wl.q, wl.kv_codes, wl.kv_e8m0, wl.kv_rowscale, idx2, wl.swa,
                               wl.swa_scale, wl.swa_pos0, wl.swa_clip, wl.sm_scale, out=out2, lse=lse2,
                               workspace=ws2)

    stages = {"score": st_score, "topk": st_topk, "attend": st_attend}
    if stage_only:
        # profiling: prepare the inputs, then `steps` calls of one entry point (cold)
        if stage_only == "copy":
            src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
            dst = torch.empty_like(src)
            stages["copy"] = lambda: dst.copy_(src)
        if stage_only == "decode_step":
            stages["decode_step"] = step
        if stage_only == "score_fp8mma":
            sc8 = torch.empty_like(scores)
            stages["score_fp8mma"] = lambda: smqa.sparse_mqa_score_fp8mma(L, wl.qI, wl.w, wl.kI, wl.kscale,
                                                                         wl.cand, scores=sc8)
        st_score()
        st_topk()
        torch.cuda.synchronize()
        timer.cold(stages[stage_only], steps, warmup)
        return {"workload": name, "stage_only": stage_only}

    print(f"[bench] {name}: warmup + eager check", file=sys.stderr, flush=True)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ref_out, ref_lse, ref_idx = out.clone(), lse.clone(), idx.clone()

    print(f"[bench] {name}: cold steps x{reps}", file=sys.stderr, flush=True)
    step_us = timer.cold(step, reps, warmup=0)
    ok = bool(torch.equal(out, ref_out) and torch.equal(lse, ref_lse) and torch.equal(idx, ref_idx))

    print(f"[bench] {name}: warm graph of 10 steps", file=sys.stderr, flush=True)
    warm_us, g = timer.warm_graph(step)
    out.zero_()
    g.replay()
    torch.cuda.synchronize()
    ok &= bool(torch.equal(out, ref_out) and torch.equal(lse, ref_lse) and torch.equal(idx, ref_idx))
    del g

    st_us = {}
    st_score()
    st_topk()
    torch.cuda.synchronize()
    for nm, fn in stages.items():
        print(f"[bench] {name}: stage {nm} x{reps_stage} cold", file=sys.stderr, flush=True)
        st_us[nm] = timer.cold(fn, reps_stage)

    # candidate-mode scoring (late indexer layers: a fixed list of 16K candidate positions per
    # query) next to dense scoring of the same batch: the pages' sparse-logits comparison
    cand = None
    if wl.cand is None and wl.swa_clip is None:
        wlc = synth.generate(name, seed=0, device="cuda", n_cand=N_CAND)
        Lc = smqa.Batch(wlc.seq_start, wlc.q_start, wlc.q_pos, wlc.max_ctx)
        sc_c = torch.empty((wlc.T, N_CAND), dtype=torch.float32, device=dev)

        def st_cand():
            smqa.sparse_mqa_score(Lc, wlc.qI, wlc.w, wlc.kI, wlc.kscale, wlc.cand, scores=sc_c)
        print(f"[bench] {name}: candidate scoring x{reps_stage} cold", file=sys.stderr, flush=True)
        cu = timer.cold(st_cand, reps_stage)
        st_us["score_cand"] = cu
        cand = {"n_cand": N_CAND, "score_us": stats(cu),
                "dense_over_candidate_time": round(stats(st_us["score"])["median"] / stats(cu)["median"], 2)}
        del wlc, sc_c

    # the indexer contraction on the FP8 matrix cores (sparse_mqa_score_fp8mma) beside the
    # bf16 form: cold time, roofline against the FP8 peak, and its largest relative
    # difference from the bf16 form's scores (which are exact products with fp32 sums)
    score_forms = None
    if wl.Di == 128:
        scores8 = torch.empty_like(scores)

        def st_score8():
            smqa.sparse_mqa_score_fp8mma(L, wl.qI, wl.w, wl.kI, wl.kscale, wl.cand, scores=scores8)

        print(f"[bench] {name}: FP8 matrix-core scoring x{reps_stage} cold", file=sys.stderr, flush=True)
        u8 = timer.cold(st_score8, reps_stage)
        st_score()
        st_score8()
        torch.cuda.synchronize()
        fin = torch.isfinite(scores)
        rel = ((scores8 - scores).abs() / scores.abs().clamp_min(1e-30))[fin]
        w8 = dict(w["score"], mfma="fp8")
        score_forms = {
            "bf16_us": stats(st_us["score"]), "fp8_mfma_us": stats(u8),
            "fp8_over_bf16_time": round(stats(u8)["median"] / stats(st_us["score"])["median"], 3),
            "max_rel_diff_fp8_vs_bf16": float(rel.max()) if rel.numel() else 0.0,
            "fp8_roofline": roofline("score", w8, stats(u8)["median"] * 1e-6),
        }
        del scores8

    # the same attention over the FP8 and NVFP4 global caches and in MegaAttention's fused
    # form, on the same selection (cold)
    formats = None
    if wl.Hq % 32 == 0 and wl.D <= 1664:
        fmt_us = {"mx_fp4": stats(st_us["attend"])}
        wl8 = synth.with_fp8_kv(wl)
        print(f"[bench] {name}: FP8-cache attention", file=sys.stderr, flush=True)
        fmt_us["fp8"] = stats(timer.cold(lambda: smqa.sparse_mqa_attend_fp8kv(
            L, wl.q, wl8.kv_fp8, wl8.kv_fp8_scale, idx2, wl.swa, wl.swa_scale, wl.swa_pos0, wl.swa_clip,
            wl.sm_scale, out=out2, lse=lse2, workspace=ws2), reps_stage))
        del wl8
        wln = synth.with_nvfp4_kv(wl)
        print(f"[bench] {name}: NVFP4-cache attention", file=sys.stderr, flush=True)
        fmt_us["nvfp4"] = stats(timer.cold(lambda: smqa.sparse_mqa_attend_nvfp4(
            L, wl.q, wln.kv_nv_codes, wln.kv_nv_scales, wl.kv_rowscale, wln.kv_nv_global, idx2, wl.swa,
            wl.swa_scale, wl.swa_pos0, wl.swa_clip, wl.sm_scale, out=out2, lse=lse2, workspace=ws2),
            reps_stage))
        del wln
        # Q.K^T on the scaled matrix cores with the query quantised to MXFP8 (row f4)
        print(f"[bench] {name}: MXFP8-query scaled-MFMA attention", file=sys.stderr, flush=True)
        fmt_us["mx_fp4_mxfp8_query"] = stats(timer.cold(lambda: smqa.sparse_mqa_attend_mxfp8q(
            L, wl.q, wl.kv_codes, wl.kv_e8m0, wl.kv_rowscale, idx2, wl.swa, wl.swa_scale, wl.swa_pos0,
            wl.swa_clip, wl.sm_scale, out=out2, lse=lse2, workspace=ws2), reps_stage))
        R = 32
        th = torch.arange(wl.T * R, device=dev, dtype=torch.float32).view(wl.T, R) * 0.001
        rc, rsn = th.cos().contiguous(), th.sin().contiguous()
        o8 = torch.empty((wl.T, wl.Hq, wl.D), dtype=torch.uint8, device=dev)
        osc = torch.empty((wl.T, wl.Hq), dtype=torch.float32, device=dev)
        print(f"[bench] {name}: fused RoPE/FP8 attention", file=sys.stderr, flush=True)
        fmt_us["fused_rope_fp8"] = stats(timer.cold(lambda: smqa.sparse_mqa_attend_fused(
            L, wl.q, rc, rsn, wl.kv_codes, wl.kv_e8m0, wl.kv_rowscale, idx2, wl.swa, wl.swa_scale,
            wl.swa_pos0, wl.swa_clip, wl.sm_scale, out_fp8=o8, out_scale=osc, want_out=False, lse=lse2,
            workspace=ws2), reps_stage))
        rs = 4 if wl.kv_rowscale is not None else 0
        m = fmt_us["mx_fp4"]["median"]
        formats = {"attend_us": fmt_us,
                   "fp8_over_mx_fp4_time": round(fmt_us["fp8"]["median"] / m, 3),
                   "nvfp4_over_mx_fp4_time": round(fmt_us["nvfp4"]["median"] / m, 3),
                   "mxfp8_query_over_mx_fp4_time": round(fmt_us["mx_fp4_mxfp8_query"]["median"] / m, 3),
                   "mxfp8_query_roofline": roofline("attend", w["attend"],
                                                    fmt_us["mx_fp4_mxfp8_query"]["mean"] * 1e-6),
                   "global_row_bytes": {"mx_fp4": wl.D // 2 + wl.D // 32 + rs,
                                        "nvfp4": wl.D // 2 + wl.D // 16 + rs, "fp8": wl.D + 4}}

    step_st = stats(step_us)
    st_stats = {k: stats(v) for k, v in st_us.items()}
    # roofline figures divide algorithmic work by the mean per-call time (what a profiler's
    # average kernel duration reports)
    st_roof = {k: roofline(k, w[k], st_stats[k]["mean"] * 1e-6, name) for k in st_us if k in w}
    main_stages = ("score", "topk", "attend")
    dom = max(main_stages, key=lambda k: st_stats[k]["median"])
    res = {
        "workload": name, "T": wl.T, "B": wl.B, "scored_positions": J,
        "step_us_cold": step_st,
        "step_us_warm_graph10": round(warm_us, 2),
        "outputs_match_eager": ok,
        "tokens_scored_per_s_step": J / (step_st["median"] * 1e-6),
        "tokens_scored_per_s_score_stage": J / (st_stats["score"]["median"] * 1e-6),
        "stage_us_cold": st_stats,
        "stage_roofline": st_roof,
        "candidate_scoring": cand,
        "score_forms": score_forms,
        "global_cache_formats": formats,
        "dominant_stage": dom,
        "roofline": st_roof[dom],
        "config": dict(wl.meta["params"], lengths=(wl.meta["lengths"] if wl.B <= 8 else
                                                  [min(wl.meta["lengths"]), max(wl.meta["lengths"])])),
    }
    del wl
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------- CPU oracle baseline

def cpu_info():
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas, threads = None, None
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            blas = f"{info[0].get('internal_api')} {info[0].get('version')}"
            threads = max(i.get("num_threads", 1) for i in info)
    except Exception:
        pass
    return model, blas, threads


def cu_clock_mhz():
    """Highest core (sclk) clock level of GPU 0 in MHz, from `rocm-smi -s` run as a child process,
    or None."""
    import re
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", "-s"], capture_output=True, text=True, timeout=30)
    except (OSError, subprocess.SubprocessError):
        return None
    txt = r.stdout
    i = txt.find("Supported sclk frequencies")
    if i < 0:
        return None
    j = txt.find("Supported", i + 10)
    vals = [float(v) for v in re.findall(r"(\d+(?:\.\d+)?)\s*Mhz", txt[i:j if j > 0 else None], flags=re.I)]
    return max(vals) if vals else None


def cpu_baseline(name, seconds):
    """The fp64 oracle's decode step on the same bytes the GPU run used (drawn on the GPU,
    copied to the host), repeated for about `seconds`."""
    import numpy as np
    import torch
    import synth
    from oracle import ref

    wl = synth.generate(name, seed=0, device="cuda").cpu()
    J, _ = work(wl)
    a = {n: (None if getattr(wl, n) is None else getattr(wl, n).numpy())
         for n in ("seq_start", "q_start", "q_pos", "qI", "w", "kI", "kscale", "kv_codes", "kv_e8m0",
                   "kv_rowscale", "swa", "swa_scale", "swa_pos0", "swa_clip")}
    a["q"] = wl.q.view(torch.int16).numpy().view(np.uint16)
    a.update(k=wl.k, W=wl.W, sm_scale=wl.sm_scale)
    model, blas, threads = cpu_info()
    reps = 0
    t0 = time.perf_counter()
    while True:
        ref.decode_step(a)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": J * reps / el, "unit": UNIT, "cores": threads or len(os.sched_getaffinity(0)),
            "kind": "oracle",
            "sample": f"{reps} full fp64 oracle decode steps of {name} on the GPU run's bytes "
                      f"({J} scored positions each), {el:.1f} s",
            "s_per_step": el / reps, "cpu_model": model, "blas": blas}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (the method's "
              f"multi-GPU sharding is described, not built)", file=sys.stderr)
        sys.exit(2)
    # the oracle's BLAS uses every core this process may run on
    os.environ.setdefault("OPENBLAS_NUM_THREADS", str(len(os.sched_getaffinity(0))))
    import torch
    import fp8_kv_cache_sparse_amd as smqa
    smqa.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    timer = Timer("cuda", args.flush)
    if args.stage_only:
        measure(args.workload, args.steps, args.warmup, timer, stage_only=args.stage_only)
        print(json.dumps({"stage_only": args.stage_only, "workload": args.workload}))
        return
    main_res = measure(args.workload, args.steps, args.warmup, timer, primary=True)
    extra = {}
    for nm in [x for x in args.also.split(",") if x and x != args.workload]:
        extra[nm] = measure(nm, args.steps, args.warmup, timer)
    hbm_rows = [r for res in [main_res, *extra.values()] for r in res.get("stage_roofline", {}).values()
                if r["bound"] == "hbm"]
    hbm_ref = hbm_reference(timer, "cuda", [r["algorithmic_bytes"] for r in hbm_rows])
    # HBM-bound stages also against the streaming read measured on this machine: of 1 GiB, and
    # of exactly the stage's algorithmic bytes
    if hbm_ref.get("stream_read_GBs"):
        same = hbm_ref.get("stream_read_same_bytes", {})
        for r in hbm_rows:
            r["frac_of_stream_read"] = round(r["achieved"] / hbm_ref["stream_read_GBs"], 4)
            ref = same.get(str(min(int(r["algorithmic_bytes"]) // 16 * 16, 1 << 30)))
            if ref:
                r["frac_of_same_bytes_read"] = round(r["achieved"] / ref["GBs"], 4)
    cpu = None if args.no_cpu else cpu_baseline(args.workload, args.cpu_seconds)
    cfg = main_res["config"]
    med = main_res["step_us_cold"]["median"]
    line = {
        "metric": METRIC,
        # context tokens scored per second of the score call (cold median); the whole
        # decode_step's rate and time are reported beside it
        "value": main_res["tokens_scored_per_s_score_stage"],
        "tokens_scored_per_s_step": main_res["tokens_scored_per_s_step"],
        "unit": UNIT,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": med / 1e3,
        "us_per_step": med,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16/fp16 MFMA, fp32 accumulate",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": cfg["B"], "ctx": cfg["lengths"],
                   "indexer": f"{cfg['Hi']}x{cfg['Di']} e4m3", "k": cfg["k"],
                   "attention": f"{cfg['Hq']} heads x {cfg['D']} latent (e2m1 + e8m0/32"
                                f"{' + f32 row scale' if cfg['rowscale'] else ''})",
                   "window": cfg["W"], "parallelism": "none (1 GPU)", "seed": 0,
                   "cu_clock_max_MHz": cu_clock_mhz(),
                   "timing": f"cold ({args.flush} of 512 MiB before each rep), median of per-call HIP events"},
        "roofline": main_res["roofline"],
        "cpu_baseline": cpu,
        "hbm_measured_GBs": hbm_ref,
        "detail": main_res,
        "also": extra,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
