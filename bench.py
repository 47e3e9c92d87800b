#!/usr/bin/env python3
"""Benchmark of the sparse-MQA decode step on one MI355X.

One step = one decode_step call over the whole batch: indexer scoring of every
context position, top-k selection and sparse MQA attention over the selected FP4
latent rows plus the FP8 window (the three stages of the method, in one call).
Inputs are the seeded synthetic workloads of ``synth`` (already resident in HBM
when timing starts).  Metric: context positions scored per second (higher is
better) and microseconds per step, at 8K context (decode_8k, the primary line)
and at 512K context (decode_512k, reported alongside).

The step is timed three ways: eager (one C-ABI call per step from Python), as a
replayed HIP graph of one call, and as a replayed graph of 10 consecutive calls
(the GPU-side steady state of a captured decode, no host work between steps);
graph outputs are checked bitwise against the eager step first.  ``value`` uses
the fastest.  Per-stage kernel
time comes from HIP events around repeated calls of each stage's entry point
on the same stream.  ``cpu_baseline`` times the fp64 CPU oracle on a bounded
sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--workload decode_8k] [--also decode_512k]
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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_8k")
    ap.add_argument("--also", default="decode_512k", help="comma list of extra workloads ('' = none)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--stage-only", default="", help="time only this stage entry point (profiling)")
    return ap.parse_args()


# ---------------------------------------------------------------- algorithmic work per stage

def work(wl):
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
    return J, out


# kernels behind each stage's entry point (what rocprofv3 lists for it)
STAGE_KERNELS = {
    "score": "score_kernel | score_stream_kernel (one query per sequence, long rows)",
    "topk": "topk_small_kernel (rows <= 16384) | topk_zero/hist/collect/finish_kernel",
    "attend": "sd::attend_kernel (dimension split; lat::/thr:: for other head counts and widths) "
              "+ attend_merge_kernel (split partials)",
}
TRAFFIC_MD = os.path.join(ROOT, "profiles", "pmc_traffic.md")
SOURCES = {"score": ["score.hip"], "topk": ["topk.hip"], "attend": ["attend.hip", "attend_sd.hip"]}


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


# ---------------------------------------------------------------- GPU measurement

def measure(name, steps, warmup, use_graph, stage_only="", fp8_baseline=True):
    import torch
    import synth
    import fp8_kv_cache_sparse_amd as smqa

    wl = synth.generate(name, seed=0, device="cuda")
    J, w = work(wl)
    L = smqa.Batch(wl.seq_start, wl.q_start, wl.q_pos, wl.max_ctx)
    dev = wl.q.device
    out = torch.empty((wl.T, wl.Hq, wl.D), dtype=torch.float32, device=dev)
    lse = torch.empty((wl.T, wl.Hq), dtype=torch.float32, device=dev)
    idx = torch.empty((wl.T, wl.k), dtype=torch.int32, device=dev)
    n_cand = 0 if wl.cand is None else wl.cand.shape[1]
    ws = torch.empty(smqa.decode_step_workspace_size(L, wl.k, n_cand, wl.W, wl.Hq, wl.D) + 256,
                     dtype=torch.uint8, device=dev)
    args = (L, wl.qI, wl.w, wl.kI, wl.kscale, wl.cand, wl.q, wl.kv_codes, wl.kv_e8m0, wl.kv_rowscale,
            wl.swa, wl.swa_scale, wl.swa_pos0, wl.swa_clip, wl.k, wl.sm_scale)

    def step():
        smqa.decode_step(*args, out=out, lse=lse, idx=idx, workspace=ws)

    # stage buffers
    scores = torch.empty((wl.T, max(wl.max_ctx, 1)), dtype=torch.float32, device=dev)
    idx2 = torch.empty_like(idx)
    out2, lse2 = torch.empty_like(out), torch.empty_like(lse)

    def st_score():
        smqa.sparse_mqa_score(L, wl.qI, wl.w, wl.kI, wl.kscale, wl.cand, scores=scores)

    def st_topk():
        smqa.topk_select(L, scores, wl.k, cand=wl.cand, idx=idx2, workspace=ws)

    def st_attend():
        smqa.sparse_mqa_attend(L, wl.q, wl.kv_codes, wl.kv_e8m0, wl.kv_rowscale, idx2, wl.swa,
                               wl.swa_scale, wl.swa_pos0, wl.swa_clip, wl.sm_scale, out=out2, lse=lse2,
                               workspace=ws)

    copy_src = torch.empty(256 << 20, dtype=torch.uint8, device=dev) if stage_only == "copy" else None
    copy_dst = torch.empty_like(copy_src) if copy_src is not None else None

    def st_copy():                                 # plain 256 MiB device copy: PMC calibration
        copy_dst.copy_(copy_src)

    stages = {"score": st_score, "topk": st_topk, "attend": st_attend}
    if stage_only == "copy":
        stages["copy"] = st_copy
    if stage_only == "attend_nvfp4":
        wlns = synth.with_nvfp4_kv(wl)
        stages["attend_nvfp4"] = lambda: smqa.sparse_mqa_attend_nvfp4(
            L, wl.q, wlns.kv_nv_codes, wlns.kv_nv_scales, wl.kv_rowscale, wlns.kv_nv_global, idx2,
            wl.swa, wl.swa_scale, wl.swa_pos0, wl.swa_clip, wl.sm_scale, out=out2, lse=lse2,
            workspace=ws)
    if stage_only == "attend_fp8kv":
        wl8s = synth.with_fp8_kv(wl)
        stages["attend_fp8kv"] = lambda: smqa.sparse_mqa_attend_fp8kv(
            L, wl.q, wl8s.kv_fp8, wl8s.kv_fp8_scale, idx2, wl.swa, wl.swa_scale, wl.swa_pos0,
            wl.swa_clip, wl.sm_scale, out=out2, lse=lse2, workspace=ws)
    if stage_only:
        fn = stages[stage_only]
        st_score()
        st_topk()
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        return {"workload": name, "stage_only": stage_only}

    print(f"[bench] {name}: warmup", file=sys.stderr, flush=True)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ref_out, ref_lse, ref_idx = out.clone(), lse.clone(), idx.clone()

    print(f"[bench] {name}: eager x{steps}", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    eager_s = (time.perf_counter() - t0) / steps

    graph_s = None
    chain_s = None
    graph_ok = None
    if use_graph:
        try:
            g = torch.cuda.CUDAGraph()
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                step()
            torch.cuda.current_stream().wait_stream(s)
            torch.cuda.synchronize()
            with torch.cuda.graph(g):
                step()
            torch.cuda.synchronize()
            graph_ok = True
            for _ in range(3):                     # every replay must reproduce the eager result
                out.zero_()
                g.replay()
                torch.cuda.synchronize()
                graph_ok &= bool(torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
                                 and torch.equal(idx, ref_idx))
            if graph_ok:
                print(f"[bench] {name}: graph x{steps}", file=sys.stderr, flush=True)
                for _ in range(warmup):
                    g.replay()
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                for _ in range(steps):
                    g.replay()
                torch.cuda.synchronize()
                graph_s = (time.perf_counter() - t0) / steps
                # GPU-side steady state: G consecutive steps in one graph, as inside a captured
                # decode of a whole model (no host work between the steps)
                G = max(1, min(10, steps))
                gc = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gc):
                    for _ in range(G):
                        step()
                torch.cuda.synchronize()
                out.zero_()
                gc.replay()
                torch.cuda.synchronize()
                graph_ok &= bool(torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
                                 and torch.equal(idx, ref_idx))
                reps = max(1, steps // G)
                print(f"[bench] {name}: graph of {G} steps x{reps}", file=sys.stderr, flush=True)
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                for _ in range(reps):
                    gc.replay()
                torch.cuda.synchronize()
                chain_s = (time.perf_counter() - t0) / (reps * G)
        except Exception as e:  # graph capture unavailable: report eager only
            print(f"[bench] graph capture failed: {e}", file=sys.stderr, flush=True)
            graph_ok = False

    # per-stage time with HIP events on the launch stream: each stage's entry point is
    # captured `steps` times into one graph (no host gaps between launches), replayed once
    st_us = {}
    st_score()
    st_topk()
    torch.cuda.synchronize()

    def timed_us(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if use_graph and graph_ok:
            gs = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gs):
                for _ in range(steps):
                    fn()
            torch.cuda.synchronize()
            gs.replay()
            torch.cuda.synchronize()
            best = None
            for _ in range(3):                     # the fastest of three timed replays
                e0.record()
                gs.replay()
                e1.record()
                torch.cuda.synchronize()
                t_ms = e0.elapsed_time(e1)
                best = t_ms if best is None else min(best, t_ms)
        else:
            e0.record()
            for _ in range(steps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            best = e0.elapsed_time(e1)
        return best * 1e3 / steps

    for nm, fn in stages.items():
        print(f"[bench] {name}: stage {nm} x{steps}", file=sys.stderr, flush=True)
        st_us[nm] = timed_us(fn)

    # the same attention over an FP8 global cache (E4M3 rows + row scale, the format the FP4
    # cache replaces) and over the NVFP4 layout, on the same selection: what the formats cost
    fp8kv = None
    if fp8_baseline and wl.Hq % 32 == 0 and wl.D <= 1664:
        print(f"[bench] {name}: FP8-cache attention x{steps}", file=sys.stderr, flush=True)
        wl8 = synth.with_fp8_kv(wl)
        torch.cuda.synchronize()

        def st_attend8():
            smqa.sparse_mqa_attend_fp8kv(L, wl.q, wl8.kv_fp8, wl8.kv_fp8_scale, idx2, wl.swa,
                                         wl.swa_scale, wl.swa_pos0, wl.swa_clip, wl.sm_scale,
                                         out=out2, lse=lse2, workspace=ws)
        us8 = timed_us(st_attend8)
        del wl8
        print(f"[bench] {name}: NVFP4-cache attention x{steps}", file=sys.stderr, flush=True)
        wln = synth.with_nvfp4_kv(wl)
        torch.cuda.synchronize()

        def st_attend_nv():
            smqa.sparse_mqa_attend_nvfp4(L, wl.q, wln.kv_nv_codes, wln.kv_nv_scales, wl.kv_rowscale,
                                         wln.kv_nv_global, idx2, wl.swa, wl.swa_scale, wl.swa_pos0,
                                         wl.swa_clip, wl.sm_scale, out=out2, lse=lse2, workspace=ws)
        usn = timed_us(st_attend_nv)
        del wln
        # MegaAttention's fused form on the MX cache: query RoPE (64 rotary dims), the same
        # attention, inverse RoPE and per-row FP8 output in one call
        fused_us = None
        if wl.D >= 64:
            R = 32
            th = torch.arange(wl.T * R, device=dev, dtype=torch.float32).view(wl.T, R) * 0.001
            rc, rsn = th.cos().contiguous(), th.sin().contiguous()
            o8 = torch.empty((wl.T, wl.Hq, wl.D), dtype=torch.uint8, device=dev)
            osc = torch.empty((wl.T, wl.Hq), dtype=torch.float32, device=dev)
            wsf = torch.empty(smqa.load().smqa_attend_fused_workspace_size(L.ref, wl.k, wl.W, wl.Hq, wl.D)
                              + 256, dtype=torch.uint8, device=dev)
            print(f"[bench] {name}: fused RoPE/FP8 attention x{steps}", file=sys.stderr, flush=True)

            def st_fused():
                smqa.sparse_mqa_attend_fused(L, wl.q, rc, rsn, wl.kv_codes, wl.kv_e8m0, wl.kv_rowscale,
                                             idx2, wl.swa, wl.swa_scale, wl.swa_pos0, wl.swa_clip,
                                             wl.sm_scale, out_fp8=o8, out_scale=osc, want_out=False,
                                             lse=lse2, workspace=wsf)
            fused_us = round(timed_us(st_fused), 2)
        rs = 4 if wl.kv_rowscale is not None else 0
        fp8kv = {"attend_us": {"mx_fp4": round(st_us["attend"], 2), "nvfp4": round(usn, 2),
                               "fp8": round(us8, 2)},
                 "fp8_over_mx_fp4_time": round(us8 / st_us["attend"], 3),
                 "nvfp4_over_mx_fp4_time": round(usn / st_us["attend"], 3),
                 "global_row_bytes": {"mx_fp4": wl.D // 2 + wl.D // 32 + rs,
                                      "nvfp4": wl.D // 2 + wl.D // 16 + rs, "fp8": wl.D + 4},
                 "kernel": "attend: sd::attend_kernel<D, F> (F = MX FP4 / NVFP4 / FP8 rows in "
                           "16-row tiles) + attend_merge_kernel",
                 "fused_rope_fp8_us": fused_us,
                 "fused_kernel": "sd::attend_kernel<D, MX> with query RoPE + attend_fused_epilogue_kernel "
                                 "(inverse RoPE, E4M3 output)"}
    dom = max(st_us, key=st_us.get)
    best_s = min(x for x in (eager_s, graph_s, chain_s) if x)
    res = {
        "workload": name, "T": wl.T, "B": wl.B, "scored_positions": J,
        "us_per_step": round(best_s * 1e6, 2),
        "us_per_step_eager": round(eager_s * 1e6, 2),
        "us_per_step_graph": None if graph_s is None else round(graph_s * 1e6, 2),
        "us_per_step_graph_chain": None if chain_s is None else round(chain_s * 1e6, 2),
        "graph_replay_matches_eager": graph_ok,
        "tokens_scored_per_s": J / best_s,
        "stage_us": {k: round(v, 2) for k, v in st_us.items()},
        "stage_roofline": {k: roofline(k, w[k], st_us[k] * 1e-6, name) for k in st_us},
        "global_cache_formats": fp8kv,
        "roofline": roofline(dom, w[dom], st_us[dom] * 1e-6, name),
        "config": dict(wl.meta["params"], lengths=(wl.meta["lengths"] if wl.B <= 8 else
                                                  [min(wl.meta["lengths"]), max(wl.meta["lengths"])])),
    }
    del wl
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------- CPU oracle baseline

def cpu_baseline(name, seconds):
    import numpy as np
    import torch
    import synth
    from oracle import ref

    wl = synth.generate(name, seed=0, device="cpu")
    J, _ = work(wl)
    a = {n: (None if getattr(wl, n) is None else getattr(wl, n).numpy())
         for n in ("seq_start", "q_start", "q_pos", "qI", "w", "kI", "kscale", "kv_codes", "kv_e8m0",
                   "kv_rowscale", "swa", "swa_scale", "swa_pos0", "swa_clip")}
    a["q"] = wl.q.view(torch.int16).numpy().view(np.uint16)
    a.update(k=wl.k, W=wl.W, sm_scale=wl.sm_scale)
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count()
    reps = 0
    t0 = time.perf_counter()
    while True:
        ref.decode_step(a)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": J * reps / el, "unit": UNIT, "cores": cores, "kind": "oracle",
            "sample": f"{reps} full fp64 oracle decode steps of {name} ({J} scored positions each), "
                      f"{el:.1f} s", "s_per_step": el / reps}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (the method's "
              f"multi-GPU sharding is described, not built)", file=sys.stderr)
        sys.exit(2)
    import torch
    import fp8_kv_cache_sparse_amd as smqa
    smqa.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.stage_only:
        measure(args.workload, args.steps, args.warmup, False, args.stage_only)
        print(json.dumps({"stage_only": args.stage_only, "workload": args.workload}))
        return
    main_res = measure(args.workload, args.steps, args.warmup, not args.no_graph)
    extra = {}
    for nm in [x for x in args.also.split(",") if x]:
        extra[nm] = measure(nm, args.steps, args.warmup, not args.no_graph)
    cpu = None if args.no_cpu else cpu_baseline(args.workload, args.cpu_seconds)
    cfg = main_res["config"]
    line = {
        "metric": METRIC,
        "value": main_res["tokens_scored_per_s"],
        "unit": UNIT,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["us_per_step"] / 1e3,
        "us_per_step": main_res["us_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16/fp16 MFMA, fp32 accumulate",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": cfg["B"], "ctx": cfg["lengths"],
                   "indexer": f"{cfg['Hi']}x{cfg['Di']} e4m3", "k": cfg["k"],
                   "attention": f"{cfg['Hq']} heads x {cfg['D']} latent (e2m1 + e8m0/32"
                                f"{' + f32 row scale' if cfg['rowscale'] else ''})",
                   "window": cfg["W"], "parallelism": "none (1 GPU)"},
        "roofline": main_res["roofline"],
        "cpu_baseline": cpu,
        "detail": main_res,
        "also": extra,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
