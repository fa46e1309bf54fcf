#!/usr/bin/env python3
"""Benchmark one denoising iteration of block-wise diffusion-LLM decoding on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]

A step is one whole iteration on synthetic inputs already resident in HBM:
dblk_attend (block queries over the dual KV cache), then
dblk_lmhead_confidence_commit (LM head, full-vocabulary softmax confidence and
argmax, and the threshold parallel decoder's commit step, which runs inside
the LM head's final merge where the shapes allow; bitwise the same as
dblk_lmhead_confidence followed by dblk_threshold_commit), back to back on one
stream, called through the C ABI.  W untimed warm-up steps, then K timed steps bracketed by device
synchronisation.  Prints ONE JSON line on stdout; progress goes to stderr.

Default workload: the LLaDA-MoE-7B-A1B-shaped block (batch 1, 16 heads x 128,
prefix 768 + block 64 + suffix 448, vocabulary 157184, threshold 0.9).

Every step starts from the workload's own tokens and mask: one pristine
copy per step is laid out in HBM before the timed region, so each commit
step decides on the generated mask rather than on one emptied by earlier
steps.

roofline: the LM head dominates (98% of the iteration's bytes at batch 1).
The duration of dblk_lmhead_confidence_commit (the LM-head kernel with the
commit step in its tail, or the LM head plus the commit kernel) is measured
with HIP events recorded on the launch stream around every call, in a second instrumented run of the same iterations right after
the timed region (an event between two kernels leaves the GPU idle for a few
microseconds, so the timed region itself holds no inner events).  With fewer
than 256 block rows the LM head is HBM-bound: achieved = algorithmic bytes
per call (W once, h of the rows computed once, their conf/argmax out; the
row kernel takes only the still-masked rows, like the GEMM) / mean duration,
against the 8 TB/s HBM peak; from 256 rows on it is an MFMA-bound GEMM over the still-
masked rows only (the decoder reads nothing else): achieved =
2*n_masked*V*d flops per call / mean duration, against the 2.5 PFLOP/s dense
bf16 peak.  traffic: HBM bytes per call from the committed rocprofv3 counter
summary, if it was taken on the current kernel source, else null.

block_loop: one block decoded until its mask is empty, timed per block from
the same pristine tokens/mask: dblk_decode_block_run (iterations enqueued a
chunk ahead of a host completion check, chunks of 2, 4 and 8),
dblk_decode_block (all L iterations enqueued at once, those after completion
skipped on the device; eager and replayed from a captured HIP graph), and a
host-driven loop that synchronises after every iteration.

cpu_baseline: the fp64 numpy oracle, full iterations of the same workload,
timed on the host for about --cpu-seconds.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
PMC_SUMMARY = os.path.join(ROOT, "profiles", "lmhead_pmc_traffic.json")
KV_COLD_BYTES = 512 << 20              # 2 x the MI355X MALL (256 MB)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def lmhead_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("lmhead.hip", "dblk_device.h", "dblk_launch.h", "commit_wave.h"):
        with open(os.path.join(ROOT, "block_wise_decoding_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def pmc_traffic(workload: str):
    """HBM bytes per LM-head launch from the committed counter summary, or None."""
    try:
        with open(PMC_SUMMARY) as f:
            s = json.load(f)
    except (OSError, ValueError):
        return None
    if s.get("kernel_source_sha256_16") != lmhead_source_hash() or s.get("workload") != workload:
        return None
    return s.get("hbm_bytes_per_launch")


def bench_block_loop(lib, dblock, torch, np, w, t, S_att, nblocks, dev):
    """Blocks decoded to completion: device loop (eager, graph) vs host-synchronised loop."""
    import ctypes
    B, L = w.B, w.L
    out = torch.empty_like(t["q"])
    conf = torch.empty(B, L, dtype=torch.float32, device=dev)
    amax = torch.empty(B, L, dtype=torch.int32, device=dev)
    tok = t["tok0"].clone()
    msk = t["msk0"].clone()
    nit = torch.empty(B, dtype=torch.int32, device=dev)
    args = dblock.decode_args(t["q"], t["kp"], t["vp"], t["kb"], t["vb"], t["ks"], t["vs"],
                              t["pl"], out, t["h"], t["W"], conf, amax, tok, msk, w.tau,
                              n_iters=nit, S=S_att)
    ws = dblock.alloc_workspace(dblock.decode_block_workspace_size(args), dev)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    pa = ctypes.byref(args)

    def reset():
        tok.copy_(t["tok0"])
        msk.copy_(t["msk0"])

    def timed(run):
        ts = []
        for _ in range(nblocks):
            reset()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            run()
            e1.record(stream)
            torch.cuda.synchronize()
            if bool(msk.any()):
                raise RuntimeError("a block loop left masked positions")
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    def device_loop():
        if lib.dblk_decode_block(pa, ws.data_ptr(), ws.numel(), sh) != 0:
            raise RuntimeError("dblk_decode_block failed")

    reset()
    device_loop()                         # warm-up; also loads every kernel before capture
    torch.cuda.synchronize()
    iters = nit.cpu().numpy()
    eager_ms = timed(device_loop)

    graph = torch.cuda.CUDAGraph()
    reset()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        dblock.dblk_decode_block(args, ws, stream=torch.cuda.current_stream(dev), device=dev)
    graph_ms = timed(graph.replay)

    M = B * L
    P = lambda x: x.data_ptr() if x.numel() else None
    ws_a = dblock.alloc_workspace(dblock.attend_workspace_size(B, w.H, L, w.D, w.P_cap, S_att), dev)
    ws_l = dblock.alloc_workspace(dblock.lmhead_workspace_size(M, w.d, w.V), dev)
    a_args = (P(t["q"]), P(t["kp"]), P(t["vp"]), P(t["kb"]), P(t["vb"]), P(t["ks"]), P(t["vs"]),
              P(t["pl"]), B, w.H, L, w.D, w.P_cap, S_att, w.S, 0.0, P(out), P(ws_a), ws_a.numel(), sh)
    lc_args = (P(t["h"]), P(t["W"]), w.d, w.V, P(conf), P(amax), P(tok), P(msk), B, L,
               float(w.tau), None, P(ws_l), ws_l.numel(), sh)

    def host_loop():
        for _ in range(L):
            st = lib.dblk_attend(*a_args)
            st |= lib.dblk_lmhead_confidence_commit(*lc_args)
            if st != 0:
                raise RuntimeError("libdblock call failed in the host loop")
            if not bool(msk.any()):          # device -> host copy: a synchronisation
                break

    host_ms = timed(host_loop)

    host_active = torch.zeros(2, dtype=torch.int32, pin_memory=True)
    n_enq = ctypes.c_int32(0)
    run_ms, run_enq = {}, {}
    for chunk in (2, 4, 8):
        def pipelined():
            if lib.dblk_decode_block_run(pa, chunk, host_active.data_ptr(), ws.data_ptr(),
                                         ws.numel(), sh, ctypes.byref(n_enq)) != 0:
                raise RuntimeError("dblk_decode_block_run failed")
        run_ms[chunk] = timed(pipelined)
        run_enq[chunk] = int(n_enq.value)
    best = min(run_ms, key=run_ms.get)
    committed = int(t["msk0"].sum())
    res = {"blocks": nblocks, "iterations_until_empty": int(iters.max()),
           "positions_committed_per_block": committed,
           "pipelined_ms_per_block": {str(c): round(v, 4) for c, v in run_ms.items()},
           "pipelined_iterations_enqueued": {str(c): v for c, v in run_enq.items()},
           "device_loop_ms_per_block": round(eager_ms, 4),
           "graph_ms_per_block": round(graph_ms, 4),
           "device_loop_iterations_enqueued": L,
           "host_sync_loop_ms_per_block": round(host_ms, 4),
           "committed_tokens_per_s": round(committed / (run_ms[best] * 1e-3), 1),
           "committed_tokens_per_s_from": f"pipelined, chunk {best}"}
    log(f"[bench] block loop: {res}")
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="c2-blk8")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--blocks", type=int, default=20,
                    help="blocks decoded by each block-loop variant (0: skip the block loop)")
    ap.add_argument("--suffix-window", type=int, default=None, metavar="S",
                    help="attend to the first S suffix rows only (suffix-pruned attention)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark, copy MIB MiB device-to-device 5 times "
                         "(reference dispatches for calibrating rocprofv3 byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from block_wise_decoding_amd import dblock
    from synth import WORKLOADS, make_inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "dispatches": 5}), flush=True)
        return
    lib = dblock.load_library()          # fails loudly if libdblock.so is not built
    w = WORKLOADS[args.workload]
    log(f"[bench] workload {w.name}: B={w.B} H={w.H} D={w.D} L={w.L} P_cap={w.P_cap} "
        f"S={w.S} V={w.V} tau={w.tau}")
    t0 = time.time()
    inp = make_inputs(w)
    log(f"[bench] inputs generated in {time.time() - t0:.1f}s")

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    q, kp, vp, kb, vb, ks, vs = (bf(inp[k]) for k in ("q", "kp", "vp", "kb", "vb", "ks", "vs"))
    # Cold attention inputs: step i reads KV set i mod R, R copies of the
    # same values at distinct addresses with >= 2 x the 256 MB MALL of
    # distinct bytes between two reuses of a set (W already exceeds it).
    att_set_bytes = sum(t.numel() * 2 for t in (q, kp, vp, kb, vb, ks, vs))
    R = max(1, -(-KV_COLD_BYTES // att_set_bytes))
    att_sets = [(q, kp, vp, kb, vb, ks, vs)] + [
        tuple(t.clone() for t in (q, kp, vp, kb, vb, ks, vs)) for _ in range(R - 1)]
    log(f"[bench] attention inputs: {R} rotating set(s) of {att_set_bytes / 1e6:.1f} MB")
    pl = torch.from_numpy(inp["prefix_len"]).to(dev)
    h, W = bf(inp["h"]), bf(inp["w"])
    tok0 = torch.from_numpy(inp["tokens"]).to(dev)
    msk0 = torch.from_numpy(inp["mask"]).to(dev)
    S_att = w.S if args.suffix_window is None else min(max(args.suffix_window, 0), w.S)
    K = args.steps
    KI = max(50, min(K, 300))
    # one pristine (tokens, mask) per step: warm-up, timed and instrumented steps
    n_copies = args.warmup + K + KI
    tok_all = tok0.unsqueeze(0).repeat(n_copies, 1, 1).contiguous()
    msk_all = msk0.unsqueeze(0).repeat(n_copies, 1, 1).contiguous()
    out = torch.empty_like(q)
    conf = torch.empty(w.M, dtype=torch.float32, device=dev)
    amax = torch.empty(w.M, dtype=torch.int32, device=dev)
    ncom = torch.empty(w.B, dtype=torch.int32, device=dev)
    ws_a = dblock.alloc_workspace(dblock.attend_workspace_size(w.B, w.H, w.L, w.D, w.P_cap, S_att), dev)
    ws_l = dblock.alloc_workspace(dblock.lmhead_workspace_size(w.M, w.d, w.V), dev)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    P = lambda t: t.data_ptr() if t.numel() else None
    a_args_r = [tuple(P(t) for t in st) + (P(pl), w.B, w.H, w.L, w.D, w.P_cap, S_att, w.S, 0.0,
                                          P(out), P(ws_a), ws_a.numel(), sh) for st in att_sets]
    tok_base, msk_base = tok_all.data_ptr(), msk_all.data_ptr()

    def lc_args(i):
        return (P(h), P(W), w.d, w.V, P(conf), P(amax), tok_base + i * w.M * 4,
                msk_base + i * w.M, w.B, w.L, float(w.tau), P(ncom), P(ws_l), ws_l.numel(), sh)

    def step(i):
        st = lib.dblk_attend(*a_args_r[i % R])
        st |= lib.dblk_lmhead_confidence_commit(*lc_args(i))
        return st

    torch.cuda.synchronize()
    for i in range(args.warmup):
        if step(i) != 0:
            raise RuntimeError("libdblock call failed during warm-up")
    torch.cuda.synchronize()

    # ---- timed region: K whole iterations, nothing else on the stream
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    bad = 0
    for i in range(args.warmup, args.warmup + K):
        bad |= step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    if bad:
        raise RuntimeError("libdblock call failed in the timed region")
    ms_step = t_start.elapsed_time(t_end) / K
    log(f"[bench] {K} steps: {ms_step * 1e3:.1f} us/step (wall {wall / K * 1e6:.1f} us/step)")

    # ---- instrumented region (same stream, same iteration): HIP events around
    # every call.  An event between two kernels costs a few microseconds of
    # idle GPU, so these timings are kept out of `value`; they give each
    # kernel's launch duration for the roofline and the stage breakdown.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(KI)]
    torch.cuda.synchronize()
    for j, e in enumerate(evs):
        e[0].record(stream); lib.dblk_attend(*a_args_r[(args.warmup + K + j) % R])
        e[1].record(stream); lib.dblk_lmhead_confidence_commit(*lc_args(args.warmup + K + j))
        e[2].record(stream)
    torch.cuda.synchronize()
    stage = {k: np.array([e[j].elapsed_time(e[j + 1]) * 1e3 for e in evs])
             for j, k in enumerate(("attend", "lmhead_commit"))}
    stages_us = {k: round(float(np.median(v)), 2) for k, v in stage.items()}
    it_inst = np.array([e[0].elapsed_time(e[2]) * 1e3 for e in evs])
    lm_ms = stage["lmhead_commit"] * 1e-3
    log(f"[bench] instrumented ({KI} steps): " +
        ", ".join(f"{k} {v.mean():.1f} us" for k, v in stage.items()))

    pl_np = inp["prefix_len"]
    kv_bytes = 2 * w.H * w.D * 2 * int(sum(int(p) + w.L + S_att for p in pl_np))
    qo_bytes = 2 * w.B * w.L * w.H * w.D * 2
    gemm = w.M >= 256                    # the library's plan: MFMA GEMM from 256 block rows on
    rows_kernel = not gemm and w.d % 256 == 0 and w.d // 256 in (1, 2, 4, 8)
    n_masked = int(inp["mask"].sum())
    # the GEMM and the rows-outer kernel take only the masked rows (compaction)
    n_rows = n_masked if (gemm or rows_kernel) else w.M
    lm_bytes = w.V * w.d * 2 + n_rows * w.d * 2 + n_rows * 8
    commit_bytes = w.M * 18
    it_bytes = kv_bytes + qo_bytes + lm_bytes + commit_bytes
    it_s = 1e3 / ms_step
    lm_us = float(lm_ms.mean()) * 1e3
    if gemm:
        # only the masked rows go through the LM head (masked-row compaction)
        lm_kernel = ("compact_masked_rows + lmhead_gemm_kernel + lmhead_gemm_merge "
                     "(+ threshold_commit_kernel)")
        flops = 2.0 * n_masked * w.V * w.d
        roof = {"bound": "mfma", "achieved": round(flops / (lm_us * 1e-6) / 1e12, 1),
                "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s"}
        roof["frac"] = round(roof["achieved"] / MFMA_BF16_PEAK_TFLOPS, 4)
        roof["algorithmic_flops_per_launch"] = flops
        roof["rows_computed"] = n_masked
    else:
        lm_kernel = "lmhead_rows_kernel" if rows_kernel else "lmhead_kernel"
        lm_kernel += (" (commit step fused)" if (w.L <= 64 and w.L & (w.L - 1) == 0)
                      else " (+ threshold_commit_kernel)")
        lm_gbs = lm_bytes / (lm_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(lm_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(lm_gbs / HBM_PEAK_GBS, 4), "rows_computed": n_rows}
    traffic = pmc_traffic(w.name) if S_att == w.S else None
    roofline = {"kernel": lm_kernel, **roof, "traffic": traffic,
                "algorithmic_bytes_per_launch": int(lm_bytes), "mean_launch_us": round(lm_us, 2)}

    block_loop = None
    if args.blocks > 0:
        block_loop = bench_block_loop(lib, dblock, torch, np, w, dict(
            q=q, kp=kp, vp=vp, kb=kb, vb=vb, ks=ks, vs=vs, pl=pl, h=h, W=W, tok0=tok0, msk0=msk0),
            S_att, args.blocks, dev)

    cpu = None
    if not args.no_cpu_baseline:
        from oracle import iteration
        try:
            from threadpoolctl import threadpool_info
            cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:
            cores = os.cpu_count() or 1
        n, c0 = 0, time.perf_counter()
        while True:
            iteration(inp, w.tau)
            n += 1
            if time.perf_counter() - c0 >= args.cpu_seconds:
                break
        t_it = (time.perf_counter() - c0) / n
        cpu = {"value": round(1.0 / t_it, 4), "unit": "iter/s", "cores": int(cores),
               "kind": "oracle",
               "sample": f"{n} full fp64 oracle iterations of {w.name} (all {w.M} block rows, "
                         f"all {w.B * w.H} (b,h) attention rows, commit), {t_it:.2f} s each"}
        log(f"[bench] oracle: {t_it:.2f} s/iteration on {cores} threads")

    res = {
        "metric": "denoise iterations/s",
        "value": round(it_s, 2),
        "unit": "iter/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.note}", "batch": w.B, "heads": w.H,
                   "head_dim": w.D, "block_len": w.L, "prefix": w.P_cap, "suffix": w.S,
                   "vocab": w.V, "threshold": w.tau, "parallelism": "none (1 GPU)"},
        "block_positions_per_s": round(w.B * w.L * it_s, 1),
        "hbm_frac_iteration": round(it_bytes / (ms_step * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
        "algorithmic_bytes_per_iteration": int(it_bytes),
        "stages_us_median_instrumented": stages_us,
        "iteration_us_instrumented": {q_: round(float(np.percentile(it_inst, p_)), 2)
                                      for q_, p_ in (("p10", 10), ("median", 50), ("p90", 90))},
        "roofline": roofline,
        # attention stage (attention kernel + split merge) against the HBM peak;
        # its instrumented time includes the events' own gaps, so this errs low
        "attention_stage": {"algorithmic_bytes": int(kv_bytes + qo_bytes),
                            "median_us_instrumented": stages_us["attend"],
                            "achieved_GBs": round((kv_bytes + qo_bytes) / (stages_us["attend"] * 1e-6) / 1e9, 1),
                            "frac": round((kv_bytes + qo_bytes) / (stages_us["attend"] * 1e-6) / 1e9
                                          / HBM_PEAK_GBS, 4),
                            "split_partials_bytes": int(dblock.attend_workspace_size(
                                w.B, w.H, w.L, w.D, w.P_cap, S_att))},
        "block_loop": block_loop,
        "cpu_baseline": cpu,
    }
    if S_att != w.S:
        res["config"]["suffix_window"] = S_att
    res["config"]["attention_input_sets"] = R
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
