#!/usr/bin/env python3
"""Benchmark one denoising iteration of block-wise diffusion-LLM decoding on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]

A step is one whole iteration on synthetic inputs already resident in HBM:
dblk_attend (block queries over the dual KV cache), then
dblk_lmhead_confidence_commit (LM head, full-vocabulary softmax confidence and
argmax, and the threshold parallel decoder's commit step, which runs inside
the LM head's final merge where the shapes allow; bitwise the same as
dblk_lmhead_confidence followed by dblk_threshold_commit), back to back on one
stream, called through the C ABI.  W untimed warm-up steps, then K timed steps
bracketed by device synchronisation.  Prints ONE JSON line on stdout;
progress goes to stderr.

Default workload: the LLaDA-MoE-7B-A1B-shaped block at block index 8 (batch
1, 16 heads x 128, prefix 768 + block 64 + suffix 448, vocabulary 157184,
threshold 0.9).  With the default, the same measurement also runs on block
indices 0 and 15 (prefix 256 / 1216, suffix 960 / 0), each in a child
process of its own, and their figures go into `block_indices`.

Every step starts from the workload's own tokens and mask: one pristine
copy per step is laid out in HBM before the timed region, so each commit
step decides on the generated mask rather than on one emptied by earlier
steps.  Attention inputs are cold: step i reads set i mod R of R copies of
q, K and V at distinct addresses, with at least 2x the 256 MB MALL of
distinct bytes between two reuses of a set (W alone already exceeds it).
`warm` repeats the timed region with one attention set reused every step.

roofline: the dominant kernel is the LM head (98% of the iteration's bytes
at batch 1).  The duration of dblk_lmhead_confidence_commit (the LM-head
kernel with the commit step in its tail, or the LM head plus the commit
kernel) is measured with HIP events recorded on the launch stream around
every call, in a second instrumented run right after the timed region (an
event between two kernels leaves the GPU idle a few microseconds, so the
timed region holds no inner events).  The bound follows from the LM head's
arithmetic intensity over the rows it must compute (the still-masked rows:
the decoder reads nothing else): 2*n*V*d flops against V*d*2 + n*d*2 + n*8
bytes.  Below the MI355X ridge (2.5 PFLOP/s / 8 TB/s = 312.5 flop/byte) it
is HBM-bound: achieved = those bytes / mean duration, against 8 TB/s (and
against the read ceiling measured by the probe below); above it,
MFMA-bound: achieved = 2*n*V*d / mean duration, against 2.5 PFLOP/s dense
bf16.  traffic: HBM bytes per call from the committed rocprofv3 counter
summary, if it was taken on the current kernel source, else null.

read_ceiling: dblk_probe_read streams a 1 GiB buffer with the LM head's
load pattern (16-byte loads, whole 128-byte lines per wave instruction),
with and without the nontemporal hint.

block_loop: one block decoded until its mask is empty, timed per block from
the same pristine tokens/mask: dblk_decode_block_run (iterations enqueued a
chunk ahead of a host completion check, chunks of 2, 4 and 8),
dblk_decode_block (all L iterations enqueued at once, those after completion
skipped on the device; eager and replayed from a captured HIP graph), and a
host-driven loop that synchronises after every iteration.

cpu_baseline: the fp64 numpy oracle, full iterations of the same workload,
timed on the host's cores for about --cpu-seconds.  Its first iteration is
also compared with the GPU's first timed step (`parity`: attention row error,
confidence error, argmax and commit mismatches, excluded count |E|).
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
RIDGE_FLOP_PER_BYTE = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
PMC_SUMMARY = os.path.join(ROOT, "profiles", "lmhead_pmc_traffic.json")
SETTLE_S = 0.05            # untimed iterations before any measurement (s)
KV_COLD_BYTES = 512 << 20              # 2 x the MI355X MALL (256 MB)
C2_SIBLINGS = {"c2-blk8": ("c2-blk0", "c2-blk15")}


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


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def read_ceiling(dblock, torch, dev, mib=1024, reps=10):
    """GB/s of dblk_probe_read over a `mib` MiB buffer (> the MALL), NT and plain."""
    buf = torch.ones(mib << 20, dtype=torch.uint8, device=dev)
    grid = 1024
    sink = torch.empty(grid * 256, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    res = {}
    for nt in (True, False):
        for _ in range(2):
            dblock.dblk_probe_read(buf, nt, grid, sink, stream)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            dblock.dblk_probe_read(buf, nt, grid, sink, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        res["nontemporal" if nt else "plain"] = round(buf.numel() / (us * 1e-6) / 1e9, 1)
    del buf, sink
    torch.cuda.empty_cache()
    return {"GBs": res, "bytes": mib << 20, "passes": reps, "grid": grid,
            "kernel": "read_probe_kernel (dblk_probe_read)"}


def cache_append_rate(dblock, torch, np, w, dev, n_calls=40):
    """dblk_cache_append on the workload's shapes: each call appends the block's
    K and V (B*H*L*D bf16 each) after every sequence's prefix.  The prefix
    capacity holds all n_calls appends, so nothing is reset between calls."""
    B, H, L, D = w.B, w.H, w.L, w.D
    cap = w.P_cap + L * (n_calls + 2)
    kp = torch.empty(B, H, cap, D, dtype=torch.bfloat16, device=dev)
    vp = torch.empty_like(kp)
    kb = torch.randn(B, H, L, D, device=dev).to(torch.bfloat16)
    vb = torch.randn(B, H, L, D, device=dev).to(torch.bfloat16)
    pl0 = torch.full((B,), w.P_cap, dtype=torch.int32, device=dev)
    pl = pl0.clone()
    stream = torch.cuda.current_stream(dev)
    dblock.dblk_cache_append(kp, vp, kb, vb, pl, stream=stream)      # warm-up
    pl.copy_(pl0)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n_calls):
        dblock.dblk_cache_append(kp, vp, kb, vb, pl, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    assert int(pl[0]) == w.P_cap + n_calls * L
    us = e0.elapsed_time(e1) * 1e3 / n_calls
    moved = 2 * 2 * B * H * L * D * 2          # K and V, read once and written once
    return {"workload": w.name, "us_per_call": round(us, 2), "bytes_per_call": moved,
            "GBs": round(moved / (us * 1e-6) / 1e9, 1),
            "frac_of_hbm_peak": round(moved / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "calls": n_calls, "kernels": "cache_append_kernel + cache_advance_kernel"}


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
    torch.cuda.synchronize()                 # the last queued chunk still writes host_active
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


def lmhead_roofline(w, n_masked, lm_us):
    """Roofline of dblk_lmhead_confidence_commit on the rows it must compute."""
    gemm = w.M >= 256                    # the library's plan: MFMA GEMM from 256 block rows on
    rows_kernel = not gemm and w.d % 256 == 0 and w.d // 256 in (1, 2, 4, 8)
    # the GEMM and the rows-outer kernel take only the masked rows (compaction)
    n = n_masked if (gemm or rows_kernel) else w.M
    lm_bytes = w.V * w.d * 2 + n * w.d * 2 + n * 8
    flops = 2.0 * n * w.V * w.d
    intensity = flops / lm_bytes
    if gemm:
        kernel = ("compact_masked_rows + lmhead_gemm_kernel + lmhead_gemm_merge "
                  "(+ threshold_commit_kernel)")
    else:
        kernel = "lmhead_rows_kernel" if rows_kernel else "lmhead_kernel"
        kernel += (" (commit step fused)" if (w.L <= 64 and w.L & (w.L - 1) == 0)
                   else " (+ threshold_commit_kernel)")
    t = lm_us * 1e-6
    if intensity >= RIDGE_FLOP_PER_BYTE:
        ach = flops / t / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4)}
    else:
        ach = lm_bytes / t / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4)}
    roof.update({"kernel": kernel, "rows_computed": n, "algorithmic_bytes_per_launch": int(lm_bytes),
                 "algorithmic_flops_per_launch": flops,
                 "intensity_flop_per_byte": round(intensity, 1),
                 "ridge_flop_per_byte": RIDGE_FLOP_PER_BYTE, "mean_launch_us": round(lm_us, 2)})
    if gemm:
        ntile = -(-n // 256)              # the GEMM walks the 256-row h tiles holding masked rows
        roof["executed_flops_per_launch"] = 2.0 * ntile * 256 * w.V * w.d
    return roof, lm_bytes


def measure(lib, dblock, torch, np, w, args, dev):
    """Timed (cold), warm and instrumented runs of one workload."""
    from synth import make_inputs
    t0 = time.time()
    inp = make_inputs(w)
    log(f"[bench] workload {w.name}: B={w.B} H={w.H} D={w.D} L={w.L} P_cap={w.P_cap} "
        f"S={w.S} V={w.V} tau={w.tau}; inputs generated in {time.time() - t0:.1f}s")

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    q, kp, vp, kb, vb, ks, vs = (bf(inp[k]) for k in ("q", "kp", "vp", "kb", "vb", "ks", "vs"))
    att_set_bytes = sum(t.numel() * 2 for t in (q, kp, vp, kb, vb, ks, vs))
    R = max(1, -(-KV_COLD_BYTES // att_set_bytes))
    att_sets = [(q, kp, vp, kb, vb, ks, vs)] + [
        tuple(t.clone() for t in (q, kp, vp, kb, vb, ks, vs)) for _ in range(R - 1)]
    pl = torch.from_numpy(inp["prefix_len"]).to(dev)
    h, W = bf(inp["h"]), bf(inp["w"])
    tok0 = torch.from_numpy(inp["tokens"]).to(dev)
    msk0 = torch.from_numpy(inp["mask"]).to(dev)
    S_att = w.S if args.suffix_window is None else min(max(args.suffix_window, 0), w.S)
    K, WU = args.steps, args.warmup
    KI = max(50, min(K, 300))
    KW = K if R > 1 else 0               # warm run only where the cold run rotates sets
    # one pristine (tokens, mask) per step: warm-up, timed, warm and instrumented steps
    n_copies = WU + K + KW + KI
    tok_all = tok0.unsqueeze(0).repeat(n_copies, 1, 1).contiguous()
    msk_all = msk0.unsqueeze(0).repeat(n_copies, 1, 1).contiguous()
    out = torch.empty_like(q)
    conf = torch.full((w.M,), -7.0, dtype=torch.float32, device=dev)
    amax = torch.full((w.M,), -9, dtype=torch.int32, device=dev)
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

    def step(i, aset):
        st = lib.dblk_attend(*a_args_r[aset])
        st |= lib.dblk_lmhead_confidence_commit(*lc_args(i))
        return st

    def timed_region(first, n, rotate):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        e0.record(stream)
        bad = 0
        for i in range(first, first + n):
            bad |= step(i, i % R if rotate else 0)
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        if bad:
            raise RuntimeError("libdblock call failed in the timed region")
        return e0.elapsed_time(e1) / n, wall / n

    # ---- settle: input generation keeps the GPU idle for seconds, and its
    # clocks take milliseconds to come back up (the first steps after idle run
    # visibly slower).  Whole iterations, untimed, for SETTLE_S seconds before
    # anything is measured; each step commits on a fresh copy of the pristine
    # tokens and mask, refilled every len(pool) steps, so every step does the
    # work of a timed one.
    pool_t = tok0.unsqueeze(0).repeat(8, 1, 1).contiguous()
    pool_m = msk0.unsqueeze(0).repeat(8, 1, 1).contiguous()
    pt, pm = pool_t.data_ptr(), pool_m.data_ptr()
    torch.cuda.synchronize()
    t_settle, n_settle = time.perf_counter(), 0
    while time.perf_counter() - t_settle < SETTLE_S or n_settle < 16:
        for j in range(8):
            a = lc_args(0)
            st = lib.dblk_attend(*a_args_r[(n_settle + j) % R])
            st |= lib.dblk_lmhead_confidence_commit(*(a[:6] + (pt + j * w.M * 4, pm + j * w.M) + a[8:]))
            if st != 0:
                raise RuntimeError("libdblock call failed while settling")
        pool_t.copy_(tok0.unsqueeze(0).expand_as(pool_t))
        pool_m.copy_(msk0.unsqueeze(0).expand_as(pool_m))
        torch.cuda.synchronize()
        n_settle += 8
    del pool_t, pool_m
    log(f"[bench] {w.name}: settled over {n_settle} untimed steps")

    # ---- instrumented region (same stream, same iteration): HIP events around
    # every call.  An event between two kernels costs a few microseconds of
    # idle GPU, so these timings are kept out of `value`; they give each
    # kernel's launch duration for the roofline and the stage breakdown.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(KI)]
    torch.cuda.synchronize()
    for j, e in enumerate(evs):
        e[0].record(stream); lib.dblk_attend(*a_args_r[j % R])
        e[1].record(stream); lib.dblk_lmhead_confidence_commit(*lc_args(j))
        e[2].record(stream)
    torch.cuda.synchronize()
    stage = {k: np.array([e[j].elapsed_time(e[j + 1]) * 1e3 for e in evs])
             for j, k in enumerate(("attend", "lmhead_commit"))}
    stages_us = {k: round(float(np.median(v)), 2) for k, v in stage.items()}
    it_inst = np.array([e[0].elapsed_time(e[2]) * 1e3 for e in evs])
    log(f"[bench] {w.name}: instrumented ({KI} steps): " +
        ", ".join(f"{k} {v.mean():.1f} us" for k, v in stage.items()))

    # ---- warm-up, then the timed region: K whole iterations, nothing else on
    # the stream
    for i in range(KI, KI + WU):
        if step(i, i % R) != 0:
            raise RuntimeError("libdblock call failed during warm-up")
    first = KI + WU
    ms_step, wall_step = timed_region(first, K, True)
    log(f"[bench] {w.name}: {K} steps: {ms_step * 1e3:.1f} us/step (wall {wall_step * 1e6:.1f} us/step)")
    # the first timed step's tokens and mask (each step commits on its own
    # copy); conf, argmax and the attention output are those of the last step,
    # which computes the same values from the same inputs
    g_first = {"tokens": tok_all[first].cpu().numpy(), "mask": msk_all[first].cpu().numpy(),
               "conf": conf.cpu().numpy(), "argmax": amax.cpu().numpy(),
               "o": out.float().cpu().numpy().astype(np.float64)}
    warm_ms = None
    if KW:
        warm_ms, _ = timed_region(first + K, KW, False)
        log(f"[bench] {w.name}: warm (one attention set): {warm_ms * 1e3:.1f} us/step")

    kv_bytes = 2 * w.H * w.D * 2 * int(sum(int(p) + w.L + S_att for p in inp["prefix_len"]))
    qo_bytes = 2 * w.B * w.L * w.H * w.D * 2
    n_masked = int(inp["mask"].sum())
    roof, lm_bytes = lmhead_roofline(w, n_masked, float(stage["lmhead_commit"].mean()))
    it_bytes = kv_bytes + qo_bytes + lm_bytes + w.M * 18
    att_us = stages_us["attend"]
    res = {
        "ms_per_step": round(ms_step, 5),
        "iterations_per_s": round(1e3 / ms_step, 2),
        "block_positions_per_s": round(w.B * w.L * 1e3 / ms_step, 1),
        "hbm_frac_iteration": round(it_bytes / (ms_step * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
        "algorithmic_bytes_per_iteration": int(it_bytes),
        "warm_ms_per_step": round(warm_ms, 5) if warm_ms else None,
        "stages_us_median_instrumented": stages_us,
        "iteration_us_instrumented": {q_: round(float(np.percentile(it_inst, p_)), 2)
                                      for q_, p_ in (("p10", 10), ("median", 50), ("p90", 90))},
        "roofline": roof,
        # attention stage against the HBM peak; its instrumented time includes
        # the events' own gaps, so this errs low
        "attention_stage": {"algorithmic_bytes": int(kv_bytes + qo_bytes),
                            "median_us_instrumented": att_us,
                            "achieved_GBs": round((kv_bytes + qo_bytes) / (att_us * 1e-6) / 1e9, 1),
                            "frac": round((kv_bytes + qo_bytes) / (att_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                            "split_partials_bytes": int(dblock.attend_workspace_size(
                                w.B, w.H, w.L, w.D, w.P_cap, S_att))},
        "attention_input_sets": R,
        "suffix_attended": S_att,
    }
    tensors = dict(q=q, kp=kp, vp=vp, kb=kb, vb=vb, ks=ks, vs=vs, pl=pl, h=h, W=W, tok0=tok0,
                   msk0=msk0)
    del att_sets, tok_all, msk_all
    return res, inp, g_first, tensors, S_att


def oracle_parity(np, w, inp, ref, g):
    """The GPU's first timed step against the oracle iteration on the same inputs."""
    from oracle import attention_row_rel_err, compare_commit, exclusion_set
    m_in = inp["mask"].astype(bool).reshape(-1)
    conf_ref = ref["conf"].reshape(w.B, w.L)
    gap_ref = ref["gap"].reshape(w.B, w.L)
    E = exclusion_set(conf_ref, gap_ref, inp["mask"], w.tau)
    ok = m_in & (ref["gap"] >= 1e-3)
    return {"attention_row_rel_err": float(attention_row_rel_err(g["o"], ref["o"])),
            "conf_max_abs_err_masked_rows": float(np.abs(g["conf"][m_in] - ref["conf"][m_in]).max()),
            "argmax_mismatches_masked_rows": int((g["argmax"][ok] != ref["argmax"][ok]).sum()),
            "commit_mismatches": int(compare_commit(g["tokens"], g["mask"], ref["tokens"],
                                                    ref["mask"], E)),
            "excluded_E": int(E.sum()), "positions": int(E.size),
            "tolerances": {"attention_row_rel_err": 1e-2, "conf_abs": 1e-3,
                           "argmax_and_commit": "exact outside E"}}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="c2-blk8")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-siblings", action="store_true",
                    help="measure the named workload only (not the other c2 block indices)")
    ap.add_argument("--no-read-ceiling", action="store_true",
                    help="skip the HBM read-ceiling probe")
    ap.add_argument("--blocks", type=int, default=20,
                    help="blocks decoded by each block-loop variant (0: skip the block loop)")
    ap.add_argument("--suffix-window", type=int, default=None, metavar="S",
                    help="attend to the first S suffix rows only (suffix-pruned attention)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark, copy MIB MiB device-to-device 5 times "
                         "(reference dispatches for calibrating rocprofv3 byte counters)")
    ap.add_argument("--read-probe", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark, measure the HBM read ceiling over MIB MiB")
    ap.add_argument("--cache-append", action="store_true",
                    help="instead of the benchmark, time dblk_cache_append on the workload's shapes")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from block_wise_decoding_amd import dblock
    from synth import WORKLOADS

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
    if args.read_probe:
        print(json.dumps({"read_ceiling": read_ceiling(dblock, torch, dev, args.read_probe)}),
              flush=True)
        return
    if args.cache_append:
        print(json.dumps({"cache_append": cache_append_rate(dblock, torch, np,
                                                            WORKLOADS[args.workload], dev)}),
              flush=True)
        return
    w = WORKLOADS[args.workload]
    prim, inp, g_first, tensors, S_att = measure(lib, dblock, torch, np, w, args, dev)

    block_loop = None
    if args.blocks > 0:
        block_loop = bench_block_loop(lib, dblock, torch, np, w, tensors, S_att, args.blocks, dev)
    del tensors
    torch.cuda.empty_cache()

    siblings = {}
    if not args.no_siblings and args.suffix_window is None:
        # each sibling in a child process of its own: measured in the same
        # process after the first workload, its 644 MB weight lands in memory
        # freed by the first one and its LM head ran ~2 us slower
        import subprocess
        for name in C2_SIBLINGS.get(w.name, ()):
            cmd = [sys.executable, os.path.abspath(__file__), "--workload", name, "--steps",
                   str(args.steps), "--warmup", str(args.warmup), "--no-siblings", "--blocks", "0",
                   "--no-cpu-baseline", "--no-read-ceiling"]
            r = json.loads(subprocess.run(cmd, check=True, capture_output=True, text=True)
                           .stdout.strip().splitlines()[-1])
            siblings[name] = {k: r[k] for k in ("ms_per_step", "value", "block_positions_per_s",
                                                  "hbm_frac_iteration", "warm_ms_per_step",
                                                  "stages_us_median_instrumented")}
            siblings[name]["iterations_per_s"] = siblings[name].pop("value")
            siblings[name]["lmhead_roofline_frac"] = r["roofline"]["frac"]
            log(f"[bench] {name} (own process): {r['ms_per_step'] * 1e3:.1f} us/step")
    ceiling = None
    roof = prim["roofline"]
    if not args.no_read_ceiling:
        ceiling = read_ceiling(dblock, torch, dev)
        log(f"[bench] read ceiling: {ceiling['GBs']}")
        if roof["bound"] == "hbm":
            roof["frac_of_measured_read_ceiling"] = round(
                roof["achieved"] / ceiling["GBs"]["nontemporal"], 4)
    roof["traffic"] = pmc_traffic(w.name) if S_att == w.S else None

    cpu, parity = None, None
    if not args.no_cpu_baseline:
        from oracle import iteration
        cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
        try:
            from threadpoolctl import threadpool_info, threadpool_limits
            limiter = threadpool_limits(limits=cores)
            blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:
            limiter, blas = None, cores
        n, c0 = 0, time.perf_counter()
        ref = None
        while True:
            r = iteration(inp, w.tau, rows=None)
            ref = ref or r
            n += 1
            if time.perf_counter() - c0 >= args.cpu_seconds:
                break
        t_it = (time.perf_counter() - c0) / n
        if limiter is not None:
            limiter.restore_original_limits()
        cpu = {"value": round(1.0 / t_it, 4), "unit": "iter/s", "cores": int(blas), "kind": "oracle",
               "affinity_cores": int(cores), "cpu_model": cpu_model(),
               "block_positions_per_s": round(w.B * w.L / t_it, 2),
               "sample": f"{n} full fp64 oracle iterations of {w.name} (all {w.M} block rows, "
                         f"all {w.B * w.H} (b,h) attention rows, commit), {t_it:.2f} s each"}
        log(f"[bench] oracle: {t_it:.2f} s/iteration on {blas} threads ({cpu['cpu_model']})")
        if S_att == w.S:
            parity = oracle_parity(np, w, inp, ref, g_first)
            log(f"[bench] parity of the first timed step: {parity}")

    ms_step = prim["ms_per_step"]
    res = {
        "metric": "denoise iterations/s",
        "value": prim["iterations_per_s"],
        "unit": "iter/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.note}", "batch": w.B, "heads": w.H,
                   "head_dim": w.D, "block_len": w.L, "prefix": w.P_cap, "suffix": w.S,
                   "vocab": w.V, "threshold": w.tau, "parallelism": "none (1 GPU)",
                   "attention_input_sets": prim["attention_input_sets"]},
        "block_positions_per_s": prim["block_positions_per_s"],
        "hbm_frac_iteration": prim["hbm_frac_iteration"],
        "algorithmic_bytes_per_iteration": prim["algorithmic_bytes_per_iteration"],
        "warm_ms_per_step": prim["warm_ms_per_step"],
        "stages_us_median_instrumented": prim["stages_us_median_instrumented"],
        "iteration_us_instrumented": prim["iteration_us_instrumented"],
        "roofline": roof,
        "read_ceiling": ceiling,
        "attention_stage": prim["attention_stage"],
        "block_indices": siblings or None,
        "block_loop": block_loop,
        "parity": parity,
        "cpu_baseline": cpu,
    }
    if S_att != w.S:
        res["config"]["suffix_window"] = S_att
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
