#!/usr/bin/env python3
"""Benchmark of the WeDLM streaming-decode step on one MI355X.

A step is one pass of the whole decode path over one batch: wedlm_reorder
(Topological Reordering + logical RoPE + KV append), wedlm_step_attn
(windowed causal GQA attention over the paged prefix cache) and
wedlm_select_commit (vocabulary confidence, commit, Eq. 11 fill, refill),
taken as one wedlm_decode_step call (the same three in three launches
instead of five; --unfused times the three calls instead, and the line
carries the other form's time beside it).  Steps stream: each one commits
tokens, so the context grows as it would in decoding.  Inputs are synthetic
and resident in HBM before timing starts.

Default workload: batch 4, 32 Q / 8 KV heads, head dim 128, 32768 cached
tokens in 16-token pages (shuffled), window 32 (16 observed), bf16; logits
[4, 32, 151936] fp32 drawn with the low/high-entropy mixture.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu]

Prints one JSON line (rank 0).  Three timed regions: (1) K whole streaming
steps, bracketed by device synchronisation, give ms_per_step and the
headline window tokens/s: launched eagerly (reported as eager_ms_per_step),
then, unless --eager, the same K steps captured once as a HIP graph with the
library's own capture API (wedlm_graph_begin / end / launch) and replayed
from the same starting state, as a serving loop would run them
(this replay gives ms_per_step and the value); (2) K back-to-back launches
of the attention call on the final state, bracketed by HIP events on its
stream, give the mean launch time the roofline divides the launch's
algorithmic bytes (K/V of every visible key read once, Q in, O out) by; (3)
the select/commit call alone, for its own bandwidth.  With the default
workload the line also carries, under "configs", the same measurement of
the other decode-step workloads (qwen3_l2048: batch 1 over a 2048-token
prefix; ragged_b32: 32 sequences with prefixes uniform in [512, 8192];
tiny_f32) and of the select/commit workload select_v152k (batch 64 x
window 16 over V = 151936), each with its attention roofline fraction
(--no-extra skips them).  Before each timed
sequence the same sequence runs untimed from the same starting state for at
least SETTLE_S seconds (and the attention call alone for ATTN_SETTLE_S
seconds before its leg), because the board reaches steady clocks only
after some tenths of a second of load.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 matrix-core peak of MI355X
# Counter-derived HBM bytes per attention launch, written from two rocprofv3
# --pmc passes (FETCH_SIZE, WRITE_SIZE) over this same command and scaled by a
# plain-copy calibration.  Used only while the attention sources still hash to
# the value recorded there and the run is the one profiled.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_traffic_long_b4.md")
ATTN_SOURCES = ["attn_bf16.hip", "attn.hip", "api.hip", "kernels.hpp", "common.hpp"]
METRIC = "window tokens/sec and decode steps/sec per GPU; attn achieved HBM GB/s vs peak"
ATTN_SETTLE = 100   # attention launches per untimed round before the roofline leg
ATTN_SETTLE_S = 0.5 # seconds of such rounds: the call's own steady clocks before it is timed
SETTLE_S = 0.25     # seconds of untimed repeats of the timed sequence before it is timed


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="long_b4",
                    choices=["long_b4", "ragged_b32", "qwen3_l2048", "tiny_f32", "select_v152k",
                             "lmhead_v152k", "dualstream_n4096", "model_qwen3_w64"],
                    help="select_v152k times the select/commit call alone (batch 64 x window 16, "
                         "V=151936, streaming from an all-masked window); lmhead_v152k the fused "
                         "LM head + select call (hidden 4096) on the same window; dualstream_n4096 the "
                         "Dual-Stream Masking attention over 4 x 4096 tokens, blocks of 32; model_qwen3_w64 "
                         "whole decode steps of a 36-layer Qwen3-8B-shaped synthetic decoder on a 4 x 64 window")
    ap.add_argument("--vocab", type=int, default=151936)
    ap.add_argument("--logit-ring", type=int, default=4, help="distinct logits buffers cycled over steps")
    ap.add_argument("--split-keys", type=int, default=0, help="override keys per split-KV work-group")
    ap.add_argument("--attn-tail", type=int, default=-1,
                    help="tail splits: sequences cut in two (-1 automatic, 0 off)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extra", action="store_true",
                    help="long_b4 only: skip the summaries of the other decode-step workloads and of the "
                         "select/commit workload that the default line carries under \"configs\"")
    ap.add_argument("--cpu-seqs", type=int, default=0, help="sequences in the CPU sample (0 = auto)")
    ap.add_argument("--unfused", action="store_true",
                    help="time the step as the three calls (reorder, attention, select/commit) "
                         "instead of one wedlm_decode_step")
    ap.add_argument("--eager", action="store_true",
                    help="time only eager launches (default: eager, then the same K steps replayed "
                         "as one captured HIP graph, which gives the reported value)")
    ap.add_argument("--cold", action="store_true",
                    help="also time each attention call after a 1 GiB scratch write (MALL cold)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (5 times): the reference for "
                         "scaling rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes")
    return ap.parse_args()


def settle(run, restart, seconds=SETTLE_S):
    """Run the timed sequence untimed, from its starting state each time,
    for at least `seconds`: the board only reaches its steady clocks after
    some tenths of a second of load (the first launches of a process, or
    the first after an idle gap such as a graph capture, run up to 30 %
    slower)."""
    import torch
    t_end = time.perf_counter() + seconds
    while True:
        restart()
        run()
        torch.cuda.synchronize()
        if time.perf_counter() >= t_end:
            break


def capture_steps(fn):
    """Record the library calls fn() makes as one HIP graph with the
    library's own capture API (wedlm_graph_begin / end), on a side stream
    ordered after the current one; replay with .launch()."""
    import torch
    import causal_attention_diffusion_amd as wd
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with wd.capture(cap) as g:
        fn()
    torch.cuda.current_stream().wait_stream(cap)
    return g


def copy_calibration(mib):
    """Plain device-to-device copy of known size, for counter calibration."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / 5
    print(json.dumps({"copy_MiB": mib, "bytes_read_per_copy": n * 4, "bytes_written_per_copy": n * 4,
                      "GB_per_s_read_plus_write": round(2 * n * 4 / dt / 1e9, 1)}), flush=True)


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path (the path would "
              "shard by sequence and KV head, or by key range with one all-gather of the split "
              "partials; that is a design, not code)", file=sys.stderr)
        sys.exit(2)

    if args.workload == "select_v152k":
        bench_select(args)
        return
    if args.workload == "lmhead_v152k":
        bench_lmhead(args)
        return
    if args.workload == "dualstream_n4096":
        bench_dual(args)
        return
    if args.workload == "model_qwen3_w64":
        bench_model(args)
        return

    result = decode_leg(args, args.workload, with_cpu=not args.no_cpu)
    if args.workload == "long_b4" and not args.no_extra:
        # the other workloads of the decode step, each timed the same way
        # (same --steps / --warmup), summarised beside the headline
        extra = {}
        for name in EXTRA_DECODE:
            extra[name] = summarise_decode(decode_leg(args, name, with_cpu=False))
            print(f"[bench] {name}: {extra[name]['ms_per_step']} ms per step", file=sys.stderr, flush=True)
        extra["select_v152k"] = summarise_select(bench_select(args, emit=False))
        print(f"[bench] select_v152k: {extra['select_v152k']['ms_per_step']} ms per step", file=sys.stderr,
              flush=True)
        result["configs"] = extra
    print(json.dumps(result), flush=True)


EXTRA_DECODE = ["qwen3_l2048", "ragged_b32", "tiny_f32"]


def summarise_decode(r):
    """The figures of one decode-step workload kept in the headline line."""
    a = r["attn"]
    return {"workload": r["config"]["workload"], "ms_per_step": r["ms_per_step"],
            "eager_ms_per_step": r["eager_ms_per_step"], "step_call": r["step_call"],
            **{k: r[k] for k in ("three_call_ms_per_step", "fused_ms_per_step") if k in r},
            "window_tokens_per_s": r["value"],
            "steps_per_s": r["steps_per_s"], "split_kv": r["config"]["split_kv"],
            "attn": {"avg_ms": a["avg_ms"], "alg_bytes_per_launch": a["alg_bytes_per_launch"],
                     "GB_per_s": a["GB_per_s"], "frac_of_hbm_peak": a["frac_of_hbm_peak"]},
            "attn_kernel_in_steps": r["attn_kernel_in_steps"],
            "select_commit": r["select_commit"], "P_c": r["P_c"],
            "dtype": r["dtype"]}


def summarise_select(r):
    return {"workload": r["config"]["workload"], "ms_per_step": r["ms_per_step"],
            "eager_ms_per_step": r["eager_ms_per_step"], "window_tokens_per_s": r["value"],
            "select_commit": r["select_commit"], "frac_of_hbm_peak": r["roofline"]["frac"], "P_c": r["P_c"]}


def decode_leg(args, workload, with_cpu):
    """K streaming decode steps (reorder + attention + select/commit) of one
    workload, then the attention call and the select/commit call alone;
    returns the result dict of the bench line."""
    import torch
    import workloads as wl
    import causal_attention_diffusion_amd as wd

    dev = torch.device("cuda:0")
    cfg = wl.CONFIGS[workload]
    scfg = wl.SelectConfig("bench", B=cfg.B, W=cfg.W, V=args.vocab, seed=1005, alpha=0.25, tau=9.0,
                           steps=0, kind="mixture")
    total_steps = args.steps + args.warmup
    spare = total_steps * cfg.W + cfg.W
    inp = wl.make_attn_inputs(cfg, spare_tokens=spare)
    t = wl.device_attn_inputs(inp, dev)
    wd.wedlm_set_attn_split_keys(args.split_keys)
    wd.wedlm_set_attn_tail(args.attn_tail)

    B, W = cfg.B, cfg.W
    mask_id = args.vocab
    # window state as produced by the previous step: flags from the workload, tokens filled
    tok0 = np.where(inp.filled == 1, (np.arange(B * W).reshape(B, W) * 7919) % args.vocab,
                    mask_id).astype(np.int32)
    tok = torch.from_numpy(tok0).to(dev)
    filled, pos, ctx = t["filled"], t["pos"], t["ctx_len"]
    max_ctx = int(inp.ctx_len.max()) + total_steps * W
    ws_attn = wd.attn_workspace_tensor(t["q_phys"], t["k_cache"], t["block_table"], max_ctx)
    ws_sel = wd.select_workspace_tensor(B, W, args.vocab, dev)
    logits = [wl.make_logits_torch(scfg, i, dev) for i in range(args.logit_ring)]
    n_commit_hist = torch.zeros((total_steps, B), dtype=torch.int32, device=dev)
    committed = torch.empty((B, W), dtype=torch.int32, device=dev)
    argmax_hist = torch.empty((total_steps, B, W), dtype=torch.int32, device=dev)  # -1 on unmasked slots
    nsplit, split_keys = wd.wedlm_attn_plan(t["q_phys"], t["k_cache"], t["block_table"], max_ctx)
    tail = wd.wedlm_attn_tail(t["q_phys"], t["k_cache"], t["block_table"], max_ctx)

    def reorder():
        wd.wedlm_reorder(filled, pos, t["q"], t["k"], t["v"], t["q_phys"], t["k_cache"], t["v_cache"],
                         t["block_table"], ctx, t["perm"], cfg.rope_base, dev_status=t["status"])

    def attention():
        wd.wedlm_step_attn(t["q_phys"], t["k_cache"], t["v_cache"], t["block_table"], ctx, t["perm"],
                           t["out"], max_ctx_len=max_ctx, workspace=ws_attn, dev_status=t["status"])

    # prefix-cacheability counters (N_new, N_total) kept by the select call
    counters = torch.zeros((B, 2), dtype=torch.int64, device=dev)

    def select(i):
        wd.wedlm_select_commit(logits[i % len(logits)], tok, filled, pos, ctx, n_commit_hist[i], committed,
                               scfg.alpha, scfg.tau, mask_id, ws_sel, argmax_out=argmax_hist[i],
                               counters=counters)

    def three_calls(i):
        reorder()
        attention()
        select(i)

    # the same step as one wedlm_decode_step (three launches instead of five)
    ws_step = wd.decode_step_workspace_tensor(t["q"], t["k_cache"], t["block_table"], max_ctx, args.vocab)

    def fused(i):
        wd.wedlm_decode_step(filled, pos, t["q"], t["k"], t["v"], t["q_phys"], t["k_cache"], t["v_cache"],
                             t["block_table"], ctx, t["perm"], t["out"], cfg.rope_base, max_ctx,
                             logits[i % len(logits)], tok, n_commit_hist[i], committed, scfg.alpha, scfg.tau,
                             mask_id, ws_step, argmax_out=argmax_hist[i], counters=counters,
                             dev_status=t["status"])

    step, other = (three_calls, fused) if args.unfused else (fused, three_calls)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ctx_start = ctx.cpu().numpy().astype(np.int64)

    # ---- timed region 1: K whole streaming steps, nothing else on the stream.
    # First launched eagerly; then (default) the same K steps captured once
    # into a HIP graph and replayed from the same post-warm-up state, once
    # untimed and once timed.  Capture records without running; a replay from
    # the same state rewrites the same cache rows with the same bytes.
    state0 = [x.clone() for x in (tok, filled, pos, ctx)]
    def restart():
        for x, y in zip((tok, filled, pos, ctx), state0):
            x.copy_(y)
        counters.zero_()

    def timed(fn):
        """(eager seconds, replayed seconds or None) of K steps of fn from the
        post-warm-up state; leaves the state the K steps produce."""
        def eager_steps():
            for i in range(args.warmup, total_steps):
                fn(i)
        settle(eager_steps, restart)
        restart()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        eager_steps()
        torch.cuda.synchronize()
        eager_s = time.perf_counter() - t0
        if args.eager:
            return eager_s, None
        state_eager = [x.clone() for x in (tok, filled, pos, ctx, counters)]
        restart()
        graph = capture_steps(eager_steps)
        settle(graph.launch, restart)
        restart()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        graph.launch()
        torch.cuda.synchronize()
        replay_s = time.perf_counter() - t0
        for x, y in zip((tok, filled, pos, ctx, counters), state_eager):
            if not torch.equal(x, y):
                print("graph replay diverged from the eager steps", file=sys.stderr)
                sys.exit(3)
        return eager_s, replay_s

    # the other form of the step first (for comparison), then the measured one;
    # both must leave the same state
    other_eager, other_replay = timed(other)
    state_other = [x.clone() for x in (tok, filled, pos, ctx, counters, n_commit_hist, t["out"])]
    eager_elapsed, replay_elapsed = timed(step)
    elapsed = eager_elapsed if replay_elapsed is None else replay_elapsed
    for x, y in zip((tok, filled, pos, ctx, counters, n_commit_hist, t["out"]), state_other):
        if not torch.equal(x, y):
            print("wedlm_decode_step and the three calls diverged", file=sys.stderr)
            sys.exit(3)
    other_elapsed = other_eager if other_replay is None else other_replay
    cnt = counters.cpu().numpy()

    # ---- the dominant kernel inside the steps: the same K steps again from
    # the same state, launched one by one as wedlm_decode_step, each step's
    # attention kernel carrying start / stop events taken from its own
    # dispatch (no marker packet between the step's launches).  Its mean
    # duration is the roofline's launch duration; the pass ends in the state
    # the timed steps left (same steps, same bytes).
    stream = torch.cuda.current_stream()
    Kst = args.steps
    kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(Kst)]
    for e0, e1 in kev:          # create the event handles
        e0.record(stream)
        e1.record(stream)
    ctx_hist = torch.empty((Kst, B), dtype=torch.int32, device=dev)
    restart()
    for j, i in enumerate(range(args.warmup, total_steps)):
        ctx_hist[j].copy_(ctx)
        wd.wedlm_decode_step(filled, pos, t["q"], t["k"], t["v"], t["q_phys"], t["k_cache"], t["v_cache"],
                             t["block_table"], ctx, t["perm"], t["out"], cfg.rope_base, max_ctx,
                             logits[i % len(logits)], tok, n_commit_hist[i], committed, scfg.alpha, scfg.tau,
                             mask_id, ws_step, argmax_out=argmax_hist[i], counters=counters,
                             dev_status=t["status"], attn_events=kev[j])
    torch.cuda.synchronize()
    for x, y in zip((tok, filled, pos, ctx, counters, n_commit_hist, t["out"]), state_other):
        if not torch.equal(x, y):
            print("the kernel-timed steps diverged from the timed steps", file=sys.stderr)
            sys.exit(3)
    kern_ms_each = [e0.elapsed_time(e1) for e0, e1 in kev]
    L_hist = ctx_hist.cpu().numpy().astype(np.int64)

    # ---- timed region 2: the attention call alone (split kernel and
    # combine), K launches back to back on the stream it runs on (the state
    # the stream ended in), bracketed by one pair of HIP events on that
    # stream.  Untimed launches of the same call come first, in rounds of
    # ATTN_SETTLE for ATTN_SETTLE_S seconds.
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_end = time.perf_counter() + ATTN_SETTLE_S
    while time.perf_counter() < t_end:
        for _ in range(ATTN_SETTLE):
            attention()
        torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        attention()
    ev1.record(stream)
    ev1.synchronize()
    attn_avg_ms = ev0.elapsed_time(ev1) / args.steps
    L_now = ctx.cpu().numpy().astype(np.int64)

    # optional: the same call with the 256 MB MALL flushed before each launch
    # (a 1 GiB scratch write), timed launch by launch
    attn_cold_ms = None
    if args.cold:
        scratch = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        tot = 0.0
        for _ in range(args.steps):
            scratch.fill_(1.0)
            ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ea.record(stream)
            attention()
            eb.record(stream)
            eb.synchronize()
            tot += ea.elapsed_time(eb)
        attn_cold_ms = tot / args.steps
        del scratch

    # ---- timed region 3: the select/commit call alone on the last logits
    # buffer (state restored after), for its own bandwidth figure
    saved = [x.clone() for x in (tok, filled, pos, ctx)]
    nmask = int((filled == 0).sum().item())
    ev2, ev3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev2.record(stream)
    for i in range(args.steps):
        for x, y in zip((tok, filled, pos, ctx), saved):
            x.copy_(y)
        select(0)
    ev3.record(stream)
    ev3.synchronize()
    evc0, evc1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    evc0.record(stream)
    for i in range(args.steps):
        for x, y in zip((tok, filled, pos, ctx), saved):
            x.copy_(y)
    evc1.record(stream)
    evc1.synchronize()
    sel_ms = (ev2.elapsed_time(ev3) - evc0.elapsed_time(evc1)) / args.steps

    status = int(t["status"].item())
    if status != 0:
        print(f"device status {status} (bad ctx/page/perm)", file=sys.stderr)
        sys.exit(3)
    K = args.steps
    ms_step = elapsed * 1e3 / K
    nc = n_commit_hist.cpu().numpy().astype(np.int64)[args.warmup:]
    Hkv, Hq, D = cfg.Hkv, cfg.Hq, cfg.D
    eb = 2 if cfg.dtype == "bf16" else 4
    # algorithmic bytes of one attention launch at the final lengths: K and V
    # of every visible key read once, Q read, O written
    mean_attn_bytes = float(((L_now + W) * Hkv * D * 2 * eb).sum() + 2 * B * W * Hq * D * eb)
    achieved_call = mean_attn_bytes / (attn_avg_ms * 1e-3) / 1e9
    # the split kernel inside the steps: each step's bytes at that step's lengths
    step_bytes = ((L_hist + W) * Hkv * D * 2 * eb).sum(axis=1) + 2 * B * W * Hq * D * eb
    kern_ms = float(np.mean(kern_ms_each))
    achieved = float(step_bytes.sum()) / (float(np.sum(kern_ms_each)) * 1e-3) / 1e9
    # algorithmic flops: row r of a window sees L_b + r + 1 keys; 2D for QK
    # and 2D for PV per (row, key, query head)
    attn_flops = float((4 * D * Hq * (W * L_now + W * (W + 1) // 2)).sum())
    mfma_peak = MFMA_BF16_PEAK_TFLOPS * 1e12 if cfg.dtype == "bf16" else 157.3e12
    tokens_per_s = B * W / (ms_step * 1e-3)
    masked_rows = (argmax_hist[args.warmup:] >= 0).sum(dim=(1, 2)).cpu().numpy()
    sel_bytes = nmask * args.vocab * 4                                     # logits rows actually read
    sel_gbs = sel_bytes / (sel_ms * 1e-3) / 1e9

    result = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "window tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic",
        "graph": not args.eager,
        "step_call": "wedlm_reorder + wedlm_step_attn + wedlm_select_commit" if args.unfused else "wedlm_decode_step",
        "eager_ms_per_step": round(eager_elapsed * 1e3 / args.steps, 4),
        ("fused_ms_per_step" if args.unfused else "three_call_ms_per_step"): round(other_elapsed * 1e3 / args.steps, 4),
        "config": {"workload": f"{cfg.name}: B={B} W={W} Hq={Hq} Hkv={Hkv} D={D} "
                               f"prefix={int(inp.ctx_len.max()) if cfg.L_range is None else str(cfg.L_range)} "
                               f"page=16 vocab={args.vocab} streaming decode step (reorder+attn+select/commit)",
                   "batch": B, "window": W, "prefix_tokens_at_start": int(ctx_start.max()),
                   "vocab": args.vocab, "split_kv": [nsplit, split_keys], "tail_splits": tail},
        "steps_per_s": round(1e3 / ms_step, 2),
        "attn_kernel_in_steps": {"kernel": f"attn_split_{'bf16' if cfg.dtype == 'bf16' else 'f32'}",
                                 "avg_ms": round(kern_ms, 5), "min_ms": round(float(np.min(kern_ms_each)), 5),
                                 "max_ms": round(float(np.max(kern_ms_each)), 5),
                                 "alg_bytes_per_launch": int(step_bytes.mean()),
                                 "GB_per_s": round(achieved, 1),
                                 "frac_of_hbm_peak": round(achieved / HBM_PEAK_GBS, 4)},
        "attn": {"avg_ms": round(attn_avg_ms, 5), "alg_bytes_per_launch": int(mean_attn_bytes),
                 "GB_per_s": round(achieved_call, 1), "frac_of_hbm_peak": round(achieved_call / HBM_PEAK_GBS, 4),
                 "prefix_tokens": [int(x) for x in L_now],
                 "alg_flops_per_launch": int(attn_flops),
                 "TFLOP_per_s": round(attn_flops / (attn_avg_ms * 1e-3) / 1e12, 1),
                 "mfma_frac_of_dense_peak": round(attn_flops / (attn_avg_ms * 1e-3) / mfma_peak, 4),
                 **({"cold_avg_ms": round(attn_cold_ms, 5),
                     "cold_GB_per_s": round(mean_attn_bytes / (attn_cold_ms * 1e-3) / 1e9, 1)}
                    if attn_cold_ms is not None else {})},
        "select_commit": {"avg_ms": round(sel_ms, 5), "masked_rows": nmask, "GB_per_s": round(sel_gbs, 1),
                          "masked_rows_per_step_in_stream": float(masked_rows.mean())},
        "tokens_committed_per_step": round(float(nc.sum(1).mean()), 3),
        # P_c = N_new / N_total over the timed steps, from the library's
        # device counters (committed tokens over window slots processed)
        "P_c": round(float(cnt[:, 0].sum()) / float(max(cnt[:, 1].sum(), 1)), 4),
        "counters": {"N_new": int(cnt[:, 0].sum()), "N_total": int(cnt[:, 1].sum()),
                     "matches_commit_history": bool(int(cnt[:, 0].sum()) == int(nc.sum())
                                                    and int(cnt[:, 1].sum()) == K * B * W)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": recorded_traffic(workload),
                     "kernel": f"attn_split_{'bf16' if cfg.dtype == 'bf16' else 'f32'}, the decode step's "
                               "attention launch, inside the timed steps (start / stop from its dispatch)"},
    }

    if with_cpu:
        result["cpu_baseline"] = cpu_baseline(cfg, args, inp)
    del t, ws_attn, ws_sel, ws_step, logits
    torch.cuda.empty_cache()
    return result


def bench_select(args, emit=True):
    """The select/commit call alone, streaming: batch 64 x window 16 over
    V=151936 fp32 logits, starting from an all-masked window at prefix 0.  A
    step is one wedlm_select_commit (vocabulary statistics of every masked
    slot, commit, Eq. 11 fill, refill); the logits of step i are buffer
    i mod --logit-ring (each 622 MB, so none stays in the 256 MB MALL)."""
    import torch
    import workloads as wl
    import causal_attention_diffusion_amd as wd

    dev = torch.device("cuda:0")
    cfg = wl.SELECT_CONFIGS["select_v152k"]
    B, W, V = cfg.B, cfg.W, cfg.V
    total = args.warmup + args.steps
    logits = [wl.make_logits_torch(cfg, i, dev) for i in range(args.logit_ring)]
    ws = wd.select_workspace_tensor(B, W, V, dev)
    init = [torch.from_numpy(x).to(dev) for x in wl.initial_window(B, W, V)]
    tok, filled, pos, ctx = [x.clone() for x in init]
    n_commit_hist = torch.zeros((total, B), dtype=torch.int32, device=dev)
    committed = torch.empty((B, W), dtype=torch.int32, device=dev)
    argmax_hist = torch.empty((total, B, W), dtype=torch.int32, device=dev)  # -1 on unmasked slots

    def step(i):
        wd.wedlm_select_commit(logits[i % len(logits)], tok, filled, pos, ctx, n_commit_hist[i], committed,
                               cfg.alpha, cfg.tau, V, ws, argmax_out=argmax_hist[i])

    def reset():
        for x, y in zip((tok, filled, pos, ctx), init):
            x.copy_(y)

    for i in range(args.warmup):
        step(i)
    # timed: K steps from the all-masked start, eagerly (HIP events on the
    # stream bracket exactly the K calls), then replayed as one HIP graph
    settle(lambda: [step(i) for i in range(args.warmup, total)], reset)
    reset()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.warmup, total):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    eager_elapsed = time.perf_counter() - t0
    call_ms = ev0.elapsed_time(ev1) / args.steps
    state_eager = [x.clone() for x in (tok, filled, pos, ctx)]
    elapsed = eager_elapsed
    if not args.eager:
        reset()
        graph = capture_steps(lambda: [step(i) for i in range(args.warmup, total)])
        settle(graph.launch, reset)
        reset()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        graph.launch()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        for x, y in zip((tok, filled, pos, ctx), state_eager):
            if not torch.equal(x, y):
                print("graph replay diverged from the eager steps", file=sys.stderr)
                sys.exit(3)

    K = args.steps
    ms_step = elapsed * 1e3 / K
    masked = (argmax_hist[args.warmup:] >= 0).sum(dim=(1, 2)).cpu().numpy().astype(np.int64)
    nc = n_commit_hist[args.warmup:].cpu().numpy().astype(np.int64)
    # algorithmic bytes: every masked slot's logits row read once
    alg_bytes = float(masked.sum()) * V * 4 / K
    achieved = alg_bytes / (call_ms * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(B * W / (ms_step * 1e-3), 1),
        "unit": "window tokens/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic", "graph": not args.eager,
        "eager_ms_per_step": round(eager_elapsed * 1e3 / K, 4),
        "config": {"workload": f"select_v152k: B={B} W={W} vocab={V} fp32 logits (low/high-entropy "
                               f"mixture), alpha={cfg.alpha} tau={cfg.tau}, {K} streaming select/commit "
                               f"steps from an all-masked window",
                   "batch": B, "window": W, "vocab": V, "logit_buffers": len(logits)},
        "steps_per_s": round(1e3 / ms_step, 2),
        "select_commit": {"avg_ms": round(call_ms, 5), "alg_bytes_per_launch": int(alg_bytes),
                          "masked_rows_per_step": round(float(masked.mean()), 2),
                          "GB_per_s": round(achieved, 1)},
        "tokens_committed_per_step": round(float(nc.sum(1).mean()), 3),
        "P_c": round(float(nc.sum()) / (K * B * W), 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "wedlm_select_commit (vocab_stats + commit_select_refill)"},
    }
    if emit and not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline_select(cfg, args)
    del logits, ws
    torch.cuda.empty_cache()
    if emit:
        print(json.dumps(result), flush=True)
    return result


def bench_lmhead(args):
    """The fused LM head + select call alone, streaming: batch 64 x window 16,
    hidden size 4096, V=151936 (Qwen3-8B's output projection), from an
    all-masked window.  Step i reads hidden-state buffer i mod --logit-ring
    (seeded device draws); the output embeddings are one seeded draw."""
    import torch
    import workloads as wl
    import causal_attention_diffusion_amd as wd

    dev = torch.device("cuda:0")
    cfg = wl.LMHEAD_CONFIGS["lmhead_v152k"]
    B, W, V, Dm = cfg.B, cfg.W, cfg.V, cfg.Dm
    total = args.warmup + args.steps
    w = wl.make_lm_head_torch(cfg, dev)
    hidden = [wl.make_hidden_torch(cfg, i, w, dev) for i in range(args.logit_ring)]
    ws = wd.lmhead_workspace_tensor(B, W, V, Dm, dev)
    init = [torch.from_numpy(x).to(dev) for x in wl.initial_window(B, W, V)]
    tok, filled, pos, ctx = [x.clone() for x in init]
    n_commit_hist = torch.zeros((total, B), dtype=torch.int32, device=dev)
    committed = torch.empty((B, W), dtype=torch.int32, device=dev)
    argmax_hist = torch.empty((total, B, W), dtype=torch.int32, device=dev)

    def step(i):
        wd.wedlm_lmhead_select_commit(hidden[i % len(hidden)], w, tok, filled, pos, ctx, n_commit_hist[i],
                                      committed, cfg.alpha, cfg.tau, V, ws, argmax_out=argmax_hist[i])

    def reset():
        for x, y in zip((tok, filled, pos, ctx), init):
            x.copy_(y)

    for i in range(args.warmup):
        step(i)
    settle(lambda: [step(i) for i in range(args.warmup, total)], reset)
    reset()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.warmup, total):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    eager_elapsed = time.perf_counter() - t0
    call_ms = ev0.elapsed_time(ev1) / args.steps
    state_eager = [x.clone() for x in (tok, filled, pos, ctx)]
    elapsed = eager_elapsed
    if not args.eager:
        reset()
        graph = capture_steps(lambda: [step(i) for i in range(args.warmup, total)])
        settle(graph.launch, reset)
        reset()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        graph.launch()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        for x, y in zip((tok, filled, pos, ctx), state_eager):
            if not torch.equal(x, y):
                print("graph replay diverged from the eager steps", file=sys.stderr)
                sys.exit(3)

    K = args.steps
    ms_step = elapsed * 1e3 / K
    masked = (argmax_hist[args.warmup:] >= 0).sum(dim=(1, 2)).cpu().numpy().astype(np.int64)
    nc = n_commit_hist[args.warmup:].cpu().numpy().astype(np.int64)
    # algorithmic work per call: 2 Dm flops per (masked row, vocabulary entry);
    # bytes: the output embeddings once plus the masked rows' hidden states
    flops = 2.0 * float(masked.mean()) * Dm * V
    alg_bytes = float(V) * Dm * 2 + float(masked.mean()) * Dm * 2
    tflops = flops / (call_ms * 1e-3) / 1e12
    result = {
        "metric": METRIC,
        "value": round(B * W / (ms_step * 1e-3), 1),
        "unit": "window tokens/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic", "graph": not args.eager,
        "eager_ms_per_step": round(eager_elapsed * 1e3 / K, 4),
        "config": {"workload": f"lmhead_v152k: B={B} W={W} hidden={Dm} vocab={V} bf16 LM head fused with "
                               f"select/commit (alpha={cfg.alpha} tau={cfg.tau}), {K} streaming steps from "
                               f"an all-masked window",
                   "batch": B, "window": W, "hidden": Dm, "vocab": V, "hidden_buffers": len(hidden)},
        "steps_per_s": round(1e3 / ms_step, 2),
        "lmhead_select_commit": {"avg_ms": round(call_ms, 5), "masked_rows_per_step": round(float(masked.mean()), 2),
                                 "alg_flops_per_launch": int(flops), "TFLOP_per_s": round(tflops, 1),
                                 "weights_GB_per_s": round(alg_bytes / (call_ms * 1e-3) / 1e9, 1),
                                 "logits_bytes_not_written_per_step": int(masked.mean() * V * 4)},
        "tokens_committed_per_step": round(float(nc.sum(1).mean()), 3),
        "P_c": round(float(nc.sum()) / (K * B * W), 4),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "wedlm_lmhead_select_commit (lmhead_stats + merge + commit)"},
    }
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline_lmhead(cfg, args, w, hidden[0])
    print(json.dumps(result), flush=True)


def bench_dual(args):
    """Dual-Stream Masking attention forward: 4 sequences of 4096 tokens,
    blocks of 32, 32 query / 8 KV heads of 128, bf16, RoPE base 1e6.  Both
    streams N(0,1); each block's observed fraction is drawn uniformly in
    [0.2, 0.8] and its observed tokens at random.  A step is one call (both
    streams of all sequences)."""
    import torch
    import causal_attention_diffusion_amd as wd

    dev = torch.device("cuda:0")
    S, N, b, Hq, Hkv, D = 4, 4096, 32, 32, 8, 128
    g = torch.Generator(device=dev)
    g.manual_seed(1401)

    def draw(h):
        return torch.randn((S, N, h, D), generator=g, device=dev).to(torch.bfloat16)

    qm, km, vm, qp, kp, vp = draw(Hq), draw(Hkv), draw(Hkv), draw(Hq), draw(Hkv), draw(Hkv)
    frac = torch.rand((S, N // b, 1), generator=g, device=dev) * 0.6 + 0.2
    flags = (torch.rand((S, N // b, b), generator=g, device=dev) < frac).reshape(S, N).to(torch.uint8)
    out_m, out_p = torch.empty_like(qm), torch.empty_like(qp)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = wd.dual_stream_workspace_tensor(qm, km, b)

    def step():
        wd.wedlm_dual_stream_attn(qm, km, vm, qp, kp, vp, flags, out_m, out_p, b, 1e6, ws, dev_status=status)

    for _ in range(args.warmup):
        step()
    settle(lambda: [step() for _ in range(args.steps)], lambda: None)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    call_ms = ev0.elapsed_time(ev1) / args.steps
    if status.item() != 0:
        print(f"device status {status.item()}", file=sys.stderr)
        sys.exit(3)
    # algorithmic bytes: every window reads K and V of its visible keys once
    # (memory: 64-token windows c see 64(c+1) keys; prediction: block i sees
    # b(i+1)), plus q, k, v of both streams in and both outputs out
    nm, nb = N // 64, N // b
    keys = S * (64 * nm * (nm + 1) // 2 + b * nb * (nb + 1) // 2)
    alg_bytes = float(keys) * Hkv * D * 2 * 2 + 2.0 * S * N * (2 * Hq + 2 * Hkv) * D * 2
    # flops: 4 D per (query head, visible key) -- memory token t sees t+1
    # keys; physical row r of prediction block i sees the i*b memory tokens
    # before the block and r+1 tokens of its own block
    pairs_m = N * (N + 1) // 2
    pairs_p = sum(i * b * b for i in range(nb)) + nb * b * (b + 1) // 2
    flops = 4.0 * D * Hq * S * (pairs_m + pairs_p)
    tflops = flops / (call_ms * 1e-3) / 1e12
    gbs = alg_bytes / (call_ms * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(2 * S * N / (call_ms * 1e-3), 1),
        "unit": "tokens/s (both streams)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(call_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic", "graph": False, "wall_ms_per_step": round(wall * 1e3 / args.steps, 4),
        "config": {"workload": f"dualstream_n4096: {S} sequences x {N} tokens, blocks of {b}, Hq={Hq} Hkv={Hkv} "
                               f"D={D} bf16, memory + prediction stream attention",
                   "sequences": S, "tokens": N, "block": b},
        # the call is bound by the matrix cores, not by HBM: the K/V of
        # both streams (S*N*Hkv*D*2 bytes each, 67 MB) fit the 256 MB MALL
        # and are re-read from there by every window
        "dual_stream": {"avg_ms": round(call_ms, 5), "alg_flops_per_launch": int(flops),
                        "TFLOP_per_s": round(tflops, 1),
                        "window_kv_bytes_per_launch": int(alg_bytes), "window_kv_GB_per_s": round(gbs, 1),
                        "unique_kv_bytes": int(2 * S * N * Hkv * D * 2 * 2)},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "wedlm_dual_stream_attn (layout + 2 x (reorder + attn_split + combine))"},
    }
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline_dual(args, [x[:1].float().cpu().numpy().astype(np.float64)
                                                          for x in (qm, km, vm, qp, kp, vp)],
                                                   flags[:1].cpu().numpy(), b)
    print(json.dumps(result), flush=True)


def bench_model(args):
    """Whole decode steps of the synthetic decoder (wedlm_model_step):
    Qwen3-8B shapes (36 layers, hidden 4096, 32 / 8 heads of 128, SwiGLU
    12288, vocabulary 151936), random bf16 weights (embeddings N(0,1),
    projections N(0, 1/fan_in), norms 1 + 0.1 N(0,1)), batch 4 x window 64,
    each sequence with a 2048-token cached prompt (K/V N(0,1) bf16 in
    shuffled 16-token pages).  Steps stream from an all-masked window."""
    import torch
    import workloads as wl
    import causal_attention_diffusion_amd as wd

    dev = torch.device("cuda:0")
    cfg = wl.MODEL_CONFIGS["model_qwen3_w64"]
    B, W, L0 = cfg.B, cfg.W, cfg.prefix
    total = args.warmup + args.steps
    max_ctx = L0 + total * W
    mp = (max_ctx + W + 15) // 16
    pool = B * mp
    g = torch.Generator(device=dev)
    g.manual_seed(cfg.seed + 11)
    w = wl.make_model_torch(cfg, dev)
    for lw in w["layers"]:
        lw["k_cache"] = torch.randn((pool, cfg.Hkv, 16, cfg.D), generator=g, device=dev).to(torch.bfloat16)
        lw["v_cache"] = torch.randn((pool, cfg.Hkv, 16, cfg.D), generator=g, device=dev).to(torch.bfloat16)
    bt = torch.randperm(pool, generator=g, device=dev).to(torch.int32).reshape(B, mp)
    handle = wd.ModelHandle(w, cfg.eps)
    shape = wd.make_shape(B, W, cfg.Hq, cfg.Hkv, cfg.D, mp, pool, wd.WEDLM_BF16)
    ws = wd.model_step_workspace_tensor(handle, shape, max_ctx, dev)
    init = [torch.from_numpy(x).to(dev) for x in wl.initial_window(B, W, cfg.vocab, L0)]
    tok, filled, pos, ctx = [x.clone() for x in init]
    n_commit_hist = torch.zeros((total, B), dtype=torch.int32, device=dev)
    committed = torch.empty((B, W), dtype=torch.int32, device=dev)
    argmax_hist = torch.empty((total, B, W), dtype=torch.int32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)

    def step(i):
        wd.wedlm_model_step(handle, shape, bt, tok, filled, pos, ctx, n_commit_hist[i], committed, cfg.alpha,
                            cfg.tau, cfg.rope_base, max_ctx, ws, argmax_out=argmax_hist[i], dev_status=status)

    def reset():
        for x, y in zip((tok, filled, pos, ctx), init):
            x.copy_(y)

    for i in range(args.warmup):
        step(i)
    settle(lambda: [step(i) for i in range(args.warmup, total)], reset)
    reset()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.warmup, total):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    eager_elapsed = time.perf_counter() - t0
    call_ms = ev0.elapsed_time(ev1) / args.steps
    if status.item() != 0:
        print(f"device status {status.item()}", file=sys.stderr)
        sys.exit(3)
    ctx_eager = ctx.clone()
    state_eager = [x.clone() for x in (tok, filled, pos, ctx)]
    elapsed = eager_elapsed
    if not args.eager:
        reset()
        graph = capture_steps(lambda: [step(i) for i in range(args.warmup, total)])
        settle(graph.launch, reset)
        reset()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        graph.launch()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        for x, y in zip((tok, filled, pos, ctx), state_eager):
            if not torch.equal(x, y):
                print("graph replay diverged from the eager steps", file=sys.stderr)
                sys.exit(3)

    K = args.steps
    ms_step = elapsed * 1e3 / K
    d, F, V, Lyr = cfg.d_model, cfg.d_ff, cfg.vocab, cfg.layers
    kvw = cfg.Hkv * cfg.D
    layer_params = 2 * d * d + 2 * kvw * d + 3 * F * d
    masked = (argmax_hist[args.warmup:] >= 0).sum(dim=(1, 2)).cpu().numpy().astype(np.float64)
    nc = n_commit_hist[args.warmup:].cpu().numpy().astype(np.int64)
    # context of the timed steps: L0 at the first, then growing by the commits
    ctx_start = L0 + np.concatenate([np.zeros((1, B), np.int64), np.cumsum(nc, 0)[:-1]], 0)
    keys_mean = float((ctx_start + W).sum(1).mean())
    # algorithmic bytes per step: every weight once (layers, final norm, LM
    # head), the window rows of the embedding, every layer's cached K/V of
    # each visible key once and the window's K/V appended
    alg_bytes = (Lyr * (layer_params + 2 * d) + d + V * d + B * W * d) * 2.0 \
        + Lyr * (keys_mean * kvw * 2 * 2 + B * W * kvw * 2 * 2)
    flops = Lyr * 2.0 * B * W * layer_params + 2.0 * float(masked.mean()) * d * V \
        + Lyr * 4.0 * cfg.Hq * cfg.D * W * keys_mean
    gbs = alg_bytes / (call_ms * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(B * W / (ms_step * 1e-3), 1),
        "unit": "window tokens/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (random weights)", "graph": not args.eager,
        "eager_ms_per_step": round(eager_elapsed * 1e3 / K, 4),
        "config": {"workload": f"model_qwen3_w64: {Lyr}-layer synthetic decoder of Qwen3-8B shapes (hidden {d}, "
                               f"{cfg.Hq}/{cfg.Hkv} heads of {cfg.D}, MLP {F}, vocab {V}), B={B} x W={W} window, "
                               f"{L0}-token cached prompt, {K} streaming steps from an all-masked window",
                   "batch": B, "window": W, "layers": Lyr, "hidden": d, "vocab": V, "prompt": L0},
        "steps_per_s": round(1e3 / ms_step, 2),
        "model_step": {"avg_ms": round(call_ms, 5), "alg_bytes_per_step": int(alg_bytes),
                       "GB_per_s": round(gbs, 1), "alg_flops_per_step": int(flops),
                       "TFLOP_per_s": round(flops / (call_ms * 1e-3) / 1e12, 1),
                       "masked_rows_per_step": round(float(masked.mean()), 2),
                       "final_ctx": ctx_eager.cpu().tolist()},
        "tokens_committed_per_step": round(float(nc.sum(1).mean()), 3),
        "P_c": round(float(nc.sum()) / (K * B * W), 4),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "wedlm_model_step (all launches of one decode step)"},
    }
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline_model(cfg, w, bt)
    print(json.dumps(result), flush=True)


def cpu_baseline_model(cfg, w_dev, bt):
    """The oracle's model step, untuned, on the host cores, for the first
    sequence of the first step (64 masked rows after the 2048-token prompt),
    on the bench's own bf16 weights and caches copied to the host.  It runs
    with the first layer, then the first four; the 36-layer step time is
    t(4) + 32 (t(4) - t(1)) / 3."""
    import oracle
    import workloads as wl

    def host(t):
        return t.float().cpu().numpy().astype(np.float64)

    L0, W = cfg.prefix, cfg.W
    top = {"embed": host(w_dev["embed"]), "final_norm": host(w_dev["final_norm"]),
           "lm_head": host(w_dev["lm_head"])}
    layers, caches = [], []
    import torch
    t = torch.arange(L0, device=bt.device)
    pg = bt[0].long()[t // 16], t % 16
    for l in range(4):
        lw = w_dev["layers"][l]
        layers.append({k: host(v) for k, v in lw.items() if k not in ("k_cache", "v_cache")})
        kc = lw["k_cache"][pg[0], :, pg[1], :]
        vc = lw["v_cache"][pg[0], :, pg[1], :]
        caches.append(([host(kc)], [host(vc)]))
    tok, filled, pos, ctx = wl.initial_window(1, W, cfg.vocab, L0)
    times = {}
    for n in (1, 4):
        wn = dict(top, layers=layers[:n])
        best = None
        for _ in range(2):
            t0 = time.perf_counter()
            oracle.model_step(wn, caches[:n], tok, filled, pos, ctx, cfg.alpha, cfg.tau, cfg.rope_base, cfg.eps,
                              cfg.Hq, cfg.Hkv)
            dt = time.perf_counter() - t0
            best = dt if best is None else min(best, dt)
        times[n] = best
    per_layer = max(times[4] - times[1], 0.0) / 3
    est = times[4] + (cfg.layers - 4) * per_layer
    return {"value": round(W / est, 3), "unit": "window tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"sequence 0 of the first step ({W} masked rows, {L0}-token prompt) with 1 and 4 layers "
                      f"({times[1]:.2f} s, {times[4]:.2f} s, best of 2); {cfg.layers}-layer step estimated as "
                      f"t4 + {cfg.layers - 4} (t4 - t1) / 3 = {est:.2f} s"}


def cpu_baseline_dual(args, arrs, flags, b):
    """The oracle on sampled tokens of the first sequence (both streams),
    scaled to tokens/s."""
    import oracle
    N = arrs[0].shape[1]
    rng = np.random.default_rng(5)
    reps, dt_s, n = 0, 0.0, 0
    while reps < 64 and dt_s < 10.0:
        toks = rng.integers(0, N, 16)
        rows = np.array([(0, st, t) for st in (0, 1) for t in toks])
        t0 = time.perf_counter()
        oracle.dual_stream_attention(*arrs, flags, b, "bf16", 1e6, rows=rows)
        dt_s += time.perf_counter() - t0
        n += len(rows)
        reps += 1
    return {"value": round(n / dt_s, 2), "unit": "tokens/s (both streams)", "cores": oracle.num_threads(),
            "kind": "oracle", "sample": f"{n} uniformly drawn tokens of one 4096-token sequence (both "
                                        f"streams, all 32 heads); {dt_s:.2f} s"}


def cpu_baseline_lmhead(cfg, args, w_dev, h_dev):
    """The oracle's LM head + select step, untuned, on the host cores, for one
    sequence of the all-masked first step (16 rows x 151936 x 4096), on the
    bench's own bf16 inputs copied to the host."""
    import oracle
    import workloads as wl
    w64 = w_dev.float().cpu().numpy().astype(np.float64)
    h64 = h_dev[:1].float().cpu().numpy().astype(np.float64)
    tok, filled, pos, ctx = wl.initial_window(1, cfg.W, cfg.V)
    reps, dt_s = 0, 0.0
    while reps < 64 and dt_s < 10.0:
        t0 = time.perf_counter()
        oracle.lmhead_select_commit(h64, w64, tok, filled, pos, ctx, cfg.alpha, cfg.tau, cfg.V)
        dt_s += time.perf_counter() - t0
        reps += 1
    return {"value": round(reps * cfg.W / dt_s, 2), "unit": "window tokens/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"1 of {cfg.B} sequences of the first step ({cfg.W} masked rows, hidden {cfg.Dm}, "
                      f"V={cfg.V}) repeated {reps}x; {dt_s:.2f} s"}


def cpu_baseline_select(cfg, args):
    """The oracle's select/commit step, untuned, on the host cores, over the
    whole batch from the all-masked start (every row masked: the largest
    step of the stream), in window tokens/s."""
    import oracle
    import workloads as wl
    lg = wl.make_logits_np(cfg, 0)
    tok, filled, pos, ctx = wl.initial_window(cfg.B, cfg.W, cfg.V)
    reps, dt_s = 0, 0.0
    while reps < 64 and dt_s < 10.0:
        t0 = time.perf_counter()
        oracle.select_commit(lg, tok, filled, pos, ctx, cfg.alpha, cfg.tau, cfg.V)
        dt_s += time.perf_counter() - t0
        reps += 1
    return {"value": round(reps * cfg.B * cfg.W / dt_s, 1), "unit": "window tokens/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"the first step ({cfg.B} x {cfg.W} masked rows over V={cfg.V}) repeated {reps}x; "
                      f"{dt_s:.2f} s"}


def attn_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        with open(os.path.join(ROOT, "causal_attention_diffusion_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(workload):
    """HBM bytes per launch of the split kernel (the roofline's kernel) from
    the committed counter summary, or None
    when the workload or the attention sources differ from the profiled
    ones (the figure belongs to that kernel build; the context grows by a
    few hundred tokens over a run, a change of well under 1 %)."""
    try:
        with open(TRAFFIC_FILE) as fh:
            kv = dict(line[2:].split(": ", 1) for line in fh.read().splitlines()
                      if line.startswith("- ") and ": " in line)
    except OSError:
        return None
    if kv.get("source_sha256", "").strip("` ") != attn_source_hash():
        return None
    if kv.get("workload", "").strip("` ") != workload:
        return None
    try:
        return int(kv["split_kernel_traffic_bytes_per_launch"].strip("` "))
    except (KeyError, ValueError):
        return None


def cpu_baseline(cfg, args, inp):
    """The oracle, untuned, on the host cores: one whole decode step (reorder,
    attention of every row, select/commit over the full vocabulary) for a
    sample of the batch's sequences, reported in window tokens/s."""
    import oracle
    import workloads as wl
    nseq = args.cpu_seqs or cfg.B
    sel = list(range(nseq))
    dt = cfg.dtype
    q = wl.storage_to_f64(inp.q[sel], dt)
    k = wl.storage_to_f64(inp.k[sel], dt)
    v = wl.storage_to_f64(inp.v[sel], dt)
    pk = [wl.storage_to_f64(inp.prefix_k[b], dt) for b in sel]
    pv = [wl.storage_to_f64(inp.prefix_v[b], dt) for b in sel]
    scfg = wl.SelectConfig("cpu", B=nseq, W=cfg.W, V=args.vocab, seed=1005, alpha=0.25, tau=9.0,
                           steps=0, kind="mixture")
    lg = wl.make_logits_np(scfg, 0)
    tok = np.where(inp.filled[sel] == 1, 1, args.vocab).astype(np.int32)
    # the same step repeated until about 10 s of CPU work (at most 4 times)
    reps, dt_s = 0, 0.0
    while reps < 4 and dt_s < 10.0:
        t0 = time.perf_counter()
        perm, qp, kw, vw = oracle.reorder(inp.filled[sel], inp.pos[sel], q, k, v, dt, cfg.rope_base)
        dk = [np.concatenate([pk[i], kw[i]], 0) for i in range(nseq)]
        dv = [np.concatenate([pv[i], vw[i]], 0) for i in range(nseq)]
        oracle.attention(qp, dk, dv, inp.ctx_len[sel], perm)
        oracle.select_commit(lg, tok, inp.filled[sel], inp.pos[sel], inp.ctx_len[sel], 0.25, 9.0, args.vocab)
        dt_s += time.perf_counter() - t0
        reps += 1
    return {"value": round(reps * nseq * cfg.W / dt_s, 3), "unit": "window tokens/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{nseq} of {cfg.B} sequences, one full step (reorder, all {cfg.W * cfg.Hq} "
                      f"attention rows per sequence, select/commit over V={args.vocab}) repeated "
                      f"{reps}x; {dt_s:.2f} s"}


if __name__ == "__main__":
    main()
