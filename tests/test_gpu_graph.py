"""Decode steps captured in a HIP graph replay exactly like the same steps
run eagerly -- captured by torch and by the library's own capture API
(wedlm_graph_*).

Three whole steps (reorder, attention, select/commit) on the Qwen3-8B-shaped
single-layer workload are captured once and replayed four times, each replay
from the same restored state, with eager work and synchronisation of the
program between replays.  Every replay must reproduce the eager run's bytes:
committed counts and tokens, attention outputs, window state and the K/V
cache.  None of the library's calls allocates, synchronises or clears memory,
so the whole step can sit in a graph."""
import numpy as np
import pytest
import torch

import workloads as wl
import causal_attention_diffusion_amd as wd

pytestmark = pytest.mark.gpu


def _decode_setup(dev, steps=3, V=4096):
    cfg = wl.CONFIGS["qwen3_l2048"]
    scfg = wl.SelectConfig("graph", B=cfg.B, W=cfg.W, V=V, seed=77, alpha=0.25, tau=6.0, steps=0,
                           kind="mixture")
    inp = wl.make_attn_inputs(cfg, spare_tokens=(steps + 1) * cfg.W)
    t = wl.device_attn_inputs(inp, dev)
    max_ctx = int(inp.ctx_len.max()) + (steps + 1) * cfg.W
    ws_attn = wd.attn_workspace_tensor(t["q_phys"], t["k_cache"], t["block_table"], max_ctx)
    ws_sel = wd.select_workspace_tensor(cfg.B, cfg.W, V, dev)
    logits = [wl.make_logits_torch(scfg, i, dev) for i in range(steps)]
    tok = torch.from_numpy(np.where(inp.filled == 1, 5, V).astype(np.int32)).to(dev)
    n_commit = torch.zeros((steps, cfg.B), dtype=torch.int32, device=dev)
    committed = torch.zeros((steps, cfg.B, cfg.W), dtype=torch.int32, device=dev)
    counters = torch.zeros((cfg.B, 2), dtype=torch.int64, device=dev)
    outs = torch.zeros((steps,) + tuple(t["out"].shape), dtype=t["out"].dtype, device=dev)
    state = (tok, t["filled"], t["pos"], t["ctx_len"], t["k_cache"], t["v_cache"])

    def run():
        for i in range(steps):
            wd.wedlm_reorder(t["filled"], t["pos"], t["q"], t["k"], t["v"], t["q_phys"], t["k_cache"],
                             t["v_cache"], t["block_table"], t["ctx_len"], t["perm"], cfg.rope_base,
                             dev_status=t["status"])
            wd.wedlm_step_attn(t["q_phys"], t["k_cache"], t["v_cache"], t["block_table"], t["ctx_len"],
                               t["perm"], outs[i], max_ctx_len=max_ctx, workspace=ws_attn,
                               dev_status=t["status"])
            wd.wedlm_select_commit(logits[i], tok, t["filled"], t["pos"], t["ctx_len"], n_commit[i],
                                   committed[i], scfg.alpha, scfg.tau, V, ws_sel, counters=counters)

    saved = [x.clone() for x in state]

    def restore():
        for x, y in zip(state, saved):
            x.copy_(y)
        for x in (n_commit, committed, outs, counters):
            x.zero_()

    def snapshot():
        return [x.clone() for x in (n_commit, committed, outs, counters) + state]

    return t, run, restore, snapshot, n_commit


def _replays_match(replay, restore, snapshot, ref, dev):
    for rep in range(4):
        restore()
        torch.randn(4096, device=dev).sum().item()   # the program's own eager work
        torch.cuda.synchronize()
        replay()
        torch.cuda.synchronize()
        got = snapshot()
        for k, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a, b), (rep, k)


def test_captured_steps_replay_like_eager(dev):
    print("[graph] qwen3_l2048 x3 steps, V=4096, torch capture", flush=True)
    t, run, restore, snapshot, n_commit = _decode_setup(dev)
    run()
    torch.cuda.synchronize()
    ref = snapshot()
    assert int(n_commit.sum().item()) > 0          # the steps did commit something

    restore()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            run()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    _replays_match(graph.replay, restore, snapshot, ref, dev)
    assert t["status"].item() == 0


def test_native_capture_replays_like_eager(dev):
    # the library's own capture API (wedlm_graph_begin / end / launch):
    # three steps = 15 kernel nodes (reorder, split attention, combine,
    # vocabulary statistics, commit) and nothing else -- no memset nodes
    print("[graph] qwen3_l2048 x3 steps, V=4096, native capture", flush=True)
    t, run, restore, snapshot, n_commit = _decode_setup(dev)
    run()
    torch.cuda.synchronize()
    ref = snapshot()
    restore()
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()
    with wd.capture(cap) as g:
        run()
    assert g.nodes() == (15, 0), g.nodes()
    _replays_match(g.launch, restore, snapshot, ref, dev)
    g.close()
    assert t["status"].item() == 0


def test_native_capture_of_model_steps(dev):
    # two whole synthetic-decoder steps (every layer, LM head, select and the
    # hidden-state copy) as one native graph, replayed like the eager run
    print("[graph] model_small x2 steps, native capture", flush=True)
    cfg = wl.MODEL_CONFIGS["model_small"]
    steps, B, W = 2, cfg.B, cfg.W
    tw = wl.make_model_torch(cfg, dev)
    mp = (steps * W + W + 15) // 16
    pool = B * mp
    for lw in tw["layers"]:
        lw["k_cache"] = torch.zeros((pool, cfg.Hkv, 16, cfg.D), dtype=torch.bfloat16, device=dev)
        lw["v_cache"] = torch.zeros_like(lw["k_cache"])
    bt = torch.arange(pool, dtype=torch.int32, device=dev).reshape(B, mp)
    handle = wd.ModelHandle(tw, cfg.eps)
    shape = wd.make_shape(B, W, cfg.Hq, cfg.Hkv, cfg.D, mp, pool, wd.WEDLM_BF16)
    ws = wd.model_step_workspace_tensor(handle, shape, steps * W, dev)
    init = [torch.from_numpy(x).to(dev) for x in wl.initial_window(B, W, cfg.vocab)]
    tok, filled, pos, ctx = [x.clone() for x in init]
    n_commit = torch.zeros((steps, B), dtype=torch.int32, device=dev)
    committed = torch.zeros((steps, B, W), dtype=torch.int32, device=dev)
    hid = torch.zeros((steps, B, W, cfg.d_model), dtype=torch.bfloat16, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    caches = [c for lw in tw["layers"] for c in (lw["k_cache"], lw["v_cache"])]
    state = [tok, filled, pos, ctx] + caches

    def run():
        for i in range(steps):
            wd.wedlm_model_step(handle, shape, bt, tok, filled, pos, ctx, n_commit[i], committed[i], cfg.alpha,
                                cfg.tau, cfg.rope_base, steps * W, ws, hidden_out=hid[i], dev_status=status)

    saved = [x.clone() for x in state]

    def restore():
        for x, y in zip(state, saved):
            x.copy_(y)
        for x in (n_commit, committed, hid):
            x.zero_()

    def snapshot():
        return [x.clone() for x in [n_commit, committed, hid] + state]

    run()
    torch.cuda.synchronize()
    ref = snapshot()
    restore()
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()
    with wd.capture(cap) as g:
        run()
    k, o = g.nodes()
    assert k > 0 and o == steps, (k, o)      # one device copy (hidden_out) per step
    _replays_match(g.launch, restore, snapshot, ref, dev)
    g.close()
    assert status.item() == 0
