"""Decode steps captured in a HIP graph replay exactly like the same steps
run eagerly.

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


def test_captured_steps_replay_like_eager(dev):
    cfg = wl.CONFIGS["qwen3_l2048"]
    steps, V = 3, 4096
    print("[graph] qwen3_l2048 x3 steps, V=4096", flush=True)
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
                                   committed[i], scfg.alpha, scfg.tau, V, ws_sel)

    saved = [x.clone() for x in state]

    def restore():
        for x, y in zip(state, saved):
            x.copy_(y)
        for x in (n_commit, committed, outs):
            x.zero_()

    def snapshot():
        return [x.clone() for x in (n_commit, committed, outs) + state]

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

    for rep in range(4):
        restore()
        torch.randn(4096, device=dev).sum().item()   # the program's own eager work
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = snapshot()
        for k, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a, b), (rep, k)
    assert t["status"].item() == 0
