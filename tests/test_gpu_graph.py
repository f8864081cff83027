"""Decode steps captured in a HIP graph replay exactly like the same steps
run eagerly -- captured by torch and by the library's own capture API
(wedlm_graph_*) -- and both match the oracle; so do the same steps taken
through the fused wedlm_decode_step.

Three whole steps (reorder, attention, select/commit) on the Qwen3-8B-shaped
single-layer workload are captured once and replayed four times, each replay
from the same restored state, with eager work and synchronisation of the
program between replays.  Every replay must reproduce the eager run's bytes:
committed counts and tokens, attention outputs, window state and the K/V
cache.  The eager run itself is checked against the oracle streamed over
the same three steps (reorder, attention over the grown cache, select /
commit / refill): integer state and commits exactly, attention within the
bf16 tolerance, the appended K bit-exact (up to the rounding-tie band of the
reorder parity test) and V exactly.  None of the library's calls allocates,
synchronises or clears memory, so the whole step can sit in a graph."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
import causal_attention_diffusion_amd as wd
from parity_checks import rounding_exact

pytestmark = pytest.mark.gpu


def _decode_setup(dev, steps=3, V=4096, fused=False, cfg=None):
    cfg = cfg or wl.CONFIGS["qwen3_l2048"]
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
    ws_step = wd.decode_step_workspace_tensor(t["q"], t["k_cache"], t["block_table"], max_ctx, V)

    def run():
        for i in range(steps):
            if fused:
                wd.wedlm_decode_step(t["filled"], t["pos"], t["q"], t["k"], t["v"], t["q_phys"], t["k_cache"],
                                     t["v_cache"], t["block_table"], t["ctx_len"], t["perm"], outs[i],
                                     cfg.rope_base, max_ctx, logits[i], tok, n_commit[i], committed[i],
                                     scfg.alpha, scfg.tau, V, ws_step, counters=counters, dev_status=t["status"])
                continue
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

    def check_oracle(snap):
        _check_against_oracle(inp, cfg, scfg, [lg.cpu().numpy() for lg in logits], snap)

    return t, run, restore, snapshot, n_commit, check_oracle


def _check_against_oracle(inp, cfg, scfg, logits, snap):
    """Stream the oracle over the same steps and compare with the eager
    run's snapshot (n_commit, committed, outs, counters, tok, filled, pos,
    ctx_len, k_cache, v_cache)."""
    g_nc, g_cm, g_out, g_cnt, g_tok, g_filled, g_pos, g_ctx, g_kc, g_vc = [x.cpu() for x in snap]
    dt, B, W, V = cfg.dtype, cfg.B, cfg.W, scfg.V
    f64 = lambda a: wl.storage_to_f64(a, dt)
    q, k, v = f64(inp.q), f64(inp.k), f64(inp.v)
    tok = np.where(inp.filled == 1, 5, V).astype(np.int32)
    filled, pos, ctx = inp.filled.copy(), inp.pos.copy(), inp.ctx_len.copy()
    cache_k = [f64(inp.prefix_k[b]) for b in range(B)]
    cache_v = [f64(inp.prefix_v[b]) for b in range(B)]
    cache_k64 = [x.copy() for x in cache_k]
    hist = []
    for i, lg in enumerate(logits):
        perm, qp, kw, vw = oracle.reorder(filled, pos, q, k, v, dt, cfg.rope_base)
        _, _, kw64, _ = oracle.reorder(filled, pos, q, k, v, "f64", cfg.rope_base)
        dk = [np.concatenate([cache_k[b][:ctx[b]], kw[b]]) for b in range(B)]
        dv = [np.concatenate([cache_v[b][:ctx[b]], vw[b]]) for b in range(B)]
        dk64 = [np.concatenate([cache_k64[b][:ctx[b]], kw64[b]]) for b in range(B)]
        out = oracle.attention(qp, dk, dv, ctx, perm)
        err = float(np.abs(f64_t(g_out[i], dt) - out).max() / np.abs(out).max())
        assert err <= 2e-2, (i, err)
        sel = oracle.select_commit(lg, tok, filled, pos, ctx, scfg.alpha, scfg.tau, V)
        assert (sel["margin"] > 1e-4).all(), sel["margin"]
        np.testing.assert_array_equal(g_nc[i].numpy(), sel["n_commit"])
        np.testing.assert_array_equal(g_cm[i].numpy(), sel["committed"])
        hist.append(sel["n_commit"])
        tok, filled, pos, ctx = sel["tok"], sel["filled"], sel["pos"], sel["ctx_len"]
        cache_k, cache_v, cache_k64 = dk, dv, dk64
        print(f"[graph oracle] step {i}: attention err {err:.3e}, commits {sel['n_commit'].tolist()}", flush=True)
    np.testing.assert_array_equal(g_tok.numpy(), tok)
    np.testing.assert_array_equal(g_filled.numpy(), filled)
    np.testing.assert_array_equal(g_pos.numpy(), pos)
    np.testing.assert_array_equal(g_ctx.numpy(), ctx)
    n_new, n_total, _ = oracle.prefix_cacheability(hist, W)
    np.testing.assert_array_equal(g_cnt.numpy(), np.stack([n_new, n_total], axis=1))
    # every cache row the steps wrote: the committed ones and the last window
    for b in range(B):
        L0 = int(inp.ctx_len[b])
        t = np.arange(L0, cache_k[b].shape[0])
        pages = inp.block_table[b, t // wl.PAGE].astype(np.int64)
        slot = (t % wl.PAGE).astype(np.int64)
        gk = f64_t(g_kc[pages, :, slot, :], dt)
        gv = f64_t(g_vc[pages, :, slot, :], dt)
        rounding_exact(gk, cache_k[b][L0:], cache_k64[b][L0:])
        np.testing.assert_array_equal(gv, cache_v[b][L0:])


def f64_t(x, dt):
    return wl.torch_storage_to_f64(x, dt)


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
    t, run, restore, snapshot, n_commit, check_oracle = _decode_setup(dev)
    run()
    torch.cuda.synchronize()
    ref = snapshot()
    assert int(n_commit.sum().item()) > 0          # the steps did commit something
    check_oracle(ref)

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
    t, run, restore, snapshot, n_commit, check_oracle = _decode_setup(dev)
    run()
    torch.cuda.synchronize()
    ref = snapshot()
    check_oracle(ref)
    restore()
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()
    with wd.capture(cap) as g:
        run()
    assert g.nodes() == (15, 0), g.nodes()
    _replays_match(g.launch, restore, snapshot, ref, dev)
    g.close()
    assert t["status"].item() == 0


def test_fused_steps_match_oracle_and_replay(dev):
    # the same three steps through wedlm_decode_step: checked against the
    # oracle's stream, then captured natively -- three launches per step (the
    # reorder with the vocabulary statistics, split attention, the combine
    # with the commit), 9 kernel nodes -- and replayed like the eager run
    print("[graph] qwen3_l2048 x3 fused steps, V=4096, native capture", flush=True)
    t, run, restore, snapshot, n_commit, check_oracle = _decode_setup(dev, fused=True)
    run()
    torch.cuda.synchronize()
    ref = snapshot()
    assert int(n_commit.sum().item()) > 0
    check_oracle(ref)
    restore()
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()
    with wd.capture(cap) as g:
        run()
    assert g.nodes() == (9, 0), g.nodes()
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


def test_tail_split_steps_match_oracle_and_replay(dev):
    # a ragged batch whose attention plan cuts its 12 longest sequences in
    # two: the cut set is ranked on the device from ctx_len at every step,
    # so replays of captured steps follow the contexts the steps grow
    base = wl.CONFIGS["ragged_b32"]
    d = {f: getattr(base, f) for f in base.__dataclass_fields__}
    d.update(name="ragged_tail_graph", L_range=(100, 1500), seed=4242)
    cfg = wl.AttnConfig(**d)
    print("[graph] ragged B=32 x3 fused steps with 12 tail splits, V=4096, native capture", flush=True)
    wd.wedlm_set_attn_tail(12)
    try:
        t, run, restore, snapshot, n_commit, check_oracle = _decode_setup(dev, fused=True, cfg=cfg)
        assert wd.wedlm_attn_tail(t["q_phys"], t["k_cache"], t["block_table"],
                                  int(t["ctx_len"].max().item()) + 4 * cfg.W) == 12
        run()
        torch.cuda.synchronize()
        ref = snapshot()
        assert int(n_commit.sum().item()) > 0
        check_oracle(ref)
        restore()
        torch.cuda.synchronize()
        cap = torch.cuda.Stream()
        with wd.capture(cap) as g:
            run()
        assert g.nodes() == (9, 0), g.nodes()
        _replays_match(g.launch, restore, snapshot, ref, dev)
        g.close()
        assert t["status"].item() == 0
    finally:
        wd.wedlm_set_attn_tail(-1)
