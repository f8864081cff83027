"""wedlm_decode_step -- a whole decode step in three launches (the reorder
beside the vocabulary pass, the split-KV attention, the split combine beside
the commit) -- leaves exactly the bytes of the three calls it stands for
(wedlm_reorder, wedlm_step_attn, wedlm_select_commit, in that order).

Two copies of one window state stream through the same steps, one through
the three calls and one through the fused call, and every tensor either
path writes is compared for equality after every step: the attention
output, q_phys, perm, both caches, the window state (tok, filled, pos,
ctx_len), n_commit, committed, argmax, entropy, the prefix-cacheability
counters and the device status.  The shapes cover the fp32 kernel with one
split and with split partials, bf16 with split partials (some splits past
the context, so the combine weighs partials it did not get keys for), a
host bound far beyond
the context (most splits empty), one split per sequence (no combine: the
commit runs alone after the split kernel), head dim 64, and more than 2048
window slots (the four-slots-per-work-group reorder).  The three-call path
is itself checked against the oracle by the parity, graph and select tests;
test_gpu_graph.py also checks the fused steps against the oracle directly."""
import numpy as np
import pytest
import torch

import workloads as wl
import causal_attention_diffusion_amd as wd

pytestmark = pytest.mark.gpu


def _cfg(base_name, **kw):
    base = wl.CONFIGS[base_name]
    d = {f: getattr(base, f) for f in base.__dataclass_fields__}
    d.update(kw)
    return wl.AttnConfig(**d)


# (case, attention config, vocabulary, steps, host bound beyond the steps)
CASES = [
    ("tiny_f32", wl.CONFIGS["tiny_f32"], 1000, 4, 0),
    ("f32_splits", _cfg("tiny_f32", name="f32_splits", B=2, L=3000, seed=93), 1000, 3, 0),
    ("qwen3_l2048_v152k", wl.CONFIGS["qwen3_l2048"], 151936, 3, 0),
    ("qwen3_l2048_far_bound", wl.CONFIGS["qwen3_l2048"], 4096, 3, 20000),
    ("ragged_b32", wl.CONFIGS["ragged_b32"], 4096, 2, 0),
    ("long_b4_l8192", _cfg("long_b4", name="long_b4_l8192", L=8192), 4096, 2, 0),
    ("d64_g4_ragged", _cfg("ragged_b32", name="d64_g4", B=6, Hq=16, Hkv=4, D=64, L_range=(100, 3000), seed=91),
     2048, 3, 0),
    ("many_slots_b128_w18", _cfg("qwen3_l2048", name="many_slots_b128_w18", B=128, W=18, L=0, L_range=(0, 300),
                                 n_obs=None, seed=4711), 1024, 2, 0),
]


class _Stream:
    """One copy of the window state, caches and per-step outputs."""

    def __init__(self, inp, dev, V, steps, max_ctx):
        cfg = inp.cfg
        self.t = wl.device_attn_inputs(inp, dev)
        B, W = cfg.B, cfg.W
        self.tok = torch.from_numpy(np.where(inp.filled == 1, (np.arange(B * W).reshape(B, W) * 7) % V, V)
                                    .astype(np.int32)).to(dev)
        self.n_commit = torch.zeros((steps, B), dtype=torch.int32, device=dev)
        self.committed = torch.zeros((steps, B, W), dtype=torch.int32, device=dev)
        self.argmax = torch.zeros((steps, B, W), dtype=torch.int32, device=dev)
        self.entropy = torch.zeros((steps, B, W), dtype=torch.float32, device=dev)
        self.outs = torch.zeros((steps,) + tuple(self.t["out"].shape), dtype=self.t["out"].dtype, device=dev)
        self.qphys = torch.zeros((steps,) + tuple(self.t["q_phys"].shape), dtype=self.t["q_phys"].dtype,
                                 device=dev)
        self.perms = torch.zeros((steps, B, W), dtype=torch.int32, device=dev)
        self.counters = torch.zeros((B, 2), dtype=torch.int64, device=dev)
        self.max_ctx = max_ctx

    def keep(self, i):
        self.qphys[i].copy_(self.t["q_phys"])
        self.perms[i].copy_(self.t["perm"])

    def result(self):
        t = self.t
        return {"out": self.outs, "q_phys": self.qphys, "perm": self.perms, "k_cache": t["k_cache"],
                "v_cache": t["v_cache"], "tok": self.tok, "filled": t["filled"], "pos": t["pos"],
                "ctx_len": t["ctx_len"], "n_commit": self.n_commit, "committed": self.committed,
                "argmax": self.argmax, "entropy": self.entropy, "counters": self.counters, "status": t["status"]}


@pytest.mark.parametrize("case", [c[0] for c in CASES])
def test_fused_step_equals_three_calls(case, dev):
    _, cfg, V, steps, beyond = next(c for c in CASES if c[0] == case)
    print(f"[step] {case}: B={cfg.B} W={cfg.W} Hq={cfg.Hq} Hkv={cfg.Hkv} D={cfg.D} {cfg.dtype} V={V} "
          f"steps={steps}", flush=True)
    inp = wl.make_attn_inputs(cfg, spare_tokens=(steps + 1) * cfg.W + beyond)
    max_ctx = int(inp.ctx_len.max()) + (steps + 1) * cfg.W + beyond
    scfg = wl.SelectConfig(case, B=cfg.B, W=cfg.W, V=V, seed=cfg.seed + 5, alpha=0.25,
                           tau=float(np.log(V) * 0.7), steps=0, kind="mixture")
    logits = [wl.make_logits_torch(scfg, i, dev) for i in range(steps)]
    a = _Stream(inp, dev, V, steps, max_ctx)
    f = _Stream(inp, dev, V, steps, max_ctx)
    t = a.t
    ws_attn = wd.attn_workspace_tensor(t["q_phys"], t["k_cache"], t["block_table"], max_ctx)
    ws_sel = wd.select_workspace_tensor(cfg.B, cfg.W, V, dev)
    ws_step = wd.decode_step_workspace_tensor(f.t["q"], f.t["k_cache"], f.t["block_table"], max_ctx, V)
    ws_step.fill_(0xFF)   # the fused call must not depend on the workspace's contents (NaN bytes here)
    nsplit, _ = wd.wedlm_attn_plan(t["q_phys"], t["k_cache"], t["block_table"], max_ctx)
    print(f"[step] {case}: {nsplit} splits", flush=True)
    for i in range(steps):
        wd.wedlm_reorder(t["filled"], t["pos"], t["q"], t["k"], t["v"], t["q_phys"], t["k_cache"], t["v_cache"],
                         t["block_table"], t["ctx_len"], t["perm"], cfg.rope_base, dev_status=t["status"])
        wd.wedlm_step_attn(t["q_phys"], t["k_cache"], t["v_cache"], t["block_table"], t["ctx_len"], t["perm"],
                           a.outs[i], max_ctx_len=max_ctx, workspace=ws_attn, dev_status=t["status"])
        a.keep(i)
        wd.wedlm_select_commit(logits[i], a.tok, t["filled"], t["pos"], t["ctx_len"], a.n_commit[i],
                               a.committed[i], scfg.alpha, scfg.tau, V, ws_sel, argmax_out=a.argmax[i],
                               entropy_out=a.entropy[i], counters=a.counters)
        u = f.t
        wd.wedlm_decode_step(u["filled"], u["pos"], u["q"], u["k"], u["v"], u["q_phys"], u["k_cache"],
                             u["v_cache"], u["block_table"], u["ctx_len"], u["perm"], f.outs[i], cfg.rope_base,
                             max_ctx, logits[i], f.tok, f.n_commit[i], f.committed[i], scfg.alpha, scfg.tau, V,
                             ws_step, argmax_out=f.argmax[i], entropy_out=f.entropy[i], counters=f.counters,
                             dev_status=u["status"])
        f.keep(i)
    torch.cuda.synchronize()
    ra, rf = a.result(), f.result()
    assert int(ra["status"].item()) == 0
    for name in ra:
        assert torch.equal(ra[name], rf[name]), f"{case}: {name} differs"
    nc = ra["n_commit"].cpu().numpy()
    print(f"[step] {case}: identical; commits per step {nc.sum(1).tolist()}", flush=True)


@pytest.mark.parametrize("fault", ["bad_page", "bad_ctx"])
def test_fused_step_reports_like_three_calls(fault, dev):
    # a block-table entry outside the page pool (sequence 1) or a context
    # length beyond the host bound (sequence 2): both forms raise the same
    # device-status bit and still leave identical bytes everywhere
    cfg = _cfg("ragged_b32", name=f"fault_{fault}", B=4, L_range=(300, 900), seed=97)
    V, steps = 1024, 1
    print(f"[step] {fault}", flush=True)
    inp = wl.make_attn_inputs(cfg, spare_tokens=2 * cfg.W)
    max_ctx = int(inp.ctx_len.max()) + cfg.W
    scfg = wl.SelectConfig("fault", B=cfg.B, W=cfg.W, V=V, seed=3, alpha=0.25, tau=4.0, steps=0, kind="mixture")
    logits = wl.make_logits_torch(scfg, 0, dev)
    a = _Stream(inp, dev, V, steps, max_ctx)
    f = _Stream(inp, dev, V, steps, max_ctx)
    t, u = a.t, f.t
    for x in (t, u):   # the fault goes into the device copies (the host draw built the cache)
        if fault == "bad_page":
            x["block_table"][1, 3] = 10 ** 6
        else:
            x["ctx_len"][2] = max_ctx + 1
    ws_attn = wd.attn_workspace_tensor(t["q_phys"], t["k_cache"], t["block_table"], max_ctx)
    ws_sel = wd.select_workspace_tensor(cfg.B, cfg.W, V, dev)
    ws_step = wd.decode_step_workspace_tensor(u["q"], u["k_cache"], u["block_table"], max_ctx, V)
    wd.wedlm_reorder(t["filled"], t["pos"], t["q"], t["k"], t["v"], t["q_phys"], t["k_cache"], t["v_cache"],
                     t["block_table"], t["ctx_len"], t["perm"], cfg.rope_base, dev_status=t["status"])
    wd.wedlm_step_attn(t["q_phys"], t["k_cache"], t["v_cache"], t["block_table"], t["ctx_len"], t["perm"],
                       a.outs[0], max_ctx_len=max_ctx, workspace=ws_attn, dev_status=t["status"])
    a.keep(0)
    wd.wedlm_select_commit(logits, a.tok, t["filled"], t["pos"], t["ctx_len"], a.n_commit[0], a.committed[0],
                           scfg.alpha, scfg.tau, V, ws_sel, argmax_out=a.argmax[0], entropy_out=a.entropy[0],
                           counters=a.counters)
    wd.wedlm_decode_step(u["filled"], u["pos"], u["q"], u["k"], u["v"], u["q_phys"], u["k_cache"], u["v_cache"],
                         u["block_table"], u["ctx_len"], u["perm"], f.outs[0], cfg.rope_base, max_ctx, logits,
                         f.tok, f.n_commit[0], f.committed[0], scfg.alpha, scfg.tau, V, ws_step,
                         argmax_out=f.argmax[0], entropy_out=f.entropy[0], counters=f.counters,
                         dev_status=u["status"])
    f.keep(0)
    torch.cuda.synchronize()
    want = 2 if fault == "bad_page" else 1   # WEDLM_DEV_BAD_PAGE / WEDLM_DEV_BAD_CTX
    ra, rf = a.result(), f.result()
    assert int(ra["status"].item()) & want, int(ra["status"].item())
    for name in ra:
        assert torch.equal(ra[name], rf[name]), f"{fault}: {name} differs"


def test_fused_step_rejects_bad_arguments(dev):
    cfg = wl.CONFIGS["qwen3_l2048"]
    inp = wl.make_attn_inputs(cfg, spare_tokens=2 * cfg.W)
    t = wl.device_attn_inputs(inp, dev)
    V = 512
    max_ctx = int(inp.ctx_len.max()) + cfg.W
    ws = wd.decode_step_workspace_tensor(t["q"], t["k_cache"], t["block_table"], max_ctx, V)
    logits = torch.zeros((cfg.B, cfg.W, V), dtype=torch.float32, device=dev)
    tok = torch.zeros((cfg.B, cfg.W), dtype=torch.int32, device=dev)
    n_commit = torch.zeros((cfg.B,), dtype=torch.int32, device=dev)
    committed = torch.zeros((cfg.B, cfg.W), dtype=torch.int32, device=dev)
    args = [t["filled"], t["pos"], t["q"], t["k"], t["v"], t["q_phys"], t["k_cache"], t["v_cache"],
            t["block_table"], t["ctx_len"], t["perm"], t["out"], cfg.rope_base, max_ctx, logits, tok, n_commit,
            committed, 0.25, 4.0, V]
    before = [x.clone() for x in (t["k_cache"], t["ctx_len"], tok)]
    with pytest.raises(wd.WedlmError, match="workspace"):
        wd.wedlm_decode_step(*args, ws[: ws.numel() - 1])
    bad = list(args)
    bad[12] = 0.5   # rope_base
    with pytest.raises(wd.WedlmError, match="rope_base"):
        wd.wedlm_decode_step(*bad, ws)
    bad = list(args)
    bad[13] = 10 ** 6   # host bound beyond the largest supported context
    with pytest.raises(wd.WedlmError):
        wd.wedlm_decode_step(*bad, ws)
    bad = list(args)
    bad[19] = float("nan")   # tau
    with pytest.raises(wd.WedlmError, match="finite"):
        wd.wedlm_decode_step(*bad, ws)
    torch.cuda.synchronize()
    for x, y in zip((t["k_cache"], t["ctx_len"], tok), before):
        assert torch.equal(x, y)   # nothing was enqueued


def test_timed_step_equals_plain_step(dev):
    # wedlm_decode_step_timed: the same bytes as wedlm_decode_step, and the
    # attention kernel's dispatch sets the two events (a positive duration
    # shorter than the whole step)
    cfg = wl.CONFIGS["qwen3_l2048"]
    V, steps = 4096, 3
    inp = wl.make_attn_inputs(cfg, spare_tokens=(steps + 1) * cfg.W)
    max_ctx = int(inp.ctx_len.max()) + (steps + 1) * cfg.W
    scfg = wl.SelectConfig("timed", B=cfg.B, W=cfg.W, V=V, seed=cfg.seed + 9, alpha=0.25,
                           tau=float(np.log(V) * 0.7), steps=0, kind="mixture")
    logits = [wl.make_logits_torch(scfg, i, dev) for i in range(steps)]
    a = _Stream(inp, dev, V, steps, max_ctx)
    f = _Stream(inp, dev, V, steps, max_ctx)
    ws_a = wd.decode_step_workspace_tensor(a.t["q"], a.t["k_cache"], a.t["block_table"], max_ctx, V)
    ws_f = wd.decode_step_workspace_tensor(f.t["q"], f.t["k_cache"], f.t["block_table"], max_ctx, V)
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in evs:
        e0.record(stream)
        e1.record(stream)
    for i in range(steps):
        for s_, ws, ev in ((a, ws_a, None), (f, ws_f, evs[i])):
            u = s_.t
            wd.wedlm_decode_step(u["filled"], u["pos"], u["q"], u["k"], u["v"], u["q_phys"], u["k_cache"],
                                 u["v_cache"], u["block_table"], u["ctx_len"], u["perm"], s_.outs[i],
                                 cfg.rope_base, max_ctx, logits[i], s_.tok, s_.n_commit[i], s_.committed[i],
                                 scfg.alpha, scfg.tau, V, ws, argmax_out=s_.argmax[i], entropy_out=s_.entropy[i],
                                 counters=s_.counters, dev_status=u["status"], attn_events=ev)
            s_.keep(i)
    torch.cuda.synchronize()
    ra, rf = a.result(), f.result()
    for name in ra:
        assert torch.equal(ra[name], rf[name]), f"timed step: {name} differs"
    ms = [e0.elapsed_time(e1) for e0, e1 in evs]
    print(f"[step] timed attention kernel: {[round(x * 1e3, 1) for x in ms]} us", flush=True)
    assert all(0.0 < x < 5.0 for x in ms), ms
