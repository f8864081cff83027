"""GPU parity of the synthetic decoder step (wedlm_model_step) against the
oracle's model step (float64, bf16 storage points mirrored).

Per step, teacher-forced (both sides start from the oracle's window state
and the oracle keeps its own caches):
  * the final normalised hidden states: max |gpu - oracle| / max |oracle|
    <= 2e-2 (bf16 storage at every projection, as for attention);
  * the window K/V the step appended to each layer's cache, same bound;
  * the select step slot by slot as the LM-head test checks it
    (tests/parity_checks.py), against the oracle's LM head + select on the
    GPU's own hidden states (argmax and the filled token may differ only
    where two logits are within 1e-3; flags, commits and positions never).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
import causal_attention_diffusion_amd as wd
from parity_checks import check_select_step

pytestmark = pytest.mark.gpu

PAGE = 16


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _bf16(bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits)).view(torch.bfloat16).to(dev)


def _f64(bits):
    return wl.bf16_bits_to_f32(bits).astype(np.float64)


def _setup(cfg, dev, max_ctx):
    wb = wl.make_model_np(cfg)
    w64 = {k: _f64(v) for k, v in wb.items() if k != "layers"}
    w64["layers"] = [{k: _f64(v) for k, v in lw.items()} for lw in wb["layers"]]
    mp = (max_ctx + cfg.W + PAGE - 1) // PAGE
    pool = cfg.B * mp
    rng = np.random.default_rng(cfg.seed + 7)
    bt = rng.permutation(pool).astype(np.int32).reshape(cfg.B, mp)       # shuffled physical pages
    tw = {k: _bf16(v, dev) for k, v in wb.items() if k != "layers"}
    tw["layers"] = []
    for lw in wb["layers"]:
        d = {k: _bf16(v, dev) for k, v in lw.items()}
        d["k_cache"] = torch.zeros((pool, cfg.Hkv, PAGE, cfg.D), dtype=torch.bfloat16, device=dev)
        d["v_cache"] = torch.zeros_like(d["k_cache"])
        tw["layers"].append(d)
    handle = wd.ModelHandle(tw, cfg.eps)
    shape = wd.make_shape(cfg.B, cfg.W, cfg.Hq, cfg.Hkv, cfg.D, mp, pool, wd.WEDLM_BF16)
    ws = wd.model_step_workspace_tensor(handle, shape, max_ctx, dev)
    return w64, tw, handle, shape, ws, torch.from_numpy(bt).to(dev), bt


def _gather_rows(cache, bt, b, t0, t1):
    """Cache rows of tokens t0 .. t1-1 of sequence b as [n, Hkv, D] float64."""
    c = cache.float().cpu().numpy()
    rows = [c[bt[b, t // PAGE], :, t % PAGE, :] for t in range(t0, t1)]
    return np.stack(rows).astype(np.float64)


def _rel(got, ref):
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30))


def _run_stream(cfg, dev, steps, max_ctx, prefix=0):
    w64, tw, handle, shape, ws, bt_t, bt = _setup(cfg, dev, max_ctx)
    B, W = cfg.B, cfg.W
    tok, filled, pos, ctx = wl.initial_window(B, W, cfg.vocab, prefix)
    caches = [([np.zeros((0, cfg.Hkv, cfg.D))] * B, [np.zeros((0, cfg.Hkv, cfg.D))] * B) for _ in range(cfg.layers)]
    if prefix:
        # a cached prompt of `prefix` tokens per sequence in every layer:
        # N(0,1) keys (taken as already rotated) and values in bf16, written to
        # the shuffled pages on the GPU and handed to the oracle as its caches
        rng = np.random.default_rng(cfg.seed + 29)
        t = np.arange(prefix)
        caches = []
        for l in range(cfg.layers):
            kv = []
            for name in ("k_cache", "v_cache"):
                bits = wl.to_storage(rng.standard_normal((B, prefix, cfg.Hkv, cfg.D)), "bf16")
                host = tw["layers"][l][name].view(torch.int16).cpu().numpy().view(np.uint16)
                for b in range(B):
                    host[bt[b, t // PAGE], :, t % PAGE, :] = bits[b]
                tw["layers"][l][name].copy_(torch.from_numpy(host.view(np.int16)).view(torch.bfloat16))
                kv.append([wl.storage_to_f64(bits[b], "bf16") for b in range(B)])
            caches.append((kv[0], kv[1]))
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    counters = torch.zeros((B, 2), dtype=torch.int64, device=dev)
    commits = []
    worst = 0.0
    for step in range(steps):
        st = [torch.from_numpy(np.ascontiguousarray(x, dt)).to(dev)
              for x, dt in ((tok, np.int32), (filled, np.uint8), (pos, np.int32), (ctx, np.int32))]
        n_commit = torch.empty(B, dtype=torch.int32, device=dev)
        committed = torch.empty((B, W), dtype=torch.int32, device=dev)
        am = torch.empty((B, W), dtype=torch.int32, device=dev)
        ent = torch.empty((B, W), dtype=torch.float32, device=dev)
        hid = torch.empty((B, W, cfg.d_model), dtype=torch.bfloat16, device=dev)
        wd.wedlm_model_step(handle, shape, bt_t, *st, n_commit, committed, cfg.alpha, cfg.tau, cfg.rope_base, max_ctx,
                            ws, argmax_out=am, entropy_out=ent, hidden_out=hid, dev_status=status, counters=counters)
        torch.cuda.synchronize()
        assert status.item() == 0
        ref = oracle.model_step(w64, caches, tok, filled, pos, ctx, cfg.alpha, cfg.tau, cfg.rope_base, cfg.eps,
                                cfg.Hq, cfg.Hkv)
        gh = hid.float().cpu().numpy().astype(np.float64)
        e = _rel(gh, ref["hidden"])
        worst = max(worst, e)
        assert e <= 2e-2, (step, e)
        for l in range(cfg.layers):
            for b in range(B):
                L = int(ctx[b])
                gk = _gather_rows(tw["layers"][l]["k_cache"], bt, b, L, L + W)
                gv = _gather_rows(tw["layers"][l]["v_cache"], bt, b, L, L + W)
                assert _rel(gk, ref["caches"][l][0][b][L:L + W]) <= 2e-2
                assert _rel(gv, ref["caches"][l][1][b][L:L + W]) <= 2e-2
        # the select step on the GPU's own hidden states
        sel = oracle.lmhead_select_commit(gh, w64["lm_head"], tok, filled, pos, ctx, cfg.alpha, cfg.tau, cfg.vocab)
        z64 = oracle.lmhead_logits(gh, w64["lm_head"])
        commits.append(sel["n_commit"])
        n_new, n_total, _ = oracle.prefix_cacheability(commits, W)
        np.testing.assert_array_equal(counters.cpu().numpy(), np.stack([n_new, n_total], axis=1))
        check_select_step(sel, z64, filled, [x.cpu().numpy() for x in st],
                          [x.cpu().numpy() for x in (n_commit, committed, am, ent)])
        # teacher forcing: continue from the select result on the GPU hidden
        # states; the oracle keeps its own caches, cut to the committed rows
        tok, filled, pos, ctx = sel["tok"], sel["filled"], sel["pos"], sel["ctx_len"]
        caches = [([ck[b][:ctx[b]] for b in range(B)], [cv[b][:ctx[b]] for b in range(B)])
                  for ck, cv in ref["caches"]]
    print(f"[model] {cfg.name}: {steps} steps, worst hidden rel err {worst:.3e}, final ctx {list(ctx)}", flush=True)
    return ctx


def test_model_small_stream(dev):
    cfg = wl.MODEL_CONFIGS["model_small"]
    ctx = _run_stream(cfg, dev, cfg.steps, max_ctx=cfg.steps * cfg.W)
    assert (ctx > 0).all()


def test_model_qwen3_layer_one_step(dev):
    # one Qwen3-8B-shaped layer (hidden 4096, 32/8 heads of 128, MLP 12288)
    # on a 4 x 64 window: 256 rows, split-K projections, two row tiles
    cfg = wl.MODEL_CONFIGS["model_qwen3_layer"]
    _run_stream(cfg, dev, 1, max_ctx=cfg.W)


def test_model_qwen3_two_layers_stream(dev):
    # two Qwen3-8B-shaped layers streamed for three steps on the 4 x 64
    # window over a 512-token cached prompt: the second layer consumes the
    # first's GPU output, and every step attends over the prompt and the
    # rows the earlier steps committed
    import dataclasses
    cfg = dataclasses.replace(wl.MODEL_CONFIGS["model_qwen3_layer"], name="model_qwen3_2layers", layers=2)
    ctx = _run_stream(cfg, dev, 3, max_ctx=512 + 3 * cfg.W, prefix=512)
    assert (ctx > 512).all()


@pytest.mark.parametrize("B,W", [(3, 48), (5, 64), (9, 64)])
def test_model_ragged_row_counts(B, W, dev):
    # window row counts that end inside a 32-row MFMA tile and inside a
    # 256-row group (144 = 128 + 16; 320 and 576 need two and three row
    # groups in every projection and in the LM head)
    import dataclasses
    cfg = dataclasses.replace(wl.MODEL_CONFIGS["model_small"], name=f"model_b{B}w{W}", B=B, W=W, layers=1,
                              seed=1600 + B * W, steps=3)
    ctx = _run_stream(cfg, dev, cfg.steps, max_ctx=cfg.steps * cfg.W)
    assert (ctx >= 0).all()
