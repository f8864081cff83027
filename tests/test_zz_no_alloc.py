"""wedlm_step_attn_noalloc (split partials in the library's own device
array, no workspace argument) against wedlm_step_attn (caller workspace),
through the C ABI on the same inputs: three calls in a row, the last on a
much smaller input, each compared element by element with the workspace
entry point.  Both run the same kernels and split plan, so the outputs must be
identical bytes (the attention tolerance would be 2e-2 for bf16).  A shape
whose partials exceed the array is refused on the host before any launch."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
import causal_attention_diffusion_amd as wd

pytestmark = pytest.mark.gpu


def _inputs(cfg, dev):
    inp, q_phys, dk, dv = wl.make_full_cache_inputs(cfg)
    perm = oracle.reorder_perm(inp.filled)
    kc, vc = wl.paged_cache(inp, dk, dv)
    dt = cfg.dtype
    t = dict(q_phys=wl.as_torch(q_phys, dt, dev), k_cache=wl.as_torch(kc, dt, dev),
             v_cache=wl.as_torch(vc, dt, dev), block_table=torch.from_numpy(inp.block_table).to(dev),
             ctx_len=torch.from_numpy(inp.ctx_len).to(dev), perm=torch.from_numpy(perm).to(dev),
             status=torch.zeros(1, dtype=torch.int32, device=dev))
    return t, int(inp.ctx_len.max())


def _both(t, max_ctx):
    out_ws = torch.full_like(t["q_phys"], 3.0)
    out_na = torch.full_like(t["q_phys"], 5.0)
    ws = wd.attn_workspace_tensor(t["q_phys"], t["k_cache"], t["block_table"], max_ctx)
    args = (t["q_phys"], t["k_cache"], t["v_cache"], t["block_table"], t["ctx_len"], t["perm"])
    wd.wedlm_step_attn_noalloc(*args, out_na, max_ctx_len=max_ctx, dev_status=t["status"])
    wd.wedlm_step_attn(*args, out_ws, max_ctx_len=max_ctx, workspace=ws, dev_status=t["status"])
    torch.cuda.synchronize()
    assert t["status"].item() == 0
    return out_na, out_ws, ws.numel()


def test_noalloc_matches_workspace_entry_point(dev):
    # ragged_b32 (tail splits: the back parts name their sequences in the
    # array), then long_b4 (8 splits, about 17 MB of partials in the array),
    # then qwen3_l2048, a smaller plan over the same array
    for name in ("ragged_b32", "long_b4", "qwen3_l2048"):
        cfg = wl.CONFIGS[name]
        print(f"[noalloc] {name}", flush=True)
        t, max_ctx = _inputs(cfg, dev)
        tail = wd.wedlm_attn_tail(t["q_phys"], t["k_cache"], t["block_table"], max_ctx)
        assert (tail > 0) == (name == "ragged_b32"), (name, tail)
        out_na, out_ws, ws_bytes = _both(t, max_ctx)
        assert 0 < ws_bytes <= wd.wedlm_step_attn_noalloc_limit()
        assert torch.equal(out_na.view(torch.int16), out_ws.view(torch.int16)), name
        print(f"[noalloc] {name}: identical to wedlm_step_attn ({ws_bytes} bytes of partials)", flush=True)
        del t
        torch.cuda.empty_cache()


def test_noalloc_refuses_oversized_plan(dev):
    # 64-key splits over a 32K context: 64 splits per (sequence, KV head) need
    # far more than the array; refused before anything is enqueued
    cfg = wl.CONFIGS["long_b4"]
    t, max_ctx = _inputs(cfg, dev)
    out = torch.full_like(t["q_phys"], 7.0)
    wd.wedlm_set_attn_split_keys(64)
    try:
        need = wd.wedlm_step_attn_workspace(t["q_phys"], t["k_cache"], t["block_table"], max_ctx)
        assert need > wd.wedlm_step_attn_noalloc_limit()
        with pytest.raises(wd.WedlmError, match="scratch"):
            wd.wedlm_step_attn_noalloc(t["q_phys"], t["k_cache"], t["v_cache"], t["block_table"], t["ctx_len"],
                                       t["perm"], out, max_ctx_len=max_ctx)
    finally:
        wd.wedlm_set_attn_split_keys(0)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
