"""GPU parity of the fused LM head + select step (wedlm_lmhead_select_commit)
against the oracle (float64 contraction of the same bf16 inputs, rounded to
fp32, then the oracle's select step).

The GPU accumulates each logit in fp32 over the hidden size, so a logit
differs from the oracle's by a few fp32 ulps of the partial sums.  Every
slot of every step is compared (tests/parity_checks.py): the commit set,
flags and positions exactly; the argmax and the filled token exactly,
except at a slot whose oracle row has two logits closer than TIE, where the
GPU's token must lie within TIE of the maximum.  Entropies agree to 1e-4
relative.  Every step is teacher-forced (both sides start from the
oracle's state), and a step whose threshold decisions lie within 1e-4 of
tau would not be a fair test: the margin is asserted.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
import causal_attention_diffusion_amd as wd
from parity_checks import check_select_step

pytestmark = pytest.mark.gpu

TIE = 1e-3


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _bf16(bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits)).view(torch.bfloat16).to(dev)


def _state(tok, filled, pos, ctx, dev):
    return [torch.from_numpy(np.ascontiguousarray(x, dt)).to(dev)
            for x, dt in ((tok, np.int32), (filled, np.uint8), (pos, np.int32), (ctx, np.int32))]


def _run(h, w, st, alpha, tau, mask_id, ws):
    B, W, _ = h.shape
    d = h.device
    n_commit = torch.empty(B, dtype=torch.int32, device=d)
    committed = torch.empty((B, W), dtype=torch.int32, device=d)
    am = torch.empty((B, W), dtype=torch.int32, device=d)
    ent = torch.empty((B, W), dtype=torch.float32, device=d)
    wd.wedlm_lmhead_select_commit(h, w, *st, n_commit, committed, alpha, tau, mask_id, ws,
                                  argmax_out=am, entropy_out=ent)
    return n_commit, committed, am, ent


def _check(ref, z64, st, outs, filled_before, rows=None):
    """ref: oracle step; z64: oracle float64 logits of the compared rows;
    filled_before: flags the step started from (compared rows)."""
    sel = slice(None) if rows is None else rows
    st_np = [x.cpu().numpy()[sel] for x in st]
    outs_np = [x.cpu().numpy()[sel] for x in outs]
    return check_select_step(ref, z64, np.asarray(filled_before), st_np, outs_np, tie=TIE)


def _stream(cfg, dev, steps, filled_pattern=None):
    lm = wl.make_lm_head_np(cfg)
    w64 = wl.bf16_bits_to_f32(lm).astype(np.float64)
    w = _bf16(lm, dev)
    ws = wd.lmhead_workspace_tensor(cfg.B, cfg.W, cfg.V, cfg.Dm, dev)
    tok, filled, pos, ctx = wl.initial_window(cfg.B, cfg.W, cfg.V)
    if filled_pattern is not None:
        filled[:] = filled_pattern
        tok[filled == 1] = 7
    total = 0
    for step in range(steps):
        hb = wl.make_hidden_np(cfg, step, lm)
        h64 = wl.bf16_bits_to_f32(hb).astype(np.float64)
        ref = oracle.lmhead_select_commit(h64, w64, tok, filled, pos, ctx, cfg.alpha, cfg.tau, cfg.V)
        z64 = oracle.lmhead_logits(h64, w64)
        st = _state(tok, filled, pos, ctx, dev)
        outs = _run(_bf16(hb, dev), w, st, cfg.alpha, cfg.tau, cfg.V, ws)
        torch.cuda.synchronize()
        _check(ref, z64, st, outs, filled)
        tok, filled, pos, ctx = ref["tok"], ref["filled"], ref["pos"], ref["ctx_len"]
        total += int(ref["n_commit"].sum())
    return total


def test_lmhead_small_stream(dev):
    # 16 rows, 12 vocabulary tiles (the last one 184 wide), 4 hidden stages
    cfg = wl.LMHEAD_CONFIGS["lmhead_small"]
    assert _stream(cfg, dev, cfg.steps) > 0


def test_lmhead_two_row_groups(dev):
    # 192 rows -> row groups of 128 and 64; 157 vocabulary tiles; 16 stages
    cfg = wl.LMHEAD_CONFIGS["lmhead_mid"]
    _stream(cfg, dev, cfg.steps)


@pytest.mark.parametrize("B,W,Dm,V", [(1, 4, 64, 100), (3, 5, 192, 257), (2, 64, 128, 512)])
def test_lmhead_edge_shapes(B, W, Dm, V, dev):
    # one hidden stage; a vocabulary shorter than one tile; a tile of one
    # entry; full 64-slot windows
    cfg = wl.LmheadConfig("e", B=B, W=W, Dm=Dm, V=V, seed=1200 + V, alpha=0.25,
                          tau=float(np.log(V) * 0.8), steps=3)
    _stream(cfg, dev, cfg.steps)


def test_lmhead_partly_filled_window(dev):
    # filled slots are skipped: only the masked rows are listed and scored
    cfg = wl.LmheadConfig("p", B=4, W=16, Dm=256, V=2000, seed=1301, alpha=0.25,
                          tau=float(np.log(2000) * 0.8), steps=4)
    pat = np.zeros((4, 16), np.uint8)
    pat[0, :5] = 1
    pat[1, 3::2] = 1
    pat[3, :] = 1                         # a window with no masked slot
    _stream(cfg, dev, cfg.steps, filled_pattern=pat)


@pytest.mark.parametrize("n_masked", [1, 127, 128, 129, 300, 512, 640, 700, 896, 1023])
def test_lmhead_masked_counts(n_masked, dev):
    """A 64 x 16 window (room for 8 row groups of 128) with n_masked masked
    slots scattered over it: every count of active row groups from 1 to 8,
    with full and partly filled last groups, maps each masked row to exactly
    one work-group per vocabulary tile (12 tiles, the last one 184 wide)."""
    B, W, V = 64, 16, 3000
    cfg = wl.LmheadConfig(f"m{n_masked}", B=B, W=W, Dm=256, V=V, seed=1400 + n_masked, alpha=0.25,
                          tau=float(np.log(V) * 0.8), steps=1)
    pat = np.ones(B * W, np.uint8)
    pat[np.random.default_rng(n_masked).choice(B * W, n_masked, replace=False)] = 0
    _stream(cfg, dev, 1, filled_pattern=pat.reshape(B, W))


def test_lmhead_no_masked_slot(dev):
    # nothing to score: commit the whole window, refill, no kernel reads
    cfg = wl.LmheadConfig("n", B=2, W=8, Dm=64, V=300, seed=1302, alpha=0.25, tau=1.0, steps=1)
    _stream(cfg, dev, 1, filled_pattern=np.ones((2, 8), np.uint8))


def test_lmhead_full_vocab_sampled_sequences(dev):
    """Qwen3-8B LM head (4096 x 151936) over a 64 x 16 all-masked window: the
    GPU scores all 1024 rows; the oracle follows 3 sequences."""
    cfg = wl.LMHEAD_CONFIGS["lmhead_v152k"]
    track = np.array([0, 37, 63])
    lm = wl.make_lm_head_np(cfg)
    w = _bf16(lm, dev)
    hb = wl.make_hidden_np(cfg, 0, lm)
    w64 = wl.bf16_bits_to_f32(lm).astype(np.float64)
    del lm
    ws = wd.lmhead_workspace_tensor(cfg.B, cfg.W, cfg.V, cfg.Dm, dev)
    tok, filled, pos, ctx = wl.initial_window(cfg.B, cfg.W, cfg.V)
    st = _state(tok, filled, pos, ctx, dev)
    outs = _run(_bf16(hb, dev), w, st, cfg.alpha, cfg.tau, cfg.V, ws)
    torch.cuda.synchronize()
    h64 = wl.bf16_bits_to_f32(hb[track]).astype(np.float64)
    ref = oracle.lmhead_select_commit(h64, w64, tok[track], filled[track], pos[track], ctx[track],
                                      cfg.alpha, cfg.tau, cfg.V)
    z64 = oracle.lmhead_logits(h64, w64)
    ties = _check(ref, z64, st, outs, filled[track], rows=track)
    print(f"[lmhead full] committed {int(ref['n_commit'].sum())} near-ties {ties}", flush=True)


def test_lmhead_deterministic(dev):
    cfg = wl.LMHEAD_CONFIGS["lmhead_mid"]
    lm = wl.make_lm_head_np(cfg)
    w = _bf16(lm, dev)
    h = _bf16(wl.make_hidden_np(cfg, 2, lm), dev)
    res = []
    for _ in range(3):
        ws = wd.lmhead_workspace_tensor(cfg.B, cfg.W, cfg.V, cfg.Dm, dev)
        st = _state(*wl.initial_window(cfg.B, cfg.W, cfg.V), dev)
        outs = _run(h, w, st, cfg.alpha, cfg.tau, cfg.V, ws)
        res.append([x.clone() for x in list(st) + list(outs)])
    torch.cuda.synchronize()
    for r in res[1:]:
        for a, b in zip(r, res[0]):
            assert torch.equal(a, b)
