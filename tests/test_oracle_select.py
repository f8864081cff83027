"""Pins for the oracle's vocab statistics and the commit / Eq. 11 select /
refill step (CPU only).

Pages: WeDLM paper-summary page, "Method" (inference paragraph: commit the
leftmost contiguous filled prefix, fill masks ranked by the penalised
entropy H~_j = H_j + alpha*d_j of Eq. 11, refill freed slots with masks),
"Key claims" (paper sec. 5.2) and the ICML abstract (commits grow a
left-to-right prefix; the window size is fixed).

Independent formulations: scipy's entropy of a softmax, numpy argmax,
closed-form entropies, a sort-based re-statement of the fill rule, and
stream invariants over many steps.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import scipy.stats

import oracle
from workloads import SELECT_CONFIGS, initial_window, make_logits_np

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- row stats
def test_constant_logits_entropy_is_log_v():
    for V in [1, 2, 7, 1000, 151936]:
        am, H = oracle.row_stats(np.full((1, V), 3.25, np.float32))
        assert am[0] == 0
        assert abs(H[0] - math.log(V)) < 1e-10


def test_single_spike_closed_form():
    for V, c in [(2, 1.0), (1000, 5.0), (151936, 12.0)]:
        z = np.zeros((1, V), np.float32)
        z[0, V // 3] = c
        am, H = oracle.row_stats(z)
        Z = math.exp(c) + V - 1
        assert am[0] == V // 3
        assert abs(H[0] - (math.log(Z) - c * math.exp(c) / Z)) < 1e-9


def test_entropy_and_argmax_vs_library():
    rng = np.random.default_rng(30)
    z = (rng.standard_normal((40, 5000)) * rng.uniform(0.1, 6, (40, 1))).astype(np.float32)
    z[3, [10, 20, 4999]] = z[3].max() + 1.0      # ties at the maximum
    am, H = oracle.row_stats(z)
    ref_H = scipy.stats.entropy(scipy.special.softmax(z.astype(np.float64), axis=1), axis=1)
    np.testing.assert_allclose(H, ref_H, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(am, np.argmax(z, axis=1))   # numpy returns the first maximum
    assert am[3] == 10


# ---------------------------------------------------------------- golden worked example
def _val(x):
    return {"ln8": math.log(8.0)}.get(x, x) if isinstance(x, str) else x


def _expr(e):
    return eval(e, {"ln10": math.log(10), "ln8": math.log(8), "ln3": math.log(3)})


def test_worked_example_threshold_and_fallback():
    d = json.load(open(os.path.join(GOLD, "select_worked_example.json")))
    tok = np.array([d["tok"]], np.int32); filled = np.array([d["filled"]], np.uint8)
    W = tok.shape[1]
    ctx = np.array([d["ctx_len"]], np.int32)
    pos = ctx[:, None] + np.arange(W)[None]
    lg = np.array([[[_val(x) for x in row] for row in d["logits"]]], np.float32)
    r = oracle.select_commit(lg, tok, filled, pos, ctx, d["alpha"], d["tau"], d["mask_id"])
    e = d["expected"]
    assert r["n_commit"].tolist() == [e["n_commit"]]
    assert r["committed"][0].tolist() == e["committed"]
    assert r["tok"][0].tolist() == e["tok"]
    assert r["filled"][0].tolist() == e["filled"]
    assert r["ctx_len"].tolist() == [e["ctx_len"]]
    assert r["pos"][0].tolist() == e["pos"]
    assert r["argmax"][0].tolist() == e["argmax"]
    for j, ex in enumerate(e["entropy_expr"]):
        if ex is None:
            assert r["entropy"][0, j] == -1.0
        else:
            assert abs(r["entropy"][0, j] - _expr(ex)) < 1e-6
    fb = d["fallback_case"]
    lg2 = np.array([[[_val(x) for x in row] for row in fb["logits"]]], np.float32)
    r2 = oracle.select_commit(lg2, tok, filled, pos, ctx, d["alpha"], fb["tau"], d["mask_id"])
    assert r2["tok"][0].tolist() == fb["expected"]["tok"]
    assert r2["filled"][0].tolist() == fb["expected"]["filled"]
    assert r2["argmax"][0].tolist() == fb["expected"]["argmax"]


# ---------------------------------------------------------------- brute force
def _reference_step(lg, tok, filled, ctx, alpha, tau, mask_id):
    """Sort-based re-statement of commit / select / refill for one sequence."""
    W = len(tok)
    k = next((i for i in range(W) if not filled[i]), W)
    emitted = list(tok[:k])
    masked = [j for j in range(W) if not filled[j]]
    tok = list(tok); filled = list(filled)
    if masked:
        j0 = masked[0]
        z = lg.astype(np.float64)
        H = {j: float(scipy.stats.entropy(scipy.special.softmax(z[j]))) for j in masked}
        a = {j: int(np.argmax(lg[j])) for j in masked}
        Ht = {j: np.float32(np.float32(H[j]) + np.float32(alpha) * np.float32(j - j0)) for j in masked}
        chosen = [j for j in masked if Ht[j] < np.float32(tau)]
        if not chosen:
            chosen = [min(masked, key=lambda j: (Ht[j], j))]
        for j in chosen:
            tok[j] = a[j]; filled[j] = 1
    tok = tok[k:] + [mask_id] * k
    filled = filled[k:] + [0] * k
    return emitted, tok, filled, ctx + k


def test_select_commit_brute_force_small():
    rng = np.random.default_rng(31)
    checked = 0
    for trial in range(400):
        B = int(rng.integers(1, 4)); W = int(rng.integers(1, 9)); V = int(rng.integers(1, 9))
        alpha = float(rng.choice([0.0, 0.1, 0.5])); tau = float(rng.uniform(0.0, 2.5))
        mask_id = V
        lg = (rng.standard_normal((B, W, V)) * rng.uniform(0.2, 4.0)).astype(np.float32)
        filled = (rng.random((B, W)) < 0.5).astype(np.uint8)
        tok = np.where(filled == 1, rng.integers(0, V, (B, W)), mask_id).astype(np.int32)
        ctx = rng.integers(0, 50, B).astype(np.int32)
        pos = ctx[:, None] + np.arange(W)[None]
        r = oracle.select_commit(lg, tok, filled, pos, ctx, alpha, tau, mask_id)
        for b in range(B):
            if r["margin"][b] < 1e-5:
                continue      # decision within fp32 noise: the two roundings may differ
            em, t2, f2, c2 = _reference_step(lg[b], tok[b], filled[b], int(ctx[b]), alpha, tau, mask_id)
            assert r["n_commit"][b] == len(em)
            assert r["committed"][b, :len(em)].tolist() == em
            assert (r["committed"][b, len(em):] == -1).all()
            assert r["tok"][b].tolist() == t2
            assert r["filled"][b].tolist() == f2
            assert r["ctx_len"][b] == c2
            assert r["pos"][b].tolist() == list(range(c2, c2 + W))
            checked += 1
    assert checked > 300


def test_commit_edge_cases():
    V, W = 5, 4
    lg = np.zeros((1, W, V), np.float32)
    ctx = np.array([7], np.int32)
    pos = ctx[:, None] + np.arange(W)
    # all filled: k = W, window refilled entirely with masks
    r = oracle.select_commit(lg, np.array([[1, 2, 3, 4]]), np.ones((1, W)), pos, ctx, 0.1, 1.0, V)
    assert r["n_commit"][0] == W and r["committed"][0].tolist() == [1, 2, 3, 4]
    assert r["tok"][0].tolist() == [V] * W and r["filled"][0].tolist() == [0] * W
    assert r["ctx_len"][0] == 11 and r["margin"][0] == np.inf
    # slot 0 masked: k = 0, nothing committed, at least one slot filled
    r = oracle.select_commit(lg, np.array([[V, 2, V, V]]), np.array([[0, 1, 0, 0]]), pos, ctx,
                             0.1, -1.0, V)
    assert r["n_commit"][0] == 0 and (r["committed"][0] == -1).all()
    assert r["filled"][0].sum() == 2 and r["filled"][0, 0] == 1   # fallback picks slot 0 (d = 0)
    assert r["ctx_len"][0] == 7


def test_missing_row_is_an_error():
    lg = np.zeros((1, 3), np.float32)
    ri = np.array([[0, -1]], np.int64)
    with pytest.raises(ValueError):
        oracle.select_commit(lg, np.array([[3, 3]]), np.zeros((1, 2)), np.array([[0, 1]]),
                             np.array([0]), 0.1, 1.0, 3, row_index=ri)


# ---------------------------------------------------------------- stream invariants
@pytest.mark.parametrize("cfg_name", ["tiny_f32"])
def test_stream_invariants_256_steps(cfg_name):
    cfg = SELECT_CONFIGS[cfg_name]
    B, W, V = 3, cfg.W, 64
    mask_id = V
    rng = np.random.default_rng(32)
    tok, filled, pos, ctx = initial_window(B, W, mask_id)
    stream = [[] for _ in range(B)]
    pending = [dict() for _ in range(B)]       # logical position -> token, once filled
    for step in range(256):
        lg = (rng.standard_normal((B, W, V)) * rng.uniform(0.5, 5.0)).astype(np.float32)
        r = oracle.select_commit(lg, tok, filled, pos, ctx, 0.25, 2.5, mask_id)
        for b in range(B):
            k = int(r["n_commit"][b])
            assert r["ctx_len"][b] == ctx[b] + k
            # committed tokens are exactly the ones filled earlier at those positions
            for i in range(k):
                p = int(ctx[b]) + i
                assert pending[b].pop(p) == r["committed"][b, i]
            stream[b].extend(r["committed"][b, :k].tolist())
            assert len(stream[b]) == r["ctx_len"][b]
            # fixed-size window, contiguous positions, masks carry mask_id
            assert r["pos"][b].tolist() == list(range(r["ctx_len"][b], r["ctx_len"][b] + W))
            assert ((r["filled"][b] == 1) | (r["tok"][b] == mask_id)).all()
            # filled tokens never revert and never change
            for i in range(W):
                p = int(r["ctx_len"][b]) + i
                if r["filled"][b, i]:
                    if p in pending[b]:
                        assert pending[b][p] == r["tok"][b, i]
                    pending[b][p] = int(r["tok"][b, i])
                else:
                    assert p not in pending[b]
            # at least one new fill when the window had masks
            had_mask = (filled[b] == 0).any()
            new_fills = int(r["filled"][b].sum()) - (int(filled[b].sum()) - k)
            assert (new_fills >= 1) == bool(had_mask)
        tok, filled, pos, ctx = r["tok"], r["filled"], r["pos"], r["ctx_len"]
    assert min(len(s) for s in stream) > 256      # more than one token per step on average


def test_tiny_config_margins_clear_fp32_noise():
    """The tiny workload's decisions (logits [8, 1000] ~ 2*N(0,1), alpha 0.25,
    tau 4.5) sit far from the threshold compared with fp32 entropy error."""
    cfg = SELECT_CONFIGS["tiny_f32"]
    lg = make_logits_np(cfg, 0)
    tok, filled, pos, ctx = initial_window(cfg.B, cfg.W, cfg.V)
    filled[0, [0, 2, 5]] = 1
    tok[0, [0, 2, 5]] = [11, 22, 33]
    r = oracle.select_commit(lg, tok, filled, pos, ctx, cfg.alpha, cfg.tau, cfg.V)
    assert r["margin"][0] > 1e-3
