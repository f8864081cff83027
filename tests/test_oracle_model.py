"""Pins for the oracle's synthetic decoder step (CPU only).

The decoder block is this library's reading (the pages name a Qwen3-8B
backbone, paper-summary page TL;DR, not its layer): pre-norm RMSNorm, GQA
attention run as a WeDLM decode step (reordered window over the cache),
SwiGLU MLP, residuals.  Pins: RMSNorm and SiLU against closed forms and
scipy; a model whose residual branches are zero reduces to the normalised
embeddings; and cached streaming steps (storage in float64) equal an
independent from-scratch forward -- complex-number RoPE, an explicit
lower-triangular mask over [committed tokens ++ reordered window] -- at
every step, with the cache holding exactly the recomputed K/V.
"""
import numpy as np
import pytest
import scipy.special

import oracle

HQ, HKV, HD, D_MODEL, D_FF, V, W, LAYERS, BASE, EPS = 4, 2, 8, 32, 48, 50, 8, 2, 1e4, 1e-6


def test_rms_norm_closed_forms():
    g = np.linspace(0.5, 1.5, 7)
    c = np.full(7, -3.0)
    np.testing.assert_allclose(oracle.rms_norm(c, g, 0.0), -g, rtol=1e-15)
    np.testing.assert_allclose(oracle.rms_norm(c, g, 1.0), -3.0 / np.sqrt(10.0) * g, rtol=1e-15)
    x = np.random.default_rng(0).standard_normal((3, 7))
    np.testing.assert_allclose(oracle.rms_norm(5.0 * x, g, 0.0), oracle.rms_norm(x, g, 0.0), rtol=1e-13)
    y = oracle.rms_norm(x, np.ones(7), 0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), 1.0, rtol=1e-13)


def test_silu_matches_scipy():
    x = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(oracle.silu(x), x * scipy.special.expit(x), rtol=1e-13, atol=1e-300)
    assert oracle.silu(np.array([0.0]))[0] == 0.0


def _model(seed, zero_branches=False):
    rng = np.random.default_rng(seed)
    q, kv = HQ * HD, HKV * HD

    def lin(o, i):
        return np.zeros((o, i)) if zero_branches else rng.standard_normal((o, i)) / np.sqrt(i)

    layers = []
    for _ in range(LAYERS):
        layers.append(dict(attn_norm=1 + 0.1 * rng.standard_normal(D_MODEL), wq=lin(q, D_MODEL) + 0,
                           wk=rng.standard_normal((kv, D_MODEL)) / np.sqrt(D_MODEL),
                           wv=rng.standard_normal((kv, D_MODEL)) / np.sqrt(D_MODEL),
                           wo=lin(D_MODEL, q), mlp_norm=1 + 0.1 * rng.standard_normal(D_MODEL),
                           w_gate=rng.standard_normal((D_FF, D_MODEL)) / np.sqrt(D_MODEL),
                           w_up=rng.standard_normal((D_FF, D_MODEL)) / np.sqrt(D_MODEL),
                           w_down=lin(D_MODEL, D_FF)))
    return dict(embed=rng.standard_normal((V + 1, D_MODEL)), final_norm=1 + 0.1 * rng.standard_normal(D_MODEL),
                lm_head=rng.standard_normal((V, D_MODEL)) * 3.0 / np.sqrt(D_MODEL), layers=layers)


def _empty_caches(B):
    return [([np.zeros((0, HKV, HD))] * B, [np.zeros((0, HKV, HD))] * B) for _ in range(LAYERS)]


def test_zero_branches_give_normalised_embeddings():
    m = _model(1, zero_branches=True)
    rng = np.random.default_rng(2)
    tok = rng.integers(0, V + 1, (2, W)).astype(np.int32)
    filled = rng.integers(0, 2, (2, W)).astype(np.uint8)
    pos = np.tile(np.arange(W, dtype=np.int32), (2, 1))
    out = oracle.model_step(m, _empty_caches(2), tok, filled, pos, np.zeros(2, np.int32), 0.25, 2.0, BASE, EPS,
                            HQ, HKV, storage="f64")
    e = m["embed"][tok]
    ref = e / np.sqrt(np.mean(e * e, -1, keepdims=True) + EPS) * m["final_norm"]
    np.testing.assert_allclose(out["hidden"], ref, rtol=1e-13)


def _rope_c(x, p):
    h = HD // 2
    w = BASE ** (-2.0 * np.arange(h) / HD)
    z = (x[..., :h] + 1j * x[..., h:]) * np.exp(1j * p[:, None, None] * w)
    return np.concatenate([z.real, z.imag], -1)


def _recompute(m, committed, tok, filled, pos):
    """From-scratch forward over committed ++ reordered window; returns the
    window's final hidden states in logical slot order and per-layer K/V."""
    L = len(committed)
    order = sorted(range(W), key=lambda i: (filled[i] == 0, i))
    ids = np.array(list(committed) + [tok[i] for i in order], dtype=np.int64)
    p = np.array(list(range(L)) + [pos[i] for i in order], dtype=np.float64)
    T = len(ids)
    x = m["embed"][ids]
    mask = np.tril(np.ones((T, T), bool))

    def norm(x, g):
        return x / np.sqrt(np.mean(x * x, -1, keepdims=True) + EPS) * g

    kv = []
    for lw in m["layers"]:
        h = norm(x, lw["attn_norm"])
        q = _rope_c((h @ lw["wq"].T).reshape(T, HQ, HD), p)
        k = _rope_c((h @ lw["wk"].T).reshape(T, HKV, HD), p)
        v = (h @ lw["wv"].T).reshape(T, HKV, HD)
        kv.append((k, v))
        o = np.zeros((T, HQ, HD))
        for hh in range(HQ):
            g = hh // (HQ // HKV)
            s = np.where(mask, (q[:, hh] @ k[:, g].T) / np.sqrt(HD), -np.inf)
            a = np.exp(s - s.max(1, keepdims=True))
            o[:, hh] = (a / a.sum(1, keepdims=True)) @ v[:, g]
        x = x + o.reshape(T, HQ * HD) @ lw["wo"].T
        h = norm(x, lw["mlp_norm"])
        gt = h @ lw["w_gate"].T
        x = x + (gt / (1 + np.exp(-gt)) * (h @ lw["w_up"].T)) @ lw["w_down"].T
    hid = norm(x, m["final_norm"])[L:]
    out = np.empty_like(hid)
    out[order] = hid
    return out, kv


@pytest.mark.parametrize("seed", [3, 4])
def test_cached_stepping_equals_recompute(seed):
    m = _model(seed)
    caches = _empty_caches(1)
    committed = []
    tok = np.full((1, W), V, np.int32)
    filled = np.zeros((1, W), np.uint8)
    pos = np.arange(W, dtype=np.int32)[None]
    ctx = np.zeros(1, np.int32)
    for step in range(12):
        out = oracle.model_step(m, caches, tok, filled, pos, ctx, 0.25, 2.6, BASE, EPS, HQ, HKV, storage="f64")
        ref, kv = _recompute(m, committed, tok[0], filled[0], pos[0])
        np.testing.assert_allclose(out["hidden"][0], ref, rtol=0, atol=1e-10)
        L = int(ctx[0])
        for l in range(LAYERS):
            np.testing.assert_allclose(out["caches"][l][0][0][:L], kv[l][0][:L], rtol=0, atol=1e-10)
            np.testing.assert_allclose(out["caches"][l][1][0][:L], kv[l][1][:L], rtol=0, atol=1e-10)
        k = int(out["n_commit"][0])
        committed.extend(out["committed"][0, :k].tolist())
        ctx = out["ctx_len"]
        caches = [([ck[0][:ctx[0]]], [cv[0][:ctx[0]]]) for ck, cv in out["caches"]]
        tok, filled, pos = out["tok"], out["filled"], out["pos"]
    assert len(committed) >= 3
