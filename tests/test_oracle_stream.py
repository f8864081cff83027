"""Cached stepping equals full recompute (CPU only).

Pages: WeDLM paper-summary page, "Method" (inference paragraph: the
committed leading prefix is cache-valid at once because attention is
strictly causal) and "Key claims" (paper sec. 5.2); risewithvishwas WeDLM
page, "Native Prefix-Cache Compatibility" (resolved tokens enter the KV cache
without recomputation or invalidation of earlier entries).

A 2-layer float64 toy model (random weights) is decoded for many streaming
steps with the oracle's reorder / attention / select-commit and a KV cache
that only ever grows by the committed rows.  At every step its logits and
its cached K/V are compared with an independent from-scratch forward (plain
numpy, complex-number RoPE, explicit lower-triangular mask) over
[committed tokens in logical order ++ reordered window].  A cache dropped
mid-stream and rebuilt from the committed tokens continues identically.
"""
import numpy as np
import pytest

import oracle

V, D_MODEL, LAYERS, HQ, HKV, HD, W, BASE = 64, 32, 2, 4, 2, 8, 8, 1e4
MASK = V


def _model(seed):
    rng = np.random.default_rng(seed)
    s = 1.0 / np.sqrt(D_MODEL)
    return dict(
        E=rng.standard_normal((V + 1, D_MODEL)),
        Wq=[rng.standard_normal((D_MODEL, HQ * HD)) * s for _ in range(LAYERS)],
        Wk=[rng.standard_normal((D_MODEL, HKV * HD)) * s for _ in range(LAYERS)],
        Wv=[rng.standard_normal((D_MODEL, HKV * HD)) * s for _ in range(LAYERS)],
        Wo=[rng.standard_normal((HQ * HD, D_MODEL)) * s * 0.5 for _ in range(LAYERS)],
        LM=rng.standard_normal((D_MODEL, V)) * 3.0 * s,
    )


def _cached_forward(m, caches, L, tok, filled, pos):
    """One decode step's forward through the oracle; appends the window's
    K/V to each layer's cache (caller truncates to the committed length)."""
    x = m["E"][tok]                                   # [W, d] logical slot order
    for l in range(LAYERS):
        q = (x @ m["Wq"][l]).reshape(1, W, HQ, HD)
        k = (x @ m["Wk"][l]).reshape(1, W, HKV, HD)
        v = (x @ m["Wv"][l]).reshape(1, W, HKV, HD)
        perm, qp, kw, vw = oracle.reorder(filled[None], pos[None], q, k, v, "f64", BASE)
        ck = np.concatenate([caches[l][0][:L], kw[0]], 0)
        cv = np.concatenate([caches[l][1][:L], vw[0]], 0)
        caches[l] = (ck, cv)
        o = oracle.attention(qp, [ck], [cv], np.array([L], np.int32), perm)[0]
        x = x + o.reshape(W, HQ * HD) @ m["Wo"][l]
    return x @ m["LM"]


def _rope_c(x, p):
    h = HD // 2
    w = BASE ** (-2.0 * np.arange(h) / HD)
    z = (x[..., :h] + 1j * x[..., h:]) * np.exp(1j * p[:, None, None] * w)
    return np.concatenate([z.real, z.imag], -1)


def _recompute(m, committed, tok, filled, pos):
    """From-scratch causal forward over committed ++ reordered window.
    Returns window logits in logical slot order and per-layer K/V."""
    L = len(committed)
    order = sorted(range(W), key=lambda i: (filled[i] == 0, i))
    ids = np.array(list(committed) + [tok[i] for i in order], dtype=np.int64)
    p = np.array(list(range(L)) + [pos[i] for i in order], dtype=np.float64)
    T = len(ids)
    x = m["E"][ids]
    mask = np.tril(np.ones((T, T), bool))
    kv = []
    for l in range(LAYERS):
        q = _rope_c((x @ m["Wq"][l]).reshape(T, HQ, HD), p)
        k = _rope_c((x @ m["Wk"][l]).reshape(T, HKV, HD), p)
        v = (x @ m["Wv"][l]).reshape(T, HKV, HD)
        kv.append((k, v))
        o = np.zeros((T, HQ, HD))
        for h in range(HQ):
            g = h // (HQ // HKV)
            s = (q[:, h] @ k[:, g].T) / np.sqrt(HD)
            s = np.where(mask, s, -np.inf)
            a = np.exp(s - s.max(1, keepdims=True))
            a /= a.sum(1, keepdims=True)
            o[:, h] = a @ v[:, g]
        x = x + o.reshape(T, HQ * HD) @ m["Wo"][l]
    logits_phys = (x @ m["LM"])[L:]
    out = np.empty_like(logits_phys)
    out[order] = logits_phys
    return out, kv


def _prefill(m, prompt):
    """Cache for a fully committed prompt, built through the oracle in one
    causal pass (every slot observed)."""
    n = len(prompt)
    caches = [(np.zeros((0, HKV, HD)), np.zeros((0, HKV, HD))) for _ in range(LAYERS)]
    x = m["E"][np.array(prompt)]
    filled = np.ones((1, n), np.uint8)
    pos = np.arange(n, dtype=np.int32)[None]
    for l in range(LAYERS):
        q = (x @ m["Wq"][l]).reshape(1, n, HQ, HD)
        k = (x @ m["Wk"][l]).reshape(1, n, HKV, HD)
        v = (x @ m["Wv"][l]).reshape(1, n, HKV, HD)
        perm, qp, kw, vw = oracle.reorder(filled, pos, q, k, v, "f64", BASE)
        caches[l] = (kw[0], vw[0])
        o = oracle.attention(qp, [kw[0]], [vw[0]], np.array([0], np.int32), perm)[0]
        x = x + o.reshape(n, HQ * HD) @ m["Wo"][l]
    return caches


def _stream(seed, steps, drop_at=None, check=True):
    m = _model(seed)
    rng = np.random.default_rng(seed + 100)
    committed = list(rng.integers(0, V, 5))
    caches = _prefill(m, committed)
    tok = np.full(W, MASK, np.int32)
    filled = np.zeros(W, np.uint8)
    L = len(committed)
    pos = (L + np.arange(W)).astype(np.int32)
    history = []
    for step in range(steps):
        if drop_at is not None and step == drop_at:
            caches = _prefill(m, committed)           # cache loss: rebuild from committed ids
        logits = _cached_forward(m, caches, L, tok, filled, pos)
        if check:
            ref, kv = _recompute(m, committed, tok, filled, pos)
            np.testing.assert_allclose(logits, ref, rtol=0, atol=1e-10)
            for l in range(LAYERS):
                np.testing.assert_allclose(caches[l][0][:L], kv[l][0][:L], rtol=0, atol=1e-10)
                np.testing.assert_allclose(caches[l][1][:L], kv[l][1][:L], rtol=0, atol=1e-10)
        r = oracle.select_commit(logits[None].astype(np.float32), tok[None], filled[None],
                                 pos[None], np.array([L], np.int32), 0.15, 3.2, MASK)
        k = int(r["n_commit"][0])
        committed.extend(r["committed"][0, :k].tolist())
        L += k
        caches = [(ck[:L], cv[:L]) for ck, cv in caches]   # keep only the committed rows
        tok, filled, pos = r["tok"][0], r["filled"][0], r["pos"][0]
        assert r["ctx_len"][0] == L == len(committed)
        history.append(list(committed))
    return history


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_cached_stepping_equals_recompute(seed):
    hist = _stream(seed, steps=40)
    # committed tokens never change: every later history extends the earlier one
    for a, b in zip(hist, hist[1:]):
        assert b[:len(a)] == a
    assert len(hist[-1]) > 40


def test_cache_loss_recovery_continues_identically():
    a = _stream(7, steps=30, check=False)
    b = _stream(7, steps=30, drop_at=13, check=False)
    assert a[-1] == b[-1]
