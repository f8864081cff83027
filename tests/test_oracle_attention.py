"""Pins for the oracle's windowed causal GQA attention (CPU only).

Pages: WeDLM paper-summary page, "Key claims" (paper sec. 3.2: mask recovery
only needs every masked slot to see all observed tokens; sec. 4.1: after
Topological Reordering a plain causal mask gives exactly that; sec. 5.2: a
decode step is causal attention of the window over the cached prefix) and
risewithvishwas WeDLM page, "Attention Mechanism" row.

Independent formulations used here:
* logical-order attention with an explicit visibility matrix (the pages'
  central equivalence, sec. 3.2 / 4.1);
* torch.nn.functional.scaled_dot_product_attention (a library routine) on
  the physical sequence with a causal boolean mask;
* closed forms: one visible key, equal scores, constant values per KV head.
"""
import itertools

import numpy as np
import pytest
import torch

import oracle


def _perm(f):
    return sorted(range(len(f)), key=lambda i: (f[i] == 0, i))


def _visible(fi, fj, i, j):
    """Logical-order visibility: observed slots see observed slots up to
    themselves; masked slots see every observed slot and masked slots up to
    themselves (the set a causal mask gives after reordering)."""
    return (fj and ((not fi) or j <= i)) or ((not fi) and (not fj) and j <= i)


def _logical_attention(qL, kL, vL, kc, vc, f, scale, G):
    """qL [W,Hq,D], kL/vL [W,Hkv,D] in logical slot order; kc/vc [L,Hkv,D]."""
    W, Hq, D = qL.shape
    out = np.zeros_like(qL)
    for i in range(W):
        for h in range(Hq):
            g = h // G
            keys = [kc[t, g] for t in range(kc.shape[0])]
            vals = [vc[t, g] for t in range(kc.shape[0])]
            for j in range(W):
                if _visible(f[i], f[j], i, j):
                    keys.append(kL[j, g]); vals.append(vL[j, g])
            s = np.array([qL[i, h] @ kk for kk in keys]) * scale
            p = np.exp(s - s.max()); p /= p.sum()
            out[i, h] = (p[:, None] * np.array(vals)).sum(0)
    return out


def _run_oracle_logical(qL, kL, vL, kc, vc, f, scale=None):
    """Reorder logical-order rows to physical order and call the oracle."""
    W = qL.shape[0]
    perm = np.array(_perm(f), np.int32)
    qp = qL[perm][None]
    dk = [np.concatenate([kc, kL[perm]], 0)]
    dv = [np.concatenate([vc, vL[perm]], 0)]
    return oracle.attention(qp, dk, dv, np.array([kc.shape[0]], np.int32), perm[None], scale=scale)[0]


@pytest.mark.parametrize("W", [1, 2, 3, 5, 8])
def test_reordered_causal_equals_explicit_visibility_all_patterns(W):
    rng = np.random.default_rng(10 + W)
    Hq, Hkv, D, L = 4, 2, 8, 5
    for bits in itertools.product([0, 1], repeat=W):
        f = np.array(bits, np.uint8)
        qL = rng.standard_normal((W, Hq, D)); kL = rng.standard_normal((W, Hkv, D))
        vL = rng.standard_normal((W, Hkv, D))
        kc = rng.standard_normal((L, Hkv, D)); vc = rng.standard_normal((L, Hkv, D))
        got = _run_oracle_logical(qL, kL, vL, kc, vc, f)
        ref = _logical_attention(qL, kL, vL, kc, vc, f, 1 / np.sqrt(D), Hq // Hkv)
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_masked_slot_sees_all_observed_tokens():
    # A masked slot's output changes when ANY observed slot's value changes,
    # including observed slots logically after it; it does not change when a
    # later masked slot changes.
    rng = np.random.default_rng(20)
    W, Hq, Hkv, D, L = 6, 2, 1, 8, 3
    f = np.array([0, 1, 0, 1, 1, 0], np.uint8)
    qL = rng.standard_normal((W, Hq, D)); kL = rng.standard_normal((W, Hkv, D))
    vL = rng.standard_normal((W, Hkv, D))
    kc = rng.standard_normal((L, Hkv, D)); vc = rng.standard_normal((L, Hkv, D))
    base = _run_oracle_logical(qL, kL, vL, kc, vc, f)
    for j in range(W):
        v2 = vL.copy(); v2[j] += 1.0
        o = _run_oracle_logical(qL, kL, v2, kc, vc, f)
        changed = np.abs(o[0] - base[0]).max() > 1e-9   # slot 0 is masked
        assert changed == (bool(f[j]) or j == 0), j


def test_matches_torch_sdpa_on_physical_sequence():
    rng = np.random.default_rng(21)
    B, W, Hq, Hkv, D = 3, 7, 8, 2, 16
    G = Hq // Hkv
    L = np.array([0, 4, 19], np.int32)
    qp = rng.standard_normal((B, W, Hq, D))
    dk = [rng.standard_normal((int(L[b]) + W, Hkv, D)) for b in range(B)]
    dv = [rng.standard_normal((int(L[b]) + W, Hkv, D)) for b in range(B)]
    f = rng.integers(0, 2, (B, W)).astype(np.uint8)
    perm = np.array([_perm(f[b]) for b in range(B)], np.int32)
    out = oracle.attention(qp, dk, dv, L, perm)
    for b in range(B):
        T = int(L[b]) + W
        q = torch.tensor(qp[b]).permute(1, 0, 2)                      # [Hq, W, D]
        k = torch.tensor(dk[b]).permute(1, 0, 2).repeat_interleave(G, 0)  # [Hq, T, D]
        v = torch.tensor(dv[b]).permute(1, 0, 2).repeat_interleave(G, 0)
        mask = torch.arange(T)[None, :] <= (int(L[b]) + torch.arange(W))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask)
        ref = ref.permute(1, 0, 2).numpy()                             # [W, Hq, D] physical
        np.testing.assert_allclose(out[b][perm[b]], ref, rtol=0, atol=1e-12)


def test_single_key_returns_its_value():
    rng = np.random.default_rng(22)
    D = 8
    qp = rng.standard_normal((1, 1, 2, D))
    k = rng.standard_normal((1, 1, D)); v = rng.standard_normal((1, 1, D))
    out = oracle.attention(qp, [k], [v], np.array([0], np.int32), np.array([[0]], np.int32))
    np.testing.assert_allclose(out[0, 0, 0], v[0, 0], atol=1e-15)
    np.testing.assert_allclose(out[0, 0, 1], v[0, 0], atol=1e-15)


def test_equal_scores_give_mean_of_visible_values():
    rng = np.random.default_rng(23)
    W, L, D = 4, 6, 8
    qp = np.zeros((1, W, 2, D))
    k = rng.standard_normal((L + W, 1, D)); v = rng.standard_normal((L + W, 1, D))
    perm = np.array([[2, 0, 3, 1]], np.int32)
    out = oracle.attention(qp, [k], [v], np.array([L], np.int32), perm)
    for r in range(W):
        np.testing.assert_allclose(out[0, perm[0, r], 1], v[:L + r + 1, 0].mean(0), atol=1e-13)


def test_gqa_head_groups_are_contiguous():
    # KV head g carries constant value c_g, so query head h returns c_{h // G}
    rng = np.random.default_rng(24)
    W, L, D, Hq, Hkv = 3, 5, 8, 8, 4
    qp = rng.standard_normal((1, W, Hq, D))
    k = rng.standard_normal((L + W, Hkv, D))
    c = np.arange(1, Hkv + 1, dtype=np.float64)
    v = np.broadcast_to(c[None, :, None], (L + W, Hkv, D)).copy()
    out = oracle.attention(qp, [k], [v], np.array([L], np.int32), np.array([[0, 1, 2]], np.int32))
    for h in range(Hq):
        np.testing.assert_allclose(out[0, :, h, :], c[h // (Hq // Hkv)], atol=1e-13)


def test_scale_argument_and_row_subset():
    rng = np.random.default_rng(25)
    W, L, D = 3, 4, 8
    qp = rng.standard_normal((1, W, 2, D))
    k = rng.standard_normal((L + W, 1, D)); v = rng.standard_normal((L + W, 1, D))
    perm = np.array([[1, 2, 0]], np.int32)
    full = oracle.attention(qp, [k], [v], np.array([L], np.int32), perm, scale=0.3)
    doubled_q = oracle.attention(qp * 2, [k], [v], np.array([L], np.int32), perm, scale=0.15)
    np.testing.assert_allclose(full, doubled_q, atol=1e-13)
    rows = np.array([[0, 2, 1], [0, 0, 0]], np.int32)     # (b, r, h)
    sub = oracle.attention(qp, [k], [v], np.array([L], np.int32), perm, scale=0.3, rows=rows)
    np.testing.assert_array_equal(sub[0, perm[0, 2], 1], full[0, perm[0, 2], 1])
    np.testing.assert_array_equal(sub[0, perm[0, 0], 0], full[0, perm[0, 0], 0])
    assert np.isnan(sub[0, perm[0, 1], 0]).all()


def test_later_physical_rows_do_not_affect_earlier_ones():
    rng = np.random.default_rng(26)
    W, L, D = 5, 3, 8
    qp = rng.standard_normal((1, W, 2, D))
    k = rng.standard_normal((L + W, 1, D)); v = rng.standard_normal((L + W, 1, D))
    perm = np.array([[0, 1, 2, 3, 4]], np.int32)
    base = oracle.attention(qp, [k], [v], np.array([L], np.int32), perm)
    k2 = k.copy(); v2 = v.copy()
    k2[L + 3] += 5.0; v2[L + 3] -= 2.0
    o = oracle.attention(qp, [k2], [v2], np.array([L], np.int32), perm)
    np.testing.assert_array_equal(o[0, :3], base[0, :3])
    assert np.abs(o[0, 3:] - base[0, 3:]).max() > 1e-6
