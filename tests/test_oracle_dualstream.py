"""Pins for the oracle's Dual-Stream Masking attention (CPU only).

WeDLM paper-summary page, "Method" (training paragraph) and "Key claims"
(sec. 4.2, Eq. 8-10): a clean memory stream and a block-masked prediction
stream share position ids; a prediction token of block i attends to the
memory tokens that precede block i.  The pins reduce the oracle to torch's
scaled_dot_product_attention (a library routine, float64, CPU) in the cases
where the mask is a plain causal or a plain prefix-plus-causal mask, check
the block locality the rule implies, and check the composition the GPU path
uses: one block equals a decode step over the memory prefix.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from workloads import f32_to_bf16_bits, bf16_bits_to_f32

BASE = 1e4


def _inputs(S, N, Hq, Hkv, D, seed, dtype="bf16"):
    rng = np.random.default_rng(seed)
    def draw(h):
        x = rng.standard_normal((S, N, h, D)).astype(np.float32)
        return bf16_bits_to_f32(f32_to_bf16_bits(x)).astype(np.float64) if dtype == "bf16" else x.astype(np.float64)
    return draw(Hq), draw(Hkv), draw(Hkv), draw(Hq), draw(Hkv), draw(Hkv), rng


def _rot(x, dtype):
    """RoPE at positions 0..N-1 and storage rounding, per token (oracle.rope)."""
    S, N, H, D = x.shape
    y = np.empty_like(x)
    for s in range(S):
        for t in range(N):
            for h in range(H):
                y[s, t, h] = [oracle.round_storage(v, dtype) for v in oracle.rope(x[s, t, h], t, BASE)]
    return y


def _sdpa(q, k, v, mask):
    """torch SDPA, float64: q [n, Hq, D], k/v [m, Hkv, D], mask [n, m] bool."""
    G = q.shape[1] // k.shape[1]
    qt = torch.from_numpy(q).permute(1, 0, 2)
    kt = torch.from_numpy(np.repeat(k, G, axis=1)).permute(1, 0, 2)
    vt = torch.from_numpy(np.repeat(v, G, axis=1)).permute(1, 0, 2)
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(mask))
    return o.permute(1, 0, 2).numpy()


def test_visibility_small_example():
    # N = 4, block 2, prediction flags [1, 0 | 0, 1]
    v = oracle.dual_stream_visible(np.array([1, 0, 0, 1]), 2)
    m = v[:4, :4]
    assert (m == np.tril(np.ones((4, 4), bool))).all()
    assert not v[:4, 4:].any()                                   # memory never sees predictions
    pm = v[4:, :4]
    assert not pm[:2].any() and (pm[2:] == [[1, 1, 0, 0]] * 2).all()
    pp = v[4:, 4:]
    expect = np.array([[1, 0, 0, 0],     # t0 observed: itself
                       [1, 1, 0, 0],     # t1 masked: observed t0 and itself
                       [0, 0, 1, 1],     # t2 masked: observed t3 (later!) and itself
                       [0, 0, 0, 1]], bool)   # t3 observed: itself only
    assert (pp == expect).all()


def test_memory_stream_is_causal_attention():
    qm, km, vm, qp, kp, vp, rng = _inputs(1, 24, 4, 2, 16, 1)
    flags = rng.integers(0, 2, (1, 24))
    om, _ = oracle.dual_stream_attention(qm, km, vm, qp, kp, vp, flags, 8, "bf16", BASE)
    q, k = _rot(qm, "bf16")[0], _rot(km, "bf16")[0]
    ref = _sdpa(q, k, vm[0], np.tril(np.ones((24, 24), bool)))
    np.testing.assert_allclose(om[0], ref, rtol=1e-10, atol=1e-12)


def test_single_block_all_observed_is_causal_attention_on_predictions():
    qm, km, vm, qp, kp, vp, _ = _inputs(1, 16, 4, 1, 16, 2)
    _, op = oracle.dual_stream_attention(qm, km, vm, qp, kp, vp, np.ones((1, 16)), 16, "bf16", BASE)
    ref = _sdpa(_rot(qp, "bf16")[0], _rot(kp, "bf16")[0], vp[0], np.tril(np.ones((16, 16), bool)))
    np.testing.assert_allclose(op[0], ref, rtol=1e-10, atol=1e-12)


def test_all_masked_block_is_prefix_plus_causal():
    N, b, c = 32, 8, 2                     # block 2: tokens 16..23
    qm, km, vm, qp, kp, vp, _ = _inputs(1, N, 2, 2, 8, 3)
    flags = np.ones((1, N), np.uint8)
    flags[0, c * b:(c + 1) * b] = 0
    _, op = oracle.dual_stream_attention(qm, km, vm, qp, kp, vp, flags, b, "bf16", BASE)
    kr = np.concatenate([_rot(km, "bf16")[0, :c * b], _rot(kp, "bf16")[0, c * b:(c + 1) * b]])
    vv = np.concatenate([vm[0, :c * b], vp[0, c * b:(c + 1) * b]])
    mask = np.zeros((b, c * b + b), bool)
    mask[:, :c * b] = True
    mask[:, c * b:] = np.tril(np.ones((b, b), bool))
    ref = _sdpa(_rot(qp, "bf16")[0, c * b:(c + 1) * b], kr, vv, mask)
    np.testing.assert_allclose(op[0, c * b:(c + 1) * b], ref, rtol=1e-10, atol=1e-12)


def test_block_locality():
    # a prediction block depends on the memory tokens before it and on its
    # own tokens only
    N, b = 32, 8
    qm, km, vm, qp, kp, vp, rng = _inputs(1, N, 2, 1, 8, 4)
    flags = rng.integers(0, 2, (1, N))
    _, op = oracle.dual_stream_attention(qm, km, vm, qp, kp, vp, flags, b, "bf16", BASE)
    km2, vm2, kp2, vp2 = km.copy(), vm.copy(), kp.copy(), vp.copy()
    km2[0, 16:] += 3.0; vm2[0, 16:] -= 2.0          # memory at and after block 2
    kp2[0, 24:] += 1.0; vp2[0, :16] *= -1.0          # other blocks' predictions
    flags2 = flags.copy(); flags2[0, :16] = 1 - flags2[0, :16]
    _, op2 = oracle.dual_stream_attention(qm, km2, vm2, qp, kp2, vp2, flags2, b, "bf16", BASE)
    np.testing.assert_array_equal(op[0, 16:24], op2[0, 16:24])
    assert not np.allclose(op[0, 24:], op2[0, 24:])  # block 3 did see the changed memory


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_block_equals_decode_step_over_memory_prefix(dtype):
    # the reduction the GPU path uses: prediction block c is one decode step
    # (window = block, reordered by its flags) over a cache holding the
    # memory stream's first c*b rotated keys
    N, b, c = 48, 16, 2
    qm, km, vm, qp, kp, vp, rng = _inputs(1, N, 4, 2, 16, 5, dtype)
    flags = rng.integers(0, 2, (1, N)).astype(np.uint8)
    _, op = oracle.dual_stream_attention(qm, km, vm, qp, kp, vp, flags, b, dtype, BASE)
    sl = slice(c * b, (c + 1) * b)
    pos = np.arange(c * b, (c + 1) * b, dtype=np.int32)[None]
    perm, qph, kw, vw = oracle.reorder(flags[:, sl], pos, qp[:, sl], kp[:, sl], vp[:, sl], dtype, BASE)
    ones = np.ones((1, N), np.uint8)
    _, _, kmr, _ = oracle.reorder(ones, np.arange(N, dtype=np.int32)[None], qm, km, vm, dtype, BASE)
    dk = [np.concatenate([kmr[0, :c * b], kw[0]])]
    dv = [np.concatenate([vm[0, :c * b], vw[0]])]
    out = oracle.attention(qph, dk, dv, np.array([c * b], np.int32), perm)
    np.testing.assert_allclose(op[0, sl], out[0], rtol=1e-10, atol=1e-12)
