"""Pins for the oracle's LM head + select step (CPU only).

The LM head maps each slot's final hidden state to vocabulary logits (the
backbone's output projection; WeDLM paper-summary page, "Method",
inference paragraph: masked slots are filled from the model's predictive
distribution).  The oracle composes a float64 contraction with the
already-pinned select step, so its pins check the contraction against
brute force and the composition against cases that reduce to the select
step on known logits.
"""
import math

import numpy as np

import oracle
import workloads as wl


def test_logits_brute_force():
    rng = np.random.default_rng(7)
    h = rng.standard_normal((2, 3, 5))
    w = rng.standard_normal((7, 5))
    z = oracle.lmhead_logits(h, w)
    assert z.shape == (2, 3, 7)
    for b in range(2):
        for j in range(3):
            for v in range(7):
                ref = math.fsum(h[b, j, k] * w[v, k] for k in range(5))
                assert abs(z[b, j, v] - ref) < 1e-12


def test_logits_transposed_operand_is_caught():
    # a transposed weight matrix is a shape error, not a silent result
    h = np.ones((1, 1, 4))
    w = np.ones((4, 6))
    try:
        oracle.lmhead_logits(h, w)
    except ValueError:
        return
    raise AssertionError("mismatched hidden size accepted")


def test_zero_hidden_gives_uniform_rows():
    B, W, Dm, V = 1, 4, 8, 37
    h = np.zeros((B, W, Dm))
    w = np.random.default_rng(1).standard_normal((V, Dm))
    tok, filled, pos, ctx = wl.initial_window(B, W, V)
    out = oracle.lmhead_select_commit(h, w, tok, filled, pos, ctx, 0.25, math.log(V) + 1.0, V)
    # every logit is 0: H = ln V and the argmax is token 0 in every masked slot
    np.testing.assert_allclose(out["entropy"], math.log(V), rtol=1e-6)
    assert (out["argmax"] == 0).all()
    assert (out["tok"] == 0).all()


def test_identity_head_reduces_to_select_step():
    # with V = Dm and an identity matrix the logits are the hidden states
    rng = np.random.default_rng(3)
    B, W, V = 3, 8, 64
    h = rng.standard_normal((B, W, V)).astype(np.float32) * 2.0
    tok, filled, pos, ctx = wl.initial_window(B, W, V)
    filled[:, [1, 4]] = 1
    tok[:, [1, 4]] = 5
    a = oracle.lmhead_select_commit(h, np.eye(V), tok, filled, pos, ctx, 0.25, 3.0, V)
    b = oracle.select_commit(h, tok, filled, pos, ctx, 0.25, 3.0, V)
    for k in ["tok", "filled", "pos", "ctx_len", "n_commit", "committed", "argmax"]:
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)
    np.testing.assert_array_equal(a["entropy"], b["entropy"])


def test_permuted_vocabulary_permutes_argmax():
    # reordering the rows of the head reorders the vocabulary: argmax moves
    # with its row, the entropy does not change
    rng = np.random.default_rng(4)
    B, W, Dm, V = 2, 6, 16, 50
    h = rng.standard_normal((B, W, Dm))
    w = rng.standard_normal((V, Dm))
    perm = rng.permutation(V)
    tok, filled, pos, ctx = wl.initial_window(B, W, V)
    a = oracle.lmhead_select_commit(h, w, tok, filled, pos, ctx, 0.25, 2.0, V)
    b = oracle.lmhead_select_commit(h, w[perm], tok, filled, pos, ctx, 0.25, 2.0, V)
    np.testing.assert_array_equal(perm[b["argmax"]], a["argmax"])
    np.testing.assert_allclose(a["entropy"], b["entropy"], rtol=1e-6)


def test_generator_spike_rows_are_low_entropy():
    # the input recipe: spiked rows have their drawn token as argmax and an
    # entropy far below the unspiked rows (whose logits are about N(0,1))
    cfg = wl.LmheadConfig("t", B=2, W=16, Dm=256, V=2000, seed=5, alpha=0.25, tau=1.0, steps=1)
    w = wl.make_lm_head_np(cfg)
    h = wl.make_hidden_np(cfg, 0, w)
    z = oracle.lmhead_logits(wl.bf16_bits_to_f32(h), wl.bf16_bits_to_f32(w))
    am, H = oracle.row_stats(z.astype(np.float32))
    top = np.sort(z, axis=-1)[..., -2:]
    spiked = (top[..., 1] - top[..., 0]) > 6.0
    assert 8 <= spiked.sum() <= 24
    assert (H[spiked] < 3.0).all() and (H[~spiked] > 6.0).all()
    assert abs(np.std(z[~spiked]) - 1.0) < 0.1
