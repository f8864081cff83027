"""Comparison helpers shared by the GPU parity tests.

rounding_exact: a value both sides round once from float64 to its storage
type must be identical, except inside a tiny band around a rounding tie,
where the two float64 routes (which differ in the last bits) may pick
different neighbours.

check_select_step: slot-by-slot comparison of one GPU commit / select /
refill step with the
oracle's, for steps whose logits the GPU computes itself (the fused LM head
and the model step): the GPU accumulates a logit in fp32, the oracle in
float64, so where a row's two largest logits are closer than the fp32
rounding of the contraction either token is a correct argmax.

Everything is compared, every step, every slot:
  * n_commit, committed, filled, pos, ctx_len: identical (entropies and
    hence every fill decision do not depend on which tied token is chosen);
  * argmax: identical, except at a near-tie slot, where the GPU's token must
    be within `tie` of the oracle's float64 maximum of that row;
  * tok: identical to the oracle's, except at the window position a slot
    filled in this step moves to (slot j -> j - n_commit) -- there the token
    is the GPU's own argmax of that slot (so it differs from the oracle's
    only at near-tie slots);
  * entropy of every masked slot within 1e-4 relative.
"""
import numpy as np

TIE_BAND = 1e-9


def rounding_exact(got, rounded, ref64):
    """got == rounded (the oracle's single rounding of ref64) everywhere,
    except where ref64 sits within TIE_BAND (relative) of the tie between
    the two: there both neighbours are correct.  Returns the number of such
    tie-band elements (expected 0 or a handful)."""
    got = np.asarray(got, np.float64)
    rounded = np.asarray(rounded, np.float64)
    ref64 = np.asarray(ref64, np.float64)
    diff = got != rounded
    if not diff.any():
        return 0
    mid = 0.5 * (got[diff] + rounded[diff])
    near = np.abs(ref64[diff] - mid) <= TIE_BAND * np.abs(ref64[diff])
    assert near.all(), (np.count_nonzero(~near), got[diff][~near][:4], rounded[diff][~near][:4],
                        ref64[diff][~near][:4])
    return int(diff.sum())


def check_select_step(ref, z64, filled_before, st, outs, tie=1e-3):
    """ref: oracle.select_commit / lmhead_select_commit result of the step;
    z64: float64 logits [B, W, V] of the oracle (rows of masked slots);
    filled_before: [B, W] flags the step started from; st: GPU window state
    after the step (tok, filled, pos, ctx_len) as numpy arrays; outs: GPU
    (n_commit, committed, argmax, entropy) as numpy arrays.  Returns the
    number of near-tie slots."""
    tok, filled, pos, ctx = st
    n_commit, committed, am, ent = outs
    assert (ref["margin"] > 1e-4).all(), ref["margin"]
    np.testing.assert_array_equal(n_commit, ref["n_commit"])
    np.testing.assert_array_equal(committed, ref["committed"])
    np.testing.assert_array_equal(filled, ref["filled"])
    np.testing.assert_array_equal(pos, ref["pos"])
    np.testing.assert_array_equal(ctx, ref["ctx_len"])
    masked = ref["argmax"] >= 0
    np.testing.assert_array_equal(am >= 0, masked)
    ties = 0
    for b, j in zip(*np.nonzero(masked)):
        a_ref, a_gpu = ref["argmax"][b, j], am[b, j]
        if a_gpu != a_ref:
            zz = z64[b, j]
            assert zz.max() - zz[a_gpu] <= tie, (b, j, a_ref, a_gpu, zz.max() - zz[a_gpu])
            ties += 1
    # expected tokens: the oracle's, with each slot filled in this step
    # carrying the GPU's (checked) argmax at its shifted position
    want = np.array(ref["tok"], copy=True)
    B, W = want.shape
    for b in range(B):
        k = int(ref["n_commit"][b])
        for i in range(W - k):
            j = i + k
            if filled_before[b, j] == 0 and ref["filled"][b, i] == 1:
                want[b, i] = am[b, j]
    np.testing.assert_array_equal(tok, want)
    e, r = ent[masked], ref["entropy"][masked]
    assert np.all(np.abs(e - r) <= 1e-4 * np.maximum(1.0, np.abs(r)))
    return ties
