"""Pins for prefix cacheability (CPU only): paper-summary page, "Key claims",
sec. 3.1, Eq. 4 -- P_c = N_new / N_total, committed tokens over the window
slots the decoder ran through.  The counts come from streams run through the oracle's
select step, checked against closed forms of two streams whose every
decision is forced."""
import numpy as np

import oracle
import workloads as wl

V = 50


def _stream(logits_fn, B, W, steps, alpha, tau, filled0=None):
    tok, filled, pos, ctx = wl.initial_window(B, W, V)
    if filled0 is not None:
        filled = filled0.copy()
        tok = np.where(filled == 1, 7, tok).astype(np.int32)
    hist = []
    for s in range(steps):
        out = oracle.select_commit(logits_fn(B, W), tok, filled, pos, ctx, alpha, tau, V)
        hist.append(out["n_commit"])
        tok, filled, pos, ctx = out["tok"], out["filled"], out["pos"], out["ctx_len"]
    return np.array(hist), ctx


def _ramp_logits(B, W):
    # slot j: one spike of height 20 - j over zeros, so entropy rises with j
    z = np.zeros((B, W, V), np.float32)
    for j in range(W):
        z[:, j, 3] = 20.0 - j
    return z


def test_one_fill_per_step_commits_one_per_step():
    # tau far below any entropy and alpha = 0: only the fallback fills, and
    # it takes slot 0 (lowest entropy) every step; step 1 commits nothing,
    # every later step commits the slot filled the step before
    B, W, S = 3, 8, 12
    hist, ctx = _stream(_ramp_logits, B, W, S, alpha=0.0, tau=-1e30)
    n_new, n_total, pc = oracle.prefix_cacheability(hist, W)
    np.testing.assert_array_equal(n_new, np.full(B, S - 1))
    np.testing.assert_array_equal(n_total, np.full(B, S * W))
    np.testing.assert_allclose(pc, (S - 1) / (S * W), rtol=1e-15)
    np.testing.assert_array_equal(ctx, n_new)   # committed tokens are exactly the cache growth


def test_everything_filled_commits_every_other_step():
    # tau above every entropy: every masked slot fills.  Commit precedes
    # select, so a step that commits the whole window leaves no masked slot
    # to fill until the refill's masks meet the next step: the stream
    # alternates between filling W slots and committing them
    B, W, S = 2, 16, 9
    hist, ctx = _stream(lambda b, w: np.zeros((b, w, V), np.float32), B, W, S, alpha=0.0, tau=1e30)
    np.testing.assert_array_equal(hist[:, 0], [0, W] * (S // 2) + [0] * (S % 2))
    n_new, n_total, pc = oracle.prefix_cacheability(hist, W)
    np.testing.assert_array_equal(n_new, np.full(B, (S // 2) * W))
    np.testing.assert_allclose(pc, (S // 2) / S, rtol=1e-15)


def test_counts_match_window_accounting():
    # on a random stream N_new equals the context growth, and N_total is
    # steps * W, whatever the decisions were
    rng = np.random.default_rng(5)
    B, W, S = 4, 16, 20
    hist, ctx = _stream(lambda b, w: rng.standard_normal((b, w, V)).astype(np.float32) * 3, B, W, S,
                        alpha=0.2, tau=2.5)
    n_new, n_total, pc = oracle.prefix_cacheability(hist, W)
    np.testing.assert_array_equal(n_new, ctx)
    np.testing.assert_array_equal(n_total, np.full(B, S * W))
    assert ((pc >= 0) & (pc <= 1)).all()
