"""Pins for the oracle's Topological Reordering, logical RoPE and storage
rounding (CPU only).

Pages: WeDLM paper-summary page, "Key claims" (paper sec. 4.1, Eq. 5-6) and
"Method" (inference paragraph); risewithvishwas WeDLM page, "Topological
Reordering" bullet.  Each check uses a formulation independent of the
oracle's code: a stable sort for the permutation, complex multiplication for
the rotation, integer bit arithmetic for bf16 rounding.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
from workloads import f32_to_bf16_bits, bf16_bits_to_f32

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- reorder
def test_reorder_golden_examples():
    d = json.load(open(os.path.join(GOLD, "reorder_examples.json")))
    for case in d["cases"]:
        perm = oracle.reorder_perm(np.array(case["filled"], np.uint8))
        assert perm.tolist() == case["perm"], case


@pytest.mark.parametrize("W", range(1, 11))
def test_reorder_all_flag_patterns_vs_stable_sort(W):
    for bits in itertools.product([0, 1], repeat=W):
        f = np.array(bits, np.uint8)
        perm = oracle.reorder_perm(f)
        ref = sorted(range(W), key=lambda i: (f[i] == 0, i))  # observed first, stable
        assert perm.tolist() == ref
        # a permutation; the leading filled run stays physically first and in place
        assert sorted(perm.tolist()) == list(range(W))
        k = next((i for i in range(W) if not f[i]), W)
        assert perm[:k].tolist() == list(range(k))


# ---------------------------------------------------------------- RoPE
def _rope_complex(x, p, base):
    """Rotation as complex multiplication: (x_c + i x_{c+D/2}) * e^{i p w_c}."""
    D = x.shape[-1]
    h = D // 2
    w = base ** (-2.0 * np.arange(h) / D)
    z = (x[..., :h] + 1j * x[..., h:]) * np.exp(1j * p * w)
    return np.concatenate([z.real, z.imag], axis=-1)


@pytest.mark.parametrize("D,base", [(64, 1e4), (128, 1e6), (8, 10.0)])
def test_rope_matches_complex_rotation(D, base):
    rng = np.random.default_rng(0)
    for p in [0, 1, 7, 64, 2063, 32799, 40000]:
        x = rng.standard_normal(D)
        # angles reach 4e4 rad: argument reduction costs ~p * 1e-16 absolute
        np.testing.assert_allclose(oracle.rope(x, p, base), _rope_complex(x, p, base),
                                   rtol=0, atol=1e-12 + 1e-15 * p)


def test_rope_identity_at_zero_and_pair_norms():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(128)
    np.testing.assert_array_equal(oracle.rope(x, 0, 1e6), x)
    y = oracle.rope(x, 12345, 1e6)
    h = 64
    np.testing.assert_allclose(x[:h] ** 2 + x[h:] ** 2, y[:h] ** 2 + y[h:] ** 2, rtol=1e-12)


def test_rope_first_pair_turns_by_p_radians():
    # c = 0 has angular frequency 1: e_0 goes to (cos p) e_0 + (sin p) e_{D/2}
    D = 16
    e0 = np.zeros(D); e0[0] = 1.0
    for p in [1, 3, 100]:
        y = oracle.rope(e0, p, 1e4)
        assert abs(y[0] - math.cos(p)) < 1e-12 and abs(y[D // 2] - math.sin(p)) < 1e-12
        assert np.abs(np.delete(y, [0, D // 2])).max() < 1e-12


def test_rope_scores_depend_only_on_relative_position():
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    for p, pk in [(70, 64), (5, 99), (33000, 12)]:
        s0 = oracle.rope(q, p, 1e4) @ oracle.rope(k, pk, 1e4)
        for shift in [1, 17, 1000]:
            s1 = oracle.rope(q, p + shift, 1e4) @ oracle.rope(k, pk + shift, 1e4)
            assert abs(s0 - s1) < 1e-9


# ---------------------------------------------------------------- storage rounding
def test_bf16_rounding_matches_bit_arithmetic():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32),
                        (rng.standard_normal(2000) * 1e-30).astype(np.float32),
                        (rng.standard_normal(2000) * 1e30).astype(np.float32)])
    ref = bf16_bits_to_f32(f32_to_bf16_bits(x)).astype(np.float64)
    got = np.array([oracle.round_storage(float(v), "bf16") for v in x])
    np.testing.assert_array_equal(got, ref)


def test_bf16_rounding_ties_to_even():
    assert oracle.round_storage(1.0 + 2.0 ** -8, "bf16") == 1.0              # tie -> even (down)
    assert oracle.round_storage(1.0 + 3 * 2.0 ** -8, "bf16") == 1.0 + 2.0 ** -6  # tie -> even (up)
    assert oracle.round_storage(1.0 + 2.0 ** -8 + 2.0 ** -30, "bf16") == 1.0 + 2.0 ** -7
    assert oracle.round_storage(-1.0 - 2.0 ** -8, "bf16") == -1.0
    assert oracle.round_storage(0.1, "f32") == float(np.float32(0.1))


# ---------------------------------------------------------------- reorder step
def test_reorder_step_places_rows_and_rotates_at_logical_positions():
    rng = np.random.default_rng(4)
    B, W, Hq, Hkv, D, base = 2, 6, 4, 2, 8, 1e4
    filled = np.array([[1, 0, 1, 0, 0, 1], [0, 0, 0, 1, 1, 0]], np.uint8)
    pos = np.array([[3, 4, 8, 9, 10, 15], [20, 21, 22, 23, 24, 25]], np.int32)
    q = rng.standard_normal((B, W, Hq, D))
    k = rng.standard_normal((B, W, Hkv, D))
    v = rng.standard_normal((B, W, Hkv, D))
    perm, qp, kw, vw = oracle.reorder(filled, pos, q, k, v, "f32", base)
    for b in range(B):
        ref = sorted(range(W), key=lambda i: (filled[b, i] == 0, i))
        assert perm[b].tolist() == ref
        for r, slot in enumerate(ref):
            p = pos[b, slot]
            np.testing.assert_allclose(qp[b, r], _rope_complex(q[b, slot], p, base).astype(np.float32),
                                       atol=1e-6, rtol=0)
            np.testing.assert_allclose(kw[b, r], _rope_complex(k[b, slot], p, base).astype(np.float32),
                                       atol=1e-6, rtol=0)
            np.testing.assert_array_equal(vw[b, r], v[b, slot])
    # stored values are exactly fp32-representable
    assert (qp.astype(np.float32).astype(np.float64) == qp).all()


def test_reorder_rejects_non_increasing_positions():
    f = np.zeros((1, 3), np.uint8)
    x = np.zeros((1, 3, 1, 4))
    with pytest.raises(ValueError):
        oracle.reorder(f, np.array([[5, 5, 6]], np.int32), x, x, x, "f32", 1e4)
