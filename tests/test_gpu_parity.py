"""GPU parity of the HIP decode-step path against the CPU oracle.

Every case draws seeded synthetic inputs from ``workloads``, runs the C-ABI
entry points through the Python binding on the GPU and compares with the
oracle on the same input bytes:
  * integer outputs (permutation, argmax, commit set, window state) bit-exact;
  * attention outputs: max |gpu - oracle| / max |oracle| <= 1e-4 (fp32) and
    2e-2 (bf16), over every output row of every workload;
  * rotated queries/keys bit-exact: both sides round the float64 rotation
    once to the storage type.  The two compute the angle by different
    routes (p * 2^(-2c/D log2 base) vs p * base^(-2c/D)), which agree to
    about 1e-12 relative, so an element whose float64 value lies within
    1e-9 relative of a rounding tie may take either neighbour; every other
    element must be identical.  Values are copied bit-exactly.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
import causal_attention_diffusion_amd as wd
from parity_checks import rounding_exact

pytestmark = pytest.mark.gpu

ATTN_TOL = {"f32": 1e-4, "bf16": 2e-2}
ATTN_CFGS = ["tiny_f32", "qwen3_l2048", "ragged_b32", "long_b4"]


def rel_err(got, ref):
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30))


def run_reorder(t, cfg):
    wd.wedlm_reorder(t["filled"], t["pos"], t["q"], t["k"], t["v"], t["q_phys"], t["k_cache"],
                     t["v_cache"], t["block_table"], t["ctx_len"], t["perm"], cfg.rope_base,
                     dev_status=t["status"])


def run_attn(t, max_ctx):
    ws = wd.attn_workspace_tensor(t["q_phys"], t["k_cache"], t["block_table"], max_ctx)
    wd.wedlm_step_attn(t["q_phys"], t["k_cache"], t["v_cache"], t["block_table"], t["ctx_len"],
                       t["perm"], t["out"], max_ctx_len=max_ctx, workspace=ws, dev_status=t["status"])


def sample_rows(cfg, L, n, seed):
    """(b, r, h) rows to check: every (b, r) at the window edges plus random ones."""
    rng = np.random.default_rng(seed)
    rows = set()
    for b in range(cfg.B):
        for r in (0, cfg.W - 1):
            rows.add((b, r, int(rng.integers(cfg.Hq))))
    while len(rows) < n + 2 * cfg.B:
        rows.add((int(rng.integers(cfg.B)), int(rng.integers(cfg.W)), int(rng.integers(cfg.Hq))))
    return np.array(sorted(rows), np.int32)


def compare_rows(got, ref, rows, perm):
    g, o = [], []
    for b, r, h in rows:
        s = perm[b, r]
        g.append(got[b, s, h]); o.append(ref[b, s, h])
    return rel_err(np.array(g), np.array(o))


def _cfg(base_name, **kw):
    base = wl.CONFIGS[base_name]
    d = {f: getattr(base, f) for f in base.__dataclass_fields__}
    d.update(kw)
    return wl.AttnConfig(**d)


# A window of more than 2048 slots (B x W) takes the four-slots-per-work-
# group launch of the reorder (the Dual-Stream pass's shape); W = 18 leaves
# a two-slot tail group per sequence.
MANY_SLOTS = _cfg("qwen3_l2048", name="many_slots_b128_w18", B=128, W=18, L=0, L_range=(0, 300), n_obs=None,
                  seed=4711)


# ---------------------------------------------------------------- reorder
@pytest.mark.parametrize("name", ATTN_CFGS + ["many_slots_b128_w18"])
def test_reorder_parity(name, dev):
    cfg = MANY_SLOTS if name == MANY_SLOTS.name else wl.CONFIGS[name]
    print(f"[reorder] {name}", flush=True)
    inp = wl.make_attn_inputs(cfg)
    t = wl.device_attn_inputs(inp, dev)
    kc0, vc0 = t["k_cache"].clone(), t["v_cache"].clone()
    run_reorder(t, cfg)
    torch.cuda.synchronize()
    assert t["status"].item() == 0
    dt = cfg.dtype
    args = (inp.filled, inp.pos, wl.storage_to_f64(inp.q, dt), wl.storage_to_f64(inp.k, dt),
            wl.storage_to_f64(inp.v, dt))
    perm, qp, kw, vw = oracle.reorder(*args, dt, cfg.rope_base)
    _, qp64, kw64, _ = oracle.reorder(*args, "f64", cfg.rope_base)   # unrounded rotation
    np.testing.assert_array_equal(t["perm"].cpu().numpy(), perm)
    ties = rounding_exact(wl.torch_storage_to_f64(t["q_phys"], dt), qp, qp64)
    touched = torch.zeros(t["k_cache"].shape[:1] + t["k_cache"].shape[2:3], dtype=torch.bool, device=dev)
    for b in range(cfg.B):
        L = int(inp.ctx_len[b])
        tok = np.arange(L, L + cfg.W)
        pages = torch.from_numpy(inp.block_table[b, tok // wl.PAGE].astype(np.int64)).to(dev)
        slots = torch.from_numpy((tok % wl.PAGE).astype(np.int64)).to(dev)
        touched[pages, slots] = True
        gk = t["k_cache"][pages, :, slots, :]          # [W, Hkv, D]
        gv = t["v_cache"][pages, :, slots, :]
        ties += rounding_exact(wl.torch_storage_to_f64(gk, dt), kw[b], kw64[b])
        np.testing.assert_array_equal(wl.torch_storage_to_f64(gv, dt), vw[b])
    print(f"[reorder] {name}: q_phys and appended K bit-exact ({ties} tie-band elements)")
    # nothing outside the window's rows changed (committed K/V never move)
    keep = ~touched
    assert torch.equal(t["k_cache"].permute(0, 2, 1, 3)[keep], kc0.permute(0, 2, 1, 3)[keep])
    assert torch.equal(t["v_cache"].permute(0, 2, 1, 3)[keep], vc0.permute(0, 2, 1, 3)[keep])


def test_reorder_retry_is_idempotent(dev):
    """A repeated wedlm_reorder on the same window state rewrites only the
    window's cache rows [L, L+W) with the same bytes: a retried step is safe."""
    cfg = wl.CONFIGS["ragged_b32"]
    print("[reorder retry] ragged_b32", flush=True)
    inp = wl.make_attn_inputs(cfg)
    t = wl.device_attn_inputs(inp, dev)
    run_reorder(t, cfg)
    torch.cuda.synchronize()
    first = {k: t[k].clone() for k in ("q_phys", "k_cache", "v_cache", "perm")}
    run_reorder(t, cfg)
    torch.cuda.synchronize()
    assert t["status"].item() == 0
    for k, v in first.items():
        assert torch.equal(t[k], v), k


# ---------------------------------------------------------------- attention alone
def _attn_alone(cfg, dev, n_rows=None, seed=None, loud_keys=()):
    inp, q_phys, dk, dv = wl.make_full_cache_inputs(cfg, seed)
    for t, f in loud_keys:          # (token, factor): that key of every sequence scaled
        for b in range(cfg.B):
            if t < dk[b].shape[0]:
                dk[b][t] = wl.to_storage(wl.storage_to_f64(dk[b][t], cfg.dtype) * f, cfg.dtype)
    perm = oracle.reorder_perm(inp.filled)
    kc, vc = wl.paged_cache(inp, dk, dv)
    dt = cfg.dtype
    t = dict(q_phys=wl.as_torch(q_phys, dt, dev), k_cache=wl.as_torch(kc, dt, dev),
             v_cache=wl.as_torch(vc, dt, dev), block_table=torch.from_numpy(inp.block_table).to(dev),
             ctx_len=torch.from_numpy(inp.ctx_len).to(dev), perm=torch.from_numpy(perm).to(dev),
             status=torch.zeros(1, dtype=torch.int32, device=dev))
    t["out"] = torch.empty_like(t["q_phys"])
    run_attn(t, int(inp.ctx_len.max()))
    torch.cuda.synchronize()
    got = wl.torch_storage_to_f64(t["out"], dt)
    rows = None if n_rows is None else sample_rows(cfg, inp.ctx_len, n_rows, cfg.seed)
    ref = oracle.attention(wl.storage_to_f64(q_phys, dt), [wl.storage_to_f64(x, dt) for x in dk],
                           [wl.storage_to_f64(x, dt) for x in dv], inp.ctx_len, perm, rows=rows)
    status = t["status"].item()
    if rows is None:
        return rel_err(got, ref), status
    return compare_rows(got, ref, rows, perm), status


@pytest.mark.parametrize("name,n_rows", [("tiny_f32", None), ("qwen3_l2048", None),
                                         ("ragged_b32", None), ("long_b4", None)])
def test_attention_parity(name, n_rows, dev):
    cfg = wl.CONFIGS[name]
    print(f"[attn] {name}", flush=True)
    err, status = _attn_alone(cfg, dev, n_rows)
    print(f"[attn] {name}: max|gpu-oracle|/max|oracle| = {err:.3e} (tol {ATTN_TOL[cfg.dtype]})")
    assert status == 0
    assert err <= ATTN_TOL[cfg.dtype], err


LOUD = [
    # (label, config overrides, keys scaled by a factor): a few keys with
    # scores of tens of nats -- attention-sink-like logits -- in the first
    # tile, in the middle of a split, late in the prefix and in the window;
    # the softmax reference must move mid-stream, and the scores must not be
    # rounded to bf16 before the exponential
    ("M128_x20", dict(B=2, W=32, L=4096, n_obs=16), ((5, 20.0), (1500, 20.0), (3000, 20.0), (4100, 20.0))),
    ("M128_x60", dict(B=2, W=32, L=4096, n_obs=16), ((3000, 60.0), (3500, 120.0))),
    ("M128_late_x60", dict(B=2, W=32, L=4096, n_obs=16), ((4100, 60.0),)),
    ("M64_x20", dict(B=3, W=16, L=3000, n_obs=4), ((0, 20.0), (777, 20.0), (2999, 20.0), (3005, 20.0))),
    ("f32_M32_x20", dict(B=2, W=8, L=2000, n_obs=3, Hq=8, Hkv=2, D=64, dtype="f32",
                         positions=("contiguous",), rope_base=1e4), ((3, 20.0), (1000, 30.0), (2003, 20.0))),
]


@pytest.mark.parametrize("label,over,loud", LOUD, ids=[x[0] for x in LOUD])
def test_attention_large_scores(label, over, loud, dev):
    cfg = _cfg("qwen3_l2048", name=label, **over)
    print(f"[loud] {label}", flush=True)
    err, status = _attn_alone(cfg, dev, loud_keys=loud)
    print(f"[loud] {label}: max|gpu-oracle|/max|oracle| = {err:.3e} (tol {ATTN_TOL[cfg.dtype]})")
    assert status == 0
    assert err <= ATTN_TOL[cfg.dtype], err


def test_attention_at_maximum_context(dev):
    """The longest context the call accepts: 524288 keys including the
    window, planned as 64 splits of 8192 keys (the combine's limit and the
    largest block-table slice), on one KV head; sampled rows vs the oracle."""
    cfg = _cfg("qwen3_l2048", name="max_ctx", B=1, W=16, L=524288 - 16, n_obs=5, Hq=4, Hkv=1,
               dtype="bf16")
    print("[attn] max context 524288", flush=True)
    err, status = _attn_alone(cfg, dev, n_rows=24)
    print(f"[attn] max context: max|gpu-oracle|/max|oracle| = {err:.3e}")
    assert status == 0
    assert err <= ATTN_TOL["bf16"], err


# ---------------------------------------------------------------- reorder + attention
@pytest.mark.parametrize("name,n_rows", [("tiny_f32", None), ("qwen3_l2048", None),
                                         ("ragged_b32", None), ("long_b4", None)])
def test_decode_step_parity(name, n_rows, dev):
    cfg = wl.CONFIGS[name]
    print(f"[step] {name}", flush=True)
    inp = wl.make_attn_inputs(cfg)
    t = wl.device_attn_inputs(inp, dev)
    run_reorder(t, cfg)
    run_attn(t, int(inp.ctx_len.max()))
    torch.cuda.synchronize()
    assert t["status"].item() == 0
    rows = None if n_rows is None else sample_rows(cfg, inp.ctx_len, n_rows, cfg.seed + 1)
    ref = oracle.decode_step_attention(inp, rows=rows)
    got = wl.torch_storage_to_f64(t["out"], cfg.dtype)
    err = rel_err(got, ref["out"]) if rows is None else compare_rows(got, ref["out"], rows, ref["perm"])
    print(f"[step] {name}: max|gpu-oracle|/max|oracle| = {err:.3e} (tol {ATTN_TOL[cfg.dtype]})")
    assert err <= ATTN_TOL[cfg.dtype], err


# ---------------------------------------------------------------- edge cases
EDGE = [
    # (label, overrides, split_keys override)
    ("W1_L0", dict(B=2, W=1, L=0, n_obs=1, Hq=32, Hkv=8, D=128, dtype="bf16"), 0),
    ("all_masked", dict(B=2, W=16, L=100, n_obs=0, dtype="bf16"), 0),
    ("all_observed", dict(B=2, W=16, L=100, n_obs=16, dtype="bf16"), 0),
    ("W64_G4", dict(B=1, W=64, L=300, n_obs=20, dtype="bf16"), 0),
    ("G1_D64", dict(B=2, W=16, L=77, n_obs=5, Hq=8, Hkv=8, D=64, dtype="bf16"), 0),
    ("G8", dict(B=2, W=16, L=129, n_obs=7, Hq=32, Hkv=4, dtype="bf16"), 0),
    ("W64_G8_rowtiles4", dict(B=1, W=64, L=200, n_obs=31, Hq=64, Hkv=8, dtype="bf16"), 0),
    # the largest head grouping the header admits: 1024 query rows per KV head
    ("W64_G16_rowtiles8", dict(B=2, W=64, L=150, n_obs=20, Hq=64, Hkv=4, dtype="bf16"), 0),
    ("f32_W64_G16_D64", dict(B=1, W=64, L=90, n_obs=40, Hq=32, Hkv=2, D=64, dtype="f32",
                             positions=("contiguous",)), 0),
    ("ragged_tails_split64", dict(B=6, W=16, L_range=(1, 200), n_obs=None, dtype="bf16"), 64),
    ("ragged_tails_split128", dict(B=6, W=16, L_range=(1, 200), n_obs=None, dtype="bf16"), 128),
    ("f32_D128_split64", dict(B=2, W=8, L=150, n_obs=3, Hq=8, Hkv=2, D=128, dtype="f32",
                              positions=("contiguous",)), 64),
    ("f32_W24_G4", dict(B=1, W=24, L=40, n_obs=9, Hq=8, Hkv=2, D=64, dtype="f32",
                        positions=("contiguous",)), 0),
]


@pytest.mark.parametrize("label,over,split", EDGE, ids=[e[0] for e in EDGE])
def test_edge_cases(label, over, split, dev):
    cfg = _cfg("qwen3_l2048", name=label, **over)
    print(f"[edge] {label}", flush=True)
    wd.wedlm_set_attn_split_keys(split)
    try:
        err, status = _attn_alone(cfg, dev)
        print(f"[edge] {label}: attention err {err:.3e}")
        assert status == 0
        assert err <= ATTN_TOL[cfg.dtype], err
        inp = wl.make_attn_inputs(cfg)
        t = wl.device_attn_inputs(inp, dev)
        run_reorder(t, cfg)
        run_attn(t, int(inp.ctx_len.max()))
        torch.cuda.synchronize()
        assert t["status"].item() == 0
        ref = oracle.decode_step_attention(inp)
        np.testing.assert_array_equal(t["perm"].cpu().numpy(), ref["perm"])
        err2 = rel_err(wl.torch_storage_to_f64(t["out"], cfg.dtype), ref["out"])
        assert err2 <= ATTN_TOL[cfg.dtype], err2
    finally:
        wd.wedlm_set_attn_split_keys(0)


# Tail splits: a one-split plan whose longest sequences get a second
# work-group for the back half of their keys (ranked on the device, ties
# by index).  (label, overrides, sequences cut)
TAIL = [
    ("tail1_B64", dict(B=64, W=16, Hq=16, Hkv=4, L=0, L_range=(0, 3000), n_obs=None), 1),
    ("tail16_B64", dict(B=64, W=16, Hq=16, Hkv=4, L=0, L_range=(0, 3000), n_obs=None), 16),
    ("tail_all_ties_B64", dict(B=64, W=16, Hq=16, Hkv=4, L=0, L_range=(1000, 1002), n_obs=None), 64),
    ("tail_empty_halves_B64", dict(B=64, W=16, Hq=16, Hkv=4, L=0, L_range=(0, 40), n_obs=None), 32),
    ("tail8_D64_B32", dict(B=32, W=16, Hq=32, Hkv=8, D=64, L=0, L_range=(10, 2000), n_obs=None), 8),
    ("tail16_W1_B64", dict(B=64, W=1, Hq=32, Hkv=4, L=0, L_range=(0, 1500), n_obs=None), 16),
]


@pytest.mark.parametrize("label,over,tail", TAIL, ids=[x[0] for x in TAIL])
def test_tail_splits(label, over, tail, dev):
    cfg = _cfg("ragged_b32", name=label, **over)
    print(f"[tail] {label}: {tail} sequences cut", flush=True)
    wd.wedlm_set_attn_tail(tail)
    try:
        err, status = _attn_alone(cfg, dev)
        print(f"[tail] {label}: attention err {err:.3e}")
        assert status == 0
        assert err <= ATTN_TOL[cfg.dtype], err
        inp = wl.make_attn_inputs(cfg)
        t = wl.device_attn_inputs(inp, dev)
        mx = int(inp.ctx_len.max())
        assert wd.wedlm_attn_tail(t["q_phys"], t["k_cache"], t["block_table"], mx) == tail
        run_reorder(t, cfg)
        run_attn(t, mx)
        torch.cuda.synchronize()
        assert t["status"].item() == 0
        ref = oracle.decode_step_attention(inp)
        err2 = rel_err(wl.torch_storage_to_f64(t["out"], cfg.dtype), ref["out"])
        assert err2 <= ATTN_TOL[cfg.dtype], err2
    finally:
        wd.wedlm_set_attn_tail(-1)


def _random_shapes(n, seed):
    """Seeded draws over the shapes the entry points accept: batch, window
    (1..64), head grouping (G = 1..8), head dim, dtype, ragged prefixes
    (some empty), observed counts and split-size overrides."""
    rng = np.random.default_rng(seed)
    heads = [(8, 8), (8, 2), (16, 4), (32, 8), (32, 4), (64, 8), (4, 2)]
    out = []
    for i in range(n):
        hq, hkv = heads[int(rng.integers(len(heads)))]
        dtype = "f32" if rng.random() < 0.3 else "bf16"
        D = int(rng.choice([64, 128]))
        B = int(rng.integers(1, 5))
        W = int(rng.integers(1, 65))
        lo = int(rng.integers(0, 300))
        L_range = (lo, lo + int(rng.integers(0, 400)))
        split = int(rng.choice([0, 0, 64, 128, 320]))
        over = dict(B=B, W=W, Hq=hq, Hkv=hkv, D=D, dtype=dtype, L=0, L_range=L_range, n_obs=None,
                    seed=9000 + i, positions=("contiguous",), rope_base=1e4 if dtype == "f32" else 1e6)
        out.append((f"r{i}_B{B}W{W}G{hq // hkv}D{D}_{dtype}_s{split}", over, split))
    return out


@pytest.mark.parametrize("label,over,split", _random_shapes(24, 2027), ids=lambda v: v if isinstance(v, str) else "")
def test_random_shapes_reorder_attention(label, over, split, dev):
    # whole reorder + attention against the oracle on seeded random shapes
    cfg = _cfg("qwen3_l2048", name=label, **over)
    print(f"[random] {label}", flush=True)
    wd.wedlm_set_attn_split_keys(split)
    try:
        inp = wl.make_attn_inputs(cfg)
        t = wl.device_attn_inputs(inp, dev)
        run_reorder(t, cfg)
        run_attn(t, int(inp.ctx_len.max()))
        torch.cuda.synchronize()
        assert t["status"].item() == 0
        ref = oracle.decode_step_attention(inp)
        np.testing.assert_array_equal(t["perm"].cpu().numpy(), ref["perm"])
        err = rel_err(wl.torch_storage_to_f64(t["out"], cfg.dtype), ref["out"])
        assert err <= ATTN_TOL[cfg.dtype], err
    finally:
        wd.wedlm_set_attn_split_keys(0)


def test_split_count_does_not_change_result(dev):
    cfg = wl.CONFIGS["qwen3_l2048"]
    outs = []
    for sk in (0, 64, 256, 2112):
        wd.wedlm_set_attn_split_keys(sk)
        try:
            inp, q_phys, dk, dv = wl.make_full_cache_inputs(cfg)
            perm = oracle.reorder_perm(inp.filled)
            kc, vc = wl.paged_cache(inp, dk, dv)
            t = dict(q_phys=wl.as_torch(q_phys, "bf16", dev), k_cache=wl.as_torch(kc, "bf16", dev),
                     v_cache=wl.as_torch(vc, "bf16", dev),
                     block_table=torch.from_numpy(inp.block_table).to(dev),
                     ctx_len=torch.from_numpy(inp.ctx_len).to(dev), perm=torch.from_numpy(perm).to(dev),
                     status=torch.zeros(1, dtype=torch.int32, device=dev))
            t["out"] = torch.empty_like(t["q_phys"])
            run_attn(t, int(inp.ctx_len.max()))
            torch.cuda.synchronize()
            outs.append(t["out"].float().cpu().numpy())
        finally:
            wd.wedlm_set_attn_split_keys(0)
    for o in outs[1:]:
        assert rel_err(o, outs[0]) <= 1e-2


@pytest.mark.parametrize("tail", [-1, 2])
def test_device_status_bad_ctx_and_page(tail, dev):
    # tail = 2: the two longest sequences cut in two; the skipped one ranks last
    wd.wedlm_set_attn_tail(tail)
    try:
        _status_bad_ctx_and_page(dev)
    finally:
        wd.wedlm_set_attn_tail(-1)


def _status_bad_ctx_and_page(dev):
    cfg = _cfg("qwen3_l2048", B=3, L=50, n_obs=4)
    inp = wl.make_attn_inputs(cfg)
    t = wl.device_attn_inputs(inp, dev)
    run_reorder(t, cfg)
    torch.cuda.synchronize()
    assert t["status"].item() == 0
    # sequence 1: ctx_len beyond the block table; sequence 2: a page id outside the pool
    bad_ctx = t["ctx_len"].clone()
    bad_ctx[1] = inp.max_pages * wl.PAGE
    bt = t["block_table"].clone()
    bt[2, 1] = inp.num_pages + 5
    t2 = dict(t, ctx_len=bad_ctx, block_table=bt, status=torch.zeros(1, dtype=torch.int32, device=dev))
    t2["out"] = torch.full_like(t["out"], 7.0)
    run_attn(t2, int(inp.ctx_len.max()))
    torch.cuda.synchronize()
    st = t2["status"].item()
    assert st & 1 and st & 2
    assert torch.count_nonzero(t2["out"][1]).item() == 0      # skipped sequence -> zeros
    assert torch.isfinite(t2["out"].float()).all()
    # the reorder entry point reports the same conditions and leaves the cache alone
    t3 = dict(t, ctx_len=bad_ctx, status=torch.zeros(1, dtype=torch.int32, device=dev))
    kc0 = t["k_cache"].clone()
    run_reorder(t3, cfg)
    torch.cuda.synchronize()
    assert t3["status"].item() & 1
    assert torch.equal(kc0, t["k_cache"])


def test_attention_deterministic(dev):
    cfg = wl.CONFIGS["ragged_b32"]
    inp, q_phys, dk, dv = wl.make_full_cache_inputs(cfg)
    perm = oracle.reorder_perm(inp.filled)
    kc, vc = wl.paged_cache(inp, dk, dv)
    t = dict(q_phys=wl.as_torch(q_phys, "bf16", dev), k_cache=wl.as_torch(kc, "bf16", dev),
             v_cache=wl.as_torch(vc, "bf16", dev), block_table=torch.from_numpy(inp.block_table).to(dev),
             ctx_len=torch.from_numpy(inp.ctx_len).to(dev), perm=torch.from_numpy(perm).to(dev),
             status=torch.zeros(1, dtype=torch.int32, device=dev))
    res = []
    for _ in range(3):
        t["out"] = torch.empty_like(t["q_phys"])
        run_attn(t, int(inp.ctx_len.max()))
        res.append(t["out"].clone())
    torch.cuda.synchronize()
    assert torch.equal(res[0], res[1]) and torch.equal(res[0], res[2])


# ---------------------------------------------------------------- select / commit
def _state_to_dev(tok, filled, pos, ctx, dev):
    return (torch.from_numpy(np.ascontiguousarray(tok, np.int32)).to(dev),
            torch.from_numpy(np.ascontiguousarray(filled, np.uint8)).to(dev),
            torch.from_numpy(np.ascontiguousarray(pos, np.int32)).to(dev),
            torch.from_numpy(np.ascontiguousarray(ctx, np.int32)).to(dev))


def _gpu_select(logits, st, alpha, tau, mask_id, ws, counters=None):
    tok, filled, pos, ctx = st
    B, W, V = logits.shape
    dev = logits.device
    n_commit = torch.empty(B, dtype=torch.int32, device=dev)
    committed = torch.empty((B, W), dtype=torch.int32, device=dev)
    am = torch.empty((B, W), dtype=torch.int32, device=dev)
    ent = torch.empty((B, W), dtype=torch.float32, device=dev)
    wd.wedlm_select_commit(logits, tok, filled, pos, ctx, n_commit, committed, alpha, tau, mask_id, ws,
                           argmax_out=am, entropy_out=ent, counters=counters)
    return n_commit, committed, am, ent


def _check_step(ref, st, outs, rows=None):
    tok, filled, pos, ctx = st
    n_commit, committed, am, ent = outs
    sel = slice(None) if rows is None else rows
    assert (ref["margin"] > 1e-4).all(), ref["margin"]
    np.testing.assert_array_equal(n_commit.cpu().numpy()[sel], ref["n_commit"])
    np.testing.assert_array_equal(committed.cpu().numpy()[sel], ref["committed"])
    np.testing.assert_array_equal(am.cpu().numpy()[sel], ref["argmax"])
    np.testing.assert_array_equal(tok.cpu().numpy()[sel], ref["tok"])
    np.testing.assert_array_equal(filled.cpu().numpy()[sel], ref["filled"])
    np.testing.assert_array_equal(pos.cpu().numpy()[sel], ref["pos"])
    np.testing.assert_array_equal(ctx.cpu().numpy()[sel], ref["ctx_len"])
    e = ent.cpu().numpy()[sel]
    assert np.all(np.abs(e - ref["entropy"]) <= 1e-4 * np.maximum(1.0, np.abs(ref["entropy"])))


def test_select_tiny_teacher_forced(dev):
    cfg = wl.SELECT_CONFIGS["tiny_f32"]
    rng = np.random.default_rng(77)
    ws = wd.select_workspace_tensor(cfg.B, cfg.W, cfg.V, dev)
    lg = wl.make_logits_np(cfg, 0)
    for trial in range(20):
        filled = (rng.random((cfg.B, cfg.W)) < 0.5).astype(np.uint8)
        tok = np.where(filled == 1, rng.integers(0, cfg.V, (cfg.B, cfg.W)), cfg.V).astype(np.int32)
        ctx = np.array([int(rng.integers(0, 100))], np.int32)
        pos = ctx[:, None] + np.arange(cfg.W)[None]
        ref = oracle.select_commit(lg, tok, filled, pos, ctx, cfg.alpha, cfg.tau, cfg.V)
        st = _state_to_dev(tok, filled, pos, ctx, dev)
        outs = _gpu_select(torch.from_numpy(lg).to(dev), st, cfg.alpha, cfg.tau, cfg.V, ws)
        torch.cuda.synchronize()
        _check_step(ref, st, outs)


@pytest.mark.parametrize("B,W,V", [(8, 16, 4096), (3, 64, 1003), (2, 5, 1), (4, 16, 16388), (2, 8, 40000), (1, 4, 16386)])
def test_select_stream_small_free_running(B, W, V, dev):
    cfg = wl.SelectConfig("s", B=B, W=W, V=V, seed=4242 + V, alpha=0.25, tau=float(np.log(V) * 0.8) if V > 1 else 1.0,
                          steps=48, kind="mixture")
    ws = wd.select_workspace_tensor(B, W, V, dev)
    tok, filled, pos, ctx = wl.initial_window(B, W, V)
    st = _state_to_dev(tok, filled, pos, ctx, dev)
    # prefix-cacheability counters (N_new, N_total) accumulate on the device
    counters = torch.zeros((B, 2), dtype=torch.int64, device=dev)
    hist = []
    for step in range(cfg.steps):
        lg = wl.make_logits_np(cfg, step)
        if V < 16:
            lg[..., 0] += 3.0
        ref = oracle.select_commit(lg, tok, filled, pos, ctx, cfg.alpha, cfg.tau, V)
        hist.append(ref["n_commit"])
        outs = _gpu_select(torch.from_numpy(lg).to(dev), st, cfg.alpha, cfg.tau, V, ws, counters=counters)
        torch.cuda.synchronize()
        if V > 1:
            _check_step(ref, st, outs)
        else:
            np.testing.assert_array_equal(st[0].cpu().numpy(), ref["tok"])
            np.testing.assert_array_equal(st[1].cpu().numpy(), ref["filled"])
        tok, filled, pos, ctx = ref["tok"], ref["filled"], ref["pos"], ref["ctx_len"]
    n_new, n_total, _ = oracle.prefix_cacheability(hist, W)
    np.testing.assert_array_equal(counters.cpu().numpy(), np.stack([n_new, n_total], axis=1))


@pytest.mark.parametrize("parts", [3, 37, 200])
def test_select_forced_parts(parts, dev):
    """More vocabulary parts than the automatic plan (the commit kernel then
    merges more than one round of 16 partials per slot): same results."""
    B, W, V = 2, 24, 40000
    cfg = wl.SelectConfig("p", B=B, W=W, V=V, seed=99 + parts, alpha=0.25, tau=6.0, steps=4, kind="mixture")
    tok, filled, pos, ctx = wl.initial_window(B, W, V)
    wd.wedlm_set_select_parts(parts)
    try:
        ws = wd.select_workspace_tensor(B, W, V, dev)
        st = _state_to_dev(tok, filled, pos, ctx, dev)
        for step in range(cfg.steps):
            lg = wl.make_logits_np(cfg, step)
            ref = oracle.select_commit(lg, tok, filled, pos, ctx, cfg.alpha, cfg.tau, V)
            outs = _gpu_select(torch.from_numpy(lg).to(dev), st, cfg.alpha, cfg.tau, V, ws)
            torch.cuda.synchronize()
            _check_step(ref, st, outs)
            tok, filled, pos, ctx = ref["tok"], ref["filled"], ref["pos"], ref["ctx_len"]
    finally:
        wd.wedlm_set_select_parts(0)


def test_select_window_full_commits_all(dev):
    B, W, V = 2, 64, 100
    ws = wd.select_workspace_tensor(B, W, V, dev)
    tok = np.arange(B * W, dtype=np.int32).reshape(B, W) % V
    filled = np.ones((B, W), np.uint8)
    ctx = np.array([5, 9], np.int32)
    pos = ctx[:, None] + np.arange(W)[None]
    lg = np.zeros((B, W, V), np.float32)
    ref = oracle.select_commit(lg, tok, filled, pos, ctx, 0.1, 1.0, V)
    st = _state_to_dev(tok, filled, pos, ctx, dev)
    outs = _gpu_select(torch.from_numpy(lg).to(dev), st, 0.1, 1.0, V, ws)
    torch.cuda.synchronize()
    _check_step(ref, st, outs)
    assert ref["n_commit"].tolist() == [64, 64]


def test_select_full_vocab_step0_full_batch(dev):
    cfg = wl.SELECT_CONFIGS["select_v152k"]
    ws = wd.select_workspace_tensor(cfg.B, cfg.W, cfg.V, dev)
    logits = wl.make_logits_torch(cfg, 0, dev)
    tok, filled, pos, ctx = wl.initial_window(cfg.B, cfg.W, cfg.V)
    st = _state_to_dev(tok, filled, pos, ctx, dev)
    outs = _gpu_select(logits, st, cfg.alpha, cfg.tau, cfg.V, ws)
    torch.cuda.synchronize()
    ref = oracle.select_commit(logits.cpu().numpy(), tok, filled, pos, ctx, cfg.alpha, cfg.tau, cfg.V)
    _check_step(ref, st, outs)


def test_select_full_vocab_256_steps_sampled_sequences(dev):
    """All 64 sequences stream 256 steps on the GPU; the oracle follows 4 of
    them (sequences are independent) and must agree bit-exactly each step."""
    cfg = wl.SELECT_CONFIGS["select_v152k"]
    track = np.array([0, 21, 42, 63])
    ws = wd.select_workspace_tensor(cfg.B, cfg.W, cfg.V, dev)
    tok, filled, pos, ctx = wl.initial_window(cfg.B, cfg.W, cfg.V)
    st = _state_to_dev(tok, filled, pos, ctx, dev)
    o_tok, o_filled, o_pos, o_ctx = tok[track], filled[track], pos[track], ctx[track]
    logits = torch.empty((cfg.B, cfg.W, cfg.V), dtype=torch.float32, device=dev)
    track_t = torch.from_numpy(track).to(dev)
    total = 0
    for step in range(cfg.steps):
        wl.make_logits_torch(cfg, step, dev, out=logits)
        host = logits.index_select(0, track_t).cpu().numpy()
        outs = _gpu_select(logits, st, cfg.alpha, cfg.tau, cfg.V, ws)
        ref = oracle.select_commit(host, o_tok, o_filled, o_pos, o_ctx, cfg.alpha, cfg.tau, cfg.V)
        torch.cuda.synchronize()
        _check_step(ref, st, outs, rows=track)
        o_tok, o_filled, o_pos, o_ctx = ref["tok"], ref["filled"], ref["pos"], ref["ctx_len"]
        total += int(ref["n_commit"].sum())
        if step % 64 == 0:
            print(f"[select stream] step {step} committed {total}", flush=True)
    # every sequence advanced and windows kept their size and contiguous positions
    c = st[3].cpu().numpy()
    p = st[2].cpu().numpy()
    assert (c > 0).all()
    np.testing.assert_array_equal(p, c[:, None] + np.arange(cfg.W)[None])


def test_select_deterministic(dev):
    cfg = wl.SELECT_CONFIGS["select_v152k"]
    logits = wl.make_logits_torch(cfg, 3, dev)
    res = []
    for _ in range(3):
        ws = wd.select_workspace_tensor(cfg.B, cfg.W, cfg.V, dev)
        tok, filled, pos, ctx = wl.initial_window(cfg.B, cfg.W, cfg.V)
        filled[:, ::3] = 1
        st = _state_to_dev(tok, filled, pos, ctx, dev)
        outs = _gpu_select(logits, st, cfg.alpha, cfg.tau, cfg.V, ws)
        res.append([x.clone() for x in list(st) + list(outs)])
    torch.cuda.synchronize()
    for r in res[1:]:
        for a, b in zip(r, res[0]):
            assert torch.equal(a, b)
