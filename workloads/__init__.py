"""Seeded synthetic inputs for the WeDLM streaming-decode step.

This module only draws random numbers and lays them out in memory (storage
casts, paged-cache scatter).  It holds none of the method's arithmetic: no
reordering, no RoPE, no attention, no entropy, no commit rule.  Both the
GPU path and the CPU oracle take their inputs from here, byte for byte.

Workloads (sizes are the ones the method's decode step runs at; the shapes
follow the Qwen3-8B backbone named in the WeDLM paper summary, TL;DR):

* ``tiny_f32``     batch 1, 4 Q / 2 KV heads, head dim 64, 64 cached tokens,
                   window 8 (3 observed), logical positions drawn from
                   [64, 80), fp32, RoPE base 1e4; logits [8, 1000] ~ 2*N(0,1).
* ``qwen3_l2048``  batch 1, 32 Q / 8 KV heads, head dim 128, 2048 cached
                   tokens in 16-token pages, window 16 with 4 observed slots,
                   bf16, RoPE base 1e6.
* ``ragged_b32``   batch 32, same heads, prefix lengths uniform in
                   [512, 8192], pages in shuffled physical order, window 16
                   with a random observed/masked split per sequence.
* ``long_b4``      batch 4, same heads, 32768 cached tokens, window 32 with
                   16 observed slots.
* ``select_v152k`` batch 64 x window 16 fp32 logits over a 151936-entry
                   vocabulary; each row is low-entropy (N(0,1) with one
                   uniformly chosen index set to 12.0) or high-entropy
                   (N(0,1)) with probability 1/2 each.
* ``lmhead_v152k`` the same window and vocabulary with the logits produced
                   on the fly by the LM head: hidden states [64, 16, 4096]
                   and an output-embedding matrix [151936, 4096], both bf16
                   (Qwen3-8B's hidden size and vocabulary).  Weights are
                   N(0, 1/4096); a hidden row is N(0,1) noise (logits about
                   N(0,1)), and with probability 1/2 it also gets
                   12 w_k / |w_k|^2 for a uniformly chosen token k, which
                   lifts logit k by 12 (the low-entropy rows).

Values are N(0,1) unless stated.  bf16 storage is the round-to-nearest-even
cast of the fp32 draw; the returned arrays hold the raw 16-bit patterns
(``uint16``) so that both sides see identical bytes.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

PAGE = 16  # tokens per KV page


@dataclass(frozen=True)
class AttnConfig:
    name: str
    B: int
    W: int
    Hq: int
    Hkv: int
    D: int
    dtype: str  # "f32" | "bf16"
    rope_base: float
    seed: int
    # prefix lengths: fixed value or (lo, hi) inclusive uniform range
    L: int = 0
    L_range: Optional[tuple] = None
    # observed slots per sequence: fixed count or None for uniform in [0, W]
    n_obs: Optional[int] = None
    # logical positions: "contiguous" (L + i) or ("sorted_from", lo, hi)
    positions: tuple = ("contiguous",)
    shuffle_pages: bool = True
    extra: dict = field(default_factory=dict)


@dataclass(frozen=True)
class SelectConfig:
    name: str
    B: int
    W: int
    V: int
    seed: int
    alpha: float
    tau: float
    steps: int
    kind: str  # "mixture" (low/high entropy rows) | "normal_scaled"
    scale: float = 1.0


CONFIGS: Dict[str, object] = {
    "tiny_f32": AttnConfig("tiny_f32", B=1, W=8, Hq=4, Hkv=2, D=64, dtype="f32",
                           rope_base=1e4, seed=1001, L=64, n_obs=3,
                           positions=("sorted_from", 64, 80)),
    "qwen3_l2048": AttnConfig("qwen3_l2048", B=1, W=16, Hq=32, Hkv=8, D=128, dtype="bf16",
                              rope_base=1e6, seed=1002, L=2048, n_obs=4),
    "ragged_b32": AttnConfig("ragged_b32", B=32, W=16, Hq=32, Hkv=8, D=128, dtype="bf16",
                             rope_base=1e6, seed=1003, L_range=(512, 8192), n_obs=None),
    "long_b4": AttnConfig("long_b4", B=4, W=32, Hq=32, Hkv=8, D=128, dtype="bf16",
                          rope_base=1e6, seed=1004, L=32768, n_obs=16),
}

@dataclass(frozen=True)
class LmheadConfig:
    name: str
    B: int
    W: int
    Dm: int      # hidden size
    V: int
    seed: int
    alpha: float
    tau: float
    steps: int


LMHEAD_CONFIGS: Dict[str, LmheadConfig] = {
    "lmhead_small": LmheadConfig("lmhead_small", B=2, W=8, Dm=256, V=3000, seed=1101, alpha=0.25,
                                 tau=float(np.log(3000) * 0.8), steps=24),
    "lmhead_mid": LmheadConfig("lmhead_mid", B=12, W=16, Dm=1024, V=40000, seed=1102, alpha=0.25,
                               tau=float(np.log(40000) * 0.8), steps=6),
    "lmhead_v152k": LmheadConfig("lmhead_v152k", B=64, W=16, Dm=4096, V=151936, seed=1105, alpha=0.25,
                                 tau=9.0, steps=256),
}


@dataclass(frozen=True)
class ModelConfig:
    """A synthetic decoder for the whole-step path: `layers` pre-norm blocks
    of d_model = Hq * D, GQA attention, SwiGLU MLP of width d_ff."""
    name: str
    layers: int
    Hq: int
    Hkv: int
    D: int
    d_ff: int
    vocab: int
    B: int
    W: int
    seed: int
    alpha: float
    tau: float
    rope_base: float = 1e6
    eps: float = 1e-6
    steps: int = 1
    prefix: int = 0     # cached prompt tokens per sequence before the first step

    @property
    def d_model(self) -> int:
        return self.Hq * self.D


MODEL_CONFIGS: Dict[str, ModelConfig] = {
    "model_small": ModelConfig("model_small", layers=2, Hq=4, Hkv=2, D=64, d_ff=512, vocab=1000, B=2, W=8,
                               seed=1501, alpha=0.25, tau=float(np.log(1000) * 0.8), steps=6),
    "model_qwen3_layer": ModelConfig("model_qwen3_layer", layers=1, Hq=32, Hkv=8, D=128, d_ff=12288, vocab=32000,
                                     B=4, W=64, seed=1502, alpha=0.25, tau=float(np.log(32000) * 0.8)),
    # Qwen3-8B shapes: 36 layers, hidden 4096, 32/8 heads of 128, MLP 12288,
    # vocabulary 151936; batch 4 x the pages' window N = 64
    "model_qwen3_w64": ModelConfig("model_qwen3_w64", layers=36, Hq=32, Hkv=8, D=128, d_ff=12288,
                                   vocab=151936, B=4, W=64, seed=1503, alpha=0.25, tau=9.0, steps=16,
                                   prefix=2048),
}


SELECT_CONFIGS: Dict[str, SelectConfig] = {
    "tiny_f32": SelectConfig("tiny_f32", B=1, W=8, V=1000, seed=1001, alpha=0.25, tau=4.5,
                             steps=1, kind="normal_scaled", scale=2.0),
    "select_v152k": SelectConfig("select_v152k", B=64, W=16, V=151936, seed=1005, alpha=0.25,
                                 tau=9.0, steps=256, kind="mixture"),
}


# ----------------------------------------------------------------------------
# storage casts (input encoding only)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16; returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & 1
    r = (u + np.uint32(0x7FFF) + lsb) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(dtype)


def storage_to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return x.astype(np.float64)
    return bf16_bits_to_f32(x).astype(np.float64)


# ----------------------------------------------------------------------------
# attention-side inputs
# ----------------------------------------------------------------------------
@dataclass
class AttnInputs:
    cfg: AttnConfig
    ctx_len: np.ndarray          # [B] int32 (committed prefix length L_b)
    filled: np.ndarray           # [B, W] uint8
    pos: np.ndarray              # [B, W] int32 (logical positions)
    q: np.ndarray                # [B, W, Hq, D] storage dtype, logical slot order, pre-RoPE
    k: np.ndarray                # [B, W, Hkv, D]
    v: np.ndarray                # [B, W, Hkv, D]
    prefix_k: List[np.ndarray]   # per sequence [L_b, Hkv, D] storage dtype (already rotated keys)
    prefix_v: List[np.ndarray]
    block_table: np.ndarray      # [B, max_pages] int32, -1 where unused
    num_pages: int

    @property
    def max_pages(self) -> int:
        return self.block_table.shape[1]


def _prefix_lengths(cfg: AttnConfig, rng: np.random.Generator) -> np.ndarray:
    if cfg.L_range is not None:
        lo, hi = cfg.L_range
        return rng.integers(lo, hi + 1, size=cfg.B).astype(np.int32)
    return np.full(cfg.B, cfg.L, dtype=np.int32)


def _flags(cfg: AttnConfig, rng: np.random.Generator) -> np.ndarray:
    filled = np.zeros((cfg.B, cfg.W), dtype=np.uint8)
    for b in range(cfg.B):
        n = cfg.n_obs if cfg.n_obs is not None else int(rng.integers(0, cfg.W + 1))
        idx = rng.choice(cfg.W, size=n, replace=False)
        filled[b, idx] = 1
    return filled


def _positions(cfg: AttnConfig, L: np.ndarray, rng: np.random.Generator) -> np.ndarray:
    pos = np.zeros((cfg.B, cfg.W), dtype=np.int32)
    for b in range(cfg.B):
        if cfg.positions[0] == "contiguous":
            pos[b] = L[b] + np.arange(cfg.W)
        else:
            _, lo, hi = cfg.positions
            pos[b] = np.sort(rng.choice(np.arange(lo, hi), size=cfg.W, replace=False))
    return pos


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def make_block_table(L_plus_W: np.ndarray, rng: np.random.Generator, shuffle: bool,
                     spare_pages: int = 0, max_pages: Optional[int] = None):
    """Assign physical pages of a shared pool to each sequence (shuffled order)."""
    need = [(int(t) + PAGE - 1) // PAGE for t in L_plus_W]
    total = sum(need) + spare_pages
    order = rng.permutation(total).astype(np.int32) if shuffle else np.arange(total, dtype=np.int32)
    mp = max(need) if max_pages is None else max_pages
    bt = np.full((len(need), mp), -1, dtype=np.int32)
    o = 0
    for b, n in enumerate(need):
        bt[b, :n] = order[o:o + n]
        o += n
    return bt, total


def make_attn_inputs(cfg: AttnConfig, seed: Optional[int] = None, L_override=None,
                     spare_tokens: int = 0) -> AttnInputs:
    """Draw one batch of window + prefix-cache inputs.

    ``spare_tokens`` reserves block-table capacity beyond L_b + W for each
    sequence (streaming runs that append across several steps).
    """
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    L = _prefix_lengths(cfg, rng) if L_override is None else np.asarray(L_override, dtype=np.int32)
    filled = _flags(cfg, rng)
    pos = _positions(cfg, L, rng)
    q = to_storage(_normal(rng, (cfg.B, cfg.W, cfg.Hq, cfg.D)), cfg.dtype)
    k = to_storage(_normal(rng, (cfg.B, cfg.W, cfg.Hkv, cfg.D)), cfg.dtype)
    v = to_storage(_normal(rng, (cfg.B, cfg.W, cfg.Hkv, cfg.D)), cfg.dtype)
    pk, pv = [], []
    for b in range(cfg.B):
        pk.append(to_storage(_normal(rng, (int(L[b]), cfg.Hkv, cfg.D)), cfg.dtype))
        pv.append(to_storage(_normal(rng, (int(L[b]), cfg.Hkv, cfg.D)), cfg.dtype))
    bt, total = make_block_table(L + cfg.W + spare_tokens, rng, cfg.shuffle_pages)
    return AttnInputs(cfg, L, filled, pos, q, k, v, pk, pv, bt, total)


def paged_cache(inp: AttnInputs, dense_k: List[np.ndarray], dense_v: List[np.ndarray]):
    """Scatter per-sequence dense [T_b, Hkv, D] K/V into [P, Hkv, PAGE, D] pages."""
    cfg = inp.cfg
    st = np.float32 if cfg.dtype == "f32" else np.uint16
    kc = np.zeros((inp.num_pages, cfg.Hkv, PAGE, cfg.D), dtype=st)
    vc = np.zeros_like(kc)
    for b in range(cfg.B):
        T = dense_k[b].shape[0]
        t = np.arange(T)
        pages = inp.block_table[b, t // PAGE]
        assert (pages >= 0).all()
        kc[pages, :, t % PAGE, :] = dense_k[b]
        vc[pages, :, t % PAGE, :] = dense_v[b]
    return kc, vc


def gather_cache(inp: AttnInputs, kc: np.ndarray, vc: np.ndarray, b: int, t0: int, t1: int):
    """Read tokens [t0, t1) of sequence b back out of a paged cache (dense order)."""
    t = np.arange(t0, t1)
    pages = inp.block_table[b, t // PAGE]
    return kc[pages, :, t % PAGE, :], vc[pages, :, t % PAGE, :]


def make_full_cache_inputs(cfg: AttnConfig, seed: Optional[int] = None):
    """Inputs for the attention call alone: q already rotated and in physical
    order, the cache already holding all L_b + W tokens, a permutation drawn
    from random observed/masked flags.  Returns (AttnInputs, q_phys, dense_k,
    dense_v, perm_flags) where perm_flags are the flags the permutation is to
    be built from (the permutation itself is method arithmetic)."""
    rng = np.random.default_rng((cfg.seed if seed is None else seed) + 7919)
    L = _prefix_lengths(cfg, rng)
    filled = _flags(cfg, rng)
    pos = _positions(cfg, L, rng)
    q_phys = to_storage(_normal(rng, (cfg.B, cfg.W, cfg.Hq, cfg.D)), cfg.dtype)
    dk, dv = [], []
    for b in range(cfg.B):
        T = int(L[b]) + cfg.W
        dk.append(to_storage(_normal(rng, (T, cfg.Hkv, cfg.D)), cfg.dtype))
        dv.append(to_storage(_normal(rng, (T, cfg.Hkv, cfg.D)), cfg.dtype))
    bt, total = make_block_table(L + cfg.W, rng, cfg.shuffle_pages)
    empty = np.zeros((0,), dtype=q_phys.dtype)
    inp = AttnInputs(cfg, L, filled, pos, empty, empty, empty, [], [], bt, total)
    return inp, q_phys, dk, dv


# ----------------------------------------------------------------------------
# select/commit-side inputs
# ----------------------------------------------------------------------------
def initial_window(B: int, W: int, mask_id: int, L0: int = 0):
    """All-masked window at prefix length L0 (tok, filled, pos, ctx_len)."""
    tok = np.full((B, W), mask_id, dtype=np.int32)
    filled = np.zeros((B, W), dtype=np.uint8)
    ctx = np.full(B, L0, dtype=np.int32)
    pos = (ctx[:, None] + np.arange(W)[None, :]).astype(np.int32)
    return tok, filled, pos, ctx


def make_logits_np(cfg: SelectConfig, step: int, B: Optional[int] = None) -> np.ndarray:
    """Host draw of one step's logits [B, W, V] fp32 (seed = cfg.seed + step)."""
    B = cfg.B if B is None else B
    rng = np.random.default_rng(cfg.seed + step)
    z = _normal(rng, (B, cfg.W, cfg.V))
    if cfg.kind == "normal_scaled":
        z *= np.float32(cfg.scale)
    else:
        low = rng.random((B, cfg.W)) < 0.5
        idx = rng.integers(0, cfg.V, size=(B, cfg.W))
        bi, wi = np.nonzero(low)
        z[bi, wi, idx[bi, wi]] = np.float32(12.0)
    return z


def make_logits_torch(cfg: SelectConfig, step: int, device, out=None):
    """Device draw of one step's logits [B, W, V] fp32 with torch's generator
    on ``device`` (seed = cfg.seed + step).  Same recipe as make_logits_np,
    different random stream; used where a host draw of the full vocabulary
    every step would dominate the run time."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(cfg.seed + step)
    shape = (cfg.B, cfg.W, cfg.V)
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=device)
    out.normal_(generator=g)
    if cfg.kind == "normal_scaled":
        out.mul_(cfg.scale)
    else:
        low = torch.rand((cfg.B, cfg.W), generator=g, device=device) < 0.5
        idx = torch.randint(0, cfg.V, (cfg.B, cfg.W), generator=g, device=device)
        spike = torch.where(low, torch.full_like(idx, 1), torch.zeros_like(idx)).to(torch.bool)
        rows = out.view(cfg.B * cfg.W, cfg.V)
        flat_idx = idx.view(-1, 1)
        cur = rows.gather(1, flat_idx)
        rows.scatter_(1, flat_idx, torch.where(spike.view(-1, 1), torch.full_like(cur, 12.0), cur))
    return out


# ----------------------------------------------------------------------------
# LM-head inputs (hidden states and output embeddings, bf16)
# ----------------------------------------------------------------------------
def make_lm_head_np(cfg: LmheadConfig) -> np.ndarray:
    """Output-embedding matrix [V, Dm], N(0, 1/Dm), as bf16 bits."""
    rng = np.random.default_rng(cfg.seed)
    w = _normal(rng, (cfg.V, cfg.Dm))
    w *= np.float32(1.0 / np.sqrt(cfg.Dm))
    return f32_to_bf16_bits(w)


def make_hidden_np(cfg: LmheadConfig, step: int, lm_head_bits: np.ndarray,
                   B: Optional[int] = None) -> np.ndarray:
    """Hidden states [B, W, Dm] of one step as bf16 bits (seed = cfg.seed +
    1000 + step): N(0,1) rows; with probability 1/2 a row also gets
    12 w_k / |w_k|^2 for a uniformly drawn token k (w_k = row k of the
    stored output embeddings), which lifts its logit k by about 12."""
    B = cfg.B if B is None else B
    rng = np.random.default_rng(cfg.seed + 1000 + step)
    h = _normal(rng, (B, cfg.W, cfg.Dm))
    low = rng.random((B, cfg.W)) < 0.5
    idx = rng.integers(0, cfg.V, size=(B, cfg.W))
    bi, wi = np.nonzero(low)
    if len(bi):
        wk = bf16_bits_to_f32(lm_head_bits[idx[bi, wi]])
        h[bi, wi] += np.float32(12.0) * wk / np.sum(wk * wk, axis=1, keepdims=True)
    return f32_to_bf16_bits(h)


def make_lm_head_torch(cfg: LmheadConfig, device):
    """Device draw of the [V, Dm] bf16 output embeddings (torch's generator,
    seed = cfg.seed; same recipe as make_lm_head_np, other random stream)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(cfg.seed)
    w = torch.empty((cfg.V, cfg.Dm), dtype=torch.float32, device=device)
    w.normal_(generator=g)
    w.mul_(1.0 / float(np.sqrt(cfg.Dm)))
    return w.to(torch.bfloat16)


def make_hidden_torch(cfg: LmheadConfig, step: int, lm_head, device):
    """Device draw of one step's [B, W, Dm] bf16 hidden states (recipe of
    make_hidden_np, torch's generator, seed = cfg.seed + 1000 + step)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(cfg.seed + 1000 + step)
    h = torch.empty((cfg.B, cfg.W, cfg.Dm), dtype=torch.float32, device=device)
    h.normal_(generator=g)
    low = torch.rand((cfg.B, cfg.W), generator=g, device=device) < 0.5
    idx = torch.randint(0, cfg.V, (cfg.B, cfg.W), generator=g, device=device)
    wk = lm_head[idx.view(-1)].float().view(cfg.B, cfg.W, cfg.Dm)
    spike = 12.0 * wk / (wk * wk).sum(dim=-1, keepdim=True)
    h += torch.where(low[..., None], spike, torch.zeros_like(spike))
    return h.to(torch.bfloat16)


# ----------------------------------------------------------------------------
# synthetic decoder weights (bf16)
# ----------------------------------------------------------------------------
def _model_shapes(cfg: ModelConfig):
    d, F, q, kv = cfg.d_model, cfg.d_ff, cfg.Hq * cfg.D, cfg.Hkv * cfg.D
    layer = [("attn_norm", (d,), None), ("wq", (q, d), d), ("wk", (kv, d), d), ("wv", (kv, d), d),
             ("wo", (d, q), q), ("mlp_norm", (d,), None), ("w_gate", (F, d), d), ("w_up", (F, d), d),
             ("w_down", (d, F), F)]
    top = [("embed", (cfg.vocab + 1, d), 0), ("final_norm", (d,), None), ("lm_head", (cfg.vocab, d), d)]
    return top, layer


def make_model_np(cfg: ModelConfig) -> dict:
    """Weights as bf16 bits: embeddings N(0,1); norm weights 1 + 0.1 N(0,1);
    every projection N(0, 1/fan_in)."""
    rng = np.random.default_rng(cfg.seed)
    top, layer = _model_shapes(cfg)

    def draw(shape, fan_in):
        x = _normal(rng, shape)
        if fan_in is None:
            x = np.float32(1.0) + np.float32(0.1) * x
        elif fan_in:
            x *= np.float32(1.0 / np.sqrt(fan_in))
        return f32_to_bf16_bits(x)

    out = {n: draw(sh, f) for n, sh, f in top}
    out["layers"] = [{n: draw(sh, f) for n, sh, f in layer} for _ in range(cfg.layers)]
    return out


def make_model_torch(cfg: ModelConfig, device) -> dict:
    """Device draw of the same recipe (torch's generator, seed = cfg.seed)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(cfg.seed)
    top, layer = _model_shapes(cfg)

    def draw(shape, fan_in):
        x = torch.empty(shape, dtype=torch.float32, device=device).normal_(generator=g)
        if fan_in is None:
            x = 1.0 + 0.1 * x
        elif fan_in:
            x *= 1.0 / float(np.sqrt(fan_in))
        return x.to(torch.bfloat16)

    out = {n: draw(sh, f) for n, sh, f in top}
    out["layers"] = [{n: draw(sh, f) for n, sh, f in layer} for _ in range(cfg.layers)]
    return out


# ----------------------------------------------------------------------------
# device upload (torch tensors; storage bytes unchanged)
# ----------------------------------------------------------------------------
def as_torch(x: np.ndarray, dtype: str, device):
    """numpy storage array -> torch tensor on `device` (bf16 bits viewed as bfloat16)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "bf16":
        t = t.view(torch.bfloat16)
    return t.to(device)


def torch_storage_to_f64(t, dtype: str) -> np.ndarray:
    """torch tensor (any device) -> float64 numpy values of its storage."""
    import torch
    if dtype == "bf16":
        return bf16_bits_to_f32(t.detach().cpu().view(torch.int16).numpy().view(np.uint16)).astype(np.float64)
    return t.detach().cpu().numpy().astype(np.float64)


def device_attn_inputs(inp: AttnInputs, device, with_window: bool = True):
    """Upload one batch: window tensors, paged cache holding the prefix,
    block table and empty outputs (q_phys, perm, out, status)."""
    import torch
    cfg = inp.cfg
    dt = cfg.dtype
    kc, vc = paged_cache(inp, inp.prefix_k, inp.prefix_v)
    t = dict(
        filled=torch.from_numpy(inp.filled).to(device),
        pos=torch.from_numpy(inp.pos).to(device),
        ctx_len=torch.from_numpy(inp.ctx_len).to(device),
        block_table=torch.from_numpy(inp.block_table).to(device),
        k_cache=as_torch(kc, dt, device),
        v_cache=as_torch(vc, dt, device),
    )
    if with_window:
        t["q"] = as_torch(inp.q, dt, device)
        t["k"] = as_torch(inp.k, dt, device)
        t["v"] = as_torch(inp.v, dt, device)
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    t["q_phys"] = torch.empty((cfg.B, cfg.W, cfg.Hq, cfg.D), dtype=tdt, device=device)
    t["out"] = torch.empty((cfg.B, cfg.W, cfg.Hq, cfg.D), dtype=tdt, device=device)
    t["perm"] = torch.empty((cfg.B, cfg.W), dtype=torch.int32, device=device)
    t["status"] = torch.zeros(1, dtype=torch.int32, device=device)
    return t
