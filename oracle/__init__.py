"""CPU oracle for the WeDLM streaming-decode step -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg import this package.  The product library never does.
The arithmetic lives in ``wedlm_oracle.c`` (plain C + OpenMP, float64);
this module only marshals numpy arrays to it.

Every function is pinned by the CPU test suite (tests/test_oracle_*.py)
against closed forms, brute force on tiny inputs and the invariants the
pages fix; none is "parity unpinned".
"""
from __future__ import annotations

import ctypes as C
import os
from typing import List, Optional, Sequence

import numpy as np

from . import build as _build

_LIB = None
F32, BF16, F64 = 0, 1, 2
_DT = {"f32": F32, "bf16": BF16, "f64": F64}


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB) or (
                os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC)):
            _build.build()
        lib = C.CDLL(_build.LIB)
        P = C.c_void_p
        i32, i64, f64 = C.c_int, C.c_int64, C.c_double
        lib.wo_num_threads.restype = i32
        lib.wo_round_storage.argtypes = [f64, i32]
        lib.wo_round_storage.restype = f64
        lib.wo_reorder_perm.argtypes = [i32, P, P]
        lib.wo_reorder_perm.restype = i32
        lib.wo_rope.argtypes = [i32, f64, C.c_int32, P, P]
        lib.wo_rope.restype = None
        lib.wo_reorder.argtypes = [i32, i32, i32, i32, i32, i32, f64, P, P, P, P, P, P, P, P, P]
        lib.wo_reorder.restype = i32
        lib.wo_attention.argtypes = [i32, i32, i32, i32, i32, f64, P, P, P, P, P, P, i64, P, P]
        lib.wo_attention.restype = None
        lib.wo_row_stats.argtypes = [i32, P, P, P]
        lib.wo_row_stats.restype = None
        lib.wo_vocab_stats.argtypes = [i64, i32, P, P, P]
        lib.wo_vocab_stats.restype = None
        lib.wo_select_commit.argtypes = [i32, i32, i32, P, P, P, P, P, P, P, P, P, P,
                                         f64, f64, C.c_int32, P]
        lib.wo_select_commit.restype = i32
        _LIB = lib
    return _LIB


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return int(_lib().wo_num_threads())


def round_storage(x: float, dtype: str) -> float:
    return float(_lib().wo_round_storage(float(x), _DT[dtype]))


def reorder_perm(filled: np.ndarray) -> np.ndarray:
    """Physical row -> logical slot, per sequence.  filled: [B, W] or [W]."""
    f = _c(np.atleast_2d(filled), np.uint8)
    B, W = f.shape
    perm = np.empty((B, W), dtype=np.int32)
    for b in range(B):
        _lib().wo_reorder_perm(W, _p(f[b]), _p(perm[b]))
    return perm if np.ndim(filled) == 2 else perm[0]


def rope(x: np.ndarray, p: int, base: float) -> np.ndarray:
    x = _c(x, np.float64)
    y = np.empty_like(x)
    _lib().wo_rope(x.shape[-1], float(base), int(p), _p(x), _p(y))
    return y


def reorder(filled, pos, q, k, v, dtype: str, base: float):
    """q/k/v as float64 values [B, W, H, D] (logical order, before RoPE).
    Returns perm [B,W], q_phys [B,W,Hq,D], k_win/v_win [B,W,Hkv,D] (physical)."""
    q = _c(q, np.float64); k = _c(k, np.float64); v = _c(v, np.float64)
    filled = _c(filled, np.uint8); pos = _c(pos, np.int32)
    B, W, Hq, D = q.shape
    Hkv = k.shape[2]
    perm = np.empty((B, W), dtype=np.int32)
    qp = np.empty_like(q)
    kw = np.empty_like(k)
    vw = np.empty_like(v)
    rc = _lib().wo_reorder(B, W, Hq, Hkv, D, _DT[dtype], float(base), _p(filled), _p(pos),
                           _p(q), _p(k), _p(v), _p(perm), _p(qp), _p(kw), _p(vw))
    if rc != 0:
        raise ValueError("positions must be strictly increasing within each window")
    return perm, qp, kw, vw


def attention(q_phys, dense_k: Sequence[np.ndarray], dense_v: Sequence[np.ndarray],
              ctx_len, perm, scale: Optional[float] = None, rows=None):
    """Windowed causal GQA attention.  q_phys [B,W,Hq,D] float64 (physical
    order); dense_k/v[b] [L_b + W, Hkv, D] float64 (logical token order).
    rows: optional int array [n, 3] of (b, r, h); only those outputs are
    computed (others stay NaN).  Returns out [B, W, Hq, D] in logical slot
    order."""
    q_phys = _c(q_phys, np.float64)
    B, W, Hq, D = q_phys.shape
    Hkv = dense_k[0].shape[1]
    ctx_len = _c(ctx_len, np.int32)
    perm = _c(perm, np.int32)
    for b in range(B):
        assert dense_k[b].shape[0] == int(ctx_len[b]) + W, "dense cache must hold L_b + W tokens"
    K = _c(np.concatenate([np.asarray(x, np.float64) for x in dense_k], axis=0), np.float64)
    V = _c(np.concatenate([np.asarray(x, np.float64) for x in dense_v], axis=0), np.float64)
    off = np.zeros(B, dtype=np.int64)
    off[1:] = np.cumsum([x.shape[0] for x in dense_k])[:-1]
    out = np.full((B, W, Hq, D), np.nan, dtype=np.float64)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    if rows is None:
        n, rp = 0, None
    else:
        # each listed output row is computed once (a row listed twice would
        # have two threads accumulating into the same output)
        rows = _c(np.unique(np.asarray(rows, np.int32).reshape(-1, 3), axis=0), np.int32)
        n, rp = rows.shape[0], rows
    _lib().wo_attention(B, W, Hq, Hkv, D, float(scale), _p(q_phys), _p(K), _p(V), _p(off),
                        _p(ctx_len), _p(perm), n, _p(rp), _p(out))
    return out


def row_stats(z: np.ndarray):
    """(argmax, entropy in nats) of each row of z [..., V] (fp32 input)."""
    z = _c(z, np.float32)
    V = z.shape[-1]
    R = z.size // V
    am = np.empty(R, dtype=np.int32)
    H = np.empty(R, dtype=np.float64)
    _lib().wo_vocab_stats(R, V, _p(z), _p(am), _p(H))
    return am.reshape(z.shape[:-1]), H.reshape(z.shape[:-1])


def select_commit(logits: np.ndarray, tok, filled, pos, ctx_len, alpha: float, tau: float,
                  mask_id: int, row_index: Optional[np.ndarray] = None):
    """One commit / Eq. 11 select / refill step.  Window state arrays are
    copied; returns a dict with the new state and the step's outputs."""
    tok = np.array(tok, dtype=np.int32, copy=True)
    filled = np.array(filled, dtype=np.uint8, copy=True)
    pos = np.array(pos, dtype=np.int32, copy=True)
    ctx = np.array(ctx_len, dtype=np.int32, copy=True)
    B, W = tok.shape
    logits = _c(logits, np.float32)
    V = logits.shape[-1]
    ri = None if row_index is None else _c(row_index, np.int64)
    n_commit = np.empty(B, dtype=np.int32)
    committed = np.empty((B, W), dtype=np.int32)
    am = np.empty((B, W), dtype=np.int32)
    ent = np.empty((B, W), dtype=np.float32)
    margin = np.empty(B, dtype=np.float64)
    rc = _lib().wo_select_commit(B, W, V, _p(logits), _p(ri), _p(tok), _p(filled), _p(pos),
                                 _p(ctx), _p(n_commit), _p(committed), _p(am), _p(ent),
                                 float(alpha), float(tau), int(mask_id), _p(margin))
    if rc != 0:
        raise ValueError("a masked slot's logits row was not supplied")
    return dict(tok=tok, filled=filled, pos=pos, ctx_len=ctx, n_commit=n_commit,
                committed=committed, argmax=am, entropy=ent, margin=margin)


def prefix_cacheability(n_commit_steps, W: int):
    """Prefix cacheability of a stream (paper-summary page, "Key claims",
    sec. 3.1, Eq. 4: P_c = N_new / N_total, committed tokens over all token
    positions the decoder ran through; only the former join the cached
    prefix whose K/V later steps reuse).  Reading:
    every step processes the W window slots of each sequence (N_total += W)
    and commits its leading filled run (N_new += n_commit).
    n_commit_steps: [steps][B] commit counts.  Returns (N_new [B], N_total
    [B], P_c [B]) with the counts as int64."""
    n = np.asarray(n_commit_steps, dtype=np.int64)
    if n.ndim == 1:
        n = n[None]
    n_new = n.sum(axis=0)
    n_total = np.full(n.shape[1], n.shape[0] * int(W), dtype=np.int64)
    return n_new, n_total, n_new / np.maximum(n_total, 1)


def lmhead_logits(hidden: np.ndarray, lm_head: np.ndarray) -> np.ndarray:
    """Logits of the LM head: z[..., v] = sum_k hidden[..., k] * lm_head[v, k]
    in float64 (numpy's matmul as the contraction).  The inputs are the
    stored values (bf16 read as float64).

    The LM head is the backbone's output projection: it maps a slot's final
    hidden state to the vocabulary logits whose softmax the select step
    scores (WeDLM paper-summary page, "Method", inference paragraph: masked
    slots are predicted from the model's output distribution; the backbone
    is Qwen3-8B, TL;DR)."""
    h = np.asarray(hidden, dtype=np.float64)
    w = np.asarray(lm_head, dtype=np.float64)
    if h.shape[-1] != w.shape[1]:
        raise ValueError("hidden size mismatch")
    return h @ w.T


def lmhead_select_commit(hidden: np.ndarray, lm_head: np.ndarray, tok, filled, pos, ctx_len,
                         alpha: float, tau: float, mask_id: int):
    """select_commit on the LM head's logits.  The fused kernel never stores
    logits; its fp32 accumulators are taken here as the float64 logits
    rounded to fp32 (the storage point of a logit)."""
    z = lmhead_logits(hidden, lm_head).astype(np.float32)
    out = select_commit(z, tok, filled, pos, ctx_len, alpha, tau, mask_id)
    out["logits"] = z
    return out


def dual_stream_visible(flags: np.ndarray, block: int) -> np.ndarray:
    """Visibility of the Dual-Stream Masking attention for one sequence of N
    tokens, as a [2N, 2N] boolean matrix over [memory stream ++ prediction
    stream] in logical order (query row, key column).

    WeDLM paper-summary page, "Method" (training paragraph) and "Key claims"
    (sec. 4.2, Eq. 8-10): a clean memory stream and a block-masked prediction
    stream share position ids; prediction tokens of block i attend to the
    memory tokens whose logical positions precede block i.  Readings where
    the page is silent: the memory stream is plainly causal; inside its own
    block a prediction token follows Topological Reordering under the causal
    mask (sec. 3.2, 4.1), i.e. token t sees token s of its block iff
    (s observed and (t masked or s <= t)) or (both masked and s <= t); the
    prediction stream sees no prediction token of another block."""
    f = np.asarray(flags, dtype=bool)
    N = f.shape[0]
    t = np.arange(N)
    vis = np.zeros((2 * N, 2 * N), dtype=bool)
    vis[:N, :N] = t[None, :] <= t[:, None]                        # memory: causal
    blk = t // block
    vis[N:, :N] = t[None, :] < (blk * block)[:, None]            # earlier blocks' clean tokens
    same = blk[:, None] == blk[None, :]
    le = t[None, :] <= t[:, None]
    fs, ft = f[None, :], f[:, None]
    vis[N:, N:] = same & ((fs & (~ft | le)) | (~ft & ~fs & le))
    return vis


def dual_stream_attention(qm, km, vm, qp, kp, vp, flags, block: int, dtype: str, base: float,
                          scale: Optional[float] = None, rows=None):
    """Dual-Stream Masking attention of S sequences (the training-time mask
    as a forward pass).  q*/k*/v* [S, N, H, D] float64 values before RoPE,
    memory (m) and prediction (p) streams in logical order; flags [S, N]
    (1 = observed) of the prediction stream.  Both streams take RoPE at the
    shared logical positions 0..N-1; rotated q and k are rounded to the
    storage dtype, as a decode step stores them.  GQA: query head h reads KV
    head h // (Hq / Hkv).  rows: optional [n, 3] of (sequence, stream 0/1,
    token) to compute (others NaN).  Returns (out_mem, out_pred), each
    [S, N, Hq, D]."""
    qm, km, vm, qp, kp, vp = [np.asarray(x, np.float64) for x in (qm, km, vm, qp, kp, vp)]
    S, N, Hq, D = qm.shape
    Hkv = km.shape[2]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    ones = np.ones((S, N), np.uint8)
    pos = np.tile(np.arange(N, dtype=np.int32), (S, 1))
    _, qmr, kmr, _ = reorder(ones, pos, qm, km, vm, dtype, base)     # RoPE + storage rounding
    _, qpr, kpr, _ = reorder(ones, pos, qp, kp, vp, dtype, base)
    out = np.full((2, S, N, Hq, D), np.nan)
    if rows is None:
        todo = [(s, st, t) for s in range(S) for st in range(2) for t in range(N)]
    else:
        todo = [tuple(int(x) for x in r) for r in np.asarray(rows).reshape(-1, 3)]
    vis_cache = {}
    for s, st, t in todo:
        if s not in vis_cache:
            vis_cache[s] = dual_stream_visible(np.asarray(flags)[s], block)
        vis = vis_cache[s][st * N + t]
        K = np.concatenate([kmr[s], kpr[s]], axis=0)[vis]             # [nk, Hkv, D]
        Vv = np.concatenate([vm[s], vp[s]], axis=0)[vis]
        q = (qmr if st == 0 else qpr)[s, t]                           # [Hq, D]
        for h in range(Hq):
            sc = K[:, h // G, :] @ q[h] * scale
            w = np.exp(sc - sc.max())
            out[st, s, t, h] = (w / w.sum()) @ Vv[:, h // G, :]
    return out[0], out[1]


def _round_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> fp32 -> bf16 (round to nearest even) -> float64: the value
    a GPU kernel stores after accumulating in fp32."""
    f = np.ascontiguousarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = (((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16).astype(np.uint32)
    return r.view(np.float32).astype(np.float64)


def rms_norm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * g over the last axis, float64."""
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(g, np.float64)


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def model_step(w: dict, caches, tok, filled, pos, ctx_len, alpha: float, tau: float, base: float, eps: float,
               Hq: int, Hkv: int, storage: str = "bf16"):
    """One decode step of the synthetic decoder (float64; values stored by
    the GPU in bf16 are rounded the same way when storage == "bf16").

    The layer is the plain pre-norm decoder block (the pages name a
    Qwen3-8B backbone, TL;DR, but not its layer; this is the reading):
      x = E[tok];  per layer: h = RMSNorm(x) g_attn;  q, k, v = h W^T;
      o = decode-step attention of the reordered window over the layer's
      cache (reorder() + attention());  x += o Wo^T;  h = RMSNorm(x) g_mlp;
      x += (silu(h Wg^T) * (h Wu^T)) Wd^T;  then RMSNorm(x) g_final, the LM
      head and the select step (lmhead_select_commit()).
    w: float64 weights (embed [V+1, d], final_norm, lm_head [V, d], layers
    list of dicts).  caches[l] = (K list, V list) of per-sequence arrays
    [>= ctx_len[b], Hkv, D] (rotated keys, logical order).  Returns the
    select result plus "hidden" [B, W, d] and "caches" with the window's K/V
    appended after ctx_len[b] in physical order."""
    rnd = _round_bf16 if storage == "bf16" else (lambda a: np.asarray(a, np.float64))
    dt = "bf16" if storage == "bf16" else "f64"
    tok = np.asarray(tok)
    B, W = tok.shape
    layers = w["layers"]
    D = layers[0]["wq"].shape[0] // Hq
    ctx = np.asarray(ctx_len, np.int32)
    x = np.asarray(w["embed"], np.float64)[tok]
    h = rnd(rms_norm(x, layers[0]["attn_norm"], eps))
    new_caches = []
    for l, lw in enumerate(layers):
        q = rnd(h @ lw["wq"].T).reshape(B, W, Hq, D)
        k = rnd(h @ lw["wk"].T).reshape(B, W, Hkv, D)
        v = rnd(h @ lw["wv"].T).reshape(B, W, Hkv, D)
        perm, qp, kw, vw = reorder(filled, pos, q, k, v, dt, base)
        dk = [np.concatenate([caches[l][0][b][:ctx[b]], kw[b]], axis=0) for b in range(B)]
        dv = [np.concatenate([caches[l][1][b][:ctx[b]], vw[b]], axis=0) for b in range(B)]
        o = rnd(attention(qp, dk, dv, ctx, perm)).reshape(B, W, Hq * D)
        x = x + o @ lw["wo"].T
        h = rnd(rms_norm(x, lw["mlp_norm"], eps))
        act = rnd(silu(h @ lw["w_gate"].T) * (h @ lw["w_up"].T))
        x = x + act @ lw["w_down"].T
        nxt = layers[l + 1]["attn_norm"] if l + 1 < len(layers) else w["final_norm"]
        h = rnd(rms_norm(x, nxt, eps))
        new_caches.append((dk, dv))
    V = w["lm_head"].shape[0]
    out = lmhead_select_commit(h, w["lm_head"], tok, filled, pos, ctx, alpha, tau, V)
    out["hidden"] = h
    out["caches"] = new_caches
    return out


def decode_step_attention(inp, scale: Optional[float] = None, rows=None):
    """Oracle for reorder + attention on one batch drawn by
    workloads.make_attn_inputs.  Returns a dict
    with perm, q_phys, k_win, v_win (physical order, storage-rounded) and out
    (logical slot order)."""
    from workloads import storage_to_f64
    cfg = inp.cfg
    dt = cfg.dtype
    perm, qp, kw, vw = reorder(inp.filled, inp.pos, storage_to_f64(inp.q, dt),
                               storage_to_f64(inp.k, dt), storage_to_f64(inp.v, dt),
                               dt, cfg.rope_base)
    dk = [np.concatenate([storage_to_f64(inp.prefix_k[b], dt), kw[b]], axis=0) for b in range(cfg.B)]
    dv = [np.concatenate([storage_to_f64(inp.prefix_v[b], dt), vw[b]], axis=0) for b in range(cfg.B)]
    out = attention(qp, dk, dv, inp.ctx_len, perm, scale=scale, rows=rows)
    return dict(perm=perm, q_phys=qp, k_win=kw, v_win=vw, out=out)
