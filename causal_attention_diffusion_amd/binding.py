"""ctypes binding of libwedlm.so: argument marshalling only.

Shapes are read off the torch tensors, pointers and the current HIP stream
are passed to the C entry points of ``include/wedlm.h``.  A non-OK status
raises WedlmError with the library's message.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libwedlm.so")
_LIB = None

WEDLM_F32, WEDLM_BF16 = 0, 1
PAGE = 16


class WedlmError(RuntimeError):
    pass


class WedlmShape(C.Structure):
    _fields_ = [("B", C.c_int32), ("W", C.c_int32), ("Hq", C.c_int32), ("Hkv", C.c_int32),
                ("D", C.c_int32), ("page_size", C.c_int32), ("max_pages", C.c_int32),
                ("num_pages", C.c_int32), ("dtype", C.c_int32)]


LAYER_FIELDS = ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down", "k_cache", "v_cache")


class WedlmStepIO(C.Structure):
    """wedlm_step_io: the pointers and scalars of one wedlm_decode_step."""
    _fields_ = [(n, C.c_void_p) for n in ("tok", "filled", "pos", "ctx_len", "q", "k", "v", "logits",
                                          "k_cache", "v_cache", "block_table", "q_phys", "perm", "out",
                                          "n_commit", "committed", "argmax_out", "entropy_out", "counters",
                                          "dev_status")] + \
               [("V", C.c_int32), ("max_ctx_len", C.c_int32), ("mask_id", C.c_int32), ("scale", C.c_float),
                ("alpha", C.c_float), ("tau", C.c_float), ("rope_base", C.c_double)]


class WedlmLayerWeights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in LAYER_FIELDS]


class WedlmModel(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("d_model", C.c_int32), ("d_ff", C.c_int32), ("vocab", C.c_int32),
                ("rms_eps", C.c_float), ("embed", C.c_void_p), ("final_norm", C.c_void_p),
                ("lm_head", C.c_void_p), ("layers", C.POINTER(WedlmLayerWeights))]


def lib_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libwedlm.so (raises if it has not been built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(_LIB_PATH):
        raise WedlmError(f"{_LIB_PATH} is not built; run `python -m causal_attention_diffusion_amd.build` "
                         "(there is no fallback path)")
    lib = C.CDLL(_LIB_PATH)
    P, i32, sz = C.c_void_p, C.c_int32, C.c_size_t
    S = C.POINTER(WedlmShape)
    lib.wedlm_reorder.argtypes = [S, P, P, P, P, P, P, P, P, P, P, P, C.c_double, P, P]
    lib.wedlm_reorder.restype = C.c_int
    lib.wedlm_step_attn_workspace.argtypes = [S, i32]
    lib.wedlm_step_attn_workspace.restype = sz
    lib.wedlm_step_attn.argtypes = [S, P, P, P, P, P, P, P, C.c_float, i32, P, sz, P, P]
    lib.wedlm_step_attn.restype = C.c_int
    lib.wedlm_step_attn_noalloc.argtypes = [S, P, P, P, P, P, P, P, C.c_float, i32, P, P]
    lib.wedlm_step_attn_noalloc.restype = C.c_int
    lib.wedlm_step_attn_noalloc_limit.argtypes = []
    lib.wedlm_step_attn_noalloc_limit.restype = sz
    lib.wedlm_select_commit_workspace.argtypes = [i32, i32, i32]
    lib.wedlm_select_commit_workspace.restype = sz
    lib.wedlm_select_commit.argtypes = [i32, i32, i32, P, P, P, P, P, P, P, P, P, P,
                                        C.c_float, C.c_float, i32, P, sz, P]
    lib.wedlm_select_commit.restype = C.c_int
    lib.wedlm_decode_step_workspace.argtypes = [S, i32, i32]
    lib.wedlm_decode_step_workspace.restype = sz
    lib.wedlm_decode_step.argtypes = [S, C.POINTER(WedlmStepIO), P, sz, P]
    lib.wedlm_decode_step.restype = C.c_int
    lib.wedlm_lmhead_select_commit_workspace.argtypes = [i32, i32, i32, i32]
    lib.wedlm_lmhead_select_commit_workspace.restype = sz
    lib.wedlm_lmhead_select_commit.argtypes = [i32, i32, i32, i32, P, P, P, P, P, P, P, P, P, P, P,
                                               C.c_float, C.c_float, i32, P, sz, P]
    lib.wedlm_lmhead_select_commit.restype = C.c_int
    lib.wedlm_dual_stream_attn_workspace.argtypes = [S, i32]
    lib.wedlm_dual_stream_attn_workspace.restype = sz
    lib.wedlm_dual_stream_attn.argtypes = [S, i32, P, P, P, P, P, P, P, P, P, C.c_double, P, sz, P, P]
    lib.wedlm_dual_stream_attn.restype = C.c_int
    Mp = C.POINTER(WedlmModel)
    lib.wedlm_model_step_workspace.argtypes = [Mp, S, i32]
    lib.wedlm_model_step_workspace.restype = sz
    lib.wedlm_model_step.argtypes = [Mp, S, P, P, P, P, P, P, P, P, P, P, P, C.c_float, C.c_float, C.c_double,
                                     i32, P, sz, P, P]
    lib.wedlm_model_step.restype = C.c_int
    lib.wedlm_attn_plan.argtypes = [S, i32, C.POINTER(i32), C.POINTER(i32)]
    lib.wedlm_attn_plan.restype = C.c_int
    lib.wedlm_set_attn_split_keys.argtypes = [i32]
    lib.wedlm_set_attn_split_keys.restype = C.c_int
    lib.wedlm_decode_step_timed.argtypes = [S, C.POINTER(WedlmStepIO), P, sz, P, P, P]
    lib.wedlm_decode_step_timed.restype = C.c_int
    lib.wedlm_attn_tail.argtypes = [S, i32]
    lib.wedlm_attn_tail.restype = i32
    lib.wedlm_set_attn_tail.argtypes = [i32]
    lib.wedlm_set_attn_tail.restype = C.c_int
    lib.wedlm_set_select_parts.argtypes = [i32]
    lib.wedlm_set_select_parts.restype = C.c_int
    lib.wedlm_graph_begin.argtypes = [P]
    lib.wedlm_graph_begin.restype = C.c_int
    lib.wedlm_graph_end.argtypes = [P, C.POINTER(C.c_void_p)]
    lib.wedlm_graph_end.restype = C.c_int
    lib.wedlm_graph_launch.argtypes = [P, P]
    lib.wedlm_graph_launch.restype = C.c_int
    lib.wedlm_graph_nodes.argtypes = [P, C.POINTER(sz), C.POINTER(sz)]
    lib.wedlm_graph_nodes.restype = C.c_int
    lib.wedlm_graph_destroy.argtypes = [P]
    lib.wedlm_graph_destroy.restype = None
    lib.wedlm_last_error.restype = C.c_char_p
    lib.wedlm_version.restype = C.c_char_p
    _LIB = lib
    return lib


def _check(rc: int):
    if rc != 0:
        raise WedlmError(f"status {rc}: {load_library().wedlm_last_error().decode()}")


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise WedlmError("tensors must be contiguous")
    if t.device.type != "cuda":
        raise WedlmError("tensors must be on the GPU")
    return t.data_ptr()


def _stream(stream) -> int:
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return WEDLM_F32
    if t.dtype == torch.bfloat16:
        return WEDLM_BF16
    raise WedlmError(f"dtype {t.dtype} not supported (float32, bfloat16)")


def make_shape(B, W, Hq, Hkv, D, max_pages, num_pages, dtype) -> WedlmShape:
    return WedlmShape(B, W, Hq, Hkv, D, PAGE, max_pages, num_pages, dtype)


def _shape_from(q, k_cache, block_table) -> WedlmShape:
    if q.dim() != 4 or k_cache.dim() != 4 or block_table.dim() != 2:
        raise WedlmError("expected q [B,W,Hq,D], cache [pages,Hkv,16,D], block_table [B,max_pages]")
    B, W, Hq, D = q.shape
    P, Hkv, page, D2 = k_cache.shape
    if page != PAGE or D2 != D:
        raise WedlmError(f"cache must be [pages, Hkv, {PAGE}, {D}], got {tuple(k_cache.shape)}")
    if block_table.shape[0] != B:
        raise WedlmError("block_table must be [B, max_pages]")
    return make_shape(B, W, Hq, Hkv, D, block_table.shape[1], P, _dtype_code(q))


def _expect(t, name, shape, dtype):
    """Shape/dtype check of one argument before its pointer reaches a kernel."""
    if t is None:
        raise WedlmError(f"{name} is required")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise WedlmError(f"{name}: expected {tuple(shape)} {dtype}, got {tuple(t.shape)} {t.dtype}")


def _opt(t, name, shape, dtype):
    if t is not None:
        _expect(t, name, shape, dtype)


# ---------------------------------------------------------------- entry points
def wedlm_reorder(filled, pos, q, k, v, q_phys, k_cache, v_cache, block_table, ctx_len, perm,
                  rope_base: float, dev_status=None, stream=None):
    import torch
    s = _shape_from(q, k_cache, block_table)
    B, W, Hkv, D = s.B, s.W, s.Hkv, s.D
    _expect(filled, "filled", (B, W), torch.uint8)
    _expect(pos, "pos", (B, W), torch.int32)
    _expect(k, "k", (B, W, Hkv, D), q.dtype)
    _expect(v, "v", (B, W, Hkv, D), q.dtype)
    _expect(q_phys, "q_phys", tuple(q.shape), q.dtype)
    _expect(v_cache, "v_cache", tuple(k_cache.shape), q.dtype)
    _expect(k_cache, "k_cache", tuple(k_cache.shape), q.dtype)
    _expect(block_table, "block_table", tuple(block_table.shape), torch.int32)
    _expect(ctx_len, "ctx_len", (B,), torch.int32)
    _expect(perm, "perm", (B, W), torch.int32)
    _opt(dev_status, "dev_status", (1,), torch.int32)
    _check(load_library().wedlm_reorder(
        C.byref(s), _ptr(filled), _ptr(pos), _ptr(q), _ptr(k), _ptr(v), _ptr(q_phys), _ptr(k_cache),
        _ptr(v_cache), _ptr(block_table), _ptr(ctx_len), _ptr(perm), float(rope_base),
        _ptr(dev_status), _stream(stream)))


def wedlm_step_attn_workspace(q_phys, k_cache, block_table, max_ctx_len: int) -> int:
    s = _shape_from(q_phys, k_cache, block_table)
    return int(load_library().wedlm_step_attn_workspace(C.byref(s), int(max_ctx_len)))


def attn_workspace_tensor(q_phys, k_cache, block_table, max_ctx_len: int):
    import torch
    n = wedlm_step_attn_workspace(q_phys, k_cache, block_table, max_ctx_len)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=q_phys.device)


def wedlm_step_attn(q_phys, k_cache, v_cache, block_table, ctx_len, perm, out, max_ctx_len: int,
                    workspace=None, scale: float = 0.0, dev_status=None, stream=None):
    import torch
    s = _shape_from(q_phys, k_cache, block_table)
    _expect(k_cache, "k_cache", tuple(k_cache.shape), q_phys.dtype)
    _expect(v_cache, "v_cache", tuple(k_cache.shape), q_phys.dtype)
    _expect(block_table, "block_table", tuple(block_table.shape), torch.int32)
    _expect(ctx_len, "ctx_len", (s.B,), torch.int32)
    _expect(perm, "perm", (s.B, s.W), torch.int32)
    _expect(out, "out", tuple(q_phys.shape), q_phys.dtype)
    _opt(dev_status, "dev_status", (1,), torch.int32)
    if workspace is not None and workspace.dtype != torch.uint8:
        raise WedlmError("workspace must be a uint8 tensor")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load_library().wedlm_step_attn(
        C.byref(s), _ptr(q_phys), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(ctx_len),
        _ptr(perm), _ptr(out), float(scale), int(max_ctx_len), _ptr(workspace), ws_bytes,
        _ptr(dev_status), _stream(stream)))


def wedlm_step_attn_noalloc(q_phys, k_cache, v_cache, block_table, ctx_len, perm, out, max_ctx_len: int,
                            scale: float = 0.0, dev_status=None, stream=None):
    """wedlm_step_attn with the split partials in the library's own device
    array (no workspace argument; calls on one GPU must not overlap)."""
    import torch
    s = _shape_from(q_phys, k_cache, block_table)
    _expect(k_cache, "k_cache", tuple(k_cache.shape), q_phys.dtype)
    _expect(v_cache, "v_cache", tuple(k_cache.shape), q_phys.dtype)
    _expect(block_table, "block_table", tuple(block_table.shape), torch.int32)
    _expect(ctx_len, "ctx_len", (s.B,), torch.int32)
    _expect(perm, "perm", (s.B, s.W), torch.int32)
    _expect(out, "out", tuple(q_phys.shape), q_phys.dtype)
    _opt(dev_status, "dev_status", (1,), torch.int32)
    _check(load_library().wedlm_step_attn_noalloc(
        C.byref(s), _ptr(q_phys), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(ctx_len),
        _ptr(perm), _ptr(out), float(scale), int(max_ctx_len), _ptr(dev_status), _stream(stream)))


def wedlm_step_attn_noalloc_limit() -> int:
    return int(load_library().wedlm_step_attn_noalloc_limit())


def wedlm_attn_plan(q_phys, k_cache, block_table, max_ctx_len: int):
    s = _shape_from(q_phys, k_cache, block_table)
    ns, sk = C.c_int32(), C.c_int32()
    _check(load_library().wedlm_attn_plan(C.byref(s), int(max_ctx_len), C.byref(ns), C.byref(sk)))
    return ns.value, sk.value


def attn_plan(B, W, Hq, Hkv, D, max_pages, num_pages, dtype, max_ctx_len):
    s = make_shape(B, W, Hq, Hkv, D, max_pages, num_pages, dtype)
    ns, sk = C.c_int32(), C.c_int32()
    _check(load_library().wedlm_attn_plan(C.byref(s), int(max_ctx_len), C.byref(ns), C.byref(sk)))
    return ns.value, sk.value


def wedlm_set_attn_split_keys(keys: int):
    _check(load_library().wedlm_set_attn_split_keys(int(keys)))


def wedlm_attn_tail(q_phys, k_cache, block_table, max_ctx_len: int) -> int:
    """Sequences the attention plan cuts in two (tail splits), 0 if none."""
    s = _shape_from(q_phys, k_cache, block_table)
    n = int(load_library().wedlm_attn_tail(C.byref(s), int(max_ctx_len)))
    if n < 0:
        raise WedlmError("wedlm_attn_tail: bad shape or bound")
    return n


def attn_tail(B, W, Hq, Hkv, D, max_pages, num_pages, dtype, max_ctx_len) -> int:
    s = make_shape(B, W, Hq, Hkv, D, max_pages, num_pages, dtype)
    return int(load_library().wedlm_attn_tail(C.byref(s), int(max_ctx_len)))


def wedlm_set_attn_tail(n: int):
    _check(load_library().wedlm_set_attn_tail(int(n)))


def wedlm_set_select_parts(parts: int):
    _check(load_library().wedlm_set_select_parts(int(parts)))


def wedlm_select_commit_workspace(B: int, W: int, V: int) -> int:
    return int(load_library().wedlm_select_commit_workspace(int(B), int(W), int(V)))


def select_workspace_tensor(B: int, W: int, V: int, device):
    """Workspace for wedlm_select_commit (no initialisation needed)."""
    import torch
    return torch.empty(max(wedlm_select_commit_workspace(B, W, V), 1), dtype=torch.uint8, device=device)


def wedlm_select_commit(logits, tok, filled, pos, ctx_len, n_commit, committed, alpha: float,
                        tau: float, mask_id: int, workspace, argmax_out=None, entropy_out=None,
                        counters=None, stream=None):
    """counters: optional [B, 2] int64 tensor accumulating (N_new, N_total):
    committed tokens and processed window slots per sequence."""
    import torch
    if logits.dim() != 3 or logits.dtype != torch.float32:
        raise WedlmError("logits must be a [B, W, V] float32 tensor")
    B, W, V = logits.shape
    _expect(tok, "tok", (B, W), torch.int32)
    _expect(filled, "filled", (B, W), torch.uint8)
    _expect(pos, "pos", (B, W), torch.int32)
    _expect(ctx_len, "ctx_len", (B,), torch.int32)
    _expect(n_commit, "n_commit", (B,), torch.int32)
    _expect(committed, "committed", (B, W), torch.int32)
    _opt(argmax_out, "argmax_out", (B, W), torch.int32)
    _opt(entropy_out, "entropy_out", (B, W), torch.float32)
    _opt(counters, "counters", (B, 2), torch.int64)
    if workspace is None or workspace.dtype != torch.uint8:
        raise WedlmError("workspace must be a uint8 tensor (select_workspace_tensor)")
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load_library().wedlm_select_commit(
        B, W, V, _ptr(logits), _ptr(tok), _ptr(filled), _ptr(pos), _ptr(ctx_len), _ptr(n_commit),
        _ptr(committed), _ptr(argmax_out), _ptr(entropy_out), _ptr(counters), float(alpha), float(tau),
        int(mask_id), _ptr(workspace), ws_bytes, _stream(stream)))


def wedlm_decode_step_workspace(q, k_cache, block_table, max_ctx_len: int, V: int) -> int:
    s = _shape_from(q, k_cache, block_table)
    return int(load_library().wedlm_decode_step_workspace(C.byref(s), int(max_ctx_len), int(V)))


def decode_step_workspace_tensor(q, k_cache, block_table, max_ctx_len: int, V: int):
    """Workspace for wedlm_decode_step (no initialisation needed)."""
    import torch
    n = wedlm_decode_step_workspace(q, k_cache, block_table, max_ctx_len, V)
    if n == 0:
        raise WedlmError(f"unsupported decode-step shape (max_ctx_len={max_ctx_len}, V={V})")
    return torch.empty(n, dtype=torch.uint8, device=q.device)


def wedlm_decode_step(filled, pos, q, k, v, q_phys, k_cache, v_cache, block_table, ctx_len, perm, out,
                      rope_base: float, max_ctx_len: int, logits, tok, n_commit, committed, alpha: float,
                      tau: float, mask_id: int, workspace, scale: float = 0.0, argmax_out=None,
                      entropy_out=None, counters=None, dev_status=None, stream=None, attn_events=None):
    """One whole decode step: the arguments of wedlm_reorder, wedlm_step_attn and
    wedlm_select_commit (same names), run as one call with fewer launches.
    attn_events: optional (start, stop) torch.cuda.Event pair (timing enabled,
    already recorded once so that they exist) that the attention kernel's
    dispatch sets (wedlm_decode_step_timed)."""
    import torch
    s = _shape_from(q, k_cache, block_table)
    B, W, Hq, Hkv, D = s.B, s.W, s.Hq, s.Hkv, s.D
    _expect(filled, "filled", (B, W), torch.uint8)
    _expect(pos, "pos", (B, W), torch.int32)
    _expect(k, "k", (B, W, Hkv, D), q.dtype)
    _expect(v, "v", (B, W, Hkv, D), q.dtype)
    _expect(q_phys, "q_phys", tuple(q.shape), q.dtype)
    _expect(k_cache, "k_cache", tuple(k_cache.shape), q.dtype)
    _expect(v_cache, "v_cache", tuple(k_cache.shape), q.dtype)
    _expect(block_table, "block_table", tuple(block_table.shape), torch.int32)
    _expect(ctx_len, "ctx_len", (B,), torch.int32)
    _expect(perm, "perm", (B, W), torch.int32)
    _expect(out, "out", (B, W, Hq, D), q.dtype)
    if logits is None or logits.dim() != 3 or logits.dtype != torch.float32 or tuple(logits.shape[:2]) != (B, W):
        raise WedlmError(f"logits must be a [{B}, {W}, V] float32 tensor")
    V = logits.shape[2]
    _expect(tok, "tok", (B, W), torch.int32)
    _expect(n_commit, "n_commit", (B,), torch.int32)
    _expect(committed, "committed", (B, W), torch.int32)
    _opt(argmax_out, "argmax_out", (B, W), torch.int32)
    _opt(entropy_out, "entropy_out", (B, W), torch.float32)
    _opt(counters, "counters", (B, 2), torch.int64)
    _opt(dev_status, "dev_status", (1,), torch.int32)
    if workspace is None or workspace.dtype != torch.uint8:
        raise WedlmError("workspace must be a uint8 tensor (decode_step_workspace_tensor)")
    io = WedlmStepIO(_ptr(tok), _ptr(filled), _ptr(pos), _ptr(ctx_len), _ptr(q), _ptr(k), _ptr(v), _ptr(logits),
                     _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(q_phys), _ptr(perm), _ptr(out),
                     _ptr(n_commit), _ptr(committed), _ptr(argmax_out), _ptr(entropy_out), _ptr(counters),
                     _ptr(dev_status), int(V), int(max_ctx_len), int(mask_id), float(scale), float(alpha),
                     float(tau), float(rope_base))
    nbytes = workspace.numel() * workspace.element_size()
    if attn_events is None:
        _check(load_library().wedlm_decode_step(C.byref(s), C.byref(io), _ptr(workspace), nbytes, _stream(stream)))
    else:
        e0, e1 = attn_events
        h0, h1 = int(e0.cuda_event), int(e1.cuda_event)
        if not h0 or not h1:
            raise WedlmError("attn_events must be recorded once before use (the handles are created lazily)")
        _check(load_library().wedlm_decode_step_timed(C.byref(s), C.byref(io), _ptr(workspace), nbytes,
                                                      _stream(stream), C.c_void_p(h0), C.c_void_p(h1)))


def wedlm_lmhead_select_commit_workspace(B: int, W: int, V: int, Dm: int) -> int:
    return int(load_library().wedlm_lmhead_select_commit_workspace(int(B), int(W), int(V), int(Dm)))


def lmhead_workspace_tensor(B: int, W: int, V: int, Dm: int, device):
    """Workspace for wedlm_lmhead_select_commit (no initialisation needed)."""
    import torch
    n = wedlm_lmhead_select_commit_workspace(B, W, V, Dm)
    if n == 0:
        raise WedlmError(f"unsupported LM-head shape B={B} W={W} V={V} Dm={Dm}")
    return torch.empty(n, dtype=torch.uint8, device=device)


def wedlm_lmhead_select_commit(hidden, lm_head, tok, filled, pos, ctx_len, n_commit, committed,
                               alpha: float, tau: float, mask_id: int, workspace, argmax_out=None,
                               entropy_out=None, counters=None, stream=None):
    """hidden [B, W, Dm] and lm_head [V, Dm] bfloat16 tensors; window state
    and outputs as for wedlm_select_commit."""
    import torch
    if hidden.dim() != 3 or hidden.dtype != torch.bfloat16 or not hidden.is_contiguous():
        raise WedlmError("hidden must be a contiguous [B, W, Dm] bfloat16 tensor")
    B, W, Dm = hidden.shape
    if lm_head.dim() != 2 or lm_head.dtype != torch.bfloat16 or lm_head.shape[1] != Dm \
            or not lm_head.is_contiguous():
        raise WedlmError("lm_head must be a contiguous [V, Dm] bfloat16 tensor")
    V = lm_head.shape[0]
    _expect(tok, "tok", (B, W), torch.int32)
    _expect(filled, "filled", (B, W), torch.uint8)
    _expect(pos, "pos", (B, W), torch.int32)
    _expect(ctx_len, "ctx_len", (B,), torch.int32)
    _expect(n_commit, "n_commit", (B,), torch.int32)
    _expect(committed, "committed", (B, W), torch.int32)
    _opt(argmax_out, "argmax_out", (B, W), torch.int32)
    _opt(entropy_out, "entropy_out", (B, W), torch.float32)
    _opt(counters, "counters", (B, 2), torch.int64)
    if workspace is None or workspace.dtype != torch.uint8:
        raise WedlmError("workspace must be a uint8 tensor (lmhead_workspace_tensor)")
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load_library().wedlm_lmhead_select_commit(
        B, W, V, Dm, _ptr(hidden), _ptr(lm_head), _ptr(tok), _ptr(filled), _ptr(pos), _ptr(ctx_len),
        _ptr(n_commit), _ptr(committed), _ptr(argmax_out), _ptr(entropy_out), _ptr(counters), float(alpha),
        float(tau), int(mask_id), _ptr(workspace), ws_bytes, _stream(stream)))


def _dual_shape(qm, km, block):
    import torch
    if qm.dim() != 4 or km.dim() != 4:
        raise WedlmError("streams must be [B, N, H, D] tensors")
    B, N, Hq, D = qm.shape
    Hkv = km.shape[2]
    dt = WEDLM_BF16 if qm.dtype == torch.bfloat16 else WEDLM_F32
    return make_shape(B, block, Hq, Hkv, D, 1, 1, dt), N


def dual_stream_workspace_tensor(qm, km, block: int):
    """Workspace for wedlm_dual_stream_attn (no initialisation needed)."""
    import torch
    shp, N = _dual_shape(qm, km, block)
    n = int(load_library().wedlm_dual_stream_attn_workspace(C.byref(shp), int(N)))
    if n == 0:
        raise WedlmError(wedlm_last_error() or "unsupported dual-stream shape")
    return torch.empty(n, dtype=torch.uint8, device=qm.device)


def wedlm_dual_stream_attn(qm, km, vm, qp, kp, vp, flags, out_m, out_p, block: int, rope_base: float,
                           workspace, dev_status=None, stream=None):
    """Memory stream qm/km/vm and prediction stream qp/kp/vp [B, N, H, D]
    (bfloat16 or float32), flags [B, N] uint8; outputs [B, N, Hq, D]."""
    import torch
    shp, N = _dual_shape(qm, km, block)
    B, _, Hq, D = qm.shape
    Hkv = km.shape[2]
    for t, name, h in ((qm, "qm", Hq), (qp, "qp", Hq), (km, "km", Hkv), (kp, "kp", Hkv), (vm, "vm", Hkv),
                       (vp, "vp", Hkv), (out_m, "out_m", Hq), (out_p, "out_p", Hq)):
        _expect(t, name, (B, N, h, D), qm.dtype)
    _expect(flags, "flags", (B, N), torch.uint8)
    _opt(dev_status, "dev_status", (1,), torch.int32)
    if workspace is None or workspace.dtype != torch.uint8:
        raise WedlmError("workspace must be a uint8 tensor (dual_stream_workspace_tensor)")
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load_library().wedlm_dual_stream_attn(
        C.byref(shp), int(N), _ptr(qm), _ptr(km), _ptr(vm), _ptr(qp), _ptr(kp), _ptr(vp), _ptr(flags),
        _ptr(out_m), _ptr(out_p), float(rope_base), _ptr(workspace), ws_bytes, _ptr(dev_status),
        _stream(stream)))


class ModelHandle:
    """The C description of a synthetic decoder whose weights and per-layer
    caches are torch tensors (kept alive here).  weights: dict with embed
    [vocab+1, d], final_norm [d], lm_head [vocab, d] and layers: list of
    dicts with the LAYER_FIELDS entries (bfloat16 tensors on the GPU)."""

    def __init__(self, weights, rms_eps: float = 1e-6):
        import torch
        self.weights = weights
        layers = weights["layers"]
        self.layer_array = (WedlmLayerWeights * len(layers))()
        for i, lw in enumerate(layers):
            for n in LAYER_FIELDS:
                t = lw[n]
                if t.dtype != torch.bfloat16 or not t.is_contiguous() or t.device.type != "cuda":
                    raise WedlmError(f"layer {i} {n}: expected a contiguous bfloat16 GPU tensor")
                setattr(self.layer_array[i], n, t.data_ptr())
        d = weights["final_norm"].shape[0]
        vocab = weights["lm_head"].shape[0]
        if tuple(weights["embed"].shape) != (vocab + 1, d):
            raise WedlmError("embed must be [vocab + 1, d_model]")
        self.model = WedlmModel(len(layers), d, layers[0]["w_gate"].shape[0], vocab, float(rms_eps),
                                _ptr(weights["embed"]), _ptr(weights["final_norm"]), _ptr(weights["lm_head"]),
                                C.cast(self.layer_array, C.POINTER(WedlmLayerWeights)))
        self.vocab = vocab
        self.d_model = d


def model_step_workspace_tensor(handle: ModelHandle, shape: WedlmShape, max_ctx_len: int, device):
    import torch
    n = int(load_library().wedlm_model_step_workspace(C.byref(handle.model), C.byref(shape), int(max_ctx_len)))
    if n == 0:
        raise WedlmError(wedlm_last_error() or "unsupported model shape")
    return torch.empty(n, dtype=torch.uint8, device=device)


def wedlm_model_step(handle: ModelHandle, shape: WedlmShape, block_table, tok, filled, pos, ctx_len, n_commit,
                     committed, alpha: float, tau: float, rope_base: float, max_ctx_len: int, workspace,
                     argmax_out=None, entropy_out=None, hidden_out=None, dev_status=None, counters=None,
                     stream=None):
    import torch
    B, W = shape.B, shape.W
    _expect(block_table, "block_table", (B, shape.max_pages), torch.int32)
    _expect(tok, "tok", (B, W), torch.int32)
    _expect(filled, "filled", (B, W), torch.uint8)
    _expect(pos, "pos", (B, W), torch.int32)
    _expect(ctx_len, "ctx_len", (B,), torch.int32)
    _expect(n_commit, "n_commit", (B,), torch.int32)
    _expect(committed, "committed", (B, W), torch.int32)
    _opt(argmax_out, "argmax_out", (B, W), torch.int32)
    _opt(entropy_out, "entropy_out", (B, W), torch.float32)
    _opt(hidden_out, "hidden_out", (B, W, handle.d_model), torch.bfloat16)
    _opt(counters, "counters", (B, 2), torch.int64)
    _opt(dev_status, "dev_status", (1,), torch.int32)
    if workspace is None or workspace.dtype != torch.uint8:
        raise WedlmError("workspace must be a uint8 tensor (model_step_workspace_tensor)")
    _check(load_library().wedlm_model_step(
        C.byref(handle.model), C.byref(shape), _ptr(block_table), _ptr(tok), _ptr(filled), _ptr(pos),
        _ptr(ctx_len), _ptr(n_commit), _ptr(committed), _ptr(argmax_out), _ptr(entropy_out), _ptr(counters),
        _ptr(hidden_out), float(alpha), float(tau), float(rope_base), int(max_ctx_len), _ptr(workspace),
        workspace.numel(), _ptr(dev_status), _stream(stream)))


def wedlm_last_error() -> str:
    return load_library().wedlm_last_error().decode()


def wedlm_version() -> str:
    return load_library().wedlm_version().decode()


class Graph:
    """A captured sequence of library calls (wedlm_graph_*), replayed with
    launch().  Made by capture(); destroyed with close() or when collected."""

    def __init__(self):
        self._h = C.c_void_p()

    def launch(self, stream=None):
        if not self._h:
            raise WedlmError("graph is empty or closed")
        _check(load_library().wedlm_graph_launch(self._h, _stream(stream)))

    def nodes(self):
        """(kernel nodes, other nodes) of the captured graph."""
        k, o = C.c_size_t(), C.c_size_t()
        _check(load_library().wedlm_graph_nodes(self._h, C.byref(k), C.byref(o)))
        return k.value, o.value

    def close(self):
        if self._h:
            load_library().wedlm_graph_destroy(self._h)
            self._h = C.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class capture:
    """Record the library calls made inside the block on `stream` (a
    torch.cuda.Stream other than the default one) into a Graph:

        with wd.capture(side_stream) as g:
            step(...)            # recorded, not run
        g.launch()               # replays every recorded call

    Inside the block `stream` is torch's current stream, so the calls need
    no stream argument.  Nothing that allocates may run inside the block."""

    def __init__(self, stream):
        import torch
        if stream is None or stream.cuda_stream == 0:
            raise WedlmError("capture needs a created stream, not the default stream")
        self.stream = stream
        self.graph = Graph()
        self._ctx = torch.cuda.stream(stream)

    def __enter__(self):
        _check(load_library().wedlm_graph_begin(self.stream.cuda_stream))
        self._ctx.__enter__()
        return self.graph

    def __exit__(self, exc_type, exc, tb):
        self._ctx.__exit__(exc_type, exc, tb)
        rc = load_library().wedlm_graph_end(self.stream.cuda_stream, C.byref(self.graph._h))
        if exc_type is None:
            _check(rc)
        return False
