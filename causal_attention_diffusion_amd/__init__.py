"""WeDLM streaming-decode step on MI355X (gfx950).

Python binding of ``libwedlm.so`` (see ``include/wedlm.h``).  The functions
carry the C names and only marshal torch tensors to device pointers; every
step of the decode path runs in the HIP kernels.  There is no CPU fallback:
if the library is not built, every call raises.

    import causal_attention_diffusion_amd as wd
    wd.wedlm_reorder(filled, pos, q, k, v, q_phys, k_cache, v_cache,
                     block_table, ctx_len, perm, rope_base)
    wd.wedlm_step_attn(q_phys, k_cache, v_cache, block_table, ctx_len, perm,
                       out, max_ctx_len=..., workspace=ws)
    wd.wedlm_select_commit(logits, tok, filled, pos, ctx_len, n_commit,
                           committed, alpha=..., tau=..., mask_id=..., workspace=ws2)

or the same three as one call with fewer launches, ``wd.wedlm_decode_step``.
"""
from .binding import (  # noqa: F401
    WEDLM_BF16,
    WEDLM_F32,
    Graph,
    capture,
    WedlmError,
    attn_plan,
    lib_path,
    ModelHandle,
    lmhead_workspace_tensor,
    model_step_workspace_tensor,
    load_library,
    make_shape,
    select_workspace_tensor,
    attn_workspace_tensor,
    decode_step_workspace_tensor,
    dual_stream_workspace_tensor,
    wedlm_decode_step,
    wedlm_decode_step_workspace,
    wedlm_dual_stream_attn,
    wedlm_attn_plan,
    wedlm_last_error,
    wedlm_lmhead_select_commit,
    wedlm_model_step,
    wedlm_lmhead_select_commit_workspace,
    wedlm_reorder,
    wedlm_select_commit,
    wedlm_select_commit_workspace,
    wedlm_set_attn_split_keys,
    wedlm_attn_tail,
    attn_tail,
    wedlm_set_attn_tail,
    wedlm_set_select_parts,
    wedlm_step_attn,
    wedlm_step_attn_noalloc,
    wedlm_step_attn_noalloc_limit,
    wedlm_step_attn_workspace,
    wedlm_version,
)
