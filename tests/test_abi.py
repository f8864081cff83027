"""C-ABI library checks that need no GPU: it loads, exports every symbol the
header declares, and its host-side validation and launch planning behave.
No call here reaches a kernel launch (every case fails validation first or
is a pure host query)."""
import ctypes as C
import os
import re
import subprocess

import pytest

import causal_attention_diffusion_amd as wd
from causal_attention_diffusion_amd.binding import WedlmShape

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wedlm.h")

OK, ERR_ARG, ERR_SHAPE, ERR_UNSUP, ERR_HIP, ERR_WS = 0, 1, 2, 3, 4, 5


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(wedlm_\w+)\s*\(", text)))


def test_header_declares_the_three_step_calls():
    f = declared_functions()
    for name in ["wedlm_reorder", "wedlm_step_attn", "wedlm_select_commit",
                 "wedlm_step_attn_workspace", "wedlm_select_commit_workspace", "wedlm_last_error"]:
        assert name in f


def test_library_exports_every_declared_symbol():
    lib = wd.load_library()
    out = subprocess.run(["nm", "-D", "--defined-only", wd.lib_path()], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (wedlm_\w+)$", out, flags=re.M))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_header_compiles_as_c():
    src = '#include "wedlm.h"\nint main(void){ wedlm_shape s; (void)s; return 0; }\n'
    p = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-I",
                        os.path.dirname(HEADER), "-x", "c", "-"], input=src, text=True, capture_output=True)
    assert p.returncode == 0, p.stderr


def _shape(**kw):
    d = dict(B=2, W=16, Hq=32, Hkv=8, D=128, page_size=16, max_pages=10, num_pages=20, dtype=1)
    d.update(kw)
    return WedlmShape(**d)


NULLS = [None] * 16


def _reorder(s):
    lib = wd.load_library()
    fake = C.c_void_p(0x1000)   # never dereferenced: validation fails before any launch
    args = [fake] * 11
    return lib.wedlm_reorder(C.byref(s) if s is not None else None, *args, 1e4, None, None)


@pytest.mark.parametrize("kw,code", [
    (dict(W=0), ERR_SHAPE), (dict(W=65), ERR_SHAPE), (dict(B=0), ERR_SHAPE),
    (dict(Hq=30, Hkv=8), ERR_SHAPE), (dict(Hq=64, Hkv=2), ERR_SHAPE),
    (dict(D=96), ERR_UNSUP), (dict(page_size=32), ERR_UNSUP),
    (dict(dtype=5), ERR_ARG), (dict(num_pages=0), ERR_SHAPE),
])
def test_reorder_rejects_bad_shapes(kw, code):
    assert _reorder(_shape(**kw)) == code
    assert wd.wedlm_last_error() != ""


def test_reorder_rejects_null_shape_and_pointers():
    lib = wd.load_library()
    assert _reorder(None) == ERR_ARG
    s = _shape()
    assert lib.wedlm_reorder(C.byref(s), *([None] * 11), 1e4, None, None) == ERR_ARG
    fake = C.c_void_p(0x1000)
    assert lib.wedlm_reorder(C.byref(s), *([fake] * 11), 0.5, None, None) == ERR_ARG   # rope_base <= 1


def test_step_attn_validation():
    lib = wd.load_library()
    s = _shape(max_pages=10)
    fake = C.c_void_p(0x1000)
    # max_ctx_len + W beyond the block table
    assert lib.wedlm_step_attn(C.byref(s), *([fake] * 7), 0.0, 200, None, 0, None, None) == ERR_SHAPE
    # NULL pointer
    assert lib.wedlm_step_attn(C.byref(s), *([None] * 7), 0.0, 100, None, 0, None, None) == ERR_ARG
    # negative scale
    assert lib.wedlm_step_attn(C.byref(s), *([fake] * 7), -1.0, 100, None, 0, None, None) == ERR_ARG
    # workspace too small (this plan needs one)
    need = lib.wedlm_step_attn_workspace(C.byref(s), 100)
    big = _shape(max_pages=4000, B=1)
    need_big = lib.wedlm_step_attn_workspace(C.byref(big), 60000)
    assert need_big > 0
    assert lib.wedlm_step_attn(C.byref(big), *([fake] * 7), 0.0, 60000, fake, need_big - 1, None,
                               None) == ERR_WS
    assert need >= 0


def test_decode_step_validation_and_workspace():
    from causal_attention_diffusion_amd.binding import WedlmStepIO
    lib = wd.load_library()
    s = _shape(max_pages=200)
    fake = 0x1000   # never dereferenced: validation fails before any launch
    io = WedlmStepIO(*([fake] * 16), None, None, None, None, 4096, 2000, 4096, 0.0, 0.25, 4.0, 1e6)
    need = lib.wedlm_decode_step_workspace(C.byref(s), 2000, 4096)
    # the split partials then the vocabulary partials, on 256-byte boundaries
    attn = lib.wedlm_step_attn_workspace(C.byref(s), 2000)
    assert need == (attn + 255) // 256 * 256 + lib.wedlm_select_commit_workspace(2, 16, 4096)
    assert lib.wedlm_decode_step(C.byref(s), None, fake, need, None) == ERR_ARG
    assert lib.wedlm_decode_step(C.byref(s), C.byref(io), fake, need - 1, None) == ERR_WS
    assert lib.wedlm_decode_step(C.byref(s), C.byref(io), None, need, None) == ERR_WS
    bad = WedlmStepIO(*([fake] * 16), None, None, None, None, 4096, 2000, 4096, 0.0, 0.25, 4.0, 0.5)
    assert lib.wedlm_decode_step(C.byref(s), C.byref(bad), fake, need, None) == ERR_ARG     # rope_base
    bad = WedlmStepIO(*([fake] * 16), None, None, None, None, 4096, 2000, 4096, 0.0, 0.25, float("inf"), 1e6)
    assert lib.wedlm_decode_step(C.byref(s), C.byref(bad), fake, need, None) == ERR_ARG     # tau
    bad = WedlmStepIO(*([fake] * 16), None, None, None, None, 4096, 5000, 4096, 0.0, 0.25, 4.0, 1e6)
    assert lib.wedlm_decode_step(C.byref(s), C.byref(bad), fake, 1 << 30, None) == ERR_SHAPE  # beyond the table
    nul = WedlmStepIO(*([fake] * 7), None, *([fake] * 8), None, None, None, None, 4096, 2000, 4096, 0.0, 0.25,
                      4.0, 1e6)   # no logits
    assert lib.wedlm_decode_step(C.byref(s), C.byref(nul), fake, need, None) == ERR_ARG
    assert lib.wedlm_decode_step_workspace(C.byref(s), 2000, 0) == 0
    # the timed form checks the same arguments before it launches anything
    assert lib.wedlm_decode_step_timed(C.byref(s), C.byref(io), fake, need - 1, None, None, None) == ERR_WS
    assert lib.wedlm_decode_step_timed(C.byref(s), C.byref(nul), fake, need, None, fake, fake) == ERR_ARG
    assert lib.wedlm_decode_step_timed(C.byref(s), None, fake, need, None, None, None) == ERR_ARG
    assert lib.wedlm_attn_tail(C.byref(_shape(W=65)), 2000) == -1
    assert lib.wedlm_attn_tail(C.byref(s), -1) == -1
    assert lib.wedlm_decode_step(C.byref(_shape(W=65)), C.byref(io), fake, need, None) == ERR_SHAPE


@pytest.mark.parametrize("B,W,Hq,Hkv,D,dt,L", [
    (4, 32, 32, 8, 128, 1, 32768), (32, 16, 32, 8, 128, 1, 8192), (1, 16, 32, 8, 128, 1, 2048),
    (1, 8, 4, 2, 64, 0, 64), (1, 64, 32, 8, 128, 1, 300), (3, 1, 8, 8, 64, 1, 0), (2, 16, 32, 4, 128, 1, 100000), (1, 64, 32, 8, 128, 1, 524224),
])
def test_attention_plan_covers_every_key(B, W, Hq, Hkv, D, dt, L):
    mp = (L + W + 15) // 16
    ns, sk = wd.attn_plan(B, W, Hq, Hkv, D, mp, B * mp, dt, L)
    tail = wd.attn_tail(B, W, Hq, Hkv, D, mp, B * mp, dt, L)
    assert ns >= 1 and sk >= 32 and sk % 32 == 0 and sk <= 32768
    if tail:
        # tail splits: the first work-group of a sequence covers it all (or
        # its front half), the second the back half of a cut sequence
        assert ns == 2 and sk >= L + W and 0 < tail <= B
    else:
        assert ns * sk >= L + W                 # the grid covers every visible key
        assert (ns - 1) * sk < L + W            # and no split is wholly past the end
    s = _shape(B=B, W=W, Hq=Hq, Hkv=Hkv, D=D, max_pages=mp, num_pages=B * mp, dtype=dt)
    ws = wd.load_library().wedlm_step_attn_workspace(C.byref(s), L)
    assert (ws == 0) == (ns == 1)


def test_tail_split_plan():
    # one split per (sequence, KV head) filling 128..256 CUs in one round:
    # the longest 3/8 of the batch are cut in two (bf16 only)
    assert wd.attn_tail(32, 16, 32, 8, 128, 513, 32 * 513, 1, 8192) == 12
    assert wd.attn_plan(32, 16, 32, 8, 128, 513, 32 * 513, 1, 8192)[0] == 2
    assert wd.attn_tail(32, 16, 32, 8, 128, 513, 32 * 513, 0, 8192) == 0       # fp32
    assert wd.attn_tail(8, 16, 32, 8, 128, 513, 8 * 513, 1, 8192) == 0         # 64 groups: under half the CUs
    assert wd.attn_tail(64, 16, 32, 8, 128, 513, 64 * 513, 1, 8192) == 0       # 512 groups: two rounds
    assert wd.attn_tail(4, 32, 32, 8, 128, 2100, 4 * 2100, 1, 32768) == 0      # several splits already
    assert wd.attn_tail(2, 64, 32, 8, 128, 200, 400, 1, 3000) == 0             # two row tiles
    try:
        wd.wedlm_set_attn_tail(0)
        assert wd.attn_tail(32, 16, 32, 8, 128, 513, 32 * 513, 1, 8192) == 0
        assert wd.attn_plan(32, 16, 32, 8, 128, 513, 32 * 513, 1, 8192)[0] == 1
        wd.wedlm_set_attn_tail(5)
        assert wd.attn_tail(8, 16, 32, 8, 128, 8, 64, 1, 100) == 5             # forced below half the CUs
        assert wd.attn_tail(3, 16, 32, 8, 128, 8, 24, 1, 100) == 3             # at most B
        assert wd.attn_tail(8, 16, 32, 8, 128, 8, 64, 0, 100) == 0             # still bf16 only
        assert wd.attn_tail(8, 16, 32, 8, 128, 513, 8 * 513, 1, 8192) == 0     # the plan has 4 splits
        with pytest.raises(wd.WedlmError):
            wd.wedlm_set_attn_tail(-2)
    finally:
        wd.wedlm_set_attn_tail(-1)


def test_split_override_validation():
    with pytest.raises(wd.WedlmError):
        wd.wedlm_set_attn_split_keys(100)
    with pytest.raises(wd.WedlmError):
        wd.wedlm_set_attn_split_keys(32768 + 64)
    wd.wedlm_set_attn_split_keys(128)
    try:
        ns, sk = wd.attn_plan(1, 16, 32, 8, 128, 200, 200, 1, 3000)
        assert sk == 128 and ns == (3000 + 16 + 127) // 128
    finally:
        wd.wedlm_set_attn_split_keys(0)


def test_select_commit_validation_and_workspace():
    lib = wd.load_library()
    fake = C.c_void_p(0x1000)
    assert lib.wedlm_select_commit(0, 16, 100, *([fake] * 10), 0.1, 1.0, 100, fake, 1 << 20, None) == ERR_SHAPE
    assert lib.wedlm_select_commit(2, 65, 100, *([fake] * 10), 0.1, 1.0, 100, fake, 1 << 20, None) == ERR_SHAPE
    assert lib.wedlm_select_commit(2, 16, 100, *([None] * 10), 0.1, 1.0, 100, fake, 1 << 20, None) == ERR_ARG
    assert lib.wedlm_select_commit(2, 16, 100, *([fake] * 10), float("nan"), 1.0, 100, fake, 1 << 20,
                                   None) == ERR_ARG
    need = lib.wedlm_select_commit_workspace(64, 16, 151936)
    assert need >= 64 * 16 * 10 * 16      # one float4 per (slot, 16384 logits)
    assert lib.wedlm_select_commit(64, 16, 151936, *([fake] * 10), 0.1, 1.0, 100, fake, need - 1,
                                   None) == ERR_WS
    assert lib.wedlm_select_commit(64, 16, 151936, *([fake] * 10), 0.1, 1.0, 100, None, need, None) == ERR_WS


def test_binding_refuses_host_tensors():
    import torch
    x = torch.zeros((1, 8, 4, 64))
    kc = torch.zeros((5, 2, 16, 64))
    bt = torch.zeros((1, 5), dtype=torch.int32)
    with pytest.raises(wd.WedlmError):
        wd.wedlm_step_attn(x, kc, kc, bt, torch.zeros(1, dtype=torch.int32),
                           torch.zeros((1, 8), dtype=torch.int32), x.clone(), max_ctx_len=10)


def test_binding_checks_shapes_before_pointers():
    import torch
    x = torch.zeros((1, 8, 4, 64))
    kc = torch.zeros((5, 2, 16, 64))
    bt = torch.zeros((1, 5), dtype=torch.int32)
    with pytest.raises(wd.WedlmError, match="perm"):
        wd.wedlm_step_attn(x, kc, kc, bt, torch.zeros(1, dtype=torch.int32),
                           torch.zeros((1, 7), dtype=torch.int32), x.clone(), max_ctx_len=10)
    with pytest.raises(wd.WedlmError, match="cache"):
        wd.wedlm_step_attn(x, torch.zeros((5, 2, 8, 64)), kc, bt, torch.zeros(1, dtype=torch.int32),
                           torch.zeros((1, 8), dtype=torch.int32), x.clone(), max_ctx_len=10)


def test_product_and_oracle_share_no_code():
    """The HIP path never imports the oracle, and the oracle never imports the
    product package; only the input generator module is shared."""
    pkg = os.path.join(ROOT, "causal_attention_diffusion_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), f
                assert "wedlm_oracle" not in text, f
                assert "workloads" not in text or f.endswith(".md"), f
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith((".py", ".c", ".h")):
            text = open(os.path.join(ROOT, "oracle", f)).read()
            assert "causal_attention_diffusion_amd" not in text, f
            assert not re.search(r'#include\s+"[^"]*(csrc|include/wedlm)', text), f


def test_lmhead_validation_and_workspace():
    lib = wd.load_library()
    fake = C.c_void_p(0x1000)
    ws = lib.wedlm_lmhead_select_commit_workspace
    assert ws(64, 16, 151936, 4096) > 64 * 16 * 594 * 16
    assert ws(1, 1, 1, 64) > 0
    for bad in [(0, 16, 100, 64), (1, 65, 100, 64), (65, 64, 100, 64), (1, 8, 0, 64), (1, 8, 100, 96),
                (1, 8, 100, 0), (1, 8, 100, 65536 + 64)]:
        assert ws(*bad) == 0, bad
    args = [fake] * 11 + [C.c_float(0.1), C.c_float(1.0), 100, fake, C.c_size_t(1 << 30), None]
    assert lib.wedlm_lmhead_select_commit(1, 8, 100, 96, *args) == ERR_SHAPE
    assert lib.wedlm_lmhead_select_commit(1, 8, 100, 64, None, *args[1:]) == ERR_ARG
    misaligned = C.c_void_p(0x1008)
    assert lib.wedlm_lmhead_select_commit(1, 8, 100, 64, misaligned, *args[1:]) == ERR_ARG
    small = args[:15] + [C.c_size_t(ws(1, 8, 100, 64) - 1), None]
    assert lib.wedlm_lmhead_select_commit(1, 8, 100, 64, *small) == ERR_WS
    nan = args[:11] + [C.c_float(float("nan"))] + args[12:]
    assert lib.wedlm_lmhead_select_commit(1, 8, 100, 64, *nan) == ERR_ARG


def test_dual_stream_validation():
    lib = wd.load_library()
    ok = wd.make_shape(1, 32, 4, 2, 64, 1, 1, wd.WEDLM_BF16)
    assert lib.wedlm_dual_stream_attn_workspace(C.byref(ok), 256) > 0
    for W, N in [(8, 256), (48, 256), (32, 100), (32, 0)]:
        bad = wd.make_shape(1, W, 4, 2, 64, 1, 1, wd.WEDLM_BF16)
        assert lib.wedlm_dual_stream_attn_workspace(C.byref(bad), N) == 0, (W, N)
    fake = C.c_void_p(0x1000)
    assert lib.wedlm_dual_stream_attn(C.byref(ok), 256, *([fake] * 8), None, 1e6, fake, 1 << 40, None,
                                      None) == ERR_ARG
    need = lib.wedlm_dual_stream_attn_workspace(C.byref(ok), 256)
    assert lib.wedlm_dual_stream_attn(C.byref(ok), 256, *([fake] * 9), 1e6, fake, need - 1, None, None) == ERR_WS


def _model_struct(d_model=256, d_ff=512, vocab=1000, addr=0x1000, misaligned_field=None):
    from causal_attention_diffusion_amd.binding import LAYER_FIELDS, WedlmLayerWeights, WedlmModel
    vals = [addr + 0x100000 * i for i in range(len(LAYER_FIELDS))]
    if misaligned_field is not None:
        vals[LAYER_FIELDS.index(misaligned_field)] += 8
    layers = (WedlmLayerWeights * 1)(WedlmLayerWeights(*vals))
    m = WedlmModel(1, d_model, d_ff, vocab, 1e-6, addr + 0x2000000, addr + 0x3000000, addr + 0x4000000,
                   C.cast(layers, C.POINTER(WedlmLayerWeights)))
    return m, layers


def test_model_step_validation_and_workspace():
    """Shape, pointer, alignment and workspace checks of wedlm_model_step
    (all fail before any launch)."""
    lib = wd.load_library()
    fake = C.c_void_p(0x1000)
    shape = wd.make_shape(2, 8, 4, 2, 64, 8, 16, wd.WEDLM_BF16)   # d_model = Hq * D = 256
    m, keep = _model_struct()
    need = lib.wedlm_model_step_workspace(C.byref(m), C.byref(shape), 64)
    assert need > 0
    bad_d, keep2 = _model_struct(d_model=512)                         # != Hq * D
    assert lib.wedlm_model_step_workspace(C.byref(bad_d), C.byref(shape), 64) == 0
    bad_ff, keep3 = _model_struct(d_ff=300)                           # not a multiple of 256
    assert lib.wedlm_model_step_workspace(C.byref(bad_ff), C.byref(shape), 64) == 0

    def call(model, ptrs=None, ws=fake, ws_bytes=None):
        p = [fake] * 7 if ptrs is None else ptrs   # block_table .. committed
        return lib.wedlm_model_step(C.byref(model), C.byref(shape), *p, None, None, None, None, C.c_float(0.25),
                                    C.c_float(2.0), C.c_double(1e4), 64, ws,
                                    C.c_size_t(need if ws_bytes is None else ws_bytes), None, None)

    assert call(bad_d) == ERR_SHAPE
    assert call(m, ptrs=[None] + [fake] * 6) == ERR_ARG
    for f in ("wq", "w_down", "attn_norm"):
        mis, keep4 = _model_struct(misaligned_field=f)
        assert call(mis) == ERR_ARG, f
    assert call(m, ws=None) == ERR_WS
    assert call(m, ws_bytes=need - 1) == ERR_WS
    assert "workspace" in wd.wedlm_last_error()


def test_graph_api_validation():
    """The capture entry points reject NULL streams and graphs before any
    HIP call; destroy(NULL) is a no-op."""
    lib = wd.load_library()
    assert lib.wedlm_graph_begin(None) == ERR_ARG
    out = C.c_void_p()
    assert lib.wedlm_graph_end(None, C.byref(out)) == ERR_ARG
    assert lib.wedlm_graph_end(C.c_void_p(0x1000), None) == ERR_ARG
    assert lib.wedlm_graph_launch(None, None) == ERR_ARG
    k, o = C.c_size_t(), C.c_size_t()
    assert lib.wedlm_graph_nodes(None, C.byref(k), C.byref(o)) == ERR_ARG
    lib.wedlm_graph_destroy(None)
    assert "NULL" in wd.wedlm_last_error()


def test_missing_library_fails_loudly():
    """Without libwedlm.so every entry point raises: there is no fallback
    path (a fresh interpreter, with the binding pointed at a path that does
    not exist)."""
    code = (
        "import causal_attention_diffusion_amd.binding as b\n"
        "b._LIB = None\n"
        "b._LIB_PATH = '/nonexistent/libwedlm.so'\n"
        "import causal_attention_diffusion_amd as wd\n"
        "for f in (lambda: b.load_library(), lambda: wd.wedlm_version()):\n"
        "    try:\n"
        "        f()\n"
        "    except b.WedlmError as e:\n"
        "        assert 'not built' in str(e) and 'no fallback' in str(e), e\n"
        "    else:\n"
        "        raise SystemExit('no error raised')\n"
        "print('raised')\n")
    r = subprocess.run(["python3", "-c", code], capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 0 and "raised" in r.stdout, r.stdout + r.stderr
