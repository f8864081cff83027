"""GPU parity of the Dual-Stream Masking attention (wedlm_dual_stream_attn)
against the oracle's direct formulation (explicit visibility over both
streams in logical order, float64).  The GPU path builds it from decode-step
windows over a shared paged cache; the oracle shares none of that.

Tolerance as for attention: max |gpu - oracle| / max |oracle| <= 2e-2 for
bf16 and 1e-4 for fp32, over every output or over sampled rows.
"""
import numpy as np
import pytest
import torch

import oracle
import causal_attention_diffusion_amd as wd
from workloads import f32_to_bf16_bits, bf16_bits_to_f32

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _case(S, N, b, Hq, Hkv, D, dtype, seed):
    rng = np.random.default_rng(seed)

    def draw(h):
        x = rng.standard_normal((S, N, h, D)).astype(np.float32)
        return f32_to_bf16_bits(x) if dtype == "bf16" else x

    arrs = [draw(Hq), draw(Hkv), draw(Hkv), draw(Hq), draw(Hkv), draw(Hkv)]
    flags = (rng.random((S, N)) < rng.uniform(0.2, 0.8, (S, N // b, 1)).repeat(b, 1).reshape(S, N)).astype(np.uint8)
    flags[0, :b] = 1                      # an all-observed block
    flags[0, b:2 * b] = 0                 # an all-masked block
    return arrs, flags


def _to_dev(a, dtype, dev):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return (t.view(torch.bfloat16) if dtype == "bf16" else t).to(dev)


def _vals(a, dtype):
    return (bf16_bits_to_f32(a) if dtype == "bf16" else a).astype(np.float64)


def _run(S, N, b, Hq, Hkv, D, dtype, seed, dev, rows=None, base=1e6):
    arrs, flags = _case(S, N, b, Hq, Hkv, D, dtype, seed)
    t = [_to_dev(a, dtype, dev) for a in arrs]
    fl = torch.from_numpy(flags).to(dev)
    out_m = torch.empty_like(t[0])
    out_p = torch.empty_like(t[3])
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = wd.dual_stream_workspace_tensor(t[0], t[1], b)
    wd.wedlm_dual_stream_attn(*t, fl, out_m, out_p, b, base, ws, dev_status=status)
    torch.cuda.synchronize()
    assert status.item() == 0
    om, op = oracle.dual_stream_attention(*[_vals(a, dtype) for a in arrs], flags, b, dtype, base, rows=rows)
    gm = out_m.float().cpu().numpy().astype(np.float64)
    gp = out_p.float().cpu().numpy().astype(np.float64)
    if rows is None:
        ref = np.concatenate([om.ravel(), op.ravel()])
        got = np.concatenate([gm.ravel(), gp.ravel()])
    else:
        ref = np.stack([(om if st == 0 else op)[s, n] for s, st, n in rows])
        got = np.stack([(gm if st == 0 else gp)[s, n] for s, st, n in rows])
    err = float(np.abs(got - ref).max() / np.abs(ref).max())
    print(f"[dual stream] S{S} N{N} b{b} {Hq}/{Hkv} D{D} {dtype}: rel err {err:.3e}", flush=True)
    assert err <= TOL[dtype], err


@pytest.mark.parametrize("S,N,b,Hq,Hkv,D,dtype", [
    (2, 128, 32, 4, 2, 64, "bf16"),
    (1, 128, 16, 4, 2, 64, "f32"),
    (1, 256, 64, 8, 2, 128, "bf16"),
    (1, 192, 16, 4, 1, 128, "bf16"),
])
def test_dual_stream_all_outputs(S, N, b, Hq, Hkv, D, dtype, dev):
    _run(S, N, b, Hq, Hkv, D, dtype, 2000 + N + b, dev)


def test_dual_stream_qwen3_shape_sampled_rows(dev):
    # 2048 tokens, blocks of 32, 32/8 heads of 128: first, middle and last
    # blocks of both streams
    N, b = 2048, 32
    rng = np.random.default_rng(7)
    toks = np.concatenate([np.arange(0, 40), np.arange(1000, 1030), np.arange(N - 40, N), rng.integers(0, N, 20)])
    rows = np.array([(0, st, n) for st in (0, 1) for n in toks])
    _run(1, N, b, 32, 8, 128, "bf16", 2100, dev, rows=rows)
