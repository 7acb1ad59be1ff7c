"""The plain entry points of the boundary, kda_chunk_fwd and kda_decode_step,
called through the C ABI on real device buffers (the other GPU tests reach
the kernels through the _ex / _gated forms, which these forward to): against
the fp64 oracle per unit, and bit for bit against the forms the binding
uses."""
import ctypes

import pytest
import torch

from linear_attention_kda_amd import inputs
from tests.gpu_cases import TOL, announce, check, oracle_prefill, to_dev

pytestmark = pytest.mark.gpu


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_plain_chunk_fwd_dense(dtype):
    import linear_attention_kda_amd as kda
    announce(f"kda_chunk_fwd through the C ABI, dense B=2 T=130 H=2 d=64 {dtype}")
    B, T, H, D = 2, 130, 2, 64
    inp = to_dev(inputs.dense(B, T, H, D, D, dtype, s0_std=0.02, seed=81))
    code = kda.KDA_BF16 if dtype == torch.bfloat16 else kda.KDA_F32
    ws = torch.empty(kda.chunk_fwd_workspace_size(B, T, H, D, D, -1, code), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(inp["v"])
    S = torch.empty((B, H, D, D), dtype=torch.float32, device="cuda")
    st = kda.lib.kda_chunk_fwd(_p(inp["q"]), _p(inp["k"]), _p(inp["v"]), _p(inp["alpha"]), _p(inp["beta"]),
                               _p(inp["S0"]), None, B, B, T, H, D, D, 0.0, code, _p(o), _p(S), _p(ws),
                               ws.numel(), _stream())
    assert st == 0, kda.status_string(st)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_prefill(inp)
    check("o", o, o_ref, TOL[dtype])
    check("S_final", S, S_ref, TOL[dtype])
    o2, S2 = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], S0=inp["S0"])
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(S, S2)


def test_plain_chunk_fwd_packed():
    import linear_attention_kda_amd as kda
    announce("kda_chunk_fwd through the C ABI, packed [70, 0, 5, 200] H=3 d=128 bf16")
    inp = to_dev(inputs.packed([70, 0, 5, 200], 3, 128, 128, torch.bfloat16, s0_std=0.02, seed=82))
    cu = inp["cu_seqlens"]
    N, T, H = cu.numel() - 1, inp["q"].shape[0], 3
    ws = torch.empty(kda.chunk_fwd_workspace_size(1, T, H, 128, 128, N, kda.KDA_BF16), dtype=torch.uint8,
                     device="cuda")
    o = torch.empty_like(inp["v"])
    S = torch.empty((N, H, 128, 128), dtype=torch.float32, device="cuda")
    st = kda.lib.kda_chunk_fwd(_p(inp["q"]), _p(inp["k"]), _p(inp["v"]), _p(inp["alpha"]), _p(inp["beta"]),
                               _p(inp["S0"]), _p(cu), N, 1, T, H, 128, 128, 0.0, kda.KDA_BF16, _p(o), _p(S),
                               _p(ws), ws.numel(), _stream())
    assert st == 0, kda.status_string(st)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_prefill(inp)
    check("o", o, o_ref, TOL[torch.bfloat16], cu=cu)
    check("S_final", S, S_ref, TOL[torch.bfloat16])


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_plain_decode_step(dtype):
    import linear_attention_kda_amd as kda
    import oracle
    announce(f"kda_decode_step through the C ABI, N=5 H=3 d=128 {dtype}")
    N, H, D = 5, 3, 128
    S0 = inputs.decode_state(N, H, D, D, 0.02, seed=83, device="cuda")
    d = to_dev(inputs.decode_token(N, H, D, D, dtype, seed=83))
    code = kda.KDA_BF16 if dtype == torch.bfloat16 else kda.KDA_F32
    S = S0.clone()
    o = torch.empty((N, H, D), dtype=dtype, device="cuda")
    st = kda.lib.kda_decode_step(_p(d["q"]), _p(d["k"]), _p(d["v"]), _p(d["alpha"]), _p(d["beta"]), _p(S),
                                 N, H, D, D, 0.0, code, _p(o), _stream())
    assert st == 0, kda.status_string(st)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.decode(d["q"], d["k"], d["v"], d["alpha"], d["beta"], S0.double().cpu().numpy())
    check("o step", o, o_ref, TOL[dtype])
    check("S step", S, S_ref, TOL[dtype])
    S2 = S0.clone()
    o2 = kda.decode_step(d["q"], d["k"], d["v"], d["alpha"], d["beta"], S2)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(S, S2)
