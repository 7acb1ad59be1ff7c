"""The block's operations around the method on the decode path
(kda_decode_tokens_module): the short causal convolution continued from a
convolution state (the three raw tokens before the launch), and the output
norm and gate (page "K3 架构图解", chapter 08 figure caption; chapter 09:
the convolution is causal).  A prefill that hands its final convolution
state to decode launches must give what one prefill over all the tokens
gives: both are checked against the block's steps in float64 (tests/
module_ref.py) feeding the oracle, and the convolution state itself is
checked value for value."""
import pytest
import torch

from linear_attention_kda_amd import inputs
from tests import module_ref as mr
from tests.gpu_cases import TOL, announce, check, oracle_prefill, to_dev
from tests.test_gpu_module_ops import _raw_block, _weights

pytestmark = pytest.mark.gpu

QK, BETA = 1, 2


def _reference(inp, w, dk):
    """Activated inputs of the whole sequence in float64, the oracle, then
    the norm and gate: (o, S_final) as float64 torch tensors."""
    ref = dict(inp)
    wq, wk, wv = w["conv"]
    ref["q"] = mr.silu_unit(mr.short_conv(inp["q"], wq))
    ref["k"] = mr.silu_unit(mr.short_conv(inp["k"], wk))
    ref["v"] = mr.short_conv(inp["v"], wv)
    ref["beta"] = torch.sigmoid(inp["beta"].detach().cpu().double())
    ref["alpha"] = torch.exp(-torch.nn.functional.softplus(inp["alpha"].detach().cpu().double()))
    o, S = oracle_prefill(ref)
    o = mr.out_gate(mr.rms_norm(torch.as_tensor(o), w["norm_weight"], w["norm_eps"]), w["out_gate"])
    return o, torch.as_tensor(S)


def _raw_tail(x, T1, t0, t1):
    return x[:, t0:t1].contiguous()


def _expected_state(inp, t_end):
    """The last three raw tokens before t_end, q | k | v, zeros before 0."""
    B, _, H, dk = inp["q"].shape
    dv = inp["v"].shape[-1]
    cs = torch.zeros((B, H, 3, 2 * dk + dv), dtype=inp["q"].dtype, device=inp["q"].device)
    for s in range(3):
        t = t_end - 3 + s
        if t >= 0:
            cs[:, :, s, :dk] = inp["q"][:, t]
            cs[:, :, s, dk:2 * dk] = inp["k"][:, t]
            cs[:, :, s, 2 * dk:] = inp["v"][:, t]
    return cs


@pytest.mark.parametrize("dtype,dk,dv,T1,chunks", [(torch.bfloat16, 128, 128, 130, (5,)),
                                                   (torch.float32, 64, 32, 70, (1, 3, 2)),
                                                   (torch.bfloat16, 32, 64, 2, (4, 1)),
                                                   (torch.float32, 16, 16, 64, (2,))])
def test_prefill_then_decode_equals_one_prefill(dtype, dk, dv, T1, chunks):
    import linear_attention_kda_amd as kda
    B, H = 2, 2
    T = T1 + sum(chunks)
    announce(f"module ops: prefill of {T1} then decode launches {chunks}, B={B} H={H} dk={dk} dv={dv} {dtype}")
    inp = _raw_block(to_dev(inputs.dense(B, T, H, dk, dv, dtype, s0_std=0.02, seed=91 + T1,
                                         gate_form="softplus_channel")), 91 + T1)
    w = _weights(H, dk, dv, dtype, inp["v"].shape, 91 + T1)
    o_ref, S_ref = _reference(inp, w, dk)
    cs = torch.empty((B, H, 3, 2 * dk + dv), dtype=dtype, device="cuda")
    pre = {n: inp[n][:, :T1].contiguous() for n in ("q", "k", "v", "alpha", "beta")}
    wp = dict(w, out_gate=w["out_gate"][:, :T1].contiguous())
    o1, S = kda.chunk_fwd(pre["q"], pre["k"], pre["v"], pre["alpha"], pre["beta"], S0=inp["S0"],
                          gate="softplus_channel", act=QK | BETA, conv_state=cs, **wp)
    torch.cuda.synchronize()
    assert torch.equal(cs, _expected_state(inp, T1))
    check("o prefill part", o1, o_ref[:, :T1].numpy(), TOL[dtype])
    t0 = T1
    for Tk in chunks:
        d = {n: inp[n][:, t0:t0 + Tk].contiguous() for n in ("q", "k", "v", "alpha", "beta")}
        wd = dict(w, out_gate=w["out_gate"][:, t0:t0 + Tk].contiguous())
        od, S = kda.decode_tokens(d["q"], d["k"], d["v"], d["alpha"], d["beta"], S, S_out=S,
                                  gate="softplus_channel", act=QK | BETA, conv_state=cs, **wd)
        torch.cuda.synchronize()
        t0 += Tk
        assert torch.equal(cs, _expected_state(inp, t0))
        check(f"o decode tokens to {t0}", od, o_ref[:, t0 - Tk:t0].numpy(), TOL[dtype])
    check("S_final", S, S_ref.numpy(), TOL[dtype])


def test_decode_from_a_sequence_start():
    # a zero convolution state: the decode launch is the sequence's start, so
    # it must equal a prefill of the same tokens (with its zero halo)
    import linear_attention_kda_amd as kda
    announce("module ops: decode of 6 tokens from a zero convolution state vs prefill, N=3 H=2 d=128 bf16")
    N, H, D, Tk = 3, 2, 128, 6
    inp = _raw_block(to_dev(inputs.dense(N, Tk, H, D, D, torch.bfloat16, s0_std=0.02, seed=95,
                                         gate_form="softplus_channel")), 95)
    w = _weights(H, D, D, torch.bfloat16, inp["v"].shape, 95)
    o_ref, S_ref = _reference(inp, w, D)
    cs = torch.zeros((N, H, 3, 3 * D), dtype=torch.bfloat16, device="cuda")
    od, S = kda.decode_tokens(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["S0"],
                              gate="softplus_channel", act=QK | BETA, conv_state=cs, **w)
    torch.cuda.synchronize()
    check("o", od, o_ref.numpy(), TOL[torch.bfloat16])
    check("S", S, S_ref.numpy(), TOL[torch.bfloat16])
    assert torch.equal(cs, _expected_state(inp, Tk))
    # the same tokens through the prefill give the same outputs up to the two
    # schedules' rounding
    op, Sp = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], S0=inp["S0"],
                           gate="softplus_channel", act=QK | BETA, **w)
    torch.cuda.synchronize()
    check("o decode vs prefill", od, op.double().cpu().numpy(), TOL[torch.bfloat16])


def test_decode_norm_gate_only():
    import linear_attention_kda_amd as kda
    announce("decode tokens with the output norm and gate only, N=4 Tk=3 H=2 d=64 fp32")
    N, H, D, Tk = 4, 2, 64, 3
    inp = to_dev(inputs.dense(N, Tk, H, D, D, torch.float32, s0_std=0.02, seed=96))
    w = _weights(H, D, D, torch.float32, inp["v"].shape, 96, conv=False)
    od, S = kda.decode_tokens(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["S0"], **w)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_prefill(inp)
    o_ref = mr.out_gate(mr.rms_norm(torch.as_tensor(o_ref), w["norm_weight"], w["norm_eps"]), w["out_gate"])
    check("o", od, o_ref.numpy(), TOL[torch.float32])
    check("S", S, S_ref, TOL[torch.float32])
