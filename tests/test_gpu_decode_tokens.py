"""Several decode tokens per launch (verification of a speculative draft):
the token-by-token schedule over Tk tokens with the state kept in registers
must equal the oracle run over those Tk tokens from S_in, equal Tk single
steps bit for bit, and leave S_in untouched unless asked to update in place."""
import pytest
import torch

from linear_attention_kda_amd import inputs
from tests.gpu_cases import TOL, announce, check, oracle_prefill, to_dev

pytestmark = pytest.mark.gpu


def _inputs(N, Tk, H, d, dtype, gate_form, seed):
    return to_dev(inputs.dense(N, Tk, H, d, d, dtype, gate="uniform", alpha_lo=0.95, s0_std=0.02,
                               seed=seed, gate_form=gate_form))


@pytest.mark.parametrize("gate_form", ["channel", "scalar"])
@pytest.mark.parametrize("dtype,d,Tk", [(torch.bfloat16, 128, 1), (torch.bfloat16, 128, 8),
                                       (torch.bfloat16, 128, 3), (torch.float32, 128, 5),
                                       (torch.float32, 32, 3), (torch.float32, 64, 5)])
def test_decode_tokens_matches_oracle(gate_form, dtype, d, Tk):
    import linear_attention_kda_amd as kda
    announce(f"decode_tokens N=4 Tk={Tk} H=3 d={d} {dtype} gate {gate_form}")
    inp = _inputs(4, Tk, 3, d, dtype, gate_form, seed=21)
    S_in = inp["S0"].clone()
    o, S_out = kda.decode_tokens(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], S_in,
                                 gate=gate_form)
    torch.cuda.synchronize()
    assert torch.equal(S_in, inp["S0"]), "S_in is the checkpoint and must not change"
    ref = dict(inp)
    if gate_form == "scalar":
        ref["alpha"] = inp["alpha"].unsqueeze(-1).expand(*inp["q"].shape).contiguous()
    o_ref, S_ref = oracle_prefill(ref)
    check("o", o, o_ref, TOL[dtype])
    check("S_out", S_out, S_ref, TOL[dtype])


@pytest.mark.parametrize("d,Tk", [(128, 4), (128, 3), (64, 4)])
def test_decode_tokens_equals_single_steps(d, Tk):
    import linear_attention_kda_amd as kda
    announce(f"decode_tokens vs single steps, N=6 Tk={Tk} H=2 d={d} bf16")
    N, H = 6, 2
    inp = _inputs(N, Tk, H, d, torch.bfloat16, "channel", seed=22)
    S_step = inp["S0"].clone()
    outs = []
    for t in range(Tk):
        outs.append(kda.decode_step(inp["q"][:, t].contiguous(), inp["k"][:, t].contiguous(),
                                    inp["v"][:, t].contiguous(), inp["alpha"][:, t].contiguous(),
                                    inp["beta"][:, t].contiguous(), S_step))
    S_multi = inp["S0"].clone()
    o, S2 = kda.decode_tokens(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], S_multi,
                              S_out=S_multi)                   # in place
    torch.cuda.synchronize()
    assert S2.data_ptr() == S_multi.data_ptr()
    assert torch.equal(torch.stack(outs, 1), o)
    assert torch.equal(S_step, S_multi)


def test_decode_tokens_zero_tokens_copies_state():
    import linear_attention_kda_amd as kda
    announce("decode_tokens Tk=0")
    inp = _inputs(3, 1, 2, 64, torch.float32, "channel", seed=23)
    q = inp["q"][:, :0].contiguous()
    o, S_out = kda.decode_tokens(q, q, q, q, inp["beta"][:, :0].contiguous(), inp["S0"])
    torch.cuda.synchronize()
    assert o.shape == (3, 0, 2, 64)
    assert torch.equal(S_out, inp["S0"])


@pytest.mark.parametrize("dk,dv,Tk", [(32, 64, 5), (64, 16, 4), (128, 32, 2), (128, 64, 3), (16, 128, 7)])
def test_decode_tokens_head_sizes(dk, dv, Tk):
    import linear_attention_kda_amd as kda
    announce(f"decode_tokens N=3 Tk={Tk} H=2 dk={dk} dv={dv} bf16")
    inp = to_dev(inputs.dense(3, Tk, 2, dk, dv, torch.bfloat16, gate="uniform", alpha_lo=0.9, s0_std=0.05,
                              seed=24 + dk + dv))
    o, S_out = kda.decode_tokens(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["S0"])
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_prefill(inp)
    check("o", o, o_ref, TOL[torch.bfloat16])
    check("S_out", S_out, S_ref, TOL[torch.bfloat16])
