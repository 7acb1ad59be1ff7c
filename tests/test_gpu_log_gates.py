"""Gates given as logarithms (kda_gate's log forms): page "Kimi Delta
Attention (KDA)", section "Two schedules of computation for one recurrence",
describes the production pipeline working with log decays.  The kernels take
exp on load; the oracle receives alpha = exp(g) computed in float64 from the
same fp32 values g, so a result must match the oracle at the usual tolerance.
g = -inf is a gate of exactly 0 (memory cleared), which takes the prep
kernel's exact path."""
import pytest
import torch

from linear_attention_kda_amd import inputs
from tests.gpu_cases import TOL, announce, check, oracle_prefill, to_dev

pytestmark = pytest.mark.gpu


def _linear(inp, dk):
    """The oracle's inputs: alpha = exp(g) in float64, broadcast per channel."""
    out = dict(inp)
    a = torch.exp(inp["alpha"].detach().cpu().double())
    lead = inp["q"].shape[:-1]
    out["alpha"] = a if a.dim() == len(lead) + 1 else a.unsqueeze(-1).expand(*lead, dk).contiguous()
    return out


def _run(inp, gate):
    import linear_attention_kda_amd as kda
    o, S = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], S0=inp.get("S0"),
                         cu_seqlens=inp.get("cu_seqlens"), gate=gate)
    torch.cuda.synchronize()
    return o, S


@pytest.mark.parametrize("form", ["log_channel", "log_scalar"])
@pytest.mark.parametrize("dtype,dk,T,H,B,s0", [
    (torch.float32, 16, 64, 2, 1, None),
    (torch.float32, 32, 130, 3, 2, 0.02),
    (torch.bfloat16, 128, 150, 4, 2, 0.02),
    (torch.bfloat16, 64, 63, 2, 1, None),
])
def test_dense_log_gates(form, dtype, dk, T, H, B, s0):
    announce(f"gate form {form} dense B={B} T={T} H={H} d={dk} {dtype}")
    inp = to_dev(inputs.dense(B, T, H, dk, dk, dtype, s0_std=s0, seed=31, gate_form=form))
    assert float(inp["alpha"].max()) <= 0.0
    o, S = _run(inp, form)
    o_ref, S_ref = oracle_prefill(_linear(inp, dk))
    check("o", o, o_ref, TOL[dtype])
    check("S_final", S, S_ref, TOL[dtype])
    # the linear form of the same gates (rounded to fp32) agrees closely too
    lin = dict(inp)
    lin["alpha"] = torch.exp(inp["alpha"])
    o2, S2 = _run(lin, form[4:])
    check("o vs linear form", o, o2.double().cpu().numpy(), TOL[dtype])


def test_packed_log_channel_gates():
    announce("gate form log_channel, packed ragged batch with a zero-length sequence, d=128 bf16")
    lengths = [70, 0, 5, 200]
    inp = to_dev(inputs.packed(lengths, 3, 128, 128, torch.bfloat16, s0_std=0.02, seed=32,
                               gate_form="log_channel"))
    o, S = _run(inp, "log_channel")
    o_ref, S_ref = oracle_prefill(_linear(inp, 128))
    check("o", o, o_ref, TOL[torch.bfloat16], cu=inp["cu_seqlens"])
    check("S_final", S, S_ref, TOL[torch.bfloat16])


@pytest.mark.parametrize("form", ["log_channel", "log_scalar"])
def test_log_gate_minus_infinity_clears_memory(form):
    announce(f"gate form {form} with -inf gates, d=128 fp32")
    inp = to_dev(inputs.dense(1, 200, 2, 128, 128, torch.float32, s0_std=0.02, seed=33, gate_form=form))
    g = inp["alpha"].clone()
    g[0, 10] = float("-inf")          # every channel (or the token's one gate)
    g[0, 100:164] = -3.0               # strong decay: a chunk product below 2^-100
    inp["alpha"] = g
    o, S = _run(inp, form)
    o_ref, S_ref = oracle_prefill(_linear(inp, 128))
    check("o", o, o_ref, TOL[torch.float32])
    check("S_final", S, S_ref, TOL[torch.float32])


@pytest.mark.parametrize("form", ["log_channel", "log_scalar"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_decode_log_gates(form, dtype):
    import linear_attention_kda_amd as kda
    import oracle
    announce(f"decode gate form {form} N=5 H=3 d=128 {dtype}, one step and 3 tokens per launch")
    N, H, D = 5, 3, 128
    S = inputs.decode_state(N, H, D, D, 0.02, seed=34, device="cuda")
    tok = inputs.decode_token(N, H, D, D, dtype, 0.95, step=0, seed=34, device="cuda")
    g = torch.log(tok["alpha"])
    tok["alpha"] = g if form == "log_channel" else g[..., 0].contiguous()
    S_np = S.double().cpu().numpy()
    o = kda.decode_step(tok["q"], tok["k"], tok["v"], tok["alpha"], tok["beta"], S, gate=form)
    torch.cuda.synchronize()
    lin = _linear(tok, D)
    o_ref, S_ref = oracle.decode(*(lin[n].cpu() for n in ("q", "k", "v", "alpha", "beta")), S_np)
    check("o", o, o_ref, TOL[dtype])
    check("S", S, S_ref, TOL[dtype])
    # three tokens per launch from the updated state
    d = to_dev(inputs.dense(N, 3, H, D, D, dtype, gate="uniform", alpha_lo=0.95, seed=35, gate_form=form))
    S_in = S.clone()
    o3, S3 = kda.decode_tokens(d["q"], d["k"], d["v"], d["alpha"], d["beta"], S_in, gate=form)
    torch.cuda.synchronize()
    ref = _linear(d, D)
    ref["S0"] = S_in
    o3_ref, S3_ref = oracle_prefill(ref)
    check("o tokens", o3, o3_ref, TOL[dtype])
    check("S tokens", S3, S3_ref, TOL[dtype])
