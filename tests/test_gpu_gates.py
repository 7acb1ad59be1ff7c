"""Gate forms on the GPU path: one gate per (token, head) shared by all key
channels (Gated DeltaNet) and no gate (DeltaNet), page "Kimi Delta Attention
(KDA)", sections "Gated DeltaNet: ..." and "DeltaNet: ...".  Both are the
per-channel recurrence with the gate broadcast over the channels (or set to
1), which is how the fp64 oracle receives them; the GPU results must also be
bitwise equal to the per-channel entry point fed the broadcast gates."""
import pytest
import torch

from linear_attention_kda_amd import inputs
from tests.gpu_cases import TOL, announce, check, oracle_prefill, to_dev

pytestmark = pytest.mark.gpu


def _expand(inp, dk):
    """The same inputs with alpha as an explicit per-channel tensor."""
    out = dict(inp)
    a = inp["alpha"]
    lead = inp["q"].shape[:-1]
    out["alpha"] = (torch.ones(*lead, dk, dtype=torch.float32, device=inp["q"].device) if a is None
                    else a.unsqueeze(-1).expand(*lead, dk).contiguous())
    return out


def _run(inp, gate):
    import linear_attention_kda_amd as kda
    o, S = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], S0=inp.get("S0"),
                         cu_seqlens=inp.get("cu_seqlens"), gate=gate)
    torch.cuda.synchronize()
    return o, S


@pytest.mark.parametrize("form", ["scalar", "none"])
@pytest.mark.parametrize("dtype,dk,T,H,B,s0", [
    (torch.float32, 16, 64, 2, 1, None),
    (torch.float32, 32, 130, 3, 2, 0.02),
    (torch.bfloat16, 128, 150, 4, 2, 0.02),
    (torch.bfloat16, 64, 63, 2, 1, None),
])
def test_dense_gate_forms(form, dtype, dk, T, H, B, s0):
    announce(f"gate form {form} dense B={B} T={T} H={H} d={dk} {dtype}")
    inp = to_dev(inputs.dense(B, T, H, dk, dk, dtype, s0_std=s0, seed=11, gate_form=form))
    o, S = _run(inp, form)
    full = _expand(inp, dk)
    o_ref, S_ref = oracle_prefill(full)
    check("o", o, o_ref, TOL[dtype])
    check("S_final", S, S_ref, TOL[dtype])
    # the per-channel entry point on the broadcast gates does the same arithmetic
    o2, S2 = _run(full, "channel")
    assert torch.equal(o, o2) and torch.equal(S, S2)


def test_packed_scalar_gates():
    announce("gate form scalar, packed ragged batch with a zero-length sequence, d=64 bf16")
    lengths = [70, 0, 5, 130]
    inp = to_dev(inputs.packed(lengths, 3, 64, 64, torch.bfloat16, s0_std=0.02, seed=12,
                               gate_form="scalar"))
    o, S = _run(inp, "scalar")
    full = _expand(inp, 64)
    o_ref, S_ref = oracle_prefill(full)
    check("o", o, o_ref, TOL[torch.bfloat16], cu=inp["cu_seqlens"])
    check("S_final", S, S_ref, TOL[torch.bfloat16])


def test_scalar_gate_zero_takes_exact_path():
    # a gate of exactly 0 clears the memory; the chunk's decay product is then
    # below the factorisation's range and the exact path runs
    announce("gate form scalar with zeros and strong decay, d=128 bf16 and fp32")
    for dtype, tol in ((torch.bfloat16, TOL[torch.bfloat16]), (torch.float32, TOL[torch.float32])):
        inp = to_dev(inputs.dense(1, 200, 2, 128, 128, dtype, s0_std=0.02, seed=13, gate_form="scalar"))
        a = inp["alpha"].clone()
        a[0, 10] = 0.0
        a[0, 100:164] = 0.05
        inp["alpha"] = a
        o, S = _run(inp, "scalar")
        o_ref, S_ref = oracle_prefill(_expand(inp, 128))
        check("o", o, o_ref, tol)
        check("S_final", S, S_ref, tol)


@pytest.mark.parametrize("form", ["scalar", "none"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_decode_gate_forms(form, dtype):
    import linear_attention_kda_amd as kda
    import oracle
    announce(f"decode gate form {form} N=5 H=3 d=128 {dtype}")
    N, H, D = 5, 3, 128
    S = inputs.decode_state(N, H, D, D, 0.02, seed=14, device="cuda")
    tok = inputs.decode_token(N, H, D, D, dtype, 0.95, step=0, seed=14, device="cuda")
    if form == "scalar":
        tok["alpha"] = tok["alpha"][..., 0].contiguous()
    else:
        tok["alpha"] = None
    S_ref = S.double().cpu().numpy()
    S_chan = S.clone()
    o = kda.decode_step(tok["q"], tok["k"], tok["v"], tok["alpha"], tok["beta"], S, gate=form)
    full = _expand(tok, D)
    o2 = kda.decode_step(full["q"], full["k"], full["v"], full["alpha"], full["beta"], S_chan,
                         gate="channel")
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.decode(*(full[n].cpu() for n in ("q", "k", "v", "alpha", "beta")), S_ref)
    check("o", o, o_ref, TOL[dtype])
    check("S", S, S_ref, TOL[dtype])
    assert torch.equal(o, o2) and torch.equal(S, S_chan)
