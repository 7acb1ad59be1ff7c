"""Input activations applied on load (kda_input_act) and gates given as
softplus logits (KDA_GATE_SOFTPLUS_*): q, k <- SiLU then unit length per
token and head, beta <- sigmoid, alpha = exp(-softplus(g)), the forms of the
delta-rule block's model code (page "22580: from GPT-2 to Kimi K3,
explained", section "DeltaNet, or Fast Weight Programmers") and of the
prefill workload's gate.  The oracle receives the activated inputs,
computed here in float64 from the same raw values."""
import pytest
import torch

from linear_attention_kda_amd import inputs
from tests.gpu_cases import TOL, announce, check, oracle_prefill, to_dev

pytestmark = pytest.mark.gpu

QK, BETA = 1, 2


def _raw(inp, seed, act=QK | BETA):
    """Raw (pre-activation) q, k and beta logits, for the activations in
    `act`, in place of the generator's activated ones (without the q, k
    activation, k stays a unit vector: a raw k of norm ~sqrt(d_k) makes the
    recurrence blow up).  The gate is left as drawn."""
    g = torch.Generator().manual_seed(seed)
    out = dict(inp)
    if act & QK:
        for n in ("q", "k"):
            x = torch.randn(inp[n].shape, generator=g)
            out[n] = x.to(inp[n].dtype).to(inp[n].device)
    if act & BETA:
        out["beta"] = torch.randn(inp["beta"].shape, generator=g).to(inp["beta"].device)
    return out


def _activated(inp, act, gate_form, dk):
    """The oracle's inputs: activations and the gate in float64."""
    out = dict(inp)
    silu = lambda x: x * torch.sigmoid(x)
    if act & QK:
        for n in ("q", "k"):
            x = silu(inp[n].detach().cpu().double())
            out[n] = x / x.norm(dim=-1, keepdim=True).clamp_min(1e-12)
    if act & BETA:
        out["beta"] = torch.sigmoid(inp["beta"].detach().cpu().double())
    a = inp["alpha"].detach().cpu().double()
    if gate_form.startswith("softplus"):
        a = torch.exp(-torch.nn.functional.softplus(a))
    lead = inp["q"].shape[:-1]
    out["alpha"] = a if a.dim() == len(lead) + 1 else a.unsqueeze(-1).expand(*lead, dk).contiguous()
    return out


def _run(inp, gate, act):
    import linear_attention_kda_amd as kda
    o, S = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], S0=inp.get("S0"),
                         cu_seqlens=inp.get("cu_seqlens"), gate=gate, act=act)
    torch.cuda.synchronize()
    return o, S


@pytest.mark.parametrize("act,gate_form", [(QK | BETA, "softplus_channel"), (QK, "channel"),
                                           (BETA, "softplus_scalar"), (0, "softplus_channel"),
                                           (QK | BETA, "scalar")])
@pytest.mark.parametrize("dtype,dk,T,H,B", [(torch.float32, 32, 130, 3, 2), (torch.bfloat16, 128, 150, 4, 2),
                                            (torch.bfloat16, 64, 63, 2, 1), (torch.float32, 16, 64, 2, 1)])
def test_dense_fused_inputs(act, gate_form, dtype, dk, T, H, B):
    announce(f"fused inputs act={act} gate {gate_form} dense B={B} T={T} H={H} d={dk} {dtype}")
    inp = _raw(to_dev(inputs.dense(B, T, H, dk, dk, dtype, s0_std=0.02, seed=51, gate_form=gate_form)), 51, act)
    o, S = _run(inp, gate_form, act)
    o_ref, S_ref = oracle_prefill(_activated(inp, act, gate_form, dk))
    check("o", o, o_ref, TOL[dtype])
    check("S_final", S, S_ref, TOL[dtype])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_fused_inputs_exact_path(dtype):
    # large softplus logits: gates near 0 push a chunk's decay product below
    # the factorisation's range, so the prep kernel's exact path (which reads
    # q and k again) must apply the activation too
    announce(f"fused inputs with strong decay (exact path), d=128 {dtype}")
    inp = _raw(to_dev(inputs.dense(1, 200, 2, 128, 128, dtype, s0_std=0.02, seed=52,
                                   gate_form="softplus_channel")), 52)
    g = inp["alpha"].clone()
    g[0, 100:164] = 3.0               # alpha = 1 / (1 + e^3) ~ 0.047 for a whole chunk
    g[0, 10, 1, :] = 80.0             # alpha = 0 in fp32
    inp["alpha"] = g
    o, S = _run(inp, "softplus_channel", QK | BETA)
    o_ref, S_ref = oracle_prefill(_activated(inp, QK | BETA, "softplus_channel", 128))
    check("o", o, o_ref, TOL[dtype])
    check("S_final", S, S_ref, TOL[dtype])


def test_packed_fused_inputs():
    announce("fused inputs, packed ragged batch with a zero-length sequence, d=128 bf16")
    inp = to_dev(inputs.packed([70, 0, 5, 200], 3, 128, 128, torch.bfloat16, s0_std=0.02, seed=53,
                               gate_form="softplus_channel"))
    inp = _raw(inp, 53)
    o, S = _run(inp, "softplus_channel", QK | BETA)
    o_ref, S_ref = oracle_prefill(_activated(inp, QK | BETA, "softplus_channel", 128))
    check("o", o, o_ref, TOL[torch.bfloat16], cu=inp["cu_seqlens"])
    check("S_final", S, S_ref, TOL[torch.bfloat16])


@pytest.mark.parametrize("gate_form", ["softplus_channel", "softplus_scalar"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_decode_fused_inputs(gate_form, dtype):
    import linear_attention_kda_amd as kda
    import oracle
    announce(f"decode with fused inputs, gate {gate_form}, N=5 H=3 d=128 {dtype}")
    N, H, D = 5, 3, 128
    S = inputs.decode_state(N, H, D, D, 0.02, seed=54, device="cuda")
    d = _raw(to_dev(inputs.dense(N, 3, H, D, D, dtype, gate="uniform", alpha_lo=0.95, seed=54,
                                 gate_form=gate_form)), 54)
    S_in = S.clone()
    o3, S3 = kda.decode_tokens(d["q"], d["k"], d["v"], d["alpha"], d["beta"], S_in, gate=gate_form,
                               act=QK | BETA)
    torch.cuda.synchronize()
    ref = _activated(d, QK | BETA, gate_form, D)
    ref["S0"] = S_in
    o3_ref, S3_ref = oracle_prefill(ref)
    check("o tokens", o3, o3_ref, TOL[dtype])
    check("S tokens", S3, S3_ref, TOL[dtype])
    # one step through decode_step
    S1 = S.clone()
    a1 = d["alpha"][:, 0].contiguous()
    o1 = kda.decode_step(d["q"][:, 0].contiguous(), d["k"][:, 0].contiguous(), d["v"][:, 0].contiguous(), a1,
                         d["beta"][:, 0].contiguous(), S1, gate=gate_form, act=QK | BETA)
    torch.cuda.synchronize()
    r1 = {n: ref[n][:, 0].contiguous() for n in ("q", "k", "v", "alpha", "beta")}
    o1_ref, S1_ref = oracle.decode(r1["q"], r1["k"], r1["v"], r1["alpha"], r1["beta"], S.double().cpu().numpy())
    check("o step", o1, o1_ref, TOL[dtype])
    check("S step", S1, S1_ref, TOL[dtype])


@pytest.mark.parametrize("dk,dv", [(64, 32), (32, 128), (128, 16)])
def test_fused_inputs_head_sizes(dk, dv):
    announce(f"fused inputs dense B=2 T=100 H=2 dk={dk} dv={dv} bf16")
    inp = _raw(to_dev(inputs.dense(2, 100, 2, dk, dv, torch.bfloat16, s0_std=0.02, seed=55 + dk,
                                   gate_form="softplus_channel")), 55 + dk)
    o, S = _run(inp, "softplus_channel", QK | BETA)
    o_ref, S_ref = oracle_prefill(_activated(inp, QK | BETA, "softplus_channel", dk))
    check("o", o, o_ref, TOL[torch.bfloat16])
    check("S_final", S, S_ref, TOL[torch.bfloat16])
