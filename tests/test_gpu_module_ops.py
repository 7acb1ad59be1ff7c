"""The operations around the method fused into the prefill
(kda_chunk_fwd_module): the short causal convolution of q, k and v, and the
output RMS norm and gate (page "K3 架构图解", chapter 08 figure caption:
the KDA module holds a short convolution, a normalisation and an output
gate; chapter 05: the RMS norm; chapter 09: the convolution is causal).
The reference runs the block's steps in float64 in the test
(tests/module_ref.py), hands the activated inputs to the oracle, and applies
the norm and gate to the oracle's outputs."""
import pytest
import torch

from linear_attention_kda_amd import inputs
from tests import module_ref as mr
from tests.gpu_cases import TOL, announce, check, oracle_prefill, to_dev

pytestmark = pytest.mark.gpu

QK, BETA = 1, 2


def _raw_block(inp, seed):
    """Raw (pre-convolution, pre-activation) q, k, v and beta logits in
    place of the generator's activated ones; the gate as drawn."""
    g = torch.Generator().manual_seed(seed)
    out = dict(inp)
    for n in ("q", "k", "v"):
        out[n] = torch.randn(inp[n].shape, generator=g).to(inp[n].dtype).to(inp[n].device)
    out["beta"] = torch.randn(inp["beta"].shape, generator=g).to(inp["beta"].device)
    return out


def _weights(H, dk, dv, dtype, o_shape, seed, conv=True, norm=True, gate=True):
    g = torch.Generator().manual_seed(seed + 1000)
    w = {}
    if conv:
        w["conv"] = tuple((torch.randn(H, d, 4, generator=g) * 0.6).cuda() for d in (dk, dk, dv))
    if norm:
        w["norm_weight"] = (1.0 + 0.2 * torch.randn(dv, generator=g)).cuda()
        w["norm_eps"] = 1e-5
    if gate:
        w["out_gate"] = torch.randn(o_shape, generator=g).to(dtype).cuda()
    return w


def _reference(inp, w, gate_form, dk):
    cu = inp.get("cu_seqlens")
    ref = dict(inp)
    if "conv" in w:
        wq, wk, wv = w["conv"]
        q, k, v = (mr.short_conv(inp[n], wt, cu) for n, wt in (("q", wq), ("k", wk), ("v", wv)))
    else:
        q, k, v = inp["q"], inp["k"], inp["v"]
    ref["q"], ref["k"], ref["v"] = mr.silu_unit(q), mr.silu_unit(k), v.detach().cpu().double()
    ref["beta"] = torch.sigmoid(inp["beta"].detach().cpu().double())
    a = inp["alpha"].detach().cpu().double()
    if gate_form.startswith("softplus"):
        a = torch.exp(-torch.nn.functional.softplus(a))
    lead = inp["q"].shape[:-1]
    ref["alpha"] = a if a.dim() == len(lead) + 1 else a.unsqueeze(-1).expand(*lead, dk).contiguous()
    o_ref, S_ref = oracle_prefill(ref)
    o_ref = torch.as_tensor(o_ref)
    if "norm_weight" in w:
        o_ref = mr.rms_norm(o_ref, w["norm_weight"], w["norm_eps"])
    if "out_gate" in w:
        o_ref = mr.out_gate(o_ref, w["out_gate"])
    return o_ref.numpy(), S_ref


def _run(inp, gate_form, w, out=None):
    import linear_attention_kda_amd as kda
    o, S = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], S0=inp.get("S0"),
                         cu_seqlens=inp.get("cu_seqlens"), gate=gate_form, act=QK | BETA, out=out, **w)
    torch.cuda.synchronize()
    return o, S


@pytest.mark.parametrize("ops", ["conv", "norm_gate", "all"])
@pytest.mark.parametrize("dtype,dk,dv,T,H,B", [(torch.bfloat16, 128, 128, 200, 3, 2),
                                               (torch.float32, 32, 32, 130, 2, 2),
                                               (torch.bfloat16, 64, 32, 70, 2, 1),
                                               (torch.float32, 16, 128, 65, 2, 1)])
def test_dense_module_ops(ops, dtype, dk, dv, T, H, B):
    announce(f"module ops {ops} dense B={B} T={T} H={H} dk={dk} dv={dv} {dtype}")
    seed = 61 + dk + T
    inp = _raw_block(to_dev(inputs.dense(B, T, H, dk, dv, dtype, s0_std=0.02, seed=seed,
                                         gate_form="softplus_channel")), seed)
    w = _weights(H, dk, dv, dtype, inp["v"].shape, seed, conv=ops in ("conv", "all"),
                 norm=ops in ("norm_gate", "all"), gate=ops in ("norm_gate", "all"))
    o, S = _run(inp, "softplus_channel", w)
    o_ref, S_ref = _reference(inp, w, "softplus_channel", dk)
    check("o", o, o_ref, TOL[dtype])
    check("S_final", S, S_ref, TOL[dtype])


def test_packed_module_ops_short_sequences():
    # sequences shorter than the convolution's reach, an empty one, and one
    # spanning several chunks: every sequence start zeroes the window
    announce("module ops, packed [70, 0, 2, 1, 5, 200, 3], d=128 bf16")
    inp = to_dev(inputs.packed([70, 0, 2, 1, 5, 200, 3], 3, 128, 128, torch.bfloat16, s0_std=0.02, seed=62,
                               gate_form="softplus_channel"))
    inp = _raw_block(inp, 62)
    w = _weights(3, 128, 128, torch.bfloat16, inp["v"].shape, 62)
    o, S = _run(inp, "softplus_channel", w)
    o_ref, S_ref = _reference(inp, w, "softplus_channel", 128)
    check("o", o, o_ref, TOL[torch.bfloat16], cu=inp["cu_seqlens"])
    check("S_final", S, S_ref, TOL[torch.bfloat16])


def test_packed_rows_outside_sequences_untouched():
    # the offsets end before the last tokens: those rows of o keep what the
    # caller put there (the norm and gate pass skips them too)
    announce("module ops, packed with trailing tokens outside every sequence, d=64 fp32")
    full = to_dev(inputs.packed([40, 90, 33], 2, 64, 64, torch.float32, s0_std=0.02, seed=63,
                                gate_form="softplus_channel"))
    full = _raw_block(full, 63)
    inp = dict(full)
    inp["cu_seqlens"] = full["cu_seqlens"][:3].contiguous()   # sequences 0 and 1 only
    inp["S0"] = full["S0"][:2].contiguous()
    w = _weights(2, 64, 64, torch.float32, inp["v"].shape, 63)
    out = torch.full(inp["v"].shape, 7.25, dtype=torch.float32, device="cuda")
    o, S = _run(inp, "softplus_channel", w, out=out)
    assert torch.all(o[130:] == 7.25)
    ref_in = dict(inp)
    for n in ("q", "k", "v", "alpha", "beta"):
        ref_in[n] = full[n][:130]
    ref_in["cu_seqlens"] = inp["cu_seqlens"]
    w_ref = dict(w)
    w_ref["out_gate"] = w["out_gate"][:130]
    o_ref, S_ref = _reference(ref_in, w_ref, "softplus_channel", 64)
    check("o", o[:130], o_ref, TOL[torch.float32], cu=inp["cu_seqlens"])
    check("S_final", S, S_ref, TOL[torch.float32])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_module_conv_exact_path(dtype):
    # strong decay on one chunk sends it down the prep's exact path, which
    # reads q and k again and must convolve them the same way
    announce(f"module ops with strong decay (exact path), d=128 {dtype}")
    inp = _raw_block(to_dev(inputs.dense(1, 200, 2, 128, 128, dtype, s0_std=0.02, seed=64,
                                         gate_form="softplus_channel")), 64)
    g = inp["alpha"].clone()
    g[0, 100:164] = 3.0
    g[0, 10, 1, :] = 80.0
    inp["alpha"] = g
    w = _weights(2, 128, 128, dtype, inp["v"].shape, 64)
    o, S = _run(inp, "softplus_channel", w)
    o_ref, S_ref = _reference(inp, w, "softplus_channel", 128)
    check("o", o, o_ref, TOL[dtype])
    check("S_final", S, S_ref, TOL[dtype])


def test_module_norm_gate_with_overlapped_schedule():
    # the norm and gate also follow the overlapped schedule's join (the
    # convolution does not take that schedule)
    import linear_attention_kda_amd as kda
    announce("norm + gate after the overlapped schedule, B=2 T=300 H=4 d=128 bf16")
    inp = _raw_block(to_dev(inputs.dense(2, 300, 4, 128, 128, torch.bfloat16, s0_std=0.02, seed=65,
                                         gate_form="softplus_channel")), 65)
    w = _weights(4, 128, 128, torch.bfloat16, inp["v"].shape, 65, conv=False)
    prev = kda.set_schedule("overlap")
    try:
        ws = torch.empty(kda.chunk_fwd_workspace_size(2, 300, 4, 128, 128), dtype=torch.uint8, device="cuda")
        o, S = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], S0=inp["S0"],
                             gate="softplus_channel", act=QK | BETA, workspace=ws, **w)
        torch.cuda.synchronize()
        sched, errs = kda.chunk_fwd_status(ws)
    finally:
        kda.set_schedule(prev)
    assert sched == "overlap" and errs == 0
    o_ref, S_ref = _reference(inp, w, "softplus_channel", 128)
    check("o", o, o_ref, TOL[torch.bfloat16])
    check("S_final", S, S_ref, TOL[torch.bfloat16])


def test_module_conv_runs_two_phase():
    import linear_attention_kda_amd as kda
    announce("convolution under a requested overlapped schedule runs two-phase, d=128 bf16")
    inp = _raw_block(to_dev(inputs.dense(1, 130, 2, 128, 128, torch.bfloat16, s0_std=0.02, seed=66,
                                         gate_form="softplus_channel")), 66)
    w = _weights(2, 128, 128, torch.bfloat16, inp["v"].shape, 66)
    prev = kda.set_schedule("overlap")
    try:
        ws = torch.empty(kda.chunk_fwd_workspace_size(1, 130, 2, 128, 128), dtype=torch.uint8, device="cuda")
        o, S = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], S0=inp["S0"],
                             gate="softplus_channel", act=QK | BETA, workspace=ws, **w)
        torch.cuda.synchronize()
        sched, errs = kda.chunk_fwd_status(ws)
    finally:
        kda.set_schedule(prev)
    assert sched == "two_phase" and errs == 0
    o_ref, S_ref = _reference(inp, w, "softplus_channel", 128)
    check("o", o, o_ref, TOL[torch.bfloat16])
    check("S_final", S, S_ref, TOL[torch.bfloat16])


def test_module_ops_in_graph_capture():
    # the convolution, the norm and gate and the final convolution state in a
    # captured call: replays with new inputs copied in match eager calls bitwise
    import linear_attention_kda_amd as kda
    announce("module ops under graph capture: 3 replays vs eager, B=2 T=150 H=2 d=128 bf16")
    B, T, H, D = 2, 150, 2, 128
    static = _raw_block(to_dev(inputs.dense(B, T, H, D, D, torch.bfloat16, s0_std=0.02, seed=67,
                                            gate_form="softplus_channel")), 67)
    w = _weights(H, D, D, torch.bfloat16, static["v"].shape, 67)
    ws = torch.empty(kda.chunk_fwd_workspace_size(B, T, H, D, D), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(static["v"])
    S = torch.empty((B, H, D, D), dtype=torch.float32, device="cuda")
    cs = torch.empty((B, H, 3, 3 * D), dtype=torch.bfloat16, device="cuda")

    def call(inp, out, S_out, state):
        kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], S0=inp["S0"], gate="softplus_channel",
                      act=QK | BETA, out=out, S_final=S_out, workspace=ws, conv_state=state, **w)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(static, o, S, cs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(static, o, S, cs)
    torch.cuda.synchronize()
    for seed in (68, 69, 70):
        new = _raw_block(to_dev(inputs.dense(B, T, H, D, D, torch.bfloat16, s0_std=0.02, seed=seed,
                                             gate_form="softplus_channel")), seed)
        for name in ("q", "k", "v", "alpha", "beta", "S0"):
            static[name].copy_(new[name])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        o_g, S_g, cs_g = o.clone(), S.clone(), cs.clone()
        o_e, S_e, cs_e = torch.empty_like(o), torch.empty_like(S), torch.empty_like(cs)
        call(new, o_e, S_e, cs_e)
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e) and torch.equal(S_g, S_e) and torch.equal(cs_g, cs_e)
