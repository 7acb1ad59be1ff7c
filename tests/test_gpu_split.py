"""Split-sequence prefill (KDA_SCHEDULE_SPLIT) on the GPU.  Each sequence is
cut into segments of whole chunks; the affine maps of the state over all
segments but the last (page "Kimi Delta Attention (KDA)": the state has a
fixed size and each step is linear in it, which is what makes long contexts
tractable) are chained into every segment's start state, and the scan runs
all segments at once.  The results equal the sequential scan's up to
rounding (the start states come from the maps), so each case is checked
against the fp64 oracle per unit, and against the two-phase schedule's
result on the same device."""
import pytest
import torch

from linear_attention_kda_amd import inputs
from tests.gpu_cases import TOL, announce, check, oracle_prefill, rel, to_dev

pytestmark = pytest.mark.gpu


def _run(inp, schedule, ws, **kw):
    import linear_attention_kda_amd as kda
    prev = kda.set_schedule(schedule)
    try:
        o, S = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], S0=inp.get("S0"),
                             workspace=ws, **kw)
        torch.cuda.synchronize()
        status = kda.chunk_fwd_status(ws)
    finally:
        kda.set_schedule(prev)
    return o, S, status


def _workspace(B, T, H):
    import linear_attention_kda_amd as kda
    n = kda.chunk_fwd_workspace_size(B, T, H, 128, 128, -1, kda.KDA_BF16)
    return torch.zeros(n, dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("B,T,H,s0", [
    (1, 3000, 2, 0.02),   # 47 chunks: three segments of 16, 16 and 15 (a ragged last chunk)
    (2, 2560, 3, None),   # 40 chunks: two segments of 20, six units
    (1, 4096, 1, 0.02),   # one unit, four segments of 16
])
def test_split_matches_oracle_and_two_phase(B, T, H, s0):
    announce(f"split-sequence vs oracle and two-phase, dense bf16 d=128 B={B} T={T} H={H} S0={s0}")
    inp = to_dev(inputs.dense(B, T, H, 128, 128, torch.bfloat16, s0_std=s0, seed=71 + T))
    ws = _workspace(B, T, H)
    o, S, st = _run(inp, "split", ws)
    assert st == ("split", 0)
    o_ref, S_ref = oracle_prefill(inp)
    check("o", o, o_ref, TOL[torch.bfloat16])
    check("S_final", S, S_ref, TOL[torch.bfloat16])
    o2, S2, st2 = _run(inp, "two_phase", ws)
    assert st2 == ("two_phase", 0)
    # the same chunks and records; only the segment start states differ by rounding
    assert rel(o, o2.double().cpu().numpy()) < 5e-3
    assert rel(S, S2.double().cpu().numpy()) < 5e-3


def test_split_in_place_state_and_strong_decay():
    # S_final written over S0; gates of 0 send chunks down the prep's exact path
    announce("split-sequence with S_final == S0 and gates of 0, B=1 T=3000 H=2")
    inp = to_dev(inputs.dense(1, 3000, 2, 128, 128, torch.bfloat16, s0_std=0.02, seed=72))
    a = inp["alpha"].clone()
    a[0, 1500:1600] = 0.05
    a[0, 2100, 1, :] = 0.0
    inp["alpha"] = a
    S0 = inp["S0"].clone()
    ref = dict(inp, S0=S0.clone())
    ws = _workspace(1, 3000, 2)
    import linear_attention_kda_amd as kda
    prev = kda.set_schedule("split")
    try:
        o, S = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], S0=S0, S_final=S0,
                             workspace=ws)
        torch.cuda.synchronize()
        assert kda.chunk_fwd_status(ws) == ("split", 0)
    finally:
        kda.set_schedule(prev)
    assert S.data_ptr() == S0.data_ptr()
    o_ref, S_ref = oracle_prefill(ref)
    check("o", o, o_ref, TOL[torch.bfloat16])
    check("S_final", S, S_ref, TOL[torch.bfloat16])


def test_split_with_module_ops():
    # the convolution's v (left in o by the prep) feeds the maps and the scan
    from tests.test_gpu_module_ops import _raw_block, _reference, _weights
    announce("split-sequence with the short convolution and norm + gate, B=1 T=2100 H=2")
    inp = _raw_block(to_dev(inputs.dense(1, 2100, 2, 128, 128, torch.bfloat16, s0_std=0.02, seed=73,
                                         gate_form="softplus_channel")), 73)
    w = _weights(2, 128, 128, torch.bfloat16, inp["v"].shape, 73)
    ws = _workspace(1, 2100, 2)
    o, S, st = _run(inp, "split", ws, gate="softplus_channel", act=3, **w)
    assert st == ("split", 0)
    o_ref, S_ref = _reference(inp, w, "softplus_channel", 128)
    check("o", o, o_ref, TOL[torch.bfloat16])
    check("S_final", S, S_ref, TOL[torch.bfloat16])


def test_split_not_supported_runs_other_schedule():
    # a shape the split cannot serve (too few chunks for two segments of 16)
    announce("split requested on B=1 T=1000 H=2: runs two-phase")
    inp = to_dev(inputs.dense(1, 1000, 2, 128, 128, torch.bfloat16, s0_std=0.02, seed=74))
    ws = _workspace(1, 1000, 2)
    o, S, st = _run(inp, "split", ws)
    assert st == ("two_phase", 0)
    o_ref, S_ref = oracle_prefill(inp)
    check("o", o, o_ref, TOL[torch.bfloat16])


def test_auto_takes_split_for_few_long_heads():
    # B=1, H=8, T=65536: the automatic schedule splits; sampled heads against
    # the oracle, all heads against two-phase
    announce("auto schedule on B=1 H=8 T=65536 d=128 bf16: split expected; heads 0 and 5 vs oracle")
    inp = to_dev(inputs.dense(1, 65536, 8, 128, 128, torch.bfloat16, s0_std=0.02, seed=75))
    ws = _workspace(1, 65536, 8)
    o, S, st = _run(inp, "auto", ws)
    assert st == ("split", 0)
    heads = [0, 5]
    o_ref, S_ref = oracle_prefill(inp, heads=heads)
    check("o", o[:, :, heads], o_ref, TOL[torch.bfloat16])
    check("S_final", S[:, heads], S_ref, TOL[torch.bfloat16])
    o2, S2, st2 = _run(inp, "two_phase", ws)
    assert st2 == ("two_phase", 0)
    assert rel(o, o2.double().cpu().numpy()) < 5e-3
    assert rel(S, S2.double().cpu().numpy()) < 5e-3


def test_split_in_graph_capture():
    # the split schedule is stream-ordered kernels only, so it can be
    # captured: replays with new inputs copied in match eager calls bitwise
    import linear_attention_kda_amd as kda
    announce("split-sequence under graph capture: 3 replays vs eager, B=1 T=3000 H=2")
    B, T, H = 1, 3000, 2
    ws = _workspace(B, T, H)
    static = to_dev(inputs.dense(B, T, H, 128, 128, torch.bfloat16, s0_std=0.02, seed=76))
    o = torch.empty_like(static["v"])
    S = torch.empty((B, H, 128, 128), dtype=torch.float32, device="cuda")
    prev = kda.set_schedule("split")
    try:
        def call():
            kda.chunk_fwd(static["q"], static["k"], static["v"], static["alpha"], static["beta"], S0=static["S0"],
                          out=o, S_final=S, workspace=ws)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            call()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            call()
        torch.cuda.synchronize()
        for seed in (77, 78, 79):
            new = to_dev(inputs.dense(B, T, H, 128, 128, torch.bfloat16, s0_std=0.02, seed=seed))
            for name in ("q", "k", "v", "alpha", "beta", "S0"):
                static[name].copy_(new[name])
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            o_g, S_g = o.clone(), S.clone()
            assert kda.chunk_fwd_status(ws) == ("split", 0)
            o_e, S_e, st = _run(new, "split", _workspace(B, T, H))
            assert st == ("split", 0)
            assert torch.equal(o_g, o_e) and torch.equal(S_g, S_e)
    finally:
        kda.set_schedule(prev)
