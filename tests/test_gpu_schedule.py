"""The overlapped prefill schedule on the GPU: chunk preparation and the scan
run at once on two disjoint sets of compute units, the scan taking each
chunk's record as soon as its ready flag is set (page "Kimi Delta Attention
(KDA)", section "Two schedules of computation for one recurrence": the
parallel chunk stage feeds the sequential scan).  Both schedules execute the
same arithmetic per chunk, so their results must be bitwise equal; one case
per group is also checked against the fp64 oracle, and the call's status
(kda_chunk_fwd_status: the schedule that ran, and the error bits for a
timed-out wait or a record from another XCD) must name the schedule and show
no error."""
import pytest
import torch

from linear_attention_kda_amd import inputs
from tests.gpu_cases import TOL, announce, check, oracle_prefill, to_dev

pytestmark = pytest.mark.gpu



def _run(inp, schedule, gate="channel", act=0, ws=None):
    import linear_attention_kda_amd as kda
    prev = kda.set_schedule(schedule)
    try:
        o, S = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], S0=inp.get("S0"),
                             gate=gate, act=act, workspace=ws)
        torch.cuda.synchronize()
    finally:
        kda.set_schedule(prev)
    return o, S


def _workspace(B, T, H):
    import linear_attention_kda_amd as kda
    n = kda.chunk_fwd_workspace_size(B, T, H, 128, 128, -1, kda.KDA_BF16)
    return torch.zeros(n, dtype=torch.uint8, device="cuda")


def _status(ws):
    import linear_attention_kda_amd as kda
    return kda.chunk_fwd_status(ws)


@pytest.mark.parametrize("B,T,H,s0", [
    (1, 64, 1, None),        # one chunk
    (1, 65, 2, 0.02),        # a ragged second chunk
    (2, 700, 3, 0.02),       # units not a multiple of eight
    (4, 2048, 16, None),     # the prefill workload's shape, 64 units
    (3, 1000, 32, 0.02),     # 96 units: 384 scan workgroups on 128 CUs, so units take turns
])
def test_overlap_equals_two_phase(B, T, H, s0):
    announce(f"schedule overlap vs two-phase, dense bf16 d=128 B={B} T={T} H={H} S0={s0}")
    inp = to_dev(inputs.dense(B, T, H, 128, 128, torch.bfloat16, s0_std=s0, seed=21))
    ws = _workspace(B, T, H)
    o1, S1 = _run(inp, "overlap", ws=ws)
    assert _status(ws) == ("overlap", 0)
    o2, S2 = _run(inp, "two_phase", ws=ws)
    assert _status(ws) == ("two_phase", 0)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_overlap_oracle():
    announce("schedule overlap vs the fp64 oracle, B=2 T=300 H=4 d=128 bf16 with S0")
    inp = to_dev(inputs.dense(2, 300, 4, 128, 128, torch.bfloat16, s0_std=0.02, seed=22))
    o, S = _run(inp, "overlap")
    o_ref, S_ref = oracle_prefill(inp)
    check("o", o, o_ref, TOL[torch.bfloat16])
    check("S_final", S, S_ref, TOL[torch.bfloat16])


@pytest.mark.parametrize("gate", ["scalar", "none", "log_channel", "softplus_channel"])
def test_overlap_gate_forms(gate):
    announce(f"schedule overlap vs two-phase, gate form {gate}, B=2 T=520 H=4")
    inp = to_dev(inputs.dense(2, 520, 4, 128, 128, torch.bfloat16, s0_std=0.02, seed=23, gate_form=gate))
    o1, S1 = _run(inp, "overlap", gate=gate)
    o2, S2 = _run(inp, "two_phase", gate=gate)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_overlap_fused_inputs_and_strong_decay():
    import linear_attention_kda_amd as kda
    announce("schedule overlap vs two-phase: fused input activations; a gate of 0 (exact prep path)")
    inp = to_dev(inputs.dense(2, 400, 4, 128, 128, torch.bfloat16, s0_std=0.02, seed=24))
    act = kda.KDA_ACT_QK_SILU_L2NORM | kda.KDA_ACT_BETA_SIGMOID
    o1, S1 = _run(inp, "overlap", act=act)
    o2, S2 = _run(inp, "two_phase", act=act)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    inp["alpha"][:, 100:140] = 0.0
    o1, S1 = _run(inp, "overlap")
    o2, S2 = _run(inp, "two_phase")
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    o_ref, S_ref = oracle_prefill(inp)
    check("o", o1, o_ref, TOL[torch.bfloat16])
    check("S_final", S1, S_ref, TOL[torch.bfloat16])


def test_overlap_repeated_calls_share_workspace():
    announce("schedule overlap: three calls in a row on one workspace with different inputs")
    B, T, H = 2, 640, 8
    ws = _workspace(B, T, H)
    for seed in (31, 32, 33):
        inp = to_dev(inputs.dense(B, T, H, 128, 128, torch.bfloat16, s0_std=0.02, seed=seed))
        o1, S1 = _run(inp, "overlap", ws=ws)
        assert _status(ws) == ("overlap", 0)
        o2, S2 = _run(inp, "two_phase")
        assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_overlap_in_graph_capture():
    """A call captured into a HIP graph while the overlapped schedule is
    requested runs two-phase (a replay keeps neither the compute-unit masks
    nor the concurrency the scan would wait on), also once the internal
    streams exist: replays with new inputs copied in, with eager work and
    synchronisation between them, match the eager two-phase results bitwise,
    and the status of each replay names the two-phase schedule."""
    import linear_attention_kda_amd as kda
    announce("overlap requested under graph capture: 3 replays vs eager two-phase, B=2 T=640 H=8")
    B, T, H = 2, 640, 8
    ws = _workspace(B, T, H)
    static = to_dev(inputs.dense(B, T, H, 128, 128, torch.bfloat16, s0_std=0.02, seed=40))
    o = torch.empty_like(static["v"])
    S = torch.empty((B, H, 128, 128), dtype=torch.float32, device="cuda")
    prev = kda.set_schedule("overlap")
    try:
        def call():
            kda.chunk_fwd(static["q"], static["k"], static["v"], static["alpha"], static["beta"], S0=static["S0"],
                          out=o, S_final=S, workspace=ws)
        call()  # eager once: creates the internal streams outside the capture
        torch.cuda.synchronize()
        assert _status(ws) == ("overlap", 0)
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
        for seed in (41, 42, 43):
            new = to_dev(inputs.dense(B, T, H, 128, 128, torch.bfloat16, s0_std=0.02, seed=seed))
            for name in ("q", "k", "v", "alpha", "beta", "S0"):
                static[name].copy_(new[name])
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            o_g, S_g = o.clone(), S.clone()
            assert _status(ws) == ("two_phase", 0)
            o_e, S_e = _run(new, "two_phase")
            assert torch.equal(o_g, o_e) and torch.equal(S_g, S_e)
    finally:
        kda.set_schedule(prev)


def test_overlap_timeout_is_reported():
    """The scan's bounded wait for a chunk record, forced to give up from the
    host (a bound of zero ticks: no wait at all), ends every kernel normally
    and is reported: kda_chunk_fwd_status shows the timeout bit, and with
    value checks on the binding raises instead of returning the wrong
    results.  A later call with the default bound is clean again."""
    import linear_attention_kda_amd as kda
    announce("overlap scan wait bound 0 (forced timeout), B=2 T=640 H=8; then the default bound")
    B, T, H = 2, 640, 8
    ws = _workspace(B, T, H)
    inp = to_dev(inputs.dense(B, T, H, 128, 128, torch.bfloat16, s0_std=0.02, seed=44))
    prev_limit = kda.set_sched_wait_limit(0)
    try:
        _run(inp, "overlap", ws=ws)
        sched, errs = _status(ws)
        assert sched == "overlap" and errs & kda.KDA_SCHED_ERR_TIMEOUT
        prev_val = kda.set_validation(True)
        try:
            prev_sched = kda.set_schedule("overlap")
            try:
                with pytest.raises(RuntimeError, match="error bits"):
                    kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], S0=inp["S0"],
                                  workspace=ws)
                torch.cuda.synchronize()
            finally:
                kda.set_schedule(prev_sched)
        finally:
            kda.set_validation(prev_val)
    finally:
        kda.set_sched_wait_limit(prev_limit)
    o1, S1 = _run(inp, "overlap", ws=ws)
    assert _status(ws) == ("overlap", 0)
    o2, S2 = _run(inp, "two_phase")
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


@pytest.mark.parametrize("T,overlap", [(8192, True), (8128, False)])
def test_auto_schedule_threshold(T, overlap):
    """The automatic schedule overlaps from 4096 chunk records (B * H *
    ceil(T / 64)): 32 heads x 128 chunks do, 32 x 127 do not, as the call's
    status shows; the results equal the two-phase schedule's bit for bit
    either way."""
    B, H = 1, 32
    announce(f"schedule auto at the overlap threshold, B={B} T={T} H={H} (overlap expected: {overlap})")
    inp = to_dev(inputs.dense(B, T, H, 128, 128, torch.bfloat16, seed=23))
    ws = _workspace(B, T, H)
    o1, S1 = _run(inp, "auto", ws=ws)
    assert _status(ws) == ("overlap" if overlap else "two_phase", 0)
    o2, S2 = _run(inp, "two_phase")
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_long_context_overlap_equals_two_phase_all_heads():
    """The long-context workload at full size (32 heads x 1024 chunks, the
    shape the automatic schedule overlaps): every head, on every XCD's share
    of the units, equals the two-phase result bit for bit."""
    announce("long-context B1 H32 T65536 d128: overlap vs two-phase, all 32 heads bitwise")
    inp = inputs.workload("long", device="cuda")
    ws = _workspace(1, 65536, 32)
    o1, S1 = _run(inp, "overlap", ws=ws)
    assert _status(ws) == ("overlap", 0)
    o2, S2 = _run(inp, "two_phase", ws=ws)
    assert _status(ws) == ("two_phase", 0)
    for h in range(32):
        assert torch.equal(o1[:, :, h], o2[:, :, h]) and torch.equal(S1[:, h], S2[:, h]), f"head {h} differs"
