"""The no-allocation prefill entry point (kda_chunk_fwd_noalloc, on the
library's static device scratch) against the existing entry point
(kda_chunk_fwd_ex, on a caller's workspace) through the C ABI: bit-identical
outputs and final states on two calls in a row, the second with a smaller
input, plus a multi-segment case, a packed batch, and the size limit."""
import pytest
import torch

from linear_attention_kda_amd import inputs
from tests.gpu_cases import TOL, announce, check, oracle_prefill, to_dev

pytestmark = pytest.mark.gpu


def _both(inp, gate="channel"):
    import linear_attention_kda_amd as kda
    args = (inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"])
    kw = dict(S0=inp.get("S0"), cu_seqlens=inp.get("cu_seqlens"), gate=gate)
    o_n, S_n = kda.chunk_fwd_noalloc(*args, **kw)
    torch.cuda.synchronize()
    o_w, S_w = kda.chunk_fwd(*args, **kw)
    torch.cuda.synchronize()
    return (o_n, S_n), (o_w, S_w)


def test_two_calls_second_smaller():
    import linear_attention_kda_amd as kda
    # first: the prefill workload (B=4 H=16 T=2048 d=128): its 128 MB
    # workspace exceeds the 64 MiB scratch, so it runs one sequence per call
    announce("noalloc call 1: prefill workload B4 H16 T2048 d128 bf16 (one sequence per call)")
    need = kda.chunk_fwd_workspace_size(4, 2048, 16, 128, 128, -1, kda.KDA_BF16)
    assert need > kda.NOALLOC_SCRATCH_BYTES
    inp = inputs.workload("prefill", seed=3, device="cuda")
    (o_n, S_n), (o_w, S_w) = _both(inp)
    assert torch.equal(o_n, o_w) and torch.equal(S_n, S_w)
    # second, smaller: fits whole, with S0, a ragged tail, a scalar gate
    announce("noalloc call 2: B2 H4 T300 d128 bf16, S0, scalar gate (one call)")
    inp2 = to_dev(inputs.dense(2, 300, 4, 128, 128, torch.bfloat16, s0_std=0.02, seed=61, gate_form="scalar"))
    (o_n2, S_n2), (o_w2, S_w2) = _both(inp2, gate="scalar")
    assert torch.equal(o_n2, o_w2) and torch.equal(S_n2, S_w2)
    full = dict(inp2)
    full["alpha"] = inp2["alpha"].unsqueeze(-1).expand(2, 300, 4, 128).contiguous()
    o_ref, S_ref = oracle_prefill(full)
    check("o", o_n2, o_ref, TOL[torch.bfloat16])
    check("S_final", S_n2, S_ref, TOL[torch.bfloat16])


def test_segments_along_the_sequence():
    # B=2 H=64 T=8192: one sequence needs 511 MB of records, so each runs in
    # segments of 16 chunks, the state carried through S_final
    announce("noalloc segments: B2 H64 T8192 d128 bf16 with S0 (8 segments per sequence), then fp32 d32")
    inp = to_dev(inputs.dense(2, 8192, 64, 128, 128, torch.bfloat16, s0_std=0.02, seed=62))
    (o_n, S_n), (o_w, S_w) = _both(inp)
    assert torch.equal(o_n, o_w) and torch.equal(S_n, S_w)
    small = to_dev(inputs.dense(1, 130, 2, 32, 32, torch.float32, s0_std=0.1, seed=63))
    (o_n, S_n), (o_w, S_w) = _both(small)
    assert torch.equal(o_n, o_w) and torch.equal(S_n, S_w)


def test_packed_batch_and_limits():
    import linear_attention_kda_amd as kda
    announce("noalloc packed batch lens [70, 0, 5, 200] H3 d128 bf16; size limit refusals")
    inp = to_dev(inputs.packed([70, 0, 5, 200], 3, 128, 128, torch.bfloat16, s0_std=0.02, seed=64))
    (o_n, S_n), (o_w, S_w) = _both(inp)
    assert torch.equal(o_n, o_w) and torch.equal(S_n, S_w)
    # a packed batch larger than the scratch is refused before any work
    T, H = 70_000, 16
    big = dict(q=torch.zeros((T, H, 128), dtype=torch.bfloat16, device="cuda"))
    big["k"], big["v"] = big["q"].clone(), big["q"].clone()
    big["alpha"] = torch.ones((T, H, 128), device="cuda")
    big["beta"] = torch.zeros((T, H), device="cuda")
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    with pytest.raises(kda.KdaError) as e:
        kda.chunk_fwd_noalloc(big["q"], big["k"], big["v"], big["alpha"], big["beta"], cu_seqlens=cu)
    assert e.value.status == kda.KDA_ERR_TOO_LARGE
    # a dense shape where not even one chunk per head fits
    H = 1100
    q = torch.zeros((1, 64, H, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(kda.KdaError) as e:
        kda.chunk_fwd_noalloc(q, q.clone(), q.clone(), torch.ones((1, 64, H, 128), device="cuda"),
                              torch.zeros((1, 64, H), device="cuda"))
    assert e.value.status == kda.KDA_ERR_TOO_LARGE
    torch.cuda.synchronize()
