"""Edge cases of the HIP path vs the fp64 oracle (GPU): ragged and empty
lengths, every supported head size, both dtypes, gates of exactly 0 and 1,
strong decay, write strengths 0 and 1, packed batches, composition of calls
and run-to-run determinism."""
import numpy as np
import pytest
import torch

from linear_attention_kda_amd import inputs
from tests.gpu_cases import TOL, announce, check, gpu_prefill, oracle_prefill, to_dev

pytestmark = pytest.mark.gpu

F32, BF16 = torch.float32, torch.bfloat16


def _dense(B, T, H, dk, dv, dtype, seed, s0=0.1, gate="softplus", alpha_lo=0.9):
    return to_dev(inputs.dense(B, T, H, dk, dv, dtype, gate=gate, alpha_lo=alpha_lo,
                               s0_std=s0, seed=seed))


@pytest.mark.parametrize("dtype", [F32, BF16], ids=["f32", "bf16"])
@pytest.mark.parametrize("T", [0, 1, 63, 64, 65, 130])
def test_lengths(T, dtype):
    announce(f"dense B2 T{T} H3 d32 {dtype} seed{T}")
    inp = _dense(2, T, 3, 32, 32, dtype, seed=T)
    o, S = gpu_prefill(inp)
    o_ref, S_ref = oracle_prefill(inp)
    if T:
        check("o", o, o_ref, TOL[dtype])
    check("S_final", S, S_ref, TOL[dtype])


@pytest.mark.parametrize("dtype", [F32, BF16], ids=["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(16, 16), (16, 64), (64, 16), (32, 128), (128, 32), (64, 64),
                                   (128, 128)])
def test_head_sizes(dk, dv, dtype):
    announce(f"dense B1 T200 H2 dk{dk} dv{dv} {dtype}")
    inp = _dense(1, 200, 2, dk, dv, dtype, seed=dk * 7 + dv)
    o, S = gpu_prefill(inp)
    o_ref, S_ref = oracle_prefill(inp)
    check("o", o, o_ref, TOL[dtype])
    check("S_final", S, S_ref, TOL[dtype])


@pytest.mark.parametrize("dtype", [F32, BF16], ids=["f32", "bf16"])
def test_special_gates(dtype):
    """Gates of exactly 0 (a channel wiped) and exactly 1, write strengths of
    exactly 0 and 1."""
    announce(f"special gates B2 T150 H2 d64 {dtype}")
    inp = _dense(2, 150, 2, 64, 64, dtype, seed=3)
    a, b = inp["alpha"], inp["beta"]
    a[:, ::7, :, ::5] = 0.0
    a[:, 3::11] = 0.0          # whole tokens that clear the memory
    a[:, 1::4] = 1.0
    b[:, ::3] = 1.0
    b[:, 2::9] = 0.0
    o, S = gpu_prefill(inp)
    o_ref, S_ref = oracle_prefill(inp)
    check("o", o, o_ref, TOL[dtype])
    check("S_final", S, S_ref, TOL[dtype])


@pytest.mark.parametrize("dtype", [F32, BF16], ids=["f32", "bf16"])
@pytest.mark.parametrize("lo,hi", [(0.0, 0.05), (1e-30, 1e-20), (0.3, 0.6)])
def test_strong_decay(lo, hi, dtype):
    """Gates whose product over 16 tokens leaves fp32's range: the diagonal
    blocks must take the exact path."""
    announce(f"strong decay alpha~U({lo},{hi}) B1 T130 H2 d32 {dtype}")
    inp = _dense(1, 130, 2, 32, 32, dtype, seed=4)
    g = torch.Generator(device="cuda").manual_seed(9)
    inp["alpha"] = torch.empty_like(inp["alpha"]).uniform_(lo, hi, generator=g)
    o, S = gpu_prefill(inp)
    o_ref, S_ref = oracle_prefill(inp)
    check("o", o, o_ref, TOL[dtype])
    check("S_final", S, S_ref, TOL[dtype])


def test_mixed_decay_channels():
    """Realistic mix: most channels slow, a few channels decaying by ~1e-4 per
    token (whole-chunk products far below fp32's range)."""
    announce("mixed decay channels B2 T256 H4 d128 bf16")
    inp = _dense(2, 256, 4, 128, 128, BF16, seed=5)
    inp["alpha"][..., ::16] = 1e-4
    o, S = gpu_prefill(inp)
    o_ref, S_ref = oracle_prefill(inp)
    check("o", o, o_ref, TOL[BF16])
    check("S_final", S, S_ref, TOL[BF16])


@pytest.mark.parametrize("dtype", [F32, BF16], ids=["f32", "bf16"])
def test_packed_ragged(dtype):
    """Packed batch with zero-length, length-1 and ragged sequences; every
    sequence has its own S0."""
    lens = [0, 1, 63, 64, 65, 130, 5, 0, 200]
    announce(f"packed lens={lens} H3 d64 {dtype}")
    inp = to_dev(inputs.packed(lens, 3, 64, 64, dtype, s0_std=0.1, seed=6))
    o, S = gpu_prefill(inp)
    o_ref, S_ref = oracle_prefill(inp)
    check("o", o, o_ref, TOL[dtype], cu=inp["cu_seqlens"])
    check("S_final", S, S_ref, TOL[dtype])
    # zero-length sequences return their S0 exactly
    assert torch.equal(S[0], inp["S0"][0]) and torch.equal(S[7], inp["S0"][7])


def test_packed_equals_separate_runs():
    lens = [70, 3, 128, 41]
    announce(f"packed == separate, lens={lens} bf16")
    inp = to_dev(inputs.packed(lens, 2, 128, 128, BF16, s0_std=0.05, seed=7))
    o, S = gpu_prefill(inp)
    cu = inp["cu_seqlens"].cpu().tolist()
    for n in range(len(lens)):
        a, b = cu[n], cu[n + 1]
        one = {key: inp[key][a:b][None] for key in ("q", "k", "v", "alpha", "beta")}
        one["S0"] = inp["S0"][n:n + 1]
        o1, S1 = gpu_prefill(one)
        assert torch.equal(o1[0], o[a:b]), f"seq {n} outputs differ"
        assert torch.equal(S1[0], S[n]), f"seq {n} state differs"


def test_split_prefill_composes():
    """prefill(T1) then prefill(T2, S0 = its final state) == prefill(T1+T2)."""
    announce("split prefill 100 + 93, bf16 d128")
    inp = _dense(2, 193, 2, 128, 128, BF16, seed=8)
    o_ref, S_ref = oracle_prefill(inp)
    first = {k: v[:, :100] for k, v in inp.items() if k != "S0"}
    first["S0"] = inp["S0"]
    oa, Sa = gpu_prefill(first)
    second = {k: v[:, 100:].contiguous() for k, v in inp.items() if k != "S0"}
    second["S0"] = Sa
    ob, Sb = gpu_prefill(second)
    check("o", torch.cat([oa, ob], 1), o_ref, TOL[BF16])
    check("S_final", Sb, S_ref, TOL[BF16])


def test_prefill_then_decode():
    """prefill(T) followed by n decode steps == the recurrence over T + n."""
    import linear_attention_kda_amd as kda
    announce("prefill 77 then 5 decode steps, bf16 d128")
    T, n = 77, 5
    inp = _dense(3, T + n, 2, 128, 128, BF16, seed=9)
    o_ref, S_ref = oracle_prefill(inp)
    head = {k: v[:, :T] for k, v in inp.items() if k != "S0"}
    head["S0"] = inp["S0"]
    o_pf, S = gpu_prefill(head)
    outs = [o_pf]
    for t in range(T, T + n):
        tok = {k: inp[k][:, t].contiguous() for k in ("q", "k", "v", "alpha", "beta")}
        outs.append(kda.decode_step(tok["q"], tok["k"], tok["v"], tok["alpha"], tok["beta"], S)[:, None])
    torch.cuda.synchronize()
    check("o", torch.cat(outs, 1), o_ref, TOL[BF16])
    check("S_final", S, S_ref, TOL[BF16])


@pytest.mark.parametrize("dtype", [F32, BF16], ids=["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (128, 128), (64, 32)])
def test_decode_shapes(dk, dv, dtype):
    import linear_attention_kda_amd as kda
    import oracle
    announce(f"decode N5 H3 dk{dk} dv{dv} {dtype}, 3 steps")
    S = inputs.decode_state(5, 3, dk, dv, 0.1, seed=1, device="cuda")
    S_ref = S.double().cpu().numpy()
    for step in range(3):
        tok = inputs.decode_token(5, 3, dk, dv, dtype, 0.9, step=step, seed=2, device="cuda")
        o = kda.decode_step(tok["q"], tok["k"], tok["v"], tok["alpha"], tok["beta"], S)
        torch.cuda.synchronize()
        o_ref, S_ref = oracle.decode(tok["q"], tok["k"], tok["v"], tok["alpha"], tok["beta"], S_ref)
        check(f"o step {step}", o, o_ref, TOL[dtype])
    check("S", S, S_ref, TOL[dtype])


def test_scale_and_in_place_state():
    """An explicit scale of d_k^-1/2 equals the default; S_final may alias S0."""
    announce("scale default/explicit and in-place state, bf16 d64")
    inp = _dense(2, 90, 2, 64, 64, BF16, seed=10)
    o1, S1 = gpu_prefill(inp)
    o2, S2 = gpu_prefill(inp, scale=64 ** -0.5)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    import linear_attention_kda_amd as kda
    S0 = inp["S0"].clone()
    o3, S3 = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], S0=S0, S_final=S0)
    torch.cuda.synchronize()
    assert S3.data_ptr() == S0.data_ptr()
    assert torch.equal(S3, S1) and torch.equal(o3, o1)


def test_deterministic():
    """Two runs of the same call give bit-identical results."""
    announce("determinism prefill-shaped B2 T512 H4 d128 bf16")
    inp = _dense(2, 512, 4, 128, 128, BF16, seed=11)
    o1, S1 = gpu_prefill(inp)
    o2, S2 = gpu_prefill(inp)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


@pytest.mark.parametrize("B,T,H", [(5, 130, 16), (1, 700, 72)])
def test_many_units_one_cu_scan(B, T, H):
    """Batches of more than 64 (sequence, head) units at d = 128 bf16 run the
    two-phase scan with one workgroup per unit: ragged lengths, S0, against
    the oracle per unit; then bitwise equal to the same units run 64 at a
    time (the four-workgroup scan)."""
    announce(f"many units (one-CU scan): dense B{B} T{T} H{H} d128 bf16 with S0")
    inp = _dense(B, T, H, 128, 128, BF16, seed=B * 100 + H, s0=0.02)
    o, S = gpu_prefill(inp)
    o_ref, S_ref = oracle_prefill(inp)
    check("o", o, o_ref, TOL[BF16])
    check("S_final", S, S_ref, TOL[BF16])
    # the same arithmetic through the four-workgroup scan: split the heads so
    # each call has at most 64 units
    hs = max(1, 64 // B)
    for h0 in range(0, H, hs):
        sl = slice(h0, min(H, h0 + hs))
        part = {key: inp[key][:, :, sl].contiguous() for key in ("q", "k", "v", "alpha", "beta")}
        part["S0"] = inp["S0"][:, sl].contiguous()
        o_p, S_p = gpu_prefill(part)
        assert torch.equal(o_p, o[:, :, sl]) and torch.equal(S_p, S[:, sl]), f"heads {h0}.. differ"
