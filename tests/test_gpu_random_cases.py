"""Seeded random cases through the C ABI against the fp64 oracle: prefill
(dense and packed, both dtypes, every head size, every gate form, with and
without S0, every schedule), decode (one token and several, in place or
not) and the block's operations around the method (short convolution,
output norm and gate).  The shapes are drawn once from a fixed seed, so every run checks the
same cases; each is small enough for the oracle and spans ragged chunks.
Gate forms reach the oracle as per-channel gates in fp64 (broadcast, ones,
exp of the logarithm, 1 / (1 + e^g) of the softplus logit), the way the page
"Kimi Delta Attention (KDA)" defines the scalar and absent gates as special
cases of the per-channel one."""
import random

import pytest
import torch

from linear_attention_kda_amd import inputs
from tests.gpu_cases import TOL, announce, check, oracle_prefill, to_dev

pytestmark = pytest.mark.gpu

GATES = ["channel", "scalar", "none", "log_channel", "log_scalar", "softplus_channel", "softplus_scalar"]
DIMS = [16, 32, 64, 128]


def _linear_alpha(alpha, form, lead, dk):
    """Per-channel gates in fp64 for the oracle, from a gate form's tensor."""
    if form == "none":
        return torch.ones(*lead, dk, dtype=torch.float64)
    a = alpha.detach().cpu().double()
    if form.startswith("log_"):
        a = torch.exp(a)
    elif form.startswith("softplus_"):
        a = 1.0 / (1.0 + torch.exp(a))
    if form.endswith("scalar"):
        a = a.unsqueeze(-1).expand(*lead, dk).contiguous()
    return a


def _prefill_cases(n=28, seed=20261203):
    rng = random.Random(seed)
    cases = []
    for i in range(n):
        dtype = rng.choice(["bf16", "fp32"])
        dk, dv = rng.choice(DIMS), rng.choice(DIMS)
        H = rng.randint(1, 4)
        packed = rng.random() < 0.35
        if packed:
            lengths = [rng.choice([0, 1, rng.randint(2, 63), 64, rng.randint(65, 300)]) for _ in range(rng.randint(1, 4))]
            B, T = 1, sum(lengths)
        else:
            lengths = None
            B, T = rng.randint(1, 3), rng.choice([1, rng.randint(2, 63), 64, 65, rng.randint(66, 600)])
        gate = rng.choice(GATES)
        s0 = rng.random() < 0.6
        sched = rng.choice(["auto", "two_phase", "overlap", "split"])
        cases.append(dict(i=i, dtype=dtype, dk=dk, dv=dv, H=H, B=B, T=T, lengths=lengths, gate=gate, s0=s0,
                          sched=sched))
    return cases


def _id(c):
    shape = f"packed{c['lengths']}" if c["lengths"] is not None else f"B{c['B']}T{c['T']}"
    return f"{c['i']}-{c['dtype']}-{shape}-H{c['H']}-dk{c['dk']}dv{c['dv']}-{c['gate']}-{'S0' if c['s0'] else 'noS0'}-{c['sched']}"


PREFILL = _prefill_cases()


@pytest.mark.parametrize("c", PREFILL, ids=[_id(c) for c in PREFILL])
def test_random_prefill(c):
    import linear_attention_kda_amd as kda
    announce(f"random prefill {_id(c)}")
    dtype = torch.bfloat16 if c["dtype"] == "bf16" else torch.float32
    seed = 9000 + c["i"]
    if c["lengths"] is not None:
        inp = inputs.packed(c["lengths"], c["H"], c["dk"], c["dv"], dtype, s0_std=0.02 if c["s0"] else None,
                            seed=seed, gate_form=c["gate"])
        lead = inp["q"].shape[:-1]
    else:
        inp = inputs.dense(c["B"], c["T"], c["H"], c["dk"], c["dv"], dtype, s0_std=0.02 if c["s0"] else None,
                           seed=seed, gate_form=c["gate"])
        lead = inp["q"].shape[:-1]
    ref_in = dict(inp)
    ref_in["alpha"] = _linear_alpha(inp["alpha"], c["gate"], lead, c["dk"])
    o_ref, S_ref = oracle_prefill(ref_in)
    dev = to_dev(inp)
    kda.set_schedule(c["sched"])
    try:
        o, S = kda.chunk_fwd(dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"], S0=dev.get("S0"),
                             cu_seqlens=dev.get("cu_seqlens"), gate=c["gate"])
        torch.cuda.synchronize()
    finally:
        kda.set_schedule("auto")
    cu = inp.get("cu_seqlens")
    check("o", o, o_ref, TOL[dtype], cu=None if cu is None else cu)
    check("S_final", S, S_ref, TOL[dtype])


def _decode_cases(n=14, seed=20261204):
    rng = random.Random(seed)
    cases = []
    for i in range(n):
        cases.append(dict(i=i, dtype=rng.choice(["bf16", "fp32"]), dk=rng.choice(DIMS), dv=rng.choice(DIMS),
                          N=rng.randint(1, 9), H=rng.randint(1, 5), Tk=rng.choice([1, 2, 3, 4, 5, 8]),
                          gate=rng.choice(GATES), in_place=rng.random() < 0.5))
    return cases


def _did(c):
    return (f"{c['i']}-{c['dtype']}-N{c['N']}H{c['H']}-dk{c['dk']}dv{c['dv']}-Tk{c['Tk']}-{c['gate']}-"
            f"{'inplace' if c['in_place'] else 'copy'}")


DECODE = _decode_cases()


@pytest.mark.parametrize("c", DECODE, ids=[_did(c) for c in DECODE])
def test_random_decode_tokens(c):
    import linear_attention_kda_amd as kda
    announce(f"random decode_tokens {_did(c)}")
    dtype = torch.bfloat16 if c["dtype"] == "bf16" else torch.float32
    inp = inputs.dense(c["N"], c["Tk"], c["H"], c["dk"], c["dv"], dtype, gate="uniform", alpha_lo=0.9,
                       s0_std=0.05, seed=9500 + c["i"], gate_form=c["gate"])
    lead = inp["q"].shape[:-1]
    ref_in = dict(inp)
    ref_in["alpha"] = _linear_alpha(inp["alpha"], c["gate"], lead, c["dk"])
    o_ref, S_ref = oracle_prefill(ref_in)
    dev = to_dev(inp)
    S_in = dev["S0"].clone()
    S_out = S_in if c["in_place"] else None
    o, S = kda.decode_tokens(dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"], S_in, S_out=S_out,
                             gate=c["gate"])
    torch.cuda.synchronize()
    if c["in_place"]:
        assert S.data_ptr() == S_in.data_ptr()
    else:
        assert torch.equal(S_in, dev["S0"]), "S_in is the checkpoint and must not change"
    check("o", o, o_ref, TOL[dtype])
    check("S_out", S, S_ref, TOL[dtype])


def _module_cases(n=12, seed=20261205):
    rng = random.Random(seed)
    cases = []
    for i in range(n):
        packed = rng.random() < 0.4
        lengths = ([rng.choice([1, 2, 3, rng.randint(4, 63), 64, rng.randint(65, 200)]) for _ in range(rng.randint(1, 3))]
                   if packed else None)
        cases.append(dict(i=i, dtype=rng.choice(["bf16", "fp32"]), dk=rng.choice(DIMS), dv=rng.choice(DIMS),
                          H=rng.randint(1, 3), B=1 if packed else rng.randint(1, 2),
                          T=sum(lengths) if packed else rng.randint(2, 300), lengths=lengths,
                          gate=rng.choice(["channel", "scalar", "softplus_channel", "softplus_scalar"]),
                          ops=rng.choice(["conv", "norm_gate", "all"]), s0=rng.random() < 0.5,
                          sched=rng.choice(["auto", "two_phase", "split"])))
    return cases


def _mid(c):
    shape = f"packed{c['lengths']}" if c["lengths"] is not None else f"B{c['B']}T{c['T']}"
    return (f"{c['i']}-{c['dtype']}-{shape}-H{c['H']}-dk{c['dk']}dv{c['dv']}-{c['gate']}-{c['ops']}-"
            f"{'S0' if c['s0'] else 'noS0'}-{c['sched']}")


MODULE = _module_cases()


@pytest.mark.parametrize("c", MODULE, ids=[_mid(c) for c in MODULE])
def test_random_module_ops(c):
    """The block's operations around the method (short convolution, output
    norm and gate) on random shapes, against the float64 block steps of
    tests/module_ref.py around the oracle."""
    import linear_attention_kda_amd as kda
    from tests.test_gpu_module_ops import _raw_block, _reference, _run, _weights
    announce(f"random module ops {_mid(c)}")
    dtype = torch.bfloat16 if c["dtype"] == "bf16" else torch.float32
    seed = 9700 + c["i"]
    if c["lengths"] is not None:
        inp = inputs.packed(c["lengths"], c["H"], c["dk"], c["dv"], dtype, s0_std=0.02 if c["s0"] else None,
                            seed=seed, gate_form=c["gate"])
    else:
        inp = inputs.dense(c["B"], c["T"], c["H"], c["dk"], c["dv"], dtype, s0_std=0.02 if c["s0"] else None,
                           seed=seed, gate_form=c["gate"])
    inp = _raw_block(to_dev(inp), seed)
    w = _weights(c["H"], c["dk"], c["dv"], dtype, inp["v"].shape, seed, conv=c["ops"] in ("conv", "all"),
                 norm=c["ops"] in ("norm_gate", "all"), gate=c["ops"] in ("norm_gate", "all"))
    o_ref, S_ref = _reference(inp, w, c["gate"], c["dk"])
    kda.set_schedule(c["sched"])
    try:
        o, S = _run(inp, c["gate"], w)
    finally:
        kda.set_schedule("auto")
    cu = inp.get("cu_seqlens")
    check("o", o, o_ref, TOL[dtype], cu=None if cu is None else cu.cpu())
    check("S_final", S, S_ref, TOL[dtype])
