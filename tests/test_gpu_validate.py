"""Device-side value checks (kda_set_validation): each precondition the host
cannot see makes a call return KDA_ERR_INVALID_VALUE and launch nothing;
clean inputs give the same results as with the checks off."""
import pytest
import torch

from linear_attention_kda_amd import inputs
from tests.gpu_cases import announce, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture()
def kda_checked():
    import linear_attention_kda_amd as kda
    prev = kda.set_validation(True)
    try:
        yield kda
    finally:
        kda.set_validation(prev)


def _rejects(kda, fn):
    with pytest.raises(kda.KdaError) as ei:
        fn()
    assert ei.value.status == kda.KDA_ERR_INVALID_VALUE


def test_prefill_checks(kda_checked):
    kda = kda_checked
    announce("value checks, dense prefill B=2 T=100 H=3 d=64 bf16")
    inp = to_dev(inputs.dense(2, 100, 3, 64, 64, torch.bfloat16, s0_std=0.02, seed=41))
    run = lambda x, gate=None: kda.chunk_fwd(x["q"], x["k"], x["v"], x["alpha"], x["beta"], S0=x["S0"], gate=gate)
    o, S = run(inp)
    kda.set_validation(False)
    o2, S2 = run(inp)
    torch.cuda.synchronize()
    kda.set_validation(True)
    assert torch.equal(o, o2) and torch.equal(S, S2)
    for key, idx, val in (("alpha", (1, 50, 2, 7), 1.5), ("alpha", (0, 0, 0, 0), float("nan")),
                          ("beta", (0, 99, 1), -0.1), ("beta", (1, 3, 0), 1.01)):
        bad = dict(inp)
        bad[key] = inp[key].clone()
        bad[key][idx] = val
        _rejects(kda, lambda: run(bad))
    bad = dict(inp)
    bad["k"] = inp["k"].clone()
    bad["k"][0, 10, 2] *= 1.1                       # |k|^2 = 1.21
    _rejects(kda, lambda: run(bad))
    lg = dict(inp)
    lg["alpha"] = torch.log(inp["alpha"])
    run(lg, "log_channel")                          # log gates <= 0 pass
    lg["alpha"][1, 1, 1, 1] = 0.1
    _rejects(kda, lambda: run(lg, "log_channel"))


def test_packed_offsets_checked(kda_checked):
    kda = kda_checked
    announce("value checks, packed offsets")
    inp = to_dev(inputs.packed([40, 70, 30], 2, 32, 32, torch.float32, s0_std=0.02, seed=42))
    run = lambda cu: kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], S0=inp["S0"],
                                   cu_seqlens=cu)
    run(inp["cu_seqlens"])
    T = int(inp["cu_seqlens"][-1])
    for bad in ([0, 70, 40, T], [5, 40, 110, T], [0, 40, 110, T - 1]):
        cu = torch.tensor(bad, dtype=torch.int32, device="cuda")
        _rejects(kda, lambda: run(cu))


def test_decode_checks_launch_nothing(kda_checked):
    kda = kda_checked
    announce("value checks, decode step and decode tokens leave the state alone")
    N, H, D = 3, 2, 64
    S = inputs.decode_state(N, H, D, D, 0.02, seed=43, device="cuda")
    tok = inputs.decode_token(N, H, D, D, torch.bfloat16, 0.95, step=0, seed=43, device="cuda")
    bad = dict(tok)
    bad["alpha"] = tok["alpha"].clone()
    bad["alpha"][2, 1, 5] = -0.5
    S0 = S.clone()
    _rejects(kda, lambda: kda.decode_step(bad["q"], bad["k"], bad["v"], bad["alpha"], bad["beta"], S))
    torch.cuda.synchronize()
    assert torch.equal(S, S0)
    d = to_dev(inputs.dense(N, 3, H, D, D, torch.bfloat16, gate="uniform", alpha_lo=0.95, seed=44))
    d["beta"][0, 2, 1] = 2.0
    _rejects(kda, lambda: kda.decode_tokens(d["q"], d["k"], d["v"], d["alpha"], d["beta"], S, S_out=S))
    torch.cuda.synchronize()
    assert torch.equal(S, S0)
    kda.decode_step(tok["q"], tok["k"], tok["v"], tok["alpha"], tok["beta"], S)   # clean: runs
