"""Sizes whose byte offsets pass 2^31 and 2^32.

One sequence of 2^20 tokens on eight heads (d = 128, bf16) through every
prefill schedule: the context length the pages build the method for (page
"Kimi Delta Attention (KDA)", section on why the architecture matters beyond
data centres: a state of constant size for contexts of a million tokens).

At this size the chunk records take 8.2 GB, so their byte offsets pass 2^32;
alpha's pass 2^31 halfway and the outputs' reach 2^31 at the end.  The oracle
cannot walk the whole chain, so the gates are drawn below 0.9.  Each step of
the recurrence (same page, opening update) maps the old state S to
S Diag(alpha_t) (I - beta_t k_t k_t^T), whose norm is at most max alpha_t for
a unit key and beta_t in [0, 1]; a state 448 tokens back therefore reaches
the present damped by 0.9^448 < 1e-20, far below fp32 rounding.  The outputs
of the last 128 tokens of a 576-token window are then, to that residue, the
oracle's run over the window alone from a zero state; the first window
starts at token 0 from the true S0 and is exact throughout.

Decode over 81,920 (sequence, head) states (5.4 GB of fp32 state, 64 KiB
each): one step and a four-token launch, checked on the sequences whose
states sit at the start, across 2^31 and 2^32 bytes and at the end."""
import pytest
import torch

from linear_attention_kda_amd import inputs
from tests.gpu_cases import TOL, announce, check, oracle_prefill

pytestmark = pytest.mark.gpu

T, H, D = 1 << 20, 8, 128
HIST, CHECK = 448, 128            # damped history, then the checked tokens
WIN = HIST + CHECK
# windows by their last token (exclusive): the start; alpha's offsets passing
# 2^31 bytes; the records of chunk 8594 (head 7 straddles 2^32 bytes) and
# 8595; the end, where the outputs reach 2^31 bytes and S_final is read
ENDS = [WIN, (1 << 19) + CHECK, 8596 * 64, T]


@pytest.fixture(scope="module")
def million():
    announce(f"million-token inputs B1 T{T} H{H} d{D} bf16, gates U(0.45, 0.9)")
    inp = inputs.dense(1, T, H, D, D, torch.bfloat16, gate="uniform", alpha_lo=0.5, s0_std=0.02, seed=41,
                       device="cuda")
    inp["alpha"].mul_(0.9)
    torch.cuda.synchronize()
    refs = {}
    for end in ENDS:
        lo = max(0, end - WIN)
        win = {key: inp[key][:, lo:end] for key in ("q", "k", "v", "alpha", "beta")}
        win["S0"] = inp["S0"] if lo == 0 else None
        refs[end] = oracle_prefill(win)
    yield inp, refs
    del inp
    torch.cuda.empty_cache()


@pytest.mark.parametrize("sched", ["auto", "two_phase", "overlap", "split"])
def test_million_token_sequence(million, sched):
    import linear_attention_kda_amd as kda
    inp, refs = million
    announce(f"million-token prefill, schedule {sched}")
    ws = torch.empty(kda.chunk_fwd_workspace_size(1, T, H, D, D), dtype=torch.uint8, device="cuda")
    kda.set_schedule(sched)
    try:
        o, S = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], S0=inp["S0"], workspace=ws)
        ran, errs = kda.chunk_fwd_status(ws)
    finally:
        kda.set_schedule("auto")
    print(f"    ran {ran}, schedule errors {errs}", flush=True)
    assert errs == 0
    if sched != "auto":
        assert ran == sched
    for end in ENDS:
        o_ref, S_ref = refs[end]
        lo = max(0, end - WIN)
        first = 0 if lo == 0 else HIST    # checked tokens of the window
        check(f"o[{lo + first}:{end}]", o[:, lo + first:end], o_ref[:, first:], TOL[torch.bfloat16])
        if end == T:
            check("S_final", S, S_ref, TOL[torch.bfloat16])
    del o, S, ws


DN, DH = 2048, 40                  # 81,920 states of 64 KiB
# sequences holding unit 0, units 32767 / 32768 (2^31 bytes), 65535 / 65536
# (2^32 bytes) and the last unit
DSEQ = [0, 819, 1638, DN - 1]


def test_decode_state_past_4gib():
    import linear_attention_kda_amd as kda
    Tk = 4
    announce(f"decode over N{DN} H{DH} d{D} (5.4 GB of state): one step, then {Tk} tokens per launch")
    inp = inputs.dense(DN, Tk, DH, D, D, torch.bfloat16, gate="uniform", alpha_lo=0.95, s0_std=0.02, seed=43,
                       device="cuda")
    S = inp["S0"].clone()
    o1 = kda.decode_step(*(inp[key][:, 0].contiguous() for key in ("q", "k", "v", "alpha", "beta")), S)
    o4, S4 = kda.decode_tokens(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["S0"],
                               S_out=torch.empty_like(inp["S0"]))
    torch.cuda.synchronize()
    idx = torch.tensor(DSEQ, device="cuda")
    for tk, o, St in ((1, o1[:, None], S), (Tk, o4, S4)):
        sub = {key: inp[key].index_select(0, idx)[:, :tk] for key in ("q", "k", "v", "alpha", "beta")}
        sub["S0"] = inp["S0"].index_select(0, idx)
        o_ref, S_ref = oracle_prefill(sub)
        check(f"o ({tk} token)", o.index_select(0, idx), o_ref, TOL[torch.bfloat16])
        check(f"S ({tk} token)", St.index_select(0, idx), S_ref, TOL[torch.bfloat16])
