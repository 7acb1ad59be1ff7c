"""Pins for the fp64 oracle: facts the pages and plain mathematics fix.

Each ``pin_*`` takes an oracle object (``oracle.Oracle``) and raises
AssertionError when the oracle disagrees with the fact.  They are written so
that a plausible slip anywhere in the oracle (a dropped term, a wrong sign, a
swapped operand, the wrong axis for the decay, the wrong order of the steps, a
lost initial state, an off-by-one in the token or sequence indexing) breaks at
least one of them; ``test_oracle_pins.py`` checks that claim by planting such
slips in copies of the oracle source.

Citations are to the pages by title and section:
 * [KDA]  "Kimi Delta Attention (KDA)" (brain.bigb.es)
 * [K3]   "K3 架构图解" / K3 architecture illustrated (huaweidata.com)
 * [GPT2] "22580: from GPT-2 to Kimi K3, explained" (temp07.ru)
"""
from __future__ import annotations

import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TOL = 1e-12


def _unit(rng, *shape):
    x = rng.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _inputs(rng, B, T, H, dk, dv, alpha_lo=0.5, beta=None, alpha=None,
            unit_k=True):
    q = rng.standard_normal((B, T, H, dk))
    k = _unit(rng, B, T, H, dk) if unit_k else rng.standard_normal((B, T, H, dk))
    v = rng.standard_normal((B, T, H, dv))
    if alpha is None:
        alpha = rng.uniform(alpha_lo, 1.0, (B, T, H, dk))
    else:
        alpha = np.full((B, T, H, dk), float(alpha))
    if beta is None:
        beta = rng.uniform(0.0, 1.0, (B, T, H))
    else:
        beta = np.full((B, T, H), float(beta))
    return q, k, v, alpha, beta


def _close(a, b, tol=TOL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 0.0)
    assert err <= tol * scale, f"{what}: max abs err {err:.3e} (scale {scale:.3e})"


def _step_states(orc, q, k, v, alpha, beta, S0):
    """States after every token of a dense [1,T,H,...] batch, by decode steps.

    Returns (states, outs): states[t] is the state after token t-1
    (states[0] = S0), outs[t] the output of token t; shapes [H,dv,dk] / [H,dv].
    """
    T = q.shape[1]
    S = S0.copy()
    states, outs = [S0[0].copy()], []
    for t in range(T):
        o, S = orc.decode(q[:, t], k[:, t], v[:, t], alpha[:, t], beta[:, t], S)
        states.append(S[0].copy())
        outs.append(o[0])
    return states, outs


# ---------------------------------------------------------------- worked example
def pin_worked_example(orc):
    """[K3] chapter 08 ("How KDA and MLA mix"): a unit key that used to map to
    1, a new value 3, no forgetting and a full-strength write leave 1+(3-1)=3."""
    with open(os.path.join(GOLDEN, "worked_example_k3_ch08.json")) as f:
        g = json.load(f)
    one = lambda x: np.asarray(x, dtype=np.float64).reshape(1, 1, 1, -1)
    o, S = orc.fwd(one(g["q"]), one(g["k"]), one(g["v"]), one(g["alpha"]),
                   np.full((1, 1, 1), g["beta"]),
                   S0=np.asarray(g["S0"], dtype=np.float64).reshape(1, 1, 1, 1),
                   scale=g["scale"])
    _close(S.ravel(), g["expected_S"], 0.0, "worked example state")
    _close(o.ravel(), g["expected_o"], 0.0, "worked example output")


# ------------------------------------------------------ DeltaNet readback facts
def pin_readback_full_write(orc):
    """[KDA] "DeltaNet: write the error instead of the value": with beta_t = 1
    and a unit key, reading the new state back with k_t returns exactly v_t."""
    rng = np.random.default_rng(11)
    H, dk, dv, T = 2, 8, 6, 6
    q, k, v, alpha, beta = _inputs(rng, 1, T, H, dk, dv, beta=1.0)
    S0 = rng.standard_normal((1, H, dv, dk))
    states, _ = _step_states(orc, q, k, v, alpha, beta, S0)
    for t in range(T):
        for h in range(H):
            _close(states[t + 1][h] @ k[0, t, h], v[0, t, h], TOL, f"readback t={t}")


def pin_partial_write(orc):
    """[KDA] DeltaNet section: reading back with the written key interpolates,
    S_t k_t = (1-beta_t) S~_t k_t + beta_t v_t, where (section "KDA") the
    pre-write state is S~_t = S_{t-1} Diag(alpha_t), so S~_t k_t is
    S_{t-1} applied to the elementwise product alpha_t * k_t."""
    rng = np.random.default_rng(12)
    H, dk, dv, T = 2, 8, 6, 6
    q, k, v, alpha, beta = _inputs(rng, 1, T, H, dk, dv)
    S0 = rng.standard_normal((1, H, dv, dk))
    states, _ = _step_states(orc, q, k, v, alpha, beta, S0)
    for t in range(T):
        for h in range(H):
            b = beta[0, t, h]
            pre = states[t][h] @ (alpha[0, t, h] * k[0, t, h])
            _close(states[t + 1][h] @ k[0, t, h], (1 - b) * pre + b * v[0, t, h],
                   TOL, f"partial write t={t}")


def pin_locality(orc):
    """[KDA] DeltaNet section: the rank-one write leaves every direction
    orthogonal to k_t untouched, (S_t - S~_t) x = 0 for x orthogonal to k_t."""
    rng = np.random.default_rng(13)
    H, dk, dv, T = 2, 8, 6, 6
    q, k, v, alpha, beta = _inputs(rng, 1, T, H, dk, dv)
    S0 = rng.standard_normal((1, H, dv, dk))
    states, _ = _step_states(orc, q, k, v, alpha, beta, S0)
    for t in range(T):
        for h in range(H):
            kt = k[0, t, h]
            x = rng.standard_normal(dk)
            x = x - (x @ kt) * kt
            pre = states[t][h] @ (alpha[0, t, h] * x)
            _close(states[t + 1][h] @ x, pre, TOL, f"locality t={t}")


def pin_gradient_step(orc):
    """[KDA] DeltaNet section: the update is one gradient-descent step with
    learning rate beta_t on the loss 0.5*||S k_t - v_t||^2, taken from the
    decayed state.  The gradient comes from torch autograd, not from a formula."""
    import torch
    rng = np.random.default_rng(14)
    H, dk, dv, T = 1, 7, 5, 4
    q, k, v, alpha, beta = _inputs(rng, 1, T, H, dk, dv)
    S0 = rng.standard_normal((1, H, dv, dk))
    states, _ = _step_states(orc, q, k, v, alpha, beta, S0)
    for t in range(T):
        pre = torch.tensor(states[t][0] * alpha[0, t, 0][None, :],
                           dtype=torch.float64, requires_grad=True)
        kt = torch.tensor(k[0, t, 0], dtype=torch.float64)
        vt = torch.tensor(v[0, t, 0], dtype=torch.float64)
        loss = 0.5 * torch.sum((pre @ kt - vt) ** 2)
        loss.backward()
        expect = (pre - beta[0, t, 0] * pre.grad).detach().numpy()
        _close(states[t + 1][0], expect, TOL, f"gradient step t={t}")


# --------------------------------------------------------- reductions / forms
def pin_deltanet_reduction(orc):
    """[KDA] DeltaNet section, expanded form, and [GPT2] section "DeltaNet /
    Parallelizing ... with Delta rule": with alpha = 1 the update is
    S_t = S_{t-1}(I - beta_t k_t k_t^T) + beta_t v_t k_t^T, and o_t reads
    the new state (scaled by d_k^-1/2 per [KDA] opening equation)."""
    rng = np.random.default_rng(15)
    H, dk, dv, T = 2, 8, 6, 7
    q, k, v, alpha, beta = _inputs(rng, 1, T, H, dk, dv, alpha=1.0)
    S0 = rng.standard_normal((1, H, dv, dk))
    o, Sf = orc.fwd(q, k, v, alpha, beta, S0=S0)
    s = dk ** -0.5
    for h in range(H):
        S = S0[0, h].copy()
        for t in range(T):
            kt, b = k[0, t, h], beta[0, t, h]
            S = S @ (np.eye(dk) - b * np.outer(kt, kt)) + b * np.outer(v[0, t, h], kt)
            _close(o[0, t, h], s * S @ q[0, t, h], TOL, f"deltanet o t={t}")
        _close(Sf[0, h], S, TOL, "deltanet state")


def pin_frozen_state(orc):
    """[KDA] Gated DeltaNet section with alpha = 1 (no forgetting) and the
    DeltaNet correction with beta = 0 (no write): the state never changes and
    every output reads S0."""
    rng = np.random.default_rng(16)
    H, dk, dv, T = 3, 8, 6, 5
    q, k, v, alpha, beta = _inputs(rng, 1, T, H, dk, dv, alpha=1.0, beta=0.0)
    S0 = rng.standard_normal((1, H, dv, dk))
    o, Sf = orc.fwd(q, k, v, alpha, beta, S0=S0)
    _close(Sf, S0, TOL, "frozen state")
    expect = np.einsum("hvk,thk->thv", S0[0], q[0]) * dk ** -0.5
    _close(o[0], expect, TOL, "frozen outputs")


def pin_linear_attention(orc):
    """[KDA] section "Dropping softmax turns attention into state": without
    the softmax the read is o_t = sum_{i<=t} (k_i^T q_t) v_i.  With orthonormal
    keys, a zero start, alpha = 1 and beta = 1 the delta rule subtracts nothing
    (each new key is orthogonal to everything stored) so KDA gives exactly that
    sum, scaled by d_k^-1/2, and the final state is sum_i v_i k_i^T."""
    rng = np.random.default_rng(17)
    H, dk, dv, T = 2, 8, 5, 8
    q = rng.standard_normal((1, T, H, dk))
    v = rng.standard_normal((1, T, H, dv))
    k = np.empty((1, T, H, dk))
    for h in range(H):
        Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
        k[0, :, h] = Qm[:, :T].T
    alpha = np.ones((1, T, H, dk))
    beta = np.ones((1, T, H))
    o, Sf = orc.fwd(q, k, v, alpha, beta)
    s = dk ** -0.5
    for h in range(H):
        for t in range(T):
            expect = sum((k[0, i, h] @ q[0, t, h]) * v[0, i, h] for i in range(t + 1))
            _close(o[0, t, h], s * expect, TOL, f"linear attention t={t}")
        _close(Sf[0, h], sum(np.outer(v[0, i, h], k[0, i, h]) for i in range(T)),
               TOL, "linear attention state")


def pin_dplr_form(orc):
    """[KDA] section "KDA": the expanded recurrence
    S_t = S_{t-1} A_t + beta_t v_t k_t^T with the diagonal-plus-rank-one
    transition A_t = D_t - (D_t k_t)(beta_t k_t)^T, D_t = Diag(alpha_t);
    o_t = d_k^-1/2 S_t q_t.  Checked over a whole sequence, d_k != d_v,
    keys not normalised (the identity holds for any k)."""
    rng = np.random.default_rng(18)
    H, dk, dv, T = 2, 8, 6, 9
    q, k, v, alpha, beta = _inputs(rng, 1, T, H, dk, dv, alpha_lo=0.0, unit_k=False)
    S0 = rng.standard_normal((1, H, dv, dk))
    o, Sf = orc.fwd(q, k, v, alpha, beta, S0=S0)
    s = dk ** -0.5
    for h in range(H):
        S = S0[0, h].copy()
        for t in range(T):
            D = np.diag(alpha[0, t, h])
            kt, b = k[0, t, h], beta[0, t, h]
            A = D - np.outer(D @ kt, b * kt)
            S = S @ A + b * np.outer(v[0, t, h], kt)
            _close(o[0, t, h], s * S @ q[0, t, h], TOL, f"dplr o t={t}")
        _close(Sf[0, h], S, TOL, "dplr state")


def pin_transposed_form(orc):
    """[K3] chapter 08 writes the same update on the transposed state
    (d_k x d_v): decay rows with Diag(alpha), predict with the transpose,
    write beta k (v - vhat)^T, read S^T q (that page applies no scale; the
    d_k^-1/2 of [KDA] is applied here to compare).  Its state is the
    transpose of ours."""
    rng = np.random.default_rng(19)
    H, dk, dv, T = 1, 8, 6, 6
    q, k, v, alpha, beta = _inputs(rng, 1, T, H, dk, dv)
    S0 = rng.standard_normal((1, H, dv, dk))
    o, Sf = orc.fwd(q, k, v, alpha, beta, S0=S0)
    St = S0[0, 0].T.copy()  # d_k x d_v
    for t in range(T):
        Sh = np.diag(alpha[0, t, 0]) @ St
        vh = Sh.T @ k[0, t, 0]
        St = Sh + beta[0, t, 0] * np.outer(k[0, t, 0], v[0, t, 0] - vh)
        _close(o[0, t, 0], dk ** -0.5 * (St.T @ q[0, t, 0]), TOL, f"p2 form o t={t}")
    _close(Sf[0, 0], St.T, TOL, "p2 form state")


def pin_full_forget(orc):
    """alpha_t = 0 on every channel clears the memory before the write
    ([GPT2] "Gated Delta Net": a gate of zero wipes the memory), so
    S_t = beta_t v_t k_t^T and o_t = d_k^-1/2 beta_t (k_t^T q_t) v_t."""
    rng = np.random.default_rng(20)
    H, dk, dv, T = 2, 8, 6, 3
    q, k, v, alpha, beta = _inputs(rng, 1, T, H, dk, dv, alpha=0.0)
    S0 = rng.standard_normal((1, H, dv, dk))
    o, Sf = orc.fwd(q, k, v, alpha, beta, S0=S0)
    for h in range(H):
        for t in range(T):
            b = beta[0, t, h]
            _close(o[0, t, h], dk ** -0.5 * b * (k[0, t, h] @ q[0, t, h]) * v[0, t, h],
                   TOL, f"full forget o t={t}")
        _close(Sf[0, h], beta[0, -1, h] * np.outer(v[0, -1, h], k[0, -1, h]), TOL,
               "full forget state")


def pin_scale(orc):
    """[KDA] opening equation: the read is scaled by d_k^-1/2 and the state is
    not.  The default scale must equal an explicit 1/sqrt(d_k)."""
    rng = np.random.default_rng(21)
    H, dk, dv, T = 2, 16, 6, 4
    q, k, v, alpha, beta = _inputs(rng, 1, T, H, dk, dv)
    S0 = rng.standard_normal((1, H, dv, dk))
    o1, S1 = orc.fwd(q, k, v, alpha, beta, S0=S0)
    o2, S2 = orc.fwd(q, k, v, alpha, beta, S0=S0, scale=1.0)
    _close(S1, S2, 0.0, "state independent of scale")
    _close(o1, o2 * 0.25, TOL, "default scale is d_k^-1/2")


# ------------------------------------------------------------------ invariants
def pin_nonexpansive(orc):
    """[KDA] DeltaNet section: I - beta k k^T has eigenvalue 1 - beta along a
    unit k and 1 elsewhere, so it never grows a vector; with alpha in [0,1]
    each transition A_t is non-expansive.  With v = 0 the Frobenius norm of
    the state can only shrink, also for nearly parallel keys."""
    rng = np.random.default_rng(22)
    H, dk, dv, T = 2, 8, 6, 40
    q, k, v, alpha, beta = _inputs(rng, 1, T, H, dk, dv, alpha_lo=0.9)
    v[:] = 0.0
    base = _unit(rng, dk)
    k[0, T // 2:] = base + 0.05 * rng.standard_normal((T - T // 2, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    S0 = rng.standard_normal((1, H, dv, dk))
    states, _ = _step_states(orc, q, k, v, alpha, beta, S0)
    for t in range(T):
        n0 = np.linalg.norm(states[t], axis=(1, 2))
        n1 = np.linalg.norm(states[t + 1], axis=(1, 2))
        assert np.all(n1 <= n0 * (1 + 1e-14)), f"norm grew at t={t}"
    # and the map is not the identity: something decayed
    assert np.all(np.linalg.norm(states[-1], axis=(1, 2)) <
                  0.99 * np.linalg.norm(states[0], axis=(1, 2)))


# --------------------------------------------------------------- composition
def pin_split_sequence(orc):
    """The recurrence is a left-to-right scan ([KDA] opening equation), so
    running T1 tokens, then T2 tokens from the resulting state, equals one run
    over T1+T2 tokens."""
    rng = np.random.default_rng(23)
    H, dk, dv, T1, T2 = 2, 8, 6, 5, 7
    q, k, v, alpha, beta = _inputs(rng, 1, T1 + T2, H, dk, dv)
    S0 = rng.standard_normal((1, H, dv, dk))
    o, Sf = orc.fwd(q, k, v, alpha, beta, S0=S0)
    oa, Sa = orc.fwd(q[:, :T1], k[:, :T1], v[:, :T1], alpha[:, :T1], beta[:, :T1], S0=S0)
    ob, Sb = orc.fwd(q[:, T1:], k[:, T1:], v[:, T1:], alpha[:, T1:], beta[:, T1:], S0=Sa)
    _close(np.concatenate([oa, ob], axis=1), o, TOL, "split outputs")
    _close(Sb, Sf, TOL, "split state")


def pin_decode_matches_fwd(orc):
    """One decode step per token reproduces the whole-sequence forward,
    for several sequences and heads at once."""
    rng = np.random.default_rng(24)
    B, H, dk, dv, T = 3, 2, 8, 6, 5
    q, k, v, alpha, beta = _inputs(rng, B, T, H, dk, dv)
    S0 = rng.standard_normal((B, H, dv, dk))
    o, Sf = orc.fwd(q, k, v, alpha, beta, S0=S0)
    S = S0.copy()
    for t in range(T):
        ot, S = orc.decode(q[:, t], k[:, t], v[:, t], alpha[:, t], beta[:, t], S)
        _close(ot, o[:, t], TOL, f"decode o t={t}")
    _close(S, Sf, TOL, "decode state")


def pin_packed_batch(orc):
    """A packed batch with offsets (cu_seqlens) equals independent runs, one
    per sequence; no state flows between sequences; a zero-length sequence
    returns its S0 unchanged."""
    rng = np.random.default_rng(25)
    H, dk, dv = 2, 8, 6
    lens = [5, 0, 1, 9, 3]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    Ttot = int(cu[-1])
    q, k, v, alpha, beta = _inputs(rng, 1, Ttot, H, dk, dv)
    S0 = rng.standard_normal((len(lens), H, dv, dk))
    o, Sf = orc.fwd(q[0], k[0], v[0], alpha[0], beta[0], S0=S0, cu_seqlens=cu)
    for n, L in enumerate(lens):
        a, b = cu[n], cu[n + 1]
        on, Sn = orc.fwd(q[:, a:b], k[:, a:b], v[:, a:b], alpha[:, a:b],
                         beta[:, a:b], S0=S0[n:n + 1])
        _close(o[a:b], on[0], TOL, f"packed o seq {n}")
        _close(Sf[n], Sn[0], TOL, f"packed state seq {n}")
    _close(Sf[1], S0[1], 0.0, "zero-length sequence keeps S0")


def pin_empty(orc):
    """Zero tokens: the final state is the initial state (zero without S0)."""
    rng = np.random.default_rng(26)
    H, dk, dv = 2, 8, 6
    z = lambda d: np.zeros((2, 0, H, d))
    S0 = rng.standard_normal((2, H, dv, dk))
    o, Sf = orc.fwd(z(dk), z(dk), z(dv), z(dk), np.zeros((2, 0, H)), S0=S0)
    assert o.shape == (2, 0, H, dv)
    _close(Sf, S0, 0.0, "empty keeps S0")
    o, Sf = orc.fwd(z(dk), z(dk), z(dv), z(dk), np.zeros((2, 0, H)))
    _close(Sf, np.zeros_like(S0), 0.0, "empty zero state")


ALL_PINS = [
    pin_worked_example, pin_readback_full_write, pin_partial_write,
    pin_locality, pin_gradient_step, pin_deltanet_reduction, pin_frozen_state,
    pin_linear_attention, pin_dplr_form, pin_transposed_form, pin_full_forget,
    pin_scale, pin_nonexpansive, pin_split_sequence, pin_decode_matches_fwd,
    pin_packed_batch, pin_empty,
]
