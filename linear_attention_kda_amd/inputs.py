"""Seeded synthetic inputs for the KDA workloads (no KDA arithmetic here).

One generator serves the GPU path, the oracle checks and the benchmark; the
oracle always receives copies of exactly the tensors the GPU received.

Workloads (names used by tests and the benchmark):
  tiny     B=1 H=2 T=64 d_k=d_v=16 fp32; q,v ~ N(0,1); k ~ N(0,1) then unit
           L2 norm per (token, head); alpha ~ U(0.9,1) per channel;
           beta = sigmoid(N(0,1)); S0 = 0
  prefill  B=4 H=16 T=2048 d=128 bf16 q/k/v (k unit); alpha = exp(-softplus(g)),
           g ~ N(-4,1) per channel, fp32; beta = sigmoid(N(0,1)); S0 = 0
  long     B=1 H=32 T=65536 d=128, distributions of `prefill`;
           S0 ~ N(0, 0.02^2) fp32
  long_share  `long` with H=4: one GPU's share of its heads when they are
           split over eight GPUs
  decode   N=256 sequences, H=32, d=128; state ~ N(0, 0.02^2) fp32; per step
           q/k/v bf16 (k unit), alpha ~ U(0.95,1), beta = sigmoid(N(0,1))
  varlen   64 sequences, lengths round(lognormal(8.3, 0.6)) clipped to
           [128, 16384] and packed with int32 offsets; H=16, d=128 bf16;
           S0 ~ N(0, 0.02^2) per sequence; heads [0, H/4) take
           alpha ~ U(0.999, 1), heads [H/4, H/2) take beta = 1, the rest follow
           `prefill`
Random draws happen in the fixed order lengths -> q -> k -> v -> gate ->
beta -> S0 from one torch.Generator seeded with `seed` on `device`.  q/k/v
are drawn in fp32 and rounded to bf16 (round to nearest even) where the
workload is bf16.  The second parameter of N(., .) is the standard deviation.
"""
from __future__ import annotations

import torch

WORKLOADS = {
    "tiny": dict(kind="dense", B=1, H=2, T=64, dk=16, dv=16, dtype=torch.float32,
                 gate="uniform", alpha_lo=0.9, s0_std=None),
    "prefill": dict(kind="dense", B=4, H=16, T=2048, dk=128, dv=128, dtype=torch.bfloat16,
                    gate="softplus", s0_std=None),
    "long": dict(kind="dense", B=1, H=32, T=65536, dk=128, dv=128, dtype=torch.bfloat16,
                 gate="softplus", s0_std=0.02),
    "long_share": dict(kind="dense", B=1, H=4, T=65536, dk=128, dv=128, dtype=torch.bfloat16,
                       gate="softplus", s0_std=0.02),
    "decode": dict(kind="decode", N=256, H=32, dk=128, dv=128, steps=1024,
                   dtype=torch.bfloat16, alpha_lo=0.95, s0_std=0.02),
    "varlen": dict(kind="packed", n_seq=64, H=16, dk=128, dv=128, dtype=torch.bfloat16,
                   mu=8.3, sigma=0.6, lo=128, hi=16384, gate="softplus", s0_std=0.02,
                   stress=True),
}


def _unit(x: torch.Tensor) -> torch.Tensor:
    return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)


def _gate(shape, gen, device, gate: str, alpha_lo: float = 0.9, form: str = "") -> torch.Tensor:
    """Gates alpha (form ""), log(alpha) ("log") or logits g with
    alpha = exp(-softplus(g)) ("softplus"); the same draws in every form."""
    if gate == "uniform":
        a = torch.empty(shape, device=device).uniform_(alpha_lo, 1.0, generator=gen)
        if form == "softplus":
            return torch.log1p(-a) - torch.log(a)      # alpha = 1 / (1 + e^g)
        return torch.log(a) if form == "log" else a
    g = torch.empty(shape, device=device).normal_(-4.0, 1.0, generator=gen)
    if form == "softplus":
        return g
    la = -torch.nn.functional.softplus(g)
    return la if form == "log" else torch.exp(la)


def _gate_kind(gate_form: str) -> str:
    return gate_form.split("_")[0] if gate_form.startswith(("log_", "softplus_")) else ""


def _gate_shape(lead, dk, gate_form):
    """alpha's shape for a gate form: one value per key channel, one per token
    and head, or none at all."""
    if gate_form in ("channel", "log_channel", "softplus_channel"):
        return (*lead, dk)
    if gate_form in ("scalar", "log_scalar", "softplus_scalar"):
        return tuple(lead)
    if gate_form == "none":
        return None
    raise ValueError(gate_form)


def dense(B, T, H, dk, dv, dtype=torch.bfloat16, gate="softplus", alpha_lo=0.9,
          s0_std=None, seed=0, device="cpu", gate_form="channel"):
    """A dense [B, T, H, .] batch.  Returns a dict of tensors on `device`.
    gate_form "scalar" draws one gate per (token, head), "none" returns
    alpha = None, "log_channel" / "log_scalar" return log(alpha) and
    "softplus_channel" / "softplus_scalar" the logits g (alpha =
    exp(-softplus(g))) of the same draws; the draws of the other tensors do
    not change."""
    gen = torch.Generator(device=device).manual_seed(seed)
    q = torch.empty((B, T, H, dk), device=device).normal_(generator=gen)
    k = _unit(torch.empty((B, T, H, dk), device=device).normal_(generator=gen))
    v = torch.empty((B, T, H, dv), device=device).normal_(generator=gen)
    shape = _gate_shape((B, T, H), dk, gate_form)
    alpha = (_gate(shape, gen, device, gate, alpha_lo, form=_gate_kind(gate_form))
             if shape is not None else None)
    beta = torch.sigmoid(torch.empty((B, T, H), device=device).normal_(generator=gen))
    S0 = None
    if s0_std is not None:
        S0 = torch.empty((B, H, dv, dk), device=device).normal_(0.0, s0_std, generator=gen)
    return dict(q=q.to(dtype), k=k.to(dtype), v=v.to(dtype),
                alpha=alpha.contiguous() if alpha is not None else None,
                beta=beta.contiguous(), S0=S0)


def packed_lengths(n_seq, mu, sigma, lo, hi, seed=0, device="cpu"):
    gen = torch.Generator(device=device).manual_seed(seed)
    x = torch.empty(n_seq, dtype=torch.float64, device=device).log_normal_(mu, sigma, generator=gen)
    return torch.clamp(torch.round(x), lo, hi).to(torch.int64), gen


def packed(lengths, H, dk, dv, dtype=torch.bfloat16, gate="softplus", s0_std=0.02,
           stress=False, gen=None, seed=0, device="cpu", gate_form="channel"):
    """A packed batch of sequences with the given lengths (list or tensor).
    gate_form as for dense(); the stress mix applies to per-channel gates."""
    if gen is None:
        gen = torch.Generator(device=device).manual_seed(seed)
    lengths = torch.as_tensor(lengths, dtype=torch.int64).cpu()
    N = int(lengths.numel())
    cu = torch.zeros(N + 1, dtype=torch.int64)
    cu[1:] = torch.cumsum(lengths, 0)
    T = int(cu[-1])
    q = torch.empty((T, H, dk), device=device).normal_(generator=gen)
    k = _unit(torch.empty((T, H, dk), device=device).normal_(generator=gen))
    v = torch.empty((T, H, dv), device=device).normal_(generator=gen)
    shape = _gate_shape((T, H), dk, gate_form)
    alpha = _gate(shape, gen, device, gate, form=_gate_kind(gate_form)) if shape is not None else None
    beta = torch.sigmoid(torch.empty((T, H), device=device).normal_(generator=gen))
    if stress and alpha is not None and gate_form == "channel":
        q4 = H // 4
        alpha[:, :q4] = torch.empty((T, q4, dk), device=device).uniform_(0.999, 1.0, generator=gen)
        beta[:, q4:2 * q4] = 1.0
    S0 = None
    if s0_std is not None:
        S0 = torch.empty((N, H, dv, dk), device=device).normal_(0.0, s0_std, generator=gen)
    return dict(q=q.to(dtype), k=k.to(dtype), v=v.to(dtype),
                alpha=alpha.contiguous() if alpha is not None else None,
                beta=beta.contiguous(), S0=S0,
                cu_seqlens=cu.to(torch.int32).to(device), lengths=lengths)


def workload(name: str, seed: int = 0, device="cpu"):
    """Inputs of a named prefill workload (tiny, prefill, long, varlen)."""
    w = WORKLOADS[name]
    if w["kind"] == "dense":
        return dense(w["B"], w["T"], w["H"], w["dk"], w["dv"], w["dtype"], w["gate"],
                     w.get("alpha_lo", 0.9), w["s0_std"], seed, device)
    if w["kind"] == "packed":
        lengths, gen = packed_lengths(w["n_seq"], w["mu"], w["sigma"], w["lo"], w["hi"], seed, device)
        return packed(lengths, w["H"], w["dk"], w["dv"], w["dtype"], w["gate"], w["s0_std"],
                      w["stress"], gen=gen, device=device)
    raise ValueError(f"{name} is not a prefill workload")


def decode_state(N=256, H=32, dk=128, dv=128, s0_std=0.02, seed=0, device="cpu"):
    gen = torch.Generator(device=device).manual_seed(seed)
    return torch.empty((N, H, dv, dk), device=device).normal_(0.0, s0_std, generator=gen)


def decode_token(N=256, H=32, dk=128, dv=128, dtype=torch.bfloat16, alpha_lo=0.95, step=0,
                 seed=0, device="cpu"):
    """Inputs of one decode step (seeded by (seed, step))."""
    gen = torch.Generator(device=device).manual_seed(seed * 1_000_003 + 1 + step)
    q = torch.empty((N, H, dk), device=device).normal_(generator=gen)
    k = _unit(torch.empty((N, H, dk), device=device).normal_(generator=gen))
    v = torch.empty((N, H, dv), device=device).normal_(generator=gen)
    alpha = torch.empty((N, H, dk), device=device).uniform_(alpha_lo, 1.0, generator=gen)
    beta = torch.sigmoid(torch.empty((N, H), device=device).normal_(generator=gen))
    return dict(q=q.to(dtype), k=k.to(dtype), v=v.to(dtype), alpha=alpha, beta=beta)
