"""Shared helpers for the GPU parity tests (HIP path vs the fp64 oracle)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2}


def announce(msg: str) -> None:
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(d: dict, device="cuda") -> dict:
    return {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def gpu_prefill(inp: dict, scale=None):
    import linear_attention_kda_amd as kda
    o, S = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"],
                         S0=inp.get("S0"), cu_seqlens=inp.get("cu_seqlens"), scale=scale)
    torch.cuda.synchronize()
    return o, S


def oracle_prefill(inp: dict, scale=None, heads=None):
    """Oracle on the same tensors (copied to the host), optionally on a subset
    of heads.  Returns (o, S_final) as float64 numpy arrays."""
    sel = slice(None) if heads is None else list(heads)
    def pick(x, axis):
        if x is None:
            return None
        x = x.detach().cpu()
        return x if heads is None else x.index_select(axis, torch.tensor(sel))
    cu = inp.get("cu_seqlens")
    if cu is None:
        q, k, v, a = (pick(inp[n], 2) for n in ("q", "k", "v", "alpha"))
        b = pick(inp["beta"], 2)
    else:
        q, k, v, a = (pick(inp[n], 1) for n in ("q", "k", "v", "alpha"))
        b = pick(inp["beta"], 1)
    S0 = pick(inp.get("S0"), 1)
    return oracle.fwd(q, k, v, a, b, S0=S0, cu_seqlens=None if cu is None else cu.cpu(),
                      scale=scale)


def rel(x, ref) -> float:
    return oracle.rel_l2(x, ref)


def unit_axes(name: str, ndim: int):
    """The (sequence, head) axes of a checked tensor, from its name and rank:
    states S [N, H, d_v, d_k] -> (0, 1); outputs o [B, T, H, d_v] (dense
    prefill, or [N, Tk, H, d_v] for several decode tokens) -> (0, 2); outputs
    o [N, H, d_v] of a decode step -> (0, 1).  Packed outputs [T, H, d_v]
    need their offsets (check(..., cu=...))."""
    if name.startswith("S"):
        return (0, 1)
    if ndim == 4:
        return (0, 2)
    if ndim == 3:
        return (0, 1)
    raise ValueError(f"no unit axes for {name} of rank {ndim}")


def check(name, got, ref, tol, cu=None):
    """Relative L2 error against the oracle, over the whole tensor and per
    (sequence, head) unit; both must be within tol, so one wrong unit among
    many cannot hide in the whole-tensor figure."""
    r = rel(got, ref)
    if cu is not None:
        per = oracle.unit_rel_l2(got, ref, cu_seqlens=cu)
    else:
        per = oracle.unit_rel_l2(got, ref, unit_axes(name, got.ndim))
    worst = float(per.max()) if per.size else 0.0
    at = tuple(int(i) for i in np.unravel_index(int(per.argmax()), per.shape)) if per.size else ()
    print(f"    {name}: rel_l2 = {r:.3e}, worst (seq, head) {at} = {worst:.3e} (tol {tol:.0e})", flush=True)
    assert np.isfinite(r) and r <= tol, f"{name}: rel_l2 {r:.3e} > {tol:.0e}"
    assert np.isfinite(worst) and worst <= tol, f"{name}: unit {at} rel_l2 {worst:.3e} > {tol:.0e}"
    return r
