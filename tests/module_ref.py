"""fp64 references of the operations around the method in a KDA block, for
the tests of kda_chunk_fwd_module (page "K3 架构图解": chapter 08 figure
caption, the KDA module's short convolution, normalisation and output gate;
chapter 05, the RMS norm formula; chapter 09, the convolution is causal).
They are test helpers, not part of the oracle: the oracle takes the
method's inputs, and these turn a block's raw inputs into them (and its
outputs into the block's outputs), written plainly from their definitions.
Their own pins are in tests/test_module_ref.py."""
from __future__ import annotations

import torch

TAPS = 4


def _f64(x):
    return x.detach().to("cpu", torch.float64)


def short_conv(x, w, cu_seqlens=None):
    """Depthwise causal convolution over tokens within each sequence:
    y[t, h, c] = sum_{i=0..3} w[h, c, i] * x[t - 3 + i, h, c], with tokens
    before the sequence's first taken as zero.  x is dense [B, T, H, d] or
    packed [T, H, d] (with cu_seqlens); w is [H, d, 4].  Tokens outside
    every sequence come out zero."""
    x, w = _f64(x), _f64(w)

    def one(xs):  # [T, H, d], one sequence
        T = xs.shape[0]
        y = torch.zeros_like(xs)
        for t in range(T):
            for i in range(TAPS):
                s = t - (TAPS - 1) + i
                if s >= 0:
                    y[t] += w[..., i] * xs[s]
        return y

    if cu_seqlens is None:
        return torch.stack([one(x[b]) for b in range(x.shape[0])])
    cu = [int(c) for c in cu_seqlens.cpu()]
    y = torch.zeros_like(x)
    for a, b in zip(cu[:-1], cu[1:]):
        if b > a:
            y[a:b] = one(x[a:b])
    return y


def silu_unit(x):
    """SiLU, then unit length over the last axis (x / max(|x|, 1e-12))."""
    x = _f64(x)
    x = x * torch.sigmoid(x)
    return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-12)


def rms_norm(o, weight, eps):
    """RMSNorm over the last axis: weight * o / sqrt(mean(o^2) + eps)."""
    o = _f64(o) if isinstance(o, torch.Tensor) else torch.as_tensor(o, dtype=torch.float64)
    return _f64(weight) * o / torch.sqrt((o * o).mean(dim=-1, keepdim=True) + eps)


def out_gate(o, g):
    """Elementwise output gate: o * sigmoid(g)."""
    o = _f64(o) if isinstance(o, torch.Tensor) else torch.as_tensor(o, dtype=torch.float64)
    return o * torch.sigmoid(_f64(g))
