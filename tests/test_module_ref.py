"""Pins of the test-side fp64 references of the block's operations around
the method (tests/module_ref.py), on the CPU: each against a fact that
follows from its definition, not against a retyped formula."""
import math

import torch

from tests import module_ref as mr


def test_conv_impulse_response_reads_taps_backwards():
    # a unit impulse at token 2 of a sequence: outputs at tokens 2..5 are the
    # taps for the current token, one back, two back, three back
    H, d, T = 2, 3, 9
    w = torch.arange(H * d * 4, dtype=torch.float64).reshape(H, d, 4) + 1
    x = torch.zeros(1, T, H, d, dtype=torch.float64)
    x[0, 2] = 1.0
    y = mr.short_conv(x, w)[0]
    for lag in range(4):
        assert torch.equal(y[2 + lag], w[..., 3 - lag])
    assert torch.count_nonzero(y[:2]) == 0 and torch.count_nonzero(y[6:]) == 0


def test_conv_identity_and_shift_taps():
    g = torch.Generator().manual_seed(1)
    x = torch.randn(2, 7, 3, 5, generator=g, dtype=torch.float64)
    ident = torch.zeros(3, 5, 4, dtype=torch.float64)
    ident[..., 3] = 1.0
    assert torch.equal(mr.short_conv(x, ident), x)
    shift = torch.zeros(3, 5, 4, dtype=torch.float64)
    shift[..., 0] = 1.0      # three tokens back
    y = mr.short_conv(x, shift)
    assert torch.equal(y[:, 3:], x[:, :-3]) and torch.count_nonzero(y[:, :3]) == 0


def test_conv_does_not_cross_sequences():
    # packed: the first tokens of the second sequence see zeros, not the end
    # of the first; the same tokens run alone give the same outputs
    g = torch.Generator().manual_seed(2)
    x = torch.randn(10, 2, 4, generator=g, dtype=torch.float64)
    w = torch.randn(2, 4, 4, generator=g, dtype=torch.float64)
    cu = torch.tensor([0, 6, 6, 10], dtype=torch.int32)
    y = mr.short_conv(x, w, cu)
    assert torch.allclose(y[6:], mr.short_conv(x[None, 6:], w)[0], rtol=0, atol=0)
    assert torch.allclose(y[:6], mr.short_conv(x[None, :6], w)[0], rtol=0, atol=0)
    # linearity in x
    assert torch.allclose(mr.short_conv(2 * x, w, cu), 2 * y, rtol=1e-15, atol=0)


def test_rms_norm_scale_invariance_and_unit_rms():
    g = torch.Generator().manual_seed(3)
    o = torch.randn(5, 4, 16, generator=g, dtype=torch.float64)
    ones = torch.ones(16, dtype=torch.float64)
    y = mr.rms_norm(o, ones, 0.0)
    # the root mean square of each row is 1, and rescaling a row changes nothing
    assert torch.allclose((y * y).mean(-1), torch.ones(5, 4, dtype=torch.float64), rtol=1e-14)
    assert torch.allclose(mr.rms_norm(7.5 * o, ones, 0.0), y, rtol=1e-14)
    # gains act per channel
    wgt = torch.linspace(0.5, 2.0, 16, dtype=torch.float64)
    assert torch.allclose(mr.rms_norm(o, wgt, 0.0), y * wgt, rtol=1e-14)
    # a constant row c with eps: c / sqrt(c^2 + eps)
    c = torch.full((1, 16), 0.3, dtype=torch.float64)
    assert math.isclose(float(mr.rms_norm(c, ones, 0.01)[0, 0]), 0.3 / math.sqrt(0.09 + 0.01), rel_tol=1e-14)


def test_out_gate_values():
    o = torch.tensor([2.0, -4.0, 1.0], dtype=torch.float64)
    g = torch.tensor([0.0, math.log(3.0), -math.inf], dtype=torch.float64)
    # sigmoid(0) = 1/2, sigmoid(ln 3) = 3/4, sigmoid(-inf) = 0
    assert torch.allclose(mr.out_gate(o, g), torch.tensor([1.0, -3.0, 0.0], dtype=torch.float64), rtol=1e-15)


def test_silu_unit_is_unit_and_matches_silu_direction():
    g = torch.Generator().manual_seed(4)
    x = torch.randn(6, 3, 32, generator=g, dtype=torch.float64)
    y = mr.silu_unit(x)
    assert torch.allclose(y.norm(dim=-1), torch.ones(6, 3, dtype=torch.float64), rtol=1e-14)
    s = x / (1 + torch.exp(-x))
    assert torch.allclose(y * s.norm(dim=-1, keepdim=True), s, rtol=1e-13)
