"""The chunkwise schedule reaches the token-by-token result (CPU, fp64).

Page "Kimi Delta Attention (KDA)", section "Two schedules for one
recurrence", states that the recurrent and chunkwise forms give identical
states and outputs.  This checks the exact chunk equations the GPU prefill
implements against the oracle, for several chunk sizes, partial last chunks,
d_k != d_v, gates of exactly 0 and 1 and write strengths of 0 and 1.
"""
import numpy as np
import pytest

import oracle
from tests import chunkform_ref


def _case(seed, B, T, H, dk, dv, alpha_lo=0.5, special=False):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    alpha = rng.uniform(alpha_lo, 1.0, (B, T, H, dk))
    beta = rng.uniform(0.0, 1.0, (B, T, H))
    if special:
        alpha[:, ::5, :, ::3] = 0.0
        alpha[:, 1::4] = 1.0
        beta[:, ::3] = 1.0
        beta[:, 2::7] = 0.0
    S0 = 0.1 * rng.standard_normal((B, H, dv, dk))
    return q, k, v, alpha, beta, S0


@pytest.mark.parametrize("C", [1, 4, 16, 64])
@pytest.mark.parametrize("T", [1, 17, 64, 130])
def test_chunk_form_matches_recurrence(C, T):
    q, k, v, alpha, beta, S0 = _case(100 + C + T, 1, T, 2, 8, 6)
    o_ref, S_ref = oracle.fwd(q, k, v, alpha, beta, S0=S0)
    o, S = chunkform_ref.chunk_fwd(q, k, v, alpha, beta, S0=S0, C=C)
    assert np.max(np.abs(o - o_ref)) < 1e-12
    assert np.max(np.abs(S - S_ref)) < 1e-12


def test_chunk_form_special_gates():
    q, k, v, alpha, beta, S0 = _case(7, 2, 70, 2, 16, 16, special=True)
    o_ref, S_ref = oracle.fwd(q, k, v, alpha, beta, S0=S0)
    o, S = chunkform_ref.chunk_fwd(q, k, v, alpha, beta, S0=S0, C=16)
    assert np.max(np.abs(o - o_ref)) < 1e-12
    assert np.max(np.abs(S - S_ref)) < 1e-12


def test_chunk_form_strong_decay():
    """Gates far below 1 (cumulative in-chunk decay far beyond fp32's range
    when multiplied out) are still exact in this form, which never divides."""
    q, k, v, alpha, beta, S0 = _case(8, 1, 64, 1, 8, 8, alpha_lo=0.0)
    alpha *= 1e-3
    o_ref, S_ref = oracle.fwd(q, k, v, alpha, beta, S0=S0)
    o, S = chunkform_ref.chunk_fwd(q, k, v, alpha, beta, S0=S0, C=64)
    assert np.max(np.abs(o - o_ref)) < 1e-12
    assert np.max(np.abs(S - S_ref)) < 1e-12
