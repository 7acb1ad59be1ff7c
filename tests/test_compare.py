"""The comparison the parity tests rest on (oracle.rel_l2 and the per-unit
oracle.unit_rel_l2), checked on small vectors whose errors are worked out by
hand, so a slip in the helper (a missing square root, a sum over the wrong
axis, a unit taken from the wrong tokens) cannot make a bad GPU result pass."""
import math

import numpy as np
import pytest
import torch

import oracle


def test_rel_l2_hand_values():
    # |x - ref| = |(0, 2, 2)| = sqrt(8), |ref| = 1
    assert oracle.rel_l2([1.0, 2.0, 2.0], [1.0, 0.0, 0.0]) == pytest.approx(math.sqrt(8.0), rel=1e-15)
    # x = 2 ref: the error is ref itself
    assert oracle.rel_l2([2.0, -4.0, 6.0], [1.0, -2.0, 3.0]) == pytest.approx(1.0, rel=1e-15)
    # equal inputs: exactly zero
    assert oracle.rel_l2([0.5, -0.25], [0.5, -0.25]) == 0.0
    # an all-zero reference gives the absolute error |(3, 4)| = 5
    assert oracle.rel_l2([3.0, 4.0], [0.0, 0.0]) == pytest.approx(5.0, rel=1e-15)
    # |(1, 1, 1, 1)| / |(2, 2, 2, 2)| = 2 / 4 over a 2 x 2 array (whole array, not per row)
    assert oracle.rel_l2([[3.0, 1.0], [3.0, 1.0]], [[2.0, 2.0], [2.0, 2.0]]) == pytest.approx(0.5, rel=1e-15)


def test_rel_l2_takes_bf16_tensors_exactly():
    # 1 + 2^-7 is a bf16 value; the upcast must not round it away
    x = torch.tensor([1.0 + 2 ** -7, 0.0], dtype=torch.bfloat16)
    ref = torch.tensor([1.0, 0.0], dtype=torch.float64)
    assert oracle.rel_l2(x, ref) == 2 ** -7


def test_unit_rel_l2_dense_axes():
    # o [B=2, T=3, H=2, d=2]; unit (b, h) sums over t and d
    ref = np.ones((2, 3, 2, 2))
    x = ref.copy()
    x[1, 0, 0, 1] += 3.0       # unit (1, 0): error 3 over a reference of norm sqrt(6)
    x[0, 2, 1, 0] -= 0.5       # unit (0, 1): error 0.5
    per = oracle.unit_rel_l2(x, ref, (0, 2))
    want = np.array([[0.0, 0.5 / math.sqrt(6.0)], [3.0 / math.sqrt(6.0), 0.0]])
    np.testing.assert_allclose(per, want, rtol=1e-15, atol=0)
    # the same tensor read with the axes swapped gives the transpose
    np.testing.assert_allclose(oracle.unit_rel_l2(x, ref, (2, 0)), want.T, rtol=1e-15, atol=0)


def test_unit_rel_l2_states():
    # S [N=3, H=1, 2, 2]: unit n uses only S[n]
    ref = np.zeros((3, 1, 2, 2))
    ref[0, 0] = [[1.0, 0.0], [0.0, 0.0]]
    ref[1, 0] = [[0.0, 2.0], [0.0, 0.0]]
    x = ref.copy()
    x[0, 0, 1, 1] = 1.0        # error 1 against norm 1
    x[2, 0, 0, 0] = 0.25       # zero reference: absolute error 0.25
    per = oracle.unit_rel_l2(x, ref, (0, 1))
    np.testing.assert_allclose(per[:, 0], [1.0, 0.0, 0.25], rtol=1e-15, atol=0)


def test_unit_rel_l2_packed_segments():
    # packed o [T=6, H=2, d=1]; sequences own tokens [0, 2), [2, 2) (empty), [2, 6)
    cu = np.array([0, 2, 2, 6])
    ref = np.arange(1.0, 13.0).reshape(6, 2, 1)
    x = ref.copy()
    x[1, 1, 0] += 4.0          # sequence 0, head 1
    x[5, 0, 0] += 1.0          # sequence 2, head 0
    per = oracle.unit_rel_l2(x, ref, cu_seqlens=cu)
    assert per.shape == (3, 2)
    # sequence 0 head 1: tokens 0, 1 hold 2 and 4
    assert per[0, 1] == pytest.approx(4.0 / math.sqrt(4 + 16), rel=1e-15)
    # sequence 2 head 0: tokens 2..5 hold 5, 7, 9, 11
    assert per[2, 0] == pytest.approx(1.0 / math.sqrt(25 + 49 + 81 + 121), rel=1e-15)
    # untouched units and the empty sequence are exact
    assert per[0, 0] == 0.0 and per[2, 1] == 0.0 and per[1, 0] == 0.0 and per[1, 1] == 0.0
    # an error placed on the token just past a sequence's end belongs to the next one
    y = ref.copy()
    y[2, 0, 0] += 1.0
    per = oracle.unit_rel_l2(y, ref, cu_seqlens=torch.tensor(cu, dtype=torch.int32))
    assert per[0, 0] == 0.0 and per[2, 0] > 0.0


def test_unit_rel_l2_rejects_shape_mismatch():
    with pytest.raises(ValueError):
        oracle.unit_rel_l2(np.zeros((2, 2, 2)), np.zeros((2, 2, 3)))


def test_check_catches_one_wrong_unit():
    """One (sequence, head) unit of 64 off by 15 % keeps the whole-tensor
    error under the bf16 tolerance of 2e-2, so only the per-unit check in
    tests/gpu_cases.check() can catch it."""
    from tests.gpu_cases import check
    g = np.random.default_rng(0)
    ref = g.standard_normal((4, 32, 16, 8))          # o [B, T, H, d]: 64 units
    got = ref * (1.0 + 1e-3 * g.standard_normal(ref.shape))
    got[2, :, 5, :] *= 1.15
    assert oracle.rel_l2(got, ref) < 2e-2
    with pytest.raises(AssertionError, match=r"unit \(2, 5\)"):
        check("o", got, ref, 2e-2)
    S_ref = g.standard_normal((4, 16, 8, 8))
    S_got = S_ref.copy()
    S_got[3, 7] *= 1.15
    with pytest.raises(AssertionError, match=r"unit \(3, 7\)"):
        check("S_final", S_got, S_ref, 2e-2)
    # a packed batch: the unit is found from the offsets
    cu = np.array([0, 10, 10, 128])
    P_ref = g.standard_normal((128, 64, 8))
    P_got = P_ref.copy()
    P_got[10:128, 3] *= 1.15
    assert oracle.rel_l2(P_got, P_ref) < 2e-2
    with pytest.raises(AssertionError, match=r"unit \(2, 3\)"):
        check("o", P_got, P_ref, 2e-2, cu=cu)
