"""The O bound of the GPU parity checks (tests/parity.py), on the CPU: the
stated per-dtype tolerance wherever a correctly rounded output can meet it,
and only beyond that half an ulp of the dtype plus the pre-rounding slack."""

import numpy as np
import torch

from parity import PRE_ROUND_SLACK, TOL_OP, bound, ulp


def test_ulp_values():
    assert ulp(np.array([1.0]), torch.bfloat16)[0] == 2.0 ** -7
    assert ulp(np.array([3.0]), torch.bfloat16)[0] == 2.0 ** -6
    assert ulp(np.array([5.0]), torch.float16)[0] == 2.0 ** -8
    assert ulp(np.array([0.75]), torch.float32)[0] == 2.0 ** -24
    # subnormals and zero: the subnormal spacing of the dtype
    assert ulp(np.array([2.4e-5]), torch.float16)[0] == 2.0 ** -24
    assert ulp(np.array([0.0]), torch.float16)[0] == 2.0 ** -24
    assert ulp(np.array([6.2e-5]), torch.float16)[0] == 2.0 ** -24   # smallest normal binade
    assert ulp(np.array([1e-39]), torch.bfloat16)[0] == 2.0 ** -133
    assert ulp(np.array([0.0]), torch.float32)[0] == 2.0 ** -149


def test_stated_bound_where_rounding_can_meet_it():
    vmax = 4.0
    # bf16: |O| < 4 keeps 8e-3 (half an ulp in [2, 4) is 7.8e-3)
    b = bound(np.array([0.0, 0.5, 1.9, 2.0, 3.99]), torch.bfloat16, vmax)
    assert np.all(b == TOL_OP[torch.bfloat16])
    # fp16: |O| < 8 keeps 2e-3 (half an ulp in [4, 8) is 1.95e-3)
    b = bound(np.array([-7.9, 0.1, 3.0, 4.0, 7.99]), torch.float16, vmax)
    assert np.all(b == TOL_OP[torch.float16])
    # fp32: |O| < 256 keeps 1e-5
    b = bound(np.array([1.0, 200.0, -255.0]), torch.float32, vmax)
    assert np.all(b == TOL_OP[torch.float32])


def test_relaxed_only_beyond():
    vmax = 4.0
    b = bound(np.array([4.0, -6.0]), torch.bfloat16, vmax)
    assert np.allclose(b, 2.0 ** -6 + PRE_ROUND_SLACK * vmax)  # half of 2^-5
    b = bound(np.array([9.0]), torch.float16, vmax)
    assert np.allclose(b, 2.0 ** -8 + PRE_ROUND_SLACK * vmax)  # half of 2^-7
    b = bound(np.array([300.0]), torch.float32, vmax)
    assert np.allclose(b, 2.0 ** -16 + PRE_ROUND_SLACK * vmax)  # half of 2^-15
