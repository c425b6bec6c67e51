"""CPU checks of the comparison rule the GPU parity tests use (tests/pa_harness.py):
the unit in the last place of each output type and the per-element bound
max(max-abs tolerance, 1 ulp)."""
import numpy as np
import pytest

pytest.importorskip("torch")
from tests.pa_harness import TOL, compare, elementwise_bound, ulp  # noqa: E402


def test_ulp_of_each_type():
    # bf16: 8 significant bits -> spacing 2^-7 on [1, 2), 2^-8 on [0.5, 1)
    assert ulp(np.array([1.0, 1.5, 0.75, 0.25, -3.0]), "bf16").tolist() == [2 ** -7, 2 ** -7, 2 ** -8, 2 ** -9,
                                                                            2 ** -6]
    # f16: 11 significant bits
    assert ulp(np.array([1.0, 0.3, 2048.0]), "f16").tolist() == [2 ** -10, 2 ** -12, 2.0]
    assert ulp(np.array([0.0]), "f16").tolist() == [2 ** -24]
    # f32 agrees with numpy's spacing
    x = np.array([1.0, 3.5, 1e-3, 7e5], dtype=np.float32)
    assert np.array_equal(ulp(x, "f32"), np.spacing(x).astype(np.float64))
    # f16 agrees with numpy's spacing on normal numbers
    h = np.array([0.001, 0.5, 1.25, 60000.0], dtype=np.float16)
    assert np.array_equal(ulp(h, "f16"), np.spacing(h).astype(np.float64))


def test_bound_is_abs_tolerance_below_quarter_and_one_ulp_above():
    b = elementwise_bound(np.array([0.1, 0.2, 0.5, 1.0, -2.0]), "bf16")
    assert b.tolist() == [2e-3, 2e-3, 2 ** -8, 2 ** -7, 2 ** -6]
    assert elementwise_bound(np.array([1.0, 3.0]), "f16").tolist() == [2e-3, 2e-3]
    assert elementwise_bound(np.array([5.0]), "f16").tolist() == [2 ** -8]
    assert elementwise_bound(np.array([1.0]), "f32").tolist() == [TOL["f32"][0]]


def test_compare_counts_elements_beyond_the_bound():
    import torch
    ref = np.array([[[0.6, 0.1, -0.3]]])
    bf = lambda a: torch.tensor(a, dtype=torch.float64).to(torch.bfloat16)  # noqa: E731
    # one bf16 step away at 0.6 (spacing 2^-8): inside the bound
    got = bf([[[0.6 + 2 ** -8, 0.1, -0.3]]])
    rep = compare(got, ref, "bf16")
    assert rep.over_bound == 0 and rep.max_abs > 2e-3
    # two steps away: outside
    got = bf([[[0.6 + 2 * 2 ** -8, 0.1, -0.3]]])
    assert compare(got, ref, "bf16").over_bound == 1
    # a NaN is never inside the bound
    got = torch.tensor([[[float("nan"), 0.1, -0.3]]]).to(torch.bfloat16)
    assert compare(got, ref, "bf16").over_bound == 1
