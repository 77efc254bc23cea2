"""The bf16 acceptance rule of the GPU parity tests, checked on the CPU: the
bf16 unit in the last place, and what the element-wise gate accepts and
rejects."""
import numpy as np
import torch

from tests.gpu_util import assert_parity, bf16_gate, bf16_ulp, compare
from workloads import small_spec


def test_bf16_ulp_is_the_gap_to_the_next_bf16_value():
    rng = np.random.default_rng(3)
    y = rng.standard_normal(4096) * np.exp2(rng.integers(-20, 20, 4096))
    b = torch.tensor(y, dtype=torch.float32).to(torch.bfloat16)
    bits = b.view(torch.int16).to(torch.int32)
    up = (bits + 1).to(torch.int16).view(torch.bfloat16)  # next magnitude up (same sign)
    gap = (up.double() - b.double()).abs().numpy()
    # the spacing just above a bf16 value (for values that are not themselves
    # a power of two, the spacing at |y| is the same)
    bv = b.double().numpy()
    assert np.array_equal(bf16_ulp(bv), gap)
    assert bf16_ulp(0.0) == 0.0


def _case():
    rng = np.random.default_rng(5)
    w = rng.standard_normal(1000) * 0.01
    w[17] = 0.5589  # one element ~50 RMS large
    ideal = torch.tensor(w, dtype=torch.float32).to(torch.bfloat16).double().numpy()
    return w, ideal


def test_gate_accepts_a_one_ulp_flip_on_a_large_element():
    """A correct result that rounds to the other bf16 neighbour of the exact
    value, on an element 50 RMS large, passes: its literal max|x-y|/rms(y)
    is far above 2e-2, the gate's measure is 0."""
    spec = small_spec(name="tol", dtype="bf16", d=128)
    w, ideal = _case()
    flip = ideal.copy()
    flip[17] += bf16_ulp(ideal[17])
    e = compare(spec, {"o_c": torch.tensor(flip)}, {"o_c": w}, names=["o_c"], ideal={"o_c": ideal})
    assert e["o_c"]["raw"] > 0.1 and e["o_c"]["gate"] == 0.0
    assert_parity(spec, e)


def test_gate_rejects_an_error_on_a_typical_element():
    """An error of 2.5e-2 RMS beyond one ulp on one typical element fails,
    and 1.5e-2 passes: the 2e-2 of the stated bound is what is left."""
    spec = small_spec(name="tol", dtype="bf16", d=128)
    w, ideal = _case()
    r = np.sqrt(np.mean(w * w))
    for extra, ok in ((2.5e-2, False), (1.5e-2, True)):
        x = ideal.copy()
        x[3] += bf16_ulp(ideal[3]) + extra * r
        e = compare(spec, {"o_c": x}, {"o_c": w}, names=["o_c"],
                    ideal={"o_c": ideal})
        assert abs(e["o_c"]["gate"] - extra) < 1e-9
        assert (e["o_c"]["gate"] <= 2e-2) == ok


def test_gate_is_measured_against_the_bf16_operand_oracle_not_the_exact_one():
    """A GPU result equal to the exact oracle but far from the bf16-operand
    oracle fails: the gate is |x - i|, where the bf16 roundings are modelled."""
    x = np.array([1.0, -2.0, 0.5, 3.0])
    i = x + np.array([0.0, 0.0, 0.2, 0.0])
    assert bf16_gate(x, i, x) > 2e-2
    assert bf16_gate(i, i, x) == 0.0


def test_lse_is_held_to_the_literal_bound():
    spec = small_spec(name="tol", dtype="bf16", d=128)
    y = np.linspace(3.0, 12.0, 64)
    r = np.sqrt(np.mean(y * y))
    x = y.copy()
    x[5] += 3e-2 * r
    e = compare(spec, {"lse_c": x}, {"lse_c": y}, names=["lse_c"])
    assert abs(e["lse_c"]["gate"] - 3e-2) < 1e-9
