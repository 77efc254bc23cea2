"""The bf16 acceptance rule of the GPU parity tests, checked on the CPU: the
bf16 unit in the last place, and what the element-wise bound accepts and
rejects."""
import numpy as np
import torch

from tests.gpu_util import assert_parity, bf16_ulp, compare
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


def test_elementwise_bound_accepts_a_one_ulp_flip_and_rejects_real_errors():
    spec = small_spec(name="tol", dtype="bf16", d=128)
    rng = np.random.default_rng(5)
    w = rng.standard_normal(1000) * 0.01
    w[17] = 0.5589  # one element ~50 RMS large
    ideal = torch.tensor(w, dtype=torch.float32).to(torch.bfloat16).double().numpy()
    flip = ideal.copy()
    flip[17] += bf16_ulp(ideal[17])  # the other bf16 neighbour of the exact value
    e = compare(spec, {"o_c": torch.tensor(flip)}, {"o_c": w}, names=["o_c"], ideal={"o_c": ideal})
    assert e["o_c"][0] > e["o_c"][1] + 2e-2  # the norm-wise rule alone would reject it
    assert_parity(spec, e)
    bad = ideal.copy()
    bad[3] += 0.05 * np.sqrt(np.mean(w * w)) + 4 * bf16_ulp(w[3])  # a typical element, off
    e = compare(spec, {"o_c": torch.tensor(bad)}, {"o_c": w}, names=["o_c"], ideal={"o_c": ideal})
    assert not e["o_c"][2]
