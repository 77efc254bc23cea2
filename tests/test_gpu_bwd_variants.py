"""The two measured alternatives to the split backward, on the GPU ("Block
Parallelism for Efficient Distributed Long-Context Diffusion Language Model
Training", §4.3, Backward pass: dQ, dK, dV of every visible pair):

  BDATTN_DKDV=fused    dK/dV with one wave per 32 keys in both roles: the
                       same arithmetic in the same order as the split dK/dV
                       kernel, so every output is bitwise equal to the
                       default path's;
  BDATTN_BWD=fused10   the whole backward in one kernel (bf16, d = 128,
                       contiguous clean K/V), dQ added up by float atomics:
                       dK/dV bitwise equal to the default path's, dQ (whose
                       summation order the atomics decide) to the same parity
                       gate against the oracle as the default path.

The library reads both switches at every backward call.
"""
import pytest
import torch

from tests.gpu_util import assert_parity, check_fwd_bwd, say
from workloads import INPUT_NAMES, make_inputs, small_spec
import block_masked_attention_amd as bd

pytestmark = pytest.mark.gpu

CASES = [
    small_spec(L=1056, B=32, H=8, Hkv=2, d=128, dtype="bf16", std=0.5, seed=3, name="bf16 d128 ragged"),
    small_spec(L=2048, B=32, H=8, Hkv=2, d=128, dtype="bf16", std=0.5, seed=5, doc_starts=[0, 96, 800],
               name="bf16 d128 3 documents"),
    small_spec(L=1000, B=8, H=4, Hkv=4, d=128, dtype="bf16", seed=9, n_clean_q=520, clean_q_start=480,
               name="bf16 d128 partial rows"),
    small_spec(L=520, B=8, H=4, Hkv=2, d=32, dtype="bf16", seed=6, name="bf16 d32"),
    small_spec(L=512, B=16, H=4, Hkv=2, d=32, dtype="f32", seed=4, name="f32 d32"),
]


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _bwd(spec, t):
    p = bd.from_spec(spec)
    ins = [t[k] for k in INPUT_NAMES]
    f = bd.fwd(p, *ins)
    g = bd.bwd(p, *ins, *f, t["do_c"], t["do_x"])
    torch.cuda.synchronize()
    return [x.clone() for x in g]


@pytest.mark.parametrize("spec", CASES, ids=lambda s: s.name)
def test_fused_role_dkdv_is_bitwise_the_split_kernel(spec, monkeypatch):
    _need_gpu()
    t = make_inputs(spec, device="cuda")
    monkeypatch.delenv("BDATTN_DKDV", raising=False)
    want = _bwd(spec, t)
    monkeypatch.setenv("BDATTN_DKDV", "fused")
    got = _bwd(spec, t)
    same = [torch.equal(a, b) for a, b in zip(got, want)]
    say(f"  {spec.name}: fused-role dK/dV bitwise per output {same}")
    assert all(same)


@pytest.mark.parametrize("spec", [c for c in CASES if c.dtype == "bf16" and c.d == 128], ids=lambda s: s.name)
def test_one_kernel_backward(spec, monkeypatch):
    _need_gpu()
    t = make_inputs(spec, device="cuda")
    monkeypatch.delenv("BDATTN_BWD", raising=False)
    want = _bwd(spec, t)
    monkeypatch.setenv("BDATTN_BWD", "fused10")
    got = _bwd(spec, t)
    # dk_c, dv_c, dk_x, dv_x: the split kernel's arithmetic in its order
    same = [torch.equal(a, b) for a, b in zip(got[2:], want[2:])]
    say(f"  {spec.name}: one-kernel backward dK/dV bitwise per output {same}")
    assert all(same)
    # dQ against the oracle, as the default path is checked
    assert_parity(spec, check_fwd_bwd(spec, t, spec.name + " (one-kernel backward)"))
