"""The precision modes of bf16 problems (bdattn_problem.precision), on the GPU.

The bf16 configurations' stated tolerance is a maximum absolute error
normalised by the output RMS, max|x - y| / rms(y) <= 2e-2, against the exact
attention ("Block Parallelism for Efficient Distributed Long-Context
Diffusion Language Model Training", §3.2 for the definition). The default
mode cannot meet it literally: its bf16 outputs, and the bf16 rounding of the
softmax weights P and score gradients dS where they enter the P V, dV, dK and
dQ products, each cost about 2^-9 relative, which on peaked rows exceeds 2e-2
of the RMS; the default mode is therefore gated element-wise against the
bf16-operand oracle (tests/gpu_util.py). In PRECISION_SPLIT mode (float32
outputs, P and dS as two bf16 terms) the literal bound applies as stated:
every output of every bf16 problem here, and sampled rows and keys of the four
full-size bf16 workloads, are compared with the exact float64 oracle by
max|x - y| / rms(y), with no allowance.

Also: the float32-output forward (PRECISION_F32_OUT) rounds to the default
forward bit for bit (the kernels differ only in the final store), and the
split pipeline's merges of float32 partial results reproduce the complete
float32 forward.
"""
import numpy as np
import pytest
import torch

import block_masked_attention_amd as bd
from tests._helpers import f64, rms_err
from tests.gpu_util import OUT_NAMES, oracle_full, say
from tests.test_gpu_gathered import SMALL as GATHERED
from tests.test_gpu_parity import DOCS, RANDOM, RANDOM_DOCS, SMALL, _sampled, long_key_blocks
from tests.test_gpu_partial import part_inputs, part_problem, pieces
from workloads import CONFIGS, INPUT_NAMES, make_inputs, small_spec

pytestmark = pytest.mark.gpu

BOUND = 2e-2  # max|x - y| / rms(y), the stated bf16 tolerance


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run_prec(spec, t, precision=bd.PRECISION_SPLIT):
    p = bd.from_spec(spec, precision=precision)
    ins = [t[k] for k in INPUT_NAMES]
    f = bd.fwd(p, *ins)
    g = bd.bwd(p, *ins, *f, t["do_c"], t["do_x"])
    torch.cuda.synchronize()
    out = dict(zip(OUT_NAMES, tuple(f) + tuple(g)))
    for k, v in out.items():
        assert v.dtype == torch.float32, (k, v.dtype)
    return out


def literal(got, want, names=OUT_NAMES):
    """max|x - y| / rms(y) per output (x: GPU tensors or arrays)."""
    conv = lambda x: x if isinstance(x, np.ndarray) else f64(x)
    return {k: rms_err(conv(got[k]), np.asarray(want[k])) for k in names
            if np.asarray(want[k]).size}


BF16_SMALL = [(label, kw) for label, kw in SMALL if kw["dtype"] == "bf16"]
# the descriptor options the small list leaves out: packed documents and a
# gathered clean buffer (the chunks in zigzag all-gather order)
BF16_MORE = [(label, kw, {}) for label, kw in DOCS if kw["dtype"] == "bf16"] + [
    (label, kw, g) for label, kw, g in GATHERED if kw["dtype"] == "bf16"]


@pytest.mark.parametrize("label,kw", BF16_SMALL, ids=[c[0] for c in BF16_SMALL])
def test_f32_forward_rounds_to_the_bf16_forward(label, kw):
    _need_gpu()
    spec = small_spec(name=label, **kw)
    t = make_inputs(spec, device="cuda")
    ins = [t[k] for k in INPUT_NAMES]
    f16 = bd.fwd(bd.from_spec(spec), *ins)
    f32 = bd.fwd(bd.from_spec(spec, precision=bd.PRECISION_F32_OUT), *ins)
    torch.cuda.synchronize()
    assert torch.equal(f32[0].to(torch.bfloat16), f16[0]) and torch.equal(f32[1].to(torch.bfloat16), f16[1])
    assert torch.equal(f32[2], f16[2]) and torch.equal(f32[3], f16[3])


# the parity suite's seeded random problems (every descriptor option mixed in)
BF16_RANDOM = [(label, kw, {}) for label, kw in RANDOM + RANDOM_DOCS if kw["dtype"] == "bf16"]
CASES = [(label, kw, {}) for label, kw in BF16_SMALL] + BF16_MORE + BF16_RANDOM


@pytest.mark.parametrize("label,kw,g", CASES, ids=[c[0] for c in CASES])
def test_small_problems_meet_the_stated_bound(label, kw, g):
    _need_gpu()
    spec = small_spec(name=label, **kw).with_(**g)
    t = make_inputs(spec, device="cuda")
    want = oracle_full(spec, t)
    errs = literal(run_prec(spec, t), want)
    say(f"  {label} split: max|x-y|/rms(y) " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    f32 = literal(run_prec(spec, t, bd.PRECISION_F32_OUT), want)
    say(f"  {label} float32 outputs only (reported): " + " ".join(f"{k}={v:.2e}" for k, v in f32.items()))
    bad = {k: v for k, v in errs.items() if not v <= BOUND}
    assert not bad, f"{label}: above {BOUND}: {bad}"


@pytest.mark.parametrize("idx", [i for i, c in enumerate(CONFIGS) if c.dtype == "bf16"],
                         ids=[c.name for c in CONFIGS if c.dtype == "bf16"])
def test_workloads_meet_the_stated_bound(idx):
    """Each bf16 workload at full size: sampled query blocks of both streams
    (O, LSE, dQ, corrupted dK/dV) and clean key blocks (dK/dV, key block 0
    and a middle block at 8K among them) against the exact oracle."""
    _need_gpu()
    spec = CONFIGS[idx]
    say(f"[gpu] workload {spec.name}, split operands and float32 outputs")
    t = make_inputs(spec, device="cuda")
    got = run_prec(spec, t)
    groups = (0,) if spec.Hkv == 1 else (0, spec.Hkv - 1)
    have, want = _sampled(spec, t, got, kv_groups=groups, long_keys=long_key_blocks(spec))
    errs = literal(have, want, names=list(want))
    say(f"  {spec.name}: max|x-y|/rms(y) " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= BOUND}
    assert not bad, f"{spec.name}: above {BOUND}: {bad}"


def test_split_forward_merges_float32_partials():
    """Partial forwards with float32 outputs merged by bdattn_merge (float32,
    d = 128) equal the complete forward. In split mode, where P enters P V to
    about 16 bits, the only difference left is the order of rounding (each
    part weights its keys against its own maximum), so they agree to 1e-4 of
    the largest value; with bf16 P they differ at the 2^-9 level."""
    _need_gpu()
    spec = small_spec(L=1056, B=32, H=8, Hkv=2, d=128, dtype="bf16", std=0.5, seed=78)
    t = make_inputs(spec, device="cuda")
    merged = None
    for lo, hi, ck in pieces(spec):
        p = part_problem(spec, lo, hi, ck)
        p.precision = bd.PRECISION_SPLIT
        r = bd.fwd(p, *[part_inputs(t, lo, hi)[k] for k in INPUT_NAMES])
        assert r[0].dtype == torch.float32
        if merged is None:
            merged = list(r)
            continue
        merged[0], merged[2] = bd.merge(merged[0], merged[2], r[0], r[2])
        merged[1], merged[3] = bd.merge(merged[1], merged[3], r[1], r[3])
    full = bd.fwd(bd.from_spec(spec, precision=bd.PRECISION_SPLIT), *[t[k] for k in INPUT_NAMES])
    torch.cuda.synchronize()
    for a, b, name in zip(merged, full, ("o_c", "o_x", "lse_c", "lse_x")):
        err = float((a - b).abs().max() / b.abs().max().clamp_min(1e-30))
        say(f"  {name}: merged vs complete max rel {err:.2e}")
        assert err <= 1e-4, name
