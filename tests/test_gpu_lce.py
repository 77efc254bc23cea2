"""The token-chunked linear cross-entropy on the GPU ("Block Parallelism for
Efficient Distributed Long-Context Diffusion Language Model Training", §5.1:
library projections plus fused softmax/CE kernels, chunk by chunk) against
the float64 oracle (oracle/lce_oracle.py).

Gates: loss and LSE (float32 outputs) max|x-y|/rms(y) <= 2e-2, and within
1e-5 of the largest value (float32 accumulation over the vocabulary); dH
(bf16) every element within one bf16 ulp plus 2e-2 RMS of the oracle's
bf16-operand mode (G rounded to bf16 before the projections); dW (float32,
made from the bf16 G) max|x - i| <= 2e-2 rms(y) against the same mode.
"""
import numpy as np
import pytest
import torch

import block_masked_attention_amd as bd
from oracle import LinearCE
from tests._helpers import f64, rms_err
from tests.gpu_util import bf16_gate, say

pytestmark = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def make_lce(N, D, V, seed, logit_std=2.0, ignore_frac=0.1):
    g = torch.Generator(device="cpu").manual_seed(seed)
    h = torch.randn(N, D, generator=g).bfloat16()
    w = (torch.randn(V, D, generator=g) * (logit_std / D ** 0.5)).bfloat16()
    t = torch.randint(0, V, (N,), generator=g, dtype=torch.int32)
    t[torch.rand(N, generator=g) < ignore_frac] = -100
    dloss = torch.randn(N, generator=g).float()
    return h, w, t, dloss


CASES = [  # N, D, V, chunk: ragged last chunk, one chunk, many small chunks
    (1000, 256, 5000, 256),
    (300, 128, 2048, 1000),
    (96, 512, 32000, 40),
    (513, 64, 8, 128),
]


def _check(label, got, want, ideal):
    loss, lse, dh, dw = (f64(x) for x in got)
    yl, ylse = want[0], want[1]
    errs = {
        "loss": rms_err(loss, yl), "lse": rms_err(lse, ylse),
        "dh": bf16_gate(dh, ideal[2], want[2]),
        "dw": float(np.max(np.abs(dw - ideal[3]))) / float(np.sqrt(np.mean(want[3] ** 2))),
    }
    lit = {"dh": rms_err(dh, want[2]), "dw": rms_err(dw, want[3])}
    say(f"  {label} gates {errs}; literal max|x-y|/rms(y) {lit}")
    assert all(v <= 2e-2 for v in errs.values()), errs
    assert np.max(np.abs(loss - yl)) <= 1e-5 * np.max(np.abs(ylse))
    assert np.max(np.abs(lse - ylse)) <= 1e-5 * np.max(np.abs(ylse))


@pytest.mark.parametrize("N,D,V,chunk", CASES, ids=[f"N{c[0]}_D{c[1]}_V{c[2]}_chunk{c[3]}" for c in CASES])
def test_lce_matches_the_oracle(N, D, V, chunk):
    _need_gpu()
    say(f"[gpu] linear CE N={N} D={D} V={V} chunk={chunk}")
    h, w, t, dloss = make_lce(N, D, V, seed=N + V)
    hd, wd, td, gd = h.cuda(), w.cuda(), t.cuda(), dloss.cuda()
    p = bd.lce_problem(N, D, V, chunk=chunk)
    loss, lse = bd.lce_fwd(p, hd, wd, td)
    dh, dw = bd.lce_bwd(p, hd, wd, td, lse, gd)
    fused = bd.lce_fwd_bwd(p, hd, wd, td, gd)
    torch.cuda.synchronize()
    args = (f64(h), f64(w), t.numpy())
    ex = LinearCE(*args)
    yl, ylse = ex.forward()
    want = (yl, ylse) + ex.backward(dloss.double().numpy(), ylse)
    bf = LinearCE(*args, operand_rounding="bf16")
    il, ilse = bf.forward()
    ideal = (il, ilse) + bf.backward(dloss.double().numpy(), ilse)
    _check(f"N{N} separate passes", (loss, lse, dh, dw), want, ideal)
    _check(f"N{N} fused pass", fused, want, ideal)
    # the fused pass computes the same numbers as the two separate passes
    for a, b in zip((loss, lse, dh, dw), fused):
        assert torch.equal(a, b)
    # ignored tokens: no loss, no gradient
    ign = (t == -100).cuda()
    assert torch.all(loss[ign] == 0) and torch.all(dh[ign] == 0)


def test_lce_chunk_size_changes_only_rounding():
    """Chunking changes only the order of the computation: two chunk sizes
    agree to float32 rounding on the loss and within one bf16 ulp on dH."""
    _need_gpu()
    N, D, V = 700, 256, 4096
    h, w, t, dloss = (x.cuda() for x in make_lce(N, D, V, seed=5))
    a = bd.lce_fwd_bwd(bd.lce_problem(N, D, V, chunk=64), h, w, t, dloss)
    b = bd.lce_fwd_bwd(bd.lce_problem(N, D, V, chunk=700), h, w, t, dloss)
    torch.cuda.synchronize()
    la, lb = f64(a[1]), f64(b[1])
    assert np.max(np.abs(la - lb)) <= 1e-5 * np.max(np.abs(la))
    ha, hb = f64(a[2]), f64(b[2])
    assert np.all(np.abs(ha - hb) <= 2 * np.maximum(np.abs(ha), np.abs(hb)) * 2.0 ** -8 + 1e-6)
    wa, wb = f64(a[3]), f64(b[3])
    assert np.max(np.abs(wa - wb)) <= 1e-4 * np.sqrt(np.mean(wa ** 2))


def test_lce_no_tokens_gives_zero_weight_gradient():
    _need_gpu()
    D, V = 64, 512
    w = torch.randn(V, D, device="cuda").bfloat16()
    h = torch.empty(0, D, device="cuda", dtype=torch.bfloat16)
    t = torch.empty(0, device="cuda", dtype=torch.int32)
    g = torch.empty(0, device="cuda")
    loss, lse, dh, dw = bd.lce_fwd_bwd(bd.lce_problem(0, D, V, chunk=16), h, w, t, g,
                                       out=(torch.empty(0, device="cuda"), torch.empty(0, device="cuda"),
                                            torch.empty(0, D, device="cuda", dtype=torch.bfloat16),
                                            torch.full((V, D), float("nan"), device="cuda")))
    torch.cuda.synchronize()
    assert torch.all(dw == 0)
