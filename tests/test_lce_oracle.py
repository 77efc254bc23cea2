"""Pins of the linear cross-entropy oracle against things other than itself:
a scalar math.fsum loop, torch's cross_entropy with autograd (float64, CPU),
central finite differences, closed forms at W = 0, ignored tokens, and the
bf16-operand mode against a scalar reference that rounds with torch's cast.
The loss is that of "Block Parallelism for Efficient Distributed
Long-Context Diffusion Language Model Training", §5.1 (token-chunked linear
cross-entropy): softmax cross-entropy over the vocabulary projection."""
import importlib.util
import math
import os
import sys

import numpy as np
import pytest
import torch

from oracle import LinearCE

SRC = os.path.join(os.path.dirname(__file__), "..", "oracle", "lce_oracle.py")


def _case(N=9, V=11, D=5, seed=0, ignore=(2,)):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((N, D))
    w = rng.standard_normal((V, D)) * 0.7
    t = rng.integers(0, V, N)
    for i in ignore:
        t[i] = -100
    g = rng.standard_normal(N)
    return h, w, t, g


def _bf16(x):
    return torch.tensor([x], dtype=torch.float64).float().bfloat16().double().item()


def scalar_reference(h, w, t, g, rounding=None, ignore=-100):
    """Loss, LSE, dH, dW one token and one vocabulary entry at a time, sums
    by math.fsum."""
    rd = _bf16 if rounding == "bf16" else (lambda x: x)
    N, D = h.shape
    V = w.shape[0]
    loss, lse = np.zeros(N), np.zeros(N)
    dH, dW = np.zeros((N, D)), np.zeros((V, D))
    dw_terms = [[[] for _ in range(D)] for _ in range(V)]
    for i in range(N):
        z = [math.fsum(h[i, e] * w[j, e] for e in range(D)) for j in range(V)]
        m = max(z)
        s = m + math.log(math.fsum(math.exp(x - m) for x in z))
        lse[i] = s
        if t[i] == ignore:
            continue
        loss[i] = s - z[t[i]]
        G = [rd(g[i] * (math.exp(z[j] - s) - (1.0 if j == t[i] else 0.0))) for j in range(V)]
        for e in range(D):
            dH[i, e] = rd(math.fsum(G[j] * w[j, e] for j in range(V)))
            for j in range(V):
                dw_terms[j][e].append(G[j] * h[i, e])
    for j in range(V):
        for e in range(D):
            dW[j, e] = math.fsum(dw_terms[j][e])
    return loss, lse, dH, dW


@pytest.mark.parametrize("rounding", [None, "bf16"])
def test_matches_scalar_reference(rounding):
    h, w, t, g = _case()
    o = LinearCE(h, w, t, operand_rounding=rounding)
    loss, lse = o.forward()
    dH, dW = o.backward(g, lse)
    want = scalar_reference(h, w, t, g, rounding)
    for got, exp in zip((loss, lse, dH, dW), want):
        np.testing.assert_allclose(got, exp, rtol=1e-12, atol=1e-12)


def test_matches_library_cross_entropy_and_autograd():
    h, w, t, g = _case(N=40, V=37, D=8, seed=3, ignore=(0, 17))
    ht = torch.tensor(h, requires_grad=True)
    wt = torch.tensor(w, requires_grad=True)
    tt = torch.tensor(t)
    loss_t = torch.nn.functional.cross_entropy(ht @ wt.T, tt, reduction="none", ignore_index=-100)
    (loss_t * torch.tensor(g)).sum().backward()
    o = LinearCE(h, w, t)
    loss, lse = o.forward()
    dH, dW = o.backward(g, lse)
    np.testing.assert_allclose(loss, loss_t.detach().numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dH, ht.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dW, wt.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, torch.logsumexp(ht @ wt.T, 1).detach().numpy(), rtol=1e-12)


def test_finite_differences():
    h, w, t, g = _case(N=6, V=7, D=4, seed=5, ignore=(4,))
    o = LinearCE(h, w, t)
    dH, dW = o.backward(g)
    f = lambda hh, ww: float(np.dot(LinearCE(hh, ww, t).forward()[0], g))
    eps = 1e-6
    for x, grad, which in ((h, dH, 0), (w, dW, 1)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            num[idx] = ((f(xp, w) - f(xm, w)) if which == 0 else (f(h, xp) - f(h, xm))) / (2 * eps)
        assert np.max(np.abs(num - grad)) / np.max(np.abs(num)) < 1e-7


def test_zero_projection_closed_forms():
    """W = 0: every logit is 0, so loss = LSE = ln V, dH = 0 and
    dW_j = sum_i g_i (1/V - [j == t_i]) h_i."""
    h, w, t, g = _case(N=12, V=9, D=4, seed=7, ignore=(3, 8))
    w = np.zeros_like(w)
    o = LinearCE(h, w, t)
    loss, lse = o.forward()
    dH, dW = o.backward(g, lse)
    V = w.shape[0]
    valid = t != -100
    np.testing.assert_allclose(lse, np.full(len(t), math.log(V)), rtol=1e-15)
    np.testing.assert_allclose(loss, np.where(valid, math.log(V), 0.0), rtol=1e-15)
    assert np.all(dH == 0)
    want = np.zeros_like(dW)
    for i in np.flatnonzero(valid):
        want += g[i] / V * h[i]
        want[t[i]] -= g[i] * h[i]
    np.testing.assert_allclose(dW, want, rtol=1e-13, atol=1e-14)


def test_ignored_tokens_contribute_nothing():
    h, w, t, g = _case(N=10, V=8, D=4, seed=9, ignore=())
    keep = np.array([0, 2, 3, 7, 9])
    t2 = t.copy()
    t2[np.setdiff1d(np.arange(10), keep)] = -100
    a = LinearCE(h, w, t2)
    b = LinearCE(h[keep], w, t[keep])
    la, _ = a.forward()
    lb, _ = b.forward()
    np.testing.assert_allclose(la[keep], lb, rtol=1e-14)
    assert np.all(la[np.setdiff1d(np.arange(10), keep)] == 0)
    dHa, dWa = a.backward(g)
    dHb, dWb = b.backward(g[keep])
    np.testing.assert_allclose(dWa, dWb, rtol=1e-13, atol=1e-14)
    assert np.all(dHa[np.setdiff1d(np.arange(10), keep)] == 0)


def test_row_blocks_do_not_change_the_result():
    """The oracle's row blocks bound memory only."""
    h, w, t, g = _case(N=50, V=13, D=6, seed=11, ignore=(1, 30))
    a = LinearCE(h, w, t)
    b = LinearCE(h, w, t)
    b.ROWS = 7
    for x, y in zip(a.forward() + a.backward(g), b.forward() + b.backward(g)):
        np.testing.assert_allclose(x, y, rtol=1e-13, atol=1e-14)


MUTANTS = [
    ("G rounded before the dloss scale", "G *= np.where(self.valid[r], dloss[r], 0.0)[:, None]\n            G = self.rd(G)",
     "G = self.rd(G)\n            G *= np.where(self.valid[r], dloss[r], 0.0)[:, None]"),
    ("target term dropped", "G[rows, self.t[r][rows]] -= 1.0", "pass"),
    ("dH not rounded", "return self.rd(dH), dW", "return dH, dW"),
    ("dW from the rounded-twice G", "dW += G.T @ self.h[r]", "dW += self.rd(G.T @ self.h[r])"),
    ("loss without the max shift", "lse[r] = m + np.log(np.exp(z - m[:, None]).sum(axis=1))",
     "lse[r] = np.log(np.exp(z - m[:, None]).sum(axis=1))"),
    ("ignored tokens keep their gradient", "G *= np.where(self.valid[r], dloss[r], 0.0)[:, None]",
     "G *= dloss[r][:, None]"),
]


@pytest.mark.parametrize("label,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(label, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, old
    name = f"_lce_mutant_{abs(hash(label))}"
    spec = importlib.util.spec_from_loader(name, loader=None)
    mod = importlib.util.module_from_spec(spec)
    mod.__package__ = "oracle"
    sys.modules[name] = mod
    try:
        exec(compile(src.replace(old, new), SRC, "exec"), mod.__dict__)
    finally:
        del sys.modules[name]
    h, w, t, g = _case()
    caught = False
    for rounding in (None, "bf16"):
        o = mod.LinearCE(h, w, t, operand_rounding=rounding)
        loss, lse = o.forward()
        got = (loss, lse) + o.backward(g, lse)
        want = scalar_reference(h, w, t, g, rounding)
        caught |= any(not np.allclose(x, y, rtol=1e-12, atol=1e-12) for x, y in zip(got, want))
    assert caught, label
