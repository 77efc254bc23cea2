"""Pins of the oracle's backward and of its bf16-operand mode by a scalar,
per-element reference, and planted mistakes that those pins must catch.

The reference below is written from the definition of softmax attention over
the visible keys ("Block Parallelism for Efficient Distributed Long-Context
Diffusion Language Model Training", §3.2 for the visible sets) and its
textbook gradient, one query row, one head and one key at a time, with every
sum taken by ``math.fsum`` (exactly rounded). Its visible sets are the range
formulation of the test suite (clean prefix length, own corrupted block), not
the oracle's pairwise rules.

The bf16-operand mode rounds, through float32 to the nearest bfloat16 (ties
to even), at exactly these points and nowhere else:
- the softmax weights before they multiply V (forward) and dO (dV);
- dS = P (dP - D) before it multiplies K (dQ) and Q (dK);
- the stored output O, which D = <dO, O> reads;
- every stored output (O, dQ, dK, dV). LSE is float32 and not rounded.
The reference rounds with torch's bfloat16 cast, not the oracle's bit
arithmetic.
"""
import importlib.util
import math
import os
import sys

import numpy as np
import pytest
import torch

from oracle import Oracle, layout
from tests.test_oracle import _prefix_sets, make, oracle_of

ORACLE_SRC = os.path.join(os.path.dirname(__file__), "..", "oracle", "bdattn_oracle.py")


def _bf16(x: float) -> float:
    """Nearest bfloat16 of x, rounded through float32 by torch's casts."""
    return torch.tensor([x], dtype=torch.float64).float().bfloat16().double().item()


def _same(x: float) -> float:
    return x


def scalar_reference(lay, t, rounding=None):
    """Forward and backward by scalar loops. Returns the oracle's output
    tuple order: O_c, O_x, LSE_c, LSE_x, dQ_c, dQ_x, dK_c, dV_c, dK_x, dV_x."""
    rd = _bf16 if rounding == "bf16" else _same
    Q = np.concatenate([t["q_c"], t["q_x"]])
    K = np.concatenate([t["k_c"], t["k_x"]])
    V = np.concatenate([t["v_c"], t["v_x"]])
    dO = np.concatenate([t["do_c"], t["do_x"]])
    nq, nk, H, d, G = Q.shape[0], K.shape[0], lay.H, lay.d, lay.G
    sets = _prefix_sets(lay)
    O = np.zeros((nq, H, d))
    LSE = np.zeros((H, nq))
    dQ = np.zeros((nq, H, d))
    dk_terms = [[[[] for _ in range(d)] for _ in range(lay.Hkv)] for _ in range(nk)]
    dv_terms = [[[[] for _ in range(d)] for _ in range(lay.Hkv)] for _ in range(nk)]
    for i, s in enumerate(sets):
        for h in range(H):
            g = h // G
            sc = [lay.scale * math.fsum(Q[i, h, e] * K[j, g, e] for e in range(d)) for j in s]
            m = max(sc)
            w = [math.exp(x - m) for x in sc]
            z = math.fsum(w)
            lse = m + math.log(z)
            LSE[h, i] = lse
            o = [rd(math.fsum(rd(w[a]) * V[j, g, e] for a, j in enumerate(s)) / z)
                 for e in range(d)]
            O[i, h] = o
            D = math.fsum(dO[i, h, e] * o[e] for e in range(d))  # reads the stored O
            dq_terms = [[] for _ in range(d)]
            for a, j in enumerate(s):
                p = math.exp(sc[a] - lse)
                dp = math.fsum(dO[i, h, e] * V[j, g, e] for e in range(d))
                ds = rd(p * (dp - D))
                for e in range(d):
                    dq_terms[e].append(ds * K[j, g, e])
                    dk_terms[j][g][e].append(ds * Q[i, h, e])
                    dv_terms[j][g][e].append(rd(p) * dO[i, h, e])
            dQ[i, h] = [rd(lay.scale * math.fsum(x)) for x in dq_terms]
    dK = np.array([[[rd(lay.scale * math.fsum(x)) for x in row] for row in kv] for kv in dk_terms])
    dV = np.array([[[rd(math.fsum(x)) for x in row] for row in kv] for kv in dv_terms])
    nc, nkc = lay.n_clean_q, lay.n_clean_kv
    return (O[:nc], O[nc:], LSE[:, :nc], LSE[:, nc:], dQ[:nc], dQ[nc:], dK[:nkc], dV[:nkc],
            dK[nkc:], dV[nkc:])


def _inputs(lay, seed):
    """Gaussian inputs already bf16 values (as a bf16 kernel receives them)."""
    t = make(lay, seed=seed, scale=0.8)
    return {k: torch.tensor(v).float().bfloat16().double().numpy() for k, v in t.items()}


# tiny problems: the complete problem (GQA 2), and a rank's share (offset
# clean queries, a longer clean buffer, strided corrupted blocks)
CASES = [
    dict(B=2, H=2, Hkv=1, d=4, n_clean_q=8),
    dict(B=3, H=4, Hkv=2, d=5, n_clean_q=6, clean_q_start=6, n_clean_kv=15,
         corr_block_ids=[0, 2, 4]),
]


def _lay(case):
    c = dict(case)
    B, H, Hkv, d, n = c.pop("B"), c.pop("H"), c.pop("Hkv"), c.pop("d"), c.pop("n_clean_q")
    return layout(B, H, Hkv, d, n, **c)


def _oracle_outputs(oracle_cls, lay, t, rounding):
    orc = oracle_cls(lay, t["q_c"], t["k_c"], t["v_c"], t["q_x"], t["k_x"], t["v_x"],
                     t["do_c"], t["do_x"], operand_rounding=rounding)
    f = orc.forward()
    g = orc.backward(O=np.concatenate([f[0], f[1]]), LSE=np.concatenate([f[2], f[3]], axis=1))
    return f + g


NAMES = ("O_c", "O_x", "LSE_c", "LSE_x", "dQ_c", "dQ_x", "dK_c", "dV_c", "dK_x", "dV_x")


def _mismatch(oracle_cls, lay, t, rounding):
    """Names of the outputs where the oracle and the scalar reference differ
    by more than 1e-13 relative to the tensor's largest element."""
    got = _oracle_outputs(oracle_cls, lay, t, rounding)
    want = scalar_reference(lay, t, rounding)
    bad = []
    for n, x, y in zip(NAMES, got, want):
        x, y = np.asarray(x), np.asarray(y)
        if x.shape != y.shape:
            bad.append(n)
            continue
        if y.size and np.max(np.abs(x - y)) > 1e-13 * max(1.0, np.max(np.abs(y))):
            bad.append(n)
    return bad


@pytest.mark.parametrize("case", CASES, ids=["complete", "share"])
@pytest.mark.parametrize("rounding", [None, "bf16"], ids=["exact", "bf16_operands"])
def test_oracle_matches_scalar_reference(case, rounding):
    """Forward and backward of the oracle (exact and bf16-operand modes) equal
    the scalar reference element by element. In bf16 mode the rounded outputs
    agree exactly (a tie flipped by the last bit of a float64 sum is the only
    way they could differ, and these seeds have none)."""
    lay = _lay(case)
    t = _inputs(lay, seed=97)
    assert _mismatch(Oracle, lay, t, rounding) == []
    if rounding == "bf16":
        got = _oracle_outputs(Oracle, lay, t, rounding)
        want = scalar_reference(lay, t, rounding)
        for n, x, y in zip(NAMES, got, want):
            if not n.startswith("LSE"):
                assert np.array_equal(x, y), n


def test_bf16_mode_differs_from_exact_where_it_rounds():
    """The roundings matter at this size (so the pin above is not vacuous):
    every rounded output of the bf16 mode differs from the exact one."""
    lay = _lay(CASES[0])
    t = _inputs(lay, seed=97)
    ex = _oracle_outputs(Oracle, lay, t, None)
    bf = _oracle_outputs(Oracle, lay, t, "bf16")
    for n, x, y in zip(NAMES, bf, ex):
        if not n.startswith("LSE"):
            assert not np.array_equal(x, y), n


# ---------------------------------------------------------- planted mistakes
# Each entry edits one expression of the oracle's source (the text must occur
# exactly once) into a plausible slip; the edited oracle must then disagree
# with the scalar reference in exact or bf16-operand mode.
MUTANTS = [
    ("rounds dP instead of dS",
     "dS = self.rd(P * (dP - D[sl, h][:, None]))", "dS = P * (self.rd(dP) - D[sl, h][:, None])"),
    ("dropped D term", "dS = self.rd(P * (dP - D[sl, h][:, None]))", "dS = self.rd(P * dP)"),
    ("wrong sign of D", "dS = self.rd(P * (dP - D[sl, h][:, None]))",
     "dS = self.rd(P * (dP + D[sl, h][:, None]))"),
    ("P not rounded before dV", "dVg += self.rd(P).T @ self.dO[rows, h]",
     "dVg += P.T @ self.dO[rows, h]"),
    ("P not rounded before PV", "O[s:s + len(rows), h] = (self.rd(E) @ Vg)",
     "O[s:s + len(rows), h] = (E @ Vg)"),
    ("stored O not rounded", "return self.rd(O), LSE", "return O, LSE"),
    ("dQ not rounded", "return self.rd(dQ), self.rd(dK), self.rd(dV)",
     "return dQ, self.rd(dK), self.rd(dV)"),
    ("dK from dO instead of Q", "dKg += lay.scale * (dS.T @ self.Q[rows, h])",
     "dKg += lay.scale * (dS.T @ self.dO[rows, h])"),
    ("dP from Q instead of dO", "dP = self.dO[rows, h] @ Vg.T", "dP = self.Q[rows, h] @ Vg.T"),
    ("dQ without the scale", "dQ[sl, h] = lay.scale * (dS @ Kg)", "dQ[sl, h] = (dS @ Kg)"),
    ("LSE without the max shift", "LSE[h, s:s + len(rows)] = m + np.log(l)",
     "LSE[h, s:s + len(rows)] = np.log(l)"),
    ("corrupted rows see their own clean block",
     "corr_clean = ~qc & kc & (k_block < q_block)", "corr_clean = ~qc & kc & (k_block <= q_block)"),
    ("clean rows miss their own block",
     "clean_clean = qc & kc & ((k_block < q_block) | own_block)",
     "clean_clean = qc & kc & (k_block < q_block)"),
    ("corrupted rows miss their own block",
     "corr_corr = ~qc & ~kc & (k_block == q_block) & bool(corr_keys)",
     "corr_corr = ~qc & ~kc & (k_block < q_block) & bool(corr_keys)"),
    ("keys of a KV head read by the wrong q heads",
     "                for h in range(g * lay.G, (g + 1) * lay.G):\n                    S = self._scores(rows, Kg, Mc, h)\n                    # exp",
     "                for h in range(g, g + lay.G):\n                    S = self._scores(rows, Kg, Mc, h)\n                    # exp"),
]


def _mutant_oracle(old, new, tag):
    with open(ORACLE_SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"planted mistake target not unique or gone: {old!r}"
    name = f"_oracle_mutant_{tag}"
    spec = importlib.util.spec_from_loader(name, loader=None)
    mod = importlib.util.module_from_spec(spec)
    sys.modules[name] = mod  # dataclasses resolve the module by name
    try:
        exec(compile(src.replace(old, new), ORACLE_SRC, "exec"), mod.__dict__)
    finally:
        del sys.modules[name]
    return mod


@pytest.mark.parametrize("label,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(label, old, new):
    mod = _mutant_oracle(old, new, abs(hash(label)))
    caught = []
    for case in CASES:
        lay = mod.layout(**{k: v for k, v in _lay_args(case).items()})
        t = _inputs(_lay(case), seed=97)
        for rounding in (None, "bf16"):
            try:
                caught += _mismatch(mod.Oracle, lay, t, rounding)
            except (ValueError, IndexError):
                caught.append("raised")
    assert caught, f"the pins did not catch: {label}"


def _lay_args(case):
    c = dict(case)
    return dict(B=c.pop("B"), H=c.pop("H"), Hkv=c.pop("Hkv"), d=c.pop("d"),
                n_clean_q=c.pop("n_clean_q"), **c)


def test_unplanted_source_passes_the_same_check():
    """The mutation harness itself: the unedited source, loaded the same way,
    agrees with the reference (so a caught mutant is caught by its edit)."""
    mod = _mutant_oracle("import math\n", "import math\n", "identity")
    for case in CASES:
        lay = mod.layout(**_lay_args(case))
        t = _inputs(_lay(case), seed=97)
        for rounding in (None, "bf16"):
            assert _mismatch(mod.Oracle, lay, t, rounding) == []
