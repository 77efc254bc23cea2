"""CPU float64 oracle for the token-chunked linear cross-entropy.

TEST INFRASTRUCTURE ONLY. Only the test suite and the benchmark's CPU-baseline
leg may import this module. The GPU library never calls it and shares no code
with it.

What it computes: the vocabulary projection and softmax cross-entropy loss of
a language model's output layer, which "Block Parallelism for Efficient
Distributed Long-Context Diffusion Language Model Training" (§5.1,
Experimental setup) computes token-chunked, with library projections and fused
softmax/CE kernels, so that full-sequence logits are never materialised.
Chunking changes only the order of the computation, so the oracle is the plain
definition over all tokens at once:

    z_ij   = <h_i, w_j>                       (logits, token i, vocabulary entry j)
    LSE_i  = ln sum_j exp(z_ij)
    loss_i = LSE_i - z_{i, t_i}               (0 for a token whose target is ignore_index)

and its analytic backward, given the upstream gradient g_i of each token's
loss:

    G_ij   = g_i (softmax_ij - [j == t_i])    (0 on ignored tokens)
    dH_i   = sum_j G_ij w_j
    dW_j   = sum_i G_ij h_i

``operand_rounding="bf16"`` evaluates the same definition with the roundings a
bf16 implementation cannot avoid and nothing else: G is rounded to bfloat16
before it multiplies W and H (the projections take bf16 operands), and dH is
stored in bfloat16. dW and the loss stay exact (float32 outputs). Products are
exact float64 sums.
"""
from __future__ import annotations

import numpy as np

from .bdattn_oracle import round_bf16

__all__ = ["LinearCE"]


def _ident(x):
    return x


class LinearCE:
    """Linear cross-entropy over N tokens: hidden states ``h`` ``[N, D]``,
    projection ``w`` ``[V, D]``, integer ``targets`` ``[N]``; float64."""

    # tokens per row block of the dense logits (bounded memory only)
    ROWS = 512

    def __init__(self, h, w, targets, ignore_index=-100, operand_rounding=None):
        self.h = np.ascontiguousarray(np.asarray(h, dtype=np.float64))
        self.w = np.ascontiguousarray(np.asarray(w, dtype=np.float64))
        self.t = np.asarray(targets, dtype=np.int64)
        self.ignore = int(ignore_index)
        if operand_rounding not in (None, "bf16"):
            raise ValueError("operand_rounding must be None or 'bf16'")
        self.rd = round_bf16 if operand_rounding == "bf16" else _ident
        N, V = self.h.shape[0], self.w.shape[0]
        self.valid = self.t != self.ignore
        if np.any((self.t[self.valid] < 0) | (self.t[self.valid] >= V)):
            raise ValueError("targets must lie in [0, V) or equal ignore_index")
        if self.t.shape != (N,) or self.h.shape[1] != self.w.shape[1]:
            raise ValueError("shapes: h [N, D], w [V, D], targets [N]")

    def _blocks(self):
        N = self.h.shape[0]
        for s in range(0, N, self.ROWS):
            yield slice(s, min(N, s + self.ROWS))

    def forward(self):
        """(loss [N], LSE [N])."""
        N = self.h.shape[0]
        loss = np.zeros(N)
        lse = np.zeros(N)
        for r in self._blocks():
            z = self.h[r] @ self.w.T
            m = z.max(axis=1)
            lse[r] = m + np.log(np.exp(z - m[:, None]).sum(axis=1))
            v = self.valid[r]
            rows = np.flatnonzero(v)
            zt = z[rows, self.t[r][rows]]
            loss[r.start + rows] = lse[r][rows] - zt
        return loss, lse

    def backward(self, dloss, lse=None):
        """(dH [N, D], dW [V, D]) for the upstream gradient ``dloss`` [N] of
        each token's loss; ``lse`` is the forward's (recomputed if None)."""
        dloss = np.asarray(dloss, dtype=np.float64)
        if lse is None:
            _, lse = self.forward()
        dH = np.zeros_like(self.h)
        dW = np.zeros_like(self.w)
        for r in self._blocks():
            z = self.h[r] @ self.w.T
            G = np.exp(z - lse[r][:, None])
            rows = np.flatnonzero(self.valid[r])
            G[rows, self.t[r][rows]] -= 1.0
            G *= np.where(self.valid[r], dloss[r], 0.0)[:, None]
            G = self.rd(G)
            dH[r] = G @ self.w
            dW += G.T @ self.h[r]
        return self.rd(dH), dW
