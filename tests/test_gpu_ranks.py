"""Context-sharded ranks simulated on one GPU ("Block Parallelism for
Efficient Distributed Long-Context Diffusion Language Model Training", §4.3
Forward pass / Backward pass, §4.4 Proposition 1).

The 8K workload is split over P = 4 ranks. Rank r holds clean-query shard r,
the clean K/V of every position before the last one its queries see (what the
forward's all-gather delivers), and the corrupted blocks of the dual-end
assignment (block b together with block nb-1-b). Each share runs through
bdattn_fwd / bdattn_bwd as its own problem. Summing the ranks' clean dK/dV
(the backward's reduce-scatter) and placing every other output at its rows
must give the single full call's results, and those are checked against the
oracle on sampled rows.
"""
import numpy as np
import pytest
import torch

from tests._helpers import f64
from tests.gpu_util import OUT_NAMES, assert_parity, bf16_ulp, compare, run_gpu, say
from tests.test_gpu_parity import _sampled
from workloads import CONFIGS, make_inputs

pytestmark = pytest.mark.gpu


def dual_end_owner(nb, P):
    """Block b and block nb-1-b go to the same rank, pairs dealt round-robin."""
    owner = {}
    for r in range(P):
        for k in range(nb // (2 * P)):
            i = r + k * P
            owner[i] = r
            owner[nb - 1 - i] = r
    return owner


def test_dual_end_ranks_sum_to_the_full_call():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    spec = CONFIGS[1]
    B, L, P = spec.B, spec.n_clean_q, 4
    nb, shard = L // B, L // P
    say(f"[gpu] simulated ranks: {spec.name}, P={P}, dual-end corrupted blocks")
    t = make_inputs(spec, device="cuda")
    full = run_gpu(spec, t)
    owner = dual_end_owner(nb, P)
    got = {k: torch.zeros_like(v) for k, v in full.items()}
    parts_k, parts_v = [], []
    for r in range(P):
        ids = sorted(b for b, o in owner.items() if o == r)
        lo, hi = r * shard, (r + 1) * shard
        kv_end = max(hi, max(ids) * B)
        rs = spec.with_(name=f"rank{r}", n_clean_q=shard, clean_q_start=lo, n_clean_kv=kv_end,
                        n_corr_blocks=len(ids), corr_block_ids=tuple(ids))
        xr = torch.as_tensor(np.concatenate([np.arange(b * B, (b + 1) * B) for b in ids]),
                             device="cuda")
        tr = dict(q_c=t["q_c"][lo:hi], k_c=t["k_c"][:kv_end], v_c=t["v_c"][:kv_end],
                  q_x=t["q_x"][xr], k_x=t["k_x"][xr], v_x=t["v_x"][xr],
                  do_c=t["do_c"][lo:hi], do_x=t["do_x"][xr])
        tr = {k: v.contiguous() for k, v in tr.items()}
        say(f"  rank {r}: clean queries [{lo}, {hi}), clean K/V [0, {kv_end}), "
            f"{len(ids)} corrupted blocks")
        out = run_gpu(rs, tr)
        for k in ("o_c", "dq_c"):
            got[k][lo:hi] = out[k]
        got["lse_c"][:, lo:hi] = out["lse_c"]
        for k in ("o_x", "dq_x", "dk_x", "dv_x"):
            got[k][xr] = out[k]
        got["lse_x"][:, xr] = out["lse_x"]
        pk = torch.zeros_like(full["dk_c"], dtype=torch.float32)
        pv = torch.zeros_like(full["dv_c"], dtype=torch.float32)
        pk[:kv_end] = out["dk_c"].float()
        pv[:kv_end] = out["dv_c"].float()
        parts_k.append(pk)
        parts_v.append(pv)
    torch.cuda.synchronize()

    # rows owned by one rank: each share's kernels sweep the same key tiles in
    # the same order as the full call; at most a one-ulp rounding difference
    for k in ("o_c", "o_x", "dq_c", "dq_x", "dk_x", "dv_x"):
        a, b = f64(got[k]), f64(full[k])
        same = float(np.mean(a == b))
        say(f"  {k}: {100 * same:.3f}% of elements bitwise equal to the full call")
        assert np.all(np.abs(a - b) <= bf16_ulp(b)), k
    for k in ("lse_c", "lse_x"):
        a, b = f64(got[k]), f64(full[k])
        assert np.max(np.abs(a - b)) <= 1e-5 * np.max(np.abs(b)), k
    # clean dK/dV: the sum of the ranks' bf16 parts against the full call's
    # one bf16 rounding of the whole sum: apart from fp32 summation order the
    # two differ by the roundings, at most half an ulp of each part and of
    # the full value
    for k, parts in (("dk_c", parts_k), ("dv_c", parts_v)):
        s = sum(f64(p) for p in parts)
        f = f64(full[k])
        bound = sum(bf16_ulp(f64(p)) / 2 for p in parts) + bf16_ulp(f) / 2 \
            + 2.0 ** -18 * sum(np.abs(f64(p)) for p in parts)
        excess = np.max(np.abs(s - f) - bound)
        say(f"  {k}: max |sum of ranks - full| = {np.max(np.abs(s - f)):.3e} "
            f"(bound excess {excess:.3e})")
        assert excess <= 0, k

    # the rank-assembled outputs against the oracle on sampled rows
    have, want = _sampled(spec, t, got, kv_groups=(0,), with_keys=False)
    _, ideal = _sampled(spec, t, got, kv_groups=(0,), rounding="bf16", with_keys=False)
    errs = compare(spec, have, want, names=list(want), label="8k ranks", ideal=ideal)
    assert_parity(spec, errs, "8k ranks")
