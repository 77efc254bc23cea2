"""A gathered clean K/V buffer on the GPU ("Block Parallelism for Efficient
Distributed Long-Context Diffusion Language Model Training", appendix,
Efficient fused operator, Implementation 1: the clean-K/V launch masks with
each gathered key's original clean position, with no reordering copy; §4.3:
the all-gather delivers the clean chunks rank by rank, zigzag order).

One launch covers a buffer of chunks in gathered order (descriptor
kv_chunk_len / kv_chunk_pos). Checked against the oracle with every buffer
row at its original position (small problems, whole outputs), and, at the 8K
workload with P = 4 zigzag ranks, against the same launch over the buffer in
position order (bitwise: the kernels work in position order and only read
and write the buffer through the chunk map) and against the oracle on
sampled rows and keys.
"""
import zlib

import numpy as np
import pytest
import torch

from tests._helpers import f64
from tests.gpu_util import OUT_NAMES, assert_parity, check_fwd_bwd, compare, run_gpu, say
from tests.test_gpu_parity import _sampled
from workloads import CONFIGS, make_inputs, small_spec

pytestmark = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def zigzag(P, C, lo=0):
    """Start positions of the chunks in zigzag all-gather order: rank r
    brings position chunks r and 2P-1-r."""
    return tuple(lo + c * C for r in range(P) for c in (r, 2 * P - 1 - r))


SMALL = [
    ("bf16_zigzag_P4", dict(L=1024, B=32, H=8, Hkv=2, d=128, dtype="bf16", std=0.5),
     dict(kv_chunk_len=128, kv_chunk_pos=zigzag(4, 128))),
    ("bf16_share_reversed", dict(L=1024, B=16, H=4, Hkv=1, d=128, dtype="bf16", std=0.5,
                                 n_clean_q=256, clean_q_start=512, n_clean_kv=1024,
                                 corr_block_ids=[2, 9, 31, 40, 63]),
     dict(kv_chunk_len=256, kv_chunk_pos=(768, 512, 256, 0))),
    ("bf16_docs_token_causal", dict(L=1024, B=32, H=4, Hkv=2, d=128, dtype="bf16", std=0.5,
                                    clean_mask=1, doc_starts=[0, 96, 320, 704]),
     dict(kv_chunk_len=128, kv_chunk_pos=zigzag(4, 128))),
    ("f32_zigzag_d32", dict(L=512, B=16, H=4, Hkv=2, d=32, dtype="f32"),
     dict(kv_chunk_len=128, kv_chunk_pos=zigzag(2, 128))),
    ("bf16_d32_zigzag", dict(L=768, B=32, H=6, Hkv=2, d=32, dtype="bf16", std=0.5),
     dict(kv_chunk_len=128, kv_chunk_pos=zigzag(3, 128))),
]


@pytest.mark.parametrize("label,kw,g", SMALL, ids=[c[0] for c in SMALL])
def test_gathered_buffer_small(label, kw, g):
    _need_gpu()
    spec = small_spec(name=label, seed=zlib.crc32(label.encode()) % 10000, **kw).with_(**g)
    say(f"[gpu] gathered buffer {label}: chunks {spec.kv_chunk_pos}")
    t = make_inputs(spec, device="cuda")
    errs = check_fwd_bwd(spec, t, label)
    assert_parity(spec, errs, label)


def _to_buffer(spec, x):
    """Rows of a position-ordered clean tensor in the gathered buffer's order."""
    idx = torch.as_tensor(np.asarray(spec.kv_positions()) - spec.clean_kv_start, device=x.device)
    return x[idx].contiguous()


def _to_positions(spec, x):
    """Rows of a gathered-buffer tensor in position order."""
    order = np.argsort(np.asarray(spec.kv_positions()))
    return x[torch.as_tensor(order, device=x.device)].contiguous()


def test_zigzag_ranks_at_8k_over_one_gathered_buffer():
    """The 8K workload's P = 4 zigzag ranks: rank r holds the query chunks r
    and 7 - r (each a launch) and the dual-end corrupted blocks, over one
    buffer of all eight chunks in gathered order. Each launch equals the same
    launch over the position-ordered buffer bitwise (dK/dV rows permuted), and
    rank 1's launches pass the oracle gate on sampled rows and keys."""
    _need_gpu()
    base = CONFIGS[1]
    P, B, L = 4, base.B, base.n_clean_q
    C = L // (2 * P)
    nb = L // B
    owner = {}
    for r in range(P):
        for k in range(nb // (2 * P)):
            owner[r + k * P] = r
            owner[nb - 1 - (r + k * P)] = r
    t = make_inputs(base, device="cuda")
    for r in range(P):
        ids = tuple(sorted(b for b, o in owner.items() if o == r))
        for qc, with_blocks in ((r, True), (2 * P - 1 - r, False)):
            plain = base.with_(name=f"8k_rank{r}_chunk{qc}", n_clean_q=C, clean_q_start=qc * C,
                               n_corr_blocks=len(ids) if with_blocks else 0,
                               corr_block_ids=ids if with_blocks else ())
            gath = plain.with_(kv_chunk_len=C, kv_chunk_pos=zigzag(P, C))
            xr = np.concatenate([np.arange(b * B, (b + 1) * B) for b in plain.corr_block_ids]) \
                if plain.corr_block_ids else np.zeros(0, np.int64)
            xr = torch.as_tensor(xr, device="cuda")
            tp = dict(q_c=t["q_c"][qc * C:(qc + 1) * C], k_c=t["k_c"], v_c=t["v_c"],
                      q_x=t["q_x"][xr], k_x=t["k_x"][xr], v_x=t["v_x"][xr],
                      do_c=t["do_c"][qc * C:(qc + 1) * C], do_x=t["do_x"][xr])
            tp = {k: v.contiguous() for k, v in tp.items()}
            tg = dict(tp, k_c=_to_buffer(gath, tp["k_c"]), v_c=_to_buffer(gath, tp["v_c"]))
            say(f"  rank {r}, query chunk {qc}: gathered vs position-ordered buffer")
            a = run_gpu(plain, tp)
            b = run_gpu(gath, tg)
            for k in OUT_NAMES:
                y = _to_positions(gath, b[k]) if k in ("dk_c", "dv_c") else b[k]
                assert torch.equal(a[k], y), (r, qc, k)
            if r == 1:  # the oracle on sampled rows and keys, position order
                got = dict(b, dk_c=_to_positions(gath, b["dk_c"]),
                           dv_c=_to_positions(gath, b["dv_c"]))
                have, want = _sampled(plain, tp, got, kv_groups=(0,))
                _, ideal = _sampled(plain, tp, got, kv_groups=(0,), rounding="bf16")
                errs = compare(plain, have, want, names=list(want), label=plain.name,
                               ideal=ideal)
                assert_parity(plain, errs, plain.name)
