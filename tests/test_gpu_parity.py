"""Parity of the HIP path (through the C ABI) with the float64 oracle.

Tolerances: fp32 problems max|x-y|/max|y| <= 1e-4 per output tensor. bf16
problems: every element of O, dQ, dK and dV within one bf16 ulp plus 2e-2 of
the exact result's RMS of the oracle evaluated with bf16 operands and bf16
outputs; LSE (float32) max|x-y|/rms(y) <= 2e-2. The literal measure
max|x-y|/rms(y) against the exact oracle is printed for every tensor (storing
even the exact result in bf16 scores 0.02-0.15 on these outputs, whose
magnitudes vary by orders between rows).

Small problems are compared element by element on every output; in bf16 the
backward is run on the bf16-operand oracle's saved O and LSE and compared
with that oracle's backward on the same saved outputs (see
gpu_util.check_fwd_bwd for why). The five
full-size workloads are compared on sampled query blocks, sampled corrupted
blocks, the clean keys of late blocks and, at 8K, of key block 0 and the
middle block (oracle sub-problems, see gpu_util), and every output element
is checked against identities that hold at any size.
"""
import time
import zlib

import numpy as np
import pytest
import torch

from tests._helpers import f64
from tests.gpu_util import (OUT_NAMES, assert_parity, check_fwd_bwd, clear_host_cache, compare,
                            run_gpu, say, sub_clean_block, sub_clean_keys, sub_corr_block)
from workloads import CONFIGS, Spec, make_inputs, small_spec

pytestmark = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def full_parity(spec, label):
    _need_gpu()
    say(f"[gpu] {label}: {spec}")
    t = make_inputs(spec, device="cuda")
    errs = check_fwd_bwd(spec, t, label)
    assert_parity(spec, errs, label)


SMALL = [
    # fp32: the kernels' full logic at fp32 precision (1e-4)
    ("f32_L256_B16", dict(L=256, B=16, H=2, Hkv=2, d=32, dtype="f32")),
    ("f32_ragged_B8_G2", dict(L=200, B=8, H=4, Hkv=2, d=32, dtype="f32")),
    ("f32_B1", dict(L=70, B=1, H=2, Hkv=1, d=32, dtype="f32")),
    ("f32_B96", dict(L=288, B=96, H=4, Hkv=4, d=32, dtype="f32")),
    ("f32_G3", dict(L=160, B=16, H=6, Hkv=2, d=32, dtype="f32")),
    ("f32_share", dict(L=128, B=16, H=4, Hkv=1, d=32, dtype="f32", n_clean_q=64,
                        clean_q_start=64, n_clean_kv=128, corr_block_ids=[1, 3, 5, 7])),
    # bf16, head dim 128
    ("bf16_L1056_B32_G4", dict(L=1056, B=32, H=8, Hkv=2, d=128, dtype="bf16", std=0.5)),
    ("bf16_L512_B16_G1", dict(L=512, B=16, H=4, Hkv=4, d=128, dtype="bf16", std=0.5)),
    ("bf16_L640_B128_G8", dict(L=640, B=128, H=8, Hkv=1, d=128, dtype="bf16", std=0.5)),
    ("bf16_L300_B5_G2", dict(L=300, B=5, H=4, Hkv=2, d=128, dtype="bf16", std=0.5)),
    ("bf16_B1", dict(L=96, B=1, H=2, Hkv=2, d=128, dtype="bf16", std=0.5)),
    ("bf16_L768_B256", dict(L=768, B=256, H=4, Hkv=1, d=128, dtype="bf16", std=0.5)),
    ("bf16_d32_G3", dict(L=384, B=32, H=6, Hkv=2, d=32, dtype="bf16", std=0.5)),
    ("bf16_outliers", dict(L=1024, B=32, H=8, Hkv=2, d=128, dtype="bf16", std=0.5,
                           outlier_frac=0.01, outlier_mult=8.0)),
    # one rank's share: offset clean queries, long clean buffer, strided blocks
    ("bf16_share_strided", dict(L=512, B=32, H=8, Hkv=2, d=128, dtype="bf16", std=0.5,
                                n_clean_q=128, clean_q_start=384, n_clean_kv=512,
                                corr_block_ids=list(range(3, 16, 4)))),
    # dual-end pairing of blocks b and nb-1-b
    ("bf16_share_dualend", dict(L=256, B=16, H=4, Hkv=2, d=128, dtype="bf16", std=0.5,
                                n_clean_q=64, clean_q_start=64, n_clean_kv=256,
                                corr_block_ids=[1, 5, 10, 14])),
    # a rank holding no clean queries, and one holding no corrupted blocks
    ("bf16_no_clean_q", dict(L=0, B=32, H=4, Hkv=2, d=128, dtype="bf16", std=0.5,
                             n_clean_q=0, n_clean_kv=640, corr_block_ids=[0, 7, 20])),
    ("bf16_no_corrupted", dict(L=320, B=32, H=4, Hkv=2, d=128, dtype="bf16", std=0.5,
                               corr_block_ids=[])),
    # token-causal clean mask (clean queries see their own block up to their
    # position): inside the key tiles of the forward and dQ kernels, across
    # them (blocks larger than a tile), with ragged blocks, and in rank shares
    ("f32_token_causal", dict(L=256, B=16, H=2, Hkv=2, d=32, dtype="f32", clean_mask=1)),
    ("f32_token_causal_share", dict(L=128, B=16, H=4, Hkv=1, d=32, dtype="f32", n_clean_q=64,
                                    clean_q_start=64, n_clean_kv=128,
                                    corr_block_ids=[1, 3, 5, 7], clean_mask=1)),
    ("bf16_token_causal_G4", dict(L=1056, B=32, H=8, Hkv=2, d=128, dtype="bf16", std=0.5,
                                  clean_mask=1)),
    ("bf16_token_causal_B256", dict(L=768, B=256, H=4, Hkv=1, d=128, dtype="bf16", std=0.5,
                                    clean_mask=1)),
    ("bf16_token_causal_d32_B5", dict(L=300, B=5, H=6, Hkv=2, d=32, dtype="bf16", std=0.5,
                                      clean_mask=1)),
    ("bf16_token_causal_share", dict(L=512, B=32, H=8, Hkv=2, d=128, dtype="bf16", std=0.5,
                                     n_clean_q=128, clean_q_start=384, n_clean_kv=512,
                                     corr_block_ids=list(range(3, 16, 4)), clean_mask=1)),
    # complementary masking: two corrupted copies of the same target block
    ("f32_complementary", dict(L=128, B=16, H=2, Hkv=1, d=32, dtype="f32",
                               corr_block_ids=[0, 0, 1, 2, 2, 5, 7, 7])),
    ("bf16_complementary", dict(L=512, B=32, H=8, Hkv=2, d=128, dtype="bf16", std=0.5,
                                corr_block_ids=[b for b in range(16) for _ in (0, 1)])),
    ("bf16_complementary_share", dict(L=512, B=32, H=8, Hkv=2, d=128, dtype="bf16", std=0.5,
                                      n_clean_q=128, clean_q_start=384, n_clean_kv=512,
                                      corr_block_ids=[3, 3, 7, 7, 11, 11, 15, 15])),
]


@pytest.mark.parametrize("label,kw", SMALL, ids=[s[0] for s in SMALL])
def test_small_full_parity(label, kw):
    full_parity(small_spec(name=label, seed=zlib.crc32(label.encode()) % 10000, **kw), label)


def test_tiny_workload_full_parity():
    """The tiny fp32 workload (clean 256 + corrupted 256, B=16, H=Hkv=2, d=32)."""
    full_parity(CONFIGS[0], CONFIGS[0].name)


def test_repeat_calls_and_determinism():
    """No output is accumulated with atomics (the work-claim counters only
    choose which workgroup runs an item) and every output element is written
    by one thread, so repeated calls are bitwise identical."""
    _need_gpu()
    spec = small_spec(L=512, B=32, H=8, Hkv=2, d=128, dtype="bf16", std=0.5, seed=3)
    t = make_inputs(spec, device="cuda")
    a = run_gpu(spec, t)
    b = run_gpu(spec, t)
    for k in OUT_NAMES:
        assert torch.equal(a[k], b[k]), k


def test_outputs_fully_overwritten():
    """NaN-poisoned output buffers are overwritten everywhere (including
    clean keys no local query sees, which get zero gradients)."""
    _need_gpu()
    import block_masked_attention_amd as bd
    spec = small_spec(L=256, B=32, H=4, Hkv=2, d=128, dtype="bf16", std=0.5, n_clean_q=64,
                      clean_q_start=64, n_clean_kv=256, corr_block_ids=[2, 3], seed=5)
    t = make_inputs(spec, device="cuda")
    p = bd.from_spec(spec)
    nan = lambda x: torch.full_like(x, float("nan"))
    o = [nan(t["q_c"]), nan(t["q_x"]),
         torch.full((spec.H, spec.n_clean_q), float("nan"), device="cuda"),
         torch.full((spec.H, spec.n_corr), float("nan"), device="cuda")]
    o_c, o_x, lse_c, lse_x = bd.fwd(p, *[t[k] for k in ("q_c", "k_c", "v_c", "q_x", "k_x", "v_x")],
                                    out=o)
    g = [nan(t["q_c"]), nan(t["q_x"]), nan(t["k_c"]), nan(t["v_c"]), nan(t["k_x"]), nan(t["v_x"])]
    dq_c, dq_x, dk_c, dv_c, dk_x, dv_x = bd.bwd(
        p, *[t[k] for k in ("q_c", "k_c", "v_c", "q_x", "k_x", "v_x")], o_c, o_x, lse_c, lse_x,
        t["do_c"], t["do_x"], out=g)
    torch.cuda.synchronize()
    for x in (o_c, o_x, lse_c, lse_x, dq_c, dq_x, dk_c, dv_c, dk_x, dv_x):
        assert torch.isfinite(x).all()
    # clean keys past every local query's prefix (positions >= 128) are unseen
    assert (dk_c[128:] == 0).all() and (dv_c[128:] == 0).all()


# ------------------------------------------------------------- full size
def _identities(spec, t, got):
    """Identities of softmax attention that hold at any size, per KV head:
    sum_j dV_j = sum_i,h dO_i;  sum_j <dV_j, v_j> = sum_i <dO_i, O_i>;
    sum_i <dQ_i, q_i> = sum_j <dK_j, k_j>."""
    G = spec.H // spec.Hkv
    d = lambda x: x.double()
    for g in range(spec.Hkv):
        hq = slice(g * G, (g + 1) * G)
        dv = torch.cat([d(got["dv_c"][:, g]), d(got["dv_x"][:, g])])
        do = torch.cat([d(t["do_c"][:, hq]), d(t["do_x"][:, hq])]).reshape(-1, spec.d)
        lhs, rhs = dv.sum(0), do.sum(0)
        tol = 2e-2 * dv.pow(2).sum(0).sqrt() + 1e-3 * do.abs().sum(0).sqrt()
        assert ((lhs - rhs).abs() <= tol).all(), f"sum dV identity, kv head {g}"
        v = torch.cat([d(t["v_c"][:, g]), d(t["v_x"][:, g])])
        o = torch.cat([d(got["o_c"][:, hq]), d(got["o_x"][:, hq])]).reshape(-1, spec.d)
        a1, b1 = (dv * v).sum(), (do * o).sum()
        assert abs(a1 - b1) <= 2e-2 * (dv * v).abs().sum() ** 0.5 * 10 + 1e-2 * abs(b1), \
            f"<dV,v> identity, kv head {g}: {a1.item()} vs {b1.item()}"
        q = torch.cat([d(t["q_c"][:, hq]), d(t["q_x"][:, hq])]).reshape(-1, spec.d)
        dq = torch.cat([d(got["dq_c"][:, hq]), d(got["dq_x"][:, hq])]).reshape(-1, spec.d)
        k = torch.cat([d(t["k_c"][:, g]), d(t["k_x"][:, g])])
        dk = torch.cat([d(got["dk_c"][:, g]), d(got["dk_x"][:, g])])
        a2, b2 = (dq * q).sum(), (dk * k).sum()
        scale = max((dq * q).abs().sum().item(), (dk * k).abs().sum().item())
        assert abs(a2 - b2) <= 2e-2 * scale ** 0.5 * 10 + 1e-2 * max(abs(a2), abs(b2)), \
            f"<dQ,q> = <dK,k> identity, kv head {g}: {a2.item()} vs {b2.item()}"


def _sampled(spec, t, got, n_blocks=3, kv_groups=(0,), rounding=None, long_keys=(),
             with_keys=True):
    """Sampled outputs of the GPU result ``got`` and of the oracle: query
    blocks of both streams (O, LSE, dQ; corrupted dK/dV), and the clean
    dK/dV of the last key blocks (few query blocks see them) plus, for the
    first KV group, ``long_keys``: key blocks whose gradients accumulate over
    long runs of query blocks (key block 0 is seen by every query)."""
    B = spec.B
    if spec.n_clean_kv > 100_000:
        n_blocks = 1  # each sampled block carries a prefix of 10^5+ keys
    rng = np.random.default_rng(spec.seed)
    cb0, cb1 = spec.clean_q_start // B, (spec.clean_q_start + spec.n_clean_q) // B
    clean_blocks = sorted({cb0, cb1 - 1} | set(rng.integers(cb0, cb1, n_blocks).tolist())) \
        if cb1 > cb0 else []
    corr = sorted({0, spec.n_corr_blocks - 1} |
                  set(rng.integers(0, spec.n_corr_blocks, n_blocks).tolist())) \
        if spec.n_corr_blocks else []
    key_blocks = [cb1 - 1, cb1 - 3]
    if spec.doc_starts:  # query blocks on both sides of two document starts, and the
        for s in [x // B for x in spec.doc_starts[1:3]]:  # last keys before each
            clean_blocks = sorted(set(clean_blocks) | {b for b in (s - 1, s) if cb0 <= b < cb1})
            key_blocks = sorted(set(key_blocks) | {s - 1})
    want = {k: [] for k in OUT_NAMES}
    have = {k: [] for k in OUT_NAMES}
    for g in kv_groups:
        for b in clean_blocks:
            say(f"  oracle clean block {b}, kv head {g}")
            r = sub_clean_block(spec, t, b, g, rounding)
            (r0, r1), (h0, h1) = r["rows"], r["heads"]
            for k in ("o_c", "dq_c"):
                want[k].append(r[k].ravel())
                have[k].append(f64(got[k][r0:r1, h0:h1]).ravel())
            want["lse_c"].append(r["lse_c"].ravel())
            have["lse_c"].append(f64(got["lse_c"][h0:h1, r0:r1]).ravel())
        for j in corr:
            say(f"  oracle corrupted block {j}, kv head {g}")
            r = sub_corr_block(spec, t, j, g, rounding)
            (r0, r1), (h0, h1), (k0, k1) = r["rows"], r["heads"], r["kv"]
            for k in ("o_x", "dq_x"):
                want[k].append(r[k].ravel())
                have[k].append(f64(got[k][r0:r1, h0:h1]).ravel())
            want["lse_x"].append(r["lse_x"].ravel())
            have["lse_x"].append(f64(got["lse_x"][h0:h1, r0:r1]).ravel())
            for k in ("dk_x", "dv_x"):
                want[k].append(r[k].ravel())
                have[k].append(f64(got[k][r0:r1, k0:k1]).ravel())
        kbs = key_blocks if g != kv_groups[0] else sorted(set(key_blocks) | set(long_keys))
        for kb in (kbs if with_keys else ()):
            say(f"  oracle clean keys of block {kb}, kv head {g}")
            r = sub_clean_keys(spec, t, kb, g, rounding)
            (a0, a1), (k0, k1) = r["keys"], r["kv"]
            for k in ("dk_c", "dv_c"):
                want[k].append(r[k].ravel())
                have[k].append(f64(got[k][a0:a1, k0:k1]).ravel())
    clear_host_cache()
    want = {k: np.concatenate(v) for k, v in want.items() if v}
    have = {k: np.concatenate(v) for k, v in have.items() if v}
    return have, want


@pytest.mark.parametrize("idx", [0, 1, 2, 3, 4], ids=[c.name for c in CONFIGS])
def test_workload_sampled_parity(idx):
    """Each of the five workloads at full size, launched as the benchmark
    launches it."""
    workload_parity(CONFIGS[idx])


def packed(spec, n, seed=1234):
    """The workload with n documents cut at n - 1 seeded random block
    boundaries (as bench.py --docs n cuts them)."""
    nb = (spec.clean_q_start + spec.n_clean_q) // spec.B
    cuts = np.sort(np.random.default_rng(seed).choice(np.arange(1, nb), n - 1, replace=False))
    return spec.with_(doc_starts=(0,) + tuple(int(c) * spec.B for c in cuts))


@pytest.mark.parametrize("idx,n,cm", [(2, 8, 0), (3, 16, 0), (1, 128, 0), (2, 1024, 0), (2, 8, 1)],
                         ids=["64k_docs8", "256k_docs16", "8k_docs128", "64k_docs1024",
                              "64k_docs8_token_causal"])
def test_packed_documents_workload_sampled_parity(idx, n, cm):
    """Full-size workloads with packed documents, launched as `bench.py
    --docs n` launches them: 64K with 8 and 256K with 16 documents, many
    short ones (8K with 128, 64K with 1024: 64 tokens on average), and 64K
    with 8 under the token-causal clean mask; the samples include the blocks
    on both sides of two document starts (one KV group)."""
    workload_parity(packed(CONFIGS[idx].with_(clean_mask=cm), n), groups=(0,))


@pytest.mark.parametrize("idx", [1, 2], ids=[CONFIGS[i].name for i in (1, 2)])
def test_token_causal_workload_sampled_parity(idx):
    """The 8K and 64K workloads at full size with the token-causal clean mask."""
    workload_parity(CONFIGS[idx].with_(clean_mask=1))


def long_key_blocks(spec):
    """Clean key blocks checked element-wise whose dK/dV accumulate over long
    runs of query blocks: key block 0 (seen by every query) and the middle
    block, where the oracle for them costs seconds (the 8K workload: 16,384
    and 8,192 query rows, each with its full visible prefix). At 64K and
    beyond one such block costs the oracle tens of minutes (every row that
    sees it needs its whole forward); there the whole-tensor identities and
    the 8K check stand in."""
    if spec.n_clean_kv > 8192 or spec.clean_q_start:
        return ()
    nb = spec.n_clean_kv // spec.B
    return (0, nb // 2)


def workload_parity(spec, groups=None):
    _need_gpu()
    say(f"[gpu] workload {spec.name} (clean mask {spec.clean_mask}): {spec.description}")
    t0 = time.perf_counter()
    t = make_inputs(spec, device="cuda")
    got = run_gpu(spec, t)
    say(f"  inputs + fwd + bwd on the GPU: {time.perf_counter() - t0:.1f} s")
    for k, v in got.items():
        assert torch.isfinite(v).all(), f"{k} has non-finite values"
    _identities(spec, t, got)
    say(f"  identities checked: {time.perf_counter() - t0:.1f} s")
    if groups is None:
        groups = (0,) if spec.Hkv == 1 else (0, spec.Hkv - 1)
    long_keys = long_key_blocks(spec)
    have, want = _sampled(spec, t, got, kv_groups=groups, long_keys=long_keys)
    say(f"  exact oracle samples: {time.perf_counter() - t0:.1f} s")
    ideal = None
    if spec.dtype == "bf16":
        _, ideal = _sampled(spec, t, got, kv_groups=groups, rounding="bf16",
                            long_keys=long_keys)
        say(f"  bf16-operand oracle samples: {time.perf_counter() - t0:.1f} s")
    errs = compare(spec, have, want, names=list(want), label=spec.name, ideal=ideal)
    assert_parity(spec, errs, spec.name)


def _random_specs(n=16, seed=2024):
    """Seeded random small problems mixing every option of the descriptor:
    block size, GQA ratio, head dim and dtype, a rank's share (clean query
    range, clean buffer length), a subset of corrupted blocks with repeated
    ids (complementary copies), and the clean mask."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        dtype, d = [("f32", 32), ("bf16", 32), ("bf16", 128)][int(rng.integers(3))]
        B = int(rng.choice([1, 2, 3, 4, 8, 16, 32, 48, 64]))
        nb = int(rng.integers(2, max(3, 640 // B) + 1))
        Hkv = int(rng.choice([1, 2, 4]))
        H = Hkv * int(rng.choice([1, 2, 3, 4]))
        cq0 = int(rng.integers(0, nb))
        cq1 = int(rng.integers(cq0, nb + 1))
        ids = sorted(rng.choice(nb, size=int(rng.integers(0, nb + 1)), replace=False).tolist())
        if ids and rng.random() < 0.4:  # complementary copies of some blocks
            ids = sorted(ids + rng.choice(ids, size=int(rng.integers(1, len(ids) + 1))).tolist())
        if cq1 == cq0 and not ids:
            continue
        need = max(cq1, max(ids) if ids else 0)  # clean blocks the local queries see
        n_kv = int(rng.integers(need, nb + 1)) * B
        out.append((f"rand{len(out)}_{dtype}_d{d}_B{B}_H{H}_{Hkv}",
                    dict(L=cq1 * B, B=B, H=H, Hkv=Hkv, d=d, dtype=dtype,
                         std=1.0 if dtype == "f32" else 0.5,
                         n_clean_q=(cq1 - cq0) * B, clean_q_start=cq0 * B, n_clean_kv=n_kv,
                         corr_block_ids=ids, clean_mask=int(rng.integers(2)))))
    return out


RANDOM = _random_specs()

# packed documents (block-aligned starts): documents not aligned to the
# kernels' 64- and 128-row tiles, one-block documents, aligned documents (the
# backward's unmasked tiles), shares and complementary copies
DOCS = [
    ("docs_bf16_unaligned_G4", dict(L=2048, B=32, H=8, Hkv=2, d=128, dtype="bf16", std=0.5,
                                    doc_starts=[0, 96, 160, 192, 1024, 1056])),
    ("docs_bf16_aligned_B64", dict(L=1024, B=64, H=4, Hkv=1, d=128, dtype="bf16", std=0.5,
                                   doc_starts=[0, 256, 512, 768])),
    ("docs_bf16_token_causal", dict(L=1024, B=32, H=4, Hkv=2, d=128, dtype="bf16", std=0.5,
                                    doc_starts=[0, 64, 448, 480], clean_mask=1)),
    ("docs_f32_share_copies", dict(L=512, B=16, H=4, Hkv=2, d=32, dtype="f32",
                                   n_clean_q=256, clean_q_start=256, n_clean_kv=512,
                                   corr_block_ids=[3, 5, 5, 17, 18, 18, 30],
                                   doc_starts=[0, 80, 288, 400])),
    ("docs_f32_B1", dict(L=200, B=1, H=2, Hkv=1, d=32, dtype="f32",
                         doc_starts=[0, 1, 2, 70, 71, 199])),
    ("docs_bf16_d32_one_block_each", dict(L=512, B=32, H=6, Hkv=2, d=32, dtype="bf16", std=0.5,
                                          doc_starts=list(range(0, 512, 32)))),
]


@pytest.mark.parametrize("label,kw", DOCS, ids=[c[0] for c in DOCS])
def test_packed_documents(label, kw):
    full_parity(small_spec(name=label, seed=zlib.crc32(label.encode()) % 10000, **kw), label)


def _random_doc_specs(n=8, seed=77):
    """Seeded random packed problems: a random problem (as above) whose
    sequence is cut into random block-aligned documents."""
    rng = np.random.default_rng(seed)
    out = []
    for i, (label, kw) in enumerate(_random_specs(n, seed)):
        nb = kw["L"] // kw["B"]
        cuts = sorted(set(rng.choice(np.arange(1, max(2, nb)), size=int(rng.integers(1, 6))).tolist()))
        kw = dict(kw, doc_starts=[0] + [c * kw["B"] for c in cuts if c < nb])
        out.append((label.replace("rand", "randdocs"), kw))
    return out


RANDOM_DOCS = _random_doc_specs()


@pytest.mark.parametrize("label,kw", RANDOM_DOCS, ids=[r[0] for r in RANDOM_DOCS])
def test_random_packed_documents(label, kw):
    full_parity(small_spec(name=label, seed=zlib.crc32(label.encode()) % 10000, **kw), label)


@pytest.mark.parametrize("label,kw", RANDOM, ids=[r[0] for r in RANDOM])
def test_random_small_problems(label, kw):
    full_parity(small_spec(name=label, seed=zlib.crc32(label.encode()) % 10000, **kw), label)


def test_side_stream_calls_keep_their_memory():
    """fwd/bwd enqueued on a side stream, with the current stream allocating
    and overwriting freshly freed memory while that work is queued behind a
    long kernel: the results equal those of calls on the current stream
    (the workspace and outputs belong to the side stream's pool)."""
    _need_gpu()
    import block_masked_attention_amd as bd
    spec = small_spec(L=2048, B=32, H=8, Hkv=2, d=128, dtype="bf16", std=0.5, seed=12)
    t = make_inputs(spec, device="cuda")
    want = run_gpu(spec, t)
    p = bd.from_spec(spec)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    big = torch.randn(4096, 4096, device="cuda")
    with torch.cuda.stream(side):
        for _ in range(20):  # keep the side stream busy before the bdattn calls
            big = big @ big.T / 4096.0
    f = bd.fwd(p, *[t[k] for k in ("q_c", "k_c", "v_c", "q_x", "k_x", "v_x")], stream=side)
    g = bd.bwd(p, *[t[k] for k in ("q_c", "k_c", "v_c", "q_x", "k_x", "v_x")], *f,
               t["do_c"], t["do_x"], stream=side)
    for _ in range(8):  # the current stream reuses whatever the caching allocator frees
        junk = torch.full((8 << 20,), float("nan"), device="cuda")
        del junk
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for k, a in zip(OUT_NAMES, tuple(f) + tuple(g)):
        assert torch.equal(a, want[k]), k


def test_plan_cache_recycles_staging_under_in_flight_calls():
    """150 forward calls, each with a new packed-document layout, enqueued
    back to back without waiting, under a 2 MiB plan-cache budget: plans are
    evicted while their staging copies may still be queued. Every kept result
    equals a later call on the same layout, and pinned memory stays bounded."""
    _need_gpu()
    import block_masked_attention_amd as bd
    spec = small_spec(L=4096, B=32, H=8, Hkv=2, d=128, dtype="bf16", std=0.5, seed=21)
    t = make_inputs(spec, device="cuda")
    ins = [t[k] for k in ("q_c", "k_c", "v_c", "q_x", "k_x", "v_x")]
    before = bd.plan_cache_info()
    bd.plan_cache_budget(2 << 20)
    try:
        rng = np.random.default_rng(3)
        layouts, kept = [], {}
        for i in range(150):
            cuts = np.sort(rng.choice(np.arange(1, 128), 7, replace=False)) * 32
            docs = [0] + cuts.tolist()
            layouts.append(docs)
            out = bd.fwd(bd.from_spec(spec.with_(doc_starts=tuple(docs))), *ins)
            if i % 30 == 0:
                kept[i] = out
            info = bd.plan_cache_info()
            assert info["pinned_bytes"] <= (3 << 20), info
        torch.cuda.synchronize()
        assert bd.plan_cache_info()["evictions"] > before["evictions"] + 100
        for i, out in kept.items():
            again = bd.fwd(bd.from_spec(spec.with_(doc_starts=tuple(layouts[i]))), *ins)
            torch.cuda.synchronize()
            for a, b in zip(out, again):
                assert torch.equal(a, b), i
    finally:
        bd.plan_cache_budget(before["budget"])
