"""Parity of the split, partial form on the GPU ("Block Parallelism for
Efficient Distributed Long-Context Diffusion Language Model Training",
appendix, Efficient fused operator, Implementation 1): the block-diagonal
corrupted part and clean K/V shards at their original positions run as
separate partial launches (descriptor partial = 1), bdattn_merge combines
their results, and the backward of each part, given the merged O and LSE,
returns the parts of the gradients.

Checked against the float64 oracle: each partial forward against the
oracle's partial layout; the merged forward and the assembled gradients
against the oracle's complete problem. Tolerances are those of the full
parity tests (fp32: 1e-4 norm-wise; bf16: every element within one bf16 ulp
plus 2e-2 of the exact result's RMS of the bf16-operand oracle, which for the
split pipeline is evaluated with the pipeline's own roundings).
"""
import numpy as np
import pytest
import torch

import block_masked_attention_amd as bd
from oracle import Oracle, layout, merge_partials, round_bf16
from tests._helpers import f64
from tests.gpu_util import (OUT_NAMES, assert_parity, compare, oracle_full, saved_on_device,
                            say)
from workloads import GRAD_NAMES, INPUT_NAMES, make_inputs, small_spec

pytestmark = pytest.mark.gpu

CASES = [
    ("f32_split", dict(L=256, B=16, H=2, Hkv=2, d=32, dtype="f32")),
    ("bf16_split_G4", dict(L=1024, B=32, H=8, Hkv=2, d=128, dtype="bf16", std=0.5)),
    ("bf16_split_token_causal", dict(L=768, B=32, H=4, Hkv=1, d=128, dtype="bf16", std=0.5,
                                     clean_mask=1)),
    ("bf16_split_share", dict(L=512, B=32, H=8, Hkv=2, d=128, dtype="bf16", std=0.5,
                              n_clean_q=128, clean_q_start=384, n_clean_kv=512,
                              corr_block_ids=list(range(3, 16, 4)))),
    ("bf16_split_docs", dict(L=1024, B=32, H=4, Hkv=2, d=128, dtype="bf16", std=0.5,
                             doc_starts=[0, 96, 320, 352, 704])),
]


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def pieces(spec):
    """(lo, hi, corrupted keys present): the block-diagonal corrupted part,
    then the clean buffer in three shards at their original positions."""
    nkv, B = spec.n_clean_kv, spec.B
    cuts = [0, B * (nkv // B // 3), B * (2 * nkv // B // 3), nkv]
    return [(0, 0, True)] + [(a, b, False) for a, b in zip(cuts, cuts[1:]) if b > a]


def part_problem(spec, lo, hi, ck):
    return bd.problem(spec.B, spec.H, spec.Hkv, spec.d, spec.dtype, spec.n_clean_q,
                      spec.clean_q_start, hi - lo, lo, spec.n_corr_blocks, spec.corr_block_ids,
                      clean_mask=spec.clean_mask, partial=True, omit_corr_keys=not ck,
                      doc_starts=spec.doc_starts)


def part_inputs(t, lo, hi):
    u = dict(t)
    u["k_c"], u["v_c"] = t["k_c"][lo:hi].contiguous(), t["v_c"][lo:hi].contiguous()
    return u


def part_oracle(spec, t, lo, hi, ck):
    lay = layout(spec.B, spec.H, spec.Hkv, spec.d, spec.n_clean_q, spec.clean_q_start, hi - lo,
                 lo, corr_block_ids=spec.corr_block_ids, n_corr_blocks=spec.n_corr_blocks,
                 partial=True, clean_mask=spec.clean_mask, corr_keys=ck, doc_starts=spec.doc_starts)
    u = part_inputs(t, lo, hi)
    return Oracle(lay, *[f64(u[k]) for k in INPUT_NAMES], *[f64(u[k]) for k in GRAD_NAMES])


@pytest.mark.parametrize("label,kw", CASES, ids=[c[0] for c in CASES])
def test_partial_forwards_match_the_oracle(label, kw):
    """Each partial launch alone: rows that see no key present get exactly
    O = 0 and LSE = -inf; the others match the oracle's partial layout."""
    _need_gpu()
    spec = small_spec(name=label, seed=77, **kw)
    t = make_inputs(spec, device="cuda")
    for lo, hi, ck in pieces(spec):
        say(f"[gpu] {label}: partial forward over clean [{lo}, {hi}), corrupted keys {ck}")
        got = bd.fwd(part_problem(spec, lo, hi, ck), *[part_inputs(t, lo, hi)[k] for k in INPUT_NAMES])
        want = part_oracle(spec, t, lo, hi, ck).forward()
        got = dict(zip(OUT_NAMES[:4], (f64(x) for x in got)))
        want = dict(zip(OUT_NAMES[:4], want))
        for s in ("c", "x"):
            empty = np.isneginf(want["lse_" + s])
            assert np.array_equal(np.isneginf(got["lse_" + s]), empty), f"{label}: empty rows ({s})"
            assert np.all(got["o_" + s][empty.any(axis=0)] == 0) or not empty.any()
            got["lse_" + s] = np.where(empty, 0.0, got["lse_" + s])
            want["lse_" + s] = np.where(empty, 0.0, want["lse_" + s])
        ideal = part_oracle_bf16(spec, t, lo, hi, ck) if spec.dtype == "bf16" else None
        errs = compare(spec, got, want, names=list(want), label=f"{label}[{lo},{hi})",
                       ideal=ideal)
        assert_parity(spec, errs, label)


def part_oracle_bf16(spec, t, lo, hi, ck):
    lay = layout(spec.B, spec.H, spec.Hkv, spec.d, spec.n_clean_q, spec.clean_q_start, hi - lo,
                 lo, corr_block_ids=spec.corr_block_ids, n_corr_blocks=spec.n_corr_blocks,
                 partial=True, clean_mask=spec.clean_mask, corr_keys=ck, doc_starts=spec.doc_starts)
    u = part_inputs(t, lo, hi)
    f = Oracle(lay, *[f64(u[k]) for k in INPUT_NAMES], operand_rounding="bf16").forward()
    out = dict(zip(OUT_NAMES[:4], f))
    for s in ("c", "x"):
        out["lse_" + s] = np.where(np.isneginf(out["lse_" + s]), 0.0, out["lse_" + s])
    return out


@pytest.mark.parametrize("label,kw", CASES, ids=[c[0] for c in CASES])
def test_split_forward_merge_and_backward_equal_the_full_problem(label, kw):
    """The whole split pipeline: partial forwards merged with bdattn_merge
    equal the complete attention; the backward of each part with the merged
    O and LSE gives dQ parts that sum (in fp32) to the full dQ, each clean
    shard's complete dK/dV, and the corrupted keys' dK/dV from the
    block-diagonal part."""
    _need_gpu()
    spec = small_spec(name=label, seed=78, **kw)
    t = make_inputs(spec, device="cuda")
    tin = [t[k] for k in INPUT_NAMES]
    merged = None
    for lo, hi, ck in pieces(spec):
        r = bd.fwd(part_problem(spec, lo, hi, ck), *[part_inputs(t, lo, hi)[k] for k in INPUT_NAMES])
        if merged is None:
            merged = list(r)
            continue
        merged[0], merged[2] = bd.merge(merged[0], merged[2], r[0], r[2])
        merged[1], merged[3] = bd.merge(merged[1], merged[3], r[1], r[3])
    o_c, o_x, lse_c, lse_x = merged
    dq_c = torch.zeros(o_c.shape, dtype=torch.float32, device=o_c.device)
    dq_x = torch.zeros(o_x.shape, dtype=torch.float32, device=o_x.device)
    dk_c, dv_c, dk_x, dv_x = [], [], None, None
    for lo, hi, ck in pieces(spec):
        u = part_inputs(t, lo, hi)
        g = bd.bwd(part_problem(spec, lo, hi, ck), *[u[k] for k in INPUT_NAMES],
                   o_c, o_x, lse_c, lse_x, t["do_c"], t["do_x"])
        dq_c += g[0].float()
        dq_x += g[1].float()
        if hi > lo:
            dk_c.append(g[2])
            dv_c.append(g[3])
        if ck:
            dk_x, dv_x = g[4], g[5]
    torch.cuda.synchronize()
    got = dict(zip(OUT_NAMES, (o_c, o_x, lse_c, lse_x, dq_c, dq_x, torch.cat(dk_c),
                               torch.cat(dv_c), dk_x, dv_x)))
    want = oracle_full(spec, t)
    ideal = split_pipeline_bf16(spec, t) if spec.dtype == "bf16" else None
    errs = compare(spec, got, want, label=label, ideal=ideal)
    assert_parity(spec, errs, label)


def split_pipeline_bf16(spec, t):
    """The split pipeline evaluated by the oracle in bf16-operand mode, with
    the pipeline's own roundings: each part's O stored in bf16, each merge's O
    stored in bf16 (oracle.merge_partials), each part's dQ stored in bf16 and
    the parts summed, each shard's dK/dV stored in bf16."""
    merged = None
    for lo, hi, ck in pieces(spec):
        lay = part_oracle(spec, t, lo, hi, ck).lay
        u = part_inputs(t, lo, hi)
        f = Oracle(lay, *[f64(u[k]) for k in INPUT_NAMES], operand_rounding="bf16").forward()
        if merged is None:
            merged = list(f)
            continue
        for o, l in ((0, 2), (1, 3)):
            mo, ml = merge_partials([(merged[o], merged[l]), (f[o], f[l])])
            merged[o], merged[l] = round_bf16(mo), ml
    O = np.concatenate([merged[0], merged[1]])
    LSE = np.concatenate([merged[2], merged[3]], axis=1)
    out = dict(o_c=merged[0], o_x=merged[1], lse_c=merged[2], lse_x=merged[3])
    out["dq_c"], out["dq_x"], dk_c, dv_c = 0.0, 0.0, [], []
    for lo, hi, ck in pieces(spec):
        lay = part_oracle(spec, t, lo, hi, ck).lay
        u = part_inputs(t, lo, hi)
        g = Oracle(lay, *[f64(u[k]) for k in INPUT_NAMES], *[f64(u[k]) for k in GRAD_NAMES],
                   operand_rounding="bf16").backward(O=O, LSE=LSE)
        out["dq_c"] = out["dq_c"] + g[0]
        out["dq_x"] = out["dq_x"] + g[1]
        if hi > lo:
            dk_c.append(g[2])
            dv_c.append(g[3])
        if ck:
            out["dk_x"], out["dv_x"] = g[4], g[5]
    out["dk_c"], out["dv_c"] = np.concatenate(dk_c), np.concatenate(dv_c)
    return out


def _random_partials(n=10, seed=4242):
    """Seeded random partial problems: a complete problem (block size, GQA,
    share, block subset with repeats, clean mask) and a random clean K/V
    range at original positions, with the corrupted keys kept or omitted."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        dtype, d = [("f32", 32), ("bf16", 128)][int(rng.integers(2))]
        B = int(rng.choice([1, 2, 4, 16, 32, 64]))
        nb = int(rng.integers(3, max(4, 512 // B) + 1))
        Hkv = int(rng.choice([1, 2]))
        H = Hkv * int(rng.choice([1, 2, 4]))
        cq0 = int(rng.integers(0, nb))
        ids = sorted(rng.choice(nb, size=int(rng.integers(1, nb + 1)), replace=False).tolist())
        if rng.random() < 0.3:
            ids = sorted(ids + [ids[0]])
        lo = int(rng.integers(0, nb)) * B
        hi = int(rng.integers(lo // B, nb + 1)) * B
        out.append((f"rpart{len(out)}_{dtype}_B{B}_[{lo},{hi})",
                    dict(L=nb * B, B=B, H=H, Hkv=Hkv, d=d, dtype=dtype,
                         std=1.0 if dtype == "f32" else 0.5, n_clean_q=(nb - cq0) * B,
                         clean_q_start=cq0 * B, n_clean_kv=nb * B, corr_block_ids=ids,
                         clean_mask=int(rng.integers(2))), lo, hi, bool(rng.integers(2))))
    return out


RANDOM_PARTIALS = _random_partials()


@pytest.mark.parametrize("label,kw,lo,hi,ck", RANDOM_PARTIALS, ids=[r[0] for r in RANDOM_PARTIALS])
def test_random_partial_problems(label, kw, lo, hi, ck):
    """One random partial launch, forward and backward: the forward against
    the oracle's partial layout (rows with no key present exactly O = 0,
    LSE = -inf); the backward, given the complete problem's O and LSE, against
    the oracle's partial backward with the oracle's complete O and LSE."""
    _need_gpu()
    spec = small_spec(name=label, seed=91, **kw)
    t = make_inputs(spec, device="cuda")
    u = part_inputs(t, lo, hi)
    p = part_problem(spec, lo, hi, ck)
    got = dict(zip(OUT_NAMES[:4], (f64(x) for x in bd.fwd(p, *[u[k] for k in INPUT_NAMES]))))
    orc = part_oracle(spec, t, lo, hi, ck)
    want = dict(zip(OUT_NAMES[:4], orc.forward()))
    for s in ("c", "x"):
        empty = np.isneginf(want["lse_" + s])
        assert np.array_equal(np.isneginf(got["lse_" + s]), empty), f"{label}: empty rows ({s})"
        got["lse_" + s] = np.where(empty, 0.0, got["lse_" + s])
        want["lse_" + s] = np.where(empty, 0.0, want["lse_" + s])
    ideal = part_oracle_bf16(spec, t, lo, hi, ck) if spec.dtype == "bf16" else None
    errs = compare(spec, got, want, names=list(want), label=label, ideal=ideal)
    # backward through the keys present, given the complete problem's saved O
    # and LSE: in fp32 the GPU's own; in bf16 the bf16-operand oracle's, the
    # same ones its backward below takes (see gpu_util.check_fwd_bwd)
    ref = oracle_full(spec, t)
    if spec.dtype == "bf16":
        rb = oracle_full(spec, t, "bf16")
        dev, saved = saved_on_device(rb, spec, t["q_c"].device)
        full = [dev[k] for k in OUT_NAMES[:4]]
    else:
        full = bd.fwd(bd.from_spec(spec), *[t[k] for k in INPUT_NAMES])
    g = bd.bwd(p, *[u[k] for k in INPUT_NAMES], *full, t["do_c"], t["do_x"])
    ob = orc.backward(O=np.concatenate([ref["o_c"], ref["o_x"]]),
                      LSE=np.concatenate([ref["lse_c"], ref["lse_x"]], axis=1))
    names = ["dq_c", "dq_x", "dk_c", "dv_c"] + (["dk_x", "dv_x"] if ck else [])
    gw = dict(zip(OUT_NAMES[4:], g))
    bw = dict(zip(OUT_NAMES[4:], ob))
    bideal = None
    if spec.dtype == "bf16":
        obr = Oracle(orc.lay, *[f64(u[k]) for k in INPUT_NAMES], *[f64(u[k]) for k in GRAD_NAMES],
                     operand_rounding="bf16")
        bideal = dict(zip(OUT_NAMES[4:], obr.backward(
            O=np.concatenate([saved["o_c"], saved["o_x"]]),
            LSE=np.concatenate([saved["lse_c"], saved["lse_x"]], axis=1))))
    errs.update(compare(spec, {k: gw[k] for k in names}, {k: bw[k] for k in names}, names=names,
                        label=label, ideal=bideal))
    assert_parity(spec, errs, label)


def _random_doc_partials(n=6, seed=4343):
    """The random partial problems above with the sequence cut into random
    block-aligned documents."""
    rng = np.random.default_rng(seed)
    out = []
    for label, kw, lo, hi, ck in _random_partials(n, seed):
        nb = kw["L"] // kw["B"]
        cuts = sorted(set(rng.choice(np.arange(1, nb), size=int(rng.integers(1, 5))).tolist()))
        kw = dict(kw, doc_starts=[0] + [c * kw["B"] for c in cuts])
        out.append((label.replace("rpart", "rpartdocs"), kw, lo, hi, ck))
    return out


RANDOM_DOC_PARTIALS = _random_doc_partials()


@pytest.mark.parametrize("label,kw,lo,hi,ck", RANDOM_DOC_PARTIALS,
                         ids=[r[0] for r in RANDOM_DOC_PARTIALS])
def test_random_partial_problems_with_documents(label, kw, lo, hi, ck):
    """A random partial launch over packed documents, forward and backward,
    checked as the one-document random partial launches are."""
    test_random_partial_problems(label, kw, lo, hi, ck)
