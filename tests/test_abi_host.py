"""Host-side tests of the C ABI (no GPU): the library loads and exports every
declared symbol, host validation returns the documented codes, and the
library's mask render and pair count agree with the independent oracle."""
import ctypes
import os
import re

import numpy as np
import pytest

import block_masked_attention_amd as bd
from oracle import (corrupted_copies, documents, key_positions, key_tokens, layout, query_positions,
                    query_tokens, visible)
from tests.test_oracle import read_golden
from workloads import CONFIGS, small_spec

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            src = open(os.path.join(ROOT, "include", h)).read()
            names |= set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(bdattn_\w+)\s*\(", src, re.M))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert {"bdattn_fwd", "bdattn_bwd", "bdattn_validate", "bdattn_workspace_size",
            "bdattn_mask_render", "bdattn_fwd_noalloc", "bdattn_lce_fwd", "bdattn_lce_bwd",
            "bdattn_lce_fwd_bwd", "bdattn_lce_workspace_size"} <= set(names)
    L = ctypes.CDLL(bd.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    assert bd.version() == 5


def test_status_strings():
    for code in range(0, -7, -1):
        assert bd.status_string(code) != "unknown status"
    assert bd.status_string(-99) == "unknown status"


def oracle_mask(p):
    ids = None
    if p.corr_block_ids:
        ids = [p.corr_block_ids[i] for i in range(p.n_corr_blocks)]
    docs = [p.doc_starts[i] for i in range(p.n_docs)] if p.n_docs else None
    lay = layout(p.B, p.H, p.Hkv, p.d, p.n_clean_q, p.clean_q_start, p.n_clean_kv,
                 p.clean_kv_start, p.n_corr_blocks, ids, clean_mask=p.clean_mask,
                 partial=bool(p.partial), corr_keys=not p.omit_corr_keys, doc_starts=docs)
    qs, qb = query_tokens(lay)
    ks, kb = key_tokens(lay)
    qp, kp = query_positions(lay), key_positions(lay)
    qc, kc = corrupted_copies(lay, lay.n_clean_q), corrupted_copies(lay, lay.n_clean_kv)
    qd, kd = documents(lay, qp), documents(lay, kp)
    return visible(qs[:, None], qb[:, None], ks[None, :], kb[None, :], qp[:, None],
                   kp[None, :], lay.clean_mask, lay.corr_keys, qc[:, None], kc[None, :],
                   qd[:, None], kd[None, :])


CASES = [
    dict(B=2, n_clean_q=8),
    dict(B=1, n_clean_q=7),
    dict(B=16, n_clean_q=256),
    dict(B=32, n_clean_q=1056),
    dict(B=7, n_clean_q=63),
    dict(B=128, n_clean_q=384),
    dict(B=4, n_clean_q=16, clean_q_start=32, n_clean_kv=64, corr_block_ids=[2, 5, 11, 15]),
    dict(B=32, n_clean_q=0, n_clean_kv=2048, corr_block_ids=[0, 9, 33, 63]),
    dict(B=8, n_clean_q=64, n_corr_blocks=0),
    # two corrupted copies of some blocks (complementary masking)
    dict(B=4, n_clean_q=32, corr_block_ids=[0, 0, 1, 3, 3, 5, 7, 7]),
    dict(B=32, n_clean_q=1024, corr_block_ids=[b for b in range(32) for _ in (0, 1)]),
]
# the same shapes with the token-causal clean mask
CASES_TC = [dict(c, clean_mask=bd.CLEAN_TOKEN_CAUSAL) for c in CASES]
# partial problems: clean K/V ranges at original positions, with or without
# the corrupted keys (the split form of the appendix's Implementation 1)
CASES_PARTIAL = [
    dict(B=4, n_clean_q=32, n_clean_kv=12, clean_kv_start=8, partial=True, omit_corr_keys=True),
    dict(B=4, n_clean_q=32, n_clean_kv=0, partial=True),
    dict(B=2, n_clean_q=8, clean_q_start=8, n_clean_kv=6, clean_kv_start=4,
         corr_block_ids=[1, 4, 6], partial=True),
    dict(B=16, n_clean_q=256, n_clean_kv=96, clean_kv_start=160, partial=True,
         omit_corr_keys=True, clean_mask=bd.CLEAN_TOKEN_CAUSAL),
    dict(B=32, n_clean_q=1056, n_clean_kv=384, clean_kv_start=320, partial=True),
]

# packed documents: block-aligned starts, documents of one block, documents
# not aligned to the kernels' tiles, shares, token-causal, partial ranges
CASES_DOCS = [
    dict(B=2, n_clean_q=12, corr_block_ids=[0, 1, 2, 3, 5], doc_starts=[0, 4, 6]),
    dict(B=32, n_clean_q=1024, doc_starts=[0, 96, 160, 192, 512, 544]),
    dict(B=32, n_clean_q=1024, doc_starts=[0, 96, 160, 192, 512, 544],
         clean_mask=bd.CLEAN_TOKEN_CAUSAL),
    dict(B=16, n_clean_q=256, clean_q_start=256, n_clean_kv=512,
         corr_block_ids=[3, 5, 5, 17, 18, 30], doc_starts=[0, 80, 288, 400]),
    dict(B=1, n_clean_q=200, doc_starts=[0, 1, 2, 70, 71, 199]),
    dict(B=64, n_clean_q=1024, doc_starts=list(range(0, 1024, 64))),
    dict(B=16, n_clean_q=512, n_clean_kv=160, clean_kv_start=192, partial=True,
         doc_starts=[0, 208, 320]),
    dict(B=16, n_clean_q=512, n_clean_kv=128, clean_kv_start=128, partial=True,
         omit_corr_keys=True, doc_starts=[0, 144, 400]),
]


@pytest.mark.parametrize("case", CASES + CASES_TC + CASES_PARTIAL + CASES_DOCS)
def test_mask_render_matches_oracle(case):
    p = bd.problem(H=2, Hkv=1, d=32, dtype="bf16", **case)
    assert bd.validate(p) == 0
    got = bd.mask_render(p)
    want = oracle_mask(p)
    assert got.shape == want.shape and np.array_equal(got, want)
    assert bd.visible_pairs(p) == int(want.sum())


@pytest.mark.parametrize("name", ["mask_L8_B2.txt", "mask_share_B2.txt",
                                  "mask_token_causal_L8_B2.txt",
                                  "mask_complementary_L8_B2.txt",
                                  "mask_docs_L12_B2.txt"])
def test_mask_render_matches_hand_drawn_fixture(name):
    prm, want = read_golden(name)
    p = bd.problem(prm["B"], 1, 1, 32, "f32", prm["n_clean_q"], prm["clean_q_start"],
                   prm["n_clean_kv"], corr_block_ids=prm["ids"],
                   clean_mask=prm.get("clean_mask", bd.CLEAN_BLOCK_CAUSAL),
                   doc_starts=prm.get("docs"))
    assert np.array_equal(bd.mask_render(p), want)


def test_visible_pairs_closed_forms_at_full_size():
    """Pairs per head: L(L+B) for a full sequence (each stream L(L+B)/2);
    the rank-15 share is the sum of B^2 (b+1) over its clean and corrupted
    blocks."""
    for spec in CONFIGS[:4]:
        p = bd.from_spec(spec)
        L, B = spec.n_clean_q, spec.B
        assert bd.visible_pairs(p) == L * (L + B)
    spec = CONFIGS[4]
    p = bd.from_spec(spec)
    B = spec.B
    want = sum(B * B * (b + 1) for b in range(spec.clean_q_start // B,
                                              (spec.clean_q_start + spec.n_clean_q) // B))
    want += sum(B * B * (b + 1) for b in spec.corr_block_ids)
    assert bd.visible_pairs(p) == want
    # token-causal: the clean stream is causal, L(L+1)/2 pairs; the corrupted
    # stream keeps its L(L+B)/2
    for spec in CONFIGS[:4]:
        p = bd.from_spec(spec.with_(clean_mask=bd.CLEAN_TOKEN_CAUSAL))
        L, B = spec.n_clean_q, spec.B
        assert bd.visible_pairs(p) == L * (L + 1) // 2 + L * (L + B) // 2


def _p(**kw):
    base = dict(B=4, H=4, Hkv=2, d=32, dtype="bf16", n_clean_q=16)
    base.update(kw)
    return bd.problem(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(H=3, Hkv=2), -2),
    (dict(B=0), -2),
    (dict(d=64), -3),
    (dict(dtype=bd.F32, d=128), -3),
    (dict(n_clean_q=18), -2),
    (dict(clean_q_start=2, n_clean_kv=20), -2),
    (dict(n_clean_kv=12), -4),
    (dict(clean_q_start=16, n_clean_kv=16), -4),
    (dict(clean_kv_start=4, n_clean_kv=32), -4),
    (dict(corr_block_ids=[3, 2]), -1),
    (dict(corr_block_ids=[2, 1]), -1),
    (dict(corr_block_ids=[-1, 2]), -1),
    (dict(corr_block_ids=[0, 9]), -4),  # block 9 needs clean keys < 36
    (dict(n_clean_q=-4), -2),
    (dict(clean_mask=2), -1),
    (dict(clean_mask=-1), -1),
    (dict(omit_corr_keys=True), -1),  # only a partial problem may omit them
    (dict(partial=True, clean_kv_start=2, n_clean_kv=8), -2),
    (dict(doc_starts=[4, 8]), -1),
    (dict(doc_starts=[0, 8, 8]), -1),
    (dict(doc_starts=[0, 12, 8]), -1),
    (dict(doc_starts=[0, 6]), -2),
])
def test_validation_error_codes(kw, code):
    p = _p(**kw)
    assert bd.validate(p) == code
    assert bd.lib().bdattn_last_error().decode() != ""


def test_unknown_dtype_and_null_problem():
    p = _p()
    p.dtype = 7
    assert bd.validate(p) == -1
    p = _p()
    p.n_docs = -1
    assert bd.validate(p) == -1
    p = _p()
    p.n_docs = 2  # no array
    assert bd.validate(p) == -1
    assert bd.lib().bdattn_validate(None) == -1


def test_workspace_size_and_launch_errors_without_gpu_work():
    """Errors found on the host come back before anything is enqueued, so
    they are testable without a GPU: bad pass, missing workspace, NULL or
    misaligned tensor pointers."""
    p = _p()
    L = bd.lib()
    n = ctypes.c_size_t(0)
    assert L.bdattn_workspace_size(ctypes.byref(p), 2, ctypes.byref(n)) == -1
    assert L.bdattn_workspace_size(ctypes.byref(p), 0, None) == -1
    assert bd.workspace_size(p, 0) > 0 and bd.workspace_size(p, 1) > bd.workspace_size(p, 0)
    vp = ctypes.c_void_p
    good = vp(1 << 20)  # never dereferenced: every call below fails validation first
    bad = vp((1 << 20) + 8)
    args = [good] * 6 + [good, good, good, good]
    # NULL q_c
    assert L.bdattn_fwd(ctypes.byref(p), None, *args[1:], good, 1 << 30, None) == -1
    # misaligned v_x
    a2 = list(args)
    a2[5] = bad
    assert L.bdattn_fwd(ctypes.byref(p), *a2, good, 1 << 30, None) == -1
    # workspace too small / missing / misaligned
    assert L.bdattn_fwd(ctypes.byref(p), *args, good, 16, None) == -5
    assert L.bdattn_fwd(ctypes.byref(p), *args, None, 1 << 30, None) == -5
    assert L.bdattn_fwd(ctypes.byref(p), *args, vp((1 << 20) + 16), 1 << 30, None) == -5
    bargs = [good] * 6 + [good] * 6 + [good] * 6
    assert L.bdattn_bwd(ctypes.byref(p), *bargs, good, 16, None) == -5
    bargs[13] = None  # dq_x
    assert L.bdattn_bwd(ctypes.byref(p), *bargs, good, 1 << 40, None) == -1


def test_plan_covers_every_visible_tile():
    """The forward work list visits, for every query row tile, exactly the key
    tiles holding a visible key; the backward list has one item per key tile
    and KV head (so every dK/dV row is written)."""
    for case in CASES + CASES_TC + CASES_PARTIAL + CASES_DOCS:
        p = bd.problem(H=4, Hkv=2, d=32, dtype="bf16", **case)
        st = bd.plan_stats(p)
        M = bd.mask_render(p)
        nc, nkv, nx = int(p.n_clean_q), int(p.n_clean_kv), p.n_corr
        R = st["fwd_rows_per_item"]
        G = int(p.H) // int(p.Hkv)  # q heads per KV head; a work item takes 4, 2 or 1 of them
        Gw = 4 if G % 4 == 0 else (2 if G % 2 == 0 else 1)
        want_items, want_tiles = 0, 0
        for s, (r0, n) in enumerate(((0, nc), (nc, nx))):
            for t in range(0, n, R):
                rows = M[r0 + t:r0 + min(n, t + R)]
                vis = rows.any(0)
                cl = np.flatnonzero(vis[:nkv])
                ntiles = 0
                if len(cl):  # clean keys swept from 0 (documents: from the first one visible)
                    ntiles += (cl.max() // 64) + 1 - (cl.min() // 64 if p.n_docs else 0)
                xk = np.flatnonzero(vis[nkv:])
                if len(xk):
                    ntiles += (xk.max() - xk.min()) // 64 + 1
                want_items += 1
                want_tiles += ntiles
        heads_groups = int(p.H) // Gw
        assert st["fwd_items"] == want_items * heads_groups
        if p.n_docs:  # an item may start its sweep at an earlier document's first key
            assert want_tiles * heads_groups <= st["fwd_tiles"] <= (want_tiles + want_items) * heads_groups
        else:
            assert st["fwd_tiles"] == want_tiles * heads_groups
        kt = -(-nkv // 128) + (0 if p.omit_corr_keys else -(-nx // 128))
        assert st["bwd_items"] == kt * int(p.Hkv)


def test_plan_cache_stays_bounded_under_new_document_layouts():
    """A training loop with packed documents presents a new document layout
    every step. 1000 distinct layouts of a 64K problem (each plan several
    hundred KB) keep the cache within its budget, and a layout planned again
    after its eviction gets the same plan."""
    before = bd.plan_cache_info()
    bd.plan_cache_budget(8 << 20)
    try:
        rng = np.random.default_rng(7)
        L, B = 65536, 32
        first = None
        for i in range(1000):
            cuts = np.sort(rng.choice(np.arange(1, L // B), 15, replace=False)) * B
            p = bd.problem(B, 32, 8, 128, "bf16", L, doc_starts=[0] + cuts.tolist())
            st = bd.plan_stats(p)
            if first is None:
                first = (cuts, st)
            info = bd.plan_cache_info()
            assert info["host_bytes"] + info["pinned_bytes"] <= (8 << 20) + (2 << 20), info
        assert info["evictions"] >= before["evictions"] + 900
        assert info["plans"] < 100
        again = bd.plan_stats(bd.problem(B, 32, 8, 128, "bf16", L,
                                         doc_starts=[0] + first[0].tolist()))
        assert again == first[1]
    finally:
        bd.plan_cache_budget(before["budget"])


def test_plan_cache_budget_is_validated():
    with pytest.raises(bd.BdattnError):
        bd.plan_cache_budget(1000)


# a gathered clean K/V buffer: chunks of 128+ keys in any order (zigzag
# all-gather order of P ranks: rank r brings position chunks r and 2P-1-r)
def _zigzag(P, C, lo=0):
    return [lo + c * C for r in range(P) for c in (r, 2 * P - 1 - r)]


CASES_GATHERED = [
    dict(B=32, n_clean_q=1024, kv_chunk_len=128, kv_chunk_pos=_zigzag(4, 128)),
    dict(B=16, n_clean_q=512, clean_q_start=512, n_clean_kv=1024, corr_block_ids=[3, 9, 40, 63],
         kv_chunk_len=256, kv_chunk_pos=[768, 0, 512, 256]),
    dict(B=32, n_clean_q=1024, kv_chunk_len=128, kv_chunk_pos=_zigzag(4, 128),
         clean_mask=bd.CLEAN_TOKEN_CAUSAL, doc_starts=[0, 96, 320, 704]),
    dict(B=32, n_clean_q=1024, n_clean_kv=512, clean_kv_start=256, partial=True,
         kv_chunk_len=128, kv_chunk_pos=[640, 256, 512, 384]),
]


@pytest.mark.parametrize("case", CASES_GATHERED)
def test_gathered_buffer_mask_and_plan(case):
    """The library's mask of a gathered buffer equals the oracle's mask with
    each buffer row at its original position, and its plan does the same work
    as the position-ordered buffer."""
    p = bd.problem(H=4, Hkv=2, d=128, dtype="bf16", **case)
    assert bd.validate(p) == 0, bd.lib().bdattn_last_error()
    ids = [p.corr_block_ids[i] for i in range(p.n_corr_blocks)] if p.corr_block_ids else None
    docs = [p.doc_starts[i] for i in range(p.n_docs)] if p.n_docs else None
    C = case["kv_chunk_len"]
    pos = [s + r for s in case["kv_chunk_pos"] for r in range(C)]
    lay = layout(p.B, p.H, p.Hkv, p.d, p.n_clean_q, p.clean_q_start, p.n_clean_kv,
                 p.clean_kv_start, p.n_corr_blocks, ids, clean_mask=p.clean_mask,
                 partial=bool(p.partial), corr_keys=not p.omit_corr_keys, doc_starts=docs,
                 clean_kv_positions=pos)
    qs, qb = query_tokens(lay)
    ks, kb = key_tokens(lay)
    qp, kp = query_positions(lay), key_positions(lay)
    qc, kc = corrupted_copies(lay, lay.n_clean_q), corrupted_copies(lay, lay.n_clean_kv)
    qd, kd = documents(lay, qp), documents(lay, kp)
    want = visible(qs[:, None], qb[:, None], ks[None, :], kb[None, :], qp[:, None], kp[None, :],
                   lay.clean_mask, lay.corr_keys, qc[:, None], kc[None, :], qd[:, None], kd[None, :])
    assert np.array_equal(bd.mask_render(p), want)
    plain = dict(case)
    plain.pop("kv_chunk_pos")
    plain["kv_chunk_len"] = 0
    q = bd.problem(H=4, Hkv=2, d=128, dtype="bf16", **plain)
    assert bd.plan_stats(p) == bd.plan_stats(q)
    assert bd.visible_pairs(p) == bd.visible_pairs(q)
    assert bd.workspace_size(p, 1) > bd.workspace_size(q, 1)  # the tile map travels along


@pytest.mark.parametrize("kw,code", [
    (dict(kv_chunk_len=64, kv_chunk_pos=list(range(0, 1024, 64))), -2),  # not a multiple of 128
    (dict(kv_chunk_len=384, kv_chunk_pos=[0, 384]), -2),                 # does not divide 1024
    (dict(kv_chunk_len=128), -1),                                        # no positions
    (dict(kv_chunk_len=128, kv_chunk_pos=[0, 128, 256, 384, 512, 640, 768, 768]), -1),
    (dict(kv_chunk_len=128, kv_chunk_pos=[0, 128, 256, 384, 512, 640, 768, 960]), -1),
    (dict(kv_chunk_len=128, kv_chunk_pos=[128, 256, 384, 512, 640, 768, 896, 1024]), -1),
    (dict(kv_chunk_len=-128), -2),
])
def test_gathered_buffer_validation(kw, code):
    p = bd.problem(B=32, H=4, Hkv=2, d=128, dtype="bf16", n_clean_q=1024, **kw)
    assert bd.validate(p) == code


def test_lce_host_validation_and_workspace():
    """The linear cross-entropy's descriptor checks and workspace sizes, on
    the host (nothing is enqueued for an invalid call)."""
    ok = bd.lce_problem(1000, 256, 5000, chunk=256)
    assert bd.lce_workspace_size(ok, 0) == 256 * 5000 * 4
    assert bd.lce_workspace_size(ok, 1) == 256 * 5000 * 4 + 256 * 5000 * 2
    small = bd.lce_problem(10, 256, 5000, chunk=256)  # the chunk is at most the tokens
    assert bd.lce_workspace_size(small, 0) == (10 * 5000 * 4 + 255) // 256 * 256
    n = ctypes.c_size_t(0)
    for bad in (bd.lce_problem(10, 12, 5000), bd.lce_problem(10, 256, 5001),
                bd.lce_problem(10, 256, 5000, chunk=0), bd.lce_problem(1 << 20, 256, 1 << 20, chunk=4096)):
        assert bd.lib().bdattn_lce_workspace_size(ctypes.byref(bad), 0, ctypes.byref(n)) == -2
    L = bd.lib()
    vp = ctypes.c_void_p
    good = vp(1 << 20)
    # missing workspace, NULL targets, misaligned h: refused before any GPU work
    assert L.bdattn_lce_fwd(ctypes.byref(ok), good, good, good, good, good, None, 0, None) == -5
    assert L.bdattn_lce_fwd(ctypes.byref(ok), good, good, None, good, good, good, 1 << 30, None) == -1
    assert L.bdattn_lce_fwd(ctypes.byref(ok), vp((1 << 20) + 8), good, good, good, good, good,
                            1 << 30, None) == -1


def test_precision_is_validated():
    """bdattn_problem.precision is a bdattn_precision (0 default, 1 float32
    outputs, 2 float32 outputs with split operands); anything else is refused
    on the host."""
    spec = small_spec(L=64, B=16, H=2, Hkv=2, d=32, dtype="bf16")
    for v, ok in ((0, True), (1, True), (2, True), (3, False), (-1, False)):
        p = bd.from_spec(spec)
        p.precision = v
        if ok:
            assert bd.workspace_size(p, 0) > 0
        else:
            with pytest.raises(bd.BdattnError):
                bd.workspace_size(p, 0)
