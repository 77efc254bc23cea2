"""Pins of the CPU oracle against things other than itself.

Each test names what fixes the expected value: a hand-drawn mask, a closed
form, a library attention routine, scalar brute force, numerical derivatives,
or an invariant the method states ("Block Parallelism for Efficient
Distributed Long-Context Diffusion Language Model Training", §3.2 separability,
§4.3 clean-gradient accumulation, §4.4 Proposition 1 exactness).
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import (BLOCK_CAUSAL, CLEAN, CORRUPTED, TOKEN_CAUSAL, Oracle, corrupted_copies,
                    documents, key_positions, key_tokens, layout, merge_partials, query_positions,
                    query_tokens, visible)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def make(lay, seed=0, scale=1.0):
    n_c, n_kv, n_x = lay.n_clean_q, lay.n_clean_kv, lay.n_corr
    H, Hkv, d = lay.H, lay.Hkv, lay.d
    return dict(
        q_c=rnd((n_c, H, d), seed + 1, scale), k_c=rnd((n_kv, Hkv, d), seed + 2, scale),
        v_c=rnd((n_kv, Hkv, d), seed + 3, scale), q_x=rnd((n_x, H, d), seed + 4, scale),
        k_x=rnd((n_x, Hkv, d), seed + 5, scale), v_x=rnd((n_x, Hkv, d), seed + 6, scale),
        do_c=rnd((n_c, H, d), seed + 7), do_x=rnd((n_x, H, d), seed + 8))


def oracle_of(lay, t):
    return Oracle(lay, t["q_c"], t["k_c"], t["v_c"], t["q_x"], t["k_x"], t["v_x"],
                  t.get("do_c"), t.get("do_x"))


def full_mask(lay):
    qs, qb = query_tokens(lay)
    ks, kb = key_tokens(lay)
    qp, kp = query_positions(lay), key_positions(lay)
    qc, kc = corrupted_copies(lay, lay.n_clean_q), corrupted_copies(lay, lay.n_clean_kv)
    qd, kd = documents(lay, qp), documents(lay, kp)
    return visible(qs[:, None], qb[:, None], ks[None, :], kb[None, :], qp[:, None],
                   kp[None, :], lay.clean_mask, lay.corr_keys, qc[:, None], kc[None, :],
                   qd[:, None], kd[None, :])


# --------------------------------------------------------------------- mask
def read_golden(name):
    rows, params = [], {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("params"):
                for kv in line.split()[1:]:
                    k, v = kv.split("=")
                    params[k] = ([int(x) for x in v.split(",")] if k in ("ids", "docs")
                                 else int(v))
                continue
            bits = line.split()[1].replace("|", "")
            rows.append([c == "1" for c in bits])
    return params, np.array(rows, dtype=bool)


@pytest.mark.parametrize("name", ["mask_L8_B2.txt", "mask_share_B2.txt",
                                  "mask_token_causal_L8_B2.txt",
                                  "mask_complementary_L8_B2.txt",
                                  "mask_docs_L12_B2.txt"])
def test_mask_matches_hand_drawn_fixture(name):
    p, want = read_golden(name)
    lay = layout(p["B"], 1, 1, 4, p["n_clean_q"], p["clean_q_start"], p["n_clean_kv"],
                 corr_block_ids=p["ids"], clean_mask=p.get("clean_mask", BLOCK_CAUSAL),
                 doc_starts=p.get("docs"))
    got = full_mask(lay)
    assert got.shape == want.shape
    assert np.array_equal(got, want)


@pytest.mark.parametrize("L,B", [(4, 1), (8, 2), (12, 3), (16, 4), (32, 8), (24, 24)])
def test_visible_counts_closed_form(L, B):
    """Both streams see (qb+1)*B keys: clean sees blocks 0..qb; corrupted sees
    blocks 0..qb-1 clean plus its own corrupted block (§3.2)."""
    lay = layout(B, 1, 1, 4, L)
    M = full_mask(lay)
    qs, qb = query_tokens(lay)
    assert np.array_equal(M.sum(1), (qb + 1) * B)
    # clean queries never see corrupted keys; each corrupted query sees
    # exactly its own block's B corrupted keys
    assert not M[:L, L:].any()
    assert np.array_equal(M[L:, L:].sum(1), np.full(L, B))


@pytest.mark.parametrize("L,B", [(4, 1), (8, 2), (12, 3), (16, 4), (32, 8), (24, 24)])
def test_visible_counts_closed_form_token_causal(L, B):
    """Token-causal: the clean query at position p sees exactly the p + 1 clean
    keys at positions 0..p; corrupted queries still see (qb+1)*B keys."""
    lay = layout(B, 1, 1, 4, L, clean_mask=TOKEN_CAUSAL)
    M = full_mask(lay)
    _, qb = query_tokens(lay)
    assert np.array_equal(M[:L, :L], np.tril(np.ones((L, L), dtype=bool)))
    assert not M[:L, L:].any()
    assert np.array_equal(M[L:].sum(1), (qb[L:] + 1) * B)


# ------------------------------------------------------------- closed forms
def _prefix_sets(lay):
    """Visible key index sets written as ranges (clean prefix length, own
    corrupted block), a formulation independent of the pairwise rules."""
    out = []
    nkc = lay.n_clean_kv
    for i in range(lay.n_clean_q):
        pos = lay.clean_q_start + i
        if lay.clean_mask == TOKEN_CAUSAL:
            out.append(list(range(0, pos + 1)))
            continue
        b = pos // lay.B
        out.append(list(range(0, (b + 1) * lay.B)))
    for j, bid in enumerate(lay.corr_ids):
        own = list(range(nkc + j * lay.B, nkc + (j + 1) * lay.B))
        for _ in range(lay.B):
            out.append(list(range(0, bid * lay.B)) + own)
    return out


@pytest.mark.parametrize("case", [
    dict(B=4, n_clean_q=32), dict(B=1, n_clean_q=9), dict(B=8, n_clean_q=24),
    dict(B=2, n_clean_q=6, clean_q_start=10, n_clean_kv=16, corr_block_ids=[0, 3, 7]),
    dict(B=4, n_clean_q=32, clean_mask=TOKEN_CAUSAL),
    dict(B=3, n_clean_q=9, clean_q_start=6, n_clean_kv=18, corr_block_ids=[1, 2, 5],
         clean_mask=TOKEN_CAUSAL),
])
def test_q_zero_uniform_weights(case):
    """Q = 0 makes every visible score 0: O_i is the mean of v over V(i) and
    LSE_i = ln |V(i)|; dV_j = sum over rows i seeing j of dO_i / |V(i)|."""
    lay = layout(H=4, Hkv=2, d=3, **case)
    t = make(lay, seed=3)
    t["q_c"][:] = 0
    t["q_x"][:] = 0
    orc = oracle_of(lay, t)
    O_c, O_x, L_c, L_x = orc.forward()
    O = np.concatenate([O_c, O_x])
    LSE = np.concatenate([L_c, L_x], axis=1)
    V = np.concatenate([t["v_c"], t["v_x"]])
    dO = np.concatenate([t["do_c"], t["do_x"]])
    sets = _prefix_sets(lay)
    dV_want = np.zeros_like(V)
    for i, s in enumerate(sets):
        for h in range(lay.H):
            g = h // lay.G
            np.testing.assert_allclose(O[i, h], V[s, g].mean(0), rtol=0, atol=1e-13)
            assert abs(LSE[h, i] - math.log(len(s))) < 1e-13
            dV_want[s, g] += dO[i, h] / len(s)
    _, _, _, dV_c, _, dV_x = orc.backward()
    np.testing.assert_allclose(np.concatenate([dV_c, dV_x]), dV_want, rtol=0, atol=1e-12)


# --------------------------------------------------------------- brute force
def test_scalar_brute_force_forward():
    """Per-query scalar loop, math.fsum softmax, over the range formulation."""
    for B, L, d in [(1, 6, 3), (2, 8, 5), (4, 12, 8)]:
        lay = layout(B, 2, 1, d, L)
        t = make(lay, seed=11)
        orc = oracle_of(lay, t)
        O_c, O_x, L_c, L_x = orc.forward()
        O = np.concatenate([O_c, O_x])
        LSE = np.concatenate([L_c, L_x], axis=1)
        Q = np.concatenate([t["q_c"], t["q_x"]])
        K = np.concatenate([t["k_c"], t["k_x"]])
        V = np.concatenate([t["v_c"], t["v_x"]])
        for i, s in enumerate(_prefix_sets(lay)):
            for h in range(lay.H):
                sc = [math.fsum(Q[i, h, e] * K[j, 0, e] for e in range(d)) / math.sqrt(d)
                      for j in s]
                m = max(sc)
                w = [math.exp(x - m) for x in sc]
                z = math.fsum(w)
                assert abs(LSE[h, i] - (m + math.log(z))) < 1e-12
                for e in range(d):
                    o = math.fsum(w[k] * V[j, 0, e] for k, j in enumerate(s)) / z
                    assert abs(O[i, h, e] - o) < 1e-12


# ------------------------------------------------------- library attention
def _sdpa_reference(lay, t, mask):
    """torch's scaled_dot_product_attention (float64, CPU) with an explicit
    boolean mask, K/V repeated over each group, and autograd gradients."""
    nc, nkc = lay.n_clean_q, lay.n_clean_kv
    T = lambda a: torch.tensor(a, dtype=torch.float64)
    Q = T(np.concatenate([t["q_c"], t["q_x"]])).requires_grad_()
    K = T(np.concatenate([t["k_c"], t["k_x"]])).requires_grad_()
    V = T(np.concatenate([t["v_c"], t["v_x"]])).requires_grad_()
    dO = T(np.concatenate([t["do_c"], t["do_x"]]))
    Kh = K.repeat_interleave(lay.G, dim=1)
    Vh = V.repeat_interleave(lay.G, dim=1)
    O = torch.nn.functional.scaled_dot_product_attention(
        Q.transpose(0, 1)[None], Kh.transpose(0, 1)[None], Vh.transpose(0, 1)[None],
        attn_mask=torch.tensor(mask), scale=lay.scale)[0].transpose(0, 1)
    (O * dO).sum().backward()
    S = lay.scale * torch.einsum("qhd,khd->hqk", Q.detach(), Kh.detach())
    S = S.masked_fill(~torch.tensor(mask)[None], -math.inf)
    LSE = torch.logsumexp(S, dim=-1)
    n = lambda x: x.detach().numpy()
    return (n(O[:nc]), n(O[nc:]), n(LSE[:, :nc]), n(LSE[:, nc:]),
            n(Q.grad[:nc]), n(Q.grad[nc:]), n(K.grad[:nkc]), n(V.grad[:nkc]),
            n(K.grad[nkc:]), n(V.grad[nkc:]))


@pytest.mark.parametrize("case", [
    dict(B=4, H=4, Hkv=2, d=8, n_clean_q=32),
    dict(B=3, H=3, Hkv=1, d=5, n_clean_q=21),
    dict(B=2, H=2, Hkv=2, d=4, n_clean_q=8, clean_q_start=8, n_clean_kv=16,
         corr_block_ids=[1, 4, 6]),
])
def test_matches_library_attention(case):
    lay = layout(**case)
    t = make(lay, seed=5)
    orc = oracle_of(lay, t)
    got = orc.forward() + orc.backward()
    want = _sdpa_reference(lay, t, full_mask(lay))
    for a, b in zip(got, want):
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-11)


def test_block_size_one_is_causal_attention():
    """B = 1: the clean stream is causal attention; corrupted row i is row i
    of causal attention over the clean keys with key/value i replaced by the
    corrupted token's own."""
    L, H, d = 12, 2, 6
    lay = layout(1, H, H, d, L)
    t = make(lay, seed=9)
    O_c, O_x, L_c, L_x = oracle_of(lay, t).forward()
    T = lambda a: torch.tensor(a, dtype=torch.float64).transpose(0, 1)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        T(t["q_c"]), T(t["k_c"]), T(t["v_c"]), is_causal=True)[0].transpose(0, 1)
    np.testing.assert_allclose(O_c, ref.numpy(), rtol=1e-12, atol=1e-13)
    for i in range(L):
        k2 = t["k_c"].copy()
        v2 = t["v_c"].copy()
        k2[i] = t["k_x"][i]
        v2[i] = t["v_x"][i]
        q = t["q_c"].copy()
        q[i] = t["q_x"][i]
        r = torch.nn.functional.scaled_dot_product_attention(
            T(q), T(k2), T(v2), is_causal=True)[0].transpose(0, 1)
        np.testing.assert_allclose(O_x[i], r[i].numpy(), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("B", [1, 3, 4, 16])
def test_token_causal_clean_stream_is_causal_attention(B):
    """Token-causal: a clean query sees exactly the clean keys at positions up
    to its own, so the clean stream is plain causal attention at any block
    size. O_c, LSE_c and dQ_c equal torch's causal scaled_dot_product_attention
    (float64, CPU, K/V repeated over each group) and its autograd gradient."""
    L, H, Hkv, d = 48, 4, 2, 6
    lay = layout(B, H, Hkv, d, L, clean_mask=TOKEN_CAUSAL)
    t = make(lay, seed=17)
    orc = oracle_of(lay, t)
    O_c, _, L_c, _ = orc.forward()
    dq_c = orc.backward()[0]
    T = lambda a: torch.tensor(a, dtype=torch.float64)
    q = T(t["q_c"]).transpose(0, 1)[None].requires_grad_()
    k = T(t["k_c"]).repeat_interleave(H // Hkv, dim=1).transpose(0, 1)[None]
    v = T(t["v_c"]).repeat_interleave(H // Hkv, dim=1).transpose(0, 1)[None]
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
    (o * T(t["do_c"]).transpose(0, 1)[None]).sum().backward()
    np.testing.assert_allclose(O_c, o[0].transpose(0, 1).detach().numpy(), rtol=1e-12,
                               atol=1e-13)
    np.testing.assert_allclose(dq_c, q.grad[0].transpose(0, 1).numpy(), rtol=1e-10,
                               atol=1e-12)
    s = (q[0] @ k[0].transpose(-1, -2)).detach() / math.sqrt(d)
    s = s.masked_fill(~torch.ones(L, L, dtype=torch.bool).tril(), -math.inf)
    np.testing.assert_allclose(L_c, torch.logsumexp(s, dim=-1).numpy(), rtol=1e-12,
                               atol=1e-12)


def test_token_causal_equals_block_causal_at_block_size_one():
    """With one-token blocks the two readings of §3.2 coincide."""
    lay0 = layout(1, 2, 1, 4, 10)
    lay1 = layout(1, 2, 1, 4, 10, clean_mask=TOKEN_CAUSAL)
    t = make(lay0, seed=6)
    a = oracle_of(lay0, t)
    b = oracle_of(lay1, t)
    for x, y in zip(a.forward() + a.backward(), b.forward() + b.backward()):
        assert np.array_equal(x, y)


# ------------------------------------------------------ numerical gradients
@pytest.mark.parametrize("clean_mask", [BLOCK_CAUSAL, TOKEN_CAUSAL])
def test_finite_difference_gradients(clean_mask):
    lay = layout(4, 2, 1, 4, 16, clean_mask=clean_mask)
    t = make(lay, seed=21)
    orc = oracle_of(lay, t)
    grads = dict(zip(["q_c", "q_x", "k_c", "v_c", "k_x", "v_x"], orc.backward()))
    dO = np.concatenate([t["do_c"], t["do_x"]])

    def f(tt):
        o = oracle_of(lay, tt).forward()
        return float(np.sum(np.concatenate([o[0], o[1]]) * dO))

    h = 1e-6
    for name in ["q_c", "q_x", "k_c", "v_c", "k_x", "v_x"]:
        num = np.zeros_like(t[name])
        for idx in np.ndindex(t[name].shape):
            tp = {k: v.copy() for k, v in t.items()}
            tm = {k: v.copy() for k, v in t.items()}
            tp[name][idx] += h
            tm[name][idx] -= h
            num[idx] = (f(tp) - f(tm)) / (2 * h)
        err = np.max(np.abs(num - grads[name])) / np.max(np.abs(num))
        assert err < 1e-6, (name, err)


# ------------------------------------------------------------- invariants
def test_identical_streams_give_identical_outputs():
    """With the corrupted copy equal to the clean copy, corrupted block b sees
    {own block} + clean blocks < b, which is the clean query's set: outputs
    and query gradients match (block-causal reading of §3.2)."""
    lay = layout(4, 4, 2, 8, 32)
    t = make(lay, seed=4)
    for a, b in [("q_x", "q_c"), ("k_x", "k_c"), ("v_x", "v_c"), ("do_x", "do_c")]:
        t[a] = t[b].copy()
    orc = oracle_of(lay, t)
    O_c, O_x, L_c, L_x = orc.forward()
    dq_c, dq_x, *_ = orc.backward()
    np.testing.assert_allclose(O_x, O_c, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(L_x, L_c, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dq_x, dq_c, rtol=1e-11, atol=1e-12)


def test_corrupted_block_separability():
    """§3.2 / §4.2: corrupted activations of block b' affect only block b'.
    Perturbing block b' leaves every other corrupted block's outputs and
    gradients and all clean outputs and dQ bitwise unchanged; clean dK/dV
    change by exactly block b''s contribution."""
    lay = layout(4, 4, 2, 8, 32)
    B, nb = 4, 8
    t = make(lay, seed=8)
    base = oracle_of(lay, t)
    f0, g0 = base.forward(), base.backward()
    bp = 5
    rows = slice(bp * B, (bp + 1) * B)
    t2 = {k: v.copy() for k, v in t.items()}
    for name in ["q_x", "k_x", "v_x"]:
        t2[name][rows] += rnd(t2[name][rows].shape, 99)
    pert = oracle_of(lay, t2)
    f1, g1 = pert.forward(), pert.backward()
    other = np.ones(32, bool)
    other[rows] = False
    assert np.array_equal(f1[0], f0[0]) and np.array_equal(f1[2], f0[2])  # clean O, LSE
    assert np.array_equal(f1[1][other], f0[1][other])
    assert np.array_equal(f1[3][:, other], f0[3][:, other])
    assert np.array_equal(g1[0], g0[0])  # dQ_c
    for k in (1, 4, 5):  # dQ_x, dK_x, dV_x
        assert np.array_equal(g1[k][other], g0[k][other])
    # clean dK/dV change by block b''s own contribution
    qrow = pert.query_index(CORRUPTED, np.arange(bp * B, (bp + 1) * B))
    _, dk1, dv1 = pert.rows_backward(qrow)
    qrow0 = base.query_index(CORRUPTED, np.arange(bp * B, (bp + 1) * B))
    _, dk0, dv0 = base.rows_backward(qrow0)
    np.testing.assert_allclose(g1[2] - g0[2], dk1[:32] - dk0[:32], rtol=0, atol=1e-12)
    np.testing.assert_allclose(g1[3] - g0[3], dv1[:32] - dv0[:32], rtol=0, atol=1e-12)


def test_clean_gradients_are_sums_of_per_block_contributions():
    """§4.1 / §4.3: clean dK/dV accumulate the contributions of every query
    block that sees them. Zeroing dO outside one query block yields that
    block's contribution; the sum over all clean and corrupted blocks equals
    the full gradient."""
    lay = layout(4, 4, 2, 8, 32)
    B, nb = 4, 8
    t = make(lay, seed=12)
    full = oracle_of(lay, t).backward()
    acc_k = np.zeros_like(full[2])
    acc_v = np.zeros_like(full[3])
    for stream in ("c", "x"):
        for b in range(nb):
            tt = {k: v.copy() for k, v in t.items()}
            keep = np.zeros(32, bool)
            keep[b * B:(b + 1) * B] = True
            tt["do_c"][:] = 0
            tt["do_x"][:] = 0
            tt["do_" + stream][keep] = t["do_" + stream][keep]
            g = oracle_of(lay, tt).backward()
            acc_k += g[2]
            acc_v += g[3]
    np.testing.assert_allclose(acc_k, full[2], rtol=0, atol=1e-12)
    np.testing.assert_allclose(acc_v, full[3], rtol=0, atol=1e-12)


@pytest.mark.parametrize("assign", ["dual_end", "strided"])
def test_simulated_context_sharded_ranks_equal_full(assign):
    """§4.3-§4.4 (Proposition 1): P ranks, each with one clean-query shard,
    the clean K/V before its shard end, and a subset of corrupted blocks;
    summing the clean dK/dV over ranks and concatenating the rest reproduces
    the single full computation."""
    L, B, P = 32, 2, 4  # 16 blocks, 4 per rank
    nb = L // B
    lay = layout(B, 4, 2, 4, L)
    t = make(lay, seed=31)
    full_f = oracle_of(lay, t).forward()
    full_g = oracle_of(lay, t).backward()
    if assign == "dual_end":
        owner = {}
        for r in range(P):
            for k in range(nb // (2 * P)):
                i = r + k * P
                owner[i] = r
                owner[nb - 1 - i] = r
    else:
        owner = {b: b % P for b in range(nb)}
    shard = L // P
    O_c = np.zeros_like(full_f[0])
    O_x = np.zeros_like(full_f[1])
    dk_c = np.zeros_like(full_g[2])
    dv_c = np.zeros_like(full_g[3])
    dq_x = np.zeros_like(full_g[1])
    dk_x = np.zeros_like(full_g[4])
    for r in range(P):
        ids = sorted(b for b, o in owner.items() if o == r)
        lo, hi = r * shard, (r + 1) * shard
        # the clean K/V buffer is every clean position before the last one
        # a local query sees (as after the forward all-gather)
        kv_end = max(hi, max(ids) * B)
        rl = layout(B, 4, 2, 4, shard, lo, kv_end, corr_block_ids=ids)
        xr = np.concatenate([np.arange(b * B, (b + 1) * B) for b in ids])
        tr = dict(q_c=t["q_c"][lo:hi], k_c=t["k_c"][:kv_end], v_c=t["v_c"][:kv_end],
                  q_x=t["q_x"][xr], k_x=t["k_x"][xr], v_x=t["v_x"][xr],
                  do_c=t["do_c"][lo:hi], do_x=t["do_x"][xr])
        orc = oracle_of(rl, tr)
        f = orc.forward()
        g = orc.backward()
        O_c[lo:hi] = f[0]
        O_x[xr] = f[1]
        dk_c[:kv_end] += g[2]
        dv_c[:kv_end] += g[3]
        dq_x[xr] = g[1]
        dk_x[xr] = g[4]
    np.testing.assert_allclose(O_c, full_f[0], rtol=0, atol=1e-13)
    np.testing.assert_allclose(O_x, full_f[1], rtol=0, atol=1e-13)
    np.testing.assert_allclose(dk_c, full_g[2], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv_c, full_g[3], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dq_x, full_g[1], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk_x, full_g[4], rtol=0, atol=1e-12)


def test_sampled_rows_and_keys_match_full():
    """The row-sampled forward/dQ and key-sampled dK/dV used at large sizes
    agree with the full computation."""
    lay = layout(4, 4, 2, 8, 48, 16, 64, corr_block_ids=[1, 5, 9, 14])
    t = make(lay, seed=17)
    orc = oracle_of(lay, t)
    f, g = orc.forward(), orc.backward()
    rows = np.array([0, 7, 30, 47])
    O, LSE = orc.rows_forward(orc.query_index(CLEAN, rows))
    np.testing.assert_allclose(O, f[0][rows], rtol=0, atol=1e-14)
    np.testing.assert_allclose(LSE, f[2][:, rows], rtol=0, atol=1e-14)
    xr = np.array([1, 5, 15])
    dq, _, _ = orc.rows_backward(orc.query_index(CORRUPTED, xr))
    np.testing.assert_allclose(dq, g[1][xr], rtol=0, atol=1e-13)
    keys = np.array([0, 3, 33, 63])
    dk, dv = orc.keys_backward(orc.key_index(CLEAN, keys))
    np.testing.assert_allclose(dk, g[2][keys], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, g[3][keys], rtol=0, atol=1e-12)
    xk = np.array([2, 9, 15])
    dk, dv = orc.keys_backward(orc.key_index(CORRUPTED, xk))
    np.testing.assert_allclose(dk, g[4][xk], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, g[5][xk], rtol=0, atol=1e-12)


def test_planted_mistakes_are_caught(monkeypatch):
    """A plausible slip in the oracle's rules (strict vs non-strict block
    comparison) must break the hand-drawn fixture."""
    import oracle.bdattn_oracle as ob

    def wrong(q_stream, q_block, k_stream, k_block):
        qc, kc = q_stream == CLEAN, k_stream == CLEAN
        return (qc & kc & (k_block < q_block)) | (~qc & kc & (k_block < q_block)) | \
            (~qc & ~kc & (k_block == q_block))

    p, want = read_golden("mask_L8_B2.txt")
    lay = layout(p["B"], 1, 1, 4, p["n_clean_q"])
    qs, qb = query_tokens(lay)
    ks, kb = key_tokens(lay)
    assert not np.array_equal(wrong(qs[:, None], qb[:, None], ks[None], kb[None]), want)


def test_missing_clean_coverage_is_rejected():
    with pytest.raises(ValueError):
        layout(2, 1, 1, 4, 4, 4, 6)  # queries at 4..7 need clean keys up to 8
    with pytest.raises(ValueError):
        layout(2, 1, 1, 4, 4, 0, 8, corr_block_ids=[5])  # block 5 needs keys < 10


# -------------------------------------------------- bf16 operand rounding mode
def test_round_bf16_matches_library_cast():
    from oracle import round_bf16
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(10000) * 10.0 ** rng.integers(-6, 6, 10000),
                        [0.0, -0.0, 1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8),
                         65504.0, 1e-30, 3.0e38]])
    want = torch.tensor(x, dtype=torch.float32).bfloat16().double().numpy()
    assert np.array_equal(round_bf16(x), want)


def test_operand_rounding_mode_is_the_exact_oracle_plus_roundings():
    """Exact mode is unchanged; bf16 mode stays within bf16 rounding of the
    exact result and its outputs are bf16 values."""
    from oracle import round_bf16
    lay = layout(4, 4, 2, 8, 32)
    t = make(lay, seed=41, scale=0.5)
    for k in t:  # inputs as a bf16 kernel receives them
        t[k] = round_bf16(t[k])
    ex = oracle_of(lay, t)
    bf = Oracle(lay, t["q_c"], t["k_c"], t["v_c"], t["q_x"], t["k_x"], t["v_x"], t["do_c"],
                t["do_x"], operand_rounding="bf16")
    e = ex.forward() + ex.backward()
    b = bf.forward() + bf.backward()
    for i, (x, y) in enumerate(zip(b, e)):
        if i in (2, 3):  # LSE is not rounded
            np.testing.assert_allclose(x, y, rtol=1e-14)
            continue
        assert np.array_equal(round_bf16(x), x)
        err = np.max(np.abs(x - y)) / np.max(np.abs(y))
        assert 0 < err < 2e-2, (i, err)
    with pytest.raises(ValueError):
        Oracle(lay, t["q_c"], t["k_c"], t["v_c"], t["q_x"], t["k_x"], t["v_x"],
               operand_rounding="fp8")


# ------------------------------------------------- partial attention, merge
def _split_inputs(lay, t, lo, hi, corr_keys):
    """Inputs of the partial problem holding clean keys [lo, hi) of a full
    problem's buffer (and the corrupted keys if corr_keys)."""
    ids = list(lay.corr_ids)
    part = layout(lay.B, lay.H, lay.Hkv, lay.d, lay.n_clean_q, lay.clean_q_start, hi - lo, lo,
                  corr_block_ids=ids, partial=True, clean_mask=lay.clean_mask,
                  corr_keys=corr_keys)
    u = dict(t)
    u["k_c"], u["v_c"] = t["k_c"][lo:hi], t["v_c"][lo:hi]
    return part, u


@pytest.mark.parametrize("case", [
    dict(B=4, H=4, Hkv=2, d=6, n_clean_q=32),
    dict(B=4, H=4, Hkv=2, d=6, n_clean_q=32, clean_mask=TOKEN_CAUSAL),
    dict(B=2, H=2, Hkv=1, d=5, n_clean_q=8, clean_q_start=8, n_clean_kv=16,
         corr_block_ids=[1, 4, 6]),
])
def test_partials_over_a_key_partition_merge_to_the_full_attention(case):
    """Implementation 1 of the appendix: the block-diagonal corrupted part and
    clean K/V in shards at their original positions, each a partial attention,
    merged through their log-sum-exps, give the full result; and the backward
    of each part, taken with the merged O and LSE, gives the full gradients
    (dQ summed over the parts, dK/dV of each part's own keys)."""
    lay = layout(**case)
    t = make(lay, seed=31)
    full = oracle_of(lay, t)
    O_c, O_x, L_c, L_x = full.forward()
    O = np.concatenate([O_c, O_x])
    LSE = np.concatenate([L_c, L_x], axis=1)
    g_full = full.backward(O=O, LSE=LSE)
    nkv = lay.n_clean_kv
    cuts = [0, lay.B * (nkv // lay.B // 3), lay.B * (2 * nkv // lay.B // 3), nkv]
    pieces = [(0, 0, True)] + [(a, b, False) for a, b in zip(cuts, cuts[1:]) if b > a]
    parts, grads = [], []
    for lo, hi, ck in pieces:
        part, u = _split_inputs(lay, t, lo, hi, ck)
        orc = oracle_of(part, u)
        o_c, o_x, l_c, l_x = orc.forward()
        parts.append((np.concatenate([o_c, o_x]), np.concatenate([l_c, l_x], axis=1)))
        grads.append((lo, hi, ck, orc.backward(O=O, LSE=LSE)))
    Om, Lm = merge_partials(parts)
    np.testing.assert_allclose(Om, O, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(Lm, LSE, rtol=1e-12, atol=1e-12)
    dq_c = sum(g[0] for _, _, _, g in grads)
    dq_x = sum(g[1] for _, _, _, g in grads)
    np.testing.assert_allclose(dq_c, g_full[0], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dq_x, g_full[1], rtol=1e-11, atol=1e-12)
    for lo, hi, ck, g in grads:
        np.testing.assert_allclose(g[2], g_full[2][lo:hi], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(g[3], g_full[3][lo:hi], rtol=1e-11, atol=1e-12)
        want_x = (g_full[4], g_full[5]) if ck else (0 * g_full[4], 0 * g_full[5])
        np.testing.assert_allclose(g[4], want_x[0], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(g[5], want_x[1], rtol=1e-11, atol=1e-12)


def test_partial_rows_without_keys_are_the_empty_sum():
    """A row that sees no key present gets O = 0, LSE = -inf, and a part with
    no key leaves a merge unchanged."""
    lay = layout(4, 2, 1, 3, 16)
    t = make(lay, seed=2)
    part, u = _split_inputs(lay, t, 8, 16, False)  # clean keys of blocks 2..3 only
    o_c, o_x, l_c, l_x = oracle_of(part, u).forward()
    assert np.all(o_c[:8] == 0) and np.all(np.isneginf(l_c[:, :8]))  # blocks 0, 1: nothing
    assert np.all(np.isfinite(l_c[:, 8:]))
    assert np.all(o_x[:12] == 0) and np.all(np.isneginf(l_x[:, :12]))  # blocks 0..2: nothing
    assert np.all(np.isfinite(l_x[:, 12:]))
    O = np.concatenate([o_c, o_x])
    L = np.concatenate([l_c, l_x], axis=1)
    empty = (np.zeros_like(O), np.full_like(L, -np.inf))
    Om, Lm = merge_partials([(O, L), empty])
    assert np.array_equal(Om, O) and np.array_equal(Lm, L)


# ------------------------------------------------- complementary masking
def test_corrupted_copies_of_a_block_are_independent():
    """Two corrupted copies of the same block (complementary masking) each
    give exactly what a problem holding only that copy gives: outputs, query
    gradients and their own dK/dV; the clean dK/dV are the sum of the two
    problems' (§3.2 separability, applied to copies)."""
    B, H, Hkv, d, L = 4, 2, 1, 5, 16
    both = layout(B, H, Hkv, d, L, corr_block_ids=[2, 2])
    t = make(both, seed=41)
    got = oracle_of(both, t)
    O_c, O_x, L_c, L_x = got.forward()
    g = got.backward()
    dk_c, dv_c = np.zeros_like(g[2]), np.zeros_like(g[3])
    for j in range(2):
        one = layout(B, H, Hkv, d, L, corr_block_ids=[2])
        u = dict(t)
        rows = slice(j * B, (j + 1) * B)
        for k in ("q_x", "k_x", "v_x", "do_x"):
            u[k] = t[k][rows]
        # the clean stream's share: count it once, in the first problem
        if j == 1:
            u["do_c"] = np.zeros_like(t["do_c"])
        ref = oracle_of(one, u)
        o_c, o_x, l_c, l_x = ref.forward()
        r = ref.backward()
        np.testing.assert_allclose(O_x[rows], o_x, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(L_x[:, rows], l_x, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(g[1][rows], r[1], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(g[4][rows], r[4], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(g[5][rows], r[5], rtol=1e-11, atol=1e-12)
        dk_c += r[2]
        dv_c += r[3]
    np.testing.assert_allclose(g[2], dk_c, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(g[3], dv_c, rtol=1e-11, atol=1e-12)


# ------------------------------------------------------- packed documents
def test_packed_document_pair_count_closed_form():
    """Full documents of lengths L_i packed into one sequence: each is its
    own block-diffusion problem, L_i (L_i + B) pairs per head (token-causal:
    L_i (L_i + 1) / 2 + L_i (L_i + B) / 2)."""
    B = 4
    lens = [8, 4, 20, 12]
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).tolist()
    L = sum(lens)
    for cm, per in ((BLOCK_CAUSAL, lambda n: n * (n + B)),
                    (TOKEN_CAUSAL, lambda n: n * (n + 1) // 2 + n * (n + B) // 2)):
        lay = layout(B, 1, 1, 4, L, doc_starts=starts, clean_mask=cm)
        assert int(full_mask(lay).sum()) == sum(per(n) for n in lens)


def test_bad_document_starts_are_rejected():
    for bad in ([4, 8], [0, 6], [0, 8, 8], [0, 12, 8]):
        with pytest.raises(ValueError):
            layout(4, 1, 1, 4, 32, doc_starts=bad)


@pytest.mark.parametrize("clean_mask", [BLOCK_CAUSAL, TOKEN_CAUSAL])
def test_packed_documents_equal_independent_problems(clean_mask):
    """A packed sequence is the documents run one by one: each document alone
    (positions counted from its own start, its corrupted blocks renumbered
    from its first block) gives exactly the packed problem's outputs and
    gradients on its rows and keys. Corrupted blocks include a repeated id
    (two copies) and a document without any."""
    B, H, Hkv, d = 2, 4, 2, 8
    lens = [6, 2, 10, 4]  # multiples of B
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(int)
    L = sum(lens)
    ids = [0, 2, 2, 4, 5, 7, 8]  # document 3 (blocks 9, 10) has none
    lay = layout(B, H, Hkv, d, L, corr_block_ids=ids, doc_starts=starts.tolist(),
                 clean_mask=clean_mask)
    t = make(lay, seed=11)
    ref = oracle_of(lay, t)
    O_c, O_x, L_c, L_x = ref.forward()
    g = ref.backward()
    x_rows = np.repeat(np.asarray(ids), B) * B  # block position of each corrupted row
    for s0, n in zip(starts, lens):
        b0 = s0 // B
        mine = [i for i in ids if b0 <= i < b0 + n // B]
        xr = np.flatnonzero((x_rows >= s0) & (x_rows < s0 + n))
        sub = layout(B, H, Hkv, d, n, corr_block_ids=[i - b0 for i in mine],
                     clean_mask=clean_mask)
        c = slice(s0, s0 + n)
        u = dict(q_c=t["q_c"][c], k_c=t["k_c"][c], v_c=t["v_c"][c], do_c=t["do_c"][c],
                 q_x=t["q_x"][xr], k_x=t["k_x"][xr], v_x=t["v_x"][xr], do_x=t["do_x"][xr])
        one = oracle_of(sub, u)
        o_c, o_x, l_c, l_x = one.forward()
        np.testing.assert_allclose(O_c[c], o_c, rtol=0, atol=1e-13)
        np.testing.assert_allclose(L_c[:, c], l_c, rtol=0, atol=1e-13)
        np.testing.assert_allclose(O_x[xr], o_x, rtol=0, atol=1e-13)
        np.testing.assert_allclose(L_x[:, xr], l_x, rtol=0, atol=1e-13)
        h = one.backward()
        for full, part, idx in ((g[0], h[0], c), (g[1], h[1], xr), (g[2], h[2], c),
                                (g[3], h[3], c), (g[4], h[4], xr), (g[5], h[5], xr)):
            np.testing.assert_allclose(full[idx], part, rtol=0, atol=1e-12)


@pytest.mark.parametrize("slip", ["left_side", "corrupted_by_own_position", "no_documents"])
def test_planted_document_mistakes_are_caught(monkeypatch, slip):
    """Plausible slips in the document rule break the hand-drawn document
    fixture: a document boundary assigned to the earlier document, a
    corrupted query placed by its local row instead of its block's position,
    documents ignored."""
    import oracle.bdattn_oracle as ob

    right = ob.documents

    def planted(lay, pos):
        pos = np.asarray(pos, dtype=np.int64)
        if slip == "left_side":
            return np.searchsorted(np.asarray(lay.docs, np.int64), pos, side="left") - 1
        if slip == "no_documents":
            return np.zeros(pos.shape, np.int64)
        return right(lay, pos)

    p, want = read_golden("mask_docs_L12_B2.txt")
    lay = layout(p["B"], 1, 1, 4, p["n_clean_q"], p["clean_q_start"], p["n_clean_kv"],
                 corr_block_ids=p["ids"], doc_starts=p["docs"])
    monkeypatch.setattr(ob, "documents", planted)
    qs, qb = query_tokens(lay)
    ks, kb = key_tokens(lay)
    qp, kp = query_positions(lay), key_positions(lay)
    if slip == "corrupted_by_own_position":
        qp = np.concatenate([qp[:lay.n_clean_q], lay.n_clean_q + np.arange(lay.n_corr)])
    qd, kd = ob.documents(lay, qp), ob.documents(lay, kp)
    got = visible(qs[:, None], qb[:, None], ks[None, :], kb[None, :], qp[:, None], kp[None, :],
                  lay.clean_mask, lay.corr_keys,
                  corrupted_copies(lay, lay.n_clean_q)[:, None],
                  corrupted_copies(lay, lay.n_clean_kv)[None, :], qd[:, None], kd[None, :])
    assert not np.array_equal(got, want)


# ------------------------------------------ gathered clean buffer (positions)
@pytest.mark.parametrize("partial", [False, True])
def test_gathered_clean_buffer_is_a_row_permutation(partial):
    """Appendix, Implementation 1: the clean K/V may arrive gathered in any
    order, each key masked by its original position. A layout naming every
    buffer row's position gives the same O, LSE and dQ as the position-ordered
    buffer, and dK/dV permuted like the buffer rows (zigzag order of P = 4
    ranks: rank r brings chunks r and 2P-1-r)."""
    B, P, C = 2, 4, 4
    L = 2 * P * C
    lo = 0 if not partial else 8
    kw = dict(corr_block_ids=[1, 5, 6, 11, 14])
    if partial:
        kw.update(partial=True)
    chunks = [c for r in range(P) for c in (r, 2 * P - 1 - r)]
    pos = [c * C + i for c in chunks for i in range(C)]
    if partial:  # chunks of the range [8, 32) only
        pos = [p for p in pos if p >= lo]
    n_kv = len(pos)
    ordered = layout(B, 4, 2, 4, L, 0, n_kv, lo, **kw)
    gathered = layout(B, 4, 2, 4, L, 0, n_kv, lo, clean_kv_positions=pos, **kw)
    t = make(ordered, seed=61)
    perm = np.asarray(pos) - lo  # buffer row i holds ordered row perm[i]
    tg = dict(t, k_c=t["k_c"][perm], v_c=t["v_c"][perm])
    a = oracle_of(ordered, t)
    b = oracle_of(gathered, tg)
    fa, fb = a.forward(), b.forward()
    ga, gb = a.backward(), b.backward()
    for x, y in zip(fa, fb):
        np.testing.assert_allclose(y, x, rtol=0, atol=1e-13)
    for i, (x, y) in enumerate(zip(ga, gb)):
        if i in (2, 3):  # clean dK, dV follow the buffer's rows
            x = x[perm]
        np.testing.assert_allclose(y, x, rtol=0, atol=1e-12)
    # the rows really moved: the first gathered rows are not the first positions
    assert not np.array_equal(perm, np.arange(n_kv))


def test_gathered_buffer_must_cover_the_visible_keys():
    with pytest.raises(ValueError):  # position 3 is missing
        layout(2, 1, 1, 4, 4, clean_kv_positions=[0, 1, 2, 5])
    with pytest.raises(ValueError):  # a repeated position
        layout(2, 1, 1, 4, 4, clean_kv_positions=[0, 1, 1, 3])
