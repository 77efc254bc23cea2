"""The allocation-free forward (bdattn_fwd_noalloc) against bdattn_fwd,
called through the C ABI: two calls in a row, the second on a smaller
problem, each bitwise equal to the forward with a workspace (also with
float32 outputs); a problem whose scratch exceeds the library's array is
refused before any GPU work; with work claiming or the persistent grid
forced on, the claim counters in the scratch array restart at zero with
every call."""
import ctypes

import pytest
import torch

import block_masked_attention_amd as bd
from workloads import INPUT_NAMES, make_inputs, small_spec

pytestmark = pytest.mark.gpu


def _noalloc(p, t):
    dt = torch.float32 if p.dtype == bd.F32 or p.precision else torch.bfloat16
    nc, nx, H, d = int(p.n_clean_q), p.n_corr, int(p.H), int(p.d)
    o_c = torch.full((nc, H, d), float("nan"), dtype=dt, device="cuda")
    o_x = torch.full((nx, H, d), float("nan"), dtype=dt, device="cuda")
    lse_c = torch.full((H, nc), float("nan"), device="cuda")
    lse_x = torch.full((H, nx), float("nan"), device="cuda")
    torch.cuda.synchronize()
    ptr = lambda x: ctypes.c_void_p(x.data_ptr() if x.numel() else 0)
    st = bd.lib().bdattn_fwd_noalloc(ctypes.byref(p), *[ptr(t[k]) for k in INPUT_NAMES],
                                     ptr(o_c), ptr(o_x), ptr(lse_c), ptr(lse_x),
                                     ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st, (o_c, o_x, lse_c, lse_x)


def test_noalloc_forward_equals_the_workspace_forward_twice_in_a_row():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    big = small_spec(L=4096, B=32, H=8, Hkv=2, d=128, dtype="bf16", std=0.5, seed=31,
                     doc_starts=[0, 1024, 1536, 3072])
    small = small_spec(L=640, B=16, H=4, Hkv=1, d=128, dtype="bf16", std=0.5, seed=32,
                       n_clean_q=320, clean_q_start=320, n_clean_kv=640,
                       corr_block_ids=[1, 5, 9, 30, 33])
    for spec in (big, small):  # the second call's lists are shorter than the first's
        print(f"[gpu] no-alloc forward: {spec.name} L={spec.n_clean_q}", flush=True)
        t = make_inputs(spec, device="cuda")
        p = bd.from_spec(spec)
        st, got = _noalloc(p, t)
        assert st == 0, bd.lib().bdattn_last_error().decode()
        want = bd.fwd(p, *[t[k] for k in INPUT_NAMES])
        torch.cuda.synchronize()
        for a, b in zip(got, want):
            assert torch.equal(a, b)


def test_noalloc_forward_with_claimed_work(monkeypatch):
    """Work claimed from the queue counters (forced on: these problems are
    small) in the scratch array: every call starts them at zero, so three
    calls in a row (large, small, large) each equal bdattn_fwd bitwise, with
    no output left unwritten."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    monkeypatch.setenv("BDATTN_CLAIM", "1")
    big = small_spec(L=4096, B=32, H=8, Hkv=2, d=128, dtype="bf16", std=0.5, seed=34)
    small = small_spec(L=1024, B=16, H=4, Hkv=2, d=128, dtype="bf16", std=0.5, seed=35)
    for spec in (big, small, big):
        print(f"[gpu] no-alloc forward, claimed work: {spec.name} L={spec.n_clean_q}", flush=True)
        t = make_inputs(spec, device="cuda")
        p = bd.from_spec(spec)
        st, got = _noalloc(p, t)
        assert st == 0, bd.lib().bdattn_last_error().decode()
        want = bd.fwd(p, *[t[k] for k in INPUT_NAMES])
        torch.cuda.synchronize()
        for a, b in zip(got, want):
            assert not torch.isnan(a).any().item()
            assert torch.equal(a, b)


def test_noalloc_forward_on_the_persistent_grid(monkeypatch):
    """Many short documents (lists of more items than CUs) on the persistent
    grid, forced on: its workgroups claim item after item from the counters
    in the scratch array, and three calls in a row (large, smaller, large)
    each equal bdattn_fwd bitwise, with no output left unwritten."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    monkeypatch.setenv("BDATTN_CLAIM", "0")
    monkeypatch.setenv("BDATTN_PERSIST", "1")
    big = small_spec(L=16384, B=32, H=8, Hkv=2, d=128, dtype="bf16", std=0.5, seed=36,
                     doc_starts=[0] + [256 * k + 32 * (k % 5) for k in range(1, 64)])
    small = small_spec(L=8192, B=32, H=8, Hkv=2, d=128, dtype="bf16", std=0.5, seed=37,
                       doc_starts=[0] + [256 * k + 64 * (k % 3) for k in range(1, 32)])
    for spec in (big, small, big):
        print(f"[gpu] no-alloc forward, persistent grid: {spec.name} L={spec.n_clean_q}", flush=True)
        t = make_inputs(spec, device="cuda")
        p = bd.from_spec(spec)
        st, got = _noalloc(p, t)
        assert st == 0, bd.lib().bdattn_last_error().decode()
        want = bd.fwd(p, *[t[k] for k in INPUT_NAMES])
        torch.cuda.synchronize()
        for a, b in zip(got, want):
            assert not torch.isnan(a).any().item()
            assert torch.equal(a, b)


def test_noalloc_forward_with_float32_outputs():
    """The precision modes reach the allocation-free forward too: float32
    outputs (and split operands), bitwise those of bdattn_fwd."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    spec = small_spec(L=1024, B=32, H=8, Hkv=2, d=128, dtype="bf16", std=0.5, seed=33)
    t = make_inputs(spec, device="cuda")
    for prec in (bd.PRECISION_F32_OUT, bd.PRECISION_SPLIT):
        print(f"[gpu] no-alloc forward, precision {prec}", flush=True)
        p = bd.from_spec(spec, precision=prec)
        st, got = _noalloc(p, t)
        assert st == 0, bd.lib().bdattn_last_error().decode()
        want = bd.fwd(p, *[t[k] for k in INPUT_NAMES])
        torch.cuda.synchronize()
        assert got[0].dtype == torch.float32
        for a, b in zip(got, want):
            assert torch.equal(a, b)


def test_noalloc_forward_refuses_a_problem_beyond_its_scratch():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    # 4M clean tokens at 64 q heads: the work list needs more than 8 MiB
    p = bd.problem(32, 64, 8, 128, "bf16", 1 << 22)
    assert bd.workspace_size(p, 0) > (8 << 20)
    fake = ctypes.c_void_p(1 << 20)  # never touched: the size check comes first
    st = bd.lib().bdattn_fwd_noalloc(ctypes.byref(p), *[fake] * 10, None)
    assert st == -5
    assert "8388608" in bd.lib().bdattn_last_error().decode()
