"""Work claiming on the GPU: the forward, dQ and dK/dV kernels take their work
items from per-XCD queues with stealing (BDATTN_CLAIM=1; by default the host
claims only for long lists of long items), or workgroup i runs item i
(BDATTN_CLAIM=0); for short lists the forward and dQ kernels can also run on a
persistent grid of one workgroup per CU that claims item after item
(BDATTN_PERSIST=1). Every item computes the same values whichever
workgroup runs it, so both schedules must give bitwise equal outputs; the
outputs start as NaN, so an item that no workgroup ran would show. The
claimed schedules run three times each per case (the steals differ from run
to run) on the same workspaces, whose claim counters every call restarts.
Cases: small problems with every descriptor option (packed documents, a
share's rows, a gathered buffer, GQA, fp32), the 8K workload, whose 1,024
query-tile and 2,048 key-tile items span all 256 CUs, and 64 short documents
(1,024 short query-tile items: the persistent grid's case).

The library reads the switch at every call.
"""
import pytest
import torch

from tests.gpu_util import say
from tests.test_gpu_gathered import zigzag
from workloads import INPUT_NAMES, config, make_inputs, small_spec
import block_masked_attention_amd as bd

pytestmark = pytest.mark.gpu

CASES = [
    small_spec(L=1056, B=32, H=8, Hkv=2, d=128, dtype="bf16", std=0.5, seed=3, name="bf16 d128 ragged"),
    small_spec(L=2048, B=32, H=8, Hkv=2, d=128, dtype="bf16", std=0.5, seed=5, doc_starts=[0, 96, 800],
               name="bf16 d128 3 documents"),
    small_spec(L=1000, B=8, H=4, Hkv=4, d=128, dtype="bf16", seed=9, n_clean_q=520, clean_q_start=480,
               name="bf16 d128 partial rows"),
    small_spec(L=1024, B=32, H=8, Hkv=2, d=128, dtype="bf16", std=0.5, seed=11,
               name="bf16 d128 gathered").with_(kv_chunk_len=128, kv_chunk_pos=zigzag(4, 128)),
    small_spec(L=520, B=8, H=4, Hkv=2, d=32, dtype="bf16", seed=6, name="bf16 d32"),
    small_spec(L=512, B=16, H=4, Hkv=2, d=32, dtype="f32", seed=4, name="f32 d32"),
    small_spec(L=64, B=16, H=2, Hkv=2, d=32, dtype="f32", seed=8, name="f32 4 blocks (fewer items than queues)"),
]


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _nan_like(*shape, dtype):
    return torch.full(shape, float("nan"), dtype=dtype, device="cuda")


def _run(spec, t, ws):
    """fwd + bwd into NaN-filled outputs with the workspaces ws; returns the
    ten outputs."""
    p = bd.from_spec(spec)
    dt = t["q_c"].dtype
    H, Hkv, d = spec.H, spec.Hkv, spec.d
    nc, nkv, nx = spec.n_clean_q, spec.n_clean_kv, spec.n_corr
    f = [_nan_like(nc, H, d, dtype=dt), _nan_like(nx, H, d, dtype=dt),
         _nan_like(H, nc, dtype=torch.float32), _nan_like(H, nx, dtype=torch.float32)]
    g = [_nan_like(nc, H, d, dtype=dt), _nan_like(nx, H, d, dtype=dt), _nan_like(nkv, Hkv, d, dtype=dt),
         _nan_like(nkv, Hkv, d, dtype=dt), _nan_like(nx, Hkv, d, dtype=dt), _nan_like(nx, Hkv, d, dtype=dt)]
    ins = [t[k] for k in INPUT_NAMES]
    bd.fwd(p, *ins, out=f, workspace=ws[0])
    bd.bwd(p, *ins, *f, t["do_c"], t["do_x"], out=g, workspace=ws[1])
    torch.cuda.synchronize()
    return f + g


def _check(spec, monkeypatch):
    t = make_inputs(spec, device="cuda")
    # one pair of workspaces for every run: each call must restart the claim
    # counters the previous one left at the end of their queues
    p = bd.from_spec(spec)
    ws = [torch.zeros(bd.workspace_size(p, k), dtype=torch.uint8, device="cuda") for k in (0, 1)]
    monkeypatch.setenv("BDATTN_CLAIM", "0")
    monkeypatch.setenv("BDATTN_PERSIST", "0")
    want = _run(spec, t, ws)
    # a row with no visible key gets LSE = -inf and O = 0 (never NaN)
    assert not any(torch.isnan(x).any().item() for x in want), "static schedule left an output unwritten"
    # one item per workgroup, claimed; then a persistent grid claiming item
    # after item (it applies to lists with more items than CUs)
    for claim, persist in (("1", "0"), ("0", "1")):
        monkeypatch.setenv("BDATTN_CLAIM", claim)
        monkeypatch.setenv("BDATTN_PERSIST", persist)
        for rep in range(3):
            got = _run(spec, t, ws)
            holes = [torch.isnan(x).any().item() for x in got]
            same = [torch.equal(a, b) for a, b in zip(got, want)]
            say(f"  {spec.name}: claim {claim} persist {persist} run {rep}: no NaN left "
                f"{not any(holes)}, bitwise {same}")
            assert not any(holes) and all(same)


@pytest.mark.parametrize("spec", CASES, ids=lambda s: s.name)
def test_claimed_schedule_is_bitwise_the_static_one(spec, monkeypatch):
    _need_gpu()
    _check(spec, monkeypatch)


def test_claimed_schedule_8k_workload(monkeypatch):
    _need_gpu()
    _check(config("8k"), monkeypatch)


def test_persistent_grid_with_many_short_documents(monkeypatch):
    """1,024 query-tile items of 64 documents: the host's choice for such a
    list is the persistent grid, forced here against the static deal."""
    _need_gpu()
    starts = [0] + [256 * k + 32 * (k % 5) for k in range(1, 64)]
    _check(small_spec(L=16384, B=32, H=8, Hkv=2, d=128, dtype="bf16", std=0.5, seed=12,
                      doc_starts=starts, name="bf16 d128 64 documents"), monkeypatch)
