"""Seeded synthetic inputs for block-diffusion attention, shared by the oracle
tests and the GPU path.

This module holds shapes and random draws only: no attention arithmetic, no
mask rule, no scale. Both sides receive exactly the tensors drawn here.

Workloads follow the structure of "Block Parallelism for Efficient Distributed
Long-Context Diffusion Language Model Training": a length-L clean stream and a
length-L corrupted stream split into blocks of B tokens (§3.2), every eligible
target block present (§5.1, SFT / conversion workloads), and one rank's share
of a context-sharded run (§4.3) as a clean-query shard plus a subset of
corrupted blocks. The pages measure on real agent trajectories, which are not
available here; Gaussian activations of the stated shapes stand in for them.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional, Sequence, Tuple

import torch

__all__ = ["Spec", "CONFIGS", "config", "make_inputs", "INPUT_NAMES", "GRAD_NAMES"]

INPUT_NAMES = ("q_c", "k_c", "v_c", "q_x", "k_x", "v_x")
GRAD_NAMES = ("do_c", "do_x")


@dataclass(frozen=True)
class Spec:
    """Shape of one problem plus the recipe of its random values.

    Field names follow the C ABI's problem descriptor. ``B`` is the block size
    in tokens (the pages use B for the block count; here it is the size).
    ``corr_block_ids`` lists the global ids of the local corrupted blocks, in
    increasing order; ``None`` means blocks ``0 .. n_corr_blocks-1``.
    """

    name: str
    B: int
    H: int
    Hkv: int
    d: int
    dtype: str  # "f32" or "bf16"
    n_clean_q: int
    clean_q_start: int
    n_clean_kv: int
    clean_kv_start: int
    n_corr_blocks: int
    corr_block_ids: Optional[Tuple[int, ...]] = None
    # value recipe
    std: float = 1.0  # Q/K/V ~ N(0,1)*std
    outlier_frac: float = 0.0  # fraction of K token rows (each stream) scaled
    outlier_mult: float = 1.0
    seed: int = 0
    description: str = ""
    # what a clean query sees of its own block: 0 all of it (block-causal),
    # 1 the keys up to its own position (token-causal)
    clean_mask: int = 0
    # packed documents: start positions (first 0, multiples of B); None: one
    doc_starts: Optional[Tuple[int, ...]] = None
    # a gathered clean K/V buffer: chunks of kv_chunk_len rows, chunk i at
    # global positions [kv_chunk_pos[i], +kv_chunk_len); 0: position order
    kv_chunk_len: int = 0
    kv_chunk_pos: Optional[Tuple[int, ...]] = None

    def kv_positions(self):
        """Global position of every clean K/V buffer row (a list)."""
        if not self.kv_chunk_len:
            return list(range(self.clean_kv_start, self.clean_kv_start + self.n_clean_kv))
        C = self.kv_chunk_len
        return [p + r for p in self.kv_chunk_pos for r in range(C)]

    @property
    def n_corr(self) -> int:
        return self.n_corr_blocks * self.B

    def torch_dtype(self) -> torch.dtype:
        return {"f32": torch.float32, "bf16": torch.bfloat16}[self.dtype]

    def with_(self, **kw) -> "Spec":
        return replace(self, **kw)


def _full(name, L, B, H, Hkv, d, dtype, std, seed, desc, **kw) -> Spec:
    return Spec(name=name, B=B, H=H, Hkv=Hkv, d=d, dtype=dtype, n_clean_q=L,
                clean_q_start=0, n_clean_kv=L, clean_kv_start=0,
                n_corr_blocks=L // B, corr_block_ids=None, std=std, seed=seed,
                description=desc, **kw)


def _rank_share(name, L_total, P, r, B, H, Hkv, d, dtype, std, seed, desc) -> Spec:
    """One rank's share of a context split in P contiguous shards: clean
    queries of shard r, the full preceding clean K/V as an input buffer, and
    the corrupted blocks b with b mod P == r (0-indexed)."""
    shard = L_total // P
    nb = L_total // B
    ids = tuple(b for b in range(nb) if b % P == r)
    return Spec(name=name, B=B, H=H, Hkv=Hkv, d=d, dtype=dtype,
                n_clean_q=shard, clean_q_start=r * shard,
                n_clean_kv=(r + 1) * shard, clean_kv_start=0,
                n_corr_blocks=len(ids), corr_block_ids=ids, std=std, seed=seed,
                description=desc)


# The five workloads (index 0 is the small case the oracle finishes in
# seconds; index 3 is the 256K long-context headline workload).
CONFIGS: Tuple[Spec, ...] = (
    _full("tiny", 256, 16, 2, 2, 32, "f32", 1.0, 1000,
          "clean L=256 + corrupted L=256, B=16, H=Hkv=2, d=32, fp32"),
    _full("8k", 8192, 32, 16, 16, 128, "bf16", 0.5, 1001,
          "clean L=8192 + corrupted 8192, B=32, H=Hkv=16, d=128, bf16"),
    _full("64k", 65536, 32, 32, 8, 128, "bf16", 0.5, 1002,
          "clean L=65536 + corrupted 65536, B=32, GQA 32/8, d=128, bf16, 1% of key rows x8",
          outlier_frac=0.01, outlier_mult=8.0),
    _full("256k", 262144, 32, 32, 8, 128, "bf16", 0.5, 1003,
          "clean L=262144 + corrupted 262144, B=32, GQA 32/8, d=128, bf16"),
    _rank_share("512k_rank15", 524288, 16, 15, 32, 32, 8, 128, "bf16", 0.5, 1004,
                "512K context split 16 ways, rank 15: 32768 clean queries at 491520, "
                "524288-token clean K/V buffer, corrupted blocks b = 15 mod 16, B=32, "
                "GQA 32/8, d=128, bf16"),
)


def config(name_or_index) -> Spec:
    if isinstance(name_or_index, int):
        return CONFIGS[name_or_index]
    for c in CONFIGS:
        if c.name == name_or_index:
            return c
    raise KeyError(name_or_index)


def make_inputs(spec: Spec, device="cpu", seed: Optional[int] = None):
    """Draw the problem's tensors with a seeded generator on ``device``.

    Draw order: Q_c, K_c, V_c, Q_x, K_x, V_x, dO_c, dO_x, each fp32 N(0,1);
    Q/K/V are multiplied by ``spec.std``; then, if ``outlier_frac`` > 0, a
    seeded sample of floor(n*frac) token rows of K_c and then of K_x (drawn
    without replacement) is multiplied by ``outlier_mult`` across all heads
    and dims; finally every tensor is cast (round to nearest even) to the
    spec's dtype.

    Layouts are token-major: Q/dO ``[n, H, d]``, K/V ``[n, Hkv, d]``.
    Returns a dict keyed by INPUT_NAMES + GRAD_NAMES.
    """
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(spec.seed if seed is None else seed)
    n_c, n_kv, n_x = spec.n_clean_q, spec.n_clean_kv, spec.n_corr
    shapes = {
        "q_c": (n_c, spec.H, spec.d),
        "k_c": (n_kv, spec.Hkv, spec.d),
        "v_c": (n_kv, spec.Hkv, spec.d),
        "q_x": (n_x, spec.H, spec.d),
        "k_x": (n_x, spec.Hkv, spec.d),
        "v_x": (n_x, spec.Hkv, spec.d),
        "do_c": (n_c, spec.H, spec.d),
        "do_x": (n_x, spec.H, spec.d),
    }
    out = {}
    for name in INPUT_NAMES + GRAD_NAMES:
        t = torch.randn(shapes[name], generator=g, device=dev, dtype=torch.float32)
        if name in INPUT_NAMES and spec.std != 1.0:
            t.mul_(spec.std)
        out[name] = t
    if spec.outlier_frac > 0:
        for name in ("k_c", "k_x"):
            n = out[name].shape[0]
            cnt = int(n * spec.outlier_frac)
            rows = torch.randperm(n, generator=g, device=dev)[:cnt]
            out[name][rows] *= spec.outlier_mult
    dt = spec.torch_dtype()
    for k in list(out):
        out[k] = out[k].to(dt).contiguous()
    return out


def small_spec(L=256, B=16, H=2, Hkv=2, d=32, dtype="f32", seed=7, std=1.0,
               n_clean_q=None, clean_q_start=0, n_clean_kv=None,
               corr_block_ids: Optional[Sequence[int]] = None, name="small",
               outlier_frac=0.0, outlier_mult=1.0, clean_mask=0, doc_starts=None) -> Spec:
    """A full-sequence (or, with ids/offsets, one-share) problem for tests."""
    n_clean_q = L if n_clean_q is None else n_clean_q
    n_clean_kv = L if n_clean_kv is None else n_clean_kv
    if corr_block_ids is None:
        ncb, ids = L // B, None
    else:
        ids = tuple(int(i) for i in corr_block_ids)
        ncb = len(ids)
    return Spec(name=name, B=B, H=H, Hkv=Hkv, d=d, dtype=dtype,
                n_clean_q=n_clean_q, clean_q_start=clean_q_start,
                n_clean_kv=n_clean_kv, clean_kv_start=0, n_corr_blocks=ncb,
                corr_block_ids=ids, std=std, seed=seed,
                outlier_frac=outlier_frac, outlier_mult=outlier_mult, clean_mask=clean_mask,
                doc_starts=tuple(int(x) for x in doc_starts) if doc_starts else None)


__all__.append("small_spec")


# ------------------------------------------------ linear cross-entropy
@dataclass(frozen=True)
class LceSpec:
    """A token-chunked linear cross-entropy problem: N tokens with hidden
    size D over a vocabulary of V entries, `chunk` tokens per chunk."""
    name: str
    N: int
    D: int
    V: int
    chunk: int
    seed: int = 0
    logit_std: float = 2.0  # std of the logits h.w at initialisation
    ignore_frac: float = 0.0  # fraction of targets set to ignore_index (-100)
    description: str = ""


# The loss of block-diffusion training is taken on the corrupted tokens: at
# the 256K context that is 262,144 tokens per sequence. Vocabulary 131,072
# and hidden size 4,096 (an 8B-class model of the family the pages train;
# the pages state neither).
LCE_CONFIGS: Tuple[LceSpec, ...] = (
    LceSpec("lce_8k", 8192, 4096, 131072, 4096, seed=2001,
            description="8192 tokens, hidden 4096, vocabulary 131072, chunks of 4096, bf16"),
    LceSpec("lce_256k", 262144, 4096, 131072, 8192, seed=2002,
            description="262144 tokens (the corrupted stream at 256K context), hidden 4096, "
                        "vocabulary 131072, chunks of 8192, bf16"),
)


def make_lce_inputs(spec: LceSpec, device="cpu"):
    """Seeded draws: h [N, D] ~ N(0, 1), w [V, D] ~ N(0, 1) * logit_std /
    sqrt(D) (both rounded to bf16), targets uniform over [0, V) with
    ignore_frac of them set to -100 (int32), and the upstream gradient of a
    mean over the valid tokens (float32 [N])."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(spec.seed)
    h = torch.randn(spec.N, spec.D, generator=g, device=dev).to(torch.bfloat16)
    w = (torch.randn(spec.V, spec.D, generator=g, device=dev) * (spec.logit_std / spec.D ** 0.5)
         ).to(torch.bfloat16)
    t = torch.randint(0, spec.V, (spec.N,), generator=g, device=dev, dtype=torch.int32)
    if spec.ignore_frac > 0:
        t[torch.rand(spec.N, generator=g, device=dev) < spec.ignore_frac] = -100
    n_valid = int((t != -100).sum().item())
    dloss = torch.full((spec.N,), 1.0 / max(1, n_valid), device=dev, dtype=torch.float32)
    return dict(h=h, w=w, targets=t, dloss=dloss)


__all__ += ["LceSpec", "LCE_CONFIGS", "make_lce_inputs"]
