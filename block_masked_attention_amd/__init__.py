"""Python binding of libbdattn (block-diffusion attention on MI355X).

Argument marshalling only: every step of the forward and backward runs in the
library's HIP kernels. Torch supplies device memory (outputs, workspace) and
the current HIP stream. The binding fails loudly when the library is missing:
there is no fallback implementation.

The entry points mirror the C ABI in include/bdattn.h: ``fwd``, ``bwd``,
``validate``, ``workspace_size``, ``mask_render``, ``visible_pairs``,
``plan_stats``, ``version``, ``status_string``.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbdattn.so")

F32 = 0
BF16 = 1
CLEAN_BLOCK_CAUSAL = 0
CLEAN_TOKEN_CAUSAL = 1
# bdattn_precision (include/bdattn.h)
PRECISION_DEFAULT = 0
PRECISION_F32_OUT = 1
PRECISION_SPLIT = 2
STATUS = {0: "BDATTN_OK", -1: "BDATTN_ERR_INVALID_ARG", -2: "BDATTN_ERR_SHAPE",
          -3: "BDATTN_ERR_UNSUPPORTED", -4: "BDATTN_ERR_COVERAGE",
          -5: "BDATTN_ERR_WORKSPACE", -6: "BDATTN_ERR_HIP"}

__all__ = ["Problem", "problem", "BdattnError", "lib", "fwd", "bwd", "validate",
           "workspace_size", "mask_render", "visible_pairs", "plan_stats", "version",
           "status_string", "profile_enable", "profile_read", "from_spec", "F32", "BF16",
           "CLEAN_BLOCK_CAUSAL", "CLEAN_TOKEN_CAUSAL", "LIB_PATH", "merge", "plan_cache_info",
           "plan_cache_budget", "LceProblem", "lce_problem", "lce_workspace_size", "lce_fwd",
           "lce_bwd", "lce_fwd_bwd"]


class BdattnError(RuntimeError):
    def __init__(self, status: int, where: str, message: str = ""):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({message})")


class Problem(ctypes.Structure):
    """ctypes mirror of ``bdattn_problem``. Build it with ``problem(...)``,
    which also keeps the host id array alive."""
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("d", ctypes.c_int32), ("dtype", ctypes.c_int32), ("scale", ctypes.c_float),
        ("n_clean_q", ctypes.c_int64), ("clean_q_start", ctypes.c_int64),
        ("n_clean_kv", ctypes.c_int64), ("clean_kv_start", ctypes.c_int64),
        ("n_corr_blocks", ctypes.c_int64),
        ("corr_block_ids", ctypes.POINTER(ctypes.c_int32)),
        ("clean_mask", ctypes.c_int32),
        ("partial", ctypes.c_int32),
        ("omit_corr_keys", ctypes.c_int32),
        ("n_docs", ctypes.c_int32),
        ("doc_starts", ctypes.POINTER(ctypes.c_int32)),
        ("kv_chunk_len", ctypes.c_int32),
        ("kv_chunk_pos", ctypes.POINTER(ctypes.c_int32)),
        ("precision", ctypes.c_int32),
    ]

    @property
    def n_corr(self) -> int:
        return int(self.n_corr_blocks) * int(self.B)


def problem(B: int, H: int, Hkv: int, d: int, dtype, n_clean_q: int, clean_q_start: int = 0,
            n_clean_kv: Optional[int] = None, clean_kv_start: int = 0,
            n_corr_blocks: Optional[int] = None, corr_block_ids: Optional[Sequence[int]] = None,
            scale: float = 0.0, clean_mask: int = CLEAN_BLOCK_CAUSAL, partial: bool = False,
            omit_corr_keys: bool = False,
            doc_starts: Optional[Sequence[int]] = None, kv_chunk_len: int = 0,
            kv_chunk_pos: Optional[Sequence[int]] = None, precision: int = 0) -> Problem:
    """Problem descriptor. ``dtype`` is F32/BF16, "f32"/"bf16" or a torch dtype.
    Without ids the corrupted blocks are 0..n_corr_blocks-1 (default: as many
    as the clean query shard has blocks). ``clean_mask`` is CLEAN_BLOCK_CAUSAL
    or CLEAN_TOKEN_CAUSAL (what a clean query sees of its own block).
    ``partial``: attention over the keys present only (any clean range, the
    corrupted keys optional with ``omit_corr_keys``); see include/bdattn.h.
    ``doc_starts`` packs documents into the sequence: their start positions
    (the first 0, increasing, multiples of B); attention stays inside each.
    ``kv_chunk_len`` / ``kv_chunk_pos``: a gathered clean K/V buffer, chunks of
    ``kv_chunk_len`` keys whose global start positions are ``kv_chunk_pos``
    (any order, together covering the buffer's position range).
    ``precision`` (bf16 inputs): PRECISION_DEFAULT, PRECISION_F32_OUT (O, dQ,
    dK, dV in float32; the backward then reads the float32 O) or
    PRECISION_SPLIT (float32 outputs, and P and dS enter their products as two
    bf16 terms); see include/bdattn.h."""
    dt = _dtype_code(dtype)
    if n_clean_kv is None:
        n_clean_kv = n_clean_q
    p = Problem()
    p.B, p.H, p.Hkv, p.d, p.dtype, p.scale = B, H, Hkv, d, dt, float(scale)
    p.clean_mask = int(clean_mask)
    p.partial = 1 if partial else 0
    p.omit_corr_keys = 1 if omit_corr_keys else 0
    p.n_clean_q, p.clean_q_start = n_clean_q, clean_q_start
    p.n_clean_kv, p.clean_kv_start = n_clean_kv, clean_kv_start
    if corr_block_ids is not None:
        ids = np.ascontiguousarray(np.asarray(corr_block_ids, dtype=np.int32))
        p._ids = ids  # keep alive
        p.n_corr_blocks = len(ids)
        p.corr_block_ids = ids.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    else:
        if n_corr_blocks is None:
            n_corr_blocks = n_clean_q // B if B > 0 else 0
        p.n_corr_blocks = n_corr_blocks
        p.corr_block_ids = None
    if doc_starts is not None and len(doc_starts) > 0:
        docs = np.ascontiguousarray(np.asarray(doc_starts, dtype=np.int32))
        p._docs = docs  # keep alive
        p.n_docs = len(docs)
        p.doc_starts = docs.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    else:
        p.n_docs, p.doc_starts = 0, None
    p.precision = int(precision)
    p.kv_chunk_len = int(kv_chunk_len)
    if kv_chunk_pos is not None and len(kv_chunk_pos) > 0:
        cpos = np.ascontiguousarray(np.asarray(kv_chunk_pos, dtype=np.int32))
        p._cpos = cpos  # keep alive
        p.kv_chunk_pos = cpos.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    else:
        p.kv_chunk_pos = None
    return p


class LceProblem(ctypes.Structure):
    """ctypes mirror of ``bdattn_lce_problem`` (include/bdattn_lce.h)."""
    _fields_ = [("n_tokens", ctypes.c_int64), ("hidden", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("ignore_index", ctypes.c_int32)]


def lce_problem(n_tokens: int, hidden: int, vocab: int, chunk: int = 4096,
                ignore_index: int = -100) -> LceProblem:
    """Linear cross-entropy descriptor: N tokens, hidden size D, vocabulary
    V, tokens per chunk, the ignored target value."""
    p = LceProblem()
    p.n_tokens, p.hidden, p.vocab, p.chunk, p.ignore_index = n_tokens, hidden, vocab, chunk, ignore_index
    return p


def from_spec(spec, precision: int = 0) -> Problem:
    """Descriptor of a workload spec (any object with the descriptor's fields)."""
    return problem(spec.B, spec.H, spec.Hkv, spec.d, spec.dtype, spec.n_clean_q,
                   spec.clean_q_start, spec.n_clean_kv, spec.clean_kv_start,
                   spec.n_corr_blocks, spec.corr_block_ids,
                   clean_mask=getattr(spec, "clean_mask", CLEAN_BLOCK_CAUSAL),
                   partial=getattr(spec, "partial", False),
                   omit_corr_keys=getattr(spec, "omit_corr_keys", False),
                   doc_starts=getattr(spec, "doc_starts", None),
                   kv_chunk_len=getattr(spec, "kv_chunk_len", 0),
                   kv_chunk_pos=getattr(spec, "kv_chunk_pos", None), precision=precision)


def _dtype_code(dtype) -> int:
    if dtype in (F32, "f32", "float32"):
        return F32
    if dtype in (BF16, "bf16", "bfloat16"):
        return BF16
    import torch
    if dtype == torch.float32:
        return F32
    if dtype == torch.bfloat16:
        return BF16
    raise ValueError(f"unsupported dtype {dtype!r}")


_LIB = None


def lib() -> ctypes.CDLL:
    """Load libbdattn.so (built in-tree); raise if it is not there."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m block_masked_attention_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(Problem)
    vp, fp = ctypes.c_void_p, ctypes.c_void_p
    L.bdattn_version.restype = ctypes.c_int
    L.bdattn_status_string.restype = ctypes.c_char_p
    L.bdattn_status_string.argtypes = [ctypes.c_int]
    L.bdattn_last_error.restype = ctypes.c_char_p
    L.bdattn_validate.argtypes = [P]
    L.bdattn_workspace_size.argtypes = [P, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]
    L.bdattn_mask_render.argtypes = [P, ctypes.c_void_p, ctypes.c_size_t]
    L.bdattn_visible_pairs.argtypes = [P, ctypes.POINTER(ctypes.c_int64)]
    L.bdattn_plan_stats.argtypes = [P, ctypes.POINTER(ctypes.c_int64)]
    L.bdattn_fwd.argtypes = [P] + [vp] * 6 + [vp, vp, fp, fp] + [vp, ctypes.c_size_t, vp]
    L.bdattn_fwd_noalloc.argtypes = [P] + [vp] * 6 + [vp, vp, fp, fp] + [vp]
    L.bdattn_bwd.argtypes = ([P] + [vp] * 6 + [vp, vp, fp, fp, vp, vp] + [vp] * 6 +
                             [vp, ctypes.c_size_t, vp])
    L.bdattn_merge.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                               vp, fp, vp, fp, vp, fp, vp]
    LP = ctypes.POINTER(LceProblem)
    L.bdattn_lce_workspace_size.argtypes = [LP, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]
    L.bdattn_lce_fwd.argtypes = [LP, vp, vp, vp, fp, fp, vp, ctypes.c_size_t, vp]
    L.bdattn_lce_bwd.argtypes = [LP, vp, vp, vp, fp, fp, vp, fp, vp, ctypes.c_size_t, vp]
    L.bdattn_lce_fwd_bwd.argtypes = [LP, vp, vp, vp, fp, fp, fp, vp, fp, vp, ctypes.c_size_t, vp]
    L.bdattn_plan_cache_info.argtypes = [ctypes.POINTER(ctypes.c_int64)]
    L.bdattn_plan_cache_budget.argtypes = [ctypes.c_size_t]
    L.bdattn_profile_enable.argtypes = [ctypes.c_int]
    L.bdattn_profile_read.argtypes = [ctypes.POINTER(ctypes.c_double),
                                      ctypes.POINTER(ctypes.c_int64)]
    L.bdattn_profile_read_n.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                                        ctypes.POINTER(ctypes.c_int64)]
    for name in ("bdattn_validate", "bdattn_workspace_size", "bdattn_mask_render",
                 "bdattn_visible_pairs", "bdattn_plan_stats", "bdattn_fwd", "bdattn_fwd_noalloc",
                 "bdattn_bwd",
                 "bdattn_merge", "bdattn_profile_enable", "bdattn_profile_read",
                 "bdattn_plan_cache_info", "bdattn_plan_cache_budget", "bdattn_lce_workspace_size",
                 "bdattn_lce_fwd", "bdattn_lce_bwd", "bdattn_lce_fwd_bwd", "bdattn_profile_read_n"):
        getattr(L, name).restype = ctypes.c_int
    _LIB = L
    return L


def _check(status: int, where: str):
    if status != 0:
        raise BdattnError(status, where, lib().bdattn_last_error().decode())


def version() -> int:
    return lib().bdattn_version()


def status_string(status: int) -> str:
    return lib().bdattn_status_string(status).decode()


def validate(p: Problem) -> int:
    """Status of the descriptor (0 = valid); never raises."""
    return lib().bdattn_validate(ctypes.byref(p))


def workspace_size(p: Problem, pass_: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().bdattn_workspace_size(ctypes.byref(p), pass_, ctypes.byref(n)), "workspace_size")
    return n.value


def mask_render(p: Problem) -> np.ndarray:
    nq = int(p.n_clean_q) + p.n_corr
    nk = int(p.n_clean_kv) + p.n_corr
    out = np.zeros((nq, nk), dtype=np.uint8)
    _check(lib().bdattn_mask_render(ctypes.byref(p), out.ctypes.data, out.nbytes), "mask_render")
    return out.astype(bool)


def visible_pairs(p: Problem) -> int:
    n = ctypes.c_int64(0)
    _check(lib().bdattn_visible_pairs(ctypes.byref(p), ctypes.byref(n)), "visible_pairs")
    return n.value


def plan_stats(p: Problem) -> dict:
    out = (ctypes.c_int64 * 8)()
    _check(lib().bdattn_plan_stats(ctypes.byref(p), out), "plan_stats")
    keys = ("fwd_items", "fwd_tiles", "fwd_masked_tiles", "bwd_items", "bwd_qtiles",
            "bwd_masked_qtiles", "fwd_rows_per_item", "bwd_keys_per_item")
    return dict(zip(keys, list(out)))


def plan_cache_info() -> dict:
    """State of the library's plan cache (plans, their host bytes, pinned
    staging bytes, the byte budget, evictions so far)."""
    out = (ctypes.c_int64 * 5)()
    _check(lib().bdattn_plan_cache_info(out), "plan_cache_info")
    return dict(zip(("plans", "host_bytes", "pinned_bytes", "budget", "evictions"), list(out)))


def plan_cache_budget(nbytes: int) -> None:
    """Bound the plan cache (host plans plus pinned staging) to ``nbytes``."""
    _check(lib().bdattn_plan_cache_budget(ctypes.c_size_t(nbytes)), "plan_cache_budget")


PROFILED_KERNELS = ("fwd", "bwd_dq", "bwd_dkdv")


def profile_enable(on: bool = True) -> None:
    """Record HIP events around the forward kernel and the backward's dQ and
    dK/dV kernels, on the stream each call is enqueued on."""
    _check(lib().bdattn_profile_enable(1 if on else 0), "profile_enable")


LCE_PROFILED = ("lce_logits", "lce_rows", "lce_dh", "lce_dw")


def profile_read_all() -> dict:
    """profile_read for every slot: the attention kernels and the linear
    cross-entropy's logits product, row kernel, dH and dW products."""
    names = PROFILED_KERNELS + LCE_PROFILED
    ms = (ctypes.c_double * len(names))()
    n = (ctypes.c_int64 * len(names))()
    _check(lib().bdattn_profile_read_n(len(names), ms, n), "profile_read_n")
    return {k: dict(ms=ms[i], launches=n[i]) for i, k in enumerate(names)}


def profile_read() -> dict:
    """Wait for the recorded events; per kernel ("fwd", "bwd_dq", "bwd_dkdv")
    the summed milliseconds and the number of launches since the last read."""
    ms = (ctypes.c_double * 3)()
    n = (ctypes.c_int64 * 3)()
    _check(lib().bdattn_profile_read(ms, n), "profile_read")
    return {k: dict(ms=ms[i], launches=n[i]) for i, k in enumerate(PROFILED_KERNELS)}


# ------------------------------------------------------------------ torch side
def _torch():
    import torch
    return torch


def _tdtype(p: Problem):
    torch = _torch()
    return torch.float32 if p.dtype == F32 else torch.bfloat16


def _odtype(p: Problem):
    """Element type of O, dQ, dK and dV."""
    torch = _torch()
    return torch.float32 if p.dtype == F32 or p.precision else torch.bfloat16


def _expect(t, shape, dtype, name, device):
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype} != {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr() if t.numel() else 0)


def _stream(device, stream):
    torch = _torch()
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _on(stream):
    """Allocation context: device memory the library reads on ``stream`` is
    taken from that stream's pool, so torch's caching allocator does not hand
    it out again while work queued on ``stream`` still uses it."""
    return contextlib.nullcontext() if stream is None else _torch().cuda.stream(stream)


def _workspace(p: Problem, pass_: int, device, workspace):
    torch = _torch()
    need = workspace_size(p, pass_)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    if workspace.numel() < need:
        raise ValueError(f"workspace has {workspace.numel()} bytes, needs {need}")
    return workspace


def fwd(p: Problem, q_c, k_c, v_c, q_x, k_x, v_x, *, workspace=None, stream=None, out=None):
    """Forward on the GPU. Returns (o_c, o_x, lse_c, lse_x). ``stream`` (a
    torch stream; default the current one) is where the work is enqueued;
    outputs and workspace allocated here come from that stream's pool. The
    caller orders the inputs' producers before it and the outputs' users
    after it."""
    torch = _torch()
    dev = q_c.device if q_c.numel() else q_x.device
    if dev.type != "cuda":
        raise ValueError("bdattn runs on a GPU: inputs must be on a cuda (HIP) device")
    dt = _tdtype(p)
    H, Hkv, d = int(p.H), int(p.Hkv), int(p.d)
    nc, nkv, nx = int(p.n_clean_q), int(p.n_clean_kv), p.n_corr
    for t, shp, nm in ((q_c, (nc, H, d), "q_c"), (k_c, (nkv, Hkv, d), "k_c"),
                       (v_c, (nkv, Hkv, d), "v_c"), (q_x, (nx, H, d), "q_x"),
                       (k_x, (nx, Hkv, d), "k_x"), (v_x, (nx, Hkv, d), "v_x")):
        _expect(t, shp, dt, nm, dev)
    odt = _odtype(p)
    with _on(stream):
        if out is None:
            o_c = torch.empty((nc, H, d), dtype=odt, device=dev)
            o_x = torch.empty((nx, H, d), dtype=odt, device=dev)
            lse_c = torch.empty((H, nc), dtype=torch.float32, device=dev)
            lse_x = torch.empty((H, nx), dtype=torch.float32, device=dev)
        else:
            o_c, o_x, lse_c, lse_x = out
            for t, shp, tdt, nm in ((o_c, (nc, H, d), odt, "o_c"), (o_x, (nx, H, d), odt, "o_x"),
                                    (lse_c, (H, nc), torch.float32, "lse_c"),
                                    (lse_x, (H, nx), torch.float32, "lse_x")):
                _expect(t, shp, tdt, nm, dev)
        ws = _workspace(p, 0, dev, workspace)
    st = lib().bdattn_fwd(ctypes.byref(p), _ptr(q_c), _ptr(k_c), _ptr(v_c), _ptr(q_x),
                          _ptr(k_x), _ptr(v_x), _ptr(o_c), _ptr(o_x), _ptr(lse_c), _ptr(lse_x),
                          _ptr(ws), ctypes.c_size_t(ws.numel()), _stream(dev, stream))
    _check(st, "bdattn_fwd")
    return o_c, o_x, lse_c, lse_x


def bwd(p: Problem, q_c, k_c, v_c, q_x, k_x, v_x, o_c, o_x, lse_c, lse_x, do_c, do_x, *,
        workspace=None, stream=None, out=None):
    """Backward on the GPU. Returns (dq_c, dq_x, dk_c, dv_c, dk_x, dv_x)."""
    torch = _torch()
    dev = q_c.device if q_c.numel() else q_x.device
    if dev.type != "cuda":
        raise ValueError("bdattn runs on a GPU: inputs must be on a cuda (HIP) device")
    dt, odt = _tdtype(p), _odtype(p)
    H, Hkv, d = int(p.H), int(p.Hkv), int(p.d)
    nc, nkv, nx = int(p.n_clean_q), int(p.n_clean_kv), p.n_corr
    for t, shp, tdt, nm in ((q_c, (nc, H, d), dt, "q_c"), (k_c, (nkv, Hkv, d), dt, "k_c"),
                            (v_c, (nkv, Hkv, d), dt, "v_c"), (q_x, (nx, H, d), dt, "q_x"),
                            (k_x, (nx, Hkv, d), dt, "k_x"), (v_x, (nx, Hkv, d), dt, "v_x"),
                            (o_c, (nc, H, d), odt, "o_c"), (o_x, (nx, H, d), odt, "o_x"),
                            (lse_c, (H, nc), torch.float32, "lse_c"),
                            (lse_x, (H, nx), torch.float32, "lse_x"),
                            (do_c, (nc, H, d), dt, "do_c"), (do_x, (nx, H, d), dt, "do_x")):
        _expect(t, shp, tdt, nm, dev)
    with _on(stream):
        if out is None:
            dq_c = torch.empty((nc, H, d), dtype=odt, device=dev)
            dq_x = torch.empty((nx, H, d), dtype=odt, device=dev)
            dk_c = torch.empty((nkv, Hkv, d), dtype=odt, device=dev)
            dv_c = torch.empty((nkv, Hkv, d), dtype=odt, device=dev)
            # not written when the corrupted keys are omitted: returned as zeros
            alloc = torch.zeros if p.omit_corr_keys else torch.empty
            dk_x = alloc((nx, Hkv, d), dtype=odt, device=dev)
            dv_x = alloc((nx, Hkv, d), dtype=odt, device=dev)
        else:
            dq_c, dq_x, dk_c, dv_c, dk_x, dv_x = out
            for t, shp, nm in ((dq_c, (nc, H, d), "dq_c"), (dq_x, (nx, H, d), "dq_x"),
                               (dk_c, (nkv, Hkv, d), "dk_c"), (dv_c, (nkv, Hkv, d), "dv_c")):
                _expect(t, shp, odt, nm, dev)
        ws = _workspace(p, 1, dev, workspace)
    st = lib().bdattn_bwd(ctypes.byref(p), _ptr(q_c), _ptr(k_c), _ptr(v_c), _ptr(q_x),
                          _ptr(k_x), _ptr(v_x), _ptr(o_c), _ptr(o_x), _ptr(lse_c), _ptr(lse_x),
                          _ptr(do_c), _ptr(do_x), _ptr(dq_c), _ptr(dq_x), _ptr(dk_c), _ptr(dv_c),
                          _ptr(dk_x), _ptr(dv_x), _ptr(ws), ctypes.c_size_t(ws.numel()),
                          _stream(dev, stream))
    _check(st, "bdattn_bwd")
    return dq_c, dq_x, dk_c, dv_c, dk_x, dv_x


def lce_workspace_size(p: LceProblem, pass_: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().bdattn_lce_workspace_size(ctypes.byref(p), pass_, ctypes.byref(n)),
           "lce_workspace_size")
    return n.value


def _lce_check(p, h, w, targets):
    torch = _torch()
    N, D, V = int(p.n_tokens), int(p.hidden), int(p.vocab)
    dev = w.device
    if dev.type != "cuda":
        raise ValueError("the linear cross-entropy runs on a GPU")
    _expect(h, (N, D), torch.bfloat16, "h", dev)
    _expect(w, (V, D), torch.bfloat16, "w", dev)
    _expect(targets, (N,), torch.int32, "targets", dev)
    return N, D, V, dev


def lce_fwd(p: LceProblem, h, w, targets, *, workspace=None, stream=None):
    """Linear cross-entropy forward: (loss [N], lse [N]) float32. ``h``
    [N, D] and ``w`` [V, D] bf16, ``targets`` [N] int32."""
    torch = _torch()
    N, D, V, dev = _lce_check(p, h, w, targets)
    with _on(stream):
        loss = torch.empty(N, dtype=torch.float32, device=dev)
        lse = torch.empty(N, dtype=torch.float32, device=dev)
        ws = workspace if workspace is not None else torch.empty(
            lce_workspace_size(p, 0), dtype=torch.uint8, device=dev)
    _check(lib().bdattn_lce_fwd(ctypes.byref(p), _ptr(h), _ptr(w), _ptr(targets), _ptr(loss),
                                _ptr(lse), _ptr(ws), ctypes.c_size_t(ws.numel()),
                                _stream(dev, stream)), "bdattn_lce_fwd")
    return loss, lse


def lce_bwd(p: LceProblem, h, w, targets, lse, dloss, *, workspace=None, stream=None):
    """Linear cross-entropy backward from the forward's ``lse`` and the
    per-token upstream gradient ``dloss`` (float32 [N]): (dh [N, D] bf16,
    dw [V, D] float32)."""
    torch = _torch()
    N, D, V, dev = _lce_check(p, h, w, targets)
    _expect(lse, (N,), torch.float32, "lse", dev)
    _expect(dloss, (N,), torch.float32, "dloss", dev)
    with _on(stream):
        dh = torch.empty(N, D, dtype=torch.bfloat16, device=dev)
        dw = torch.empty(V, D, dtype=torch.float32, device=dev)
        ws = workspace if workspace is not None else torch.empty(
            lce_workspace_size(p, 1), dtype=torch.uint8, device=dev)
    _check(lib().bdattn_lce_bwd(ctypes.byref(p), _ptr(h), _ptr(w), _ptr(targets), _ptr(lse),
                                _ptr(dloss), _ptr(dh), _ptr(dw), _ptr(ws),
                                ctypes.c_size_t(ws.numel()), _stream(dev, stream)), "bdattn_lce_bwd")
    return dh, dw


def lce_fwd_bwd(p: LceProblem, h, w, targets, dloss, *, workspace=None, stream=None, out=None):
    """Forward and backward in one pass: (loss, lse, dh, dw)."""
    torch = _torch()
    N, D, V, dev = _lce_check(p, h, w, targets)
    _expect(dloss, (N,), torch.float32, "dloss", dev)
    with _on(stream):
        if out is None:
            loss = torch.empty(N, dtype=torch.float32, device=dev)
            lse = torch.empty(N, dtype=torch.float32, device=dev)
            dh = torch.empty(N, D, dtype=torch.bfloat16, device=dev)
            dw = torch.empty(V, D, dtype=torch.float32, device=dev)
        else:
            loss, lse, dh, dw = out
        ws = workspace if workspace is not None else torch.empty(
            lce_workspace_size(p, 1), dtype=torch.uint8, device=dev)
    _check(lib().bdattn_lce_fwd_bwd(ctypes.byref(p), _ptr(h), _ptr(w), _ptr(targets),
                                    _ptr(dloss), _ptr(loss), _ptr(lse), _ptr(dh), _ptr(dw),
                                    _ptr(ws), ctypes.c_size_t(ws.numel()), _stream(dev, stream)),
           "bdattn_lce_fwd_bwd")
    return loss, lse, dh, dw


def merge(o_a, lse_a, o_b, lse_b, *, stream=None, out=None):
    """Merge two partial results over disjoint key sets (bdattn_merge):
    o_* ``[n, H, d]`` (fp32 or bf16), lse_* ``[H, n]`` float32. Returns
    (o, lse); ``out`` may name the inputs themselves."""
    torch = _torch()
    n, H, d = (int(x) for x in o_a.shape)
    dev = o_a.device
    for t, shp, tdt, nm in ((o_a, (n, H, d), o_a.dtype, "o_a"), (o_b, (n, H, d), o_a.dtype, "o_b"),
                            (lse_a, (H, n), torch.float32, "lse_a"),
                            (lse_b, (H, n), torch.float32, "lse_b")):
        _expect(t, shp, tdt, nm, dev)
    with _on(stream):
        if out is None:
            o = torch.empty_like(o_a)
            lse = torch.empty_like(lse_a)
        else:
            o, lse = out
    st = lib().bdattn_merge(ctypes.c_int64(n), H, d, _dtype_code(o_a.dtype), _ptr(o_a),
                            _ptr(lse_a), _ptr(o_b), _ptr(lse_b), _ptr(o), _ptr(lse),
                            _stream(dev, stream))
    _check(st, "bdattn_merge")
    return o, lse
