"""CPU float64 oracle for clean-plus-corrupted block-diffusion attention.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check of the build
entry point and the benchmark's CPU-baseline leg may import this module. The
GPU library never calls it and shares no code with it.

What it computes follows "Block Parallelism for Efficient Distributed
Long-Context Diffusion Language Model Training":

* §3.2 (Block diffusion language models): a clean copy and a corrupted copy of
  the sequence, split into blocks. A clean token of block b sees the clean
  tokens of blocks < b and, of its own block, all of it (the block-causal
  reading, the default) or the tokens up to its own position (the token-causal
  reading of the section's "causal access within block b"; see ``visible``);
  a corrupted token of target block b sees its own corrupted block
  bidirectionally and the clean prefix of blocks < b, and never the corrupted
  tokens of other blocks.
* §4.4 (Proposition 1): the distributed schemes reproduce exactly the plain
  masked computation, so the oracle is the plain definition of masked softmax
  attention over the visible keys, with its textbook analytic backward. No
  tiling, no online softmax, no skipping beyond restricting each row chunk to
  the columns its own mask marks visible.
* §4.3 (Backward pass): gradients of clean K/V sum the contributions of every
  query (clean, or corrupted of a later block) that sees them.
* Appendix, "Efficient fused operator" (Implementation 1): the attention can be
  computed as partial attentions over disjoint key sets (the block-diagonal
  corrupted part, and clean K/V given by original positions), merged through
  their log-sum-exps. A *partial* layout holds only some keys: the result is
  the attention over the visible keys present (a row that sees none gets
  O = 0, LSE = -inf), and ``merge_partials`` combines such results. The clean
  keys may come in any order, each with its original clean position (the
  gathered buffer of that paragraph): a layout then names the position of
  every row of its clean K/V buffer.
* Packed documents (variable-length training sequences, §5.1; Block Diffusion,
  named in §2, generates sequences of any length): several documents share
  one sequence, each starting on a block boundary, with its blocks counted
  from its own start, and attention never crosses from one document into
  another. The four rules above then hold inside each document.

Conventions (readings where the pages are silent): blocks are 0-indexed with
block(p) = floor(p / B) on global clean positions; the scale defaults to
1/sqrt(d); LSE is the natural log of the softmax normaliser, including the
scale; q head h reads KV head floor(h / (H/Hkv)); no position encoding,
dropout or bias; LSE is not differentiated.

Every array is float64 numpy. Queries are indexed clean-local first, then
corrupted-local; keys are the clean buffer first, then the corrupted keys.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

CLEAN = 0
CORRUPTED = 1

BLOCK_CAUSAL = 0  # a clean query sees its whole own clean block
TOKEN_CAUSAL = 1  # ... or its own clean block up to its own position

__all__ = ["Layout", "layout", "visible", "query_tokens", "key_tokens", "query_positions",
           "key_positions", "corrupted_copies", "Oracle", "CLEAN", "CORRUPTED", "BLOCK_CAUSAL", "TOKEN_CAUSAL",
           "round_bf16", "merge_partials", "documents", "clean_key_positions"]


@dataclass(frozen=True)
class Layout:
    B: int
    H: int
    Hkv: int
    d: int
    scale: float
    n_clean_q: int
    clean_q_start: int
    n_clean_kv: int
    clean_kv_start: int
    corr_ids: tuple  # global ids of the local corrupted blocks, increasing
    clean_mask: int = BLOCK_CAUSAL
    partial: bool = False  # keys may be missing: attention over the keys present
    corr_keys: bool = True  # the local corrupted keys are present
    docs: tuple = ()  # start positions of packed documents (empty: one document)
    kv_pos: tuple = ()  # position of each clean K/V buffer row (empty: clean_kv_start + row)

    @property
    def G(self) -> int:
        return self.H // self.Hkv

    @property
    def n_corr(self) -> int:
        return len(self.corr_ids) * self.B

    @property
    def nq(self) -> int:
        return self.n_clean_q + self.n_corr

    @property
    def nk(self) -> int:
        return self.n_clean_kv + self.n_corr


def layout(B: int, H: int, Hkv: int, d: int, n_clean_q: int, clean_q_start: int = 0,
           n_clean_kv: Optional[int] = None, clean_kv_start: int = 0,
           n_corr_blocks: Optional[int] = None,
           corr_block_ids: Optional[Sequence[int]] = None,
           scale: Optional[float] = None, partial: bool = False,
           clean_mask: int = BLOCK_CAUSAL, corr_keys: bool = True,
           doc_starts: Optional[Sequence[int]] = None,
           clean_kv_positions: Optional[Sequence[int]] = None) -> Layout:
    """Describe one problem. Without ids, the corrupted blocks are 0..n-1
    (n defaults to the number of clean blocks of the query shard).
    ``clean_mask`` is BLOCK_CAUSAL or TOKEN_CAUSAL.

    Unless ``partial``, the clean K/V buffer must hold every clean key some
    local query sees and the corrupted keys must be present (a ValueError
    otherwise). A partial layout may hold any clean range (``clean_kv_start``
    > 0 included) and may omit the corrupted keys (``corr_keys=False``).

    ``doc_starts`` packs several documents into the sequence: their start
    positions, increasing, the first 0, each a multiple of B (a document
    starts a new block). None or a single 0 is one document.

    ``clean_kv_positions`` gives the original clean position of every row of
    the clean K/V buffer, distinct, in any order (a gathered buffer);
    ``clean_kv_start`` is then unused. Without it, row r is at position
    ``clean_kv_start + r``."""
    if n_clean_kv is None:
        n_clean_kv = n_clean_q
    if corr_block_ids is None:
        if n_corr_blocks is None:
            n_corr_blocks = n_clean_q // B
        corr_block_ids = range(n_corr_blocks)
    ids = tuple(int(i) for i in corr_block_ids)
    if H % Hkv:
        raise ValueError("H must be a multiple of Hkv")
    if clean_mask not in (BLOCK_CAUSAL, TOKEN_CAUSAL):
        raise ValueError("clean_mask must be BLOCK_CAUSAL or TOKEN_CAUSAL")
    if scale is None or scale <= 0:
        scale = 1.0 / math.sqrt(d)
    docs = tuple(int(x) for x in (doc_starts or ()))
    if docs:
        if docs[0] != 0 or any(b <= a for a, b in zip(docs, docs[1:])) or any(x % B for x in docs):
            raise ValueError("doc_starts must start at 0, increase and be multiples of B")
        if len(docs) == 1:
            docs = ()
    if not partial and not corr_keys:
        raise ValueError("only a partial layout may omit the corrupted keys")
    kv_pos = ()
    if clean_kv_positions is not None:
        kv_pos = tuple(int(x) for x in clean_kv_positions)
        if len(kv_pos) != n_clean_kv or len(set(kv_pos)) != len(kv_pos) or min(kv_pos, default=0) < 0:
            raise ValueError("clean_kv_positions: one distinct position >= 0 per buffer row")
    if not partial:
        need = 0  # one past the last clean position some query sees
        if n_clean_q:
            need = ((clean_q_start + n_clean_q - 1) // B + 1) * B
        if ids:
            need = max(need, max(ids) * B)
        if kv_pos:
            covered = need <= len(kv_pos) and set(range(need)) <= set(kv_pos)
        else:
            covered = clean_kv_start == 0 and n_clean_kv >= need
        if need and not covered:
            raise ValueError("clean K/V buffer does not cover every visible clean key")
    return Layout(B, H, Hkv, d, float(scale), n_clean_q, clean_q_start, n_clean_kv,
                  clean_kv_start, ids, clean_mask, bool(partial), bool(corr_keys), docs, kv_pos)


def clean_key_positions(lay: Layout):
    """Original clean position of every row of the clean K/V buffer."""
    if lay.kv_pos:
        return np.asarray(lay.kv_pos, dtype=np.int64)
    return lay.clean_kv_start + np.arange(lay.n_clean_kv, dtype=np.int64)


def query_tokens(lay: Layout):
    """(stream, block) of every query: clean-local rows, then corrupted."""
    pos = lay.clean_q_start + np.arange(lay.n_clean_q, dtype=np.int64)
    stream = np.concatenate([np.full(lay.n_clean_q, CLEAN, np.int8),
                             np.full(lay.n_corr, CORRUPTED, np.int8)])
    block = np.concatenate([pos // lay.B,
                            np.repeat(np.asarray(lay.corr_ids, np.int64), lay.B)])
    return stream, block


def key_tokens(lay: Layout):
    """(stream, block) of every key: the clean buffer, then corrupted."""
    pos = clean_key_positions(lay)
    stream = np.concatenate([np.full(lay.n_clean_kv, CLEAN, np.int8),
                             np.full(lay.n_corr, CORRUPTED, np.int8)])
    block = np.concatenate([pos // lay.B,
                            np.repeat(np.asarray(lay.corr_ids, np.int64), lay.B)])
    return stream, block


def query_positions(lay: Layout):
    """Sequence position of every query: clean rows at their global clean
    position, corrupted rows at their position inside the sequence (block id
    times B plus the offset in the block)."""
    clean = lay.clean_q_start + np.arange(lay.n_clean_q, dtype=np.int64)
    corr = (np.repeat(np.asarray(lay.corr_ids, np.int64), lay.B) * lay.B
            + np.tile(np.arange(lay.B, dtype=np.int64), len(lay.corr_ids)))
    return np.concatenate([clean, corr])


def key_positions(lay: Layout):
    """Sequence position of every key (clean buffer, then corrupted keys)."""
    clean = clean_key_positions(lay)
    corr = (np.repeat(np.asarray(lay.corr_ids, np.int64), lay.B) * lay.B
            + np.tile(np.arange(lay.B, dtype=np.int64), len(lay.corr_ids)))
    return np.concatenate([clean, corr])


def documents(lay: Layout, pos):
    """Index of the packed document holding each sequence position (all 0
    for a single document)."""
    pos = np.asarray(pos, dtype=np.int64)
    if not lay.docs:
        return np.zeros(pos.shape, np.int64)
    return np.searchsorted(np.asarray(lay.docs, np.int64), pos, side="right") - 1


def corrupted_copies(lay: Layout, n_clean: int):
    """Local corrupted block (copy) index of every token of a query or key
    list with ``n_clean`` clean tokens first; -1 for clean tokens. Two local
    blocks with the same id are two corrupted copies of that block
    (complementary masking)."""
    return np.concatenate([np.full(n_clean, -1, np.int64),
                           np.repeat(np.arange(len(lay.corr_ids), dtype=np.int64), lay.B)])


def visible(q_stream, q_block, k_stream, k_block, q_pos=None, k_pos=None,
            clean_mask=BLOCK_CAUSAL, corr_keys=True, q_copy=None, k_copy=None,
            q_doc=None, k_doc=None):
    """The four visibility rules of §3.2, broadcast over their arguments.

    clean query, block qb     -> clean key of block kb  iff kb < qb, or kb == qb
                                 (block-causal: the whole own block;
                                  token-causal: key position <= query position)
    clean query               -> corrupted key          never
    corrupted query, block qb -> clean key of block kb  iff kb <  qb
    corrupted query, block qb -> corrupted key, block kb iff kb == qb, of its
                                 own copy (``q_copy``/``k_copy``, when a rank
                                 holds two corrupted copies of a block)

    With packed documents (``q_doc``/``k_doc``: the document of each token)
    a pair is visible only inside one document.

    Positions are needed only for TOKEN_CAUSAL. With ``corr_keys`` False the
    corrupted keys are absent (a partial problem) and none is visible.
    """
    qc = q_stream == CLEAN
    kc = k_stream == CLEAN
    own_block = k_block == q_block
    if clean_mask == TOKEN_CAUSAL:
        own_block = own_block & (k_pos <= q_pos)
    clean_clean = qc & kc & ((k_block < q_block) | own_block)
    corr_clean = ~qc & kc & (k_block < q_block)
    corr_corr = ~qc & ~kc & (k_block == q_block) & bool(corr_keys)
    if q_copy is not None:
        corr_corr = corr_corr & (k_copy == q_copy)
    vis = clean_clean | corr_clean | corr_corr
    if q_doc is not None:
        vis = vis & (q_doc == k_doc)
    return vis


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def merge_partials(parts):
    """Attention over the union of disjoint key sets from the partial results
    over each set (appendix, Implementation 1). ``parts`` is a list of
    (O ``[n, H, d]``, LSE ``[H, n]``). Each part's O_i is its softmax-weighted
    mean over its own keys and exp(LSE_i) its softmax denominator, so
    LSE = ln sum_i exp(LSE_i) and O = sum_i exp(LSE_i - LSE) O_i. A part with
    LSE_i = -inf (no key) has weight 0; a row with no key in any part keeps
    O = 0, LSE = -inf."""
    Os = [_f64(o) for o, _ in parts]
    Ls = [_f64(l) for _, l in parts]
    top = np.max(np.stack(Ls), axis=0)
    ref = np.where(np.isfinite(top), top, 0.0)
    w = [np.exp(l - ref) for l in Ls]  # exp(-inf) = 0
    den = np.sum(w, axis=0)
    with np.errstate(divide="ignore"):
        LSE = ref + np.log(den)
    safe = np.where(den > 0, den, 1.0)
    O = np.zeros_like(Os[0])
    for wi, oi in zip(w, Os):
        O += (wi / safe).T[:, :, None] * oi
    return O, LSE


def round_bf16(x):
    """Round to the nearest bfloat16 value (ties to even), through float32
    (as a kernel that rounds its fp32 results does). bfloat16 keeps the top
    16 bits of a float32: add half of the dropped part, with the tie going
    to the even kept value, then truncate."""
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def _ident(x):
    return x


class Oracle:
    """Plain masked softmax attention and its analytic backward, in float64.

    Construct with the layout and the inputs (Q/dO ``[n, H, d]``, K/V
    ``[n, Hkv, d]``) exactly as the GPU receives them (upcast, never rounded).

    ``operand_rounding="bf16"`` gives the same definition evaluated with the
    roundings a bf16 matrix-core implementation cannot avoid, and nothing
    else: the softmax weights are rounded to bf16 before they multiply V (and
    dO), dS is rounded to bf16 before it multiplies K (and Q), the saved O
    that D = <dO, O> reads is the bf16 output, and every output is stored in
    bf16. Products are still exact sums in float64. It measures what bf16
    arithmetic at those points costs; the default (None) is the exact oracle.
    """

    # rows x columns of one chunk's dense score matrix (bounded memory only)
    CHUNK_ELEMS = 1 << 24

    def __init__(self, lay: Layout, q_c, k_c, v_c, q_x, k_x, v_x, do_c=None, do_x=None,
                 operand_rounding=None):
        self.lay = lay
        if operand_rounding not in (None, "bf16"):
            raise ValueError("operand_rounding must be None or 'bf16'")
        self.rd = round_bf16 if operand_rounding == "bf16" else _ident
        self.Q = np.concatenate([_f64(q_c), _f64(q_x)]).reshape(lay.nq, lay.H, lay.d)
        K = np.concatenate([_f64(k_c), _f64(k_x)]).reshape(lay.nk, lay.Hkv, lay.d)
        V = np.concatenate([_f64(v_c), _f64(v_x)]).reshape(lay.nk, lay.Hkv, lay.d)
        # keys of each KV head as one contiguous [nk, d] array
        self.Kh = [np.ascontiguousarray(K[:, g]) for g in range(lay.Hkv)]
        self.Vh = [np.ascontiguousarray(V[:, g]) for g in range(lay.Hkv)]
        del K, V
        if do_c is not None:
            self.dO = np.concatenate([_f64(do_c), _f64(do_x)]).reshape(lay.nq, lay.H, lay.d)
        else:
            self.dO = None
        self.qs, self.qb = query_tokens(lay)
        self.ks, self.kb = key_tokens(lay)
        self.qp, self.kp = query_positions(lay), key_positions(lay)
        self.qcp, self.kcp = corrupted_copies(lay, lay.n_clean_q), corrupted_copies(lay, lay.n_clean_kv)
        self.qd, self.kd = documents(lay, self.qp), documents(lay, self.kp)

    # ---------------------------------------------------------------- helpers
    def _mask(self, qidx, kidx=None):
        if kidx is None:
            kidx = slice(None)
        return visible(self.qs[qidx, None], self.qb[qidx, None],
                       self.ks[None, kidx], self.kb[None, kidx],
                       self.qp[qidx, None], self.kp[None, kidx], self.lay.clean_mask,
                       self.lay.corr_keys, self.qcp[qidx, None], self.kcp[None, kidx],
                       self.qd[qidx, None], self.kd[None, kidx])

    @staticmethod
    def _columns(cols):
        """Index of the visible key columns: a slice when they are one
        contiguous run (a view, no copy), else the index array."""
        if len(cols) and cols[-1] - cols[0] + 1 == len(cols):
            return slice(int(cols[0]), int(cols[-1]) + 1)
        return cols

    def _chunks(self, qidx):
        qidx = np.asarray(qidx, dtype=np.int64)
        step = max(1, min(2048, self.CHUNK_ELEMS // max(1, self.lay.nk)))
        for s in range(0, len(qidx), step):
            yield s, qidx[s:s + step]

    def _scores(self, rows, Kg, Mc, h):
        """Masked scores S = scale * q k^T over the gathered keys Kg of the
        row's KV head, -inf where not visible."""
        S = self.lay.scale * (self.Q[rows, h] @ Kg.T)
        S[~Mc] = -np.inf
        return S

    # ---------------------------------------------------------------- forward
    def rows_forward(self, qidx):
        """O ``[n, H, d]`` and LSE ``[H, n]`` of the given query rows."""
        qidx = np.asarray(qidx, dtype=np.int64)
        lay = self.lay
        O = np.zeros((len(qidx), lay.H, lay.d))
        LSE = np.zeros((lay.H, len(qidx)))
        for s, rows in self._chunks(qidx):
            M = self._mask(rows)
            seen = M.any(axis=1)
            if not seen.all() and not lay.partial:
                raise ValueError("a query row sees no key")
            # a row that sees no key present (partial layouts only): the empty
            # sum, O = 0 and LSE = ln 0 = -inf
            LSE[:, s:s + len(rows)] = -np.inf
            cols = np.flatnonzero(M.any(axis=0))
            if len(cols) == 0:
                continue
            Mc = M[:, cols]
            cs = self._columns(cols)
            for g in range(lay.Hkv):
                Kg, Vg = self.Kh[g][cs], self.Vh[g][cs]  # visible keys of KV head g
                for h in range(g * lay.G, (g + 1) * lay.G):
                    S = self._scores(rows, Kg, Mc, h)
                    m = np.where(seen, S.max(axis=1), 0.0)
                    E = np.exp(S - m[:, None])
                    l = E.sum(axis=1)
                    with np.errstate(divide="ignore"):
                        LSE[h, s:s + len(rows)] = m + np.log(l)
                    O[s:s + len(rows), h] = (self.rd(E) @ Vg) / np.where(seen, l, 1.0)[:, None]
        return self.rd(O), LSE

    def forward(self):
        """Full forward: (O_c, O_x, LSE_c, LSE_x)."""
        O, LSE = self.rows_forward(np.arange(self.lay.nq))
        nc = self.lay.n_clean_q
        return O[:nc], O[nc:], LSE[:, :nc], LSE[:, nc:]

    # --------------------------------------------------------------- backward
    def _row_stats(self, qidx, O=None, LSE=None):
        if O is None or LSE is None:
            O, LSE = self.rows_forward(qidx)
        D = np.einsum("nhd,nhd->nh", self.dO[qidx], self.rd(O))  # D_i = <dO_i, O_i>
        return O, LSE, D

    def rows_backward(self, qidx, kidx=None, O=None, LSE=None):
        """Gradients contributed by the given query rows.

        Returns dQ of those rows ``[n, H, d]`` and the dK, dV ``[nk, Hkv, d]``
        those rows contribute (summed over the rows and the q heads of each KV
        group). ``kidx`` restricts the key columns considered (all columns a
        row sees must be included for dQ to be complete).
        """
        if self.dO is None:
            raise ValueError("no upstream gradient given")
        lay = self.lay
        qidx = np.asarray(qidx, dtype=np.int64)
        O, LSE, D = self._row_stats(qidx, O, LSE)
        dQ = np.zeros((len(qidx), lay.H, lay.d))
        dK = np.zeros((lay.nk, lay.Hkv, lay.d))
        dV = np.zeros((lay.nk, lay.Hkv, lay.d))
        for s, rows in self._chunks(qidx):
            sl = slice(s, s + len(rows))
            M = self._mask(rows)
            if kidx is not None:
                keep = np.zeros(lay.nk, bool)
                keep[kidx] = True
                M = M & keep[None, :]
            cols = np.flatnonzero(M.any(axis=0))
            if len(cols) == 0:
                continue
            Mc = M[:, cols]
            cs = self._columns(cols)
            for g in range(lay.Hkv):
                Kg, Vg = self.Kh[g][cs], self.Vh[g][cs]  # visible keys of KV head g
                dKg = np.zeros_like(Kg)
                dVg = np.zeros_like(Vg)
                for h in range(g * lay.G, (g + 1) * lay.G):
                    S = self._scores(rows, Kg, Mc, h)
                    # exp(-inf) = 0 off the mask; a row whose LSE is -inf (no
                    # key at all) has no weight anywhere
                    Lr = np.where(np.isfinite(LSE[h, sl]), LSE[h, sl], np.inf)
                    P = np.exp(S - Lr[:, None])
                    dP = self.dO[rows, h] @ Vg.T
                    dS = self.rd(P * (dP - D[sl, h][:, None]))
                    dQ[sl, h] = lay.scale * (dS @ Kg)
                    dKg += lay.scale * (dS.T @ self.Q[rows, h])
                    dVg += self.rd(P).T @ self.dO[rows, h]
                dK[cs, g] += dKg
                dV[cs, g] += dVg
        return self.rd(dQ), self.rd(dK), self.rd(dV)

    def backward(self, O=None, LSE=None):
        """Full backward: (dQ_c, dQ_x, dK_c, dV_c, dK_x, dV_x)."""
        lay = self.lay
        dQ, dK, dV = self.rows_backward(np.arange(lay.nq), O=O, LSE=LSE)
        nc, nkc = lay.n_clean_q, lay.n_clean_kv
        return dQ[:nc], dQ[nc:], dK[:nkc], dV[:nkc], dK[nkc:], dV[nkc:]

    def keys_backward(self, kidx):
        """dK, dV ``[len(kidx), Hkv, d]`` of the given key columns: every
        query that sees one of them contributes (its full row is used for its
        LSE and D)."""
        kidx = np.asarray(kidx, dtype=np.int64)
        seen = np.zeros(self.lay.nq, bool)
        for s, rows in self._chunks(np.arange(self.lay.nq)):
            seen[rows] = self._mask(rows, kidx).any(axis=1)
        qidx = np.flatnonzero(seen)
        if len(qidx) == 0:
            z = np.zeros((len(kidx), self.lay.Hkv, self.lay.d))
            return z, z.copy()
        _, dK, dV = self.rows_backward(qidx, kidx=kidx)
        return dK[kidx], dV[kidx]

    def query_index(self, stream, local_rows):
        """Global query index of local rows of a stream."""
        local_rows = np.asarray(local_rows, dtype=np.int64)
        return local_rows if stream == CLEAN else self.lay.n_clean_q + local_rows

    def key_index(self, stream, local_rows):
        local_rows = np.asarray(local_rows, dtype=np.int64)
        return local_rows if stream == CLEAN else self.lay.n_clean_kv + local_rows
