// Visibility rule of block-diffusion attention, compiled for host and device.
//
// "Block Parallelism for Efficient Distributed Long-Context Diffusion Language
// Model Training", §3.2 (Block diffusion language models):
//   clean query of block qb      sees clean keys of blocks kb <= qb (block-
//                                causal), or, token-causal, clean keys of
//                                blocks kb < qb and those of its own block at
//                                positions up to its own; never corrupted keys;
//   corrupted query of block qb  sees clean keys of blocks kb < qb and the
//                                corrupted keys of its own block.
// Blocks are 0-indexed on global clean positions: block(p) = p / B.
// Packed documents (several variable-length sequences in one): each document
// starts on a block boundary and no pair crosses two documents.
//
// Every row's visible keys are two intervals: clean keys [clo, cb) of the
// clean K/V buffer (clo = 0, or the start of the row's document) and an
// interval [xlo, xhi) of the local corrupted keys. This O(n) bound form is
// what the planner, the kernels and the host mask render all evaluate.
#pragma once

#include <stdint.h>

#if defined(__HIP__)
#define BD_HD __attribute__((host, device, always_inline)) inline
#else
#define BD_HD inline
#endif

// Visible key intervals of one query row.
struct BdRowBounds {
  int32_t clo;  // clean keys [clo, cb) are visible
  int32_t cb;
  int32_t xlo;  // corrupted keys [xlo, xhi) are visible (empty for clean rows)
  int32_t xhi;
};

// Clean query at global position gpos: clean keys of blocks 0..block(gpos),
// or, token-causal, clean keys at positions 0..gpos.
BD_HD BdRowBounds bd_clean_row(int32_t gpos, int32_t B, bool token_causal) {
  BdRowBounds r;
  r.clo = 0;
  r.cb = token_causal ? gpos + 1 : (gpos / B + 1) * B;
  r.xlo = 0;
  r.xhi = 0;
  return r;
}

// Corrupted query at local corrupted row `row`, whose block has global id
// `block_id`: clean keys of blocks < block_id, corrupted keys of its own block
// (local block index row / B, packed contiguously).
BD_HD BdRowBounds bd_corr_row(int32_t row, int32_t block_id, int32_t B) {
  BdRowBounds r;
  r.clo = 0;
  r.cb = block_id * B;
  r.xlo = (row / B) * B;
  r.xhi = r.xlo + B;
  return r;
}

// Packed documents: one entry per global block, describing the block's
// document.
struct BdDocSpan {
  int32_t lo;   // first position of the document
  int32_t hi;   // one past its last position (2^31 - 1 for the last document)
  int32_t xhi;  // B times the local corrupted blocks whose ids lie before hi / B
  int32_t pad;
};

// The bounds of a row inside its document (`s`: the entry of the row's block,
// its own for a clean row, its id's for a corrupted row): no clean key before
// the document's start. The rules keep every other bound inside it.
BD_HD BdRowBounds bd_in_document(BdRowBounds r, const BdDocSpan& s) {
  r.clo = s.lo;
  return r;
}

// The same bounds relative to a clean K/V buffer holding global positions
// [kv0, kv0 + nkv) (the whole prefix when kv0 = 0 and the buffer covers it):
// the visible clean keys present are buffer indices [clo - kv0, cb - kv0),
// clipped to the buffer; without the corrupted keys, none of those is visible.
BD_HD BdRowBounds bd_in_buffer(BdRowBounds r, int32_t kv0, int32_t nkv, bool corr_keys) {
  const int32_t c = r.cb - kv0, l = r.clo - kv0;
  r.cb = c < 0 ? 0 : (c > nkv ? nkv : c);
  r.clo = l < 0 ? 0 : (l > nkv ? nkv : l);
  if (!corr_keys) r.xlo = r.xhi = 0;
  return r;
}

// Is clean key `k` (buffer index) visible to the row (bounds in buffer terms)?
BD_HD bool bd_sees_clean(const BdRowBounds& r, int32_t k) { return k >= r.clo && k < r.cb; }

// Is local corrupted key `k` visible to the row?
BD_HD bool bd_sees_corr(const BdRowBounds& r, int32_t k) { return k >= r.xlo && k < r.xhi; }
