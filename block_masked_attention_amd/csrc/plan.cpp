// Host planner for block-diffusion attention: validation, pair counts, mask
// render and the longest-first work lists of the forward and backward kernels.
#include "plan.h"

#include <math.h>
#include <string.h>

#include <algorithm>
#include <numeric>

namespace bdattn {

namespace {

constexpr int64_t kMax32 = (int64_t(1) << 31) - 1;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int32_t ceil_div(int64_t a, int64_t b) { return int32_t((a + b - 1) / b); }

// Bounds of a local row in terms of the keys present (clean buffer indices).
BdRowBounds row_bounds(const Problem& P, int stream, int32_t row) {
  const int32_t blk = stream == 0 ? (P.clean_q_start + row) / P.B : P.ids[row / P.B];
  BdRowBounds r = stream == 0 ? bd_clean_row(P.clean_q_start + row, P.B, P.token_causal != 0)
                              : bd_corr_row(row, blk, P.B);
  if (!P.spans.empty()) r = bd_in_document(r, P.spans[blk]);
  return bd_in_buffer(r, P.clean_kv_start, P.n_clean_kv, P.corr_keys != 0);
}

// Document entry of every global block a row or key can name: document start,
// end, and the local corrupted rows before the end.
void build_spans(Problem* P) {
  int64_t nb = (int64_t(P->clean_q_start) + P->n_clean_q) / P->B;
  nb = std::max<int64_t>(nb, (int64_t(P->clean_kv_start) + P->n_clean_kv) / P->B);
  if (!P->ids.empty()) nb = std::max<int64_t>(nb, int64_t(P->ids.back()) + 1);
  P->spans.assign(size_t(nb), BdDocSpan{0, 0, 0, 0});
  size_t d = 0;
  for (int64_t b = 0; b < nb; ++b) {
    const int64_t pos = b * P->B;
    while (d + 1 < P->docs.size() && P->docs[d + 1] <= pos) ++d;
    BdDocSpan& s = P->spans[size_t(b)];
    s.lo = P->docs[d];
    s.hi = d + 1 < P->docs.size() ? P->docs[d + 1] : int32_t(kMax32);
    const int64_t end_blk = d + 1 < P->docs.size() ? P->docs[d + 1] / P->B : kMax32;
    s.xhi = int32_t(std::lower_bound(P->ids.begin(), P->ids.end(), end_blk) - P->ids.begin()) * P->B;
  }
}

// Work-list order. Longest first balances the CUs. With packed documents,
// the query-tile list (forward and dQ) also keeps the items of one document
// together, so the K/V tiles they share stay in the L2: documents longest
// first (by their items' summed cost), then each document's items longest
// first. One document keeps the plain longest-first order. (The same grouping
// of the key-tile list measured faster with 16 documents at 256K, but 11%
// slower with 1024, so that list stays longest first.)
// `doc` of an item is the index of its document in P.docs (0..n_docs-1).
template <class T>
void order_items(std::vector<T>* tiles, size_t n_docs) {
  if (n_docs <= 1) {
    std::stable_sort(tiles->begin(), tiles->end(),
                     [](const T& a, const T& b) { return a.cost > b.cost; });
    return;
  }
  std::vector<int64_t> doc_cost(n_docs, 0);
  for (const T& t : *tiles) doc_cost[size_t(t.doc)] += t.cost;
  std::stable_sort(tiles->begin(), tiles->end(), [&](const T& a, const T& b) {
    const int64_t ca = doc_cost[size_t(a.doc)], cb = doc_cost[size_t(b.doc)];
    if (ca != cb) return ca > cb;
    if (a.doc != b.doc) return a.doc < b.doc;
    return a.cost > b.cost;
  });
}

}  // namespace

int load_problem(const bdattn_problem* p, Problem* out, std::string* msg) {
  if (!p) {
    *msg = "problem descriptor is NULL";
    return BDATTN_ERR_INVALID_ARG;
  }
  if (p->dtype != BDATTN_F32 && p->dtype != BDATTN_BF16) {
    *msg = "unknown dtype";
    return BDATTN_ERR_INVALID_ARG;
  }
  if (p->clean_mask != BDATTN_CLEAN_BLOCK_CAUSAL && p->clean_mask != BDATTN_CLEAN_TOKEN_CAUSAL) {
    *msg = "unknown clean_mask";
    return BDATTN_ERR_INVALID_ARG;
  }
  if ((p->partial != 0 && p->partial != 1) || (p->omit_corr_keys != 0 && p->omit_corr_keys != 1)) {
    *msg = "partial and omit_corr_keys must be 0 or 1";
    return BDATTN_ERR_INVALID_ARG;
  }
  if (p->omit_corr_keys && !p->partial) {
    *msg = "only a partial problem may omit the corrupted keys";
    return BDATTN_ERR_INVALID_ARG;
  }
  if (p->precision < BDATTN_PRECISION_DEFAULT || p->precision > BDATTN_PRECISION_SPLIT) {
    *msg = "unknown precision";
    return BDATTN_ERR_INVALID_ARG;
  }
  if (p->B < 1 || p->H < 1 || p->Hkv < 1) {
    *msg = "B, H and Hkv must be >= 1";
    return BDATTN_ERR_SHAPE;
  }
  if (p->H % p->Hkv) {
    *msg = "H must be a multiple of Hkv";
    return BDATTN_ERR_SHAPE;
  }
  if (p->d != 32 && p->d != 128) {
    *msg = "head dim must be 32 or 128";
    return BDATTN_ERR_UNSUPPORTED;
  }
  if (p->n_clean_q < 0 || p->clean_q_start < 0 || p->n_clean_kv < 0 || p->clean_kv_start < 0 ||
      p->n_corr_blocks < 0) {
    *msg = "negative size or offset";
    return BDATTN_ERR_SHAPE;
  }
  const int64_t B = p->B;
  if (p->n_clean_q % B || p->clean_q_start % B || p->n_clean_kv % B) {
    *msg = "n_clean_q, clean_q_start and n_clean_kv must be multiples of B";
    return BDATTN_ERR_SHAPE;
  }
  if (p->partial && p->clean_kv_start % B) {
    *msg = "clean_kv_start must be a multiple of B";
    return BDATTN_ERR_SHAPE;
  }
  if (p->clean_q_start + p->n_clean_q > kMax32 || p->n_clean_kv > kMax32 ||
      p->n_corr_blocks * B > kMax32 || p->clean_kv_start + p->n_clean_kv > kMax32) {
    *msg = "sizes must stay below 2^31 rows";
    return BDATTN_ERR_SHAPE;
  }
  Problem P;
  P.B = p->B;
  P.H = p->H;
  P.Hkv = p->Hkv;
  P.d = p->d;
  P.dtype = p->dtype;
  P.token_causal = p->clean_mask == BDATTN_CLEAN_TOKEN_CAUSAL ? 1 : 0;
  P.clean_kv_start = int32_t(p->clean_kv_start);
  P.partial = p->partial;
  P.precision = p->dtype == BDATTN_BF16 ? p->precision : BDATTN_PRECISION_DEFAULT;
  P.corr_keys = p->omit_corr_keys ? 0 : 1;
  P.scale = p->scale > 0.f ? p->scale : float(1.0 / sqrt(double(p->d)));
  P.n_clean_q = int32_t(p->n_clean_q);
  P.clean_q_start = int32_t(p->clean_q_start);
  P.n_clean_kv = int32_t(p->n_clean_kv);
  P.n_corr_blocks = int32_t(p->n_corr_blocks);
  P.ids.resize(P.n_corr_blocks);
  if (p->corr_block_ids) {
    for (int32_t i = 0; i < P.n_corr_blocks; ++i) {
      int32_t v = p->corr_block_ids[i];
      if (v < 0 || (i > 0 && v < P.ids[i - 1])) {
        *msg = "corr_block_ids must be >= 0 and non-decreasing";
        return BDATTN_ERR_INVALID_ARG;
      }
      if (int64_t(v) * B > kMax32) {
        *msg = "corrupted block id beyond 2^31 positions";
        return BDATTN_ERR_SHAPE;
      }
      P.ids[i] = v;
    }
  } else {
    std::iota(P.ids.begin(), P.ids.end(), 0);
  }
  if (p->n_docs < 0 || (p->n_docs > 0 && !p->doc_starts)) {
    *msg = "n_docs must be >= 0, with doc_starts given when > 0";
    return BDATTN_ERR_INVALID_ARG;
  }
  for (int32_t i = 0; i < p->n_docs; ++i) {
    const int32_t v = p->doc_starts[i];
    if ((i == 0 && v != 0) || (i > 0 && v <= P.docs.back())) {
      *msg = "doc_starts must start at 0 and increase";
      return BDATTN_ERR_INVALID_ARG;
    }
    if (v % P.B) {
      *msg = "doc_starts must be multiples of B";
      return BDATTN_ERR_SHAPE;
    }
    P.docs.push_back(v);
  }
  if (P.docs.size() > 1) build_spans(&P);
  else P.docs.clear();
  if (p->kv_chunk_len < 0) {
    *msg = "kv_chunk_len must be >= 0";
    return BDATTN_ERR_SHAPE;
  }
  if (p->kv_chunk_len > 0) {  // a gathered clean buffer: chunks at their positions
    const int64_t C = p->kv_chunk_len;
    if (C % 128 || C % B || P.n_clean_kv % C) {
      *msg = "kv_chunk_len must be a multiple of 128 and of B that divides n_clean_kv";
      return BDATTN_ERR_SHAPE;
    }
    const int64_t n = P.n_clean_kv / C;
    if (n > 0 && !p->kv_chunk_pos) {
      *msg = "kv_chunk_pos is NULL";
      return BDATTN_ERR_INVALID_ARG;
    }
    // chunk c of the position range [clean_kv_start, +n_clean_kv) -> buffer chunk
    std::vector<int32_t> at(size_t(n), -1);
    for (int64_t i = 0; i < n; ++i) {
      const int64_t rel = int64_t(p->kv_chunk_pos[i]) - p->clean_kv_start;
      if (rel < 0 || rel % C || rel / C >= n || at[size_t(rel / C)] >= 0) {
        *msg = "the chunks of kv_chunk_pos must cover [clean_kv_start, clean_kv_start + "
               "n_clean_kv) exactly, each starting on a chunk boundary";
        return BDATTN_ERR_INVALID_ARG;
      }
      at[size_t(rel / C)] = int32_t(i);
    }
    const int32_t tpc = int32_t(C / FWD_TK);
    P.kv_map.resize(size_t(n) * tpc);
    for (int64_t c = 0; c < n; ++c)
      for (int32_t t = 0; t < tpc; ++t) P.kv_map[size_t(c * tpc + t)] = at[size_t(c)] * tpc + t;
  }
  if (P.partial) {  // any clean range: the attention over the keys present
    *out = std::move(P);
    return BDATTN_OK;
  }
  // Coverage: the buffer starts at position 0 and holds every clean key a
  // local query sees: the whole last block of the query shard, and the
  // prefix before the last local corrupted block.
  int64_t need = 0;
  if (P.n_clean_q > 0) need = int64_t(P.clean_q_start) + P.n_clean_q;
  if (P.n_corr_blocks > 0) need = std::max<int64_t>(need, int64_t(P.ids.back()) * B);
  if (p->clean_kv_start != 0 && (need > 0 || p->n_clean_kv > 0)) {
    *msg = "the clean K/V buffer must start at global position 0";
    return BDATTN_ERR_COVERAGE;
  }
  if (P.n_clean_kv < need) {
    *msg = "the clean K/V buffer misses clean keys a local query sees";
    return BDATTN_ERR_COVERAGE;
  }
  *out = std::move(P);
  return BDATTN_OK;
}

int fwd_heads_per_group(const Problem& P) {
  int G = P.G();
  if (G % 4 == 0) return 4;
  if (G % 2 == 0) return 2;
  return 1;
}

int fwd_rows_per_item(const Problem& P) {
  return FWD_WAVES * FWD_ROWS_PER_WAVE / fwd_heads_per_group(P);
}

size_t n_q_items(const Problem& P) {
  const int Gw = fwd_heads_per_group(P), R = fwd_rows_per_item(P);
  size_t tiles = size_t(ceil_div(P.n_clean_q, R)) + size_t(ceil_div(P.n_corr(), R));
  return tiles * size_t(P.H / Gw);
}

size_t n_kv_items(const Problem& P) {
  size_t tiles = size_t(ceil_div(P.n_clean_kv, BWD_TK)) +
                 (P.corr_keys ? size_t(ceil_div(P.n_corr(), BWD_TK)) : 0);
  return tiles * size_t(P.Hkv);
}

WsLayout workspace_layout(const Problem& P, int pass) {
  WsLayout w;
  size_t off = 0;
  w.claim = off;
  off = align_up(off + sizeof(int32_t) * kClaimCounters, WS_ALIGN);
  w.ids = off;
  off = align_up(off + sizeof(int32_t) * std::max<size_t>(1, P.ids.size()), WS_ALIGN);
  w.spans = off;
  off = align_up(off + sizeof(BdDocSpan) * P.spans.size(), WS_ALIGN);
  w.kv_map = off;
  off = align_up(off + sizeof(int32_t) * P.kv_map.size(), WS_ALIGN);
  w.q_items = off;
  w.q_items_bytes = n_q_items(P) * sizeof(FwdItem);
  off = align_up(off + std::max<size_t>(1, w.q_items_bytes), WS_ALIGN);
  if (pass == 1) {
    w.kv_items = off;
    w.kv_items_bytes = n_kv_items(P) * sizeof(BwdItem);
    off = align_up(off + std::max<size_t>(1, w.kv_items_bytes), WS_ALIGN);
  }
  w.staged = off;
  if (pass == 1) {
    const size_t rc = sizeof(float) * size_t(P.H) * row_pad(P.n_clean_q);
    const size_t rx = sizeof(float) * size_t(P.H) * row_pad(P.n_corr());
    w.d_c = off;
    off = align_up(off + rc, WS_ALIGN);
    w.l2_c = off;
    off = align_up(off + rc, WS_ALIGN);
    w.d_x = off;
    off = align_up(off + rx, WS_ALIGN);
    w.l2_x = off;
    off = align_up(off + rx, WS_ALIGN);
  }
  w.total = off;
  return w;
}

void build_plan(const Problem& P, Plan* plan) {
  plan->P = P;
  plan->Gw = fwd_heads_per_group(P);
  plan->fwd_rows = fwd_rows_per_item(P);
  plan->fwd.clear();
  plan->bwd.clear();
  plan->fwd_tiles = plan->fwd_masked_tiles = plan->bwd_qtiles = plan->bwd_masked_qtiles = 0;

  // ---------------- forward: (stream, row tile) sorted by key tiles, longest first
  {
    const int R = plan->fwd_rows;
    const int NHG = P.H / plan->Gw;
    struct T { int32_t tile, stream; int64_t cost, masked; int32_t doc; };
    std::vector<T> tiles;
    for (int s = 0; s < 2; ++s) {
      const int32_t n = s == 0 ? P.n_clean_q : P.n_corr();
      for (int32_t t = 0; t * int64_t(R) < n; ++t) {
        const int32_t r0 = t * R, r1 = std::min<int32_t>(n, r0 + R);
        BdRowBounds first = row_bounds(P, s, r0), last = row_bounds(P, s, r1 - 1);
        // clean key tiles [j0, nct) are swept; [jf0, jf1) need no mask (the
        // kernels' split of the same bounds)
        const int32_t j0 = first.clo / FWD_TK;
        const int32_t nct = last.cb <= first.clo ? j0 : ceil_div(last.cb, FWD_TK);
        const int32_t jf0 = std::min(nct, std::max(j0, ceil_div(last.clo, FWD_TK)));
        const int32_t jf1 = std::max(jf0, std::min(nct, first.cb / FWD_TK));
        int64_t cost = nct - j0, masked = (jf0 - j0) + (nct - jf1);
        if (s == 1) {
          const int32_t nxt = ceil_div(last.xhi - first.xlo, FWD_TK);
          cost += nxt;
          masked += nxt;
        }
        int32_t doc = 0;  // index of the document of the tile's first row
        if (!P.spans.empty()) {
          const int32_t lo = P.spans[size_t(s == 0 ? (P.clean_q_start + r0) / P.B : P.ids[r0 / P.B])].lo;
          doc = int32_t(std::lower_bound(P.docs.begin(), P.docs.end(), lo) - P.docs.begin());
        }
        tiles.push_back({t, s, cost, masked, doc});
      }
    }
    order_items(&tiles, P.spans.empty() ? 0 : P.docs.size());
    plan->fwd.reserve(tiles.size() * NHG);
    // consecutive workgroup ids land on different XCDs; keep one head group
    // per id residue so an XCD's L2 sees one KV head's prefix
    for (const T& t : tiles) {
      for (int hg = 0; hg < NHG; ++hg) plan->fwd.push_back({t.tile, (hg << 1) | t.stream});
      plan->fwd_tiles += t.cost * NHG;
      plan->fwd_masked_tiles += t.masked * NHG;
    }
  }

  // ---------------- backward: key tiles sorted by query rows swept, longest first
  {
    const int G = P.G();
    const int32_t nx = P.n_corr();
    struct T { int32_t ktile, stream; BwdItem rows; int64_t cost, qt, masked; int32_t doc; };
    std::vector<T> tiles;
    auto qtiles = [](int32_t r0, int32_t r1) -> int64_t {
      if (r1 <= r0) return 0;
      return (r1 - 1) / BWD_TQ - r0 / BWD_TQ + 1;
    };
    for (int32_t kt = 0; kt * int64_t(BWD_TK) < P.n_clean_kv; ++kt) {
      const int32_t k0 = kt * BWD_TK, k1 = std::min<int32_t>(P.n_clean_kv, k0 + BWD_TK);
      const int32_t g0 = P.clean_kv_start + k0;  // global position of the tile's first key
      const int32_t kb = g0 / P.B;
      // clean rows of blocks >= kb (token-causal: at positions >= g0);
      // corrupted rows of blocks with id > kb
      const int32_t first_row_pos = P.token_causal ? g0 : kb * P.B;
      int32_t c0 = std::min<int32_t>(P.n_clean_q, std::max<int32_t>(0, first_row_pos - P.clean_q_start));
      int32_t j = int32_t(std::upper_bound(P.ids.begin(), P.ids.end(), kb) - P.ids.begin());
      int32_t x0 = j * P.B;
      // packed documents: no row after the end of the last key's document
      // sees the tile
      int32_t c1 = P.n_clean_q, x1 = nx;
      bool one_doc = true;
      if (!P.spans.empty()) {
        const BdDocSpan& first = P.spans[size_t(g0 / P.B)];
        const BdDocSpan& last = P.spans[size_t((P.clean_kv_start + k1 - 1) / P.B)];
        c1 = int32_t(std::min<int64_t>(P.n_clean_q,
                                       std::max<int64_t>(0, int64_t(last.hi) - P.clean_q_start)));
        c1 = std::max(c0, c1);
        x1 = std::max(x0, last.xhi);
        one_doc = first.hi == last.hi;
      }
      // a q tile needs the mask unless it lies inside the swept rows and its
      // first row sees the whole key tile (row bounds are nondecreasing, so
      // the unmasked tiles are the top ones of each stream); with documents,
      // only when every key of the tile is in one document, and below the
      // last tile boundary before that document's end unless the document
      // ends with the stream (rows past a stream's end contribute nothing)
      int32_t cfe = !one_doc ? c0 : (c1 == P.n_clean_q ? c1 : c1 / BWD_TQ * BWD_TQ);
      int32_t xfe = !one_doc ? x0 : (x1 == nx ? x1 : x1 / BWD_TQ * BWD_TQ);
      int64_t qt = qtiles(c0, c1) + qtiles(x0, x1), masked = qt;
      int32_t cf = cfe, xf = xfe;
      for (int32_t r = c0 / BWD_TQ * BWD_TQ; r + BWD_TQ <= cfe || (r < cfe && cfe == P.n_clean_q);
           r += BWD_TQ) {
        if (r >= c0 && row_bounds(P, 0, r).cb >= k1 && k1 - k0 == BWD_TK) {
          cf = r;
          masked -= qtiles(cf, cfe);
          break;
        }
      }
      for (int32_t r = x0 / BWD_TQ * BWD_TQ; r + BWD_TQ <= xfe || (r < xfe && xfe == nx);
           r += BWD_TQ) {
        if (r >= x0 && row_bounds(P, 1, r).cb >= k1 && k1 - k0 == BWD_TK) {
          xf = r;
          masked -= qtiles(xf, xfe);
          break;
        }
      }
      if (cf >= cfe) cf = cfe = c1;  // no unmasked tile: the kernel reads [c1, c1)
      if (xf >= xfe) xf = xfe = x1;
      BwdItem it{kt, 0, c0, c1, x0, x1, cf, xf, cfe, xfe};
      tiles.push_back({kt, 0, it, (c1 - c0) + int64_t(x1 - x0), qt, masked, 0});
    }
    for (int32_t kt = 0; P.corr_keys && kt * int64_t(BWD_TK) < nx; ++kt) {
      const int32_t k0 = kt * BWD_TK, k1 = std::min<int32_t>(nx, k0 + BWD_TK);
      const int32_t x0 = k0 / P.B * P.B, x1 = std::min<int32_t>(nx, ceil_div(k1, P.B) * P.B);
      BwdItem it{kt, 1, 0, 0, x0, x1, 0, x1, 0, x1};
      const int64_t qt = qtiles(x0, x1);
      tiles.push_back({kt, 1, it, x1 - x0, qt, qt, 0});
    }
    order_items(&tiles, 0);
    plan->bwd.reserve(tiles.size() * P.Hkv);
    for (const T& t : tiles) {
      for (int g = 0; g < P.Hkv; ++g) {
        BwdItem it = t.rows;
        it.hs = (g << 1) | t.stream;
        plan->bwd.push_back(it);
      }
      plan->bwd_qtiles += t.qt * G * P.Hkv;
      plan->bwd_masked_qtiles += t.masked * G * P.Hkv;
    }
  }
}

int64_t visible_pairs(const Problem& P) {
  int64_t pairs = 0;
  for (int32_t r = 0; r < P.n_clean_q; ++r) {
    const BdRowBounds b = row_bounds(P, 0, r);
    pairs += b.cb - b.clo;
  }
  for (int32_t r = 0; r < P.n_corr(); ++r) {
    const BdRowBounds b = row_bounds(P, 1, r);
    pairs += int64_t(b.cb - b.clo) + (b.xhi - b.xlo);
  }
  return pairs;
}

void mask_render(const Problem& P, uint8_t* out) {
  const int64_t nq = int64_t(P.n_clean_q) + P.n_corr();
  const int64_t nk = int64_t(P.n_clean_kv) + P.n_corr();
  for (int64_t q = 0; q < nq; ++q) {
    const int stream = q < P.n_clean_q ? 0 : 1;
    const int32_t row = int32_t(stream == 0 ? q : q - P.n_clean_q);
    BdRowBounds b = row_bounds(P, stream, row);
    uint8_t* o = out + q * nk;
    // (a gathered buffer: the key at buffer row k sits at position-order index
    // map(k); rows follow the buffer)
    for (int32_t k = 0; k < P.n_clean_kv; ++k) {
      const int32_t kb = P.kv_map.empty() ? k : P.kv_map[k / FWD_TK] * FWD_TK + k % FWD_TK;
      o[kb] = bd_sees_clean(b, k) ? 1 : 0;
    }
    for (int32_t k = 0; k < P.n_corr(); ++k) o[P.n_clean_kv + k] = bd_sees_corr(b, k) ? 1 : 0;
  }
}

}  // namespace bdattn
