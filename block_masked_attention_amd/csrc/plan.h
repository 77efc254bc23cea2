// Host planner: problem validation, exact pair counts, and the work lists the
// kernels consume. No HIP calls here, so it builds with any host compiler.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/bdattn.h"
#include "bdattn_mask.h"

namespace bdattn {

// Forward and backward dQ: a workgroup of FWD_WAVES waves covers
// FWD_ROWS_PER_WAVE query rows per wave and sweeps the visible keys in tiles
// of FWD_TK.
#ifndef BDATTN_FWD_WAVES
#define BDATTN_FWD_WAVES 8
#endif
constexpr int FWD_WAVES = BDATTN_FWD_WAVES;
// Waves of the forward that copy its key tiles: with 8 waves, the older wave
// of each SIMD (waves w and w + 4 share one), which runs ahead of its partner;
// with 4 (one per SIMD), all of them
#ifndef BDATTN_FWD_COPY_WAVES
#define BDATTN_FWD_COPY_WAVES (BDATTN_FWD_WAVES == 8 ? 4 : BDATTN_FWD_WAVES)
#endif
constexpr int FWD_COPY_WAVES = BDATTN_FWD_COPY_WAVES;
constexpr int FWD_ROWS_PER_WAVE = 32;
constexpr int FWD_TK = 64;
// Backward dK/dV: a workgroup owns BWD_TK keys of one KV head, 32 per SIMD
// (two waves of 64 lanes each in the split kernel), and sweeps the query rows
// that see them in tiles of BWD_TQ.
#ifndef BDATTN_BWD_TQ
#define BDATTN_BWD_TQ 64
#endif
constexpr int BWD_TK = 128;
constexpr int BWD_TQ = BDATTN_BWD_TQ;

constexpr size_t WS_ALIGN = 256;

// Work claiming (the forward, dQ and dK/dV kernels). A work list, sorted
// longest first, is dealt over kClaimQueues queues: queue x holds items x,
// x + 8, x + 16, ... The hardware places workgroup i on XCD i mod 8, and that
// workgroup first claims from queue i mod 8, so while every XCD keeps pace
// each runs the items of the static deal. XCDs do not run at one speed, so
// the grid has claim_extra(n) workgroups beyond the n items: an XCD that has
// emptied its queue takes the next items of another, and workgroups that
// find every queue empty end at once. The counters (one per queue) sit in
// the workspace's uploaded head and so restart at zero with every launch.
constexpr int kClaimQueues = 8;
constexpr int kClaimCounters = 3 * kClaimQueues;  // forward or dQ, dK/dV, spare
BD_HD int32_t claim_extra(int32_t n) { return kClaimQueues * ((n + 31) / 32); }  // n / 4, rounded up

// One claim: the next item of the first queue, from `home` on, that still
// holds one, or -1 when every queue is empty. load(y) reads counter y (an
// older value is harmless: the counters only grow, so it can only cost an
// extra fetch_add); fetch_add(y) adds 1 to counter y and returns its old
// value. Each item is returned exactly once over all claims: queue y's items
// go to the fetch_adds that return 0 .. len - 1, and a claim gives up only
// after seeing every queue at or past its length. (A negative counter, which
// only a clobbered workspace can hold, yields no item.)
template <class Load, class FetchAdd>
BD_HD int32_t claim_next(int home, int32_t n, Load load, FetchAdd fetch_add) {
  for (int v = 0; v < kClaimQueues; ++v) {
    const int y = (home + v) % kClaimQueues;
    const int32_t len = n > y ? (n - y + kClaimQueues - 1) / kClaimQueues : 0;
    if (v && load(y) >= len) continue;
    const int32_t c = fetch_add(y);
    if (c >= 0 && c < len) return y + kClaimQueues * c;
  }
  return -1;
}

// One forward work item: `tile` of `rows` query rows (stream bit 0 of hs),
// head group hs >> 1 (Gw consecutive q heads).
struct FwdItem {
  int32_t tile;
  int32_t hs;
};

// One backward work item: key tile `ktile` of the key stream (bit 0 of hs) of
// KV head hs >> 1; sweeps clean query rows [c0, c1) and corrupted rows
// [x0, x1). Query tiles (BWD_TQ rows, aligned) inside [cf, cfe) (clean) /
// [xf, xfe) (corrupted) see every key of the tile and skip the mask; the end
// is c1 / x1, or with packed documents the last tile boundary below it (the
// top tile then holds rows of a later document and keeps the mask). cf = cfe
// / xf = xfe when no tile skips it.
struct BwdItem {
  int32_t ktile;
  int32_t hs;
  int32_t c0, c1, x0, x1;
  int32_t cf, xf, cfe, xfe;
};

struct Problem {
  int32_t B, H, Hkv, d, dtype;
  int32_t token_causal = 0;  // clean_mask == BDATTN_CLEAN_TOKEN_CAUSAL
  int32_t clean_kv_start = 0;  // global position of clean buffer row 0 (partial problems)
  int32_t partial = 0;         // attention over the keys present only
  int32_t corr_keys = 1;       // the local corrupted keys are present
  int32_t precision = 0;       // bdattn_precision (bf16 inputs; not part of the plan)
  float scale;  // resolved (> 0)
  int32_t n_clean_q, clean_q_start, n_clean_kv, n_corr_blocks;
  std::vector<int32_t> ids;  // always materialised (0..n-1 when NULL)
  std::vector<int32_t> docs;  // packed document starts (empty: one document)
  std::vector<BdDocSpan> spans;  // per global block, with documents (else empty)
  // gathered clean K/V buffer: buffer tile (FWD_TK keys) of each clean key
  // tile in position order (empty: the buffer is in position order)
  std::vector<int32_t> kv_map;
  int32_t n_corr() const { return n_corr_blocks * B; }
  int32_t G() const { return H / Hkv; }
};

// Validate and copy a descriptor. Returns a bdattn_status; `msg` explains.
int load_problem(const bdattn_problem* p, Problem* out, std::string* msg);

// Heads per forward workgroup: the largest of 4, 2, 1 dividing H/Hkv.
int fwd_heads_per_group(const Problem& P);
int fwd_rows_per_item(const Problem& P);

struct Plan {
  Problem P;
  int Gw = 1;        // q heads per forward workgroup
  int fwd_rows = 0;  // query rows per forward workgroup
  std::vector<FwdItem> fwd;
  std::vector<BwdItem> bwd;
  // statistics
  int64_t fwd_tiles = 0, fwd_masked_tiles = 0, bwd_qtiles = 0, bwd_masked_qtiles = 0;
};

void build_plan(const Problem& P, Plan* plan);

// Workspace layout (byte offsets from the workspace start). Forward: the
// corrupted block ids and the query-tile work list. Backward: the ids, the
// query-tile list (dQ kernel), the key-tile list (dK/dV kernel) and
// -D = -rowsum(dO * O) of each stream.
// The backward's per-row data of each stream, -D = -rowsum(dO * O) and
// LSE * log2(e), are float [H][round_up(n, BWD_TQ)]: every query tile's
// values are one contiguous run, and rows past n hold -D = 0, LSE = +inf.
struct WsLayout {
  size_t claim = 0;  // kClaimCounters int32 work-claim counters (zero when uploaded)
  size_t ids = 0, spans = 0, kv_map = 0, q_items = 0, q_items_bytes = 0, kv_items = 0,
         kv_items_bytes = 0;
  size_t d_c = 0, d_x = 0, l2_c = 0, l2_x = 0;  // bwd row data
  size_t staged = 0;  // bytes copied from the host (ids and work lists)
  size_t total = 0;
};
BD_HD int32_t row_pad(int32_t n) { return (n + BWD_TQ - 1) / BWD_TQ * BWD_TQ; }
WsLayout workspace_layout(const Problem& P, int pass);
size_t n_q_items(const Problem& P);
size_t n_kv_items(const Problem& P);

int64_t visible_pairs(const Problem& P);
void mask_render(const Problem& P, uint8_t* out);

}  // namespace bdattn
