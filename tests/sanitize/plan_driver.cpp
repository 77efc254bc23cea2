// Host-only driver of the bdattn planner, built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_sanitize.py (test infrastructure).
//
// Reads one problem descriptor per line on stdin:
//   B H Hkv d dtype n_clean_q clean_q_start n_clean_kv clean_kv_start
//   n_corr_blocks clean_mask partial omit_corr_keys has_ids n_ids ids...
//   n_docs docs... kv_chunk_len n_chunks chunk_pos...
// and for each prints the validation status and, for a valid problem, the
// exact pair count, both workspace sizes, the planner statistics and, over
// the dense mask's visible entries (flat index i = row * n_keys + key), their
// count, the sum of i and the sum of i*i modulo 2^64, so that the test can
// compare them with the production library. It also checks every planned
// work item against the problem's row and tile ranges.
#include <stdio.h>
#include <stdlib.h>

#include <string>
#include <vector>

#include "plan.h"

namespace {

bool check_items(const bdattn::Plan& plan, std::string* why) {
  const bdattn::Problem& P = plan.P;
  const int64_t n_rows[2] = {P.n_clean_q, P.n_corr()};
  for (const bdattn::FwdItem& it : plan.fwd) {
    const int s = it.hs & 1, hg = it.hs >> 1;
    if (it.tile < 0 || int64_t(it.tile) * plan.fwd_rows >= n_rows[s] || hg < 0 ||
        hg >= P.H / plan.Gw) {
      *why = "forward item out of range";
      return false;
    }
  }
  const int64_t n_keys[2] = {P.n_clean_kv, P.n_corr()};
  for (const bdattn::BwdItem& it : plan.bwd) {
    const int s = it.hs & 1, g = it.hs >> 1;
    if (it.ktile < 0 || int64_t(it.ktile) * bdattn::BWD_TK >= n_keys[s] || g < 0 || g >= P.Hkv) {
      *why = "backward item out of range";
      return false;
    }
    if (it.c0 < 0 || it.c0 > it.c1 || it.c1 > P.n_clean_q || it.x0 < 0 || it.x0 > it.x1 ||
        it.x1 > P.n_corr() || it.cf > it.cfe || it.xf > it.xfe || it.cfe > P.n_clean_q ||
        it.xfe > P.n_corr()) {
      *why = "backward item rows out of range";
      return false;
    }
  }
  return true;
}

}  // namespace

int main() {
  char line[1 << 16];
  while (fgets(line, sizeof line, stdin)) {
    std::vector<long long> v;
    char* p = line;
    char* end = nullptr;
    for (long long x = strtoll(p, &end, 10); end != p; x = strtoll(p, &end, 10)) {
      v.push_back(x);
      p = end;
    }
    if (v.size() < 16) continue;
    bdattn_problem d = {};
    size_t i = 0;
    d.B = int32_t(v[i++]);
    d.H = int32_t(v[i++]);
    d.Hkv = int32_t(v[i++]);
    d.d = int32_t(v[i++]);
    d.dtype = int32_t(v[i++]);
    d.scale = 0.f;
    d.n_clean_q = v[i++];
    d.clean_q_start = v[i++];
    d.n_clean_kv = v[i++];
    d.clean_kv_start = v[i++];
    d.n_corr_blocks = v[i++];
    d.clean_mask = int32_t(v[i++]);
    d.partial = int32_t(v[i++]);
    d.omit_corr_keys = int32_t(v[i++]);
    const bool has_ids = v[i++] != 0;
    const size_t n_ids = size_t(v[i++]);
    std::vector<int32_t> ids(n_ids);
    for (size_t k = 0; k < n_ids; ++k) ids[k] = int32_t(v[i++]);
    const size_t n_docs = size_t(v[i++]);
    std::vector<int32_t> docs(n_docs);
    for (size_t k = 0; k < n_docs; ++k) docs[k] = int32_t(v[i++]);
    d.kv_chunk_len = i < v.size() ? int32_t(v[i++]) : 0;
    const size_t n_cp = i < v.size() ? size_t(v[i++]) : 0;
    std::vector<int32_t> cpos(n_cp);
    for (size_t k = 0; k < n_cp && i < v.size(); ++k) cpos[k] = int32_t(v[i++]);
    d.kv_chunk_pos = n_cp ? cpos.data() : nullptr;
    d.corr_block_ids = has_ids ? ids.data() : nullptr;
    d.n_docs = int32_t(n_docs);
    d.doc_starts = n_docs ? docs.data() : nullptr;

    bdattn::Problem P;
    std::string msg;
    const int st = bdattn::load_problem(&d, &P, &msg);
    if (st != BDATTN_OK) {
      printf("%d\n", st);
      continue;
    }
    bdattn::Plan plan;
    bdattn::build_plan(P, &plan);
    std::string why;
    if (!check_items(plan, &why)) {
      printf("ITEM %s\n", why.c_str());
      return 3;
    }
    const int64_t nq = int64_t(P.n_clean_q) + P.n_corr(), nk = int64_t(P.n_clean_kv) + P.n_corr();
    std::vector<uint8_t> mask(size_t(nq * nk));
    bdattn::mask_render(P, mask.data());
    uint64_t ones = 0, s1 = 0, s2 = 0;
    for (size_t k = 0; k < mask.size(); ++k) {
      if (!mask[k]) continue;
      ones += 1;
      s1 += uint64_t(k);
      s2 += uint64_t(k) * uint64_t(k);
    }
    printf("0 %lld %zu %zu %zu %lld %lld %zu %lld %lld %d %d %llu %llu %llu\n",
           (long long)bdattn::visible_pairs(P), bdattn::workspace_layout(P, 0).total,
           bdattn::workspace_layout(P, 1).total, plan.fwd.size(), (long long)plan.fwd_tiles,
           (long long)plan.fwd_masked_tiles, plan.bwd.size(), (long long)plan.bwd_qtiles,
           (long long)plan.bwd_masked_qtiles, plan.fwd_rows, bdattn::BWD_TK,
           (unsigned long long)ones, (unsigned long long)s1, (unsigned long long)s2);
  }
  return 0;
}
