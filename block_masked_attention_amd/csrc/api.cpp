// C ABI of bdattn (include/bdattn.h): validation, plan cache, workspace upload
// and kernel launches.
#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>

#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/bdattn.h"
#include "launch.h"
#include "plan.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const std::string& msg) {
  g_last_error = msg;
  return status;
}

// One cached plan per distinct problem (ids included), kept for the life of
// the process: the work list and the ids are staged once into pinned host
// memory, from which every call copies them asynchronously into the caller's
// workspace. Entries are never freed, so a copy still in flight always reads
// live memory.
struct Entry {
  bdattn::Plan plan;
  std::mutex mu;
  void* staged[2] = {nullptr, nullptr};
  size_t staged_bytes[2] = {0, 0};
};

struct PlanCache {
  std::mutex mu;
  std::map<std::string, Entry*> entries;
};

PlanCache& cache() {
  static PlanCache* c = new PlanCache;  // never destroyed (outlives the HIP runtime)
  return *c;
}

std::string plan_key(const bdattn::Problem& P) {
  std::string k;
  const int32_t head[] = {P.B, P.H, P.Hkv, P.d, P.dtype, P.n_clean_q, P.clean_q_start,
                          P.n_clean_kv, P.n_corr_blocks, P.token_causal, P.clean_kv_start,
                          P.partial, P.corr_keys};
  k.append((const char*)head, sizeof(head));
  k.append((const char*)P.ids.data(), P.ids.size() * sizeof(int32_t));
  const int32_t nd = int32_t(P.docs.size());
  k.append((const char*)&nd, sizeof(nd));
  k.append((const char*)P.docs.data(), P.docs.size() * sizeof(int32_t));
  return k;
}

Entry* get_entry(const bdattn::Problem& P) {
  PlanCache& c = cache();
  const std::string key = plan_key(P);
  std::lock_guard<std::mutex> lock(c.mu);
  auto it = c.entries.find(key);
  if (it != c.entries.end()) return it->second;
  Entry* e = new Entry;
  bdattn::build_plan(P, &e->plan);
  c.entries[key] = e;
  return e;
}

int load(const bdattn_problem* p, bdattn::Problem* P) {
  std::string msg;
  int st = bdattn::load_problem(p, P, &msg);
  if (st != BDATTN_OK) return fail(st, msg);
  return BDATTN_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Every tensor of nonzero size needs a non-null 16-byte aligned pointer.
int check_ptr(const void* p, int64_t elems, const char* name) {
  if (elems == 0) return BDATTN_OK;
  if (!p) return fail(BDATTN_ERR_INVALID_ARG, std::string(name) + " is NULL");
  if (!aligned16(p)) return fail(BDATTN_ERR_INVALID_ARG, std::string(name) + " is not 16-byte aligned");
  return BDATTN_OK;
}

// Copy the corrupted block ids, the document table and the work lists (staged once in pinned host
// memory) into the workspace head, asynchronously on the caller's stream.
int upload(Entry* e, int pass, const bdattn::WsLayout& w, char* ws, hipStream_t s) {
  const size_t bytes = w.staged;
  void* src = nullptr;
  {
    std::lock_guard<std::mutex> lock(e->mu);
    if (!e->staged[pass]) {
      void* h = nullptr;
      hipError_t er = hipHostMalloc(&h, bytes, hipHostMallocDefault);
      if (er != hipSuccess) return fail(BDATTN_ERR_HIP, std::string("hipHostMalloc: ") + hipGetErrorString(er));
      memset(h, 0, bytes);
      const bdattn::Plan& plan = e->plan;
      memcpy((char*)h + w.ids, plan.P.ids.data(), plan.P.ids.size() * sizeof(int32_t));
      memcpy((char*)h + w.spans, plan.P.spans.data(), plan.P.spans.size() * sizeof(BdDocSpan));
      memcpy((char*)h + w.q_items, plan.fwd.data(), w.q_items_bytes);
      if (pass == 1) memcpy((char*)h + w.kv_items, plan.bwd.data(), w.kv_items_bytes);
      e->staged[pass] = h;
      e->staged_bytes[pass] = bytes;
    }
    src = e->staged[pass];
  }
  hipError_t er = hipMemcpyAsync(ws, src, bytes, hipMemcpyHostToDevice, s);
  if (er != hipSuccess) return fail(BDATTN_ERR_HIP, std::string("hipMemcpyAsync: ") + hipGetErrorString(er));
  return BDATTN_OK;
}

// Benchmark instrumentation: per-thread list of (kernel index, events)
// recorded by the launches while profiling is on. Kernel 0 = forward,
// 1 = backward dQ, 2 = backward dK/dV.
constexpr int kProfKernels = 3;
struct Prof {
  bool on = false;
  std::vector<std::pair<int, bdattn::KernelEvents>> recs;
};
thread_local Prof g_prof;

// Fills ev[0..n-1] with fresh events for kernels first..first+n-1; returns
// ev, or nullptr when profiling is off or an event cannot be created.
const bdattn::KernelEvents* prof_events(int first, int n, bdattn::KernelEvents* ev) {
  if (!g_prof.on) return nullptr;
  for (int i = 0; i < n; ++i) {
    bool ok = hipEventCreate(&ev[i].start) == hipSuccess;
    if (ok && hipEventCreate(&ev[i].stop) != hipSuccess) {
      (void)hipEventDestroy(ev[i].start);
      ok = false;
    }
    if (!ok) {
      for (int k = 0; k < i; ++k) {
        (void)hipEventDestroy(ev[k].start);
        (void)hipEventDestroy(ev[k].stop);
      }
      return nullptr;
    }
  }
  for (int i = 0; i < n; ++i) g_prof.recs.push_back({first + i, ev[i]});
  return ev;
}

}  // namespace

extern "C" {

int bdattn_profile_enable(int on) {
  g_prof.on = on != 0;
  return BDATTN_OK;
}

int bdattn_profile_read(double* ms, int64_t* launches) {
  double t[kProfKernels] = {0, 0, 0};
  int64_t n[kProfKernels] = {0, 0, 0};
  int st = BDATTN_OK;
  for (auto& r : g_prof.recs) {
    float x = 0.f;
    if (hipEventSynchronize(r.second.stop) == hipSuccess &&
        hipEventElapsedTime(&x, r.second.start, r.second.stop) == hipSuccess) {
      t[r.first] += x;
      n[r.first] += 1;
    } else {
      st = fail(BDATTN_ERR_HIP, "profile event wait failed");
    }
    (void)hipEventDestroy(r.second.start);
    (void)hipEventDestroy(r.second.stop);
  }
  g_prof.recs.clear();
  for (int k = 0; k < kProfKernels; ++k) {
    if (ms) ms[k] = t[k];
    if (launches) launches[k] = n[k];
  }
  return st;
}

int bdattn_version(void) { return BDATTN_VERSION; }

const char* bdattn_status_string(int status) {
  switch (status) {
    case BDATTN_OK: return "ok";
    case BDATTN_ERR_INVALID_ARG: return "invalid argument";
    case BDATTN_ERR_SHAPE: return "invalid shape";
    case BDATTN_ERR_UNSUPPORTED: return "unsupported head dim or dtype";
    case BDATTN_ERR_COVERAGE: return "clean K/V buffer does not cover the visible keys";
    case BDATTN_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    case BDATTN_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* bdattn_last_error(void) { return g_last_error.c_str(); }

int bdattn_validate(const bdattn_problem* p) {
  bdattn::Problem P;
  int st = load(p, &P);
  if (st != BDATTN_OK) return st;
  if (!bdattn::have_kernels(P.dtype, P.d))
    return fail(BDATTN_ERR_UNSUPPORTED, "no kernel for this dtype and head dim (fp32 needs d = 32)");
  return BDATTN_OK;
}

int bdattn_workspace_size(const bdattn_problem* p, int pass, size_t* bytes) {
  if (!bytes) return fail(BDATTN_ERR_INVALID_ARG, "bytes is NULL");
  if (pass != 0 && pass != 1) return fail(BDATTN_ERR_INVALID_ARG, "pass must be 0 or 1");
  bdattn::Problem P;
  int st = load(p, &P);
  if (st != BDATTN_OK) return st;
  *bytes = bdattn::workspace_layout(P, pass).total;
  return BDATTN_OK;
}

int bdattn_mask_render(const bdattn_problem* p, uint8_t* host_out, size_t cap) {
  bdattn::Problem P;
  int st = load(p, &P);
  if (st != BDATTN_OK) return st;
  const size_t nq = size_t(P.n_clean_q) + P.n_corr();
  const size_t nk = size_t(P.n_clean_kv) + P.n_corr();
  if (!host_out || cap < nq * nk) return fail(BDATTN_ERR_INVALID_ARG, "output buffer too small");
  bdattn::mask_render(P, host_out);
  return BDATTN_OK;
}

int bdattn_visible_pairs(const bdattn_problem* p, int64_t* pairs) {
  if (!pairs) return fail(BDATTN_ERR_INVALID_ARG, "pairs is NULL");
  bdattn::Problem P;
  int st = load(p, &P);
  if (st != BDATTN_OK) return st;
  *pairs = bdattn::visible_pairs(P);
  return BDATTN_OK;
}

int bdattn_plan_stats(const bdattn_problem* p, int64_t out[8]) {
  if (!out) return fail(BDATTN_ERR_INVALID_ARG, "out is NULL");
  bdattn::Problem P;
  int st = load(p, &P);
  if (st != BDATTN_OK) return st;
  const bdattn::Plan* plan = &get_entry(P)->plan;
  out[0] = int64_t(plan->fwd.size());
  out[1] = plan->fwd_tiles;
  out[2] = plan->fwd_masked_tiles;
  out[3] = int64_t(plan->bwd.size());
  out[4] = plan->bwd_qtiles;
  out[5] = plan->bwd_masked_qtiles;
  out[6] = plan->fwd_rows;
  out[7] = bdattn::BWD_TK;
  return BDATTN_OK;
}

int bdattn_fwd(const bdattn_problem* p, const void* q_c, const void* k_c, const void* v_c,
               const void* q_x, const void* k_x, const void* v_x, void* o_c, void* o_x,
               float* lse_c, float* lse_x, void* workspace, size_t ws_bytes, void* hip_stream) {
  bdattn::Problem P;
  int st = bdattn_validate(p);
  if (st != BDATTN_OK) return st;
  load(p, &P);
  const int64_t nqc = int64_t(P.n_clean_q) * P.H * P.d, nqx = int64_t(P.n_corr()) * P.H * P.d;
  const int64_t nkc = int64_t(P.n_clean_kv) * P.Hkv * P.d, nkx = int64_t(P.n_corr()) * P.Hkv * P.d;
  if ((st = check_ptr(q_c, nqc, "q_c")) || (st = check_ptr(k_c, nkc, "k_c")) ||
      (st = check_ptr(v_c, nkc, "v_c")) || (st = check_ptr(q_x, nqx, "q_x")) ||
      (st = check_ptr(k_x, nkx, "k_x")) || (st = check_ptr(v_x, nkx, "v_x")) ||
      (st = check_ptr(o_c, nqc, "o_c")) || (st = check_ptr(o_x, nqx, "o_x")) ||
      (st = check_ptr(lse_c, nqc, "lse_c")) || (st = check_ptr(lse_x, nqx, "lse_x")))
    return st;
  Entry* entry = get_entry(P);
  const bdattn::Plan* plan = &entry->plan;
  const bdattn::WsLayout w = bdattn::workspace_layout(P, 0);
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) % bdattn::WS_ALIGN) || ws_bytes < w.total)
    return fail(BDATTN_ERR_WORKSPACE, "forward workspace missing, misaligned or smaller than " +
                                          std::to_string(w.total) + " bytes");
  hipStream_t s = (hipStream_t)hip_stream;
  char* ws = (char*)workspace;
  if ((st = upload(entry, 0, w, ws, s))) return st;
  bdattn::FwdArgs a;
  a.q_c = q_c; a.k_c = k_c; a.v_c = v_c; a.q_x = q_x; a.k_x = k_x; a.v_x = v_x;
  a.o_c = o_c; a.o_x = o_x; a.lse_c = lse_c; a.lse_x = lse_x;
  a.ids = (const int32_t*)(ws + w.ids);
  a.docs = P.spans.empty() ? nullptr : (const BdDocSpan*)(ws + w.spans);
  a.items = (const bdattn::FwdItem*)(ws + w.q_items);
  a.n_items = int32_t(plan->fwd.size());
  a.B = P.B; a.H = P.H; a.Hkv = P.Hkv; a.Gw = plan->Gw; a.rows_per_item = plan->fwd_rows;
  a.n_clean_q = P.n_clean_q; a.clean_q_start = P.clean_q_start; a.n_clean_kv = P.n_clean_kv;
  a.n_corr = P.n_corr();
  a.token_causal = P.token_causal;
  a.clean_kv_start = P.clean_kv_start;
  a.corr_keys = P.corr_keys;
  a.scale_log2 = float(double(P.scale) * 1.4426950408889634);
  bdattn::KernelEvents ev[1];
  hipError_t e = bdattn::launch_fwd(a, P.dtype, P.d, s, prof_events(0, 1, ev));
  if (e != hipSuccess) return fail(BDATTN_ERR_HIP, std::string("forward launch: ") + hipGetErrorString(e));
  return BDATTN_OK;
}

int bdattn_bwd(const bdattn_problem* p, const void* q_c, const void* k_c, const void* v_c,
               const void* q_x, const void* k_x, const void* v_x, const void* o_c, const void* o_x,
               const float* lse_c, const float* lse_x, const void* do_c, const void* do_x, void* dq_c,
               void* dq_x, void* dk_c, void* dv_c, void* dk_x, void* dv_x, void* workspace,
               size_t ws_bytes, void* hip_stream) {
  bdattn::Problem P;
  int st = bdattn_validate(p);
  if (st != BDATTN_OK) return st;
  load(p, &P);
  const int64_t nqc = int64_t(P.n_clean_q) * P.H * P.d, nqx = int64_t(P.n_corr()) * P.H * P.d;
  const int64_t nkc = int64_t(P.n_clean_kv) * P.Hkv * P.d, nkx = int64_t(P.n_corr()) * P.Hkv * P.d;
  if ((st = check_ptr(q_c, nqc, "q_c")) || (st = check_ptr(k_c, nkc, "k_c")) ||
      (st = check_ptr(v_c, nkc, "v_c")) || (st = check_ptr(q_x, nqx, "q_x")) ||
      (st = check_ptr(k_x, nkx, "k_x")) || (st = check_ptr(v_x, nkx, "v_x")) ||
      (st = check_ptr(o_c, nqc, "o_c")) || (st = check_ptr(o_x, nqx, "o_x")) ||
      (st = check_ptr(lse_c, nqc, "lse_c")) || (st = check_ptr(lse_x, nqx, "lse_x")) ||
      (st = check_ptr(do_c, nqc, "do_c")) || (st = check_ptr(do_x, nqx, "do_x")) ||
      (st = check_ptr(dq_c, nqc, "dq_c")) || (st = check_ptr(dq_x, nqx, "dq_x")) ||
      (st = check_ptr(dk_c, nkc, "dk_c")) || (st = check_ptr(dv_c, nkc, "dv_c")) ||
      (st = check_ptr(dk_x, P.corr_keys ? nkx : 0, "dk_x")) ||
      (st = check_ptr(dv_x, P.corr_keys ? nkx : 0, "dv_x")))
    return st;
  Entry* entry = get_entry(P);
  const bdattn::Plan* plan = &entry->plan;
  const bdattn::WsLayout w = bdattn::workspace_layout(P, 1);
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) % bdattn::WS_ALIGN) || ws_bytes < w.total)
    return fail(BDATTN_ERR_WORKSPACE, "backward workspace missing, misaligned or smaller than " +
                                          std::to_string(w.total) + " bytes");
  hipStream_t s = (hipStream_t)hip_stream;
  char* ws = (char*)workspace;
  if ((st = upload(entry, 1, w, ws, s))) return st;
  bdattn::BwdArgs a;
  a.q_c = q_c; a.k_c = k_c; a.v_c = v_c; a.q_x = q_x; a.k_x = k_x; a.v_x = v_x;
  a.o_c = o_c; a.o_x = o_x; a.do_c = do_c; a.do_x = do_x; a.lse_c = lse_c; a.lse_x = lse_x;
  a.dq_c = dq_c; a.dq_x = dq_x; a.dk_c = dk_c; a.dv_c = dv_c; a.dk_x = dk_x; a.dv_x = dv_x;
  a.ids = (const int32_t*)(ws + w.ids);
  a.docs = P.spans.empty() ? nullptr : (const BdDocSpan*)(ws + w.spans);
  a.q_items = (const bdattn::FwdItem*)(ws + w.q_items);
  a.n_q_items = int32_t(plan->fwd.size());
  a.kv_items = (const bdattn::BwdItem*)(ws + w.kv_items);
  a.n_kv_items = int32_t(plan->bwd.size());
  a.d_c = (float*)(ws + w.d_c);
  a.d_x = (float*)(ws + w.d_x);
  a.l2_c = (float*)(ws + w.l2_c);
  a.l2_x = (float*)(ws + w.l2_x);
  a.B = P.B; a.H = P.H; a.Hkv = P.Hkv; a.Gw = plan->Gw; a.rows_per_item = plan->fwd_rows;
  a.n_clean_q = P.n_clean_q; a.clean_q_start = P.clean_q_start; a.n_clean_kv = P.n_clean_kv;
  a.n_corr = P.n_corr();
  a.token_causal = P.token_causal;
  a.clean_kv_start = P.clean_kv_start;
  a.corr_keys = P.corr_keys;
  a.scale = P.scale;
  a.scale_log2 = float(double(P.scale) * 1.4426950408889634);
  bdattn::KernelEvents ev[2];
  hipError_t e = bdattn::launch_bwd(a, P.dtype, P.d, s, prof_events(1, 2, ev));
  if (e != hipSuccess) return fail(BDATTN_ERR_HIP, std::string("backward launch: ") + hipGetErrorString(e));
  return BDATTN_OK;
}

int bdattn_merge(int64_t n_rows, int32_t H, int32_t d, int32_t dtype, const void* o_a,
                 const float* lse_a, const void* o_b, const float* lse_b, void* o, float* lse,
                 void* hip_stream) {
  if (dtype != BDATTN_F32 && dtype != BDATTN_BF16) return fail(BDATTN_ERR_INVALID_ARG, "unknown dtype");
  if (n_rows < 0 || H < 1) return fail(BDATTN_ERR_SHAPE, "n_rows must be >= 0 and H >= 1");
  if (!bdattn::have_kernels(dtype, d))
    return fail(BDATTN_ERR_UNSUPPORTED, "no merge kernel for this head dim and dtype");
  if (n_rows > (int64_t(1) << 40) / (int64_t(H) * d))
    return fail(BDATTN_ERR_SHAPE, "merge problem too large");
  const int64_t no = n_rows * H * d, nl = n_rows * H;
  int st;
  if ((st = check_ptr(o_a, no, "o_a")) || (st = check_ptr(o_b, no, "o_b")) ||
      (st = check_ptr(o, no, "o")) || (st = check_ptr(lse_a, nl, "lse_a")) ||
      (st = check_ptr(lse_b, nl, "lse_b")) || (st = check_ptr(lse, nl, "lse")))
    return st;
  hipError_t e = bdattn::launch_merge(n_rows, H, d, dtype, o_a, lse_a, o_b, lse_b, o, lse,
                                      (hipStream_t)hip_stream);
  if (e != hipSuccess) return fail(BDATTN_ERR_HIP, std::string("merge launch: ") + hipGetErrorString(e));
  return BDATTN_OK;
}

}  // extern "C"
