// C ABI of bdattn (include/bdattn.h): validation, plan cache, workspace upload
// and kernel launches.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <list>
#include <memory>
#include <mutex>
#include <string>
#include <unordered_map>
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

// Plan cache: one plan per distinct problem (ids and document starts
// included), least recently used first out, bounded by bytes (the plans' host
// memory plus their pinned staging buffers) and by entry count. A call copies
// its plan's work lists from a pinned staging buffer into the caller's
// workspace with an asynchronous copy on the caller's stream, and records an
// event after it. A staging buffer is reused or freed only once the event of
// its last copy has completed, so a copy still in flight always reads live,
// unchanged memory. Buffers of evicted plans go to a spare pool and are handed
// to new plans, so a stream of distinct problems (a new packed-document layout
// every training step) allocates pinned memory only while the pool is short.
struct Staged {
  void* ptr = nullptr;
  size_t cap = 0;
  hipEvent_t done = nullptr;     // recorded after the last copy from ptr
  hipStream_t stream = nullptr;  // the stream of that copy
  bool used = false;
};

void release_staged(Staged* st);

struct Entry {
  std::string key;
  bdattn::Plan plan;
  size_t host_bytes = 0;
  std::mutex mu;  // guards staged
  Staged staged[2];
  ~Entry() {
    for (Staged& st : staged) release_staged(&st);
  }
};

size_t plan_host_bytes(const bdattn::Plan& plan) {
  return sizeof(bdattn::Plan) + plan.fwd.capacity() * sizeof(bdattn::FwdItem) +
         plan.bwd.capacity() * sizeof(bdattn::BwdItem) +
         plan.P.ids.capacity() * sizeof(int32_t) + plan.P.docs.capacity() * sizeof(int32_t) +
         plan.P.spans.capacity() * sizeof(BdDocSpan);
}

constexpr size_t kDefaultBudget = size_t(256) << 20;
constexpr size_t kMaxEntries = 1024;

struct PlanCache {
  std::mutex mu;  // guards everything below except the spare pool
  std::list<std::shared_ptr<Entry>> lru;  // front: most recently used
  std::unordered_map<std::string, std::list<std::shared_ptr<Entry>>::iterator> index;
  size_t host_bytes = 0;
  size_t budget = kDefaultBudget;
  int64_t evictions = 0;
  std::mutex spare_mu;  // guards spare, spare_bytes, pinned_bytes
  std::vector<Staged> spare;  // staging buffers of evicted plans
  size_t spare_bytes = 0;
  size_t pinned_bytes = 0;  // every live staging buffer, in entries and spare
};

PlanCache& cache() {
  static PlanCache* c = new PlanCache;  // never destroyed (outlives the HIP runtime)
  return *c;
}

bool copy_done(const Staged& st) { return !st.used || hipEventQuery(st.done) != hipErrorNotReady; }

void free_staged(Staged* st) {
  if (st->done) (void)hipEventDestroy(st->done);
  if (st->ptr) (void)hipHostFree(st->ptr);
  *st = Staged();
}

// An evicted plan's staging buffer joins the spare pool. Completed spare
// buffers beyond a quarter of the budget are freed, oldest first.
void release_staged(Staged* st) {
  if (!st->ptr) return;
  PlanCache& c = cache();
  std::vector<Staged> drop;
  {
    std::lock_guard<std::mutex> lock(c.spare_mu);
    c.spare.push_back(*st);
    c.spare_bytes += st->cap;
    const size_t keep = c.budget / 4;
    for (size_t i = 0; i < c.spare.size() && c.spare_bytes > keep;) {
      if (copy_done(c.spare[i])) {
        c.spare_bytes -= c.spare[i].cap;
        c.pinned_bytes -= c.spare[i].cap;
        drop.push_back(c.spare[i]);
        c.spare.erase(c.spare.begin() + long(i));
      } else {
        ++i;
      }
    }
  }
  *st = Staged();
  for (Staged& d : drop) free_staged(&d);
}

// A staging buffer of at least `bytes`: a completed spare one that is not
// more than twice too large, else a new pinned allocation.
int take_staged(size_t bytes, Staged* out, std::string* msg) {
  PlanCache& c = cache();
  {
    std::lock_guard<std::mutex> lock(c.spare_mu);
    for (size_t i = 0; i < c.spare.size(); ++i) {
      Staged& st = c.spare[i];
      if (st.cap >= bytes && st.cap <= 2 * bytes + (size_t(64) << 10) && copy_done(st)) {
        *out = st;
        c.spare_bytes -= st.cap;
        c.spare.erase(c.spare.begin() + long(i));
        return BDATTN_OK;
      }
    }
  }
  Staged st;
  st.cap = std::max(bytes, size_t(64) << 10);
  hipError_t er = hipHostMalloc(&st.ptr, st.cap, hipHostMallocDefault);
  if (er != hipSuccess) {
    *msg = std::string("hipHostMalloc: ") + hipGetErrorString(er);
    return BDATTN_ERR_HIP;
  }
  er = hipEventCreateWithFlags(&st.done, hipEventDisableTiming);
  if (er != hipSuccess) {
    (void)hipHostFree(st.ptr);
    *msg = std::string("hipEventCreate: ") + hipGetErrorString(er);
    return BDATTN_ERR_HIP;
  }
  {
    std::lock_guard<std::mutex> lock(c.spare_mu);
    c.pinned_bytes += st.cap;
  }
  *out = st;
  return BDATTN_OK;
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
  const int32_t nm = int32_t(P.kv_map.size());
  k.append((const char*)&nm, sizeof(nm));
  k.append((const char*)P.kv_map.data(), P.kv_map.size() * sizeof(int32_t));
  return k;
}

// The plan of P, built on first use. The returned reference keeps the entry
// alive even if it is evicted meanwhile.
std::shared_ptr<Entry> get_entry(const bdattn::Problem& P) {
  PlanCache& c = cache();
  std::string key = plan_key(P);
  {
    std::lock_guard<std::mutex> lock(c.mu);
    auto it = c.index.find(key);
    if (it != c.index.end()) {
      c.lru.splice(c.lru.begin(), c.lru, it->second);
      return *it->second;
    }
  }
  auto e = std::make_shared<Entry>();
  bdattn::build_plan(P, &e->plan);  // outside the lock: planning may take milliseconds
  e->host_bytes = plan_host_bytes(e->plan);
  e->key = std::move(key);
  std::vector<std::shared_ptr<Entry>> evicted;  // released after the lock
  std::lock_guard<std::mutex> lock(c.mu);
  auto it = c.index.find(e->key);
  if (it != c.index.end()) {  // another thread built it meanwhile
    c.lru.splice(c.lru.begin(), c.lru, it->second);
    return *it->second;
  }
  c.lru.push_front(e);
  c.index[e->key] = c.lru.begin();
  c.host_bytes += e->host_bytes;
  // pinned bytes held by live plans; an evicted plan's buffers leave that
  // count when the plan is released (after the lock)
  size_t live_pinned;
  {
    std::lock_guard<std::mutex> l2(c.spare_mu);
    live_pinned = c.pinned_bytes - c.spare_bytes;
  }
  while (c.lru.size() > 1 &&
         (c.lru.size() > kMaxEntries || c.host_bytes + live_pinned > c.budget)) {
    std::shared_ptr<Entry> old = c.lru.back();
    c.lru.pop_back();
    c.index.erase(old->key);
    c.host_bytes -= old->host_bytes;
    {
      std::lock_guard<std::mutex> l3(old->mu);
      live_pinned -= std::min(live_pinned, old->staged[0].cap + old->staged[1].cap);
    }
    ++c.evictions;
    evicted.push_back(std::move(old));
  }
  return e;
}

}  // namespace

// The error channel of bdattn_last_error, for the library's other sources.
int bdattn::record_error(int status, const std::string& msg) { return fail(status, msg); }

namespace {

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

// Copy the corrupted block ids, the document table and the work lists
// (staged once per plan in pinned host memory) into the workspace head,
// asynchronously on the caller's stream, and record the copy's completion.
// A copy from the same buffer on another stream first waits for the previous
// copy, so the recorded event always covers every copy still reading it.
int upload(Entry* e, int pass, const bdattn::WsLayout& w, char* ws, hipStream_t s) {
  const size_t bytes = w.staged;
  std::lock_guard<std::mutex> lock(e->mu);
  Staged& st = e->staged[pass];
  if (!st.ptr) {
    std::string msg;
    int rc = take_staged(bytes, &st, &msg);
    if (rc != BDATTN_OK) return fail(rc, msg);
    char* h = (char*)st.ptr;
    memset(h, 0, bytes);
    const bdattn::Plan& plan = e->plan;
    memcpy(h + w.ids, plan.P.ids.data(), plan.P.ids.size() * sizeof(int32_t));
    memcpy(h + w.spans, plan.P.spans.data(), plan.P.spans.size() * sizeof(BdDocSpan));
    memcpy(h + w.kv_map, plan.P.kv_map.data(), plan.P.kv_map.size() * sizeof(int32_t));
    memcpy(h + w.q_items, plan.fwd.data(), w.q_items_bytes);
    if (pass == 1) memcpy(h + w.kv_items, plan.bwd.data(), w.kv_items_bytes);
  }
  hipError_t er = hipSuccess;
  if (st.used && st.stream != s && hipEventQuery(st.done) == hipErrorNotReady)
    er = hipStreamWaitEvent(s, st.done, 0);
  if (er == hipSuccess) er = hipMemcpyAsync(ws, st.ptr, bytes, hipMemcpyHostToDevice, s);
  if (er == hipSuccess) er = hipEventRecord(st.done, s);
  if (er != hipSuccess) return fail(BDATTN_ERR_HIP, std::string("workspace upload: ") + hipGetErrorString(er));
  st.used = true;
  st.stream = s;
  return BDATTN_OK;
}

// Benchmark instrumentation: per-thread list of (kernel index, events)
// recorded by the launches while profiling is on. Kernel 0 = forward,
// 1 = backward dQ, 2 = backward dK/dV.
constexpr int kProfKernels = bdattn::kProfiledKernels;
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

// Scratch of the allocation-free forward: one array per device, holding
// the block ids, the document table and the query-tile work list of the last
// such call on that device. In host code `scratch` names a host-side stand-in;
// the device address comes from hipGetSymbolAddress, once per device, with
// that device current.
constexpr size_t kScratchBytes = size_t(8) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_address(void** out) {
  int dev = -1;
  hipError_t er = hipGetDevice(&dev);
  if (er != hipSuccess) return fail(BDATTN_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(er));
  if (dev < 0 || dev >= kMaxDevices) return fail(BDATTN_ERR_HIP, "device index out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    er = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (er != hipSuccess || !ptr)
      return fail(BDATTN_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(er));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return BDATTN_OK;
}

// Work-list copy of the allocation-free forward: from the plan's host
// vectors (pageable memory, consumed before each copy call returns), so no
// pinned staging buffer is taken.
int upload_direct(const bdattn::Plan& plan, const bdattn::WsLayout& w, char* ws, hipStream_t s) {
  static const int32_t zeros[bdattn::kClaimCounters] = {};  // the work-claim counters
  struct Part { size_t off; const void* src; size_t bytes; };
  const Part parts[] = {{w.claim, zeros, sizeof(zeros)},
                        {w.ids, plan.P.ids.data(), plan.P.ids.size() * sizeof(int32_t)},
                        {w.spans, plan.P.spans.data(), plan.P.spans.size() * sizeof(BdDocSpan)},
                        {w.kv_map, plan.P.kv_map.data(), plan.P.kv_map.size() * sizeof(int32_t)},
                        {w.q_items, plan.fwd.data(), w.q_items_bytes}};
  for (const Part& pt : parts) {
    if (!pt.bytes) continue;
    hipError_t er = hipMemcpyAsync(ws + pt.off, pt.src, pt.bytes, hipMemcpyHostToDevice, s);
    if (er != hipSuccess) return fail(BDATTN_ERR_HIP, std::string("scratch upload: ") + hipGetErrorString(er));
  }
  return BDATTN_OK;
}

// Work claiming across the XCDs' queues (kClaimQueues in plan.h) for a list
// of n_items items that sweep `steps` tiles in all. It pays when the list is
// long (16 or more items per CU of the 256, so an XCD's last items can go to
// another) and its items are long enough (32 tiles or more on average) to
// hide the claim's atomic round trip, about 1.5 us; else workgroup i runs
// item i (the static deal). BDATTN_CLAIM=0 forces the static deal and
// BDATTN_CLAIM=1 forces claiming.
bool claim_on(size_t n_items, int64_t steps) {
  const char* e = getenv("BDATTN_CLAIM");
  if (e && !strcmp(e, "0")) return false;
  if (e && !strcmp(e, "1")) return true;
  return n_items >= 4096 && steps >= 32 * int64_t(n_items);
}

// Compute units of the current device (cached per device; 0 if unknown).
int cu_count() {
  static std::mutex mu;
  static int count[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  std::lock_guard<std::mutex> lock(mu);
  if (!count[dev] &&
      hipDeviceGetAttribute(&count[dev], hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    count[dev] = 0;
  return count[dev];
}

// Persistent grid for a query-tile list of n_items items that sweep `steps`
// tiles in all, when not claiming one item per workgroup: one workgroup per
// CU, each claiming item after item from the queues, pays when items are
// short (under 128 tiles on average, so that an item's start-up and the
// latency of its stores weigh) and there are more items than CUs. Returns
// the grid size, or 0. BDATTN_PERSIST=0 / 1 forces it off / on (on: whenever
// there are more items than CUs).
// The persistent query-tile kernels are built for bf16 at head dim 128, the
// default precision and a clean K/V buffer in position order.
bool persist_kernels(const bdattn::Problem& P) {
  return P.dtype == BDATTN_BF16 && P.d == 128 && P.precision == 0 && P.kv_map.empty();
}

int32_t persist_grid(size_t n_items, int64_t steps, bool claiming) {
  const char* e = getenv("BDATTN_PERSIST");
  if (claiming || (e && !strcmp(e, "0"))) return 0;
  const int cus = cu_count();
  if (cus <= 0 || n_items <= size_t(cus)) return 0;
  if (e && !strcmp(e, "1")) return cus;
  return steps < 128 * int64_t(n_items) ? cus : 0;
}

}  // namespace

const bdattn::KernelEvents* bdattn::profile_events(int first, int n, KernelEvents* ev) {
  return prof_events(first, n, ev);
}

extern "C" {

int bdattn_profile_enable(int on) {
  g_prof.on = on != 0;
  return BDATTN_OK;
}

int bdattn_profile_read(double* ms, int64_t* launches) {
  double t[kProfKernels] = {};
  int64_t n[kProfKernels] = {};
  int st = BDATTN_OK;
  if ((st = bdattn_profile_read_n(kProfKernels, t, n))) return st;
  for (int k = 0; k < 3; ++k) {
    if (ms) ms[k] = t[k];
    if (launches) launches[k] = n[k];
  }
  return BDATTN_OK;
}

int bdattn_profile_read_n(int count, double* ms, int64_t* launches) {
  if (count < 0 || count > kProfKernels)
    return fail(BDATTN_ERR_INVALID_ARG, "count must lie in [0, " + std::to_string(kProfKernels) + "]");
  double t[kProfKernels] = {};
  int64_t n[kProfKernels] = {};
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
  for (int k = 0; k < count; ++k) {
    if (ms) ms[k] = t[k];
    if (launches) launches[k] = n[k];
  }
  return st;
}

int bdattn_plan_cache_info(int64_t out[5]) {
  if (!out) return fail(BDATTN_ERR_INVALID_ARG, "out is NULL");
  PlanCache& c = cache();
  std::lock_guard<std::mutex> lock(c.mu);
  std::lock_guard<std::mutex> l2(c.spare_mu);
  out[0] = int64_t(c.lru.size());
  out[1] = int64_t(c.host_bytes);
  out[2] = int64_t(c.pinned_bytes);
  out[3] = int64_t(c.budget);
  out[4] = c.evictions;
  return BDATTN_OK;
}

int bdattn_plan_cache_budget(size_t bytes) {
  if (bytes < (size_t(1) << 20)) return fail(BDATTN_ERR_INVALID_ARG, "plan cache budget below 1 MiB");
  PlanCache& c = cache();
  std::lock_guard<std::mutex> lock(c.mu);
  c.budget = bytes;
  return BDATTN_OK;
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
  std::shared_ptr<Entry> entry = get_entry(P);
  const bdattn::Plan* plan = &entry->plan;
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

}  // extern "C"

namespace {

// The forward's shared body. With `ws` set, the work lists go into the
// caller's workspace from the plan's pinned staging copy; with `ws` null
// (the allocation-free forward), into this device's `scratch` array, copied
// straight from the plan's host vectors.
int fwd_impl(const bdattn_problem* p, const void* q_c, const void* k_c, const void* v_c,
             const void* q_x, const void* k_x, const void* v_x, void* o_c, void* o_x,
             float* lse_c, float* lse_x, void* workspace, size_t ws_bytes, void* hip_stream,
             bool noalloc) {
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
  const bdattn::WsLayout w = bdattn::workspace_layout(P, 0);
  hipStream_t s = (hipStream_t)hip_stream;
  if (noalloc) {
    if (w.total > kScratchBytes)
      return fail(BDATTN_ERR_WORKSPACE, "the problem needs " + std::to_string(w.total) +
                                            " bytes of forward scratch; the allocation-free "
                                            "forward holds " + std::to_string(kScratchBytes));
    if ((st = scratch_address(&workspace))) return st;
  } else if (!workspace || (reinterpret_cast<uintptr_t>(workspace) % bdattn::WS_ALIGN) ||
             ws_bytes < w.total) {
    return fail(BDATTN_ERR_WORKSPACE, "forward workspace missing, misaligned or smaller than " +
                                          std::to_string(w.total) + " bytes");
  }
  std::shared_ptr<Entry> entry = get_entry(P);
  const bdattn::Plan* plan = &entry->plan;
  char* ws = (char*)workspace;
  if ((st = noalloc ? upload_direct(*plan, w, ws, s) : upload(entry.get(), 0, w, ws, s))) return st;
  bdattn::FwdArgs a;
  a.q_c = q_c; a.k_c = k_c; a.v_c = v_c; a.q_x = q_x; a.k_x = k_x; a.v_x = v_x;
  a.o_c = o_c; a.o_x = o_x; a.lse_c = lse_c; a.lse_x = lse_x;
  a.ids = (const int32_t*)(ws + w.ids);
  a.docs = P.spans.empty() ? nullptr : (const BdDocSpan*)(ws + w.spans);
  a.kv_map = P.kv_map.empty() ? nullptr : (const int32_t*)(ws + w.kv_map);
  a.n_kv_map = int32_t(P.kv_map.size());
  a.items = (const bdattn::FwdItem*)(ws + w.q_items);
  a.n_items = int32_t(plan->fwd.size());
  a.claim = claim_on(plan->fwd.size(), plan->fwd_tiles) ? (int32_t*)(ws + w.claim) : nullptr;
  a.persist = persist_kernels(P) ? persist_grid(plan->fwd.size(), plan->fwd_tiles, a.claim != nullptr) : 0;
  if (a.persist) a.claim = (int32_t*)(ws + w.claim);  // the persistent grid claims its items
  a.B = P.B; a.H = P.H; a.Hkv = P.Hkv; a.Gw = plan->Gw; a.rows_per_item = plan->fwd_rows;
  a.n_clean_q = P.n_clean_q; a.clean_q_start = P.clean_q_start; a.n_clean_kv = P.n_clean_kv;
  a.n_corr = P.n_corr();
  a.token_causal = P.token_causal;
  a.clean_kv_start = P.clean_kv_start;
  a.corr_keys = P.corr_keys;
  a.precision = P.precision;
  a.scale_log2 = float(double(P.scale) * 1.4426950408889634);
  bdattn::KernelEvents ev[1];
  hipError_t e = bdattn::launch_fwd(a, P.dtype, P.d, s, noalloc ? nullptr : prof_events(0, 1, ev));
  if (e != hipSuccess) return fail(BDATTN_ERR_HIP, std::string("forward launch: ") + hipGetErrorString(e));
  return BDATTN_OK;
}

}  // namespace

extern "C" {

int bdattn_fwd(const bdattn_problem* p, const void* q_c, const void* k_c, const void* v_c,
               const void* q_x, const void* k_x, const void* v_x, void* o_c, void* o_x,
               float* lse_c, float* lse_x, void* workspace, size_t ws_bytes, void* hip_stream) {
  return fwd_impl(p, q_c, k_c, v_c, q_x, k_x, v_x, o_c, o_x, lse_c, lse_x, workspace, ws_bytes,
                  hip_stream, false);
}

int bdattn_fwd_noalloc(const bdattn_problem* p, const void* q_c, const void* k_c,
                       const void* v_c, const void* q_x, const void* k_x, const void* v_x,
                       void* o_c, void* o_x, float* lse_c, float* lse_x, void* hip_stream) {
  return fwd_impl(p, q_c, k_c, v_c, q_x, k_x, v_x, o_c, o_x, lse_c, lse_x, nullptr, 0,
                  hip_stream, true);
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
  std::shared_ptr<Entry> entry = get_entry(P);
  const bdattn::Plan* plan = &entry->plan;
  const bdattn::WsLayout w = bdattn::workspace_layout(P, 1);
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) % bdattn::WS_ALIGN) || ws_bytes < w.total)
    return fail(BDATTN_ERR_WORKSPACE, "backward workspace missing, misaligned or smaller than " +
                                          std::to_string(w.total) + " bytes");
  hipStream_t s = (hipStream_t)hip_stream;
  char* ws = (char*)workspace;
  if ((st = upload(entry.get(), 1, w, ws, s))) return st;
  bdattn::BwdArgs a;
  a.q_c = q_c; a.k_c = k_c; a.v_c = v_c; a.q_x = q_x; a.k_x = k_x; a.v_x = v_x;
  a.o_c = o_c; a.o_x = o_x; a.do_c = do_c; a.do_x = do_x; a.lse_c = lse_c; a.lse_x = lse_x;
  a.dq_c = dq_c; a.dq_x = dq_x; a.dk_c = dk_c; a.dv_c = dv_c; a.dk_x = dk_x; a.dv_x = dv_x;
  a.ids = (const int32_t*)(ws + w.ids);
  a.docs = P.spans.empty() ? nullptr : (const BdDocSpan*)(ws + w.spans);
  a.kv_map = P.kv_map.empty() ? nullptr : (const int32_t*)(ws + w.kv_map);
  a.n_kv_map = int32_t(P.kv_map.size());
  a.q_items = (const bdattn::FwdItem*)(ws + w.q_items);
  a.n_q_items = int32_t(plan->fwd.size());
  a.kv_items = (const bdattn::BwdItem*)(ws + w.kv_items);
  a.n_kv_items = int32_t(plan->bwd.size());
  int32_t* const ctr = (int32_t*)(ws + w.claim);
  a.claim_q = claim_on(plan->fwd.size(), plan->fwd_tiles) ? ctr : nullptr;
  a.claim_kv = claim_on(plan->bwd.size(), plan->bwd_qtiles) ? ctr + bdattn::kClaimQueues : nullptr;
  a.persist = persist_kernels(P) ? persist_grid(plan->fwd.size(), plan->fwd_tiles, a.claim_q != nullptr) : 0;
  if (a.persist) a.claim_q = ctr;  // the persistent grid claims its items
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
  a.precision = P.precision;
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
  // float32 results of bf16 problems (BDATTN_PRECISION_F32_OUT / SPLIT) merge
  // as float32 at their head dim
  if (!bdattn::have_kernels(dtype, d) && !(dtype == BDATTN_F32 && bdattn::have_kernels(BDATTN_BF16, d)))
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
