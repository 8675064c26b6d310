// Host side of the library: the C ABI of include/mlora.h - argument checks,
// status codes, the paged adapter pool's allocator and pinned-staging loads,
// and the launch plan of each step.  No device memory is allocated here.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <functional>
#include <map>
#include <cmath>
#include <mutex>
#include <string>
#include <thread>
#include <utility>
#include <vector>

#include "internal.h"

using mlora::PoolView;

namespace {

thread_local std::string g_err;

mlora_status fail(mlora_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

// Scratch of the entry point that allocates nothing (mlora_forward_static):
// device memory the library owns for the life of the process, one copy per
// GPU (each device holds its own at its own address), shared by every call
// on that GPU.  In host code `scratch` names a host-side stand-in, not the
// device memory: its device address comes from hipGetSymbolAddress, taken
// once per device with that device current.
constexpr size_t kStaticScratchBytes = size_t(20) << 20;
constexpr int kMaxDevices = 64;
static_assert(kStaticScratchBytes == MLORA_STATIC_SCRATCH_BYTES, "the header states the scratch size");
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// the device address of `scratch` on device `dev` (the current device)
mlora_status static_scratch(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return fail(MLORA_EINVAL, "device %d outside [0, %d)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return fail(MLORA_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MLORA_OK;
}

// armed launch timing: launch i gets events ev[2i] (kernel start) and
// ev[2i+1] (kernel end)
constexpr int kTimingMax = 2048;
struct Timing {
  std::mutex mu;
  std::atomic<int> armed{0};  // launches still to mark
  int used = 0;               // launches marked so far
  std::vector<hipEvent_t> ev;
  std::vector<const char*> name;  // name[i]: kernel of launch i
};
Timing g_timing;

mlora_status hip_check(hipError_t e, const char* what) {
  if (e == hipSuccess) return MLORA_OK;
  return fail(MLORA_EHIP, "%s: %s", what, hipGetErrorString(e));
}

#define HIP_TRY(call)                                   \
  do {                                                  \
    mlora_status st_ = hip_check((call), #call);        \
    if (st_ != MLORA_OK) return st_;                    \
  } while (0)

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Free-page ranges of one arena: start -> length, merged on release.
class RangeAlloc {
 public:
  typedef std::vector<std::pair<int64_t, int64_t>> Runs;

  void init(int64_t n) {
    free_.clear();
    if (n > 0) free_[0] = n;
    nfree_ = n;
  }
  int64_t nfree() const { return nfree_; }

  // `count` pages as one run if some free range holds them (first fit), else
  // gathered from the lowest free ranges.  False (nothing taken) if short.
  bool alloc(int64_t count, Runs& runs) {
    runs.clear();
    if (count > nfree_) return false;
    for (auto& kv : free_) {
      if (kv.second >= count) {
        const int64_t s = kv.first;
        runs.push_back({s, count});
        take(s, count);
        return true;
      }
    }
    int64_t need = count;
    while (need > 0) {
      auto it = free_.begin();
      const int64_t s = it->first, n = std::min(need, it->second);
      runs.push_back({s, n});
      take(s, n);
      need -= n;
    }
    return true;
  }

  void release(const Runs& runs) {
    for (const auto& r : runs) put(r.first, r.second);
  }

 private:
  void take(int64_t s, int64_t c) {
    auto it = free_.find(s);
    const int64_t len = it->second;
    free_.erase(it);
    if (len > c) free_[s + c] = len - c;
    nfree_ -= c;
  }
  void put(int64_t s, int64_t c) {
    nfree_ += c;
    auto next = free_.lower_bound(s);
    if (next != free_.begin()) {
      auto prev = std::prev(next);
      if (prev->first + prev->second == s) {
        s = prev->first;
        c += prev->second;
        free_.erase(prev);
      }
    }
    next = free_.lower_bound(s);
    if (next != free_.end() && s + c == next->first) {
      c += next->second;
      free_.erase(next);
    }
    free_[s] = c;
  }
  std::map<int64_t, int64_t> free_;
  int64_t nfree_ = 0;
};

struct MetaLayout {
  size_t rank, scale, dpt, upt, total;
};

MetaLayout meta_layout(int32_t A, int32_t P, int32_t R) {
  MetaLayout m;
  const size_t pt = (size_t)A * P * R * sizeof(int32_t);
  m.rank = 0;
  m.scale = align256((size_t)A * 4);
  m.dpt = m.scale + align256((size_t)A * 4);
  m.upt = m.dpt + align256(pt);
  m.total = m.upt + align256(pt);
  return m;
}

constexpr size_t kStageBytes = size_t(8) << 20;  // two pinned staging buffers of 8 MiB
constexpr int kMaxSplitChunks = 8;               // din slices used by the split variant
constexpr int kMaxExpandChunks = 1024;           // partial-t slices an expand accepts
constexpr int kRowsMax = 1024;                   // largest batch of the per-row path

}  // namespace

struct mlora_pool {
  int device = 0;
  mlora_pool_desc d{};
  MetaLayout ml{};
  RangeAlloc dfree, ufree;
  std::vector<int32_t> rank;
  std::vector<float> scale;
  std::vector<RangeAlloc::Runs> druns, uruns;
  int32_t n_resident = 0;
  void* stage[2] = {nullptr, nullptr};
  hipEvent_t ev[2] = {nullptr, nullptr};
  bool pending[2] = {false, false};
  int cur = 0;
  // Cross-stream lifecycle.  An unloaded adapter's pages are parked with an
  // event recorded on the unload's stream behind every earlier reader there;
  // a load (on any stream) that takes them first makes its stream wait for
  // that event on the device.  Pages a load released but did not use stay
  // behind `guard`, which every later load waits for.  ready[id] is recorded
  // on the load's stream after the adapter's copies (mlora_pool_ready).
  struct Parked {
    RangeAlloc::Runs d, u;
    int64_t pages;
    hipEvent_t last_reader;
  };
  std::vector<Parked> parked;
  hipEvent_t guard = nullptr;
  bool guarded = false;
  std::vector<hipEvent_t> ready;
  std::vector<hipEvent_t> spare;  // recorded events no longer referenced
  std::mutex mu;
  // testing aid (mlora_pool_fail_next_load): the next load fails at this
  // step once its copies are staged (0 = off)
  int fail_step = 0;

  PoolView view() const {
    PoolView v;
    const char* m = static_cast<const char*>(d.meta);
    v.rank = reinterpret_cast<const int32_t*>(m + ml.rank);
    v.scale = reinterpret_cast<const float*>(m + ml.scale);
    v.down_page = reinterpret_cast<const int32_t*>(m + ml.dpt);
    v.up_page = reinterpret_cast<const int32_t*>(m + ml.upt);
    v.down = static_cast<const uint16_t*>(d.down_pages);
    v.up = static_cast<const uint16_t*>(d.up_pages);
    v.din = d.din;
    v.dout = d.dout;
    v.n_proj = d.n_proj;
    v.max_adapters = d.max_adapters;
    v.max_rank = d.max_rank;
    return v;
  }
};

namespace {

// Packs host data into pinned staging and issues stream-ordered copies to
// the device, merging copies whose staging and device ranges are both
// contiguous.  A staging buffer is refilled only after the event recorded
// behind its last copies has completed.
class Stager {
 public:
  Stager(mlora_pool* p, hipStream_t s) : p_(p), s_(s) {}

  // reserve `bytes` of staging for a copy to device address `dst`
  mlora_status reserve(void* dst, size_t bytes, char** host) {
    if (bytes > kStageBytes) return fail(MLORA_EINVAL, "staging: one copy of %zu bytes exceeds %zu", bytes, kStageBytes);
    if (used_ + bytes > kStageBytes) {
      mlora_status st = flush();
      if (st != MLORA_OK) return st;
    }
    if (!open_) {
      const int b = p_->cur;
      if (p_->pending[b]) {
        HIP_TRY(hipEventSynchronize(p_->ev[b]));
        p_->pending[b] = false;
      }
      open_ = true;
      used_ = 0;
      copies_.clear();
    }
    char* base = static_cast<char*>(p_->stage[p_->cur]);
    *host = base + used_;
    if (!copies_.empty() && copies_.back().src + copies_.back().bytes == used_ &&
        static_cast<char*>(copies_.back().dst) + copies_.back().bytes == static_cast<char*>(dst)) {
      copies_.back().bytes += bytes;
    } else {
      copies_.push_back({used_, dst, bytes});
    }
    used_ += bytes;
    return MLORA_OK;
  }

  // work that fills the reserved staging slots; run before their copies go out
  void on_flush(std::function<void()> f) { fill_ = std::move(f); }

  mlora_status flush() {
    if (!open_) return MLORA_OK;
    if (fill_) fill_();
    const int b = p_->cur;
    char* base = static_cast<char*>(p_->stage[b]);
    for (const auto& c : copies_) HIP_TRY(hipMemcpyAsync(c.dst, base + c.src, c.bytes, hipMemcpyHostToDevice, s_));
    HIP_TRY(hipEventRecord(p_->ev[b], s_));
    p_->pending[b] = true;
    p_->cur ^= 1;
    open_ = false;
    used_ = 0;
    copies_.clear();
    return MLORA_OK;
  }

 private:
  struct Copy {
    size_t src;
    void* dst;
    size_t bytes;
  };
  mlora_pool* p_;
  hipStream_t s_;
  std::function<void()> fill_;
  bool open_ = false;
  size_t used_ = 0;
  std::vector<Copy> copies_;
};

mlora_status take_event(mlora_pool* p, hipEvent_t* e) {
  if (!p->spare.empty()) {
    *e = p->spare.back();
    p->spare.pop_back();
    return MLORA_OK;
  }
  return hip_check(hipEventCreateWithFlags(e, hipEventDisableTiming), "hipEventCreate(pool)");
}

// Makes `s` wait on the device for the last readers of every parked page
// run, then returns those runs to the free lists behind the guard event
// (recorded on `s` after the waits, so any later load waits for it too).
// Runs whose readers are known to have finished need no wait.
mlora_status unpark(mlora_pool* p, hipStream_t s) {
  bool waited = false;
  size_t done = 0;  // entries released so far (dropped from the list even on an error)
  mlora_status st = MLORA_OK;
  for (; done < p->parked.size(); ++done) {
    auto& k = p->parked[done];
    const hipError_t q = hipEventQuery(k.last_reader);
    if (q == hipErrorNotReady) {
      st = hip_check(hipStreamWaitEvent(s, k.last_reader, 0), "hipStreamWaitEvent(last reader)");
      if (st != MLORA_OK) break;
      waited = true;
    } else if (q != hipSuccess) {
      st = hip_check(q, "hipEventQuery(last reader)");
      break;
    }
    p->dfree.release(k.d);
    p->ufree.release(k.u);
    p->spare.push_back(k.last_reader);  // the wait above holds the record it saw
  }
  p->parked.erase(p->parked.begin(), p->parked.begin() + done);
  if (waited) {
    // the guard covers the waits enqueued above (even when a later entry
    // failed); without a guard, the host waits for them instead, so the
    // released pages are never reused ahead of their readers
    mlora_status gs = p->guard ? MLORA_OK : take_event(p, &p->guard);
    if (gs == MLORA_OK) gs = hip_check(hipEventRecord(p->guard, s), "hipEventRecord(guard)");
    if (gs != MLORA_OK) {
      (void)hipStreamSynchronize(s);
      return gs;
    }
    p->guarded = true;
  }
  return st;
}

int64_t parked_pages(const mlora_pool* p) {
  int64_t n = 0;
  for (const auto& k : p->parked) n += k.pages;
  return n;
}

mlora_status check_pool(const mlora_pool* p) {
  if (!p) return fail(MLORA_EINVAL, "pool is NULL");
  int dev = -1;
  HIP_TRY(hipGetDevice(&dev));
  if (dev != p->device) return fail(MLORA_EINVAL, "pool lives on device %d but device %d is current", p->device, dev);
  return MLORA_OK;
}

// page index of the i-th page of a run list
inline int64_t page_at(const RangeAlloc::Runs& runs, int64_t i) {
  for (const auto& r : runs) {
    if (i < r.second) return r.first + i;
    i -= r.second;
  }
  return -1;
}

}  // namespace

extern "C" {

const char* mlora_version(void) { return "mlora-mi355x 0.1 (gfx950)"; }

const char* mlora_status_string(int s) {
  switch (s) {
    case MLORA_OK: return "ok";
    case MLORA_EINVAL: return "invalid argument";
    case MLORA_ENOSPC: return "no free pages";
    case MLORA_EEXIST: return "adapter already resident";
    case MLORA_ENOENT: return "adapter not resident";
    case MLORA_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* mlora_last_error(void) { return g_err.c_str(); }

size_t mlora_pool_meta_bytes(int32_t max_adapters, int32_t n_proj, int32_t max_rank) {
  if (max_adapters < 1 || n_proj < 1 || max_rank < 1) return 0;
  return meta_layout(max_adapters, n_proj, max_rank).total;
}

mlora_status mlora_pool_create(const mlora_pool_desc* desc, void* stream, mlora_pool** out) {
  g_err.clear();
  if (!desc || !out) return fail(MLORA_EINVAL, "desc and out must not be NULL");
  *out = nullptr;
  const mlora_pool_desc& d = *desc;
  if (d.din < 1 || d.dout < 1 || d.n_proj < 1) return fail(MLORA_EINVAL, "din, dout and n_proj must be >= 1");
  if (d.max_adapters < 1 || d.max_adapters > MLORA_MAX_ADAPTERS)
    return fail(MLORA_EINVAL, "max_adapters must be in [1, %d]", MLORA_MAX_ADAPTERS);
  if (d.max_rank < 1 || d.max_rank > MLORA_MAX_RANK) return fail(MLORA_EINVAL, "max_rank must be in [1, %d]", MLORA_MAX_RANK);
  if (d.reserved != 0) return fail(MLORA_EINVAL, "reserved must be 0");
  if (d.n_down_pages < 0 || d.n_up_pages < 0 || d.n_down_pages > INT32_MAX || d.n_up_pages > INT32_MAX)
    return fail(MLORA_EINVAL, "page counts must be in [0, 2^31)");
  if (!d.meta) return fail(MLORA_EINVAL, "meta must not be NULL");
  if ((d.n_down_pages && !d.down_pages) || (d.n_up_pages && !d.up_pages))
    return fail(MLORA_EINVAL, "page arenas must not be NULL");
  if ((reinterpret_cast<uintptr_t>(d.meta) & 255u) != 0) return fail(MLORA_EINVAL, "meta must be 256-byte aligned");
  if ((size_t)d.din * 2 > kStageBytes || (size_t)d.dout * 2 > kStageBytes) return fail(MLORA_EINVAL, "din/dout too large");

  mlora_pool* p = new mlora_pool();
  p->d = d;
  p->ml = meta_layout(d.max_adapters, d.n_proj, d.max_rank);
  p->dfree.init(d.n_down_pages);
  p->ufree.init(d.n_up_pages);
  p->rank.assign(d.max_adapters, 0);
  p->scale.assign(d.max_adapters, 0.f);
  p->druns.resize(d.max_adapters);
  p->uruns.resize(d.max_adapters);
  p->ready.assign(d.max_adapters, nullptr);
  auto cleanup = [&](mlora_status st) {
    for (int b = 0; b < 2; ++b) {
      if (p->stage[b]) (void)hipHostFree(p->stage[b]);
      if (p->ev[b]) (void)hipEventDestroy(p->ev[b]);
    }
    delete p;
    return st;
  };
  mlora_status st = hip_check(hipGetDevice(&p->device), "hipGetDevice");
  for (int b = 0; b < 2 && st == MLORA_OK; ++b) {
    st = hip_check(hipHostMalloc(&p->stage[b], kStageBytes, hipHostMallocDefault), "hipHostMalloc(staging)");
    if (st == MLORA_OK) st = hip_check(hipEventCreateWithFlags(&p->ev[b], hipEventDisableTiming), "hipEventCreate");
  }
  hipStream_t s = as_stream(stream);
  char* meta = static_cast<char*>(d.meta);
  if (st == MLORA_OK) st = hip_check(hipMemsetAsync(meta, 0, p->ml.dpt, s), "hipMemsetAsync(meta)");
  if (st == MLORA_OK) st = hip_check(hipMemsetAsync(meta + p->ml.dpt, 0xff, p->ml.total - p->ml.dpt, s), "hipMemsetAsync(page tables)");
  if (st != MLORA_OK) return cleanup(st);
  *out = p;
  return MLORA_OK;
}

mlora_status mlora_pool_destroy(mlora_pool* p) {
  g_err.clear();
  if (!p) return fail(MLORA_EINVAL, "pool is NULL");
  mlora_status st = MLORA_OK;
  for (int b = 0; b < 2; ++b) {
    if (p->pending[b] && st == MLORA_OK) st = hip_check(hipEventSynchronize(p->ev[b]), "hipEventSynchronize");
    if (p->stage[b]) (void)hipHostFree(p->stage[b]);
    if (p->ev[b]) (void)hipEventDestroy(p->ev[b]);
  }
  for (auto& k : p->parked) (void)hipEventDestroy(k.last_reader);
  for (hipEvent_t e : p->ready)
    if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : p->spare) (void)hipEventDestroy(e);
  if (p->guard) (void)hipEventDestroy(p->guard);
  delete p;
  return st;
}

mlora_status mlora_pool_load(mlora_pool* p, int32_t id, int32_t rank, float scale, const uint16_t* down,
                             const uint16_t* up, void* stream) {
  g_err.clear();
  mlora_status st = check_pool(p);
  if (st != MLORA_OK) return st;
  std::lock_guard<std::mutex> lock(p->mu);
  const mlora_pool_desc& d = p->d;
  if (id < 0 || id >= d.max_adapters) return fail(MLORA_EINVAL, "adapter id %d outside [0, %d)", id, d.max_adapters);
  if (rank < 1 || rank > d.max_rank) return fail(MLORA_EINVAL, "rank %d outside [1, %d]", rank, d.max_rank);
  if (!down || !up) return fail(MLORA_EINVAL, "down and up must not be NULL");
  if (p->rank[id] != 0) return fail(MLORA_EEXIST, "adapter %d is already resident (unload it first)", id);
  const int64_t npages = (int64_t)d.n_proj * rank;
  hipStream_t s = as_stream(stream);
  // parked pages join the free lists once this stream waits for their
  // last readers; free pages released that way are written only after
  // the guard
  if ((p->dfree.nfree() < npages || p->ufree.nfree() < npages) && !p->parked.empty()) {
    if ((st = unpark(p, s)) != MLORA_OK) return st;
  }
  if (p->guarded) {
    const hipError_t q = hipEventQuery(p->guard);
    if (q == hipSuccess)
      p->guarded = false;
    else if (q == hipErrorNotReady)
      HIP_TRY(hipStreamWaitEvent(s, p->guard, 0));
    else
      return hip_check(q, "hipEventQuery(guard)");
  }
  RangeAlloc::Runs dr, ur;
  if (!p->dfree.alloc(npages, dr))
    return fail(MLORA_ENOSPC, "Down arena: %lld pages needed, %lld free", (long long)npages, (long long)p->dfree.nfree());
  if (!p->ufree.alloc(npages, ur)) {
    p->dfree.release(dr);
    return fail(MLORA_ENOSPC, "Up arena: %lld pages needed, %lld free", (long long)npages, (long long)p->ufree.nfree());
  }
  auto undo = [&](mlora_status s) {
    p->dfree.release(dr);
    p->ufree.release(ur);
    return s;
  };
  // the ready event is taken before any device work, so nothing after the
  // metadata copies can fail for want of an event
  if (!p->ready[id] && (st = take_event(p, &p->ready[id])) != MLORA_OK) return undo(st);
  const int fail_step = p->fail_step;
  p->fail_step = 0;
  char* meta = static_cast<char*>(d.meta);
  // A failure once copies may have been issued (page rows by a staging
  // flush; the page tables, scale and rank by the last one): the device
  // may already hold this adapter's rank, and copies into its pages may
  // still be in flight.  So the rank is set back to 0 on the stream, and
  // the pages are parked behind an event recorded after it, as an unload
  // parks them: a later load reuses them only once that stream has passed
  // this point.  Without an event the host waits for the stream instead.
  auto abort_load = [&](mlora_status s0) {
    (void)hipMemsetAsync(meta + p->ml.rank + (size_t)id * 4, 0, 4, s);
    hipEvent_t e = nullptr;
    if (take_event(p, &e) == MLORA_OK && hipEventRecord(e, s) == hipSuccess) {
      p->parked.push_back({dr, ur, npages, e});
    } else {
      if (e) p->spare.push_back(e);
      (void)hipStreamSynchronize(s);
      p->dfree.release(dr);
      p->ufree.release(ur);
    }
    return s0;
  };

  Stager sg(p, s);
  const size_t drow = (size_t)d.din * 2, urow = (size_t)d.dout * 2;
  char* dbase = static_cast<char*>(d.down_pages);
  char* ubase = static_cast<char*>(d.up_pages);
  std::vector<int32_t> dpt((size_t)d.n_proj * d.max_rank, -1), upt((size_t)d.n_proj * d.max_rank, -1);
  // Page rows are packed into the reserved staging slots just before each
  // flush, by several host threads when the chunk is large: Down rows are
  // copies, Up rows a transpose (the host work bounds a load's rate).
  struct Fill {
    char* h;
    int64_t i;  // page row of the adapter: i = p*rank + q
    bool upr;   // Up row (column q of Up for projection p), else Down row
  };
  std::vector<Fill> fills;
  auto fill_range = [&](size_t b, size_t e) {
    for (size_t k = b; k < e; ++k) {
      const Fill& f = fills[k];
      if (!f.upr) {
        std::memcpy(f.h, down + (size_t)f.i * d.din, drow);
      } else {
        uint16_t* row = reinterpret_cast<uint16_t*>(f.h);
        const uint16_t* src = up + (size_t)(f.i / rank) * d.dout * rank + f.i % rank;
        for (int32_t c = 0; c < d.dout; ++c) row[c] = src[(size_t)c * rank];
      }
    }
  };
  sg.on_flush([&]() {
    const size_t n = fills.size();
    const size_t bytes = n * std::max(drow, urow);
    const unsigned hw = std::max(1u, std::thread::hardware_concurrency());
    const size_t nt = bytes < ((size_t)4 << 20) ? 1 : std::min<size_t>(std::min(hw, 8u), n);
    if (nt <= 1) {
      fill_range(0, n);
    } else {
      std::vector<std::thread> ts;
      size_t t = 1;
      try {
        for (; t < nt; ++t) ts.emplace_back(fill_range, n * t / nt, n * (t + 1) / nt);
      } catch (...) {  // no thread to spare: this thread packs the rest
      }
      fill_range(0, n / nt);
      fill_range(n * t / nt, n);
      for (auto& th : ts) th.join();
    }
    fills.clear();
  });
  // Down rows: page i of the run list holds row (p, q), i = p*rank + q
  for (int64_t i = 0; i < npages; ++i) {
    const int64_t pg = page_at(dr, i);
    char* h = nullptr;
    if ((st = sg.reserve(dbase + pg * drow, drow, &h)) != MLORA_OK) return abort_load(st);
    fills.push_back({h, i, false});
    dpt[(size_t)(i / rank) * d.max_rank + (i % rank)] = (int32_t)pg;
  }
  // Up^T rows: page i holds column q of Up for projection p
  for (int64_t i = 0; i < npages; ++i) {
    const int64_t pg = page_at(ur, i);
    char* h = nullptr;
    if ((st = sg.reserve(ubase + pg * urow, urow, &h)) != MLORA_OK) return abort_load(st);
    fills.push_back({h, i, true});
    upt[(size_t)(i / rank) * d.max_rank + (i % rank)] = (int32_t)pg;
  }
  // metadata: page tables, scale, then rank (all ordered on the stream)
  const size_t ptb = dpt.size() * sizeof(int32_t);
  const size_t pt_off = (size_t)id * d.n_proj * d.max_rank * sizeof(int32_t);
  char* h = nullptr;
  if ((st = sg.reserve(meta + p->ml.dpt + pt_off, ptb, &h)) != MLORA_OK) return abort_load(st);
  std::memcpy(h, dpt.data(), ptb);
  if ((st = sg.reserve(meta + p->ml.upt + pt_off, ptb, &h)) != MLORA_OK) return abort_load(st);
  std::memcpy(h, upt.data(), ptb);
  if ((st = sg.reserve(meta + p->ml.scale + (size_t)id * 4, 4, &h)) != MLORA_OK) return abort_load(st);
  std::memcpy(h, &scale, 4);
  if ((st = sg.reserve(meta + p->ml.rank + (size_t)id * 4, 4, &h)) != MLORA_OK) return abort_load(st);
  std::memcpy(h, &rank, 4);
  if (fail_step == 1) return abort_load(fail(MLORA_EHIP, "injected failure before the last staging flush"));
  if ((st = sg.flush()) != MLORA_OK) return abort_load(st);
  if (fail_step == 2) return abort_load(fail(MLORA_EHIP, "injected failure after the metadata copies"));
  if ((st = hip_check(hipEventRecord(p->ready[id], s), "hipEventRecord(ready)")) != MLORA_OK) return abort_load(st);

  p->rank[id] = rank;
  p->scale[id] = scale;
  p->druns[id] = dr;
  p->uruns[id] = ur;
  ++p->n_resident;
  return MLORA_OK;
}

mlora_status mlora_pool_fail_next_load(mlora_pool* p, int32_t step) {
  g_err.clear();
  mlora_status st = check_pool(p);
  if (st != MLORA_OK) return st;
  if (step < 0 || step > 2) return fail(MLORA_EINVAL, "failure step %d outside [0, 2]", step);
  std::lock_guard<std::mutex> lock(p->mu);
  p->fail_step = step;
  return MLORA_OK;
}

mlora_status mlora_pool_unload(mlora_pool* p, int32_t id, void* stream) {
  g_err.clear();
  mlora_status st = check_pool(p);
  if (st != MLORA_OK) return st;
  std::lock_guard<std::mutex> lock(p->mu);
  if (id < 0 || id >= p->d.max_adapters) return fail(MLORA_EINVAL, "adapter id %d outside [0, %d)", id, p->d.max_adapters);
  if (p->rank[id] == 0) return fail(MLORA_ENOENT, "adapter %d is not resident", id);
  char* meta = static_cast<char*>(p->d.meta);
  hipStream_t s = as_stream(stream);
  // the pages are parked behind every reader enqueued so far on `stream`
  hipEvent_t e = nullptr;
  mlora_status est = take_event(p, &e);
  if (est != MLORA_OK) return est;
  est = hip_check(hipMemsetAsync(meta + p->ml.rank + (size_t)id * 4, 0, 4, s), "hipMemsetAsync(rank)");
  if (est == MLORA_OK) est = hip_check(hipEventRecord(e, s), "hipEventRecord(last reader)");
  if (est != MLORA_OK) {
    p->spare.push_back(e);
    return est;
  }
  p->parked.push_back({p->druns[id], p->uruns[id], (int64_t)p->d.n_proj * p->rank[id], e});
  p->druns[id].clear();
  p->uruns[id].clear();
  p->rank[id] = 0;
  p->scale[id] = 0.f;
  --p->n_resident;
  return MLORA_OK;
}

mlora_status mlora_pool_ready(mlora_pool* p, int32_t id, void* stream) {
  g_err.clear();
  mlora_status st = check_pool(p);
  if (st != MLORA_OK) return st;
  std::lock_guard<std::mutex> lock(p->mu);
  if (id < 0 || id >= p->d.max_adapters) return fail(MLORA_EINVAL, "adapter id %d outside [0, %d)", id, p->d.max_adapters);
  if (p->rank[id] == 0) return fail(MLORA_ENOENT, "adapter %d is not resident", id);
  return hip_check(hipStreamWaitEvent(as_stream(stream), p->ready[id], 0), "hipStreamWaitEvent(ready)");
}

mlora_status mlora_pool_query(const mlora_pool* p, int32_t id, int32_t* rank, float* scale) {
  g_err.clear();
  if (!p) return fail(MLORA_EINVAL, "pool is NULL");
  if (id < 0 || id >= p->d.max_adapters) return fail(MLORA_EINVAL, "adapter id %d outside [0, %d)", id, p->d.max_adapters);
  std::lock_guard<std::mutex> lock(const_cast<mlora_pool*>(p)->mu);
  if (rank) *rank = p->rank[id];
  if (scale) *scale = p->scale[id];
  return p->rank[id] ? MLORA_OK : fail(MLORA_ENOENT, "adapter %d is not resident", id);
}

mlora_status mlora_pool_free_pages(const mlora_pool* p, int64_t* free_down, int64_t* free_up, int32_t* n_resident) {
  g_err.clear();
  if (!p) return fail(MLORA_EINVAL, "pool is NULL");
  std::lock_guard<std::mutex> lock(const_cast<mlora_pool*>(p)->mu);
  const int64_t pk = parked_pages(p);  // usable by the next load (which waits for their readers)
  if (free_down) *free_down = p->dfree.nfree() + pk;
  if (free_up) *free_up = p->ufree.nfree() + pk;
  if (n_resident) *n_resident = p->n_resident;
  return MLORA_OK;
}

size_t mlora_segments_bytes(int32_t n) {
  if (n < 0) return 0;
  return align256(((size_t)MLORA_SEG_TILES(n) + 2 * (size_t)n) * sizeof(int32_t));
}

mlora_status mlora_build_segments(const mlora_pool* p, const int32_t* row_adapter, int32_t n, void* seg_ws,
                                  void* stream) {
  g_err.clear();
  mlora_status st = check_pool(p);
  if (st != MLORA_OK) return st;
  if (n < 0 || n > MLORA_MAX_ROWS) return fail(MLORA_EINVAL, "n_rows %d outside [0, %d]", n, MLORA_MAX_ROWS);
  if (!seg_ws || (n > 0 && !row_adapter)) return fail(MLORA_EINVAL, "row_adapter and seg_ws must not be NULL");
  if ((reinterpret_cast<uintptr_t>(seg_ws) & 7u) != 0) return fail(MLORA_EINVAL, "seg_ws must be 8-byte aligned");
  const PoolView v = p->view();
  return hip_check(mlora::launch_seg_build(row_adapter, n, v.rank, v.max_adapters, static_cast<int32_t*>(seg_ws),
                                           as_stream(stream)),
                   "segment builder launch");
}

mlora_status mlora_segments_header(const void* seg_ws, int32_t* header, void* stream) {
  g_err.clear();
  if (!seg_ws || !header) return fail(MLORA_EINVAL, "seg_ws and header must not be NULL");
  HIP_TRY(hipMemcpyAsync(header, seg_ws, MLORA_SEG_HEADER * sizeof(int32_t), hipMemcpyDeviceToHost, as_stream(stream)));
  HIP_TRY(hipStreamSynchronize(as_stream(stream)));
  return MLORA_OK;
}

mlora_status mlora_segments_status(const void* seg_ws, int32_t* status, void* stream) {
  g_err.clear();
  if (!seg_ws || !status) return fail(MLORA_EINVAL, "seg_ws and status must not be NULL");
  HIP_TRY(hipMemcpyAsync(status, static_cast<const int32_t*>(seg_ws) + MLORA_SEG_STATUS, sizeof(int32_t),
                         hipMemcpyDeviceToHost, as_stream(stream)));
  HIP_TRY(hipStreamSynchronize(as_stream(stream)));
  return MLORA_OK;
}

mlora_status mlora_base_gemm(const uint16_t* X, const uint16_t* W0, uint16_t* Y, int32_t n, int32_t din,
                             int32_t dout, void* stream) {
  g_err.clear();
  if (n < 0 || din < 1 || dout < 1) return fail(MLORA_EINVAL, "need n_rows >= 0, din >= 1, dout >= 1");
  if (n == 0) return MLORA_OK;
  if (!X || !W0 || !Y) return fail(MLORA_EINVAL, "X, W0 and Y must not be NULL");
  return hip_check(mlora::launch_base_gemm(X, W0, Y, n, din, dout, as_stream(stream)), "base GEMM launch");
}

int32_t mlora_shrink_max_chunks(int32_t din) { return din < 1 ? 0 : (din + 511) / 512; }

namespace {
mlora_status check_branch_args(const mlora_pool* p, int32_t proj, const void* seg_ws, int32_t n) {
  mlora_status st = check_pool(p);
  if (st != MLORA_OK) return st;
  if (proj < 0 || proj >= p->d.n_proj) return fail(MLORA_EINVAL, "proj %d outside [0, %d)", proj, p->d.n_proj);
  if (n < 0 || n > MLORA_MAX_ROWS) return fail(MLORA_EINVAL, "n_rows %d outside [0, %d]", n, MLORA_MAX_ROWS);
  if (!seg_ws) return fail(MLORA_EINVAL, "seg_ws must not be NULL");
  return MLORA_OK;
}
int chunk_elems_for(int din, int n_chunks) {
  const int per = (din + n_chunks - 1) / n_chunks;
  return (per + 511) / 512 * 512;
}
}  // namespace

mlora_status mlora_shrink(const mlora_pool* p, int32_t proj, const uint16_t* X, const void* seg_ws, int32_t n,
                          float* T, int32_t n_chunks, void* stream) {
  g_err.clear();
  mlora_status st = check_branch_args(p, proj, seg_ws, n);
  if (st != MLORA_OK) return st;
  if (n_chunks < 1 || n_chunks > mlora_shrink_max_chunks(p->d.din))
    return fail(MLORA_EINVAL, "n_chunks %d outside [1, %d]", n_chunks, mlora_shrink_max_chunks(p->d.din));
  if (n == 0) return MLORA_OK;
  if (!X || !T) return fail(MLORA_EINVAL, "X and T must not be NULL");
  return hip_check(mlora::launch_shrink(p->view(), proj, X, static_cast<const int32_t*>(seg_ws), n, T, n_chunks,
                                        chunk_elems_for(p->d.din, n_chunks), as_stream(stream)),
                   "shrink launch");
}

mlora_status mlora_expand(const mlora_pool* p, int32_t proj, const float* T, int32_t n_chunks, const void* seg_ws,
                          uint16_t* Y, int32_t n, void* stream) {
  g_err.clear();
  mlora_status st = check_branch_args(p, proj, seg_ws, n);
  if (st != MLORA_OK) return st;
  if (n_chunks < 1 || n_chunks > kMaxExpandChunks)
    return fail(MLORA_EINVAL, "n_chunks %d outside [1, %d]", n_chunks, kMaxExpandChunks);
  if (n == 0) return MLORA_OK;
  if (!T || !Y) return fail(MLORA_EINVAL, "T and Y must not be NULL");
  return hip_check(mlora::launch_expand(p->view(), proj, T, n_chunks, static_cast<const int32_t*>(seg_ws), Y, n,
                                        as_stream(stream)),
                   "expand launch");
}

mlora_status mlora_fused(const mlora_pool* p, int32_t proj, const uint16_t* X, const void* seg_ws, uint16_t* Y,
                         int32_t n, void* stream) {
  g_err.clear();
  mlora_status st = check_branch_args(p, proj, seg_ws, n);
  if (st != MLORA_OK) return st;
  if (n == 0) return MLORA_OK;
  if (!X || !Y) return fail(MLORA_EINVAL, "X and Y must not be NULL");
  return hip_check(mlora::launch_fused(p->view(), proj, X, static_cast<const int32_t*>(seg_ws), Y, n,
                                       as_stream(stream)),
                   "fused launch");
}

namespace {
// work layout of the per-row path: T [n][max_rank] fp32 | split-K partials
struct RowsWork {
  float* T;
  float* part;
};
// T region: room for the decode form's K-slice partials of T as well, then
// the per-row descriptors
size_t rows_t_bytes(const mlora_pool* p, int n) {
  return align256((size_t)mlora::rows_t_slices(n) * n * p->d.max_rank * sizeof(float) +
                  (size_t)n * mlora::row_desc_words(p->d.max_rank) * sizeof(int32_t));
}
size_t rows_work_bytes(const mlora_pool* p, int n) {
  return rows_t_bytes(p, n) + align256(mlora::gemm_lora_part_floats(n, p->d.dout, p->d.din) * sizeof(float));
}
RowsWork rows_work(const mlora_pool* p, int n, void* work) {
  char* w = static_cast<char*>(work);
  RowsWork r;
  r.T = reinterpret_cast<float*>(w);
  r.part = reinterpret_cast<float*>(w + rows_t_bytes(p, n));
  return r;
}
mlora_status check_rows_work(const mlora_pool* p, int n, const void* work, size_t work_bytes) {
  if (n > kRowsMax) return fail(MLORA_EINVAL, "n_rows %d above %d for the per-row path", n, kRowsMax);
  const size_t need = rows_work_bytes(p, n);
  if (!work || work_bytes < need) return fail(MLORA_EINVAL, "work: %zu bytes given, %zu needed", work_bytes, need);
  if ((reinterpret_cast<uintptr_t>(work) & 255u) != 0) return fail(MLORA_EINVAL, "work must be 256-byte aligned");
  return MLORA_OK;
}
}  // namespace

mlora_status mlora_shrink_rows(const mlora_pool* p, int32_t proj, const uint16_t* X, const void* seg_ws, int32_t n,
                               void* work, size_t work_bytes, void* stream) {
  g_err.clear();
  mlora_status st = check_branch_args(p, proj, seg_ws, n);
  if (st != MLORA_OK) return st;
  if (n == 0) return MLORA_OK;
  if (!X) return fail(MLORA_EINVAL, "X must not be NULL");
  if ((st = check_rows_work(p, n, work, work_bytes)) != MLORA_OK) return st;
  const RowsWork w = rows_work(p, n, work);
  return hip_check(mlora::launch_shrink_rows(p->view(), proj, X, static_cast<const int32_t*>(seg_ws), n, w.T,
                                             as_stream(stream)),
                   "per-row shrink launch");
}

mlora_status mlora_gemm_lora(const mlora_pool* p, int32_t proj, const uint16_t* X, const uint16_t* W0,
                             const void* seg_ws, void* work, size_t work_bytes, uint16_t* Y, int32_t n, void* stream) {
  g_err.clear();
  mlora_status st = check_branch_args(p, proj, seg_ws, n);
  if (st != MLORA_OK) return st;
  if (n == 0) return MLORA_OK;
  if (!X || !W0 || !Y) return fail(MLORA_EINVAL, "X, W0 and Y must not be NULL");
  if ((st = check_rows_work(p, n, work, work_bytes)) != MLORA_OK) return st;
  const RowsWork w = rows_work(p, n, work);
  return hip_check(mlora::launch_gemm_lora(p->view(), proj, X, W0, static_cast<const int32_t*>(seg_ws), w.T, w.part,
                                           Y, n, false, as_stream(stream)),
                   "GEMM + expand launch");
}

namespace {
// din slices for the split variant: enough waves to spread a small batch
// over the chip, never more than kMaxSplitChunks
// Operands of the large-batch GEMM's low-rank term, in `work` after the
// shrink's slices: tb [n][wt] bf16 | koff [max_adapters] | over, kx (one
// word each) | tx [n][txw] bf16 | upt, room for upt_units rank rows of dout.
// upt_units is every adapter of the batch padded to the largest rank, or as
// many rank rows as fit in a 256 MiB budget for the operands if that is
// less: then a batch whose distinct adapters (known only on the device) need
// more has its low-rank term added by a separate expand instead of the
// epilogue (may_overrun).  txw (the widest rank-concatenated batch, Ux
// living in the upt region) is the largest multiple of 64 up to
// kMaxConcatRanks that upt_units holds.
constexpr size_t kMaxEpilogueBytes = 256u << 20;
struct EpilogueLayout {
  size_t koff, over, kx, tx, upt, total;
  long upt_units;
  int txw;
  bool may_overrun;
};
EpilogueLayout epilogue_layout(const mlora_pool* p, int n) {
  const int wt = mlora::t_rows_width(p->d.max_rank);
  EpilogueLayout L{};
  L.koff = align256((size_t)n * wt * 2);
  L.over = L.koff + align256((size_t)p->d.max_adapters * 4);
  L.kx = L.over + 4;
  const long worst = (long)mlora::lora_upt_units(n, p->d.max_adapters, p->d.max_rank);
  L.txw = (int)std::min<long>(mlora::kMaxConcatRanks, worst / 64 * 64);
  L.tx = L.over + 256;
  L.upt = L.tx + align256((size_t)n * L.txw * 2);
  const size_t row = (size_t)p->d.dout * 2;
  const long budget = L.upt < kMaxEpilogueBytes ? (long)((kMaxEpilogueBytes - L.upt) / row) / 16 * 16 : 0;
  L.upt_units = std::min(worst, budget);
  if (L.upt_units < L.txw) L.txw = (int)(L.upt_units / 64 * 64);
  L.may_overrun = L.upt_units < worst;
  L.total = L.upt + align256((size_t)L.upt_units * row);
  return L;
}
size_t lora_operands_bytes(const mlora_pool* p, int n) { return epilogue_layout(p, n).total; }
// The GEMM epilogue needs room for at least one adapter of the largest rank.
bool big_epilogue_fits(const mlora_pool* p, int n) {
  return epilogue_layout(p, n).upt_units >= mlora::t_rows_width(p->d.max_rank) &&
         (size_t)p->d.n_up_pages * p->d.dout < (1u << 31);
}

int split_chunks(const mlora_pool* p, int n) {
  const int din = p->d.din;
  int c;
  if (n >= mlora::kShrinkTilesMinRows && din % 32 == 0) {
    // matrix-core shrink: enough (tile, slice) workgroups for two per CU
    // (prefill, 70 tile slots: 8 slices take 13.9 us, 4 slices 17.4 us)
    const int cap = mlora::shrink_tile_cap(p->view(), n);
    c = (512 + cap - 1) / cap;
  } else {
    const int items = MLORA_SEG_MAX_ITEMS(n);
    c = (1024 + items - 1) / items;
  }
  c = std::min(c, kMaxSplitChunks);
  c = std::min(c, mlora_shrink_max_chunks(din));
  return std::max(c, 1);
}
// AUTO: decode-sized batches take the per-row path (shrink per row, expand
// inside the base GEMM kernel); larger batches the grouped split path
int32_t auto_variant(const mlora_pool* p, int n) {
  (void)p;
  return n <= kRowsMax ? MLORA_VARIANT_ROWS : MLORA_VARIANT_SPLIT;
}
}  // namespace

namespace {
// Bytes of `work` the launch plan of `variant` (AUTO resolved) uses for n
// rows: ROWS its T region and split-K partials; FUSED the same partials
// (its base GEMM splits K through them when the buffer holds them, else it
// takes the one-pass form); SPLIT its shrink slices, plus the epilogue's
// operands for large batches, and the split-K partials of its base GEMM.
size_t plan_work_bytes(const mlora_pool* p, int n, int variant) {
  if (n <= 0) return 0;
  const size_t rows = n <= kRowsMax ? rows_work_bytes(p, n) : 0;
  if (variant != MLORA_VARIANT_SPLIT) return rows;
  const int chunks = std::max(split_chunks(p, n), 1);
  size_t b = align256((size_t)chunks * n * p->d.max_rank * sizeof(float));
  if (big_epilogue_fits(p, n)) b += lora_operands_bytes(p, n);
  return std::max(b, rows);
}
}  // namespace

size_t mlora_work_bytes(const mlora_pool* p, int32_t n) {
  if (!p || n < 0) return 0;
  // the largest need among the variants (so one buffer serves them all)
  return std::max(plan_work_bytes(p, n, MLORA_VARIANT_SPLIT), plan_work_bytes(p, n, MLORA_VARIANT_ROWS));
}

mlora_status mlora_plan(const mlora_pool* p, int32_t n, int32_t variant, int32_t* out_variant, int32_t* out_chunks) {
  g_err.clear();
  if (!p) return fail(MLORA_EINVAL, "pool is NULL");
  if (n < 0 || n > MLORA_MAX_ROWS) return fail(MLORA_EINVAL, "n_rows %d outside [0, %d]", n, MLORA_MAX_ROWS);
  if (variant < MLORA_VARIANT_AUTO || variant > MLORA_VARIANT_ROWS) return fail(MLORA_EINVAL, "unknown variant %d", variant);
  if (variant == MLORA_VARIANT_AUTO) variant = auto_variant(p, n);
  if (variant == MLORA_VARIANT_ROWS && n > kRowsMax)
    return fail(MLORA_EINVAL, "the per-row variant takes at most %d rows", kRowsMax);
  if (out_variant) *out_variant = variant;
  if (out_chunks) *out_chunks = variant == MLORA_VARIANT_SPLIT ? split_chunks(p, n) : 0;
  return MLORA_OK;
}

mlora_status mlora_apply(const mlora_pool* p, int32_t proj, const uint16_t* X, const uint16_t* W0,
                         const void* seg_ws, uint16_t* Y, int32_t n, void* work, size_t work_bytes, int32_t variant,
                         void* stream) {
  g_err.clear();
  mlora_status st = check_branch_args(p, proj, seg_ws, n);
  if (st != MLORA_OK) return st;
  if (variant < MLORA_VARIANT_AUTO || variant > MLORA_VARIANT_ROWS) return fail(MLORA_EINVAL, "unknown variant %d", variant);
  if (variant == MLORA_VARIANT_ROWS && n > kRowsMax)
    return fail(MLORA_EINVAL, "the per-row variant takes at most %d rows", kRowsMax);
  if (n == 0) return MLORA_OK;
  if (!X || !W0 || !Y) return fail(MLORA_EINVAL, "X, W0 and Y must not be NULL");
  const mlora_pool_desc& d = p->d;
  hipStream_t s = as_stream(stream);
  const PoolView v = p->view();
  const int32_t* ws = static_cast<const int32_t*>(seg_ws);
  if (variant == MLORA_VARIANT_AUTO) variant = auto_variant(p, n);
  if (variant == MLORA_VARIANT_SPLIT || variant == MLORA_VARIANT_ROWS) {
    const size_t need = plan_work_bytes(p, n, variant);
    if (!work || work_bytes < need) return fail(MLORA_EINVAL, "work: %zu bytes given, %zu needed", work_bytes, need);
    if (!aligned16(work)) return fail(MLORA_EINVAL, "work must be 16-byte aligned");
  }
  if (variant == MLORA_VARIANT_ROWS) {
    if ((st = check_rows_work(p, n, work, work_bytes)) != MLORA_OK) return st;
    const RowsWork w = rows_work(p, n, work);
    return hip_check(mlora::launch_gemm_lora(v, proj, X, W0, ws, w.T, w.part, Y, n, true, s),
                     "per-row shrink + GEMM + expand launch");
  }
  if (variant == MLORA_VARIANT_SPLIT && big_epilogue_fits(p, n) && mlora::big_lora_ok(v, X, W0, n)) {
    // large batch: shrink, the low-rank operands, then one GEMM that adds
    // the low-rank term itself (Y written once)
    const int chunks = split_chunks(p, n);
    float* T = static_cast<float*>(work);
    char* w = static_cast<char*>(work) + align256((size_t)chunks * n * d.max_rank * sizeof(float));
    const int wt = mlora::t_rows_width(d.max_rank);
    const EpilogueLayout L = epilogue_layout(p, n);
    uint16_t* tb = reinterpret_cast<uint16_t*>(w);
    int32_t* koff = reinterpret_cast<int32_t*>(w + L.koff);
    int32_t* over = reinterpret_cast<int32_t*>(w + L.over);
    int32_t* kx = reinterpret_cast<int32_t*>(w + L.kx);
    uint16_t* tx = L.txw > 0 ? reinterpret_cast<uint16_t*>(w + L.tx) : nullptr;
    uint16_t* upt = reinterpret_cast<uint16_t*>(w + L.upt);
    st = hip_check(mlora::launch_shrink(v, proj, X, ws, n, T, chunks, chunk_elems_for(d.din, chunks), s), "shrink launch");
    if (st != MLORA_OK) return st;
    st = hip_check(mlora::launch_lora_prep(v, proj, ws, n, T, chunks, tb, wt, koff, upt, L.upt_units, over, tx,
                                           L.txw, kx, s),
                   "low-rank operand launch");
    if (st != MLORA_OK) return st;
    const mlora::LoraOperands lo{tb, koff, upt, wt, L.may_overrun ? over : nullptr, tx, L.txw, tx ? kx : nullptr};
    st = hip_check(mlora::launch_big_lora(v, X, W0, ws, lo, Y, n, s), "GEMM + low-rank term launch");
    if (st != MLORA_OK || !L.may_overrun) return st;
    return hip_check(mlora::launch_expand_over(v, proj, T, chunks, ws, Y, n, over, s), "overrun expand launch");
  }
  // the base GEMM: split over K with its partials in `work` (per-row
  // layout) when the batch and the buffer allow, else the plain form
  hipError_t ge = hipErrorNotSupported;
  if (n <= kRowsMax && work && work_bytes >= rows_work_bytes(p, n) &&
      (reinterpret_cast<uintptr_t>(work) & 255u) == 0)
    ge = mlora::launch_base_split(X, W0, Y, n, d.din, d.dout, rows_work(p, n, work).part, s);
  if (ge == hipErrorNotSupported) ge = mlora::launch_base_gemm(X, W0, Y, n, d.din, d.dout, s);
  st = hip_check(ge, "base GEMM launch");
  if (st != MLORA_OK) return st;
  if (variant == MLORA_VARIANT_FUSED)
    return hip_check(mlora::launch_fused(v, proj, X, ws, Y, n, s), "fused launch");
  const int chunks = split_chunks(p, n);
  float* T = static_cast<float*>(work);
  st = hip_check(mlora::launch_shrink(v, proj, X, ws, n, T, chunks, chunk_elems_for(d.din, chunks), s), "shrink launch");
  if (st != MLORA_OK) return st;
  return hip_check(mlora::launch_expand(v, proj, T, chunks, ws, Y, n, s), "expand launch");
}

mlora_status mlora_forward(const mlora_pool* p, int32_t proj, const uint16_t* X, const uint16_t* W0,
                           const int32_t* row_adapter, void* seg_ws, uint16_t* Y, int32_t n, void* work,
                           size_t work_bytes, int32_t variant, void* stream) {
  g_err.clear();
  mlora_status st = check_pool(p);
  if (st != MLORA_OK) return st;
  if (n < 0 || n > MLORA_MAX_ROWS) return fail(MLORA_EINVAL, "n_rows %d outside [0, %d]", n, MLORA_MAX_ROWS);
  if (!seg_ws || (n > 0 && !row_adapter)) return fail(MLORA_EINVAL, "row_adapter and seg_ws must not be NULL");
  if ((reinterpret_cast<uintptr_t>(seg_ws) & 7u) != 0) return fail(MLORA_EINVAL, "seg_ws must be 8-byte aligned");
  if ((st = check_branch_args(p, proj, seg_ws, n)) != MLORA_OK) return st;
  if (variant < MLORA_VARIANT_AUTO || variant > MLORA_VARIANT_ROWS) return fail(MLORA_EINVAL, "unknown variant %d", variant);
  if (variant == MLORA_VARIANT_ROWS && n > kRowsMax)
    return fail(MLORA_EINVAL, "the per-row variant takes at most %d rows", kRowsMax);
  if (n > 0 && (!X || !W0 || !Y)) return fail(MLORA_EINVAL, "X, W0 and Y must not be NULL");
  const int32_t resolved = variant == MLORA_VARIANT_AUTO ? auto_variant(p, n) : variant;
  if (n > 0 && (resolved == MLORA_VARIANT_SPLIT || resolved == MLORA_VARIANT_ROWS)) {
    // the work checks of mlora_apply, before anything is launched
    const size_t need = plan_work_bytes(p, n, resolved);
    if (!work || work_bytes < need) return fail(MLORA_EINVAL, "work: %zu bytes given, %zu needed", work_bytes, need);
    if (!aligned16(work)) return fail(MLORA_EINVAL, "work must be 16-byte aligned");
    if (resolved == MLORA_VARIANT_ROWS && (st = check_rows_work(p, n, work, work_bytes)) != MLORA_OK) return st;
  }
  if (n > 0 && resolved == MLORA_VARIANT_ROWS) {
    const RowsWork w = rows_work(p, n, work);
    const hipError_t e = mlora::launch_forward_rows(p->view(), proj, X, W0, row_adapter, static_cast<int32_t*>(seg_ws),
                                                    w.T, w.part, Y, n, as_stream(stream));
    if (e != hipErrorNotSupported) return hip_check(e, "segment build + per-row shrink + GEMM + expand launch");
  }
  if ((st = mlora_build_segments(p, row_adapter, n, seg_ws, stream)) != MLORA_OK) return st;
  return mlora_apply(p, proj, X, W0, seg_ws, Y, n, work, work_bytes, variant, stream);
}

mlora_status mlora_forward_static(const mlora_pool* p, int32_t proj, const uint16_t* X, const uint16_t* W0,
                                  const int32_t* row_adapter, void* seg_ws, uint16_t* Y, int32_t n, int32_t variant,
                                  void* stream) {
  g_err.clear();
  mlora_status st = check_pool(p);
  if (st != MLORA_OK) return st;
  if (n < 0 || n > MLORA_MAX_ROWS) return fail(MLORA_EINVAL, "n_rows %d outside [0, %d]", n, MLORA_MAX_ROWS);
  if (variant < MLORA_VARIANT_AUTO || variant > MLORA_VARIANT_ROWS) return fail(MLORA_EINVAL, "unknown variant %d", variant);
  const size_t need = plan_work_bytes(p, n, variant == MLORA_VARIANT_AUTO ? auto_variant(p, n) : variant);
  if (need > kStaticScratchBytes)
    return fail(MLORA_EINVAL, "a batch of %d rows needs %zu bytes of scratch; the static scratch holds %zu "
                "(use mlora_forward with a work buffer)", n, need, kStaticScratchBytes);
  void* work = nullptr;
  if ((st = static_scratch(p->device, &work)) != MLORA_OK) return st;
  return mlora_forward(p, proj, X, W0, row_adapter, seg_ws, Y, n, work, kStaticScratchBytes, variant, stream);
}

mlora_status mlora_timing_arm(int32_t n_launches) {
  g_err.clear();
  if (n_launches < 1 || n_launches > kTimingMax) return fail(MLORA_EINVAL, "n_launches %d outside [1, %d]", n_launches, kTimingMax);
  std::lock_guard<std::mutex> lk(g_timing.mu);
  while ((int)g_timing.ev.size() < 2 * n_launches) {
    hipEvent_t e;
    mlora_status st = hip_check(hipEventCreate(&e), "hipEventCreate(timing)");
    if (st != MLORA_OK) return st;
    g_timing.ev.push_back(e);
  }
  g_timing.name.assign(n_launches, nullptr);
  g_timing.used = 0;
  g_timing.armed.store(n_launches);
  return MLORA_OK;
}

mlora_status mlora_timing_read(float* ms, int32_t capacity, int32_t* out_n) {
  g_err.clear();
  std::lock_guard<std::mutex> lk(g_timing.mu);
  g_timing.armed.store(0);
  const int used = g_timing.used;
  if (out_n) *out_n = used;
  if (!ms || capacity < used) return fail(MLORA_EINVAL, "room for %d intervals, %d launches marked", capacity, used);
  mlora_status st = MLORA_OK;
  for (int i = 0; i < used && st == MLORA_OK; ++i) {
    st = hip_check(hipEventSynchronize(g_timing.ev[2 * i + 1]), "hipEventSynchronize(timing)");
    if (st == MLORA_OK)
      st = hip_check(hipEventElapsedTime(&ms[i], g_timing.ev[2 * i], g_timing.ev[2 * i + 1]), "hipEventElapsedTime");
  }
  return st;
}

const char* mlora_timing_name(int32_t i) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  return (i >= 0 && i < g_timing.used) ? g_timing.name[i] : nullptr;
}

mlora_status mlora_merge(const mlora_pool* p, int32_t id, int32_t proj, uint16_t* W0, float sign, void* stream) {
  g_err.clear();
  if (!p) return fail(MLORA_EINVAL, "pool is NULL");
  if (!W0) return fail(MLORA_EINVAL, "W0 must not be NULL");
  if (!std::isfinite(sign)) return fail(MLORA_EINVAL, "sign must be finite");
  if (id < 0 || id >= p->d.max_adapters) return fail(MLORA_EINVAL, "adapter id %d outside [0, %d)", id, p->d.max_adapters);
  if (proj < 0 || proj >= p->d.n_proj) return fail(MLORA_EINVAL, "projection %d outside [0, %d)", proj, p->d.n_proj);
  int32_t rank;
  float scale;
  {
    std::lock_guard<std::mutex> lock(const_cast<mlora_pool*>(p)->mu);
    rank = p->rank[id];
    scale = p->scale[id];
  }
  if (rank <= 0) return fail(MLORA_ENOENT, "adapter %d is not resident", id);
  return hip_check(mlora::launch_merge(p->view(), id, proj, rank, sign * scale, W0, as_stream(stream)),
                   "merge launch");
}

mlora_status mlora_hbm_copy(void* dst, const void* src, size_t bytes, void* stream) {
  g_err.clear();
  if (!dst || !src || bytes % 16 != 0 || !aligned16(dst) || !aligned16(src))
    return fail(MLORA_EINVAL, "copy needs non-NULL 16-byte aligned pointers and a multiple of 16 bytes");
  return hip_check(mlora::launch_hbm_copy(dst, src, bytes, as_stream(stream)), "copy launch");
}

mlora_status mlora_hbm_read(const void* src, size_t bytes, uint32_t* out, void* stream) {
  g_err.clear();
  if (!src || !out || bytes % 16 != 0 || !aligned16(src))
    return fail(MLORA_EINVAL, "read needs a non-NULL 16-byte aligned source, a multiple of 16 bytes and an output word");
  return hip_check(mlora::launch_hbm_read(src, bytes, out, as_stream(stream)), "read launch");
}

mlora_status mlora_hbm_read_lds(const void* src, size_t bytes, uint32_t* out, void* stream) {
  g_err.clear();
  if (!src || !out || bytes % 1024 != 0 || bytes > 0x7fffffffu || !aligned16(src))
    return fail(MLORA_EINVAL,
                "LDS-DMA read needs a non-NULL 16-byte aligned source, a multiple of 1024 bytes below 2 GiB and an "
                "output word");
  return hip_check(mlora::launch_hbm_read_lds(src, bytes, out, as_stream(stream)), "LDS-DMA read launch");
}

}  // extern "C"

namespace mlora {
TimingSlot timing_next(const char* kernel) {
  TimingSlot t;
  if (g_timing.armed.load(std::memory_order_relaxed) <= 0) return t;
  std::lock_guard<std::mutex> lk(g_timing.mu);
  if (g_timing.armed.load() <= 0) return t;
  g_timing.armed.fetch_sub(1);
  const int i = g_timing.used++;
  g_timing.name[i] = kernel;
  t.start = g_timing.ev[2 * i];
  t.stop = g_timing.ev[2 * i + 1];
  t.on = true;
  return t;
}
}  // namespace mlora
