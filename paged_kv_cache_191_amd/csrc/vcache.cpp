// Contiguous KV cache on demand-mapped virtual memory (HIP VMM).
//
// Follows "Makale Bülteni — vAttention" (cmlonder.com), section "İddia ve
// Gerçeklik: vAttention": the cache reserves, up front, a virtually
// contiguous buffer large enough for every sequence's maximum context, which
// costs no physical memory; physical pages are created and mapped into it
// only as sequences grow, so the attention kernels read one plain tensor and
// the GPU's page tables do the translation. The same section notes that the
// mapping calls are slow enough to need pre-allocation and deferred
// reclamation; here released pages stay mapped-out but allocated in a pool
// and are mapped again before new ones are created.
//
// Layout: K and V are each [max_seqs, Hkv, max_context, D] (the library's
// contiguous layout with seq_stride = max_context). The unit of mapping is a
// page of page_tokens rows of one (sequence, KV head) in one tensor, so
// a sequence of L tokens holds 2 * Hkv * ceil(L / page_tokens) pages.
//
// The same section has vAttention run the mapping calls ahead of need, off
// the critical path. kv_vcache_prefetch queues such a request for the
// cache's own mapping thread (started by the first request); a reserve that
// finds the pages mapped returns at once, and one that needs a page being
// mapped waits for it. All state is guarded by one mutex, held by whichever
// thread runs the mapping calls.

#include <hip/hip_runtime.h>

#include <condition_variable>
#include <deque>
#include <mutex>
#include <new>
#include <string>
#include <thread>
#include <utility>
#include <vector>

#include "kvpaged_internal.h"

struct kv_vcache {
  int device = 0;
  int32_t max_seqs = 0, max_context = 0, hkv = 0, head_dim = 0;
  int32_t page_tokens = 0;
  size_t esize = 0;
  size_t page_bytes = 0;
  size_t tensor_bytes = 0;         // reserved bytes of one tensor
  char* base[2] = {nullptr, nullptr};  // K, V
  std::vector<int32_t> pages;      // mapped pages per sequence (per region)
  // handles[((t * max_seqs + s) * hkv + g) * pages_per_region + p]
  std::vector<hipMemGenericAllocationHandle_t> handles;
  int32_t pages_per_region = 0;
  std::vector<hipMemGenericAllocationHandle_t> pool;  // created, not mapped
  int64_t mapped_pages = 0;
  int64_t created_pages = 0;
  // mapping thread
  mutable std::mutex mu;           // guards every field of the cache
  std::condition_variable cv;      // a request queued, or one served
  std::deque<std::pair<int32_t, int32_t>> queue;  // (seq, tokens) to back
  std::thread worker;
  bool stop = false;
  bool busy = false;               // the thread is serving a request
  kv_status async_status = KV_OK;  // first failure of a request since sync
  std::string async_msg;
};

namespace {

hipMemAllocationProp page_prop(int device) {
  hipMemAllocationProp prop = {};
  prop.type = hipMemAllocationTypePinned;
  prop.location.type = hipMemLocationTypeDevice;
  prop.location.id = device;
  return prop;
}

kv_status hip_fail(const char* what, hipError_t e) {
  return kvp_fail(e == hipErrorOutOfMemory ? KV_ENOMEM : KV_EHIP, "%s: %s",
                  what, hipGetErrorString(e));
}

// Wait for all work queued on the cache's device: a kernel still in flight
// may read pages that are about to be unmapped.
kv_status drain_device(const kv_vcache* c) {
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return hip_fail("kv_vcache: hipGetDevice", e);
  if (cur != c->device && (e = hipSetDevice(c->device)) != hipSuccess)
    return hip_fail("kv_vcache: hipSetDevice", e);
  e = hipDeviceSynchronize();
  if (cur != c->device) (void)hipSetDevice(cur);
  if (e != hipSuccess) return hip_fail("kv_vcache: hipDeviceSynchronize", e);
  return KV_OK;
}

// Unmap pages [keep, mapped) of every region of sequence s; their handles go
// back to the pool. With `drain`, the device's queued work is waited for
// first (false only when the caller has just done so).
kv_status unmap_tail(kv_vcache* c, int32_t s, int32_t keep,
                     bool drain = true) {
  const int32_t have = c->pages[s];
  if (have <= keep) return KV_OK;
  if (drain) {
    const kv_status st = drain_device(c);
    if (st != KV_OK) return st;
  }
  try {  // room in the pool for every handle unmapped below
    c->pool.reserve(c->pool.size() + (size_t)(have - keep) * 2 * c->hkv);
  } catch (const std::bad_alloc&) {
    return kvp_fail(KV_ENOMEM, "kv_vcache: host allocation");
  }
  for (int t = 0; t < 2; ++t)
    for (int32_t g = 0; g < c->hkv; ++g)
      for (int32_t p = keep; p < have; ++p) {
        const size_t region =
            ((size_t)t * c->max_seqs + s) * c->hkv + g;
        char* va = c->base[t] +
                   ((size_t)s * c->hkv + g) * c->max_context * c->head_dim *
                       c->esize +
                   (size_t)p * c->page_bytes;
        hipError_t e = hipMemUnmap(va, c->page_bytes);
        if (e != hipSuccess) return hip_fail("kv_vcache: hipMemUnmap", e);
        c->pool.push_back(c->handles[region * c->pages_per_region + p]);
        --c->mapped_pages;
      }
  c->pages[s] = keep;
  return KV_OK;
}

}  // namespace

extern "C" kv_status kv_vcache_granularity(size_t* bytes) {
  if (!bytes) return kvp_fail(KV_EINVAL, "kv_vcache_granularity: NULL");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail("kv_vcache_granularity: hipGetDevice", e);
  hipMemAllocationProp prop = page_prop(dev);
  e = hipMemGetAllocationGranularity(bytes, &prop,
                                     hipMemAllocationGranularityMinimum);
  if (e != hipSuccess)
    return hip_fail("kv_vcache_granularity: hipMemGetAllocationGranularity", e);
  return KV_OK;
}

extern "C" kv_status kv_vcache_create(int32_t max_seqs, int32_t max_context,
                                      int32_t num_kv_heads, int32_t head_dim,
                                      kv_dtype dtype, int32_t page_tokens,
                                      kv_vcache** out) {
  if (!out) return kvp_fail(KV_EINVAL, "kv_vcache_create: out is NULL");
  *out = nullptr;
  if (max_seqs <= 0 || max_context <= 0 || num_kv_heads <= 0 ||
      head_dim <= 0 || page_tokens <= 0 || page_tokens % 16 != 0 ||
      max_context % page_tokens != 0)
    return kvp_fail(KV_EINVAL,
                    "kv_vcache_create: bad shape (S=%d Lmax=%d Hkv=%d D=%d "
                    "page_tokens=%d; page_tokens must be a multiple of 16 "
                    "dividing Lmax)",
                    max_seqs, max_context, num_kv_heads, head_dim, page_tokens);
  if (dtype != KV_F32 && dtype != KV_BF16)
    return kvp_fail(KV_EINVAL, "kv_vcache_create: unknown dtype %d",
                    (int)dtype);
  const size_t esize = dtype == KV_F32 ? 4 : 2;
  const size_t page_bytes = (size_t)page_tokens * head_dim * esize;
  size_t gran = 0;
  kv_status st = kv_vcache_granularity(&gran);
  if (st != KV_OK) return st;
  if (gran == 0 || page_bytes % gran != 0)
    return kvp_fail(KV_EINVAL,
                    "kv_vcache_create: a page of %d tokens is %zu bytes, not "
                    "a multiple of the mapping granularity %zu",
                    page_tokens, page_bytes, gran);
  kv_vcache* c = new (std::nothrow) kv_vcache;
  if (!c) return kvp_fail(KV_ENOMEM, "kv_vcache_create: host allocation");
  hipError_t e = hipGetDevice(&c->device);
  if (e != hipSuccess) {
    delete c;
    return hip_fail("kv_vcache_create: hipGetDevice", e);
  }
  c->max_seqs = max_seqs;
  c->max_context = max_context;
  c->hkv = num_kv_heads;
  c->head_dim = head_dim;
  c->page_tokens = page_tokens;
  c->esize = esize;
  c->page_bytes = page_bytes;
  c->pages_per_region = max_context / page_tokens;
  c->tensor_bytes = (size_t)max_seqs * num_kv_heads * max_context * head_dim *
                    esize;
  try {
    c->pages.assign(max_seqs, 0);
    c->handles.assign((size_t)2 * max_seqs * num_kv_heads *
                          c->pages_per_region,
                      hipMemGenericAllocationHandle_t{});
  } catch (const std::bad_alloc&) {
    delete c;
    return kvp_fail(KV_ENOMEM, "kv_vcache_create: host allocation");
  }
  for (int t = 0; t < 2; ++t) {
    void* va = nullptr;
    e = hipMemAddressReserve(&va, c->tensor_bytes, 0, nullptr, 0);
    if (e != hipSuccess) {
      if (t == 1) (void)hipMemAddressFree(c->base[0], c->tensor_bytes);
      delete c;
      return hip_fail("kv_vcache_create: hipMemAddressReserve", e);
    }
    c->base[t] = (char*)va;
  }
  *out = c;
  return KV_OK;
}

extern "C" void kv_vcache_destroy(kv_vcache* c) {
  if (!c) return;
  {
    std::lock_guard<std::mutex> lk(c->mu);
    c->stop = true;
    c->queue.clear();
  }
  c->cv.notify_all();
  if (c->worker.joinable()) c->worker.join();
  (void)drain_device(c);  // nothing may still read the pages
  for (int32_t s = 0; s < c->max_seqs; ++s) (void)unmap_tail(c, s, 0, false);
  for (auto h : c->pool) (void)hipMemRelease(h);
  for (int t = 0; t < 2; ++t)
    if (c->base[t]) (void)hipMemAddressFree(c->base[t], c->tensor_bytes);
  delete c;
}

extern "C" kv_status kv_vcache_ptrs(const kv_vcache* c, void** k, void** v) {
  if (!c || !k || !v) return kvp_fail(KV_EINVAL, "kv_vcache_ptrs: NULL");
  *k = c->base[0];
  *v = c->base[1];
  return KV_OK;
}

namespace {

int32_t pages_for(const kv_vcache* c, int32_t tokens) {
  return (int32_t)(((int64_t)tokens + c->page_tokens - 1) / c->page_tokens);
}

// Map the pages of sequence seq below page `want` that are not mapped yet;
// *pages_mapped (may be NULL) = pages mapped here. The caller holds c->mu.
kv_status map_upto(kv_vcache* c, int32_t seq, int32_t want,
                   int32_t* pages_mapped) {
  const int32_t have = c->pages[seq];
  if (pages_mapped) *pages_mapped = 0;
  if (want <= have) return KV_OK;
  hipMemAllocationProp prop = page_prop(c->device);
  hipMemAccessDesc acc = {};
  acc.location.type = hipMemLocationTypeDevice;
  acc.location.id = c->device;
  acc.flags = hipMemAccessFlagsProtReadWrite;
  // Map page by page, region by region; on a failure, unmap what this call
  // mapped (handles back to the pool) so that the mapping is as it was.
  struct Done {
    char* va;
    hipMemGenericAllocationHandle_t h;
  };
  // Host storage for every page this call may map, and for returning them
  // to the pool, is reserved first: nothing below can throw (this also runs
  // on the mapping thread, where an escaping exception would end the
  // process).
  const size_t n_map = (size_t)(want - have) * 2 * c->hkv;
  std::vector<Done> done;
  try {
    done.reserve(n_map);
    c->pool.reserve(c->pool.size() + n_map);
  } catch (const std::bad_alloc&) {
    return kvp_fail(KV_ENOMEM, "kv_vcache: host allocation");
  }
  kv_status st = KV_OK;
  for (int32_t p = have; p < want && st == KV_OK; ++p)
    for (int t = 0; t < 2 && st == KV_OK; ++t)
      for (int32_t g = 0; g < c->hkv && st == KV_OK; ++g) {
        const size_t region = ((size_t)t * c->max_seqs + seq) * c->hkv + g;
        char* va = c->base[t] +
                   ((size_t)seq * c->hkv + g) * c->max_context * c->head_dim *
                       c->esize +
                   (size_t)p * c->page_bytes;
        hipMemGenericAllocationHandle_t h;
        bool fresh = false;
        if (!c->pool.empty()) {
          h = c->pool.back();
          c->pool.pop_back();
        } else {
          hipError_t e = hipMemCreate(&h, c->page_bytes, &prop, 0);
          if (e != hipSuccess) {
            st = hip_fail("kv_vcache: hipMemCreate", e);
            break;
          }
          fresh = true;
          ++c->created_pages;
        }
        hipError_t e = hipMemMap(va, c->page_bytes, 0, h, 0);
        if (e == hipSuccess) {
          e = hipMemSetAccess(va, c->page_bytes, &acc, 1);
          if (e != hipSuccess) (void)hipMemUnmap(va, c->page_bytes);
        }
        if (e != hipSuccess) {
          if (fresh) {
            (void)hipMemRelease(h);
            --c->created_pages;
          } else {
            c->pool.push_back(h);
          }
          st = hip_fail("kv_vcache: hipMemMap/hipMemSetAccess", e);
          break;
        }
        c->handles[region * c->pages_per_region + p] = h;
        done.push_back({va, h});
      }
  if (st != KV_OK) {
    for (size_t i = done.size(); i-- > 0;) {
      (void)hipMemUnmap(done[i].va, c->page_bytes);
      c->pool.push_back(done[i].h);
    }
    return st;
  }
  c->mapped_pages += (int64_t)done.size();
  c->pages[seq] = want;
  if (pages_mapped) *pages_mapped = (int32_t)done.size();
  return KV_OK;
}

// The mapping thread: serves queued requests in order until stopped.
void worker_main(kv_vcache* c) {
  (void)hipSetDevice(c->device);
  std::unique_lock<std::mutex> lk(c->mu);
  for (;;) {
    c->cv.wait(lk, [c] { return c->stop || !c->queue.empty(); });
    if (c->stop) return;
    const std::pair<int32_t, int32_t> r = c->queue.front();
    c->queue.pop_front();
    c->busy = true;
    const kv_status st = map_upto(c, r.first, pages_for(c, r.second), nullptr);
    if (st != KV_OK && c->async_status == KV_OK) {
      c->async_status = st;
      try {
        c->async_msg = kv_last_error();
      } catch (...) {
        c->async_msg.clear();  // the status alone is reported
      }
    }
    c->busy = false;
    c->cv.notify_all();
  }
}

}  // namespace

extern "C" kv_status kv_vcache_reserve(kv_vcache* c, int32_t seq,
                                       int32_t num_tokens,
                                       int32_t* pages_mapped) {
  if (!c) return kvp_fail(KV_EINVAL, "kv_vcache_reserve: cache is NULL");
  if (seq < 0 || seq >= c->max_seqs || num_tokens < 0 ||
      num_tokens > c->max_context)
    return kvp_fail(KV_EINVAL,
                    "kv_vcache_reserve: seq %d / tokens %d outside [0, %d) / "
                    "[0, %d]",
                    seq, num_tokens, c->max_seqs, c->max_context);
  std::lock_guard<std::mutex> lk(c->mu);
  return map_upto(c, seq, pages_for(c, num_tokens), pages_mapped);
}

extern "C" kv_status kv_vcache_prefetch(kv_vcache* c, int32_t seq,
                                        int32_t num_tokens) {
  if (!c) return kvp_fail(KV_EINVAL, "kv_vcache_prefetch: cache is NULL");
  if (seq < 0 || seq >= c->max_seqs || num_tokens < 0 ||
      num_tokens > c->max_context)
    return kvp_fail(KV_EINVAL,
                    "kv_vcache_prefetch: seq %d / tokens %d outside [0, %d) / "
                    "[0, %d]",
                    seq, num_tokens, c->max_seqs, c->max_context);
  std::lock_guard<std::mutex> lk(c->mu);
  if (pages_for(c, num_tokens) <= c->pages[seq]) return KV_OK;
  if (!c->worker.joinable()) {
    try {
      c->worker = std::thread(worker_main, c);
    } catch (...) {
      return kvp_fail(KV_ENOMEM, "kv_vcache_prefetch: cannot start the "
                      "mapping thread");
    }
  }
  try {
    c->queue.emplace_back(seq, num_tokens);
  } catch (const std::bad_alloc&) {
    return kvp_fail(KV_ENOMEM, "kv_vcache_prefetch: host allocation");
  }
  c->cv.notify_all();
  return KV_OK;
}

extern "C" kv_status kv_vcache_sync(kv_vcache* c) {
  if (!c) return kvp_fail(KV_EINVAL, "kv_vcache_sync: cache is NULL");
  std::unique_lock<std::mutex> lk(c->mu);
  c->cv.wait(lk, [c] { return c->queue.empty() && !c->busy; });
  const kv_status st = c->async_status;
  const std::string msg = c->async_msg;
  c->async_status = KV_OK;
  c->async_msg.clear();
  if (st != KV_OK) return kvp_fail(st, "kv_vcache_prefetch (earlier): %s",
                                   msg.c_str());
  return KV_OK;
}

extern "C" kv_status kv_vcache_release(kv_vcache* c, int32_t seq) {
  if (!c) return kvp_fail(KV_EINVAL, "kv_vcache_release: cache is NULL");
  if (seq < 0 || seq >= c->max_seqs)
    return kvp_fail(KV_EINVAL, "kv_vcache_release: seq %d outside [0, %d)",
                    seq, c->max_seqs);
  std::lock_guard<std::mutex> lk(c->mu);
  // queued requests for this sequence are dropped, not served later
  for (auto it = c->queue.begin(); it != c->queue.end();)
    it = it->first == seq ? c->queue.erase(it) : it + 1;
  return unmap_tail(c, seq, 0);
}

extern "C" int32_t kv_vcache_seq_pages(const kv_vcache* c, int32_t seq) {
  if (!c || seq < 0 || seq >= c->max_seqs) return -1;
  std::lock_guard<std::mutex> lk(c->mu);
  return c->pages[seq];
}

extern "C" int64_t kv_vcache_mapped_bytes(const kv_vcache* c) {
  if (!c) return -1;
  std::lock_guard<std::mutex> lk(c->mu);
  return c->mapped_pages * (int64_t)c->page_bytes;
}

extern "C" int64_t kv_vcache_held_bytes(const kv_vcache* c) {
  if (!c) return -1;
  std::lock_guard<std::mutex> lk(c->mu);
  return c->created_pages * (int64_t)c->page_bytes;
}
