// Host side of the paged-KV library: block pool with refcounts and
// copy-on-write, sequence growth, slot mapping, and the error channel.
//
// Steps follow "PagedAttention Nedir?" (bitcanli.com), section
// "PagedAttention Nasıl Çalışır?" (blocks, on-demand allocation, block table,
// reuse), and "Makale Bülteni — PagedAttention ve vLLM", section "İddia ve
// Gerçeklik" (a free block is taken when the current one is full; shared
// blocks are copied on write). The pages leave the choice of free block
// open; this pool is a FIFO queue so that results are reproducible.

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <new>
#include <algorithm>
#include <vector>

#include "kvpaged_internal.h"

// ----------------------------------------------------------------- errors --
static thread_local char g_err[512] = "";

extern "C" const char* kv_last_error(void) { return g_err; }

kv_status kvp_fail(kv_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

// ------------------------------------------------------------------- pool --
// The free queue is a ring buffer of capacity num_blocks: a block is either
// in the queue or referenced, never both, so it can never overflow.
struct kv_pool {
  int32_t num_blocks;
  int32_t block_size;
  std::vector<int32_t> ring;
  int32_t head;   // index of the next block to hand out
  int32_t count;  // number of free blocks
  std::vector<int32_t> rc;

  int32_t pop() {
    int32_t b = ring[head];
    head = (head + 1 == num_blocks) ? 0 : head + 1;
    --count;
    return b;
  }
  void push(int32_t b) {
    int32_t tail = head + count;
    if (tail >= num_blocks) tail -= num_blocks;
    ring[tail] = b;
    ++count;
  }
  bool valid(int32_t b) const { return b >= 0 && b < num_blocks; }
};

extern "C" int64_t kv_blocks_needed(int64_t num_tokens, int32_t block_size) {
  if (num_tokens < 0 || block_size <= 0) return -1;
  return (num_tokens + block_size - 1) / block_size;
}

extern "C" kv_status kv_pool_create(int32_t num_blocks, int32_t block_size,
                                    const int32_t* init_free_order,
                                    kv_pool** out) {
  if (!out) return kvp_fail(KV_EINVAL, "kv_pool_create: out is NULL");
  *out = nullptr;
  if (num_blocks < 0 || block_size <= 0)
    return kvp_fail(KV_EINVAL, "kv_pool_create: num_blocks=%d block_size=%d",
                    num_blocks, block_size);
  kv_pool* p = new (std::nothrow) kv_pool;
  if (!p) return kvp_fail(KV_ENOMEM, "kv_pool_create: host allocation failed");
  p->num_blocks = num_blocks;
  p->block_size = block_size;
  p->head = 0;
  p->count = num_blocks;
  std::vector<char> seen;
  try {
    p->ring.assign(num_blocks, 0);
    p->rc.assign(num_blocks, 0);
    if (init_free_order) seen.assign(num_blocks, 0);
  } catch (const std::bad_alloc&) {
    delete p;
    return kvp_fail(KV_ENOMEM, "kv_pool_create: host allocation failed");
  }
  if (init_free_order) {
    for (int32_t i = 0; i < num_blocks; ++i) {
      int32_t b = init_free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete p;
        return kvp_fail(KV_EINVAL,
                        "kv_pool_create: init_free_order is not a permutation "
                        "(entry %d = %d)", i, b);
      }
      seen[b] = 1;
      p->ring[i] = b;
    }
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) p->ring[i] = i;
  }
  *out = p;
  return KV_OK;
}

extern "C" void kv_pool_destroy(kv_pool* pool) { delete pool; }

extern "C" kv_status kv_block_alloc(kv_pool* pool, int32_t n,
                                    int32_t* out_ids) {
  if (!pool || n < 0 || (n > 0 && !out_ids))
    return kvp_fail(KV_EINVAL, "kv_block_alloc: bad argument (n=%d)", n);
  if (n > pool->count)
    return kvp_fail(KV_ENOMEM, "kv_block_alloc: %d blocks asked, %d free", n,
                    pool->count);
  for (int32_t i = 0; i < n; ++i) {
    int32_t b = pool->pop();
    pool->rc[b] = 1;
    out_ids[i] = b;
  }
  return KV_OK;
}

extern "C" kv_status kv_block_free(kv_pool* pool, int32_t n,
                                   const int32_t* ids) {
  if (!pool || n < 0 || (n > 0 && !ids))
    return kvp_fail(KV_EINVAL, "kv_block_free: bad argument (n=%d)", n);
  for (int32_t i = 0; i < n; ++i)
    if (!pool->valid(ids[i]))
      return kvp_fail(KV_EINVAL, "kv_block_free: id %d outside the pool",
                      ids[i]);
  // An id may repeat: check the total drop per id before changing anything.
  std::vector<int32_t> drop;
  try {
    drop.assign(pool->num_blocks, 0);
  } catch (const std::bad_alloc&) {
    return kvp_fail(KV_ENOMEM, "kv_block_free: host allocation failed");
  }
  for (int32_t i = 0; i < n; ++i) ++drop[ids[i]];
  for (int32_t i = 0; i < n; ++i)
    if (drop[ids[i]] > pool->rc[ids[i]])
      return kvp_fail(KV_EREFCOUNT,
                      "kv_block_free: block %d has refcount %d, %d drops",
                      ids[i], pool->rc[ids[i]], drop[ids[i]]);
  for (int32_t i = 0; i < n; ++i) {
    int32_t b = ids[i];
    if (--pool->rc[b] == 0) pool->push(b);
  }
  return KV_OK;
}

extern "C" kv_status kv_block_share(kv_pool* pool, int32_t n,
                                    const int32_t* ids) {
  if (!pool || n < 0 || (n > 0 && !ids))
    return kvp_fail(KV_EINVAL, "kv_block_share: bad argument (n=%d)", n);
  for (int32_t i = 0; i < n; ++i)
    if (!pool->valid(ids[i]))
      return kvp_fail(KV_EINVAL, "kv_block_share: id %d outside the pool",
                      ids[i]);
  for (int32_t i = 0; i < n; ++i)
    if (pool->rc[ids[i]] == 0)
      return kvp_fail(KV_EREFCOUNT, "kv_block_share: block %d is free",
                      ids[i]);
  for (int32_t i = 0; i < n; ++i) ++pool->rc[ids[i]];
  return KV_OK;
}

extern "C" kv_status kv_block_cow(kv_pool* pool, int32_t id, int32_t* out_id,
                                  int32_t* need_copy) {
  if (!pool || !out_id || !need_copy)
    return kvp_fail(KV_EINVAL, "kv_block_cow: NULL argument");
  if (!pool->valid(id))
    return kvp_fail(KV_EINVAL, "kv_block_cow: id %d outside the pool", id);
  if (pool->rc[id] == 0)
    return kvp_fail(KV_EREFCOUNT, "kv_block_cow: block %d is free", id);
  if (pool->rc[id] == 1) {
    *out_id = id;
    *need_copy = 0;
    return KV_OK;
  }
  if (pool->count == 0)
    return kvp_fail(KV_ENOMEM, "kv_block_cow: no free block for the copy");
  int32_t b = pool->pop();
  pool->rc[b] = 1;
  --pool->rc[id];
  *out_id = b;
  *need_copy = 1;
  return KV_OK;
}

extern "C" int32_t kv_block_refcount(const kv_pool* pool, int32_t id) {
  if (!pool || !pool->valid(id)) return KV_EINVAL;
  return pool->rc[id];
}

extern "C" int32_t kv_pool_num_free(const kv_pool* pool) {
  return pool ? pool->count : KV_EINVAL;
}
extern "C" int32_t kv_pool_num_blocks(const kv_pool* pool) {
  return pool ? pool->num_blocks : KV_EINVAL;
}
extern "C" int32_t kv_pool_block_size(const kv_pool* pool) {
  return pool ? pool->block_size : KV_EINVAL;
}

extern "C" int32_t kv_pool_free_list(const kv_pool* pool, int32_t* out,
                                     int32_t cap) {
  if (!pool) return KV_EINVAL;
  int32_t idx = pool->head;
  for (int32_t i = 0; i < pool->count && i < cap && out; ++i) {
    out[i] = pool->ring[idx];
    idx = (idx + 1 == pool->num_blocks) ? 0 : idx + 1;
  }
  return pool->count;
}

// ------------------------------------------------------- sequence growth --
// Undo-log entry: a failing batch leaves pool, tables and lengths as they
// were.
namespace {
struct TableEdit {
  int32_t* where;
  int32_t old;
};
}  // namespace

extern "C" kv_status kv_seq_append(kv_pool* pool, int32_t* block_tables,
                                   int32_t bt_stride, int32_t* seq_lens,
                                   const int32_t* n_new, int32_t num_seqs,
                                   int64_t* out_slots, int32_t* out_cow_pairs,
                                   int32_t cow_capacity,
                                   int32_t* out_num_cow) {
  if (!pool || !block_tables || !seq_lens || num_seqs < 0 || bt_stride <= 0 ||
      cow_capacity < 0 || (cow_capacity > 0 && !out_cow_pairs))
    return kvp_fail(KV_EINVAL, "kv_seq_append: bad argument");
  const int32_t B = pool->block_size;
  int64_t total = 0;
  for (int32_t s = 0; s < num_seqs; ++s) total += n_new ? (n_new[s] > 0 ? n_new[s] : 0) : 1;
  if (total > 0 && !out_slots)
    return kvp_fail(KV_EINVAL, "kv_seq_append: out_slots is NULL");

  // Appending only pops from the free queue (never pushes), so a rollback
  // restores head/count and replays the undo logs of refcounts and table
  // entries in reverse.
  const int32_t saved_head = pool->head, saved_count = pool->count;
  std::vector<TableEdit> edits, rc_edits;
  // Room for every undo record first, so that nothing below can throw: a
  // sequence takes at most add / B + 1 new blocks (one table and one
  // refcount record each) and copies at most one shared block (one table
  // and two refcount records).
  {
    const int64_t fresh = std::min<int64_t>(pool->count, total / B + num_seqs);
    const int64_t cows = std::min<int64_t>(cow_capacity, num_seqs);
    try {
      edits.reserve((size_t)(fresh + cows));
      rc_edits.reserve((size_t)(fresh + 2 * cows));
    } catch (const std::bad_alloc&) {
      return kvp_fail(KV_ENOMEM, "kv_seq_append: host allocation failed");
    }
  }
  auto set_rc = [&](int32_t b, int32_t v) {
    rc_edits.push_back({&pool->rc[b], pool->rc[b]});
    pool->rc[b] = v;
  };
  auto rollback = [&](kv_status st, const char* what, int32_t s) {
    for (size_t i = rc_edits.size(); i-- > 0;) *rc_edits[i].where = rc_edits[i].old;
    pool->head = saved_head;
    pool->count = saved_count;
    for (size_t i = edits.size(); i-- > 0;) *edits[i].where = edits[i].old;
    return kvp_fail(st, "kv_seq_append: seq %d: %s", s, what);
  };

  int64_t k = 0;
  int32_t ncow = 0;
  for (int32_t s = 0; s < num_seqs; ++s) {
    int32_t add = n_new ? n_new[s] : 1;
    int32_t* row = block_tables + (int64_t)s * bt_stride;
    int32_t len = seq_lens[s];
    if (add < 0 || len < 0)
      return rollback(KV_EINVAL, "negative length or token count", s);
    for (int32_t t = 0; t < add; ++t) {
      int32_t p = len + t;
      int32_t lb = p / B, off = p % B;
      if (lb >= bt_stride)
        return rollback(KV_EINVAL, "table row too short", s);
      if (off == 0) {
        if (pool->count == 0) return rollback(KV_ENOMEM, "pool exhausted", s);
        int32_t b = pool->pop();
        set_rc(b, 1);
        edits.push_back({row + lb, row[lb]});
        row[lb] = b;
      } else {
        int32_t b = row[lb];
        if (!pool->valid(b))
          return rollback(KV_EINVAL, "table entry outside the pool", s);
        if (pool->rc[b] == 0)
          return rollback(KV_EREFCOUNT, "table names a free block", s);
        if (pool->rc[b] > 1) {
          if (pool->count == 0)
            return rollback(KV_ENOMEM, "no free block for copy-on-write", s);
          if (ncow >= cow_capacity)
            return rollback(KV_EINVAL, "cow_capacity too small", s);
          int32_t nb = pool->pop();
          set_rc(nb, 1);
          set_rc(b, pool->rc[b] - 1);
          out_cow_pairs[2 * ncow] = b;
          out_cow_pairs[2 * ncow + 1] = nb;
          ++ncow;
          edits.push_back({row + lb, b});
          row[lb] = nb;
        }
      }
      out_slots[k++] = (int64_t)row[lb] * B + off;
    }
  }
  for (int32_t s = 0; s < num_seqs; ++s) seq_lens[s] += n_new ? n_new[s] : 1;
  if (out_num_cow) *out_num_cow = ncow;
  return KV_OK;
}

extern "C" kv_status kv_slot_mapping(const int32_t* block_tables,
                                     int32_t bt_stride, const int32_t* seq_ids,
                                     const int32_t* positions, int32_t n,
                                     int32_t block_size, int64_t* out_slots) {
  if (n < 0 || block_size <= 0 || bt_stride <= 0 ||
      (n > 0 && (!block_tables || !seq_ids || !positions || !out_slots)))
    return kvp_fail(KV_EINVAL, "kv_slot_mapping: bad argument");
  for (int32_t i = 0; i < n; ++i) {
    int32_t p = positions[i];
    if (p < 0) {
      out_slots[i] = -1;
      continue;
    }
    int32_t lb = p / block_size;
    if (lb >= bt_stride || seq_ids[i] < 0)
      return kvp_fail(KV_EINVAL,
                      "kv_slot_mapping: entry %d (seq %d, pos %d) outside the "
                      "table", i, seq_ids[i], p);
    out_slots[i] = (int64_t)block_tables[(int64_t)seq_ids[i] * bt_stride + lb] *
                       block_size + p % block_size;
  }
  return KV_OK;
}
