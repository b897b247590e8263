// Prefix cache: finds the blocks of a block pool that already hold the K/V
// of a prompt's leading tokens.
//
// Follows "PagedAttention Nedir?" (bitcanli.com), section "Prefix Sharing
// Nasıl Çalışır?": K/V computed for the common start of requests is reused
// only when the token sequence matches under the same model context; the
// keys that find reusable blocks take both a block's contents and the
// context before it into account; reuse needs the blocks to still be
// cached.
//
// Rules (fixed so that results are reproducible):
//   * only full blocks are keyed. Key of block i = FNV-1a-64 (Fowler, Noll,
//     Vo) over the little-endian bytes of (key of block i-1, 0 for the
//     first; salt; the block's token ids as int32). The salt stands for the
//     model and adapter context;
//   * an entry keeps its block id, parent key and token ids, and a key
//     matches only if those are equal: a hash collision is a miss;
//   * lookup walks a prompt's full blocks from the first and stops at the
//     first miss; each block found gets one more pool reference for the
//     caller;
//   * insert walks the same chain over the caller's blocks: a missing key is
//     added and the cache takes one reference to the caller's block; an equal
//     entry is kept; a colliding key ends the walk;
//   * every block a lookup or insert passes is stamped with an increasing
//     tick, from the chain's last block to its first, so chains age tail
//     first; evict frees the blocks only the cache references (refcount 1),
//     oldest stamp first.

#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <unordered_map>
#include <vector>

#include "kvpaged_internal.h"

namespace {

constexpr uint64_t kFnvOffset = 0xCBF29CE484222325ull;
constexpr uint64_t kFnvPrime = 0x100000001B3ull;

uint64_t fnv1a(const unsigned char* p, size_t n, uint64_t h) {
  for (size_t i = 0; i < n; ++i) {
    h ^= p[i];
    h *= kFnvPrime;
  }
  return h;
}

void put_le(unsigned char* out, uint64_t v, int bytes) {
  for (int i = 0; i < bytes; ++i) out[i] = (unsigned char)(v >> (8 * i));
}

struct Entry {
  int32_t block;
  uint64_t parent;
  std::vector<int32_t> tokens;
  uint64_t last_use;
};

}  // namespace

struct kv_prefix_cache {
  kv_pool* pool = nullptr;
  int32_t block_size = 0;
  uint64_t salt = 0;
  uint64_t tick = 0;
  std::unordered_map<uint64_t, Entry> entries;
};

extern "C" uint64_t kv_prefix_block_key(uint64_t parent, uint64_t salt,
                                        const int32_t* tokens, int32_t n) {
  unsigned char w[8];
  uint64_t h = kFnvOffset;
  put_le(w, parent, 8);
  h = fnv1a(w, 8, h);
  put_le(w, salt, 8);
  h = fnv1a(w, 8, h);
  for (int32_t i = 0; i < n; ++i) {
    put_le(w, (uint32_t)tokens[i], 4);
    h = fnv1a(w, 4, h);
  }
  return h;
}

extern "C" kv_status kv_prefix_cache_create(kv_pool* pool, uint64_t salt,
                                            kv_prefix_cache** out) {
  if (!pool || !out)
    return kvp_fail(KV_EINVAL, "kv_prefix_cache_create: NULL argument");
  kv_prefix_cache* c = new (std::nothrow) kv_prefix_cache;
  if (!c) return kvp_fail(KV_ENOMEM, "kv_prefix_cache_create: host allocation");
  c->pool = pool;
  c->block_size = kv_pool_block_size(pool);
  c->salt = salt;
  *out = c;
  return KV_OK;
}

extern "C" void kv_prefix_cache_destroy(kv_prefix_cache* c) {
  if (!c) return;
  for (auto& kvp : c->entries) {
    const int32_t b = kvp.second.block;
    (void)kv_block_free(c->pool, 1, &b);
  }
  delete c;
}

namespace {

// Walk the full blocks of tokens[0, n): for each, its key and parent key.
struct Link {
  uint64_t key, parent;
  const int32_t* toks;
};

std::vector<Link> chain(const kv_prefix_cache* c, const int32_t* tokens,
                        int32_t n) {
  std::vector<Link> out;
  const int32_t B = c->block_size;
  uint64_t parent = 0;
  for (int32_t i = 0; i + B <= n; i += B) {
    const uint64_t k = kv_prefix_block_key(parent, c->salt, tokens + i, B);
    out.push_back({k, parent, tokens + i});
    parent = k;
  }
  return out;
}

bool equal_entry(const Entry& e, const Link& l, int32_t B) {
  return e.parent == l.parent &&
         memcmp(e.tokens.data(), l.toks, (size_t)B * sizeof(int32_t)) == 0;
}

void touch(kv_prefix_cache* c, const std::vector<Entry*>& passed) {
  for (size_t i = passed.size(); i-- > 0;) passed[i]->last_use = ++c->tick;
}

}  // namespace

extern "C" kv_status kv_prefix_cache_lookup(kv_prefix_cache* c,
                                            const int32_t* tokens, int32_t n,
                                            int32_t* out_blocks,
                                            int32_t* num_blocks) {
  if (!c || !num_blocks || n < 0 || (n > 0 && !tokens) ||
      (n >= c->block_size && !out_blocks))
    return kvp_fail(KV_EINVAL, "kv_prefix_cache_lookup: bad argument");
  std::vector<Entry*> found;
  try {
    for (const Link& l : chain(c, tokens, n)) {
      auto it = c->entries.find(l.key);
      if (it == c->entries.end() || !equal_entry(it->second, l, c->block_size))
        break;
      found.push_back(&it->second);
    }
  } catch (const std::bad_alloc&) {
    return kvp_fail(KV_ENOMEM, "kv_prefix_cache_lookup: host allocation");
  }
  std::vector<int32_t> ids;
  try {
    ids.resize(found.size());
  } catch (const std::bad_alloc&) {
    return kvp_fail(KV_ENOMEM, "kv_prefix_cache_lookup: host allocation");
  }
  for (size_t i = 0; i < found.size(); ++i) ids[i] = found[i]->block;
  if (!ids.empty()) {
    const kv_status st = kv_block_share(c->pool, (int32_t)ids.size(),
                                        ids.data());
    if (st != KV_OK) return st;  // a cached block was freed behind the cache
    memcpy(out_blocks, ids.data(), ids.size() * sizeof(int32_t));
  }
  touch(c, found);
  *num_blocks = (int32_t)ids.size();
  return KV_OK;
}

extern "C" kv_status kv_prefix_cache_insert(kv_prefix_cache* c,
                                            const int32_t* tokens, int32_t n,
                                            const int32_t* blocks,
                                            int32_t* num_inserted) {
  if (!c || n < 0 || (n > 0 && !tokens) || (n >= c->block_size && !blocks))
    return kvp_fail(KV_EINVAL, "kv_prefix_cache_insert: bad argument");
  const int32_t B = c->block_size;
  std::vector<Link> links;
  try {
    links = chain(c, tokens, n);
  } catch (const std::bad_alloc&) {
    return kvp_fail(KV_ENOMEM, "kv_prefix_cache_insert: host allocation");
  }
  // Validate first (all-or-nothing): the blocks to be added must be live.
  size_t stop = links.size();
  for (size_t i = 0; i < links.size(); ++i) {
    auto it = c->entries.find(links[i].key);
    if (it != c->entries.end()) {
      if (!equal_entry(it->second, links[i], B)) {
        stop = i;
        break;
      }
      continue;
    }
    if (kv_block_refcount(c->pool, blocks[i]) <= 0)
      return kvp_fail(KV_EINVAL,
                      "kv_prefix_cache_insert: block %d (chain position %zu) "
                      "is not a live block of the pool",
                      blocks[i], i);
  }
  std::vector<Entry*> passed;
  int32_t added = 0;
  try {
    for (size_t i = 0; i < stop; ++i) {
      auto it = c->entries.find(links[i].key);
      if (it == c->entries.end()) {
        Entry e;
        e.block = blocks[i];
        e.parent = links[i].parent;
        e.tokens.assign(links[i].toks, links[i].toks + B);
        e.last_use = 0;
        const kv_status st = kv_block_share(c->pool, 1, &e.block);
        if (st != KV_OK) return st;  // not reached: validated above
        it = c->entries.emplace(links[i].key, std::move(e)).first;
        ++added;
      }
      passed.push_back(&it->second);
    }
  } catch (const std::bad_alloc&) {
    return kvp_fail(KV_ENOMEM, "kv_prefix_cache_insert: host allocation");
  }
  touch(c, passed);
  if (num_inserted) *num_inserted = added;
  return KV_OK;
}

extern "C" int32_t kv_prefix_cache_evict(kv_prefix_cache* c, int32_t n,
                                         int32_t* freed) {
  if (!c || n < 0) {
    kvp_fail(KV_EINVAL, "kv_prefix_cache_evict: bad argument");
    return -1;
  }
  std::vector<std::pair<uint64_t, uint64_t>> cands;  // (last_use, key)
  try {
    for (auto& kvp : c->entries)
      if (kv_block_refcount(c->pool, kvp.second.block) == 1)
        cands.push_back({kvp.second.last_use, kvp.first});
  } catch (const std::bad_alloc&) {
    kvp_fail(KV_ENOMEM, "kv_prefix_cache_evict: host allocation");
    return -1;
  }
  std::sort(cands.begin(), cands.end());
  int32_t done = 0;
  for (size_t i = 0; i < cands.size() && done < n; ++i) {
    auto it = c->entries.find(cands[i].second);
    const int32_t b = it->second.block;
    if (kv_block_free(c->pool, 1, &b) != KV_OK) break;
    c->entries.erase(it);
    if (freed) freed[done] = b;
    ++done;
  }
  return done;
}

extern "C" int32_t kv_prefix_cache_size(const kv_prefix_cache* c) {
  return c ? (int32_t)c->entries.size() : -1;
}
