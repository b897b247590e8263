// Internal declarations shared by the host and device translation units.
#pragma once
#include "../../include/kvpaged.h"

// Record a message for kv_last_error() and return `st`.
kv_status kvp_fail(kv_status st, const char* fmt, ...);

#include <hip/hip_runtime.h>

// Device address of a pointer the device can use: device memory as is,
// pinned host memory through its device mapping; NULL otherwise.
void* kvp_device_view(const void* p);

// One launch of the shared-prefix partial attention (prefill.hip): the
// decode queries of the members of each group against the group's shared
// tokens, read through the first member's table, split into nsplit pieces
// of ksplit keys. Writes plen[member] (shared tokens the member's own pass
// skips) and the partials po/pml. bf16, head_dim 128, block_size % 16 ==
// 0 (any Hq / Hkv).
struct KvpPrefixJob {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* bt;
  int32_t bt_stride;
  int32_t num_blocks;
  int32_t block_size;
  const int32_t* ctx;
  int32_t members;
  int32_t hq;
  int32_t hkv;
  const int32_t* group_starts;
  const int32_t* shared_lens;
  int32_t num_groups;
  int32_t max_group_size;
  int32_t nsplit;
  int32_t ksplit;
  float scale_log2;
  int32_t* plen;
  float* po;
  float* pml;
};
kv_status kvp_prefix_partials(const KvpPrefixJob& job, hipStream_t st);
