// Decode for callers that cannot allocate device memory (code under HIP
// graph capture, serving loops, harnesses that forbid hipMalloc): the same
// kernels as paged_attn_decode, with their workspace in a file-scope device
// array instead of a caller-supplied buffer. Each GPU holds its own copy of
// the array, found once per device with hipGetSymbolAddress; the host-side
// name of the array is not a device address and is never passed to a kernel.

#include <hip/hip_runtime.h>

#include <mutex>

#include "kvpaged_internal.h"

namespace {
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
__device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch array (the host-side symbol is
// not an address a kernel may use). NULL after recording an error.
void* scratch_for_current_device(const char* name) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    kvp_fail(KV_EHIP, "%s: no current device (or device id >= %d)", name,
             kMaxDevices);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      kvp_fail(KV_EHIP, "%s: hipGetSymbolAddress of the scratch array "
               "failed: %s", name, hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

extern "C" kv_status paged_attn_decode_noalloc(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    int32_t num_blocks, const int32_t* block_tables, int32_t bt_stride,
    const int32_t* context_lens, int32_t max_context, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, float scale, kv_dtype dtype, void* stream) {
  const char* name = "paged_attn_decode_noalloc";
  const size_t need = kv_decode_workspace_bytes(
      num_seqs, num_q_heads, num_kv_heads, head_dim, max_context);
  if (need > kNoAllocScratchBytes)
    return kvp_fail(KV_EINVAL, "%s: this shape needs %zu bytes of scratch, "
                    "more than the %zu the library holds per device", name,
                    need, kNoAllocScratchBytes);
  void* ws = nullptr;
  if (num_seqs > 0) {
    ws = scratch_for_current_device(name);
    if (!ws) return KV_EHIP;
  }
  return paged_attn_decode(out, q, k_cache, v_cache, num_blocks, block_tables,
                           bt_stride, context_lens, max_context, num_seqs,
                           num_q_heads, num_kv_heads, head_dim, block_size,
                           scale, dtype, ws, kNoAllocScratchBytes, stream);
}
