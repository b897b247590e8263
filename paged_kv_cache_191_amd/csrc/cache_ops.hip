// Cache writes: the slot-mapped row scatter of new K/V tokens and the
// whole-block copies of copy-on-write.
//
// A new token's K and V rows go into the slot its block table assigns
// ["PagedAttention Nedir?" (bitcanli.com), "PagedAttention Nasıl Çalışır?",
// steps 2-3]; a shared block is copied before it is written
// ["Makale Bülteni — PagedAttention ve vLLM", "İddia ve Gerçeklik"].
// Both are plain byte moves bounded by HBM bandwidth: each head row is moved
// in 16-byte (or 4/2-byte) units, consecutive lanes on consecutive units.
// Caches are head-major inside a block: [blocks, Hkv, block_size, D].

#include "device_common.h"
#include "fp8_codec.h"

namespace {

using namespace kvp;

// Rows of `per_token` units (Hkv heads x units_per_head) per token; a
// workgroup of 256 threads covers `tpb` = 256 / per_token tokens at a time
// (per_token <= 256), thread (token k, unit u) moving unit u of K and of V,
// so the index arithmetic is done once per thread and the loop only walks
// tokens. Destinations are head-major inside a block: unit u of head h of
// slot goes to ((slot / B) * Hkv + h) * B + slot % B (in head rows).
// bs_shift = log2(B) for power-of-two block sizes (else -1).
template <typename U>
__global__ __launch_bounds__(256) void scatter_rows_kernel(
    const U* __restrict__ k, const U* __restrict__ v,
    const int64_t* __restrict__ slots, int32_t num_tokens, U* k_cache,
    U* v_cache, int64_t num_slots, int32_t block_size, int32_t bs_shift,
    int32_t num_kv_heads, int32_t units_per_head) {
  const int per_token = num_kv_heads * units_per_head;
  const int tpb = blockDim.x / per_token;
  const int tk = threadIdx.x / per_token;
  if (tk >= tpb) return;
  const int u = threadIdx.x - tk * per_token;
  const int h = u / units_per_head;
  const int uu = u - h * units_per_head;
  for (int64_t t = (int64_t)blockIdx.x * tpb + tk; t < num_tokens;
       t += (int64_t)gridDim.x * tpb) {
    const int64_t slot = slots[t];
    if (slot < 0 || slot >= num_slots) continue;
    int64_t blk, off;
    if (bs_shift >= 0) {
      blk = slot >> bs_shift;
      off = slot & (block_size - 1);
    } else {
      blk = slot / block_size;
      off = slot - blk * block_size;
    }
    const int64_t src = t * per_token + u;
    const int64_t dst =
        ((blk * num_kv_heads + h) * block_size + off) * units_per_head + uu;
    const U kx = k[src];
    const U vx = v[src];
    k_cache[dst] = kx;
    v_cache[dst] = vx;
  }
}

// The same for rows of more than 256 units: one item = one unit of one
// token (K and V).
template <typename U>
__global__ __launch_bounds__(256) void scatter_wide_rows_kernel(
    const U* __restrict__ k, const U* __restrict__ v,
    const int64_t* __restrict__ slots, int32_t num_tokens, U* k_cache,
    U* v_cache, int64_t num_slots, int32_t block_size, int32_t num_kv_heads,
    int32_t units_per_head) {
  const int64_t per_token = (int64_t)num_kv_heads * units_per_head;
  const int64_t total = (int64_t)num_tokens * per_token;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / per_token;
    const int64_t r = i - t * per_token;
    const int64_t h = r / units_per_head;
    const int64_t uu = r - h * units_per_head;
    const int64_t slot = slots[t];
    if (slot < 0 || slot >= num_slots) continue;
    const int64_t blk = slot / block_size;
    const int64_t off = slot - blk * block_size;
    const int64_t dst =
        ((blk * num_kv_heads + h) * block_size + off) * units_per_head + uu;
    k_cache[dst] = k[i];
    v_cache[dst] = v[i];
  }
}

// Pairs are independent (no destination is read or written by another
// pair), so they are copied in parallel: blockIdx.y walks the pairs,
// blockIdx.x/threads walk the units of one block of K and of V.
template <typename U>
__global__ __launch_bounds__(256) void copy_blocks_kernel(
    U* k_cache, U* v_cache, const int32_t* __restrict__ src_dst, int32_t n,
    int32_t num_blocks, int64_t units_per_block) {
  const int64_t total = 2 * units_per_block;
  for (int32_t p = blockIdx.y; p < n; p += gridDim.y) {
    const int32_t src = src_dst[2 * p], dst = src_dst[2 * p + 1];
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) continue;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
      const bool is_v = i >= units_per_block;
      const int64_t u = is_v ? i - units_per_block : i;
      U* c = is_v ? v_cache : k_cache;
      c[(int64_t)dst * units_per_block + u] =
          c[(int64_t)src * units_per_block + u];
    }
  }
}

// One workgroup per sequence: the table entry of the new token's logical
// block (patched first when the host took a new block), its slot, the K and
// V rows of every head in unit-sized pieces, then the length. Only this
// workgroup touches row s of the table and context_lens[s]. Src/Dst: a unit
// of the source row and of the cache (the same type, copied; or 8 bf16
// values -> 8 fp8 E4M3 codes, quantised with 1 / scale by `Conv`).
template <typename Src, typename Dst, typename Conv>
__global__ __launch_bounds__(256) void append_token_kernel(
    const Src* __restrict__ k, const Src* __restrict__ v,
    const int32_t* new_blocks, int32_t* bt, int32_t bt_stride, int32_t* ctx,
    Dst* k_cache, Dst* v_cache, int32_t num_blocks, int32_t block_size,
    int32_t num_kv_heads, int32_t units_per_head, Conv conv) {
  const int s = blockIdx.x;
  const int L = ctx[s];
  const int nb = new_blocks[s];
  const bool ok_pos = L >= 0 && (int64_t)L < (int64_t)bt_stride * block_size;
  const int idx = ok_pos ? L / block_size : 0;
  int32_t* entry = bt + (int64_t)s * bt_stride + idx;
  const int blk = nb >= 0 ? nb : (ok_pos ? *entry : -1);
  const bool ok = ok_pos && blk >= 0 && blk < num_blocks;
  if (ok) {
    const int64_t off = L - (int64_t)idx * block_size;
    const int64_t per_tensor = (int64_t)num_kv_heads * units_per_head;
    for (int64_t i = threadIdx.x; i < 2 * per_tensor; i += blockDim.x) {
      const bool is_v = i >= per_tensor;
      const int64_t r = is_v ? i - per_tensor : i;
      const int64_t h = r / units_per_head;
      const int64_t u = r - h * units_per_head;
      const Src* src = is_v ? v : k;
      Dst* dst = is_v ? v_cache : k_cache;
      dst[(((int64_t)blk * num_kv_heads + h) * block_size + off) *
              units_per_head + u] =
          conv(src[(int64_t)s * per_tensor + r], is_v, h);
    }
  }
  // every thread has read ctx[s] and the table entry before they change
  __syncthreads();
  if (ok && threadIdx.x == 0) {
    if (nb >= 0) *entry = nb;
    ctx[s] = L + 1;
  }
}

struct CopyUnit {
  template <typename U>
  __device__ U operator()(U x, bool, int64_t) const { return x; }
};

size_t elem_size(kv_dtype dt) { return dt == KV_F32 ? 4 : 2; }

// fp8 variant of scatter_rows_kernel: one item = 8 values of one head row
// (16 source bytes of bf16 -> 8 cache bytes of codes).
__global__ __launch_bounds__(256) void scatter_rows_fp8_kernel(
    const u32x4* __restrict__ k, const u32x4* __restrict__ v,
    const int64_t* __restrict__ slots, int32_t num_tokens, u32x2* k_cache,
    u32x2* v_cache, int64_t num_slots, int32_t block_size,
    int32_t num_kv_heads, int32_t units_per_head, float k_inv, float v_inv,
    const float* __restrict__ k_scales, const float* __restrict__ v_scales) {
  const int64_t per_token = (int64_t)num_kv_heads * units_per_head;
  const int64_t per_tensor = (int64_t)num_tokens * per_token;
  const int64_t total = 2 * per_tensor;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const bool is_v = i >= per_tensor;
    const int64_t j = is_v ? i - per_tensor : i;
    const int64_t t = j / per_token;
    const int64_t r = j - t * per_token;
    const int64_t h = r / units_per_head;
    const int64_t u = r - h * units_per_head;
    const int64_t slot = slots[t];
    if (slot < 0 || slot >= num_slots) continue;
    const int64_t blk = slot / block_size;
    const int64_t off = slot - blk * block_size;
    const u32x4 x = (is_v ? v : k)[t * per_token + r];
    const float inv =
        is_v ? fp8_inv(v_scales, v_inv, h) : fp8_inv(k_scales, k_inv, h);
    u32x2 c;
    c[0] = fp8_pack4(x[0], x[1], inv);
    c[1] = fp8_pack4(x[2], x[3], inv);
    (is_v ? v_cache : k_cache)
        [((blk * num_kv_heads + h) * block_size + off) * units_per_head + u] =
        c;
  }
}

// 8 bf16 values of head h -> 8 E4M3 codes, with the K or V scale (per
// tensor, or per head when the arrays are given)
struct Fp8Unit {
  float k_inv, v_inv;
  const float* k_scales;
  const float* v_scales;
  __device__ u32x2 operator()(u32x4 x, bool is_v, int64_t h) const {
    const float inv =
        is_v ? fp8_inv(v_scales, v_inv, h) : fp8_inv(k_scales, k_inv, h);
    u32x2 c;
    c[0] = fp8_pack4(x[0], x[1], inv);
    c[1] = fp8_pack4(x[2], x[3], inv);
    return c;
  }
};

}  // namespace

namespace {
// Shared body of the fp8 cache writes: one scale per tensor (k_scale,
// v_scale) or, when k_scales / v_scales are given, one per KV head.
kv_status reshape_and_cache_fp8(const char* name, const void* k,
                                const void* v, const int64_t* slots,
                                int32_t num_tokens, void* k_cache,
                                void* v_cache, int64_t num_slots,
                                int32_t block_size, int32_t num_kv_heads,
                                int32_t head_dim, float k_scale, float v_scale,
                                const float* k_scales, const float* v_scales,
                                void* stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      head_dim % 8 != 0 || num_slots < 0 || block_size <= 0 ||
      num_slots % block_size != 0)
    return kvp_fail(KV_EINVAL, "%s: bad shape (D=%d slots=%lld block_size=%d;"
                    " D must be a multiple of 8)", name, head_dim,
                    (long long)num_slots, block_size);
  if (!(k_scale > 0.f) || !(k_scale < INFINITY) || !(v_scale > 0.f) ||
      !(v_scale < INFINITY))
    return kvp_fail(KV_EINVAL, "%s: k_scale and v_scale must be finite and "
                    "> 0", name);
  if (num_tokens == 0) return KV_OK;
  if (!k || !v || !slots || !k_cache || !v_cache)
    return kvp_fail(KV_EINVAL, "%s: NULL pointer", name);
  if (((uintptr_t)k | (uintptr_t)v) % 16 || ((uintptr_t)k_cache |
                                              (uintptr_t)v_cache) % 8)
    return kvp_fail(KV_EINVAL, "%s: k/v must be 16-byte and the caches "
                    "8-byte aligned", name);
  const float k_inv = 1.f / k_scale, v_inv = 1.f / v_scale;
  hipStream_t st = (hipStream_t)stream;
  const int threads = 256;
  const int32_t uph = head_dim / 8;
  const int64_t items = 2 * (int64_t)num_tokens * num_kv_heads * uph;
  const int64_t g = (items + threads - 1) / threads;
  scatter_rows_fp8_kernel<<<(int)(g < 65536 ? g : 65536), threads, 0, st>>>(
      (const u32x4*)k, (const u32x4*)v, slots, num_tokens, (u32x2*)k_cache,
      (u32x2*)v_cache, num_slots, block_size, num_kv_heads, uph, k_inv, v_inv,
      k_scales, v_scales);
  KVP_LAUNCH_CHECK(name);
  return KV_OK;
}
}  // namespace

extern "C" kv_status kv_reshape_and_cache_fp8(
    const void* k, const void* v, const int64_t* slots, int32_t num_tokens,
    void* k_cache, void* v_cache, int64_t num_slots, int32_t block_size,
    int32_t num_kv_heads, int32_t head_dim, float k_scale, float v_scale,
    void* stream) {
  return reshape_and_cache_fp8("kv_reshape_and_cache_fp8", k, v, slots,
                               num_tokens, k_cache, v_cache, num_slots,
                               block_size, num_kv_heads, head_dim, k_scale,
                               v_scale, nullptr, nullptr, stream);
}

extern "C" kv_status kv_reshape_and_cache_fp8_per_head(
    const void* k, const void* v, const int64_t* slots, int32_t num_tokens,
    void* k_cache, void* v_cache, int64_t num_slots, int32_t block_size,
    int32_t num_kv_heads, int32_t head_dim, const float* k_scales,
    const float* v_scales, void* stream) {
  const char* name = "kv_reshape_and_cache_fp8_per_head";
  if (num_tokens > 0 && (!k_scales || !v_scales))
    return kvp_fail(KV_EINVAL, "%s: NULL scale array", name);
  return reshape_and_cache_fp8(name, k, v, slots, num_tokens, k_cache,
                               v_cache, num_slots, block_size, num_kv_heads,
                               head_dim, 1.f, 1.f, k_scales, v_scales, stream);
}

extern "C" kv_status kv_reshape_and_cache(const void* k, const void* v,
                                          const int64_t* slots,
                                          int32_t num_tokens, void* k_cache,
                                          void* v_cache, int64_t num_slots,
                                          int32_t block_size,
                                          int32_t num_kv_heads,
                                          int32_t head_dim, kv_dtype dtype,
                                          void* stream) {
  if (dtype != KV_F32 && dtype != KV_BF16)
    return kvp_fail(KV_EINVAL, "kv_reshape_and_cache: unknown dtype %d",
                    (int)dtype);
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || num_slots < 0 ||
      block_size <= 0 || num_slots % block_size != 0)
    return kvp_fail(KV_EINVAL, "kv_reshape_and_cache: bad shape (slots=%lld "
                    "block_size=%d)", (long long)num_slots, block_size);
  if (num_tokens == 0) return KV_OK;
  if (!k || !v || !slots || !k_cache || !v_cache)
    return kvp_fail(KV_EINVAL, "kv_reshape_and_cache: NULL pointer");
  const int64_t head_bytes = (int64_t)head_dim * elem_size(dtype);
  hipStream_t st = (hipStream_t)stream;
  int bs_shift = -1;
  if ((block_size & (block_size - 1)) == 0)
    for (bs_shift = 0; (1 << bs_shift) < block_size; ++bs_shift) {}
  auto go = [&](auto unit) {
    using U = decltype(unit);
    const int64_t uph = head_bytes / (int64_t)sizeof(U);
    const int64_t per_token = uph * num_kv_heads;
    if (per_token <= 256) {
      const int64_t tpb = 256 / per_token;
      const int64_t g = (num_tokens + tpb - 1) / tpb;
      scatter_rows_kernel<U><<<(int)(g < 65536 ? g : 65536), 256, 0, st>>>(
          (const U*)k, (const U*)v, slots, num_tokens, (U*)k_cache,
          (U*)v_cache, num_slots, block_size, bs_shift, num_kv_heads,
          (int32_t)uph);
    } else {
      const int64_t g = (num_tokens * per_token + 255) / 256;
      scatter_wide_rows_kernel<U>
          <<<(int)(g < 65536 ? g : 65536), 256, 0, st>>>(
              (const U*)k, (const U*)v, slots, num_tokens, (U*)k_cache,
              (U*)v_cache, num_slots, block_size, num_kv_heads,
              (int32_t)uph);
    }
  };
  if (head_bytes % 16 == 0) go(u32x4{});
  else if (head_bytes % 4 == 0) go(uint32_t{});
  else go(uint16_t{});
  KVP_LAUNCH_CHECK("kv_reshape_and_cache");
  return KV_OK;
}

namespace {
template <typename U>
void launch_copy(void* k_cache, void* v_cache, const int32_t* src_dst,
                 int32_t n, int32_t num_blocks, int64_t units, hipStream_t st) {
  const int threads = 256;
  const int64_t per_pair = (2 * units + threads - 1) / threads;
  dim3 grid((unsigned)(per_pair < 1024 ? per_pair : 1024),
            (unsigned)(n < 65535 ? n : 65535));
  copy_blocks_kernel<U><<<grid, threads, 0, st>>>(
      (U*)k_cache, (U*)v_cache, src_dst, n, num_blocks, units);
}
}  // namespace

extern "C" kv_status kv_copy_blocks(void* k_cache, void* v_cache,
                                    const int32_t* src_dst, int32_t n,
                                    int32_t num_blocks, int32_t block_size,
                                    int32_t num_kv_heads, int32_t head_dim,
                                    kv_dtype dtype, void* stream) {
  if (dtype != KV_F32 && dtype != KV_BF16)
    return kvp_fail(KV_EINVAL, "kv_copy_blocks: unknown dtype %d", (int)dtype);
  if (n < 0 || num_blocks < 0 || block_size <= 0 || num_kv_heads <= 0 ||
      head_dim <= 0)
    return kvp_fail(KV_EINVAL, "kv_copy_blocks: bad shape");
  if (n == 0) return KV_OK;
  if (!k_cache || !v_cache || !src_dst)
    return kvp_fail(KV_EINVAL, "kv_copy_blocks: NULL pointer");
  const int64_t block_bytes =
      (int64_t)block_size * num_kv_heads * head_dim * elem_size(dtype);
  hipStream_t st = (hipStream_t)stream;
  if (block_bytes % 16 == 0)
    launch_copy<u32x4>(k_cache, v_cache, src_dst, n, num_blocks,
                       block_bytes / 16, st);
  else if (block_bytes % 4 == 0)
    launch_copy<uint32_t>(k_cache, v_cache, src_dst, n, num_blocks,
                          block_bytes / 4, st);
  else
    launch_copy<uint16_t>(k_cache, v_cache, src_dst, n, num_blocks,
                          block_bytes / 2, st);
  KVP_LAUNCH_CHECK("kv_copy_blocks");
  return KV_OK;
}

// ---------------------------------------------------------------------------
// Copies of whole blocks between two pools of the same shape, either of which
// may be pinned host memory the device addresses directly: blocks swapped out
// to CPU memory when the device pool is full, and back in ["Makale Bülteni —
// PagedAttention ve vLLM", section "İddia ve Gerçeklik"].
namespace {
template <typename U>
__global__ __launch_bounds__(256) void swap_blocks_kernel(
    const U* __restrict__ sk, const U* __restrict__ sv, U* __restrict__ dk,
    U* __restrict__ dv, const int32_t* __restrict__ pairs, int32_t n,
    int32_t src_blocks, int32_t dst_blocks, int64_t units_per_block) {
  const int64_t total = 2 * units_per_block;
  for (int32_t p = blockIdx.y; p < n; p += gridDim.y) {
    const int32_t src = pairs[2 * p], dst = pairs[2 * p + 1];
    if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) continue;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
      const bool is_v = i >= units_per_block;
      const int64_t u = is_v ? i - units_per_block : i;
      (is_v ? dv : dk)[(int64_t)dst * units_per_block + u] =
          (is_v ? sv : sk)[(int64_t)src * units_per_block + u];
    }
  }
}

}  // namespace

void* kvp_device_view(const void* p) {
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();  // pageable host memory: clear the error
    return nullptr;
  }
  if (a.type == hipMemoryTypeDevice || a.type == hipMemoryTypeManaged)
    return const_cast<void*>(p);
  if (a.type == hipMemoryTypeHost) return a.devicePointer;
  return nullptr;
}

extern "C" kv_status kv_swap_blocks(const void* src_k, const void* src_v,
                                    int32_t src_blocks, void* dst_k,
                                    void* dst_v, int32_t dst_blocks,
                                    const int32_t* pairs, int32_t n,
                                    int32_t block_size, int32_t num_kv_heads,
                                    int32_t head_dim, kv_dtype dtype,
                                    void* stream) {
  if (dtype != KV_F32 && dtype != KV_BF16)
    return kvp_fail(KV_EINVAL, "kv_swap_blocks: unknown dtype %d", (int)dtype);
  if (n < 0 || src_blocks < 0 || dst_blocks < 0 || block_size <= 0 ||
      num_kv_heads <= 0 || head_dim <= 0)
    return kvp_fail(KV_EINVAL, "kv_swap_blocks: bad shape");
  if (n == 0) return KV_OK;
  if (!src_k || !src_v || !dst_k || !dst_v || !pairs)
    return kvp_fail(KV_EINVAL, "kv_swap_blocks: NULL pointer");
  const void* ptrs[5] = {src_k, src_v, dst_k, dst_v, pairs};
  void* dev[5];
  for (int i = 0; i < 5; ++i) {
    dev[i] = kvp_device_view(ptrs[i]);
    if (!dev[i])
      return kvp_fail(KV_EINVAL,
                      "kv_swap_blocks: %s is not device or pinned host memory",
                      i == 4 ? "pairs" : (i < 2 ? "a source pool" :
                                          "a destination pool"));
  }
  const int64_t block_bytes =
      (int64_t)block_size * num_kv_heads * head_dim * elem_size(dtype);
  hipStream_t st = (hipStream_t)stream;
  const int threads = 256;
  auto go = [&](auto unit) {
    using U = decltype(unit);
    const int64_t units = block_bytes / (int64_t)sizeof(U);
    const int64_t per_pair = (2 * units + threads - 1) / threads;
    dim3 grid((unsigned)(per_pair < 1024 ? per_pair : 1024),
              (unsigned)(n < 65535 ? n : 65535));
    swap_blocks_kernel<U><<<grid, threads, 0, st>>>(
        (const U*)dev[0], (const U*)dev[1], (U*)dev[2], (U*)dev[3],
        (const int32_t*)dev[4], n, src_blocks, dst_blocks, units);
  };
  if (block_bytes % 16 == 0) go(u32x4{});
  else if (block_bytes % 4 == 0) go(uint32_t{});
  else go(uint16_t{});
  KVP_LAUNCH_CHECK("kv_swap_blocks");
  return KV_OK;
}

extern "C" kv_status kv_append_token(const void* k, const void* v,
                                     const int32_t* new_blocks,
                                     int32_t* block_tables, int32_t bt_stride,
                                     int32_t* context_lens, int32_t num_seqs,
                                     void* k_cache, void* v_cache,
                                     int32_t num_blocks, int32_t block_size,
                                     int32_t num_kv_heads, int32_t head_dim,
                                     kv_dtype dtype, void* stream) {
  const char* name = "kv_append_token";
  if (dtype != KV_F32 && dtype != KV_BF16)
    return kvp_fail(KV_EINVAL, "%s: unknown dtype %d", name, (int)dtype);
  if (num_seqs < 0 || bt_stride <= 0 || num_blocks <= 0 || block_size <= 0 ||
      num_kv_heads <= 0 || head_dim <= 0)
    return kvp_fail(KV_EINVAL, "%s: bad shape (S=%d stride=%d N=%d B=%d "
                    "Hkv=%d D=%d)", name, num_seqs, bt_stride, num_blocks,
                    block_size, num_kv_heads, head_dim);
  if (num_seqs == 0) return KV_OK;
  if (!k || !v || !new_blocks || !block_tables || !context_lens || !k_cache ||
      !v_cache)
    return kvp_fail(KV_EINVAL, "%s: NULL pointer", name);
  const int32_t* nb = (const int32_t*)kvp_device_view(new_blocks);
  if (!nb)
    return kvp_fail(KV_EINVAL, "%s: new_blocks is not device or pinned host "
                    "memory", name);
  const int64_t head_bytes = (int64_t)head_dim * elem_size(dtype);
  // the widest unit that divides a head row and every row address
  const uintptr_t align = (uintptr_t)k | (uintptr_t)v | (uintptr_t)k_cache |
                          (uintptr_t)v_cache | (uintptr_t)head_bytes;
  hipStream_t st = (hipStream_t)stream;
  const int threads = 256;
  if (align % 16 == 0)
    append_token_kernel<<<num_seqs, threads, 0, st>>>(
        (const u32x4*)k, (const u32x4*)v, nb, block_tables, bt_stride,
        context_lens, (u32x4*)k_cache, (u32x4*)v_cache, num_blocks,
        block_size, num_kv_heads, (int32_t)(head_bytes / 16), CopyUnit{});
  else if (align % 4 == 0)
    append_token_kernel<<<num_seqs, threads, 0, st>>>(
        (const uint32_t*)k, (const uint32_t*)v, nb, block_tables, bt_stride,
        context_lens, (uint32_t*)k_cache, (uint32_t*)v_cache, num_blocks,
        block_size, num_kv_heads, (int32_t)(head_bytes / 4), CopyUnit{});
  else
    append_token_kernel<<<num_seqs, threads, 0, st>>>(
        (const uint16_t*)k, (const uint16_t*)v, nb, block_tables, bt_stride,
        context_lens, (uint16_t*)k_cache, (uint16_t*)v_cache, num_blocks,
        block_size, num_kv_heads, (int32_t)(head_bytes / 2), CopyUnit{});
  KVP_LAUNCH_CHECK(name);
  return KV_OK;
}

namespace {
kv_status append_token_fp8(const char* name, const void* k, const void* v,
                           const int32_t* new_blocks, int32_t* block_tables,
                           int32_t bt_stride, int32_t* context_lens,
                           int32_t num_seqs, void* k_cache, void* v_cache,
                           int32_t num_blocks, int32_t block_size,
                           int32_t num_kv_heads, int32_t head_dim,
                           float k_scale, float v_scale, const float* k_scales,
                           const float* v_scales, void* stream) {
  if (num_seqs < 0 || bt_stride <= 0 || num_blocks <= 0 || block_size <= 0 ||
      num_kv_heads <= 0 || head_dim <= 0 || head_dim % 8 != 0)
    return kvp_fail(KV_EINVAL, "%s: bad shape (S=%d stride=%d N=%d B=%d "
                    "Hkv=%d D=%d; D must be a multiple of 8)", name, num_seqs,
                    bt_stride, num_blocks, block_size, num_kv_heads, head_dim);
  if (!(k_scale > 0.f) || !(k_scale < INFINITY) || !(v_scale > 0.f) ||
      !(v_scale < INFINITY))
    return kvp_fail(KV_EINVAL, "%s: k_scale and v_scale must be finite and "
                    "> 0", name);
  if (num_seqs == 0) return KV_OK;
  if (!k || !v || !new_blocks || !block_tables || !context_lens || !k_cache ||
      !v_cache)
    return kvp_fail(KV_EINVAL, "%s: NULL pointer", name);
  if (((uintptr_t)k | (uintptr_t)v) % 16 ||
      ((uintptr_t)k_cache | (uintptr_t)v_cache) % 8)
    return kvp_fail(KV_EINVAL, "%s: k/v must be 16-byte and the caches "
                    "8-byte aligned", name);
  const int32_t* nb = (const int32_t*)kvp_device_view(new_blocks);
  if (!nb)
    return kvp_fail(KV_EINVAL, "%s: new_blocks is not device or pinned host "
                    "memory", name);
  append_token_kernel<<<num_seqs, 256, 0, (hipStream_t)stream>>>(
      (const u32x4*)k, (const u32x4*)v, nb, block_tables, bt_stride,
      context_lens, (u32x2*)k_cache, (u32x2*)v_cache, num_blocks, block_size,
      num_kv_heads, head_dim / 8,
      Fp8Unit{1.f / k_scale, 1.f / v_scale, k_scales, v_scales});
  KVP_LAUNCH_CHECK(name);
  return KV_OK;
}
}  // namespace

extern "C" kv_status kv_append_token_fp8(
    const void* k, const void* v, const int32_t* new_blocks,
    int32_t* block_tables, int32_t bt_stride, int32_t* context_lens,
    int32_t num_seqs, void* k_cache, void* v_cache, int32_t num_blocks,
    int32_t block_size, int32_t num_kv_heads, int32_t head_dim, float k_scale,
    float v_scale, void* stream) {
  return append_token_fp8("kv_append_token_fp8", k, v, new_blocks,
                          block_tables, bt_stride, context_lens, num_seqs,
                          k_cache, v_cache, num_blocks, block_size,
                          num_kv_heads, head_dim, k_scale, v_scale, nullptr,
                          nullptr, stream);
}

extern "C" kv_status kv_append_token_fp8_per_head(
    const void* k, const void* v, const int32_t* new_blocks,
    int32_t* block_tables, int32_t bt_stride, int32_t* context_lens,
    int32_t num_seqs, void* k_cache, void* v_cache, int32_t num_blocks,
    int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
    const float* k_scales, const float* v_scales, void* stream) {
  const char* name = "kv_append_token_fp8_per_head";
  if (num_seqs > 0 && (!k_scales || !v_scales))
    return kvp_fail(KV_EINVAL, "%s: NULL scale array", name);
  return append_token_fp8(name, k, v, new_blocks, block_tables, bt_stride,
                          context_lens, num_seqs, k_cache, v_cache,
                          num_blocks, block_size, num_kv_heads, head_dim, 1.f,
                          1.f, k_scales, v_scales, stream);
}
