/*
 * kvpaged.h - C ABI of the paged-KV attention library for MI355X (gfx950).
 *
 * What it implements (pages cited by title and section):
 *   - The KV cache of each sequence lives in fixed-size blocks of token
 *     slots; blocks are taken as the sequence grows; a block table maps
 *     logical blocks to physical ones; the attention kernel reads K/V
 *     through that table; freed blocks are reused ["PagedAttention Nedir?"
 *     (bitcanli.com), section "PagedAttention Nasıl Çalışır?", steps 1-5].
 *   - A free block is taken from the pool when the current block is full;
 *     empty slots exist only in a sequence's last block; parallel samples
 *     share blocks by reference with copy-on-write ["Makale Bülteni —
 *     PagedAttention ve vLLM", section "İddia ve Gerçeklik"].
 *   - The contiguous variant keeps one contiguous K/V buffer per sequence,
 *     reserved for the maximum context, so the kernel sees a plain tensor
 *     ["Makale Bülteni — vAttention", section "İddia ve Gerçeklik"].
 *
 * Conventions:
 *   - Every function returns a kv_status (or a documented value); no
 *     exception or abort crosses the ABI. On an error return, host state
 *     (pool, tables, lengths) is unchanged and kv_last_error() describes it.
 *   - Host-side functions (kv_pool_*, kv_block_*, kv_seq_append,
 *     kv_slot_mapping, kv_blocks_needed) touch no GPU.
 *   - Device ops take device pointers owned by the caller, enqueue work on
 *     `stream` (a hipStream_t; NULL = the default stream), return after the
 *     launch, and allocate no device memory. Launch failures return KV_EHIP.
 *   - Layouts (row-major, element type = `dtype`):
 *       paged K/V pool        [num_blocks, Hkv, block_size, D]
 *       contiguous K/V        [num_seqs, Hkv, seq_stride, D]
 *       new K/V rows          [num_tokens, Hkv, D]
 *       decode q / out        [num_seqs, Hq, D]
 *       prefill q / out       [total_q, Hq, D]   (sequence s owns rows
 *                                                 cu_q_lens[s]..cu_q_lens[s+1])
 *       block table           int32 [num_seqs, bt_stride]
 *     Both caches are head-major inside a block (or sequence): the D values
 *     of one head for consecutive tokens are contiguous. A slot numbers the
 *     tokens of a cache: slot = block * block_size + offset for the paged
 *     pool, s * seq_stride + position for the contiguous layout (whose
 *     "block" is the whole sequence).
 *   - Query head h reads KV head h / (Hq / Hkv). Attention is softmax of
 *     scale * q.k over the visible keys, accumulated in fp32; out has the
 *     dtype of q. scale must be finite and > 0 (KV_EINVAL otherwise).
 *   - The allocator is single-threaded: one host thread per pool.
 */
#ifndef KVPAGED_H
#define KVPAGED_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KV_OK = 0,
  KV_EINVAL = -1,       /* bad argument (null pointer, out-of-range id, shape) */
  KV_ENOMEM = -2,       /* the pool has too few free blocks                     */
  KV_EREFCOUNT = -3,    /* free/share/cow of a block whose refcount is 0        */
  KV_EHIP = -4,         /* a HIP runtime call or kernel launch failed           */
  KV_EUNSUPPORTED = -5  /* valid, but no kernel covers this shape/dtype         */
} kv_status;

typedef enum { KV_F32 = 0, KV_BF16 = 1 } kv_dtype;

typedef struct kv_pool kv_pool; /* opaque host-side block metadata */

/* Thread-local description of the last non-OK status on this thread. */
const char* kv_last_error(void);

/* ---------------------------------------------------------------------
 * Block arithmetic ["PagedAttention Nasıl Çalışır?", worked example:
 * 35 tokens in 16-slot blocks take 3 blocks].
 * Returns ceil(num_tokens / block_size), or -1 if num_tokens < 0 or
 * block_size <= 0. */
int64_t kv_blocks_needed(int64_t num_tokens, int32_t block_size);

/* ---------------------------------------------------------------------
 * Block pool [steps 2 and 5 of "PagedAttention Nasıl Çalışır?";
 * copy-on-write from "İddia ve Gerçeklik" of the PagedAttention newsletter].
 * Policy: the free blocks form a FIFO queue, initially init_free_order
 * (a permutation of 0..num_blocks-1; NULL means ascending). Allocation pops
 * from the head; a block whose refcount drops to 0 is pushed at the tail,
 * in argument order. The caller owns the returned pool. */
kv_status kv_pool_create(int32_t num_blocks, int32_t block_size,
                         const int32_t* init_free_order, kv_pool** out);
void kv_pool_destroy(kv_pool* pool); /* NULL is a no-op */

/* Take n blocks (refcount 1) into out_ids[0..n). All or nothing:
 * KV_ENOMEM if fewer than n are free. */
kv_status kv_block_alloc(kv_pool* pool, int32_t n, int32_t* out_ids);

/* Drop one reference per listed id (ids may repeat). KV_EINVAL for an id
 * outside the pool, KV_EREFCOUNT if an id would drop below 0. */
kv_status kv_block_free(kv_pool* pool, int32_t n, const int32_t* ids);

/* Add one reference per listed id (fork). KV_EREFCOUNT for a free block. */
kv_status kv_block_share(kv_pool* pool, int32_t n, const int32_t* ids);

/* Copy-on-write check before writing into block `id`. Refcount 1: *out_id
 * = id, *need_copy = 0. Refcount > 1: a new block (refcount 1) is taken,
 * id loses one reference, *out_id = new block, *need_copy = 1 (the caller
 * copies the contents, e.g. with kv_copy_blocks). KV_ENOMEM if no block is
 * free, KV_EREFCOUNT if id is free. */
kv_status kv_block_cow(kv_pool* pool, int32_t id, int32_t* out_id,
                       int32_t* need_copy);

/* Refcount of id, or KV_EINVAL (< 0) for an id outside the pool. */
int32_t kv_block_refcount(const kv_pool* pool, int32_t id);
int32_t kv_pool_num_free(const kv_pool* pool);
int32_t kv_pool_num_blocks(const kv_pool* pool);
int32_t kv_pool_block_size(const kv_pool* pool);

/* Copy the free queue, head first, into out[0..min(cap, num_free)).
 * Returns the number of free blocks. */
int32_t kv_pool_free_list(const kv_pool* pool, int32_t* out, int32_t cap);

/* ---------------------------------------------------------------------
 * Sequence growth (host; steps 2-3 of "PagedAttention Nasıl Çalışır?").
 * Sequences s = 0..num_seqs-1, in order, each gain n_new[s] tokens (NULL:
 * one token each). For the token at position p = seq_lens[s]:
 *   - if p % block_size == 0, a new block is allocated and written to
 *     block_tables[s * bt_stride + p / block_size];
 *   - otherwise, if the block holding p is shared (refcount > 1), it is
 *     copied on write: the table entry is replaced by the new block and
 *     the pair (old, new) is appended to out_cow_pairs;
 *   - its slot, table[p / block_size] * block_size + p % block_size, is
 *     appended to out_slots (sequence order, then position order).
 * seq_lens[s] grows by n_new[s]. block_tables and seq_lens are host
 * arrays, read and written. out_slots needs sum(n_new) entries;
 * out_cow_pairs holds [cow_capacity, 2] int32; *out_num_cow receives the
 * number of pairs. All or nothing: KV_ENOMEM when the pool runs dry,
 * KV_EINVAL when a table row or cow_capacity is too small. */
kv_status kv_seq_append(kv_pool* pool, int32_t* block_tables,
                        int32_t bt_stride, int32_t* seq_lens,
                        const int32_t* n_new, int32_t num_seqs,
                        int64_t* out_slots, int32_t* out_cow_pairs,
                        int32_t cow_capacity, int32_t* out_num_cow);

/* Slot of each (seq_ids[i], positions[i]) from a host block table:
 * block_tables[seq * bt_stride + pos / block_size] * block_size +
 * pos % block_size; a negative position gives -1 (padding). Host only. */
kv_status kv_slot_mapping(const int32_t* block_tables, int32_t bt_stride,
                          const int32_t* seq_ids, const int32_t* positions,
                          int32_t n, int32_t block_size, int64_t* out_slots);

/* ---------------------------------------------------------------------
 * Cache write [step 2: a new token's K and V go into its slot].
 * k, v: new rows [num_tokens, Hkv, D]; slots: device int64 [num_tokens].
 * For every head h, k[i, h, :] goes to k_cache[slot / block_size, h,
 * slot % block_size, :] (same for v). The caches hold num_slots tokens
 * (paged: num_blocks * block_size; contiguous: num_seqs * seq_stride with
 * block_size = seq_stride). Slots < 0 (padding) and slots >= num_slots are
 * skipped. Bit copy. */
kv_status kv_reshape_and_cache(const void* k, const void* v,
                               const int64_t* slots, int32_t num_tokens,
                               void* k_cache, void* v_cache, int64_t num_slots,
                               int32_t block_size, int32_t num_kv_heads,
                               int32_t head_dim, kv_dtype dtype, void* stream);

/* Device side of one decode append for a batch, one new token per
 * sequence, with the block table and the lengths kept in device memory
 * ["PagedAttention Nedir?" (bitcanli.com), "PagedAttention Nasıl
 * Çalışır?", steps 2-3: the new token goes into the slot its table assigns,
 * a block taken from the pool when the last one is full]. For each
 * sequence s, with L = context_lens[s]:
 *   1. if new_blocks[s] >= 0, it is stored as block_tables[s][L / B] (the
 *      block the host allocator took for that logical block: a fresh block
 *      when L % B == 0, or the copy-on-write target, whose copy must
 *      already be enqueued on the stream);
 *   2. k[s, h, :] and v[s, h, :] go to slot
 *      block_tables[s][L / B] * B + L % B, laid out as kv_reshape_and_cache
 *      writes it;
 *   3. context_lens[s] becomes L + 1.
 * k, v: [num_seqs, Hkv, D] device rows. block_tables (int32 [num_seqs,
 * bt_stride]) and context_lens (int32 [num_seqs]) are device memory and are
 * updated in place. new_blocks: int32 [num_seqs], -1 = keep the entry;
 * device memory or pinned host memory (hipHostMalloc, torch's pin_memory),
 * which the kernel reads directly, so that a step uploads nothing; other
 * host memory -> KV_EINVAL. The kernel reads new_blocks when it runs, not
 * at the call: the host must not rewrite it before then (e.g. wait for an
 * event recorded after the call). A sequence with L outside [0, bt_stride * B),
 * or whose block is outside [0, num_blocks), is left unchanged. The
 * contiguous layout is the case block_size = seq_stride with
 * block_tables[s][0] = s. The result equals kv_seq_append's table and slots
 * followed by kv_reshape_and_cache. Enqueued on `stream`; allocates
 * nothing. */
kv_status kv_append_token(const void* k, const void* v,
                          const int32_t* new_blocks, int32_t* block_tables,
                          int32_t bt_stride, int32_t* context_lens,
                          int32_t num_seqs, void* k_cache, void* v_cache,
                          int32_t num_blocks, int32_t block_size,
                          int32_t num_kv_heads, int32_t head_dim,
                          kv_dtype dtype, void* stream);

/* Copy-on-write data move: for i < n, block src_dst[2i] -> src_dst[2i+1]
 * of both caches (device int32 pairs). The pairs must be independent: no
 * destination may be another pair's source or destination (the pairs
 * kv_seq_append emits always are); they are copied in parallel. Pairs
 * naming a block outside [0, num_blocks) are skipped. Bit copy. */
kv_status kv_copy_blocks(void* k_cache, void* v_cache,
                         const int32_t* src_dst, int32_t n, int32_t num_blocks,
                         int32_t block_size, int32_t num_kv_heads,
                         int32_t head_dim, kv_dtype dtype, void* stream);

/* ---------------------------------------------------------------------
 * Decode attention: one query per sequence against all context_lens[s]
 * tokens of its context (the query's own K/V is written first)
 * [step 4 of "PagedAttention Nasıl Çalışır?"; the kernel-side table read
 * described in "İddia ve Gerçeklik" of the vAttention newsletter].
 *
 * The work is balanced across the GPU independently of the length mix: per
 * KV head, the tokens of all sequences are laid end to end and cut into
 * kv_decode_chunks() equal chunks, one workgroup each; a sequence cut by a
 * chunk boundary leaves partial softmax results that a second kernel merges
 * exactly. The workspace (device memory, caller-owned, at least
 * kv_decode_workspace_bytes() bytes; never NULL for num_seqs > 0) starts
 * with a 256-byte header, followed, for head_dim 128, by those partials
 * (an fp32 call uses the header only). max_context bounds every
 * context_lens[s]: a value outside [0, max_context] (or beyond the table's
 * bt_stride * block_size tokens, or the contiguous seq_stride) is clamped
 * into range, which keeps memory accesses in bounds, and the number of
 * sequences clamped in the call is stored in the header;
 * kv_decode_clamped_count() reads it, so a stale bound is visible rather
 * than silently shortening the attention. Table entries outside
 * [0, num_blocks) are clamped into range (not counted), which keeps memory
 * accesses in bounds but makes that output meaningless. context_lens[s] ==
 * 0 gives a zero output row. Calls sharing one workspace must be ordered
 * (same stream). */
int32_t kv_decode_chunks(int32_t num_q_heads, int32_t num_kv_heads);
size_t kv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim,
                                 int32_t max_context);

/* One decode step with the step's token appended, in one op: the same
 * result and the same cache, table and length updates as kv_append_token
 * (k_new, v_new, new_blocks, block_tables, context_lens, ...) followed by
 * paged_attn_decode over the lengths it advanced ["PagedAttention Nedir?"
 * (bitcanli.com), "PagedAttention Nasıl Çalışır?", steps 2-4: the new
 * token's K/V take the slot its table assigns, then the query attends to
 * the whole context]. The attention reads the new token from k_new / v_new
 * rather than from the cache, so the cache write (the K and V rows, the
 * table entry when new_blocks[s] >= 0, context_lens[s] + 1) is done by the
 * merge kernel after the attention and no separate append launch is made.
 * Arguments as in kv_append_token and paged_attn_decode; context_lens
 * holds the lengths before the token and is advanced in place; the
 * workspace is kv_decode_workspace_bytes(). new_blocks (device or pinned
 * host memory) is copied into the workspace by the op's first kernel; the
 * caller may rewrite it once the op has completed on `stream`. A sequence
 * whose token position lies outside [0, bt_stride * block_size) is not
 * advanced and attends to its stored context only. A position inside the table whose
 * block is invalid (new_blocks[s] < 0 and an entry outside
 * [0, num_blocks)) is a caller error: the token is attended to but not
 * stored, and the length is not advanced. Shapes other than bf16,
 * head_dim 128, block_size % 16 == 0 (or rows not 16-byte aligned) run the
 * two calls in order. */
kv_status paged_attn_decode_append(
    void* out, const void* q, const void* k_new, const void* v_new,
    const int32_t* new_blocks, void* k_cache, void* v_cache,
    int32_t num_blocks, int32_t* block_tables, int32_t bt_stride,
    int32_t* context_lens, int32_t max_context, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, float scale, kv_dtype dtype, void* workspace,
    size_t workspace_bytes, void* stream);

/* Number of sequences whose context_lens entry the last decode call on this
 * workspace clamped (see above): waits for `stream`, then copies the count
 * from the workspace header into *count. KV_EHIP if the copy fails. */
kv_status kv_decode_clamped_count(const void* workspace, void* stream,
                                  int32_t* count);

kv_status paged_attn_decode(void* out, const void* q, const void* k_cache,
                            const void* v_cache, int32_t num_blocks,
                            const int32_t* block_tables, int32_t bt_stride,
                            const int32_t* context_lens, int32_t max_context,
                            int32_t num_seqs, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim,
                            int32_t block_size, float scale, kv_dtype dtype,
                            void* workspace, size_t workspace_bytes,
                            void* stream);

/* paged_attn_decode for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. Same arguments and result as paged_attn_decode, without the
 * workspace: the kernels use a scratch array of 16 MiB that the library
 * holds in each GPU's memory from load until the process ends (found once
 * per device with hipGetSymbolAddress). Calls allocate nothing (no
 * hipMalloc, hipFree or allocating library routine). A shape whose
 * workspace (kv_decode_workspace_bytes) exceeds 16 MiB -> KV_EINVAL. Every
 * call on a GPU shares that GPU's scratch and leaves its contents behind:
 * calls that overlap on one GPU (different streams, or threads) race and
 * must be ordered by the caller. The clamp count of this call stays in the
 * scratch (use paged_attn_decode to read it). */
kv_status paged_attn_decode_noalloc(void* out, const void* q,
                                    const void* k_cache, const void* v_cache,
                                    int32_t num_blocks,
                                    const int32_t* block_tables,
                                    int32_t bt_stride,
                                    const int32_t* context_lens,
                                    int32_t max_context, int32_t num_seqs,
                                    int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t block_size,
                                    float scale, kv_dtype dtype, void* stream);

/* Same on the contiguous layout [num_seqs, Hkv, seq_stride, D]. */
kv_status contig_attn_decode(void* out, const void* q, const void* k,
                             const void* v, int32_t seq_stride,
                             const int32_t* context_lens, int32_t max_context,
                             int32_t num_seqs, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t head_dim,
                             float scale, kv_dtype dtype, void* workspace,
                             size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------
 * Decode with shared prefixes. Same result as paged_attn_decode (same
 * arguments up to block_size), for batches where groups of consecutive
 * sequences hold the same first tokens in the same physical blocks: a
 * prompt forked with kv_block_share, its blocks at refcount > 1
 * ["Makale Bülteni — PagedAttention ve vLLM", "İddia ve Gerçeklik";
 * "PagedAttention Nedir?", "Prefix Sharing Nasıl Çalışır?"]. The shared
 * tokens' K/V are read once per group instead of once per sequence.
 *   group_starts  device int32 [num_groups + 1]: group g is sequences
 *                 group_starts[g] .. group_starts[g+1]-1; the groups must
 *                 partition 0..num_seqs-1 in order (a sequence that shares
 *                 nothing is a group of one with shared_lens 0).
 *   shared_lens   device int32 [num_groups]: leading tokens of every
 *                 member's context that sit in the same physical blocks as
 *                 the group's first member's; read through that member's
 *                 table. Must not exceed any member's context_lens.
 *   num_groups, max_group_size (largest group), max_shared_len (largest
 *                 shared_lens entry): host bounds that size the launch.
 * Shared tokens are used in whole 16-token groups (the rest of a partial
 * group is read per sequence). Values outside these rules keep memory
 * accesses in bounds but make the affected outputs meaningless.
 * The workspace must hold kv_decode_shared_prefix_workspace_bytes() bytes.
 * The sharing pass needs bf16, head_dim 128, block_size % 16 == 0 and at
 * most 4096 sequences; other calls (and max_shared_len < 16) run
 * paged_attn_decode unchanged. */
size_t kv_decode_shared_prefix_workspace_bytes(int32_t num_seqs,
                                               int32_t num_q_heads,
                                               int32_t num_kv_heads,
                                               int32_t head_dim,
                                               int32_t max_context,
                                               int32_t max_shared_len);

kv_status paged_attn_decode_shared_prefix(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    int32_t num_blocks, const int32_t* block_tables, int32_t bt_stride,
    const int32_t* context_lens, int32_t max_context, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, const int32_t* group_starts,
    const int32_t* shared_lens, int32_t num_groups, int32_t max_group_size,
    int32_t max_shared_len, float scale, kv_dtype dtype, void* workspace,
    size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------
 * Chunked prefill attention. Sequence s has cu_q_lens[s+1]-cu_q_lens[s]
 * queries at absolute positions q_start_pos[s] + i and a context of
 * context_lens[s] tokens already in the cache (including this chunk's
 * own K/V). With causal != 0 a query at position p sees keys 0..p (and
 * < context_lens[s]); otherwise all context keys. max_q_len bounds every
 * sequence's query count (the grid covers max_q_len rows per sequence; the
 * rows of a sequence with more queries are left unspecified). cu_q_lens,
 * q_start_pos and context_lens are device int32 arrays, read by the kernel
 * without a bound it could check: cu_q_lens starts at 0 and does not
 * decrease, and q and out hold cu_q_lens[num_seqs] rows of
 * [num_q_heads, head_dim]. [The prefill kernels the vAttention newsletter
 * compares in "İddia ve Gerçeklik".] */
kv_status paged_attn_prefill(void* out, const void* q,
                             const int32_t* cu_q_lens,
                             const int32_t* q_start_pos, int32_t max_q_len,
                             const void* k_cache, const void* v_cache,
                             int32_t num_blocks, const int32_t* block_tables,
                             int32_t bt_stride, const int32_t* context_lens,
                             int32_t num_seqs, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t head_dim,
                             int32_t block_size, float scale, int32_t causal,
                             kv_dtype dtype, void* stream);

kv_status contig_attn_prefill(void* out, const void* q,
                              const int32_t* cu_q_lens,
                              const int32_t* q_start_pos, int32_t max_q_len,
                              const void* k, const void* v, int32_t seq_stride,
                              const int32_t* context_lens, int32_t num_seqs,
                              int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, float scale, int32_t causal,
                              kv_dtype dtype, void* stream);

/* Copy blocks between two pools of the same [blocks, Hkv, block_size, D]
 * shape: the swap of blocks out to CPU memory when the device pool is full,
 * and back in ["Makale Bülteni — PagedAttention ve vLLM", section "İddia
 * ve Gerçeklik"]. pairs: int32 [n, 2] of (block of the source pool
 * src_k/src_v with src_blocks blocks, block of the destination pool with
 * dst_blocks blocks); a pair with an id outside its pool is skipped. Each
 * pool and `pairs` may be device memory or pinned host memory (hipHostMalloc,
 * e.g. torch's pin_memory) that the device addresses directly; other host
 * memory -> KV_EINVAL. Destinations must be distinct and must not be read
 * by another pair. Enqueued on `stream`; allocates nothing. */
kv_status kv_swap_blocks(const void* src_k, const void* src_v,
                         int32_t src_blocks, void* dst_k, void* dst_v,
                         int32_t dst_blocks, const int32_t* pairs, int32_t n,
                         int32_t block_size, int32_t num_kv_heads,
                         int32_t head_dim, kv_dtype dtype, void* stream);

/* ---------------------------------------------------------------------
 * FP8 K/V cache. Lower-precision storage of the cache is a separate lever
 * from paging ["PagedAttention Nedir?" (bitcanli.com), section "KV Cache'i
 * Sıkıştırıyor mu?"]; FP8 is among the serving stack's quantisation schemes
 * ["Makale Bülteni — PagedAttention ve vLLM", section "Kod ve Entegrasyon
 * Haritası"]. Format: OCP E4M3 ("E4M3FN": bias 7, no infinities, largest
 * finite 448), one byte per value, in the same [blocks, Hkv, block_size, D]
 * (or [S, Hkv, seq_stride, D]) layout as the bf16 caches. A value x is
 * stored as E4M3(clamp(x * fl32(1 / scale), -448, 448)): fp32 product with
 * the reciprocal rounded to fp32, saturation of overflows and infinities to
 * +-448, round to nearest, ties to even; a NaN stays NaN (the code
 * S.1111.111 with x's sign). A code reads back as E4M3 value * scale.
 * Scales: one per tensor (k_scale for K, v_scale for V, finite and > 0), or
 * with the *_per_head calls one per KV head (device float arrays k_scales,
 * v_scales of Hkv entries; each must be finite and > 0, else the codes or
 * outputs of that head are meaningless). */

/* kv_reshape_and_cache for an fp8 cache: k, v are bf16 rows [num_tokens,
 * Hkv, D] (16-byte aligned), the caches hold codes (8-byte aligned);
 * D % 8 == 0. Slots as in kv_reshape_and_cache. */
kv_status kv_reshape_and_cache_fp8(const void* k, const void* v,
                                   const int64_t* slots, int32_t num_tokens,
                                   void* k_cache, void* v_cache,
                                   int64_t num_slots, int32_t block_size,
                                   int32_t num_kv_heads, int32_t head_dim,
                                   float k_scale, float v_scale, void* stream);

/* kv_append_token for fp8 caches: k, v are bf16 rows [num_seqs, Hkv, D]
 * (16-byte aligned), the caches hold codes (8-byte aligned), D % 8 == 0;
 * each value is stored as in kv_reshape_and_cache_fp8. Table, lengths and
 * new_blocks as in kv_append_token. */
kv_status kv_append_token_fp8(const void* k, const void* v,
                              const int32_t* new_blocks,
                              int32_t* block_tables, int32_t bt_stride,
                              int32_t* context_lens, int32_t num_seqs,
                              void* k_cache, void* v_cache,
                              int32_t num_blocks, int32_t block_size,
                              int32_t num_kv_heads, int32_t head_dim,
                              float k_scale, float v_scale, void* stream);

/* paged_attn_decode / contig_attn_decode over fp8 caches: q and out are
 * bf16; attention is computed on the dequantised K (k_scale folded into the
 * softmax scale) and V (v_scale applied to the output). Workspace as for
 * the bf16 calls (kv_decode_workspace_bytes). Only head_dim 128 and, paged,
 * block_size a multiple of 16 (else KV_EUNSUPPORTED). */
kv_status paged_attn_decode_fp8(void* out, const void* q, const void* k_cache,
                                const void* v_cache, int32_t num_blocks,
                                const int32_t* block_tables, int32_t bt_stride,
                                const int32_t* context_lens,
                                int32_t max_context, int32_t num_seqs,
                                int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size,
                                float scale, float k_scale, float v_scale,
                                void* workspace, size_t workspace_bytes,
                                void* stream);

kv_status contig_attn_decode_fp8(void* out, const void* q, const void* k,
                                 const void* v, int32_t seq_stride,
                                 const int32_t* context_lens,
                                 int32_t max_context, int32_t num_seqs,
                                 int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, float scale, float k_scale,
                                 float v_scale, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* The fp8 calls above with one scale per KV head: k_scales, v_scales are
 * device float arrays [Hkv]; head h's rows are stored with
 * fl32(1 / k_scales[h]) (K) and fl32(1 / v_scales[h]) (V), and the decode
 * folds k_scales[g] into the score scale of KV head g and applies
 * v_scales[g] to its outputs. Other arguments, layouts and errors as in the
 * per-tensor calls; NULL scale arrays -> KV_EINVAL. */
kv_status kv_reshape_and_cache_fp8_per_head(
    const void* k, const void* v, const int64_t* slots, int32_t num_tokens,
    void* k_cache, void* v_cache, int64_t num_slots, int32_t block_size,
    int32_t num_kv_heads, int32_t head_dim, const float* k_scales,
    const float* v_scales, void* stream);

kv_status kv_append_token_fp8_per_head(
    const void* k, const void* v, const int32_t* new_blocks,
    int32_t* block_tables, int32_t bt_stride, int32_t* context_lens,
    int32_t num_seqs, void* k_cache, void* v_cache, int32_t num_blocks,
    int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
    const float* k_scales, const float* v_scales, void* stream);

kv_status paged_attn_decode_fp8_per_head(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    int32_t num_blocks, const int32_t* block_tables, int32_t bt_stride,
    const int32_t* context_lens, int32_t max_context, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, float scale, const float* k_scales,
    const float* v_scales, void* workspace, size_t workspace_bytes,
    void* stream);

kv_status contig_attn_decode_fp8_per_head(
    void* out, const void* q, const void* k, const void* v, int32_t seq_stride,
    const int32_t* context_lens, int32_t max_context, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, float scale,
    const float* k_scales, const float* v_scales, void* workspace,
    size_t workspace_bytes, void* stream);

/* paged_attn_decode_append on fp8 E4M3 caches: the same result and the
 * same cache, table and length updates as kv_append_token_fp8 (or
 * kv_append_token_fp8_per_head) followed by paged_attn_decode_fp8 (or
 * _per_head) over the advanced lengths, in one op. k_new / v_new are bf16;
 * the attention takes the new token as the codes the cache will hold (its
 * rows quantised with the head's 1 / scale, then widened back), so the
 * result is that of the two calls; the merge kernel stores those codes,
 * the table entry and the length after the attention. Scales, arguments
 * and errors as in those calls; head_dim 128 and block_size % 16 == 0
 * only (others: KV_EUNSUPPORTED, nothing written); k_new / v_new 16-byte
 * and the caches 8-byte aligned (else KV_EINVAL). */
kv_status paged_attn_decode_append_fp8(
    void* out, const void* q, const void* k_new, const void* v_new,
    const int32_t* new_blocks, void* k_cache, void* v_cache,
    int32_t num_blocks, int32_t* block_tables, int32_t bt_stride,
    int32_t* context_lens, int32_t max_context, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, float scale, float k_scale, float v_scale,
    void* workspace, size_t workspace_bytes, void* stream);

kv_status paged_attn_decode_append_fp8_per_head(
    void* out, const void* q, const void* k_new, const void* v_new,
    const int32_t* new_blocks, void* k_cache, void* v_cache,
    int32_t num_blocks, int32_t* block_tables, int32_t bt_stride,
    int32_t* context_lens, int32_t max_context, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, float scale, const float* k_scales,
    const float* v_scales, void* workspace, size_t workspace_bytes,
    void* stream);

/* ---------------------------------------------------------------------
 * Prefix cache over a block pool ["PagedAttention Nedir?" (bitcanli.com),
 * section "Prefix Sharing Nasıl Çalışır?"]: the K/V of a prompt's leading
 * tokens is reused only for an equal token sequence under the same model
 * context, found by keys that cover a block's contents and the context
 * before it, while the blocks are still cached. Host functions; no GPU.
 *   Key of full block i of a prompt (kv_prefix_block_key): FNV-1a-64 over
 *   the little-endian bytes of (key of block i-1, 0 for the first; salt;
 *   the block's block_size token ids as int32). The salt identifies the
 *   model / adapter context. Only full blocks are keyed.
 *   An entry keeps its block id, parent key and tokens; a key matches only
 *   if they are equal (a hash collision is a miss, never a wrong reuse).
 *   Blocks a lookup or insert passes are stamped with increasing ticks from
 *   the chain's last block to its first; eviction frees blocks only the
 *   cache references (refcount 1), oldest stamp first.
 * The cache holds one pool reference per cached block; the pool must
 * outlive it. One host thread per pool. */
typedef struct kv_prefix_cache kv_prefix_cache;

uint64_t kv_prefix_block_key(uint64_t parent, uint64_t salt,
                             const int32_t* tokens, int32_t block_size);

kv_status kv_prefix_cache_create(kv_pool* pool, uint64_t salt,
                                 kv_prefix_cache** out);
/* Drops the cache's references (blocks only it held return to the pool). */
void kv_prefix_cache_destroy(kv_prefix_cache* cache);

/* Longest cached run of full blocks at the start of tokens[0, n): their ids
 * go to out_blocks (room for n / block_size), their count to *num_blocks,
 * and each gets one more reference for the caller's block table. */
kv_status kv_prefix_cache_lookup(kv_prefix_cache* cache, const int32_t* tokens,
                                 int32_t n, int32_t* out_blocks,
                                 int32_t* num_blocks);

/* blocks[i] holds the K/V of tokens [i*B, (i+1)*B) (the caller's table row,
 * written). Adds the full blocks not cached yet (one cache reference each),
 * keeps equal entries, stops at a colliding key; *num_inserted (may be NULL)
 * = entries added. KV_EINVAL (nothing changed) if a block to add is not
 * live. */
kv_status kv_prefix_cache_insert(kv_prefix_cache* cache, const int32_t* tokens,
                                 int32_t n, const int32_t* blocks,
                                 int32_t* num_inserted);

/* Free up to n blocks only the cache references, least recently used
 * first; their ids go to freed (room for n; may be NULL). Returns the count
 * (-1 on a bad argument). */
int32_t kv_prefix_cache_evict(kv_prefix_cache* cache, int32_t n,
                              int32_t* freed);

/* Entries held (-1 if cache is NULL). */
int32_t kv_prefix_cache_size(const kv_prefix_cache* cache);

/* ---------------------------------------------------------------------
 * Contiguous KV cache on demand-mapped virtual memory ["Makale Bülteni —
 * vAttention", section "İddia ve Gerçeklik: vAttention"]: a virtually
 * contiguous buffer is reserved for every sequence's maximum context at
 * creation (no physical memory); physical pages are created and mapped
 * into it only as sequences grow, so the contiguous kernels above
 * (contig_attn_decode, contig_attn_prefill, kv_reshape_and_cache with
 * slot = s * max_context + position) run on it unchanged.
 *   Layout: K and V each [max_seqs, Hkv, max_context, D] of `dtype`
 *   (seq_stride = max_context). The unit of mapping is a page of
 *   page_tokens rows of one (sequence, KV head) in one tensor: a sequence
 *   of L tokens holds 2 * Hkv * ceil(L / page_tokens) pages.
 *   page_tokens: a multiple of 16 that divides max_context, whose pages
 *   (page_tokens * D * sizeof(dtype) bytes) are a multiple of the device's
 *   mapping granularity (kv_vcache_granularity).
 * Host functions; they run HIP virtual-memory calls (hipMemAddressReserve,
 * hipMemCreate, hipMemMap, hipMemSetAccess, hipMemUnmap) on the device that
 * is current at kv_vcache_create, and launch no kernel. A kernel may read
 * or write only tokens [0, L) of a sequence reserved up to L: other
 * addresses of the range are unmapped. Released pages keep their physical
 * memory in the cache's pool and are mapped again before new pages are
 * created; kv_vcache_destroy frees everything. kv_vcache_release (when it
 * unmaps anything) and kv_vcache_destroy first wait for all work queued on
 * the cache's device (hipDeviceSynchronize), so a kernel still reading the
 * pages finishes before they are unmapped; they are therefore not for use
 * inside a captured graph.
 * Errors: KV_EINVAL (arguments), KV_ENOMEM (device memory), KV_EHIP (other
 * HIP failures); a failed reserve leaves the mapping unchanged. The calls
 * on a cache come from one host thread; the cache's own mapping thread
 * serves kv_vcache_prefetch requests (the newsletter's mapping ahead of
 * need, off the critical path). One mutex guards the cache, so a call that
 * arrives while that thread runs a request waits for the request. */
typedef struct kv_vcache kv_vcache;

/* Minimum mapping granularity of the current device, in bytes. */
kv_status kv_vcache_granularity(size_t* bytes);

kv_status kv_vcache_create(int32_t max_seqs, int32_t max_context,
                           int32_t num_kv_heads, int32_t head_dim,
                           kv_dtype dtype, int32_t page_tokens,
                           kv_vcache** out);
void kv_vcache_destroy(kv_vcache* cache);

/* Device base addresses of the K and V ranges. */
kv_status kv_vcache_ptrs(const kv_vcache* cache, void** k, void** v);

/* Map pages so that tokens [0, num_tokens) of sequence seq are backed;
 * *pages_mapped (may be NULL) = pages this call mapped. Never unmaps. */
kv_status kv_vcache_reserve(kv_vcache* cache, int32_t seq, int32_t num_tokens,
                            int32_t* pages_mapped);

/* Queue a request that tokens [0, num_tokens) of sequence seq be backed,
 * for the cache's mapping thread (started by the first request), and
 * return at once. A later kv_vcache_reserve over the same tokens then finds
 * the pages mapped, or waits for the request being served. Argument errors
 * are returned here; failures of the mapping itself are reported by
 * kv_vcache_sync (and the pages stay unmapped, so a later reserve maps them
 * or reports its own error). */
kv_status kv_vcache_prefetch(kv_vcache* cache, int32_t seq,
                             int32_t num_tokens);

/* Wait until every queued request has been served; return (and clear) the
 * first failure any of them met since the last sync. */
kv_status kv_vcache_sync(kv_vcache* cache);

/* Unmap all pages of sequence seq (their memory stays in the pool); queued
 * requests for seq are dropped. */
kv_status kv_vcache_release(kv_vcache* cache, int32_t seq);

/* Pages mapped per region of sequence seq (-1 on a bad argument). */
int32_t kv_vcache_seq_pages(const kv_vcache* cache, int32_t seq);

/* Physical bytes mapped now / held (mapped + pooled); -1 if cache is NULL. */
int64_t kv_vcache_mapped_bytes(const kv_vcache* cache);
int64_t kv_vcache_held_bytes(const kv_vcache* cache);

#ifdef __cplusplus
}
#endif

#endif /* KVPAGED_H */
