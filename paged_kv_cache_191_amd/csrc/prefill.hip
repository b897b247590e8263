// Chunked-prefill attention over a paged or contiguous KV cache.
//
// Every query of a chunk attends, causally, to the keys at or before its
// absolute position, reading K/V through the block table. The vAttention
// newsletter ("İddia ve Gerçeklik") reports paged FlashAttention-2 and
// FlashInfer prefill kernels running 37-42% slower than contiguous ones on
// A100; the paged and contiguous variants here share one kernel body, with
// only the tile loader's row addressing different.
//
// Fast path (bf16, head_dim 128, block_size % 16 == 0):
//   * A workgroup of 8 waves owns 64 query rows of one sequence and 4 query
//     heads of one KV head (grouped-query packing: the K/V tile in LDS serves
//     all four heads and all 64 rows). Each wave owns one head and 32 rows.
//     A group whose size is not a multiple of 4 ends in a partly empty block
//     of heads; its spare waves repeat a valid head and store nothing.
//   * Keys advance in tiles of 64, gathered through the block table (16
//     consecutive keys share a block) with 16-byte direct global-to-LDS
//     loads into double buffers: unpadded 256-byte rows, XOR-swizzled so
//     that the MFMA operand reads hit distinct banks.
//   * Per tile a wave computes S^T = K Q^T (keys x queries) with
//     v_mfma_f32_32x32x16_bf16, an online softmax in the log2 domain (one
//     query per lane column), and O^T += V^T P^T with the same MFMA (V^T
//     through transposing LDS reads); P stays in the lanes that computed it.
//   * The two halves of the workgroup alternate between MFMA and softmax
//     work (see prefill_pp_kernel).
//   * Causal and context masks are selects (-inf scores), only in the tiles
//     that need them.
// Generic path (other dtypes/shapes): one wave per (query row, head).
//
// The same tile loop also serves decode with a shared prefix: the queries
// of all member sequences of a group (one decode query each, any number of
// members) attend to the group's shared tokens, which are read once per
// group through the first member's block table. The key range is split
// into pieces; each piece leaves an unnormalised partial (max, sum, output)
// per (member, head) that the decode kernels fold in exactly.

#include <type_traits>

#include "device_common.h"

namespace {

using namespace kvp;

constexpr int kD = 128;
constexpr int kBN = 64;            // keys per tile
// LDS reads issued ahead of the first MFMA of a QK / PV block (deeper
// read-ahead measured no faster and costs registers)
constexpr int kQkAhead = 2;
constexpr int kPvAhead = 2;

struct PrefillArgs {
  void* out;
  const void* q;
  const int32_t* cu_q;
  const int32_t* q_start;
  int32_t max_q_len;
  const void* k;
  const void* v;
  const int32_t* bt;
  int32_t bt_stride;
  int32_t num_blocks;
  int32_t block_size;
  int32_t bs_shift;       // log2(block_size) when it is a power of two, else -1
  int32_t seq_stride;
  const int32_t* ctx;
  int32_t num_seqs;
  int32_t hq;
  int32_t hkv;
  int32_t group;
  int32_t head_dim;
  float scale_log2;
  int32_t causal;
  // shared-prefix partials (cu_q = group starts, num_seqs = groups)
  const int32_t* shared;  // [groups] shared tokens of each group
  int32_t* plen;          // [members] shared tokens each member skips
  float* po;              // [nsplit, members, Hq, D] partial outputs
  float* pml;             // [nsplit, members, Hq, 2] (reference max, sum)
  int32_t members;
  int32_t nsplit;
  int32_t ksplit;         // keys per piece (multiple of 64)
  int32_t rowblocks;      // query blocks of 64 members per group
};

__device__ __forceinline__ int clamp_ctx(const PrefillArgs& a, int s,
                                         bool paged) {
  int c = a.ctx[s];
  c = c < 0 ? 0 : c;
  if (paged) {
    const int64_t cap = (int64_t)a.bt_stride * a.block_size;
    if (c > cap) c = (int)cap;
  } else if (c > a.seq_stride) {
    c = a.seq_stride;
  }
  return c;
}

// K and V tiles in LDS: row-major [64 keys][128 d], 256-byte rows with no
// padding; the 16-byte chunk c of row r is stored at chunk c ^ swizzle(r),
// so that the rows read together land in distinct LDS banks:
//   K (read by ds_read_b128, 16 rows at one chunk): swizzle = r & 15;
//   V (read by transpose reads, 4 rows x 32-64 bytes): swizzle =
//     {0, 6, 12, 10}[r & 3].
__device__ __forceinline__ int k_elem(int row, int d) {
  return row * kD + ((((d >> 3) ^ (row & 15))) << 3) + (d & 7);
}
__device__ __forceinline__ int v_elem(int row, int d) {
  const int swz = (0xAC60 >> (4 * (row & 3))) & 15;
  return row * kD + ((((d >> 3) ^ swz)) << 3) + (d & 7);
}

// Lanes l and l ^ 32 combined without LDS: v_permlane32_swap exchanges the
// upper half-wave of one operand with the lower half-wave of the other, so
// with both operands v each lane receives {own value, partner's value} in
// some order; a symmetric operation of the pair gives the combined value.
// Issued as inline assembly: the optimizer folds a symmetric operation of
// the builtin's two results to its first result. The s_nop covers the wait
// states between a VALU write and the swap's read of that register.
struct f32pair { float a, b; };
__device__ __forceinline__ f32pair halves_pair(float v) {
  float a = v, b = v;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return {a, b};
}
__device__ __forceinline__ float halves_max(float v) {
  const f32pair r = halves_pair(v);
  return fmaxf(r.a, r.b);
}
__device__ __forceinline__ float halves_sum(float v) {
  const f32pair r = halves_pair(v);
  return r.a + r.b;
}

typedef __attribute__((address_space(1))) const void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

// ---------------------------------------------------------------------------
// Two-group ("ping-pong") variant of the MFMA path. A workgroup of 8 waves
// owns 64 query rows x 4 query heads of one KV head: waves 0-3 (group 0)
// take rows 0-31, waves 4-7 (group 1) rows 32-63, one head per wave, and
// both groups read the same K/V tiles from LDS. A SIMD runs the matrix
// unit and the vector ALU at the same time only for different waves, so
// the groups are kept half a step apart by workgroup barriers: in each
// phase one group issues its MFMA block (PV of the previous tile, QK of the
// next) while the other runs the softmax of its current tile. Per tile t:
//   phase A(t): group 0 softmax(t)           group 1 PV(t-1), QK(t)
//   phase B(t): group 0 PV(t), QK(t+1)       group 1 softmax(t)
// K tiles are loaded two tiles ahead and V tiles one tile ahead into static
// double buffers. Group 0 issues all of a tile's loads, one every second
// MFMA of its QK block in B phases, so that the requests reach the memory
// pipeline spread out while the other group's softmax runs undisturbed.
// ---------------------------------------------------------------------------
constexpr int kPPWaves = 8;
constexpr int kPPRows = 64;

// Barrier between phases. wait_vm: first wait for this wave's tile loads
// and LDS reads (at the end of A phases: the next phase reads the loaded
// tiles, and loads into the buffers read so far start after it). B phases
// end without a wait: no LDS buffer is rewritten before the next A phase
// ends. The scheduling barriers and empty asm statements keep the compiler
// from moving instructions or memory accesses across the barrier.
__device__ __forceinline__ void phase_barrier(bool wait_vm) {
  if (wait_vm) __builtin_amdgcn_s_waitcnt(0);  // vmcnt, expcnt, lgkmcnt: 0
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

template <bool PAGED, bool PREFIX, bool POW2>
__global__ __launch_bounds__(kPPWaves * kWave, 1) void prefill_pp_kernel(
    PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) bf16 sk0[kBN * kD];
  __shared__ __attribute__((aligned(16))) bf16 sk1[kBN * kD];
  __shared__ __attribute__((aligned(16))) bf16 sv0[kBN * kD];
  __shared__ __attribute__((aligned(16))) bf16 sv1[kBN * kD];
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  using NoMask = std::false_type;
  using Mask = std::true_type;

  const int tid = threadIdx.x;
  // head blocks of 4 query heads inside each KV head's group (the last one
  // partly empty when the group size is not a multiple of 4)
  const int hb_per_kv = (a.group + 3) / 4;
  const int hblocks = a.hkv * hb_per_kv;
  int bx, by, bz, split = 0;
  if (PREFIX) {
    int t = xcd_order(blockIdx.x, gridDim.x);
    bx = t % a.rowblocks;
    t /= a.rowblocks;
    by = t % hblocks;
    t /= hblocks;
    split = t % a.nsplit;
    bz = t / a.nsplit;
  } else {
    const int t = xcd_order(
        blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z),
        gridDim.x * gridDim.y * gridDim.z);
    bx = t % gridDim.x;
    by = (t / gridDim.x) % gridDim.y;
    bz = t / (gridDim.x * gridDim.y);
  }
  const int s = bz;
  int qbeg, nq;
  if (PREFIX) {
    qbeg = min(max(a.cu_q[s], 0), a.members);
    nq = min(max(a.cu_q[s + 1], qbeg), a.members) - qbeg;
  } else {
    qbeg = a.cu_q[s];
    nq = a.cu_q[s + 1] - qbeg;
  }
  const int q0 = (PREFIX ? bx : (gridDim.x - 1 - bx)) * kPPRows;
  if (q0 >= nq) return;
  const int nrows = min(kPPRows, nq - q0);
  const int trow = PREFIX ? qbeg : s;
  const int ctx = clamp_ctx(a, trow, PAGED);
  int kv_beg = 0, kv_end, pos_first = 0;
  if (PREFIX) {
    const int P = min(max(a.shared[s], 0), ctx) & ~15;
    if (by == 0 && split == 0)
      for (int i = tid; i < nrows; i += kPPWaves * kWave) {
        const int m = qbeg + q0 + i;
        a.plen[m] = min(P, clamp_ctx(a, m, PAGED)) & ~15;
      }
    if (P == 0) return;
    kv_beg = split * a.ksplit;
    kv_end = min(P, kv_beg + a.ksplit);
  } else {
    pos_first = a.q_start[s] + q0;
    const int pos_last = pos_first + nrows - 1;
    kv_end = a.causal ? min(ctx, pos_last + 1) : ctx;
    kv_end = kv_end < 0 ? 0 : kv_end;
  }

  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = w >> 2;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int g2 = lane >> 5;
  const int kvh = by / hb_per_kv;
  const int h_in_grp = (by % hb_per_kv) * 4 + (w & 3);
  // A wave past the group's last head repeats that head's work (its tile
  // loads and barriers are the workgroup's) and stores nothing.
  const bool h_ok = h_in_grp < a.group;
  const int h = kvh * a.group + (h_ok ? h_in_grp : a.group - 1);
  const int row0 = q0 + 32 * grp;  // first query row of this group
  if (PREFIX && kv_beg >= kv_end) {
    if (h_ok && row0 + l32 < nrows + q0 && g2 == 0) {
      const int64_t idx =
          ((int64_t)split * a.members + qbeg + row0 + l32) * a.hq + h;
      a.pml[2 * idx] = -INFINITY;
      a.pml[2 * idx + 1] = 0.f;
    }
    return;
  }
  if (kv_end <= kv_beg) {
    // no key at all (empty context): zero rows
    if (!PREFIX && h_ok && row0 + l32 < q0 + nrows) {
      bf16* op = (bf16*)a.out + ((int64_t)(qbeg + row0 + l32) * a.hq + h) * kD +
                 64 * g2;
#pragma unroll
      for (int i = 0; i < 8; ++i) st16(op + 8 * i, u32x4{0, 0, 0, 0});
    }
    return;
  }

  // Q^T (B operand of S^T = K Q^T): lane holds query l32 of its group,
  // d = 16 ks + 8 g2 + e. Rows past the block repeat its last row.
  bf16x8 qop[8];
  {
    const int qr = qbeg + min(row0 + l32, q0 + nrows - 1);
    const bf16* qp = (const bf16*)a.q + ((int64_t)qr * a.hq + h) * kD + 8 * g2;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qop[ks] = as_bf16x8(ld16(qp + 16 * ks));
  }
  const int my_pos = pos_first + 32 * grp + l32;

  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m_run = -INFINITY, l_part = 0.f;
  f32x16 sacc[2];
  u32x4 pk[4];  // P^T of the last softmax, packed for the PV MFMAs

  const int n_tiles = (kv_end + kBN - 1) / kBN;
  const int j_beg = kv_beg / kBN;
  // Tiles below n_full need no mask for this group's rows.
  int n_full = kv_end / kBN;
  if (!PREFIX && a.causal) n_full = min(n_full, (pos_first + 32 * grp + 1) / kBN);
  n_full = max(n_full, j_beg);

  // ---- tile loads: wave w moves keys 8w..8w+7 of a tile (2 instructions
  // of 4 rows per tensor); table entries are read one step ahead.
  const int ld_row = lane >> 4;
  const int ld_pc = lane & 15;
  const int64_t head_row0 =
      (int64_t)kvh * (PAGED ? a.block_size : a.seq_stride);
  typedef __attribute__((address_space(4))) const int32_t* cptr_t;
  // block index and offset of a key position (shift and mask for the usual
  // power-of-two block sizes: no branch inside the tile loop)
  auto blk_of = [&](int x) __attribute__((always_inline)) {
    if constexpr (POW2) return x >> a.bs_shift;
    else return x / a.block_size;
  };
  auto off_in_blk = [&](int x) __attribute__((always_inline)) {
    if constexpr (POW2) return x & (a.block_size - 1);
    else return x % a.block_size;
  };
  // Key slot `slot` (0..7) of a tile: keys 8 slot .. 8 slot + 7.
  auto group_base = [&](int j, int slot) __attribute__((always_inline)) {
    return min((j * kBN + 8 * slot) & ~15, (kv_end - 1) & ~15);
  };
  auto table_block = [&](int j, int slot) __attribute__((always_inline)) {
    if (!PAGED) return 0;
    j = min(j, n_tiles - 1);
    return ((cptr_t)a.bt)[(int64_t)trow * a.bt_stride +
                          blk_of(group_base(j, slot))];
  };
  // Per-lane parts of the load addresses: the 16-byte chunk each lane moves
  // (swizzled), as a byte offset inside a head row. The swizzle depends on
  // the row modulo 16, the same for slots w and w + 4.
  int chunk_off[2][2];  // [K/V][n]
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int row = 8 * w + 4 * n + ld_row;
    chunk_off[0][n] = 16 * (ld_pc ^ (row & 15));
    chunk_off[1][n] = 16 * (ld_pc ^ ((0xAC60 >> (4 * (row & 3))) & 15));
  }
  // One 16-byte-per-lane load: rows 8 slot + 4 n .. + 3 of tile j (block
  // table entry b) into buffer `buf`.
  // Wave-uniform address parts: this head's first row in each tensor, and
  // the bytes of one block (all heads) of a tensor.
  const int64_t head_row_seq =
      PAGED ? head_row0 : (int64_t)s * a.hkv * a.seq_stride + head_row0;
  const char* k_head = (const char*)a.k + head_row_seq * (kD * 2);
  const char* v_head = (const char*)a.v + head_row_seq * (kD * 2);
  const uint64_t blk_bytes = (uint64_t)a.hkv * a.block_size * (kD * 2);
  auto load1 = [&](auto is_v, auto buf, int j, int b, int slot, int n)
      __attribute__((always_inline)) {
    constexpr bool V = decltype(is_v)::value;
    bf16* dst = V ? (decltype(buf)::value ? sv1 : sv0)
                  : (decltype(buf)::value ? sk1 : sk0);
    // wave-uniform byte address of head row `base` (the first row of the
    // 16-key group), plus a 32-bit per-lane offset: row within the group
    // (keys past the context re-read the last one) and 16-byte chunk
    const char* gbase = V ? v_head : k_head;
    int base = 0;
    if (PAGED) {
      base = group_base(j, slot);
      b = b < 0 ? 0 : (b >= a.num_blocks ? a.num_blocks - 1 : b);
      gbase += (uint64_t)(uint32_t)b * blk_bytes +
               (uint32_t)off_in_blk(base) * (kD * 2);
    }
    const int u = j * kBN + 8 * slot + 4 * n - base;
    const int lim = kv_end - 1 - base;
    const uint32_t off = (uint32_t)(min(u + ld_row, lim) * (kD * 2) +
                                    chunk_off[V ? 1 : 0][n]);
    const uint32_t lds =
        (uint32_t)(uintptr_t)(lptr_t)(&dst[(8 * slot + 4 * n) * kD]);
    // Issued as inline assembly: the compiler then keeps its own LDS read
    // counters exact (it treats a direct-to-LDS load as an unordered LDS
    // event and would drain every LDS read behind it). Completion is
    // awaited explicitly: every phase that follows a load phase ends with
    // s_waitcnt 0 before the barrier (phase_barrier(true)).
    // m0 is named as clobbered; no other code of this kernel uses m0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    asm volatile(
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %2"
        :
        : "v"(off), "s"(lds), "s"(gbase)
        : "m0");
#pragma clang diagnostic pop
  };
  // All eight waves: each moves its own slot w.
  auto load = [&](auto is_v, auto buf, int j, int b)
      __attribute__((always_inline)) {
    load1(is_v, buf, j, b, w, 0);
    load1(is_v, buf, j, b, w, 1);
  };
  using KT = std::false_type;
  using VT = std::true_type;

  // ---- MFMA blocks
  // The scheduler is asked to keep each LDS read two steps ahead of its
  // MFMA (short read-ahead keeps register use down).
  // Tile loads of phase B(t), slot w or w + 4 for group 0, w - 4 or w for
  // group 1 (sl = 0, 1), rows 4 n ..: group 0 moves K(t+2) into the K buffer
  // of parity t, one load every fourth MFMA of its QK block; group 1 moves
  // V(t+1) into the V buffer of parity t + 1 before its softmax. A K tile
  // past the last is clamped to it (the buffer written is free).
  int kb_next[2] = {0, 0};  // table entries: K(t+2) (group 0), V(t+1) (group 1)
  const int slot0 = grp == 0 ? w : w - 4;
  auto tile_load = [&](auto par, int sl, int n, int t)
      __attribute__((always_inline)) {
    constexpr int PAR = decltype(par)::value;
    if (grp == 0)
      load1(KT{}, std::integral_constant<int, PAR>{}, min(t + 2, n_tiles - 1),
            kb_next[sl], slot0 + 4 * sl, n);
    else
      load1(VT{}, std::integral_constant<int, 1 - PAR>{}, t + 1, kb_next[sl],
            slot0 + 4 * sl, n);
  };
  // table entries of the next phase B's loads (tile t + 3 or t + 2)
  auto next_entries = [&](int t) __attribute__((always_inline)) {
#pragma unroll
    for (int sl = 0; sl < 2; ++sl)
      kb_next[sl] = table_block(t + (grp == 0 ? 3 : 2), slot0 + 4 * sl);
  };
  // QK of K buffer `buf`; with LD, group 0's loads of phase B(t) interleaved.
  auto qk = [&](auto buf, auto ld, auto par, int t)
      __attribute__((always_inline)) {
    constexpr bool LD = decltype(ld)::value;
    const bf16* K_ = decltype(buf)::value ? sk1 : sk0;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8 ka = as_bf16x8(
            ld16(&K_[k_elem(32 * kb + l32, 16 * ks + 8 * g2)]));
        sacc[kb] = mfma32(ka, qop[ks], sacc[kb]);
        const int i = 8 * kb + ks;
        if (LD && (i & 3) == 3) tile_load(par, i >> 3, (i >> 2) & 1, t);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x100, kQkAhead, 0);
#pragma unroll
    for (int i = 0; i < 16 - kQkAhead; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kQkAhead, 0);
    __builtin_amdgcn_sched_barrier(0);
    if (LD) next_entries(t);
  };
  const int trs = lane & 15;
  const int trd = 16 * ((lane >> 4) & 1) + 4 * (trs & 3);
  auto pv = [&](auto buf) __attribute__((always_inline)) {
    const bf16* V_ = decltype(buf)::value ? sv1 : sv0;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const bf16x8 pop = as_bf16x8(pk[kk]);
      const int r0 = 16 * kk + 4 * g2 + (trs >> 2);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const u32x2 lo = lds_read_tr16(&V_[v_elem(r0, 32 * db + trd)]);
        const u32x2 hi = lds_read_tr16(&V_[v_elem(r0 + 8, 32 * db + trd)]);
        const bf16x8 va = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
        oacc[db] = mfma32(va, pop, oacc[db]);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kPvAhead, 0);
#pragma unroll
    for (int i = 0; i < 16 - kPvAhead; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kPvAhead, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  using NoLd = std::false_type;
  using Ld = std::true_type;
  // ---- softmax of tile j (vector ALU): masks, lazy rescale, P^T packed.
  auto softmax = [&](int j, auto masked) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(masked)::value;
    const int tile0 = j * kBN;
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (MASK) {
          const int key = tile0 + 32 * kb + 8 * (r >> 2) + 4 * g2 + (r & 3);
          const bool dead = key >= kv_end || (a.causal && key > my_pos);
          sacc[kb][r] = dead ? -INFINITY : sacc[kb][r];
        }
        mx = fmaxf(mx, sacc[kb][r]);
      }
    mx = halves_max(mx) * a.scale_log2;
    if (__any(mx > m_run + 8.f)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_run - m_new);
      m_run = m_new;
      l_part *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db) oacc[db] *= alpha;
    }
    const float m_ref = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        sacc[kb][r] = fast_exp2(__builtin_fmaf(sacc[kb][r], a.scale_log2,
                                               -m_ref));
    // P^T: lane holds query l32; k-slot e of MFMA kk <-> key
    // 16 kk + 8 (e / 4) + 4 g2 + e % 4 of the tile.
    float psum = 0.f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int kb = kk >> 1;
      const int rb = 8 * (kk & 1);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pk[kk][e] = pack_bf16(sacc[kb][rb + 2 * e], sacc[kb][rb + 2 * e + 1]);
        psum += sacc[kb][rb + 2 * e] + sacc[kb][rb + 2 * e + 1];
      }
    }
    l_part += psum;
    // Pin the results here: the softmax must finish in its own phase, not
    // sink into the next MFMA block of this wave.
    asm volatile("" : "+v"(pk[0]), "+v"(pk[1]), "+v"(pk[2]), "+v"(pk[3]),
                 "+v"(l_part), "+v"(m_run));
  };

  // ---- prologue: K(j_beg) (and, at the start of the first phase, K(j_beg+1)
  // and V(j_beg)), one slot per wave.
  {
    const int b0 = table_block(j_beg, w);
    if (j_beg & 1) load(KT{}, B1{}, j_beg, b0);
    else load(KT{}, B0{}, j_beg, b0);
    next_entries(j_beg - 1);
    phase_barrier(true);
    // first phase ("B(j_beg - 1)"): loads K(j_beg+1), V(j_beg); group 0
    // computes QK(j_beg); group 1 waits.
    if (j_beg + 1 < n_tiles) {
      const int b1 = table_block(j_beg + 1, w);
      if ((j_beg + 1) & 1) load(KT{}, B1{}, j_beg + 1, b1);
      else load(KT{}, B0{}, j_beg + 1, b1);
    }
    if (j_beg & 1) load(VT{}, B1{}, j_beg, b0);
    else load(VT{}, B0{}, j_beg, b0);
    if (grp == 0) {
      if (j_beg & 1) qk(B1{}, NoLd{}, B0{}, 0);
      else qk(B0{}, NoLd{}, B0{}, 0);
    }
  }
  phase_barrier(false);

  if (grp == 0) {
    // A(t): softmax(t); B(t): PV(t) from V[t&1], QK(t+1) from K[(t+1)&1]
    // with the loads of K(t+2) interleaved
    auto iter = [&](auto par, int t, auto masked) __attribute__((always_inline)) {
      constexpr int PAR = decltype(par)::value;
      softmax(t, masked);
      phase_barrier(true);
      if constexpr (PAR) pv(B1{}); else pv(B0{});
      if (t + 1 < n_tiles) {
        if constexpr (PAR) qk(B0{}, Ld{}, par, t); else qk(B1{}, Ld{}, par, t);
      }
      phase_barrier(false);
    };
    auto run = [&](int t0, int t1, auto masked) __attribute__((always_inline)) {
      int t = t0;
      if ((t & 1) && t < t1) iter(B1{}, t++, masked);
      for (; t + 1 < t1; t += 2) {
        iter(B0{}, t, masked);
        iter(B1{}, t + 1, masked);
      }
      if (t < t1) iter(B0{}, t, masked);
    };
    run(j_beg, n_full, NoMask{});
    run(n_full, n_tiles, Mask{});
  } else {
    // A(t): PV(t-1) from V[(t-1)&1], QK(t) from K[t&1]; B(t): loads of
    // V(t+1), softmax(t)
    auto iter = [&](auto par, int t, auto masked, auto with_pv)
        __attribute__((always_inline)) {
      constexpr int PAR = decltype(par)::value;
      if constexpr (decltype(with_pv)::value) {
        if constexpr (PAR) pv(B0{}); else pv(B1{});
      }
      if constexpr (PAR) qk(B1{}, NoLd{}, par, t); else qk(B0{}, NoLd{}, par, t);
      phase_barrier(true);
      if (t + 1 < n_tiles) {
#pragma unroll
        for (int k = 0; k < 4; ++k) tile_load(par, k >> 1, k & 1, t);
        next_entries(t);
      }
      softmax(t, masked);
      phase_barrier(false);
    };
    auto run = [&](int t0, int t1, auto masked) __attribute__((always_inline)) {
      int t = t0;
      if (t == j_beg && t < t1) {  // first tile: no PV yet
        if (t & 1) iter(B1{}, t, masked, std::false_type{});
        else iter(B0{}, t, masked, std::false_type{});
        ++t;
      }
      if ((t & 1) && t < t1) iter(B1{}, t++, masked, std::true_type{});
      for (; t + 1 < t1; t += 2) {
        iter(B0{}, t, masked, std::true_type{});
        iter(B1{}, t + 1, masked, std::true_type{});
      }
      if (t < t1) iter(B0{}, t, masked, std::true_type{});
    };
    run(j_beg, n_full, NoMask{});
    run(n_full, n_tiles, Mask{});
    // last phase: PV(n_tiles - 1)
    if ((n_tiles - 1) & 1) pv(B1{});
    else pv(B0{});
  }

  // ---- outputs of this group's rows
  l_part = halves_sum(l_part);
  const bool row_ok = h_ok && row0 + l32 < q0 + nrows;
  if (PREFIX) {
    if (row_ok) {
      const int64_t idx =
          ((int64_t)split * a.members + qbeg + row0 + l32) * a.hq + h;
      float* po = a.po + idx * kD + 4 * g2;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4)
          *reinterpret_cast<f32x4*>(po + 32 * db + 8 * a4) =
              f32x4{oacc[db][4 * a4], oacc[db][4 * a4 + 1],
                    oacc[db][4 * a4 + 2], oacc[db][4 * a4 + 3]};
      if (g2 == 0) {
        a.pml[2 * idx] = m_run;
        a.pml[2 * idx + 1] = l_part;
      }
    }
    return;
  }
  if (row_ok) {
    const float inv = l_part > 0.f ? 1.f / l_part : 0.f;
    bf16* op = (bf16*)a.out + ((int64_t)(qbeg + row0 + l32) * a.hq + h) * kD +
               4 * g2;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        u32x2 v2;
        v2[0] = pack_bf16(oacc[db][4 * a4] * inv, oacc[db][4 * a4 + 1] * inv);
        v2[1] =
            pack_bf16(oacc[db][4 * a4 + 2] * inv, oacc[db][4 * a4 + 3] * inv);
        *reinterpret_cast<u32x2*>(op + 32 * db + 8 * a4) = v2;
      }
  }
}

// Generic path: one wave per (query head, query row, sequence).
template <typename T, bool PAGED>
__global__ __launch_bounds__(kWave) void prefill_generic_kernel(PrefillArgs a) {
  const int h = blockIdx.x;
  const int i = blockIdx.y;
  const int s = blockIdx.z;
  const int qbeg = a.cu_q[s];
  const int nq = a.cu_q[s + 1] - qbeg;
  if (i >= nq) return;
  const int lane = threadIdx.x;
  const int D = a.head_dim;
  const int g = h / a.group;
  const int ctx = clamp_ctx(a, s, PAGED);
  const int pos = a.q_start[s] + i;
  int nvis = a.causal ? min(ctx, pos + 1) : ctx;
  nvis = nvis < 0 ? 0 : nvis;
  float qv[4], acc[4];
  const T* qp = (const T*)a.q + ((int64_t)(qbeg + i) * a.hq + h) * D;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int d = lane + kWave * k;
    qv[k] = d < D ? to_f32<T>(qp[d]) : 0.f;
    acc[k] = 0.f;
  }
  float m_run = -INFINITY, l = 0.f;
  for (int p = 0; p < nvis; ++p) {
    int64_t row;  // head row of (key p, KV head g)
    if (PAGED) {
      int b = a.bt[(int64_t)s * a.bt_stride + p / a.block_size];
      b = b < 0 ? 0 : (b >= a.num_blocks ? a.num_blocks - 1 : b);
      row = ((int64_t)b * a.hkv + g) * a.block_size + p % a.block_size;
    } else {
      row = ((int64_t)s * a.hkv + g) * a.seq_stride + p;
    }
    const T* kp = (const T*)a.k + row * D;
    const T* vp = (const T*)a.v + row * D;
    float dot = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int d = lane + kWave * k;
      if (d < D) dot += qv[k] * to_f32<T>(kp[d]);
    }
    dot = wave_sum(dot);
    const float x = dot * a.scale_log2;
    const float m_new = fmaxf(m_run, x);
    const float alpha = fast_exp2(m_run - m_new);
    const float pr = fast_exp2(x - m_new);
    l = l * alpha + pr;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int d = lane + kWave * k;
      const float vv = d < D ? to_f32<T>(vp[d]) : 0.f;
      acc[k] = acc[k] * alpha + pr * vv;
    }
    m_run = m_new;
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  T* op = (T*)a.out + ((int64_t)(qbeg + i) * a.hq + h) * D;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int d = lane + kWave * k;
    if (d < D) op[d] = from_f32<T>(acc[k] * inv);
  }
}

kv_status run_prefill(const char* name, bool paged, PrefillArgs a,
                      kv_dtype dtype, hipStream_t st) {
  if (dtype != KV_F32 && dtype != KV_BF16)
    return kvp_fail(KV_EINVAL, "%s: unknown dtype %d", name, (int)dtype);
  if (!(a.scale_log2 > 0.f) || !(a.scale_log2 < INFINITY))
    return kvp_fail(KV_EINVAL, "%s: scale must be finite and > 0", name);
  if (a.num_seqs < 0 || a.hq <= 0 || a.hkv <= 0 || a.hq % a.hkv != 0 ||
      a.head_dim <= 0 || a.max_q_len < 0)
    return kvp_fail(KV_EINVAL, "%s: bad shape (S=%d Hq=%d Hkv=%d D=%d)", name,
                    a.num_seqs, a.hq, a.hkv, a.head_dim);
  if (paged && (a.block_size <= 0 || a.bt_stride <= 0 || a.num_blocks <= 0))
    return kvp_fail(KV_EINVAL, "%s: bad paging arguments", name);
  if (paged && (int64_t)a.num_blocks * a.block_size * a.hkv > INT32_MAX)
    return kvp_fail(KV_EUNSUPPORTED, "%s: pool of more than 2^31 head rows",
                    name);
  if (!paged && a.seq_stride <= 0)
    return kvp_fail(KV_EINVAL, "%s: seq_stride must be > 0", name);
  if (a.num_seqs == 0 || a.max_q_len == 0) return KV_OK;
  if (!a.out || !a.q || !a.cu_q || !a.q_start || !a.k || !a.v || !a.ctx ||
      (paged && !a.bt))
    return kvp_fail(KV_EINVAL, "%s: NULL pointer", name);
  a.group = a.hq / a.hkv;
  a.bs_shift = (a.block_size > 0 && (a.block_size & (a.block_size - 1)) == 0)
                   ? __builtin_ctz((unsigned)a.block_size)
                   : -1;
  const bool fast = dtype == KV_BF16 && a.head_dim == kD &&
                    (!paged || a.block_size % 16 == 0);
  if (fast) {
    dim3 grid((a.max_q_len + kPPRows - 1) / kPPRows,
              a.hkv * ((a.group + 3) / 4), a.num_seqs);
    if ((int64_t)grid.x * grid.y * grid.z > INT32_MAX)
      return kvp_fail(KV_EUNSUPPORTED, "%s: too many query blocks", name);
    if (!paged)
      prefill_pp_kernel<false, false, false><<<grid, kPPWaves * kWave, 0, st>>>(a);
    else if (a.bs_shift >= 0)
      prefill_pp_kernel<true, false, true><<<grid, kPPWaves * kWave, 0, st>>>(a);
    else
      prefill_pp_kernel<true, false, false><<<grid, kPPWaves * kWave, 0, st>>>(a);
    KVP_LAUNCH_CHECK(name);
    return KV_OK;
  }
  if (a.head_dim > 4 * kWave)
    return kvp_fail(KV_EUNSUPPORTED, "%s: head_dim %d > 256", name,
                    a.head_dim);
  if (a.max_q_len > 65535)
    return kvp_fail(KV_EUNSUPPORTED, "%s: generic path takes <= 65535 queries "
                    "per sequence", name);
  dim3 grid(a.hq, a.max_q_len, a.num_seqs);
  if (dtype == KV_F32) {
    if (paged)
      prefill_generic_kernel<float, true><<<grid, kWave, 0, st>>>(a);
    else
      prefill_generic_kernel<float, false><<<grid, kWave, 0, st>>>(a);
  } else {
    if (paged)
      prefill_generic_kernel<bf16, true><<<grid, kWave, 0, st>>>(a);
    else
      prefill_generic_kernel<bf16, false><<<grid, kWave, 0, st>>>(a);
  }
  KVP_LAUNCH_CHECK(name);
  return KV_OK;
}

}  // namespace

kv_status kvp_prefix_partials(const KvpPrefixJob& j, hipStream_t st) {
  PrefillArgs a = {};
  a.q = j.q;
  a.k = j.k;
  a.v = j.v;
  a.bt = j.bt;
  a.bt_stride = j.bt_stride;
  a.num_blocks = j.num_blocks;
  a.block_size = j.block_size;
  a.bs_shift = (j.block_size > 0 && (j.block_size & (j.block_size - 1)) == 0)
                   ? __builtin_ctz((unsigned)j.block_size)
                   : -1;
  a.ctx = j.ctx;
  a.cu_q = j.group_starts;
  a.num_seqs = j.num_groups;
  a.hq = j.hq;
  a.hkv = j.hkv;
  a.group = j.hq / j.hkv;
  a.head_dim = kD;
  a.scale_log2 = j.scale_log2;
  a.causal = 0;
  a.shared = j.shared_lens;
  a.plen = j.plen;
  a.po = j.po;
  a.pml = j.pml;
  a.members = j.members;
  a.nsplit = j.nsplit;
  a.ksplit = j.ksplit;
  a.rowblocks = (j.max_group_size + kPPRows - 1) / kPPRows;
  const int64_t n = (int64_t)a.rowblocks * (a.hkv * ((a.group + 3) / 4)) *
                    a.nsplit *
                    j.num_groups;
  if (n > INT32_MAX)
    return kvp_fail(KV_EUNSUPPORTED, "shared-prefix decode: too many groups");
  if (a.bs_shift >= 0)
    prefill_pp_kernel<true, true, true><<<(unsigned)n, kPPWaves * kWave, 0, st>>>(a);
  else
    prefill_pp_kernel<true, true, false><<<(unsigned)n, kPPWaves * kWave, 0, st>>>(a);
  KVP_LAUNCH_CHECK("paged_attn_decode_shared_prefix");
  return KV_OK;
}

extern "C" kv_status paged_attn_prefill(
    void* out, const void* q, const int32_t* cu_q_lens,
    const int32_t* q_start_pos, int32_t max_q_len, const void* k_cache,
    const void* v_cache, int32_t num_blocks, const int32_t* block_tables,
    int32_t bt_stride, const int32_t* context_lens, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, float scale, int32_t causal, kv_dtype dtype,
    void* stream) {
  PrefillArgs a = {};
  a.out = out;
  a.q = q;
  a.cu_q = cu_q_lens;
  a.q_start = q_start_pos;
  a.max_q_len = max_q_len;
  a.k = k_cache;
  a.v = v_cache;
  a.bt = block_tables;
  a.bt_stride = bt_stride;
  a.num_blocks = num_blocks;
  a.block_size = block_size;
  a.ctx = context_lens;
  a.num_seqs = num_seqs;
  a.hq = num_q_heads;
  a.hkv = num_kv_heads;
  a.head_dim = head_dim;
  a.scale_log2 = scale * kLog2e;
  a.causal = causal ? 1 : 0;
  return run_prefill("paged_attn_prefill", true, a, dtype, (hipStream_t)stream);
}

extern "C" kv_status contig_attn_prefill(
    void* out, const void* q, const int32_t* cu_q_lens,
    const int32_t* q_start_pos, int32_t max_q_len, const void* k,
    const void* v, int32_t seq_stride, const int32_t* context_lens,
    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, float scale, int32_t causal, kv_dtype dtype,
    void* stream) {
  PrefillArgs a = {};
  a.out = out;
  a.q = q;
  a.cu_q = cu_q_lens;
  a.q_start = q_start_pos;
  a.max_q_len = max_q_len;
  a.k = k;
  a.v = v;
  a.seq_stride = seq_stride;
  a.block_size = 16;
  a.ctx = context_lens;
  a.num_seqs = num_seqs;
  a.hq = num_q_heads;
  a.hkv = num_kv_heads;
  a.head_dim = head_dim;
  a.scale_log2 = scale * kLog2e;
  a.causal = causal ? 1 : 0;
  return run_prefill("contig_attn_prefill", false, a, dtype,
                     (hipStream_t)stream);
}
