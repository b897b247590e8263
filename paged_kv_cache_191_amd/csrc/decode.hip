// Decode attention over a paged or contiguous KV cache.
//
// One query per sequence attends to every token of its context, reading K
// and V through the sequence's block table ["PagedAttention Nedir?"
// (bitcanli.com), "PagedAttention Nasıl Çalışır?", step 4]. The vAttention
// newsletter ("İddia ve Gerçeklik") locates the cost of paging in this
// loop: a table read per block, extra branching, and registers holding page
// indices; the contiguous variant reads a plain [S, Hkv, Lmax, D] buffer.
// Both variants share one kernel body; only the row addressing differs, so
// their timing difference is the table lookup.
//
// Fast path (bf16, head_dim 128, block_size % 16 == 0, any GQA group):
//   * Balanced split ("stream-K"): per KV head, the 32-token tiles of all
//     sequences (ceil(L / 32) per sequence) are laid end to end and cut into
//     n_chunks equal chunks; workgroup (unit, chunk) streams one chunk. Every
//     workgroup moves the same bytes whatever the length mix, and a piece of
//     a sequence always starts on a tile boundary, so no tile is read by two
//     workgroups. The chunk size is derived on the device from the context
//     lengths, so the grid needs no host-side sums.
//   * A chunk covers pieces ("segments") of one or more sequences. The 4
//     waves of the workgroup share each segment tile by tile, then merge
//     their softmax states through LDS. A segment that is a whole sequence
//     writes the output; a cut sequence leaves a partial (max, sum,
//     unnormalised output) that decode_combine_kernel merges exactly.
//   * All query heads of a KV head (up to 16) share one MFMA column block,
//     so each K/V byte is read once from HBM.
//   * Per 32-token tile a wave computes S^T = K Q^T with
//     v_mfma_f32_16x16x32_bf16 (tokens x heads), an online softmax in the
//     log2 domain with lazy rescaling, and O^T += V^T P^T with the same MFMA.
//   * K is loaded straight into the MFMA A-operand layout (each lane 16 B of
//     one token row). V is loaded as whole 256-byte head rows (16 lanes per
//     row) and transposed inside each lane's registers with v_perm_b32: the
//     token order of the PV product is the order in which S^T leaves P in
//     registers, so P never moves between lanes. K/V loads are non-temporal
//     (read once).
//   * Head-row bases of a wave's 16-token groups are fetched once per
//     segment (one lane per group) and broadcast with v_readlane, so each
//     half-tile's address is wave-uniform.
//   * Tiles are 32-aligned in sequence positions (16-token groups never
//     straddle a block); a half tile wholly past the context re-reads the
//     last context group (rows already in flight, served by the cache);
//     tokens past the context are selected out (score -inf, V 0), never
//     multiplied by 0, so NaN in unused slots cannot leak.
// Generic path (fp32, or shapes the fast path does not cover): one
// workgroup of 8 waves per (query head, sequence), lanes over head_dim; the
// tokens go to the waves in groups of 8, each wave keeps its own softmax
// state, and the 8 states are merged exactly through LDS.
//
// Contexts: a context_lens entry outside [0, bound], bound = min(max_context,
// the table's or the sequence's capacity), is clamped into it so that every
// access stays in bounds. The number of such sequences of the last call is
// kept in the workspace header (kv_decode_clamped_count reads it), so that a
// stale bound is visible instead of silently shortening the attention.
//
// Shared prefix (paged_attn_decode_shared_prefix): when groups of sequences
// hold the same first tokens in the same physical blocks (a forked prompt,
// blocks at refcount > 1 ["Makale Bülteni — PagedAttention ve vLLM",
// "İddia ve Gerçeklik"; "PagedAttention Nedir?", "Prefix Sharing Nasıl
// Çalışır?"]), an MFMA pass (prefill.hip) attends every member's query to
// the shared tokens, reading them once per group, and leaves exact partials.
// The stream-K pass above then covers only each sequence's own tokens and
// folds those partials in; the result is the same attention.

#include <stdlib.h>

#include "device_common.h"
#include "fp8_codec.h"

namespace {

using namespace kvp;

constexpr int kD = 128;       // head_dim of the MFMA path
constexpr int kWaves = 4;     // waves per workgroup in the MFMA path
constexpr int kTile = 32;     // tokens per wave iteration
constexpr int kHeadBlk = 16;  // query heads per MFMA column block
constexpr int kMaxSeqs = 4096;  // sequences per launch of the MFMA path
constexpr int kGroupsPerLoad = 64;  // 16-token groups prefetched per wave
constexpr float kRescaleLog2 = 8.f;  // lazy-rescale threshold (log2 units)

struct DecodeArgs {
  void* out;
  const void* q;
  const void* k;
  const void* v;
  const int32_t* bt;
  int32_t bt_stride;
  int32_t num_blocks;
  int32_t block_size;
  int32_t seq_stride;   // contiguous layout: token rows per sequence
  const int32_t* ctx;
  int32_t max_ctx;      // clamp bound of context_lens
  int32_t num_seqs;
  int32_t hq;
  int32_t hkv;
  int32_t group;        // hq / hkv
  int32_t head_blocks;  // ceil(group / 16)
  int32_t head_dim;
  float scale_log2;     // scale * log2(e) (fp8 K/V per tensor: times k_scale)
  float v_scale;        // fp8 K/V: scale of V (outputs are multiplied by it)
  const float* k_scales;  // fp8 K/V per KV head [Hkv] (NULL: per tensor)
  const float* v_scales;
  int32_t* ws_hdr;      // workspace header: [0] = sequences clamped
  int32_t clamp_add;    // 0: store the count, 1: add it (later launches)
  int32_t n_chunks;     // chunks per (KV head, head block)
  float* ws_o;          // [n_chunks, 2, Hq, D] unnormalised partial outputs
  float* ws_ml;         // [n_chunks, 2, Hq, 2] (reference max, sum)
  int32_t* ws_cs;       // [S + 1] tile offsets of the sequences
  int32_t* ws_nb;       // [S] with append: new_blocks copied to the device
  float* ws_inv;        // [2 Hkv] fp8 with append: 1 / scale, K then V heads
  // shared prefix (all NULL / 0 for plain decode)
  const int32_t* plen;  // [S] leading tokens covered by the prefix partials
  const float* pre_o;   // [n_psplit, pre_stride, Hq, D]
  const float* pre_ml;  // [n_psplit, pre_stride, Hq, 2]
  int32_t n_psplit;
  int32_t pre_stride;   // sequences between two pieces of pre_o / pre_ml
  float* whole_o;       // [S, Hq, D] own part of a sequence in one chunk
  float* whole_ml;      // [S, Hq, 2]
  // decode with this step's token appended (k_new NULL: plain decode)
  const void* k_new;    // [S, Hkv, D] the token's K and V (bf16)
  const void* v_new;
  const int32_t* new_blocks;  // [S] block for table[s][L / B] (-1: keep)
  int32_t* bt_w;        // the table, lengths and caches, written by the
  int32_t* ctx_w;       // merge kernel once the attention is done
  void* k_cache_w;
  void* v_cache_w;
  int32_t kv8;          // the caches hold fp8 E4M3 codes
  float k_inv, v_inv;   // fp8 K/V with append: 1 / scale of the tensor (the
                        // token is stored as codes; k_scales / v_scales per
                        // head when given)
};

__device__ __forceinline__ int clamp_len(const DecodeArgs& a, int c,
                                         bool paged) {
  c = c < 0 ? 0 : c;
  c = c > a.max_ctx ? a.max_ctx : c;
  if (paged) {
    const int64_t cap = (int64_t)a.bt_stride * a.block_size;
    if (c > cap) c = (int)cap;
  } else if (c > a.seq_stride) {
    c = a.seq_stride;
  }
  return c;
}

__device__ __forceinline__ int clamp_ctx(const DecodeArgs& a, int s,
                                         bool paged) {
  return clamp_len(a, a.ctx[s], paged);
}

// A stored length as the attention sees it: with this step's token
// appended (k_new set), one more when the token's position lies inside the
// table (the condition under which it is stored).
template <bool APPEND>
__device__ __forceinline__ int with_new(const DecodeArgs& a, int stored) {
  if (!APPEND) return stored;
  const int64_t cap = (int64_t)a.bt_stride * a.block_size;
  return stored + (stored >= 0 && stored < cap ? 1 : 0);
}

// Workgroup 0 of a launch records how many of its sequences were clamped.
__device__ __forceinline__ void record_clamped(const DecodeArgs& a, int n) {
  if (!a.ws_hdr) return;
  if (a.clamp_add) a.ws_hdr[0] += n;
  else a.ws_hdr[0] = n;
}

// Leading tokens of sequence s (context L) that the prefix partials cover;
// a multiple of 16, so the sequence's own tiles start on a 16-token group.
__device__ __forceinline__ int shared_of(const DecodeArgs& a, int s, int L) {
  if (!a.plen) return 0;
  int p = a.plen[s];
  p = p < 0 ? 0 : (p > L ? L : p);
  return p & ~15;
}

// Folds piece (mi, li, acc_i[8]) into the running (M, Ls, acc).
__device__ __forceinline__ void fold_piece(float& M, float& Ls, float* acc,
                                           float mi, float li, f32x4 lo4,
                                           f32x4 hi4) {
  if (mi == -INFINITY) return;
  const float m_new = fmaxf(M, mi);
  const float old_scale = fast_exp2(M - m_new);
  const float new_scale = fast_exp2(mi - m_new);
  M = m_new;
  Ls = Ls * old_scale + li * new_scale;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    acc[e] = acc[e] * old_scale + lo4[e] * new_scale;
    acc[4 + e] = acc[4 + e] * old_scale + hi4[e] * new_scale;
  }
}

__device__ __forceinline__ int tiles_of(int tokens) {
  return (tokens + kTile - 1) / kTile;
}

// Tiles per chunk for T tiles in total.
__device__ __forceinline__ int chunk_tiles(int total, int n_chunks) {
  const int c = (total + n_chunks - 1) / n_chunks;
  return c < 1 ? 1 : c;
}

// ---------------------------------------------------------------------------
// MFMA fast path
// ---------------------------------------------------------------------------
// 8 fp8 E4M3 values (two dwords) -> 8 bf16 (exact: every E4M3 value is a
// bf16 value).
__device__ __forceinline__ u32x4 fp8x8_to_bf16(u32x2 w) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    r[2 * i] = __builtin_bit_cast(
        uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, false));
    r[2 * i + 1] = __builtin_bit_cast(
        uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, true));
  }
  return r;
}

// KV8: K/V cache in fp8 E4M3 (one byte per value, converted to bf16 in
// registers; K's scale is folded into scale_log2, V's applied to outputs).
// APPEND: this step's token is read from k_new / v_new (bf16; paged only).
// With KV8 it enters the attention as the codes the cache will hold.
template <bool PAGED, bool KV8, bool APPEND = false>
__global__ __launch_bounds__(kWaves * kWave, 3) void decode_sk_kernel(
    DecodeArgs a) {
  constexpr int ES = KV8 ? 1 : 2;  // bytes per K/V value
  constexpr int KL = KV8 ? 2 : 4;  // 16-byte K loads per token row per tile
  __shared__ int s_cs[kMaxSeqs + 1];
  __shared__ int s_part[kWaves];
  __shared__ int s_clamped;
  __shared__ u32x4 s_newrow[2 * kD * 2 / 16];  // this step's K and V rows
  __shared__ float sm_o[kWaves][kHeadBlk][kD];
  __shared__ float sm_ml[kWaves][kHeadBlk][2];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int lane = tid & 63;
  const int r16 = lane & 15;
  const int grp = lane >> 4;
  // KV heads vary fastest across consecutive workgroups, so the workgroups
  // of one chunk run together.
  const int hblk = blockIdx.x % a.head_blocks;
  const int g = blockIdx.x / a.head_blocks;
  const int chunk = blockIdx.y;
  const int S = a.num_seqs;

  // --- tile offsets of the sequences (exclusive scan of the tile counts) ---
  // Thread tid owns sequences [lo, hi): their tile counts go to s_cs, then
  // the 256 per-thread sums are scanned (shuffles inside each wave, the
  // four wave totals through LDS) and s_cs is turned into offsets in place.
  {
    if (tid == 0) s_clamped = 0;
    const int per = (S + kWaves * kWave - 1) / (kWaves * kWave);
    const int lo = tid * per;
    const int hi = min(S, lo + per);
    int sum = 0, clamped = 0;
    for (int i = lo; i < hi; ++i) {
      const int raw = with_new<APPEND>(a, a.ctx[i]);
      const int L = clamp_len(a, raw, PAGED);
      clamped += L != raw;
      const int n = tiles_of(L - shared_of(a, i, L));
      s_cs[i] = n;
      sum += n;
    }
    int inc = sum;  // inclusive scan over the lanes of this wave
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int y = __shfl_up(inc, o);
      if (lane >= o) inc += y;
    }
    if (lane == kWave - 1) s_part[w] = inc;
    __syncthreads();
    if (clamped) atomicAdd(&s_clamped, clamped);
    int base = 0;  // tiles of the waves before this one
    for (int ww = 0; ww < w; ++ww) base += s_part[ww];
    int run = base + inc - sum;
    for (int i = lo; i < hi; ++i) {
      const int n = s_cs[i];
      s_cs[i] = run;
      run += n;
    }
    if (tid == kWaves * kWave - 1) s_cs[S] = base + inc;
    __syncthreads();
  }
  const int total = s_cs[S];
  if (blockIdx.x == 0 && chunk == 0) {
    for (int i = tid; i <= S; i += kWaves * kWave) a.ws_cs[i] = s_cs[i];
    if (tid == 0) record_clamped(a, s_clamped);
    // With append, the merge kernel stores the token: the block ids (pinned
    // host memory, possibly) and the fp8 reciprocals go to the workspace
    // now, long before it runs, so that it reads them from device memory.
    if constexpr (APPEND) {
      for (int i = tid; i < S; i += kWaves * kWave)
        a.ws_nb[i] = a.new_blocks[i];
      if constexpr (KV8) {
        for (int i = tid; i < 2 * a.hkv; i += kWaves * kWave)
          a.ws_inv[i] = i < a.hkv ? fp8_inv(a.k_scales, a.k_inv, i)
                                  : fp8_inv(a.v_scales, a.v_inv, i - a.hkv);
      }
    }
  }
  const int C = chunk_tiles(total, a.n_chunks);
  const int c0 = chunk * C;
  if (c0 >= total) return;
  const int c1 = min(total, c0 + C);

  // sequence holding tile c0: largest s with s_cs[s] <= c0
  int s = 0;
  {
    int lo = 0, hi = S - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_cs[mid] <= c0) lo = mid; else hi = mid - 1;
    }
    s = lo;
  }

  // fp8 K/V: per-head scales fold into this KV head's score scale and
  // output scale
  const float scale_log2 = a.k_scales ? a.scale_log2 * a.k_scales[g]
                                      : a.scale_log2;
  const float v_scale = a.v_scales ? a.v_scales[g] : a.v_scale;
  // fp8 with append: the reciprocals the token's codes are made with
  float k_inv = 0.f, v_inv = 0.f;
  if constexpr (KV8 && APPEND) {
    k_inv = fp8_inv(a.k_scales, a.k_inv, g);
    v_inv = fp8_inv(a.v_scales, a.v_inv, g);
  }
  const int h_in_group = hblk * kHeadBlk + r16;
  const bool h_valid = h_in_group < a.group;
  const int nh = min(kHeadBlk, a.group - hblk * kHeadBlk);
  const char* kbase = (const char*)a.k;
  const char* vbase = (const char*)a.v;

  for (int pos = c0; pos < c1; ++s) {
    const int seq_lo = s_cs[s];
    const int nt = s_cs[s + 1] - seq_lo;
    if (nt == 0) continue;
    // segment: tiles [lo_t, hi_t) of the sequence, tokens [lo, hi)
    const int lo_t = pos - seq_lo;
    const int hi_t = min(c1 - seq_lo, nt);
    pos = seq_lo + hi_t;
    const int stored = a.ctx[s];
    const int raw = with_new<APPEND>(a, stored);
    const int L = clamp_len(a, raw, PAGED);
    // this step's token (position `stored`) is read from k_new / v_new,
    // not from the cache
    const bool new_in = APPEND && raw != stored && L == raw;
    const int L_cache = new_in ? L - 1 : L;
    const int P = shared_of(a, s, L);  // tokens before the own tiles
    const int lo = P + kTile * lo_t;
    const int hi = min(P + kTile * hi_t, L);
    const int hi_c = min(hi, L_cache);  // end of the cached tokens

    const int qh = g * a.group + (h_valid ? h_in_group : 0);
    // Q^T: B operand, head r16; d = 32 i + 8 grp + e (bf16 K) or
    // d = 32 grp + 8 i + e (fp8 K), matching the K operands
    bf16x8 qop[4];
    {
      const bf16* qp = (const bf16*)a.q + ((int64_t)s * a.hq + qh) * kD +
                       (KV8 ? 32 : 8) * grp;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x4 qraw = ld16(qp + (KV8 ? 8 : 32) * i);
        if (!h_valid) qraw = u32x4{0, 0, 0, 0};
        qop[i] = as_bf16x8(qraw);
      }
    }

    float m_run = -INFINITY;  // reference max (log2 domain) of head r16
    float l_part = 0.f;       // this lane's share of the denominator
    f32x4 o[8];               // O^T: o[m][r] = O[head r16][32 grp + 8 r + m]
#pragma unroll
    for (int m = 0; m < 8; ++m) o[m] = f32x4{0.f, 0.f, 0.f, 0.f};

    // This step's token is folded in by the last wave (the one with the
    // fewest of the segment's tiles) after its tiles; its K and V rows
    // (16 + 16 units of 16 bytes) are read now, one unit per lane, so that
    // they arrive while the tiles stream.
    const bool fold_new = APPEND && new_in && hi_t == nt && w == kWaves - 1;
    u32x4 new_unit = u32x4{0, 0, 0, 0};
    if (fold_new && lane < 2 * kD * 2 / 16) {
      const int64_t row = ((int64_t)s * a.hkv + g) * kD;
      const bf16* src = lane < kD * 2 / 16
                            ? (const bf16*)a.k_new + row + 8 * lane
                            : (const bf16*)a.v_new + row + 8 * (lane - 16);
      new_unit = ld16(src);
    }

    // tiles covering [lo, hi); wave w takes tiles w, w+4, ...
    const int t_al = lo;
    // tiles holding cached tokens (this step's token alone needs none)
    const int n_tiles = (max(hi_c - lo, 0) + kTile - 1) / kTile;
    // start of the last cached group (the first group when none is)
    const int last_grp_pos = max(hi_c - 1, 0) & ~15;
    const int64_t seq_row0 = ((int64_t)s * a.hkv + g) * a.seq_stride;

    for (int kb0 = 0; kb0 < n_tiles; kb0 += kWaves * (kGroupsPerLoad / 2)) {
      // head row of each 16-token group of this wave's next tiles
      int row_lane = 0;
      if (PAGED) {
        const int k = kb0 + w + kWaves * (lane >> 1);
        int gpos = t_al + kTile * k + 16 * (lane & 1);
        gpos = min(gpos, last_grp_pos);
        int b = a.bt[(int64_t)s * a.bt_stride + gpos / a.block_size];
        b = b < 0 ? 0 : (b >= a.num_blocks ? a.num_blocks - 1 : b);
        row_lane = (b * a.hkv + g) * a.block_size + gpos % a.block_size;
      }
      // Addresses: a wave-uniform pointer to the head row of the first
      // token of the 16-token group of half hf of this wave's j-th tile
      // (groups past the context are replaced by the last context group),
      // plus a 32-bit per-lane byte offset: row `off` of the group, in
      // 0..15 (clamped to the context's last row for the contiguous
      // layout), and the lane's 16-byte chunk.
      auto half_start = [&](int j, int hf) -> int {
        return min(t_al + kTile * (kb0 + w + kWaves * j) + 16 * hf,
                   last_grp_pos);
      };
      auto half_ptr = [&](const char* base, int j, int hf) -> const char* {
        int64_t row;
        if (PAGED)
          row = __builtin_amdgcn_readlane(row_lane, 2 * j + hf);
        else
          row = seq_row0 + half_start(j, hf);
        return base + row * (kD * ES);
      };
      auto lane_off = [&](int j, int hf, int off, int chunk) -> uint32_t {
        const int r = PAGED ? off : min(off, hi_c - 1 - half_start(j, hf));
        return (uint32_t)(r * (kD * ES) + 8 * ES * chunk);
      };
      // 8 consecutive K/V values of a row, as stored; to_bf16 widens them
      // once they are needed (after every load of the tile is issued)
      auto ld8v = [&](const char* p) __attribute__((always_inline)) {
        if constexpr (KV8)
          return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
        else
          return ld16_stream(p);
      };
      using Raw = decltype(ld8v(kbase));
      auto to_bf16 = [](Raw r) __attribute__((always_inline)) -> u32x4 {
        if constexpr (KV8)
          return fp8x8_to_bf16(r);
        else
          return r;
      };
      const int k_end = min(n_tiles, kb0 + kWaves * (kGroupsPerLoad / 2));
      // Raw K of a tile: kraw[hf][i] = 16 bytes of token r16 of half hf.
      //   bf16: i < 4, d = 32 i + 8 grp .. +7 (one MFMA operand each);
      //   fp8:  i < 2, d = 32 grp + 16 i .. +15 (two MFMA operands each).
      // Raw V: rows tau(grp, e) = 16 (e / 4) + 4 grp + e % 4, d-chunk r16.
      auto load_tile = [&](int j, u32x4 (&kraw)[2][KL], Raw (&vraw)[8])
          __attribute__((always_inline)) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const char* kp = half_ptr(kbase, j, hf);
          if constexpr (KV8) {
            const uint32_t ko = lane_off(j, hf, r16, 4 * grp);
#pragma unroll
            for (int i = 0; i < KL; ++i) kraw[hf][i] = ld16_stream(kp + ko + 16 * i);
          } else {
            const uint32_t ko = lane_off(j, hf, r16, grp);
#pragma unroll
            for (int i = 0; i < KL; ++i) kraw[hf][i] = ld16_stream(kp + ko + 64 * i);
          }
        }
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const char* vp = half_ptr(vbase, j, hf);
#pragma unroll
          for (int e = 4 * hf; e < 4 * hf + 4; ++e)
            vraw[e] = ld8v(vp + lane_off(j, hf, 4 * grp + (e & 3), r16));
        }
      };
      // K operand i (8 bf16) of half hf
      auto k_op = [&](const u32x4 (&kraw)[2][KL], int hf, int i)
          __attribute__((always_inline)) -> bf16x8 {
        if constexpr (KV8) {
          const u32x4 r = kraw[hf][i >> 1];
          return as_bf16x8(fp8x8_to_bf16(
              (i & 1) ? u32x2{r[2], r[3]} : u32x2{r[0], r[1]}));
        } else {
          return as_bf16x8(kraw[hf][i]);
        }
      };
      auto compute_tile = [&](int j, const u32x4 (&kraw)[2][KL],
                              const Raw (&vraw)[8])
          __attribute__((always_inline)) {
        const int t = t_al + kTile * (kb0 + w + kWaves * j);
        f32x4 sc[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          sc[hf] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int i = 0; i < 4; ++i)
            sc[hf] = mfma16(k_op(kraw, hf, i), qop[i], sc[hf]);
        }

        const bool full = t + kTile <= hi_c;
        float x[2][4];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float v = sc[hf][r] * scale_log2;
            const int p = t + 16 * hf + 4 * grp + r;
            x[hf][r] = (full || p < hi_c) ? v : -INFINITY;
          }
        float mx =
            fmaxf(fmaxf(fmaxf(x[0][0], x[0][1]), fmaxf(x[0][2], x[0][3])),
                  fmaxf(fmaxf(x[1][0], x[1][1]), fmaxf(x[1][2], x[1][3])));
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        // Lazy rescaling: the reference max moves only when a score exceeds
        // it by more than 2^8 (so p <= 256); the final division by the sum
        // makes the result independent of the reference.
        if (__any(mx > m_run + kRescaleLog2)) {
          const float m_new = fmaxf(m_run, mx);
          const float alpha = fast_exp2(m_run - m_new);
          m_run = m_new;
          l_part *= alpha;
#pragma unroll
          for (int m = 0; m < 8; ++m) o[m] *= alpha;
        }
        float p[2][4];
        float psum = 0.f;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            p[hf][r] = fast_exp2(x[hf][r] - m_run);
            psum += p[hf][r];
          }
        l_part += psum;

        // P^T: B operand of O^T += V^T P^T, k-slot e <-> token tau(grp, e)
        u32x4 pb;
        pb[0] = pack_bf16(p[0][0], p[0][1]);
        pb[1] = pack_bf16(p[0][2], p[0][3]);
        pb[2] = pack_bf16(p[1][0], p[1][1]);
        pb[3] = pack_bf16(p[1][2], p[1][3]);
        const bf16x8 pop = as_bf16x8(pb);
        u32x4 vr[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) vr[e] = to_bf16(vraw[e]);
        if (!full) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int pe = t + 16 * (e >> 2) + 4 * grp + (e & 3);
            if (pe >= hi_c) vr[e] = u32x4{0, 0, 0, 0};
          }
        }
        // V^T rows d = 8 r16 + m: element e of A_m is V[tau(grp, e)][8r16+m]
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          u32x4 am;
          const int wd = m >> 1;
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4)
            am[q4] = (m & 1) ? pick_hi(vr[2 * q4][wd], vr[2 * q4 + 1][wd])
                             : pick_lo(vr[2 * q4][wd], vr[2 * q4 + 1][wd]);
          o[m] = mfma16(as_bf16x8(am), pop, o[m]);
        }
      };
      // One tile at a time for both cache types (issuing two fp8 tiles'
      // loads before computing either measured 1.5-2.6% slower).
      for (int j = 0; kb0 + w + kWaves * j < k_end; ++j) {
        u32x4 kraw[2][KL];
        Raw vraw[8];
        load_tile(j, kraw, vraw);
        // All loads of the tile are issued before the first MFMA waits for
        // any of them (the scheduler would otherwise start on the K half and
        // issue the V loads late, halving the bytes in flight).
        __builtin_amdgcn_sched_barrier(0);
        compute_tile(j, kraw, vraw);
      }
    }

    // This step's token, at the sequence's end (one key): its rows go
    // through LDS into the lanes' layouts, then a dot product per head and
    // p V.
    if constexpr (APPEND) {
      if (fold_new) {
        if (lane < 2 * kD * 2 / 16) {
          if constexpr (KV8) {
            // the values the cache will hold: the unit's codes, widened
            // back to bf16 as the tiles widen theirs (scales stay folded
            // into scale_log2 and the output)
            const float inv = lane < kD * 2 / 16 ? k_inv : v_inv;
            new_unit = fp8x8_to_bf16(u32x2{fp8_pack4(new_unit[0], new_unit[1], inv),
                                           fp8_pack4(new_unit[2], new_unit[3], inv)});
          }
          s_newrow[lane] = new_unit;
        }
        // the same wave reads what it wrote
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
        float dot = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // K at d = 32 i + 8 grp + e (bf16 K) or 32 grp + 8 i + e (fp8
          // K), as in qop[i]
          const u32x4 kr = s_newrow[KV8 ? 4 * grp + i : 4 * i + grp];
          const u32x4 qr = as_u32x4(qop[i]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            dot = __builtin_fmaf(bf16_lo(qr[e]), bf16_lo(kr[e]), dot);
            dot = __builtin_fmaf(bf16_hi(qr[e]), bf16_hi(kr[e]), dot);
          }
        }
        dot += __shfl_xor(dot, 16);
        dot += __shfl_xor(dot, 32);
        const float x = dot * scale_log2;
        if (__any(x > m_run + kRescaleLog2)) {
          const float m_new = fmaxf(m_run, x);
          const float alpha = fast_exp2(m_run - m_new);
          m_run = m_new;
          l_part *= alpha;
#pragma unroll
          for (int m = 0; m < 8; ++m) o[m] *= alpha;
        }
        const float pn = fast_exp2(x - m_run);
        if (grp == 0) l_part += pn;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          // V at d = 32 grp + 8 r + m, as in o[m][r]: unit 16 + 4 grp + r
          const u32x4 vr = s_newrow[16 + 4 * grp + r];
#pragma unroll
          for (int m = 0; m < 8; ++m) {
            const uint32_t wv = vr[m >> 1];
            o[m][r] += pn * ((m & 1) ? bf16_hi(wv) : bf16_lo(wv));
          }
        }
      }
    }

    // --- merge the waves' states of this segment through LDS ---
    l_part += __shfl_xor(l_part, 16);
    l_part += __shfl_xor(l_part, 32);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float* dst = &sm_o[w][r16][32 * grp + 8 * r];
      *reinterpret_cast<f32x4*>(dst) =
          f32x4{o[0][r], o[1][r], o[2][r], o[3][r]};
      *reinterpret_cast<f32x4*>(dst + 4) =
          f32x4{o[4][r], o[5][r], o[6][r], o[7][r]};
    }
    if (grp == 0) {
      sm_ml[w][r16][0] = m_run;
      sm_ml[w][r16][1] = l_part;
    }
    __syncthreads();
    const bool whole = lo_t == 0 && hi_t == nt;
    // slot 0: a continuation (lo > 0); slot 1: first piece of a sequence
    // that continues in later chunks.
    const int slot = lo_t > 0 ? 0 : 1;
    for (int it = tid; it < kHeadBlk * (kD / 8); it += kWaves * kWave) {
      const int h = it / (kD / 8);
      const int c = it % (kD / 8);
      if (h >= nh) continue;
      float M = -INFINITY;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, sm_ml[ww][h][0]);
      float Ls = 0.f;
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (M != -INFINITY) {
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) {
          const float mw = sm_ml[ww][h][0];
          if (mw == -INFINITY) continue;
          const float cw = fast_exp2(mw - M);
          Ls += cw * sm_ml[ww][h][1];
          const f32x4 lo4 = *reinterpret_cast<const f32x4*>(&sm_o[ww][h][8 * c]);
          const f32x4 hi4 =
              *reinterpret_cast<const f32x4*>(&sm_o[ww][h][8 * c + 4]);
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            acc[jj] += cw * lo4[jj];
            acc[4 + jj] += cw * hi4[jj];
          }
        }
      }
      if constexpr (KV8) {
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) acc[jj] *= v_scale;
      }
      const int head = g * a.group + hblk * kHeadBlk + h;
      if (whole && P > 0) {
        // own part done; decode_combine_kernel adds the prefix partials
        const int64_t idx = (int64_t)s * a.hq + head;
        float* po = a.whole_o + idx * kD + 8 * c;
        *reinterpret_cast<f32x4*>(po) = f32x4{acc[0], acc[1], acc[2], acc[3]};
        *reinterpret_cast<f32x4*>(po + 4) =
            f32x4{acc[4], acc[5], acc[6], acc[7]};
        if (c == 0) {
          a.whole_ml[2 * idx] = M;
          a.whole_ml[2 * idx + 1] = Ls;
        }
      } else if (whole) {
        const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
        u32x4 ov;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          ov[jj] = pack_bf16(acc[2 * jj] * inv, acc[2 * jj + 1] * inv);
        st16((bf16*)a.out + ((int64_t)s * a.hq + head) * kD + 8 * c, ov);
      } else {
        const int64_t idx = ((int64_t)chunk * 2 + slot) * a.hq + head;
        float* po = a.ws_o + idx * kD + 8 * c;
        *reinterpret_cast<f32x4*>(po) = f32x4{acc[0], acc[1], acc[2], acc[3]};
        *reinterpret_cast<f32x4*>(po + 4) =
            f32x4{acc[4], acc[5], acc[6], acc[7]};
        if (c == 0) {
          a.ws_ml[2 * idx] = M;
          a.ws_ml[2 * idx + 1] = Ls;
        }
      }
    }
    __syncthreads();
  }
}

// Exact merge of the partials of a sequence that spans several chunks
// (and of its shared-prefix partials, if any):
// o = sum_i 2^(m_i - M) O_i / sum_i 2^(m_i - M) l_i with M = max_i m_i, for
// every query head. Grid (sequence, query head), one wave each: lane
// (j, c) = (lane / 16, lane % 16) folds pieces j, j+4, ... of d chunk c (8
// values) with a running max; the four lane groups are then merged by
// shuffles. Also writes zeros for empty contexts.
constexpr int kCombineThreads = kWave;

// This step's token of sequence s (decode with append), stored as
// kv_append_token (fp8 caches: kv_append_token_fp8) stores it: the K and V
// rows of every KV head into the
// slot of position context_lens[s], the table entry when new_blocks[s] >= 0,
// then the length + 1; nothing when the position lies outside the table or
// names no valid block. One wave per sequence (an extra column of the
// merge grid), after the attention: no other workgroup of the op reads
// these entries any more.
__device__ void append_token_of(const DecodeArgs& a, int s, int lane) {
  constexpr int kUnits = kD * 2 / 16;  // 16-byte units of a head row
  constexpr int kAhead = 4;            // units per lane read up front
  const int per_tensor = a.hkv * kUnits;
  const int stored = a.ctx_w[s];
  const int64_t cap = (int64_t)a.bt_stride * a.block_size;
  const bool ok_pos = stored >= 0 && stored < cap;
  const int idx = ok_pos ? stored / a.block_size : 0;
  int32_t* entry = a.bt_w + (int64_t)s * a.bt_stride + idx;
  // the block id (copied to the workspace by the stream-K kernel) and the
  // current entry, and the first rows, all in flight together
  const int nb = a.ws_nb[s];
  const int old = ok_pos ? *entry : -1;
  auto src_of = [&](int i) {
    const bool is_v = i >= per_tensor;
    const int r = is_v ? i - per_tensor : i;
    return (const u32x4*)(is_v ? a.v_new : a.k_new) + (int64_t)s * per_tensor +
           r;
  };
  // 1 / scale of unit i's head (fp8 caches), as kv_append_token_fp8 takes
  // it (computed by the stream-K kernel)
  auto inv_of = [&](int i) -> float {
    const bool is_v = i >= per_tensor;
    const int hh = (is_v ? i - per_tensor : i) / kUnits;
    return a.ws_inv[(is_v ? a.hkv : 0) + hh];
  };
  // unit i (8 values) into its row: as is, or (fp8 caches) as 8 codes made
  // with inv
  auto put = [&](int i, int blk, int off, u32x4 x, float inv) {
    const bool is_v = i >= per_tensor;
    const int r = is_v ? i - per_tensor : i;
    const int hh = r / kUnits;
    const int64_t at =
        (((int64_t)blk * a.hkv + hh) * a.block_size + off) * kUnits +
        (r - hh * kUnits);
    void* base = is_v ? a.v_cache_w : a.k_cache_w;
    if (a.kv8)
      ((u32x2*)base)[at] =
          u32x2{fp8_pack4(x[0], x[1], inv), fp8_pack4(x[2], x[3], inv)};
    else
      ((u32x4*)base)[at] = x;
  };
  u32x4 x[kAhead];
  float xinv[kAhead];
#pragma unroll
  for (int k = 0; k < kAhead; ++k) {
    const int i = lane + k * kWave;
    if (i < 2 * per_tensor) {
      x[k] = *src_of(i);
      xinv[k] = a.kv8 ? inv_of(i) : 0.f;
    }
  }
  const int blk = nb >= 0 ? nb : old;
  if (!(ok_pos && blk >= 0 && blk < a.num_blocks)) return;
  const int off = stored - idx * a.block_size;
#pragma unroll
  for (int k = 0; k < kAhead; ++k) {
    const int i = lane + k * kWave;
    if (i < 2 * per_tensor) put(i, blk, off, x[k], xinv[k]);
  }
  for (int i = lane + kAhead * kWave; i < 2 * per_tensor; i += kWave)
    put(i, blk, off, *src_of(i), a.kv8 ? inv_of(i) : 0.f);
  if (lane == 0) {
    if (nb >= 0) *entry = nb;
    a.ctx_w[s] = stored + 1;
  }
}

__global__ __launch_bounds__(kCombineThreads) void decode_combine_kernel(
    DecodeArgs a) {
  const int s = blockIdx.x;
  const int h = blockIdx.y;
  const int lane = threadIdx.x;
  if (h == a.hq) {  // the extra column of a decode with append
    append_token_of(a, s, lane);
    return;
  }
  const int c = lane & 15;
  const int j = lane >> 4;
  const int* cs = a.ws_cs;
  const int total = cs[a.num_seqs];
  const int seq_lo = cs[s], seq_hi = cs[s + 1];
  bf16* out = (bf16*)a.out + ((int64_t)s * a.hq + h) * kD;
  // the shared-prefix path is paged only
  const int P = a.plen ? shared_of(a, s, clamp_ctx(a, s, true)) : 0;
  const int n_pre = P > 0 ? a.n_psplit : 0;
  int n_own = 0, ca = 0;
  bool own_whole = false;  // own part in one chunk, left in whole_o
  if (seq_hi > seq_lo) {
    const int C = chunk_tiles(total, a.n_chunks);
    ca = seq_lo / C;
    const int cb = (seq_hi - 1) / C;
    if (ca == cb) {
      if (n_pre == 0) return;  // written whole by decode_sk_kernel
      own_whole = true;
      n_own = 1;
    } else {
      n_own = cb - ca + 1;
    }
  } else if (n_pre == 0) {
    if (j == 0) st16(out + 8 * c, u32x4{0, 0, 0, 0});
    return;
  }
  const int n = n_own + n_pre;
  float M = -INFINITY, L = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
  for (int i = j; i < n; i += 4) {
    const float* po;
    const float* pml;
    if (own_whole && i == 0) {
      const int64_t idx = (int64_t)s * a.hq + h;
      po = a.whole_o + idx * kD;
      pml = a.whole_ml + 2 * idx;
    } else if (i < n_own) {
      // own piece i: chunk ca + i; slot 1 (first piece) for i == 0, else 0
      const int64_t idx =
          ((int64_t)(ca + i) * 2 + (i == 0 ? 1 : 0)) * a.hq + h;
      po = a.ws_o + idx * kD;
      pml = a.ws_ml + 2 * idx;
    } else {
      const int64_t idx =
          ((int64_t)(i - n_own) * a.pre_stride + s) * a.hq + h;
      po = a.pre_o + idx * kD;
      pml = a.pre_ml + 2 * idx;
    }
    fold_piece(M, L, acc, pml[0], pml[1],
               *reinterpret_cast<const f32x4*>(po + 8 * c),
               *reinterpret_cast<const f32x4*>(po + 8 * c + 4));
  }
  // merge the four lane groups (lanes c, c + 16, c + 32, c + 48)
  float Mall = fmaxf(M, __shfl_xor(M, 16));
  Mall = fmaxf(Mall, __shfl_xor(Mall, 32));
  const float f = M == -INFINITY ? 0.f : fast_exp2(M - Mall);
  L *= f;
  L += __shfl_xor(L, 16);
  L += __shfl_xor(L, 32);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    acc[e] *= f;
    acc[e] += __shfl_xor(acc[e], 16);
    acc[e] += __shfl_xor(acc[e], 32);
  }
  if (j == 0) {
    const float inv = L > 0.f ? 1.f / L : 0.f;
    u32x4 ov;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      ov[e] = pack_bf16(acc[2 * e] * inv, acc[2 * e + 1] * inv);
    st16(out + 8 * c, ov);
  }
}

// ---------------------------------------------------------------------------
// Generic path: one workgroup of kGenWaves waves per (query head, sequence);
// lanes over head_dim (<= 256). The tokens are taken in groups of
// kGenTokens, group j by wave j % kGenWaves, each wave with its own online
// softmax; the waves' (max, sum, output) are then merged exactly through
// LDS. The loads of a group (table entries, then their K and V rows) are
// issued together, so a wave waits on memory once per group rather than
// twice per token; tokens past the context re-read the last one and are
// skipped.
// ---------------------------------------------------------------------------
constexpr int kGenTokens = 8;
constexpr int kGenWaves = 8;

template <typename T, bool PAGED>
__global__ __launch_bounds__(kGenWaves * kWave) void decode_generic_kernel(
    DecodeArgs a) {
  __shared__ float sm_acc[kGenWaves][4][kWave];
  __shared__ float sm_ml[kGenWaves][2];
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int g = h / a.group;
  const int D = a.head_dim;
  const int ctx = clamp_ctx(a, s, PAGED);
  float qv[4], acc[4];
  const T* qp = (const T*)a.q + ((int64_t)s * a.hq + h) * D;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int d = lane + kWave * i;
    qv[i] = d < D ? to_f32<T>(qp[d]) : 0.f;
    acc[i] = 0.f;
  }
  float m_run = -INFINITY, l = 0.f;
  for (int p0 = kGenTokens * w; p0 < ctx; p0 += kGenTokens * kGenWaves) {
    float kk[kGenTokens][4], vv[kGenTokens][4];
#pragma unroll
    for (int t = 0; t < kGenTokens; ++t) {
      const int p = min(p0 + t, ctx - 1);
      int64_t row;  // head row of (token p, KV head g)
      if (PAGED) {
        int b = a.bt[(int64_t)s * a.bt_stride + p / a.block_size];
        b = b < 0 ? 0 : (b >= a.num_blocks ? a.num_blocks - 1 : b);
        row = ((int64_t)b * a.hkv + g) * a.block_size + p % a.block_size;
      } else {
        row = ((int64_t)s * a.hkv + g) * a.seq_stride + p;
      }
      const T* kp = (const T*)a.k + row * D;
      const T* vp = (const T*)a.v + row * D;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = lane + kWave * i;
        kk[t][i] = d < D ? to_f32<T>(kp[d]) : 0.f;
        vv[t][i] = d < D ? to_f32<T>(vp[d]) : 0.f;
      }
    }
    float x[kGenTokens];
#pragma unroll
    for (int t = 0; t < kGenTokens; ++t) {
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) dot += qv[i] * kk[t][i];
      x[t] = wave_sum(dot) * a.scale_log2;
    }
#pragma unroll
    for (int t = 0; t < kGenTokens; ++t) {
      if (p0 + t >= ctx) break;  // wave-uniform
      const float m_new = fmaxf(m_run, x[t]);
      const float alpha = fast_exp2(m_run - m_new);
      const float pr = fast_exp2(x[t] - m_new);
      l = l * alpha + pr;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = acc[i] * alpha + pr * vv[t][i];
      m_run = m_new;
    }
  }
  // exact merge of the waves: o = sum_w 2^(m_w - M) acc_w / sum_w 2^(m_w - M) l_w
  if (lane == 0) {
    sm_ml[w][0] = m_run;
    sm_ml[w][1] = l;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) sm_acc[w][i][lane] = acc[i];
  __syncthreads();
  if (w != 0) return;
  float M = -INFINITY;
#pragma unroll
  for (int ww = 0; ww < kGenWaves; ++ww) M = fmaxf(M, sm_ml[ww][0]);
  float L = 0.f, o[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ww = 0; ww < kGenWaves; ++ww) {
    const float mw = sm_ml[ww][0];
    const float f = mw == -INFINITY ? 0.f : fast_exp2(mw - M);
    L += f * sm_ml[ww][1];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] += f * sm_acc[ww][i][lane];
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  T* op = (T*)a.out + ((int64_t)s * a.hq + h) * D;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int d = lane + kWave * i;
    if (d < D) op[d] = from_f32<T>(o[i] * inv);
  }
  // wave 0 of the first workgroup counts the clamped contexts
  if (blockIdx.x == 0 && blockIdx.y == 0 && a.ws_hdr) {
    int n = 0;
    for (int i = lane; i < a.num_seqs; i += kWave) {
      const int raw = a.ctx[i];
      n += clamp_len(a, raw, PAGED) != raw;
    }
#pragma unroll
    for (int o2 = 32; o2 > 0; o2 >>= 1) n += __shfl_xor(n, o2);
    if (lane == 0) record_clamped(a, n);
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
            hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

int env_chunks_override() {
  static int cached = -2;
  if (cached == -2) {
    const char* e = getenv("KVPAGED_DECODE_CHUNKS");
    cached = e ? atoi(e) : 0;
  }
  return cached;
}

// Chunks per (KV head, head block): enough workgroups for one resident
// round (3 workgroups of 4 waves per CU), split evenly over the units.
int choose_chunks(int num_kv_heads, int head_blocks) {
  const int ov = env_chunks_override();
  if (ov > 0) return ov;
  const int units = num_kv_heads * head_blocks;
  const int target = device_cus() * 3;
  const int n = (target + units - 1) / units;
  return n < 1 ? 1 : n;
}

// Workspace: a 256-byte header (int32 [0] = sequences whose context was
// clamped in the last call), then the stream-K partials and tile offsets,
// and for a decode with append the step's block ids and fp8 reciprocals.
constexpr size_t kWsHeader = 256;

// [header][o][ml][cs: S + 1][nb: S][inv: 2 Hkv]
size_t sk_workspace_bytes(int num_seqs, int hq, int hkv, int n_chunks) {
  const size_t o = (size_t)n_chunks * 2 * hq * kD * sizeof(float);
  const size_t ml = (size_t)n_chunks * 2 * hq * 2 * sizeof(float);
  const size_t cs = (size_t)(num_seqs + 1) * sizeof(int32_t);
  const size_t nb = (size_t)num_seqs * sizeof(int32_t);
  const size_t inv = (size_t)2 * hkv * sizeof(float);
  return kWsHeader + o + ml + cs + nb + inv;
}

bool fast_path_ok(kv_dtype dtype, int head_dim, int block_size, bool paged) {
  return dtype == KV_BF16 && head_dim == kD &&
         (!paged || block_size % 16 == 0);
}

// kv8: K/V cache in fp8 E4M3 (q and out stay bf16, dtype must be KV_BF16);
// only the fast path reads it.
kv_status run_decode(const char* name, bool paged, DecodeArgs a,
                     kv_dtype dtype, void* workspace, size_t ws_bytes,
                     hipStream_t st, bool kv8 = false) {
  if (dtype != KV_F32 && dtype != KV_BF16)
    return kvp_fail(KV_EINVAL, "%s: unknown dtype %d", name, (int)dtype);
  if (!(a.scale_log2 > 0.f) || !(a.scale_log2 < INFINITY))
    return kvp_fail(KV_EINVAL, "%s: scale must be finite and > 0", name);
  if (a.num_seqs < 0 || a.hq <= 0 || a.hkv <= 0 || a.hq % a.hkv != 0 ||
      a.head_dim <= 0 || a.max_ctx < 0)
    return kvp_fail(KV_EINVAL,
                    "%s: bad shape (S=%d Hq=%d Hkv=%d D=%d max_context=%d)",
                    name, a.num_seqs, a.hq, a.hkv, a.head_dim, a.max_ctx);
  if (paged && (a.block_size <= 0 || a.bt_stride <= 0 || a.num_blocks <= 0))
    return kvp_fail(KV_EINVAL, "%s: bad paging arguments (B=%d stride=%d N=%d)",
                    name, a.block_size, a.bt_stride, a.num_blocks);
  if (paged && (int64_t)a.num_blocks * a.block_size * a.hkv > INT32_MAX)
    return kvp_fail(KV_EUNSUPPORTED, "%s: pool of more than 2^31 head rows",
                    name);
  if (!paged && a.seq_stride <= 0)
    return kvp_fail(KV_EINVAL, "%s: seq_stride must be > 0", name);
  if (a.num_seqs == 0) return KV_OK;
  if (!a.out || !a.q || !a.k || !a.v || !a.ctx || (paged && !a.bt))
    return kvp_fail(KV_EINVAL, "%s: NULL pointer", name);
  a.group = a.hq / a.hkv;
  a.kv8 = kv8;

  const bool fast = fast_path_ok(dtype, a.head_dim, a.block_size, paged);
  if (kv8 && !fast)
    return kvp_fail(KV_EUNSUPPORTED,
                    "%s: fp8 K/V needs head_dim %d and block_size a multiple "
                    "of 16 (got D=%d B=%d)", name, kD, a.head_dim,
                    a.block_size);
  if (fast) {
    a.head_blocks = (a.group + kHeadBlk - 1) / kHeadBlk;
    a.n_chunks = choose_chunks(a.hkv, a.head_blocks);
    const int per_launch = a.num_seqs < kMaxSeqs ? a.num_seqs : kMaxSeqs;
    if ((int64_t)per_launch * a.max_ctx > INT32_MAX)
      return kvp_fail(KV_EUNSUPPORTED, "%s: more than 2^31 context tokens in "
                      "one launch", name);
    const size_t need =
        sk_workspace_bytes(per_launch, a.hq, a.hkv, a.n_chunks);
    if (!workspace || ws_bytes < need)
      return kvp_fail(KV_EINVAL, "%s: workspace of %zu bytes needed, %zu given",
                      name, need, ws_bytes);
    a.ws_hdr = (int32_t*)workspace;
    a.ws_o = (float*)((char*)workspace + kWsHeader);
    a.ws_ml = a.ws_o + (size_t)a.n_chunks * 2 * a.hq * kD;
    a.ws_cs = (int32_t*)(a.ws_ml + (size_t)a.n_chunks * 2 * a.hq * 2);
    a.ws_nb = a.ws_cs + per_launch + 1;
    a.ws_inv = (float*)(a.ws_nb + per_launch);
    // Batches of more than kMaxSeqs sequences run as several launches on
    // the same stream, in order, sharing the workspace.
    for (int s0 = 0; s0 < a.num_seqs; s0 += kMaxSeqs) {
      DecodeArgs b = a;
      b.num_seqs = min(kMaxSeqs, a.num_seqs - s0);
      b.clamp_add = s0 > 0;
      b.out = (bf16*)a.out + (size_t)s0 * a.hq * kD;
      b.q = (const bf16*)a.q + (size_t)s0 * a.hq * kD;
      b.ctx = a.ctx + s0;
      if (a.k_new) {
        b.k_new = (const bf16*)a.k_new + (size_t)s0 * a.hkv * kD;
        b.v_new = (const bf16*)a.v_new + (size_t)s0 * a.hkv * kD;
        b.new_blocks = a.new_blocks + s0;
        b.bt_w = a.bt_w + (size_t)s0 * a.bt_stride;
        b.ctx_w = a.ctx_w + s0;
      }
      if (a.plen) {
        b.plen = a.plen + s0;
        b.pre_o = a.pre_o + (size_t)s0 * a.hq * kD;
        b.pre_ml = a.pre_ml + (size_t)s0 * a.hq * 2;
        b.whole_o = a.whole_o + (size_t)s0 * a.hq * kD;
        b.whole_ml = a.whole_ml + (size_t)s0 * a.hq * 2;
      }
      if (paged) {
        b.bt = a.bt + (size_t)s0 * a.bt_stride;
      } else {
        const size_t seq_bytes =
            (size_t)a.hkv * a.seq_stride * kD * (kv8 ? 1 : sizeof(bf16));
        b.k = (const char*)a.k + (size_t)s0 * seq_bytes;
        b.v = (const char*)a.v + (size_t)s0 * seq_bytes;
      }
      dim3 grid(a.hkv * a.head_blocks, a.n_chunks);
      if (paged && kv8 && a.k_new)
        decode_sk_kernel<true, true, true><<<grid, kWaves * kWave, 0, st>>>(
            b);
      else if (paged && kv8)
        decode_sk_kernel<true, true><<<grid, kWaves * kWave, 0, st>>>(b);
      else if (paged && a.k_new)
        decode_sk_kernel<true, false, true><<<grid, kWaves * kWave, 0, st>>>(
            b);
      else if (paged)
        decode_sk_kernel<true, false><<<grid, kWaves * kWave, 0, st>>>(b);
      else if (kv8)
        decode_sk_kernel<false, true><<<grid, kWaves * kWave, 0, st>>>(b);
      else
        decode_sk_kernel<false, false><<<grid, kWaves * kWave, 0, st>>>(b);
      KVP_LAUNCH_CHECK(name);
      // (with append, one more column per sequence stores its token)
      dim3 g2(b.num_seqs, a.hq + (a.k_new ? 1 : 0));
      decode_combine_kernel<<<g2, kCombineThreads, 0, st>>>(b);
      KVP_LAUNCH_CHECK(name);
    }
    return KV_OK;
  }
  if (a.head_dim > 4 * kWave)
    return kvp_fail(KV_EUNSUPPORTED, "%s: head_dim %d > 256", name,
                    a.head_dim);
  if (!workspace || ws_bytes < kWsHeader)
    return kvp_fail(KV_EINVAL, "%s: workspace of %zu bytes needed, %zu given",
                    name, kWsHeader, ws_bytes);
  a.ws_hdr = (int32_t*)workspace;
  dim3 grid(a.hq, a.num_seqs);
  if (dtype == KV_F32) {
    if (paged)
      decode_generic_kernel<float, true><<<grid, kGenWaves * kWave, 0, st>>>(a);
    else
      decode_generic_kernel<float, false><<<grid, kGenWaves * kWave, 0, st>>>(a);
  } else {
    if (paged)
      decode_generic_kernel<bf16, true><<<grid, kGenWaves * kWave, 0, st>>>(a);
    else
      decode_generic_kernel<bf16, false><<<grid, kGenWaves * kWave, 0, st>>>(a);
  }
  KVP_LAUNCH_CHECK(name);
  return KV_OK;
}

// Shared-prefix pieces: enough MFMA workgroups for one per CU (a prefill
// workgroup of 8 waves fills a CU), at least 256 keys per piece, pieces a
// multiple of 64 keys. More pieces make shorter workgroups, whose pipeline
// fill then dominates (2, 4 and 16 pieces measured slower than 8 for 256
// members of 32 / 8 heads).
int env_psplit_override() {
  static int cached = -2;
  if (cached == -2) {
    const char* e = getenv("KVPAGED_PREFIX_SPLITS");
    cached = e ? atoi(e) : 0;
  }
  return cached;
}

void choose_psplit(int num_seqs, int hq, int hkv, int max_shared,
                   int* nsplit, int* ksplit) {
  const int ms = max_shared < 16 ? 16 : max_shared;
  const int rowblocks = (num_seqs + 63) / 64;  // 64 query rows each
  // prefix-pass workgroups per piece: row blocks x head blocks of 4 within
  // each KV head's group
  const int per_split = rowblocks * hkv * ((hq / hkv + 3) / 4);
  int n = (device_cus() + per_split - 1) / per_split;
  if (env_psplit_override() > 0) n = env_psplit_override();
  const int max_n = (ms + 255) / 256;
  n = n < 1 ? 1 : (n > max_n ? max_n : n);
  const int ks = (((ms + n - 1) / n) + 63) & ~63;
  *ksplit = ks;
  *nsplit = (ms + ks - 1) / ks;
}

bool shared_fast_ok(kv_dtype dtype, int hq, int hkv, int head_dim,
                    int block_size) {
  return dtype == KV_BF16 && head_dim == kD && block_size % 16 == 0 &&
         hkv > 0 && hq % hkv == 0;
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// [plen: S int32][pre_o: nsplit pieces][whole_o][pre_ml][whole_ml]
size_t shared_extra_bytes(int num_seqs, int hq, int nsplit) {
  return align256((size_t)num_seqs * sizeof(int32_t)) +
         (size_t)(nsplit + 1) * num_seqs * hq * (kD + 2) * sizeof(float);
}

}  // namespace

extern "C" size_t kv_decode_shared_prefix_workspace_bytes(
    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t max_context, int32_t max_shared_len) {
  const size_t base = kv_decode_workspace_bytes(num_seqs, num_q_heads,
                                                num_kv_heads, head_dim,
                                                max_context);
  if (num_seqs <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads ||
      !shared_fast_ok(KV_BF16, num_q_heads, num_kv_heads, head_dim, 16))
    return base;
  int nsplit, ksplit;
  choose_psplit(num_seqs, num_q_heads, num_kv_heads, max_shared_len, &nsplit,
                &ksplit);
  return align256(base) + shared_extra_bytes(num_seqs, num_q_heads, nsplit);
}

extern "C" kv_status paged_attn_decode_shared_prefix(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    int32_t num_blocks, const int32_t* block_tables, int32_t bt_stride,
    const int32_t* context_lens, int32_t max_context, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, const int32_t* group_starts,
    const int32_t* shared_lens, int32_t num_groups, int32_t max_group_size,
    int32_t max_shared_len, float scale, kv_dtype dtype, void* workspace,
    size_t workspace_bytes, void* stream) {
  const char* name = "paged_attn_decode_shared_prefix";
  DecodeArgs a = {};
  a.out = out;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.bt = block_tables;
  a.bt_stride = bt_stride;
  a.num_blocks = num_blocks;
  a.block_size = block_size;
  a.ctx = context_lens;
  a.max_ctx = max_context;
  a.num_seqs = num_seqs;
  a.hq = num_q_heads;
  a.hkv = num_kv_heads;
  a.head_dim = head_dim;
  a.scale_log2 = scale * kLog2e;
  hipStream_t st = (hipStream_t)stream;
  if (num_groups < 0 || max_group_size < 0 || max_shared_len < 0 ||
      max_context < 0 || num_seqs < 0)
    return kvp_fail(KV_EINVAL, "%s: negative size argument", name);
  if (num_seqs > 0 && (num_groups < 1 || num_groups > num_seqs ||
                       max_group_size < 1 || max_group_size > num_seqs))
    return kvp_fail(KV_EINVAL,
                    "%s: need 1 <= num_groups <= num_seqs and 1 <= "
                    "max_group_size <= num_seqs", name);
  // Shapes without the MFMA prefix pass, or no shared tokens: the plain
  // decode computes the same attention.
  if (num_seqs <= 0 || max_shared_len < 16 ||
      !shared_fast_ok(dtype, num_q_heads, num_kv_heads, head_dim,
                      block_size) ||
      num_seqs > kMaxSeqs)
    return run_decode(name, true, a, dtype, workspace, workspace_bytes, st);
  if (!group_starts || !shared_lens || !workspace)
    return kvp_fail(KV_EINVAL, "%s: NULL pointer", name);
  const size_t need = kv_decode_shared_prefix_workspace_bytes(
      num_seqs, num_q_heads, num_kv_heads, head_dim, max_context,
      max_shared_len);
  if (workspace_bytes < need)
    return kvp_fail(KV_EINVAL, "%s: workspace of %zu bytes needed, %zu given",
                    name, need, workspace_bytes);
  int nsplit, ksplit;
  choose_psplit(num_seqs, num_q_heads, num_kv_heads, max_shared_len, &nsplit,
                &ksplit);
  const size_t base = align256(kv_decode_workspace_bytes(
      num_seqs, num_q_heads, num_kv_heads, head_dim, max_context));
  char* wp = (char*)workspace + base;
  int32_t* plen = (int32_t*)wp;
  // outputs first (rows of kD floats stay 16-byte aligned), then the
  // (max, sum) pairs
  float* pre_o = (float*)(wp + align256((size_t)num_seqs * sizeof(int32_t)));
  float* whole_o = pre_o + (size_t)nsplit * num_seqs * num_q_heads * kD;
  float* pre_ml = whole_o + (size_t)num_seqs * num_q_heads * kD;
  float* whole_ml = pre_ml + (size_t)nsplit * num_seqs * num_q_heads * 2;
  if (block_size <= 0 || bt_stride <= 0 || num_blocks <= 0 || !block_tables ||
      !context_lens || !q || !k_cache || !v_cache || !out)
    return kvp_fail(KV_EINVAL, "%s: bad paging arguments or NULL pointer",
                    name);
  if ((int64_t)num_blocks * block_size * num_kv_heads > INT32_MAX)
    return kvp_fail(KV_EUNSUPPORTED, "%s: pool of more than 2^31 head rows",
                    name);
  if (!(a.scale_log2 > 0.f) || !(a.scale_log2 < INFINITY))
    return kvp_fail(KV_EINVAL, "%s: scale must be finite and > 0", name);
  KvpPrefixJob job = {};
  job.q = q;
  job.k = k_cache;
  job.v = v_cache;
  job.bt = block_tables;
  job.bt_stride = bt_stride;
  job.num_blocks = num_blocks;
  job.block_size = block_size;
  job.ctx = context_lens;
  job.members = num_seqs;
  job.hq = num_q_heads;
  job.hkv = num_kv_heads;
  job.group_starts = group_starts;
  job.shared_lens = shared_lens;
  job.num_groups = num_groups;
  job.max_group_size = max_group_size;
  job.nsplit = nsplit;
  job.ksplit = ksplit;
  job.scale_log2 = a.scale_log2;
  job.plen = plen;
  job.po = pre_o;
  job.pml = pre_ml;
  kv_status r = kvp_prefix_partials(job, st);
  if (r != KV_OK) return r;
  a.plen = plen;
  a.pre_o = pre_o;
  a.pre_ml = pre_ml;
  a.n_psplit = nsplit;
  a.pre_stride = num_seqs;
  a.whole_o = whole_o;
  a.whole_ml = whole_ml;
  return run_decode(name, true, a, dtype, workspace, workspace_bytes, st);
}

extern "C" int32_t kv_decode_chunks(int32_t num_q_heads, int32_t num_kv_heads) {
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads)
    return KV_EINVAL;
  const int hb = (num_q_heads / num_kv_heads + kHeadBlk - 1) / kHeadBlk;
  return choose_chunks(num_kv_heads, hb);
}

extern "C" size_t kv_decode_workspace_bytes(int32_t num_seqs,
                                            int32_t num_q_heads,
                                            int32_t num_kv_heads,
                                            int32_t head_dim,
                                            int32_t max_context) {
  (void)max_context;
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      num_q_heads % num_kv_heads || head_dim <= 0)
    return 0;
  if (head_dim != kD) return kWsHeader;  // generic path: the header only
  const int hb = (num_q_heads / num_kv_heads + kHeadBlk - 1) / kHeadBlk;
  const int n = choose_chunks(num_kv_heads, hb);
  const int per_launch = num_seqs < kMaxSeqs ? num_seqs : kMaxSeqs;
  return sk_workspace_bytes(per_launch, num_q_heads, num_kv_heads, n);
}

extern "C" kv_status paged_attn_decode(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    int32_t num_blocks, const int32_t* block_tables, int32_t bt_stride,
    const int32_t* context_lens, int32_t max_context, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, float scale, kv_dtype dtype, void* workspace,
    size_t workspace_bytes, void* stream) {
  DecodeArgs a = {};
  a.out = out;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.bt = block_tables;
  a.bt_stride = bt_stride;
  a.num_blocks = num_blocks;
  a.block_size = block_size;
  a.ctx = context_lens;
  a.max_ctx = max_context;
  a.num_seqs = num_seqs;
  a.hq = num_q_heads;
  a.hkv = num_kv_heads;
  a.head_dim = head_dim;
  a.scale_log2 = scale * kLog2e;
  return run_decode("paged_attn_decode", true, a, dtype, workspace,
                    workspace_bytes, (hipStream_t)stream);
}

extern "C" kv_status paged_attn_decode_append(
    void* out, const void* q, const void* k_new, const void* v_new,
    const int32_t* new_blocks, void* k_cache, void* v_cache,
    int32_t num_blocks, int32_t* block_tables, int32_t bt_stride,
    int32_t* context_lens, int32_t max_context, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, float scale, kv_dtype dtype, void* workspace,
    size_t workspace_bytes, void* stream) {
  const char* name = "paged_attn_decode_append";
  if (num_seqs < 0)
    return kvp_fail(KV_EINVAL, "%s: num_seqs must be >= 0", name);
  if (num_seqs == 0) return KV_OK;
  const bool aligned = (((uintptr_t)k_new | (uintptr_t)v_new) & 15) == 0;
  if (!fast_path_ok(dtype, head_dim, block_size, true) || !aligned) {
    // shapes the stream-K kernel does not cover (or rows not 16-byte
    // aligned): the two calls it fuses
    const kv_status st = kv_append_token(
        k_new, v_new, new_blocks, block_tables, bt_stride, context_lens,
        num_seqs, k_cache, v_cache, num_blocks, block_size, num_kv_heads,
        head_dim, dtype, stream);
    if (st != KV_OK) return st;
    return paged_attn_decode(out, q, k_cache, v_cache, num_blocks,
                             block_tables, bt_stride, context_lens,
                             max_context, num_seqs, num_q_heads, num_kv_heads,
                             head_dim, block_size, scale, dtype, workspace,
                             workspace_bytes, stream);
  }
  if (!k_new || !v_new || !new_blocks)
    return kvp_fail(KV_EINVAL, "%s: NULL pointer", name);
  const int32_t* nb = (const int32_t*)kvp_device_view(new_blocks);
  if (!nb)
    return kvp_fail(KV_EINVAL, "%s: new_blocks is not device or pinned host "
                    "memory", name);
  DecodeArgs a = {};
  a.out = out;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.bt = block_tables;
  a.bt_stride = bt_stride;
  a.num_blocks = num_blocks;
  a.block_size = block_size;
  a.ctx = context_lens;
  a.max_ctx = max_context;
  a.num_seqs = num_seqs;
  a.hq = num_q_heads;
  a.hkv = num_kv_heads;
  a.head_dim = head_dim;
  a.scale_log2 = scale * kLog2e;
  a.k_new = k_new;
  a.v_new = v_new;
  a.new_blocks = nb;
  a.bt_w = block_tables;
  a.ctx_w = context_lens;
  a.k_cache_w = k_cache;
  a.v_cache_w = v_cache;
  return run_decode(name, true, a, dtype, workspace, workspace_bytes,
                    (hipStream_t)stream);
}

namespace {
// paged_attn_decode_append on fp8 E4M3 caches: per-tensor scales (k_scales
// NULL) or one per KV head.
kv_status decode_append_fp8(const char* name, void* out, const void* q,
                            const void* k_new, const void* v_new,
                            const int32_t* new_blocks, void* k_cache,
                            void* v_cache, int32_t num_blocks,
                            int32_t* block_tables, int32_t bt_stride,
                            int32_t* context_lens, int32_t max_context,
                            int32_t num_seqs, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim,
                            int32_t block_size, float scale, float k_scale,
                            float v_scale, const float* k_scales,
                            const float* v_scales, void* workspace,
                            size_t workspace_bytes, void* stream) {
  if (num_seqs < 0)
    return kvp_fail(KV_EINVAL, "%s: num_seqs must be >= 0", name);
  if (num_seqs == 0) return KV_OK;
  if (!k_scales && (!(k_scale > 0.f) || !(k_scale < INFINITY) ||
                    !(v_scale > 0.f) || !(v_scale < INFINITY)))
    return kvp_fail(KV_EINVAL, "%s: k_scale and v_scale must be finite and "
                    "> 0", name);
  if (!fast_path_ok(KV_BF16, head_dim, block_size, true))
    return kvp_fail(KV_EUNSUPPORTED,
                    "%s: fp8 K/V needs head_dim %d and block_size a multiple "
                    "of 16 (got D=%d B=%d)", name, kD, head_dim, block_size);
  if (!k_new || !v_new || !new_blocks || !k_cache || !v_cache)
    return kvp_fail(KV_EINVAL, "%s: NULL pointer", name);
  if (((uintptr_t)k_new | (uintptr_t)v_new) % 16 ||
      ((uintptr_t)k_cache | (uintptr_t)v_cache) % 8)
    return kvp_fail(KV_EINVAL, "%s: k_new/v_new must be 16-byte and the "
                    "caches 8-byte aligned", name);
  const int32_t* nb = (const int32_t*)kvp_device_view(new_blocks);
  if (!nb)
    return kvp_fail(KV_EINVAL, "%s: new_blocks is not device or pinned host "
                    "memory", name);
  DecodeArgs a = {};
  a.out = out;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.bt = block_tables;
  a.bt_stride = bt_stride;
  a.num_blocks = num_blocks;
  a.block_size = block_size;
  a.ctx = context_lens;
  a.max_ctx = max_context;
  a.num_seqs = num_seqs;
  a.hq = num_q_heads;
  a.hkv = num_kv_heads;
  a.head_dim = head_dim;
  // as the fp8 decode: per-tensor scales fold into the score scale and the
  // output, per-head ones are applied in the kernel
  a.scale_log2 = scale * (k_scales ? 1.f : k_scale) * kLog2e;
  a.v_scale = k_scales ? 1.f : v_scale;
  a.k_scales = k_scales;
  a.v_scales = v_scales;
  // the token's codes, as kv_append_token_fp8 computes them
  a.k_inv = k_scales ? 1.f : 1.f / k_scale;
  a.v_inv = k_scales ? 1.f : 1.f / v_scale;
  a.k_new = k_new;
  a.v_new = v_new;
  a.new_blocks = nb;
  a.bt_w = block_tables;
  a.ctx_w = context_lens;
  a.k_cache_w = k_cache;
  a.v_cache_w = v_cache;
  return run_decode(name, true, a, KV_BF16, workspace, workspace_bytes,
                    (hipStream_t)stream, true);
}
}  // namespace

extern "C" kv_status paged_attn_decode_append_fp8(
    void* out, const void* q, const void* k_new, const void* v_new,
    const int32_t* new_blocks, void* k_cache, void* v_cache,
    int32_t num_blocks, int32_t* block_tables, int32_t bt_stride,
    int32_t* context_lens, int32_t max_context, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, float scale, float k_scale, float v_scale,
    void* workspace, size_t workspace_bytes, void* stream) {
  return decode_append_fp8(
      "paged_attn_decode_append_fp8", out, q, k_new, v_new, new_blocks,
      k_cache, v_cache, num_blocks, block_tables, bt_stride, context_lens,
      max_context, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
      scale, k_scale, v_scale, nullptr, nullptr, workspace, workspace_bytes,
      stream);
}

extern "C" kv_status paged_attn_decode_append_fp8_per_head(
    void* out, const void* q, const void* k_new, const void* v_new,
    const int32_t* new_blocks, void* k_cache, void* v_cache,
    int32_t num_blocks, int32_t* block_tables, int32_t bt_stride,
    int32_t* context_lens, int32_t max_context, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, float scale, const float* k_scales,
    const float* v_scales, void* workspace, size_t workspace_bytes,
    void* stream) {
  const char* name = "paged_attn_decode_append_fp8_per_head";
  if (num_seqs > 0 && (!k_scales || !v_scales))
    return kvp_fail(KV_EINVAL, "%s: NULL scale array", name);
  return decode_append_fp8(name, out, q, k_new, v_new, new_blocks, k_cache,
                           v_cache, num_blocks, block_tables, bt_stride,
                           context_lens, max_context, num_seqs, num_q_heads,
                           num_kv_heads, head_dim, block_size, scale, 1.f, 1.f,
                           k_scales, v_scales, workspace, workspace_bytes,
                           stream);
}

extern "C" kv_status paged_attn_decode_fp8(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    int32_t num_blocks, const int32_t* block_tables, int32_t bt_stride,
    const int32_t* context_lens, int32_t max_context, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, float scale, float k_scale, float v_scale,
    void* workspace, size_t workspace_bytes, void* stream) {
  const char* name = "paged_attn_decode_fp8";
  if (!(k_scale > 0.f) || !(k_scale < INFINITY) || !(v_scale > 0.f) ||
      !(v_scale < INFINITY))
    return kvp_fail(KV_EINVAL, "%s: k_scale and v_scale must be finite and "
                    "> 0", name);
  DecodeArgs a = {};
  a.out = out;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.bt = block_tables;
  a.bt_stride = bt_stride;
  a.num_blocks = num_blocks;
  a.block_size = block_size;
  a.ctx = context_lens;
  a.max_ctx = max_context;
  a.num_seqs = num_seqs;
  a.hq = num_q_heads;
  a.hkv = num_kv_heads;
  a.head_dim = head_dim;
  a.scale_log2 = scale * k_scale * kLog2e;
  a.v_scale = v_scale;
  return run_decode(name, true, a, KV_BF16, workspace, workspace_bytes,
                    (hipStream_t)stream, true);
}

extern "C" kv_status contig_attn_decode_fp8(
    void* out, const void* q, const void* k, const void* v, int32_t seq_stride,
    const int32_t* context_lens, int32_t max_context, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, float scale,
    float k_scale, float v_scale, void* workspace, size_t workspace_bytes,
    void* stream) {
  const char* name = "contig_attn_decode_fp8";
  if (!(k_scale > 0.f) || !(k_scale < INFINITY) || !(v_scale > 0.f) ||
      !(v_scale < INFINITY))
    return kvp_fail(KV_EINVAL, "%s: k_scale and v_scale must be finite and "
                    "> 0", name);
  DecodeArgs a = {};
  a.out = out;
  a.q = q;
  a.k = k;
  a.v = v;
  a.seq_stride = seq_stride;
  a.block_size = 16;
  a.ctx = context_lens;
  a.max_ctx = max_context;
  a.num_seqs = num_seqs;
  a.hq = num_q_heads;
  a.hkv = num_kv_heads;
  a.head_dim = head_dim;
  a.scale_log2 = scale * k_scale * kLog2e;
  a.v_scale = v_scale;
  return run_decode(name, false, a, KV_BF16, workspace, workspace_bytes,
                    (hipStream_t)stream, true);
}

extern "C" kv_status contig_attn_decode(
    void* out, const void* q, const void* k, const void* v, int32_t seq_stride,
    const int32_t* context_lens, int32_t max_context, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, float scale,
    kv_dtype dtype, void* workspace, size_t workspace_bytes, void* stream) {
  DecodeArgs a = {};
  a.out = out;
  a.q = q;
  a.k = k;
  a.v = v;
  a.seq_stride = seq_stride;
  a.block_size = 16;
  a.ctx = context_lens;
  a.max_ctx = max_context;
  a.num_seqs = num_seqs;
  a.hq = num_q_heads;
  a.hkv = num_kv_heads;
  a.head_dim = head_dim;
  a.scale_log2 = scale * kLog2e;
  return run_decode("contig_attn_decode", false, a, dtype, workspace,
                    workspace_bytes, (hipStream_t)stream);
}

extern "C" kv_status paged_attn_decode_fp8_per_head(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    int32_t num_blocks, const int32_t* block_tables, int32_t bt_stride,
    const int32_t* context_lens, int32_t max_context, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, float scale, const float* k_scales,
    const float* v_scales, void* workspace, size_t workspace_bytes,
    void* stream) {
  const char* name = "paged_attn_decode_fp8_per_head";
  if (num_seqs > 0 && (!k_scales || !v_scales))
    return kvp_fail(KV_EINVAL, "%s: NULL scale array", name);
  DecodeArgs a = {};
  a.out = out;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.bt = block_tables;
  a.bt_stride = bt_stride;
  a.num_blocks = num_blocks;
  a.block_size = block_size;
  a.ctx = context_lens;
  a.max_ctx = max_context;
  a.num_seqs = num_seqs;
  a.hq = num_q_heads;
  a.hkv = num_kv_heads;
  a.head_dim = head_dim;
  a.scale_log2 = scale * kLog2e;
  a.v_scale = 1.f;
  a.k_scales = k_scales;
  a.v_scales = v_scales;
  return run_decode(name, true, a, KV_BF16, workspace, workspace_bytes,
                    (hipStream_t)stream, true);
}

extern "C" kv_status contig_attn_decode_fp8_per_head(
    void* out, const void* q, const void* k, const void* v, int32_t seq_stride,
    const int32_t* context_lens, int32_t max_context, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, float scale,
    const float* k_scales, const float* v_scales, void* workspace,
    size_t workspace_bytes, void* stream) {
  const char* name = "contig_attn_decode_fp8_per_head";
  if (num_seqs > 0 && (!k_scales || !v_scales))
    return kvp_fail(KV_EINVAL, "%s: NULL scale array", name);
  DecodeArgs a = {};
  a.out = out;
  a.q = q;
  a.k = k;
  a.v = v;
  a.seq_stride = seq_stride;
  a.block_size = 16;
  a.ctx = context_lens;
  a.max_ctx = max_context;
  a.num_seqs = num_seqs;
  a.hq = num_q_heads;
  a.hkv = num_kv_heads;
  a.head_dim = head_dim;
  a.scale_log2 = scale * kLog2e;
  a.v_scale = 1.f;
  a.k_scales = k_scales;
  a.v_scales = v_scales;
  return run_decode(name, false, a, KV_BF16, workspace, workspace_bytes,
                    (hipStream_t)stream, true);
}

extern "C" kv_status kv_decode_clamped_count(const void* workspace,
                                             void* stream, int32_t* count) {
  if (!workspace || !count)
    return kvp_fail(KV_EINVAL, "kv_decode_clamped_count: NULL pointer");
  hipStream_t st = (hipStream_t)stream;
  int32_t v = 0;
  if (hipMemcpyAsync(&v, workspace, sizeof(v), hipMemcpyDeviceToHost, st) !=
          hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return kvp_fail(KV_EHIP, "kv_decode_clamped_count: copy failed: %s",
                    hipGetErrorString(hipGetLastError()));
  *count = v;
  return KV_OK;
}
