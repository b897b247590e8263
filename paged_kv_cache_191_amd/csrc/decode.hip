// Decode attention over a paged or contiguous KV cache.
//
// One query per sequence attends to every token of its context, reading K
// and V through the sequence's block table ["PagedAttention Nedir?"
// (bitcanli.com), "PagedAttention Nasıl Çalışır?", step 4]. The vAttention
// newsletter ("İddia ve Gerçeklik") locates the cost of paging in this
// loop: a table read per block, extra branching, and registers holding page
// indices; the contiguous variant reads a plain [S, Lmax, Hkv, D] buffer.
// Both variants below share one kernel body; only the row addressing
// differs, so their timing difference is the table lookup.
//
// Fast path (bf16, head_dim 128, block_size % 16 == 0, any GQA group):
//   * A workgroup owns one (sequence, KV head, head block of <= 16 query
//     heads, partition of `part` tokens); its 4 waves split the partition.
//     All query heads of a KV head are packed into one MFMA so each K/V byte
//     is read once from HBM.
//   * Per 32-token tile a wave computes S^T = K Q^T with
//     v_mfma_f32_16x16x32_bf16 (tokens x heads), an online softmax in the
//     log2 domain, and O^T += V^T P^T with the same MFMA (d x heads).
//   * K is loaded straight into the MFMA A-operand layout (each lane 16 B
//     of one token row). V is loaded as whole 256-byte token rows (16 lanes
//     per row, fully coalesced) and transposed inside each lane's registers
//     with v_perm_b32: the k (token) order of the PV product is chosen to be
//     the order in which the S^T product leaves P in registers, so P never
//     moves between lanes.
//   * Block ids of the wave's range are fetched once (one lane per 16-token
//     group) and broadcast with v_readlane, so each half-tile's base address
//     is wave-uniform.
//   * Masked tokens (past the context or the wave's range) are selected out
//     (score -> -inf, V -> 0), never multiplied by 0, so NaN in unused slots
//     cannot leak.
//   * Partitions of one (sequence, head) are merged exactly by
//     decode_combine_kernel using (max, sum, unnormalised output).
// Generic path (fp32, or shapes the fast path does not cover): one wave per
// (sequence, query head), lanes over head_dim, tokens in order.

#include <stdlib.h>

#include "device_common.h"

namespace {

using namespace kvp;

constexpr int kD = 128;      // head_dim of the MFMA path
constexpr int kWaves = 4;    // waves per workgroup in the MFMA path
constexpr int kTile = 32;    // tokens per wave iteration
constexpr int kHeadBlk = 16; // query heads per MFMA column block
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
  float scale_log2;     // scale * log2(e)
  int32_t part;         // tokens per partition (multiple of kWaves * kTile)
  int32_t max_parts;    // partition slots per (seq, head) in the workspace
  float* ws_o;          // [S, Hq, max_parts, D] unnormalised partial outputs
  float* ws_ml;         // [S, Hq, max_parts, 2] (max, sum) per partial
};

__device__ __forceinline__ int clamp_ctx(const DecodeArgs& a, int s,
                                         bool paged) {
  int c = a.ctx[s];
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

// ---------------------------------------------------------------------------
// MFMA fast path
// ---------------------------------------------------------------------------
template <bool PAGED>
__global__ __launch_bounds__(kWaves * kWave) void decode_mfma_kernel(
    DecodeArgs a) {
  // KV heads vary fastest across consecutive workgroups, so the workgroups
  // of one partition run together and read whole token rows (all heads).
  const int hblk = blockIdx.x % a.head_blocks;
  const int g = blockIdx.x / a.head_blocks;
  const int part_idx = blockIdx.y;
  const int s = blockIdx.z;
  const int ctx = clamp_ctx(a, s, PAGED);
  const int nparts = ctx > 0 ? (ctx + a.part - 1) / a.part : 1;
  if (part_idx >= nparts) return;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int lane = tid & 63;
  const int r16 = lane & 15;
  const int grp = lane >> 4;

  const int t_begin = part_idx * a.part;
  const int t_end = min(ctx, t_begin + a.part);
  const int per_wave = a.part / kWaves;
  const int w0 = t_begin + w * per_wave;
  const int w1 = min(t_end, w0 + per_wave);

  const int h_in_group = hblk * kHeadBlk + r16;
  const bool h_valid = h_in_group < a.group;
  const int qh = g * a.group + (h_valid ? h_in_group : 0);

  // Q^T as the B operand of S^T = K Q^T: lane holds head r16, d = 32i+8grp+e.
  bf16x8 qop[4];
  {
    const bf16* qp = (const bf16*)a.q + ((int64_t)s * a.hq + qh) * kD + 8 * grp;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x4 raw = ld16(qp + 32 * i);
      if (!h_valid) raw = u32x4{0, 0, 0, 0};
      qop[i] = as_bf16x8(raw);
    }
  }

  float m_run = -INFINITY;  // running max (log2 domain) of head r16
  float l_part = 0.f;       // this lane's share of the softmax denominator
  f32x4 o[8];               // O^T: o[m][r] = O[head r16][32 grp + 8 r + m]
#pragma unroll
  for (int m = 0; m < 8; ++m) o[m] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Head rows of D elements: head g of token `off` in block b is row
  // (b * Hkv + g) * block_size + off (contiguous: (s * Hkv + g) * stride +
  // position), so one head's tokens of a block are contiguous.
  const bf16* kbase = (const bf16*)a.k;
  const bf16* vbase = (const bf16*)a.v;

  // Head row of the first token of every 16-token group of this wave's
  // range, one group per lane (the range holds at most 64 groups).
  // 16-token groups never straddle a block (block_size % 16 == 0 and w0 is
  // a multiple of 32), so a group's rows are row .. row + 15.
  int row_lane = 0;
  if (PAGED && w0 < w1) {
    const int ngroups = (w1 - w0 + 15) >> 4;
    if (lane < ngroups) {
      const int pos = w0 + 16 * lane;
      int b = a.bt[(int64_t)s * a.bt_stride + pos / a.block_size];
      b = b < 0 ? 0 : (b >= a.num_blocks ? a.num_blocks - 1 : b);
      row_lane = (b * a.hkv + g) * a.block_size + pos % a.block_size;
    }
  }
  // Last 16-token group that holds a valid token; groups past it re-read it
  // (in bounds) and are masked.
  const int last_grp = w1 > w0 ? ((w1 - 1 - w0) >> 4) : 0;
  const int64_t seq_row0 = ((int64_t)s * a.hkv + g) * a.seq_stride;

  // Row of the token `off` places after the start of group gi. Contiguous
  // rows are clamped to the last valid token so that a ragged tail never
  // reads past the sequence (masked afterwards).
  auto row_of = [&](int gi, int off) -> int64_t {
    gi = gi > last_grp ? last_grp : gi;
    if (PAGED) return (int64_t)__builtin_amdgcn_readlane(row_lane, gi) + off;
    const int pos = min(w0 + 16 * gi + off, w1 - 1);
    return seq_row0 + pos;
  };

  for (int t = w0; t < w1; t += kTile) {
    const int gi0 = (t - w0) >> 4;
    // K: A operand of S^T (token r16 of each half, d = 32 i + 8 grp + e).
    u32x4 kr[2][4];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const bf16* kp = kbase + row_of(gi0 + hf, r16) * kD + 8 * grp;
#pragma unroll
      for (int i = 0; i < 4; ++i) kr[hf][i] = ld16_stream(kp + 32 * i);
    }
    // V: token rows tau(grp, e) = 16 (e / 4) + 4 grp + e % 4, d-chunk r16.
    u32x4 vr[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bf16* vp =
          vbase + row_of(gi0 + (e >> 2), 4 * grp + (e & 3)) * kD + 8 * r16;
      vr[e] = ld16_stream(vp);
    }

    // S^T = K Q^T, two 16-token halves.
    f32x4 sc[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      sc[hf] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sc[hf] = mfma16(as_bf16x8(kr[hf][i]), qop[i], sc[hf]);
    }

    // Scores in the log2 domain; tokens past the wave's range -> -inf.
    const bool full = (t + kTile) <= w1;
    float x[2][4];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = sc[hf][r] * a.scale_log2;
        const int pos = t + 16 * hf + 4 * grp + r;
        x[hf][r] = (full || pos < w1) ? v : -INFINITY;
      }
    float mx = fmaxf(fmaxf(fmaxf(x[0][0], x[0][1]), fmaxf(x[0][2], x[0][3])),
                     fmaxf(fmaxf(x[1][0], x[1][1]), fmaxf(x[1][2], x[1][3])));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // Lazy rescaling: the reference max only moves when a score exceeds it
    // by more than 2^8, so p <= 256 and most tiles skip the O rescale. The
    // final division by l makes the result independent of the reference.
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

    // P^T as the B operand of O^T += V^T P^T: k-slot e <-> token tau(grp, e).
    u32x4 pb;
    pb[0] = pack_bf16(p[0][0], p[0][1]);
    pb[1] = pack_bf16(p[0][2], p[0][3]);
    pb[2] = pack_bf16(p[1][0], p[1][1]);
    pb[3] = pack_bf16(p[1][2], p[1][3]);
    const bf16x8 pop = as_bf16x8(pb);

    if (!full) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int pos = t + 16 * (e >> 2) + 4 * grp + (e & 3);
        if (pos >= w1) vr[e] = u32x4{0, 0, 0, 0};
      }
    }
    // V^T rows d = 8 r16 + m: element e of A_m is V[tau(grp, e)][8 r16 + m].
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      u32x4 am;
      const int wd = m >> 1;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        am[j] = (m & 1) ? pick_hi(vr[2 * j][wd], vr[2 * j + 1][wd])
                        : pick_lo(vr[2 * j][wd], vr[2 * j + 1][wd]);
      o[m] = mfma16(as_bf16x8(am), pop, o[m]);
    }
  }

  // Denominator of head r16: sum over the four lane groups.
  l_part += __shfl_xor(l_part, 16);
  l_part += __shfl_xor(l_part, 32);

  // Merge the waves' partial results through LDS.
  __shared__ float sm_o[kWaves][kHeadBlk][kD];
  __shared__ float sm_ml[kWaves][kHeadBlk][2];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float* dst = &sm_o[w][r16][32 * grp + 8 * r];
    *reinterpret_cast<f32x4*>(dst) = f32x4{o[0][r], o[1][r], o[2][r], o[3][r]};
    *reinterpret_cast<f32x4*>(dst + 4) =
        f32x4{o[4][r], o[5][r], o[6][r], o[7][r]};
  }
  if (grp == 0) {
    sm_ml[w][r16][0] = m_run;
    sm_ml[w][r16][1] = l_part;
  }
  __syncthreads();

  const int nh = min(kHeadBlk, a.group - hblk * kHeadBlk);
  for (int it = tid; it < kHeadBlk * (kD / 8); it += kWaves * kWave) {
    const int h = it / (kD / 8);
    const int c = it % (kD / 8);
    if (h >= nh) continue;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, sm_ml[ww][h][0]);
    float L = 0.f;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (M != -INFINITY) {
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) {
        const float mw = sm_ml[ww][h][0];
        if (mw == -INFINITY) continue;
        const float cw = fast_exp2(mw - M);
        L += cw * sm_ml[ww][h][1];
        const f32x4 lo = *reinterpret_cast<const f32x4*>(&sm_o[ww][h][8 * c]);
        const f32x4 hi =
            *reinterpret_cast<const f32x4*>(&sm_o[ww][h][8 * c + 4]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[j] += cw * lo[j];
          acc[4 + j] += cw * hi[j];
        }
      }
    }
    const int head = g * a.group + hblk * kHeadBlk + h;
    if (nparts == 1) {
      const float inv = L > 0.f ? 1.f / L : 0.f;
      u32x4 ov;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        ov[j] = pack_bf16(acc[2 * j] * inv, acc[2 * j + 1] * inv);
      st16((bf16*)a.out + ((int64_t)s * a.hq + head) * kD + 8 * c, ov);
    } else {
      const int64_t slot = ((int64_t)s * a.hq + head) * a.max_parts + part_idx;
      float* po = a.ws_o + slot * kD + 8 * c;
      *reinterpret_cast<f32x4*>(po) = f32x4{acc[0], acc[1], acc[2], acc[3]};
      *reinterpret_cast<f32x4*>(po + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
      if (c == 0) {
        a.ws_ml[2 * slot] = M;
        a.ws_ml[2 * slot + 1] = L;
      }
    }
  }
}

// Exact merge of the partitions of one (sequence, query head):
// o = sum_i 2^(m_i - M) O_i / sum_i 2^(m_i - M) l_i with M = max_i m_i.
template <typename T, bool PAGED>
__global__ __launch_bounds__(kWave) void decode_combine_kernel(DecodeArgs a) {
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  const int ctx = clamp_ctx(a, s, PAGED);
  const int nparts = ctx > 0 ? (ctx + a.part - 1) / a.part : 1;
  if (nparts <= 1) return;
  const int lane = threadIdx.x;
  const int64_t base = ((int64_t)s * a.hq + h) * a.max_parts;
  const float* ml = a.ws_ml + 2 * base;
  // max and weighted sum over the partitions, lanes in parallel
  float M = -INFINITY;
  for (int i = lane; i < nparts; i += kWave) M = fmaxf(M, ml[2 * i]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  float L = 0.f;
  for (int i = lane; i < nparts; i += kWave) {
    const float mi = ml[2 * i];
    if (mi != -INFINITY) L += fast_exp2(mi - M) * ml[2 * i + 1];
  }
  L = wave_sum(L);
  const float inv = L > 0.f ? 1.f / L : 0.f;
  T* out = (T*)a.out + ((int64_t)s * a.hq + h) * a.head_dim;
  const float* po = a.ws_o + base * a.head_dim;
  for (int d = lane; d < a.head_dim; d += kWave) {
    float acc = 0.f;
    for (int i = 0; i < nparts; ++i) {
      const float mi = ml[2 * i];
      if (mi == -INFINITY) continue;
      acc += fast_exp2(mi - M) * po[(int64_t)i * a.head_dim + d];
    }
    out[d] = from_f32<T>(acc * inv);
  }
}

// ---------------------------------------------------------------------------
// Generic path: one wave per (query head, sequence); lanes over head_dim
// (<= 256); one token at a time with an online softmax.
// ---------------------------------------------------------------------------
template <typename T, bool PAGED>
__global__ __launch_bounds__(kWave) void decode_generic_kernel(DecodeArgs a) {
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  const int lane = threadIdx.x;
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
  for (int p = 0; p < ctx; ++p) {
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
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = lane + kWave * i;
      if (d < D) dot += qv[i] * to_f32<T>(kp[d]);
    }
    dot = wave_sum(dot);
    const float x = dot * a.scale_log2;
    const float m_new = fmaxf(m_run, x);
    const float alpha = fast_exp2(m_run - m_new);
    const float pr = fast_exp2(x - m_new);
    l = l * alpha + pr;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = lane + kWave * i;
      const float vv = d < D ? to_f32<T>(vp[d]) : 0.f;
      acc[i] = acc[i] * alpha + pr * vv;
    }
    m_run = m_new;
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  T* op = (T*)a.out + ((int64_t)s * a.hq + h) * D;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int d = lane + kWave * i;
    if (d < D) op[d] = from_f32<T>(acc[i] * inv);
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
int env_part_override() {
  static int cached = -2;
  if (cached == -2) {
    const char* e = getenv("KVPAGED_DECODE_PART");
    cached = e ? atoi(e) : 0;
  }
  return cached;
}

// Tokens per partition of the MFMA path: the largest of 4096..128 that
// still gives at least ~2048 workgroups for the longest context.
int choose_part(int num_seqs, int num_kv_heads, int head_blocks,
                int max_context) {
  const int ov = env_part_override();
  if (ov > 0) {
    int p = (ov + kWaves * kTile - 1) / (kWaves * kTile) * (kWaves * kTile);
    return p > 4096 ? 4096 : p;
  }
  const int64_t units = (int64_t)num_seqs * num_kv_heads * head_blocks;
  int part = 4096;
  while (part > kWaves * kTile) {
    const int64_t parts = (max_context + part - 1) / part;
    if (units * parts >= 2048) break;
    part >>= 1;
  }
  return part;
}

bool fast_path_ok(kv_dtype dtype, int head_dim, int block_size, bool paged) {
  return dtype == KV_BF16 && head_dim == kD &&
         (!paged || block_size % 16 == 0);
}

kv_status run_decode(const char* name, bool paged, DecodeArgs a,
                     kv_dtype dtype, void* workspace, size_t ws_bytes,
                     hipStream_t st) {
  if (dtype != KV_F32 && dtype != KV_BF16)
    return kvp_fail(KV_EINVAL, "%s: unknown dtype %d", name, (int)dtype);
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

  if (fast_path_ok(dtype, a.head_dim, a.block_size, paged)) {
    a.head_blocks = (a.group + kHeadBlk - 1) / kHeadBlk;
    a.part = choose_part(a.num_seqs, a.hkv, a.head_blocks, a.max_ctx);
    a.max_parts = a.max_ctx > 0 ? (a.max_ctx + a.part - 1) / a.part : 1;
    if (a.max_parts > 1) {
      const size_t need = (size_t)a.num_seqs * a.hq * a.max_parts *
                          (a.head_dim + 2) * sizeof(float);
      if (!workspace || ws_bytes < need)
        return kvp_fail(KV_EINVAL, "%s: workspace of %zu bytes needed, %zu given",
                        name, need, ws_bytes);
      a.ws_o = (float*)workspace;
      a.ws_ml = a.ws_o + (size_t)a.num_seqs * a.hq * a.max_parts * a.head_dim;
    }
    dim3 grid(a.hkv * a.head_blocks, a.max_parts, a.num_seqs);
    if (paged)
      decode_mfma_kernel<true><<<grid, kWaves * kWave, 0, st>>>(a);
    else
      decode_mfma_kernel<false><<<grid, kWaves * kWave, 0, st>>>(a);
    KVP_LAUNCH_CHECK(name);
    if (a.max_parts > 1) {
      dim3 g2(a.hq, a.num_seqs);
      if (paged)
        decode_combine_kernel<bf16, true><<<g2, kWave, 0, st>>>(a);
      else
        decode_combine_kernel<bf16, false><<<g2, kWave, 0, st>>>(a);
      KVP_LAUNCH_CHECK(name);
    }
    return KV_OK;
  }
  if (a.head_dim > 4 * kWave)
    return kvp_fail(KV_EUNSUPPORTED, "%s: head_dim %d > 256", name,
                    a.head_dim);
  dim3 grid(a.hq, a.num_seqs);
  if (dtype == KV_F32) {
    if (paged)
      decode_generic_kernel<float, true><<<grid, kWave, 0, st>>>(a);
    else
      decode_generic_kernel<float, false><<<grid, kWave, 0, st>>>(a);
  } else {
    if (paged)
      decode_generic_kernel<bf16, true><<<grid, kWave, 0, st>>>(a);
    else
      decode_generic_kernel<bf16, false><<<grid, kWave, 0, st>>>(a);
  }
  KVP_LAUNCH_CHECK(name);
  return KV_OK;
}

}  // namespace

extern "C" int32_t kv_decode_partition(int32_t num_seqs, int32_t num_q_heads,
                                       int32_t num_kv_heads,
                                       int32_t max_context) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      num_q_heads % num_kv_heads || max_context < 0)
    return KV_EINVAL;
  const int hb = (num_q_heads / num_kv_heads + kHeadBlk - 1) / kHeadBlk;
  return choose_part(num_seqs, num_kv_heads, hb, max_context);
}

extern "C" size_t kv_decode_workspace_bytes(int32_t num_seqs,
                                            int32_t num_q_heads,
                                            int32_t num_kv_heads,
                                            int32_t head_dim,
                                            int32_t max_context) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      num_q_heads % num_kv_heads || head_dim <= 0 || max_context <= 0)
    return 0;
  const int hb = (num_q_heads / num_kv_heads + kHeadBlk - 1) / kHeadBlk;
  const int part = choose_part(num_seqs, num_kv_heads, hb, max_context);
  const int64_t parts = (max_context + part - 1) / part;
  if (parts <= 1) return 0;
  return (size_t)num_seqs * num_q_heads * parts * (head_dim + 2) *
         sizeof(float);
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
