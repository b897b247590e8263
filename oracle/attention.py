"""fp64 oracle: block arithmetic, slot mapping, and exact attention.

TEST INFRASTRUCTURE (see the package docstring): never called by the native
library.

What the pages fix, in my words:
  * The KV cache of a sequence is cut into blocks of a fixed number of token
    slots; tokens fill the blocks in order; a block table maps each logical
    block to a physical block anywhere in memory; attention finds K and V of
    a token through that table [explainer, "PagedAttention Nedir?" and
    "PagedAttention Nasıl Çalışır?" steps 1-4; PagedAttention newsletter,
    "İddia ve Gerçeklik"].
  * Worked example: with 16-slot blocks a 35-token sequence needs three
    blocks and leaves 13 slots of the last one empty [explainer, "PagedAttention
    Nasıl Çalışır?", example after the steps].
  * Only the last block of a sequence can hold empty slots [PagedAttention
    newsletter, "İddia ve Gerçeklik"].
  * Paging changes where the same K/V values sit, not the values, and keeps
    the logical token order [explainer, "KV Cache'i Sıkıştırıyor mu?" and
    "PagedAttention Nedir?"]. Attention over paged K/V is therefore ordinary
    attention over the logically ordered tokens.
  * The attention is exact (FlashAttention's title calls it exact; it avoids
    writing the full score matrix, which changes memory traffic, not the
    result) [explainer, "FlashAttention ile Aynı mı?" and "Kaynaklar"].

Readings where the pages are silent (each also listed in the design notes):
  * slot = table[p // B] * B + p % B; a negative slot means "padding, skip".
  * grouped-query attention: query head h reads KV head h // (Hq / Hkv).
  * scores are scale * (q . k); softmax over the visible keys; a query with
    no visible key returns zeros.
  * decode: the query attends to all L tokens of its sequence (its own K/V
    is written first). Chunked prefill: query at absolute position p sees
    keys 0..p (causal), or all context keys when not causal.

Arrays: K/V pools are [num_blocks, B, Hkv, D] (any float dtype; rows are
converted to float64 after gathering). Contiguous K/V are [S, Lmax, Hkv, D].
Queries are [S, Hq, D] (decode) or [T, Hq, D] (prefill).
"""
from __future__ import annotations

import numpy as np


# --------------------------------------------------------------------------
# Block arithmetic [explainer, "PagedAttention Nasıl Çalışır?"]
# --------------------------------------------------------------------------
def blocks_needed(num_tokens: int, block_size: int) -> int:
    """Blocks a sequence of ``num_tokens`` tokens occupies: tokens fill
    blocks of ``block_size`` slots in order, so the count is the ceiling of
    the quotient (0 tokens -> 0 blocks)."""
    if num_tokens < 0 or block_size <= 0:
        raise ValueError("num_tokens >= 0 and block_size > 0 required")
    full, rest = divmod(num_tokens, block_size)
    return full + (1 if rest else 0)


def unused_slots(num_tokens: int, block_size: int) -> int:
    """Empty slots left in a sequence's blocks; all of them sit in the last
    block [PagedAttention newsletter, "İddia ve Gerçeklik"]."""
    return blocks_needed(num_tokens, block_size) * block_size - num_tokens


def pool_blocks_exact(lengths, block_size: int) -> int:
    """A pool with no slack: the sum of every sequence's block count."""
    return int(sum(blocks_needed(int(n), block_size) for n in lengths))


def waste_fraction(lengths, block_size: int) -> float:
    """Fraction of allocated slots that are empty."""
    alloc = sum(blocks_needed(int(n), block_size) * block_size
                for n in lengths)
    used = sum(int(n) for n in lengths)
    return 0.0 if alloc == 0 else (alloc - used) / alloc


# --------------------------------------------------------------------------
# Slot mapping [explainer steps 3-4; PagedAttention newsletter]
# --------------------------------------------------------------------------
def slot_of(table_row, pos: int, block_size: int) -> int:
    """Physical slot of logical position ``pos``: the table gives the
    physical block of logical block pos // B; the token sits at offset
    pos % B inside it. Slots number the pool's token rows block by block."""
    logical_block, offset = divmod(int(pos), block_size)
    return int(table_row[logical_block]) * block_size + offset


def slot_mapping(block_table, seq_ids, positions, block_size: int
                 ) -> np.ndarray:
    """slot_of for each (seq, position) pair; a negative position maps to
    -1 (padding)."""
    out = np.empty(len(positions), dtype=np.int64)
    for i, (s, p) in enumerate(zip(seq_ids, positions)):
        out[i] = -1 if p < 0 else slot_of(block_table[s], p, block_size)
    return out


def scatter_rows(pool: np.ndarray, rows: np.ndarray, slots) -> None:
    """Write token rows into their slots (the cache write of a new token's
    K or V): ``pool[slot // B, slot % B] = row``; slot < 0 is skipped."""
    block_size = pool.shape[1]
    for r, slot in enumerate(slots):
        if slot < 0:
            continue
        blk, off = divmod(int(slot), block_size)
        pool[blk, off] = rows[r]


def gather_rows(pool: np.ndarray, table_row, length: int) -> np.ndarray:
    """K or V of one sequence in logical order, as float64 [L, Hkv, D],
    read slot by slot through the block table."""
    block_size = pool.shape[1]
    out = np.empty((length,) + pool.shape[2:], dtype=np.float64)
    for p in range(length):
        blk, off = divmod(slot_of(table_row, p, block_size), block_size)
        out[p] = pool[blk, off]
    return out


def copy_blocks(pool: np.ndarray, pairs) -> None:
    """Copy whole physical blocks, src -> dst, in the given order (the data
    side of copy-on-write) [PagedAttention newsletter, "İddia ve
    Gerçeklik"]."""
    for src, dst in pairs:
        pool[int(dst)] = pool[int(src)]


# --------------------------------------------------------------------------
# Exact attention (definition)
# --------------------------------------------------------------------------
def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float
           ) -> np.ndarray:
    """Softmax attention of one query head over n keys, in float64.

    q [D], K [n, D], V [n, D] -> o [D]
      z_j = scale * sum_e q_e K_je
      o   = sum_j exp(z_j - max z) V_j / sum_j exp(z_j - max z)
    Subtracting max z leaves the result unchanged in exact arithmetic and
    keeps exp finite. n == 0 returns zeros.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    if K.shape[0] == 0:
        return np.zeros(V.shape[1], dtype=np.float64)
    z = scale * (K @ q)
    w = np.exp(z - z.max())
    return (w @ V) / w.sum()


def kv_head_of(h: int, num_q_heads: int, num_kv_heads: int) -> int:
    """Grouped-query mapping: consecutive groups of Hq/Hkv query heads share
    one KV head."""
    if num_q_heads % num_kv_heads:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    return h // (num_q_heads // num_kv_heads)


def attend_heads(q_heads: np.ndarray, K: np.ndarray, V: np.ndarray,
                 scale: float) -> np.ndarray:
    """All query heads of one token: q_heads [Hq, D], K/V [n, Hkv, D]."""
    hq = q_heads.shape[0]
    hkv = K.shape[1]
    out = np.empty((hq, V.shape[2]), dtype=np.float64)
    for h in range(hq):
        g = kv_head_of(h, hq, hkv)
        out[h] = attend(q_heads[h], K[:, g], V[:, g], scale)
    return out


# --------------------------------------------------------------------------
# Decode: one query per sequence against its whole context
# --------------------------------------------------------------------------
def decode_logical(q: np.ndarray, ks, vs, scale: float) -> np.ndarray:
    """q [S, Hq, D]; ks[s], vs[s] logical [L_s, Hkv, D] -> o [S, Hq, D]."""
    out = np.empty(q.shape, dtype=np.float64)
    for s in range(q.shape[0]):
        out[s] = attend_heads(np.asarray(q[s], dtype=np.float64),
                              ks[s], vs[s], scale)
    return out


def decode_paged(q, k_pool, v_pool, block_tables, context_lens,
                 scale: float, seqs=None) -> np.ndarray:
    """Decode reading K/V through the block table (one sequence at a time;
    ``seqs`` restricts the work to some sequences, the rest are NaN)."""
    out = np.full(q.shape, np.nan, dtype=np.float64)
    for s in (range(q.shape[0]) if seqs is None else seqs):
        K = gather_rows(k_pool, block_tables[s], int(context_lens[s]))
        V = gather_rows(v_pool, block_tables[s], int(context_lens[s]))
        out[s] = attend_heads(np.asarray(q[s], dtype=np.float64), K, V,
                              scale)
    return out


def decode_contig(q, k, v, context_lens, scale: float) -> np.ndarray:
    """Decode on the contiguous layout [S, Lmax, Hkv, D] (the vAttention
    view: one contiguous buffer per sequence) [vAttention newsletter,
    "İddia ve Gerçeklik"]."""
    ks = [np.asarray(k[s, :int(context_lens[s])], dtype=np.float64)
          for s in range(q.shape[0])]
    vs = [np.asarray(v[s, :int(context_lens[s])], dtype=np.float64)
          for s in range(q.shape[0])]
    return decode_logical(q, ks, vs, scale)


# --------------------------------------------------------------------------
# Chunked prefill
# --------------------------------------------------------------------------
def visible_keys(pos: int, context_len: int, causal: bool) -> int:
    """How many leading keys a query at absolute position ``pos`` sees."""
    if causal:
        return max(0, min(pos + 1, context_len))
    return context_len


def prefill_logical(q, cu_q_lens, q_start_pos, ks, vs, scale: float,
                    causal: bool, rows=None) -> np.ndarray:
    """q [T, Hq, D]; sequence s owns query rows cu_q_lens[s]..cu_q_lens[s+1]
    at absolute positions q_start_pos[s] + i; ks[s], vs[s] hold its context.
    ``rows`` restricts the work to a subset of query rows (others are NaN).
    """
    T = q.shape[0]
    out = np.full(q.shape, np.nan, dtype=np.float64)
    wanted = None if rows is None else set(int(r) for r in rows)
    S = len(cu_q_lens) - 1
    for s in range(S):
        L = ks[s].shape[0]
        for r in range(int(cu_q_lens[s]), int(cu_q_lens[s + 1])):
            if wanted is not None and r not in wanted:
                continue
            pos = int(q_start_pos[s]) + (r - int(cu_q_lens[s]))
            n = visible_keys(pos, L, causal)
            out[r] = attend_heads(np.asarray(q[r], dtype=np.float64),
                                  ks[s][:n], vs[s][:n], scale)
    assert out.shape[0] == T
    return out


def prefill_paged(q, cu_q_lens, q_start_pos, k_pool, v_pool, block_tables,
                  context_lens, scale: float, causal: bool, rows=None
                  ) -> np.ndarray:
    """Chunked prefill reading K/V through the block table, one sequence at
    a time (only sequences owning a requested row are gathered)."""
    S = len(cu_q_lens) - 1
    out = np.full(q.shape, np.nan, dtype=np.float64)
    wanted = None if rows is None else np.asarray(rows)
    empty = np.zeros((0,) + k_pool.shape[2:])
    for s in range(S):
        lo, hi = int(cu_q_lens[s]), int(cu_q_lens[s + 1])
        if wanted is not None and not ((wanted >= lo) & (wanted < hi)).any():
            continue
        K = gather_rows(k_pool, block_tables[s], int(context_lens[s]))
        V = gather_rows(v_pool, block_tables[s], int(context_lens[s]))
        ks = [empty] * S
        vs = [empty] * S
        ks[s], vs[s] = K, V
        sub = None if wanted is None else wanted[(wanted >= lo) & (wanted < hi)]
        part = prefill_logical(q, cu_q_lens, q_start_pos, ks, vs, scale,
                               causal, rows=sub if sub is not None else
                               range(lo, hi))
        out[lo:hi] = part[lo:hi]
    return out


def prefill_contig(q, cu_q_lens, q_start_pos, k, v, context_lens,
                   scale: float, causal: bool, rows=None) -> np.ndarray:
    S = len(cu_q_lens) - 1
    ks = [np.asarray(k[s, :int(context_lens[s])], dtype=np.float64)
          for s in range(S)]
    vs = [np.asarray(v[s, :int(context_lens[s])], dtype=np.float64)
          for s in range(S)]
    return prefill_logical(q, cu_q_lens, q_start_pos, ks, vs, scale, causal,
                           rows)


# --------------------------------------------------------------------------
# Split of the key range and its exact merge
# --------------------------------------------------------------------------
def attend_partial(q, K, V, scale: float):
    """Unnormalised attention over a key subset: returns (m, l, acc) with
    m = max z, l = sum exp(z - m), acc = sum exp(z - m) V. An empty subset
    gives (-inf, 0, 0)."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    if K.shape[0] == 0:
        return -np.inf, 0.0, np.zeros(V.shape[1], dtype=np.float64)
    z = scale * (K @ q)
    m = z.max()
    w = np.exp(z - m)
    return m, w.sum(), w @ V


def merge_partials(parts) -> np.ndarray:
    """Combine (m_i, l_i, acc_i) of disjoint key subsets into the softmax
    over their union: with M = max m_i and c_i = exp(m_i - M),
    o = sum c_i acc_i / sum c_i l_i. Exact in real arithmetic."""
    ms = [p[0] for p in parts if p[1] > 0]
    if not ms:
        return np.zeros_like(parts[0][2])
    M = max(ms)
    num = np.zeros_like(parts[0][2])
    den = 0.0
    for m, l, acc in parts:
        if l == 0:
            continue
        c = np.exp(m - M)
        num = num + c * acc
        den = den + c * l
    return num / den
