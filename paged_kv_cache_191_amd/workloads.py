"""Seeded synthetic inputs for attention over a paged KV cache.

This module holds shapes and random draws only. It computes none of the
method's arithmetic: no block counts, no slot numbers, no attention. Where a
pool size depends on block counts, the caller passes a function that computes
it, so each side (the oracle in tests, the native library on the device side)
supplies its own.

Every value comes from NumPy's PCG64 generator. Large tensors are drawn in
fixed chunks of ``CHUNK`` elements; chunk ``c`` of stream ``t`` is drawn from
``default_rng([seed, t, c])``. The result therefore does not depend on how
many threads draw it. Streams: 0 = lengths, 1 = free-block order, 2 = Q,
3 = K, 4 = V.

bf16 inputs are drawn as fp32 and rounded to bf16 (round to nearest even, by
torch's conversion); both sides read the rounded values.

The workloads stand in for the model shapes the pages name for vAttention's
evaluation (Yi-6B, Llama-3-8B, Yi-34B, contexts up to 192K) [vAttention
newsletter, "Kod ve Entegrasyon Haritası"]; no dataset or trace is used.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Callable, Optional, Sequence

import numpy as np
import torch

CHUNK = 1 << 22

STREAM_LENGTHS = 0
STREAM_FREE_ORDER = 1
STREAM_Q = 2
STREAM_K = 3
STREAM_V = 4


@dataclass(frozen=True)
class Workload:
    """Shape and value recipe of one synthetic workload.

    kind: "decode"  - one query per sequence against its whole context;
          "prefill" - every token of every sequence is a query, processed in
                      chunks of ``chunk`` tokens with a causal mask;
          "prefix"  - decode where every sequence starts with the same
                      ``prefix_len`` tokens (shared blocks) and then its own
                      suffix.
    lengths: fixed per-sequence lengths, or None to draw them uniformly from
        ``length_range`` (inclusive at both ends). For "prefix" these are the
        suffix lengths.
    pool_blocks: fixed pool size; None means the caller sizes it.
    """

    name: str
    kind: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str  # "f32" | "bf16"
    dist: str  # "uniform" (U[-1, 1)) | "normal" (N(0, 1))
    seed: int
    lengths: Optional[tuple] = None
    length_range: Optional[tuple] = None
    pool_blocks: Optional[int] = None
    chunk: int = 0
    prefix_len: int = 0
    model: str = ""

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "decode_tiny_f32": Workload(
        name="decode_tiny_f32", kind="decode", num_seqs=4, num_q_heads=8,
        num_kv_heads=8, head_dim=64, block_size=16, dtype="f32",
        dist="uniform", seed=1, lengths=(35, 16, 1, 100), pool_blocks=32,
        model="tiny"),
    "llama3_8b_decode": Workload(
        name="llama3_8b_decode", kind="decode", num_seqs=64, num_q_heads=32,
        num_kv_heads=8, head_dim=128, block_size=16, dtype="bf16",
        dist="normal", seed=2, length_range=(512, 4096),
        model="Llama-3-8B-shaped layer"),
    "yi6b_chunked_prefill_b16": Workload(
        name="yi6b_chunked_prefill_b16", kind="prefill", num_seqs=4,
        num_q_heads=32, num_kv_heads=4, head_dim=128, block_size=16,
        dtype="bf16", dist="normal", seed=3, lengths=(32768,) * 4,
        chunk=2048, model="Yi-6B-shaped layer"),
    "yi6b_chunked_prefill_b64": Workload(
        name="yi6b_chunked_prefill_b64", kind="prefill", num_seqs=4,
        num_q_heads=32, num_kv_heads=4, head_dim=128, block_size=64,
        dtype="bf16", dist="normal", seed=3, lengths=(32768,) * 4,
        chunk=2048, model="Yi-6B-shaped layer"),
    "yi34b_long_decode": Workload(
        name="yi34b_long_decode", kind="decode", num_seqs=4, num_q_heads=56,
        num_kv_heads=8, head_dim=128, block_size=64, dtype="bf16",
        dist="normal", seed=4, lengths=(196608,) * 4,
        model="Yi-34B-shaped layer"),
    "prefix_share_decode": Workload(
        name="prefix_share_decode", kind="prefix", num_seqs=256,
        num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
        dtype="bf16", dist="normal", seed=5, length_range=(64, 1024),
        prefix_len=4096, model="Llama-3-8B-shaped layer"),
}


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _draw_f32(seed: int, stream: int, n: int, dist: str) -> np.ndarray:
    """n fp32 values of ``dist`` from (seed, stream), chunked as the module
    docstring states."""
    out = np.empty(n, dtype=np.float32)
    nchunks = (n + CHUNK - 1) // CHUNK

    def fill(c: int) -> None:
        lo = c * CHUNK
        hi = min(n, lo + CHUNK)
        g = np.random.default_rng([seed, stream, c])
        if dist == "normal":
            out[lo:hi] = g.standard_normal(hi - lo, dtype=np.float32)
        elif dist == "uniform":
            u = g.random(hi - lo, dtype=np.float32)
            out[lo:hi] = u * np.float32(2.0) - np.float32(1.0)
        else:
            raise ValueError(f"unknown distribution {dist!r}")

    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


def _storage(a: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(a)
    if dtype == "f32":
        return t
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    raise ValueError(f"unknown dtype {dtype!r}")


def torch_dtype(dtype: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def draw_lengths(w: Workload) -> np.ndarray:
    """Per-sequence lengths (suffix lengths for kind "prefix")."""
    if w.lengths is not None:
        if len(w.lengths) != w.num_seqs:
            raise ValueError("lengths must have num_seqs entries")
        return np.asarray(w.lengths, dtype=np.int64)
    lo, hi = w.length_range
    g = np.random.default_rng([w.seed, STREAM_LENGTHS])
    return g.integers(lo, hi + 1, size=w.num_seqs, dtype=np.int64)


def draw_free_order(w: Workload, num_blocks: int) -> np.ndarray:
    """A seeded permutation of 0..num_blocks-1: the pool's initial free order."""
    g = np.random.default_rng([w.seed, STREAM_FREE_ORDER])
    return g.permutation(num_blocks).astype(np.int32)


@dataclass
class Inputs:
    """One drawn workload.

    lengths: per-sequence token counts of the logical K/V (full context for
        "decode"/"prefill"; suffix only for "prefix").
    cu: token offsets of each sequence's rows in ``k``/``v`` (for "prefix"
        the shared prefix rows come first, at ``prefix_rows``).
    q: "decode"/"prefix": [S, Hq, D]; "prefill": [sum(lengths), Hq, D].
    k, v: [rows, Hkv, D] logical K/V in sequence order.
    free_order: int32 permutation of the pool ids.
    """

    workload: Workload
    lengths: np.ndarray
    cu: np.ndarray
    free_order: np.ndarray
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    prefix_rows: int = 0

    def seq_rows(self, s: int) -> slice:
        return slice(int(self.cu[s]), int(self.cu[s + 1]))


def draw(w: Workload,
         pool_blocks_for: Optional[Callable[[np.ndarray], int]] = None
         ) -> Inputs:
    """Draw a workload. ``pool_blocks_for(lengths)`` sizes the pool when the
    workload does not fix it; it is the caller's arithmetic, not this
    module's."""
    lens = draw_lengths(w)
    if w.pool_blocks is not None:
        n_pool = int(w.pool_blocks)
    else:
        if pool_blocks_for is None:
            raise ValueError(f"{w.name}: pool size depends on the caller")
        n_pool = int(pool_blocks_for(lens))
    free_order = draw_free_order(w, n_pool)

    hq, hkv, d = w.num_q_heads, w.num_kv_heads, w.head_dim
    prefix_rows = w.prefix_len if w.kind == "prefix" else 0
    total_rows = prefix_rows + int(lens.sum())
    cu = np.zeros(w.num_seqs + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lens) + prefix_rows
    cu[0] = prefix_rows
    q_rows = int(lens.sum()) if w.kind == "prefill" else w.num_seqs

    q = _storage(_draw_f32(w.seed, STREAM_Q, q_rows * hq * d, w.dist),
                 w.dtype).view(q_rows, hq, d)
    k = _storage(_draw_f32(w.seed, STREAM_K, total_rows * hkv * d, w.dist),
                 w.dtype).view(total_rows, hkv, d)
    v = _storage(_draw_f32(w.seed, STREAM_V, total_rows * hkv * d, w.dist),
                 w.dtype).view(total_rows, hkv, d)
    return Inputs(workload=w, lengths=lens, cu=cu, free_order=free_order,
                  q=q, k=k, v=v, prefix_rows=prefix_rows)


def logical_rows(inp: Inputs, s: int) -> np.ndarray:
    """Row indices (into ``inp.k``/``inp.v``) of sequence s's tokens in
    logical order: the shared prefix first (kind "prefix"), then its own."""
    own = np.arange(inp.cu[s], inp.cu[s + 1], dtype=np.int64)
    if inp.prefix_rows:
        return np.concatenate(
            [np.arange(inp.prefix_rows, dtype=np.int64), own])
    return own


def context_lengths(inp: Inputs) -> np.ndarray:
    """Tokens per sequence in logical order (prefix + own rows)."""
    return inp.lengths + inp.prefix_rows


def sample_rows(seed: int, n_rows: int, k: int,
                must: Sequence[int] = ()) -> np.ndarray:
    """A seeded, sorted sample of ``k`` distinct row indices in [0, n_rows),
    always containing ``must``."""
    g = np.random.default_rng([seed, 99])
    base = set(int(m) for m in must if 0 <= m < n_rows)
    k = min(k, n_rows)
    if k > len(base):
        pick = g.choice(n_rows, size=min(n_rows, k), replace=False)
        for p in pick:
            if len(base) >= k:
                break
            base.add(int(p))
    return np.array(sorted(base), dtype=np.int64)
