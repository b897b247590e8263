"""Benchmark of the paged-KV hot path on one MI355X.

The default run measures every configuration of the workload set, each
against its kernel's roofline, next to its contiguous (vAttention layout)
counterpart, and next to the fp64 CPU oracle timed on a bounded sample:

  decode_tiny_f32      4 sequences (contexts 35, 16, 1, 100), 8/8 heads,
                       head_dim 64, fp32, block 16: the generic decode path,
                       latency-bound (time only, no roofline claim);
  llama3_8b_decode     (the headline) 64 sequences, 32 q / 8 kv heads,
                       block 16, contexts uniform in 512..4096; paged,
                       contiguous, contiguous on demand-mapped memory, and
                       paged over fp8 E4M3 caches with per-head scales;
  yi6b_chunked_prefill 4 x 32768 tokens in 2048-token chunks, 32 q / 4 kv
                       heads, causal: paged B=16, paged B=64, contiguous,
                       contiguous on demand-mapped memory;
  yi34b_long_decode    4 sequences of 196608 tokens, 56 q / 8 kv heads,
                       block 64 (split-K over the context); paged,
                       contiguous, demand-mapped, fp8;
  prefix_share_decode  256 sequences sharing a 4096-token prefix (256 blocks
                       at refcount 256, written once) plus own suffixes
                       uniform in 64..1024, 32 q / 8 kv heads, block 16: the
                       shared-prefix decode, plain paged decode, contiguous
                       (prefix copied per sequence), and the copy-on-write
                       case (a 4104-token prefix whose last block is half
                       full, copied by 255 of the 256 sequences);
  block_swap           2048 blocks out to pinned host memory and back.
All values are synthetic N(0, 1) bf16 (U[-1, 1) fp32 for the small decode)
of the model layers the vAttention evaluation names; head_dim 128.

A decode step is one step of a batch of sequences, each growing by one token:
  host   kv_seq_append: allocation when a block fills (copy-on-write of a
         shared, partly filled block), slot mapping; the block ids it took
         go to a pinned int32 [S] buffer;
  device kv_append_token (the new block ids read from that pinned buffer
         into the device block table, slot, cache write of the new token's
         K/V, length + 1; the table and lengths stay on the device),
         paged_attn_decode (stream-K partitions + exact merge).
The contiguous layouts take the same kernel with one "block" per sequence;
the fp8 decode its fp8 form (kv_append_token_fp8_per_head).
Four independent replicas of the whole batch (pools, tables, queries) rotate
so that no step finds its K/V in the 256 MB last-level cache. Each replica's
two device launches are marshalled once (kv.bind) and re-issued every step,
so the host keeps ahead of the GPU. The timed steps queue nothing else
besides one completion event per step (the replica's pinned buffer is
refilled only after the step that reads it); a second pass of as many steps
brackets each decode op with HIP events for its GPU time. Every event is
created without the system-scope fence (HipEvent), and every timed function
first waits out the slower reads that follow large memory releases
(settle).

`value` = decode algorithmic bytes of the headline workload (K+V once per KV
head, q, o, block-table entries, lengths) summed over the timed steps / wall
time of those steps. With a shared prefix the prefix counts once (unique
bytes); the bytes the sequences read logically are reported beside it as
"effective" GB/s, which can exceed the HBM peak because the shared blocks are
served from cache. The same JSON line carries:
  roofline      - the headline decode op (HIP events around each call on its
                  stream, without the system-scope fence) against 8 TB/s, with the HBM traffic counted by
                  hardware counters when they were taken on these sources;
  rooflines     - the same record for every other measured kernel: decode
                  ops of each workload and layout, the prefill passes
                  (algorithmic FLOPs against 2.5 PFLOP/s bf16), the cache
                  writes and the copy-on-write block copy;
  prefill       - the paged B=16 prefill's roofline record, with every
                  layout's figures beside it;
  paged_vs_contig_overhead - (t_paged - t_contig) / t_contig per
                  configuration (per block size for the prefill);
  plain_read_GBps / frac_of_plain_read (in each decode record) - the rate
                  of a plain streaming read of the same byte count on the
                  same GPU in the same run (libkvprobe.so, the best of 1-4
                  workgroups per CU), and the record's rate against it: the
                  practical read ceiling, next to the published peak;
  cpu_oracle    - the fp64 oracle, single-threaded, per configuration;
  cpu_baseline  - the headline workload's entry of cpu_oracle;
  configs       - every figure of every configuration.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC = ("decode KV-read HBM GB/s (% of peak) + prefill TFLOP/s (% MFMA "
          "peak), paged vs contig")
DECODE_WORKLOADS = ("llama3_8b_decode", "yi34b_long_decode",
                    "prefix_share_decode")
COW_PREFIX = 4104
# appends timed on their own after the timed decode steps
APPEND_TIMING_STEPS = 8


def decode_steps_total(steps: int, warmup: int) -> int:
    """Decode steps a run takes from its replicas: warm-up, the timed
    steps, the same number again with per-op events, and the cache-write
    timing."""
    return warmup + 2 * steps + APPEND_TIMING_STEPS
# GPU spin before each of them (about 40 us at 2.4 GHz)
SPIN_CYCLES = 100_000


class HipEvent:
    """A HIP event created with hipEventDisableSystemFence, recorded on
    torch's current stream. A torch event's record carries a system-scope
    fence: the caches are written back and invalidated at every record, and
    the next kernel pays for it (1-2 us per decode step). The bench's events
    only mark completion (a replica's pinned block-id buffer may be reused
    once the step that reads it has run) and take timestamps, which needs no
    fence. Calls the HIP runtime torch loaded (same soname)."""
    _lib = None

    @classmethod
    def _hip(cls):
        if cls._lib is None:
            import ctypes
            import torch  # noqa: F401  (its HIP runtime is the one resolved)
            lib = ctypes.CDLL("libamdhip64.so.7")
            P = ctypes.c_void_p
            lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(P),
                                                    ctypes.c_uint]
            lib.hipEventRecord.argtypes = [P, P]
            lib.hipEventSynchronize.argtypes = [P]
            lib.hipEventElapsedTime.argtypes = [
                ctypes.POINTER(ctypes.c_float), P, P]
            lib.hipEventDestroy.argtypes = [P]
            cls._lib = lib
        return cls._lib

    @staticmethod
    def _ok(rc: int, what: str) -> None:
        if rc != 0:
            raise RuntimeError(f"{what} returned {rc}")

    def __init__(self, enable_timing: bool = False):
        import ctypes
        self._h = ctypes.c_void_p()
        flags = 0x20000000 | (0 if enable_timing else 0x2)  # no fence; timing
        self._ok(self._hip().hipEventCreateWithFlags(ctypes.byref(self._h),
                                                      flags),
                 "hipEventCreateWithFlags")

    def record(self) -> None:
        import ctypes
        import torch
        self._ok(self._hip().hipEventRecord(
            self._h, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)),
            "hipEventRecord")

    def synchronize(self) -> None:
        self._ok(self._hip().hipEventSynchronize(self._h),
                 "hipEventSynchronize")

    def elapsed_time(self, end: "HipEvent") -> float:
        import ctypes
        ms = ctypes.c_float()
        self._ok(self._hip().hipEventElapsedTime(ctypes.byref(ms), self._h,
                                                 end._h),
                 "hipEventElapsedTime")
        return ms.value

    def __del__(self):
        # not while the interpreter shuts down: the HIP runtime may be gone
        if (self._lib is not None and getattr(self, "_h", None) and
                not sys.is_finalizing()):
            self._lib.hipEventDestroy(self._h)


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# page of the demand-mapped contiguous cache in the prefill pass, in tokens
# of one head (--vmm-page-tokens)
VMM_PREFILL_PAGE_TOKENS = 1024
# pages one process maps at most in a decode run (each page is one device
# allocation; larger pages are used when the contexts would need more)
VMM_MAX_PAGES = 16384

TRAFFIC_PROFILES = {
    "llama3_8b_decode": os.path.join(ROOT, "profiles",
                                     "hbm_traffic_decode_llama3_8b.txt"),
    "yi34b_long_decode": os.path.join(ROOT, "profiles",
                                      "hbm_traffic_decode_yi34b.txt"),
    "prefix_share_decode": os.path.join(ROOT, "profiles",
                                        "hbm_traffic_decode_prefix_share.txt"),
    "yi6b_chunked_prefill_paged_b16": os.path.join(
        ROOT, "profiles", "hbm_traffic_prefill_yi6b_paged_b16.txt"),
}


# profiles that count a whole prefill pass (16 chunk launches)
PASS_PROFILES = ("yi6b_chunked_prefill_paged_b16",)


def recorded_traffic(workload: str = "llama3_8b_decode", fp8: bool = False,
                     fused: bool = False):
    """HBM bytes per decode launch from the committed counter summary
    (FETCH_SIZE/WRITE_SIZE, calibrated on a plain copy; the fp8 op's or the
    fused op's line when asked), or None when no summary exists for the
    workload or the decode sources differ from the ones the counters were
    taken on."""
    import hashlib
    path = TRAFFIC_PROFILES.get(workload)
    if path is None:
        return None
    try:
        text = open(path).read().splitlines()
    except OSError:
        return None
    value = None
    key = ("fp8_fused_traffic_bytes_per_launch:" if fp8 and fused else
           "fp8_traffic_bytes_per_launch:" if fp8 else
           "fused_traffic_bytes_per_launch:" if fused else
           "traffic_bytes_per_pass:" if workload in PASS_PROFILES else
           "traffic_bytes_per_launch:")
    for line in text:
        if line.startswith(key):
            value = int(line.split(":")[1])
        elif line.startswith("source_sha256 "):
            rel, digest = line[len("source_sha256 "):].rsplit(": ", 1)
            with open(os.path.join(ROOT, rel), "rb") as f:
                if hashlib.sha256(f.read()).hexdigest() != digest.strip():
                    return None
    return value


def decode_bytes(ctx: np.ndarray, hq: int, hkv: int, d: int, B: int,
                 paged: bool, esize: int = 2, shared: int = 0,
                 kv_esize: int = 0) -> int:
    """Algorithmic bytes of one decode call: K and V of every context token
    once per KV head (``kv_esize`` bytes per value, default ``esize``), q and
    o, the block-table entries in use, lengths. ``shared`` leading tokens of
    every context sit in the same physical blocks for all sequences and count
    once."""
    toks = int(ctx.sum()) - shared * (len(ctx) - 1) if shared else \
        int(ctx.sum())
    kvb = toks * hkv * d * 2 * (kv_esize or esize)
    qo = 2 * len(ctx) * hq * d * esize
    table = int(sum(-(-int(n) // B) for n in ctx)) * 4 if paged else 0
    return kvb + qo + table + 4 * len(ctx)


# device bytes released outside torch's allocator (demand-mapped pages)
# since the last settle()
_native_freed = 0


def settle(device) -> None:
    """Gives torch's cached device memory back to the driver, then waits
    while the driver works through what was released since the last call.
    Reads have measured about 5% slower for a while after large releases
    (13 GB: about 0.2 s; 40 GB: about 1 s), so every timed function calls
    this first: no timed region starts inside that window."""
    global _native_freed
    import torch
    torch.cuda.synchronize(device)
    peak = torch.cuda.max_memory_reserved(device)
    torch.cuda.empty_cache()
    freed = max(0, peak - torch.cuda.memory_reserved(device)) + _native_freed
    _native_freed = 0
    torch.cuda.reset_peak_memory_stats(device)
    time.sleep(0.05 + 0.05 * freed / 1e9)


def pool_blocks(kv, w, lengths, headroom: int = 0) -> int:
    """Blocks for every sequence with no slack, plus ``headroom``; with a
    shared prefix, its blocks once plus each sequence's blocks past the last
    full prefix block."""
    B = w.block_size
    if w.kind == "prefix":
        P = w.prefix_len
        own = sum(kv.kv_blocks_needed(P + int(n), B) - P // B
                  for n in lengths)
        return kv.kv_blocks_needed(P, B) + own + headroom
    return sum(kv.kv_blocks_needed(int(n), B) for n in lengths) + headroom


def rounded(d: dict) -> dict:
    """Numbers to 4 decimals; other values (names, nested dicts) as they
    are."""
    return {k: round(v, 4) if isinstance(v, float) else v
            for k, v in d.items()}


def stats_ms(ms) -> dict:
    ms = np.asarray(ms, dtype=np.float64)
    return {"mean": float(ms.mean()), "median": float(np.median(ms)),
            "p10": float(np.percentile(ms, 10)),
            "p90": float(np.percentile(ms, 90))}


class DecodeReplica:
    """One independent copy of the decode batch, paged or contiguous. The
    contexts minus their newest token are written through the product path
    (append + cache write); with a shared prefix, sequence 0 writes it and
    the others take shared references to its blocks (fork)."""

    def __init__(self, inp, k_dev, v_dev, new_k, new_v, paged: bool,
                 steps: int, device, shared_op: bool = False,
                 vmm_page_tokens: int = 0, fp8_scales=None,
                 fused: bool = False):
        import torch
        from paged_kv_cache_191_amd import kvpaged as kv
        from paged_kv_cache_191_amd import workloads as W
        self.kv = kv
        self.torch = torch
        w = inp.workload
        self.w = w
        self.paged = paged
        # the step's append fused into the decode op (paged, bf16 or fp8)
        self.fused = fused and paged and not shared_op
        S, B = w.num_seqs, w.block_size
        ctx = W.context_lengths(inp).astype(np.int64)
        self.lmax = int(ctx.max()) + steps + 1
        # demand-mapped contiguous cache: Lmax in whole pages
        self.vmm = vmm_page_tokens if not paged else 0
        if self.vmm:
            self.lmax = -(-self.lmax // self.vmm) * self.vmm
        self.cap = -(-self.lmax // B)
        n_pool = len(inp.free_order)
        # host mirror of [lens int32 S | table int32 S*cap], uploaded once
        # after the set-up writes; the device copy is then kept current by
        # the append kernel
        nbytes = 4 * S + 4 * S * self.cap
        self.h_buf = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
        self.d_buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        hb = self.h_buf.numpy()
        self.h_lens = hb[:4 * S].view(np.int32)
        self.h_table = hb[4 * S:].view(np.int32).reshape(S, self.cap)
        self.d_lens = self.d_buf[:4 * S].view(torch.int32)
        self.d_table = self.d_buf[4 * S:].view(torch.int32).view(S, self.cap)
        self.q = inp.q.to(device)
        self.out = torch.empty_like(self.q)
        self.new_k, self.new_v = new_k, new_v
        tdt = inp.k.dtype
        # fp8 E4M3 caches (paged only), one scale per KV head
        self.fp8 = fp8_scales is not None and paged
        if self.fp8:
            tdt = torch.uint8
            self.k_scales, self.v_scales = fp8_scales
        self.h_table[:] = -1
        self.h_lens[:] = 0
        self.shared = 0
        if paged:
            self.pool = kv.KVPool(n_pool, B, inp.free_order)
            self.k = torch.empty((n_pool, w.num_kv_heads, B, w.head_dim),
                                 dtype=tdt, device=device)
            self.v = torch.empty_like(self.k)

            def write(s, first, count):
                n_new = np.zeros(S, dtype=np.int32)
                n_new[s] = count
                slots, pairs = self.pool.seq_append(self.h_table, self.h_lens,
                                                    n_new)
                assert len(pairs) == 0
                rows = torch.from_numpy(
                    W.logical_rows(inp, s)[first:first + count]).to(device)
                d_slots = torch.from_numpy(slots).to(device)
                if self.fp8:
                    kv.kv_reshape_and_cache_fp8_per_head(
                        k_dev[rows], v_dev[rows], d_slots, self.k, self.v,
                        self.k_scales, self.v_scales)
                else:
                    kv.kv_reshape_and_cache(k_dev[rows], v_dev[rows],
                                            d_slots, self.k, self.v)

            P = inp.prefix_rows
            if P:
                write(0, 0, P)
                nb = kv.kv_blocks_needed(P, B)
                for s in range(1, S):
                    self.pool.share(self.h_table[0, :nb].tolist())
                    self.h_table[s, :nb] = self.h_table[0, :nb]
                    self.h_lens[s] = P
                self.shared = (P // B) * B
            for s in range(S):
                first = int(self.h_lens[s])
                write(s, first, int(ctx[s]) - 1 - first)
        elif self.vmm:
            # pages mapped as each sequence's context is written
            self.vc = kv.VCache(S, self.lmax, w.num_kv_heads, w.head_dim,
                                tdt, self.vmm)
            self.k, self.v = self.vc.k, self.vc.v
            self.map_s = 0.0
            self.map_pages = 0
            for s in range(S):
                n = int(ctx[s]) - 1
                t0 = time.perf_counter()
                self.map_pages += self.vc.reserve(s, n)
                self.map_s += time.perf_counter() - t0
                rows = torch.from_numpy(W.logical_rows(inp, s)[:n]).to(device)
                slots = torch.arange(s * self.lmax, s * self.lmax + n,
                                     dtype=torch.int64, device=device)
                kv.kv_reshape_and_cache(k_dev[rows], v_dev[rows], slots,
                                        self.k, self.v)
                self.h_lens[s] = n
            self.mapped_tok = np.array(
                [self.vc.seq_pages(s) * self.vmm for s in range(S)])
            self.step_map_s = []
            self.step_map_pages = []
        else:
            self.k = torch.empty((S, w.num_kv_heads, self.lmax, w.head_dim),
                                 dtype=tdt, device=device)
            self.v = torch.empty_like(self.k)
            for s in range(S):
                n = int(ctx[s]) - 1
                rows = torch.from_numpy(W.logical_rows(inp, s)[:n]).to(device)
                self.k[s, :, :n] = k_dev[rows].transpose(0, 1)
                self.v[s, :, :n] = v_dev[rows].transpose(0, 1)
                self.h_lens[s] = n
        # shared_op: decode through paged_attn_decode_shared_prefix with
        # one group (all sequences) sharing the prefix's whole blocks
        self.shared_op = shared_op and paged and self.shared > 0
        if self.shared_op:
            self.ws = kv.decode_shared_prefix_workspace(
                S, w.num_q_heads, w.num_kv_heads, w.head_dim, self.lmax,
                self.shared, device)
            self.g_starts = torch.tensor([0, S], dtype=torch.int32,
                                         device=device)
            self.g_shared = torch.tensor([self.shared], dtype=torch.int32,
                                         device=device)
        else:
            self.ws = kv.decode_workspace(S, w.num_q_heads, w.num_kv_heads,
                                          w.head_dim, self.lmax, device)
        # Device-resident table and lengths for kv_append_token, uploaded
        # once here. Contiguous layouts: one block per sequence
        # (table[s] = [s], block_size = Lmax).
        self.h_newb = torch.full((S,), -1, dtype=torch.int32,
                                 pin_memory=True)
        self.d_buf.copy_(self.h_buf)
        if paged:
            self.a_table = self.d_table
        else:
            self.a_table = torch.arange(S, dtype=torch.int32,
                                        device=device).view(S, 1)
        # The pinned block-id buffer is rewritten only after the append that
        # read it has run: `uploaded` is an event recorded after that append
        # (the decode op's start event in a step).
        self.uploaded = HipEvent()
        self.uploaded.record()
        # the replica's own event for steps without timing events (recorded
        # again each step: the next host_append of this replica has waited
        # on it by then)
        self.done_ev = HipEvent()
        self.scale = 1.0 / float(np.sqrt(w.head_dim))
        self._bind_launches()
        torch.cuda.synchronize()

    def _bind_launches(self) -> None:
        """The step's two device launches, marshalled once (kv.bind): the
        cache write and the decode op re-issue the same native calls every
        step, as a serving loop in C++ would. The decode's context bound is
        the replica's capacity, lmax, which holds every length of the run
        (the bound only clamps lengths)."""
        kv = self.kv
        if self.fused and self.fp8:
            self._write = None
            self._decode = kv.bind(
                kv.paged_attn_decode_append_fp8_per_head, self.out, self.q,
                self.new_k, self.new_v, self.h_newb, self.k, self.v,
                self.d_table, self.d_lens, self.lmax, self.scale,
                self.k_scales, self.v_scales, self.ws)
            return
        if self.fused:
            self._write = None
            self._decode = kv.bind(
                kv.paged_attn_decode_append, self.out, self.q, self.new_k,
                self.new_v, self.h_newb, self.k, self.v, self.d_table,
                self.d_lens, self.lmax, self.scale, self.ws)
            return
        if self.fp8:
            self._write = kv.bind(
                kv.kv_append_token_fp8_per_head, self.new_k, self.new_v,
                self.h_newb, self.a_table, self.d_lens, self.k, self.v,
                self.k_scales, self.v_scales)
            self._decode = kv.bind(
                kv.paged_attn_decode_fp8_per_head, self.out, self.q, self.k,
                self.v, self.d_table, self.d_lens, self.lmax, self.scale,
                self.k_scales, self.v_scales, self.ws)
            return
        self._write = kv.bind(kv.kv_append_token, self.new_k, self.new_v,
                              self.h_newb, self.a_table, self.d_lens, self.k,
                              self.v)
        if self.shared_op:
            self._decode = kv.bind(
                kv.paged_attn_decode_shared_prefix, self.out, self.q, self.k,
                self.v, self.d_table, self.d_lens, self.lmax, self.g_starts,
                self.g_shared, self.w.num_seqs, self.shared, self.scale,
                self.ws)
        elif self.paged:
            self._decode = kv.bind(kv.paged_attn_decode, self.out, self.q,
                                   self.k, self.v, self.d_table, self.d_lens,
                                   self.lmax, self.scale, self.ws)
        else:
            self._decode = kv.bind(kv.contig_attn_decode, self.out, self.q,
                                   self.k, self.v, self.d_lens, self.lmax,
                                   self.scale, self.ws)

    def host_append(self) -> None:
        """Host part of a step. Paged: kv_seq_append (allocation, slot
        mapping) on the host mirror, and the block ids it took (-1 where the
        entry did not change) into the pinned buffer the append kernel
        reads. Contiguous: the host lengths advance (and, demand-mapped, the
        pages a new token needs are mapped)."""
        self.uploaded.synchronize()
        if self.paged:
            S = self.w.num_seqs
            ar = np.arange(S)
            idx = self.h_lens // self.w.block_size
            before = self.h_table[ar, idx]
            _, pairs = self.pool.seq_append(self.h_table, self.h_lens)
            assert len(pairs) == 0
            after = self.h_table[ar, idx]
            self.h_newb.numpy()[:] = np.where(after != before, after, -1)
        else:
            self.h_lens += 1
            if self.vmm:
                # map a page for the sequences whose new token starts one
                t0 = time.perf_counter()
                n = 0
                for s in np.nonzero(self.h_lens > self.mapped_tok)[0]:
                    n += self.vc.reserve(int(s), int(self.h_lens[s]))
                    self.mapped_tok[s] = self.vc.seq_pages(int(s)) * self.vmm
                self.step_map_s.append(time.perf_counter() - t0)
                self.step_map_pages.append(n)

    def close(self) -> None:
        global _native_freed
        if self.vmm:
            _native_freed += self.vc.mapped_bytes
            self.vc.close()

    def cache_write(self, done=None) -> None:
        """Device part of the append: the new token's row in the cache, the
        table entry and the length on the device. `done` (an event, default
        a new one) is recorded after it and marks the pinned buffer free."""
        self._write()
        self.uploaded = done if done is not None else self.done_ev
        self.uploaded.record()

    def device_step(self, ev=None) -> None:
        """Cache write, then the decode op, bracketed by ev[0], ev[1]; ev[0]
        also marks the end of the cache write. Fused: the one op (append and
        decode), bracketed by ev[0], ev[1]; its end frees the pinned
        buffer."""
        if self.fused:
            if ev is not None:
                ev[0].record()
            self._decode()
            self.uploaded = ev[1] if ev is not None else self.done_ev
            self.uploaded.record()
            return
        self.cache_write(ev[0] if ev is not None else None)
        self._decode()
        if ev is not None:
            ev[1].record()


def new_token_kv(w, device):
    """K/V of the token each sequence appends per step (seeded, bf16)."""
    import torch
    g = np.random.default_rng([w.seed, 50])
    shape = (w.num_seqs, w.num_kv_heads, w.head_dim)
    mk = [torch.from_numpy(g.standard_normal(shape, dtype=np.float32)).to(
        torch.bfloat16).to(device) for _ in range(2)]
    return mk[0], mk[1]


def fp8_head_scales(k_dev, v_dev):
    """Per-KV-head scales of the fp8 caches: the largest |value| of each
    head over the workload's rows maps to E4M3's largest finite value, 448
    (set-up, before the timed steps)."""
    return tuple((t.abs().amax(dim=(0, 2)).float() / 448.0).contiguous()
                 for t in (k_dev, v_dev))


def run_decode(inp, paged: bool, steps: int, warmup: int, reps: int,
               device, shared_op: bool = False, vmm_page_tokens: int = 0,
               fp8: bool = False, fused: bool = False):
    settle(device)
    import torch
    w = inp.workload
    new_k, new_v = new_token_kv(w, device)
    k_dev, v_dev = inp.k.to(device), inp.v.to(device)
    scales = fp8_head_scales(k_dev, v_dev) if fp8 else None
    reps_ = [DecodeReplica(inp, k_dev, v_dev, new_k, new_v, paged,
                           decode_steps_total(steps, warmup), device,
                           shared_op, vmm_page_tokens, scales, fused)
             for _ in range(reps)]
    del k_dev, v_dev
    for i in range(warmup):
        r = reps_[i % reps]
        r.host_append()
        r.device_step()
    torch.cuda.synchronize()
    kv_es = 1 if fp8 else 0

    def step_bytes(r, lens=None):
        args = (r.h_lens if lens is None else lens, w.num_q_heads,
                w.num_kv_heads, w.head_dim, w.block_size, paged)
        return (decode_bytes(*args, shared=r.shared, kv_esize=kv_es),
                decode_bytes(*args, kv_esize=kv_es))

    # The timed steps: host append, cache write and decode op, nothing else
    # queued (the per-op events are a second pass below). The lengths each
    # step attends over are copied aside; their bytes are counted after the
    # timed region.
    lens_seen = []
    t0 = time.perf_counter()
    for i in range(steps):
        r = reps_[i % reps]
        r.host_append()
        lens_seen.append((r, r.h_lens.copy()))
        r.device_step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_bytes = logical_bytes = 0
    for r, lens in lens_seen:
        b, lb = step_bytes(r, lens)
        total_bytes += b
        logical_bytes += lb
    # The same steps again (the contexts one token per replica round
    # longer), each decode op bracketed by events: its GPU time.
    evs = [tuple(HipEvent(enable_timing=True) for _ in range(2))
           for _ in range(steps)]
    op_bytes = op_logical = 0
    for i in range(steps):
        r = reps_[i % reps]
        r.host_append()
        b, lb = step_bytes(r)
        op_bytes += b
        op_logical += lb
        r.device_step(evs[i])
    torch.cuda.synchronize()
    op = stats_ms([a.elapsed_time(b) for a, b in evs])
    # The cache write alone (the append kernel),
    # timed after the timed steps so that its events stay out of them. A
    # short spin kernel keeps the GPU busy while the host queues the events
    # and the write, so the interval is GPU time, not launch latency.
    # (The fused op has no separate cache write.)
    rc_ev = []
    for i in range(0 if fused else APPEND_TIMING_STEPS):
        r = reps_[i % reps]
        r.host_append()
        e = tuple(HipEvent(enable_timing=True) for _ in range(2))
        torch.cuda._sleep(SPIN_CYCLES)
        e[0].record()
        r.cache_write(e[1])
        rc_ev.append(e)
    torch.cuda.synchronize()
    rc = stats_ms([a.elapsed_time(b) for a, b in rc_ev]) if rc_ev else None
    res = {
        "wall_s": wall,
        "ms_per_step": 1e3 * wall / steps,
        "step_GBps": total_bytes / wall / 1e9,
        "decode_op_ms_mean": op["mean"],
        "decode_op_ms_median": op["median"],
        "decode_op_ms_p10": op["p10"],
        "decode_op_ms_p90": op["p90"],
        "bytes_per_step": total_bytes / steps,
        "cache_write": (("fused into paged_attn_decode_append_fp8_per_head"
                         if fp8 else "fused into paged_attn_decode_append")
                        if fused else "kv_append_token" if not fp8 else
                        "kv_append_token_fp8_per_head"),
    }
    if rc is not None:
        res["cache_write_us_median"] = 1e3 * rc["median"]
    res["op_bytes_per_step"] = op_bytes / steps
    res["decode_op_GBps"] = res["op_bytes_per_step"] / (op["mean"] * 1e-3) / 1e9
    if logical_bytes != total_bytes:
        res["logical_bytes_per_step"] = logical_bytes / steps
        res["decode_op_effective_GBps"] = (op_logical / steps) / (
            op["mean"] * 1e-3) / 1e9
    # the new rows: K and V, read once (bf16) and written once
    tok_bytes = w.num_seqs * w.num_kv_heads * w.head_dim * 2 * (
        2 + (1 if fp8 else 2))
    if rc is not None:
        res["cache_write_GBps"] = tok_bytes / (rc["median"] * 1e-3) / 1e9
    if vmm_page_tokens and not paged:
        P = vmm_page_tokens
        r0 = reps_[0]
        page_bytes = P * w.head_dim * 2
        used = float(r0.h_lens.sum()) * w.num_kv_heads * w.head_dim * 2 * 2
        mapped = r0.vc.mapped_bytes
        # the same contexts in 64 KiB and 2 MiB pages

        def mapped_with(page_b):
            tok = page_b // (w.head_dim * 2)
            return float(np.sum(-(-r0.h_lens // tok))) * \
                w.num_kv_heads * 2 * page_b
        step_s = [x for r in reps_ for x in r.step_map_s]
        step_pages = [x for r in reps_ for x in r.step_map_pages]
        res["vmm"] = {
            "page_tokens": P, "page_bytes": page_bytes,
            "fill_map_us_per_page": 1e6 * sum(r.map_s for r in reps_) /
            max(1, sum(r.map_pages for r in reps_)),
            "fill_pages_per_replica": r0.map_pages,
            "step_pages_mapped_mean": float(np.mean(step_pages)),
            "step_map_host_us_mean": 1e6 * float(np.mean(step_s)),
            "step_map_host_us_max": 1e6 * float(np.max(step_s)),
            "mapped_bytes": mapped, "used_bytes": used,
            "waste": 1.0 - used / mapped,
            "waste_64KiB_pages": 1.0 - used / mapped_with(64 << 10),
            "waste_2MiB_pages": 1.0 - used / mapped_with(2 << 20),
        }
    if fp8:
        res["fp8_k_scales"] = [round(float(x), 6) for x in scales[0].cpu()]
        res["fp8_v_scales"] = [round(float(x), 6) for x in scales[1].cpu()]
    for r in reps_:
        r.close()
    del reps_
    torch.cuda.empty_cache()
    return res


def run_tiny_decode(device, launches: int = 50):
    """The small fp32 decode configuration (4 sequences, contexts 35, 16, 1
    and 100, 8/8 heads, head_dim 64, block 16, 32-block pool): the generic
    path, latency-bound, so its time is reported without a roofline. Each
    launch is timed with events behind a GPU spin (kernel time, not launch
    latency)."""
    settle(device)
    import torch
    from paged_kv_cache_191_amd import kvpaged as kv
    from paged_kv_cache_191_amd import workloads as W
    w = W.WORKLOADS["decode_tiny_f32"]
    B, S = w.block_size, w.num_seqs
    inp = W.draw(w, lambda L: pool_blocks(kv, w, L))
    n_pool = len(inp.free_order)
    pool = kv.KVPool(n_pool, B, inp.free_order)
    cap = -(-int(inp.lengths.max()) // B)
    table = np.full((S, cap), -1, dtype=np.int32)
    lens = np.zeros(S, dtype=np.int32)
    slots, _ = pool.seq_append(table, lens, inp.lengths.astype(np.int32))
    kc = torch.zeros((n_pool, w.num_kv_heads, B, w.head_dim),
                     dtype=torch.float32, device=device)
    vc = torch.zeros_like(kc)
    kv.kv_reshape_and_cache(inp.k.to(device), inp.v.to(device),
                            torch.from_numpy(slots).to(device), kc, vc)
    q = inp.q.to(device)
    out = torch.empty_like(q)
    bt = torch.from_numpy(table).to(device)
    ctx = torch.from_numpy(lens).to(device)
    scale = 1.0 / float(np.sqrt(w.head_dim))
    times = []
    for i in range(launches + 10):
        ev = [HipEvent(enable_timing=True) for _ in range(2)]
        torch.cuda._sleep(SPIN_CYCLES)
        ev[0].record()
        kv.paged_attn_decode(out, q, kc, vc, bt, ctx, int(lens.max()), scale)
        ev[1].record()
        if i >= 10:
            times.append(ev)
    torch.cuda.synchronize()
    us = stats_ms([a.elapsed_time(b) for a, b in times])
    pool.close()
    return {"tokens": int(lens.sum()), "dtype": "f32",
            "decode_op_us_median": 1e3 * us["median"],
            "decode_op_us_p10": 1e3 * us["p10"],
            "decode_op_us_p90": 1e3 * us["p90"]}


def run_swap(w, device, n_blocks: int = 2048, reps: int = 5):
    """Swap of n_blocks blocks of the workload's pool shape (K and V) out to a
    pinned host pool and back in (kv_swap_blocks), timed with events: the
    PCIe cost of preempting sequences when the device pool is full."""
    settle(device)
    import torch
    from paged_kv_cache_191_amd import kvpaged as kv
    shape = (n_blocks, w.num_kv_heads, w.block_size, w.head_dim)
    dk = torch.randn(shape, dtype=torch.float32, device=device).to(
        torch.bfloat16)
    dv = torch.randn(shape, dtype=torch.float32, device=device).to(
        torch.bfloat16)
    hk = torch.empty(shape, dtype=torch.bfloat16).pin_memory()
    hv = torch.empty(shape, dtype=torch.bfloat16).pin_memory()
    perm = np.random.default_rng([w.seed, 60]).permutation(n_blocks)
    pairs = torch.from_numpy(np.stack([perm, np.arange(n_blocks)], 1).astype(
        np.int32)).to(device)
    back = torch.from_numpy(np.stack([np.arange(n_blocks), perm], 1).astype(
        np.int32)).to(device)
    t_out, t_in = [], []
    for i in range(reps + 1):
        e = [HipEvent(enable_timing=True) for _ in range(3)]
        e[0].record()
        kv.kv_swap_blocks(dk, dv, hk, hv, pairs)
        e[1].record()
        kv.kv_swap_blocks(hk, hv, dk, dv, back)
        e[2].record()
        torch.cuda.synchronize()
        if i:
            t_out.append(e[0].elapsed_time(e[1]))
            t_in.append(e[1].elapsed_time(e[2]))
    nbytes = 2 * dk.numel() * 2
    res = {"blocks": n_blocks, "bytes": nbytes,
           "out_ms_median": float(np.median(t_out)),
           "in_ms_median": float(np.median(t_in))}
    res["out_GBps"] = nbytes / (res["out_ms_median"] * 1e-3) / 1e9
    res["in_GBps"] = nbytes / (res["in_ms_median"] * 1e-3) / 1e9
    del dk, dv, hk, hv
    torch.cuda.empty_cache()
    return res


def run_cow(w, steps: int, warmup: int, device):
    """Copy-on-write step: 256 sequences forked from a COW_PREFIX-token
    prefix whose last block is half full each append one token; 255 of them
    copy that block (kv_copy_blocks), the last finds it unshared and writes
    in place; the decode then shares the prefix's whole blocks. Every repetition starts from a fresh allocator with the same
    free order, so the prefix rows (written once) stay valid."""
    settle(device)
    import torch
    from paged_kv_cache_191_amd import kvpaged as kv
    from paged_kv_cache_191_amd import workloads as W
    wc = w.replace(prefix_len=COW_PREFIX, name="prefix_share_cow")
    S, B, P = wc.num_seqs, wc.block_size, COW_PREFIX
    nb_prefix = kv.kv_blocks_needed(P, B)
    n_pool = nb_prefix + S
    inp = W.draw(wc, lambda L: n_pool)
    cap = kv.kv_blocks_needed(P + 1, B)
    tdt = inp.k.dtype
    kc = torch.empty((n_pool, wc.num_kv_heads, B, wc.head_dim), dtype=tdt,
                     device=device)
    vc = torch.empty_like(kc)
    new_k, new_v = new_token_kv(wc, device)
    q = inp.q.to(device)
    out = torch.empty_like(q)
    shared = (P // B) * B  # whole blocks still shared after the copies
    ws = kv.decode_shared_prefix_workspace(S, wc.num_q_heads, wc.num_kv_heads,
                                           wc.head_dim, P + 1, shared, device)
    g_starts = torch.tensor([0, S], dtype=torch.int32, device=device)
    g_shared = torch.tensor([shared], dtype=torch.int32, device=device)
    scale = 1.0 / float(np.sqrt(wc.head_dim))
    times, host_us, n_pairs = [], [], 0
    for i in range(warmup + steps):
        t_h = time.perf_counter()
        pool = kv.KVPool(n_pool, B, inp.free_order)
        table = np.full((S, cap), -1, dtype=np.int32)
        lens = np.zeros(S, dtype=np.int32)
        n_new = np.zeros(S, dtype=np.int32)
        n_new[0] = P
        slots0, _ = pool.seq_append(table, lens, n_new)
        # fork: one reference to each prefix block per other sequence, in
        # one call (kv_block_share counts repeated ids once per occurrence)
        pool.share(np.tile(table[0, :nb_prefix], S - 1))
        table[1:, :nb_prefix] = table[0, :nb_prefix]
        lens[1:] = P
        slots, pairs = pool.seq_append(table, lens)
        host_us.append(1e6 * (time.perf_counter() - t_h))
        n_pairs = len(pairs)
        if i == 0:
            rows = torch.arange(P, device=device)
            kv.kv_reshape_and_cache(inp.k.to(device)[rows],
                                    inp.v.to(device)[rows],
                                    torch.from_numpy(slots0).to(device), kc,
                                    vc)
        d_pairs = torch.from_numpy(pairs).to(device)
        d_slots = torch.from_numpy(slots).to(device)
        d_table = torch.from_numpy(table).to(device)
        d_lens = torch.from_numpy(lens).to(device)
        ev = [HipEvent(enable_timing=True) for _ in range(3)]
        # keep the GPU busy while the step is queued, so that the events
        # time the kernels and not the launch latency after the host work
        torch.cuda._sleep(SPIN_CYCLES)
        ev[0].record()
        kv.kv_copy_blocks(kc, vc, d_pairs)
        ev[1].record()
        kv.kv_reshape_and_cache(new_k, new_v, d_slots, kc, vc)
        kv.paged_attn_decode_shared_prefix(out, q, kc, vc, d_table, d_lens,
                                           int(lens.max()), g_starts,
                                           g_shared, S, shared, scale, ws)
        ev[2].record()
        torch.cuda.synchronize()
        if i >= warmup:
            times.append((ev[0].elapsed_time(ev[1]),
                          ev[0].elapsed_time(ev[2])))
        pool.close()
    copy_ms = stats_ms([a for a, _ in times])
    step_ms = stats_ms([b for _, b in times])
    copy_bytes = 2 * n_pairs * B * wc.num_kv_heads * wc.head_dim * 2 * 2
    del kc, vc
    torch.cuda.empty_cache()
    return {"prefix_tokens": P, "cow_copies": n_pairs,
            "copy_blocks_us_median": 1e3 * copy_ms["median"],
            "copy_blocks_GBps": copy_bytes / (copy_ms["median"] * 1e-3) / 1e9,
            "step_incl_cow_us_median": 1e3 * step_ms["median"],
            "step_incl_cow_us_p10": 1e3 * step_ms["p10"],
            "step_incl_cow_us_p90": 1e3 * step_ms["p90"],
            "host_fork_and_append_us_median": float(np.median(host_us))}


def prefill_pass(inp, layout: str, device):
    settle(device)
    import torch
    from paged_kv_cache_191_amd import kvpaged as kv
    w = inp.workload
    S, B, C = w.num_seqs, w.block_size, w.chunk
    N = int(inp.lengths.max())
    scale = 1.0 / float(np.sqrt(w.head_dim))
    tdt = inp.k.dtype
    q_dev = inp.q.to(device)
    k_dev = inp.k.to(device)
    v_dev = inp.v.to(device)
    vcache = None
    map_s, map_pages = [], []
    if layout == "contig":
        kc = torch.empty((S, w.num_kv_heads, N, w.head_dim), dtype=tdt,
                         device=device)
        vc = torch.empty_like(kc)
    elif layout == "vattn":
        # contiguous layout on demand-mapped memory: pages are mapped as
        # each chunk's rows are written
        vcache = kv.VCache(S, N, w.num_kv_heads, w.head_dim, tdt,
                           VMM_PREFILL_PAGE_TOKENS)
        kc, vc = vcache.k, vcache.v
    else:
        n_pool = len(inp.free_order)
        kc = torch.empty((n_pool, w.num_kv_heads, B, w.head_dim), dtype=tdt,
                         device=device)
        vc = torch.empty_like(kc)
    cap = -(-N // B)
    out = torch.empty((S * C, w.num_q_heads, w.head_dim), dtype=tdt,
                      device=device)
    flops_total = 0.0
    times = []

    def one_pass(timed: bool):
        nonlocal flops_total
        pool = kv.KVPool(len(inp.free_order), B, inp.free_order) \
            if layout == "paged" else None
        table = np.full((S, cap), -1, dtype=np.int32)
        lens = np.zeros(S, dtype=np.int32)
        if vcache is not None:
            # start from unmapped sequences; pages come back from the pool
            torch.cuda.synchronize()
            for s in range(S):
                vcache.release(s)
        t_map, n_map = 0.0, 0
        for c0 in range(0, N, C):
            n_new = np.full(S, C, dtype=np.int32)
            if vcache is not None:
                t0 = time.perf_counter()
                for s in range(S):
                    n_map += vcache.reserve(s, c0 + C)
                t_map += time.perf_counter() - t0
            if pool is not None:
                slots, _ = pool.seq_append(table, lens, n_new)
            else:
                slots = (np.arange(S)[:, None] * N + lens[:, None] +
                         np.arange(C)[None, :]).reshape(-1).astype(np.int64)
                lens += C
            rows = (np.arange(S)[:, None] * N + c0 +
                    np.arange(C)[None, :]).reshape(-1)
            rows_d = torch.from_numpy(rows).to(device)
            k_new, v_new = k_dev[rows_d], v_dev[rows_d]
            d_slots = torch.from_numpy(slots).to(device)
            cu = torch.arange(0, S * C + 1, C, dtype=torch.int32,
                              device=device)
            start = torch.full((S,), c0, dtype=torch.int32, device=device)
            ctx = torch.from_numpy(lens.copy()).to(device)
            d_table = torch.from_numpy(table).to(device)
            q = q_dev[rows_d]
            ev = [HipEvent(enable_timing=True) for _ in range(3)]
            torch.cuda._sleep(SPIN_CYCLES)   # GPU busy while this is queued
            ev[0].record()
            kv.kv_reshape_and_cache(k_new, v_new, d_slots, kc, vc)
            ev[1].record()
            if layout != "paged":
                kv.contig_attn_prefill(out, q, cu, start, C, kc, vc, ctx,
                                       scale, True)
            else:
                kv.paged_attn_prefill(out, q, cu, start, C, kc, vc, d_table,
                                      ctx, scale, True)
            ev[2].record()
            if timed:
                times.append(ev)
                # unmasked causal pairs of this chunk, 4*d*Hq flops each
                pairs = S * (C * c0 + C * (C + 1) // 2)
                flops_total += 4.0 * w.head_dim * w.num_q_heads * pairs
        torch.cuda.synchronize()
        if timed:
            map_s.append(t_map)
            map_pages.append(n_map)

    one_pass(False)
    t0 = time.perf_counter()
    one_pass(True)
    wall = time.perf_counter() - t0
    attn_ms = sum(e[1].elapsed_time(e[2]) for e in times)
    rc_ms = [e[0].elapsed_time(e[1]) for e in times]
    # new rows per chunk: K and V, read once and written once
    rc_bytes = S * C * w.num_kv_heads * w.head_dim * 2 * 2 * 2
    res = {"attn_ms": attn_ms, "pass_wall_ms": 1e3 * wall,
           "TFLOPs": flops_total / (attn_ms * 1e-3) / 1e12,
           "tflop": flops_total / 1e12,
           "reshape_and_cache_us_median": 1e3 * float(np.median(rc_ms)),
           "reshape_and_cache_GBps": rc_bytes / (float(np.median(rc_ms)) *
                                                 1e-3) / 1e9}
    if vcache is not None:
        res["vmm_page_tokens"] = VMM_PREFILL_PAGE_TOKENS
        res["vmm_pages_mapped_per_pass"] = map_pages[0]
        res["vmm_map_host_ms_per_pass"] = 1e3 * map_s[0]
        res["vmm_map_us_per_page"] = 1e6 * map_s[0] / max(1, map_pages[0])
        torch.cuda.synchronize()
        global _native_freed
        _native_freed += vcache.mapped_bytes
        vcache.close()
    del kc, vc, q_dev, k_dev, v_dev, out
    torch.cuda.empty_cache()
    return res


def memory_waste(inp, lmax_reserved: int) -> dict:
    """Unused slots of the paged pool (the tail of each sequence's last
    block; a shared prefix held once) next to a contiguous reservation of
    ``lmax_reserved`` tokens per sequence (a shared prefix copied into every
    sequence), at the drawn contexts."""
    from paged_kv_cache_191_amd import kvpaged as kv
    from paged_kv_cache_191_amd import workloads as W
    w = inp.workload
    held = pool_blocks(kv, w, inp.lengths) * w.block_size
    unique = int(inp.lengths.sum()) + int(inp.prefix_rows)
    logical = int(W.context_lengths(inp).sum())
    reserved = len(inp.lengths) * lmax_reserved
    return {"paged_held_tokens": held,
            "paged_waste": round(1.0 - unique / held, 5),
            "contig_reserved_tokens": reserved,
            "contig_reservation_waste": round(1.0 - logical / reserved, 5),
            "contig_reserved_over_paged_held": round(reserved / held, 3)}


# ---------------------------------------------------------------------------
# The fp64 oracle on this host (a reported baseline, not the target)
# ---------------------------------------------------------------------------
def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def _one_thread():
    """A context that holds NumPy's BLAS pools at one thread: the oracle's
    time goes to its per-token gather loop in Python, which runs on one core
    whatever the BLAS threads (more threads measured slower)."""
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(limits=1)
    except Exception:                                  # noqa: BLE001
        import contextlib
        return contextlib.nullcontext()


def _oracle_pool(inp, seqs, upto=None):
    """The oracle's model allocator over the whole workload (host metadata
    only) and float32 pools holding the rows of `seqs` (the prefix, if any,
    written once by sequence 0 and shared by fork). Set-up, not timed."""
    from oracle import allocator as A
    from oracle import attention as O
    from paged_kv_cache_191_amd import workloads as W
    w = inp.workload
    S, B = w.num_seqs, w.block_size
    ctx = W.context_lengths(inp)
    if upto is not None:
        ctx = np.minimum(ctx, upto)
    pool = A.ModelPool(len(inp.free_order), B, inp.free_order)
    tables, lens = [[] for _ in range(S)], [0] * S
    kp = np.zeros((len(inp.free_order), B, w.num_kv_heads, w.head_dim),
                  dtype=np.float32)
    vp = np.zeros_like(kp)
    wanted = set(int(s) for s in seqs)
    P = int(inp.prefix_rows)

    def write(s, first, count, store):
        n_new = [0] * S
        n_new[s] = count
        st, slots, _ = A.append_tokens(pool, tables, lens, n_new, 1 << 30)
        assert st == A.OK
        if store and count:
            rows = W.logical_rows(inp, s)[first:first + count]
            O.scatter_rows(kp, inp.k[rows].float().numpy(), slots)
            O.scatter_rows(vp, inp.v[rows].float().numpy(), slots)

    if P:
        write(0, 0, P, True)
        nb = O.blocks_needed(P, B)
        for s in range(1, S):
            assert pool.share(tables[0][:nb]) == A.OK
            tables[s] = list(tables[0][:nb])
            lens[s] = P
    for s in range(S):
        write(s, lens[s], int(ctx[s]) - lens[s], s in wanted)
    return tables, lens, kp, vp


def oracle_decode_rate(inp, seqs, budget_s: float):
    """The oracle's paged decode (gather through the table, bf16 -> fp64,
    attention) of the sequences `seqs`, cycled until `budget_s` has passed;
    GB/s of the K/V, q, o and table bytes it reads (a shared prefix counts
    once per sequence: the oracle has no sharing)."""
    from oracle import attention as O
    w = inp.workload
    tables, lens, kp, vp = _oracle_pool(inp, seqs)
    q = inp.q.float().numpy()
    scale = 1.0 / float(np.sqrt(w.head_dim))
    esize = 4 if w.dtype == "f32" else 2
    done, nbytes = 0, 0
    with _one_thread():
        t0 = time.perf_counter()
        while True:
            s = int(seqs[done % len(seqs)])
            O.decode_paged(q, kp, vp, tables, lens, scale, seqs=[s])
            nbytes += decode_bytes(np.array([lens[s]]), w.num_q_heads,
                                   w.num_kv_heads, w.head_dim, w.block_size,
                                   True, esize=esize)
            done += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        dt = time.perf_counter() - t0
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s",
            "cores": 1, "kind": "oracle",
            "sample": f"{done} sequence decodes over sequences "
                      f"{sorted(set(int(x) for x in seqs))[:8]}"
                      f"{'...' if len(set(seqs)) > 8 else ''} of the "
                      f"{w.name} batch, {dt:.1f} s of fp64 oracle time on one "
                      f"thread (gather through the table, bf16->fp64, "
                      f"attention)",
            "nproc": os.cpu_count(), "cpu_model": _cpu_model()}


def oracle_prefill_rate(inp, budget_s: float):
    """The oracle's chunked prefill of sampled query rows of the last chunk
    of sequence 0 (the heaviest rows: each sees up to 32768 keys), one call
    per row, cycled until `budget_s` has passed; GFLOP/s of the rows'
    algorithmic work (4 d Hq per visible key). The time covers the
    oracle's gather of the sequence's K/V through the table and its
    attention."""
    from oracle import attention as O
    w = inp.workload
    C = w.chunk
    N = int(inp.lengths[0])
    tables, lens, kp, vp = _oracle_pool(inp, [0])
    c0 = N - C
    rows_all = np.arange(c0, N)
    sample = rows_all[np.linspace(0, C - 1, 8).astype(int)]
    q = inp.q[int(inp.cu[0]) + c0:int(inp.cu[0]) + N].float().numpy()
    scale = 1.0 / float(np.sqrt(w.head_dim))
    cu = [0, C]
    done, flops = 0, 0.0
    with _one_thread():
        t0 = time.perf_counter()
        while True:
            p = int(sample[done % len(sample)])
            O.prefill_paged(q, cu, [c0], kp, vp, tables[:1], [N], scale,
                            True, rows=[p - c0])
            flops += 4.0 * w.head_dim * w.num_q_heads * (p + 1)
            done += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e9, 4), "unit": "GFLOP/s",
            "cores": 1, "kind": "oracle",
            "sample": f"{done} query rows (all 32 heads) at positions "
                      f"{c0}..{N - 1} of sequence 0's last chunk, one oracle "
                      f"call each, {dt:.1f} s of fp64 oracle time on one "
                      f"thread (gather of the sequence's K/V through the "
                      f"table, bf16->fp64, causal attention); the whole "
                      f"pass is {35.185:.3f} TFLOP",
            "nproc": os.cpu_count(), "cpu_model": _cpu_model()}


# ---------------------------------------------------------------------------
# Records
# ---------------------------------------------------------------------------
def roofline_record(bound: str, achieved: float, peak: float, unit: str,
                    traffic=None, **extra) -> dict:
    r = {"bound": bound, "achieved": round(achieved, 1), "peak": peak,
         "unit": unit, "frac": round(achieved / peak, 4), "traffic": traffic}
    r.update(extra)
    return r


DECODE_KERNEL = "paged_attn_decode (decode_sk_kernel + decode_combine_kernel)"
FUSED_KERNEL = ("paged_attn_decode_append (decode_sk_kernel + "
                "decode_combine_kernel, the step's append fused)")
SHARED_KERNEL = ("paged_attn_decode_shared_prefix (prefill_pp_kernel<true,"
                 "true> + decode_sk_kernel + decode_combine_kernel)")


def decode_roofline(res: dict, kernel: str, traffic=None) -> dict:
    return roofline_record(
        "hbm", res["decode_op_GBps"], HBM_PEAK_GBPS, "GB/s", traffic,
        kernel=kernel, bytes_per_launch=int(res["op_bytes_per_step"]),
        ms_per_launch=round(res["decode_op_ms_mean"], 4))


PROBE_LIB = os.path.join(ROOT, "paged_kv_cache_191_amd", "libkvprobe.so")
_probe = None


def probe_lib():
    """libkvprobe.so: the plain streaming-read kernel (measurement only)."""
    global _probe
    if _probe is None:
        import ctypes
        from paged_kv_cache_191_amd import kvpaged as kv
        if not os.path.exists(PROBE_LIB):
            raise RuntimeError(f"{PROBE_LIB} is not built: run "
                               "__graft_entry__.build()")
        lib = kv.load_native(PROBE_LIB)
        lib.kvprobe_threads.restype = ctypes.c_int
        lib.kvprobe_threads.argtypes = []
        lib.kvprobe_stream_read.restype = ctypes.c_int
        lib.kvprobe_stream_read.argtypes = [
            ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
            ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
        _probe = lib
    return _probe


def plain_read(nbytes: int, device, reps: int = 20,
               per_cu=(1, 2, 3, 4)) -> dict:
    """The read rate a plain streaming kernel reaches for ``nbytes`` bytes on
    this GPU: libkvprobe's kernel (each workgroup one contiguous range, 16-B
    non-temporal loads, 8 in flight per lane), best median over 1-4
    workgroups per CU. Two buffers alternate, as the decode's replicas do,
    so that no read finds its bytes in the last-level cache; they are
    written before they are timed, as the caches are."""
    settle(device)
    import torch
    lib = probe_lib()
    nb = int(nbytes) // 16 * 16
    cus = torch.cuda.get_device_properties(device).multi_processor_count
    sink = torch.empty(max(per_cu) * cus * lib.kvprobe_threads(),
                       dtype=torch.int32, device=device)
    bufs = [torch.ones(nb, dtype=torch.uint8, device=device)
            for _ in range(2)]
    stream = torch.cuda.current_stream(device)
    warm = 3
    best = None
    for k in per_cu:
        evs = []
        for r in range(warm + reps):
            e0 = HipEvent(enable_timing=True)
            e1 = HipEvent(enable_timing=True)
            e0.record()
            rc = lib.kvprobe_stream_read(
                bufs[r % 2].data_ptr(), nb, sink.data_ptr(),
                sink.numel() * 4, k * cus, stream.cuda_stream)
            e1.record()
            if rc != 0:
                raise RuntimeError(f"kvprobe_stream_read returned {rc}")
            evs.append((e0, e1))
        torch.cuda.synchronize()
        med = float(np.median([a.elapsed_time(b) for a, b in evs[warm:]]))
        if best is None or med < best[0]:
            best = (med, k)
    del bufs, sink
    return {"bytes": nb, "us": round(best[0] * 1e3, 3),
            "GBps": round(nb / (best[0] * 1e-3) / 1e9, 1),
            "workgroups_per_cu": best[1]}


def add_read_ceilings(rl: dict, device) -> dict:
    """Times a plain read of each decode record's algorithmic bytes and adds
    it to the record: ``plain_read_GBps`` and the record's rate as a
    fraction of it (``frac_of_plain_read``)."""
    seen = {}
    for rec in rl.values():
        nb = rec.get("bytes_per_launch")
        if rec.get("bound") != "hbm" or not nb:
            continue
        key = round(nb / 2**20)  # layouts whose bytes differ by < 1 MiB
        if key not in seen:
            seen[key] = plain_read(nb, device)
        pr = seen[key]
        rec["plain_read_GBps"] = pr["GBps"]
        rec["frac_of_plain_read"] = round(rec["achieved"] / pr["GBps"], 4)
    return {str(v["bytes"]): v for v in seen.values()}


def overhead(t_paged: float, t_contig: float) -> float:
    return round(t_paged / t_contig - 1.0, 4)


def nested_round(d):
    if isinstance(d, dict):
        return {k: nested_round(v) for k, v in d.items()}
    if isinstance(d, float):
        return round(d, 4)
    return d


CTX_DESC = {"llama3_8b_decode": "U{512..4096}",
            "yi34b_long_decode": "196608",
            "prefix_share_decode": "4096 shared + U{64..1024}"}
LMAX_RESERVED = {"llama3_8b_decode": 4096, "yi34b_long_decode": 196608,
                 "prefix_share_decode": 4096 + 1024}


def bench_decode_config(name: str, args, device) -> dict:
    """Every layout of one decode workload, with its rooflines, the
    paged-vs-contiguous overhead and the oracle's rate."""
    from paged_kv_cache_191_amd import kvpaged as kv
    from paged_kv_cache_191_amd import workloads as W
    wd = W.WORKLOADS[name]
    headroom = wd.num_seqs * (-(-decode_steps_total(args.steps, args.warmup)
                                // wd.block_size) + 1)
    log(f"{name}: drawing")
    inp = W.draw(wd, lambda L: pool_blocks(kv, wd, L, headroom))
    runs = {}
    prefix = wd.kind == "prefix"
    if not prefix:
        # The headline form runs first. Every leg starts with settle(): a
        # leg timed right after another one had released its caches (the
        # contiguous leg's 4.4 GB) measured up to 4% slower.
        log(f"{name}: paged decode steps, append fused into the decode op")
        runs["paged_fused"] = run_decode(inp, True, args.steps, args.warmup,
                                         args.replicas, device, fused=True)
    log(f"{name}: paged decode steps")
    runs["paged"] = run_decode(inp, True, args.steps, args.warmup,
                               args.replicas, device, shared_op=prefix)
    if prefix:
        log(f"{name}: paged decode steps without prefix sharing")
        runs["paged_without_sharing"] = run_decode(
            inp, True, args.steps, args.warmup, args.replicas, device)
    if not args.no_contig:
        log(f"{name}: contiguous decode steps")
        runs["contig"] = run_decode(inp, False, args.steps, args.warmup,
                                    args.replicas, device)
        if not args.no_vmm and not prefix:
            log(f"{name}: contiguous decode steps on demand-mapped memory")
            ctx = W.context_lengths(inp)
            pt = args.vmm_page_tokens
            while args.replicas * 2 * wd.num_kv_heads * int(
                    np.sum(-(-(ctx + args.steps + args.warmup) // pt))) \
                    > VMM_MAX_PAGES:
                pt *= 2
            try:
                runs["contig_demand_mapped"] = run_decode(
                    inp, False, args.steps, args.warmup, args.replicas,
                    device, vmm_page_tokens=pt)
            except kv.KVError as e:
                log(f"demand-mapped decode failed: {e}")
                runs["contig_demand_mapped"] = {"error": str(e)}
    if not args.no_fp8 and not prefix:
        log(f"{name}: paged decode steps over fp8 caches (per-head scales)")
        runs["paged_fp8"] = run_decode(inp, True, args.steps, args.warmup,
                                       args.replicas, device, fp8=True)
        log(f"{name}: the same, append fused into the fp8 decode op")
        runs["paged_fp8_fused"] = run_decode(
            inp, True, args.steps, args.warmup, args.replicas, device,
            fp8=True, fused=True)
    cow = None
    if prefix and not args.no_cow:
        log(f"{name}: copy-on-write step")
        cow = run_cow(wd, args.steps, args.warmup, device)

    paged = runs["paged"]
    rl = {name: decode_roofline(paged, SHARED_KERNEL if prefix else
                                DECODE_KERNEL, recorded_traffic(name))}
    if "paged_without_sharing" in runs:
        rl[name + "_without_sharing"] = decode_roofline(
            runs["paged_without_sharing"], DECODE_KERNEL)
    if "contig" in runs:
        rl[name + "_contig"] = decode_roofline(
            runs["contig"], "contig_attn_decode (decode_sk_kernel + "
            "decode_combine_kernel)")
    vm = runs.get("contig_demand_mapped")
    if vm and "error" not in vm:
        rl[name + "_contig_demand_mapped"] = decode_roofline(
            vm, "contig_attn_decode on demand-mapped memory")
    if "paged_fused" in runs:
        rl[name + "_fused"] = decode_roofline(
            runs["paged_fused"], FUSED_KERNEL,
            recorded_traffic(name, fused=True))
    if "paged_fp8" in runs:
        rl[name + "_fp8"] = decode_roofline(
            runs["paged_fp8"], "paged_attn_decode_fp8_per_head "
            "(decode_sk_kernel<true,true,false> + decode_combine_kernel)",
            recorded_traffic(name, fp8=True))
    if "paged_fp8_fused" in runs:
        rl[name + "_fp8_fused"] = decode_roofline(
            runs["paged_fp8_fused"], "paged_attn_decode_append_fp8_per_head "
            "(decode_sk_kernel<true,true,true> + decode_combine_kernel)",
            recorded_traffic(name, fp8=True, fused=True))
    if prefix:
        # headline bytes: the shared prefix once (unique); the plain decode
        # reads it once per sequence, mostly from cache
        rl[name]["bytes"] = "unique"
        rl[name + "_without_sharing"]["bytes"] = "unique"
        if name + "_contig" in rl:
            rl[name + "_contig"]["bytes"] = "logical (prefix per sequence)"
    if cow:
        rl["copy_blocks_cow"] = roofline_record(
            "hbm", cow["copy_blocks_GBps"], HBM_PEAK_GBPS, "GB/s",
            kernel="kv_copy_blocks (copy_blocks_kernel)",
            us_per_launch=round(cow["copy_blocks_us_median"], 3),
            blocks=cow["cow_copies"])
    ovh = {}
    if "contig" in runs:
        ovh[name] = overhead(paged["decode_op_ms_mean"],
                             runs["contig"]["decode_op_ms_mean"])
        if prefix:
            ovh[name + "_without_sharing"] = overhead(
                runs["paged_without_sharing"]["decode_op_ms_mean"],
                runs["contig"]["decode_op_ms_mean"])
    if vm and "error" not in vm:
        ovh[name + "_vs_demand_mapped"] = overhead(
            paged["decode_op_ms_mean"], vm["decode_op_ms_mean"])
    ceilings = None
    if not args.no_read_ceiling:
        log(f"{name}: plain reads of the same byte counts")
        ceilings = add_read_ceilings(rl, device)
    out = {"inp": inp, "runs": runs, "rooflines": rl, "overhead": ovh,
           "cow": cow, "memory": memory_waste(inp, LMAX_RESERVED[name]),
           "read_ceiling": ceilings}
    if "paged_fp8" in runs:
        out["fp8_speedup_vs_bf16"] = round(
            paged["decode_op_ms_mean"] /
            runs["paged_fp8"]["decode_op_ms_mean"], 4)
    return out


def bench_prefill(args, device) -> dict:
    from paged_kv_cache_191_amd import kvpaged as kv
    from paged_kv_cache_191_amd import workloads as W
    layouts = {}
    wanted = args.prefill_layouts.split(",")
    pin16 = None
    for name, layout in (("yi6b_chunked_prefill_b16", "paged_b16"),
                         ("yi6b_chunked_prefill_b64", "paged_b64"),
                         ("yi6b_chunked_prefill_b16", "contig"),
                         ("yi6b_chunked_prefill_b16", "contig_vmm")):
        if layout not in wanted:
            continue
        wp = W.WORKLOADS[name]
        log(f"prefill {layout}")
        pin = W.draw(wp, lambda L: pool_blocks(kv, wp, L))
        if layout == "paged_b16":
            pin16 = pin
        r = prefill_pass(pin, {"contig": "contig", "contig_vmm": "vattn"}
                         .get(layout, "paged"), device)
        r["frac_of_peak"] = r["TFLOPs"] / MFMA_BF16_PEAK_TFLOPS
        layouts[layout] = r
    kernels = {"paged_b16": "paged_attn_prefill (prefill_pp_kernel<true,"
                            "false,true>)",
               "paged_b64": "paged_attn_prefill (prefill_pp_kernel<true,"
                            "false,true>)",
               "contig": "contig_attn_prefill (prefill_pp_kernel<false,"
                         "false,false>)",
               "contig_vmm": "contig_attn_prefill on demand-mapped memory"}
    rl, ovh = {}, {}
    for lay, r in layouts.items():
        rl["yi6b_chunked_prefill_" + lay] = roofline_record(
            "mfma", r["TFLOPs"], MFMA_BF16_PEAK_TFLOPS, "TFLOP/s",
            recorded_traffic("yi6b_chunked_prefill_" + lay),
            kernel=kernels[lay], tflop_per_pass=round(r["tflop"], 4),
            ms_per_pass=round(r["attn_ms"], 4))
        # the chunk's cache write: 2 x (read + write) of the new rows
        rl["yi6b_reshape_and_cache_" + lay] = roofline_record(
            "hbm", r["reshape_and_cache_GBps"], HBM_PEAK_GBPS, "GB/s",
            kernel="kv_reshape_and_cache (scatter_rows_kernel)",
            us_per_launch=round(r["reshape_and_cache_us_median"], 3))
    if "contig" in layouts:
        for lay in ("paged_b16", "paged_b64", "contig_vmm"):
            if lay in layouts:
                ovh["yi6b_chunked_prefill_" + lay] = overhead(
                    layouts[lay]["attn_ms"], layouts["contig"]["attn_ms"])
    return {"layouts": layouts, "rooflines": rl, "overhead": ovh,
            "inp": pin16}


def calibration_copy(device) -> None:
    """One plain 1 GiB device copy: the reference kernel for hardware
    traffic counters."""
    import torch
    src = torch.ones(1 << 30, dtype=torch.uint8, device=device)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


ALL_CONFIGS = ("decode_tiny_f32", "llama3_8b_decode", "yi6b_chunked_prefill",
               "yi34b_long_decode", "prefix_share_decode", "block_swap")


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--configs", default=",".join(ALL_CONFIGS),
                    help="configurations to run (default: all)")
    ap.add_argument("--workload", default=None, choices=DECODE_WORKLOADS,
                    help="run this decode workload only (no prefill, no "
                         "other configuration); for profiling")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode configurations (prefill / "
                         "profiling runs); no bench line is printed")
    ap.add_argument("--prefill-layouts",
                    default="paged_b16,paged_b64,contig,contig_vmm")
    ap.add_argument("--no-contig", action="store_true")
    ap.add_argument("--no-vmm", action="store_true",
                    help="skip the contiguous decode on demand-mapped memory")
    ap.add_argument("--vmm-page-tokens", type=int, default=1024,
                    help="page of the demand-mapped cache, in tokens of one "
                         "head (1024 x 128 bf16 values = 256 KiB; one "
                         "allocation per page, and a process holds some "
                         "tens of thousands at most)")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the paged decode over fp8 E4M3 caches")
    ap.add_argument("--no-cow", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-headline", type=float, default=10.0,
                    help="seconds of oracle time for the headline workload "
                         "(the cpu_baseline record)")
    ap.add_argument("--cpu-budget", type=float, default=4.0,
                    help="seconds of oracle time per configuration")
    ap.add_argument("--no-read-ceiling", action="store_true",
                    help="skip the plain streaming reads of each decode "
                         "record's byte count")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="also run one plain 1 GiB device copy (reference "
                         "kernel for hardware traffic counters)")
    args = ap.parse_args()
    global VMM_PREFILL_PAGE_TOKENS
    VMM_PREFILL_PAGE_TOKENS = args.vmm_page_tokens
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not "
              "supported (decode and prefill shard by sequence or head with "
              "no exchange; the multi-GPU path is not built)",
              file=sys.stderr)
        return 2

    import torch
    from paged_kv_cache_191_amd import kvpaged as kv
    kv.lib()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    device = torch.device("cuda:0")
    if args.calibration_copy:
        calibration_copy(device)

    configs = [c for c in args.configs.split(",") if c]
    if args.workload:
        configs = [args.workload]
    if args.no_prefill:
        configs = [c for c in configs if c != "yi6b_chunked_prefill"]
    if args.no_decode:
        configs = [c for c in configs if c == "yi6b_chunked_prefill"]
    unknown = set(configs) - set(ALL_CONFIGS)
    if unknown:
        print(f"unknown configurations {sorted(unknown)}", file=sys.stderr)
        return 2
    cpu = not args.no_cpu_baseline

    t_start = time.perf_counter()
    rooflines, ovh, cpu_oracle, details = {}, {}, {}, {}
    decoded = {}
    prefill = None
    for name in configs:
        if name == "decode_tiny_f32":
            log("small fp32 decode (latency)")
            tiny = run_tiny_decode(device)
            tiny["note"] = ("generic path, latency-bound: no roofline "
                            "claim")
            details[name] = nested_round(tiny)
            if cpu:
                from paged_kv_cache_191_amd import workloads as W
                wt = W.WORKLOADS[name]
                it = W.draw(wt, lambda L: pool_blocks(kv, wt, L))
                cpu_oracle[name] = oracle_decode_rate(
                    it, list(range(wt.num_seqs)), min(args.cpu_budget, 2.0))
        elif name == "yi6b_chunked_prefill":
            prefill = bench_prefill(args, device)
            rooflines.update(prefill["rooflines"])
            ovh.update(prefill["overhead"])
            details[name] = {k: nested_round(v) for k, v in
                             prefill["layouts"].items()}
            if cpu and prefill["inp"] is not None:
                log("prefill: oracle on sampled rows")
                cpu_oracle[name] = oracle_prefill_rate(prefill["inp"],
                                                       args.cpu_budget)
            prefill["inp"] = None
        elif name == "block_swap":
            from paged_kv_cache_191_amd import workloads as W
            log("block swap to pinned host memory and back")
            details[name] = run_swap(W.WORKLOADS["llama3_8b_decode"], device)
        else:
            r = bench_decode_config(name, args, device)
            decoded[name] = r
            rooflines.update(r["rooflines"])
            ovh.update(r["overhead"])
            d = {k: nested_round(v) for k, v in r["runs"].items()}
            d["cache_write_note"] = (
                "cache_write_* fields: the step's append kernel, a few "
                "hundred KB per launch: latency-bound, no roofline claim")
            d["memory"] = r["memory"]
            if r["cow"]:
                d["copy_on_write"] = nested_round(r["cow"])
            if "fp8_speedup_vs_bf16" in r:
                d["fp8_speedup_vs_bf16"] = r["fp8_speedup_vs_bf16"]
            if r["read_ceiling"]:
                d["plain_read"] = r["read_ceiling"]
            details[name] = d
            if cpu:
                w = r["inp"].workload
                log(f"{name}: oracle on a sample")
                if name == "yi34b_long_decode":
                    seqs = [0]
                elif name == "prefix_share_decode":
                    seqs = list(range(0, w.num_seqs, 37))
                else:
                    seqs = list(range(w.num_seqs))
                budget = (args.cpu_budget_headline
                          if name == "llama3_8b_decode" else args.cpu_budget)
                cpu_oracle[name] = oracle_decode_rate(r["inp"], seqs, budget)
            r["inp"] = None
    log(f"all configurations done in {time.perf_counter() - t_start:.1f} s")

    if not decoded:
        log(f"no decode configuration: no bench line. prefill: "
            f"{json.dumps(nested_round(details.get('yi6b_chunked_prefill')))}")
        return 0
    head = "llama3_8b_decode" if "llama3_8b_decode" in decoded else \
        next(iter(decoded))
    runs_h = decoded[head]["runs"]
    fused_h = "paged_fused" in runs_h
    hp = runs_h["paged_fused"] if fused_h else runs_h["paged"]
    wd = __import__("paged_kv_cache_191_amd.workloads",
                    fromlist=["WORKLOADS"]).WORKLOADS[head]
    line = {
        "metric": METRIC,
        "value": round(hp["step_GBps"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(hp["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": wd.name,
            "num_seqs": wd.num_seqs, "num_q_heads": wd.num_q_heads,
            "num_kv_heads": wd.num_kv_heads, "head_dim": wd.head_dim,
            "block_size": wd.block_size, "context": CTX_DESC[wd.name],
            "step": ("append+paged_attn_decode_append" if fused_h else
                     "append+kv_append_token+" + (
                         "paged_attn_decode_shared_prefix"
                         if wd.kind == "prefix" else "paged_attn_decode")),
            "replicas": args.replicas,
            "configs_run": configs,
        },
        "roofline": rooflines[head + "_fused" if fused_h else head],
    }
    if prefill and "paged_b16" in prefill["layouts"]:
        p16 = dict(rooflines["yi6b_chunked_prefill_paged_b16"])
        p16["overhead_vs_contig"] = ovh.get(
            "yi6b_chunked_prefill_paged_b16")
        p16["layouts"] = {
            lay: {"TFLOPs": round(r["TFLOPs"], 1),
                  "frac": round(r["frac_of_peak"], 4),
                  "attn_ms": round(r["attn_ms"], 4),
                  "overhead_vs_contig": ovh.get(
                      "yi6b_chunked_prefill_" + lay)}
            for lay, r in prefill["layouts"].items()}
        line["prefill"] = p16
    line["rooflines"] = rooflines
    line["paged_vs_contig_overhead"] = ovh
    line["cpu_oracle"] = cpu_oracle
    line["configs"] = details
    line["cpu_baseline"] = cpu_oracle.get(head)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
