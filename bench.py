"""Benchmark of the paged-KV hot path on one MI355X.

A step is one decode step of the Llama-3-8B-shaped batch (64 sequences,
32 query / 8 KV heads, head_dim 128, bf16, block size 16, contexts uniform in
512..4096, Q/K/V ~ N(0, 1)):
  host   kv_seq_append: allocation when a block fills, slot mapping;
  upload one pinned host->device copy of slots, lengths and block table;
  device kv_reshape_and_cache of the new token's K/V, paged_attn_decode
         (partitions + exact merge).
Each sequence grows by one token per step. Four independent replicas of the
whole batch (pools, tables, queries) rotate so that no step finds its K/V in
the 256 MB last-level cache.

`value` = decode algorithmic bytes (K+V once per KV head, q, o, block table,
lengths) summed over the timed steps / wall time of those steps.
The same JSON line carries:
  roofline     - the decode op alone (HIP events around each call on its
                 stream) against 8 TB/s;
  contig       - the same steps on the contiguous layout, and the
                 paged-vs-contiguous overhead of the decode op;
  prefill      - one chunked-prefill pass of the Yi-6B-shaped workload (4 x
                 32768 tokens, 2048-token chunks, 32/4 heads) per layout
                 (paged B=16, paged B=64, contiguous): TFLOP/s of the
                 attention calls against 2.5 PFLOP/s bf16;
  cpu_baseline - the fp64 oracle on this host's cores on the same decode
                 workload.
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


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def decode_bytes(lens: np.ndarray, hq: int, hkv: int, d: int, B: int,
                 paged: bool, esize: int = 2) -> int:
    """Algorithmic bytes of one decode call: K and V of every context token
    once per KV head, q and o, the block-table entries in use, lengths."""
    kvb = int(lens.sum()) * hkv * d * 2 * esize
    qo = 2 * len(lens) * hq * d * esize
    table = int(sum(-(-int(n) // B) for n in lens)) * 4 if paged else 0
    return kvb + qo + table + 4 * len(lens)


class DecodeReplica:
    """One independent copy of the decode batch, paged or contiguous."""

    def __init__(self, inp, new_k, new_v, paged: bool, steps: int, device):
        import torch
        from paged_kv_cache_191_amd import kvpaged as kv
        self.kv = kv
        self.torch = torch
        w = inp.workload
        self.w = w
        self.paged = paged
        S, B = w.num_seqs, w.block_size
        ctx = inp.lengths.astype(np.int64)
        self.lmax = int(ctx.max()) + steps + 1
        self.cap = -(-self.lmax // B)
        n_pool = len(inp.free_order)
        # pinned host staging: [slots int64 S | lens int32 S | table int32 S*cap]
        nbytes = 8 * S + 4 * S + 4 * S * self.cap
        self.h_buf = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
        self.d_buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        hb = self.h_buf.numpy()
        self.h_slots = hb[:8 * S].view(np.int64)
        self.h_lens = hb[8 * S:12 * S].view(np.int32)
        self.h_table = hb[12 * S:].view(np.int32).reshape(S, self.cap)
        self.d_slots = self.d_buf[:8 * S].view(torch.int64)
        self.d_lens = self.d_buf[8 * S:12 * S].view(torch.int32)
        self.d_table = self.d_buf[12 * S:].view(torch.int32).view(S, self.cap)
        self.q = inp.q.to(device)
        self.out = torch.empty_like(self.q)
        self.new_k, self.new_v = new_k, new_v
        tdt = inp.k.dtype
        self.h_table[:] = -1
        self.h_lens[:] = 0
        if paged:
            self.pool = kv.KVPool(n_pool, B, inp.free_order)
            self.k = torch.empty((n_pool, w.num_kv_heads, B, w.head_dim),
                                 dtype=tdt, device=device)
            self.v = torch.empty_like(self.k)
            # contexts minus the newest token, written through the product
            # path (append + cache write), one sequence at a time
            for s in range(S):
                n_new = np.zeros(S, dtype=np.int32)
                n_new[s] = int(ctx[s]) - 1
                slots, _ = self.pool.seq_append(self.h_table, self.h_lens,
                                                n_new)
                rows = torch.arange(int(inp.cu[s]), int(inp.cu[s + 1]) - 1)
                kv.kv_reshape_and_cache(inp.k[rows].to(device),
                                        inp.v[rows].to(device),
                                        torch.from_numpy(slots).to(device),
                                        self.k, self.v)
        else:
            self.k = torch.empty((S, w.num_kv_heads, self.lmax, w.head_dim),
                                 dtype=tdt, device=device)
            self.v = torch.empty_like(self.k)
            for s in range(S):
                n = int(ctx[s]) - 1
                rows = slice(int(inp.cu[s]), int(inp.cu[s]) + n)
                self.k[s, :, :n] = inp.k[rows].to(device).transpose(0, 1)
                self.v[s, :, :n] = inp.v[rows].to(device).transpose(0, 1)
                self.h_lens[s] = n
        self.ws = kv.decode_workspace(S, w.num_q_heads, w.num_kv_heads,
                                      w.head_dim, self.lmax, device)
        # the staging buffer is rewritten only after its last upload is done
        self.uploaded = torch.cuda.Event()
        self.uploaded.record()
        self.scale = 1.0 / float(np.sqrt(w.head_dim))
        torch.cuda.synchronize()

    def host_append(self) -> None:
        """Host part of a step: allocation and slot mapping (paged), or the
        contiguous slot s * Lmax + position."""
        self.uploaded.synchronize()
        if self.paged:
            slots, pairs = self.pool.seq_append(self.h_table, self.h_lens)
            assert len(pairs) == 0
            self.h_slots[:] = slots
        else:
            S = self.w.num_seqs
            self.h_slots[:] = np.arange(S, dtype=np.int64) * self.lmax + \
                self.h_lens
            self.h_lens += 1

    def device_step(self, ev=None) -> None:
        kv = self.kv
        self.d_buf.copy_(self.h_buf, non_blocking=True)
        self.uploaded.record()
        kv.kv_reshape_and_cache(self.new_k, self.new_v, self.d_slots, self.k,
                                self.v)
        max_ctx = int(self.h_lens.max())
        if ev is not None:
            ev[0].record()
        if self.paged:
            kv.paged_attn_decode(self.out, self.q, self.k, self.v,
                                 self.d_table, self.d_lens, max_ctx,
                                 self.scale, self.ws)
        else:
            kv.contig_attn_decode(self.out, self.q, self.k, self.v,
                                  self.d_lens, max_ctx, self.scale, self.ws)
        if ev is not None:
            ev[1].record()


def run_decode(inp, paged: bool, steps: int, warmup: int, reps: int,
               device):
    import torch
    w = inp.workload
    g = np.random.default_rng([w.seed, 50])
    shape = (w.num_seqs, w.num_kv_heads, w.head_dim)
    new_k = torch.from_numpy(g.standard_normal(shape, dtype=np.float32)).to(
        torch.bfloat16).to(device)
    new_v = torch.from_numpy(g.standard_normal(shape, dtype=np.float32)).to(
        torch.bfloat16).to(device)
    reps_ = [DecodeReplica(inp, new_k, new_v, paged, steps + warmup, device)
             for _ in range(reps)]
    for i in range(warmup):
        r = reps_[i % reps]
        r.host_append()
        r.device_step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True),
            torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    total_bytes = 0
    t0 = time.perf_counter()
    for i in range(steps):
        r = reps_[i % reps]
        r.host_append()
        total_bytes += decode_bytes(r.h_lens, w.num_q_heads, w.num_kv_heads,
                                    w.head_dim, w.block_size, paged)
        r.device_step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    op_ms = [a.elapsed_time(b) for a, b in evs]
    res = {
        "wall_s": wall,
        "ms_per_step": 1e3 * wall / steps,
        "step_GBps": total_bytes / wall / 1e9,
        "decode_op_ms_mean": float(np.mean(op_ms)),
        "decode_op_ms_p10": float(np.percentile(op_ms, 10)),
        "decode_op_ms_p90": float(np.percentile(op_ms, 90)),
        "bytes_per_step": total_bytes / steps,
    }
    res["decode_op_GBps"] = res["bytes_per_step"] / (
        res["decode_op_ms_mean"] * 1e-3) / 1e9
    del reps_
    torch.cuda.empty_cache()
    return res


def prefill_pass(inp, layout: str, device):
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
    if layout == "contig":
        kc = torch.empty((S, w.num_kv_heads, N, w.head_dim), dtype=tdt,
                         device=device)
        vc = torch.empty_like(kc)
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
            if layout != "contig" else None
        table = np.full((S, cap), -1, dtype=np.int32)
        lens = np.zeros(S, dtype=np.int32)
        for c0 in range(0, N, C):
            n_new = np.full(S, C, dtype=np.int32)
            if pool is not None:
                slots, _ = pool.seq_append(table, lens, n_new)
            else:
                slots = (np.arange(S)[:, None] * N + lens[:, None] +
                         np.arange(C)[None, :]).reshape(-1).astype(np.int64)
                lens += C
            rows = (np.arange(S)[:, None] * N + c0 +
                    np.arange(C)[None, :]).reshape(-1)
            rows_d = torch.from_numpy(rows).to(device)
            kv.kv_reshape_and_cache(k_dev[rows_d], v_dev[rows_d],
                                    torch.from_numpy(slots).to(device), kc, vc)
            cu = torch.arange(0, S * C + 1, C, dtype=torch.int32,
                              device=device)
            start = torch.full((S,), c0, dtype=torch.int32, device=device)
            ctx = torch.from_numpy(lens.copy()).to(device)
            q = q_dev[rows_d]
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            if layout == "contig":
                kv.contig_attn_prefill(out, q, cu, start, C, kc, vc, ctx,
                                       scale, True)
            else:
                kv.paged_attn_prefill(out, q, cu, start, C, kc, vc,
                                      torch.from_numpy(table).to(device), ctx,
                                      scale, True)
            e1.record()
            if timed:
                times.append((e0, e1))
                # unmasked causal pairs of this chunk, 4*d*Hq flops each
                pairs = S * (C * c0 + C * (C + 1) // 2)
                flops_total += 4.0 * w.head_dim * w.num_q_heads * pairs
        torch.cuda.synchronize()

    one_pass(False)
    t0 = time.perf_counter()
    one_pass(True)
    wall = time.perf_counter() - t0
    attn_ms = sum(a.elapsed_time(b) for a, b in times)
    del kc, vc, q_dev, k_dev, v_dev, out
    torch.cuda.empty_cache()
    return {"attn_ms": attn_ms, "pass_wall_ms": 1e3 * wall,
            "TFLOPs": flops_total / (attn_ms * 1e-3) / 1e12,
            "tflop": flops_total / 1e12}


def cpu_baseline(inp, budget_s: float = 12.0):
    """The fp64 oracle (as it stands) on this host: paged decode of the
    same workload, gather + conversion + attention timed, pool build not."""
    from oracle import allocator as A
    from oracle import attention as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] +
                      [1])
    except Exception:
        threads = 1
    w = inp.workload
    B = w.block_size
    S = w.num_seqs
    pool = A.ModelPool(len(inp.free_order), B, inp.free_order)
    tables, lens = [[] for _ in range(S)], [0] * S
    st, slots, _ = A.append_tokens(pool, tables, lens, inp.lengths.tolist(),
                                   1 << 30)
    kp = np.zeros((len(inp.free_order), B, w.num_kv_heads, w.head_dim),
                  dtype=np.float32)
    vp = np.zeros_like(kp)
    O.scatter_rows(kp, inp.k.float().numpy(), slots)
    O.scatter_rows(vp, inp.v.float().numpy(), slots)
    q = inp.q.float().numpy()
    scale = 1.0 / float(np.sqrt(w.head_dim))
    done, nbytes = 0, 0
    t0 = time.perf_counter()
    while True:
        s = done % S
        O.decode_paged(q, kp, vp, tables, lens, scale, seqs=[s])
        nbytes += decode_bytes(np.array([lens[s]]), w.num_q_heads,
                               w.num_kv_heads, w.head_dim, B, True)
        done += 1
        if time.perf_counter() - t0 >= budget_s and done >= S:
            break
    dt = time.perf_counter() - t0
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{done} sequence decodes of the {w.name} batch "
                      f"({done / S:.2f} passes), {dt:.1f} s of fp64 oracle "
                      f"time (gather through the table, bf16->fp64, "
                      f"attention)"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-contig", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not "
              "supported (decode and prefill shard by sequence or head with "
              "no exchange; the multi-GPU path is not built)",
              file=sys.stderr)
        return 2

    import torch
    from paged_kv_cache_191_amd import kvpaged as kv
    from paged_kv_cache_191_amd import workloads as W
    kv.lib()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    device = torch.device("cuda:0")

    wd = W.WORKLOADS["llama3_8b_decode"]
    headroom = wd.num_seqs * (-(-(args.steps + args.warmup) // wd.block_size)
                              + 1)
    log("drawing llama3_8b_decode")
    inp = W.draw(wd, lambda L: sum(kv.kv_blocks_needed(int(n), wd.block_size)
                                   for n in L) + headroom)
    log("paged decode steps")
    paged = run_decode(inp, True, args.steps, args.warmup, args.replicas,
                       device)
    contig = None
    if not args.no_contig:
        log("contiguous decode steps")
        contig = run_decode(inp, False, args.steps, args.warmup,
                            args.replicas, device)

    prefill = None
    if not args.no_prefill:
        prefill = {}
        for name, layout in (("yi6b_chunked_prefill_b16", "paged_b16"),
                             ("yi6b_chunked_prefill_b64", "paged_b64"),
                             ("yi6b_chunked_prefill_b16", "contig")):
            wp = W.WORKLOADS[name]
            log(f"prefill {layout}")
            pin = W.draw(wp, lambda L: sum(
                kv.kv_blocks_needed(int(n), wp.block_size) for n in L))
            r = prefill_pass(pin, "contig" if layout == "contig" else "paged",
                             device)
            r["frac_of_peak"] = r["TFLOPs"] / MFMA_BF16_PEAK_TFLOPS
            prefill[layout] = r
        for b in ("paged_b16", "paged_b64"):
            prefill[b]["overhead_vs_contig"] = (
                prefill[b]["attn_ms"] / prefill["contig"]["attn_ms"] - 1.0)

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (fp64 oracle)")
        cpu = cpu_baseline(inp, args.cpu_budget)

    achieved = paged["decode_op_GBps"]
    line = {
        "metric": METRIC,
        "value": round(paged["step_GBps"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(paged["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "llama3_8b_decode",
            "num_seqs": wd.num_seqs, "num_q_heads": wd.num_q_heads,
            "num_kv_heads": wd.num_kv_heads, "head_dim": wd.head_dim,
            "block_size": wd.block_size, "context": "U{512..4096}",
            "step": "append+upload+reshape_and_cache+paged_attn_decode",
            "replicas": args.replicas,
        },
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None,
            "kernel": "paged_attn_decode (decode_mfma_kernel + "
                      "decode_combine_kernel)",
            "bytes_per_launch": int(paged["bytes_per_step"]),
            "ms_per_launch": round(paged["decode_op_ms_mean"], 4),
        },
        "decode_paged": {k: round(v, 4) for k, v in paged.items()},
    }
    if contig:
        line["decode_contig"] = {k: round(v, 4) for k, v in contig.items()}
        line["decode_paged_vs_contig_overhead"] = round(
            paged["decode_op_ms_mean"] / contig["decode_op_ms_mean"] - 1.0, 4)
    if prefill:
        line["prefill"] = {k: {kk: round(vv, 4) for kk, vv in v.items()}
                           for k, v in prefill.items()}
    line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
