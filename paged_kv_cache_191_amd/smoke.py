"""One small invocation of the hot path on cuda:0, checked against the fp64
oracle: allocation and slot mapping through the native allocator, cache
write, paged decode (fp32 generic path and bf16 MFMA path), one decode step
through the device-side append (block table and lengths on the device) and
paged chunked prefill (bf16 MFMA path). Raises on any mismatch."""
from __future__ import annotations

import numpy as np
import torch

from . import kvpaged as kv
from . import workloads as W


def _fill(inp, B, cap, dev):
    w = inp.workload
    S = w.num_seqs
    pool = kv.KVPool(len(inp.free_order), B, inp.free_order)
    tables = np.full((S, cap), -1, dtype=np.int32)
    lens = np.zeros(S, dtype=np.int32)
    slots, pairs = pool.seq_append(tables, lens, inp.lengths.astype(np.int32))
    assert len(pairs) == 0
    tdt = W.torch_dtype(w.dtype)
    kc = torch.full((len(inp.free_order), w.num_kv_heads, B, w.head_dim),
                    float("nan"), dtype=tdt, device=dev)
    vc = torch.full_like(kc, float("nan"))
    kv.kv_reshape_and_cache(inp.k.to(dev), inp.v.to(dev),
                            torch.from_numpy(slots).to(dev), kc, vc)
    return pool, tables, lens, kc, vc


def run() -> None:
    from oracle import allocator as A
    from oracle import attention as O

    dev = torch.device("cuda:0")
    kv.lib()
    # --- decode, fp32 (pages' worked-example-sized config) and bf16 -------
    for w in (W.WORKLOADS["decode_tiny_f32"],
              W.WORKLOADS["llama3_8b_decode"].replace(
                  num_seqs=4, length_range=(1, 700), name="smoke_bf16")):
        B = w.block_size
        inp = W.draw(w, lambda L: O.pool_blocks_exact(L, B))
        S = w.num_seqs
        cap = max(1, -(-int(inp.lengths.max()) // B))
        pool, tables, lens, kc, vc = _fill(inp, B, cap, dev)
        mp = A.ModelPool(len(inp.free_order), B, inp.free_order)
        mt, ml = [[] for _ in range(S)], [0] * S
        st, mslots, _ = A.append_tokens(mp, mt, ml, inp.lengths.tolist(), cap)
        assert st == A.OK
        for s in range(S):
            if mt[s] != tables[s, :len(mt[s])].tolist():
                raise AssertionError("allocation differs from the oracle")
        n_pool = len(inp.free_order)
        kp = np.full((n_pool, B, w.num_kv_heads, w.head_dim), np.nan,
                     dtype=np.float32)
        vp = np.full_like(kp, np.nan)
        O.scatter_rows(kp, inp.k.float().numpy(), mslots)
        O.scatter_rows(vp, inp.v.float().numpy(), mslots)
        got = kc.permute(0, 2, 1, 3).float().cpu().numpy()
        if not np.array_equal(got, kp, equal_nan=True):
            raise AssertionError("cache write differs from the oracle")
        q = inp.q.to(dev)
        out = torch.empty_like(q)
        scale = 1.0 / float(np.sqrt(w.head_dim))
        kv.paged_attn_decode(out, q, kc, vc, torch.from_numpy(tables).to(dev),
                             torch.from_numpy(lens).to(dev),
                             int(lens.max()), scale)
        torch.cuda.synchronize()
        want = O.decode_paged(inp.q.float().numpy(), kp, vp, mt, ml, scale)
        err = float(np.abs(out.float().cpu().numpy() - want).max())
        tol = 1e-4 if w.dtype == "f32" else 2e-2
        print(f"smoke decode {w.name}: max-abs {err:.2e} (tol {tol})",
              flush=True)
        if not err <= tol:
            raise AssertionError(f"decode {w.name}: max-abs {err}")
    # --- one decode step through the device-side append (bf16) ------------
    w = W.WORKLOADS["llama3_8b_decode"].replace(
        num_seqs=4, length_range=(1, 700), name="smoke_step")
    B, S = w.block_size, w.num_seqs
    inp = W.draw(w, lambda L: O.pool_blocks_exact(L, B) + S)
    cap = max(1, -(-(int(inp.lengths.max()) + 1) // B))
    pool, tables, lens, kc, vc = _fill(inp, B, cap, dev)
    mp = A.ModelPool(len(inp.free_order), B, inp.free_order)
    mt, ml = [[] for _ in range(S)], [0] * S
    st, mslots, _ = A.append_tokens(mp, mt, ml, inp.lengths.tolist(), cap)
    kp = np.full((len(inp.free_order), B, w.num_kv_heads, w.head_dim),
                 np.nan, dtype=np.float32)
    vp = np.full_like(kp, np.nan)
    O.scatter_rows(kp, inp.k.float().numpy(), mslots)
    O.scatter_rows(vp, inp.v.float().numpy(), mslots)
    bt_d = torch.from_numpy(tables).to(dev)
    lens_d = torch.from_numpy(lens).to(dev)
    ar = np.arange(S)
    idx = lens // B
    before = tables[ar, idx].copy()
    _, pairs = pool.seq_append(tables, lens)        # one token each
    after = tables[ar, idx]
    new_blocks = torch.from_numpy(
        np.where(after != before, after, -1).astype(np.int32)).pin_memory()
    g = np.random.default_rng([w.seed, 77])
    shape = (S, w.num_kv_heads, w.head_dim)
    k_new = torch.from_numpy(g.standard_normal(shape, dtype=np.float32)).to(
        torch.bfloat16)
    v_new = torch.from_numpy(g.standard_normal(shape, dtype=np.float32)).to(
        torch.bfloat16)
    kv.kv_append_token(k_new.to(dev), v_new.to(dev), new_blocks, bt_d, lens_d,
                       kc, vc)
    q = inp.q.to(dev)
    out = torch.empty_like(q)
    scale = 1.0 / float(np.sqrt(w.head_dim))
    kv.paged_attn_decode(out, q, kc, vc, bt_d, lens_d, int(lens.max()), scale)
    torch.cuda.synchronize()
    st, mslots, _ = A.append_tokens(mp, mt, ml, [1] * S, cap)
    assert st == A.OK and len(pairs) == 0
    O.scatter_rows(kp, k_new.float().numpy(), mslots)
    O.scatter_rows(vp, v_new.float().numpy(), mslots)
    if lens_d.cpu().tolist() != ml or any(
            mt[s] != bt_d[s, :len(mt[s])].cpu().tolist() for s in range(S)):
        raise AssertionError("device table or lengths differ from the oracle")
    want = O.decode_paged(inp.q.float().numpy(), kp, vp, mt, ml, scale)
    err = float(np.abs(out.float().cpu().numpy() - want).max())
    print(f"smoke decode step (device append): max-abs {err:.2e} (tol 2e-2)",
          flush=True)
    if not err <= 2e-2:
        raise AssertionError(f"decode step: max-abs {err}")
    # --- chunked prefill, bf16 MFMA path -----------------------------------
    w = W.WORKLOADS["yi6b_chunked_prefill_b16"].replace(
        num_seqs=2, lengths=(200, 77), name="smoke_prefill")
    B = w.block_size
    inp = W.draw(w, lambda L: O.pool_blocks_exact(L, B))
    cap = max(1, -(-200 // B))
    pool, tables, lens, kc, vc = _fill(inp, B, cap, dev)
    mp = A.ModelPool(len(inp.free_order), B, inp.free_order)
    mt, ml = [[], []], [0, 0]
    st, mslots, _ = A.append_tokens(mp, mt, ml, inp.lengths.tolist(), cap)
    kp = np.full((len(inp.free_order), B, w.num_kv_heads, w.head_dim), np.nan,
                 dtype=np.float32)
    vp = np.full_like(kp, np.nan)
    O.scatter_rows(kp, inp.k.float().numpy(), mslots)
    O.scatter_rows(vp, inp.v.float().numpy(), mslots)
    cu = np.array([0, 200, 277], dtype=np.int32)
    start = np.zeros(2, dtype=np.int32)
    ctx = inp.lengths.astype(np.int32)
    q = inp.q.to(dev)
    out = torch.empty_like(q)
    scale = 1.0 / float(np.sqrt(w.head_dim))
    kv.paged_attn_prefill(out, q, torch.from_numpy(cu).to(dev),
                          torch.from_numpy(start).to(dev), 200, kc, vc,
                          torch.from_numpy(tables).to(dev),
                          torch.from_numpy(ctx).to(dev), scale, True)
    torch.cuda.synchronize()
    want = O.prefill_paged(inp.q.float().numpy(), cu, start, kp, vp, mt, ctx,
                           scale, True)
    err = float(np.abs(out.float().cpu().numpy() - want).max())
    print(f"smoke prefill: max-abs {err:.2e} (tol 2e-2)", flush=True)
    if not err <= 2e-2:
        raise AssertionError(f"prefill: max-abs {err}")
    print("smoke OK", flush=True)
