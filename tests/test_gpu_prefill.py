"""GPU parity of the chunked-prefill kernels (paged at two block sizes, and
contiguous) against the fp64 oracle, through the C ABI."""
import sys

import numpy as np
import pytest
import torch

import helpers as H
from native import ensure_built
from oracle import attention as O
from paged_kv_cache_191_amd import kvpaged as kv
from paged_kv_cache_191_amd import workloads as W

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _setup():
    ensure_built()
    assert torch.cuda.is_available(), "GPU tests need a GPU"


def _draw(w):
    return W.draw(w, lambda lens: H.pool_blocks_for(w, lens))


def _chunk_meta(inp, c0, C):
    """Queries of chunk [c0, c0 + C) of every sequence: q rows, cu_q_lens,
    q_start_pos, context lengths after the chunk."""
    lens = inp.lengths
    S = len(lens)
    rows, cu, start, ctx = [], [0], [], []
    for s in range(S):
        lo = min(c0, int(lens[s]))
        hi = min(c0 + C, int(lens[s]))
        rows.extend(range(int(inp.cu[s]) + lo, int(inp.cu[s]) + hi))
        cu.append(cu[-1] + hi - lo)
        start.append(lo)
        ctx.append(hi)
    return (np.array(rows, dtype=np.int64), np.array(cu, dtype=np.int32),
            np.array(start, dtype=np.int32), np.array(ctx, dtype=np.int32))


def _run_prefill(inp, layout, nat, kc, vc, rows, cu, start, ctx, causal=True):
    w = inp.workload
    q = inp.q[torch.from_numpy(rows)].cuda().contiguous()
    out = torch.full_like(q, float("nan"))
    cu_d = torch.from_numpy(cu).cuda()
    st_d = torch.from_numpy(start).cuda()
    ctx_d = torch.from_numpy(ctx).cuda()
    max_q = int(np.diff(cu).max()) if len(cu) > 1 else 0
    if layout == "contig":
        kv.contig_attn_prefill(out, q, cu_d, st_d, max_q, kc, vc, ctx_d,
                               H.scale_of(w), causal)
    else:
        kv.paged_attn_prefill(out, q, cu_d, st_d, max_q, nat.k_cache,
                              nat.v_cache, nat.bt, ctx_d, H.scale_of(w),
                              causal)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


@pytest.mark.parametrize("B,layout", [(16, "paged"), (64, "paged"),
                                      (48, "paged"), (16, "contig")])
def test_chunked_prefill_small(B, layout):
    # Yi-6B head shape, two ragged sequences, chunks that span several
    # 32-query blocks and 64-key tiles with ragged tails.
    w = W.WORKLOADS["yi6b_chunked_prefill_b16"].replace(
        num_seqs=2, lengths=(300, 421), chunk=128, block_size=B,
        name=f"prefill_small_{layout}_{B}")
    inp = _draw(w)
    C = w.chunk
    total = int(inp.lengths.max())
    cap = H.tables_capacity(total, B)
    # Cache filled chunk by chunk through the product path.
    nat = H.build_native(inp, B, cap, upto=0)
    orc = H.build_oracle(inp, B)
    kc, vc = H.contig_from_inputs(inp, total) if layout == "contig" else (None, None)
    for c0 in range(0, total, C):
        n_new = np.clip(np.minimum(inp.lengths, c0 + C) - c0, 0, None)
        slots, pairs = nat.pool.seq_append(nat.tables, nat.lens, n_new)
        assert len(pairs) == 0
        rows = np.concatenate([np.arange(inp.cu[s] + c0, inp.cu[s] + c0 + n)
                               for s, n in enumerate(n_new)]).astype(np.int64)
        kv.kv_reshape_and_cache(inp.k[rows].cuda(), inp.v[rows].cuda(),
                                torch.from_numpy(slots).cuda(), nat.k_cache,
                                nat.v_cache)
        nat.bt = torch.from_numpy(nat.tables).cuda()
        qrows, cu, start, ctx = _chunk_meta(inp, c0, C)
        got = _run_prefill(inp, layout, nat, kc, vc, qrows, cu, start, ctx)
        q_all = inp.q[torch.from_numpy(qrows)].float().numpy()
        want = O.prefill_paged(q_all, cu, start, orc.k_pool, orc.v_pool,
                               orc.tables, ctx, H.scale_of(w), True)
        err = H.max_abs(got, want)
        _log(f"{w.name} chunk@{c0}: max-abs {err:.3e}")
        assert err <= H.tolerance(w), (c0, err)


@pytest.mark.parametrize("variant", ["noncausal", "f32_generic",
                                     "g7", "g1", "g5", "b8_generic",
                                     "yi34b_g7_b64"])
def test_prefill_variants(variant):
    # Head groups that are not a multiple of 4 (g1, g5, g7, the Yi-34B shape
    # 56 q / 8 kv heads) run the MFMA kernel with a partly empty last block
    # of heads; fp32, and block sizes that are not a multiple of 16, run the
    # generic kernel.
    base = W.WORKLOADS["yi6b_chunked_prefill_b16"]
    causal = True
    nq = [20, 33]
    if variant == "noncausal":
        w = base.replace(num_seqs=2, lengths=(70, 131), name=variant)
        causal = False
    elif variant == "f32_generic":
        w = base.replace(num_seqs=2, lengths=(40, 77), dtype="f32",
                         dist="uniform", num_q_heads=8, num_kv_heads=2,
                         head_dim=64, name=variant)
    elif variant == "b8_generic":
        w = base.replace(num_seqs=2, lengths=(50, 97), num_q_heads=8,
                         num_kv_heads=2, block_size=8, name=variant)
    elif variant == "yi34b_g7_b64":
        # two 64-row query blocks and a ragged one per sequence
        w = base.replace(num_seqs=2, lengths=(300, 421), num_q_heads=56,
                         num_kv_heads=8, block_size=64, name=variant)
        nq = [150, 131]
    else:
        g = int(variant[1:])
        w = base.replace(num_seqs=2, lengths=(50, 97), num_q_heads=2 * g,
                         num_kv_heads=2, name=variant)
    inp = _draw(w)
    B = w.block_size
    nat = H.build_native(inp, B, H.tables_capacity(int(inp.lengths.max()), B))
    orc = H.build_oracle(inp, B)
    # Query the last `nq` tokens of each sequence against its full context.
    rows = np.concatenate([np.arange(inp.cu[s + 1] - n, inp.cu[s + 1])
                           for s, n in enumerate(nq)]).astype(np.int64)
    cu = np.array([0, nq[0], nq[0] + nq[1]], dtype=np.int32)
    ctx = inp.lengths.astype(np.int32)
    start = (ctx - np.array(nq)).astype(np.int32)
    got = _run_prefill(inp, "paged", nat, None, None, rows, cu, start, ctx,
                       causal)
    want = O.prefill_paged(inp.q[torch.from_numpy(rows)].float().numpy(), cu,
                           start, orc.k_pool, orc.v_pool, orc.tables, ctx,
                           H.scale_of(w), causal)
    err = H.max_abs(got, want)
    _log(f"{variant}: max-abs {err:.3e}")
    assert err <= H.tolerance(w)


@pytest.mark.parametrize("name,layout", [
    ("yi6b_chunked_prefill_b16", "paged"),
    ("yi6b_chunked_prefill_b64", "paged"),
    ("yi6b_chunked_prefill_b16", "contig")])
def test_prefill_full_size_sampled(name, layout):
    # Full Yi-6B-shaped workload (4 x 32768 tokens). The cache holds all
    # tokens; chunk i's queries attend causally with context (i+1)*C, so
    # later tokens are present but must stay masked. Sampled rows of three
    # chunks (first/last rows, block boundaries, random) against the oracle.
    w = W.WORKLOADS[name]
    _log(f"drawing {name}")
    inp = _draw(w)
    B = w.block_size
    total = int(inp.lengths.max())
    cap = H.tables_capacity(total, B)
    nat = H.build_native(inp, B, cap)
    orc = H.build_oracle(inp, B)
    kc, vc = H.contig_from_inputs(inp, total) if layout == "contig" else (None, None)
    C = w.chunk
    for ci in (0, 7, 15):
        c0 = ci * C
        qrows, cu, start, ctx = _chunk_meta(inp, c0, C)
        got = _run_prefill(inp, layout, nat, kc, vc, qrows, cu, start, ctx)
        must = [0, C - 1, C, 2 * C - 1, 15, 16, 63, 64, 65, 3 * C + 31,
                4 * C - 1]
        sample = W.sample_rows(100 + ci, len(qrows), 256, must)
        q_all = inp.q[torch.from_numpy(qrows)].float().numpy()
        want = O.prefill_paged(q_all, cu, start, orc.k_pool, orc.v_pool,
                               orc.tables, ctx, H.scale_of(w), True,
                               rows=sample)
        err = H.max_abs(got[sample], want[sample])
        _log(f"{name} {layout} chunk {ci}: {len(sample)} rows, max-abs {err:.3e}")
        assert err <= H.tolerance(w), (ci, err)
        assert np.isfinite(got).all()


@pytest.mark.parametrize("chunks", [(1, 2, 3, 4, 5, 6),
                                    (8, 9, 10, 11, 12, 13, 14)])
def test_prefill_full_size_every_chunk(chunks):
    # The same Yi-6B-shaped workload, paged B = 16: the 13 chunks the test
    # above leaves out, 256 whole rows each (every sequence's first and last
    # row of the chunk, block boundaries, the rest seeded), so that every
    # chunk of the pass is checked against the oracle. Two halves keep each
    # test's CPU oracle time short.
    name = "yi6b_chunked_prefill_b16"
    w = W.WORKLOADS[name]
    _log(f"drawing {name}")
    inp = _draw(w)
    B = w.block_size
    total = int(inp.lengths.max())
    nat = H.build_native(inp, B, H.tables_capacity(total, B))
    orc = H.build_oracle(inp, B)
    C = w.chunk
    assert max(chunks) < total // C
    for ci in chunks:
        qrows, cu, start, ctx = _chunk_meta(inp, ci * C, C)
        got = _run_prefill(inp, "paged", nat, None, None, qrows, cu, start,
                           ctx)
        must = ([int(x) for x in cu[:-1]] + [int(x) - 1 for x in cu[1:]] +
                [15, 16, 63, 64, 65, C + 15, C + 16])
        sample = W.sample_rows(100 + ci, len(qrows), 256, must)
        q_all = inp.q[torch.from_numpy(qrows)].float().numpy()
        want = O.prefill_paged(q_all, cu, start, orc.k_pool, orc.v_pool,
                               orc.tables, ctx, H.scale_of(w), True,
                               rows=sample)
        err = H.max_abs(got[sample], want[sample])
        _log(f"{name} chunk {ci}: {len(sample)} rows, max-abs {err:.3e}")
        assert err <= H.tolerance(w), (ci, err)
        assert np.isfinite(got).all()


def test_prefill_repeat_is_bit_identical():
    w = W.WORKLOADS["yi6b_chunked_prefill_b16"].replace(
        num_seqs=2, lengths=(500, 333), name="prefill_repeat")
    inp = _draw(w)
    nat = H.build_native(inp, 16, H.tables_capacity(500, 16))
    qrows, cu, start, ctx = _chunk_meta(inp, 0, 500)
    a = _run_prefill(inp, "paged", nat, None, None, qrows, cu, start, ctx)
    b = _run_prefill(inp, "paged", nat, None, None, qrows, cu, start, ctx)
    assert np.array_equal(a, b)
