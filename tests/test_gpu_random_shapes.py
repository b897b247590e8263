"""GPU parity on seeded random shapes, through the C ABI: paged and
contiguous decode, and paged and contiguous chunked prefill (causal and
not), against the fp64 oracle. Each seed draws the batch size, head
grouping, head_dim, block size, dtype and context lengths, so the fast
(MFMA) and generic paths, block sizes that are and are not powers of two,
GQA groups that fill one or two MFMA column blocks, and empty contexts are
all covered."""
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


def _decode_shape(seed):
    g = np.random.default_rng([1000, seed])
    hkv = int(g.choice([1, 2, 4, 8]))
    group = int(g.choice([1, 2, 4, 7, 8, 16, 20]))
    fast = seed % 4 != 3                 # every fourth seed: generic path
    return dict(
        num_seqs=int(g.integers(1, 33)), num_kv_heads=hkv,
        num_q_heads=hkv * group,
        head_dim=128 if fast else int(g.choice([64, 96])),
        block_size=int(g.choice([16, 32, 48, 64])) if fast else
        int(g.choice([8, 16, 24])),
        dtype="bf16" if fast or seed % 8 == 3 else "f32",
        length_range=(0, int(g.integers(1, 900))),
        dist="normal" if fast else "uniform")


@pytest.mark.parametrize("seed", range(12))
def test_decode_random_shapes(seed):
    spec = _decode_shape(seed)
    w = W.WORKLOADS["llama3_8b_decode"].replace(name=f"rand_decode_{seed}",
                                               seed=1000 + seed, **spec)
    inp = W.draw(w, lambda lens: H.pool_blocks_for(w, lens))
    ctx = W.context_lengths(inp)
    B = w.block_size
    cap = H.tables_capacity(int(max(ctx.max(), 1)), B)
    nat = H.build_native(inp, B, cap)
    orc = H.build_oracle(inp, B)
    q = inp.q.cuda()
    max_ctx = int(max(ctx.max(), 1))
    scale = H.scale_of(w)
    out = torch.full_like(q, float("nan"))
    kv.paged_attn_decode(out, q, nat.k_cache, nat.v_cache, nat.bt, nat.ctx,
                         max_ctx, scale)
    kc, vc = H.contig_from_inputs(inp, max_ctx)
    oc = torch.full_like(q, float("nan"))
    kv.contig_attn_decode(oc, q, kc, vc, nat.ctx, max_ctx, scale)
    torch.cuda.synchronize()
    want = O.decode_paged(inp.q.float().numpy(), orc.k_pool, orc.v_pool,
                          orc.tables, ctx, scale)
    tol = H.tolerance(w)
    for name, got in (("paged", out), ("contig", oc)):
        err = H.max_abs(got.float().cpu().numpy(), want)
        _log(f"{w.name} {spec} {name}: max-abs {err:.2e} (tol {tol})")
        assert err <= tol, (name, err)


def _prefill_shape(seed):
    g = np.random.default_rng([2000, seed])
    hkv = int(g.choice([1, 2, 4]))
    group = int(g.choice([1, 2, 3, 4, 5, 7, 8, 12]))
    S = int(g.integers(1, 4))
    return dict(num_seqs=S, num_kv_heads=hkv, num_q_heads=hkv * group,
                block_size=int(g.choice([16, 32, 48, 64])),
                lengths=tuple(int(x) for x in g.integers(1, 700, size=S)),
                length_range=None), bool(g.integers(0, 2))


@pytest.mark.parametrize("seed", range(8))
def test_prefill_random_shapes(seed):
    spec, causal = _prefill_shape(seed)
    w = W.WORKLOADS["yi6b_chunked_prefill_b16"].replace(
        name=f"rand_prefill_{seed}", seed=2000 + seed, **spec)
    inp = W.draw(w, lambda lens: H.pool_blocks_for(w, lens))
    B = w.block_size
    lens = inp.lengths.astype(np.int32)
    nat = H.build_native(inp, B, H.tables_capacity(int(lens.max()), B))
    orc = H.build_oracle(inp, B)
    # one chunk per sequence: its last n_q tokens against its whole context
    g = np.random.default_rng([2100, seed])
    nq = np.array([int(g.integers(1, L + 1)) for L in lens], dtype=np.int32)
    rows = np.concatenate([np.arange(inp.cu[s + 1] - n, inp.cu[s + 1])
                           for s, n in enumerate(nq)]).astype(np.int64)
    cu = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    start = (lens - nq).astype(np.int32)
    q = inp.q[torch.from_numpy(rows)].cuda().contiguous()
    out = torch.full_like(q, float("nan"))
    kv.paged_attn_prefill(out, q, torch.from_numpy(cu).cuda(),
                          torch.from_numpy(start).cuda(), int(nq.max()),
                          nat.k_cache, nat.v_cache, nat.bt,
                          torch.from_numpy(lens).cuda(), H.scale_of(w),
                          causal)
    # the contiguous layout of the same data (unused tail rows NaN)
    kc, vc = H.contig_from_inputs(inp, int(lens.max()))
    oc = torch.full_like(q, float("nan"))
    kv.contig_attn_prefill(oc, q, torch.from_numpy(cu).cuda(),
                           torch.from_numpy(start).cuda(), int(nq.max()), kc,
                           vc, torch.from_numpy(lens).cuda(), H.scale_of(w),
                           causal)
    torch.cuda.synchronize()
    want = O.prefill_paged(inp.q[torch.from_numpy(rows)].float().numpy(), cu,
                           start, orc.k_pool, orc.v_pool, orc.tables, lens,
                           H.scale_of(w), causal)
    for name, got in (("paged", out), ("contig", oc)):
        err = H.max_abs(got.float().cpu().numpy(), want)
        _log(f"{w.name} {spec} causal={causal} q={nq.tolist()} {name}: "
             f"max-abs {err:.2e}")
        assert err <= H.tolerance(w), (name, err)
