"""GPU parity of paged_attn_decode_append (the decode step with its token
appended in one op) against the two calls it fuses, kv_append_token then
paged_attn_decode, and against the fp64 oracle, through the C ABI. The
caches, tables and lengths it leaves must equal the two calls' bit for bit;
its outputs differ from theirs only in rounding (the new token's weight is
applied in fp32 instead of through the bf16 MFMA operand)."""
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


def _bits(t):
    """Bit pattern of a cache (NaN-initialised pools compare as bits)."""
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else \
        t.view(torch.int32)


class Side:
    """One copy of the batch at contexts `stored` (device caches, table and
    lengths), to be advanced by one step either fused or unfused."""

    def __init__(self, inp, B, cap, stored):
        self.nat = H.build_native(inp, B, cap, upto=stored)
        self.S = inp.workload.num_seqs
        self.B = B
        self.newb = torch.full((self.S,), -1, dtype=torch.int32,
                               pin_memory=True)
        self.lens = torch.from_numpy(self.nat.lens.copy()).cuda()
        self.bt = torch.from_numpy(self.nat.tables).cuda()

    def host_append(self, ok):
        """kv_seq_append for the sequences in `ok`; their new block ids (or
        -1) into the pinned buffer."""
        nat, S, B = self.nat, self.S, self.B
        idx = np.minimum(nat.lens // B, nat.tables.shape[1] - 1)
        before = nat.tables[np.arange(S), idx].copy()
        n_new = np.asarray(ok, dtype=np.int32)
        _, pairs = nat.pool.seq_append(nat.tables, nat.lens, n_new)
        assert len(pairs) == 0
        after = nat.tables[np.arange(S), idx]
        self.newb.numpy()[:] = np.where((after != before) & (n_new > 0),
                                        after, -1)


def _run_step(inp, B, cap, stored, ok, k_new, v_new, max_context,
              fused: bool, dtype_ws=None):
    """One step on a fresh copy; returns (out, side, workspace)."""
    w = inp.workload
    side = Side(inp, B, cap, stored)
    side.host_append(ok)
    q = inp.q.cuda()
    out = torch.full_like(q, float("nan"))
    ws = kv.decode_workspace(w.num_seqs, w.num_q_heads, w.num_kv_heads,
                             w.head_dim, max_context, q.device)
    nat = side.nat
    if fused:
        kv.paged_attn_decode_append(out, q, k_new, v_new, side.newb,
                                    nat.k_cache, nat.v_cache, side.bt,
                                    side.lens, max_context, H.scale_of(w), ws)
    else:
        kv.kv_append_token(k_new, v_new, side.newb, side.bt, side.lens,
                           nat.k_cache, nat.v_cache)
        kv.paged_attn_decode(out, q, nat.k_cache, nat.v_cache, side.bt,
                             side.lens, max_context, H.scale_of(w), ws)
    torch.cuda.synchronize()
    return out, side, ws


def _new_rows(inp, stored):
    """K/V of each sequence's token at position stored[s] (the draw's next
    row), so that the oracle sees the same context."""
    S = inp.workload.num_seqs
    rows = []
    for s in range(S):
        lr = W.logical_rows(inp, s)
        rows.append(lr[min(int(stored[s]), len(lr) - 1)])
    r = torch.from_numpy(np.array(rows))
    return inp.k[r].cuda().contiguous(), inp.v[r].cuda().contiguous()


def _compare(inp, B, cap, stored, ok, max_context, ctx_after):
    w = inp.workload
    k_new, v_new = _new_rows(inp, stored)
    of, sf, wsf = _run_step(inp, B, cap, stored, ok, k_new, v_new,
                            max_context, True)
    ou, su, wsu = _run_step(inp, B, cap, stored, ok, k_new, v_new,
                            max_context, False)
    # the same cache, table and lengths, bit for bit
    assert torch.equal(_bits(sf.nat.k_cache), _bits(su.nat.k_cache))
    assert torch.equal(_bits(sf.nat.v_cache), _bits(su.nat.v_cache))
    assert torch.equal(sf.bt, su.bt)
    assert torch.equal(sf.lens, su.lens)
    assert sf.lens.cpu().numpy().tolist() == list(ctx_after_stored(
        stored, ok))
    assert kv.kv_decode_clamped_count(wsf) == kv.kv_decode_clamped_count(wsu)
    got, ref = of.float().cpu().numpy(), ou.float().cpu().numpy()
    d = H.max_abs(got, ref)
    _within_rounding(got, ref)
    orc = H.build_oracle(inp, B)
    want = O.decode_paged(inp.q.float().numpy(), orc.k_pool, orc.v_pool,
                          orc.tables, np.asarray(ctx_after), H.scale_of(w))
    e = H.max_abs(got, want)
    _log(f"{w.name}: fused vs two calls max-abs {d:.2e}, vs oracle {e:.2e}")
    assert e <= H.tolerance(w), e
    return sf, wsf


def _within_rounding(got, ref):
    """The fused op and the two calls differ by the rounding of the output
    to bf16 (2^-8 relative, 2^-7 allowed) plus the new token's weight taken
    in fp32 instead of as a bf16 MFMA operand (2^-9 relative per weight,
    which near-cancelling sums can leave as about 1e-3 absolute; 4e-3
    allowed)."""
    bound = 2.0 ** -7 * np.maximum(np.abs(got), np.abs(ref)) + 4e-3
    bad = np.abs(got - ref) > bound
    assert not bad.any(), (np.argwhere(bad)[:5], got[bad][:5], ref[bad][:5])


def ctx_after_stored(stored, ok):
    return [int(a) + int(b) for a, b in zip(stored, ok)]


def test_decode_append_edge_lengths():
    # first token of a sequence (stored 0), last slot of a block (15), the
    # first slot of a new block (16, 32), long contexts; a bound that cuts
    # the longest sequence's new token (clamped in both paths)
    lengths = (1, 16, 17, 33, 200, 1000)
    w = W.WORKLOADS["llama3_8b_decode"].replace(
        num_seqs=len(lengths), lengths=lengths, length_range=None,
        name="append_edges")
    inp = W.draw(w, lambda L: H.pool_blocks_for(w, L, 8))
    ctx = np.array(lengths, dtype=np.int32)
    stored = ctx - 1
    B = w.block_size
    cap = H.tables_capacity(int(ctx.max()), B)
    ok = np.ones(len(lengths), dtype=np.int32)
    _compare(inp, B, cap, stored, ok, int(ctx.max()), ctx)
    # bound 200: the 1000-token sequence attends to its first 200 tokens
    # only (and is counted as clamped), its token is still stored
    sf, ws = _compare(inp, B, cap, stored, ok, 200,
                      np.minimum(ctx, 200))
    assert kv.kv_decode_clamped_count(ws) == 1


def test_decode_append_full_table():
    # a sequence whose table is full: its token has no slot, it is neither
    # stored nor attended to, and its length stays
    lengths = (33, 21)
    w = W.WORKLOADS["llama3_8b_decode"].replace(
        num_seqs=2, lengths=lengths, length_range=None, name="append_full")
    inp = W.draw(w, lambda L: H.pool_blocks_for(w, L, 4))
    stored = np.array([32, 20], dtype=np.int32)
    B = w.block_size
    cap = 2                    # 32 tokens: sequence 0 is full
    ok = np.array([0, 1], dtype=np.int32)
    _compare(inp, B, cap, stored, ok, cap * B, np.array([32, 21]))


@pytest.mark.parametrize("name,S,B", [("llama3_8b_decode", 64, 16),
                                      ("yi34b_long_decode", 4, 64)])
def test_decode_append_workload_shapes(name, S, B):
    # Llama-3-8B (64 sequences, 32/8 heads) and a Yi-34B-shaped batch
    # (56/8 heads, block 64; contexts shortened to keep the oracle quick)
    w = W.WORKLOADS[name]
    if name.startswith("yi34b"):
        w = w.replace(lengths=(5000, 3001, 64, 129), length_range=None,
                      name="yi34b_shape_append")
    inp = W.draw(w, lambda L: H.pool_blocks_for(w, L, S))
    ctx = W.context_lengths(inp).astype(np.int32)
    stored = ctx - 1
    cap = H.tables_capacity(int(ctx.max()), B)
    _compare(inp, B, cap, stored, np.ones(S, dtype=np.int32),
             int(ctx.max()), ctx)


def test_decode_append_many_sequences():
    # more sequences than one launch takes (4096): the launches share the
    # workspace, each copying its own block ids into it; short contexts,
    # the first token of some sequences among them
    w = W.WORKLOADS["llama3_8b_decode"].replace(
        num_seqs=4100, num_q_heads=8, num_kv_heads=2, length_range=(1, 48),
        name="append_many_seqs")
    inp = W.draw(w, lambda L: H.pool_blocks_for(w, L, w.num_seqs))
    ctx = W.context_lengths(inp).astype(np.int32)
    assert (ctx == 1).any()
    B = w.block_size
    cap = H.tables_capacity(int(ctx.max()), B)
    _compare(inp, B, cap, ctx - 1, np.ones(w.num_seqs, dtype=np.int32),
             int(ctx.max()), ctx)


def test_decode_append_many_steps():
    # 40 steps of 16 sequences, every one fused against the two calls on
    # their own copies (new rows drawn per step): caches, tables and lengths
    # stay bit-identical, outputs within rounding
    w = W.WORKLOADS["llama3_8b_decode"].replace(num_seqs=16, name="append40")
    inp = W.draw(w, lambda L: H.pool_blocks_for(w, L, 16 * 4))
    ctx = W.context_lengths(inp).astype(np.int32)
    B = w.block_size
    steps = 40
    cap = H.tables_capacity(int(ctx.max()) + steps, B)
    sides = [Side(inp, B, cap, ctx) for _ in range(2)]
    q = inp.q.cuda()
    g = torch.Generator().manual_seed(11)
    ws = [kv.decode_workspace(w.num_seqs, w.num_q_heads, w.num_kv_heads,
                              w.head_dim, cap * B, q.device) for _ in range(2)]
    worst = 0.0
    for step in range(steps):
        k_new = torch.randn(w.num_seqs, w.num_kv_heads, w.head_dim,
                            generator=g).to(torch.bfloat16).cuda()
        v_new = torch.randn(k_new.shape, generator=g).to(torch.bfloat16).cuda()
        outs = []
        for i, side in enumerate(sides):
            side.host_append(np.ones(w.num_seqs, dtype=np.int32))
            nat = side.nat
            out = torch.full_like(q, float("nan"))
            if i == 0:
                kv.paged_attn_decode_append(
                    out, q, k_new, v_new, side.newb, nat.k_cache, nat.v_cache,
                    side.bt, side.lens, cap * B, H.scale_of(w), ws[0])
            else:
                kv.kv_append_token(k_new, v_new, side.newb, side.bt,
                                   side.lens, nat.k_cache, nat.v_cache)
                kv.paged_attn_decode(out, q, nat.k_cache, nat.v_cache,
                                     side.bt, side.lens, cap * B,
                                     H.scale_of(w), ws[1])
            torch.cuda.synchronize()
            outs.append(out.float().cpu().numpy())
        a, b = sides
        assert torch.equal(_bits(a.nat.k_cache), _bits(b.nat.k_cache))
        assert torch.equal(_bits(a.nat.v_cache), _bits(b.nat.v_cache))
        assert torch.equal(a.bt, b.bt) and torch.equal(a.lens, b.lens)
        worst = max(worst, H.max_abs(outs[0], outs[1]))
        _within_rounding(outs[0], outs[1])
    _log(f"40 fused steps: states bit-identical, outputs max-abs {worst:.2e}")


@pytest.mark.parametrize("hq,hkv", [(8, 8), (40, 2), (12, 4)])
def test_decode_append_head_groups(hq, hkv):
    # one query head per KV head, a group of 20 (two 16-head column blocks,
    # so two workgroups fold the token for each KV head), a group of 3
    lengths = (1, 31, 32, 33, 500, 64)
    w = W.WORKLOADS["llama3_8b_decode"].replace(
        num_seqs=len(lengths), lengths=lengths, length_range=None,
        num_q_heads=hq, num_kv_heads=hkv, name=f"append_g{hq // hkv}")
    inp = W.draw(w, lambda L: H.pool_blocks_for(w, L, 8))
    ctx = np.array(lengths, dtype=np.int32)
    B = w.block_size
    cap = H.tables_capacity(int(ctx.max()), B)
    _compare(inp, B, cap, ctx - 1, np.ones(len(lengths), dtype=np.int32),
             int(ctx.max()), ctx)


@pytest.mark.parametrize("variant", ["f32", "b8"])
def test_decode_append_fallback_shapes(variant):
    # shapes outside the stream-K kernel run the two calls: identical
    w = W.WORKLOADS["decode_tiny_f32"] if variant == "f32" else \
        W.WORKLOADS["llama3_8b_decode"].replace(
            num_seqs=4, lengths=(40, 9, 64, 100), length_range=None,
            block_size=8, name="append_b8")
    inp = W.draw(w, lambda L: H.pool_blocks_for(w, L, 8))
    ctx = W.context_lengths(inp).astype(np.int32)
    stored = ctx - 1
    B = w.block_size
    cap = H.tables_capacity(int(ctx.max()), B)
    k_new, v_new = _new_rows(inp, stored)
    ok = np.ones(w.num_seqs, dtype=np.int32)
    of, sf, _ = _run_step(inp, B, cap, stored, ok, k_new, v_new,
                          int(ctx.max()), True)
    ou, su, _ = _run_step(inp, B, cap, stored, ok, k_new, v_new,
                          int(ctx.max()), False)
    assert torch.equal(_bits(sf.nat.k_cache), _bits(su.nat.k_cache))
    assert torch.equal(sf.lens, su.lens)
    assert torch.equal(_bits(of), _bits(ou))
