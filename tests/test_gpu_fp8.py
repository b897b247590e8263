"""GPU parity of the fp8 E4M3 K/V cache through the C ABI: the quantising
cache write bit for bit against the oracle's codec (oracle/fp8.py), and
decode over fp8 caches against the fp64 oracle run on the dequantised
values, with one scale per tensor or one per KV head. Unused cache bytes
start as 0x7F (an E4M3 NaN), so a kernel that reads a slot past a context
fails the comparison."""
import sys

import numpy as np
import pytest
import torch

import helpers as H
from native import ensure_built
from oracle import attention as O
from oracle import fp8 as F
from paged_kv_cache_191_amd import kvpaged as kv
from paged_kv_cache_191_amd import workloads as W

pytestmark = pytest.mark.gpu

NAN_CODE = 0x7F


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _setup():
    ensure_built()
    assert torch.cuda.is_available(), "GPU tests need a GPU"


def _per_head(scale) -> bool:
    return isinstance(scale, np.ndarray)


def _inv(scale):
    """The fp32 reciprocal the cache write multiplies by: a number, or for
    per-head scales an [Hkv, 1] array that broadcasts over rows [.., Hkv,
    D]."""
    if _per_head(scale):
        return (np.float32(1.0) / scale.astype(np.float32))[:, None]
    return float(np.float32(1.0) / np.float32(scale))


def _scale_b(scale):
    """A scale as the oracle's dequantisation takes it ([Hkv, 1] per head)."""
    return scale[:, None] if _per_head(scale) else scale


def _dev_scales(scale):
    return torch.from_numpy(scale.astype(np.float32)).cuda()


def _write_fp8(k, v, slots, kc, vc, ks, vs):
    """kv_reshape_and_cache_fp8, or its per-head form for array scales."""
    if _per_head(ks):
        kv.kv_reshape_and_cache_fp8_per_head(k, v, slots, kc, vc,
                                             _dev_scales(ks), _dev_scales(vs))
    else:
        kv.kv_reshape_and_cache_fp8(k, v, slots, kc, vc, ks, vs)


def _fill_fp8(inp, nat, k_scale, v_scale):
    """fp8 paged caches [N, Hkv, B, D] holding every context row of the
    native tables (written in one cache-write call)."""
    w = inp.workload
    B = w.block_size
    kc = torch.full(tuple(nat.k_cache.shape), NAN_CODE, dtype=torch.uint8,
                    device="cuda")
    vc = torch.full_like(kc, NAN_CODE)
    ctx = W.context_lengths(inp)
    seq_ids = np.concatenate([np.full(int(n), s, dtype=np.int32)
                              for s, n in enumerate(ctx)])
    pos = np.concatenate([np.arange(int(n), dtype=np.int32) for n in ctx])
    slots = kv.kv_slot_mapping(nat.tables, seq_ids, pos, B)
    rows = np.concatenate([W.logical_rows(inp, s) for s in range(len(ctx))])
    r = torch.from_numpy(rows)
    _write_fp8(inp.k[r].cuda(), inp.v[r].cuda(),
               torch.from_numpy(slots).cuda(), kc, vc, k_scale, v_scale)
    torch.cuda.synchronize()
    return kc, vc


def _oracle_codes(inp, orc, k_scale, v_scale, seqs=None):
    """Oracle code pools [N, B, Hkv, D] (0x7F where unused) for the
    sequences `seqs` (all by default), scattered by the oracle's tables."""
    w = inp.workload
    B = w.block_size
    n_pool = orc.k_pool.shape[0]
    kp = np.full((n_pool, B, w.num_kv_heads, w.head_dim), NAN_CODE,
                 dtype=np.uint8)
    vp = kp.copy()
    ctx = W.context_lengths(inp)
    seqs = list(range(len(ctx)) if seqs is None else seqs)
    per_row = w.num_kv_heads * w.head_dim

    def flush(batch):
        rows = [W.logical_rows(inp, s) for s in batch]
        sid = [s for s, r in zip(batch, rows) for _ in range(len(r))]
        if not sid:
            return
        pos = [p for r in rows for p in range(len(r))]
        slots = O.slot_mapping(orc.tables, sid, pos, B)
        allr = np.concatenate(rows)
        O.scatter_rows(kp, F.quantize(inp.k[allr].float().numpy(),
                                      _inv(k_scale)), slots)
        O.scatter_rows(vp, F.quantize(inp.v[allr].float().numpy(),
                                      _inv(v_scale)), slots)

    # sequences batched into oracle calls of about 4M values (the oracle
    # encodes each distinct product once per call)
    batch, n = [], 0
    for s in seqs:
        batch.append(s)
        n += int(ctx[s]) * per_row
        if n >= 4 << 20:
            flush(batch)
            batch, n = [], 0
    flush(batch)
    return kp, vp


def _dequant_pool(codes, scale):
    """Values of an oracle code pool [N, B, Hkv, D] (NaN where 0x7F)."""
    return F.dequantize(codes, _scale_b(scale))


def _small_workload(seed=11):
    return W.WORKLOADS["llama3_8b_decode"].replace(
        num_seqs=7, lengths=(1, 15, 16, 17, 300, 129, 64), length_range=None,
        name="fp8_small", seed=seed)


# ------------------------------------------------------------ cache write --
def test_fp8_cache_write_special_values():
    """Rounding, clamping and the non-finite inputs, one value per lane."""
    vals = [np.nan, np.inf, -np.inf, -0.0, 0.0, 448.0, 464.0, -464.0, 1e30,
            -1e30, 2.0 ** -9, 2.0 ** -10, -(2.0 ** -10), 3 * 2.0 ** -10,
            2.0 ** -11, 1.0625, 1.1875, -1.0625, 0.01171875, 0.013671875,
            240.0, 248.0, 232.0, 2.0 ** -6, 7 * 2.0 ** -9, 15 * 2.0 ** -10]
    D = 128
    row = np.zeros(D, dtype=np.float32)
    row[:len(vals)] = vals
    g = np.random.default_rng(7)
    row[len(vals):] = g.standard_normal(D - len(vals)).astype(np.float32) * 50
    k = torch.from_numpy(np.stack([row, -row])[:, None, :]).to(torch.bfloat16)
    v = torch.from_numpy(np.stack([row * 0.25, row * 3])[:, None, :]).to(
        torch.bfloat16)
    for ks, vs in ((1.0, 1.0), (0.5, 3.0), (0.0123, 7.5)):
        kc = torch.full((1, 1, 16, D), NAN_CODE, dtype=torch.uint8,
                        device="cuda")
        vc = torch.full_like(kc, NAN_CODE)
        kv.kv_reshape_and_cache_fp8(k.cuda(), v.cuda(),
                                    torch.tensor([3, 0], dtype=torch.int64,
                                                 device="cuda"), kc, vc, ks, vs)
        torch.cuda.synchronize()
        got_k = kc.cpu().numpy()[0, 0]
        got_v = vc.cpu().numpy()[0, 0]
        want_k = F.quantize(k.float().numpy()[:, 0], _inv(ks))
        want_v = F.quantize(v.float().numpy()[:, 0], _inv(vs))
        assert np.array_equal(got_k[3], want_k[0]), (ks, vs)
        assert np.array_equal(got_k[0], want_k[1]), (ks, vs)
        assert np.array_equal(got_v[3], want_v[0]), (ks, vs)
        assert np.array_equal(got_v[0], want_v[1]), (ks, vs)
        untouched = [r for r in range(16) if r not in (0, 3)]
        assert (got_k[untouched] == NAN_CODE).all()
        assert (got_v[untouched] == NAN_CODE).all()


@pytest.mark.parametrize("scales", [(0.0123, 0.02), (0.005, 1.0)])
def test_fp8_cache_write_bit_exact(scales):
    """Ragged contexts through the native tables; (0.005, 1.0) saturates many
    K values and puts many V values in the subnormal range."""
    ks, vs = scales
    w = _small_workload()
    inp = W.draw(w, lambda lens: H.pool_blocks_for(w, lens, 4))
    cap = H.tables_capacity(int(W.context_lengths(inp).max()), w.block_size)
    nat = H.build_native(inp, w.block_size, cap)
    orc = H.build_oracle(inp, w.block_size)
    kc, vc = _fill_fp8(inp, nat, ks, vs)
    kp, vp = _oracle_codes(inp, orc, ks, vs)
    assert np.array_equal(kc.permute(0, 2, 1, 3).cpu().numpy(), kp)
    assert np.array_equal(vc.permute(0, 2, 1, 3).cpu().numpy(), vp)


def test_fp8_cache_write_errors():
    k = torch.zeros((2, 1, 128), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((1, 1, 16, 128), dtype=torch.uint8, device="cuda")
    slots = torch.zeros(2, dtype=torch.int64, device="cuda")
    for ks, vs in ((0.0, 1.0), (1.0, -1.0), (float("inf"), 1.0),
                   (1.0, float("nan"))):
        with pytest.raises(kv.KVError):
            kv.kv_reshape_and_cache_fp8(k, k, slots, kc, kc.clone(), ks, vs)
    k12 = torch.zeros((2, 1, 12), dtype=torch.bfloat16, device="cuda")
    kc12 = torch.zeros((1, 1, 16, 12), dtype=torch.uint8, device="cuda")
    with pytest.raises(kv.KVError):
        kv.kv_reshape_and_cache_fp8(k12, k12, slots, kc12, kc12.clone(), 1, 1)
    with pytest.raises(TypeError):
        kv.kv_reshape_and_cache_fp8(k, k, slots, kc.to(torch.int32),
                                    kc.clone(), 1.0, 1.0)


# ----------------------------------------------------------------- decode --
def _decode_fp8_both(inp, nat, orc, kc, vc, kp, vp, ks, vs, seqs=None,
                     contig=True):
    w = inp.workload
    scale = H.scale_of(w)
    ctx = W.context_lengths(inp)
    max_ctx = int(ctx.max())
    q = inp.q.cuda()
    out = torch.empty_like(q)
    if _per_head(ks):
        kv.paged_attn_decode_fp8_per_head(out, q, kc, vc, nat.bt, nat.ctx,
                                          max_ctx, scale, _dev_scales(ks),
                                          _dev_scales(vs))
    else:
        kv.paged_attn_decode_fp8(out, q, kc, vc, nat.bt, nat.ctx, max_ctx,
                                 scale, ks, vs)
    outs = {"paged": out}
    if contig:
        # contiguous fp8 caches [S, Hkv, Lmax, D] written by the same call,
        # slot = s * Lmax + pos
        S = w.num_seqs
        ck = torch.full((S, w.num_kv_heads, max_ctx, w.head_dim), NAN_CODE,
                        dtype=torch.uint8, device="cuda")
        cv = torch.full_like(ck, NAN_CODE)
        rows = np.concatenate([W.logical_rows(inp, s) for s in range(S)])
        slots = np.concatenate([s * max_ctx + np.arange(int(ctx[s]))
                                for s in range(S)]).astype(np.int64)
        r = torch.from_numpy(rows)
        _write_fp8(inp.k[r].cuda(), inp.v[r].cuda(),
                   torch.from_numpy(slots).cuda(), ck, cv, ks, vs)
        oc = torch.empty_like(q)
        if _per_head(ks):
            kv.contig_attn_decode_fp8_per_head(oc, q, ck, cv, nat.ctx,
                                               max_ctx, scale,
                                               _dev_scales(ks),
                                               _dev_scales(vs))
        else:
            kv.contig_attn_decode_fp8(oc, q, ck, cv, nat.ctx, max_ctx, scale,
                                      ks, vs)
        outs["contig"] = oc
    torch.cuda.synchronize()
    want = O.decode_paged(inp.q.float().numpy(), _dequant_pool(kp, ks),
                          _dequant_pool(vp, vs), orc.tables, ctx, scale,
                          seqs=seqs)
    return {k: v.float().cpu().numpy() for k, v in outs.items()}, want


def _check(outs, want, name, seqs=None):
    tol = 2e-2   # bf16 q, P and output, as for the bf16 cache
    sel = slice(None) if seqs is None else list(seqs)
    for lay, got in outs.items():
        err = H.max_abs(got[sel], want[sel])
        _log(f"{name} {lay}: max-abs {err:.3e} (tol {tol})")
        assert err <= tol, (lay, err)


@pytest.mark.parametrize("scales", [(0.0123, 0.02), (0.03, 0.004)])
def test_decode_fp8_small(scales):
    ks, vs = scales
    w = _small_workload(seed=12)
    inp = W.draw(w, lambda lens: H.pool_blocks_for(w, lens, 4))
    cap = H.tables_capacity(int(W.context_lengths(inp).max()), w.block_size)
    nat = H.build_native(inp, w.block_size, cap)
    orc = H.build_oracle(inp, w.block_size)
    kc, vc = _fill_fp8(inp, nat, ks, vs)
    kp, vp = _oracle_codes(inp, orc, ks, vs)
    outs, want = _decode_fp8_both(inp, nat, orc, kc, vc, kp, vp, ks, vs)
    _check(outs, want, f"fp8_small{scales}")
    # a one-token context returns that token's dequantised V row
    G = w.num_q_heads // w.num_kv_heads
    v0 = _dequant_pool(vp, vs)[orc.tables[0][0], 0]
    v0 = v0[np.arange(w.num_q_heads) // G]
    assert H.max_abs(outs["paged"][0], v0) <= 2e-2
    assert np.array_equal(outs["paged"], outs["contig"])


def test_decode_fp8_long_context_split():
    # Yi-34B shape (G = 7, B = 64), shortened: sequences cut into chunks
    w = W.WORKLOADS["yi34b_long_decode"].replace(
        num_seqs=3, lengths=(9000, 2049, 70), name="fp8_yi34b_short")
    inp = W.draw(w, lambda lens: H.pool_blocks_for(w, lens))
    ctx = W.context_lengths(inp)
    cap = H.tables_capacity(int(ctx.max()), w.block_size)
    nat = H.build_native(inp, w.block_size, cap)
    orc = H.build_oracle(inp, w.block_size)
    ks, vs = 0.0123, 0.0123
    kc, vc = _fill_fp8(inp, nat, ks, vs)
    kp, vp = _oracle_codes(inp, orc, ks, vs)
    outs, want = _decode_fp8_both(inp, nat, orc, kc, vc, kp, vp, ks, vs)
    _check(outs, want, w.name)
    assert np.array_equal(outs["paged"], outs["contig"])


def test_decode_fp8_full_size():
    """Llama-3-8B-shaped decode batch (64 sequences, 512..4096 tokens), the
    launch the benchmark times: every code of the pool and every output
    against the oracle (about 35 s of oracle quantisation)."""
    w = W.WORKLOADS["llama3_8b_decode"]
    _log("drawing llama3_8b_decode")
    inp = W.draw(w, lambda lens: H.pool_blocks_for(w, lens))
    ctx = W.context_lengths(inp)
    cap = H.tables_capacity(int(ctx.max()), w.block_size)
    nat = H.build_native(inp, w.block_size, cap)
    orc = H.build_oracle(inp, w.block_size)
    ks, vs = 0.0123, 0.0123
    kc, vc = _fill_fp8(inp, nat, ks, vs)
    kp, vp = _oracle_codes(inp, orc, ks, vs)
    # every sequence's codes are the oracle's, bit for bit
    kd = kc.permute(0, 2, 1, 3).cpu().numpy()
    vd = vc.permute(0, 2, 1, 3).cpu().numpy()
    for s in range(w.num_seqs):
        blocks = orc.tables[s]
        assert np.array_equal(kd[blocks], kp[blocks])
        assert np.array_equal(vd[blocks], vp[blocks])
    outs, want = _decode_fp8_both(inp, nat, orc, kc, vc, kp, vp, ks, vs,
                                  contig=False)
    _check(outs, want, w.name)


def test_decode_fp8_many_sequences():
    """4100 sequences (two launches), contexts 0..48, per-head scales:
    paged and contiguous fp8 caches against the oracle."""
    w = _small_workload(seed=21).replace(
        num_seqs=4100, lengths=None, length_range=(0, 48), num_q_heads=8,
        num_kv_heads=2, name="fp8_many_seqs")
    inp = W.draw(w, lambda lens: H.pool_blocks_for(w, lens, 4))
    ctx = W.context_lengths(inp)
    assert (ctx == 0).any()
    cap = H.tables_capacity(int(max(ctx.max(), 1)), w.block_size)
    nat = H.build_native(inp, w.block_size, cap)
    orc = H.build_oracle(inp, w.block_size)
    ks, vs = _head_scales(10, w.num_kv_heads)
    kc, vc = _fill_fp8(inp, nat, ks, vs)
    kp, vp = _oracle_codes(inp, orc, ks, vs)
    outs, want = _decode_fp8_both(inp, nat, orc, kc, vc, kp, vp, ks, vs)
    _check(outs, want, w.name)


def test_decode_fp8_errors():
    q = torch.zeros((1, 8, 128), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((2, 2, 16, 128), dtype=torch.uint8, device="cuda")
    bt = torch.zeros((1, 2), dtype=torch.int32, device="cuda")
    ctx = torch.ones(1, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    with pytest.raises(kv.KVError):
        kv.paged_attn_decode_fp8(out, q, kc, kc, bt, ctx, 1, 0.1, 0.0, 1.0)
    with pytest.raises(kv.KVError):
        kv.paged_attn_decode_fp8(out, q, kc, kc, bt, ctx, 1, 0.1, 1.0,
                                 float("inf"))
    # head_dim 64: no fp8 kernel
    q64 = torch.zeros((1, 8, 64), dtype=torch.bfloat16, device="cuda")
    kc64 = torch.zeros((2, 2, 16, 64), dtype=torch.uint8, device="cuda")
    with pytest.raises(kv.KVError, match="UNSUPPORTED"):
        kv.paged_attn_decode_fp8(torch.empty_like(q64), q64, kc64, kc64, bt,
                                 ctx, 1, 0.1, 1.0, 1.0)


def _fp8_shape(seed):
    g = np.random.default_rng([3000, seed])
    hkv = int(g.choice([1, 2, 4, 8]))
    group = (1, 2, 4, 7, 8, 16, 20, 5)[seed % 8]    # each size once
    S = int(g.integers(2, 33))
    lens = g.integers(1, int(g.integers(2, 1500)), size=S, endpoint=True)
    if seed % 2 == 0:
        lens[S // 2] = 0                           # an empty context
    spec = dict(num_seqs=S, num_kv_heads=hkv, num_q_heads=hkv * group,
                head_dim=128, block_size=(16, 32, 48, 64)[seed % 4],
                lengths=tuple(int(x) for x in lens), length_range=None)
    scales = tuple(float(np.float32(x)) for x in g.uniform(0.012, 0.05, 2))
    return spec, scales


@pytest.mark.parametrize("seed", range(8))
def test_decode_fp8_random_shapes(seed):
    """Seeded random shapes over fp8 caches: batch size, KV heads, head
    groups that fill one or two MFMA column blocks, block sizes, context
    lengths (empty ones included) and per-tensor scales; paged and
    contiguous against the oracle on the dequantised codes."""
    spec, (ks, vs) = _fp8_shape(seed)
    w = W.WORKLOADS["llama3_8b_decode"].replace(name=f"fp8_rand_{seed}",
                                               seed=3000 + seed, **spec)
    inp = W.draw(w, lambda lens: H.pool_blocks_for(w, lens))
    ctx = W.context_lengths(inp)
    cap = H.tables_capacity(int(ctx.max()), w.block_size)
    nat = H.build_native(inp, w.block_size, cap)
    orc = H.build_oracle(inp, w.block_size)
    kc, vc = _fill_fp8(inp, nat, ks, vs)
    kp, vp = _oracle_codes(inp, orc, ks, vs)
    outs, want = _decode_fp8_both(inp, nat, orc, kc, vc, kp, vp, ks, vs)
    _log(f"{w.name} {spec} scales {ks:.4f} {vs:.4f} contexts "
         f"{int(ctx.min())}..{int(ctx.max())}")
    _check(outs, want, w.name)
    assert np.array_equal(outs["paged"], outs["contig"])


# ------------------------------------------------------- per-head scales --
def _head_scales(seed, hkv):
    """Seeded per-head K and V scales, spread over a factor of about 8 so
    that a scale taken from the wrong head changes the codes."""
    g = np.random.default_rng([4000, seed])
    return (g.uniform(0.006, 0.05, hkv).astype(np.float32),
            g.uniform(0.006, 0.05, hkv).astype(np.float32))


def test_fp8_per_head_cache_write_bit_exact():
    w = _small_workload(seed=13)
    inp = W.draw(w, lambda lens: H.pool_blocks_for(w, lens, 4))
    cap = H.tables_capacity(int(W.context_lengths(inp).max()), w.block_size)
    nat = H.build_native(inp, w.block_size, cap)
    orc = H.build_oracle(inp, w.block_size)
    ks, vs = _head_scales(0, w.num_kv_heads)
    kc, vc = _fill_fp8(inp, nat, ks, vs)
    kp, vp = _oracle_codes(inp, orc, ks, vs)
    assert np.array_equal(kc.permute(0, 2, 1, 3).cpu().numpy(), kp)
    assert np.array_equal(vc.permute(0, 2, 1, 3).cpu().numpy(), vp)
    # the per-head codes differ from those of any single tensor scale
    kp0, _ = _oracle_codes(inp, orc, float(ks[0]), float(vs[0]))
    assert not np.array_equal(kp, kp0)


def test_fp8_per_head_special_values():
    """NaN (both signs), infinities and saturation under per-head scales."""
    D, hkv = 128, 2
    g = np.random.default_rng(8)
    rows = g.standard_normal((3, hkv, D)).astype(np.float32) * 60
    rows[0, 0, 2:4] = [np.inf, -np.inf]
    rows[1, 1, :2] = [1e30, -1e30]
    k = torch.from_numpy(rows).to(torch.bfloat16)
    v = torch.from_numpy(-rows).to(torch.bfloat16)
    # NaNs of both signs, as bf16 bit patterns (torch's fp32 -> bf16
    # conversion would make every NaN 0xFFFF)
    for t in (k, v):
        bits = t.view(torch.int16)
        bits[0, 0, 0] = 0x7FC0                 # +NaN
        bits[0, 0, 1] = -64                    # 0xFFC0, -NaN
        bits[1, 1, 2] = 0x7F81                 # +NaN, low payload
    ks = np.array([0.5, 0.02], dtype=np.float32)
    vs = np.array([3.0, 0.0123], dtype=np.float32)
    kc = torch.full((2, hkv, 16, D), NAN_CODE, dtype=torch.uint8,
                    device="cuda")
    vc = torch.full_like(kc, NAN_CODE)
    slots = torch.tensor([17, -1, 2], dtype=torch.int64, device="cuda")
    _write_fp8(k.cuda(), v.cuda(), slots, kc, vc, ks, vs)
    torch.cuda.synchronize()
    want_k = F.quantize(k.float().numpy(), _inv(ks))
    want_v = F.quantize(v.float().numpy(), _inv(vs))
    got_k = kc.permute(0, 2, 1, 3).cpu().numpy()
    got_v = vc.permute(0, 2, 1, 3).cpu().numpy()
    for t, slot in ((0, 17), (2, 2)):
        b, o = divmod(slot, 16)
        assert np.array_equal(got_k[b, o], want_k[t]), t
        assert np.array_equal(got_v[b, o], want_v[t]), t
    assert want_k[0, 0, :2].tolist() == [0x7F, 0xFF]
    assert want_k[1, 1, 2] == 0x7F
    # the padded row (slot -1) wrote nothing
    written = {(1, 1), (0, 2)}
    for b in range(2):
        for o in range(16):
            if (b, o) not in written:
                assert (got_k[b, o] == NAN_CODE).all()
                assert (got_v[b, o] == NAN_CODE).all()


def test_fp8_per_head_append_token():
    """The device append with per-head scales equals the per-head cache
    write of the same rows into the same slots, and the oracle's codes."""
    w = _small_workload(seed=14)
    S, B, hkv, D = w.num_seqs, w.block_size, w.num_kv_heads, w.head_dim
    ks, vs = _head_scales(1, hkv)
    g = np.random.default_rng(15)
    lens = np.array(w.lengths, dtype=np.int32)
    cap = H.tables_capacity(int(lens.max()) + 1, B)
    n_pool = sum(-(-int(n + 1) // B) for n in lens) + 4
    pool = kv.KVPool(n_pool, B)
    table = np.full((S, cap), -1, dtype=np.int32)
    cur = np.zeros(S, dtype=np.int32)
    pool.seq_append(table, cur, lens)
    before = table.copy()
    _, pairs = pool.seq_append(table, cur)          # one more token each
    assert len(pairs) == 0
    newb = np.where(table != before, table, -1).max(axis=1).astype(np.int32)
    rows = torch.from_numpy(
        g.standard_normal((S, hkv, D)).astype(np.float32) * 5).to(
        torch.bfloat16)
    vrows = torch.from_numpy(
        g.standard_normal((S, hkv, D)).astype(np.float32) * 5).to(
        torch.bfloat16)
    kc = torch.full((n_pool, hkv, B, D), NAN_CODE, dtype=torch.uint8,
                    device="cuda")
    vc = torch.full_like(kc, NAN_CODE)
    kc2, vc2 = kc.clone(), vc.clone()
    d_table = torch.from_numpy(before).cuda()
    d_lens = torch.from_numpy(lens.copy()).cuda()
    kv.kv_append_token_fp8_per_head(rows.cuda(), vrows.cuda(),
                                    torch.from_numpy(newb).cuda(), d_table,
                                    d_lens, kc, vc, _dev_scales(ks),
                                    _dev_scales(vs))
    slots = np.array([table[s, lens[s] // B] * B + lens[s] % B
                      for s in range(S)], dtype=np.int64)
    _write_fp8(rows.cuda(), vrows.cuda(), torch.from_numpy(slots).cuda(),
               kc2, vc2, ks, vs)
    torch.cuda.synchronize()
    assert torch.equal(kc, kc2) and torch.equal(vc, vc2)
    assert np.array_equal(d_table.cpu().numpy(), table)
    assert np.array_equal(d_lens.cpu().numpy(), lens + 1)
    want_k = F.quantize(rows.float().numpy(), _inv(ks))
    got_k = kc.permute(0, 2, 1, 3).cpu().numpy()
    for s in range(S):
        b, o = divmod(int(slots[s]), B)
        assert np.array_equal(got_k[b, o], want_k[s]), s
    pool.close()


def test_decode_fp8_per_head_small():
    w = _small_workload(seed=16)
    inp = W.draw(w, lambda lens: H.pool_blocks_for(w, lens, 4))
    cap = H.tables_capacity(int(W.context_lengths(inp).max()), w.block_size)
    nat = H.build_native(inp, w.block_size, cap)
    orc = H.build_oracle(inp, w.block_size)
    ks, vs = _head_scales(2, w.num_kv_heads)
    kc, vc = _fill_fp8(inp, nat, ks, vs)
    kp, vp = _oracle_codes(inp, orc, ks, vs)
    outs, want = _decode_fp8_both(inp, nat, orc, kc, vc, kp, vp, ks, vs)
    _check(outs, want, "fp8_per_head_small")
    assert np.array_equal(outs["paged"], outs["contig"])


@pytest.mark.parametrize("seed", range(4))
def test_decode_fp8_per_head_random_shapes(seed):
    """Random shapes as above with one scale per KV head."""
    spec, _ = _fp8_shape(seed + 8)
    w = W.WORKLOADS["llama3_8b_decode"].replace(name=f"fp8_ph_rand_{seed}",
                                               seed=3100 + seed, **spec)
    inp = W.draw(w, lambda lens: H.pool_blocks_for(w, lens))
    ctx = W.context_lengths(inp)
    cap = H.tables_capacity(int(ctx.max()), w.block_size)
    nat = H.build_native(inp, w.block_size, cap)
    orc = H.build_oracle(inp, w.block_size)
    ks, vs = _head_scales(10 + seed, w.num_kv_heads)
    kc, vc = _fill_fp8(inp, nat, ks, vs)
    kp, vp = _oracle_codes(inp, orc, ks, vs)
    outs, want = _decode_fp8_both(inp, nat, orc, kc, vc, kp, vp, ks, vs)
    _log(f"{w.name} {spec} per-head scales contexts "
         f"{int(ctx.min())}..{int(ctx.max())}")
    _check(outs, want, w.name)
    assert np.array_equal(outs["paged"], outs["contig"])


def test_fp8_per_head_errors():
    k = torch.zeros((2, 2, 128), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((1, 2, 16, 128), dtype=torch.uint8, device="cuda")
    slots = torch.zeros(2, dtype=torch.int64, device="cuda")
    good = torch.ones(2, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):      # one scale per KV head
        kv.kv_reshape_and_cache_fp8_per_head(
            k, k, slots, kc, kc.clone(), torch.ones(3, device="cuda"), good)
    with pytest.raises(TypeError):
        kv.kv_reshape_and_cache_fp8_per_head(
            k, k, slots, kc, kc.clone(), good.double(), good)
    st = kv.lib().kv_reshape_and_cache_fp8_per_head(
        k.data_ptr(), k.data_ptr(), slots.data_ptr(), 2, kc.data_ptr(),
        kc.data_ptr(), 16, 16, 2, 128, None, good.data_ptr(), None)
    assert st == kv.KV_EINVAL


# ------------------------------------------------- decode with the append --
def _fill_fp8_upto(inp, nat, stored, k_scale, v_scale):
    """fp8 paged caches holding the first stored[s] rows of each sequence
    (the native tables were built up to those lengths)."""
    w = inp.workload
    B, S = w.block_size, w.num_seqs
    kc = torch.full(tuple(nat.k_cache.shape), NAN_CODE, dtype=torch.uint8,
                    device="cuda")
    vc = torch.full_like(kc, NAN_CODE)
    n = [int(x) for x in stored]
    if sum(n):
        seq_ids = np.concatenate([np.full(c, s, dtype=np.int32)
                                  for s, c in enumerate(n)])
        pos = np.concatenate([np.arange(c, dtype=np.int32) for c in n])
        slots = kv.kv_slot_mapping(nat.tables, seq_ids, pos, B)
        rows = np.concatenate([W.logical_rows(inp, s)[:c]
                               for s, c in enumerate(n)])
        r = torch.from_numpy(rows)
        _write_fp8(inp.k[r].cuda(), inp.v[r].cuda(),
                   torch.from_numpy(slots).cuda(), kc, vc, k_scale, v_scale)
    torch.cuda.synchronize()
    return kc, vc


def _append_fp8_step(inp, stored, ks, vs, fused, max_context=None):
    """One decode step that appends each sequence's next row (position
    stored[s] of the draw) to fp8 caches holding stored[s] rows: fused
    (paged_attn_decode_append_fp8[_per_head]) or as the two calls. Returns
    (out, k codes, v codes, table, lengths)."""
    w = inp.workload
    B, S = w.block_size, w.num_seqs
    ctx = np.asarray(stored, dtype=np.int32) + 1
    cap = H.tables_capacity(int(ctx.max()), B)
    nat = H.build_native(inp, B, cap, upto=stored)
    kc, vc = _fill_fp8_upto(inp, nat, stored, ks, vs)
    bt = torch.from_numpy(nat.tables).cuda()
    lens = torch.from_numpy(nat.lens.copy()).cuda()
    # the host allocator takes the blocks the new tokens start
    idx = np.minimum(nat.lens // B, cap - 1)
    before = nat.tables[np.arange(S), idx].copy()
    _, pairs = nat.pool.seq_append(nat.tables, nat.lens)
    assert len(pairs) == 0
    after = nat.tables[np.arange(S), idx]
    newb = torch.from_numpy(
        np.where(after != before, after, -1).astype(np.int32)).pin_memory()
    rows = torch.from_numpy(np.array(
        [W.logical_rows(inp, s)[int(stored[s])] for s in range(S)]))
    k_new = inp.k[rows].cuda().contiguous()
    v_new = inp.v[rows].cuda().contiguous()
    q = inp.q.cuda()
    out = torch.full_like(q, float("nan"))
    scale = H.scale_of(w)
    mc = int(ctx.max()) if max_context is None else max_context
    if _per_head(ks):
        dks, dvs = _dev_scales(ks), _dev_scales(vs)
        if fused:
            kv.paged_attn_decode_append_fp8_per_head(
                out, q, k_new, v_new, newb, kc, vc, bt, lens, mc, scale, dks,
                dvs)
        else:
            kv.kv_append_token_fp8_per_head(k_new, v_new, newb, bt, lens, kc,
                                            vc, dks, dvs)
            kv.paged_attn_decode_fp8_per_head(out, q, kc, vc, bt, lens, mc,
                                              scale, dks, dvs)
    else:
        if fused:
            kv.paged_attn_decode_append_fp8(out, q, k_new, v_new, newb, kc,
                                            vc, bt, lens, mc, scale, ks, vs)
        else:
            kv.kv_append_token_fp8(k_new, v_new, newb, bt, lens, kc, vc, ks,
                                   vs)
            kv.paged_attn_decode_fp8(out, q, kc, vc, bt, lens, mc, scale, ks,
                                     vs)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), kc, vc, bt, lens


def _within_rounding(got, ref):
    """The fused op and the two calls differ by the output's rounding to
    bf16 (2^-7 relative allowed) plus the new token's weight taken in fp32
    rather than as a bf16 MFMA operand (4e-3 absolute allowed)."""
    bound = 2.0 ** -7 * np.maximum(np.abs(got), np.abs(ref)) + 4e-3
    bad = np.abs(got - ref) > bound
    assert not bad.any(), (np.argwhere(bad)[:5], got[bad][:5], ref[bad][:5])


def _fused_vs_two_calls(inp, stored, ks, vs, seqs=None):
    w = inp.workload
    ctx = np.asarray(stored, dtype=np.int32) + 1
    of, kf, vf, btf, lf = _append_fp8_step(inp, stored, ks, vs, True)
    ou, ku, vu, btu, lu = _append_fp8_step(inp, stored, ks, vs, False)
    # the same codes, table and lengths, bit for bit
    assert torch.equal(kf, ku) and torch.equal(vf, vu)
    assert torch.equal(btf, btu) and torch.equal(lf, lu)
    assert lf.cpu().numpy().tolist() == ctx.tolist()
    _within_rounding(of, ou)
    # and the oracle over the codes of every context row
    orc = H.build_oracle(inp, w.block_size)
    kp, vp = _oracle_codes(inp, orc, ks, vs, seqs=seqs)
    want = O.decode_paged(inp.q.float().numpy(), _dequant_pool(kp, ks),
                          _dequant_pool(vp, vs), orc.tables, ctx,
                          H.scale_of(w), seqs=seqs)
    sel = slice(None) if seqs is None else list(seqs)
    err = H.max_abs(of[sel], want[sel])
    _log(f"{w.name}: fused fp8 vs two calls max-abs "
         f"{H.max_abs(of, ou):.2e}, vs oracle {err:.2e}")
    assert err <= 2e-2, err


@pytest.mark.parametrize("spec", ["tensor", "head"])
def test_decode_append_fp8_small(spec):
    """First token of a sequence, the last and first slots of a block, and
    longer contexts: the fused fp8 op against the two calls and the
    oracle, with one scale per tensor or per KV head."""
    w = _small_workload(seed=17)
    inp = W.draw(w, lambda lens: H.pool_blocks_for(w, lens, 4))
    stored = W.context_lengths(inp).astype(np.int32) - 1
    ks, vs = ((0.0123, 0.02) if spec == "tensor"
              else _head_scales(5, w.num_kv_heads))
    _fused_vs_two_calls(inp, stored, ks, vs)


def test_decode_append_fp8_workload_shape():
    """The Llama-3-8B batch (64 sequences, 32 / 8 heads, block 16) with
    per-head scales; the oracle on sampled sequences."""
    w = W.WORKLOADS["llama3_8b_decode"]
    inp = W.draw(w, lambda lens: H.pool_blocks_for(w, lens, w.num_seqs))
    stored = W.context_lengths(inp).astype(np.int32) - 1
    ks, vs = _head_scales(6, w.num_kv_heads)
    _fused_vs_two_calls(inp, stored, ks, vs, seqs=[0, 17, 40, 63])


def test_decode_append_fp8_many_sequences():
    """More sequences than one launch takes (4096), per-head scales: every
    launch copies its block ids and the reciprocal scales into the shared
    workspace."""
    w = _small_workload(seed=19).replace(
        num_seqs=4100, lengths=None, length_range=(1, 48), num_q_heads=8,
        num_kv_heads=2, name="fp8_append_many_seqs")
    inp = W.draw(w, lambda lens: H.pool_blocks_for(w, lens, w.num_seqs))
    stored = W.context_lengths(inp).astype(np.int32) - 1
    _fused_vs_two_calls(inp, stored, *_head_scales(9, w.num_kv_heads))


@pytest.mark.parametrize("hq,hkv", [(56, 8), (8, 8)])
def test_decode_append_fp8_head_groups(hq, hkv):
    """Head groups of 7 and of 1 per KV head."""
    lengths = (1, 31, 32, 33, 400, 64)
    w = _small_workload(seed=18).replace(
        num_seqs=len(lengths), lengths=lengths, num_q_heads=hq,
        num_kv_heads=hkv, name=f"fp8_append_g{hq // hkv}")
    inp = W.draw(w, lambda lens: H.pool_blocks_for(w, lens, 8))
    stored = np.array(lengths, dtype=np.int32) - 1
    _fused_vs_two_calls(inp, stored, *_head_scales(7, hkv))


def test_decode_append_fp8_errors():
    """Shapes the fp8 decode does not cover fail before anything is
    written; a missing scale array is refused."""
    S, hkv, D = 2, 2, 128
    q = torch.zeros((S, 4, D), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    k_new = torch.zeros((S, hkv, D), dtype=torch.bfloat16, device="cuda")
    newb = torch.tensor([0, 1], dtype=torch.int32).pin_memory()
    bt = torch.zeros((S, 2), dtype=torch.int32, device="cuda")
    lens = torch.zeros(S, dtype=torch.int32, device="cuda")
    kc8 = torch.full((4, hkv, 8, D), NAN_CODE, dtype=torch.uint8,
                     device="cuda")
    with pytest.raises(kv.KVError):      # block_size 8
        kv.paged_attn_decode_append_fp8(out, q, k_new, k_new, newb, kc8,
                                        kc8.clone(), bt, lens, 16, 0.1, 1.0,
                                        1.0)
    torch.cuda.synchronize()
    assert (kc8 == NAN_CODE).all() and (lens == 0).all()
    kc = torch.full((4, hkv, 16, D), NAN_CODE, dtype=torch.uint8,
                    device="cuda")
    with pytest.raises(kv.KVError):      # scale must be > 0
        kv.paged_attn_decode_append_fp8(out, q, k_new, k_new, newb, kc,
                                        kc.clone(), bt, lens, 32, 0.1, 0.0,
                                        1.0)
    good = torch.ones(hkv, dtype=torch.float32, device="cuda")
    ws = kv.decode_workspace(S, 4, hkv, D, 32, q.device)
    st = kv.lib().paged_attn_decode_append_fp8_per_head(
        out.data_ptr(), q.data_ptr(), k_new.data_ptr(), k_new.data_ptr(),
        newb.data_ptr(), kc.data_ptr(), kc.data_ptr(), 4, bt.data_ptr(), 2,
        lens.data_ptr(), 32, S, 4, hkv, D, 16, 0.1, None, good.data_ptr(),
        ws.data_ptr(), ws.numel(), None)
    assert st == kv.KV_EINVAL
    torch.cuda.synchronize()
    assert (kc == NAN_CODE).all() and (lens == 0).all()
