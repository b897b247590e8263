"""Pins of the fp64 oracle against things other than itself: the pages'
worked example, hand-worked fixtures, closed forms, brute force in 50-digit
decimal arithmetic, torch's scaled_dot_product_attention in float64 on the
CPU, and invariants the pages state."""
import json
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest
import torch

from oracle import allocator as A
from oracle import attention as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- blocks --
def test_worked_example_block_count():
    g = _golden("worked_example.json")
    assert O.blocks_needed(g["tokens"], g["block_size"]) == g["blocks"]
    assert O.unused_slots(g["tokens"], g["block_size"]) == g["unused_slots"]


def test_worked_example_through_allocator():
    g = _golden("worked_example.json")
    pool = A.ModelPool(8, g["block_size"])
    tables, lens = [[]], [0]
    st, slots, pairs = A.append_tokens(pool, tables, lens, [g["tokens"]], 8)
    assert st == A.OK and pairs == []
    assert len(tables[0]) == g["blocks"]
    assert len(tables[0]) * g["block_size"] - lens[0] == g["unused_slots"]
    assert pool.num_free() == 8 - g["blocks"]


def test_decode_tiny_block_counts():
    g = _golden("decode_tiny_blocks.json")
    B = g["block_size"]
    assert [O.blocks_needed(n, B) for n in g["lengths"]] == g["blocks"]
    assert [O.unused_slots(n, B) for n in g["lengths"]] == g["unused_slots"]
    assert O.pool_blocks_exact(g["lengths"], B) == g["total_blocks"]
    assert O.waste_fraction(g["lengths"], B) == pytest.approx(
        g["total_unused"] / g["allocated_slots"])


def test_waste_confined_to_last_block():
    # Only the last block may hold empty slots: 0 <= waste <= B-1.
    for B in (1, 2, 3, 7, 16, 64):
        for n in range(0, 300):
            w = O.unused_slots(n, B)
            assert 0 <= w <= B - 1
            if n == 0:
                assert O.blocks_needed(n, B) == 0
            else:
                # all blocks but the last are full
                assert (O.blocks_needed(n, B) - 1) * B < n <= O.blocks_needed(n, B) * B


# ------------------------------------------------------------------ slots --
def test_slot_example():
    g = _golden("slot_example.json")
    got = [O.slot_of(g["table"], p, g["block_size"]) for p in g["positions"]]
    assert got == g["slots"]
    got2 = O.slot_mapping([g["table"]], [0] * len(g["positions"]),
                          g["positions"], g["block_size"])
    assert got2.tolist() == g["slots"]
    assert O.slot_mapping([g["table"]], [0], [-1], 4).tolist() == [-1]


def test_slot_bijection():
    rng = np.random.default_rng(11)
    B = 8
    lens = [37, 8, 1, 64, 0, 15]
    pool = A.ModelPool(64, B, free_order=rng.permutation(64))
    tables, cur = [[] for _ in lens], [0] * len(lens)
    st, slots, _ = A.append_tokens(pool, tables, cur, lens, 64)
    assert st == A.OK
    seen = set()
    for s, n in enumerate(lens):
        own = [O.slot_of(tables[s], p, B) for p in range(n)]
        assert len(set(own)) == n
        assert all(x // B in tables[s] for x in own)
        assert not (seen & set(own))
        seen |= set(own)
    assert len(seen) == sum(lens)
    assert slots == [O.slot_of(tables[s], p, B)
                     for s, n in enumerate(lens) for p in range(n)]



def test_scatter_skips_padding_slots():
    # A negative slot is padding: nothing is written anywhere (in particular
    # not at the pool's last slot, where a negative index would land).
    pool = np.full((3, 4, 1, 2), np.nan)
    rows = np.arange(8, dtype=np.float64).reshape(4, 1, 2)
    O.scatter_rows(pool, rows, [-1, 5, -1, 2])
    want = np.full((3, 4, 1, 2), np.nan)
    want[1, 1] = rows[1]          # slot 5 = block 1, offset 1
    want[0, 2] = rows[3]          # slot 2 = block 0, offset 2
    assert np.array_equal(pool, want, equal_nan=True)

# --------------------------------------------------------------- softmax --
def _decimal_attend(q, K, V, scale):
    getcontext().prec = 50
    qd = [Decimal(float(x)) for x in q]
    sc = Decimal(float(scale))
    ws = []
    for row in K:
        z = sc * sum(Decimal(float(a)) * b for a, b in zip(row, qd))
        ws.append(z.exp())
    den = sum(ws)
    out = []
    for e in range(V.shape[1]):
        num = sum(w * Decimal(float(V[j, e])) for j, w in enumerate(ws))
        out.append(float(num / den))
    return np.array(out)


@pytest.mark.parametrize("seed", range(12))
def test_attend_matches_decimal_bruteforce(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 6))
    d = int(rng.integers(1, 5))
    q = rng.normal(size=d) * 3
    K = rng.normal(size=(n, d)) * 3
    V = rng.normal(size=(n, d))
    scale = float(rng.uniform(0.1, 2.0))
    got = O.attend(q, K, V, scale)
    want = _decimal_attend(q, K, V, scale)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_attend_partial_matches_decimal():
    rng = np.random.default_rng(5)
    q = rng.normal(size=3)
    K = rng.normal(size=(4, 3))
    V = rng.normal(size=(4, 3))
    m, l, acc = O.attend_partial(q, K, V, 0.7)
    np.testing.assert_allclose(acc / l, _decimal_attend(q, K, V, 0.7),
                               atol=1e-12, rtol=0)


# ---------------------------------------------- library cross-check (SDPA) --
def _sdpa(q, k, v, scale, causal=False, mask=None):
    """torch SDPA in float64 on the CPU; q [Hq, T, D], k/v [Hkv, L, D]."""
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None],
        torch.from_numpy(v)[None], attn_mask=mask, is_causal=causal,
        scale=scale, enable_gqa=True)[0].numpy()


@pytest.mark.parametrize("hq,hkv", [(8, 8), (32, 8), (56, 8), (4, 1)])
def test_decode_matches_sdpa(hq, hkv):
    rng = np.random.default_rng(hq * 100 + hkv)
    d, lens, scale = 16, [1, 5, 40], 0.25
    q = rng.normal(size=(len(lens), hq, d))
    ks = [rng.normal(size=(n, hkv, d)) for n in lens]
    vs = [rng.normal(size=(n, hkv, d)) for n in lens]
    got = O.decode_logical(q, ks, vs, scale)
    for s, n in enumerate(lens):
        want = _sdpa(q[s][:, None, :], ks[s].transpose(1, 0, 2),
                     vs[s].transpose(1, 0, 2), scale)[:, 0, :]
        np.testing.assert_allclose(got[s], want, atol=1e-12, rtol=0)


def test_causal_prefill_matches_sdpa():
    rng = np.random.default_rng(3)
    hq, hkv, d, n, scale = 8, 2, 16, 37, 0.3
    q = rng.normal(size=(n, hq, d))
    k = rng.normal(size=(n, hkv, d))
    v = rng.normal(size=(n, hkv, d))
    got = O.prefill_logical(q, [0, n], [0], [k], [v], scale, causal=True)
    want = _sdpa(q.transpose(1, 0, 2), k.transpose(1, 0, 2),
                 v.transpose(1, 0, 2), scale, causal=True).transpose(1, 0, 2)
    np.testing.assert_allclose(got, want, atol=1e-12, rtol=0)


def test_noncausal_prefill_matches_sdpa():
    rng = np.random.default_rng(4)
    hq, hkv, d, nq, L, scale = 4, 2, 8, 5, 19, 0.5
    q = rng.normal(size=(nq, hq, d))
    k = rng.normal(size=(L, hkv, d))
    v = rng.normal(size=(L, hkv, d))
    got = O.prefill_logical(q, [0, nq], [L - nq], [k], [v], scale,
                            causal=False)
    want = _sdpa(q.transpose(1, 0, 2), k.transpose(1, 0, 2),
                 v.transpose(1, 0, 2), scale).transpose(1, 0, 2)
    np.testing.assert_allclose(got, want, atol=1e-12, rtol=0)


# ---------------------------------------------------------- closed forms --
def test_single_key_returns_its_value_exactly():
    rng = np.random.default_rng(0)
    V = rng.normal(size=(1, 6))
    o = O.attend(rng.normal(size=6), rng.normal(size=(1, 6)), V, 0.125)
    assert np.array_equal(o, V[0])


def test_zero_query_gives_mean_of_values():
    rng = np.random.default_rng(1)
    V = rng.normal(size=(9, 4))
    o = O.attend(np.zeros(4), rng.normal(size=(9, 4)), V, 1.0)
    np.testing.assert_allclose(o, V.mean(axis=0), atol=1e-14, rtol=0)


def test_equal_keys_give_mean_of_values():
    rng = np.random.default_rng(2)
    K = np.tile(rng.normal(size=(1, 4)), (7, 1))
    V = rng.normal(size=(7, 4))
    o = O.attend(rng.normal(size=4), K, V, 1.0)
    np.testing.assert_allclose(o, V.mean(axis=0), atol=1e-14, rtol=0)


def test_dominant_logit_selects_its_value():
    rng = np.random.default_rng(3)
    K = np.zeros((6, 2))
    K[4] = [50.0, 0.0]
    V = rng.normal(size=(6, 3))
    o = O.attend(np.array([1.0, 0.0]), K, V, 1.0)
    np.testing.assert_allclose(o, V[4], atol=1e-20 + 6 * np.exp(-50) * 5,
                               rtol=0)


def test_empty_context_gives_zeros():
    assert np.array_equal(O.attend(np.ones(3), np.zeros((0, 3)),
                                   np.zeros((0, 3)), 1.0), np.zeros(3))


# ------------------------------------------------------------ invariants --
def _paged_setup(lens, B, n_pool, order_seed, hkv=2, d=4, data_seed=0):
    rng = np.random.default_rng(data_seed)
    ks = [rng.normal(size=(n, hkv, d)) for n in lens]
    vs = [rng.normal(size=(n, hkv, d)) for n in lens]
    order = np.random.default_rng(order_seed).permutation(n_pool)
    pool = A.ModelPool(n_pool, B, free_order=order)
    tables, cur = [[] for _ in lens], [0] * len(lens)
    st, slots, _ = A.append_tokens(pool, tables, cur, lens, 64)
    assert st == A.OK
    kp = np.full((n_pool, B, hkv, d), np.nan)
    vp = np.full((n_pool, B, hkv, d), np.nan)
    O.scatter_rows(kp, np.concatenate(ks), slots)
    O.scatter_rows(vp, np.concatenate(vs), slots)
    return ks, vs, kp, vp, tables


def test_physical_permutation_invariance_and_contig_equality():
    lens, B = [35, 16, 1, 100], 16
    q = np.random.default_rng(9).normal(size=(4, 4, 4))
    outs = []
    for order_seed in (1, 2, 3):
        ks, vs, kp, vp, tables = _paged_setup(lens, B, 32, order_seed)
        outs.append(O.decode_paged(q, kp, vp, tables, lens, 0.5))
    assert np.array_equal(outs[0], outs[1])
    assert np.array_equal(outs[0], outs[2])
    assert np.isfinite(outs[0]).all()  # NaN-filled unused slots never read
    Lmax = max(lens)
    kc = np.full((4, Lmax, 2, 4), np.nan)
    vc = np.full((4, Lmax, 2, 4), np.nan)
    for s, n in enumerate(lens):
        kc[s, :n] = ks[s]
        vc[s, :n] = vs[s]
    assert np.array_equal(outs[0], O.decode_contig(q, kc, vc, lens, 0.5))
    assert np.array_equal(outs[0], O.decode_logical(q, ks, vs, 0.5))


def test_chunked_prefill_equals_one_shot():
    rng = np.random.default_rng(21)
    n, C, hq, hkv, d = 50, 16, 4, 2, 8
    q = rng.normal(size=(n, hq, d))
    k = rng.normal(size=(n, hkv, d))
    v = rng.normal(size=(n, hkv, d))
    one = O.prefill_logical(q, [0, n], [0], [k], [v], 0.3, causal=True)
    parts = []
    for c0 in range(0, n, C):
        c1 = min(n, c0 + C)
        parts.append(O.prefill_logical(q[c0:c1], [0, c1 - c0], [c0],
                                       [k[:c1]], [v[:c1]], 0.3, causal=True))
    assert np.array_equal(np.concatenate(parts), one)


def test_prefill_paged_equals_contig():
    lens, B = [20, 33], 8
    ks, vs, kp, vp, tables = _paged_setup(lens, B, 16, 4, hkv=2, d=4)
    rng = np.random.default_rng(8)
    nq = [5, 9]
    q = rng.normal(size=(sum(nq), 4, 4))
    cu = [0, nq[0], nq[0] + nq[1]]
    start = [lens[0] - nq[0], lens[1] - nq[1]]
    a = O.prefill_paged(q, cu, start, kp, vp, tables, lens, 0.5, True)
    kc = np.full((2, 40, 2, 4), np.nan)
    vc = np.full((2, 40, 2, 4), np.nan)
    for s, n in enumerate(lens):
        kc[s, :n], vc[s, :n] = ks[s], vs[s]
    b = O.prefill_contig(q, cu, start, kc, vc, lens, 0.5, True)
    assert np.array_equal(a, b)
    assert np.isfinite(a).all()


@pytest.mark.parametrize("seed", range(6))
def test_split_merge_equals_unsplit(seed):
    rng = np.random.default_rng(seed)
    n, d = int(rng.integers(1, 300)), 8
    q = rng.normal(size=d) * 2
    K = rng.normal(size=(n, d)) * 2
    V = rng.normal(size=(n, d))
    cuts = sorted(set(rng.integers(0, n + 1, size=5).tolist()) | {0, n})
    parts = [O.attend_partial(q, K[a:b], V[a:b], 0.3)
             for a, b in zip(cuts[:-1], cuts[1:])]
    np.testing.assert_allclose(O.merge_partials(parts),
                               O.attend(q, K, V, 0.3), atol=1e-12, rtol=0)


def test_copy_blocks_copies_whole_blocks_in_order():
    pool = np.arange(4 * 2 * 3, dtype=np.float64).reshape(4, 2, 3)
    orig = pool.copy()
    O.copy_blocks(pool, [(0, 2), (2, 3)])
    assert np.array_equal(pool[2], orig[0])
    assert np.array_equal(pool[3], orig[0])  # sequential: 2 already holds 0
    assert np.array_equal(pool[0], orig[0])
    assert np.array_equal(pool[1], orig[1])
