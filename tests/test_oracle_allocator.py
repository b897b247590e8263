"""Pins of the model allocator: a hand-worked trace of the FIFO/refcount
policy, the pages' worked example, invariants over random operation
sequences, and the copy-on-write fan-out of a shared half-full block."""
import json
import os

import numpy as np
import pytest

from oracle import allocator as A
from oracle import attention as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _run_op(pool, op):
    kind = op["op"]
    if kind == "alloc":
        st, ids = pool.alloc(op["n"])
        return {"status": st, "ids": ids}
    if kind == "free":
        return {"status": pool.free_blocks(op["ids"])}
    if kind == "share":
        return {"status": pool.share(op["ids"])}
    if kind == "cow":
        st, out, need = pool.cow(op["id"])
        return {"status": st, "out": out, "need_copy": need}
    raise ValueError(kind)


def test_golden_trace():
    with open(os.path.join(GOLDEN, "allocator_trace.json")) as f:
        g = json.load(f)
    pool = A.ModelPool(g["num_blocks"], g["block_size"], g["free_order"])
    for op in g["ops"]:
        got = _run_op(pool, op)
        assert got["status"] == op["status"], op
        for key in ("ids", "out", "need_copy"):
            if key in op and key in got:
                assert got[key] == op[key], op
        if "num_free" in op:
            assert pool.num_free() == op["num_free"], op
        for b, rc in op.get("refcount", {}).items():
            assert pool.refcount(int(b)) == rc, op


def _check_invariants(pool, refs):
    live = {b for b in range(pool.num_blocks) if pool.rc[b] > 0}
    free = set(pool.free)
    assert len(free) == len(pool.free)          # no duplicates in the queue
    assert not (live & free)
    assert len(live) + len(free) == pool.num_blocks
    assert sum(pool.rc) == sum(refs.values())
    for b, n in refs.items():
        assert pool.rc[b] == n


@pytest.mark.parametrize("seed", range(20))
def test_random_traces_keep_invariants(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 9))
    pool = A.ModelPool(n, 4, rng.permutation(n))
    refs = {}
    for _ in range(200):
        r = rng.integers(0, 4)
        if r == 0:
            st, ids = pool.alloc(int(rng.integers(0, 4)))
            if st == A.OK:
                for b in ids:
                    refs[b] = 1
        elif r == 1 and refs:
            b = int(rng.choice(list(refs)))
            assert pool.free_blocks([b]) == A.OK
            refs[b] -= 1
            if refs[b] == 0:
                del refs[b]
        elif r == 2 and refs:
            b = int(rng.choice(list(refs)))
            assert pool.share([b]) == A.OK
            refs[b] += 1
        elif r == 3 and refs:
            b = int(rng.choice(list(refs)))
            before = pool.num_free()
            st, out, need = pool.cow(b)
            if st == A.OK and need:
                refs[b] -= 1
                refs[out] = 1
                assert pool.num_free() == before - 1
            elif st == A.OK:
                assert out == b and refs[b] == 1
            else:
                assert st == A.ENOMEM and before == 0
        _check_invariants(pool, refs)
    for b, c in list(refs.items()):
        assert pool.free_blocks([b] * c) == A.OK
    assert pool.num_free() == n


def test_free_order_is_fifo():
    pool = A.ModelPool(5, 2, [4, 3, 2, 1, 0])
    assert pool.alloc(5) == (A.OK, [4, 3, 2, 1, 0])
    assert pool.free_blocks([1, 3, 0]) == A.OK
    assert list(pool.free) == [1, 3, 0]
    assert pool.alloc(2) == (A.OK, [1, 3])


def test_errors_leave_state_unchanged():
    pool = A.ModelPool(3, 2)
    assert pool.alloc(4) == (A.ENOMEM, [])
    assert pool.num_free() == 3
    assert pool.alloc(-1)[0] == A.EINVAL
    st, ids = pool.alloc(1)
    assert pool.free_blocks([ids[0], ids[0]]) == A.EREFCOUNT
    assert pool.refcount(ids[0]) == 1
    assert pool.share([ids[0], 7]) == A.EINVAL
    assert pool.refcount(ids[0]) == 1
    assert pool.cow(9)[0] == A.EINVAL
    assert pool.refcount(99) == A.EINVAL


def test_append_all_or_nothing():
    pool = A.ModelPool(3, 4)
    tables, lens = [[], []], [0, 0]
    st, slots, pairs = A.append_tokens(pool, tables, lens, [8, 8], 8)
    assert st == A.ENOMEM and slots == [] and pairs == []
    assert tables == [[], []] and lens == [0, 0] and pool.num_free() == 3
    st, slots, _ = A.append_tokens(pool, tables, lens, [3, 1], 1)
    assert st == A.OK and lens == [3, 1]
    st, _, _ = A.append_tokens(pool, tables, lens, [2, 0], 1)  # needs block 1
    assert st == A.EINVAL and lens == [3, 1]


def test_copy_on_write_fanout_of_half_full_shared_block():
    # A parent with 2.5 blocks of prefix is forked into 4 sequences that
    # share every block; each then appends one token in ascending order.
    B, n_seq = 4, 4
    pool = A.ModelPool(16, B, list(range(16)))
    tables, lens = [[]], [0]
    assert A.append_tokens(pool, tables, lens, [10], 8)[0] == A.OK
    parent = tables[0]
    for _ in range(n_seq - 1):
        assert pool.share(parent) == A.OK
        tables.append(list(parent))
        lens.append(10)
    assert all(pool.refcount(b) == n_seq for b in parent)
    st, slots, pairs = A.append_tokens(pool, tables, lens, [1] * n_seq, 8)
    assert st == A.OK
    # first three copy the half-full block; the last one finds refcount 1
    assert pairs == [(2, 3), (2, 4), (2, 5)]
    assert [t[2] for t in tables] == [3, 4, 5, 2]
    assert slots == [3 * B + 2, 4 * B + 2, 5 * B + 2, 2 * B + 2]
    assert pool.refcount(2) == 1
    assert pool.refcount(0) == n_seq and pool.refcount(1) == n_seq
    for t in tables:
        assert A.release_sequence(pool, t) == A.OK
    assert pool.num_free() == 16


def test_decode_step_allocates_only_at_block_boundary():
    B = 16
    pool = A.ModelPool(8, B)
    tables, lens = [[]], [0]
    for n in range(1, 40):
        before = pool.num_free()
        st, slots, _ = A.append_tokens(pool, tables, lens, [1], 8)
        assert st == A.OK
        took = before - pool.num_free()
        assert took == (1 if (n - 1) % B == 0 else 0)
        assert len(tables[0]) == O.blocks_needed(n, B)
