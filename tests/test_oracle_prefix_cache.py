"""Pins of the prefix-cache model (oracle/prefix_cache.py): the FNV-1a-64
test vectors of its key function, and the behaviour the explainer states
["PagedAttention Nedir?", "Prefix Sharing Nasıl Çalışır?"]: reuse only for
an equal token sequence under the same model context, keyed by block
contents and the context before them, only while the blocks are cached."""
import pytest

from oracle.allocator import ModelPool
from oracle.prefix_cache import ModelPrefixCache, block_key, fnv1a64


@pytest.mark.parametrize("data,want", [
    (b"", 0xCBF29CE484222325),        # offset basis
    (b"a", 0xAF63DC4C8601EC8C),
    (b"foobar", 0x85944171F73967E8),
])
def test_fnv1a64_published_vectors(data, want):
    assert fnv1a64(data) == want


def test_key_depends_on_parent_salt_and_every_token():
    toks = list(range(100, 116))
    k = block_key(0, 7, toks)
    assert block_key(1, 7, toks) != k
    assert block_key(0, 8, toks) != k
    for i in range(16):
        t = list(toks)
        t[i] += 1
        assert block_key(0, 7, t) != k
    # token ids are 32-bit little-endian after the two 64-bit words
    assert k == fnv1a64(b"\0" * 8 + (7).to_bytes(8, "little") +
                        b"".join(t.to_bytes(4, "little") for t in toks))


def _setup(B=4, N=16, salt=3):
    pool = ModelPool(N, B)
    return pool, ModelPrefixCache(pool, salt)


def _seq(pool, n_blocks):
    st, ids = pool.alloc(n_blocks)
    assert st == 0
    return ids


def test_same_prompt_reuses_full_blocks_only():
    pool, pc = _setup()
    prompt = list(range(11))                # 2 full blocks + 3 tokens
    blocks = _seq(pool, 3)
    assert pc.insert(prompt, blocks) == 2
    assert [pool.refcount(b) for b in blocks] == [2, 2, 1]
    got = pc.lookup(prompt + [99])
    assert got == blocks[:2]
    assert [pool.refcount(b) for b in blocks] == [3, 3, 1]


def test_other_model_context_misses():
    pool, pc = _setup(salt=3)
    prompt = list(range(8))
    pc.insert(prompt, _seq(pool, 2))
    other = ModelPrefixCache(pool, salt=4)
    other.entries = pc.entries              # same table, other salt
    assert other.lookup(prompt) == []


@pytest.mark.parametrize("j", range(12))
def test_first_difference_bounds_the_hit(j):
    pool, pc = _setup()
    prompt = list(range(12))
    blocks = _seq(pool, 3)
    pc.insert(prompt, blocks)
    q = list(prompt)
    q[j] = -1
    assert pc.lookup(q) == blocks[:j // 4]


def test_hash_collision_is_a_miss():
    pool = ModelPool(16, 4)
    pc = ModelPrefixCache(pool, 0, key_fn=lambda parent, salt, toks: 42)
    a = _seq(pool, 1)
    assert pc.insert([1, 2, 3, 4], a) == 1
    assert pc.lookup([1, 2, 3, 5]) == []
    assert pc.insert([1, 2, 3, 5], _seq(pool, 1)) == 0
    assert pc.lookup([1, 2, 3, 4]) == a


def test_eviction_is_lru_tail_first_and_spares_held_blocks():
    pool, pc = _setup()
    prompt = list(range(12))
    blocks = _seq(pool, 3)
    pc.insert(prompt, blocks)
    pool.free_blocks(blocks)                # the request ends
    assert [pool.refcount(b) for b in blocks] == [1, 1, 1]
    held = _seq(pool, 2)                    # another chain, still in use
    pc.insert(list(range(50, 58)), held)
    assert pc.evict(1) == [blocks[2]]       # tail of the older chain first
    assert pc.lookup(prompt) == blocks[:2]  # refreshes, adds references
    pool.free_blocks(blocks[:2])
    assert pc.evict(10) == [blocks[1], blocks[0]]
    assert pc.size() == 2                   # the held chain stays
    assert pool.num_free() == 16 - 2


def test_lookup_makes_blocks_recent():
    pool, pc = _setup()
    a, b = _seq(pool, 1), _seq(pool, 1)
    pc.insert([1, 1, 1, 1], a)
    pc.insert([2, 2, 2, 2], b)
    pool.free_blocks(a + b)
    pc.lookup([1, 1, 1, 1])
    pool.free_blocks(a)
    assert pc.evict(1) == b
