"""kv.bind's refusals, on the host: no launch is made (CPU only)."""
import pytest

from native import ensure_built
from paged_kv_cache_191_amd import kvpaged as kv


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()


def test_bind_needs_a_workspace():
    # a decode that would allocate its own workspace cannot be bound: the
    # buffer would be freed when bind returns
    with pytest.raises(ValueError, match="workspace"):
        kv.bind(kv.paged_attn_decode, None, None, None, None, None, None,
                16, 0.1)


def test_bind_refuses_a_call_that_is_not_one_launch():
    # a host query makes no launch at all
    with pytest.raises(ValueError, match="single launch"):
        kv.bind(kv.kv_decode_chunks, 32, 8)


def test_bind_leaves_the_binding_usable():
    with pytest.raises(ValueError):
        kv.bind(kv.kv_decode_chunks, 32, 8)
    assert kv._RECORD is None
    assert kv.kv_decode_chunks(32, 8) > 0
