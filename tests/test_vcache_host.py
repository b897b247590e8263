"""Argument checks of the demand-mapped contiguous cache (kv_vcache_*) that
return before any HIP call: these run without a GPU."""
import ctypes

import pytest

from native import ensure_built
from paged_kv_cache_191_amd import kvpaged as kv


@pytest.fixture(scope="module")
def lib():
    ensure_built()
    return kv.lib()


@pytest.mark.parametrize("args", [
    (0, 4096, 8, 128, kv.KV_BF16, 256),     # no sequences
    (4, 0, 8, 128, kv.KV_BF16, 256),        # no context
    (4, 4096, 0, 128, kv.KV_BF16, 256),     # no KV heads
    (4, 4096, 8, 0, kv.KV_BF16, 256),       # no head_dim
    (4, 4096, 8, 128, kv.KV_BF16, 200),     # page not a multiple of 16
    (4, 4096, 8, 128, kv.KV_BF16, 384),     # page does not divide Lmax
    (4, 4096, 8, 128, 7, 256),              # unknown dtype
])
def test_create_rejects_bad_arguments(lib, args):
    h = ctypes.c_void_p(123)
    assert lib.kv_vcache_create(*args, ctypes.byref(h)) == kv.KV_EINVAL
    assert h.value is None
    assert b"kv_vcache_create" in lib.kv_last_error()


def test_null_cache_calls(lib):
    n = ctypes.c_int32(5)
    assert lib.kv_vcache_reserve(None, 0, 16, ctypes.byref(n)) == kv.KV_EINVAL
    assert lib.kv_vcache_release(None, 0) == kv.KV_EINVAL
    assert lib.kv_vcache_seq_pages(None, 0) == -1
    assert lib.kv_vcache_mapped_bytes(None) == -1
    assert lib.kv_vcache_held_bytes(None) == -1
    k, v = ctypes.c_void_p(), ctypes.c_void_p()
    assert lib.kv_vcache_ptrs(None, ctypes.byref(k), ctypes.byref(v)) == \
        kv.KV_EINVAL
    assert lib.kv_vcache_create(4, 4096, 8, 128, kv.KV_BF16, 256,
                                None) == kv.KV_EINVAL
    lib.kv_vcache_destroy(None)  # no-op
