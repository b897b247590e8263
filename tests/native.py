"""Test helper: load the native library, building it once if it is missing."""
import os

from paged_kv_cache_191_amd import kvpaged as kv


def ensure_built():
    if not os.path.exists(kv.LIB_PATH):
        from paged_kv_cache_191_amd import build
        build.build()
    return kv.lib()
