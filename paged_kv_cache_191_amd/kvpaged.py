"""Python binding of libkvpaged.so (include/kvpaged.h).

Argument marshalling only: every step runs in the native library (host
allocator in C++, device ops in HIP kernels). Device tensors are torch CUDA
tensors, passed as raw pointers on torch's current stream. If the library
is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkvpaged.so")

KV_OK = 0
KV_EINVAL = -1
KV_ENOMEM = -2
KV_EREFCOUNT = -3
KV_EHIP = -4
KV_EUNSUPPORTED = -5
KV_F32 = 0
KV_BF16 = 1

STATUS_NAMES = {KV_OK: "KV_OK", KV_EINVAL: "KV_EINVAL",
                KV_ENOMEM: "KV_ENOMEM", KV_EREFCOUNT: "KV_EREFCOUNT",
                KV_EHIP: "KV_EHIP", KV_EUNSUPPORTED: "KV_EUNSUPPORTED"}

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_F = ctypes.c_float
_SZ = ctypes.c_size_t
_PI32 = ctypes.POINTER(ctypes.c_int32)
_PI64 = ctypes.POINTER(ctypes.c_int64)

# name -> (restype, argtypes); mirrors include/kvpaged.h
SIGNATURES = {
    "kv_last_error": (ctypes.c_char_p, []),
    "kv_blocks_needed": (_I64, [_I64, _I32]),
    "kv_pool_create": (_I32, [_I32, _I32, _PI32, ctypes.POINTER(_P)]),
    "kv_pool_destroy": (None, [_P]),
    "kv_block_alloc": (_I32, [_P, _I32, _PI32]),
    "kv_block_free": (_I32, [_P, _I32, _PI32]),
    "kv_block_share": (_I32, [_P, _I32, _PI32]),
    "kv_block_cow": (_I32, [_P, _I32, _PI32, _PI32]),
    "kv_block_refcount": (_I32, [_P, _I32]),
    "kv_pool_num_free": (_I32, [_P]),
    "kv_pool_num_blocks": (_I32, [_P]),
    "kv_pool_block_size": (_I32, [_P]),
    "kv_pool_free_list": (_I32, [_P, _PI32, _I32]),
    "kv_seq_append": (_I32, [_P, _PI32, _I32, _PI32, _PI32, _I32, _PI64,
                             _PI32, _I32, _PI32]),
    "kv_slot_mapping": (_I32, [_PI32, _I32, _PI32, _PI32, _I32, _I32,
                               _PI64]),
    "kv_reshape_and_cache": (_I32, [_P, _P, _P, _I32, _P, _P, _I64, _I32,
                                    _I32, _I32, _I32, _P]),
    "kv_copy_blocks": (_I32, [_P, _P, _P, _I32, _I32, _I32, _I32, _I32,
                              _I32, _P]),
    "kv_append_token": (_I32, [_P, _P, _P, _P, _I32, _P, _I32, _P, _P,
                                _I32, _I32, _I32, _I32, _I32, _P]),
    "kv_append_token_fp8": (_I32, [_P, _P, _P, _P, _I32, _P, _I32, _P, _P,
                                    _I32, _I32, _I32, _I32, _F, _F, _P]),
    "kv_swap_blocks": (_I32, [_P, _P, _I32, _P, _P, _I32, _P, _I32, _I32,
                              _I32, _I32, _I32, _P]),
    "kv_reshape_and_cache_fp8": (_I32, [_P, _P, _P, _I32, _P, _P, _I64, _I32,
                                        _I32, _I32, _F, _F, _P]),
    "paged_attn_decode_fp8": (_I32, [_P, _P, _P, _P, _I32, _P, _I32, _P, _I32,
                                     _I32, _I32, _I32, _I32, _I32, _F, _F, _F,
                                     _P, _SZ, _P]),
    "contig_attn_decode_fp8": (_I32, [_P, _P, _P, _P, _I32, _P, _I32, _I32,
                                      _I32, _I32, _I32, _F, _F, _F, _P, _SZ,
                                      _P]),
    "kv_reshape_and_cache_fp8_per_head": (_I32, [_P, _P, _P, _I32, _P, _P,
                                                 _I64, _I32, _I32, _I32, _P,
                                                 _P, _P]),
    "kv_append_token_fp8_per_head": (_I32, [_P, _P, _P, _P, _I32, _P, _I32,
                                            _P, _P, _I32, _I32, _I32, _I32,
                                            _P, _P, _P]),
    "paged_attn_decode_fp8_per_head": (_I32, [_P, _P, _P, _P, _I32, _P, _I32,
                                              _P, _I32, _I32, _I32, _I32,
                                              _I32, _I32, _F, _P, _P, _P,
                                              _SZ, _P]),
    "contig_attn_decode_fp8_per_head": (_I32, [_P, _P, _P, _P, _I32, _P, _I32,
                                               _I32, _I32, _I32, _I32, _F, _P,
                                               _P, _P, _SZ, _P]),
    "kv_decode_clamped_count": (_I32, [_P, _P, _PI32]),
    "kv_decode_chunks": (_I32, [_I32, _I32]),
    "kv_decode_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32]),
    "paged_attn_decode": (_I32, [_P, _P, _P, _P, _I32, _P, _I32, _P, _I32,
                                 _I32, _I32, _I32, _I32, _I32, _F, _I32, _P,
                                 _SZ, _P]),
    "paged_attn_decode_append": (_I32, [_P, _P, _P, _P, _P, _P, _P, _I32,
                                        _P, _I32, _P, _I32, _I32, _I32, _I32,
                                        _I32, _I32, _F, _I32, _P, _SZ, _P]),
    "paged_attn_decode_append_fp8": (_I32, [_P, _P, _P, _P, _P, _P, _P, _I32,
                                            _P, _I32, _P, _I32, _I32, _I32,
                                            _I32, _I32, _I32, _F, _F, _F, _P,
                                            _SZ, _P]),
    "paged_attn_decode_append_fp8_per_head": (_I32, [_P, _P, _P, _P, _P, _P,
                                                     _P, _I32, _P, _I32, _P,
                                                     _I32, _I32, _I32, _I32,
                                                     _I32, _I32, _F, _P, _P,
                                                     _P, _SZ, _P]),
    "paged_attn_decode_noalloc": (_I32, [_P, _P, _P, _P, _I32, _P, _I32, _P,
                                         _I32, _I32, _I32, _I32, _I32, _I32,
                                         _F, _I32, _P]),
    "contig_attn_decode": (_I32, [_P, _P, _P, _P, _I32, _P, _I32, _I32,
                                  _I32, _I32, _I32, _F, _I32, _P, _SZ, _P]),
    "kv_decode_shared_prefix_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32,
                                                      _I32, _I32]),
    "paged_attn_decode_shared_prefix": (_I32, [_P, _P, _P, _P, _I32, _P, _I32,
                                               _P, _I32, _I32, _I32, _I32,
                                               _I32, _I32, _P, _P, _I32, _I32,
                                               _I32, _F, _I32, _P, _SZ, _P]),
    "paged_attn_prefill": (_I32, [_P, _P, _P, _P, _I32, _P, _P, _I32, _P,
                                  _I32, _P, _I32, _I32, _I32, _I32, _I32, _F,
                                  _I32, _I32, _P]),
    "contig_attn_prefill": (_I32, [_P, _P, _P, _P, _I32, _P, _P, _I32, _P,
                                   _I32, _I32, _I32, _I32, _F, _I32, _I32,
                                   _P]),
    "kv_prefix_block_key": (ctypes.c_uint64, [ctypes.c_uint64,
                                              ctypes.c_uint64, _PI32, _I32]),
    "kv_prefix_cache_create": (_I32, [_P, ctypes.c_uint64,
                                      ctypes.POINTER(_P)]),
    "kv_prefix_cache_destroy": (None, [_P]),
    "kv_prefix_cache_lookup": (_I32, [_P, _PI32, _I32, _PI32, _PI32]),
    "kv_prefix_cache_insert": (_I32, [_P, _PI32, _I32, _PI32, _PI32]),
    "kv_prefix_cache_evict": (_I32, [_P, _I32, _PI32]),
    "kv_prefix_cache_size": (_I32, [_P]),
    "kv_vcache_granularity": (_I32, [ctypes.POINTER(_SZ)]),
    "kv_vcache_create": (_I32, [_I32, _I32, _I32, _I32, _I32, _I32,
                                ctypes.POINTER(_P)]),
    "kv_vcache_destroy": (None, [_P]),
    "kv_vcache_ptrs": (_I32, [_P, ctypes.POINTER(_P), ctypes.POINTER(_P)]),
    "kv_vcache_reserve": (_I32, [_P, _I32, _I32, _PI32]),
    "kv_vcache_release": (_I32, [_P, _I32]),
    "kv_vcache_prefetch": (_I32, [_P, _I32, _I32]),
    "kv_vcache_sync": (_I32, [_P]),
    "kv_vcache_seq_pages": (_I32, [_P, _I32]),
    "kv_vcache_mapped_bytes": (_I64, [_P]),
    "kv_vcache_held_bytes": (_I64, [_P]),
}

_lib = None


def load_native(path: str) -> ctypes.CDLL:
    """dlopen a library of this package, with one HIP runtime per process.

    torch carries its own libamdhip64 under the same soname as ROCm's. When
    torch is imported first, a library loaded afterwards binds to torch's
    runtime; loaded first, it brings in ROCm's, torch then loads its own
    beside it, and launches through the first find no device. So torch (when
    installed) is imported before the library."""
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    return ctypes.CDLL(path)


def lib() -> ctypes.CDLL:
    """Load libkvpaged.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -c 'import "
                f"__graft_entry__ as g; g.build()'` first")
        handle = load_native(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


class KVError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib().kv_last_error().decode(errors="replace")
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {msg}")


def _check(st: int, where: str) -> None:
    if st != KV_OK:
        raise KVError(st, where)


def _i32p(a: np.ndarray):
    return a.ctypes.data_as(_PI32)


def _i64p(a: np.ndarray):
    return a.ctypes.data_as(_PI64)


def _as_i32(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


# ----------------------------------------------------------------- host ---
def kv_blocks_needed(num_tokens: int, block_size: int) -> int:
    return int(lib().kv_blocks_needed(int(num_tokens), int(block_size)))


def kv_last_error() -> str:
    return lib().kv_last_error().decode(errors="replace")


class KVPool:
    """Owner of a native kv_pool (host block metadata)."""

    def __init__(self, num_blocks: int, block_size: int,
                 free_order: Optional[Sequence[int]] = None):
        self._h = None
        handle = _P()
        order = None if free_order is None else _as_i32(free_order)
        st = lib().kv_pool_create(int(num_blocks), int(block_size),
                                  None if order is None else _i32p(order),
                                  ctypes.byref(handle))
        _check(st, "kv_pool_create")
        self._h = handle
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)

    def close(self) -> None:
        if self._h is not None and self._h.value:
            lib().kv_pool_destroy(self._h)
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def handle(self):
        return self._h

    # Status-returning forms (used by the parity tests).
    def alloc_status(self, n: int) -> Tuple[int, list]:
        out = np.zeros(max(n, 1), dtype=np.int32)
        st = lib().kv_block_alloc(self._h, int(n), _i32p(out))
        return st, (out[:n].tolist() if st == KV_OK else [])

    def free_status(self, ids) -> int:
        a = _as_i32(ids)
        return lib().kv_block_free(self._h, len(a), _i32p(a))

    def share_status(self, ids) -> int:
        a = _as_i32(ids)
        return lib().kv_block_share(self._h, len(a), _i32p(a))

    def cow_status(self, b: int) -> Tuple[int, int, int]:
        out, need = ctypes.c_int32(-1), ctypes.c_int32(0)
        st = lib().kv_block_cow(self._h, int(b), ctypes.byref(out),
                                ctypes.byref(need))
        if st != KV_OK:
            return st, -1, 0
        return st, out.value, need.value

    # Raising forms.
    def alloc(self, n: int) -> list:
        st, ids = self.alloc_status(n)
        _check(st, "kv_block_alloc")
        return ids

    def free(self, ids) -> None:
        _check(self.free_status(ids), "kv_block_free")

    def share(self, ids) -> None:
        _check(self.share_status(ids), "kv_block_share")

    def cow(self, b: int) -> Tuple[int, int]:
        st, out, need = self.cow_status(b)
        _check(st, "kv_block_cow")
        return out, need

    def refcount(self, b: int) -> int:
        return int(lib().kv_block_refcount(self._h, int(b)))

    def num_free(self) -> int:
        return int(lib().kv_pool_num_free(self._h))

    def free_list(self) -> list:
        n = self.num_free()
        out = np.zeros(max(n, 1), dtype=np.int32)
        lib().kv_pool_free_list(self._h, _i32p(out), n)
        return out[:n].tolist()

    def seq_append_status(self, tables: np.ndarray, lens: np.ndarray,
                          n_new=None, cow_capacity: Optional[int] = None):
        """kv_seq_append on host arrays tables [S, stride] int32 and lens
        [S] int32 (both updated in place). Returns (status, slots int64,
        cow pairs int32 [n, 2])."""
        assert tables.dtype == np.int32 and tables.flags.c_contiguous
        assert lens.dtype == np.int32 and lens.flags.c_contiguous
        S = lens.shape[0]
        nn = None if n_new is None else _as_i32(n_new)
        total = S if nn is None else int(np.clip(nn, 0, None).sum())
        slots = np.zeros(max(total, 1), dtype=np.int64)
        cap = S if cow_capacity is None else int(cow_capacity)
        pairs = np.zeros((max(cap, 1), 2), dtype=np.int32)
        ncow = ctypes.c_int32(0)
        st = lib().kv_seq_append(self._h, _i32p(tables), tables.shape[1],
                                 _i32p(lens),
                                 None if nn is None else _i32p(nn), S,
                                 _i64p(slots), _i32p(pairs), cap,
                                 ctypes.byref(ncow))
        if st != KV_OK:
            return st, np.zeros(0, np.int64), np.zeros((0, 2), np.int32)
        return st, slots[:total], pairs[:ncow.value]

    def seq_append(self, tables, lens, n_new=None, cow_capacity=None):
        st, slots, pairs = self.seq_append_status(tables, lens, n_new,
                                                  cow_capacity)
        _check(st, "kv_seq_append")
        return slots, pairs


def kv_pool_create(num_blocks: int, block_size: int, free_order=None
                   ) -> KVPool:
    return KVPool(num_blocks, block_size, free_order)


def kv_slot_mapping(block_tables: np.ndarray, seq_ids, positions,
                    block_size: int) -> np.ndarray:
    bt = _as_i32(block_tables)
    sid = _as_i32(seq_ids)
    pos = _as_i32(positions)
    out = np.zeros(max(len(pos), 1), dtype=np.int64)
    st = lib().kv_slot_mapping(_i32p(bt), bt.shape[1], _i32p(sid), _i32p(pos),
                               len(pos), int(block_size), _i64p(out))
    _check(st, "kv_slot_mapping")
    return out[:len(pos)]


class PrefixCache:
    """Owner of a native kv_prefix_cache over a KVPool (kv_prefix_cache_*).
    The pool must stay open while the cache lives; close() drops the cache's
    block references."""

    def __init__(self, pool: KVPool, salt: int):
        self._h = None
        self.pool = pool
        h = _P()
        _check(lib().kv_prefix_cache_create(pool.handle,
                                            int(salt) & (2**64 - 1),
                                            ctypes.byref(h)),
               "kv_prefix_cache_create")
        self._h = h

    def close(self) -> None:
        if self._h is not None and self._h.value:
            lib().kv_prefix_cache_destroy(self._h)
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def lookup(self, tokens) -> list:
        t = _as_i32(tokens)
        out = np.zeros(max(1, len(t) // self.pool.block_size), dtype=np.int32)
        n = ctypes.c_int32(0)
        _check(lib().kv_prefix_cache_lookup(self._h, _i32p(t), len(t),
                                            _i32p(out), ctypes.byref(n)),
               "kv_prefix_cache_lookup")
        return out[:n.value].tolist()

    def insert(self, tokens, blocks) -> int:
        t = _as_i32(tokens)
        b = _as_i32(blocks)
        if len(b) < len(t) // self.pool.block_size:
            raise ValueError("fewer blocks than full blocks of tokens")
        n = ctypes.c_int32(0)
        _check(lib().kv_prefix_cache_insert(self._h, _i32p(t), len(t),
                                            _i32p(b), ctypes.byref(n)),
               "kv_prefix_cache_insert")
        return int(n.value)

    def evict(self, n: int) -> list:
        out = np.zeros(max(1, int(n)), dtype=np.int32)
        k = lib().kv_prefix_cache_evict(self._h, int(n), _i32p(out))
        if k < 0:
            raise KVError(KV_EINVAL, "kv_prefix_cache_evict")
        return out[:k].tolist()

    def size(self) -> int:
        return int(lib().kv_prefix_cache_size(self._h))


def kv_prefix_block_key(parent: int, salt: int, tokens) -> int:
    t = _as_i32(tokens)
    return int(lib().kv_prefix_block_key(int(parent) & (2**64 - 1),
                                         int(salt) & (2**64 - 1), _i32p(t),
                                         len(t)))


# --------------------------------------------------------------- device ---
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return KV_F32
    if t.dtype == torch.bfloat16:
        return KV_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(t, name: str, dtype=None):
    """Pointer of a contiguous CUDA tensor (None passes NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _ndim(t, n: int, name: str) -> None:
    if len(t.shape) != n:
        raise ValueError(f"{name} must have {n} dimensions, has shape "
                         f"{tuple(t.shape)}")


def _rows(t, n: int, name: str) -> None:
    """t holds at least n rows (entries of its first dimension): the
    kernels index rows 0..n-1 of it without a bound they could check."""
    if len(t.shape) < 1 or t.shape[0] < n:
        raise ValueError(f"{name} needs at least {n} rows, has shape "
                         f"{tuple(t.shape)}")


def _same(a, b, an: str, bn: str) -> None:
    if tuple(a.shape) != tuple(b.shape):
        raise ValueError(f"{an} {tuple(a.shape)} and {bn} {tuple(b.shape)} "
                         "differ in shape")


def _attn_shapes(out, q, k, v, head_dim_of_k: int, S: int,
                 per_seq=()) -> None:
    """Shape agreement the attention kernels assume: out like q, V like K,
    one head_dim, and one row per sequence in every per-sequence input."""
    _ndim(q, 3, "q")
    _same(out, q, "out", "q")
    _ndim(k, 4, "k cache")
    _same(v, k, "v cache", "k cache")
    if head_dim_of_k != q.shape[2]:
        raise ValueError(f"head_dim of q ({q.shape[2]}) and of the cache "
                         f"({head_dim_of_k}) differ")
    for t, name in per_seq:
        _rows(t, S, name)


# While bind() records a launch, _invoke notes the native call instead of
# making it.
_RECORD: Optional[list] = None


def _invoke(name: str, *args):
    if _RECORD is not None:
        _RECORD.append((name, args))
        return KV_OK
    return getattr(lib(), name)(*args)


def bind(wrapper, *args, **kwargs):
    """Marshals one device launch once and returns a callable that issues it
    again (same pointers, sizes, scale and stream: the stream current at bind
    time unless `stream` is given) with no further Python-side checks, for
    loops that run an op many times on the same buffers. The callable keeps
    the arguments alive. A wrapper that would allocate its own workspace is
    refused (the buffer would not outlive this call)."""
    import inspect
    global _RECORD
    sig = inspect.signature(wrapper)
    given = sig.bind(*args, **kwargs).arguments
    if "workspace" in sig.parameters and given.get("workspace") is None:
        raise ValueError(f"bind({wrapper.__name__}) needs a workspace")
    if _RECORD is not None:
        raise RuntimeError("bind() is not reentrant")
    _RECORD = []
    try:
        wrapper(*args, **kwargs)
        rec = _RECORD
    finally:
        _RECORD = None
    if len(rec) != 1:
        raise ValueError(f"{wrapper.__name__} is not a single launch")
    name, cargs = rec[0]
    fn = getattr(lib(), name)
    # arguments converted to their ctypes types once
    cargs = tuple(t(a) if a is not None and not isinstance(a, t) else a
                  for t, a in zip(fn.argtypes, cargs))

    def call() -> None:
        st = fn(*cargs)
        if st != KV_OK:
            raise KVError(st, name)
    call.keep = (args, kwargs)
    return call


def _stream(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def kv_reshape_and_cache(k, v, slots, k_cache, v_cache, stream=None) -> None:
    """k, v [T, Hkv, D]; caches [blocks, Hkv, block_size, D] (paged) or
    [S, Hkv, seq_stride, D] (contiguous; slot = s * seq_stride + pos)."""
    torch = _torch()
    n, hkv, d = k.shape
    nb, chkv, bs, cd = k_cache.shape
    if (chkv, cd) != (hkv, d):
        raise ValueError("cache and rows disagree on Hkv or head_dim")
    _same(v, k, "v", "k")
    _same(v_cache, k_cache, "v_cache", "k_cache")
    _ndim(slots, 1, "slots")
    _rows(slots, n, "slots")
    st = _invoke("kv_reshape_and_cache",
        _dev(k, "k"), _dev(v, "v", k.dtype), _dev(slots, "slots", torch.int64),
        n, _dev(k_cache, "k_cache", k.dtype), _dev(v_cache, "v_cache", k.dtype),
        nb * bs, bs, hkv, d, _dtype_code(k), _stream(stream))
    _check(st, "kv_reshape_and_cache")


def _fp8_cache(t, name):
    """Device pointer of an fp8 E4M3 cache (torch.uint8 codes or
    torch.float8_e4m3fn)."""
    torch = _torch()
    if t.dtype not in (torch.uint8, torch.float8_e4m3fn):
        raise TypeError(f"{name} must be uint8 or float8_e4m3fn, got {t.dtype}")
    return _dev(t, name)


def kv_reshape_and_cache_fp8(k, v, slots, k_cache, v_cache, k_scale: float,
                             v_scale: float, stream=None) -> None:
    """bf16 rows k, v [T, Hkv, D] -> fp8 E4M3 codes in the caches (layout
    as kv_reshape_and_cache): code = E4M3(x * fl32(1 / scale))."""
    torch = _torch()
    n, hkv, d = k.shape
    nb, chkv, bs, cd = k_cache.shape
    if (chkv, cd) != (hkv, d) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("caches and rows disagree on shape")
    _same(v, k, "v", "k")
    _ndim(slots, 1, "slots")
    _rows(slots, n, "slots")
    st = _invoke("kv_reshape_and_cache_fp8",
        _dev(k, "k", torch.bfloat16), _dev(v, "v", torch.bfloat16),
        _dev(slots, "slots", torch.int64), n, _fp8_cache(k_cache, "k_cache"),
        _fp8_cache(v_cache, "v_cache"), nb * bs, bs, hkv, d, float(k_scale),
        float(v_scale), _stream(stream))
    _check(st, "kv_reshape_and_cache_fp8")


def _head_scales(t, hkv: int, name: str):
    """Pointer of a device float32 [Hkv] array of per-head scales."""
    torch = _torch()
    if tuple(t.shape) != (hkv,):
        raise ValueError(f"{name} must have shape ({hkv},), has "
                         f"{tuple(t.shape)}")
    return _dev(t, name, torch.float32)


def kv_reshape_and_cache_fp8_per_head(k, v, slots, k_cache, v_cache,
                                      k_scales, v_scales,
                                      stream=None) -> None:
    """kv_reshape_and_cache_fp8 with one scale per KV head: k_scales,
    v_scales are device float32 [Hkv]."""
    torch = _torch()
    n, hkv, d = k.shape
    nb, chkv, bs, cd = k_cache.shape
    if (chkv, cd) != (hkv, d) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("caches and rows disagree on shape")
    _same(v, k, "v", "k")
    _ndim(slots, 1, "slots")
    _rows(slots, n, "slots")
    st = _invoke("kv_reshape_and_cache_fp8_per_head",
        _dev(k, "k", torch.bfloat16), _dev(v, "v", torch.bfloat16),
        _dev(slots, "slots", torch.int64), n, _fp8_cache(k_cache, "k_cache"),
        _fp8_cache(v_cache, "v_cache"), nb * bs, bs, hkv, d,
        _head_scales(k_scales, hkv, "k_scales"),
        _head_scales(v_scales, hkv, "v_scales"), _stream(stream))
    _check(st, "kv_reshape_and_cache_fp8_per_head")


def kv_copy_blocks(k_cache, v_cache, src_dst, stream=None) -> None:
    torch = _torch()
    nb, hkv, bs, d = k_cache.shape
    _same(v_cache, k_cache, "v_cache", "k_cache")
    if len(src_dst.shape) != 2 or src_dst.shape[1] != 2:
        raise ValueError("src_dst must be [n, 2]")
    st = _invoke("kv_copy_blocks",
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache", k_cache.dtype),
        _dev(src_dst, "src_dst", torch.int32), src_dst.shape[0], nb, bs, hkv,
        d, _dtype_code(k_cache), _stream(stream))
    _check(st, "kv_copy_blocks")


def kv_append_token(k, v, new_blocks, block_tables, context_lens, k_cache,
                    v_cache, stream=None) -> None:
    """One decode token per sequence, table and lengths on the device:
    k, v [S, Hkv, D]; new_blocks int32 [S] (device or pinned host, -1 = keep
    the entry) is installed at block_tables[s][L / B] first; the rows go to
    slot block_tables[s][L / B] * B + L % B; context_lens[s] += 1. Caches
    [blocks, Hkv, block_size, D]."""
    torch = _torch()
    S, hkv, d = k.shape
    nb, chkv, bs, cd = k_cache.shape
    if (chkv, cd) != (hkv, d) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("caches and rows disagree on shape")
    if tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v differ in shape")
    if block_tables.shape[0] != S or context_lens.shape[0] != S or \
            new_blocks.shape[0] != S:
        raise ValueError("block_tables, context_lens and new_blocks need one "
                         "row per sequence")
    if not new_blocks.is_contiguous() or new_blocks.dtype != torch.int32:
        raise ValueError("new_blocks must be a contiguous int32 tensor")
    _ndim(new_blocks, 1, "new_blocks")
    _ndim(block_tables, 2, "block_tables")
    _ndim(context_lens, 1, "context_lens")
    st = _invoke("kv_append_token",
        _dev(k, "k"), _dev(v, "v", k.dtype), new_blocks.data_ptr(),
        _dev(block_tables, "block_tables", torch.int32),
        block_tables.shape[1], _dev(context_lens, "context_lens", torch.int32),
        S, _dev(k_cache, "k_cache", k.dtype), _dev(v_cache, "v_cache", k.dtype),
        nb, bs, hkv, d, _dtype_code(k), _stream(stream))
    _check(st, "kv_append_token")


def kv_append_token_fp8(k, v, new_blocks, block_tables, context_lens,
                        k_cache, v_cache, k_scale: float, v_scale: float,
                        stream=None) -> None:
    """kv_append_token into fp8 E4M3 caches: bf16 rows k, v [S, Hkv, D]
    stored as E4M3(x * fl32(1 / scale))."""
    torch = _torch()
    S, hkv, d = k.shape
    nb, chkv, bs, cd = k_cache.shape
    if (chkv, cd) != (hkv, d) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("caches and rows disagree on shape")
    if tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v differ in shape")
    if block_tables.shape[0] != S or context_lens.shape[0] != S or \
            new_blocks.shape[0] != S:
        raise ValueError("block_tables, context_lens and new_blocks need one "
                         "row per sequence")
    if not new_blocks.is_contiguous() or new_blocks.dtype != torch.int32:
        raise ValueError("new_blocks must be a contiguous int32 tensor")
    _ndim(new_blocks, 1, "new_blocks")
    _ndim(block_tables, 2, "block_tables")
    _ndim(context_lens, 1, "context_lens")
    st = _invoke("kv_append_token_fp8",
        _dev(k, "k", torch.bfloat16), _dev(v, "v", torch.bfloat16),
        new_blocks.data_ptr(), _dev(block_tables, "block_tables", torch.int32),
        block_tables.shape[1], _dev(context_lens, "context_lens", torch.int32),
        S, _fp8_cache(k_cache, "k_cache"), _fp8_cache(v_cache, "v_cache"), nb,
        bs, hkv, d, float(k_scale), float(v_scale), _stream(stream))
    _check(st, "kv_append_token_fp8")


def kv_append_token_fp8_per_head(k, v, new_blocks, block_tables,
                                 context_lens, k_cache, v_cache, k_scales,
                                 v_scales, stream=None) -> None:
    """kv_append_token_fp8 with one scale per KV head (device float32
    [Hkv])."""
    torch = _torch()
    S, hkv, d = k.shape
    nb, chkv, bs, cd = k_cache.shape
    if (chkv, cd) != (hkv, d) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("caches and rows disagree on shape")
    if tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v differ in shape")
    if block_tables.shape[0] != S or context_lens.shape[0] != S or \
            new_blocks.shape[0] != S:
        raise ValueError("block_tables, context_lens and new_blocks need one "
                         "row per sequence")
    if not new_blocks.is_contiguous() or new_blocks.dtype != torch.int32:
        raise ValueError("new_blocks must be a contiguous int32 tensor")
    _ndim(new_blocks, 1, "new_blocks")
    _ndim(block_tables, 2, "block_tables")
    _ndim(context_lens, 1, "context_lens")
    st = _invoke("kv_append_token_fp8_per_head",
        _dev(k, "k", torch.bfloat16), _dev(v, "v", torch.bfloat16),
        new_blocks.data_ptr(), _dev(block_tables, "block_tables", torch.int32),
        block_tables.shape[1], _dev(context_lens, "context_lens", torch.int32),
        S, _fp8_cache(k_cache, "k_cache"), _fp8_cache(v_cache, "v_cache"), nb,
        bs, hkv, d, _head_scales(k_scales, hkv, "k_scales"),
        _head_scales(v_scales, hkv, "v_scales"), _stream(stream))
    _check(st, "kv_append_token_fp8_per_head")


def kv_swap_blocks(src_k, src_v, dst_k, dst_v, pairs, stream=None) -> None:
    """Copy blocks src -> dst between two pools [blocks, Hkv, B, D] (device
    tensors or pinned host tensors); pairs int32 [n, 2] (device or pinned)."""
    sb, hkv, bs, d = src_k.shape
    db = dst_k.shape[0]
    if tuple(dst_k.shape[1:]) != (hkv, bs, d):
        raise ValueError("the pools differ in Hkv, block_size or head_dim")
    _same(src_v, src_k, "src_v", "src_k")
    _same(dst_v, dst_k, "dst_v", "dst_k")
    if len(pairs.shape) != 2 or pairs.shape[1] != 2:
        raise ValueError("pairs must be [n, 2]")
    for t, name in ((src_k, "src_k"), (src_v, "src_v"), (dst_k, "dst_k"),
                    (dst_v, "dst_v"), (pairs, "pairs")):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    for t in (src_v, dst_k, dst_v):
        if t.dtype != src_k.dtype:
            raise TypeError("the pools differ in dtype")
    torch = _torch()
    if pairs.dtype != torch.int32:
        raise TypeError("pairs must be int32")
    st = _invoke("kv_swap_blocks", src_k.data_ptr(), src_v.data_ptr(), sb,
                              dst_k.data_ptr(), dst_v.data_ptr(), db,
                              pairs.data_ptr(), pairs.shape[0], bs, hkv, d,
                              _dtype_code(src_k), _stream(stream))
    _check(st, "kv_swap_blocks")


def kv_decode_chunks(num_q_heads, num_kv_heads) -> int:
    return int(lib().kv_decode_chunks(num_q_heads, num_kv_heads))


def kv_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                              max_context) -> int:
    return int(lib().kv_decode_workspace_bytes(num_seqs, num_q_heads,
                                               num_kv_heads, head_dim,
                                               max_context))


def decode_workspace(num_seqs, num_q_heads, num_kv_heads, head_dim,
                     max_context, device="cuda"):
    """A device buffer of kv_decode_workspace_bytes (torch-allocated)."""
    torch = _torch()
    n = kv_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads,
                                  head_dim, max_context)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def paged_attn_decode(out, q, k_cache, v_cache, block_tables, context_lens,
                      max_context: int, scale: float, workspace=None,
                      stream=None) -> None:
    torch = _torch()
    S, hq, d = q.shape
    nb, hkv, bs, dk = k_cache.shape
    _attn_shapes(out, q, k_cache, v_cache, dk, S,
                 ((block_tables, "block_tables"),
                  (context_lens, "context_lens")))
    _ndim(block_tables, 2, "block_tables")
    if workspace is None:
        workspace = decode_workspace(S, hq, hkv, d, max_context, q.device)
    st = _invoke("paged_attn_decode",
        _dev(out, "out", q.dtype), _dev(q, "q"),
        _dev(k_cache, "k_cache", q.dtype), _dev(v_cache, "v_cache", q.dtype),
        nb, _dev(block_tables, "block_tables", torch.int32),
        block_tables.shape[1], _dev(context_lens, "context_lens", torch.int32),
        int(max_context), S, hq, hkv, d, bs, float(scale), _dtype_code(q),
        _dev(workspace, "workspace"), workspace.numel(), _stream(stream))
    _check(st, "paged_attn_decode")


def paged_attn_decode_append(out, q, k_new, v_new, new_blocks, k_cache,
                             v_cache, block_tables, context_lens,
                             max_context: int, scale: float, workspace=None,
                             stream=None) -> None:
    """kv_append_token(k_new, v_new, new_blocks, block_tables, context_lens,
    k_cache, v_cache) then paged_attn_decode over the advanced lengths, as
    one op (the attention reads the new token from k_new / v_new; the merge
    kernel stores it). context_lens is advanced in place."""
    torch = _torch()
    S, hq, d = q.shape
    nb, hkv, bs, dk = k_cache.shape
    _attn_shapes(out, q, k_cache, v_cache, dk, S,
                 ((block_tables, "block_tables"),
                  (context_lens, "context_lens")))
    _append_args(q, k_new, v_new, new_blocks, k_cache, block_tables)
    if workspace is None:
        workspace = decode_workspace(S, hq, hkv, d, max_context, q.device)
    st = _invoke("paged_attn_decode_append",
        _dev(out, "out", q.dtype), _dev(q, "q"),
        _dev(k_new, "k_new", q.dtype), _dev(v_new, "v_new", q.dtype),
        new_blocks.data_ptr(), _dev(k_cache, "k_cache", q.dtype),
        _dev(v_cache, "v_cache", q.dtype), nb,
        _dev(block_tables, "block_tables", torch.int32),
        block_tables.shape[1], _dev(context_lens, "context_lens", torch.int32),
        int(max_context), S, hq, hkv, d, bs, float(scale), _dtype_code(q),
        _dev(workspace, "workspace"), workspace.numel(), _stream(stream))
    _check(st, "paged_attn_decode_append")


def _append_args(q, k_new, v_new, new_blocks, k_cache, block_tables):
    """Shape checks shared by the decode-with-append wrappers."""
    torch = _torch()
    S, hq, d = q.shape
    hkv = k_cache.shape[1]
    _ndim(block_tables, 2, "block_tables")
    if tuple(k_new.shape) != (S, hkv, d) or tuple(v_new.shape) != (S, hkv, d):
        raise ValueError("k_new and v_new must be [num_seqs, Hkv, D]")
    if new_blocks.shape[0] != S or not new_blocks.is_contiguous() or \
            new_blocks.dtype != torch.int32:
        raise ValueError("new_blocks must be a contiguous int32 [num_seqs]")


def paged_attn_decode_append_fp8(out, q, k_new, v_new, new_blocks, k_cache,
                                 v_cache, block_tables, context_lens,
                                 max_context: int, scale: float,
                                 k_scale: float, v_scale: float,
                                 workspace=None, stream=None) -> None:
    """kv_append_token_fp8 then paged_attn_decode_fp8 over the advanced
    lengths, as one op (k_new / v_new bf16, caches fp8 E4M3 codes).
    context_lens is advanced in place."""
    torch = _torch()
    S, hq, d = q.shape
    nb, hkv, bs, dk = k_cache.shape
    _attn_shapes(out, q, k_cache, v_cache, dk, S,
                 ((block_tables, "block_tables"),
                  (context_lens, "context_lens")))
    _append_args(q, k_new, v_new, new_blocks, k_cache, block_tables)
    if workspace is None:
        workspace = decode_workspace(S, hq, hkv, d, max_context, q.device)
    st = _invoke("paged_attn_decode_append_fp8",
        _dev(out, "out", torch.bfloat16), _dev(q, "q", torch.bfloat16),
        _dev(k_new, "k_new", torch.bfloat16),
        _dev(v_new, "v_new", torch.bfloat16), new_blocks.data_ptr(),
        _fp8_cache(k_cache, "k_cache"), _fp8_cache(v_cache, "v_cache"), nb,
        _dev(block_tables, "block_tables", torch.int32),
        block_tables.shape[1], _dev(context_lens, "context_lens", torch.int32),
        int(max_context), S, hq, hkv, d, bs, float(scale), float(k_scale),
        float(v_scale), _dev(workspace, "workspace"), workspace.numel(),
        _stream(stream))
    _check(st, "paged_attn_decode_append_fp8")


def paged_attn_decode_append_fp8_per_head(out, q, k_new, v_new, new_blocks,
                                          k_cache, v_cache, block_tables,
                                          context_lens, max_context: int,
                                          scale: float, k_scales, v_scales,
                                          workspace=None,
                                          stream=None) -> None:
    """paged_attn_decode_append_fp8 with one scale per KV head (device
    float32 [Hkv])."""
    torch = _torch()
    S, hq, d = q.shape
    nb, hkv, bs, dk = k_cache.shape
    _attn_shapes(out, q, k_cache, v_cache, dk, S,
                 ((block_tables, "block_tables"),
                  (context_lens, "context_lens")))
    _append_args(q, k_new, v_new, new_blocks, k_cache, block_tables)
    if workspace is None:
        workspace = decode_workspace(S, hq, hkv, d, max_context, q.device)
    st = _invoke("paged_attn_decode_append_fp8_per_head",
        _dev(out, "out", torch.bfloat16), _dev(q, "q", torch.bfloat16),
        _dev(k_new, "k_new", torch.bfloat16),
        _dev(v_new, "v_new", torch.bfloat16), new_blocks.data_ptr(),
        _fp8_cache(k_cache, "k_cache"), _fp8_cache(v_cache, "v_cache"), nb,
        _dev(block_tables, "block_tables", torch.int32),
        block_tables.shape[1], _dev(context_lens, "context_lens", torch.int32),
        int(max_context), S, hq, hkv, d, bs, float(scale),
        _head_scales(k_scales, hkv, "k_scales"),
        _head_scales(v_scales, hkv, "v_scales"),
        _dev(workspace, "workspace"), workspace.numel(), _stream(stream))
    _check(st, "paged_attn_decode_append_fp8_per_head")


def paged_attn_decode_noalloc(out, q, k_cache, v_cache, block_tables,
                              context_lens, max_context: int, scale: float,
                              stream=None) -> None:
    """paged_attn_decode on the library's per-device scratch: nothing is
    allocated (for callers that cannot allocate, e.g. under graph
    capture). Overlapping calls on one GPU race."""
    torch = _torch()
    S, hq, d = q.shape
    nb, hkv, bs, dk = k_cache.shape
    _attn_shapes(out, q, k_cache, v_cache, dk, S,
                 ((block_tables, "block_tables"),
                  (context_lens, "context_lens")))
    _ndim(block_tables, 2, "block_tables")
    st = _invoke("paged_attn_decode_noalloc",
        _dev(out, "out", q.dtype), _dev(q, "q"),
        _dev(k_cache, "k_cache", q.dtype), _dev(v_cache, "v_cache", q.dtype),
        nb, _dev(block_tables, "block_tables", torch.int32),
        block_tables.shape[1], _dev(context_lens, "context_lens", torch.int32),
        int(max_context), S, hq, hkv, d, bs, float(scale), _dtype_code(q),
        _stream(stream))
    _check(st, "paged_attn_decode_noalloc")


def paged_attn_decode_fp8(out, q, k_cache, v_cache, block_tables,
                          context_lens, max_context: int, scale: float,
                          k_scale: float, v_scale: float, workspace=None,
                          stream=None) -> None:
    """paged_attn_decode over fp8 E4M3 caches; q, out bf16."""
    torch = _torch()
    S, hq, d = q.shape
    nb, hkv, bs, dk = k_cache.shape
    _attn_shapes(out, q, k_cache, v_cache, dk, S,
                 ((block_tables, "block_tables"),
                  (context_lens, "context_lens")))
    _ndim(block_tables, 2, "block_tables")
    if workspace is None:
        workspace = decode_workspace(S, hq, hkv, d, max_context, q.device)
    st = _invoke("paged_attn_decode_fp8",
        _dev(out, "out", torch.bfloat16), _dev(q, "q", torch.bfloat16),
        _fp8_cache(k_cache, "k_cache"), _fp8_cache(v_cache, "v_cache"), nb,
        _dev(block_tables, "block_tables", torch.int32),
        block_tables.shape[1], _dev(context_lens, "context_lens", torch.int32),
        int(max_context), S, hq, hkv, d, bs, float(scale), float(k_scale),
        float(v_scale), _dev(workspace, "workspace"), workspace.numel(),
        _stream(stream))
    _check(st, "paged_attn_decode_fp8")


def contig_attn_decode_fp8(out, q, k, v, context_lens, max_context: int,
                           scale: float, k_scale: float, v_scale: float,
                           workspace=None, stream=None) -> None:
    """contig_attn_decode over fp8 E4M3 caches [S, Hkv, Lmax, D]."""
    torch = _torch()
    S, hq, d = q.shape
    _, hkv, lmax, dk = k.shape
    _attn_shapes(out, q, k, v, dk, S,
                 ((k, "k"), (context_lens, "context_lens")))
    if workspace is None:
        workspace = decode_workspace(S, hq, hkv, d, max_context, q.device)
    st = _invoke("contig_attn_decode_fp8",
        _dev(out, "out", torch.bfloat16), _dev(q, "q", torch.bfloat16),
        _fp8_cache(k, "k"), _fp8_cache(v, "v"), lmax,
        _dev(context_lens, "context_lens", torch.int32), int(max_context), S,
        hq, hkv, d, float(scale), float(k_scale), float(v_scale),
        _dev(workspace, "workspace"), workspace.numel(), _stream(stream))
    _check(st, "contig_attn_decode_fp8")


def paged_attn_decode_fp8_per_head(out, q, k_cache, v_cache, block_tables,
                                   context_lens, max_context: int,
                                   scale: float, k_scales, v_scales,
                                   workspace=None, stream=None) -> None:
    """paged_attn_decode_fp8 with one scale per KV head (device float32
    [Hkv])."""
    torch = _torch()
    S, hq, d = q.shape
    nb, hkv, bs, dk = k_cache.shape
    _attn_shapes(out, q, k_cache, v_cache, dk, S,
                 ((block_tables, "block_tables"),
                  (context_lens, "context_lens")))
    _ndim(block_tables, 2, "block_tables")
    if workspace is None:
        workspace = decode_workspace(S, hq, hkv, d, max_context, q.device)
    st = _invoke("paged_attn_decode_fp8_per_head",
        _dev(out, "out", torch.bfloat16), _dev(q, "q", torch.bfloat16),
        _fp8_cache(k_cache, "k_cache"), _fp8_cache(v_cache, "v_cache"), nb,
        _dev(block_tables, "block_tables", torch.int32),
        block_tables.shape[1], _dev(context_lens, "context_lens", torch.int32),
        int(max_context), S, hq, hkv, d, bs, float(scale),
        _head_scales(k_scales, hkv, "k_scales"),
        _head_scales(v_scales, hkv, "v_scales"),
        _dev(workspace, "workspace"), workspace.numel(), _stream(stream))
    _check(st, "paged_attn_decode_fp8_per_head")


def contig_attn_decode_fp8_per_head(out, q, k, v, context_lens,
                                    max_context: int, scale: float, k_scales,
                                    v_scales, workspace=None,
                                    stream=None) -> None:
    """contig_attn_decode_fp8 with one scale per KV head."""
    torch = _torch()
    S, hq, d = q.shape
    _, hkv, lmax, dk = k.shape
    _attn_shapes(out, q, k, v, dk, S,
                 ((k, "k"), (context_lens, "context_lens")))
    if workspace is None:
        workspace = decode_workspace(S, hq, hkv, d, max_context, q.device)
    st = _invoke("contig_attn_decode_fp8_per_head",
        _dev(out, "out", torch.bfloat16), _dev(q, "q", torch.bfloat16),
        _fp8_cache(k, "k"), _fp8_cache(v, "v"), lmax,
        _dev(context_lens, "context_lens", torch.int32), int(max_context), S,
        hq, hkv, d, float(scale), _head_scales(k_scales, hkv, "k_scales"),
        _head_scales(v_scales, hkv, "v_scales"),
        _dev(workspace, "workspace"), workspace.numel(), _stream(stream))
    _check(st, "contig_attn_decode_fp8_per_head")


def kv_decode_clamped_count(workspace, stream=None) -> int:
    """Sequences whose context length the last decode call on `workspace`
    clamped (waits for the stream)."""
    n = ctypes.c_int32(0)
    st = _invoke("kv_decode_clamped_count", _dev(workspace, "workspace"),
                                       _stream(stream), ctypes.byref(n))
    _check(st, "kv_decode_clamped_count")
    return int(n.value)


def kv_decode_shared_prefix_workspace_bytes(num_seqs, num_q_heads,
                                            num_kv_heads, head_dim,
                                            max_context, max_shared_len) -> int:
    return int(lib().kv_decode_shared_prefix_workspace_bytes(
        num_seqs, num_q_heads, num_kv_heads, head_dim, max_context,
        max_shared_len))


def decode_shared_prefix_workspace(num_seqs, num_q_heads, num_kv_heads,
                                   head_dim, max_context, max_shared_len,
                                   device="cuda"):
    """A device buffer of kv_decode_shared_prefix_workspace_bytes."""
    torch = _torch()
    n = kv_decode_shared_prefix_workspace_bytes(
        num_seqs, num_q_heads, num_kv_heads, head_dim, max_context,
        max_shared_len)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def paged_attn_decode_shared_prefix(out, q, k_cache, v_cache, block_tables,
                                    context_lens, max_context: int,
                                    group_starts, shared_lens,
                                    max_group_size: int, max_shared_len: int,
                                    scale: float, workspace=None,
                                    stream=None) -> None:
    """group_starts: device int32 [G + 1]; shared_lens: device int32 [G]."""
    torch = _torch()
    S, hq, d = q.shape
    nb, hkv, bs, dk = k_cache.shape
    _attn_shapes(out, q, k_cache, v_cache, dk, S,
                 ((block_tables, "block_tables"),
                  (context_lens, "context_lens")))
    _ndim(block_tables, 2, "block_tables")
    G = shared_lens.shape[0]
    if group_starts.shape[0] != G + 1:
        raise ValueError("group_starts must have num_groups + 1 entries")
    if workspace is None:
        workspace = decode_shared_prefix_workspace(S, hq, hkv, d, max_context,
                                                   max_shared_len, q.device)
    st = _invoke("paged_attn_decode_shared_prefix",
        _dev(out, "out", q.dtype), _dev(q, "q"),
        _dev(k_cache, "k_cache", q.dtype), _dev(v_cache, "v_cache", q.dtype),
        nb, _dev(block_tables, "block_tables", torch.int32),
        block_tables.shape[1], _dev(context_lens, "context_lens", torch.int32),
        int(max_context), S, hq, hkv, d, bs,
        _dev(group_starts, "group_starts", torch.int32),
        _dev(shared_lens, "shared_lens", torch.int32), G,
        int(max_group_size), int(max_shared_len), float(scale),
        _dtype_code(q), _dev(workspace, "workspace"), workspace.numel(),
        _stream(stream))
    _check(st, "paged_attn_decode_shared_prefix")


def contig_attn_decode(out, q, k, v, context_lens, max_context: int,
                       scale: float, workspace=None, stream=None) -> None:
    torch = _torch()
    S, hq, d = q.shape
    _, hkv, lmax, dk = k.shape
    _attn_shapes(out, q, k, v, dk, S,
                 ((k, "k"), (context_lens, "context_lens")))
    if workspace is None:
        workspace = decode_workspace(S, hq, hkv, d, max_context, q.device)
    st = _invoke("contig_attn_decode",
        _dev(out, "out", q.dtype), _dev(q, "q"), _dev(k, "k", q.dtype),
        _dev(v, "v", q.dtype), lmax,
        _dev(context_lens, "context_lens", torch.int32), int(max_context), S,
        hq, hkv, d, float(scale), _dtype_code(q), _dev(workspace, "workspace"),
        workspace.numel(), _stream(stream))
    _check(st, "contig_attn_decode")


def paged_attn_prefill(out, q, cu_q_lens, q_start_pos, max_q_len: int,
                       k_cache, v_cache, block_tables, context_lens,
                       scale: float, causal: bool = True, stream=None) -> None:
    torch = _torch()
    T, hq, d = q.shape
    nb, hkv, bs, dk = k_cache.shape
    _ndim(cu_q_lens, 1, "cu_q_lens")
    S = cu_q_lens.shape[0] - 1
    _attn_shapes(out, q, k_cache, v_cache, dk, S,
                 ((block_tables, "block_tables"),
                  (context_lens, "context_lens"),
                  (q_start_pos, "q_start_pos")))
    _ndim(block_tables, 2, "block_tables")
    st = _invoke("paged_attn_prefill",
        _dev(out, "out", q.dtype), _dev(q, "q"),
        _dev(cu_q_lens, "cu_q_lens", torch.int32),
        _dev(q_start_pos, "q_start_pos", torch.int32), int(max_q_len),
        _dev(k_cache, "k_cache", q.dtype), _dev(v_cache, "v_cache", q.dtype),
        nb, _dev(block_tables, "block_tables", torch.int32),
        block_tables.shape[1], _dev(context_lens, "context_lens", torch.int32),
        S, hq, hkv, d, bs, float(scale), 1 if causal else 0, _dtype_code(q),
        _stream(stream))
    _check(st, "paged_attn_prefill")


def contig_attn_prefill(out, q, cu_q_lens, q_start_pos, max_q_len: int, k, v,
                        context_lens, scale: float, causal: bool = True,
                        stream=None) -> None:
    torch = _torch()
    T, hq, d = q.shape
    _ndim(cu_q_lens, 1, "cu_q_lens")
    S = cu_q_lens.shape[0] - 1
    _, hkv, lmax, dk = k.shape
    _attn_shapes(out, q, k, v, dk, S,
                 ((k, "k"), (context_lens, "context_lens"),
                  (q_start_pos, "q_start_pos")))
    st = _invoke("contig_attn_prefill",
        _dev(out, "out", q.dtype), _dev(q, "q"),
        _dev(cu_q_lens, "cu_q_lens", torch.int32),
        _dev(q_start_pos, "q_start_pos", torch.int32), int(max_q_len),
        _dev(k, "k", q.dtype), _dev(v, "v", q.dtype), lmax,
        _dev(context_lens, "context_lens", torch.int32), S, hq, hkv, d,
        float(scale), 1 if causal else 0, _dtype_code(q), _stream(stream))
    _check(st, "contig_attn_prefill")


# ------------------------------------------- demand-mapped contiguous cache --
class DeviceView:
    """A device range owned by the library (the K or V range of a VCache),
    with the attributes the wrappers above read from a tensor: shape, dtype,
    is_cuda, is_contiguous(), data_ptr(), numel()."""

    is_cuda = True

    def __init__(self, ptr: int, shape, dtype):
        self._ptr = int(ptr)
        self.shape = tuple(int(x) for x in shape)
        self.dtype = dtype

    def is_contiguous(self) -> bool:
        return True

    def data_ptr(self) -> int:
        return self._ptr

    def numel(self) -> int:
        return int(np.prod(self.shape))


def kv_vcache_granularity() -> int:
    g = _SZ(0)
    _check(lib().kv_vcache_granularity(ctypes.byref(g)),
           "kv_vcache_granularity")
    return int(g.value)


class VCache:
    """Contiguous K/V [max_seqs, Hkv, max_context, D] on virtual memory whose
    pages are mapped as sequences grow (kv_vcache_* in kvpaged.h). `k` and
    `v` are DeviceViews for contig_attn_decode / contig_attn_prefill /
    kv_reshape_and_cache; only tokens reserved for a sequence may be read or
    written. Call close() (after synchronizing the work that reads it)."""

    def __init__(self, max_seqs: int, max_context: int, num_kv_heads: int,
                 head_dim: int, dtype, page_tokens: int):
        torch = _torch()
        code = KV_BF16 if dtype == torch.bfloat16 else (
            KV_F32 if dtype == torch.float32 else None)
        if code is None:
            raise TypeError(f"unsupported dtype {dtype}")
        h = _P()
        _check(lib().kv_vcache_create(max_seqs, max_context, num_kv_heads,
                                      head_dim, code, page_tokens,
                                      ctypes.byref(h)), "kv_vcache_create")
        self._h = h
        k, v = _P(), _P()
        _check(lib().kv_vcache_ptrs(h, ctypes.byref(k), ctypes.byref(v)),
               "kv_vcache_ptrs")
        shape = (max_seqs, num_kv_heads, max_context, head_dim)
        self.k = DeviceView(k.value, shape, dtype)
        self.v = DeviceView(v.value, shape, dtype)
        self.page_tokens = page_tokens
        self.max_context = max_context

    def _handle(self):
        if self._h is None:
            raise ValueError("VCache is closed")
        return self._h

    def reserve(self, seq: int, num_tokens: int) -> int:
        n = ctypes.c_int32(0)
        _check(lib().kv_vcache_reserve(self._handle(), int(seq),
                                       int(num_tokens), ctypes.byref(n)),
               "kv_vcache_reserve")
        return int(n.value)

    def prefetch(self, seq: int, num_tokens: int) -> None:
        """Queue the mapping of tokens [0, num_tokens) of seq for the cache's
        mapping thread; returns at once."""
        _check(lib().kv_vcache_prefetch(self._handle(), int(seq),
                                        int(num_tokens)),
               "kv_vcache_prefetch")

    def sync(self) -> None:
        """Wait for every queued mapping request; raise the first failure."""
        _check(lib().kv_vcache_sync(self._handle()), "kv_vcache_sync")

    def release(self, seq: int) -> None:
        _check(lib().kv_vcache_release(self._handle(), int(seq)),
               "kv_vcache_release")

    def seq_pages(self, seq: int) -> int:
        return int(lib().kv_vcache_seq_pages(self._handle(), int(seq)))

    @property
    def mapped_bytes(self) -> int:
        return int(lib().kv_vcache_mapped_bytes(self._handle()))

    @property
    def held_bytes(self) -> int:
        return int(lib().kv_vcache_held_bytes(self._handle()))

    def close(self) -> None:
        if self._h is not None:
            lib().kv_vcache_destroy(self._h)
            self._h = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
