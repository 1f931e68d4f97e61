"""Python binding of ``libpkv.so``, the gfx950 paged-KV attention library.

Argument marshalling only: every function forwards to the C entry point of
the same name declared in ``include/pkv.h``; all work runs in the library's
HIP kernels. Pointer arguments accept an integer device address or any object
with ``data_ptr()`` (e.g. a torch tensor); ``stream`` accepts a HIP stream
handle as an integer, an object with ``cuda_stream`` (torch's stream), or
None for the null stream. A non-OK status raises :class:`PkvError`.

The library is built in-tree by ``__graft_entry__.build()`` (or
``python -m paged_kv_decode_reshape_amd._build``); calling any function
without it raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "PkvError", "F32", "BF16", "FP8_E4M3", "KERNEL_APPEND", "KERNEL_DECODE_PARTITION",
    "KERNEL_DECODE_REDUCE", "KERNEL_PREFILL", "KERNEL_DECODE_PREFIX", "KERNEL_GATHER", "library_path", "load",
    "kv_pool_bytes", "kv_pool_create", "kv_pool_set_fp8_scales", "kv_pool_destroy",
    "reshape_and_cache", "copy_blocks",
    "paged_attention_decode_workspace_bytes", "paged_attention_decode", "paged_attention_decode_noalloc",
    "paged_attention_decode_append",
    "paged_attention_decode_multi_workspace_bytes", "paged_attention_decode_multi",
    "paged_attention_decode_shared_workspace_bytes", "paged_attention_decode_shared",
    "paged_attention_prefill_chunk", "paged_kv_gather_checksum", "pkv_timing_enable", "pkv_timing_disable",
    "pkv_timing_read", "pkv_timing_read_launches", "pkv_last_error", "pkv_debug_read_errors",
    "DEBUG_SLOT", "DEBUG_BLOCK", "DEBUG_CONTEXT", "DEBUG_CHUNK", "library_variant", "EXPORTED_SYMBOLS",
]

F32, BF16, FP8_E4M3 = 0, 1, 2
KERNEL_APPEND, KERNEL_DECODE_PARTITION, KERNEL_DECODE_REDUCE, KERNEL_PREFILL = 0, 1, 2, 3
KERNEL_DECODE_PREFIX = 4
KERNEL_GATHER = 5
DEBUG_SLOT, DEBUG_BLOCK, DEBUG_CONTEXT, DEBUG_CHUNK = 1, 2, 4, 8

_STATUS = {0: "PKV_OK", -1: "PKV_ERR_INVALID_ARG", -2: "PKV_ERR_UNSUPPORTED",
           -3: "PKV_ERR_HIP", -4: "PKV_ERR_WORKSPACE"}

_HERE = os.path.dirname(os.path.abspath(__file__))
# Two builds of the same sources: "release" (libpkv.so) and "debug"
# (libpkv_debug.so, device-value checks compiled in). Calls go to the
# variant selected by library_variant(), the release library by default.
_LIB_FILES = {"release": "libpkv.so", "debug": "libpkv_debug.so"}
_libs = {}
_variant = "release"

c_int, c_float, c_size_t, c_void_p = ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p
_P = ctypes.POINTER

# name -> (restype, argtypes); the C-ABI of include/pkv.h
_SIGNATURES = {
    "pkv_last_error": (ctypes.c_char_p, []),
    "kv_pool_bytes": (c_int, [c_int, c_int, c_int, c_int, c_int, _P(c_size_t), _P(c_size_t)]),
    "kv_pool_create": (c_int, [_P(c_void_p), c_int, c_int, c_int, c_int, c_int, c_int,
                               _P(c_void_p), _P(c_void_p)]),
    "kv_pool_set_fp8_scales": (c_int, [c_void_p, c_int, _P(c_float), _P(c_float)]),
    "kv_pool_destroy": (c_int, [c_void_p]),
    "reshape_and_cache": (c_int, [c_void_p, c_int, c_void_p, c_void_p, c_void_p, c_int, c_void_p]),
    "copy_blocks": (c_int, [c_void_p, c_void_p, c_int, c_void_p]),
    "paged_attention_decode_workspace_bytes": (c_int, [c_void_p, c_int, c_int, c_int, c_int,
                                                       _P(c_size_t)]),
    "paged_attention_decode": (c_int, [c_void_p, c_int, c_void_p, c_void_p, c_void_p, c_void_p,
                                       c_int, c_int, c_int, c_float, c_int, c_void_p, c_size_t,
                                       c_void_p]),
    "paged_attention_decode_noalloc": (c_int, [c_void_p, c_int, c_void_p, c_void_p, c_void_p, c_void_p,
                                               c_int, c_int, c_int, c_float, c_int, c_void_p]),
    "paged_attention_decode_append": (c_int, [c_void_p, c_int, c_void_p, c_void_p, c_void_p, c_void_p,
                                              c_void_p, c_void_p, c_int, c_int, c_int, c_float, c_int,
                                              c_void_p, c_size_t, c_void_p]),
    "paged_attention_decode_multi_workspace_bytes": (c_int, [c_void_p, c_int, c_int, c_int, c_int, c_int,
                                                             _P(c_size_t)]),
    "paged_attention_decode_multi": (c_int, [c_void_p, c_int, c_void_p, c_void_p, c_int, c_void_p,
                                             c_void_p, c_int, c_int, c_int, c_float, c_int, c_void_p,
                                             c_size_t, c_void_p]),
    "paged_attention_decode_shared_workspace_bytes": (c_int, [c_void_p, c_int, c_int, c_int, c_int,
                                                              _P(c_size_t)]),
    "paged_attention_decode_shared": (c_int, [c_void_p, c_int, c_void_p, c_void_p, c_void_p, c_void_p,
                                              c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_int,
                                              c_float, c_int, c_void_p, c_size_t, c_void_p]),
    "paged_attention_prefill_chunk": (c_int, [c_void_p, c_int, c_void_p, c_void_p, c_void_p,
                                              c_void_p, c_void_p, c_int, c_int, c_int, c_int,
                                              c_int, c_float, c_void_p]),
    "paged_kv_gather_checksum": (c_int, [c_void_p, c_int, c_void_p, c_void_p, c_void_p, c_int, c_int,
                                         c_void_p, c_size_t, c_void_p]),
    "pkv_timing_enable": (c_int, [c_int, ctypes.c_uint]),
    "pkv_timing_disable": (c_int, []),
    "pkv_timing_read": (c_int, [c_int, _P(c_int), _P(ctypes.c_double)]),
    "pkv_timing_read_launches": (c_int, [c_int, _P(c_float), c_int, _P(c_int)]),
    "pkv_debug_read_errors": (c_int, [_P(ctypes.c_uint), c_int]),
}
EXPORTED_SYMBOLS = tuple(_SIGNATURES)


class PkvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


def library_path(variant: str | None = None) -> str:
    v = variant or _variant
    # A test build of the same entry points (the host-sanitized library) can
    # stand in for the release library.
    if v == "release" and os.environ.get("PKV_LIBRARY_PATH"):
        return os.environ["PKV_LIBRARY_PATH"]
    return os.path.join(_HERE, _LIB_FILES[v])


def load(variant: str | None = None):
    """Load the selected library variant (once). Raises if it has not been built."""
    v = variant or _variant
    if v not in _libs:
        path = library_path(v)
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                               "(there is no fallback implementation)")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype, fn.argtypes = res, args
        _libs[v] = lib
    return _libs[v]


class library_variant:
    """Context manager: calls inside go to the given variant ("release" or
    "debug"). Pool handles belong to the variant that created them."""

    def __init__(self, variant: str):
        if variant not in _LIB_FILES:
            raise ValueError(f"unknown library variant {variant!r}")
        self.variant = variant

    def __enter__(self):
        global _variant
        self.prev, _variant = _variant, self.variant
        load()
        return self

    def __exit__(self, *exc):
        global _variant
        _variant = self.prev
        return False


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _stream(s):
    if s is None:
        return None
    if isinstance(s, int):
        return s
    return int(s.cuda_stream)


def _check(status: int):
    if status != 0:
        raise PkvError(status, load().pkv_last_error().decode())


def pkv_last_error() -> str:
    return load().pkv_last_error().decode()


def kv_pool_bytes(num_blocks, block_size, num_kv_heads, head_dim, dtype):
    k, v = c_size_t(), c_size_t()
    _check(load().kv_pool_bytes(num_blocks, block_size, num_kv_heads, head_dim, dtype,
                                ctypes.byref(k), ctypes.byref(v)))
    return k.value, v.value


def kv_pool_create(num_layers, num_blocks, block_size, num_kv_heads, head_dim, dtype,
                   k_layers, v_layers):
    """Returns the opaque pool handle (an integer). The caller keeps the device
    memory alive and calls kv_pool_destroy when done."""
    n = len(k_layers)
    karr = (c_void_p * n)(*[_ptr(t) for t in k_layers])
    varr = (c_void_p * n)(*[_ptr(t) for t in v_layers])
    handle = c_void_p()
    _check(load().kv_pool_create(ctypes.byref(handle), num_layers, num_blocks, block_size,
                                 num_kv_heads, head_dim, dtype, karr, varr))
    return handle.value


def kv_pool_set_fp8_scales(pool, k_scales, v_scales):
    """k_scales, v_scales: one float per layer of the pool."""
    k, v = list(k_scales), list(v_scales)
    if len(k) != len(v):
        raise ValueError("k_scales and v_scales differ in length")
    _check(load().kv_pool_set_fp8_scales(pool, len(k), (c_float * len(k))(*k), (c_float * len(v))(*v)))


def kv_pool_destroy(pool):
    _check(load().kv_pool_destroy(pool))


def reshape_and_cache(pool, layer, key, value, slot_mapping, num_tokens, stream=None):
    _check(load().reshape_and_cache(pool, layer, _ptr(key), _ptr(value), _ptr(slot_mapping),
                                    num_tokens, _stream(stream)))


def copy_blocks(pool, block_pairs, num_pairs, stream=None):
    _check(load().copy_blocks(pool, _ptr(block_pairs), num_pairs, _stream(stream)))


def paged_attention_decode_workspace_bytes(pool, num_seqs, num_q_heads, max_blocks_per_seq,
                                           partition_size=0):
    out = c_size_t()
    _check(load().paged_attention_decode_workspace_bytes(pool, num_seqs, num_q_heads,
                                                         max_blocks_per_seq, partition_size,
                                                         ctypes.byref(out)))
    return out.value


def paged_attention_decode(pool, layer, out, query, block_tables, context_lens, num_seqs,
                           num_q_heads, max_blocks_per_seq, scale, partition_size=0,
                           workspace=None, workspace_bytes=0, stream=None):
    _check(load().paged_attention_decode(pool, layer, _ptr(out), _ptr(query), _ptr(block_tables),
                                         _ptr(context_lens), num_seqs, num_q_heads,
                                         max_blocks_per_seq, float(scale), partition_size,
                                         _ptr(workspace), workspace_bytes, _stream(stream)))


def paged_attention_decode_noalloc(pool, layer, out, query, block_tables, context_lens, num_seqs,
                                   num_q_heads, max_blocks_per_seq, scale, partition_size=0, stream=None):
    _check(load().paged_attention_decode_noalloc(pool, layer, _ptr(out), _ptr(query), _ptr(block_tables),
                                                 _ptr(context_lens), num_seqs, num_q_heads,
                                                 max_blocks_per_seq, float(scale), partition_size,
                                                 _stream(stream)))


def paged_attention_decode_append(pool, layer, out, query, key, value, block_tables, context_lens, num_seqs,
                                  num_q_heads, max_blocks_per_seq, scale, partition_size=0,
                                  workspace=None, workspace_bytes=0, stream=None):
    _check(load().paged_attention_decode_append(pool, layer, _ptr(out), _ptr(query), _ptr(key), _ptr(value),
                                                _ptr(block_tables), _ptr(context_lens), num_seqs,
                                                num_q_heads, max_blocks_per_seq, float(scale),
                                                partition_size, _ptr(workspace), workspace_bytes,
                                                _stream(stream)))


def paged_attention_decode_multi_workspace_bytes(pool, num_seqs, queries_per_seq, num_q_heads,
                                                 max_blocks_per_seq, partition_size=0):
    out = c_size_t()
    _check(load().paged_attention_decode_multi_workspace_bytes(pool, num_seqs, queries_per_seq,
                                                               num_q_heads, max_blocks_per_seq,
                                                               partition_size, ctypes.byref(out)))
    return out.value


def paged_attention_decode_multi(pool, layer, out, query, queries_per_seq, block_tables, context_lens,
                                 num_seqs, num_q_heads, max_blocks_per_seq, scale, partition_size=0,
                                 workspace=None, workspace_bytes=0, stream=None):
    _check(load().paged_attention_decode_multi(pool, layer, _ptr(out), _ptr(query), queries_per_seq,
                                               _ptr(block_tables), _ptr(context_lens), num_seqs,
                                               num_q_heads, max_blocks_per_seq, float(scale),
                                               partition_size, _ptr(workspace), workspace_bytes,
                                               _stream(stream)))


def paged_attention_decode_shared_workspace_bytes(pool, num_seqs, num_q_heads, max_blocks_per_seq,
                                                  partition_size=0):
    out = c_size_t()
    _check(load().paged_attention_decode_shared_workspace_bytes(pool, num_seqs, num_q_heads,
                                                                max_blocks_per_seq, partition_size,
                                                                ctypes.byref(out)))
    return out.value


def paged_attention_decode_shared(pool, layer, out, query, block_tables, context_lens, group_starts,
                                  prefix_lens, num_seqs, num_groups, max_group_size, num_q_heads,
                                  max_blocks_per_seq, scale, partition_size=0, workspace=None,
                                  workspace_bytes=0, stream=None):
    _check(load().paged_attention_decode_shared(pool, layer, _ptr(out), _ptr(query), _ptr(block_tables),
                                                _ptr(context_lens), _ptr(group_starts),
                                                _ptr(prefix_lens), num_seqs, num_groups, max_group_size,
                                                num_q_heads, max_blocks_per_seq, float(scale),
                                                partition_size, _ptr(workspace), workspace_bytes,
                                                _stream(stream)))


def paged_attention_prefill_chunk(pool, layer, out, query, cu_q_lens, block_tables,
                                  context_lens, num_seqs, total_q_tokens, max_q_len,
                                  num_q_heads, max_blocks_per_seq, scale, stream=None):
    _check(load().paged_attention_prefill_chunk(pool, layer, _ptr(out), _ptr(query),
                                                _ptr(cu_q_lens), _ptr(block_tables),
                                                _ptr(context_lens), num_seqs, total_q_tokens,
                                                max_q_len, num_q_heads, max_blocks_per_seq,
                                                float(scale), _stream(stream)))


def paged_kv_gather_checksum(pool, layer, checksum, block_tables, context_lens, num_seqs,
                             max_blocks_per_seq, workspace, workspace_bytes, stream=None):
    _check(load().paged_kv_gather_checksum(pool, layer, _ptr(checksum), _ptr(block_tables),
                                           _ptr(context_lens), num_seqs, max_blocks_per_seq,
                                           _ptr(workspace), workspace_bytes, _stream(stream)))


def pkv_timing_enable(max_launches, kinds=None):
    """Record launches of the given kernel kinds (an iterable of KERNEL_*
    values; None records every kind)."""
    mask = 0 if kinds is None else sum(1 << int(k) for k in set(kinds))
    _check(load().pkv_timing_enable(max_launches, mask))


def pkv_timing_disable():
    _check(load().pkv_timing_disable())


def pkv_timing_read(kind):
    """Returns (launches, total_ms) for one kernel kind."""
    n, ms = c_int(), ctypes.c_double()
    _check(load().pkv_timing_read(kind, ctypes.byref(n), ctypes.byref(ms)))
    return n.value, ms.value


def pkv_timing_read_launches(kind, capacity):
    """Durations in ms of up to ``capacity`` recorded launches of one kernel kind, in launch order."""
    buf = (c_float * max(capacity, 1))()
    n = c_int()
    _check(load().pkv_timing_read_launches(kind, buf, capacity, ctypes.byref(n)))
    return [float(buf[i]) for i in range(n.value)]


def pkv_debug_read_errors(clear=True):
    """Bits (DEBUG_*) the device-value checks of the debug library set since
    the last clear; waits for the device."""
    f = ctypes.c_uint()
    _check(load().pkv_debug_read_errors(ctypes.byref(f), 1 if clear else 0))
    return f.value
