"""numpy front end of the C oracle (liboracle.so, built from pa_oracle.c).

TEST INFRASTRUCTURE ONLY: called by the tests, the smoke check and the CPU-baseline leg
of the benchmark; never by the product. Arrays are numpy; bf16 data is passed as its raw
uint16 bits, fp32 as float32. Every function returns new arrays (the caches passed to the
cache-write and block-copy oracles are copied first) and raises on a bad input.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# PA_ORACLE_LIBRARY: another build of the same source (the sanitizer check uses it)
_LIB_PATH = os.environ.get("PA_ORACLE_LIBRARY") or os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16 = 0, 1
_ERRORS = {-1: "bad argument", -2: "block table names a block outside the pool",
           -3: "duplicate slot / overlapping copy pair"}


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: run oracle/build.py (or __graft_entry__.build())")
        lib = ctypes.CDLL(_LIB_PATH)
        vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        lib.oracle_decode.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                      f32, i32, vp, i32, i32]
        lib.oracle_decode_multi.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                            i32, i32, f32, i32, vp, i32, i32]
        lib.oracle_gather.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32]
        lib.oracle_reshape_and_cache.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32]
        lib.oracle_copy_blocks.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32]
        lib.oracle_max_threads.argtypes = []
        for fn in (lib.oracle_decode, lib.oracle_decode_multi, lib.oracle_gather, lib.oracle_reshape_and_cache,
                   lib.oracle_copy_blocks, lib.oracle_max_threads):
            fn.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a):
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"cache element type must be float32 or uint16 (bf16 bits), got {a.dtype}")


def _check(status, what):
    if status != 0:
        raise ValueError(f"{what}: {_ERRORS.get(status, status)}")


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def decode(q, k_cache, v_cache, block_tables, seq_lens, scale, rows=None, threads=0):
    """Paged decode attention in fp64.

    q [B, Hq, D]; k_cache / v_cache [num_blocks, Hkv, block_size, D] (same dtype as q);
    block_tables int32 [B, max_blocks]; seq_lens int32 [B]; scale is rounded to fp32
    exactly as the kernel receives it. rows: optional list of flat query rows b * Hq + h;
    then the result is [len(rows), D], else [B, Hq, D]. Returns float64.
    """
    lib = _load()
    q = np.ascontiguousarray(q)
    k_cache = np.ascontiguousarray(k_cache)
    v_cache = np.ascontiguousarray(v_cache)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    code = _dtype_code(k_cache)
    if q.dtype != k_cache.dtype or v_cache.dtype != k_cache.dtype:
        raise TypeError("q, k_cache and v_cache must share one element type")
    B, Hq, D = q.shape
    nb, Hkv, bs, D2 = k_cache.shape
    if D2 != D or v_cache.shape != k_cache.shape or bt.shape[0] != B or sl.shape != (B,):
        raise ValueError("shape mismatch")
    max_blocks = bt.shape[1] if bt.ndim == 2 else 0
    if rows is None:
        out = np.zeros((B, Hq, D), dtype=np.float64)
        rp, nr = None, 0
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int32)
        out = np.zeros((len(rows), D), dtype=np.float64)
        rp, nr = _ptr(rows), len(rows)
    st = lib.oracle_decode(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(bt), _ptr(sl),
                           B, Hq, Hkv, D, bs, nb, max_blocks, float(np.float32(scale)), code,
                           rp, nr, int(threads))
    _check(st, "oracle_decode")
    return out


def decode_multi(q, k_cache, v_cache, block_tables, seq_lens, q_starts, scale, rows=None,
                 threads=0):
    """Multi-query paged attention with a causal mask, in fp64.

    q [total_q, Hq, D]: the last n_b = q_starts[b+1] - q_starts[b] tokens of each sequence,
    in position order; query j of sequence b attends to tokens 0 .. seq_lens[b] - n_b + j.
    q_starts int32 [B + 1]. rows: optional list of flat rows qi * Hq + h; then the result
    is [len(rows), D], else [total_q, Hq, D]. Returns float64.
    """
    lib = _load()
    q = np.ascontiguousarray(q)
    k_cache = np.ascontiguousarray(k_cache)
    v_cache = np.ascontiguousarray(v_cache)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    qs = np.ascontiguousarray(q_starts, dtype=np.int32)
    code = _dtype_code(k_cache)
    if q.dtype != k_cache.dtype or v_cache.dtype != k_cache.dtype:
        raise TypeError("q, k_cache and v_cache must share one element type")
    total, Hq, D = q.shape
    nb, Hkv, bs, D2 = k_cache.shape
    B = sl.shape[0]
    if (D2 != D or v_cache.shape != k_cache.shape or bt.shape[0] != B or qs.shape != (B + 1,)
            or int(qs[-1]) != total):
        raise ValueError("shape mismatch")
    max_blocks = bt.shape[1] if bt.ndim == 2 else 0
    if rows is None:
        out = np.zeros((total, Hq, D), dtype=np.float64)
        rp, nr = None, 0
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int32)
        out = np.zeros((len(rows), D), dtype=np.float64)
        rp, nr = _ptr(rows), len(rows)
    st = lib.oracle_decode_multi(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(bt),
                                 _ptr(sl), _ptr(qs), B, Hq, Hkv, D, bs, nb, max_blocks,
                                 float(np.float32(scale)), code, rp, nr, int(threads))
    _check(st, "oracle_decode_multi")
    return out


def gather(k_cache, v_cache, table, seq_len, kv_head):
    """Contiguous fp64 K and V ([L, D] each) of one sequence and one KV head."""
    lib = _load()
    k_cache = np.ascontiguousarray(k_cache)
    v_cache = np.ascontiguousarray(v_cache)
    table = np.ascontiguousarray(table, dtype=np.int32)
    nb, Hkv, bs, D = k_cache.shape
    L = int(seq_len)
    ko = np.zeros((L, D), dtype=np.float64)
    vo = np.zeros((L, D), dtype=np.float64)
    st = lib.oracle_gather(_ptr(ko), _ptr(vo), _ptr(k_cache), _ptr(v_cache), _ptr(table), L,
                           int(kv_head), Hkv, D, bs, nb, _dtype_code(k_cache))
    _check(st, "oracle_gather")
    return ko, vo


def reshape_and_cache(k_cache, v_cache, key, value, slot_mapping):
    """Return copies of the caches with key/value [T, Hkv, D] written at slot_mapping [T]."""
    lib = _load()
    kc = np.array(k_cache, copy=True, order="C")
    vc = np.array(v_cache, copy=True, order="C")
    key = np.ascontiguousarray(key)
    value = np.ascontiguousarray(value)
    sm = np.ascontiguousarray(slot_mapping, dtype=np.int32)
    nb, Hkv, bs, D = kc.shape
    if key.dtype != kc.dtype or value.dtype != kc.dtype:
        raise TypeError("key/value must have the cache's element type")
    T = sm.shape[0]
    if key.shape != (T, Hkv, D) or value.shape != (T, Hkv, D):
        raise ValueError("key/value must be [T, Hkv, D]")
    st = lib.oracle_reshape_and_cache(_ptr(kc), _ptr(vc), _ptr(key), _ptr(value), _ptr(sm), T,
                                      Hkv, D, bs, nb, kc.itemsize)
    _check(st, "oracle_reshape_and_cache")
    return kc, vc


def copy_blocks(k_cache, v_cache, block_pairs):
    """Return copies of the caches after copying each (src, dst) block pair."""
    lib = _load()
    kc = np.array(k_cache, copy=True, order="C")
    vc = np.array(v_cache, copy=True, order="C")
    pairs = np.ascontiguousarray(block_pairs, dtype=np.int32).reshape(-1, 2)
    nb, Hkv, bs, D = kc.shape
    st = lib.oracle_copy_blocks(_ptr(kc), _ptr(vc), _ptr(pairs), pairs.shape[0], Hkv, D, bs, nb,
                                kc.itemsize)
    _check(st, "oracle_copy_blocks")
    return kc, vc
