"""ctypes binding of libpa.so (include/pa.h), with the C names.

Argument marshalling only: tensors are passed by data pointer with their shapes, the
current HIP stream of their device is used unless one is given, and a non-zero status is
raised as PaError carrying pa_last_error(). Every step of the hot path runs in libpa's
kernels; there is no fallback. Importing this module raises if libpa.so is missing.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# PA_LIBRARY: another build of the same sources (the sanitizer check uses it)
LIB_PATH = os.environ.get("PA_LIBRARY") or os.path.join(_HERE, "libpa.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} not found: build it with __graft_entry__.build() "
                      "(or python paged_kv_cache_298_amd/build.py)")
_lib = ctypes.CDLL(LIB_PATH)

PA_F32, PA_BF16 = 0, 1
PA_PATH_AUTO, PA_PATH_PARTITION, PA_PATH_STREAM = 0, 1, 2
PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_NO_BLOCKS, PA_ERR_HIP = 0, -1, -2, -3, -4

_vp, _i32, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
_P32 = ctypes.POINTER(ctypes.c_int32)

_SIGS = {
    "pa_decode": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                         _f32, _i32, _vp, _sz, _vp]),
    "pa_decode_append": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                _i32, _i32, _i32, _f32, _i32, _vp, _sz, _vp]),
    "pa_decode_noalloc": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                 _i32, _f32, _i32, _vp]),
    "pa_decode_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_decode_partition_tokens": (_i32, [_i32, _i32]),
    "pa_set_partition_tokens": (_i32, [_i32]),
    "pa_set_decode_path": (_i32, [_i32]),
    "pa_set_stream_waves": (_i32, [_i32, _i32]),
    "pa_set_multi_order": (_i32, [_i32]),
    "pa_decode_shared": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                _i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp, _sz, _vp]),
    "pa_decode_shared_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_decode_multi": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                               _i32, _i32, _i32, _i32, _f32, _i32, _vp, _sz, _vp]),
    "pa_decode_multi_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_reshape_and_cache": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                    _vp]),
    "pa_copy_blocks": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp]),
    "pa_read_tiles": (_i32, [_vp, _vp, _sz, _vp, _i32, _i32, _vp, _vp]),
    "pa_set_validation": (_i32, [_i32]),
    "pa_validation_enabled": (_i32, []),
    "pa_validate_decode": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _vp]),
    "pa_validate_slots": (_i32, [_vp, _i32, _i32, _i32, _vp]),
    "pa_validate_block_pairs": (_i32, [_vp, _i32, _i32, _vp]),
    "pa_validate_groups": (_i32, [_vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp]),
    "pa_validate_query_starts": (_i32, [_vp, _vp, _i32, _i32, _i32, _vp]),
    "pa_validate_append": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp]),
    "pa_status_string": (ctypes.c_char_p, [_i32]),
    "pa_last_error": (ctypes.c_char_p, []),
    "pa_abi_version": (_i32, []),
    "pa_alloc_create": (_vp, [_i32, _i32, _vp]),
    "pa_alloc_destroy": (None, [_vp]),
    "pa_alloc_allocate": (_i32, [_vp, _i32, _vp]),
    "pa_alloc_free": (_i32, [_vp, _vp, _i32]),
    "pa_alloc_fork": (_i32, [_vp, _vp, _i32, _vp]),
    "pa_alloc_append_token": (_i32, [_vp, _vp, _P32, _i32, _P32, _P32, _P32, _P32]),
    "pa_alloc_refcount": (_i32, [_vp, _i32]),
    "pa_alloc_num_free": (_i32, [_vp]),
    "pa_alloc_free_list": (_i32, [_vp, _vp, _i32]),
    "pa_alloc_block_size": (_i32, [_vp]),
    "pa_pcache_create": (_vp, [_vp]),
    "pa_pcache_destroy": (None, [_vp]),
    "pa_pcache_acquire": (_i32, [_vp, _vp, _i32, _vp, _i32, _P32, _P32]),
    "pa_pcache_publish": (_i32, [_vp, _vp, _i32, _vp, _i32]),
    "pa_pcache_evict": (_i32, [_vp, _i32]),
    "pa_pcache_num_entries": (_i32, [_vp]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTS = tuple(_SIGS)


# flags of the debug validation pass (include/pa.h)
PA_BAD_LENGTH, PA_BAD_TABLE_ENTRY, PA_BAD_SLOT, PA_DUP_SLOT = 0x1, 0x2, 0x4, 0x8
PA_BAD_PAIR, PA_DUP_DST, PA_DST_IS_SRC, PA_BAD_GROUP, PA_BAD_QUERY_STARTS = 0x10, 0x20, 0x40, 0x80, 0x100
PA_BAD_APPEND_SLOT = 0x200


class PaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{_lib.pa_status_string(status).decode()}: {message}")
        self.status = status


def _check(status):
    if status != PA_OK:
        raise PaError(status, _lib.pa_last_error().decode())
    return status


def _kv_dtype(t):
    if t.dtype == torch.bfloat16:
        return PA_BF16
    if t.dtype == torch.float32:
        return PA_F32
    raise TypeError(f"element type must be torch.bfloat16 or torch.float32, got {t.dtype}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _expect(t, name, dtype, shape, device):
    """t must be a tensor of this element type and shape (None: any extent) on `device`:
    the library reads and writes by these sizes, so a mismatch would be read as other data
    or written past the tensor."""
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != len(shape) or any(s is not None and s != d for s, d in zip(shape, t.shape)):
        want = tuple("*" if s is None else s for s in shape)
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {want}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _expect_caches(k_cache, v_cache):
    """The caches: [num_blocks, Hkv, block_size, D], same type and shape, on a GPU."""
    if k_cache.dim() != 4:
        raise ValueError(f"k_cache has shape {tuple(k_cache.shape)}, expected (num_blocks, Hkv, block_size, D)")
    if not k_cache.is_cuda:
        raise ValueError(f"the caches must be on a GPU, k_cache is on {k_cache.device}")
    _kv_dtype(k_cache)
    _expect(v_cache, "v_cache", k_cache.dtype, tuple(k_cache.shape), k_cache.device)
    return k_cache.shape


def _expect_decode(out, q, k_cache, v_cache, block_tables, seq_lens, workspace):
    """Arguments of the decode entry points: out [B, Hq, D] fp32, q [B, Hq, D] and the caches
    of one element type, block_tables int32 [B, max_blocks], seq_lens int32 [B]."""
    nb, Hkv, bs, D = _expect_caches(k_cache, v_cache)
    dev = k_cache.device
    if q is None or q.dim() != 3:
        raise ValueError("q must be [B, Hq, D]")
    B, Hq = q.shape[0], q.shape[1]
    _expect(q, "q", k_cache.dtype, (B, Hq, D), dev)
    _expect(out, "out", torch.float32, (B, Hq, D), dev)
    _expect(block_tables, "block_tables", torch.int32, (B, None), dev)
    _expect(seq_lens, "seq_lens", torch.int32, (B,), dev)
    if workspace is not None:
        _expect(workspace, "workspace", torch.uint8, (None,), dev)


def _workspace(need, like, stream):
    """A workspace the library may fill as it likes (no zero fill, which would race with a
    launch on another stream), kept from reuse by torch's allocator until the work queued on
    `stream` has finished with it."""
    ws = torch.empty(need, dtype=torch.uint8, device=like.device)
    if stream is not None:
        s = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(
            int(stream.cuda_stream if hasattr(stream, "cuda_stream") else stream), device=like.device)
        if s != torch.cuda.current_stream(like.device):
            ws.record_stream(s)
    return ws


def _stream(t, stream):
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))
    if t.is_cuda:
        return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)
    return ctypes.c_void_p(0)


def abi_version():
    return int(_lib.pa_abi_version())


def pa_decode_workspace_bytes(B, Hq, Hkv, D, block_size, max_blocks, kv_dtype):
    return int(_lib.pa_decode_workspace_bytes(B, Hq, Hkv, D, block_size, max_blocks, kv_dtype))


def pa_decode_partition_tokens(block_size, max_blocks):
    return int(_lib.pa_decode_partition_tokens(block_size, max_blocks))


def pa_set_partition_tokens(tokens):
    _check(_lib.pa_set_partition_tokens(int(tokens)))


def pa_set_decode_path(path):
    _check(_lib.pa_set_decode_path(int(path)))


def pa_set_stream_waves(waves, min_slice=0):
    _check(_lib.pa_set_stream_waves(int(waves), int(min_slice)))


def pa_set_multi_order(longest_first):
    _check(_lib.pa_set_multi_order(int(longest_first)))


def pa_decode(out, q, k_cache, v_cache, block_tables, seq_lens, scale, workspace=None,
              stream=None):
    """out [B, Hq, D] fp32 <- paged decode attention. k_cache/v_cache are
    [num_blocks, Hkv, block_size, D]; block_tables int32 [B, max_blocks]; seq_lens int32 [B].
    workspace: a uint8 tensor of at least pa_decode_workspace_bytes(...) bytes (allocated
    here on q's device when None and needed)."""
    _expect_decode(out, q, k_cache, v_cache, block_tables, seq_lens, workspace)
    B, Hq, D = q.shape
    nb, Hkv, bs, _ = k_cache.shape
    max_blocks = block_tables.shape[1]
    need = pa_decode_workspace_bytes(B, Hq, Hkv, D, bs, max_blocks, _kv_dtype(k_cache))
    if workspace is None and need:
        workspace = _workspace(need, q, stream)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib.pa_decode(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                          _ptr(seq_lens), B, Hq, Hkv, D, bs, nb, max_blocks, float(scale),
                          _kv_dtype(k_cache), _ptr(workspace), ws_bytes, _stream(q, stream)))
    return out


def pa_decode_append(out, q, k_cache, v_cache, key, value, slot_mapping, block_tables, seq_lens,
                     scale, workspace=None, stream=None):
    """One decode step: write each sequence's newest K/V row (key/value [B, Hkv, D]) to its slot
    (slot_mapping int32 [B]: the slot of position seq_lens[b] - 1, or < 0 for none) and run
    pa_decode over the batch including it; the same result as pa_reshape_and_cache followed by
    pa_decode."""
    _expect_decode(out, q, k_cache, v_cache, block_tables, seq_lens, workspace)
    B, Hq, D = q.shape
    for name, t in (("key", key), ("value", value)):
        _expect(t, name, k_cache.dtype, (B, k_cache.shape[1], D), k_cache.device)
    _expect(slot_mapping, "slot_mapping", torch.int32, (B,), k_cache.device)
    nb, Hkv, bs, _ = k_cache.shape
    max_blocks = block_tables.shape[1]
    need = pa_decode_workspace_bytes(B, Hq, Hkv, D, bs, max_blocks, _kv_dtype(k_cache))
    if workspace is None and need:
        workspace = _workspace(need, q, stream)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib.pa_decode_append(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(key), _ptr(value),
                                 _ptr(slot_mapping), _ptr(block_tables), _ptr(seq_lens), B, Hq, Hkv, D, bs,
                                 nb, max_blocks, float(scale), _kv_dtype(k_cache), _ptr(workspace),
                                 ws_bytes, _stream(q, stream)))
    return out


def pa_decode_noalloc(out, q, k_cache, v_cache, block_tables, seq_lens, scale, stream=None):
    """pa_decode on the library's per-device scratch: no workspace, nothing allocated."""
    _expect_decode(out, q, k_cache, v_cache, block_tables, seq_lens, None)
    B, Hq, D = q.shape
    nb, Hkv, bs, _ = k_cache.shape
    _check(_lib.pa_decode_noalloc(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                  _ptr(seq_lens), B, Hq, Hkv, D, bs, nb, block_tables.shape[1],
                                  float(scale), _kv_dtype(k_cache), _stream(q, stream)))
    return out


def pa_decode_shared_workspace_bytes(B, Hq, D, block_size, max_blocks, max_shared_tokens):
    return int(_lib.pa_decode_shared_workspace_bytes(B, Hq, D, block_size, max_blocks,
                                                     max_shared_tokens))


def pa_decode_shared(out, q, k_cache, v_cache, block_tables, seq_lens, groups, max_members,
                     max_shared_tokens, scale, workspace=None, stream=None):
    """pa_decode for groups of consecutive sequences sharing their leading blocks.
    groups: int32 [n_groups, 3] on the device (first sequence, members, shared tokens),
    sorted by first sequence; max_members / max_shared_tokens: host bounds over the groups."""
    _expect_decode(out, q, k_cache, v_cache, block_tables, seq_lens, workspace)
    if groups is not None and groups.shape[0]:
        _expect(groups, "groups", torch.int32, (None, 3), k_cache.device)
    B, Hq, D = q.shape
    nb, Hkv, bs, _ = k_cache.shape
    max_blocks = block_tables.shape[1]
    n_groups = 0 if groups is None else groups.shape[0]
    need = pa_decode_shared_workspace_bytes(B, Hq, D, bs, max_blocks, max_shared_tokens)
    if workspace is None and need:
        workspace = _workspace(need, q, stream)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib.pa_decode_shared(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                 _ptr(block_tables), _ptr(seq_lens),
                                 _ptr(groups) if n_groups else None, n_groups, int(max_members),
                                 int(max_shared_tokens), B, Hq, Hkv, D, bs, nb, max_blocks,
                                 float(scale), _kv_dtype(k_cache), _ptr(workspace), ws_bytes,
                                 _stream(q, stream)))
    return out


def pa_decode_multi_workspace_bytes(B, total_q, max_q, Hq, Hkv, D, block_size, max_blocks):
    return int(_lib.pa_decode_multi_workspace_bytes(B, total_q, max_q, Hq, Hkv, D, block_size,
                                                    max_blocks))


def pa_decode_multi(out, q, k_cache, v_cache, block_tables, seq_lens, q_starts, max_q, scale,
                    workspace=None, stream=None):
    """Causal multi-query attention: q [total_q, Hq, D] holds each sequence's last n_b
    tokens (q_starts int32 [B + 1] on the device); query j of sequence b attends to tokens
    0 .. seq_lens[b] - n_b + j. max_q: host bound on any n_b."""
    _, _, _, D = _expect_caches(k_cache, v_cache)
    dev = k_cache.device
    if q is None or q.dim() != 3:
        raise ValueError("q must be [total_q, Hq, D]")
    _expect(q, "q", k_cache.dtype, (q.shape[0], q.shape[1], D), dev)
    _expect(out, "out", torch.float32, tuple(q.shape), dev)
    _expect(seq_lens, "seq_lens", torch.int32, (None,), dev)
    _expect(block_tables, "block_tables", torch.int32, (seq_lens.shape[0], None), dev)
    _expect(q_starts, "q_starts", torch.int32, (seq_lens.shape[0] + 1,), dev)
    if workspace is not None:
        _expect(workspace, "workspace", torch.uint8, (None,), dev)
    total_q, Hq, D = q.shape
    nb, Hkv, bs, _ = k_cache.shape
    B = seq_lens.shape[0]
    max_blocks = block_tables.shape[1]
    need = pa_decode_multi_workspace_bytes(B, total_q, max_q, Hq, Hkv, D, bs, max_blocks)
    if workspace is None and need:
        workspace = _workspace(need, q, stream)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib.pa_decode_multi(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                _ptr(block_tables), _ptr(seq_lens), _ptr(q_starts), B, total_q,
                                int(max_q), Hq, Hkv, D, bs, nb, max_blocks, float(scale),
                                _kv_dtype(k_cache), _ptr(workspace), ws_bytes,
                                _stream(q, stream)))
    return out


def pa_reshape_and_cache(k_cache, v_cache, key, value, slot_mapping, stream=None):
    """Write key/value [T, Hkv, D] into the caches at slot_mapping int32 [T] (s < 0 skips)."""
    nb, Hkv, bs, D = _expect_caches(k_cache, v_cache)
    _expect(slot_mapping, "slot_mapping", torch.int32, (None,), k_cache.device)
    for name, t in (("key", key), ("value", value)):
        _expect(t, name, k_cache.dtype, (slot_mapping.shape[0], Hkv, D), k_cache.device)
    T = slot_mapping.shape[0]
    _check(_lib.pa_reshape_and_cache(_ptr(k_cache), _ptr(v_cache), _ptr(key), _ptr(value),
                                     _ptr(slot_mapping), T, Hkv, D, bs, nb, _kv_dtype(k_cache),
                                     _stream(k_cache, stream)))


def pa_copy_blocks(k_cache, v_cache, block_pairs, stream=None):
    """Copy whole blocks src -> dst for each row of block_pairs int32 [N, 2]."""
    nb, Hkv, bs, D = _expect_caches(k_cache, v_cache)
    _expect(block_pairs, "block_pairs", torch.int32, (None, 2), k_cache.device)
    N = block_pairs.shape[0]
    _check(_lib.pa_copy_blocks(_ptr(k_cache), _ptr(v_cache), _ptr(block_pairs), N, Hkv, D, bs, nb,
                               _kv_dtype(k_cache), _stream(k_cache, stream)))


READ_SINK_LEN = 4096   # uint32 entries pa_read_tiles' sink must hold


def pa_read_tiles(k_cache, v_cache, tile_offsets, tile_bytes, sink, stream=None):
    """Read-ceiling aid: stream the listed tiles of both caches (int64 byte offsets, in
    order) as the stream decode kernel reads its groups, XOR-folding every word into
    sink (uint32 [READ_SINK_LEN]); no attention arithmetic."""
    if sink.dtype != torch.int32 or sink.numel() < READ_SINK_LEN:
        raise ValueError(f"sink must be an int32 tensor of at least {READ_SINK_LEN} entries")
    if not k_cache.is_cuda:
        raise ValueError(f"the caches must be on a GPU, k_cache is on {k_cache.device}")
    _expect(v_cache, "v_cache", k_cache.dtype, tuple(k_cache.shape), k_cache.device)
    _expect(tile_offsets, "tile_offsets", torch.int64, (None,), k_cache.device)
    _expect(sink, "sink", torch.int32, (sink.numel(),), k_cache.device)
    _check(_lib.pa_read_tiles(_ptr(k_cache), _ptr(v_cache), k_cache.numel() * k_cache.element_size(),
                              _ptr(tile_offsets), tile_offsets.numel(), int(tile_bytes), _ptr(sink),
                              _stream(k_cache, stream)))


class BlockAllocator:
    """The host refcounted block allocator (pa_alloc_*). Block ids and tables are plain
    Python lists / int32 numpy arrays; nothing here touches the GPU."""

    def __init__(self, num_blocks, block_size, initial_free_order=None):
        import numpy as np
        self._np = np
        self.block_size = int(block_size)
        self.num_blocks = int(num_blocks)
        arr = None
        if initial_free_order is not None:
            arr = np.ascontiguousarray(initial_free_order, dtype=np.int32)
            if arr.shape != (self.num_blocks,):
                raise ValueError("initial_free_order must list every block id once")
        h = _lib.pa_alloc_create(self.num_blocks, self.block_size,
                                 arr.ctypes.data_as(_vp) if arr is not None else None)
        if not h:
            raise PaError(PA_ERR_INVALID_ARG, _lib.pa_last_error().decode())
        self._h = ctypes.c_void_p(h)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h and _lib is not None:          # not during interpreter shutdown
            _lib.pa_alloc_destroy(h)
            self._h = None

    def _arr(self, xs):
        return self._np.ascontiguousarray(xs, dtype=self._np.int32)

    def allocate(self, n):
        out = self._np.zeros(max(int(n), 1), dtype=self._np.int32)
        _check(_lib.pa_alloc_allocate(self._h, int(n), out.ctypes.data_as(_vp)))
        return [int(x) for x in out[:int(n)]]

    def free(self, blocks):
        a = self._arr(blocks)
        _check(_lib.pa_alloc_free(self._h, a.ctypes.data_as(_vp), a.shape[0]))

    def fork(self, blocks):
        a = self._arr(blocks)
        out = self._np.zeros(max(a.shape[0], 1), dtype=self._np.int32)
        _check(_lib.pa_alloc_fork(self._h, a.ctypes.data_as(_vp), a.shape[0],
                                  out.ctypes.data_as(_vp)))
        return [int(x) for x in out[:a.shape[0]]]

    def append_token(self, table, seq_len, table_cap=None):
        """table: list of block ids (updated in place). Returns (new_len, slot, cow) with cow
        None or (src, dst)."""
        cap = int(table_cap) if table_cap is not None else len(table) + 1
        buf = self._np.zeros(max(cap, len(table), 1), dtype=self._np.int32)
        buf[:len(table)] = table
        n = ctypes.c_int32(len(table))
        L = ctypes.c_int32(int(seq_len))
        slot, src, dst = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check(_lib.pa_alloc_append_token(self._h, buf.ctypes.data_as(_vp), ctypes.byref(n), cap,
                                          ctypes.byref(L), ctypes.byref(slot), ctypes.byref(src),
                                          ctypes.byref(dst)))
        table[:] = [int(x) for x in buf[:n.value]]
        cow = None if src.value < 0 else (src.value, dst.value)
        return L.value, slot.value, cow

    def refcount(self, block):
        r = _lib.pa_alloc_refcount(self._h, int(block))
        return _check(r) if r < 0 else int(r)

    def num_free(self):
        return int(_lib.pa_alloc_num_free(self._h))

    def free_list(self):
        out = self._np.zeros(max(self.num_blocks, 1), dtype=self._np.int32)
        n = _lib.pa_alloc_free_list(self._h, out.ctypes.data_as(_vp), self.num_blocks)
        return [int(x) for x in out[:n]]


class PrefixCache:
    """The prefix cache over a BlockAllocator (pa_pcache_*): full blocks found by their
    token ids and everything before them are shared by new sequences. Host only."""

    def __init__(self, allocator):
        self._alloc = allocator          # keeps the allocator alive as long as the cache
        self._np = allocator._np
        h = _lib.pa_pcache_create(allocator._h)
        if not h:
            raise PaError(PA_ERR_INVALID_ARG, _lib.pa_last_error().decode())
        self._h = ctypes.c_void_p(h)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h and _lib is not None:          # not during interpreter shutdown
            _lib.pa_pcache_destroy(h)
            self._h = None

    def acquire(self, tokens):
        """Table for a new sequence with these prompt tokens: (table, cached_tokens)."""
        t = self._np.ascontiguousarray(tokens, dtype=self._np.int32)
        bs = self._alloc.block_size
        cap = max((t.shape[0] + bs - 1) // bs, 1)
        out = self._np.zeros(cap, dtype=self._np.int32)
        n, cached = ctypes.c_int32(), ctypes.c_int32()
        _check(_lib.pa_pcache_acquire(self._h, t.ctypes.data_as(_vp), t.shape[0],
                                      out.ctypes.data_as(_vp), cap, ctypes.byref(n),
                                      ctypes.byref(cached)))
        return [int(x) for x in out[:n.value]], cached.value

    def publish(self, tokens, table):
        t = self._np.ascontiguousarray(tokens, dtype=self._np.int32)
        tb = self._np.ascontiguousarray(table, dtype=self._np.int32)
        _check(_lib.pa_pcache_publish(self._h, t.ctypes.data_as(_vp), t.shape[0],
                                      tb.ctypes.data_as(_vp), tb.shape[0]))

    def evict(self, n):
        r = _lib.pa_pcache_evict(self._h, int(n))
        return _check(r) if r < 0 else int(r)

    def num_entries(self):
        return int(_lib.pa_pcache_num_entries(self._h))


# ---------------------------------------------------------------- debug validation

def pa_set_validation(on):
    """Debug mode: every kernel entry point checks its index arrays on the host first and
    raises PaError (PA_ERR_INVALID_ARG) on a violation, with nothing enqueued."""
    _check(_lib.pa_set_validation(1 if on else 0))


def pa_validation_enabled():
    return bool(_lib.pa_validation_enabled())


def _host_i32(a):
    import numpy as np
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def _validate(fn, *args):
    """(status, flags, message) of a host validator; status PA_OK or PA_ERR_INVALID_ARG."""
    flags = ctypes.c_uint32(0)
    st = fn(*args, ctypes.byref(flags))
    return st, int(flags.value), (_lib.pa_last_error().decode() if st != PA_OK else "")


def pa_validate_decode(block_tables, seq_lens, block_size, num_blocks):
    t, tp = _host_i32(block_tables)
    l, lp = _host_i32(seq_lens)
    return _validate(_lib.pa_validate_decode, tp, lp, int(t.shape[0]), int(block_size),
                     int(num_blocks), int(t.shape[1]))


def pa_validate_slots(slot_mapping, block_size, num_blocks):
    s, sp = _host_i32(slot_mapping)
    return _validate(_lib.pa_validate_slots, sp, int(s.shape[0]), int(block_size), int(num_blocks))


def pa_validate_block_pairs(block_pairs, num_blocks):
    p, pp = _host_i32(block_pairs)
    return _validate(_lib.pa_validate_block_pairs, pp, int(p.reshape(-1, 2).shape[0]), int(num_blocks))


def pa_validate_groups(groups, block_tables, seq_lens, block_size, max_members, max_shared_tokens):
    g, gp = _host_i32(groups)
    t, tp = _host_i32(block_tables)
    l, lp = _host_i32(seq_lens)
    return _validate(_lib.pa_validate_groups, gp, int(g.reshape(-1, 3).shape[0]), tp, lp,
                     int(t.shape[0]), int(block_size), int(t.shape[1]), int(max_members),
                     int(max_shared_tokens))


def pa_validate_append(slot_mapping, block_tables, seq_lens, block_size, num_blocks):
    s_, sp = _host_i32(slot_mapping)
    t, tp = _host_i32(block_tables)
    l, lp = _host_i32(seq_lens)
    return _validate(_lib.pa_validate_append, sp, tp, lp, int(t.shape[0]), int(block_size), int(num_blocks),
                     int(t.shape[1]))


def pa_validate_query_starts(q_starts, seq_lens, max_q):
    q, qp = _host_i32(q_starts)
    l, lp = _host_i32(seq_lens)
    return _validate(_lib.pa_validate_query_starts, qp, lp, int(l.shape[0]), int(q[-1]), int(max_q))
