"""Caches larger than 4 GiB, with blocks placed past byte offset 2^32 of each cache.

Every entry point that addresses the caches (block copy, cache write, decode on the stream
and partition decompositions, the fused append, the scratch-backed decode, shared-prefix
decode, multi-query decode on both of its decompositions) is run twice on the same batch:
once on a cache that holds just the batch's blocks, once on a 4.5 GiB cache (147,456
blocks of 32 KiB: Hkv 8, block_size 16, head_dim 128, bf16) holding the same blocks at
other indices, most of them past 4 GiB. Outputs and written blocks must be bit-identical
(placement does not change the arithmetic), and the decode must match the oracle.
"""
import numpy as np
import pytest
import torch

from paged_kv_cache_298_amd import workloads as W
from tests._gpu_helpers import (DEV, TOL, DevWorkload, check_inputs, gpu_step, max_err, note,
                                oracle_step, to_dev, to_host)

pytestmark = pytest.mark.gpu

HKV, BS, D, HQ = 8, 16, 128, 32
BIG = 147456          # blocks per cache: 4.5 GiB at 32 KiB per block


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_298_amd import pa as _pa
    _pa.pa_set_decode_path(_pa.PA_PATH_AUTO)
    _pa.pa_set_stream_waves(0, 0)
    _pa.pa_set_partition_tokens(0)
    return _pa


@pytest.fixture(scope="module")
def big():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    note(f"large caches: 2 x {BIG} blocks of {HKV * BS * D * 2} bytes")
    k = torch.empty((BIG, HKV, BS, D), dtype=torch.bfloat16, device=DEV)
    v = torch.empty((BIG, HKV, BS, D), dtype=torch.bfloat16, device=DEV)
    assert k.numel() * 2 > 1 << 32
    return k, v


class Placed:
    """The batch's blocks copied into the large caches at indices `phys` (most past 4 GiB,
    an eighth below), with tables, slots and clone pairs renamed to match."""

    def __init__(self, wl, big, seed):
        self.k, self.v = big
        nb, hkv, bs, d = self.k.shape
        assert (wl.Hkv, wl.block_size, wl.D) == (hkv, bs, d)
        low = -(-(1 << 32) // (self.k[0].numel() * self.k.element_size()))   # first block at 4 GiB
        rng = np.random.default_rng(seed)
        n = wl.num_blocks
        n_low = n // 8
        phys = np.concatenate([rng.choice(np.arange(low, nb), size=n - n_low, replace=False),
                               rng.choice(np.arange(0, low), size=n_low, replace=False)])
        rng.shuffle(phys)
        self.phys = phys.astype(np.int64)
        assert self.phys.max() < nb and (self.phys >= low).sum() > n // 2
        self.idx = torch.from_numpy(self.phys).to(DEV)
        self.k.index_copy_(0, self.idx, to_dev(wl.k_cache))
        self.v.index_copy_(0, self.idx, to_dev(wl.v_cache))
        # every entry renamed, those past a sequence's length too (they stay in the pool)
        tables = self.phys[np.clip(wl.block_tables, 0, n - 1)].astype(np.int32)
        assert tables.min() >= 0 and tables.max() < nb
        self.bt = to_dev(tables)
        s = wl.slot_mapping.astype(np.int64)
        slots = np.where(s >= 0, self.phys[np.clip(s, 0, None) // bs] * bs + s % bs, -1)
        assert slots.max(initial=0) < nb * bs
        self.slots = to_dev(slots.astype(np.int32))
        self.pairs = (to_dev(self.phys[wl.cow_pairs].astype(np.int32))
                      if wl.cow_pairs.shape[0] else None)

    def blocks(self):
        """The batch's blocks in their original order, from the large caches."""
        return (to_host(self.k.index_select(0, self.idx)),
                to_host(self.v.index_select(0, self.idx)))


def _batch(seed, B=12):
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, 2049, size=B).astype(np.int32)
    lens[0], lens[1] = 1, 2048
    return W.make_workload("big", B, HQ, HKV, D, BS, lens, W.BF16, seed=seed)


def _same_bits(a, b):
    return np.array_equal(np.asarray(a).view(np.uint32), np.asarray(b).view(np.uint32))


@pytest.mark.parametrize("path", ["stream", "partition"])
def test_decode_step_past_4gib(pa, oracle, big, path):
    """copy_blocks -> reshape_and_cache -> pa_decode, small cache against large cache."""
    # forked prompts: the step clones each fork's last prompt block before writing
    wl = W.make_shared_prefix("big-cow", 3, 4, 256, 40, HQ, HKV, D, BS, W.BF16, seed=71)
    assert wl.cow_pairs.shape[0] > 0
    check_inputs(wl)
    mode = pa.PA_PATH_STREAM if path == "stream" else pa.PA_PATH_PARTITION
    pa.pa_set_decode_path(mode)
    try:
        note(f"large cache decode step ({path}): B={wl.B} pairs={wl.cow_pairs.shape[0]}")
        dw = DevWorkload(wl)
        pa.pa_copy_blocks(dw.k, dw.v, dw.pairs)
        pa.pa_reshape_and_cache(dw.k, dw.v, dw.nk, dw.nv, dw.slots)
        pa.pa_decode(dw.out, dw.q, dw.k, dw.v, dw.bt, dw.sl, wl.scale)
        torch.cuda.synchronize()
        small = dw.out.cpu().numpy()

        pl = Placed(wl, big, seed=5)
        out = torch.empty_like(dw.out)
        pa.pa_copy_blocks(pl.k, pl.v, pl.pairs)
        pa.pa_reshape_and_cache(pl.k, pl.v, dw.nk, dw.nv, pl.slots)
        pa.pa_decode(out, dw.q, pl.k, pl.v, pl.bt, dw.sl, wl.scale)
        torch.cuda.synchronize()
        large = out.cpu().numpy()
    finally:
        pa.pa_set_decode_path(pa.PA_PATH_AUTO)
    assert _same_bits(large, small)
    kb, vb = pl.blocks()
    assert _same_bits(kb, to_host(dw.k)) and _same_bits(vb, to_host(dw.v))
    ref, kc, vc = oracle_step(oracle, wl)
    assert _same_bits(kb, kc) and _same_bits(vb, vc)
    err = max_err(large, ref)
    note(f"  max abs err {err:.3e}")
    assert err <= TOL[wl.dtype]


def test_append_and_noalloc_past_4gib(pa, oracle, big):
    """pa_decode_append (cache write inside the decode launch) and pa_decode_noalloc."""
    wl = _batch(72)
    check_inputs(wl)
    note(f"large cache append / noalloc: B={wl.B}")
    dw = DevWorkload(wl)
    pa.pa_decode_append(dw.out, dw.q, dw.k, dw.v, dw.nk, dw.nv, dw.slots, dw.bt, dw.sl, wl.scale)
    torch.cuda.synchronize()
    small = dw.out.cpu().numpy()
    pl = Placed(wl, big, seed=6)
    out = torch.empty_like(dw.out)
    pa.pa_decode_append(out, dw.q, pl.k, pl.v, dw.nk, dw.nv, pl.slots, pl.bt, dw.sl, wl.scale)
    torch.cuda.synchronize()
    assert _same_bits(out.cpu().numpy(), small)
    kb, vb = pl.blocks()
    assert _same_bits(kb, to_host(dw.k)) and _same_bits(vb, to_host(dw.v))
    out2 = torch.empty_like(dw.out)
    pa.pa_decode_noalloc(out2, dw.q, pl.k, pl.v, pl.bt, dw.sl, wl.scale)
    torch.cuda.synchronize()
    assert _same_bits(out2.cpu().numpy(), small)
    ref, _, _ = oracle_step(oracle, wl)
    assert max_err(small, ref) <= TOL[wl.dtype]


def test_shared_prefix_past_4gib(pa, oracle, big):
    wl = W.make_shared_prefix("big-sp", 3, 4, 512, 60, HQ, HKV, D, BS, W.BF16, seed=73)
    check_inputs(wl)
    shared = 512 - BS
    groups = np.array([(p * 4, 4, shared) for p in range(3)], np.int32)
    note(f"large cache shared prefix: B={wl.B} groups={groups.tolist()}")
    dw = DevWorkload(wl)
    pa.pa_copy_blocks(dw.k, dw.v, dw.pairs)
    pa.pa_reshape_and_cache(dw.k, dw.v, dw.nk, dw.nv, dw.slots)
    g = to_dev(groups)
    pa.pa_decode_shared(dw.out, dw.q, dw.k, dw.v, dw.bt, dw.sl, g, 4, shared, wl.scale)
    torch.cuda.synchronize()
    small = dw.out.cpu().numpy()
    pl = Placed(wl, big, seed=7)
    out = torch.empty_like(dw.out)
    pa.pa_copy_blocks(pl.k, pl.v, pl.pairs)
    pa.pa_reshape_and_cache(pl.k, pl.v, dw.nk, dw.nv, pl.slots)
    pa.pa_decode_shared(out, dw.q, pl.k, pl.v, pl.bt, dw.sl, g, 4, shared, wl.scale)
    torch.cuda.synchronize()
    assert _same_bits(out.cpu().numpy(), small)
    ref, _, _ = oracle_step(oracle, wl)
    assert max_err(small, ref) <= TOL[wl.dtype]


@pytest.mark.parametrize("n_new", [4, 200], ids=["draft-stream", "chunk-tiles"])
def test_multi_query_past_4gib(pa, oracle, big, n_new):
    """Four draft tokens per sequence (the stream decomposition) and 200-token chunks (the
    query-tile items)."""
    rng = np.random.default_rng(74 + n_new)
    B = 6
    lens = rng.integers(n_new + 1, 1500, size=B).astype(np.int32)
    wl = W.make_workload("big-mq", B, HQ, HKV, D, BS, lens, W.BF16, seed=75 + n_new,
                         n_new=[n_new] * B)
    check_inputs(wl)
    note(f"large cache multi-query n_new={n_new}: lens={lens.tolist()}")
    q, sl, qs = to_dev(wl.q), to_dev(wl.seq_lens), to_dev(wl.q_starts)
    nk, nv = to_dev(wl.new_key), to_dev(wl.new_value)
    max_q = int(np.diff(wl.q_starts).max())

    k, v, bt = to_dev(wl.k_cache), to_dev(wl.v_cache), to_dev(wl.block_tables)
    out = torch.empty((wl.q.shape[0], HQ, D), dtype=torch.float32, device=DEV)
    pa.pa_reshape_and_cache(k, v, nk, nv, to_dev(wl.slot_mapping))
    pa.pa_decode_multi(out, q, k, v, bt, sl, qs, max_q, wl.scale)
    torch.cuda.synchronize()
    small = out.cpu().numpy()

    pl = Placed(wl, big, seed=8)
    out2 = torch.empty_like(out)
    pa.pa_reshape_and_cache(pl.k, pl.v, nk, nv, pl.slots)
    pa.pa_decode_multi(out2, q, pl.k, pl.v, pl.bt, sl, qs, max_q, wl.scale)
    torch.cuda.synchronize()
    assert _same_bits(out2.cpu().numpy(), small)
    kb, vb = pl.blocks()
    assert _same_bits(kb, to_host(k)) and _same_bits(vb, to_host(v))
    kc, vc = oracle.reshape_and_cache(wl.k_cache, wl.v_cache, wl.new_key, wl.new_value,
                                      wl.slot_mapping)
    ref = oracle.decode_multi(wl.q, kc, vc, wl.block_tables, wl.seq_lens, wl.q_starts, wl.scale)
    err = max_err(small, ref)
    note(f"  max abs err {err:.3e}")
    assert err <= TOL[wl.dtype]


def test_read_tiles_past_4gib(pa, big):
    """pa_read_tiles over the batch's tiles in the large caches: the XOR of its sink equals
    the XOR of the same tiles in the small caches, computed on the host."""
    wl = _batch(76)
    check_inputs(wl)
    pl = Placed(wl, big, seed=9)
    tables = pl.phys[np.clip(wl.block_tables, 0, wl.num_blocks - 1)].astype(np.int32)
    offs = W.group_tile_offsets(tables, wl.seq_lens, HKV, D, 2, BS)
    tile = BS * D * 2
    assert offs.min() >= 0 and offs.max() + tile <= BIG * HKV * tile   # host guard
    assert (offs >= 1 << 32).sum() > len(offs) // 2
    note(f"large cache read_tiles: {len(offs)} tiles, max offset {int(offs.max())}")
    sink = torch.zeros(pa.READ_SINK_LEN, dtype=torch.int32, device=DEV)
    pa.pa_read_tiles(pl.k, pl.v, torch.from_numpy(offs).to(DEV), tile, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    small = W.group_tile_offsets(wl.block_tables, wl.seq_lens, HKV, D, 2, BS)
    kr = np.ascontiguousarray(wl.k_cache).view(np.uint8).reshape(-1)
    vr = np.ascontiguousarray(wl.v_cache).view(np.uint8).reshape(-1)
    idx = (small[:, None] + np.arange(tile)[None, :]).reshape(-1)
    want = (np.bitwise_xor.reduce(kr[idx].view(np.uint32)) ^
            np.bitwise_xor.reduce(vr[idx].view(np.uint32)))
    assert got == want


SHAPES = [
    # dtype, head_dim, block_size: the 8-token blocks of the stream kernel (two tiles per
    # group), head_dim 64, fp32 caches (partition kernel), 128-token blocks
    (W.BF16, 128, 8), (W.BF16, 64, 32), (W.F32, 128, 16), (W.BF16, 128, 128),
]


@pytest.mark.parametrize("case", SHAPES, ids=lambda c: f"{c[0]}-D{c[1]}-bs{c[2]}")
def test_other_shapes_past_4gib(pa, oracle, case):
    """reshape_and_cache then pa_decode with other block sizes, head sizes and fp32 caches,
    in caches of 4.5 GiB each."""
    dtype, d, bs = case
    tdt = torch.bfloat16 if dtype == W.BF16 else torch.float32
    blk = HKV * bs * d * (2 if dtype == W.BF16 else 4)
    nb = (9 << 29) // blk                                   # 4.5 GiB per cache
    rng = np.random.default_rng(bs + d)
    lens = rng.integers(1, 1500, size=8).astype(np.int32)
    lens[0] = 1
    wl = W.make_workload("big-shape", 8, 32, HKV, d, bs, lens, dtype, seed=bs + d)
    check_inputs(wl)
    note(f"large cache {dtype} D={d} bs={bs}: {nb} blocks of {blk} bytes per cache")
    dw = DevWorkload(wl)
    small = gpu_step(pa, dw)
    k = torch.empty((nb, HKV, bs, d), dtype=tdt, device=DEV)
    v = torch.empty((nb, HKV, bs, d), dtype=tdt, device=DEV)
    try:
        pl = Placed(wl, (k, v), seed=bs)
        out = torch.empty_like(dw.out)
        pa.pa_reshape_and_cache(pl.k, pl.v, dw.nk, dw.nv, pl.slots)
        pa.pa_decode(out, dw.q, pl.k, pl.v, pl.bt, dw.sl, wl.scale)
        torch.cuda.synchronize()
        assert _same_bits(out.cpu().numpy(), small)
        kb, vb = pl.blocks()
        assert _same_bits(kb, to_host(dw.k)) and _same_bits(vb, to_host(dw.v))
    finally:
        del k, v
        torch.cuda.empty_cache()
    ref, _, _ = oracle_step(oracle, wl)
    err = max_err(small, ref)
    note(f"  max abs err {err:.3e}")
    assert err <= TOL[wl.dtype]
