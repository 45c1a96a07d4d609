"""Parity of the HIP path (through the C ABI) with the oracle, on an MI355X.

Attention: max-abs error over every output element <= 1e-5 (fp32 caches) or 2e-2 (bf16
caches, fp32 accumulation). Cache write and block copy: bit-exact over the whole cache.
Invariants (placement, sharing, poison, determinism) are checked bit for bit on the GPU.
bf16 caches go through the stream decomposition by default; the partition decomposition
is forced where a test names it, and the stream decomposition is run with few waves where
rows must be split across many slices.
"""
import contextlib

import numpy as np
import pytest
import torch

from paged_kv_cache_298_amd import workloads as W
from tests._gpu_helpers import (DEV, TOL, DevWorkload, gpu_step, max_err, note, oracle_step,
                                scale_k_by_position, to_dev, to_host)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_298_amd import pa as _pa
    _pa.pa_set_partition_tokens(0)
    _pa.pa_set_decode_path(_pa.PA_PATH_AUTO)
    _pa.pa_set_stream_waves(0, 0)
    return _pa


@contextlib.contextmanager
def _path(pa, path, waves=0, min_slice=0, part_tokens=0):
    pa.pa_set_decode_path(path)
    pa.pa_set_stream_waves(waves, min_slice)
    pa.pa_set_partition_tokens(part_tokens)
    try:
        yield
    finally:
        pa.pa_set_decode_path(pa.PA_PATH_AUTO)
        pa.pa_set_stream_waves(0, 0)
        pa.pa_set_partition_tokens(0)


def _parity(pa, oracle, wl, rows=None, tag=""):
    note(f"{wl.name} {tag} B={wl.B} Hq={wl.Hq} Hkv={wl.Hkv} D={wl.D} bs={wl.block_size} "
         f"dtype={wl.dtype} lens[:8]={list(wl.seq_lens[:8])}")
    dw = DevWorkload(wl)
    got = gpu_step(pa, dw)
    ref, kc, vc = oracle_step(oracle, wl, rows=rows)
    if rows is not None:
        got = got.reshape(wl.B * wl.Hq, wl.D)[rows]
    err = max_err(got, ref)
    note(f"  max abs err {err:.3e} (tol {TOL[wl.dtype]})")
    assert err <= TOL[wl.dtype]
    return dw, kc, vc


def test_config1_tiny_fp32(pa, oracle):
    wl = W.config(1)
    dw, kc, vc = _parity(pa, oracle, wl)
    assert np.array_equal(to_host(dw.k).view(np.uint32), kc.view(np.uint32))
    assert np.array_equal(to_host(dw.v).view(np.uint32), vc.view(np.uint32))


SMALL = [
    # B, Hq, Hkv, D, bs, dtype, lens
    (4, 8, 2, 128, 16, W.BF16, [1, 15, 16, 17]),
    (5, 32, 8, 128, 16, W.BF16, [255, 256, 257, 513, 700]),
    (3, 16, 2, 128, 32, W.BF16, [31, 32, 1000]),
    (3, 8, 8, 64, 64, W.BF16, [63, 64, 65]),
    (4, 16, 2, 64, 16, W.BF16, [2, 100, 300, 1500]),
    (2, 4, 2, 128, 64, W.BF16, [3000, 129]),
    (3, 8, 4, 128, 16, W.F32, [1, 40, 600]),
    (3, 8, 1, 64, 32, W.F32, [5, 64, 333]),
    (2, 2, 2, 128, 64, W.F32, [70, 1]),
    (4, 4, 4, 64, 16, W.F32, [16, 17, 255, 1024]),
    # 8-token blocks (a 16-token group spans two blocks; bf16 stream decomposition only)
    (4, 16, 4, 128, 8, W.BF16, [7, 8, 9, 300]),
    (3, 8, 8, 64, 8, W.BF16, [1, 17, 1001]),
    (2, 64, 8, 128, 8, W.BF16, [15, 2000]),
    # 128-token blocks
    (3, 16, 4, 64, 128, W.BF16, [1, 128, 1000]),
    (3, 32, 8, 128, 128, W.BF16, [127, 129, 4000]),
    (3, 16, 4, 64, 128, W.F32, [100, 129, 700]),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"G{c[1] // c[2]}-D{c[3]}-bs{c[4]}-{c[5]}")
def test_small_shapes(pa, oracle, case):
    B, Hq, Hkv, D, bs, dt, lens = case
    wl = W.make_workload("small", B, Hq, Hkv, D, bs, lens, dt, seed=sum(lens) + D)
    _parity(pa, oracle, wl)


@pytest.mark.parametrize("L", [1, 15, 16, 17, 63, 64, 65, 255, 256, 257, 511, 512, 513])
def test_edge_lengths(pa, oracle, L):
    wl = W.make_workload("edge", 2, 32, 8, 128, 16, [L, max(1, L // 2)], W.BF16, seed=L,
                         max_blocks=64)
    _parity(pa, oracle, wl, tag=f"L={L}")


def test_empty_sequences_give_zero_rows(pa, oracle):
    wl = W.make_workload("empty", 4, 8, 2, 128, 16, [0, 37, 0, 300], W.BF16, seed=3,
                         max_blocks=32)
    dw, _, _ = _parity(pa, oracle, wl)
    out = dw.out.cpu().numpy()
    assert np.array_equal(out[0], np.zeros_like(out[0]))
    assert np.array_equal(out[2], np.zeros_like(out[2]))


def test_config2_llama8b_full(pa, oracle):
    _parity(pa, oracle, W.config(2))


def test_config3_shared_prefix_full(pa, oracle):
    wl = W.config(3)
    dw, kc, vc = _parity(pa, oracle, wl)
    # the clones and the written slots are bit-exact over the whole cache
    assert np.array_equal(to_host(dw.k), kc)
    assert np.array_equal(to_host(dw.v), vc)


def test_config4_llama70b_full(pa, oracle):
    _parity(pa, oracle, W.config(4))


def test_config5_long_context_full(pa, oracle):
    """All 4 x 32 rows of the long-context batch (rows split over up to ~60 slices)."""
    _parity(pa, oracle, W.config(5))


@pytest.mark.parametrize("waves", [0, 37, 100])
def test_stream_rows_over_many_slices_reuse_workspace(pa, oracle, waves):
    """Long rows split over many slices (odd wave counts too), merged in slice order by the
    merge kernel; one workspace, filled with garbage first (it needs no initialisation),
    serves consecutive calls on different inputs."""
    lens = [5000, 1, 20000, 0, 7000, 64, 16, 333]
    wls = [W.make_workload("slices", 8, 32, 8, 128, 64, lens, W.BF16, seed=400 + i, max_blocks=320)
           for i in range(2)]
    with _path(pa, pa.PA_PATH_STREAM, waves=waves, min_slice=1):
        ws = torch.full((pa.pa_decode_workspace_bytes(8, 32, 8, 128, 64, 320, pa.PA_BF16),), 0x7f,
                        dtype=torch.uint8, device=DEV)
        for rep in range(3):
            wl = wls[rep % 2]
            note(f"many slices waves={waves} rep={rep}")
            dw = DevWorkload(wl)
            pa.pa_reshape_and_cache(dw.k, dw.v, dw.nk, dw.nv, dw.slots)
            pa.pa_decode(dw.out, dw.q, dw.k, dw.v, dw.bt, dw.sl, wl.scale, workspace=ws)
            torch.cuda.synchronize()
            ref, _, _ = oracle_step(oracle, wl)
            err = max_err(dw.out.cpu().numpy(), ref)
            note(f"  max abs err {err:.3e}")
            assert err <= TOL[wl.dtype]


def test_stream_workspace_sized_by_device_waves(pa):
    """The stream records are sized for the waves the device runs at once (one per SIMD),
    capped by what the batch can fill: 4.2 MB for the Llama-3-8B batch on 256 CUs."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    up = lambda x: (x + 255) // 256 * 256
    for (B, Hq, Hkv, D, bs, mb) in ((64, 32, 8, 128, 16, 256), (32, 64, 8, 128, 32, 256), (4, 2, 1, 64, 16, 3)):
        G = Hq // Hkv
        nw = 4 * cus
        ns = max(1, min(nw, B * Hkv * (-(-bs * mb // 16)) // 8))
        ml = up(2 * ns * G * D * 4)
        total = up(up(ml + 2 * ns * G * 8) + nw * 16) + 16
        assert pa.pa_decode_workspace_bytes(B, Hq, Hkv, D, bs, mb, pa.PA_BF16) == total


def test_cow_through_the_append_path(pa, oracle):
    """A prompt that ends inside a block (2040 tokens, bs 16) forked 4 ways; each fork
    appends one token through the reference block manager: three clone the shared last
    block (copy old -> new), the last writes in place."""
    from oracle.block_manager import Pool, SeqTable
    bs, prompt, nf = 16, 2040, 4
    base = W.make_workload("cow", 1, 32, 8, 128, bs, [prompt], W.BF16, seed=77, max_blocks=160,
                           num_blocks=200, keep_logical=True)
    mgr = Pool(base.num_blocks, bs,
               free_order=[int(x) for x in np.random.default_rng(1).permutation(base.num_blocks)])
    root = SeqTable(mgr, prompt)
    seqs = [root] + [root.branch() for _ in range(nf - 1)]
    rng = np.random.default_rng(2)
    k = np.full_like(base.k_cache, W.NAN_BF16)
    v = np.full_like(base.v_cache, W.NAN_BF16)
    for t in range(prompt):   # the shared prompt, in the manager's blocks
        k[root.table[t // bs], :, t % bs] = base.logical_k[0][t]
        v[root.table[t // bs], :, t % bs] = base.logical_v[0][t]
    pairs, slots = [], []
    for s in seqs:
        slot, cow = s.add_token()
        slots.append(slot)
        if cow:
            pairs.append(cow)
    assert len(pairs) == nf - 1
    tables = np.zeros((nf, 160), np.int32)
    for i, s in enumerate(seqs):
        tables[i, :len(s.table)] = s.table
    nk = W.bf16_from_f32(rng.standard_normal((nf, 8, 128), dtype=np.float32))
    nv = W.bf16_from_f32(rng.standard_normal((nf, 8, 128), dtype=np.float32))
    q = W.bf16_from_f32(rng.standard_normal((nf, 32, 128), dtype=np.float32))
    wl = W.Workload(name="cow", dtype=W.BF16, B=nf, Hq=32, Hkv=8, D=128, block_size=bs,
                    num_blocks=base.num_blocks, max_blocks=160, scale=base.scale, q=q,
                    k_cache=k, v_cache=v, block_tables=tables,
                    seq_lens=np.full(nf, prompt + 1, np.int32), new_key=nk, new_value=nv,
                    slot_mapping=np.array(slots, np.int32),
                    cow_pairs=np.array(pairs, np.int32))
    dw, kc, vc = _parity(pa, oracle, wl)
    assert np.array_equal(to_host(dw.k), kc) and np.array_equal(to_host(dw.v), vc)


# ------------------------------------------------------------------ bit-exact kernels

def test_steps_built_by_the_product_allocator(pa, oracle):
    """Every table, slot and copy-on-write pair comes from the product allocator
    (pa_alloc_allocate / fork / append_token): four prompts (2040, 2048, 333 and 17 tokens,
    the first ending inside a block) are written by pa_reshape_and_cache, forked 16, 8, 4
    and 2 ways, then every sequence appends three tokens, one per step, each step being
    pa_copy_blocks (the clones its appends asked for) -> pa_reshape_and_cache; then
    pa_decode. Caches must equal the oracle's replay of the same calls bit for bit, and the
    output must match the oracle's attention."""
    from tests._gpu_helpers import to_dev
    bs, Hq, Hkv, D, max_blocks, nb = 16, 32, 8, 128, 160, 640
    rng = np.random.default_rng(2040)
    alloc = pa.BlockAllocator(nb, bs, initial_free_order=rng.permutation(nb).astype(np.int32))
    k = np.full((nb, Hkv, bs, D), W.NAN_BF16, np.uint16)
    v = np.full_like(k, W.NAN_BF16)
    kd, vd = to_dev(k), to_dev(v)
    kc, vc = k, v

    def rand_rows(n):
        return W.bf16_from_f32(rng.standard_normal((n, Hkv, D), dtype=np.float32))

    def write(nk, nv, slots):
        nonlocal kc, vc
        st = pa.pa_validate_slots(slots, bs, nb)
        assert st[0] == pa.PA_OK, st
        pa.pa_reshape_and_cache(kd, vd, to_dev(nk), to_dev(nv), to_dev(np.asarray(slots, np.int32)))
        kc, vc = oracle.reshape_and_cache(kc, vc, nk, nv, np.asarray(slots, np.int32))

    tables, lens = [], []
    for L, forks in ((2040, 16), (2048, 8), (333, 4), (17, 2)):
        t = alloc.allocate(-(-L // bs))
        note(f"allocator-driven: prompt of {L} tokens in blocks {t[:4]}..., {forks} forks")
        write(rand_rows(L), rand_rows(L), [t[p // bs] * bs + p % bs for p in range(L)])
        tables += [t] + [alloc.fork(t) for _ in range(forks - 1)]
        lens += [L] * forks
    n_pairs = 0
    for rnd in range(3):
        slots, pairs = [], []
        for i in range(len(tables)):
            lens[i], slot, cow = alloc.append_token(tables[i], lens[i], table_cap=max_blocks)
            slots.append(slot)
            if cow:
                pairs.append(cow)
        note(f"allocator-driven step {rnd}: {len(pairs)} clone pairs")
        if pairs:
            pairs = np.asarray(pairs, np.int32)
            st = pa.pa_validate_block_pairs(pairs, nb)
            assert st[0] == pa.PA_OK, st
            pa.pa_copy_blocks(kd, vd, to_dev(pairs))
            kc, vc = oracle.copy_blocks(kc, vc, pairs)
            n_pairs += len(pairs)
        write(rand_rows(len(slots)), rand_rows(len(slots)), slots)
    # step 0 clones the shared partial last blocks: 15 (2040 tokens), 3 (333) and 1 (17)
    assert n_pairs == 15 + 3 + 1
    B = len(tables)
    bt = np.zeros((B, max_blocks), np.int32)
    for i, t in enumerate(tables):
        bt[i, :len(t)] = t
    sl = np.asarray(lens, np.int32)
    assert pa.pa_validate_decode(bt, sl, bs, nb)[0] == pa.PA_OK
    q = W.bf16_from_f32(rng.standard_normal((B, Hq, D), dtype=np.float32))
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    pa.pa_decode(out, to_dev(q), kd, vd, to_dev(bt), to_dev(sl), scale)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(kd), kc) and np.array_equal(to_host(vd), vc)
    ref = oracle.decode(q, kc, vc, bt, sl, scale)
    err = max_err(out.cpu().numpy(), ref)
    note(f"  allocator-driven decode: B={B} max abs err {err:.3e}")
    assert err <= TOL[W.BF16]


def test_reshape_and_cache_every_token_of_config2_bit_exact(pa, oracle):
    wl = W.config(2, keep_logical=True)
    bs = wl.block_size
    slots, keys, vals = [], [], []
    for b in range(wl.B):
        L = int(wl.seq_lens[b])
        t = np.arange(L)
        slots.append(wl.block_tables[b, t // bs] * bs + t % bs)
        keys.append(wl.logical_k[b])
        vals.append(wl.logical_v[b])
    slots = np.concatenate(slots).astype(np.int32)
    order = np.random.default_rng(0).permutation(len(slots))
    slots, keys, vals = slots[order], np.concatenate(keys)[order], np.concatenate(vals)[order]
    slots[::97] = -1                                   # padding entries are skipped
    empty = np.full_like(wl.k_cache, W.NAN_BF16)
    note(f"reshape_and_cache T={len(slots)}")
    kd, vd = (torch.from_numpy(empty.view(np.int16)).view(torch.bfloat16).to(DEV) for _ in range(2))
    from tests._gpu_helpers import to_dev
    pa.pa_reshape_and_cache(kd, vd, to_dev(keys), to_dev(vals), to_dev(slots))
    torch.cuda.synchronize()
    kr, vr = oracle.reshape_and_cache(empty, empty, keys, vals, slots)
    assert np.array_equal(to_host(kd), kr)
    assert np.array_equal(to_host(vd), vr)


def test_copy_blocks_bit_exact_fp32(pa, oracle):
    rng = np.random.default_rng(8)
    kc = rng.standard_normal((300, 4, 32, 64)).astype(np.float32)
    vc = rng.standard_normal((300, 4, 32, 64)).astype(np.float32)
    src = rng.choice(150, 90, replace=False)
    dst = 150 + rng.choice(150, 90, replace=False)
    pairs = np.stack([src, dst], 1).astype(np.int32)
    from tests._gpu_helpers import to_dev
    note("copy_blocks fp32 90 pairs")
    kd, vd = to_dev(kc), to_dev(vc)
    pa.pa_copy_blocks(kd, vd, to_dev(pairs))
    torch.cuda.synchronize()
    kr, vr = oracle.copy_blocks(kc, vc, pairs)
    assert np.array_equal(to_host(kd).view(np.uint32), kr.view(np.uint32))
    assert np.array_equal(to_host(vd).view(np.uint32), vr.view(np.uint32))


# ------------------------------------------------------------------ invariants (bitwise)

def test_placement_does_not_change_a_bit(pa):
    outs = []
    for placement in ("permute", "identity", "reversed"):
        wl = W.make_workload("perm", 6, 32, 8, 128, 16, [5, 300, 1024, 17, 2000, 64], W.BF16,
                             seed=44, placement=placement)
        note(f"placement {placement}")
        outs.append(gpu_step(pa, DevWorkload(wl)))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_poison_does_not_change_a_bit(pa):
    outs = []
    for poison in (True, False):
        wl = W.make_workload("poison", 5, 32, 8, 128, 32, [1, 31, 33, 700, 4000], W.BF16,
                             seed=12, poison=poison)
        note(f"poison {poison}")
        o = gpu_step(pa, DevWorkload(wl))
        assert np.isfinite(o).all()
        outs.append(o)
    assert np.array_equal(outs[0], outs[1])


def test_shared_prefix_equals_private_copies_bitwise(pa):
    wl = W.make_shared_prefix("s", 2, 4, 512, 40, 32, 8, 128, 16, W.BF16, seed=19,
                              keep_logical=True)
    note("shared prefix")
    shared = gpu_step(pa, DevWorkload(wl))
    priv = W.make_workload("p", wl.B, wl.Hq, wl.Hkv, wl.D, 16, wl.seq_lens, W.BF16, seed=1,
                           keep_logical=True)
    priv.q[:] = wl.q
    for b in range(wl.B):
        L = int(wl.seq_lens[b])
        for t in range(L - 1):
            blk = priv.block_tables[b, t // 16]
            priv.k_cache[blk, :, t % 16] = wl.logical_k[b][t]
            priv.v_cache[blk, :, t % 16] = wl.logical_v[b][t]
        priv.new_key[b] = wl.logical_k[b][L - 1]
        priv.new_value[b] = wl.logical_v[b][L - 1]
    note("private copies")
    private = gpu_step(pa, DevWorkload(priv))
    assert np.array_equal(shared, private)


def test_repeated_calls_are_bitwise_equal(pa):
    wl = W.config(4)
    dw = DevWorkload(wl)
    note("determinism cfg4")
    a = gpu_step(pa, dw).copy()
    for _ in range(3):
        pa.pa_decode(dw.out, dw.q, dw.k, dw.v, dw.bt, dw.sl, wl.scale)
    torch.cuda.synchronize()
    assert np.array_equal(a, dw.out.cpu().numpy())


@pytest.mark.parametrize("path", ["stream", "partition"])
def test_side_stream_with_library_workspace(pa, path):
    """pa_decode on a stream other than the current one, with the workspace left to the
    binding (uninitialised memory, held from reuse until that stream's work is done), while
    the current stream allocates and fills memory of the same size meanwhile: the bits of
    the call on the current stream."""
    wl = W.config(2)
    dw = DevWorkload(wl)
    mode = pa.PA_PATH_STREAM if path == "stream" else pa.PA_PATH_PARTITION
    with _path(pa, mode):
        note(f"side stream ({path}): reference on the current stream")
        ref = gpu_step(pa, dw).copy()
        need = pa.pa_decode_workspace_bytes(wl.B, wl.Hq, wl.Hkv, wl.D, wl.block_size,
                                            wl.max_blocks, pa.PA_BF16)
        side = torch.cuda.Stream()
        out = torch.empty_like(dw.out)
        side.wait_stream(torch.cuda.current_stream())
        note(f"side stream ({path}): 3 calls, workspace from the binding")
        for _ in range(3):
            pa.pa_decode(out, dw.q, dw.k, dw.v, dw.bt, dw.sl, wl.scale, stream=side)
            junk = torch.full((need,), 0x7f, dtype=torch.uint8, device=DEV)   # current stream
            del junk
        torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("P", [64, 128, 512, 1024])
def test_partition_length_changes_only_rounding(pa, oracle, P):
    wl = W.make_workload("split", 4, 32, 8, 128, 64, [100, 1023, 1025, 4000], W.BF16, seed=P,
                         max_blocks=64)
    with _path(pa, pa.PA_PATH_PARTITION, part_tokens=P):
        _parity(pa, oracle, wl, tag=f"partition P={P}")


@pytest.mark.parametrize("case", [c for c in SMALL if c[5] == W.BF16 and c[4] >= 16],
                         ids=lambda c: f"G{c[1] // c[2]}-D{c[3]}-bs{c[4]}")
def test_partition_path_bf16_small_shapes(pa, oracle, case):
    B, Hq, Hkv, D, bs, dt, lens = case
    wl = W.make_workload("small", B, Hq, Hkv, D, bs, lens, dt, seed=sum(lens) + D)
    with _path(pa, pa.PA_PATH_PARTITION):
        _parity(pa, oracle, wl, tag="partition")


def test_partition_path_config2(pa, oracle):
    with _path(pa, pa.PA_PATH_PARTITION):
        _parity(pa, oracle, W.config(2), tag="partition")


# rows cut across many slices: few waves, one group per slice allowed
SPLIT = [
    # B, Hq, Hkv, D, bs, lens, waves
    (6, 32, 8, 128, 16, [0, 1, 17, 300, 0, 2049], 4),
    (6, 32, 8, 128, 16, [0, 1, 17, 300, 0, 2049], 12),
    (5, 16, 2, 64, 32, [4000, 1, 33, 0, 640], 8),
    (3, 8, 8, 64, 64, [1, 1, 1], 64),             # more waves than groups
    (4, 8, 1, 128, 16, [1500, 3, 16, 4096], 4),   # slices of ~90 groups: window refresh
    (2, 64, 8, 128, 16, [2000, 999], 20),         # 8 query heads per KV head
    (3, 4, 4, 128, 32, [77, 0, 5000], 36),
    (4, 32, 8, 128, 8, [1, 9, 300, 2049], 12),    # 8-token blocks
    (3, 16, 2, 64, 128, [700, 0, 3000], 8),       # 128-token blocks
]


@pytest.mark.parametrize("case", SPLIT, ids=lambda c: f"G{c[1] // c[2]}-D{c[3]}-bs{c[4]}-w{c[6]}")
def test_stream_rows_split_across_slices(pa, oracle, case):
    B, Hq, Hkv, D, bs, lens, waves = case
    cap = -(-max(lens) // bs) * bs
    wl = W.make_workload("split", B, Hq, Hkv, D, bs, lens, W.BF16, seed=sum(lens) + waves,
                         max_blocks=max(1, cap // bs))
    with _path(pa, pa.PA_PATH_STREAM, waves=waves, min_slice=1):
        dw, _, _ = _parity(pa, oracle, wl, tag=f"stream waves={waves}")
    out = dw.out.cpu().numpy()
    for b, L in enumerate(lens):
        if L == 0:
            assert np.array_equal(out[b], np.zeros_like(out[b]))


def test_stream_config2_few_waves(pa, oracle):
    with _path(pa, pa.PA_PATH_STREAM, waves=100, min_slice=1):
        _parity(pa, oracle, W.config(2), tag="stream waves=100")


def test_stream_workspace_reused_across_calls(pa, oracle):
    """One workspace serves consecutive calls on different inputs (no stale partial state is
    read), with few waves so that many rows are merged, then with the default wave count."""
    from tests._gpu_helpers import to_dev
    wls = [W.make_workload("reuse", 6, 32, 8, 128, 16, [0, 1, 17, 300, 700, 2049], W.BF16,
                           seed=100 + i, max_blocks=129) for i in range(3)]
    need = 0
    for waves in (12, 0):   # the size depends on the wave settings: room for both
        with _path(pa, pa.PA_PATH_STREAM, waves=waves, min_slice=1):
            need = max(need, pa.pa_decode_workspace_bytes(6, 32, 8, 128, 16, 129, pa.PA_BF16))
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    for waves in (12, 0):
        with _path(pa, pa.PA_PATH_STREAM, waves=waves, min_slice=1):
            for wl in wls:
                note(f"workspace reuse waves={waves} seed={wl.seed if hasattr(wl, 'seed') else ''}")
                dw = DevWorkload(wl)
                pa.pa_reshape_and_cache(dw.k, dw.v, dw.nk, dw.nv, dw.slots)
                pa.pa_decode(dw.out, dw.q, dw.k, dw.v, dw.bt, dw.sl, wl.scale, workspace=ws)
                torch.cuda.synchronize()
                ref, _, _ = oracle_step(oracle, wl)
                err = max_err(dw.out.cpu().numpy(), ref)
                note(f"  max abs err {err:.3e}")
                assert err <= TOL[wl.dtype]


def test_stream_split_invariant_to_placement_and_poison(pa):
    outs = []
    for placement, poison in (("permute", True), ("identity", False), ("reversed", True)):
        wl = W.make_workload("perm", 6, 32, 8, 128, 16, [5, 300, 1024, 17, 2000, 64], W.BF16,
                             seed=44, placement=placement, poison=poison)
        note(f"stream split placement {placement} poison {poison}")
        with _path(pa, pa.PA_PATH_STREAM, waves=12, min_slice=1):
            o = gpu_step(pa, DevWorkload(wl))
        assert np.isfinite(o).all()
        outs.append(o)
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


@pytest.mark.parametrize("bs", [8, 128])
def test_placement_invariance_new_block_sizes(pa, bs):
    outs = []
    for placement in ("permute", "identity", "reversed"):
        wl = W.make_workload("perm", 5, 32, 8, 128, bs, [5, 300, 1024, 17, 2000], W.BF16,
                             seed=45, placement=placement)
        note(f"placement {placement} bs={bs}")
        outs.append(gpu_step(pa, DevWorkload(wl)))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


# ------------------------------------------------------------------ shared prefixes

def _shared_step(pa, wl, groups, max_members, max_shared):
    """copy_blocks -> reshape_and_cache -> pa_decode_shared, on the current stream."""
    from tests._gpu_helpers import to_dev
    dw = DevWorkload(wl)
    if dw.pairs is not None:
        pa.pa_copy_blocks(dw.k, dw.v, dw.pairs)
    pa.pa_reshape_and_cache(dw.k, dw.v, dw.nk, dw.nv, dw.slots)
    g = to_dev(np.asarray(groups, np.int32).reshape(-1, 3)) if len(groups) else None
    pa.pa_decode_shared(dw.out, dw.q, dw.k, dw.v, dw.bt, dw.sl, g, max_members, max_shared,
                        wl.scale)
    torch.cuda.synchronize()
    return dw.out.cpu().numpy()


def _shared_parity(pa, oracle, wl, groups, max_members, max_shared, tag):
    note(f"shared prefix {tag}: B={wl.B} Hq={wl.Hq} Hkv={wl.Hkv} D={wl.D} bs={wl.block_size} "
         f"groups={groups[:2]}...")
    got = _shared_step(pa, wl, groups, max_members, max_shared)
    ref, _, _ = oracle_step(oracle, wl)
    err = max_err(got, ref)
    note(f"  max abs err {err:.3e}")
    assert err <= TOL[wl.dtype]
    return got


SHARED = [
    # prompts, candidates, prompt tokens, extra tokens, Hq, Hkv, D, bs
    (3, 4, 512, 40, 32, 8, 128, 16),
    (2, 8, 256, 300, 64, 8, 128, 32),      # G = 8, 8 members: 64 query rows per KV head
    (2, 3, 384, 20, 16, 4, 64, 16),        # D = 64
    (2, 2, 1024, 100, 32, 8, 128, 128),    # 128-token blocks
]


@pytest.mark.parametrize("case", SHARED, ids=lambda c: f"p{c[0]}x{c[1]}-L{c[2]}-G{c[4] // c[5]}-D{c[6]}-bs{c[7]}")
def test_shared_prefix_decode(pa, oracle, case):
    npr, nc, plen, extra, Hq, Hkv, D, bs = case
    wl = W.make_shared_prefix("sp", npr, nc, plen, extra, Hq, Hkv, D, bs, W.BF16, seed=plen + bs)
    shared = plen - bs                       # the last prompt block is cloned per candidate
    groups = [(p * nc, nc, shared) for p in range(npr)]
    _shared_parity(pa, oracle, wl, groups, nc, shared, "all prompts")


def test_shared_prefix_mixed_members_and_rounding(pa, oracle):
    """Only some prompts form groups (the others are read per sequence), a shared count that
    is not a multiple of 16 (used as 480), and one member with no tokens of its own."""
    wl = W.make_shared_prefix("mix", 3, 4, 512, 60, 32, 8, 128, 16, W.BF16, seed=9)
    wl.seq_lens[9] = 496 - 7 - 2             # member of the third group: L = 487 > 480
    wl.seq_lens[8] = 480                     # exactly the rounded shared tokens
    groups = [(0, 4, 496), (8, 4, 489)]
    _shared_parity(pa, oracle, wl, groups, 4, 496, "mixed")


def test_shared_prefix_many_groups(pa, oracle):
    """More than 64 groups (the group search then takes more than one step), with prompts
    left out of every third group so that some sequences fall between groups."""
    wl = W.make_shared_prefix("many", 100, 2, 64, 20, 8, 2, 64, 16, W.BF16, seed=5)
    groups = [(p * 2, 2, 48) for p in range(100) if p % 3 != 1]
    assert len(groups) > 64
    _shared_parity(pa, oracle, wl, groups, 2, 48, "many groups")


def test_shared_prefix_no_groups_is_plain_decode(pa, oracle):
    wl = W.make_shared_prefix("none", 2, 4, 256, 30, 32, 8, 128, 16, W.BF16, seed=3)
    _shared_parity(pa, oracle, wl, [], 1, 0, "no groups")


def test_shared_prefix_config3_full(pa, oracle):
    wl = W.config(3)
    nc, shared = 8, 2048 - 16
    groups = [(p * nc, nc, shared) for p in range(16)]
    got = _shared_parity(pa, oracle, wl, groups, nc, shared, "config 3")
    dw = DevWorkload(wl)
    plain = gpu_step(pa, dw)                  # the same rows through pa_decode
    assert float(np.max(np.abs(plain - got))) <= TOL[wl.dtype]


def test_shared_prefix_repeatable(pa):
    outs = []
    for seed in (21, 21):
        wl = W.make_shared_prefix("inv", 2, 4, 512, 40, 32, 8, 128, 16, W.BF16, seed=seed)
        outs.append(_shared_step(pa, wl, [(0, 4, 496), (4, 4, 496)], 4, 496))
    assert np.array_equal(outs[0], outs[1])


def test_one_token_returns_its_value_exactly(pa):
    for dt in (W.F32, W.BF16):
        wl = W.make_workload("one", 3, 8, 2, 128, 16, [1, 1, 1], dt, seed=5, keep_logical=True)
        note(f"one token {dt}")
        out = gpu_step(pa, DevWorkload(wl))
        for b in range(3):
            v = wl.logical_v[b][0]
            v = W.bf16_to_f32(v) if dt == W.BF16 else v
            for h in range(8):
                assert np.array_equal(out[b, h], v[h // 4])


# ------------------------------------------------------------------ read-ceiling aid

@pytest.mark.parametrize("D,dtype", [(128, W.BF16), (64, W.BF16), (128, W.F32)],
                         ids=["d128-bf16", "d64-bf16", "d128-f32"])
def test_read_tiles_xor_matches_host(pa, D, dtype):
    """pa_read_tiles reads exactly the listed tiles of both caches: the XOR of its sink
    equals the XOR of every 32-bit word of those tiles, computed on the host."""
    rng = np.random.default_rng(D)
    L = rng.integers(1, 700, size=24).astype(np.int32)
    wl = W.make_workload(f"read-{D}", 24, 32, 8, D, 16, L, dtype, seed=D, poison=True)
    elt = 2 if dtype == W.BF16 else 4
    offs = W.group_tile_offsets(wl.block_tables, wl.seq_lens, wl.Hkv, wl.D, elt, 16)
    tile = 16 * D * elt
    kr = np.ascontiguousarray(wl.k_cache).view(np.uint8).reshape(-1)
    vr = np.ascontiguousarray(wl.v_cache).view(np.uint8).reshape(-1)
    assert offs.min() >= 0 and offs.max() + tile <= kr.size   # host guard before the launch
    note(f"read_tiles D={D} {dtype} tiles={len(offs)} tile_bytes={tile}")
    k, v = to_dev(wl.k_cache), to_dev(wl.v_cache)
    sink = torch.zeros(pa.READ_SINK_LEN, dtype=torch.int32, device=DEV)
    pa.pa_read_tiles(k, v, torch.from_numpy(offs).to(DEV), tile, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    idx = (offs[:, None] + np.arange(tile)[None, :]).reshape(-1)
    want = (np.bitwise_xor.reduce(kr[idx].view(np.uint32)) ^
            np.bitwise_xor.reduce(vr[idx].view(np.uint32)))
    assert got == want


@pytest.mark.parametrize("path", ["stream", "partition"])
def test_score_ramp_decode(pa, oracle, path):
    """K rows scaled up with position (scores climbing by hundreds of log2 units over a
    sequence, so the running maximum moves at almost every group), rows split over slices."""
    wl = W.make_workload("ramp-decode", 8, 32, 8, 128, 16, [1, 17, 700, 2000, 3000, 64, 1500, 900],
                         W.BF16, seed=63)
    scale_k_by_position(wl, lambda b, pos, L: 1.0 + pos / 40.0)
    mode = pa.PA_PATH_STREAM if path == "stream" else pa.PA_PATH_PARTITION
    with _path(pa, mode, waves=64 if path == "stream" else 0):
        _parity(pa, oracle, wl, tag=f"ramp {path}")


def test_binding_refuses_mismatched_tensors(pa):
    """Tensors whose element type, shape or device differ from what the kernels read and
    write are refused by the binding before any launch (a half-size fp16 output would
    otherwise be written past its end; int64 tables would be read as other entries)."""
    wl = W.make_workload("refuse", 3, 32, 8, 128, 16, [40, 300, 17], W.BF16, seed=3)
    dw = DevWorkload(wl)
    note("binding refuses mismatched tensors")
    bad = [
        dict(out=dw.out.half()),                              # output must be fp32
        dict(out=dw.out[:2]),                                  # B rows
        dict(q=dw.q.float()),                                  # q in the caches' type
        dict(block_tables=dw.bt.long()),                       # int32 tables
        dict(seq_lens=dw.sl[:2]),                              # one length per sequence
        dict(seq_lens=dw.sl.cpu()),                            # on the caches' device
        dict(v_cache=dw.v[:-1]),                               # same shape as k_cache
    ]
    base = dict(out=dw.out, q=dw.q, k_cache=dw.k, v_cache=dw.v, block_tables=dw.bt, seq_lens=dw.sl)
    for change in bad:
        args = dict(base, **change)
        with pytest.raises((TypeError, ValueError)):
            pa.pa_decode(args["out"], args["q"], args["k_cache"], args["v_cache"],
                         args["block_tables"], args["seq_lens"], wl.scale)
    with pytest.raises(ValueError):
        pa.pa_reshape_and_cache(dw.k, dw.v, dw.nk[:2], dw.nv, dw.slots)
    with pytest.raises(TypeError):
        pa.pa_copy_blocks(dw.k, dw.v, torch.zeros((1, 2), dtype=torch.int64, device=DEV))
    torch.cuda.synchronize()
    # the correct call still runs
    got = gpu_step(pa, dw)
    assert np.isfinite(got).all()
