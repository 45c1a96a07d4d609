"""pa_decode_append (one decode step in one launch: the newest tokens' cache write and the
decode that reads them) against pa_reshape_and_cache followed by pa_decode, on an MI355X
through the C ABI: outputs and both caches bit for bit, on every seeded workload and on both
decompositions, and the output against the fp64 oracle within the bf16 / fp32 bounds."""
import numpy as np
import pytest
import torch

from paged_kv_cache_298_amd import workloads as W
from tests._gpu_helpers import (DEV, TOL, DevWorkload, check_inputs, max_err, note, oracle_step,
                                to_dev, to_host)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_298_amd import pa as _pa
    _pa.pa_set_decode_path(_pa.PA_PATH_AUTO)
    _pa.pa_set_stream_waves(0, 0)
    _pa.pa_set_partition_tokens(0)
    return _pa


def _both(pa, wl, slots=None):
    """(two-launch output, k, v), (fused output, k, v), on separate copies of the inputs."""
    check_inputs(wl)
    slots = wl.slot_mapping if slots is None else slots
    st = pa.pa_validate_append(slots, wl.block_tables, wl.seq_lens, wl.block_size, wl.num_blocks)
    assert st[0] == pa.PA_OK, st
    res = []
    for fused in (False, True):
        dw = DevWorkload(wl)
        sl = to_dev(np.asarray(slots, np.int32))
        if dw.pairs is not None:
            pa.pa_copy_blocks(dw.k, dw.v, dw.pairs)
        dw.out.fill_(float("nan"))
        if fused:
            pa.pa_decode_append(dw.out, dw.q, dw.k, dw.v, dw.nk, dw.nv, sl, dw.bt, dw.sl, wl.scale)
        else:
            pa.pa_reshape_and_cache(dw.k, dw.v, dw.nk, dw.nv, sl)
            pa.pa_decode(dw.out, dw.q, dw.k, dw.v, dw.bt, dw.sl, wl.scale)
        torch.cuda.synchronize()
        res.append((dw.out.cpu().numpy(), to_host(dw.k), to_host(dw.v)))
    return res


def _same_bits(a, b):
    return np.array_equal(np.ascontiguousarray(a).view(np.uint8), np.ascontiguousarray(b).view(np.uint8))


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_append_equals_write_then_decode(pa, oracle, cfg):
    wl = W.config(cfg)
    note(f"append vs write+decode, workload {cfg}: {wl.name}")
    (o2, k2, v2), (o1, k1, v1) = _both(pa, wl)
    assert _same_bits(k1, k2) and _same_bits(v1, v2)
    assert _same_bits(o1, o2)
    if cfg in (1, 3):
        ref, kc, _ = oracle_step(oracle, wl)
        err = max_err(o1, ref)
        note(f"  max abs err {err:.3e}")
        assert err <= TOL[wl.dtype] and _same_bits(k1, kc)


@pytest.mark.parametrize("waves", [12, 100])
@pytest.mark.parametrize("bs", [8, 16, 64])
def test_append_with_rows_split_over_slices(pa, oracle, bs, waves):
    """Rows split across many slices, blocks of 8 (a 16-token group spans two blocks), 16
    and 64 tokens, lengths that put the newest token at every position of its group."""
    lens = [1, 15, 16, 17, 31, 32, 33, 250, 700, 1]
    wl = W.make_workload(f"append-bs{bs}", len(lens), 32, 8, 128, bs, lens, W.BF16, seed=bs + waves,
                         max_blocks=-(-704 // bs))
    pa.pa_set_decode_path(pa.PA_PATH_STREAM)
    pa.pa_set_stream_waves(waves, 1)
    try:
        note(f"append bs={bs} waves={waves}")
        (o2, k2, v2), (o1, k1, v1) = _both(pa, wl)
    finally:
        pa.pa_set_decode_path(pa.PA_PATH_AUTO)
        pa.pa_set_stream_waves(0, 0)
    assert _same_bits(k1, k2) and _same_bits(v1, v2) and _same_bits(o1, o2)
    ref, _, _ = oracle_step(oracle, wl)
    assert max_err(o1, ref) <= TOL[W.BF16]


def test_append_rows_without_a_new_token_read_the_cache(pa, oracle):
    """Sequences whose slot is -1 have no new token in this call: their position L - 1 is
    read from the cache (written beforehand here), as the two-launch form reads it."""
    lens = [40, 17, 300, 5, 64, 129]
    wl = W.make_workload("append-pad", 6, 32, 8, 128, 16, lens, W.BF16, seed=9)
    slots = wl.slot_mapping.copy()
    slots[[1, 4, 5]] = -1                    # written by an earlier call; no new token now
    res = []
    for fused in (False, True):
        dw = DevWorkload(wl)
        pa.pa_reshape_and_cache(dw.k, dw.v, dw.nk, dw.nv, to_dev(np.where(slots < 0, wl.slot_mapping, -1).astype(np.int32)))
        sl = to_dev(slots.astype(np.int32))
        if fused:
            pa.pa_decode_append(dw.out, dw.q, dw.k, dw.v, dw.nk, dw.nv, sl, dw.bt, dw.sl, wl.scale)
        else:
            pa.pa_reshape_and_cache(dw.k, dw.v, dw.nk, dw.nv, sl)
            pa.pa_decode(dw.out, dw.q, dw.k, dw.v, dw.bt, dw.sl, wl.scale)
        torch.cuda.synchronize()
        res.append((dw.out.cpu().numpy(), to_host(dw.k)))
    assert _same_bits(res[0][0], res[1][0]) and _same_bits(res[0][1], res[1][1])
    ref, _, _ = oracle_step(oracle, wl)      # every newest token ends up in the cache
    assert max_err(res[1][0], ref) <= TOL[W.BF16]


def test_append_repeats_bitwise_and_returns_its_status(pa):
    wl = W.config(2)
    dw = DevWorkload(wl)
    sl = to_dev(wl.slot_mapping)
    outs = []
    for _ in range(2):
        pa.pa_decode_append(dw.out, dw.q, dw.k, dw.v, dw.nk, dw.nv, sl, dw.bt, dw.sl, wl.scale)
        torch.cuda.synchronize()
        outs.append(dw.out.cpu().numpy().copy())
    assert _same_bits(outs[0], outs[1])
    with pytest.raises(pa.PaError):
        pa._check(pa._lib.pa_decode_append(None, None, None, None, None, None, None, None, None, 4, 32, 8,
                                           128, 16, 64, 3, 0.1, pa.PA_BF16, None, 0, None))
