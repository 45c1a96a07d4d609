"""The decode step captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

The library launches kernels only on the stream it is given and records no memset or copy,
so a step captures as it is. Each test replays the graph several times with new queries,
lengths and cache contents written eagerly between the replays, and compares every replay
bit for bit with the same calls made eagerly on the same inputs.
"""
import numpy as np
import pytest
import torch

from paged_kv_cache_298_amd import workloads as W
from tests._gpu_helpers import DEV, DevWorkload, check_inputs, note, to_dev

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


def _batch():
    rng = np.random.default_rng(31)
    lens = rng.integers(17, 2000, size=24).astype(np.int32)
    wl = W.make_workload("graph", 24, 32, 8, 128, 16, lens, W.BF16, seed=31)
    check_inputs(wl)
    return wl


def _bits(t):
    return t.cpu().numpy().view(np.uint32).copy()


def _inputs_for_replay(dw, wl, r, shorten):
    """New queries and new-token rows for replay r; with `shorten`, lengths up to two
    tokens shorter too (the decode then reads fewer cached tokens; tables stay valid)."""
    rng = np.random.default_rng(100 + r)
    dw.q.copy_(torch.from_numpy(rng.standard_normal(dw.q.shape).astype(np.float32)).to(DEV).to(dw.q.dtype))
    dw.nk.copy_(torch.from_numpy(rng.standard_normal(dw.nk.shape).astype(np.float32)).to(DEV).to(dw.nk.dtype))
    if shorten:
        lens = wl.seq_lens - rng.integers(0, 3, size=wl.B).astype(np.int32)
        dw.sl.copy_(to_dev(np.maximum(lens, 1).astype(np.int32)))


@pytest.mark.parametrize("entry", ["pa_decode", "pa_decode_noalloc", "pa_decode_append"])
def test_graph_replays_equal_eager_calls(pa, entry):
    wl = _batch()
    dw = DevWorkload(wl)
    need = pa.pa_decode_workspace_bytes(wl.B, wl.Hq, wl.Hkv, wl.D, 16, wl.max_blocks, pa.PA_BF16)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=DEV)
    out = torch.empty_like(dw.out)

    def step(o, w):
        if entry == "pa_decode":
            pa.pa_reshape_and_cache(dw.k, dw.v, dw.nk, dw.nv, dw.slots)
            pa.pa_decode(o, dw.q, dw.k, dw.v, dw.bt, dw.sl, wl.scale, workspace=w)
        elif entry == "pa_decode_noalloc":
            pa.pa_reshape_and_cache(dw.k, dw.v, dw.nk, dw.nv, dw.slots)
            pa.pa_decode_noalloc(o, dw.q, dw.k, dw.v, dw.bt, dw.sl, wl.scale)
        else:
            pa.pa_decode_append(o, dw.q, dw.k, dw.v, dw.nk, dw.nv, dw.slots, dw.bt, dw.sl,
                                wl.scale, workspace=w)

    note(f"graph {entry}: warm-up on a side stream, then capture")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(out, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(out, ws)
    torch.cuda.synchronize()

    ref_out = torch.empty_like(dw.out)
    ref_ws = torch.empty_like(ws)
    for r in range(4):
        # the fused append writes the token at position L - 1: its lengths stay as built
        _inputs_for_replay(dw, wl, r, shorten=entry != "pa_decode_append")
        torch.cuda.synchronize()
        note(f"graph {entry}: replay {r}")
        g.replay()
        torch.cuda.synchronize()
        got = _bits(out)
        step(ref_out, ref_ws)                     # the same step, eagerly
        torch.cuda.synchronize()
        want = _bits(ref_out)
        assert np.isfinite(out.cpu().numpy()).all()
        assert np.array_equal(got, want), f"replay {r}"
