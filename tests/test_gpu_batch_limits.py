"""Batches at the stream decomposition's size limit and one past it.

The stream kernel keeps each sequence's clamped length and the prefix of its 16-token
groups in LDS, so it takes up to 4096 sequences (4096 x 3 + 1 words with the fused cache
write); a bf16 batch of 4097 sequences runs on the partition decomposition instead. Every
output row is compared with the oracle; the fused append is compared bit for bit with the
cache write followed by the decode.
"""
import numpy as np
import pytest
import torch

from paged_kv_cache_298_amd import workloads as W
from tests._gpu_helpers import (DEV, TOL, DevWorkload, check_inputs, gpu_step, max_err, note,
                                oracle_step, to_host)

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


def _many(B, seed):
    """B short sequences (1-80 tokens, a few of 300-700, every 97th empty)."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, 81, size=B).astype(np.int32)
    lens[rng.choice(B, size=B // 64, replace=False)] = rng.integers(300, 701, size=B // 64)
    lens[::97] = 0
    return W.make_workload(f"many-{B}", B, 32, 8, 128, 16, lens, W.BF16, seed=seed,
                           max_blocks=48)


@pytest.mark.parametrize("B", [4096, 4097], ids=["stream-at-limit", "partition-past-limit"])
def test_largest_batches_match_the_oracle(pa, oracle, B):
    wl = _many(B, seed=B)
    check_inputs(wl)
    ws = pa.pa_decode_workspace_bytes(B, 32, 8, 128, 16, 48, pa.PA_BF16)
    note(f"batch limit B={B}: workspace {ws} bytes, lens max {int(wl.seq_lens.max())}")
    got = gpu_step(pa, DevWorkload(wl))
    ref, _, _ = oracle_step(oracle, wl)
    err = max_err(got, ref)
    note(f"  max abs err {err:.3e}")
    assert err <= TOL[wl.dtype]
    assert not got[wl.seq_lens == 0].any()          # empty sequences: zero rows


def test_append_at_the_batch_limit(pa):
    """pa_decode_append at B = 4096 (the fused launch's LDS holds 3 B + 1 words) gives the
    bits of pa_reshape_and_cache followed by pa_decode, caches included."""
    wl = _many(4096, seed=7)
    check_inputs(wl)
    note("append at B=4096: separate launches")
    a = DevWorkload(wl)
    sep = gpu_step(pa, a)
    note("append at B=4096: one launch")
    b = DevWorkload(wl)
    pa.pa_decode_append(b.out, b.q, b.k, b.v, b.nk, b.nv, b.slots, b.bt, b.sl, wl.scale)
    torch.cuda.synchronize()
    assert np.array_equal(b.out.cpu().numpy().view(np.uint32), sep.view(np.uint32))
    assert np.array_equal(to_host(b.k), to_host(a.k)) and np.array_equal(to_host(b.v), to_host(a.v))
