"""Parity of pa_decode_multi (causal multi-query attention: prefill, prompt chunks, draft
tokens) with the oracle, on an MI355X, through the C ABI.

Each step writes the chunk's K/V with pa_reshape_and_cache, then runs pa_decode_multi.
Max-abs error over every output element <= 2e-2 (bf16 caches, fp32 accumulation), at
full size too.
"""
import numpy as np
import pytest
import torch

from paged_kv_cache_298_amd import workloads as W
from tests._gpu_helpers import (DEV, TOL, check_inputs, max_err, note, scale_k_by_position,
                                to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_298_amd import pa as _pa
    return _pa


def _check_chunks(wl):
    qs = wl.q_starts
    n = np.diff(qs)
    assert qs[0] == 0 and qs[-1] == wl.q.shape[0] and np.all(n >= 0) and np.all(n <= wl.seq_lens)


def _multi_gpu(pa, wl, repeat=1):
    check_inputs(wl)
    _check_chunks(wl)
    k, v = to_dev(wl.k_cache), to_dev(wl.v_cache)
    q, bt, sl, qs = to_dev(wl.q), to_dev(wl.block_tables), to_dev(wl.seq_lens), to_dev(wl.q_starts)
    out = torch.full((wl.q.shape[0], wl.Hq, wl.D), float("nan"), dtype=torch.float32, device=DEV)
    pa.pa_reshape_and_cache(k, v, to_dev(wl.new_key), to_dev(wl.new_value), to_dev(wl.slot_mapping))
    max_q = int(np.diff(wl.q_starts).max(initial=0))
    outs = []
    for _ in range(repeat):
        pa.pa_decode_multi(out, q, k, v, bt, sl, qs, max_q, wl.scale)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy().copy())
    return outs, (k, v, bt, sl)


def _multi_oracle(oracle, wl, rows=None):
    kc, vc = oracle.reshape_and_cache(wl.k_cache, wl.v_cache, wl.new_key, wl.new_value,
                                      wl.slot_mapping)
    return oracle.decode_multi(wl.q, kc, vc, wl.block_tables, wl.seq_lens, wl.q_starts,
                               wl.scale, rows=rows)


def _parity(pa, oracle, wl, tag, rows=None):
    n = np.diff(wl.q_starts)
    note(f"multi {tag}: B={wl.B} Hq={wl.Hq} Hkv={wl.Hkv} D={wl.D} bs={wl.block_size} "
         f"lens[:6]={list(wl.seq_lens[:6])} n[:6]={list(n[:6])} total_q={int(wl.q_starts[-1])}")
    (got,), _ = _multi_gpu(pa, wl)
    ref = _multi_oracle(oracle, wl, rows=rows)
    if rows is not None:
        got = got.reshape(-1, wl.D)[rows]
    assert np.all(np.isfinite(got))
    err = max_err(got, ref)
    note(f"  max abs err {err:.3e}")
    assert err <= TOL[wl.dtype]
    return got


MULTI = [
    # name, lens, n_new, Hq, Hkv, D, bs
    ("tiny", [5, 16, 40], [5, 3, 17], 8, 2, 64, 16),
    ("prompts", [300, 700], [300, 700], 32, 8, 128, 32),            # whole prompts (prefill)
    ("chunks-g8", [1500, 2100], [256, 512], 64, 8, 128, 64),        # 66-group partitions
    ("mixed", [40, 1, 333, 90, 17], [0, 1, 33, 90, 4], 16, 4, 64, 128),
    ("g1", [100, 250, 64], [7, 250, 1], 4, 4, 128, 16),
    ("d64-g8-bs64", [700, 130, 1], [70, 130, 1], 64, 8, 64, 64),   # one-token prompt
    ("g2-long", [3000, 2500], [40, 1], 16, 8, 128, 32),             # split partitions, G=2
    ("g5-mixed", [9000, 300, 5000], [600, 300, 40], 40, 8, 128, 16),  # G=5, partitions
]


@pytest.mark.parametrize("case", MULTI, ids=lambda c: c[0])
def test_multi_matches_oracle(pa, oracle, case):
    name, lens, n_new, Hq, Hkv, D, bs = case
    wl = W.make_workload(f"mq-{name}", len(lens), Hq, Hkv, D, bs, lens, W.BF16,
                         seed=sum(lens) + bs, n_new=n_new)
    _parity(pa, oracle, wl, name)


def test_draft_tokens_split_partitions(pa, oracle):
    """Four draft tokens per sequence on ragged lengths: one query tile per (sequence, KV
    head), so the tokens are split into partitions and merged."""
    rng = np.random.default_rng(41)
    lens = rng.integers(4, 1200, size=16)
    wl = W.make_workload("mq-draft", 16, 32, 8, 128, 16, lens, W.BF16, seed=41, n_new=[4] * 16)
    from paged_kv_cache_298_amd import pa as _pa
    assert _pa.pa_decode_multi_workspace_bytes(16, 64, 4, 32, 8, 128, 16, wl.max_blocks) > 0
    _parity(pa, oracle, wl, "draft")


def test_one_query_per_sequence_matches_pa_decode(pa, oracle):
    rng = np.random.default_rng(3)
    lens = rng.integers(1, 900, size=12)
    wl = W.make_workload("mq-one", 12, 32, 8, 128, 16, lens, W.BF16, seed=3, n_new=[1] * 12)
    got = _parity(pa, oracle, wl, "one query")
    dec = W.make_workload("mq-one", 12, 32, 8, 128, 16, lens, W.BF16, seed=3)
    assert np.array_equal(dec.q, wl.q) and np.array_equal(dec.k_cache, wl.k_cache)
    k, v = to_dev(dec.k_cache), to_dev(dec.v_cache)
    pa.pa_reshape_and_cache(k, v, to_dev(dec.new_key), to_dev(dec.new_value), to_dev(dec.slot_mapping))
    out = torch.empty((12, 32, 128), dtype=torch.float32, device=DEV)
    pa.pa_decode(out, to_dev(dec.q), k, v, to_dev(dec.block_tables), to_dev(dec.seq_lens), dec.scale)
    torch.cuda.synchronize()
    assert max_err(got, out.cpu().numpy()) <= TOL[W.BF16]


def test_multi_repeatable_bitwise(pa):
    wl = W.make_workload("mq-rep", 3, 32, 8, 128, 16, [400, 90, 1300], W.BF16, seed=5,
                         n_new=[64, 90, 8])
    outs, _ = _multi_gpu(pa, wl, repeat=2)
    assert np.array_equal(outs[0], outs[1])


def test_placement_leaves_multi_bitwise_equal(pa):
    outs = []
    for placement in ("permute", "identity"):
        wl = W.make_workload("mq-pl", 3, 32, 8, 128, 16, [400, 90, 1300], W.BF16, seed=5,
                             n_new=[64, 90, 8], placement=placement)
        (o,), _ = _multi_gpu(pa, wl)
        outs.append(o)
    assert np.array_equal(outs[0], outs[1])


def test_draft_tokens_llama3_batch_full(pa, oracle):
    """The Llama-3-8B batch's lengths with four draft tokens per sequence, at full size,
    every one of its 256 x 32 query rows against the oracle (the multi-query bench batch)."""
    rng = np.random.default_rng(29802)
    lens = rng.integers(1, 4097, size=64).astype(np.int32)
    lens = np.maximum(lens, 4)
    wl = W.make_workload("mq-llama3-draft", 64, 32, 8, 128, 16, lens, W.BF16, seed=29802,
                         max_blocks=256, n_new=[4] * 64)
    _parity(pa, oracle, wl, "llama3 draft")


def test_prompt_chunks_bench_batch_full(pa, oracle):
    """The chunked-prefill bench batch: 1024-token chunks of 4 sequences after 0, 1024, 2048
    and 3072 cached tokens (64 query tiles per row, lazy rescale over up to 4096 tokens),
    every output row against the oracle."""
    wl = W.make_workload("chunks", 4, 32, 8, 128, 16, [1024, 2048, 3072, 4096], W.BF16, 29806,
                         max_blocks=256, n_new=[1024] * 4)
    _parity(pa, oracle, wl, "chunk bench batch")


def test_loose_max_q_bound_and_empty_chunks(pa, oracle):
    """max_q larger than any chunk (it only sizes the tiles), and a batch in which most
    sequences have no queries at all."""
    wl = W.make_workload("mq-loose", 5, 32, 8, 128, 16, [50, 900, 17, 333, 64], W.BF16, seed=77,
                         n_new=[0, 9, 0, 0, 2])
    _check_chunks(wl)
    k, v = to_dev(wl.k_cache), to_dev(wl.v_cache)
    pa.pa_reshape_and_cache(k, v, to_dev(wl.new_key), to_dev(wl.new_value), to_dev(wl.slot_mapping))
    out = torch.full((11, 32, 128), float("nan"), dtype=torch.float32, device=DEV)
    note("multi loose max_q=64 for chunks of at most 9")
    pa.pa_decode_multi(out, to_dev(wl.q), k, v, to_dev(wl.block_tables), to_dev(wl.seq_lens),
                       to_dev(wl.q_starts), 64, wl.scale)
    torch.cuda.synchronize()
    ref = _multi_oracle(oracle, wl)
    assert max_err(out.cpu().numpy(), ref) <= TOL[W.BF16]


def test_more_sequences_than_the_longest_first_order_holds(pa, oracle):
    """2100 sequences (the longest-first order handles up to 2048; beyond that the waves
    take the query tiles in grid order): every row against the oracle."""
    rng = np.random.default_rng(2100)
    lens = rng.integers(6, 41, size=2100)
    wl = W.make_workload("mq-many", 2100, 8, 2, 64, 16, lens, W.BF16, seed=2100, n_new=[6] * 2100)
    _parity(pa, oracle, wl, "2100 sequences (grid order)")


# ------------------------------------------------ the stream decomposition (<= 16 columns)

STREAM = [
    # name, lens, n_new, Hq, Hkv, D, bs   (max n x G <= 16: one score tile per row)
    ("g4-n4", [300, 1, 77, 1000, 17, 640], [4, 1, 3, 4, 0, 2], 32, 8, 128, 16),
    ("g8-n2", [500, 33, 900], [2, 1, 2], 64, 8, 128, 32),
    ("g2-n3", [129, 400, 3, 64], [3, 3, 3, 1], 16, 8, 128, 16),    # 6 of 8 columns used
    ("g1-n16", [700, 16, 300], [16, 16, 5], 8, 8, 64, 64),
    # 4 columns (record-split merge); each sequence's last group holds one or two tokens
    # that the chunk's first query does not see, so with many waves a slice can hold only
    # segments in which some column sees no token
    ("g2-n2-edge-d64", [33, 49, 17, 1000, 34], [2, 2, 2, 2, 3], 16, 8, 64, 16),
    ("g2-n2-edge-d128", [33, 65, 17, 600, 34], [2, 2, 2, 2, 2], 16, 8, 128, 16),
]


@pytest.mark.parametrize("waves", [0, 96], ids=["all-waves", "96-waves"])
@pytest.mark.parametrize("case", STREAM, ids=lambda c: c[0])
def test_stream_decomposition_matches_oracle(pa, oracle, case, waves):
    """Draft-sized chunks go through the decode kernel's slices (equal groups per wave,
    rows split across waves and merged); with 96 waves most rows are split."""
    name, lens, n_new, Hq, Hkv, D, bs = case
    wl = W.make_workload(f"mqs-{name}", len(lens), Hq, Hkv, D, bs, lens, W.BF16,
                         seed=sum(lens) + 3 * bs, n_new=n_new)
    pa.pa_set_stream_waves(waves, 1 if waves else 0)
    try:
        _parity(pa, oracle, wl, f"stream {name} waves={waves}")
    finally:
        pa.pa_set_stream_waves(0, 0)


def test_stream_and_tile_decompositions_agree(pa):
    rng = np.random.default_rng(12)
    lens = rng.integers(4, 2000, size=24)
    wl = W.make_workload("mqs-agree", 24, 32, 8, 128, 16, lens, W.BF16, seed=12, n_new=[4] * 24)
    (a,), _ = _multi_gpu(pa, wl)
    pa.pa_set_decode_path(pa.PA_PATH_PARTITION)        # query tiles instead
    try:
        (b,), _ = _multi_gpu(pa, wl)
    finally:
        pa.pa_set_decode_path(pa.PA_PATH_AUTO)
    assert max_err(a, b) <= TOL[W.BF16]


@pytest.mark.parametrize("case", MULTI[1:] + [
    ("chunk-bench", [1024, 2048, 3072, 4096], [1024] * 4, 32, 8, 128, 16),
    ("long-tile-last", [4096, 4064], [4096, 64], 32, 8, 128, 16),
], ids=lambda c: c[0])
def test_longest_first_and_grid_order_give_the_same_bits(pa, case):
    """The query-tile work is handed out longest first by default; the plain grid order
    runs the same units, each with the same arithmetic, so every output bit agrees."""
    name, lens, n_new, Hq, Hkv, D, bs = case
    wl = W.make_workload(f"mq-order-{name}", len(lens), Hq, Hkv, D, bs, lens, W.BF16, seed=77,
                         n_new=n_new)
    note(f"multi order {name}: lens={lens} n={n_new}")
    outs = []
    try:
        for order in (1, 0):
            pa.pa_set_multi_order(order)
            (o,), _ = _multi_gpu(pa, wl)
            outs.append(o)
    finally:
        pa.pa_set_multi_order(1)
    assert np.all(np.isfinite(outs[0]))
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))


RAMPS = [
    # name, profile of the K row scale over positions: scores whose maxima climb steadily
    # (many small moves of the softmax reference, and moves just under and past the lazy
    # threshold), fall (the reference set early, later probabilities vanish), or jump
    ("rising", lambda b, pos, L: 1.0 + pos / 40.0),
    ("falling", lambda b, pos, L: 1.0 + (L - pos) / 40.0),
    ("spikes", lambda b, pos, L: 60.0 if (pos * 7919 + b) % 389 == 0 else 1.0),
]


@pytest.mark.parametrize("ramp", RAMPS, ids=lambda r: r[0])
@pytest.mark.parametrize("shape", ["chunks", "draft"])
def test_score_ramps_through_the_softmax_reference(pa, oracle, shape, ramp):
    """Score ranges of hundreds of log2 units: the chunk items' lazy reference and the stream
    kernel's running maximum against the oracle."""
    name, prof = ramp
    if shape == "chunks":
        wl = W.make_workload(f"ramp-{name}", 3, 32, 8, 128, 16, [1200, 2000, 700], W.BF16,
                             seed=61, n_new=[600, 300, 700])
    else:
        wl = W.make_workload(f"ramp-{name}-draft", 6, 32, 8, 128, 16,
                             [1200, 2000, 700, 64, 3000, 4], W.BF16, seed=62, n_new=[4] * 6)
    scale_k_by_position(wl, prof)
    _parity(pa, oracle, wl, f"{shape} {name}")


LONG = [
    # name, lens, n_new: a 16,384-token prompt as one prefill (1,024 query tiles per KV
    # head, one partition), a 2,048-token chunk at the end of a 32,768-token context, and a
    # 256-token chunk there (few tiles: the context is cut into partitions, then merged)
    ("prefill-16k", [16384], [16384]),
    ("chunk-at-32k", [32768, 900], [2048, 100]),
    ("short-chunk-at-32k", [32768, 900], [256, 100]),
]


@pytest.mark.parametrize("case", LONG, ids=lambda c: c[0])
def test_long_prefill_and_late_chunk(pa, oracle, case):
    """The longest query ranges: every (query, head) row is computed on the GPU and 512
    rows spread over the whole range (the first and last of each sequence included) are
    compared with the oracle one by one."""
    name, lens, n_new = case
    wl = W.make_workload(f"mq-{name}", len(lens), 32, 8, 128, 16, lens, W.BF16,
                         seed=sum(lens), n_new=n_new)
    total = int(wl.q_starts[-1])
    rng = np.random.default_rng(7)
    firsts = [int(wl.q_starts[b]) * wl.Hq for b in range(wl.B)]
    lasts = [int(wl.q_starts[b + 1]) * wl.Hq - 1 for b in range(wl.B)]
    rows = np.unique(np.concatenate([firsts, lasts, rng.integers(0, total * wl.Hq, size=508)]))
    _parity(pa, oracle, wl, name, rows=rows.astype(np.int32))
