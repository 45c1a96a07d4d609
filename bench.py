"""Benchmark: one decode step of paged attention on one MI355X.

A step is the whole hot path over one batch: clone shared blocks (copy_blocks, when the
workload has copy-on-write pairs), then pa_decode_append, which writes each sequence's
newest K/V to its slot (the reshape_and_cache step) and runs paged decode attention over
the batch in one launch (stream decode kernel + split-row merge). The same step as separate
launches (reshape_and_cache, then pa_decode) is timed too, for context. Inputs
are seeded synthetic data resident in HBM before timing starts; successive steps rotate
over R replicas of (pool, q, tables, ...) so the working set exceeds the 256 MB Infinity
Cache. Prints ONE JSON line.

  value        effective KV GB/s of the step: sum_b L_b * Hkv * D * 2 * elt / step time
  roofline     pa_decode alone: the same KV bytes / its mean duration (HIP events around
               each call, on the stream it runs on) against 8 TB/s
  cpu_baseline the fp64 oracle (OpenMP, all host threads) on the same step, repeated for a
               bounded ~10 s sample
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBS = 8000.0
METRIC = "paged decode attention effective KV GB/s (% of HBM peak); µs per decode step"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_pa_decode.json")
# the sources the decode kernels are compiled from (the traffic summary is tied to them)
DECODE_SRCS = [os.path.join(ROOT, "paged_kv_cache_298_amd", "csrc", f)
               for f in ("pa_decode.hip", "pa_device.h")]


def _log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _to_dev(a, torch, dev):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(a).to(dev)


def _decode_source_sha():
    h = hashlib.sha256()
    for path in DECODE_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic_for(config_name):
    """HBM bytes per pa_decode launch from the committed rocprofv3 counter summary, only
    while the kernel source is the one the counters were taken from."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha") != _decode_source_sha():
        return None
    entry = rec.get("workloads", {}).get(config_name)
    return entry.get("bytes_per_launch") if entry else None


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _cpu_baseline(wl, budget_s, one_thread=False):
    """The fp64 oracle on the whole step (copy_blocks if any, cache write, decode of every
    row), repeated for about budget_s on all the host threads OpenMP offers; with
    one_thread, also on one thread for about half as long (at least one step)."""
    from oracle import oracle as orc
    threads = orc.max_threads()

    def run(n_threads, budget):
        reps, t0 = 0, time.perf_counter()
        while True:
            kc, vc = wl.k_cache, wl.v_cache
            if wl.cow_pairs.shape[0]:
                kc, vc = orc.copy_blocks(kc, vc, wl.cow_pairs)
            kc, vc = orc.reshape_and_cache(kc, vc, wl.new_key, wl.new_value, wl.slot_mapping)
            orc.decode(wl.q, kc, vc, wl.block_tables, wl.seq_lens, wl.scale, threads=n_threads)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget or reps >= 200:
                return el / reps, reps, el

    per, reps, el = run(threads, budget_s)
    out = {"value": round(wl.kv_bytes() / per / 1e9, 3), "unit": "GB/s", "cores": threads,
           "kind": "oracle", "seconds_per_step": round(per, 4), "cpu_model": _cpu_model(),
           "sample": f"the full step (cache write + fp64 decode of all {wl.B} sequences) "
                     f"repeated {reps}x, {el:.1f} s"}
    if one_thread:
        per1, reps1, el1 = run(1, budget_s / 2)
        out["one_thread"] = {"value": round(wl.kv_bytes() / per1 / 1e9, 4), "unit": "GB/s",
                             "seconds_per_step": round(per1, 4),
                             "sample": f"the same step on 1 thread, repeated {reps1}x, {el1:.1f} s"}
        orc.decode(wl.q[:1], wl.k_cache, wl.v_cache, wl.block_tables[:1], wl.seq_lens[:1], wl.scale,
                   threads=threads)   # OpenMP keeps the last thread count: restore it
    return out


def _cpu_timed(run, budget_s):
    """Repeat the oracle call `run` for about budget_s seconds (at least once); returns
    (seconds per call, repetitions, elapsed, threads)."""
    from oracle import oracle as orc
    reps, t0 = 0, time.perf_counter()
    while True:
        run()
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 200:
            break
    return el / reps, reps, el, orc.max_threads()


def _copy_calibration(torch, pa, dev, launches=5):
    """pa_copy_blocks of 2048 distinct blocks onto 2048 others, K and V, bf16, Hkv=8,
    bs=16, D=128 (32 KiB per block and cache): 128 MiB read and 128 MiB written per launch."""
    nb, npairs = 4096, 2048
    k = torch.zeros((nb, 8, 16, 128), dtype=torch.bfloat16, device=dev)
    v = torch.zeros_like(k)
    pairs = torch.stack([torch.arange(npairs), torch.arange(npairs) + npairs], 1).to(torch.int32).to(dev)
    for _ in range(launches):
        pa.pa_copy_blocks(k, v, pairs)
    torch.cuda.synchronize()
    per = 2 * npairs * 8 * 16 * 128 * 2
    print(json.dumps({"calibration": "pa_copy_blocks", "launches": launches,
                      "bytes_read_per_launch": per, "bytes_written_per_launch": per}), flush=True)


def _read_calibration(torch, pa, W, dev, launches=5):
    """pa_read_tiles over the Llama-3-8B batch's tile list: non-temporal 16-byte loads, as
    the decode kernel issues them, of a known number of bytes (every K and V tile of the
    batch once), the reference for scaling rocprofv3 FETCH_SIZE of the decode kernel."""
    wl = W.config(2, poison=False)
    k, v = _to_dev(wl.k_cache, torch, dev), _to_dev(wl.v_cache, torch, dev)
    offs = torch.from_numpy(W.group_tile_offsets(wl.block_tables, wl.seq_lens, wl.Hkv, wl.D, 2,
                                                 wl.block_size)).to(dev)
    sink = torch.zeros(pa.READ_SINK_LEN, dtype=torch.int32, device=dev)
    for _ in range(launches):
        pa.pa_read_tiles(k, v, offs, 16 * wl.D * 2, sink)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "pa_read_tiles (non-temporal)", "launches": launches,
                      "bytes_read_per_launch": int(offs.numel()) * 16 * wl.D * 2 * 2,
                      "bytes_written_per_launch": 4 * pa.READ_SINK_LEN}), flush=True)


def _sweep_block_size(torch, pa, W, dev, args):
    """The same 64 sequences (lengths of the Llama-3-8B batch) stored in blocks of
    8, 16, 32, 64 and 128 tokens, with the physical blocks permuted at random or laid out
    in order; each point times pa_decode alone (HIP events around each call, two replicas
    rotated) and prints one JSON line."""
    L = W.config(2, poison=False).seq_lens
    steps = max(20, min(args.steps, 100))
    for bs in (8, 16, 32, 64, 128):
        for placement in ("permute", "identity"):
            wl = W.make_workload(f"llama3-8b-bs{bs}", 64, 32, 8, 128, bs, L, W.BF16, 29802,
                                 max_blocks=4096 // bs, poison=False, placement=placement)
            ws_bytes = pa.pa_decode_workspace_bytes(wl.B, wl.Hq, wl.Hkv, wl.D, bs,
                                                    wl.max_blocks, pa.PA_BF16)
            reps = [dict(q=_to_dev(wl.q, torch, dev), k=_to_dev(wl.k_cache, torch, dev),
                         v=_to_dev(wl.v_cache, torch, dev), bt=_to_dev(wl.block_tables, torch, dev),
                         sl=_to_dev(wl.seq_lens, torch, dev),
                         out=torch.empty((wl.B, wl.Hq, wl.D), dtype=torch.float32, device=dev))
                    for _ in range(2)]
            ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
            stream = torch.cuda.current_stream(dev)
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(steps)]
            for i in range(10 + steps):
                r = reps[i % 2]
                if i >= 10:
                    ev[i - 10][0].record(stream)
                pa.pa_decode(r["out"], r["q"], r["k"], r["v"], r["bt"], r["sl"], wl.scale,
                             workspace=ws, stream=stream)
                if i >= 10:
                    ev[i - 10][1].record(stream)
            torch.cuda.synchronize()
            us = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
            print(json.dumps({"sweep": "block_size", "block_size": bs, "placement": placement,
                              "decode_us_mean": round(float(us.mean()), 2),
                              "decode_us_p50": round(float(np.median(us)), 2),
                              "kv_bytes": wl.kv_bytes(),
                              "GBps": round(wl.kv_bytes() / (us.mean() * 1e-6) / 1e9, 1),
                              "table_entries": int(sum((x + bs - 1) // bs for x in L))}), flush=True)
            del reps, ws
            torch.cuda.empty_cache()


def _sweep_group_size(torch, pa, W, dev, args):
    """The same 64 sequences (lengths of the Llama-3-8B batch, Hkv = 8, D = 128, bs = 16, the
    same K/V bytes) with G = Hq / Hkv = 1, 2, 4 and 8 query heads per KV head; pa_decode
    alone, HIP events around each call, two replicas rotated. One JSON line per G."""
    L = W.config(2, poison=False).seq_lens
    steps = max(100, min(args.steps, 300))
    for G in (1, 2, 4, 8):
        wl = W.make_workload(f"llama3-8b-G{G}", 64, 8 * G, 8, 128, 16, L, W.BF16, 29802,
                             max_blocks=256, poison=False)
        ws_bytes = pa.pa_decode_workspace_bytes(wl.B, wl.Hq, wl.Hkv, wl.D, 16, wl.max_blocks, pa.PA_BF16)
        reps = [dict(q=_to_dev(wl.q, torch, dev), k=_to_dev(wl.k_cache, torch, dev),
                     v=_to_dev(wl.v_cache, torch, dev), bt=_to_dev(wl.block_tables, torch, dev),
                     sl=_to_dev(wl.seq_lens, torch, dev),
                     out=torch.empty((wl.B, wl.Hq, wl.D), dtype=torch.float32, device=dev),
                     ws=torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device=dev))
                for _ in range(2)]
        stream = torch.cuda.current_stream(dev)
        t = _per_call_us(torch, lambda r: pa.pa_decode(r["out"], r["q"], r["k"], r["v"], r["bt"], r["sl"],
                                                       wl.scale, workspace=r["ws"], stream=stream),
                         reps, steps, 30, stream)
        kv = wl.kv_bytes()
        print(json.dumps({"sweep": "group_size", "G": G, "Hq": wl.Hq, "Hkv": wl.Hkv, "kv_bytes": kv,
                          "decode_us": t, "GBps": round(kv / (t["mean"] * 1e-6) / 1e9, 1),
                          "frac": round(kv / (t["mean"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}), flush=True)
        del reps
        torch.cuda.empty_cache()


def _per_call_us(torch, fn, reps, steps, warmup, stream):
    """Mean, p10, p50 and p90 of fn's duration in us: HIP events around each call on its
    stream, rotating over the replicas."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for i in range(warmup):
        fn(reps[i % len(reps)])
    torch.cuda.synchronize()
    for i in range(steps):
        ev[i][0].record(stream)
        fn(reps[i % len(reps)])
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
    return {"mean": round(float(us.mean()), 2), "p10": round(float(np.percentile(us, 10)), 2),
            "p50": round(float(np.median(us)), 2), "p90": round(float(np.percentile(us, 90)), 2)}


def _shared_prefix(torch, pa, W, dev, args):
    """The shared-prefix batch (16 prompts of 2048 tokens, 8 candidates each): the step
    copy_blocks + reshape_and_cache + pa_decode_shared, and the decode alone through
    pa_decode_shared and through pa_decode; one JSON line. Logical bytes count every
    sequence's tokens; unique bytes count each shared block once."""
    wl = W.config(3, poison=False)
    groups = wl.share_groups
    max_members, max_shared = int(groups[:, 1].max()), int(groups[:, 2].max())
    shared_of = np.zeros(wl.B, np.int64)
    for first, members, sh in groups:
        shared_of[first:first + members] = sh
    row = wl.Hkv * wl.D * 2 * 2
    unique = (int(groups[:, 2].astype(np.int64).sum()) + int((wl.seq_lens - shared_of).sum())) * row
    logical = wl.kv_bytes()
    per_replica = 2 * wl.k_cache.nbytes + wl.q.nbytes + wl.block_tables.nbytes
    R = args.replicas or max(2, math.ceil((1 << 30) / per_replica))
    ws_sh = pa.pa_decode_shared_workspace_bytes(wl.B, wl.Hq, wl.D, wl.block_size, wl.max_blocks,
                                                max_shared)
    ws_pl = pa.pa_decode_workspace_bytes(wl.B, wl.Hq, wl.Hkv, wl.D, wl.block_size, wl.max_blocks,
                                         pa.PA_BF16)
    _log(f"{wl.name}: B={wl.B} logical={logical} unique={unique} replicas={R}")
    reps = [dict(q=_to_dev(wl.q, torch, dev), k=_to_dev(wl.k_cache, torch, dev),
                 v=_to_dev(wl.v_cache, torch, dev), bt=_to_dev(wl.block_tables, torch, dev),
                 sl=_to_dev(wl.seq_lens, torch, dev), nk=_to_dev(wl.new_key, torch, dev),
                 nv=_to_dev(wl.new_value, torch, dev), slots=_to_dev(wl.slot_mapping, torch, dev),
                 pairs=_to_dev(wl.cow_pairs, torch, dev), groups=_to_dev(groups, torch, dev),
                 out=torch.empty((wl.B, wl.Hq, wl.D), dtype=torch.float32, device=dev),
                 ws_sh=torch.zeros(max(ws_sh, 1), dtype=torch.uint8, device=dev),
                 ws_pl=torch.zeros(max(ws_pl, 1), dtype=torch.uint8, device=dev))
            for _ in range(R)]
    stream = torch.cuda.current_stream(dev)

    def shared(r):
        pa.pa_decode_shared(r["out"], r["q"], r["k"], r["v"], r["bt"], r["sl"], r["groups"],
                            max_members, max_shared, wl.scale, workspace=r["ws_sh"], stream=stream)

    def plain(r):
        pa.pa_decode(r["out"], r["q"], r["k"], r["v"], r["bt"], r["sl"], wl.scale,
                     workspace=r["ws_pl"], stream=stream)

    def step(r):
        pa.pa_copy_blocks(r["k"], r["v"], r["pairs"], stream=stream)
        pa.pa_reshape_and_cache(r["k"], r["v"], r["nk"], r["nv"], r["slots"], stream=stream)
        shared(r)

    steps = max(20, min(args.steps, 200))
    st = _per_call_us(torch, step, reps, steps, args.warmup, stream)
    sh = _per_call_us(torch, shared, reps, steps, args.warmup, stream)
    pl = _per_call_us(torch, plain, reps, steps, args.warmup, stream)
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import oracle as orc
        kc, vc = orc.copy_blocks(wl.k_cache, wl.v_cache, wl.cow_pairs)
        kc, vc = orc.reshape_and_cache(kc, vc, wl.new_key, wl.new_value, wl.slot_mapping)
        per, n, el, thr = _cpu_timed(lambda: orc.decode(wl.q, kc, vc, wl.block_tables, wl.seq_lens,
                                                        wl.scale), args.cpu_seconds)
        cpu = {"value": round(logical / per / 1e9, 3), "unit": "GB/s (logical KV)", "cores": thr,
               "kind": "oracle", "seconds_per_call": round(per, 4),
               "sample": f"fp64 decode of all {wl.B} sequences (every sequence reads its own "
                         f"copy of the prompt), repeated {n}x, {el:.1f} s"}
    unique_gbs = unique / (sh["mean"] * 1e-6) / 1e9
    print(json.dumps({
        "bench": "shared_prefix", "workload": W.CONFIG_NAMES[3], "replicas_rotated": R,
        "groups": int(len(groups)), "members": max_members, "shared_tokens": max_shared,
        "logical_kv_bytes": logical, "unique_kv_bytes": unique,
        "step_us": st, "decode_shared_us": sh, "decode_us": pl,
        "shared_logical_GBps": round(logical / (sh["mean"] * 1e-6) / 1e9, 1),
        "shared_unique_GBps": round(unique / (sh["mean"] * 1e-6) / 1e9, 1),
        "plain_logical_GBps": round(logical / (pl["mean"] * 1e-6) / 1e9, 1),
        "speedup_vs_pa_decode": round(pl["mean"] / sh["mean"], 3),
        "roofline": {"bound": "hbm", "kernel": "pa_decode_shared (one launch + merge)",
                     "achieved": round(unique_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(unique_gbs / HBM_PEAK_GBS, 4),
                     "bytes": "unique KV bytes (each shared block once)"},
        "cpu_baseline": cpu}), flush=True)


MFMA_BF16_PEAK_TFLOPS = 2500.0


def _multi_query(torch, pa, W, dev, args):
    """pa_decode_multi on two batches; one JSON line each.

    draft: the Llama-3-8B batch's 64 lengths (at least 4) with the last 4 tokens of each
    sequence as queries (speculative decoding's check of 4 draft tokens). HBM-bound: the
    KV bytes are those of a decode step.
    chunks: 4 sequences whose newest 1024 tokens are a prompt chunk, after 0, 1024, 2048
    and 3072 cached tokens (chunked prefill). Matrix-core bound: 4 D flops per (query
    head, visible token), bf16 MFMA peak 2.5 PFLOP/s.
    Each is the cache write of the chunk followed by pa_decode_multi, timed with HIP events
    around each pa_decode_multi call, rotating enough replicas to exceed 1 GiB.
    """
    rng = np.random.default_rng(29802)
    L2 = np.maximum(rng.integers(1, 4097, size=64).astype(np.int32), 4)
    cases = [
        ("draft-4-llama3-8b", W.make_workload("draft", 64, 32, 8, 128, 16, L2, W.BF16, 29802,
                                             max_blocks=256, poison=False, n_new=[4] * 64)),
        ("chunk-1024x4-llama3-8b", W.make_workload("chunks", 4, 32, 8, 128, 16,
                                                   [1024, 2048, 3072, 4096], W.BF16, 29806,
                                                   max_blocks=256, poison=False,
                                                   n_new=[1024] * 4)),
    ]
    steps = max(20, min(args.steps, 200))
    for name, wl in cases:
        qs = wl.q_starts
        n = np.diff(qs)
        max_q, total_q = int(n.max()), int(qs[-1])
        kv = wl.kv_bytes()
        vis = sum(int(L - k + j + 1) for L, k in zip(wl.seq_lens, n) for j in range(int(k)))
        flops = 4.0 * wl.D * wl.Hq * vis
        ws_bytes = pa.pa_decode_multi_workspace_bytes(wl.B, total_q, max_q, wl.Hq, wl.Hkv, wl.D,
                                                      wl.block_size, wl.max_blocks)
        per_replica = 2 * wl.k_cache.nbytes + wl.q.nbytes
        R = args.replicas or max(2, math.ceil((1 << 30) / per_replica))
        reps = [dict(q=_to_dev(wl.q, torch, dev), k=_to_dev(wl.k_cache, torch, dev),
                     v=_to_dev(wl.v_cache, torch, dev), bt=_to_dev(wl.block_tables, torch, dev),
                     sl=_to_dev(wl.seq_lens, torch, dev), qs=_to_dev(qs, torch, dev),
                     nk=_to_dev(wl.new_key, torch, dev), nv=_to_dev(wl.new_value, torch, dev),
                     slots=_to_dev(wl.slot_mapping, torch, dev),
                     out=torch.empty((total_q, wl.Hq, wl.D), dtype=torch.float32, device=dev),
                     ws=torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device=dev))
                for _ in range(R)]
        stream = torch.cuda.current_stream(dev)
        for r in reps:
            pa.pa_reshape_and_cache(r["k"], r["v"], r["nk"], r["nv"], r["slots"], stream=stream)

        def multi(r):
            pa.pa_decode_multi(r["out"], r["q"], r["k"], r["v"], r["bt"], r["sl"], r["qs"], max_q,
                               wl.scale, workspace=r["ws"], stream=stream)

        t = _per_call_us(torch, multi, reps, steps, args.warmup, stream)
        sec = t["mean"] * 1e-6
        hbm_bound = max_q * wl.G <= 16            # one query tile per (sequence, KV head)
        if hbm_bound:
            roof = {"bound": "hbm", "achieved": round(kv / sec / 1e9, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(kv / sec / 1e9 / HBM_PEAK_GBS, 4)}
        else:
            roof = {"bound": "mfma", "achieved": round(flops / sec / 1e12, 1),
                    "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(flops / sec / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
        roof["kernel"] = "pa_decode_multi"
        cpu = None
        if not args.no_cpu_baseline:
            from oracle import oracle as orc
            kc, vc = orc.reshape_and_cache(wl.k_cache, wl.v_cache, wl.new_key, wl.new_value,
                                           wl.slot_mapping)
            per, nrep, el, thr = _cpu_timed(lambda: orc.decode_multi(
                wl.q, kc, vc, wl.block_tables, wl.seq_lens, qs, wl.scale), args.cpu_seconds)
            cpu = {"value": round(kv / per / 1e9, 3) if hbm_bound else round(flops / per / 1e12, 4),
                   "unit": "GB/s" if hbm_bound else "TFLOP/s", "cores": thr, "kind": "oracle",
                   "seconds_per_call": round(per, 3),
                   "sample": f"fp64 causal multi-query attention of all {total_q} queries, "
                             f"repeated {nrep}x, {el:.1f} s"}
        line = {"bench": "multi_query", "workload": name, "B": wl.B, "queries": total_q,
                "max_q": max_q, "Hq": wl.Hq, "Hkv": wl.Hkv, "D": wl.D, "block_size": wl.block_size,
                "seq_lens": [int(x) for x in wl.seq_lens] if wl.B <= 8 else "llama3-8b batch",
                "replicas_rotated": R, "decode_multi_us": t, "kv_bytes": kv,
                "kv_GBps": round(kv / sec / 1e9, 1), "kv_frac_of_hbm": round(kv / sec / 1e9 / HBM_PEAK_GBS, 4),
                "flops": flops, "TFLOPs": round(flops / sec / 1e12, 1),
                "mfma_frac": round(flops / sec / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                "roofline": roof, "cpu_baseline": cpu}
        print(json.dumps(line), flush=True)
        del reps
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2, help="workload 1-5 (2 = the headline)")
    ap.add_argument("--replicas", type=int, default=0, help="0 = enough to exceed 1 GiB")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep-block-size", action="store_true",
                    help="pa_decode on the Llama-3-8B-shaped batch for block sizes 8..128, "
                         "permuted vs in-order block placement; one JSON line per point")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run pa_copy_blocks over a known number of bytes (the reference "
                         "for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE) and print them")
    ap.add_argument("--sweep-group-size", action="store_true",
                    help="pa_decode on the Llama-3-8B lengths with G = 1, 2, 4, 8 query heads per "
                         "KV head (same K/V bytes); one JSON line per G")
    ap.add_argument("--read-calibration", action="store_true",
                    help="only run pa_read_tiles (non-temporal loads) over the Llama-3-8B "
                         "batch's tiles, a known number of bytes, and print them")
    ap.add_argument("--shared-prefix", action="store_true",
                    help="the shared-prefix batch through pa_decode_shared and pa_decode; "
                         "one JSON line")
    ap.add_argument("--multi-query", action="store_true",
                    help="pa_decode_multi on draft tokens (Llama-3-8B batch) and on prompt "
                         "chunks; one JSON line each")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the decode path "
              "shards by sequence or KV head with no exchange; only N=1 is built)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from paged_kv_cache_298_amd import pa
    from paged_kv_cache_298_amd import workloads as W

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        _copy_calibration(torch, pa, dev)
        return
    if args.sweep_group_size:
        _sweep_group_size(torch, pa, W, dev, args)
        return
    if args.read_calibration:
        _read_calibration(torch, pa, W, dev)
        return
    if args.sweep_block_size:
        _sweep_block_size(torch, pa, W, dev, args)
        return
    if args.shared_prefix:
        _shared_prefix(torch, pa, W, dev, args)
        return
    if args.multi_query:
        _multi_query(torch, pa, W, dev, args)
        return
    _log(f"generating workload {args.config}")
    wl = W.config(args.config, poison=False)
    kv_bytes = wl.kv_bytes()
    per_replica = 2 * wl.k_cache.nbytes + wl.q.nbytes + wl.block_tables.nbytes
    R = args.replicas or max(2, math.ceil((1 << 30) / per_replica))
    _log(f"{wl.name}: B={wl.B} kv_bytes={kv_bytes} pool={wl.num_blocks} blocks, replicas={R}")

    reps = []
    ws_bytes = pa.pa_decode_workspace_bytes(wl.B, wl.Hq, wl.Hkv, wl.D, wl.block_size, wl.max_blocks,
                                            pa.PA_BF16 if wl.dtype == "bf16" else pa.PA_F32)
    for _ in range(R):
        reps.append(dict(
            q=_to_dev(wl.q, torch, dev), k=_to_dev(wl.k_cache, torch, dev),
            v=_to_dev(wl.v_cache, torch, dev), bt=_to_dev(wl.block_tables, torch, dev),
            sl=_to_dev(wl.seq_lens, torch, dev), nk=_to_dev(wl.new_key, torch, dev),
            nv=_to_dev(wl.new_value, torch, dev), slots=_to_dev(wl.slot_mapping, torch, dev),
            pairs=_to_dev(wl.cow_pairs, torch, dev) if wl.cow_pairs.shape[0] else None,
            out=torch.empty((wl.B, wl.Hq, wl.D), dtype=torch.float32, device=dev),
            ws=torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device=dev)))
    stream = torch.cuda.current_stream(dev)

    def step(r):
        # one decode step: the clones (when the batch has copy-on-write pairs), then the
        # newest tokens' cache write and the decode in one launch
        if r["pairs"] is not None:
            pa.pa_copy_blocks(r["k"], r["v"], r["pairs"], stream=stream)
        pa.pa_decode_append(r["out"], r["q"], r["k"], r["v"], r["nk"], r["nv"], r["slots"], r["bt"],
                            r["sl"], wl.scale, workspace=r["ws"], stream=stream)

    def step_two_launches(r):
        if r["pairs"] is not None:
            pa.pa_copy_blocks(r["k"], r["v"], r["pairs"], stream=stream)
        pa.pa_reshape_and_cache(r["k"], r["v"], r["nk"], r["nv"], r["slots"], stream=stream)
        pa.pa_decode(r["out"], r["q"], r["k"], r["v"], r["bt"], r["sl"], wl.scale,
                     workspace=r["ws"], stream=stream)

    def decode_only(r):
        pa.pa_decode(r["out"], r["q"], r["k"], r["v"], r["bt"], r["sl"], wl.scale,
                     workspace=r["ws"], stream=stream)

    # ---- whole step
    for i in range(args.warmup):
        step(reps[i % R])
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(reps[i % R])
    ev1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - w0) * 1e3 / args.steps
    ms_step = ev0.elapsed_time(ev1) / args.steps
    _log(f"step: {ms_step * 1e3:.1f} us (events), {wall_ms * 1e3:.1f} us (wall)")
    # the same step as separate launches (pa_reshape_and_cache, then pa_decode), for context
    for i in range(args.warmup):
        step_two_launches(reps[i % R])
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(args.steps):
        step_two_launches(reps[i % R])
    ev1.record(stream)
    torch.cuda.synchronize()
    us_two = ev0.elapsed_time(ev1) / args.steps * 1e3
    _log(f"step as separate cache-write and decode launches: {us_two:.1f} us")

    # ---- pa_decode alone: events around every call, on its stream; at least 200 calls
    # after at least 30 warm-up calls, so the mean and percentiles are stable
    n_dec, w_dec = max(args.steps, 200), max(args.warmup, 30)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n_dec)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n_dec)]
    for i in range(w_dec):
        decode_only(reps[i % R])
    torch.cuda.synchronize()
    for i in range(n_dec):
        starts[i].record(stream)
        decode_only(reps[i % R])
        ends[i].record(stream)
    torch.cuda.synchronize()
    dec_us = np.array([s.elapsed_time(e) * 1e3 for s, e in zip(starts, ends)])
    dec_mean = float(dec_us.mean())
    _log(f"pa_decode: mean {dec_mean:.1f} us, p10 {np.percentile(dec_us, 10):.1f}, "
         f"p50 {np.median(dec_us):.1f}, p90 {np.percentile(dec_us, 90):.1f}")

    # ---- hot (one replica, Infinity Cache may help) for context
    for i in range(args.warmup):
        decode_only(reps[0])
    torch.cuda.synchronize()
    n_hot = 50
    for i in range(n_hot):
        starts[i].record(stream)
        decode_only(reps[0])
        ends[i].record(stream)
    torch.cuda.synchronize()
    hot_us = float(np.mean([starts[i].elapsed_time(ends[i]) * 1e3 for i in range(n_hot)]))

    # ---- the read ceiling of this access pattern: the same 16-token group tiles, in the
    # decode kernel's order and slices, read with no arithmetic (pa_read_tiles)
    read = None
    if wl.block_size >= 16:
        elt = 2 if wl.dtype == "bf16" else 4
        offs = torch.from_numpy(W.group_tile_offsets(wl.block_tables, wl.seq_lens, wl.Hkv, wl.D,
                                                     elt, wl.block_size)).to(dev)
        sink = torch.zeros(pa.READ_SINK_LEN, dtype=torch.int32, device=dev)
        tile = 16 * wl.D * elt
        rd = _per_call_us(torch, lambda r: pa.pa_read_tiles(r["k"], r["v"], offs, tile, sink,
                                                           stream=stream),
                          reps, n_dec, w_dec, stream)
        read = {"kernel": "pa_read_tiles: the decode kernel's tiles, order and slices, no arithmetic",
                "us_mean": rd["mean"], "us_p50": rd["p50"],
                "GBps": round(kv_bytes / (rd["mean"] * 1e-6) / 1e9, 2),
                "decode_frac_of_read": round(rd["mean"] / dec_mean, 4)}
        _log(f"read ceiling: mean {rd['mean']:.1f} us ({read['GBps']:.0f} GB/s of KV); "
             f"pa_decode at {read['decode_frac_of_read']:.3f} of it")

    achieved = kv_bytes / (dec_mean * 1e-6) / 1e9
    value = kv_bytes / (ms_step * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        _log("cpu baseline (oracle)")
        cpu = _cpu_baseline(wl, args.cpu_seconds, one_thread=args.config in (1, 2))

    traffic = _traffic_for(wl.name)
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "us_per_step": round(ms_step * 1e3, 2),
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": W.CONFIG_NAMES[args.config], "global_batch": wl.B,
                   "kv_bytes_per_step": kv_bytes, "replicas_rotated": R,
                   "step": "copy_blocks (if CoW pairs) + pa_decode_append (cache write + decode, one launch)",
                   "us_per_step_separate_launches": round(us_two, 2)},
        "roofline": {"bound": "hbm", "kernel": "pa_decode (decode kernel + split-row merge)",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "decode_us_mean": round(dec_mean, 2),
                     "decode_us_p10": round(float(np.percentile(dec_us, 10)), 2),
                     "decode_us_p50": round(float(np.median(dec_us)), 2),
                     "decode_us_p90": round(float(np.percentile(dec_us, 90)), 2),
                     "decode_us_hot_one_replica": round(hot_us, 2), "decode_calls_timed": n_dec,
                     "read_ceiling": read},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
