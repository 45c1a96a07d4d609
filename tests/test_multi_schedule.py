"""Host model of pa_decode_multi's work split (CPU only).

The launch plan (query tiles of 16 nset rows, token partitions of P tokens) and each
item's index arithmetic are repeated here in Python: for every (sequence, KV head, query
row), the partitions that hold its visible tokens 0 .. p must cover them exactly once,
partition 0 alone must write a row whose tokens fit in it, and otherwise the merge must
find exactly the records that were written. Table rows, cache tiles, q rows, output rows
and record slots the items touch must lie inside their buffers.
"""
import numpy as np
import pytest

MIN_WAVES, MIN_PART = 2048, 256


def plan(B, max_q, Hq, Hkv, cap):
    rows = max_q * (Hq // Hkv)
    nset = 4 if rows > 32 else (2 if rows > 16 else 1)
    n_tiles = max(1, -(-rows // (16 * nset)))
    P = max(16, -(-cap // 16) * 16)
    units = B * Hkv * n_tiles
    while P > MIN_PART and units * (-(-cap // P)) < MIN_WAVES:
        P = max(MIN_PART, (P // 2 + 15) // 16 * 16)
    return nset, n_tiles, P, max(1, -(-cap // P))


def run(lens, n_new, Hq, Hkv, bs, max_blocks):
    B = len(lens)
    cap = bs * max_blocks
    q_starts = np.concatenate([[0], np.cumsum(n_new)])
    total_q, max_q = int(q_starts[-1]), max(n_new)
    nset, n_tiles, P, n_parts = plan(B, max_q, Hq, Hkv, cap)
    G = Hq // Hkv
    covered = {}                 # (qi, h) -> list of token ranges
    direct, records = set(), set()
    for item in range(Hkv * n_tiles * n_parts * B):
        g = item % Hkv
        rest = item // Hkv
        tile = n_tiles - 1 - rest % n_tiles
        rest //= n_tiles
        part = rest % n_parts
        b = rest // n_parts
        assert b < B
        L = min(max(lens[b], 0), cap)
        qs = min(max(int(q_starts[b]), 0), total_q)
        n = min(max(int(q_starts[b + 1]) - qs, 0), L, max_q, total_q - qs)
        row0 = tile * 16 * nset
        M = min(16 * nset, n * G - row0)
        if M <= 0:
            continue
        base = L - n
        pos_last = base + (row0 + M - 1) // G
        t0 = part * P
        if t0 > pos_last:
            continue
        ntok = min(pos_last + 1, t0 + P) - t0
        ng = -(-ntok // 16)
        for gq in range(ng):                      # table entries and tiles the ring reads
            i = min((t0 + gq * 16) >> (bs.bit_length() - 1), max_blocks - 1)
            assert 0 <= i < max_blocks and (t0 + gq * 16) % bs + 16 <= bs
        for qr in range(M):
            row = row0 + qr
            j, hh = divmod(row, G)
            pos = base + j
            grow = (qs + j) * Hq + g * G + hh
            assert 0 <= qs + j < total_q and grow < total_q * Hq
            if pos < t0:
                continue
            covered.setdefault(grow, []).append((t0, min(t0 + ntok, pos + 1)))
            if pos < P:
                assert part == 0
                direct.add(grow)
            else:
                assert part < n_parts
                records.add((grow, part))
    # every row: tokens 0..pos covered exactly once; written directly or fully merged
    for b in range(B):
        L, n = lens[b], n_new[b]
        for j in range(n):
            pos = L - n + j
            for h in range(Hq):
                grow = (int(q_starts[b]) + j) * Hq + h
                rs = sorted(covered[grow])
                assert rs[0][0] == 0 and rs[-1][1] == pos + 1
                assert all(a[1] == c[0] for a, c in zip(rs, rs[1:]))
                np_row = pos // P + 1
                if np_row == 1:
                    assert grow in direct
                else:
                    assert {(grow, k) for k in range(np_row)} <= records
    return nset, n_tiles, P, n_parts


@pytest.mark.parametrize("lens, n_new, Hq, Hkv, bs", [
    ([5, 16, 40], [5, 3, 17], 8, 2, 16),
    ([300, 700], [300, 700], 32, 8, 32),
    ([1500, 2100], [256, 512], 64, 8, 64),
    ([40, 1, 333, 90, 17], [0, 1, 33, 90, 4], 16, 4, 128),
    ([100, 250, 64], [7, 250, 1], 4, 4, 16),
    ([4000, 17, 2500, 999], [4, 4, 4, 4], 32, 8, 16),
])
def test_every_visible_token_once_every_row_written(lens, n_new, Hq, Hkv, bs):
    max_blocks = -(-max(lens) // bs)
    run(lens, n_new, Hq, Hkv, bs, max_blocks)


def test_plans_of_the_benchmark_shapes():
    # four draft tokens on the Llama-3-8B batch: one tile per (sequence, KV head), split
    assert plan(64, 4, 32, 8, 4096) == (1, 1, 1024, 4)
    # whole 1024-token chunks of four sequences: 64 tiles each, no split
    assert plan(4, 1024, 32, 8, 4096) == (4, 64, 4096, 1)
    # a 66-group partition needs two table windows
    assert plan(2, 512, 64, 8, 2112)[2] == 1056
