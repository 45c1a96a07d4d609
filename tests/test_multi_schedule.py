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


# ---------------------------------------------------------------- longest-first order
# The kernel hands query-tile units (sequence, partition, tile) to the waves in decreasing
# work: ntok, the partition's tokens that the tile's last query sees, counted in classes of
# Q tokens; within a class by sequence, partition, then tile from the last. Each block
# derives the order from the lengths (histogram of classes, scan, then rank -> unit). The
# arithmetic below repeats the kernel's, integer for integer.

LPT_BUCKETS = 1024


def _tiles_from(y, base, n, nt, G, rshift):
    d = y - base - 1
    if d < 0:
        return nt
    if n <= d:
        return 0
    return nt + 1 - ((d * G + (1 << rshift)) >> rshift)


def _seqs(lens, n_new, cap, max_q):
    q_starts = np.concatenate([[0], np.cumsum(n_new)]).astype(int)
    total_q = int(q_starts[-1])
    out = []
    for b in range(len(lens)):
        L = min(max(int(lens[b]), 0), cap)
        qs = min(max(int(q_starts[b]), 0), total_q)
        n = min(max(int(q_starts[b + 1]) - qs, 0), L, max_q, total_q - qs)
        out.append((L - n, n))
    return out


def lpt_units(lens, n_new, Hq, Hkv, cap):
    """[(b, part, tile)] in the order the kernel's ranks 0, 1, ... map to."""
    B, G = len(lens), Hq // Hkv
    nset, n_tiles, P, n_parts = plan(B, max(n_new), Hq, Hkv, cap)
    rshift = 4 + {1: 0, 2: 1, 4: 2}[nset]
    qsh = 8
    while (P + (1 << qsh) - 1) >> qsh > LPT_BUCKETS:
        qsh += 1
    K = (P + (1 << qsh) - 1) >> qsh
    seq = _seqs(lens, n_new, cap, max(n_new))

    def class_tiles(k, part, base, n, nt):
        lo = part * P + ((k - 1) << qsh)
        a = _tiles_from(lo + 1, base, n, nt, G, rshift)
        c = _tiles_from(lo + (1 << qsh) + 1, base, n, nt, G, rshift) if k < K else 0
        return a, c

    hist = [0] * K
    NP = B * n_parts
    for pr in range(NP):
        b, part = divmod(pr, n_parts)
        base, n = seq[b]
        L = base + n
        if n <= 0 or part * P >= L:
            continue
        nt = (n * G + 16 * nset - 1) >> rshift
        tf = nt - _tiles_from(part * P + 1, base, n, nt, G, rshift)
        vf = base + (min((tf + 1) << rshift, n * G) - 1) // G + 1
        k_lo = (min(vf, (part + 1) * P) - part * P + (1 << qsh) - 1) >> qsh
        k_hi = (min(L, (part + 1) * P) - part * P + (1 << qsh) - 1) >> qsh
        for k in range(k_lo, k_hi + 1):
            a, c = class_tiles(k, part, base, n, nt)
            if a > c:
                hist[K - k] += a - c
    start = np.concatenate([[0], np.cumsum(hist)[:-1]]).astype(int)
    total = int(start[-1] + hist[-1])
    units = []
    for rank in range(total):
        lo_, hi_ = 0, K - 1
        while lo_ < hi_:
            mid = (lo_ + hi_ + 1) >> 1
            if start[mid] <= rank:
                lo_ = mid
            else:
                hi_ = mid - 1
        k, j = K - lo_, rank - int(start[lo_])
        found = None
        for pr in range(NP):                       # the kernel scans 64 pairs at a time
            b, part = divmod(pr, n_parts)
            base, n = seq[b]
            if n <= 0 or part * P >= base + n:
                continue
            nt = (n * G + 16 * nset - 1) >> rshift
            a, c = class_tiles(k, part, base, n, nt)
            cnt = max(a - c, 0)
            if j < cnt:
                found = (b, part, nt - c - 1 - j)
                break
            j -= cnt
        assert found is not None
        units.append(found)
    return units, (nset, n_tiles, P, n_parts, qsh)


def _grid_units(lens, n_new, Hq, Hkv, cap):
    """The units the grid order runs (M > 0 and a partition start at or before the tile's
    last position), with their ntok."""
    B, G = len(lens), Hq // Hkv
    nset, n_tiles, P, n_parts = plan(B, max(n_new), Hq, Hkv, cap)
    seq = _seqs(lens, n_new, cap, max(n_new))
    out = {}
    for b in range(B):
        base, n = seq[b]
        for part in range(n_parts):
            for tile in range(n_tiles):
                row0 = tile * 16 * nset
                M = min(16 * nset, n * G - row0)
                if M <= 0:
                    continue
                pos_last = base + (row0 + M - 1) // G
                if part * P > pos_last:
                    continue
                out[(b, part, tile)] = min(pos_last + 1, (part + 1) * P) - part * P
    return out


LPT_CASES = [
    ([5, 16, 40], [5, 3, 17], 8, 2, 16),
    ([300, 700], [300, 700], 32, 8, 32),
    ([1500, 2100], [256, 512], 64, 8, 64),
    ([40, 1, 333, 90, 17], [0, 1, 33, 90, 4], 16, 4, 128),
    ([100, 250, 64], [7, 250, 1], 4, 4, 16),
    ([1024, 2048, 3072, 4096], [1024] * 4, 32, 8, 16),        # the prompt-chunk batch
    ([4096, 4064], [4096, 64], 32, 8, 16),                     # a long tile behind a prefill
    ([9000, 300, 5000], [600, 300, 40], 40, 8, 16),             # G = 5
]


@pytest.mark.parametrize("lens, n_new, Hq, Hkv, bs", LPT_CASES)
def test_longest_first_runs_every_unit_once_in_class_order(lens, n_new, Hq, Hkv, bs):
    cap = bs * -(-max(lens) // bs)
    units, (nset, n_tiles, P, n_parts, qsh) = lpt_units(lens, n_new, Hq, Hkv, cap)
    grid = _grid_units(lens, n_new, Hq, Hkv, cap)
    assert len(units) == len(set(units)) and set(units) == set(grid)   # a bijection
    assert len(units) <= len(lens) * n_tiles * n_parts                 # ranks within the grid
    cls = [-(-grid[u] // (1 << qsh)) for u in units]
    assert cls == sorted(cls, reverse=True)                            # longest class first
    for a, c, ka, kc in zip(units, units[1:], cls, cls[1:]):
        if ka == kc:                                                   # then sequence, partition,
            assert (a[0], a[1], -a[2]) < (c[0], c[1], -c[2])           # tile from the last


def _makespan(works, slots=256, fixed=2.0):
    import heapq
    h = [0.0] * slots
    for w in works:
        t = heapq.heappop(h)
        heapq.heappush(h, t + w + fixed)
    return max(h)


def test_longest_first_balances_the_chunk_batch():
    """The prompt-chunk batch (four 1024-token chunks after 0 .. 3072 cached tokens) on 256
    four-wave blocks, each unit's 8 KV heads taking two blocks of equal work: in grid order
    the long chunks' tiles start last and the slowest CU runs about a quarter over the
    average; longest first it runs at the average."""
    lens, n_new, Hq, Hkv, cap = [1024, 2048, 3072, 4096], [1024] * 4, 32, 8, 4096
    grid = _grid_units(lens, n_new, Hq, Hkv, cap)
    units, (nset, n_tiles, P, n_parts, _) = lpt_units(lens, n_new, Hq, Hkv, cap)
    steps = lambda u: -(-grid[u] // 32)                     # 32 tokens per softmax step
    natural = [(b, part, n_tiles - 1 - t) for b in range(4) for part in range(n_parts)
               for t in range(n_tiles)]
    natural = [u for u in natural if u in grid]
    per_block = lambda order: [steps(u) for u in order for _ in range(Hkv // 4)]
    ideal = sum(per_block(units)) / 256 + 2.0
    assert _makespan(per_block(natural)) > 1.2 * ideal
    assert _makespan(per_block(units)) < 1.02 * ideal


def test_longest_first_on_random_batches():
    """Random batches (lengths, chunk sizes, head ratios, block sizes, partitions): the
    longest-first ranks still cover every unit of the grid order exactly once, in class
    order, within the grid's rank range."""
    rng = np.random.default_rng(7301)
    for _ in range(40):
        B = int(rng.integers(1, 9))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.choice([1, 2, 3, 4, 5, 8]))
        bs = int(rng.choice([16, 32, 64, 128]))
        lens = [int(x) for x in rng.integers(0, 3000, size=B)]
        n_new = [int(rng.integers(0, L + 1)) if L > 0 else 0 for L in lens]
        if max(n_new) * G <= 16:           # one score tile per row: the stream path, not tiles
            n_new[0] = min(lens[0], 17) if lens[0] else 0
            if max(n_new) * G <= 16:
                continue
        cap = bs * max(1, -(-max(max(lens), 1) // bs))
        units, (nset, n_tiles, P, n_parts, qsh) = lpt_units(lens, n_new, G * Hkv, Hkv, cap)
        grid = _grid_units(lens, n_new, G * Hkv, Hkv, cap)
        assert len(units) == len(set(units)) and set(units) == set(grid)
        assert len(units) <= B * n_tiles * n_parts
        cls = [-(-grid[u] // (1 << qsh)) for u in units]
        assert cls == sorted(cls, reverse=True)
