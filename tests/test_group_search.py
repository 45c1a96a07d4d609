"""Host model of the shared-prefix group search (CPU only).

The decode kernels find the group holding sequence b with a 64-way search over the groups'
first sequences: each of a wavefront's 64 lanes tests one candidate (every stride-th of the
remaining range), a ballot names the last candidate starting at or before b, and the search
continues inside the stride that follows it. This model repeats the same index arithmetic in
Python and checks it against bisection on sorted inputs, and that it stays in range (and
ends) on unsorted ones.
"""
import bisect

import numpy as np
import pytest


def _search(firsts, b):
    lo, n, found, steps = 0, len(firsts), -1, 0
    while n > 0:
        steps += 1
        stride = (n + 63) >> 6
        hits = [lane for lane in range(64) if lane * stride < n and firsts[lo + lane * stride] <= b]
        if not hits:
            break
        found = lo + max(hits) * stride
        if stride == 1:
            break
        end = lo + n
        lo = found + 1
        n = min(stride - 1, end - lo)
    return found, steps


@pytest.mark.parametrize("n", [0, 1, 2, 63, 64, 65, 100, 4095, 4096, 4097, 20000])
def test_matches_bisection(n):
    rng = np.random.default_rng(n)
    firsts = np.sort(rng.choice(max(4 * n, 8), size=n, replace=False)).tolist()
    probes = set(rng.integers(-2, 4 * n + 10, size=200).tolist()) | set(firsts) | {f - 1 for f in firsts}
    for b in probes:
        want = bisect.bisect_right(firsts, b) - 1
        got, steps = _search(firsts, b)
        assert got == want, (n, b)
        assert steps <= (1 if n <= 64 else 2 if n <= 4096 else 3)


def test_unsorted_stays_in_range():
    rng = np.random.default_rng(7)
    for n in (5, 64, 300, 5000):
        firsts = rng.integers(0, 100, size=n).tolist()
        for b in range(-1, 101, 7):
            got, steps = _search(firsts, b)
            assert -1 <= got < n and steps <= 3


def test_workload_share_groups_meet_the_preconditions():
    """The groups the shared-prompt generator reports: sorted, disjoint, and every member's
    table entries over the shared tokens equal the first member's."""
    from paged_kv_cache_298_amd import workloads as W
    for wl in (W.config(3, poison=False),
               W.make_shared_prefix("g", 3, 4, 512, 40, 32, 8, 128, 16, W.BF16, seed=2),
               W.make_shared_prefix("g", 2, 3, 384, 20, 16, 4, 64, 32, W.BF16, seed=4)):
        g = wl.share_groups
        assert g.shape[1] == 3 and len(g) > 0
        assert np.all(np.diff(g[:, 0]) >= g[:-1, 1])
        for first, members, shared in g:
            nb = shared // wl.block_size
            assert shared % wl.block_size == 0 and nb > 0
            for b in range(first, first + members):
                assert wl.seq_lens[b] >= shared
                assert np.array_equal(wl.block_tables[b, :nb], wl.block_tables[first, :nb])
            # the next block is private to each member (the copy-on-write clone)
            if members > 1:
                assert len({int(wl.block_tables[b, nb]) for b in range(first, first + members)}) == members
