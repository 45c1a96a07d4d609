"""Host model of the stream decomposition's bookkeeping (CPU only).

The bf16 decode kernel lays the (sequence, KV head) rows, cut into 16-token groups, end to
end and gives each of nwe waves the slice [w*T//nwe, (w+1)*T//nwe) of the T groups. A wave
writes the output of every row it covers whole, and a partial record for a row it covers
only in part (slot 0 for its first row segment, slot 1 for its last); the merge kernel
looks at the row holding the first group of slice w and merges it when the row began in
slice w - 1. This model walks the same index arithmetic in Python and checks that every
group is consumed once, every row's output is produced exactly once, and every record the
merge reads was written by the wave and slot it names and lies inside the record buffer.
"""
import numpy as np
import pytest


def _schedule(lens, Hkv, nw, min_slice):
    n = [(L + 15) // 16 for L in lens]
    C = np.concatenate([[0], np.cumsum(n)]).astype(np.int64)
    T = int(C[-1]) * Hkv
    nwe = 0 if T == 0 else min(nw, max(1, T // min_slice))
    produced = {}          # (b, g) -> how many times the output row was written
    records = {}           # rec index -> (b, g)
    consumed = np.zeros(T, dtype=np.int64)
    desc = {}

    def locate(s):
        b = int(np.searchsorted(C[1:] * Hkv, s, side="right"))
        off = s - int(C[b]) * Hkv
        g, j = divmod(off, n[b])
        return b, g, j

    for b, L in enumerate(lens):
        if L == 0:
            for g in range(Hkv):
                produced[(b, g)] = produced.get((b, g), 0) + 1
    for w in range(nwe):
        s0, s1 = w * T // nwe, (w + 1) * T // nwe
        assert s1 > s0
        b, g, j = locate(s0)
        desc[w] = (b, g, s0 - j, n[b])
        first, seg_j0 = True, j
        for t in range(s1 - s0):
            s = s0 + t
            assert locate(s) == (b, g, j)
            consumed[s] += 1
            if j == n[b] - 1 or t == s1 - s0 - 1:
                if seg_j0 == 0 and j == n[b] - 1:
                    produced[(b, g)] = produced.get((b, g), 0) + 1
                else:
                    rec = 2 * w + (0 if first else 1)
                    assert rec not in records
                    records[rec] = (b, g)
                if t < s1 - s0 - 1:
                    g += 1
                    if g == Hkv:
                        g = 0
                        b += 1
                        while n[b] == 0:
                            b += 1
                    j, seg_j0, first = 0, 0, False
            else:
                j += 1
    # the merge
    for w in range(1, nwe):
        b, g, start, rn = desc[w]
        s0w = w * T // nwe
        s0p = (w - 1) * T // nwe
        if start >= s0w or start < s0p:
            continue
        last = start + rn - 1
        wb = ((last + 1) * nwe - 1) // T
        assert wb * T // nwe <= last < (wb + 1) * T // nwe
        recs = [2 * (w - 1) + (0 if start == s0p else 1)] + [2 * x for x in range(w, wb + 1)]
        for rec in recs:
            assert records.get(rec) == (b, g), (rec, records.get(rec), (b, g))
            assert rec < 2 * nw
        produced[(b, g)] = produced.get((b, g), 0) + 1
    return T, nwe, consumed, produced


@pytest.mark.parametrize("seed", range(12))
def test_every_row_once_every_group_once(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 40))
    Hkv = int(rng.choice([1, 2, 8]))
    kind = seed % 4
    if kind == 0:
        lens = rng.integers(0, 600, size=B)
    elif kind == 1:
        lens = rng.integers(0, 3, size=B)            # empty and one-group rows
    elif kind == 2:
        lens = rng.integers(2000, 5000, size=B)      # long rows: slices span many windows
    else:
        lens = np.where(rng.random(B) < 0.5, 0, rng.integers(1, 300, size=B))
    lens = [int(x) for x in lens]
    nw = int(rng.choice([4, 8, 64, 2048]))
    min_slice = int(rng.choice([1, 8]))
    T, nwe, consumed, produced = _schedule(lens, Hkv, nw, min_slice)
    assert np.all(consumed == 1)
    assert set(produced) == {(b, g) for b in range(B) for g in range(Hkv)}
    assert all(v == 1 for v in produced.values())


def test_llama3_batch_shape():
    # the Llama-3-8B batch: 64 sequences, 8 KV heads, lengths up to 4096, 2048 waves
    rng = np.random.default_rng(29802)
    lens = [int(x) for x in rng.integers(1, 4097, size=64)]
    T, nwe, consumed, produced = _schedule(lens, 8, 2048, 8)
    assert nwe == 2048 and np.all(consumed == 1)
    assert all(v == 1 for v in produced.values()) and len(produced) == 64 * 8


def test_all_empty_and_fewer_groups_than_waves():
    T, nwe, consumed, produced = _schedule([0, 0, 0], 2, 64, 8)
    assert T == 0 and nwe == 0 and len(produced) == 6
    T, nwe, consumed, produced = _schedule([1, 0, 17], 2, 64, 1)
    assert T == 6 and nwe == 6 and np.all(consumed == 1)
    assert all(v == 1 for v in produced.values())


# ------------------------------------------------------------------ the merge's arithmetic
#
# The merge kernel folds a split row's records (m_i, l_i, o_i): m_i is the segment's
# reference in log2 units, l_i its sum and o_i its unnormalised output. Narrow rows deal
# the records to four waves in contiguous runs, each folded with a running reference in
# batches, then combine the four states in wave order; wide rows let one wave fold every
# record. A multi-query column may see no token of a segment (m_i = -inf, l_i = 0,
# o_i = 0); the row's first record always has a finite reference. This models that
# arithmetic in float32 and compares it with the plain merge in float64.

def _fold(ms, ls, os_, batch, D):
    M, l, o = np.float32(-np.inf), np.float32(0), np.zeros(D, dtype=np.float32)
    for x0 in range(0, len(ms), batch):
        mb = ms[x0:x0 + batch]
        Mb = np.float32(max([M] + list(mb)))
        Mr = np.float32(0) if Mb == -np.inf else Mb       # the kernel's guard
        a = np.exp2(np.float32(M - Mr))
        o, l = o * a, l * a
        for k in range(x0, min(x0 + batch, len(ms))):
            wgt = np.exp2(np.float32(ms[k] - Mr))
            o = o + wgt * os_[k]
            l = l + wgt * ls[k]
        M = Mb
    return M, l, o


def _merge_four_runs(ms, ls, os_, batch):
    nrec = len(ms)
    per = (nrec + 3) // 4
    runs = [(min(nrec, q * per), min(nrec, min(nrec, q * per) + per)) for q in range(4)]
    covered = [x for a, b in runs for x in range(a, b)]
    assert covered == list(range(nrec))                   # contiguous runs, in order
    st = [_fold(ms[a:b], ls[a:b], os_[a:b], batch, len(os_[0])) for a, b in runs]
    Mx = np.float32(max(s[0] for s in st))
    acc = np.zeros_like(os_[0], dtype=np.float32)
    lsum = np.float32(0)
    for M, l, o in st:
        wgt = np.exp2(np.float32(M - Mx))
        acc, lsum = acc + wgt * o, lsum + wgt * l
    return acc / lsum


def _plain_merge(ms, ls, os_):
    m = np.array(ms, dtype=np.float64)
    M = m[np.isfinite(m)].max()
    w = np.where(np.isfinite(m), np.exp2(np.where(np.isfinite(m), m, 0) - M), 0.0)
    return (w[:, None] * np.asarray(os_, np.float64)).sum(0) / (w * np.asarray(ls, np.float64)).sum()


@pytest.mark.parametrize("seed", range(10))
def test_merge_runs_match_plain_merge(seed):
    rng = np.random.default_rng(100 + seed)
    nrec = int(rng.integers(2, 60))
    D = 8
    ms = list(rng.normal(0, 6, size=nrec).astype(np.float32))
    ls = list(rng.uniform(1, 16, size=nrec).astype(np.float32))
    os_ = [rng.normal(0, 1, size=D).astype(np.float32) * l for l in ls]
    # a column that sees no token of some later segments (never of the first)
    for x in rng.choice(np.arange(1, nrec), size=int(rng.integers(0, nrec)), replace=False):
        ms[x], ls[x], os_[x] = np.float32(-np.inf), np.float32(0), np.zeros(D, np.float32)
    ref = _plain_merge(ms, ls, os_)
    for batch in (4, 8, 16):
        got = _merge_four_runs(ms, ls, os_, batch)             # narrow rows
        assert np.all(np.isfinite(got)) and np.max(np.abs(got - ref)) < 1e-4
        M, l, o = _fold(ms, ls, os_, batch, D)                 # wide rows: one fold
        assert np.max(np.abs(o / l - ref)) < 1e-4


def test_merge_guard_is_needed_for_an_all_empty_run():
    # records 4..7 see no token: with 8 records the fourth wave's run holds only those
    ms = [np.float32(1.0)] * 4 + [np.float32(-np.inf)] * 4
    ls = [np.float32(1.0)] * 4 + [np.float32(0.0)] * 4
    os_ = [np.ones(4, np.float32)] * 4 + [np.zeros(4, np.float32)] * 4
    assert np.allclose(_merge_four_runs(ms, ls, os_, 8), 1.0)
    with np.errstate(invalid="ignore"):
        M = np.float32(-np.inf)
        assert np.isnan(np.exp2(np.float32(M - M)))           # what the guard avoids
