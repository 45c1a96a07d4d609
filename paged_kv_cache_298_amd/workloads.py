"""Seeded synthetic workloads for paged decode attention (numpy only).

This module only draws inputs: sequence lengths, a physical placement of blocks, q and
the per-sequence K/V rows in logical order, and stores them in the paged pool layout
[num_blocks, Hkv, block_size, D]. It computes no attention and is shared, as plain input
data, by the GPU tests, the benchmark and the oracle checks.

Recipe (all draws from numpy's PCG64 ``default_rng(seed)``, in this order): sequence
lengths, placement permutation, q, K per sequence in logical order, V per sequence in
logical order, then any extra masks. Normal draws are float32 and, for bf16 workloads,
are rounded to bf16 by round-to-nearest-even on the float32 bits; the stored bits are the
input both sides read. The newest token of every sequence (position L-1) is not stored in
the pool: it is handed over as ``new_key``/``new_value`` with its ``slot_mapping`` entry,
so one decode step is: clone shared blocks (``cow_pairs``), write the new tokens, attend.

``poison=True`` (parity inputs) fills every slot that holds no valid token, every spare
block and every not-yet-copied clone with NaN, and points block-table entries past a
sequence's last block at a NaN spare block; ``poison=False`` (timing inputs) uses zeros
and block 0.
"""
from dataclasses import dataclass, field
import math

import numpy as np

F32, BF16 = "f32", "bf16"
NAN_BF16 = np.uint16(0x7FC0)
NAN_F32_BITS = np.uint32(0x7FC00000)


def bf16_from_f32(x):
    """Round float32 values to bf16 (round to nearest, ties to even); returns uint16 bits.
    Inputs must be finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store_dtype(dtype):
    return np.uint16 if dtype == BF16 else np.float32


def _draw(rng, shape, dtype):
    x = rng.standard_normal(shape, dtype=np.float32)
    return bf16_from_f32(x) if dtype == BF16 else x


def _fill_value(dtype, poison):
    if not poison:
        return np.uint16(0) if dtype == BF16 else np.float32(0.0)
    return NAN_BF16 if dtype == BF16 else NAN_F32_BITS.view(np.float32)


@dataclass
class Workload:
    name: str
    dtype: str
    B: int
    Hq: int
    Hkv: int
    D: int
    block_size: int
    num_blocks: int
    max_blocks: int
    scale: float
    q: np.ndarray                  # [B, Hq, D]
    k_cache: np.ndarray            # [num_blocks, Hkv, block_size, D] (newest tokens absent)
    v_cache: np.ndarray
    block_tables: np.ndarray       # int32 [B, max_blocks]
    seq_lens: np.ndarray           # int32 [B] (including the newest token)
    new_key: np.ndarray            # [B, Hkv, D]: K of each sequence's newest token
    new_value: np.ndarray
    slot_mapping: np.ndarray       # int32 [B]: physical slot of position seq_lens[b] - 1
    cow_pairs: np.ndarray          # int32 [N, 2] (src, dst) blocks to clone before writing
    logical_k: list = field(default_factory=list)   # per sequence [L, Hkv, D], if kept
    logical_v: list = field(default_factory=list)
    # int32 [n_groups, 3] (first sequence, members, tokens whose table entries all members
    # share), for workloads built with shared prompts; empty otherwise
    share_groups: np.ndarray = field(default_factory=lambda: np.zeros((0, 3), np.int32))
    # int32 [B + 1] query offsets of a multi-query workload (None: one query per sequence)
    q_starts: np.ndarray = None

    @property
    def G(self):
        return self.Hq // self.Hkv

    def kv_bytes(self):
        """Bytes of valid K and V the decode step must read: sum_b L_b * Hkv * D * 2 * elt."""
        elt = 2 if self.dtype == BF16 else 4
        return int(np.sum(self.seq_lens, dtype=np.int64)) * self.Hkv * self.D * 2 * elt


def _scatter_sequence(pool, table, rows, bs, skip_last):
    """Store rows [L, Hkv, D] (logical order) into the blocks table[0:n]; the last
    int(skip_last) rows are left out (the newest tokens, written by the step itself)."""
    L = rows.shape[0]
    if L == 0:
        return
    n = (L + bs - 1) // bs
    stored = L - int(skip_last)
    for j in range(n):
        lo, hi = j * bs, min((j + 1) * bs, stored)
        if hi <= lo:
            continue
        # rows [lo, hi) of the sequence go to slots [0, hi-lo) of block table[j]
        pool[table[j], :, 0:hi - lo, :] = rows[lo:hi].transpose(1, 0, 2)


def make_workload(name, B, Hq, Hkv, D, block_size, seq_lens, dtype, seed, *,
                  max_blocks=None, pool_factor=1.25, num_blocks=None, placement="permute",
                  poison=True, keep_logical=False, k_row_scale_mask=None, rng=None,
                  scale=None, n_new=None):
    """General builder. seq_lens are given (already drawn); the placement permutation, q,
    K and V are then drawn from rng (or default_rng(seed)) in that order.

    n_new (multi-query workloads): per sequence, how many of its newest tokens are queries
    at once (0 <= n_new[b] <= seq_lens[b]). Those tokens are left out of the cache and
    handed to the step as new_key / new_value [sum n_new, Hkv, D] with their slots; q is
    then [sum n_new, Hq, D] in position order and q_starts [B + 1] its offsets. Without
    it, each sequence has one query and one new token (the decode step)."""
    rng = np.random.default_rng(seed) if rng is None else rng
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    bs = int(block_size)
    nblk = (seq_lens.astype(np.int64) + bs - 1) // bs
    total = int(nblk.sum())
    if max_blocks is None:
        max_blocks = max(1, int(nblk.max()) if B else 1)
    if num_blocks is None:
        num_blocks = max(total + 1, int(math.ceil(pool_factor * total)))
    # the permutation is always drawn, so that q/K/V do not depend on the placement
    perm = rng.permutation(num_blocks).astype(np.int32)
    if placement == "identity":
        perm = np.arange(num_blocks, dtype=np.int32)
    elif placement == "reversed":
        perm = np.arange(num_blocks - 1, -1, -1, dtype=np.int32)
    elif placement != "permute":
        raise ValueError(placement)
    spare = int(perm[total]) if total < num_blocks else 0
    fill_entry = spare if poison else 0
    tables = np.full((B, max_blocks), fill_entry, dtype=np.int32)
    cursor = 0
    for b in range(B):
        tables[b, :nblk[b]] = perm[cursor:cursor + nblk[b]]
        cursor += int(nblk[b])
    sdt = _store_dtype(dtype)
    if n_new is not None:
        n_new = np.asarray(n_new, dtype=np.int32)
        if n_new.shape != (B,) or np.any(n_new < 0) or np.any(n_new > seq_lens):
            raise ValueError("n_new must give 0 <= n_new[b] <= seq_lens[b] per sequence")
        q_starts = np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32)
        q = _draw(rng, (int(q_starts[-1]), Hq, D), dtype)
    else:
        q_starts = None
        q = _draw(rng, (B, Hq, D), dtype)
    ks = [_draw(rng, (int(L), Hkv, D), dtype) for L in seq_lens]
    vs = [_draw(rng, (int(L), Hkv, D), dtype) for L in seq_lens]
    if k_row_scale_mask is not None:
        # extra draw, last: per (sequence, token) Bernoulli mask; those K rows are scaled
        # (all KV heads) after rounding; k_row_scale_mask = (probability, factor)
        prob, factor = k_row_scale_mask
        for b in range(B):
            m = rng.random(int(seq_lens[b])) < prob
            if dtype == BF16:
                kf = bf16_to_f32(ks[b][m]) * np.float32(factor)
                ks[b][m] = bf16_from_f32(kf)
            else:
                ks[b][m] = ks[b][m] * np.float32(factor)
    fill = _fill_value(dtype, poison)
    k_cache = np.full((num_blocks, Hkv, bs, D), fill, dtype=sdt)
    v_cache = np.full((num_blocks, Hkv, bs, D), fill, dtype=sdt)
    if n_new is None:
        new_key = np.zeros((B, Hkv, D), dtype=sdt)
        new_value = np.zeros((B, Hkv, D), dtype=sdt)
        slots = np.full((B,), -1, dtype=np.int32)
        for b in range(B):
            L = int(seq_lens[b])
            _scatter_sequence(k_cache, tables[b], ks[b], bs, skip_last=True)
            _scatter_sequence(v_cache, tables[b], vs[b], bs, skip_last=True)
            if L > 0:
                new_key[b] = ks[b][L - 1]
                new_value[b] = vs[b][L - 1]
                slots[b] = tables[b, (L - 1) // bs] * bs + (L - 1) % bs
    else:
        T = int(q_starts[-1])
        new_key = np.zeros((T, Hkv, D), dtype=sdt)
        new_value = np.zeros((T, Hkv, D), dtype=sdt)
        slots = np.full((T,), -1, dtype=np.int32)
        for b in range(B):
            L, n = int(seq_lens[b]), int(n_new[b])
            _scatter_sequence(k_cache, tables[b], ks[b], bs, skip_last=n)
            _scatter_sequence(v_cache, tables[b], vs[b], bs, skip_last=n)
            for j in range(n):
                pos, i = L - n + j, int(q_starts[b]) + j
                new_key[i] = ks[b][pos]
                new_value[i] = vs[b][pos]
                slots[i] = tables[b, pos // bs] * bs + pos % bs
    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(D)))
    return Workload(name=name, dtype=dtype, B=B, Hq=Hq, Hkv=Hkv, D=D, block_size=bs,
                    num_blocks=num_blocks, max_blocks=max_blocks, scale=scale, q=q,
                    k_cache=k_cache, v_cache=v_cache, block_tables=tables, seq_lens=seq_lens,
                    new_key=new_key, new_value=new_value, slot_mapping=slots,
                    cow_pairs=np.zeros((0, 2), dtype=np.int32),
                    logical_k=ks if keep_logical else [], logical_v=vs if keep_logical else [],
                    q_starts=q_starts)


def make_shared_prefix(name, n_prompts, n_cand, prompt_len, div_max, Hq, Hkv, D, block_size,
                       dtype, seed, *, poison=True, keep_logical=False, pool_factor=1.25,
                       clone_last_prompt_block=True):
    """Parallel sampling: n_prompts prompts of prompt_len tokens, each forked into n_cand
    candidates that share the prompt's blocks and add 1..div_max tokens of their own.

    When clone_last_prompt_block, every candidate but the last of each prompt gets a
    private clone of the prompt's last block (the copy-on-write of diverging forks): its
    table points at the clone, the clone holds nothing until the step copies it, and the
    (original, clone) pair is listed in cow_pairs. prompt_len must then be a multiple of
    the block size, so that no candidate token lives in the cloned block (a prompt that
    ends inside a block is built through the block manager's append path instead).
    """
    rng = np.random.default_rng(seed)
    bs = int(block_size)
    if clone_last_prompt_block and prompt_len % bs != 0:
        raise NotImplementedError("clone of a partly filled prompt block: use the append path")
    B = n_prompts * n_cand
    d = rng.integers(1, div_max + 1, size=B).astype(np.int32)          # seq_lens draw
    seq_lens = (prompt_len + d).astype(np.int32)
    p_blocks = (prompt_len + bs - 1) // bs
    # blocks holding only the candidate's own tokens, after the shared prompt blocks
    own = ((seq_lens.astype(np.int64) + bs - 1) // bs) - p_blocks
    n_clones = n_prompts * (n_cand - 1) if clone_last_prompt_block else 0
    needed = n_prompts * p_blocks + int(own.sum()) + n_clones
    num_blocks = int(math.ceil(pool_factor * needed)) + 1
    perm = rng.permutation(num_blocks).astype(np.int32)              # placement draw
    max_blocks = int(((seq_lens.astype(np.int64) + bs - 1) // bs).max())
    cursor = 0
    prompt_tables = []
    for p in range(n_prompts):
        prompt_tables.append(perm[cursor:cursor + p_blocks].copy())
        cursor += p_blocks
    tables = np.zeros((B, max_blocks), dtype=np.int32)
    pairs = []
    for p in range(n_prompts):
        for c in range(n_cand):
            b = p * n_cand + c
            t = list(prompt_tables[p])
            if clone_last_prompt_block and c < n_cand - 1:
                clone = int(perm[cursor]); cursor += 1
                pairs.append((int(t[-1]), clone))
                t[-1] = clone
            t.extend(int(x) for x in perm[cursor:cursor + own[b]])
            cursor += int(own[b])
            tables[b, :len(t)] = t
    spare = int(perm[cursor]) if cursor < num_blocks else 0
    for b in range(B):
        n_b = (int(seq_lens[b]) + bs - 1) // bs
        tables[b, n_b:] = spare if poison else 0
    sdt = _store_dtype(dtype)
    q = _draw(rng, (B, Hq, D), dtype)
    kp = [_draw(rng, (prompt_len, Hkv, D), dtype) for _ in range(n_prompts)]
    kd = [_draw(rng, (int(x), Hkv, D), dtype) for x in d]
    vp = [_draw(rng, (prompt_len, Hkv, D), dtype) for _ in range(n_prompts)]
    vd = [_draw(rng, (int(x), Hkv, D), dtype) for x in d]
    fill = _fill_value(dtype, poison)
    k_cache = np.full((num_blocks, Hkv, bs, D), fill, dtype=sdt)
    v_cache = np.full((num_blocks, Hkv, bs, D), fill, dtype=sdt)
    for p in range(n_prompts):
        _scatter_sequence(k_cache, prompt_tables[p], kp[p], bs, skip_last=False)
        _scatter_sequence(v_cache, prompt_tables[p], vp[p], bs, skip_last=False)
    new_key = np.zeros((B, Hkv, D), dtype=sdt)
    new_value = np.zeros((B, Hkv, D), dtype=sdt)
    slots = np.zeros((B,), dtype=np.int32)
    logical_k, logical_v = [], []
    for p in range(n_prompts):
        for c in range(n_cand):
            b = p * n_cand + c
            L = int(seq_lens[b])
            # the candidate's own tokens start at position prompt_len
            for t in range(prompt_len, L - 1):
                blk = tables[b, t // bs]
                k_cache[blk, :, t % bs, :] = kd[b][t - prompt_len]
                v_cache[blk, :, t % bs, :] = vd[b][t - prompt_len]
            new_key[b] = kd[b][-1]
            new_value[b] = vd[b][-1]
            slots[b] = tables[b, (L - 1) // bs] * bs + (L - 1) % bs
            if keep_logical:
                logical_k.append(np.concatenate([kp[p], kd[b]], axis=0))
                logical_v.append(np.concatenate([vp[p], vd[b]], axis=0))
    scale = float(np.float32(1.0 / math.sqrt(D)))
    # the cloned last prompt block is no longer a shared table entry
    shared_tokens = (p_blocks - 1) * bs if clone_last_prompt_block and n_cand > 1 else prompt_len
    return Workload(name=name, dtype=dtype, B=B, Hq=Hq, Hkv=Hkv, D=D, block_size=bs,
                    num_blocks=num_blocks, max_blocks=max_blocks, scale=scale, q=q,
                    k_cache=k_cache, v_cache=v_cache, block_tables=tables, seq_lens=seq_lens,
                    new_key=new_key, new_value=new_value, slot_mapping=slots,
                    cow_pairs=np.asarray(pairs, dtype=np.int32).reshape(-1, 2),
                    logical_k=logical_k, logical_v=logical_v,
                    share_groups=np.asarray([(p * n_cand, n_cand, shared_tokens)
                                             for p in range(n_prompts)], np.int32).reshape(-1, 3))


CONFIG_NAMES = {
    1: "tiny-fp32: B=4, L={1,7,16,33}, Hq=Hkv=2, D=64, bs=16, 64-block pool",
    2: "llama3-8b-layer-bf16: B=64, Hq=32, Hkv=8, D=128, bs=16, L~U[1,4096]",
    3: "shared-prefix-bf16: 16 prompts x 2048 tokens x 8 candidates (+1..256), Hq=32, Hkv=8, D=128, bs=16",
    4: "llama3-70b-layer-bf16: B=32, Hq=64, Hkv=8, D=128, bs=32, L log-uniform [128,8192]",
    5: "long-context-bf16: B=4, L={32768,65536,100000,131072}, Hq=32, Hkv=8, D=128, bs=64",
}


def config(n, poison=True, keep_logical=False):
    """The five named workloads (seed 29800 + n)."""
    seed = 29800 + n
    if n == 1:
        # fixed lengths; 64-block pool, placement is a permutation of all 64 blocks
        return make_workload("cfg1", 4, 2, 2, 64, 16, [1, 7, 16, 33], F32, seed,
                             max_blocks=3, num_blocks=64, poison=poison,
                             keep_logical=keep_logical)
    if n == 2:
        rng = np.random.default_rng(seed)
        L = rng.integers(1, 4097, size=64).astype(np.int32)
        return make_workload("cfg2", 64, 32, 8, 128, 16, L, BF16, seed, max_blocks=256,
                             poison=poison, keep_logical=keep_logical, rng=rng)
    if n == 3:
        return make_shared_prefix("cfg3", 16, 8, 2048, 256, 32, 8, 128, 16, BF16, seed,
                                  poison=poison, keep_logical=keep_logical)
    if n == 4:
        rng = np.random.default_rng(seed)
        u = rng.uniform(math.log(128), math.log(8192), size=32)
        L = np.clip(np.floor(np.exp(u)), 128, 8192).astype(np.int32)
        return make_workload("cfg4", 32, 64, 8, 128, 32, L, BF16, seed, max_blocks=256,
                             poison=poison, keep_logical=keep_logical, rng=rng)
    if n == 5:
        rng = np.random.default_rng(seed)
        L = np.array([32768, 65536, 100000, 131072], dtype=np.int32)
        return make_workload("cfg5", 4, 32, 8, 128, 64, L, BF16, seed, max_blocks=2048,
                             poison=poison, keep_logical=keep_logical, rng=rng,
                             k_row_scale_mask=(0.01, 8.0))
    raise ValueError(f"no config {n}")


def kv_bytes_per_token(layers, kv_heads, head_dim, elt_bytes):
    """Bytes of K plus V per token: 2 (K and V) x elt_bytes x layers x kv_heads x head_dim."""
    return 2 * elt_bytes * layers * kv_heads * head_dim


def group_tile_offsets(block_tables, seq_lens, Hkv, D, elt_bytes, block_size):
    """Byte offsets (int64, into either cache) of every 16-token group tile that the stream
    decode kernel reads, in its order: sequences, then KV heads, then groups. A tile is
    16 rows of D elements of one KV head inside one block (block_size >= 16)."""
    assert block_size >= 16 and block_size % 16 == 0
    row = D * elt_bytes
    tile = block_size * row                 # one (block, KV head) tile
    blk = Hkv * tile                        # one physical block
    out = []
    for b, L in enumerate(np.asarray(seq_lens)):
        n = (int(L) + 15) // 16
        if n == 0:
            continue
        j = np.arange(n, dtype=np.int64)
        phys = np.asarray(block_tables[b], dtype=np.int64)[(j * 16) // block_size]
        base = phys * blk + ((j * 16) % block_size) * row
        for g in range(Hkv):
            out.append(base + g * tile)
    return np.concatenate(out) if out else np.zeros(0, dtype=np.int64)
