"""Reference KV block pool: the oracle of the host allocator that builds block tables.

TEST INFRASTRUCTURE ONLY. Only tests/, the smoke check and the benchmark's CPU baseline
use it; the product allocator (C++, pa_alloc_*) is checked against it operation by
operation.

What the pages fix about the pool ([P2] "Paged Attention", infra.pidoku.co.in, section 4
"Tiny example" and section 5 "Copy-on-write sharing"; [P4] "PagedAttention & KV-Cache
Management in High-Throughput LLM Serving", subroutine-cs.cc, section 3), stated as the
behaviour this module implements:
  (a) free physical ids are handed out last in, first out; a fresh pool of N ids holds
      id 0 on top and id N-1 at the bottom;
  (b) a request for n ids is met whole or not at all; it receives the n topmost ids,
      listed from the deepest of them up to the top one, and each starts with one holder;
  (c) giving ids back lowers each one's holder count; an id with no holder left goes back
      on top of the free ids, in the order the ids were given;
  (d) sharing a table with a new sequence adds one holder to each of its ids, and the new
      table lists the same ids;
  (e) token pos of a sequence lives in slot table[pos // bs] * bs + pos % bs.

Readings taken where the pages leave a step open:
  * the pages disagree on which free id comes first: the [P2] listing takes the top of a
    stack, the [P4] Python manager pops the front of a list; (a)-(b) follow [P2];
  * giving back an id more often than it is held is an error, and an error leaves the
    pool unchanged;
  * writing a token (copy-on-write, [P2] section 5: a shared block is copied before it is
    written): a token that starts a new logical block gets a fresh id; a token that falls
    into a block other sequences still hold gets a fresh private id in that place, the
    shared id loses this sequence as a holder, and when the block already holds tokens of
    this sequence the copy (shared -> fresh) is reported; a request that cannot be met
    leaves the sequence and the pool unchanged.
"""
from collections import Counter


class OutOfBlocks(Exception):
    pass


class Pool:
    """Holder count per physical id (0 = free) and the free ids, bottom of the stack
    first."""

    def __init__(self, num_blocks, block_size, free_order=None):
        self.block_size = int(block_size)
        self.holders = [0] * int(num_blocks)
        if free_order is None:
            self.stack = [int(num_blocks) - 1 - i for i in range(int(num_blocks))]
        else:
            self.stack = [int(b) for b in free_order]
            if sorted(self.stack) != list(range(int(num_blocks))):
                raise ValueError("free_order must list every block id once")

    def count_for(self, tokens):
        """Blocks that hold `tokens` tokens."""
        return -(-int(tokens) // self.block_size)

    def take(self, n):
        n = int(n)
        if n < 0:
            raise ValueError("negative block count")
        if n > len(self.stack):
            raise OutOfBlocks(f"out of KV blocks: need {n}, have {len(self.stack)}")
        top_first = [self.stack.pop() for _ in range(n)]
        for b in top_first:
            self.holders[b] = 1
        return top_first[::-1]

    def give_back(self, ids):
        for b, k in Counter(ids).items():
            if not 0 <= b < len(self.holders) or self.holders[b] < k:
                raise ValueError(f"block {b} given back more often than it is held")
        for b in ids:
            self.holders[b] -= 1
            if self.holders[b] == 0:
                self.stack.append(b)

    def share(self, ids):
        if any(not 0 <= b < len(self.holders) or self.holders[b] == 0 for b in ids):
            raise ValueError("sharing a block that is not allocated")
        for b in ids:
            self.holders[b] += 1
        return list(ids)

    def holders_of(self, b):
        return self.holders[b]

    def in_use(self):
        return sum(1 for h in self.holders if h > 0)


class SeqTable:
    """One sequence: its table of physical ids and its length in tokens."""

    def __init__(self, pool, tokens=0, table=None):
        self.pool = pool
        self.table = pool.take(pool.count_for(tokens)) if table is None else list(table)
        self.length = int(tokens)

    def slot(self, pos):
        bs = self.pool.block_size
        return self.table[pos // bs] * bs + pos % bs

    def branch(self):
        """A second sequence holding the same blocks (parallel sampling, beams)."""
        return SeqTable(self.pool, self.length, self.pool.share(self.table))

    def add_token(self):
        """Write one more token. Returns (slot, copy), copy = (shared id, fresh id) or
        None."""
        pool, bs = self.pool, self.pool.block_size
        blk, off = divmod(self.length, bs)
        if blk > len(self.table):
            raise ValueError("block table shorter than the sequence")
        copy = None
        if blk == len(self.table):
            self.table.append(pool.take(1)[0])
        elif pool.holders_of(self.table[blk]) > 1:
            shared = self.table[blk]
            fresh = pool.take(1)[0]
            pool.holders[shared] -= 1
            self.table[blk] = fresh
            if off:
                copy = (shared, fresh)
        self.length += 1
        return self.slot(self.length - 1), copy
