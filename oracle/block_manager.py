"""Reference block manager: the host-side allocator that builds block tables.

TEST INFRASTRUCTURE ONLY (the oracle of the allocator): an independent, plain-Python
statement of the block manager on [P2] "Paged Attention" (infra.pidoku.co.in, §4 "Tiny
example"), extended with the copy-on-write append rule that page and [P4] "PagedAttention
& KV-Cache Management in High-Throughput LLM Serving" (subroutine-cs.cc, §3) describe in
prose. The product allocator (C++) is checked against it operation by operation.

Readings taken where the pages leave a step open:
  * free list order: a stack whose top is the end of the list, initially N-1 ... 0, and an
    allocation of n takes the top n in list order ([P2] §4); the Python manager on [P4] §4
    pops from the front instead, so the two pages' orders differ.
  * freeing a block whose count is already zero is an error (the page's map would silently
    go negative); an error leaves the state unchanged.
  * append with copy-on-write: position pos = current length; if it starts a new logical
    block a fresh block is appended; if it falls inside a block that other sequences also
    reference, that block is replaced by a fresh one, and a copy (old -> new) is emitted
    when the block already holds tokens of this sequence; a failed allocation leaves the
    sequence unchanged (the page's code bumps the length first).
"""


class OutOfBlocks(Exception):
    pass


class BlockManager:
    def __init__(self, num_blocks, block_size, initial_free=None):
        self.block_size = int(block_size)
        self.num_blocks = int(num_blocks)
        if initial_free is None:
            self.free = list(range(self.num_blocks - 1, -1, -1))
        else:
            self.free = [int(b) for b in initial_free]
        self.refcount = {}

    def blocks_needed(self, tokens):
        return (int(tokens) + self.block_size - 1) // self.block_size

    def allocate(self, n):
        n = int(n)
        if n < 0:
            raise ValueError("negative block count")
        if len(self.free) < n:
            raise OutOfBlocks(f"out of KV blocks: need {n}, have {len(self.free)}")
        cut = len(self.free) - n
        taken = self.free[cut:]
        del self.free[cut:]
        for b in taken:
            self.refcount[b] = 1
        return taken

    def free_blocks(self, blocks):
        need = {}
        for b in blocks:
            need[b] = need.get(b, 0) + 1
        for b, k in need.items():
            if self.refcount.get(b, 0) < k:
                raise ValueError(f"block {b} freed more times than it is referenced")
        for b in blocks:
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                del self.refcount[b]
                self.free.append(b)

    def fork(self, blocks):
        for b in blocks:
            if self.refcount.get(b, 0) <= 0:
                raise ValueError(f"fork of unallocated block {b}")
        for b in blocks:
            self.refcount[b] += 1
        return list(blocks)

    def ref(self, block):
        return self.refcount.get(block, 0)


class Sequence:
    def __init__(self, mgr, prompt_len=0, table=None):
        self.mgr = mgr
        if table is None:
            self.table = mgr.allocate(mgr.blocks_needed(prompt_len))
        else:
            self.table = list(table)
        self.length = int(prompt_len)

    def physical_index(self, pos):
        bs = self.mgr.block_size
        return self.table[pos // bs] * bs + pos % bs

    def fork(self):
        return Sequence(self.mgr, self.length, self.mgr.fork(self.table))

    def append_token(self):
        """Add one token. Returns (slot, cow) where cow is None or (src_block, dst_block)."""
        mgr = self.mgr
        bs = mgr.block_size
        pos = self.length
        j = pos // bs
        cow = None
        if j == len(self.table):
            self.table.append(mgr.allocate(1)[0])
        elif j > len(self.table):
            raise ValueError("block table shorter than the sequence")
        else:
            cur = self.table[j]
            if mgr.ref(cur) > 1:
                new = mgr.allocate(1)[0]
                mgr.refcount[cur] -= 1
                self.table[j] = new
                if pos % bs != 0:
                    cow = (cur, new)
        self.length += 1
        return self.physical_index(pos), cow
