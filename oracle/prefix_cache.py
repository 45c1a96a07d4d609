"""Reference prefix cache: the oracle of the C++ prefix cache (pa_pcache_*).

TEST INFRASTRUCTURE ONLY. A plain-Python statement of [P2] "Paged Attention"
(infra.pidoku.co.in), §5 "The relationship to prefix caching": hash the token ids of each
block, keep a map to block ids, and let a new sequence whose leading blocks are cached
point at them with one more reference. It runs on the reference block manager
(oracle/block_manager.py) and is checked against the product operation by operation.

Readings (the page gives three sentences): a block is identified by its tokens and all
tokens before it, so the map key here is exact -- (parent entry, the block's tokens) --
with no hashing at all; only full blocks are cached; the cache holds its own reference on
each cached block; when a new sequence needs more free blocks than exist, cached blocks no
sequence holds are released least recently used first; an acquire that cannot be met
changes nothing. "Use" is a counter stamped on every hit and every publish.
"""
from oracle.block_manager import OutOfBlocks


class PrefixCacheRef:
    def __init__(self, mgr):
        self.mgr = mgr
        self.bs = mgr.block_size
        self.entries = {}        # (parent id, tokens tuple) -> id
        self.info = {}           # id -> [block, stamp, key]
        self.next_id = 1
        self.clock = 0

    def _touch(self, eid):
        self.clock += 1
        self.info[eid][1] = self.clock

    def _evictable(self, exclude=()):
        return [e for e, (blk, _, _) in self.info.items()
                if self.mgr.holders_of(blk) == 1 and e not in exclude]

    def _evict(self, n, exclude=()):
        done = 0
        for e in sorted(self._evictable(exclude), key=lambda e: self.info[e][1]):
            if done == n:
                break
            blk, _, key = self.info.pop(e)
            del self.entries[key]
            self.mgr.give_back([blk])
            done += 1
        return done

    def acquire(self, tokens):
        bs = self.bs
        tokens = [int(t) for t in tokens]
        total = (len(tokens) + bs - 1) // bs
        hits, parent = [], 0
        for i in range(len(tokens) // bs):
            e = self.entries.get((parent, tuple(tokens[i * bs:(i + 1) * bs])))
            if e is None:
                break
            hits.append(e)
            parent = e
        need = total - len(hits)
        spare = len(self.mgr.stack)
        if spare < need and spare + len(self._evictable(exclude=set(hits))) < need:
            raise OutOfBlocks(f"out of KV blocks: need {need}")
        table = self.mgr.share([self.info[e][0] for e in hits])
        if spare < need:
            self._evict(need - spare, exclude=set(hits))
        table += self.mgr.take(need)
        for e in hits:
            self._touch(e)
        return table, len(hits) * bs

    def publish(self, tokens, table):
        bs = self.bs
        tokens = [int(t) for t in tokens]
        full = len(tokens) // bs
        if full > len(table) or any(self.mgr.holders_of(b) < 1 for b in table[:full]):
            raise ValueError("publish: table does not hold the tokens")
        parent = 0
        for i in range(full):
            key = (parent, tuple(tokens[i * bs:(i + 1) * bs]))
            e = self.entries.get(key)
            if e is None:
                e = self.next_id
                self.next_id += 1
                self.mgr.share([table[i]])
                self.entries[key] = e
                self.info[e] = [table[i], 0, key]
            self._touch(e)
            parent = e

    def evict(self, n):
        return self._evict(n)

    def num_entries(self):
        return len(self.info)
