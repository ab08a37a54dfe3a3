"""Plain model of the host block manager (test infrastructure, like the rest
of oracle/: only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
use it).

Follows the allocator sketches on the pages: a free list of physical blocks,
a block table per sequence and a reference count per block (第三讲
"核心数据结构：Block Table": a sequence gets ceil(tokens / block_size) blocks
or the request fails; Continuous Batching §3.2: fork shares the parent's
blocks and raises their counts, free lowers them and returns a block whose
count reaches zero; vLLM notes "Sharing KV Cache" and 第三讲 "共享前缀": a
sequence that appends into a block another sequence still references first
gets a fresh block holding a copy -- copy-on-write).

Policy details the pages leave open, fixed here (and in the C++ manager):
  - free blocks are handed out lowest id first;
  - appending when the last block is full (or the sequence has no block)
    takes a fresh block; appending into a partially filled block whose count
    exceeds one copies it (the pair (old, new) is reported for copy_blocks)
    and lowers the old block's count;
  - a failed call changes nothing (a batch append stops at the first
    sequence that cannot get a block; the ones before it are done).
"""
import bisect


class BlockManagerError(Exception):
    def __init__(self, kind):
        super().__init__(kind)
        self.kind = kind            # "no_blocks" | "sequence" | "value"


class BlockManagerRef:
    def __init__(self, num_blocks, block_size):
        if num_blocks < 1 or block_size < 1:
            raise BlockManagerError("value")
        self.bs = block_size
        self.nb = num_blocks
        self.free = list(range(num_blocks))          # sorted ascending
        self.ref = {}
        self.seqs = {}                               # id -> [blocks, tokens]

    # -- helpers -----------------------------------------------------------
    def _take(self):
        return self.free.pop(0)

    def _release(self, b):
        self.ref[b] -= 1
        if self.ref[b] == 0:
            del self.ref[b]
            bisect.insort(self.free, b)

    # -- operations ----------------------------------------------------------
    def add_sequence(self, sid, num_tokens):
        if sid in self.seqs or num_tokens < 0:
            raise BlockManagerError("sequence" if sid in self.seqs else "value")
        need = -(-num_tokens // self.bs)
        if need > len(self.free):
            raise BlockManagerError("no_blocks")
        blocks = [self._take() for _ in range(need)]
        for b in blocks:
            self.ref[b] = 1
        self.seqs[sid] = [blocks, num_tokens]

    def fork(self, parent, child):
        if parent not in self.seqs or child in self.seqs:
            raise BlockManagerError("sequence")
        blocks, n = self.seqs[parent]
        for b in blocks:
            self.ref[b] += 1
        self.seqs[child] = [list(blocks), n]

    def free_sequence(self, sid):
        if sid not in self.seqs:
            raise BlockManagerError("sequence")
        blocks, _ = self.seqs.pop(sid)
        for b in blocks:
            self._release(b)

    def append(self, sid):
        """One new token: returns (slot, (src, dst) or None)."""
        if sid not in self.seqs:
            raise BlockManagerError("sequence")
        blocks, n = self.seqs[sid]
        off = n % self.bs
        if off == 0:                                  # last block full, or none
            if not self.free:
                raise BlockManagerError("no_blocks")
            b = self._take()
            self.ref[b] = 1
            blocks.append(b)
            pair = None
        else:
            b = blocks[-1]
            pair = None
            if self.ref[b] > 1:                       # shared: copy on write
                if not self.free:
                    raise BlockManagerError("no_blocks")
                nb_ = self._take()
                self.ref[nb_] = 1
                self.ref[b] -= 1
                blocks[-1] = nb_
                pair = (b, nb_)
                b = nb_
        self.seqs[sid][1] = n + 1
        return b * self.bs + off, pair

    def append_batch(self, sids):
        """Returns (slots, copy pairs, number done); raises after the done ones."""
        slots, pairs = [], []
        for i, sid in enumerate(sids):
            try:
                slot, pair = self.append(sid)
            except BlockManagerError as e:
                e.done, e.slots, e.pairs = i, slots, pairs
                raise
            slots.append(slot)
            if pair:
                pairs.append(pair)
        return slots, pairs, len(sids)

    def table(self, sid):
        if sid not in self.seqs:
            raise BlockManagerError("sequence")
        blocks, n = self.seqs[sid]
        return list(blocks), n

    def token_slots(self, sid, first, count):
        blocks, n = self.table(sid)
        if first < 0 or count < 0 or first + count > n:
            raise BlockManagerError("value")
        return [blocks[t // self.bs] * self.bs + t % self.bs for t in range(first, first + count)]

    def num_free(self):
        return len(self.free)

    def check(self):
        """Internal consistency: every block is free or referenced, counts
        equal the number of tables naming the block."""
        count = {}
        for blocks, n in self.seqs.values():
            assert len(blocks) == -(-n // self.bs)
            for b in blocks:
                count[b] = count.get(b, 0) + 1
        assert count == self.ref
        assert not (set(self.free) & set(self.ref))
        assert len(self.free) + len(self.ref) == self.nb
        assert self.free == sorted(self.free)
