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

Prefix cache (TGI notes §5.2-5.3: a trie from prompt tokens to blocks with a
reference count and last access time per node; lookup of the longest cached
prefix on allocation, insertion of the prompt's blocks when the request is
freed, eviction of unreferenced leaves oldest first; vLLM notes "Prefix
Caching": a request whose leading blocks hold the same tokens as cached ones
points its table at those blocks):
  - one trie node per full block, keyed by that block's token ids;
  - a prompt matches cached blocks from its first block on, only within its
    first n - 1 tokens (its last token is always computed);
  - freeing a sequence added with its tokens enters its full prompt blocks:
    where a node with the same tokens exists it is kept (and touched), else
    the sequence's block becomes a new node;
  - a block is free, referenced, or cached with no reference; new blocks come
    from the free list first, then from evicting the unreferenced leaf with
    the oldest access (ties: lowest block id), repeatedly;
  - access times come from a counter that every successful cached add and
    every free advances.
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
        self.prompt = {}                             # id -> prompt token ids (cached adds)
        self.root = {}                               # token tuple -> node
        self.nodes = {}                              # block -> node (cached blocks)
        self.clock = 0

    # -- helpers -----------------------------------------------------------
    def _leaves(self):
        """Cached blocks that no sequence references and that have no children."""
        return [b for b, nd in self.nodes.items() if b not in self.ref and not nd["children"]]

    def _obtainable(self, pinned=()):
        """Blocks an allocation can get: free ones, plus cached ones whose whole
        subtree is unreferenced (evicting leaves in turn frees all of them)."""
        def clear(nd):
            ok = nd["block"] not in self.ref and nd["block"] not in pinned
            for child in nd["children"].values():
                ok = clear(child) and ok
            count[0] += ok
            return ok
        count = [0]
        for nd in self.root.values():
            clear(nd)
        return len(self.free) + count[0]

    def _take(self):
        if self.free:
            return self.free.pop(0)
        b = min(self._leaves(), key=lambda x: (self.nodes[x]["access"], x))   # LRU leaf
        nd = self.nodes.pop(b)
        siblings = self.root if nd["parent"] is None else nd["parent"]["children"]
        del siblings[nd["key"]]
        return b

    def _release(self, b):
        self.ref[b] -= 1
        if self.ref[b] == 0:
            del self.ref[b]
            if b not in self.nodes:
                bisect.insort(self.free, b)

    # -- operations ----------------------------------------------------------
    def add_sequence(self, sid, num_tokens):
        if sid in self.seqs or num_tokens < 0:
            raise BlockManagerError("sequence" if sid in self.seqs else "value")
        need = -(-num_tokens // self.bs)
        if need > self._obtainable():
            raise BlockManagerError("no_blocks")
        blocks = []
        for _ in range(need):
            b = self._take()
            self.ref[b] = 1
            blocks.append(b)
        self.seqs[sid] = [blocks, num_tokens]

    def add_sequence_cached(self, sid, tokens):
        """A prompt by its token ids: returns the number of leading tokens whose
        blocks came from the cache."""
        tokens = [int(t) for t in tokens]
        n = len(tokens)
        if sid in self.seqs:
            raise BlockManagerError("sequence")
        hits, level = [], self.root
        for j in range(max(n - 1, 0) // self.bs):            # within the first n - 1 tokens
            nd = level.get(tuple(tokens[j * self.bs:(j + 1) * self.bs]))
            if nd is None:
                break
            hits.append(nd["block"])
            level = nd["children"]
        need = -(-n // self.bs) - len(hits)
        if need > self._obtainable(pinned=set(hits)):
            raise BlockManagerError("no_blocks")
        self.clock += 1
        for b in hits:
            self.ref[b] = self.ref.get(b, 0) + 1
            self.nodes[b]["access"] = self.clock
        blocks = list(hits)
        for _ in range(need):
            b = self._take()
            self.ref[b] = 1
            blocks.append(b)
        self.seqs[sid] = [blocks, n]
        self.prompt[sid] = tokens
        return len(hits) * self.bs

    def fork(self, parent, child):
        if parent not in self.seqs or child in self.seqs:
            raise BlockManagerError("sequence")
        blocks, n = self.seqs[parent]
        for b in blocks:
            self.ref[b] += 1
        self.seqs[child] = [list(blocks), n]
        if parent in self.prompt:
            self.prompt[child] = list(self.prompt[parent])

    def free_sequence(self, sid):
        if sid not in self.seqs:
            raise BlockManagerError("sequence")
        self.clock += 1
        blocks, _ = self.seqs.pop(sid)
        tokens = self.prompt.pop(sid, None)
        if tokens:
            level, parent = self.root, None
            for j in range(len(tokens) // self.bs):          # the prompt's full blocks
                key = tuple(tokens[j * self.bs:(j + 1) * self.bs])
                nd = level.get(key)
                if nd is None:
                    nd = {"block": blocks[j], "key": key, "parent": parent, "children": {},
                          "access": 0}
                    level[key] = nd
                    self.nodes[blocks[j]] = nd
                nd["access"] = self.clock
                level, parent = nd["children"], nd
        for b in blocks:
            self._release(b)

    def append(self, sid):
        """One new token: returns (slot, (src, dst) or None)."""
        if sid not in self.seqs:
            raise BlockManagerError("sequence")
        blocks, n = self.seqs[sid]
        off = n % self.bs
        if off == 0:                                  # last block full, or none
            if not self.free and not self._leaves():
                raise BlockManagerError("no_blocks")
            b = self._take()
            self.ref[b] = 1
            blocks.append(b)
            pair = None
        else:
            b = blocks[-1]
            pair = None
            if self.ref[b] > 1:                       # shared: copy on write
                if not self.free and not self._leaves():
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

    def num_cached(self):
        return len(self.nodes)

    def check(self):
        """Internal consistency: every block is free or referenced, counts
        equal the number of tables naming the block."""
        count = {}
        for blocks, n in self.seqs.values():
            assert len(blocks) == -(-n // self.bs)
            for b in blocks:
                count[b] = count.get(b, 0) + 1
        assert count == self.ref
        cached = set(self.nodes)
        assert not (set(self.free) & set(self.ref)) and not (set(self.free) & cached)
        assert len(self.free) + len(set(self.ref) | cached) == self.nb
        assert self.free == sorted(self.free)
        # trie: every node is reachable from the root under its own key, once
        seen = []

        def walk(level, parent):
            for key, nd in level.items():
                assert nd["key"] == key and nd["parent"] is parent and len(key) == self.bs
                assert self.nodes[nd["block"]] is nd
                seen.append(nd["block"])
                walk(nd["children"], nd)
        walk(self.root, None)
        assert sorted(seen) == sorted(cached)
