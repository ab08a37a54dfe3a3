"""Oracle results for a few sequences of a large workload.

TEST INFRASTRUCTURE ONLY (tests/, smoke(), bench.py's cpu_baseline leg).

A full-size pool can be many GB; the oracle only needs the physical blocks
that the chosen sequences use.  Those blocks are renumbered 0..n-1 (the
result of the method does not depend on where blocks sit: invariance to a
permutation of physical blocks, pinned in tests/test_oracle_attention.py),
the chosen sequences' tokens are written with reshape_and_cache_ref into that
compact pool, and paged_attention_ref runs on it.

`w` is duck-typed: any object with the Workload attributes (numpy arrays for
the query, the per-token bulk and decode-step K/V with their slots, block
tables and context lengths, plus the formats and scales).
"""
import numpy as np

from .paged import paged_attention_ref, reshape_and_cache_ref

_POISON = {"f32": np.float32(np.nan), "f16": np.float16(np.nan), "bf16": np.uint16(0x7FC0),
           "fp8": np.uint8(0x7F)}
_DTYPE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16, "fp8": np.uint8}


class CompactPool:
    def __init__(self, w, seqs):
        seqs = np.asarray(seqs, dtype=np.int64)
        BS = w.BS
        L = w.context_lens[seqs].astype(np.int64)
        nb = -(-L // BS)
        used = sorted({int(b) for s, n in zip(seqs, nb) for b in w.block_tables[s, :n]})
        self.phys = np.array(used, dtype=np.int64)
        remap = np.full(w.NB, -1, dtype=np.int64)
        remap[self.phys] = np.arange(len(used))
        self.remap = remap
        n = max(1, len(used))
        dt = _DTYPE[w.cache_fmt]
        self.k = np.full((n, w.Hk, w.D, BS), _POISON[w.cache_fmt], dtype=dt)
        self.v = self.k.copy()
        for keys, vals, slots in ((w.key_bulk, w.value_bulk, w.slot_bulk),
                                  (w.key_new, w.value_new, w.slot_new)):
            slots = np.asarray(slots, dtype=np.int64)
            ok = (slots >= 0) & (slots < w.NB * BS)
            blk = np.where(ok, slots // BS, 0)
            take = ok & (remap[blk] >= 0)
            idx = np.nonzero(take)[0]
            cs = remap[blk[idx]] * BS + slots[idx] % BS
            reshape_and_cache_ref(keys[idx], vals[idx], self.k, self.v, cs, w.src_fmt,
                                  w.cache_fmt, w.k_scale, w.v_scale)
        bt = w.block_tables[seqs].astype(np.int64)
        self.tables = np.where(bt >= 0, remap[np.maximum(bt, 0)], -1)
        self.seqs = seqs

    def attention(self, w):
        return paged_attention_ref(w.query[self.seqs], self.k, self.v, self.tables,
                                   w.context_lens[self.seqs], w.scale, w.q_fmt, w.cache_fmt,
                                   w.k_scale, w.v_scale)
