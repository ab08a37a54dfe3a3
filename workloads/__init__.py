"""Seeded synthetic inputs for paged decode attention and the KV writer.

Shared by the tests, bench.py and smoke(): this module draws random numbers,
casts them to storage formats and builds block tables with a small test-only
block allocator.  It holds none of the attention or quantisation arithmetic and
imports neither the oracle nor the HIP library.

The five workloads are shaped like the pages' examples (a LLaMA-7B-shaped
batch, long contexts split into 512-token partitions, parallel sampling with a
shared prefix, an FP8 KV batch); no dataset is involved anywhere.

Recipe (all draws numpy PCG64; the tree of seeds comes from
numpy.random.SeedSequence(seed).spawn):
  child 0: context lengths;  child 1: the pool permutation that the allocator
  hands out blocks from;  child 2: the query [S, H, D];  child 3: one child per
  owner of tokens (a sequence, or for the shared-prefix workload one per prompt
  prefix and one per sample suffix), each drawing K then V as [n_tok, Hk, D].
  Values are float32 standard normal, cast to the storage format with round to
  nearest even (numpy for float16, torch CPU for bfloat16).

Storage formats as in the oracle: 'f32' float32, 'f16' float16, 'bf16' uint16
bit patterns, 'fp8' uint8 codes (the writer produces those from bf16 or f16).
"""

from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

BLOCK_SIZE = 16


# --------------------------------------------------------------------------- #
# storage casts (input preparation only)
# --------------------------------------------------------------------------- #
def cast_f32(x: np.ndarray, fmt: str) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    if fmt == "f32":
        return x
    if fmt == "f16":
        return x.astype(np.float16)
    if fmt == "bf16":
        import torch
        return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    raise ValueError(fmt)


def np_storage_dtype(fmt: str):
    return {"f32": np.float32, "f16": np.float16, "bf16": np.uint16, "fp8": np.uint8}[fmt]


# --------------------------------------------------------------------------- #
# test-only block allocator (builds block tables; not part of the library)
# --------------------------------------------------------------------------- #
class BlockAllocator:
    """Free list + reference counts, after the allocator sketches on the pages
    (第三讲 "核心数据结构：Block Table": allocate ceil(tokens / block_size) blocks
    or fail when the free list runs short; Continuous Batching §3.2: fork shares
    the parent's blocks and increments their counts, free decrements and
    returns a block when its count reaches zero)."""

    def __init__(self, order: np.ndarray):
        self.free = [int(b) for b in order]
        self.free.reverse()                 # pop() hands out order[0], order[1], ...
        self.ref = {}

    def allocate(self, n_blocks: int) -> list[int]:
        if n_blocks > len(self.free):
            raise MemoryError(f"pool exhausted: need {n_blocks}, {len(self.free)} free")
        out = [self.free.pop() for _ in range(n_blocks)]
        for b in out:
            self.ref[b] = 1
        return out

    def fork(self, blocks: list[int]) -> list[int]:
        for b in blocks:
            self.ref[b] += 1
        return list(blocks)

    def release(self, blocks: list[int]) -> None:
        for b in blocks:
            self.ref[b] -= 1
            if self.ref[b] == 0:
                del self.ref[b]
                self.free.append(b)

    def check(self, n_pool: int) -> None:
        live = set(self.ref)
        assert not (live & set(self.free)), "block both live and free"
        assert len(set(self.free)) == len(self.free), "duplicate free block"
        assert len(live) + len(self.free) == n_pool, "leaked block"


# --------------------------------------------------------------------------- #
# workload container
# --------------------------------------------------------------------------- #
@dataclasses.dataclass
class Workload:
    name: str
    S: int
    H: int
    Hk: int
    D: int
    NB: int
    MB: int
    q_fmt: str
    cache_fmt: str
    scale: float
    k_scale: float
    v_scale: float
    context_lens: np.ndarray        # [S] int32
    block_tables: np.ndarray        # [S, MB] int32, padding -1
    query: np.ndarray               # [S, H, D] storage of q_fmt
    key_bulk: np.ndarray            # [T, Hk, D] storage of src_fmt (tokens before the new one)
    value_bulk: np.ndarray
    slot_bulk: np.ndarray           # [T] int64
    key_new: np.ndarray             # [S, Hk, D]: the token each sequence appends (position L-1)
    value_new: np.ndarray
    slot_new: np.ndarray            # [S] int64 (-1 for an empty sequence)
    shared_groups: list = dataclasses.field(default_factory=list)  # [(seq ids, n prefix blocks)]
    BS: int = BLOCK_SIZE

    @property
    def src_fmt(self) -> str:
        return self.q_fmt

    @property
    def g(self) -> int:
        return self.H // self.Hk

    def group_arrays(self):
        """(group_starts [G + 1], group_prefix_blocks [G], largest group size) for
        the shared-prefix decode: the sharing groups in batch order, every other
        sequence a group of its own without a prefix."""
        starts, prefix = [0], []
        s = 0
        groups = {seqs[0]: (seqs, pb) for seqs, pb in self.shared_groups}
        while s < self.S:
            if s in groups:
                seqs, pb = groups[s]
                assert seqs == list(range(s, s + len(seqs))), "groups must be contiguous"
                s += len(seqs)
                prefix.append(pb)
            else:
                s += 1
                prefix.append(0)
            starts.append(s)
        sizes = np.diff(starts)
        return (np.array(starts, np.int32), np.array(prefix, np.int32),
                int(sizes.max()) if len(sizes) else 1)

    def kv_elem_bytes(self) -> int:
        return {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1}[self.cache_fmt]

    def q_elem_bytes(self) -> int:
        return {"f32": 4, "f16": 2, "bf16": 2}[self.q_fmt]

    def decode_bytes(self, unique: bool = True) -> int:
        """Algorithmic HBM bytes of one decode call: every (token, KV head) of K
        and V once, q in and out once, the used block-table entries and the
        lengths.  With unique=True a physical block shared by several sequences
        is counted once."""
        L = self.context_lens.astype(np.int64)
        nb = -(-L // self.BS)
        kv_tok = int(L.sum())
        if unique and self.shared_groups:
            for seqs, nblk in self.shared_groups:
                kv_tok -= (len(seqs) - 1) * nblk * self.BS
        kv = kv_tok * self.Hk * self.D * 2 * self.kv_elem_bytes()
        qo = self.S * self.H * self.D * 2 * self.q_elem_bytes()
        return kv + qo + int(nb.sum()) * 4 + self.S * 4

    def writer_bytes(self, n_tokens: int) -> int:
        """Bytes read + written by the writer for n_tokens new tokens."""
        src = {"f32": 4, "f16": 2, "bf16": 2}[self.src_fmt]
        return n_tokens * self.Hk * self.D * 2 * (src + self.kv_elem_bytes()) + n_tokens * 8


def _slot(table_row, pos: int, bs: int = BLOCK_SIZE) -> int:
    return int(table_row[pos // bs]) * bs + pos % bs


def _draw_kv(seed_seqs, n_tokens, Hk, D, fmt, threads=16):
    """One (K, V) pair of [n, Hk, D] arrays per owner, drawn in parallel from
    independent child generators (results do not depend on the thread count)."""
    def one(args):
        ss, n = args
        rng = np.random.default_rng(ss)
        k = rng.standard_normal((n, Hk, D), dtype=np.float32)
        v = rng.standard_normal((n, Hk, D), dtype=np.float32)
        return cast_f32(k, fmt), cast_f32(v, fmt)
    with ThreadPoolExecutor(threads) as ex:
        return list(ex.map(one, zip(seed_seqs, n_tokens)))


def build(name: str, S: int, H: int, Hk: int, D: int, NB: int, q_fmt: str,
          cache_fmt: str, lens: np.ndarray | None = None, lens_fn=None,
          seed: int = 0, scale: float | None = None, k_scale: float = 1.0,
          v_scale: float = 1.0, prefix_tokens: int = 0, n_samples: int = 1,
          MB: int | None = None, threads: int = 16, block_size: int = BLOCK_SIZE) -> Workload:
    """General builder.  Either `lens` (explicit context lengths) or `lens_fn(rng)`.

    With n_samples > 1 the S sequences form S / n_samples groups; each group
    shares one prefix of `prefix_tokens` tokens (a whole number of blocks,
    allocated once and forked to every sample), followed by per-sample suffix
    tokens on private blocks; lens then gives the suffix lengths.
    """
    root = np.random.SeedSequence(seed)
    c_len, c_perm, c_q, c_kv = root.spawn(4)
    if lens is None:
        lens = lens_fn(np.random.default_rng(c_len))
    lens = np.asarray(lens, dtype=np.int64)
    bs = int(block_size)
    assert prefix_tokens % bs == 0
    perm = np.random.default_rng(c_perm).permutation(NB)
    alloc = BlockAllocator(perm)

    tables: list[list[int]] = []
    ctx = np.zeros(S, dtype=np.int64)
    owners = []                 # (kind, index, n tokens) in draw order
    shared_groups = []
    if n_samples > 1:
        assert S % n_samples == 0
        n_groups = S // n_samples
        for gi in range(n_groups):
            pre = alloc.allocate(prefix_tokens // bs)
            owners.append(("prefix", gi, prefix_tokens))
            seqs = []
            for j in range(n_samples):
                s = gi * n_samples + j
                suf = int(lens[s])
                row = alloc.fork(pre) + alloc.allocate(-(-suf // bs))
                tables.append(row)
                ctx[s] = prefix_tokens + suf
                owners.append(("suffix", s, suf))
                seqs.append(s)
            alloc.release(pre)          # the prompt itself no longer holds the prefix
            shared_groups.append((seqs, prefix_tokens // bs))
    else:
        for s in range(S):
            tables.append(alloc.allocate(-(-int(lens[s]) // bs)))
            ctx[s] = lens[s]
            owners.append(("seq", s, int(lens[s])))
    alloc.check(NB)

    nb = np.array([len(t) for t in tables], dtype=np.int64)
    if MB is None:
        MB = max(1, int(nb.max()) if S else 1)
    bt = np.full((S, MB), -1, dtype=np.int32)
    for s, t in enumerate(tables):
        bt[s, :len(t)] = t

    q = cast_f32(np.random.default_rng(c_q).standard_normal((S, H, D), dtype=np.float32), q_fmt)

    src_fmt = q_fmt
    kv = _draw_kv(c_kv.spawn(len(owners)), [o[2] for o in owners], Hk, D, src_fmt, threads)

    # Bulk tokens: every token except each sequence's last one, which is the
    # decode-step append.  Shared prefixes are written once.
    kb, vb, sb = [], [], []
    k_new = np.zeros((S, Hk, D), dtype=np_storage_dtype(src_fmt))
    v_new = np.zeros_like(k_new)
    s_new = np.full(S, -1, dtype=np.int64)
    for (kind, idx, n), (k, v) in zip(owners, kv):
        if kind == "prefix":
            row = tables[idx * n_samples]
            kb.append(k)
            vb.append(v)
            sb.append(np.array([_slot(row, p, bs) for p in range(n)], dtype=np.int64))
            continue
        s = idx
        base = prefix_tokens if kind == "suffix" else 0
        row = tables[s]
        if n == 0:
            if kind == "suffix":
                raise ValueError("empty suffix")
            continue
        kb.append(k[:n - 1])
        vb.append(v[:n - 1])
        sb.append(np.array([_slot(row, base + p, bs) for p in range(n - 1)], dtype=np.int64))
        k_new[s] = k[n - 1]
        v_new[s] = v[n - 1]
        s_new[s] = _slot(row, base + n - 1, bs)
    Tb = sum(len(x) for x in sb)
    key_bulk = np.concatenate(kb) if kb else np.zeros((0, Hk, D), np_storage_dtype(src_fmt))
    value_bulk = np.concatenate(vb) if vb else np.zeros_like(key_bulk)
    slot_bulk = np.concatenate(sb) if sb else np.zeros(0, np.int64)
    assert len(key_bulk) == Tb

    return Workload(name=name, S=S, H=H, Hk=Hk, D=D, NB=NB, MB=MB, q_fmt=q_fmt,
                    cache_fmt=cache_fmt,
                    scale=(1.0 / math.sqrt(D)) if scale is None else float(scale),
                    k_scale=k_scale, v_scale=v_scale,
                    context_lens=ctx.astype(np.int32), block_tables=bt, query=q,
                    key_bulk=key_bulk, value_bulk=value_bulk, slot_bulk=slot_bulk,
                    key_new=k_new, value_new=v_new, slot_new=s_new,
                    shared_groups=shared_groups, BS=bs)


# --------------------------------------------------------------------------- #
# the five named workloads
# --------------------------------------------------------------------------- #
FP8_SCALE = 6.0 / 448.0      # maps +-6 standard deviations onto the E4M3 maximum

WORKLOADS = {
    # 4 seqs x 4 heads (MHA), head 64, fp32, lengths U{1..200}, 64-block pool
    "tiny": dict(S=4, H=4, Hk=4, D=64, NB=64, q_fmt="f32", cache_fmt="f32", seed=1001,
                 lens_fn=lambda r: r.integers(1, 200, size=4, endpoint=True)),
    # LLaMA-7B-shaped layer: 64 seqs x 32 heads x 128, fp16, lengths U{128..2048}
    "llama7b_b64": dict(S=64, H=32, Hk=32, D=128, NB=16384, q_fmt="f16", cache_fmt="f16",
                        seed=1002,
                        lens_fn=lambda r: r.integers(128, 2048, size=64, endpoint=True)),
    # long contexts: 8 seqs x 32 heads x 128, bf16, lengths U{16384..32768}
    "long32k": dict(S=8, H=32, Hk=32, D=128, NB=40000, q_fmt="bf16", cache_fmt="bf16",
                    seed=1003,
                    lens_fn=lambda r: r.integers(16384, 32768, size=8, endpoint=True)),
    # parallel sampling: 16 prompts x 8 samples, 1024-token shared prefix, GQA 64/8
    "shared_prefix_gqa": dict(S=128, H=64, Hk=8, D=128, NB=4096, q_fmt="bf16",
                              cache_fmt="bf16", seed=1004, prefix_tokens=1024, n_samples=8,
                              lens_fn=lambda r: r.integers(1, 256, size=128, endpoint=True)),
    # fp8 KV: 256 seqs, GQA 32/8, lognormal lengths (median 512, sigma 1) in [16, 8192]
    "fp8_mixed": dict(S=256, H=32, Hk=8, D=128, NB=32768, q_fmt="bf16", cache_fmt="fp8",
                      seed=1005, k_scale=FP8_SCALE, v_scale=FP8_SCALE,
                      lens_fn=lambda r: np.clip(np.rint(np.exp(r.normal(np.log(512.0), 1.0,
                                                                        size=256))),
                                                16, 8192).astype(np.int64)),
}


def make(name: str, threads: int = 16, **overrides) -> Workload:
    spec = dict(WORKLOADS[name])
    spec.update(overrides)
    return build(name=name, threads=threads, **spec)
