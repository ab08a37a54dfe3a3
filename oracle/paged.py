"""Plain CPU oracle of paged decode attention and of the slot-mapped KV writer.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py.  The product path never imports, calls or links
anything under oracle/.

Sources (the four pages this project is built from):
  [TGI]  "TGI PagedAttention 深度解析：分块 KV Cache、前缀复用与连续批处理的内存优化"
  [L3]   "第三讲：PagedAttention与vLLM——让KV Cache不再'吃'显存"
  [CB]   "Continuous Batching与PagedAttention：LLM推理引擎的核心技术"
  [VN]   "怎么加快大模型推理 10分钟学懂VLLM内部原理 (vLLM notes)"

What is computed (readings of the pages are named R-n and listed with their
reasons in the design notes of the repository):

* Pool layout.  Each cache is [num_blocks, num_kv_heads, head_size, BLOCK_SIZE]:
  per (block, head) the BLOCK_SIZE tokens of one head sit together, token index
  fastest ([TGI] §4.2, the paragraph on physical layout; [L3] "注意力计算的'分页'实现",
  the docstring of the forward pseudocode).  K and V use the same layout (R-1).
* Block table.  Logical block j of sequence s lives in physical block
  block_tables[s, j] ([TGI] §4.3; [L3] "核心数据结构：Block Table").
* Writer.  Each new token i is stored at slot slot_mapping[i]; slot =
  block * BLOCK_SIZE + offset (R-4); negative or out-of-pool slots write
  nothing.  Either the bits are copied, or the value is quantised to FP8 after a
  float32 division by a per-tensor scale ([TGI] §4.1, KV write side; R-9, R-10).
* Attention.  The forward pseudocode of [L3] ("注意力计算的'分页'实现") walks the
  logical blocks, reads each physical block through the table, multiplies the
  query with the key block, concatenates the per-block scores over all tokens
  and ends with "softmax and the weighted sum".  Filled in: scores are scaled by
  an explicit `scale` (R-3), tokens at positions >= context_len are excluded
  (R-6), query head h reads KV head h // (H / Hk) (R-2), an empty context gives
  zeros (R-7).  The partitioned variant ([TGI] §4.1: V2 splits a long sequence
  into 512-token partitions computed in parallel and merges them) must give the
  same result; it is here as a self-check of the merge arithmetic.

Arrays are numpy.  Storage formats: 'f32' (float32), 'f16' (float16), 'bf16'
(uint16 bit patterns), 'fp8' (uint8 OCP E4M3FN codes).  All attention
arithmetic is float64 and the result is returned unrounded.
"""

import math

import numpy as np

from .fp8_e4m3 import decode_e4m3, quantize_e4m3

FORMATS = ("f32", "f16", "bf16", "fp8")


# --------------------------------------------------------------------------- #
# storage formats
# --------------------------------------------------------------------------- #
def to_float32(a, fmt):
    """Exact float32 value of stored 16/32-bit elements (not for fp8)."""
    a = np.asarray(a)
    if fmt == "f32":
        return a.astype(np.float32)
    if fmt == "f16":
        return a.astype(np.float16).astype(np.float32)
    if fmt == "bf16":
        return (a.astype(np.uint16).astype(np.uint32) << 16).view(np.float32)
    raise ValueError(fmt)


def to_float64(a, fmt, fp8_scale=1.0):
    """Exact float64 value of stored elements; fp8 codes are decoded and scaled."""
    if fmt == "fp8":
        return decode_e4m3(a) * float(fp8_scale)
    return to_float32(a, fmt).astype(np.float64)


# --------------------------------------------------------------------------- #
# the writer
# --------------------------------------------------------------------------- #
def reshape_and_cache_ref(key, value, key_cache, value_cache, slot_mapping,
                          src_fmt, cache_fmt, k_scale=1.0, v_scale=1.0):
    """Write each new token's K and V into the paged caches, in place.

    key, value:            [T, Hk, D] in src_fmt
    key_cache, value_cache [NB, Hk, D, BS] in cache_fmt (== src_fmt, or 'fp8')
    slot_mapping           [T] int64; slot = block * BS + offset

    [TGI] §4.1 (KV write side: new keys/values are written into the block cache
    by their slot index, with an FP8 quantised variant).
    """
    NB, Hk, D, BS = key_cache.shape
    slots = np.asarray(slot_mapping, dtype=np.int64)
    seen = set()
    for i, s in enumerate(slots.tolist()):
        if s < 0 or s >= NB * BS:
            continue                       # no write (R-4)
        assert s not in seen, "duplicate slots are a precondition violation"
        seen.add(s)
        b, o = divmod(s, BS)
        if cache_fmt == src_fmt:
            key_cache[b, :, :, o] = key[i]          # bit copy
            value_cache[b, :, :, o] = value[i]
        elif cache_fmt == "fp8":
            key_cache[b, :, :, o] = quantize_e4m3(to_float32(key[i], src_fmt), k_scale)
            value_cache[b, :, :, o] = quantize_e4m3(to_float32(value[i], src_fmt), v_scale)
        else:
            raise ValueError((src_fmt, cache_fmt))


# --------------------------------------------------------------------------- #
# block-table gather
# --------------------------------------------------------------------------- #
def gather_ref(cache, block_table_row, context_len):
    """Logical KV of one sequence, in storage format: [Hk, L, D].

    Logical block j is physical block block_table_row[j] ([TGI] §4.3;
    [L3] "注意力计算的'分页'实现": physical_block_idx = block_table[logical_block_idx]);
    inside a block the token index is the last axis ([TGI] §4.2).
    """
    NB, Hk, D, BS = cache.shape
    L = int(context_len)
    nb = -(-L // BS)
    phys = np.asarray(block_table_row[:nb], dtype=np.int64)
    blocks = cache[phys]                       # [nb, Hk, D, BS]
    tok = blocks.transpose(1, 0, 3, 2)         # [Hk, nb, BS, D]
    return tok.reshape(Hk, nb * BS, D)[:, :L, :]


# --------------------------------------------------------------------------- #
# attention
# --------------------------------------------------------------------------- #
def softmax_weights_ref(q_vec, k_tokens, scale):
    """Softmax weights of one query over L keys ([L3] forward pseudocode: scores
    query . key, then softmax).  float64; k_tokens is [L, D]."""
    x = scale * (k_tokens @ q_vec)
    m = x.max()
    w = np.exp(x - m)
    return w / w.sum()


def paged_attention_ref(query, key_cache, value_cache, block_tables, context_lens,
                        scale, q_fmt, cache_fmt, k_scale=1.0, v_scale=1.0):
    """Decode attention of one query token per sequence over its paged KV.

    query [S, H, D] (q_fmt); caches [NB, Hk, D, BS] (cache_fmt);
    block_tables [S, MB] int; context_lens [S] int.  Returns float64 [S, H, D].
    """
    S, H, D = query.shape
    Hk = key_cache.shape[1]
    assert H % Hk == 0
    g = H // Hk
    q64 = to_float64(query, q_fmt)
    out = np.zeros((S, H, D), dtype=np.float64)
    for s in range(S):
        L = int(context_lens[s])
        if L <= 0:
            continue                                    # R-7: empty context -> 0
        Kl = to_float64(gather_ref(key_cache, block_tables[s], L), cache_fmt, k_scale)
        Vl = to_float64(gather_ref(value_cache, block_tables[s], L), cache_fmt, v_scale)
        for h in range(H):
            kvh = h // g                                # R-2
            w = softmax_weights_ref(q64[s, h], Kl[kvh], scale)
            out[s, h] = w @ Vl[kvh]
    return out


def paged_attention_partitioned_ref(query, key_cache, value_cache, block_tables,
                                    context_lens, scale, q_fmt, cache_fmt,
                                    k_scale=1.0, v_scale=1.0, partition_size=512,
                                    num_partitions=None):
    """Same result, computed per partition and merged ([TGI] §4.1: V2 splits long
    sequences into _PARTITION_SIZE = 512 token partitions, computes them in
    parallel and merges them).

    Per partition p: m_p = max score, l_p = sum exp(score - m_p),
    o_p = sum exp(score - m_p) * v.  Merge: M = max_p m_p,
    out = sum_p exp(m_p - M) o_p / sum_p exp(m_p - M) l_p.
    A partition with no token has l_p = 0 and weight 0.  `num_partitions`
    (default: just enough for the sequence) lets trailing empty partitions in.
    """
    S, H, D = query.shape
    Hk = key_cache.shape[1]
    g = H // Hk
    q64 = to_float64(query, q_fmt)
    out = np.zeros((S, H, D), dtype=np.float64)
    for s in range(S):
        L = int(context_lens[s])
        if L <= 0:
            continue
        Kl = to_float64(gather_ref(key_cache, block_tables[s], L), cache_fmt, k_scale)
        Vl = to_float64(gather_ref(value_cache, block_tables[s], L), cache_fmt, v_scale)
        n_p = num_partitions if num_partitions is not None else -(-L // partition_size)
        for h in range(H):
            kvh = h // g
            ms, ls, os_ = [], [], []
            for p in range(n_p):
                lo, hi = p * partition_size, min((p + 1) * partition_size, L)
                if hi <= lo:
                    ms.append(-math.inf)
                    ls.append(0.0)
                    os_.append(np.zeros(D))
                    continue
                x = scale * (Kl[kvh, lo:hi] @ q64[s, h])
                m = x.max()
                e = np.exp(x - m)
                ms.append(m)
                ls.append(e.sum())
                os_.append(e @ Vl[kvh, lo:hi])
            M = max(ms)
            num = np.zeros(D)
            den = 0.0
            for m, l, o in zip(ms, ls, os_):
                if l == 0.0:
                    continue
                w = math.exp(m - M)
                num += w * o
                den += w * l
            out[s, h] = num / den
    return out


# --------------------------------------------------------------------------- #
# copy-on-write block copy
# --------------------------------------------------------------------------- #
def copy_blocks_ref(key_cache, value_cache, src_dst_pairs):
    """Copy whole physical blocks (all heads, all tokens), in place, for each
    (src, dst) pair: the copy step of copy-on-write ([VN] "Sharing KV Cache":
    when a branch appends to a block whose ref count exceeds 1, a new block is
    allocated, the old block's contents are copied into it and the branch's
    block table is pointed at the copy; [L3] "共享前缀").  All sources are read
    before any destination is written.
    """
    pairs = [(int(a), int(b)) for a, b in src_dst_pairs]
    k_src = [key_cache[a].copy() for a, _ in pairs]
    v_src = [value_cache[a].copy() for a, _ in pairs]
    for (a, b), k, v in zip(pairs, k_src, v_src):
        key_cache[b] = k
        value_cache[b] = v
