"""The prefix cache driving the device calls: requests whose prompts share
leading blocks with earlier, finished requests take the cached blocks (their
KV written by the earlier request) and write only the rest; under pool
pressure cached blocks are evicted and reused.  Each token's key and value
are a fixed function of the token ids up to it (as in a model, where a
token's KV depends on its whole prefix), so a cached block is valid for a
new request exactly when its tokens and all before them match.  Every decode
output must equal dense attention over the request's own KV history,
computed by the oracle from that history alone."""
import sys
import zlib

import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads.gpu import TORCH_DTYPE, to_device

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import paged_kv_cache_139_amd as pkv

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def kv_of(prefix, Hk, D, q_fmt):
    """Key and value [Hk, D] of the last token of `prefix` (token ids)."""
    seed = zlib.crc32(np.asarray(prefix, np.int64).tobytes())
    f = np.random.default_rng(seed).standard_normal((2, Hk, D), dtype=np.float32)
    return workloads.cast_f32(f[0], q_fmt), workloads.cast_f32(f[1], q_fmt)


def stored(x, q_fmt, cache_fmt, scale, Hk, D):
    """What the cache holds for source rows x [n, Hk, D] (the oracle's writer)."""
    n = len(x)
    dt = workloads.np_storage_dtype(cache_fmt)
    tmp = np.zeros((max(1, -(-n // 16)), Hk, D, 16), dt)
    oracle.reshape_and_cache_ref(x, x, tmp, tmp.copy(), np.arange(n, dtype=np.int64), q_fmt,
                                 cache_fmt, scale, scale)
    return tmp.transpose(0, 3, 1, 2).reshape(-1, Hk, D)[:n]


def dense(q, hk, hv, scale, q_fmt, cache_fmt, ks, vs, bs):
    S = len(hk)
    Hk, D = hk[0].shape[1], hk[0].shape[2]
    lens = np.array([len(k) for k in hk], np.int32)
    nbs = [-(-int(n) // bs) for n in lens]
    dt = workloads.np_storage_dtype(cache_fmt)
    kc = np.zeros((max(1, sum(nbs)), Hk, D, bs), dt)
    vc = np.zeros_like(kc)
    bt = np.full((S, max(1, max(nbs))), -1, np.int32)
    pos = 0
    for s in range(S):
        bt[s, :nbs[s]] = np.arange(pos, pos + nbs[s])
        for t in range(int(lens[s])):
            kc[pos + t // bs, :, :, t % bs] = hk[s][t]
            vc[pos + t // bs, :, :, t % bs] = hv[s][t]
        pos += nbs[s]
    return oracle.paged_attention_ref(q, kc, vc, bt, lens, scale, q_fmt, cache_fmt, ks, vs)


@pytest.mark.parametrize("q_fmt,cache_fmt,H,Hk", [("bf16", "bf16", 4, 2), ("f16", "fp8", 8, 2),
                                                  ("f16", "f16", 4, 4)])
def test_requests_share_cached_prompt_blocks(q_fmt, cache_fmt, H, Hk):
    say(f"prefix cache {q_fmt}/{cache_fmt} H={H} Hk={Hk}")
    rng = np.random.default_rng(H * 7 + Hk)
    D, BS, NB = 64, 16, 24
    fp8 = cache_fmt == "fp8"
    ks = vs = 0.05 if fp8 else 1.0
    scale = D ** -0.5
    bm = pkv.BlockManager(NB, BS)
    if fp8:
        kc = torch.full((NB, Hk, D, BS), 0x7F, dtype=torch.uint8, device=DEV)
    else:
        kc = torch.full((NB, Hk, D, BS), float("nan"), dtype=TORCH_DTYPE[cache_fmt], device=DEV)
    vc = kc.clone()
    live = {}                     # id -> token ids of the request so far
    hits = []
    system = list(rng.integers(0, 50, size=40))          # a shared 40-token system prompt

    def start(rid, prompt):
        cached = bm.add_sequence_cached(rid, prompt)
        hits.append(cached)
        n = len(prompt)
        if n > cached:                                      # write only the uncached tokens
            k = np.stack([kv_of(prompt[:i + 1], Hk, D, q_fmt)[0] for i in range(cached, n)])
            v = np.stack([kv_of(prompt[:i + 1], Hk, D, q_fmt)[1] for i in range(cached, n)])
            pkv.reshape_and_cache(to_device(k, q_fmt, DEV), to_device(v, q_fmt, DEV), kc, vc,
                                  torch.tensor(bm.token_slots(rid, cached, n - cached),
                                               dtype=torch.int64, device=DEV), ks, vs)
        live[rid] = list(prompt)

    def step():
        ids = sorted(live)
        slots, pairs, done = bm.append_tokens(ids)
        assert done == len(ids) and not pairs
        new = [int(rng.integers(0, 50)) for _ in ids]
        for i, rid in enumerate(ids):
            live[rid].append(new[i])
        k = np.stack([kv_of(live[r], Hk, D, q_fmt)[0] for r in ids])
        v = np.stack([kv_of(live[r], Hk, D, q_fmt)[1] for r in ids])
        pkv.reshape_and_cache(to_device(k, q_fmt, DEV), to_device(v, q_fmt, DEV), kc, vc,
                              torch.tensor(slots, dtype=torch.int64, device=DEV), ks, vs)
        MB = max(len(bm.table(r)[0]) for r in ids)
        bt, lens = bm.build_block_tables(ids, MB)
        q = workloads.cast_f32(rng.standard_normal((len(ids), H, D), dtype=np.float32), q_fmt)
        out = torch.empty((len(ids), H, D), dtype=TORCH_DTYPE[q_fmt], device=DEV)
        pkv.paged_attention_decode(out, to_device(q, q_fmt, DEV), kc, vc,
                                   torch.from_numpy(bt).to(DEV), torch.from_numpy(lens).to(DEV),
                                   scale, ks, vs, 32)
        torch.cuda.synchronize()
        hk, hv = [], []
        for r in ids:                              # each request's history from its tokens
            toks = live[r]
            rows = [kv_of(toks[:i + 1], Hk, D, q_fmt) for i in range(len(toks))]
            hk.append(stored(np.stack([x[0] for x in rows]), q_fmt, cache_fmt, ks, Hk, D))
            hv.append(stored(np.stack([x[1] for x in rows]), q_fmt, cache_fmt, vs, Hk, D))
        ref = dense(q, hk, hv, scale, q_fmt, cache_fmt, ks, vs, BS)
        gpu = out.float().cpu().numpy().astype(np.float64)
        assert np.isfinite(gpu).all()
        bound = 5e-2 if fp8 else 2e-3 + 1e-2 * np.abs(ref)
        assert (np.abs(gpu - ref) <= bound).all(), np.abs(gpu - ref).max()

    def finish(rid):
        bm.free_sequence(rid)
        del live[rid]

    start(0, system + list(rng.integers(0, 50, size=9)))        # 49 tokens: 3 full blocks
    for _ in range(3):
        step()
    finish(0)                                                    # its 3 prompt blocks cached
    start(1, system + list(rng.integers(0, 50, size=30)))        # shares 2 blocks (32 tokens)
    start(2, system[:35])                                        # shares 2 blocks
    for _ in range(4):
        step()
    finish(1)
    start(3, system + list(rng.integers(0, 50, size=60)))        # shares 2 again
    for _ in range(3):
        step()
    finish(2)
    finish(3)
    # pool pressure: a long unrelated prompt takes free blocks, then evicts cached ones
    start(4, list(rng.integers(50, 90, size=16 * 18 + 3)))
    step()
    assert bm.num_cached() < 8
    finish(4)
    start(5, system + [1, 2, 3])                                 # whatever is still cached
    start(6, list(rng.integers(0, 50, size=20)))
    for _ in range(2):
        step()
    assert hits[:4] == [0, 32, 32, 32], hits
    bm.close()
