"""Decode at the extremes of its size range, against the oracle.

- one sequence of 131072 tokens (8192 blocks): 64 partitions of the default
  size (the merge's statistics fill exactly one wave) and 8192 partitions of
  16 tokens (128 rounds of 64 statistics), on both kernels;
- 4096 sequences of 1..64 tokens with 32 heads (131072 (sequence, head)
  items, most ids past the last item of their partition), sampled;
- a pool whose byte offsets pass 2^32 (tiles read and written above 4 GiB)."""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads.gpu import DeviceWorkload

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import paged_kv_cache_139_amd as pkv

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def close(gpu, ref, fp8, what):
    assert np.isfinite(gpu).all(), what
    err = np.abs(gpu - ref)
    bound = 5e-2 if fp8 else 2e-3 + 1e-2 * np.abs(ref)
    assert (err <= bound).all(), f"{what}: max error {err.max()}"


@pytest.mark.parametrize("q_fmt,cache_fmt,H,Hk", [("bf16", "bf16", 8, 8), ("bf16", "fp8", 8, 2)])
@pytest.mark.parametrize("P", [0, 16])
def test_one_very_long_sequence(q_fmt, cache_fmt, H, Hk, P):
    say(f"131072 tokens {q_fmt}/{cache_fmt} H={H} Hk={Hk} P={P}: generating inputs")
    L = 131072
    fp8 = cache_fmt == "fp8"
    w = workloads.build("long1", S=2, H=H, Hk=Hk, D=128, NB=L // 16 + 40, q_fmt=q_fmt,
                        cache_fmt=cache_fmt, lens=np.array([L, 77]), seed=31 + P,
                        k_scale=6 / 448 if fp8 else 1.0, v_scale=6 / 448 if fp8 else 1.0)
    dw = DeviceWorkload(w, DEV, P).fill()
    dw.decode_append()
    torch.cuda.synchronize()
    gpu = dw.out_f64()
    cp = oracle.CompactPool(w, [0, 1])
    close(gpu, cp.attention(w), fp8, f"L={L} P={P}")


@pytest.mark.parametrize("q_fmt,cache_fmt,H,Hk", [("f16", "f16", 32, 32), ("bf16", "fp8", 32, 8)])
def test_many_short_sequences(q_fmt, cache_fmt, H, Hk):
    say(f"4096 sequences {q_fmt}/{cache_fmt} H={H} Hk={Hk}: generating inputs")
    rng = np.random.default_rng(77)
    lens = rng.integers(1, 65, size=4096)
    fp8 = cache_fmt == "fp8"
    nb = int(np.sum(-(-lens // 16)))
    w = workloads.build("many", S=4096, H=H, Hk=Hk, D=128, NB=nb + 64, q_fmt=q_fmt,
                        cache_fmt=cache_fmt, lens=lens, seed=5,
                        k_scale=6 / 448 if fp8 else 1.0, v_scale=6 / 448 if fp8 else 1.0)
    dw = DeviceWorkload(w, DEV, 16).fill()          # 16-token partitions: up to 4 per sequence
    dw.decode_append()
    torch.cuda.synchronize()
    gpu = dw.out_f64()
    seqs = [0, 1, 1000, 2047, 3333, 4095] + [int(s) for s in np.argsort(lens)[-3:]]
    cp = oracle.CompactPool(w, seqs)
    close(gpu[seqs], cp.attention(w), fp8, "many sequences")


def test_pool_offsets_past_4gib():
    """Blocks placed at the top of a 4.6 GB pool per cache (byte offsets beyond
    2^32): the writer and decode with append address them."""
    say("pool past 4 GiB: generating inputs")
    NB, Hk, D = 140000, 8, 128                      # 140000 * 8 * 128 * 16 * 2 B = 4.6 GB per cache
    lens = np.array([300, 1000, 17, 2048])
    w = workloads.build("big", S=4, H=32, Hk=Hk, D=D, NB=NB, q_fmt="bf16", cache_fmt="bf16",
                        lens=lens, seed=12)
    # move every used block to the top of the pool
    bt = w.block_tables.copy()
    used = bt[bt >= 0]
    top = np.arange(NB - len(used), NB)
    remap = dict(zip(used.tolist(), top.tolist()))
    w.block_tables = np.where(bt >= 0, np.vectorize(lambda b: remap.get(int(b), b))(bt),
                              bt).astype(np.int32)
    for name in ("slot_bulk", "slot_new"):
        sl = getattr(w, name)
        b, o = sl // 16, sl % 16
        setattr(w, name, np.where(sl >= 0, np.vectorize(lambda x: remap.get(int(x), x))(b) * 16 + o,
                                  sl).astype(np.int64))
    assert (w.block_tables[w.block_tables >= 0].astype(np.int64) * Hk * D * 16 * 2 >= 2 ** 32).all()
    dw = DeviceWorkload(w, DEV).fill()
    dw.decode_append()
    torch.cuda.synchronize()
    gpu = dw.out_f64()
    cp = oracle.CompactPool(w, [0, 1, 2, 3])
    close(gpu, cp.attention(w), False, "pool past 4 GiB")
