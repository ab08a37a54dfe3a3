"""GPU parity at the head sizes beyond 64 and 128: 32, 80, 96, 112, 120, 192
and 256.  The vector kernel reads R rows per load (R = 64 / element bytes);
where head_size is not a multiple of R its last load is partly past the
last row, which these sizes exercise for every cache type (120 for all of
them, 80 / 112 for 16-bit and E4M3 caches, 32 / 96 / 192 for E4M3).  The
matrix cores take the 16-bit caches at 32, 80, 96 and 112 with grouped heads.

Decode is within |gpu - ref| <= 2e-3 + 1e-2 |ref| (16/32-bit caches) or 5e-2
(FP8) of the oracle; decode with append leaves caches and output bit-equal to
the writer followed by decode, and caches equal to the oracle's pool."""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads.gpu import DeviceWorkload, to_numpy_storage

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import paged_kv_cache_139_amd as pkv

DEV = "cuda:0"
HEAD_SIZES = [32, 80, 96, 112, 120, 192, 256]
DTYPES = [("f32", "f32"), ("f16", "f16"), ("bf16", "bf16"), ("f16", "fp8"), ("bf16", "fp8")]
LENS = np.array([1, 7, 16, 17, 33, 100, 0, 257, 520])


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host_pool(w):
    dt = workloads.np_storage_dtype(w.cache_fmt)
    poison = {"f32": np.nan, "f16": np.nan, "bf16": 0x7FC0, "fp8": 0x7F}[w.cache_fmt]
    kc = np.full((w.NB, w.Hk, w.D, w.BS), poison, dtype=dt)
    vc = kc.copy()
    for keys, vals, slots in ((w.key_bulk, w.value_bulk, w.slot_bulk),
                              (w.key_new, w.value_new, w.slot_new)):
        oracle.reshape_and_cache_ref(keys, vals, kc, vc, slots, w.src_fmt, w.cache_fmt,
                                     w.k_scale, w.v_scale)
    return kc, vc


def assert_close(gpu, ref, fp8, what):
    assert np.isfinite(gpu).all(), f"{what}: non-finite output"
    err = np.abs(gpu - ref)
    bound = 5e-2 if fp8 else 2e-3 + 1e-2 * np.abs(ref)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} elements out of tolerance; worst at {i}: "
                             f"gpu {gpu[i]!r} ref {ref[i]!r}")


def small(BS, q_fmt, cache_fmt, D, H, Hk, seed):
    fp8 = cache_fmt == "fp8"
    nb = int(np.sum(-(-LENS // BS)))
    return workloads.build("hd", S=len(LENS), H=H, Hk=Hk, D=D, NB=nb + 9, q_fmt=q_fmt,
                           cache_fmt=cache_fmt, lens=LENS, seed=seed, block_size=BS,
                           k_scale=0.02 if fp8 else 1.0, v_scale=0.03 if fp8 else 1.0)


def bits(a):
    return np.ascontiguousarray(a).view(np.uint8)


def tbits(t):
    return t.contiguous().view(torch.uint8).cpu().numpy()


def run_decode(BS, q_fmt, cache_fmt, D, H, Hk, P):
    w = small(BS, q_fmt, cache_fmt, D, H, Hk, 11 * D + 3 * H + BS + P)
    dw = DeviceWorkload(w, DEV, P).fill()
    dw.out.fill_(float("nan"))
    dw.step()
    torch.cuda.synchronize()
    kc, vc = host_pool(w)
    assert np.array_equal(bits(to_numpy_storage(dw.k_cache, cache_fmt)), bits(kc))
    assert np.array_equal(bits(to_numpy_storage(dw.v_cache, cache_fmt)), bits(vc))
    ref = oracle.paged_attention_ref(w.query, kc, vc, w.block_tables, w.context_lens, w.scale,
                                     q_fmt, cache_fmt, w.k_scale, w.v_scale)
    gpu = dw.out_f64()
    assert_close(gpu, ref, cache_fmt == "fp8", f"D={D} BS={BS}")
    assert np.array_equal(gpu[LENS == 0], np.zeros_like(gpu[LENS == 0]))


@pytest.mark.parametrize("D", HEAD_SIZES)
@pytest.mark.parametrize("q_fmt,cache_fmt", DTYPES)
@pytest.mark.parametrize("H,Hk", [(4, 4), (8, 2), (20, 1)])
@pytest.mark.parametrize("P", [0, 48])
def test_decode_head_size(D, q_fmt, cache_fmt, H, Hk, P):
    say(f"decode D={D} {q_fmt}/{cache_fmt} H={H} Hk={Hk} P={P}")
    run_decode(16, q_fmt, cache_fmt, D, H, Hk, P)


@pytest.mark.parametrize("BS", [8, 32])
@pytest.mark.parametrize("D", HEAD_SIZES)
@pytest.mark.parametrize("q_fmt,cache_fmt", DTYPES)
def test_decode_head_size_block_size(BS, D, q_fmt, cache_fmt):
    say(f"decode D={D} BS={BS} {q_fmt}/{cache_fmt}")
    run_decode(BS, q_fmt, cache_fmt, D, 8, 2, 48)


@pytest.mark.parametrize("BS", [8, 16, 32])
@pytest.mark.parametrize("D", HEAD_SIZES)
@pytest.mark.parametrize("q_fmt,cache_fmt,H,Hk", [("f32", "f32", 4, 4), ("bf16", "bf16", 8, 2),
                                                  ("f16", "f16", 4, 4), ("f16", "fp8", 8, 2),
                                                  ("bf16", "fp8", 4, 4)])
def test_append_head_size(BS, D, q_fmt, cache_fmt, H, Hk):
    """Decode with append equals the writer (slots from the tables) followed by
    decode, bit for bit; lanes past the last row store nothing."""
    say(f"append D={D} BS={BS} {q_fmt}/{cache_fmt} H={H} Hk={Hk}")
    P = 48
    w = small(BS, q_fmt, cache_fmt, D, H, Hk, 5 * D + BS + H)
    dw = DeviceWorkload(w, DEV, P).fill()
    torch.cuda.synchronize()
    ka, va = dw.k_cache.clone(), dw.v_cache.clone()
    out_a = torch.full_like(dw.out, float("nan"))
    pkv.paged_attention_decode_append(out_a, dw.query, dw.key_new, dw.value_new, ka, va,
                                      dw.block_tables, dw.context_lens, w.scale, w.k_scale,
                                      w.v_scale, P, dw.workspace)
    dw.write_new()
    out_b = torch.full_like(dw.out, float("nan"))
    pkv.paged_attention_decode(out_b, dw.query, dw.k_cache, dw.v_cache, dw.block_tables,
                               dw.context_lens, w.scale, w.k_scale, w.v_scale, P, dw.workspace)
    torch.cuda.synchronize()
    for x, y, name in ((ka, dw.k_cache, "key cache"), (va, dw.v_cache, "value cache"),
                       (out_a, out_b, "output")):
        assert np.array_equal(tbits(x), tbits(y)), f"D={D} BS={BS}: {name} differs"
    kc, vc = host_pool(w)
    assert np.array_equal(tbits(ka), bits(kc))
    assert np.array_equal(tbits(va), bits(vc))


@pytest.mark.parametrize("D,q_fmt,cache_fmt,H,Hk", [(80, "f16", "f16", 16, 16),
                                                    (96, "bf16", "bf16", 32, 8),
                                                    (112, "bf16", "fp8", 28, 4),
                                                    (256, "bf16", "bf16", 16, 4),
                                                    (256, "f16", "fp8", 8, 1),
                                                    (192, "f32", "f32", 8, 8)])
def test_batch_head_size(D, q_fmt, cache_fmt, H, Hk):
    """A batch of 16 sequences of 128..4096 tokens (one and two default
    partitions) at the given head size: sampled sequences against the oracle."""
    say(f"batch D={D} {q_fmt}/{cache_fmt} H={H} Hk={Hk}: generating inputs")
    rng = np.random.default_rng(D + H)
    lens = rng.integers(128, 4097, size=16)
    fp8 = cache_fmt == "fp8"
    nb = int(np.sum(-(-lens // 16)))
    w = workloads.build("hd_batch", S=16, H=H, Hk=Hk, D=D, NB=nb + 64, q_fmt=q_fmt,
                        cache_fmt=cache_fmt, lens=lens, seed=D * 7 + H, block_size=16,
                        k_scale=6 / 448 if fp8 else 1.0, v_scale=6 / 448 if fp8 else 1.0)
    dw = DeviceWorkload(w, DEV).fill()
    dw.decode_append()
    torch.cuda.synchronize()
    gpu = dw.out_f64()
    assert np.isfinite(gpu).all()
    seqs = [0, 7, int(np.argmax(lens)), 15]
    cp = oracle.CompactPool(w, seqs)
    assert_close(gpu[seqs], cp.attention(w), fp8, f"batch D={D}")
