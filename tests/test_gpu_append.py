"""paged_attention_decode_append: a whole decode step in one call.

Its caches must equal, bit for bit, those left by reshape_and_cache (slots
taken from the block tables) followed by paged_attention_decode on the same
inputs, and so must its output (the same arithmetic on the same bits); the
output is also checked against the oracle over the oracle's own pool
(|gpu - ref| <= 2e-3 + 1e-2 |ref|, or 5e-2 for FP8 caches)."""
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
LENS = np.array([1, 7, 8, 9, 15, 16, 17, 31, 32, 33, 100, 0, 257, 520])


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def table_slots(bt, lens, bs, nb):
    """Slot of each sequence's position L - 1 from its block table; -1 for none."""
    mb = bt.shape[1]
    out = np.full(len(lens), -1, np.int64)
    for s, L in enumerate(int(x) for x in lens):
        if 1 <= L <= mb * bs:
            b = int(bt[s, (L - 1) // bs])
            if 0 <= b < nb:
                out[s] = b * bs + (L - 1) % bs
    return out


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


def both_paths(w, P, edit=None):
    """(appended caches, output) and (writer + decode caches, output) from one filled pool;
    edit(dw) may change the device tables / lengths first."""
    dw = DeviceWorkload(w, DEV, P).fill()
    if edit is not None:
        edit(dw)
    torch.cuda.synchronize()
    ka, va = dw.k_cache.clone(), dw.v_cache.clone()
    out_a = torch.full_like(dw.out, float("nan"))
    pkv.paged_attention_decode_append(out_a, dw.query, dw.key_new, dw.value_new, ka, va,
                                      dw.block_tables, dw.context_lens, w.scale, w.k_scale,
                                      w.v_scale, P, dw.workspace)
    slots = table_slots(dw.block_tables.cpu().numpy(), dw.context_lens.cpu().numpy(), w.BS, w.NB)
    pkv.reshape_and_cache(dw.key_new, dw.value_new, dw.k_cache, dw.v_cache,
                          torch.from_numpy(slots).to(DEV), w.k_scale, w.v_scale)
    out_b = torch.full_like(dw.out, float("nan"))
    pkv.paged_attention_decode(out_b, dw.query, dw.k_cache, dw.v_cache, dw.block_tables,
                               dw.context_lens, w.scale, w.k_scale, w.v_scale, P, dw.workspace)
    torch.cuda.synchronize()
    return (ka, va, out_a), (dw.k_cache, dw.v_cache, out_b), slots


def bits(t):
    return t.contiguous().view(torch.uint8).cpu().numpy()


def check_same(a, b, what):
    for x, y, name in zip(a, b, ("key cache", "value cache", "output")):
        assert np.array_equal(bits(x), bits(y)), f"{what}: {name} differs"


def small(BS, q_fmt, cache_fmt, D, H, Hk, seed):
    fp8 = cache_fmt == "fp8"
    nb = int(np.sum(-(-LENS // BS)))
    return workloads.build("append", S=len(LENS), H=H, Hk=Hk, D=D, NB=nb + 9, q_fmt=q_fmt,
                           cache_fmt=cache_fmt, lens=LENS, seed=seed, block_size=BS,
                           k_scale=0.02 if fp8 else 1.0, v_scale=0.03 if fp8 else 1.0)


DTYPES = [("f32", "f32"), ("f16", "f16"), ("bf16", "bf16"), ("f16", "fp8"), ("bf16", "fp8")]


@pytest.mark.parametrize("BS", [8, 16, 32])
@pytest.mark.parametrize("q_fmt,cache_fmt", DTYPES)
@pytest.mark.parametrize("H,Hk", [(4, 4), (32, 1), (8, 2)])
@pytest.mark.parametrize("P", [0, 48])
def test_append_equals_writer_then_decode(BS, q_fmt, cache_fmt, H, Hk, P):
    """MHA and 32 heads per KV head: the vector kernel stores the token; 4 heads per
    KV head at block size 16 with a 16-bit query: the matrix-core path, writer first."""
    say(f"append BS={BS} {q_fmt}/{cache_fmt} H={H} Hk={Hk} P={P}")
    D = 64 if H == 32 else 128
    w = small(BS, q_fmt, cache_fmt, D, H, Hk, BS + H + P)
    a, b, slots = both_paths(w, P)
    assert np.array_equal(slots, w.slot_new)
    check_same(a, b, f"BS={BS}")
    kc, vc = host_pool(w)
    assert np.array_equal(bits(a[0]), np.ascontiguousarray(kc).view(np.uint8))
    assert np.array_equal(bits(a[1]), np.ascontiguousarray(vc).view(np.uint8))
    ref = oracle.paged_attention_ref(w.query, kc, vc, w.block_tables, w.context_lens, w.scale,
                                     q_fmt, cache_fmt, w.k_scale, w.v_scale)
    gpu = a[2].float().cpu().numpy().astype(np.float64)
    assert np.isfinite(gpu).all()
    bound = 5e-2 if cache_fmt == "fp8" else 2e-3 + 1e-2 * np.abs(ref)
    assert (np.abs(gpu - ref) <= bound).all(), np.abs(gpu - ref).max()


@pytest.mark.parametrize("BS", [8, 16, 32])
@pytest.mark.parametrize("q_fmt,cache_fmt,H,Hk", [("f16", "f16", 4, 4), ("bf16", "fp8", 4, 4),
                                                  ("bf16", "bf16", 8, 2)])
def test_append_without_a_slot(BS, q_fmt, cache_fmt, H, Hk):
    """A table entry outside the pool at position L - 1, or a length past the table:
    no token is stored (as the writer skips such slots) and both paths still agree."""
    say(f"append without slot BS={BS} {q_fmt}/{cache_fmt} H={H} Hk={Hk}")
    w = small(BS, q_fmt, cache_fmt, 128, H, Hk, 7 * BS + H)

    def edit(dw):
        lens = dw.context_lens.cpu().numpy()
        s1 = int(np.flatnonzero(lens == 100)[0])
        dw.block_tables[s1, (100 - 1) // BS] = w.NB + 3          # outside the pool
        s2 = int(np.flatnonzero(lens == 33)[0])
        dw.context_lens[s2] = w.MB * BS + 5                      # past the table

    a, b, slots = both_paths(w, 0, edit)
    assert (slots < 0).sum() >= 3                                # those two and L = 0
    check_same(a, b, f"BS={BS}")


@pytest.mark.parametrize("name", ["llama7b_b64", "fp8_mixed"])
def test_append_full_size(name):
    """The LLaMA-7B batch (vector kernel) and the FP8 batch (matrix cores, writer
    first): caches and outputs of the two paths equal at full size."""
    say(f"append full size {name}")
    w = workloads.make(name)
    a, b, _ = both_paths(w, 0)
    check_same(a, b, name)
