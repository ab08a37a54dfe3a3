"""A seeded random sweep over the decode calls' option space, each case
against the oracle: head size x block size x dtype pair x query heads per KV
head x partition size x packed or row-strided tensors x plain or with
append, on random lengths (0, 1 and block edges included) and a shuffled
pool.  Decode is within |gpu - ref| <= 2e-3 + 1e-2 |ref| (16/32-bit caches)
or 5e-2 (FP8) of the oracle; with append the caches are bit-equal to the
oracle's pool and the output bit-equal to the writer followed by decode."""
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
HEAD_SIZES = [32, 64, 80, 96, 112, 120, 128, 192, 256]
DTYPES = [("f32", "f32"), ("f16", "f16"), ("bf16", "bf16"), ("f16", "fp8"), ("bf16", "fp8")]
GROUPS = [1, 1, 2, 4, 4, 8, 16, 20]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def tbits(t):
    return t.contiguous().view(torch.uint8).cpu().numpy()


def case(seed):
    rng = np.random.default_rng(4000 + seed)
    D = int(rng.choice(HEAD_SIZES))
    q_fmt, cache_fmt = DTYPES[int(rng.integers(len(DTYPES)))]
    BS = int(rng.choice([8, 16, 16, 32]))
    g = int(rng.choice(GROUPS))
    Hk = int(rng.integers(1, 4))
    S = int(rng.integers(1, 7))
    edges = [0, 1, BS - 1, BS, BS + 1, 2 * BS, 16 * 3 + 1]
    lens = np.array([int(rng.choice(edges)) if rng.random() < 0.4 else int(rng.integers(1, 700))
                     for _ in range(S)])
    P = int(rng.choice([0, 16, 48, 128]))
    strided = bool(rng.random() < 0.4)
    append = bool(rng.random() < 0.5)
    return dict(D=D, q_fmt=q_fmt, cache_fmt=cache_fmt, BS=BS, H=g * Hk, Hk=Hk, lens=lens, P=P,
                strided=strided, append=append, seed=seed)


def widen(t, pad):
    """A row-strided copy of t [N, A, D]: rows of A*D + pad elements."""
    n = t.shape[0]
    buf = torch.full((n, t.shape[1] * t.shape[2] + pad), float("nan"), dtype=t.dtype,
                     device=t.device)
    buf[:, :t.shape[1] * t.shape[2]] = t.reshape(n, -1)
    return buf[:, :t.shape[1] * t.shape[2]].view(t.shape)


@pytest.mark.parametrize("seed", range(80))
def test_random_case(seed):
    c = case(seed)
    say(f"sweep {seed}: D={c['D']} {c['q_fmt']}/{c['cache_fmt']} BS={c['BS']} H={c['H']} "
        f"Hk={c['Hk']} lens={list(c['lens'])} P={c['P']} strided={c['strided']} "
        f"append={c['append']}")
    fp8 = c["cache_fmt"] == "fp8"
    lens = c["lens"]
    nb = int(np.sum(-(-lens // c["BS"])))
    w = workloads.build("sweep", S=len(lens), H=c["H"], Hk=c["Hk"], D=c["D"], NB=nb + 7,
                        q_fmt=c["q_fmt"], cache_fmt=c["cache_fmt"], lens=lens, seed=c["seed"],
                        block_size=c["BS"], k_scale=0.03 if fp8 else 1.0,
                        v_scale=0.02 if fp8 else 1.0)
    P = c["P"]
    dw = DeviceWorkload(w, DEV, P).fill()
    q, kn, vn = dw.query, dw.key_new, dw.value_new
    out = torch.full_like(dw.out, float("nan"))
    if c["strided"]:
        q, kn, vn = widen(q, 8), widen(kn, 16), widen(vn, 24)
        out = widen(out, 8)
    if c["append"]:
        kc, vc = dw.k_cache.clone(), dw.v_cache.clone()
        pkv.paged_attention_decode_append(out, q, kn, vn, kc, vc, dw.block_tables,
                                          dw.context_lens, w.scale, w.k_scale, w.v_scale, P,
                                          dw.workspace)
        dw.write_new()
        ref_out = torch.full_like(dw.out, float("nan"))
        pkv.paged_attention_decode(ref_out, dw.query, dw.k_cache, dw.v_cache, dw.block_tables,
                                   dw.context_lens, w.scale, w.k_scale, w.v_scale, P,
                                   dw.workspace)
        torch.cuda.synchronize()
        assert np.array_equal(tbits(kc), tbits(dw.k_cache)), "key cache"
        assert np.array_equal(tbits(vc), tbits(dw.v_cache)), "value cache"
        assert np.array_equal(tbits(out), tbits(ref_out)), "output vs writer + decode"
    else:
        dw.write_new()
        pkv.paged_attention_decode(out, q, dw.k_cache, dw.v_cache, dw.block_tables,
                                   dw.context_lens, w.scale, w.k_scale, w.v_scale, P,
                                   dw.workspace)
        torch.cuda.synchronize()
    dt = workloads.np_storage_dtype(w.cache_fmt)
    poison = {"f32": np.nan, "f16": np.nan, "bf16": 0x7FC0, "fp8": 0x7F}[w.cache_fmt]
    kc_h = np.full((w.NB, w.Hk, w.D, w.BS), poison, dtype=dt)
    vc_h = kc_h.copy()
    for keys, vals, slots in ((w.key_bulk, w.value_bulk, w.slot_bulk),
                              (w.key_new, w.value_new, w.slot_new)):
        oracle.reshape_and_cache_ref(keys, vals, kc_h, vc_h, slots, w.src_fmt, w.cache_fmt,
                                     w.k_scale, w.v_scale)
    assert np.array_equal(tbits(dw.k_cache), np.ascontiguousarray(kc_h).view(np.uint8))
    ref = oracle.paged_attention_ref(w.query, kc_h, vc_h, w.block_tables, w.context_lens,
                                     w.scale, w.q_fmt, w.cache_fmt, w.k_scale, w.v_scale)
    gpu = out.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(gpu).all()
    bound = 5e-2 if fp8 else 2e-3 + 1e-2 * np.abs(ref)
    err = np.abs(gpu - ref)
    assert (err <= bound).all(), f"max error {err.max()}"
    assert np.array_equal(gpu[lens == 0], np.zeros_like(gpu[lens == 0]))
