"""Pins of the oracle's writer, gather and attention (CPU only).

Each test ties the oracle to something other than itself: the worked example
printed on a page, brute-force scalar loops, a library routine (torch SDPA),
closed forms, or invariants of the method.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN_TABLE = os.path.join(os.path.dirname(__file__), "golden",
                            "worked_example_block_table.txt")


# --------------------------------------------------------------------------- #
# small paged problems built by hand (any block size)
# --------------------------------------------------------------------------- #
def make_problem(seed, S, H, Hk, D, BS, lens, NB=None, fmt="f32", contiguous=False):
    rng = np.random.default_rng(seed)
    nbs = [-(-L // BS) for L in lens]
    NB = NB or (sum(nbs) + 3)
    ids = np.arange(NB) if contiguous else rng.permutation(NB)
    MB = max(1, max(nbs) if nbs else 1)
    bt = np.full((len(lens), MB), -1, np.int64)
    k_tok, v_tok = [], []
    pos = 0
    dt = workloads.np_storage_dtype(fmt)
    kc = np.full((NB, Hk, D, BS), np.nan, np.float32).astype(dt) if fmt != "bf16" else \
        np.full((NB, Hk, D, BS), 0x7FC0, np.uint16)
    vc = kc.copy()
    for s, L in enumerate(lens):
        bt[s, :nbs[s]] = ids[pos:pos + nbs[s]]
        pos += nbs[s]
        k = workloads.cast_f32(rng.standard_normal((L, Hk, D), dtype=np.float32), fmt)
        v = workloads.cast_f32(rng.standard_normal((L, Hk, D), dtype=np.float32), fmt)
        slots = np.array([bt[s, t // BS] * BS + t % BS for t in range(L)], np.int64)
        oracle.reshape_and_cache_ref(k, v, kc, vc, slots, fmt, fmt)
        k_tok.append(k)
        v_tok.append(v)
    q = workloads.cast_f32(rng.standard_normal((len(lens), H, D), dtype=np.float32), fmt)
    return dict(q=q, kc=kc, vc=vc, bt=bt, lens=np.array(lens), k_tok=k_tok, v_tok=v_tok,
                fmt=fmt, Hk=Hk, BS=BS)


def bits(a):
    return np.ascontiguousarray(a).view(np.uint8)


def run_ref(p, scale=0.3, **kw):
    return oracle.paged_attention_ref(p["q"], p["kc"], p["vc"], p["bt"], p["lens"], scale,
                                      p["fmt"], p["fmt"], **kw)


def brute_force(p, scale):
    """Pure-Python scalar loops straight from the definition: no numpy arithmetic."""
    q, kc, vc, bt, lens = p["q"].tolist(), p["kc"], p["vc"], p["bt"].tolist(), p["lens"]
    kc = oracle.to_float64(kc, p["fmt"]).tolist()
    vc = oracle.to_float64(vc, p["fmt"]).tolist()
    if p["fmt"] != "f32":
        q = oracle.to_float64(p["q"], p["fmt"]).tolist()
    S, H, D = len(q), len(q[0]), len(q[0][0])
    Hk, BS = p["Hk"], p["BS"]
    g = H // Hk
    out = [[[0.0] * D for _ in range(H)] for _ in range(S)]
    for s in range(S):
        L = int(lens[s])
        if L == 0:
            continue
        for h in range(H):
            kvh = h // g
            where = [(bt[s][t // BS], t % BS) for t in range(L)]
            x = []
            for b, o in where:
                acc = 0.0
                for d in range(D):
                    acc += q[s][h][d] * kc[b][kvh][d][o]
                x.append(scale * acc)
            m = max(x)
            e = [math.exp(v - m) for v in x]
            z = sum(e)
            for d in range(D):
                acc = 0.0
                for (b, o), w in zip(where, e):
                    acc += w * vc[b][kvh][d][o]
                out[s][h][d] = acc / z
    return np.array(out)


# --------------------------------------------------------------------------- #
# P9: brute force on tiny shapes, several block sizes and GQA factors
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("BS", [16, 2, 1])
@pytest.mark.parametrize("H,Hk", [(2, 2), (4, 2), (3, 1)])
def test_brute_force(BS, H, Hk):
    p = make_problem(11 + BS + H, S=3, H=H, Hk=Hk, D=8, BS=BS, lens=[1, 17, 40])
    ref = run_ref(p, 0.3)
    bf = brute_force(p, 0.3)
    np.testing.assert_allclose(ref, bf, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_brute_force_16bit_storage(fmt):
    p = make_problem(5, S=2, H=4, Hk=2, D=8, BS=16, lens=[23, 5], fmt=fmt)
    np.testing.assert_allclose(run_ref(p, 0.5), brute_force(p, 0.5), rtol=1e-12, atol=1e-13)


def test_brute_force_on_the_tiny_workload():
    w = workloads.make("tiny")
    kc = np.full((w.NB, w.Hk, w.D, 16), np.nan, np.float32)
    vc = kc.copy()
    oracle.reshape_and_cache_ref(w.key_bulk, w.value_bulk, kc, vc, w.slot_bulk, "f32", "f32")
    oracle.reshape_and_cache_ref(w.key_new, w.value_new, kc, vc, w.slot_new, "f32", "f32")
    p = dict(q=w.query, kc=kc, vc=vc, bt=w.block_tables, lens=w.context_lens, fmt="f32",
             Hk=w.Hk, BS=16)
    ref = oracle.paged_attention_ref(w.query, kc, vc, w.block_tables, w.context_lens,
                                     w.scale, "f32", "f32")
    assert np.isfinite(ref).all()
    np.testing.assert_allclose(ref, brute_force(p, w.scale), rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------- #
# P4 / P11: dense attention from a library routine
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("BS", [16, 1])
@pytest.mark.parametrize("H,Hk", [(4, 4), (8, 2)])
def test_identity_table_equals_torch_sdpa(BS, H, Hk):
    lens = [1, 15, 16, 17, 70]
    p = make_problem(3, S=len(lens), H=H, Hk=Hk, D=16, BS=BS, lens=lens, contiguous=True)
    scale = 0.25
    ref = run_ref(p, scale)
    for s, L in enumerate(lens):
        q = torch.from_numpy(p["q"][s].astype(np.float64)).view(1, H, 1, 16)
        k = torch.from_numpy(p["k_tok"][s].astype(np.float64)).permute(1, 0, 2)   # [Hk, L, D]
        v = torch.from_numpy(p["v_tok"][s].astype(np.float64)).permute(1, 0, 2)
        k = k.repeat_interleave(H // Hk, dim=0).unsqueeze(0)
        v = v.repeat_interleave(H // Hk, dim=0).unsqueeze(0)
        dense = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale)
        np.testing.assert_allclose(ref[s], dense[0, :, 0, :].numpy(), rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------- #
# closed forms (P1, P2, P3, P14) and softmax invariants (P7)
# --------------------------------------------------------------------------- #
def test_single_token_returns_its_value_exactly():
    p = make_problem(4, S=3, H=4, Hk=2, D=8, BS=16, lens=[1, 1, 1])
    ref = run_ref(p, 1.7)
    for s in range(3):
        for h in range(4):
            assert np.array_equal(ref[s, h], p["v_tok"][s][0, h // 2].astype(np.float64))


def test_zero_query_gives_mean_of_values():
    p = make_problem(6, S=2, H=2, Hk=2, D=8, BS=16, lens=[33, 7])
    p["q"][:] = 0
    ref = run_ref(p, 1.0)
    for s in range(2):
        np.testing.assert_allclose(ref[s], p["v_tok"][s].astype(np.float64).mean(0),
                                   rtol=1e-12, atol=1e-14)


def test_zero_scale_gives_mean_of_values():
    p = make_problem(8, S=1, H=2, Hk=1, D=8, BS=16, lens=[50])
    ref = run_ref(p, 0.0)
    mean = p["v_tok"][0].astype(np.float64).mean(0)       # [Hk, D]
    np.testing.assert_allclose(ref[0], np.repeat(mean, 2, axis=0), rtol=1e-12, atol=1e-14)


def test_constant_values_pass_through():
    p = make_problem(9, S=2, H=2, Hk=2, D=8, BS=16, lens=[20, 45])
    for s in range(2):
        for t in range(p["lens"][s]):
            b, o = p["bt"][s, t // 16], t % 16
            p["vc"][b, :, :, o] = 2.5
    ref = run_ref(p, 0.9)
    np.testing.assert_allclose(ref, 2.5, rtol=1e-14)


def test_one_dominant_logit():
    p = make_problem(10, S=1, H=1, Hk=1, D=8, BS=16, lens=[40])
    p["q"][:] = 0
    p["q"][0, 0, 0] = 1.0
    p["kc"][:, :, 0, :] = 0.0
    star = 23
    p["kc"][p["bt"][0, star // 16], 0, 0, star % 16] = 50.0
    ref = run_ref(p, 1.0)
    vstar = p["v_tok"][0][star, 0].astype(np.float64)
    bound = 39 * math.exp(-50.0) * 2 * np.abs(p["v_tok"][0]).max()
    assert np.abs(ref[0, 0] - vstar).max() <= bound + 1e-15


def test_softmax_weights_are_a_distribution():
    rng = np.random.default_rng(12)
    for L in (1, 2, 16, 300):
        k = rng.standard_normal((L, 32)) * 3
        q = rng.standard_normal(32) * 3
        w = oracle.softmax_weights_ref(q, k, 0.7)
        assert (w >= 0).all() and abs(w.sum() - 1.0) <= 1e-12
        # the largest score gets the largest weight
        assert np.argmax(w) == np.argmax(k @ q)


def test_empty_context_gives_zeros():
    p = make_problem(13, S=3, H=2, Hk=2, D=8, BS=16, lens=[5, 0, 9])
    ref = run_ref(p, 0.5)
    assert np.array_equal(ref[1], np.zeros((2, 8)))
    assert np.isfinite(ref).all()


def test_poison_outside_the_context_is_never_read():
    p = make_problem(14, S=2, H=2, Hk=1, D=8, BS=16, lens=[19, 3])
    ref = run_ref(p, 0.5)
    assert np.isfinite(ref).all()       # tail slots and unused blocks hold NaN


# --------------------------------------------------------------------------- #
# P5: physical placement does not matter; P6: sharing does not matter
# --------------------------------------------------------------------------- #
def test_physical_block_permutation_is_bit_invariant():
    p = make_problem(15, S=3, H=4, Hk=2, D=16, BS=16, lens=[5, 64, 100])
    ref = run_ref(p, 0.3)
    NB = p["kc"].shape[0]
    pi = np.random.default_rng(99).permutation(NB)
    kc2 = np.empty_like(p["kc"])
    vc2 = np.empty_like(p["vc"])
    kc2[pi] = p["kc"]
    vc2[pi] = p["vc"]
    bt2 = np.where(p["bt"] >= 0, pi[np.maximum(p["bt"], 0)], -1)
    ref2 = oracle.paged_attention_ref(p["q"], kc2, vc2, bt2, p["lens"], 0.3, "f32", "f32")
    assert np.array_equal(ref, ref2)


def test_shared_prefix_equals_private_copies():
    w = workloads.build("sp", S=8, H=8, Hk=2, D=16, NB=128, q_fmt="bf16", cache_fmt="bf16",
                        lens=np.array([1, 5, 16, 17, 3, 30, 2, 9]), seed=3,
                        prefix_tokens=64, n_samples=4)
    kc = np.full((w.NB, w.Hk, w.D, 16), 0x7FC0, np.uint16)
    vc = kc.copy()
    oracle.reshape_and_cache_ref(w.key_bulk, w.value_bulk, kc, vc, w.slot_bulk, "bf16", "bf16")
    oracle.reshape_and_cache_ref(w.key_new, w.value_new, kc, vc, w.slot_new, "bf16", "bf16")
    shared = oracle.paged_attention_ref(w.query, kc, vc, w.block_tables, w.context_lens,
                                        w.scale, "bf16", "bf16")
    # give every sample a private copy of its prefix blocks
    bt = w.block_tables.copy()
    used = set(int(b) for b in bt.ravel() if b >= 0)
    spare = [b for b in range(w.NB) if b not in used]
    for seqs, nblk in w.shared_groups:
        assert len(seqs) == 4 and nblk == 4
        for s in seqs[1:]:
            for j in range(nblk):
                nb_ = spare.pop()
                kc[nb_] = kc[bt[s, j]]
                vc[nb_] = vc[bt[s, j]]
                bt[s, j] = nb_
    private = oracle.paged_attention_ref(w.query, kc, vc, bt, w.context_lens, w.scale,
                                         "bf16", "bf16")
    assert np.array_equal(shared, private)


# --------------------------------------------------------------------------- #
# P8: partitioned computation and its merge
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("P", [16, 32, 512])
def test_partitioned_equals_unpartitioned(P):
    p = make_problem(16, S=4, H=4, Hk=2, D=16, BS=16, lens=[1, 31, 100, 257])
    ref = run_ref(p, 0.4)
    part = oracle.paged_attention_partitioned_ref(p["q"], p["kc"], p["vc"], p["bt"], p["lens"],
                                                  0.4, "f32", "f32", partition_size=P)
    np.testing.assert_allclose(part, ref, rtol=1e-12, atol=1e-14)
    # trailing partitions that hold no token contribute nothing
    part2 = oracle.paged_attention_partitioned_ref(p["q"], p["kc"], p["vc"], p["bt"],
                                                   p["lens"], 0.4, "f32", "f32",
                                                   partition_size=P,
                                                   num_partitions=-(-257 // P) + 2)
    np.testing.assert_allclose(part2, ref, rtol=1e-12, atol=1e-14)


def test_partitioned_large_logits():
    p = make_problem(17, S=1, H=1, Hk=1, D=8, BS=16, lens=[200])
    p["q"] *= 40.0
    ref = run_ref(p, 1.0)
    assert np.isfinite(ref).all()
    part = oracle.paged_attention_partitioned_ref(p["q"], p["kc"], p["vc"], p["bt"], p["lens"],
                                                  1.0, "f32", "f32", partition_size=32)
    np.testing.assert_allclose(part, ref, rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------- #
# P10: the worked example printed on the page; P13: writer invariants
# --------------------------------------------------------------------------- #
def _golden_table():
    rows = []
    with open(GOLDEN_TABLE) as f:
        for line in f:
            line = line.split("#")[0].split()
            if line:
                rows.append((int(line[0]), int(line[1])))
    return rows


def test_worked_example_gather_order():
    rows = _golden_table()
    assert rows == [(0, 7), (1, 3), (2, 9)]
    NB, Hk, D, BS = 10, 2, 4, 16
    cache = np.zeros((NB, Hk, D, BS), np.float32)
    for b in range(NB):
        cache[b] = b                                   # every element names its block
    table = np.array([phys for _, phys in rows])
    L = 3 * BS - 5
    got = oracle.gather_ref(cache, table, L)           # [Hk, L, D]
    assert got.shape == (Hk, L, D)
    expect_blocks = [phys for _, phys in rows for _ in range(BS)][:L]
    assert np.array_equal(got[0, :, 0], np.array(expect_blocks, np.float32))


def test_gather_reads_token_axis_last():
    NB, Hk, D, BS = 4, 2, 3, 16
    cache = np.arange(NB * Hk * D * BS, dtype=np.float32).reshape(NB, Hk, D, BS)
    got = oracle.gather_ref(cache, np.array([2, 0]), 20)
    for t in range(20):
        b = [2, 0][t // BS]
        for h in range(Hk):
            for d in range(D):
                assert got[h, t, d] == cache[b, h, d, t % BS]


@pytest.mark.parametrize("fmt,cache_fmt", [("f32", "f32"), ("f16", "f16"), ("bf16", "bf16"),
                                           ("bf16", "fp8"), ("f16", "fp8")])
def test_writer_round_trip_and_untouched_slots(fmt, cache_fmt):
    rng = np.random.default_rng(21)
    NB, Hk, D, BS, T = 8, 2, 4, 16, 40
    cdt = workloads.np_storage_dtype(cache_fmt)
    kc = rng.integers(0, 256, size=(NB, Hk, D, BS * np.dtype(cdt).itemsize),
                      dtype=np.uint8).view(cdt)
    vc = rng.integers(0, 256, size=kc.shape[:3] + (BS * np.dtype(cdt).itemsize,),
                      dtype=np.uint8).view(cdt)
    k0, v0 = kc.copy(), vc.copy()
    slots = rng.choice(NB * BS, size=T, replace=False).astype(np.int64)
    slots[3] = -1                    # skipped
    slots[7] = NB * BS + 5           # skipped (outside the pool)
    key = workloads.cast_f32(rng.standard_normal((T, Hk, D), dtype=np.float32), fmt)
    val = workloads.cast_f32(rng.standard_normal((T, Hk, D), dtype=np.float32), fmt)
    oracle.reshape_and_cache_ref(key, val, kc, vc, slots, fmt, cache_fmt, 0.05, 0.07)
    written = np.zeros((NB, BS), bool)
    for i, s in enumerate(slots):
        if 0 <= s < NB * BS:
            b, o = divmod(int(s), BS)
            written[b, o] = True
            if cache_fmt == fmt:
                assert np.array_equal(bits(kc[b, :, :, o]), bits(key[i]))
                assert np.array_equal(bits(vc[b, :, :, o]), bits(val[i]))
            else:
                kx = oracle.to_float32(key[i], fmt)
                back = oracle.decode_e4m3(kc[b, :, :, o]) * 0.05
                assert np.all(np.abs(back - kx) <= np.maximum(np.abs(kx) * 2.0 ** -4,
                                                              2.0 ** -10 * 0.05) + 1e-12)
    for b in range(NB):
        for o in range(BS):
            if not written[b, o]:
                assert np.array_equal(bits(kc[b, :, :, o]), bits(k0[b, :, :, o]))
                assert np.array_equal(bits(vc[b, :, :, o]), bits(v0[b, :, :, o]))


def test_workload_write_then_gather_round_trip():
    w = workloads.build("rt", S=5, H=4, Hk=2, D=8, NB=40, q_fmt="f16", cache_fmt="f16",
                        lens=np.array([1, 16, 17, 60, 33]), seed=4)
    kc = np.full((w.NB, w.Hk, w.D, 16), np.nan, np.float16)
    vc = kc.copy()
    oracle.reshape_and_cache_ref(w.key_bulk, w.value_bulk, kc, vc, w.slot_bulk, "f16", "f16")
    oracle.reshape_and_cache_ref(w.key_new, w.value_new, kc, vc, w.slot_new, "f16", "f16")
    # every sequence's logical tokens come back in order; bulk tokens are stored
    # sequence after sequence, the decode-step token last
    off = 0
    for s in range(w.S):
        L = int(w.context_lens[s])
        got = oracle.gather_ref(kc, w.block_tables[s], L)          # [Hk, L, D]
        expect = np.concatenate([w.key_bulk[off:off + L - 1], w.key_new[s:s + 1]])
        off += L - 1
        assert np.array_equal(got.transpose(1, 0, 2), expect)


def test_allocator_invariants_and_exhaustion():
    a = workloads.BlockAllocator(np.random.default_rng(0).permutation(10))
    x = a.allocate(4)
    y = a.fork(x)
    z = a.allocate(3)
    a.check(10)
    a.release(x)
    a.check(10)
    assert all(a.ref[b] == 1 for b in y)
    a.release(y)
    a.release(z)
    a.check(10)
    assert len(a.free) == 10
    with pytest.raises(MemoryError):
        a.allocate(11)


# --------------------------------------------------------------------------- #
# copy-on-write block copy
# --------------------------------------------------------------------------- #
def test_copy_blocks_then_repoint_keeps_logical_kv():
    p = make_problem(30, S=2, H=2, Hk=2, D=8, BS=16, lens=[40, 20], NB=12)
    ref = run_ref(p, 0.3)
    used = set(int(b) for b in p["bt"].ravel() if b >= 0)
    free = [b for b in range(12) if b not in used]
    pairs = [(int(p["bt"][0, 1]), free[0]), (int(p["bt"][1, 0]), free[1])]
    k0, v0 = p["kc"].copy(), p["vc"].copy()
    oracle.copy_blocks_ref(p["kc"], p["vc"], pairs)
    for src, dst in pairs:
        assert np.array_equal(bits(p["kc"][dst]), bits(k0[src]))
        assert np.array_equal(bits(p["vc"][dst]), bits(v0[src]))
    others = [b for b in range(12) if b not in (free[0], free[1])]
    assert np.array_equal(bits(p["kc"][others]), bits(k0[others]))
    p["bt"][0, 1] = free[0]
    p["bt"][1, 0] = free[1]
    assert np.array_equal(run_ref(p, 0.3), ref)


# --------------------------------------------------------------------------- #
# the compact-pool reference used for sampled checks of full-size workloads
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("cache_fmt", ["bf16", "fp8"])
def test_compact_pool_matches_full_pool(cache_fmt):
    w = workloads.build("cp", S=6, H=8, Hk=2, D=16, NB=60, q_fmt="bf16", cache_fmt=cache_fmt,
                        lens=np.array([3, 40, 1, 77, 16, 20]), seed=8,
                        k_scale=0.05 if cache_fmt == "fp8" else 1.0,
                        v_scale=0.07 if cache_fmt == "fp8" else 1.0)
    dt = workloads.np_storage_dtype(cache_fmt)
    kc = np.full((w.NB, w.Hk, w.D, 16), 0x7FC0 if cache_fmt == "bf16" else 0x7F, dt)
    vc = kc.copy()
    for keys, vals, slots in ((w.key_bulk, w.value_bulk, w.slot_bulk),
                              (w.key_new, w.value_new, w.slot_new)):
        oracle.reshape_and_cache_ref(keys, vals, kc, vc, slots, "bf16", cache_fmt,
                                     w.k_scale, w.v_scale)
    full = oracle.paged_attention_ref(w.query, kc, vc, w.block_tables, w.context_lens, w.scale,
                                      "bf16", cache_fmt, w.k_scale, w.v_scale)
    seqs = [4, 1, 3]
    cp = oracle.CompactPool(w, seqs)
    assert np.array_equal(cp.attention(w), full[seqs])
    # the compact pool holds exactly the chosen sequences' blocks
    for i, s in enumerate(seqs):
        nb = -(-int(w.context_lens[s]) // 16)
        for j in range(nb):
            assert np.array_equal(bits(cp.k[cp.tables[i, j]]), bits(kc[w.block_tables[s, j]]))
