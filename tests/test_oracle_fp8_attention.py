"""Pins of the oracle's attention over FP8 caches (CPU only).

paged_attention_ref decodes stored E4M3 codes and multiplies keys by k_scale
and values by v_scale (TGI PagedAttention 深度解析 §4.1: the KV writer stores
FP8-quantised keys and values; the read side undoes the per-tensor scale).
These tests tie that path to things other than the oracle itself:

* a pure-Python scalar loop straight from the definition of attention, with
  every code decoded by torch's float8_e4m3fn dtype (a library routine, not
  the oracle's codec table), at k_scale != v_scale != 1;
* closed forms: one cached token gives exactly decode(code) * v_scale;
  a zero query gives the mean of the decoded values times v_scale;
  (scale s, k_scale 2) gives the same bits as (scale 2s, k_scale 1);
  doubling v_scale doubles the output exactly;
* discrimination: the same brute force with the scales swapped, or with a
  scale applied as a divide, disagrees with the oracle, so those mistakes
  cannot pass the pins above.
"""
import math

import numpy as np
import pytest
import torch

import oracle

FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)


def lib_decode(codes):
    """Exact values of E4M3FN codes by torch's float8_e4m3fn (float64 result)."""
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def fp8_problem(seed, S, H, Hk, D, BS, lens, code_pool=FINITE):
    """Random finite codes in the used slots, the NaN code 0x7F everywhere
    else (tails of last blocks, unused blocks), random physical placement."""
    rng = np.random.default_rng(seed)
    nbs = [-(-L // BS) for L in lens]
    NB = sum(nbs) + 3
    ids = rng.permutation(NB)
    MB = max(1, max(nbs))
    bt = np.full((S, MB), -1, np.int64)
    kc = np.full((NB, Hk, D, BS), 0x7F, np.uint8)
    vc = kc.copy()
    pos = 0
    for s, L in enumerate(lens):
        bt[s, :nbs[s]] = ids[pos:pos + nbs[s]]
        pos += nbs[s]
        for t in range(L):
            b, o = bt[s, t // BS], t % BS
            kc[b, :, :, o] = rng.choice(code_pool, size=(Hk, D))
            vc[b, :, :, o] = rng.choice(code_pool, size=(Hk, D))
    q = rng.standard_normal((S, H, D)).astype(np.float32)
    q16 = torch.from_numpy(q).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return dict(q=q16, kc=kc, vc=vc, bt=bt, lens=np.array(lens), Hk=Hk, BS=BS)


def bf16_values(bits16):
    """Exact float64 values of bf16 bit patterns, by torch's bfloat16 dtype."""
    t = torch.from_numpy(np.ascontiguousarray(bits16).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def brute_force_fp8(p, scale, k_scale, v_scale, k_op=None, v_op=None):
    """Scalar loops: x_t = scale * sum_d q_d * (dec(K_t,d) k_scale), softmax over
    t < L, out_d = sum_t w_t * dec(V_t,d) v_scale.  k_op / v_op replace the
    'multiply by the scale' step (to show that mistakes there are caught)."""
    k_op = k_op or (lambda x, s: x * s)
    v_op = v_op or (lambda x, s: x * s)
    q = bf16_values(p["q"]).tolist()
    kd = lib_decode(p["kc"]).tolist()
    vd = lib_decode(p["vc"]).tolist()
    bt = p["bt"].tolist()
    Hk, BS = p["Hk"], p["BS"]
    S, H, D = len(q), len(q[0]), len(q[0][0])
    g = H // Hk
    out = [[[0.0] * D for _ in range(H)] for _ in range(S)]
    for s in range(S):
        L = int(p["lens"][s])
        if L == 0:
            continue
        where = [(bt[s][t // BS], t % BS) for t in range(L)]
        for h in range(H):
            c = h // g
            x = []
            for b, o in where:
                acc = 0.0
                for d in range(D):
                    acc += q[s][h][d] * k_op(kd[b][c][d][o], k_scale)
                x.append(scale * acc)
            m = max(x)
            e = [math.exp(v - m) for v in x]
            z = sum(e)
            for d in range(D):
                acc = 0.0
                for (b, o), wt in zip(where, e):
                    acc += wt * v_op(vd[b][c][d][o], v_scale)
                out[s][h][d] = acc / z
    return np.array(out)


def run_oracle(p, scale, k_scale, v_scale):
    return oracle.paged_attention_ref(p["q"], p["kc"], p["vc"], p["bt"], p["lens"], scale,
                                      "bf16", "fp8", k_scale, v_scale)


# small codes keep the logits in a range where the scales visibly matter
SMALL_CODES = np.array([c for c in FINITE if abs(oracle.e4m3_value_of_code(int(c))) <= 4.0],
                       np.uint8)


@pytest.mark.parametrize("BS", [16, 2])
@pytest.mark.parametrize("H,Hk", [(2, 2), (4, 2), (3, 1)])
def test_fp8_brute_force(BS, H, Hk):
    p = fp8_problem(40 + BS + H, S=3, H=H, Hk=Hk, D=8, BS=BS, lens=[1, 19, 37],
                    code_pool=SMALL_CODES)
    scale, ks, vs = 0.31, 0.37, 2.9
    ref = run_oracle(p, scale, ks, vs)
    bf = brute_force_fp8(p, scale, ks, vs)
    assert np.isfinite(ref).all()
    np.testing.assert_allclose(ref, bf, rtol=1e-12, atol=1e-13)


def test_fp8_brute_force_catches_scale_mistakes():
    """Swapped scales, a scale applied as a divide, or a missing scale each
    move the result far outside the brute-force tolerance above."""
    p = fp8_problem(7, S=2, H=4, Hk=2, D=8, BS=16, lens=[23, 40], code_pool=SMALL_CODES)
    scale, ks, vs = 0.31, 0.37, 2.9
    ref = run_oracle(p, scale, ks, vs)
    wrong = {
        "swapped": brute_force_fp8(p, scale, vs, ks),
        "k divide": brute_force_fp8(p, scale, ks, vs, k_op=lambda x, s: x / s),
        "v divide": brute_force_fp8(p, scale, ks, vs, v_op=lambda x, s: x / s),
        "no k scale": brute_force_fp8(p, scale, 1.0, vs),
        "no v scale": brute_force_fp8(p, scale, ks, 1.0),
    }
    for what, bad in wrong.items():
        assert np.abs(bad - ref).max() > 1e-3, what


def test_fp8_one_token_is_the_decoded_value_times_v_scale():
    """L = 1: softmax of one score is 1, so out = dec(V code) * v_scale exactly,
    whatever k_scale, for all 254 finite codes."""
    Hk, D, H = 2, 127, 4
    vcodes = FINITE.reshape(Hk, D)
    p = fp8_problem(3, S=1, H=H, Hk=Hk, D=D, BS=16, lens=[1])
    b = p["bt"][0, 0]
    p["vc"][b, :, :, 0] = vcodes
    for ks, vs in ((0.5, 3.0), (7.0, 0.013), (1.0, 1.0)):
        out = run_oracle(p, 0.2, ks, vs)
        expect = lib_decode(vcodes) * vs
        assert np.array_equal(out[0], np.repeat(expect, H // Hk, axis=0)), (ks, vs)


def test_fp8_zero_query_gives_mean_times_v_scale():
    """q = 0: every score is 0, the weights are uniform, out = mean_t dec(V) v_scale."""
    p = fp8_problem(9, S=2, H=2, Hk=1, D=16, BS=16, lens=[5, 33])
    p["q"][...] = 0
    out = run_oracle(p, 0.7, 3.0, 0.25)
    for s, L in enumerate(p["lens"]):
        v = np.stack([lib_decode(p["vc"][p["bt"][s, t // 16], 0, :, t % 16]) for t in range(L)])
        np.testing.assert_allclose(out[s, 0], v.mean(0) * 0.25, rtol=1e-13, atol=1e-15)


def test_fp8_k_scale_folds_into_the_score_scale():
    """k_scale multiplies every key, so (scale s, k_scale 2) and (scale 2s,
    k_scale 1) give the same float64 scores (power-of-two factors are exact)
    and the same output bits; a k_scale of 1 and a non-trivial one differ."""
    p = fp8_problem(11, S=3, H=4, Hk=2, D=16, BS=16, lens=[2, 17, 50])
    a = run_oracle(p, 0.3, 2.0, 0.7)
    b = run_oracle(p, 0.6, 1.0, 0.7)
    assert np.array_equal(a, b)
    assert np.abs(run_oracle(p, 0.3, 1.0, 0.7) - a).max() > 1e-6


def test_fp8_v_scale_scales_the_output():
    """Doubling v_scale doubles every output element exactly."""
    p = fp8_problem(12, S=3, H=4, Hk=4, D=8, BS=2, lens=[3, 9, 30])
    a = run_oracle(p, 0.4, 0.9, 0.75)
    b = run_oracle(p, 0.4, 0.9, 1.5)
    assert np.array_equal(2.0 * a, b)


def test_fp8_masked_tail_codes_do_not_matter():
    """NaN codes past L in the last block never reach the output; other
    finite codes there give the same bits."""
    p = fp8_problem(13, S=2, H=2, Hk=2, D=8, BS=16, lens=[5, 20])
    a = run_oracle(p, 0.5, 0.6, 0.8)
    assert np.isfinite(a).all()
    for s, L in enumerate(p["lens"]):
        b = p["bt"][s, (L - 1) // 16]
        p["kc"][b, :, :, L % 16:] = 0x38
        p["vc"][b, :, :, L % 16:] = 0x38
    assert np.array_equal(run_oracle(p, 0.5, 0.6, 0.8), a)
