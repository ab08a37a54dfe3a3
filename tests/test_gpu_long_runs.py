"""Partitions longer than 4096 tokens, against the oracle.

A work item's run is split among its 4 waves, and each wave fetches its block
ids 64 table entries at a time.  Partitions of 4096 tokens or fewer never give
a wave more than 64 tiles; longer ones (8192 tokens, and one partition per
sequence) walk several 64-entry chunks per wave, on the vector kernel at
block sizes 8, 16 and 32 and on the matrix-core kernel with 16-bit caches
(32-token tiles at block sizes 8, 16 and 32) and FP8 caches (16-token steps,
whole blocks at 32), plain and with the new token appended in the same
call.  Lengths put
chunk and block edges at the ends of the runs."""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads.gpu import DeviceWorkload

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
LENS = np.array([20000, 4097, 16 * 64 * 4 + 1, 777, 16 * 64 * 8])


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("append", [False, True])
@pytest.mark.parametrize("P", [8192, 65536])
@pytest.mark.parametrize("BS,q_fmt,cache_fmt,H,Hk", [(16, "f16", "f16", 4, 4),
                                                     (8, "bf16", "bf16", 2, 2),
                                                     (32, "f16", "f16", 2, 2),
                                                     (8, "f16", "fp8", 2, 2),
                                                     (16, "bf16", "bf16", 8, 2),
                                                     (16, "bf16", "fp8", 8, 2),
                                                     (8, "f16", "f16", 8, 2),
                                                     (32, "bf16", "bf16", 8, 2),
                                                     (32, "bf16", "fp8", 8, 2)])
def test_runs_past_64_tiles_per_wave(BS, q_fmt, cache_fmt, H, Hk, P, append):
    say(f"long runs BS={BS} {q_fmt}/{cache_fmt} H={H} Hk={Hk} P={P} append={append}")
    fp8 = cache_fmt == "fp8"
    nb = int(np.sum(-(-LENS // BS)))
    w = workloads.build("longruns", S=len(LENS), H=H, Hk=Hk, D=128, NB=nb + 11, q_fmt=q_fmt,
                        cache_fmt=cache_fmt, lens=LENS, seed=BS * 7 + H + P % 1000,
                        block_size=BS, k_scale=0.03 if fp8 else 1.0,
                        v_scale=0.02 if fp8 else 1.0)
    dw = DeviceWorkload(w, DEV, P).fill()
    if append:
        dw.decode_append()
    else:
        dw.write_new()
        dw.decode()
    torch.cuda.synchronize()
    gpu = dw.out_f64()
    ref = oracle.CompactPool(w, list(range(len(LENS)))).attention(w)
    assert np.isfinite(gpu).all()
    bound = 5e-2 if fp8 else 2e-3 + 1e-2 * np.abs(ref)
    err = np.abs(gpu - ref)
    assert (err <= bound).all(), f"max error {err.max()}"
