"""Benchmark of one decode step on one MI355X: append each sequence's new token
with reshape_and_cache, then paged_attention_decode over the whole batch.

    python bench.py [--steps K] [--warmup W] [--workload llama7b_b64] [--partition P]

Prints ONE JSON line.  `value` is the step's algorithmic HBM bytes (decode: K
and V of every cached (token, KV head) once, q in and out, the used block-table
entries and lengths; writer: new K/V read + written) divided by the measured
time per step, inputs resident in HBM.  `roofline` is for the decode call (its
partition kernel and, when a sequence spans several partitions, the merge
kernel), timed with HIP events on the launch stream.  `cpu_baseline` times the
float64 oracle on a bounded sample of the same workload on the host.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama7b_b64")
    ap.add_argument("--partition", type=int, default=0, help="tokens per partition (0: default)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate budget of the oracle timing (0 disables it)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy 3 times (reference for the "
                         "FETCH_SIZE / WRITE_SIZE counters) and exit")
    return ap.parse_args()


def copy_calibration():
    """A plain copy of known size: its counter readings scale the decode's."""
    import torch
    n = 1 << 30
    x = torch.ones(n // 2, dtype=torch.float16, device="cuda:0")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n,
                      "launches": 3}), flush=True)


def cpu_baseline(w, budget_s):
    """Time the oracle (writer for the step's new tokens + attention) on whole
    sequences of the workload until about budget_s seconds have been spent."""
    import oracle
    from threadpoolctl import threadpool_limits
    rng = np.random.default_rng(0)
    order = rng.permutation(w.S)
    done, t_oracle, nbytes, seq_heads = [], 0.0, 0, 0
    e_kv = w.kv_elem_bytes()
    e_q = w.q_elem_bytes()
    passes = 0
    with threadpool_limits(limits=1):
        while t_oracle < budget_s and passes < 20:
            passes += 1
            for s in order:
                cp = oracle.CompactPool(w, [int(s)])      # setup: not timed
                kn = w.key_new[s:s + 1]
                vn = w.value_new[s:s + 1]
                sl = w.slot_new[s:s + 1]
                slot_c = np.where(sl >= 0, cp.remap[np.maximum(sl, 0) // 16] * 16 + sl % 16, -1)
                t0 = time.perf_counter()
                oracle.reshape_and_cache_ref(kn, vn, cp.k, cp.v, slot_c, w.src_fmt, w.cache_fmt,
                                             w.k_scale, w.v_scale)
                cp.attention(w)
                t_oracle += time.perf_counter() - t0
                L = int(w.context_lens[s])
                nbytes += (L * w.Hk * w.D * 2 * e_kv + w.H * w.D * 2 * e_q
                           + (-(-L // 16)) * 4 + 4)
                seq_heads += w.H
                done.append(int(s))
                if t_oracle >= budget_s:
                    break
    return {"value": round(nbytes / t_oracle / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "seq_heads_per_s": round(seq_heads / t_oracle, 2),
            "sample": f"{len(done)} sequence passes over {len(set(done))} of the {w.S} "
                      f"sequences of the same workload ({seq_heads} (sequence, head) pairs): "
                      f"writer for the decode token + attention, float64 numpy, 1 thread, "
                      f"{t_oracle:.1f} s",
            "cpu": _cpu_model()}


HERE = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILES = {  # workload -> counter summary of its dominant kernel (default partition)
    "llama7b_b64": ("profiles/decode_valu_f16_llama7b_b64_traffic.txt",
                    ("paged_kv_cache_139_amd/csrc/decode_valu.hip",
                     "paged_kv_cache_139_amd/csrc/device_common.h",
                     "paged_kv_cache_139_amd/csrc/internal.h")),
}


def measured_traffic(workload, partition_is_default):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    when there is none for this workload or the kernel sources changed since."""
    import hashlib
    if workload not in TRAFFIC_FILES or not partition_is_default:
        return None
    path, sources = TRAFFIC_FILES[workload]
    try:
        kv = {}
        for line in open(os.path.join(HERE, path)):
            if line.strip() and not line.startswith("#"):
                k, v = line.split(None, 1)
                kv[k] = v.strip()
        h = hashlib.sha256()
        for src in sources:
            h.update(open(os.path.join(HERE, src), "rb").read())
    except OSError:
        return None
    if kv.get("kernel_source_sha256") != h.hexdigest():
        return None
    return float(kv["traffic_bytes_per_launch"])


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the decode path has no multi-GPU mode "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads
    from workloads.gpu import DeviceWorkload

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        copy_calibration()
        return
    t0 = time.time()
    w = workloads.make(args.workload)
    dw = DeviceWorkload(w, "cuda:0", args.partition).fill()
    torch.cuda.synchronize()
    setup_s = time.time() - t0

    for _ in range(args.warmup):
        dw.step()
    torch.cuda.synchronize()

    K = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(K):
        dw.write_new()
        ev[i][0].record()
        dw.decode()
        ev[i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    dec_ms = np.array([a.elapsed_time(b) for a, b in ev])

    ms_per_step = wall * 1e3 / K
    dec_bytes = w.decode_bytes(unique=True)
    step_bytes = dec_bytes + w.writer_bytes(w.S)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    dec_avg_ms = float(dec_ms.mean())
    achieved = dec_bytes / (dec_avg_ms * 1e-3) / 1e9
    traffic_bytes = measured_traffic(w.name, args.partition in (0, None))
    traffic = None if traffic_bytes is None else traffic_bytes / (dec_avg_ms * 1e-3) / 1e9

    from paged_kv_cache_139_amd import DEFAULT_PARTITION_SIZE
    part = args.partition or DEFAULT_PARTITION_SIZE
    kernel = "decode_mfma_kernel" if (w.q_fmt != "f32" and 2 <= w.g <= 16) else "decode_valu_kernel"
    merged = w.MB * w.BS > part
    kernel_label = (f"paged_attention_decode call: {kernel}" +
                    (" + merge_kernel" if merged else " (one launch: no sequence spans two partitions)"))
    rec = {
        "metric": "decode attention effective KV GB/s (% of HBM peak) + seq-heads/sec",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "f16": "f16", "bf16": "bf16"}[w.q_fmt] +
                 ("+fp8kv" if w.cache_fmt == "fp8" else ""),
        "data": "synthetic",
        "config": {"workload": w.name, "num_seqs": w.S, "num_heads": w.H,
                   "num_kv_heads": w.Hk, "head_size": w.D, "block_size": w.BS,
                   "pool_blocks": w.NB, "max_blocks_per_seq": w.MB,
                   "total_context_tokens": int(w.context_lens.sum()),
                   "partition_size": part, "kv_dtype": w.cache_fmt},
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "seq_heads_per_s": round(w.S * w.H / (ms_per_step * 1e-3), 1),
        "step_bytes": int(step_bytes),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None if traffic is None else round(traffic, 2),
            "traffic_bytes_per_launch": None if traffic_bytes is None else int(traffic_bytes),
            "kernel": kernel_label,
            "avg_us": round(dec_avg_ms * 1e3, 2),
            "p10_us": round(float(np.percentile(dec_ms, 10)) * 1e3, 2),
            "p90_us": round(float(np.percentile(dec_ms, 90)) * 1e3, 2),
            "bytes_per_launch": int(dec_bytes),
        },
        "setup_s": round(setup_s, 1),
    }
    if args.cpu_seconds > 0:
        rec["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
