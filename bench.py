"""Benchmark of the paged decode step on one MI355X.

    python bench.py [--steps K] [--warmup W]                  # the whole suite, one JSON line
    python bench.py --single --workload NAME [--partition P]  # one configuration
    python bench.py --single --writer-bulk --workload NAME    # the writer's bulk fill alone
    python bench.py --read-ceiling                            # decode vs plain reads of its bytes

Default (the suite): the headline is the LLaMA-7B-shaped batch (64 seqs x 32
heads x 128, f16) decoded by one paged_attention_decode_append call per step
(the new token is stored by the decode kernel; one launch).  `value` is that
step's algorithmic HBM bytes (K and V of every cached (token, KV head) once, q
in and out, the used block-table entries and lengths, and the new tokens read
and written) over the mean event time of the step, inputs resident in HBM.
`roofline` is for that call, timed with HIP events on the launch stream.
`cpu_baseline` times the float64 oracle on a bounded sample of the same batch
on the host.  The same line carries, under "suite", the other large workloads
(long contexts at 512- and 2048-token partitions, the parallel-sampling batch
through the shared-prefix call, the FP8 batch), each with its own roofline,
and under "writer_bulk" the writer's bulk fills of the LLaMA-7B and FP8
batches (bytes read + written over the launch time).  Every `traffic` figure
comes from committed rocprofv3 FETCH_SIZE / WRITE_SIZE summaries in profiles/,
and only while the kernel sources they were taken on are unchanged.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published

# The suite: (workload, partition size (0: library default), decode call).
# "append": one paged_attention_decode_append call per step;
# "shared_prefix_append": one paged_attention_decode_shared_prefix_append call;
# "shared_prefix": reshape_and_cache for the new tokens, then
# paged_attention_decode_shared_prefix; "plain": reshape_and_cache, then
# paged_attention_decode.
# A fourth field, when present, is the cache block size (default 16; the pool
# keeps the same token capacity).
HEADLINE = ("llama7b_b64", 0, "append")
SUITE = [
    ("long32k", 512, "append"),
    ("long32k", 0, "append"),
    ("shared_prefix_gqa", 0, "shared_prefix_append"),
    ("llama7b_b64", 0, "append", 8),
    ("llama7b_b64", 0, "append", 32),
    ("fp8_mixed", 0, "append"),
    ("fp8_mixed", 0, "append", 8),
    ("fp8_mixed", 0, "append", 32),
    ("shared_prefix_gqa", 0, "append", 8),
    ("shared_prefix_gqa", 0, "append", 32),
]
WRITER_BULK = ["llama7b_b64", "fp8_mixed"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--suite-steps", type=int, default=20,
                    help="timed steps of each non-headline configuration of the suite")
    ap.add_argument("--single", action="store_true",
                    help="one configuration (--workload, --partition, ...) instead of the suite")
    ap.add_argument("--workload", default="llama7b_b64")
    ap.add_argument("--partition", type=int, default=0, help="tokens per partition (0: default)")
    ap.add_argument("--block-size", type=int, default=16, choices=(8, 16, 32),
                    help="cache block size in tokens (the pool keeps the same token capacity)")
    ap.add_argument("--shared-prefix", choices=("auto", "on", "off"), default="auto",
                    help="decode through paged_attention_decode_shared_prefix with the "
                         "workload's sharing groups (auto: when its sequences share prefix "
                         "blocks; off: paged_attention_decode)")
    ap.add_argument("--append", choices=("auto", "on", "off"), default="auto",
                    help="the step as one call whose decode kernel stores the new tokens "
                         "itself (paged_attention_decode_append, or the shared-prefix call's "
                         "append variant; auto: on; off: reshape_and_cache, then the decode "
                         "call)")
    ap.add_argument("--writer-bulk", action="store_true",
                    help="with --single: time reshape_and_cache writing all of the workload's "
                         "cached tokens (every token but each sequence's last) in one call")
    ap.add_argument("--flush-mb", type=int, default=1024,
                    help="MiB of scratch read (untimed) before every step, so that the step "
                         "starts with L2 and the 256 MB last-level cache holding other data "
                         "(0: none)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate budget of the oracle timing (0 disables it)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy 3 times (reference for the "
                         "FETCH_SIZE / WRITE_SIZE counters) and exit")
    ap.add_argument("--copy-blocks", action="store_true",
                    help="time copy_blocks instead of the decode step: --pairs (src, dst) "
                         "pairs over --layers layers of LLaMA-7B-shaped f16 caches")
    ap.add_argument("--block-manager", action="store_true",
                    help="time the host block manager's decode-step bookkeeping (no GPU): "
                         "--pairs prompts x 4 samples, append + tables per step")
    ap.add_argument("--read-ceiling", action="store_true",
                    help="time the plain decode call beside the reference read kernels of "
                         "libpkvprobe.so on the same bytes: the decode's tiles read with no "
                         "arithmetic, and one contiguous stream (--workload: a comma list; "
                         "default llama7b_b64,long32k,fp8_mixed)")
    ap.add_argument("--pairs", type=int, default=256)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--profile-summary", metavar="DIR",
                    help="no GPU: write profiles/<kernel>_<workload>.txt from the rocprofv3 "
                         "--stats output in DIR (with bench.log, the bench line of that run)")
    ap.add_argument("--traffic-summary", metavar="DIR",
                    help="no GPU: write profiles/<kernel>_<workload>_traffic.txt from the "
                         "FETCH_SIZE / WRITE_SIZE runs in DIR/{fetch,write}_{bench,copy} "
                         "(with DIR/bench.log, the bench line of the FETCH_SIZE run)")
    return ap.parse_args()


def say(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


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


def read_ceiling_bench(args):
    """The decode's bytes read with no arithmetic, for context beside the
    published peak: the plain decode call (default partitions, block size 16),
    the same (block, KV head) tiles read by libpkvprobe.so's tile kernel in the
    decode's work order (items longest first, 4 waves per item and KV head),
    and one contiguous stream of as many bytes.  Cold caches before every call
    (the read flush); medians over --steps calls."""
    import ctypes
    import torch
    from paged_kv_cache_139_amd import DEFAULT_PARTITION_SIZE
    from workloads.gpu import DeviceWorkload
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "paged_kv_cache_139_amd",
                        "libpkvprobe.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: run paged_kv_cache_139_amd/build.py")
    lib = ctypes.CDLL(path)
    vp, ci = ctypes.c_void_p, ctypes.c_int
    lib.pkvprobe_stream_read.argtypes = [vp, ctypes.c_size_t, vp, ci, vp]
    lib.pkvprobe_tile_read.argtypes = [vp] * 6 + [ci] * 5 + [vp, vp]
    names = (args.workload.split(",") if args.workload != "llama7b_b64" or args.single
             else ["llama7b_b64", "long32k", "fp8_mixed"])
    flush = Flush(args.flush_mb)
    dev = "cuda:0"
    for name in names:
        w = make_workload(name, 16)
        esize = {"fp8": 1, "f16": 2, "bf16": 2, "f32": 4}[w.cache_fmt]
        tile = w.D * 16 * esize
        dw = DeviceWorkload(w, dev, 0).fill()
        lens = w.context_lens.astype(np.int64)
        nblk = (lens + 15) // 16
        assert nblk.max() <= w.MB and dw.block_tables.dtype == torch.int32
        steps_per_part = DEFAULT_PARTITION_SIZE // 16
        items = []
        for s_ in range(w.S):
            n = int(nblk[s_])
            nparts = max(1, -(-n // steps_per_part))
            for p_ in range(nparts):
                items.append((p_ * n // nparts, (p_ + 1) * n // nparts, s_))
        items.sort(key=lambda t: t[0] - t[1])               # longest first (stable)
        it = [torch.tensor([t[k] for t in items], dtype=torch.int32, device=dev)
              for k in (2, 0, 1)]
        nbytes = int(nblk.sum()) * w.Hk * 2 * tile
        sink = torch.empty(max(len(items) * w.Hk, 1024) * 256, dtype=torch.int32, device=dev)
        stream_buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)

        def stream_ptr():
            return torch.cuda.current_stream().cuda_stream

        def tiles():
            r = lib.pkvprobe_tile_read(dw.k_cache.data_ptr(), dw.v_cache.data_ptr(),
                                       dw.block_tables.data_ptr(), it[0].data_ptr(),
                                       it[1].data_ptr(), it[2].data_ptr(), len(items), w.Hk,
                                       w.MB, w.NB, tile, sink.data_ptr(), stream_ptr())
            assert r == 0, r

        def stream():
            r = lib.pkvprobe_stream_read(stream_buf.data_ptr(), nbytes, sink.data_ptr(), 1024,
                                         stream_ptr())
            assert r == 0, r

        rec = {"read_ceiling": name, "bytes": nbytes, "tile_bytes": tile, "items": len(items),
               "calls": args.steps}
        for key, fn in (("decode", dw.decode), ("tile_probe", tiles), ("stream", stream)):
            for _ in range(max(args.warmup, 1)):
                flush()
                fn()
            torch.cuda.synchronize()
            ts = []
            for _ in range(args.steps):
                flush()
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record()
                fn()
                b.record()
                torch.cuda.synchronize()
                ts.append(a.elapsed_time(b) * 1e3)
            us = float(np.median(ts))
            rec[key + "_us"] = round(us, 2)
            rec[key + "_GBps"] = round(nbytes / us / 1e3, 1)
        rec["decode_of_stream_rate"] = round(rec["stream_us"] / rec["decode_us"], 4)
        rec["decode_of_tile_probe_rate"] = round(rec["tile_probe_us"] / rec["decode_us"], 4)
        print(json.dumps(rec), flush=True)
        del dw, stream_buf, sink
        torch.cuda.empty_cache()


def copy_blocks_bench(args):
    """copy_blocks on a copy-on-write burst: `pairs` blocks copied in each of
    `layers` layers, K and V, caches [2048, 32, 128, 16] f16 per layer."""
    import torch
    import paged_kv_cache_139_amd as pkv
    NB, Hk, D = 2048, 32, 128
    dev = "cuda:0"
    kcs = [torch.randn((NB, Hk, D, 16), dtype=torch.float16, device=dev)
           for _ in range(args.layers)]
    vcs = [torch.randn((NB, Hk, D, 16), dtype=torch.float16, device=dev)
           for _ in range(args.layers)]
    ids = np.random.default_rng(0).permutation(NB)
    pairs = np.stack([ids[:args.pairs], ids[args.pairs:2 * args.pairs]], 1).astype(np.int64)
    mapping = torch.from_numpy(pairs).to(dev)
    for _ in range(args.warmup):
        pkv.copy_blocks(kcs, vcs, mapping)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record()
        pkv.copy_blocks(kcs, vcs, mapping)
        b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    block_bytes = Hk * D * 16 * 2
    nbytes = args.pairs * args.layers * 2 * block_bytes * 2          # K and V, read + write
    # the timed configuration's result: every destination equals its source
    # (first and last layer, bitwise)
    for li in (0, args.layers - 1):
        k_host = kcs[li].cpu().numpy()
        v_host = vcs[li].cpu().numpy()
        ok = all(np.array_equal(k_host[d], k_host[s]) and np.array_equal(v_host[d], v_host[s])
                 for s, d in pairs)
        assert ok, f"layer {li}: a copied block differs from its source"
    avg = float(ms.mean())
    gbs = nbytes / (avg * 1e-3) / 1e9
    rec = {"metric": "copy_blocks HBM GB/s (bytes read + written)", "value": round(gbs, 2),
           "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(wall * 1e3 / args.steps, 5), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
           "config": {"workload": f"cow_copy_{args.pairs}x{args.layers}l_llama7b",
                      "pairs": args.pairs, "layers": args.layers, "pool_blocks": NB,
                      "num_kv_heads": Hk, "head_size": D, "block_size": 16},
           "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                        "kernel": "copy_blocks_kernel", "avg_us": round(avg * 1e3, 2),
                        "p10_us": round(float(np.percentile(ms, 10)) * 1e3, 2),
                        "p90_us": round(float(np.percentile(ms, 90)) * 1e3, 2),
                        "bytes_per_launch": int(nbytes)}}
    print(json.dumps(rec), flush=True)


def block_manager_bench(args):
    """Host bookkeeping of one decode step with the library's block manager:
    append one token to every live sequence (slots + copy-on-write pairs) and
    build the batch's block tables.  Prompts of U{128..2048} tokens, each
    forked into 4 samples (so the first step copies their partial blocks)."""
    import paged_kv_cache_139_amd as pkv
    rng = np.random.default_rng(0)
    n_prompts, samples, bs = args.pairs, 4, 16
    lens = rng.integers(128, 2048, size=n_prompts, endpoint=True)
    steps = args.steps
    nb = int(sum(-(-int(L) // bs) * samples for L in lens)) + n_prompts * samples * (steps // bs + 2)
    bm = pkv.BlockManager(nb, bs)
    ids = []
    for i, L in enumerate(lens):
        bm.add_sequence(i * samples, int(L))
        ids.append(i * samples)
        for j in range(1, samples):
            bm.fork(i * samples, i * samples + j)
            ids.append(i * samples + j)
    mb = int(lens.max()) // bs + steps // bs + 2
    t = []
    copies = 0
    for _ in range(steps):
        t0 = time.perf_counter()
        slots, pairs, _ = bm.append_tokens(ids)
        bm.build_block_tables(ids, mb)
        t.append(time.perf_counter() - t0)
        copies += len(pairs)
    t = np.array(t) * 1e6
    rec = {"metric": "host block manager: decode-step bookkeeping (append + block tables)",
           "value": round(float(np.median(t)), 2), "unit": "us per step",
           "higher_is_better": False, "steps": steps, "n_gpus": 0, "data": "synthetic",
           "config": {"workload": f"block_manager_{n_prompts}x{samples}", "sequences": len(ids),
                      "block_size": bs, "pool_blocks": nb, "max_blocks_per_seq": mb},
           "p10_us": round(float(np.percentile(t, 10)), 2),
           "p90_us": round(float(np.percentile(t, 90)), 2),
           "first_step_us": round(float(t[0]), 2), "copy_on_write_pairs": copies,
           "appends_per_s": round(len(ids) / (float(np.median(t)) * 1e-6), 1),
           "cpu": _cpu_model()}
    print(json.dumps(rec), flush=True)


# --------------------------------------------------------------------------- #
# the oracle on the host (cpu_baseline)
# --------------------------------------------------------------------------- #
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
    rec = {"value": round(nbytes / t_oracle / 1e9, 4), "unit": "GB/s", "cores": 1,
           "kind": "oracle",
           "seq_heads_per_s": round(seq_heads / t_oracle, 2),
           "sample": f"{len(done)} sequence passes over {len(set(done))} of the {w.S} "
                     f"sequences of the same workload ({seq_heads} (sequence, head) pairs): "
                     f"writer for the decode token + attention, float64 numpy, 1 thread, "
                     f"{t_oracle:.1f} s",
           "cpu": _cpu_model()}
    rec["all_cores"] = cpu_baseline_all_cores(w, budget_s / 2)
    return rec


def one_sequence_oracle(w, s):
    """The oracle's work for sequence s of a step (writer for its new token, then
    attention); returns its algorithmic bytes and (sequence, head) pairs."""
    import oracle
    cp = oracle.CompactPool(w, [int(s)])
    sl = w.slot_new[s:s + 1]
    slot_c = np.where(sl >= 0, cp.remap[np.maximum(sl, 0) // 16] * 16 + sl % 16, -1)
    oracle.reshape_and_cache_ref(w.key_new[s:s + 1], w.value_new[s:s + 1], cp.k, cp.v, slot_c,
                                 w.src_fmt, w.cache_fmt, w.k_scale, w.v_scale)
    cp.attention(w)
    L = int(w.context_lens[s])
    return (L * w.Hk * w.D * 2 * w.kv_elem_bytes() + w.H * w.D * 2 * w.q_elem_bytes()
            + (-(-L // 16)) * 4 + 4), w.H


_POOL_W = None          # the workload, inherited by the forked oracle workers


def _pool_task(s):
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        return one_sequence_oracle(_POOL_W, s)


def cpu_baseline_all_cores(w, budget_s):
    """The same oracle work spread over the host's cores: one forked process per
    core (at most 16, the host share of one GPU), each taking whole sequences
    with its numerical library on one thread, for about budget_s seconds of
    wall time (the per-sequence copy-out of the pool is included here).  Runs
    before this process touches the GPU, so the workers inherit no GPU state."""
    import multiprocessing as mp
    global _POOL_W
    workers = max(1, min(16, os.cpu_count() or 1))
    order = [int(s) for s in np.random.default_rng(1).permutation(w.S)] * 20
    nbytes = pairs = count = 0
    _POOL_W = w
    pool = mp.get_context("fork").Pool(workers)
    try:
        t0 = time.perf_counter()
        for b, h in pool.imap_unordered(_pool_task, order):
            nbytes += b
            pairs += h
            count += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        wall = time.perf_counter() - t0
    finally:
        pool.terminate()
        pool.join()
        _POOL_W = None
    return {"value": round(nbytes / wall / 1e9, 4), "unit": "GB/s", "cores": workers,
            "seq_heads_per_s": round(pairs / wall, 2),
            "sample": f"{count} sequence passes of the same workload in {workers} processes, "
                      f"{wall:.1f} s wall"}


# --------------------------------------------------------------------------- #
# kernels, profile files and the counter summaries they are checked against
# --------------------------------------------------------------------------- #
HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = "paged_kv_cache_139_amd/csrc/"
KERNEL_SOURCES = {  # code path -> the sources its kernels come from
    "decode_valu": (CSRC + "decode_valu.hip", CSRC + "device_common.h", CSRC + "internal.h"),
    "decode_mfma": (CSRC + "decode_mfma.hip", CSRC + "decode_valu.hip",
                    CSRC + "device_common.h", CSRC + "internal.h"),
    "decode_shared_prefix": (CSRC + "decode_mfma.hip", CSRC + "decode_valu.hip",
                             CSRC + "device_common.h", CSRC + "internal.h"),
    "reshape_and_cache": (CSRC + "writer.hip", CSRC + "device_common.h", CSRC + "internal.h"),
}
DT_NAMES = {"0": "f32", "1": "f16", "2": "bf16", "3": "fp8"}


def decode_kernel_of(q_fmt, g, block_size=16):
    mfma = q_fmt != "f32" and 2 <= g <= 16
    return "decode_mfma_kernel" if mfma else "decode_valu_kernel"


def call_kernels(rec):
    """(name of the call's code path, its kernels in launch order) for a bench
    record."""
    c = rec["config"]
    if c.get("decode_call") == "writer_bulk":
        return "reshape_and_cache", ["reshape_and_cache_kernel"]
    kernel = decode_kernel_of(rec["dtype"].split("+")[0], c["num_heads"] // c["num_kv_heads"],
                              c.get("block_size", 16))
    if c.get("decode_call", "").startswith("shared_prefix"):
        if kernel == "decode_mfma_kernel":        # one launch on the matrix cores
            return "decode_shared_prefix", ["decode_group_kernel"]
        return "decode_shared_prefix", ["decode_prefix_kernel", kernel, "merge_kernel"]
    merged = c["max_blocks_per_seq"] * c["block_size"] > c["partition_size"]
    return kernel.replace("_kernel", ""), [kernel] + (["merge_kernel"] if merged else [])


def profile_stem(rec):
    """profiles/ file stem for a bench record: code path, q dtype, workload (the
    partition size when it is not the default, the block size when it is not 16,
    _append for the one-call step, _bulk for the writer's bulk fill)."""
    from paged_kv_cache_139_amd import DEFAULT_PARTITION_SIZE
    path, _ = call_kernels(rec)
    c = rec["config"]
    tail = ""
    if c.get("decode_call") != "writer_bulk" and c.get("partition_size") != DEFAULT_PARTITION_SIZE:
        tail += f"_p{c['partition_size']}"
    if c.get("block_size", 16) != 16:
        tail += f"_bs{c['block_size']}"
    if c.get("decode_call") in ("append", "shared_prefix_append"):
        tail += "_append"
    if c.get("decode_call") == "writer_bulk":
        tail += "_bulk"
    q_dtype = rec["dtype"].split("+")[0].split("->")[0]      # query / source dtype
    return f"{path}_{q_dtype}_{c['workload']}{tail}"


def bench_flags(rec):
    """The bench.py flags that reproduce a bench record's configuration alone."""
    from paged_kv_cache_139_amd import DEFAULT_PARTITION_SIZE
    c = rec["config"]
    flags = f" --single --workload {c['workload']}"
    if c.get("decode_call") == "writer_bulk":
        return flags + " --writer-bulk"
    if c.get("partition_size") != DEFAULT_PARTITION_SIZE:
        flags += f" --partition {c['partition_size']}"
    if c.get("decode_call", "").startswith("shared_prefix"):
        flags += " --shared-prefix on"
    elif c["workload"] == "shared_prefix_gqa":
        flags += " --shared-prefix off"
    if c.get("decode_call") in ("plain", "shared_prefix"):
        flags += " --append off"
    if c.get("block_size", 16) != 16:
        flags += f" --block-size {c['block_size']}"
    return flags


def traffic_file(rec):
    return os.path.join("profiles", profile_stem(rec) + "_traffic.txt")


def strip_comments(text):
    """C/C++ source without its comments and blank space: // and /* */ comments
    outside string and character literals are dropped, every run of white space
    becomes one space.  A change to comments or layout then keeps the hash."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def sources_sha256(path):
    """SHA-256 of a code path's kernel sources with comments and layout removed
    (strip_comments): the counters stay valid across comment-only edits, and
    any change to the code itself invalidates them."""
    import hashlib
    h = hashlib.sha256()
    for src in KERNEL_SOURCES[path]:
        with open(os.path.join(HERE, src), encoding="utf-8") as f:
            h.update(strip_comments(f.read()).encode("utf-8"))
    return h.hexdigest()


def measured_traffic(rec, default_run):
    """HBM bytes per call from the committed rocprofv3 counter summary for this
    configuration, or None when there is none, the kernel's sources changed
    since the counters were taken, or the run does not use the cache flush the
    counters were taken with."""
    if not default_run:
        return None
    try:
        kv = {}
        with open(os.path.join(HERE, traffic_file(rec))) as f:
            for line in f:
                if line.strip() and not line.startswith("#"):
                    k, v = line.split(None, 1)
                    kv[k] = v.strip()
        sha = sources_sha256(call_kernels(rec)[0])
    except OSError:
        return None
    if kv.get("kernel_source_sha256") != sha:
        return None
    return float(kv["traffic_bytes_per_launch"])


def _bench_line(path):
    with open(path) as f:
        for line in f:
            if line.startswith("{") and '"metric"' in line:
                return json.loads(line)
    raise SystemExit(f"no bench line in {path}")


def _short_kernel(name):
    import re
    name = re.sub(r"^void ", "", name)
    name = re.sub(r"pkv::\(anonymous namespace\)::", "", name)
    name = re.sub(r"\(pkv::DT\)(\d)", lambda m: DT_NAMES[m.group(1)], name)
    return re.sub(r"\(pkv::DecodePtrs.*$|\(unsigned char const\*.*$", "", name)


def _csv_rows(directory, suffix):
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(directory, "**", "*" + suffix), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {directory}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def profile_summary(directory):
    """profiles/<path>_<q dtype>_<workload>....txt from one rocprofv3 --stats run
    of a --single bench configuration."""
    rec = _bench_line(os.path.join(directory, "bench.log"))
    c = rec["config"]
    rows = _csv_rows(directory, "kernel_stats.csv")
    if rec["metric"].startswith("copy_blocks"):
        return _copy_profile_summary(directory, rec, rows)
    path, kernels = call_kernels(rec)
    wl = c["workload"]
    flags = bench_flags(rec)
    what = ("the writer's bulk fill of" if c.get("decode_call") == "writer_bulk"
            else "paged decode on")
    out = [f"# rocprofv3 kernel statistics: {what} the {wl} workload"
           + (f" at block size {c['block_size']}" if c.get("block_size", 16) != 16 else ""),
           f"# ({c['num_seqs']} seqs x {c['num_heads']} heads ({c['num_kv_heads']} KV heads) x "
           f"head {c['head_size']}, {rec['dtype']}, {c['total_context_tokens']} context tokens,",
           f"#  {c['pool_blocks']}-block pool, {c['partition_size']}-token partitions; "
           f"{rec['warmup']} warm-up + {rec['steps']} timed calls plus one bulk fill;",
           f"#  a {rec.get('timing', {}).get('cache_flush_mib_read_before_each_step', 0)} MiB "
           f"read (torch sum) before every call empties the caches of its data)",
           "# command, from the repository root on one MI355X:",
           f"#   rocprofv3 --kernel-trace --stats -d {directory} -o bench --output-format csv -- \\",
           f"#       python -u bench.py --cpu-seconds 0{flags}",
           f"# bench record of the same process: {rec['roofline']['avg_us']} us per call "
           f"(HIP events), {rec['roofline']['achieved']} GB/s, frac {rec['roofline']['frac']}",
           "",
           f"{'kernel':<58} {'calls':>6} {'avg_us':>9} {'min_us':>9} {'max_us':>9}"]
    call_us = 0.0
    for r in rows:
        name = _short_kernel(r["Name"])
        a = float(r["AverageNs"]) / 1e3
        out.append(f"{name[:58]:<58} {int(r['Calls']):>6} {a:>9.2f} "
                   f"{float(r['MinNs']) / 1e3:>9.2f} {float(r['MaxNs']) / 1e3:>9.2f}")
        if any(k in r["Name"] for k in kernels):
            call_us += a
    b = rec["roofline"]["bytes_per_launch"]
    out += ["",
            f"# call = {' + '.join(kernels)}"
            f": {call_us:.2f} us by kernel averages; {b} algorithmic bytes per call ->",
            f"#   {b / (call_us * 1e-6) / 1e9:.0f} GB/s ({b / (call_us * 1e-6) / 8e12:.3f} of 8 TB/s)."]
    path = os.path.join("profiles", profile_stem(rec) + ".txt")
    with open(os.path.join(HERE, path), "w") as f:
        f.write("\n".join(out) + "\n")
    print(f"wrote {path}")


def _copy_profile_summary(directory, rec, rows):
    c = rec["config"]
    out = [f"# rocprofv3 kernel statistics: copy_blocks on a copy-on-write burst of {c['pairs']} "
           f"(src, dst) pairs",
           f"# in each of {c['layers']} layers, K and V caches [{c['pool_blocks']}, "
           f"{c['num_kv_heads']}, {c['head_size']}, {c['block_size']}] f16 per layer",
           f"# ({rec['warmup']} warm-up + {rec['steps']} timed calls; 32 layers = one launch)",
           "# command, from the repository root on one MI355X:",
           f"#   rocprofv3 --kernel-trace --stats -d {directory} -o bench --output-format csv -- \\",
           "#       python -u bench.py --copy-blocks",
           f"# bench line of the same process: {rec['roofline']['avg_us']} us per call (HIP "
           f"events), {rec['value']} GB/s read + written, frac {rec['roofline']['frac']}",
           "",
           f"{'kernel':<58} {'calls':>6} {'avg_us':>9} {'min_us':>9} {'max_us':>9}"]
    avg = 0.0
    for r in rows:
        name = _short_kernel(r["Name"])
        a = float(r["AverageNs"]) / 1e3
        out.append(f"{name[:58]:<58} {int(r['Calls']):>6} {a:>9.2f} "
                   f"{float(r['MinNs']) / 1e3:>9.2f} {float(r['MaxNs']) / 1e3:>9.2f}")
        if "copy_blocks_kernel" in r["Name"]:
            avg = a
    b = rec["roofline"]["bytes_per_launch"]
    out += ["", f"# copy_blocks_kernel: {avg:.2f} us; {b} bytes read + written per call -> "
                f"{b / (avg * 1e-6) / 1e9:.0f} GB/s ({b / (avg * 1e-6) / 8e12:.3f} of 8 TB/s)."]
    path = os.path.join("profiles", f"copy_blocks_f16_{c['workload']}.txt")
    with open(os.path.join(HERE, path), "w") as f:
        f.write("\n".join(out) + "\n")
    print(f"wrote {path}")


def traffic_summary(directory):
    """profiles/<stem>_traffic.txt from FETCH_SIZE and WRITE_SIZE runs of a
    --single bench configuration and of its plain-copy calibration."""
    rec = _bench_line(os.path.join(directory, "bench.log"))
    path, kernels = call_kernels(rec)
    wl = rec["config"]["workload"]
    bulk = rec["config"].get("decode_call") == "writer_bulk"

    def per_call(sub, counter):
        rows = _csv_rows(os.path.join(directory, sub), "counter_collection.csv")
        total, calls = 0.0, 0
        for r in rows:
            if r["Counter_Name"] != counter:
                continue
            if kernels[0] in r["Kernel_Name"]:
                calls += 1
            if any(k in r["Kernel_Name"] for k in kernels):
                total += float(r["Counter_Value"])
        return total / calls, calls

    def copy_kib(sub, counter):
        rows = _csv_rows(os.path.join(directory, sub), "counter_collection.csv")
        vals = [float(r["Counter_Value"]) for r in rows
                if r["Counter_Name"] == counter and "copyBuffer" in r["Kernel_Name"]]
        return sum(vals) / len(vals)

    fetch, calls = per_call("fetch_bench", "FETCH_SIZE")
    write, _ = per_call("write_bench", "WRITE_SIZE")
    cf, cw = copy_kib("fetch_copy", "FETCH_SIZE"), copy_kib("write_copy", "WRITE_SIZE")
    fs, ws = 1048576.0 / cf, 1048576.0 / cw
    traffic = (fetch * fs + write * ws) * 1024
    alg = rec["roofline"]["bytes_per_launch"]
    cmd = f"python -u bench.py --steps 5 --warmup 1 --cpu-seconds 0{bench_flags(rec)}"
    what = ("one bulk reshape_and_cache call" if bulk else
            f"one call ({' + '.join(kernels)})")
    lines = [
        f"# HBM traffic of {what} on the {wl} workload,",
        "# from rocprofv3 hardware counters on one MI355X.",
        "# Each counter in a run of its own; a plain 1 GiB device copy calibrates them.",
        "# commands, from the repository root:",
        f"#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d {directory}/fetch_bench -o bench -- {cmd}",
        f"#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d {directory}/write_bench -o bench -- {cmd}",
        f"#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d {directory}/fetch_copy -o copy -- python -u bench.py --copy-calibration",
        f"#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d {directory}/write_copy -o copy -- python -u bench.py --copy-calibration",
        f"# The copy (__amd_rocclr_copyBuffer, 1073741824 bytes read and written) reads",
        f"# {cf:.1f} KiB on FETCH_SIZE and {cw:.1f} KiB on WRITE_SIZE; each reading of the",
        f"# call is scaled by 1048576 KiB / the copy's reading of the same counter.",
        f"# bench.py reports traffic only while kernel_source_sha256 matches the sources",
        f"# ({', '.join(os.path.basename(x) for x in KERNEL_SOURCES[path])}; comments and",
        f"# layout stripped before hashing).",
        f"kernel_source_sha256 {sources_sha256(path)}",
        f"decode_fetch_kib_per_launch {fetch:.1f}",
        f"decode_write_kib_per_launch {write:.1f}",
        f"decode_launches_counted {calls}",
        f"copy_fetch_kib {cf:.1f}",
        f"copy_write_kib {cw:.1f}",
        f"fetch_scale {fs:.5f}",
        f"write_scale {ws:.5f}",
        f"traffic_bytes_per_launch {traffic:.0f}",
        f"algorithmic_bytes_per_launch {alg}",
        f"traffic_over_algorithmic {traffic / alg:.4f}",
    ]
    path = traffic_file(rec)
    with open(os.path.join(HERE, path), "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {path}")


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# --------------------------------------------------------------------------- #
# GPU measurements
# --------------------------------------------------------------------------- #
def make_workload(name, block_size=16):
    import workloads
    if block_size == 16:
        return workloads.make(name)
    nb = workloads.WORKLOADS[name]["NB"] * 16 // block_size
    return workloads.make(name, block_size=block_size, NB=nb)


class Flush:
    """Cold caches: a read (not a write, whose dirty lines would be written back
    during the timed call) of `mb` MiB before every timed call evicts the call's
    data from L2 and the last-level cache; the flush is outside the events."""

    def __init__(self, mb):
        import torch
        self.mb = mb
        self.scratch = (torch.ones(mb << 18, dtype=torch.float32, device="cuda:0")
                        if mb > 0 else None)

    def __call__(self):
        if self.scratch is not None:
            self.scratch.sum()


def time_calls(fn, flush, steps, warmup, two_part=None):
    """Mean-able per-call event times (ms) of fn() over `steps` calls after
    `warmup`, each preceded by the flush.  two_part: (first, second) callables
    timed back to back as one step, with an event between them; then returns
    (step times, second-part times)."""
    import torch
    for _ in range(warmup):
        flush()
        if two_part:
            two_part[0]()
            two_part[1]()
        else:
            fn()
    torch.cuda.synchronize()
    ev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b, c in ev:
        flush()
        a.record()
        if two_part:
            two_part[0]()
            b.record()
            two_part[1]()
        else:
            fn()
        c.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step = np.array([a.elapsed_time(c) for a, _, c in ev])
    second = np.array([b.elapsed_time(c) for _, b, c in ev]) if two_part else step
    return step, second, wall


def rate_stats(ms, nbytes):
    avg = float(ms.mean())
    gbs = nbytes / (avg * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
            "traffic_bytes_per_launch": None,
            "avg_us": round(avg * 1e3, 2), "median_us": round(float(np.median(ms)) * 1e3, 2),
            "p10_us": round(float(np.percentile(ms, 10)) * 1e3, 2),
            "p90_us": round(float(np.percentile(ms, 90)) * 1e3, 2),
            "bytes_per_launch": int(nbytes)}


def attach_traffic(rec, flush_mb, ms):
    t = measured_traffic(rec, flush_mb == 1024)
    if t is not None:
        rec["roofline"]["traffic"] = round(t / (float(ms.mean()) * 1e-3) / 1e9, 2)
        rec["roofline"]["traffic_bytes_per_launch"] = int(t)


def workload_config(w, part, call):
    return {"workload": w.name, "num_seqs": w.S, "num_heads": w.H, "num_kv_heads": w.Hk,
            "head_size": w.D, "block_size": w.BS, "pool_blocks": w.NB,
            "max_blocks_per_seq": w.MB, "total_context_tokens": int(w.context_lens.sum()),
            "partition_size": part, "kv_dtype": w.cache_fmt, "decode_call": call}


def dtype_label(w):
    return w.q_fmt + ("+fp8kv" if w.cache_fmt == "fp8" else "")


def measure_step(w, part, call, steps, warmup, flush, flush_mb):
    """One decode step of workload w, timed over `steps` steps: call "append"
    (paged_attention_decode_append), "shared_prefix_append"
    (paged_attention_decode_shared_prefix_append), "plain" (reshape_and_cache,
    then paged_attention_decode) or "shared_prefix" (reshape_and_cache, then
    paged_attention_decode_shared_prefix).  Returns the bench record."""
    import torch
    from paged_kv_cache_139_amd import DEFAULT_PARTITION_SIZE
    from workloads.gpu import DeviceWorkload
    t0 = time.time()
    shared = call.startswith("shared_prefix")
    dw = DeviceWorkload(w, "cuda:0", part, shared_prefix=shared).fill()
    torch.cuda.synchronize()
    setup_s = time.time() - t0
    append = call in ("append", "shared_prefix_append")
    if append:
        step_ms, dec_ms, wall = time_calls(dw.decode_append, flush, steps, warmup)
    else:
        step_ms, dec_ms, wall = time_calls(None, flush, steps, warmup,
                                           two_part=(dw.write_new, dw.decode))
    part = part or DEFAULT_PARTITION_SIZE
    kernel = decode_kernel_of(w.q_fmt, w.g, w.BS)
    merged = w.MB * w.BS > part
    if shared:
        passes = ("decode_group_kernel (prefix once per 16-row tile, then each member's "
                  "blocks; no merge)" if kernel == "decode_mfma_kernel"
                  else f"decode_prefix_kernel + {kernel} + merge_kernel")
        label = (f"paged_attention_decode_shared_prefix{'_append' if append else ''} call: "
                 f"{passes}" + (" and stores the new tokens" if append else ""))
    elif append:
        label = (f"paged_attention_decode_append call: {kernel} stores the new tokens" +
                 (" + merge_kernel" if merged else " (no sequence spans two partitions)"))
    else:
        label = (f"paged_attention_decode call: {kernel}" +
                 (" + merge_kernel" if merged else
                  " (one launch: no sequence spans two partitions)"))
    dec_bytes = w.decode_bytes(unique=True)
    step_bytes = dec_bytes + w.writer_bytes(w.S)
    if append:                                   # the call also moves the new tokens
        dec_bytes = step_bytes
    ms_per_step = float(step_ms.mean())
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    rec = {
        "metric": "decode attention effective KV GB/s (% of HBM peak) + seq-heads/sec",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": dtype_label(w), "data": "synthetic",
        "config": workload_config(w, part, call),
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "seq_heads_per_s": round(w.S * w.H / (ms_per_step * 1e-3), 1),
        "step_bytes": int(step_bytes),
        "roofline": {**rate_stats(dec_ms, dec_bytes), "kernel": label},
        "setup_s": round(setup_s, 1),
        "timing": {"step": ("HIP events around the one decode-with-append call"
                            if append else
                            "HIP events around reshape_and_cache + the decode call") +
                           ", mean over steps",
                   "cache_flush_mib_read_before_each_step": flush_mb,
                   "wall_ms_per_step_incl_flush": round(wall * 1e3 / steps, 5)},
    }
    if not append:
        wr_ms = float(np.mean(step_ms - dec_ms))
        rec["writer"] = {"avg_us": round(wr_ms * 1e3, 2), "bytes": int(w.writer_bytes(w.S)),
                         "GBps": round(w.writer_bytes(w.S) / (wr_ms * 1e-3) / 1e9, 2)}
    if w.shared_groups:
        logical = w.decode_bytes(unique=False)
        rec["logical_kv"] = {"bytes": int(logical),
                             "GBps": round(logical / (float(np.mean(dec_ms)) * 1e-3) / 1e9, 2),
                             "note": "every sequence's whole context counted, shared blocks "
                                     "once per sequence"}
    attach_traffic(rec, flush_mb, dec_ms)
    del dw
    torch.cuda.empty_cache()
    return rec


def measure_writer_bulk(w, steps, warmup, flush, flush_mb):
    """reshape_and_cache writing every cached token of workload w (all but each
    sequence's last, in sequence order: the bulk fill of the pools) in one call,
    from sources already in HBM; bytes = K and V read in the source format and
    written in the cache format, plus the slots."""
    import torch
    import paged_kv_cache_139_amd as pkv
    from workloads.gpu import DeviceWorkload, to_device
    dev = "cuda:0"
    dw = DeviceWorkload(w, dev)
    k = to_device(w.key_bulk, w.src_fmt, dev)
    v = to_device(w.value_bulk, w.src_fmt, dev)
    s = torch.from_numpy(w.slot_bulk).to(dev)
    T = len(w.slot_bulk)

    def call():
        pkv.reshape_and_cache(k, v, dw.k_cache, dw.v_cache, s, w.k_scale, w.v_scale)
    ms, _, wall = time_calls(call, flush, steps, warmup)
    nbytes = w.writer_bytes(T)
    rec = {"metric": "reshape_and_cache bulk fill HBM GB/s (bytes read + written)",
           "dtype": w.src_fmt + "->" + w.cache_fmt, "steps": steps, "warmup": warmup,
           "config": {**workload_config(w, 0, "writer_bulk"), "tokens": T},
           "roofline": {**rate_stats(ms, nbytes),
                        "kernel": "reshape_and_cache_kernel (one launch over all tokens)"},
           "tokens_per_s": round(T / (float(ms.mean()) * 1e-3), 1),
           "timing": {"call": "HIP events around one reshape_and_cache call, mean over calls",
                      "cache_flush_mib_read_before_each_step": flush_mb,
                      "wall_ms_per_call_incl_flush": round(wall * 1e3 / steps, 5)}}
    attach_traffic(rec, flush_mb, ms)
    del dw, k, v, s
    torch.cuda.empty_cache()
    return rec


def compact(rec):
    """The parts of a configuration's record kept inside the suite line."""
    keep = ("config", "dtype", "steps", "ms_per_step", "value", "pct_hbm_peak",
            "seq_heads_per_s", "step_bytes", "roofline", "writer", "logical_kv",
            "tokens_per_s")
    return {k: rec[k] for k in keep if k in rec}


def main():
    args = parse()
    if args.profile_summary:
        profile_summary(args.profile_summary)
        return
    if args.traffic_summary:
        traffic_summary(args.traffic_summary)
        return
    if args.block_manager:
        block_manager_bench(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the decode path has no multi-GPU mode "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration or args.copy_blocks or args.read_ceiling:
        assert torch.cuda.is_available(), "bench.py needs a GPU"
        if args.read_ceiling:
            read_ceiling_bench(args)
        elif args.copy_calibration:
            copy_calibration()
        else:
            copy_blocks_bench(args)
        return

    if args.single:
        w = make_workload(args.workload, args.block_size)
        cpu = (cpu_baseline(w, args.cpu_seconds)
               if args.cpu_seconds > 0 and not args.writer_bulk else None)
        assert torch.cuda.is_available(), "bench.py needs a GPU"
        flush = Flush(args.flush_mb)
        if args.writer_bulk:
            rec = measure_writer_bulk(w, args.steps, args.warmup, flush, args.flush_mb)
            rec.update({"value": rec["roofline"]["achieved"], "unit": "GB/s", "n_gpus": 1,
                        "ms_per_step": round(rec["roofline"]["avg_us"] / 1e3, 5),
                        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
                        "data": "synthetic"})
        else:
            shared = args.shared_prefix == "on" or (args.shared_prefix == "auto" and
                                                    bool(w.shared_groups))
            split = args.append == "off"
            call = (("shared_prefix" if split else "shared_prefix_append") if shared else
                    ("plain" if split else "append"))
            rec = measure_step(w, args.partition, call, args.steps, args.warmup, flush,
                               args.flush_mb)
        if cpu is not None:
            rec["cpu_baseline"] = cpu
        print(json.dumps(rec), flush=True)
        return

    # the suite: the headline configuration first (with the oracle's timing,
    # which forks worker processes and so runs before the GPU is touched)
    t_all = time.time()
    name, part, call = HEADLINE
    say(f"{name}: generating inputs")
    w = make_workload(name)
    cpu = cpu_baseline(w, args.cpu_seconds) if args.cpu_seconds > 0 else None
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    flush = Flush(args.flush_mb)
    say(f"{name}: {args.steps} timed steps")
    rec = measure_step(w, part, call, args.steps, args.warmup, flush, args.flush_mb)
    suite = {}
    bulk = {}
    for wname in WRITER_BULK:
        wb = w if wname == name else make_workload(wname)
        say(f"writer bulk fill of {wname}")
        bulk[wname] = compact(measure_writer_bulk(wb, args.suite_steps, args.warmup, flush,
                                                  args.flush_mb))
        if wb is not w:
            del wb
    del w
    for sname, spart, scall, *rest in SUITE:
        sbs = rest[0] if rest else 16
        say(f"{sname} partition {spart or 'default'} {scall} block size {sbs}: "
            f"{args.suite_steps} timed steps")
        ws = make_workload(sname, sbs)
        key = (f"{sname}" + (f"_p{spart}" if spart else "") + (f"_bs{sbs}" if sbs != 16 else "")
               + f"_{scall}")
        suite[key] = compact(measure_step(ws, spart, scall, args.suite_steps, args.warmup,
                                          flush, args.flush_mb))
        del ws
    rec["suite"] = suite
    rec["writer_bulk"] = bulk
    rec["suite_wall_s"] = round(time.time() - t_all, 1)
    if cpu is not None:
        rec["cpu_baseline"] = cpu
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
