"""bench.py's host-side helpers (no GPU): the source hash that guards the
committed counter summaries ignores comments and layout but not code, profile
file names per configuration, and the refusal of more than one GPU."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_strip_comments_keeps_code_and_literals():
    src = 'int a = 1; // note\n/* block\n comment */ const char* s = "//x/*y*/";\nchar c = \'/\';'
    assert bench.strip_comments(src) == 'int a = 1; const char* s = "//x/*y*/"; char c = \'/\';'
    assert bench.strip_comments("a\n\n   b") == "a b"
    # a comment-only edit keeps the text; a code edit does not
    assert bench.strip_comments("x = 1; // one") == bench.strip_comments("x = 1;   /* uno */")
    assert bench.strip_comments("x = 1;") != bench.strip_comments("x = 2;")


def test_every_code_path_hashes():
    for path in bench.KERNEL_SOURCES:
        assert len(bench.sources_sha256(path)) == 64


def rec(workload, call, part=2048, q="bf16", H=32, Hk=8, bs=16):
    return {"dtype": q, "config": {"workload": workload, "decode_call": call,
                                   "partition_size": part, "num_heads": H, "num_kv_heads": Hk,
                                   "block_size": bs, "max_blocks_per_seq": 2048}}


def test_profile_stems_name_each_configuration():
    assert bench.profile_stem(rec("long32k", "append", 512, H=32, Hk=32)) == \
        "decode_valu_bf16_long32k_p512_append"
    assert bench.profile_stem(rec("long32k", "append", H=32, Hk=32)) == \
        "decode_valu_bf16_long32k_append"
    assert bench.profile_stem(rec("fp8_mixed", "append")) == "decode_mfma_bf16_fp8_mixed_append"
    assert bench.profile_stem(rec("shared_prefix_gqa", "shared_prefix", H=64)) == \
        "decode_shared_prefix_bf16_shared_prefix_gqa"
    assert bench.profile_stem(rec("shared_prefix_gqa", "shared_prefix_append", H=64)) == \
        "decode_shared_prefix_bf16_shared_prefix_gqa_append"
    assert bench.call_kernels(rec("shared_prefix_gqa", "shared_prefix_append", H=64))[1] == \
        ["decode_group_kernel"]
    assert bench.profile_stem(rec("llama7b_b64", "writer_bulk", 0, q="f16")) == \
        "reshape_and_cache_f16_llama7b_b64_bulk"
    assert bench.bench_flags(rec("long32k", "append", 512, H=32, Hk=32)) == \
        " --single --workload long32k --partition 512"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
