"""Build libpagedkv.so (gfx950) in-tree with hipcc, and beside it
libpkvprobe.so, the benchmark's reference read kernels (csrc/read_probe.hip).

    python paged_kv_cache_139_amd/build.py      # or __graft_entry__.build()

(run as a file: importing the package first would load the library it
rebuilds)

Each .hip file is compiled on its own (in parallel), then linked into one
shared library next to this file.  The library is always rebuilt.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(HERE, "libpagedkv.so")
PROBE_PATH = os.path.join(HERE, "libpkvprobe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]

SOURCES = ["api.hip", "writer.hip", "decode_valu.hip", "decode_mfma.hip", "copy_blocks.hip",
           "block_manager.cpp"]
PROBE_SOURCES = ["read_probe.hip"]


def _compile(src, verbose):
    obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if verbose and out.strip():
        print(out)
    return obj


def _link(objs, path, verbose):
    tmp = path + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, path)
    if verbose:
        print("built", path)


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with ThreadPoolExecutor(len(srcs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    _link(objs[:len(SOURCES)], LIB_PATH, verbose)
    _link(objs[len(SOURCES):], PROBE_PATH, verbose)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
