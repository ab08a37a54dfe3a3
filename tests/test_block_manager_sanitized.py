"""The host block manager (csrc/block_manager.cpp) built with g++ under
AddressSanitizer and UndefinedBehaviorSanitizer, driven by tests/c/
bm_sanitized.cpp through a seeded random sequence of calls on four pool and
block sizes, with the contract checks listed there.  Host code only: no GPU
code is built or run."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ROCM_INCLUDE = "/opt/rocm/include"


def _sanitizers_link(tmp_path):
    probe = tmp_path / "probe.cpp"
    probe.write_text("int main() { return 0; }\n")
    r = subprocess.run(["g++", "-fsanitize=address,undefined", str(probe), "-o",
                        str(tmp_path / "probe")], capture_output=True, text=True)
    return r.returncode == 0


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INCLUDE),
                    reason="needs g++ and the ROCm headers")
def test_block_manager_under_sanitizers(tmp_path):
    if not _sanitizers_link(tmp_path):
        pytest.skip("the sanitizer runtimes are not installed")
    exe = str(tmp_path / "bm_sanitized")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", f"-I{os.path.join(ROOT, 'include')}", f"-I{ROCM_INCLUDE}",
           os.path.join(HERE, "c", "bm_sanitized.cpp"),
           os.path.join(ROOT, "paged_kv_cache_139_amd", "csrc", "block_manager.cpp"),
           "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0 and run.stdout.strip().endswith("all ok"), (
        run.stdout[-2000:] + run.stderr[-4000:])
