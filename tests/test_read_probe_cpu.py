"""The benchmark's reference read kernels (libpkvprobe.so): built beside the
library, both entry points exported, and argument errors returned before any
launch (no GPU needed for those calls)."""
import ctypes
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PATH = os.path.join(ROOT, "paged_kv_cache_139_amd", "libpkvprobe.so")


@pytest.fixture(scope="module")
def lib():
    assert os.path.exists(PATH), "build first: python paged_kv_cache_139_amd/build.py"
    lib = ctypes.CDLL(PATH)
    vp, ci = ctypes.c_void_p, ctypes.c_int
    lib.pkvprobe_stream_read.argtypes = [vp, ctypes.c_size_t, vp, ci, vp]
    lib.pkvprobe_tile_read.argtypes = [vp] * 6 + [ci] * 5 + [vp, vp]
    return lib


def test_exports(lib):
    assert hasattr(lib, "pkvprobe_stream_read") and hasattr(lib, "pkvprobe_tile_read")


def test_stream_argument_errors(lib):
    p = 4096
    assert lib.pkvprobe_stream_read(None, 64, p, 4, None) == -1          # no buffer
    assert lib.pkvprobe_stream_read(p, 64, None, 4, None) == -1          # no sink
    assert lib.pkvprobe_stream_read(p, 65, p, 4, None) == -1             # not 16-byte words
    assert lib.pkvprobe_stream_read(p, 64, p, 0, None) == -1             # no work-groups
    assert lib.pkvprobe_stream_read(p, 64, p, 65537, None) == -1


def test_tile_argument_errors(lib):
    p = 4096
    ok = [p, p, p, p, p, p, 4, 2, 8, 16, 4096, p, None]

    def call(**kw):
        a = list(ok)
        names = ["k", "v", "bt", "s", "j0", "j1", "n", "hk", "mb", "nb", "tile", "sink", "st"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return lib.pkvprobe_tile_read(*a)

    assert call(k=None) == -1
    assert call(sink=None) == -1
    assert call(n=-1) == -1
    assert call(hk=0) == -1
    assert call(mb=0) == -1
    assert call(nb=0) == -1
    assert call(tile=3072) == -1                                       # not a supported tile
    assert call(n=1 << 30, hk=4) == -1                                 # grid too large
    assert call(n=0) == 0                                              # nothing to launch
