"""ctypes binding of libpagedkv.so: argument marshalling only.

Every computation runs in the library's HIP kernels; torch supplies device
memory and the current stream.  Importing this module loads the library and
raises ImportError when it is missing (build it with
``python paged_kv_cache_139_amd/build.py``): there is no fallback.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedkv.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing; build it with "
                      "`python paged_kv_cache_139_amd/build.py`")
_lib = ctypes.CDLL(LIB_PATH)

# pkv_dtype
F32, F16, BF16, FP8_E4M3 = 0, 1, 2, 3
BLOCK_SIZE = 16
DEFAULT_PARTITION_SIZE = 2048

_c_i32 = ctypes.c_int32
_c_f32 = ctypes.c_float
_vp = ctypes.c_void_p

_lib.pkv_status_string.restype = ctypes.c_char_p
_lib.pkv_status_string.argtypes = [ctypes.c_int]
_lib.reshape_and_cache.restype = ctypes.c_int
_lib.reshape_and_cache.argtypes = [_vp, _vp, _vp, _vp, _vp, _c_i32, _c_i32, _c_i32, _c_i32,
                                   _c_i32, ctypes.c_int, ctypes.c_int, _c_f32, _c_f32, _vp]
_lib.paged_attention_decode_workspace_bytes.restype = ctypes.c_size_t
_lib.paged_attention_decode_workspace_bytes.argtypes = [_c_i32] * 6
_lib.paged_attention_decode.restype = ctypes.c_int
_lib.paged_attention_decode.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _c_i32, _c_i32, _c_i32,
                                        _c_i32, _c_i32, _c_i32, _c_i32, _c_f32, ctypes.c_int,
                                        ctypes.c_int, _c_f32, _c_f32, _c_i32, _vp,
                                        ctypes.c_size_t, _vp]
_lib.paged_attention_decode_noalloc.restype = ctypes.c_int
_lib.paged_attention_decode_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _c_i32, _c_i32,
                                                 _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_f32,
                                                 ctypes.c_int, ctypes.c_int, _c_f32, _c_f32,
                                                 _c_i32, _vp]
_lib.paged_kv_gather.restype = ctypes.c_int
_lib.paged_attention_decode_append.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_i32,
                                                _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                                ctypes.c_float, ctypes.c_int, ctypes.c_int,
                                                ctypes.c_float, ctypes.c_float, _c_i32, _vp,
                                                ctypes.c_size_t, _vp]
_lib.paged_attention_decode_append.restype = ctypes.c_int
_lib.paged_kv_gather.argtypes = [_vp, _vp, _vp, _vp, _vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                 ctypes.c_int, _vp]
_c_i64 = ctypes.c_int64
_lib.reshape_and_cache_strided.restype = ctypes.c_int
_lib.reshape_and_cache_strided.argtypes = [_vp, _vp, _vp, _vp, _vp, _c_i32, _c_i32, _c_i32,
                                           _c_i32, _c_i32, _c_i64, _c_i64, ctypes.c_int,
                                           ctypes.c_int, _c_f32, _c_f32, _vp]
_lib.paged_attention_decode_strided.restype = ctypes.c_int
_lib.paged_attention_decode_strided.argtypes = [
    _vp, _vp, _vp, _vp, _vp, _vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
    _c_i64, _c_i64, _c_f32, ctypes.c_int, ctypes.c_int, _c_f32, _c_f32, _c_i32, _vp,
    ctypes.c_size_t, _vp]
_lib.paged_attention_decode_append_strided.restype = ctypes.c_int
_lib.paged_attention_decode_append_strided.argtypes = [
    _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
    _c_i32, _c_i64, _c_i64, _c_i64, _c_i64, _c_f32, ctypes.c_int, ctypes.c_int, _c_f32, _c_f32,
    _c_i32, _vp, ctypes.c_size_t, _vp]

_lib.paged_attention_decode_shared_prefix_workspace_bytes.restype = ctypes.c_size_t
_lib.paged_attention_decode_shared_prefix_workspace_bytes.argtypes = [_c_i32] * 6
_lib.paged_attention_decode_shared_prefix.restype = ctypes.c_int
_lib.paged_attention_decode_shared_prefix.argtypes = [
    _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
    _c_i32, _c_i32, _c_i32, _c_f32, ctypes.c_int, ctypes.c_int, _c_f32, _c_f32, _c_i32, _vp,
    ctypes.c_size_t, _vp]
_lib.paged_attention_decode_shared_prefix_append.restype = ctypes.c_int
_lib.paged_attention_decode_shared_prefix_append.argtypes = [
    _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
    _c_i32, _c_i32, _c_i32, _c_i32, _c_f32, ctypes.c_int, ctypes.c_int, _c_f32, _c_f32, _c_i32,
    _vp, ctypes.c_size_t, _vp]
_lib.copy_blocks.restype = ctypes.c_int
_lib.copy_blocks.argtypes = [ctypes.POINTER(_vp), ctypes.POINTER(_vp), _c_i32, _vp, _c_i32,
                             _c_i32, _c_i32, _c_i32, _c_i32, ctypes.c_int, _vp]

_i64p = ctypes.POINTER(ctypes.c_int64)
_i32p = ctypes.POINTER(ctypes.c_int32)
_lib.pkv_bm_create.restype = ctypes.c_int
_lib.pkv_bm_create.argtypes = [_c_i32, _c_i32, ctypes.POINTER(_vp)]
_lib.pkv_bm_destroy.restype = None
_lib.pkv_bm_destroy.argtypes = [_vp]
_lib.pkv_bm_num_free_blocks.restype = ctypes.c_int32
_lib.pkv_bm_num_free_blocks.argtypes = [_vp]
_lib.pkv_bm_add_sequence.restype = ctypes.c_int
_lib.pkv_bm_add_sequence.argtypes = [_vp, ctypes.c_int64, ctypes.c_int64]
_lib.pkv_bm_fork.restype = ctypes.c_int
_lib.pkv_bm_fork.argtypes = [_vp, ctypes.c_int64, ctypes.c_int64]
_lib.pkv_bm_free_sequence.restype = ctypes.c_int
_lib.pkv_bm_free_sequence.argtypes = [_vp, ctypes.c_int64]
_lib.pkv_bm_append_tokens.restype = ctypes.c_int
_lib.pkv_bm_append_tokens.argtypes = [_vp, _i64p, _c_i32, _i64p, _i64p, _i32p, _i32p]
_lib.pkv_bm_get_block_table.restype = ctypes.c_int
_lib.pkv_bm_get_block_table.argtypes = [_vp, ctypes.c_int64, _i32p, _c_i32, _i32p, _i64p]
_lib.pkv_bm_token_slots.restype = ctypes.c_int
_lib.pkv_bm_token_slots.argtypes = [_vp, ctypes.c_int64, ctypes.c_int64, _c_i32, _i64p]
_lib.pkv_bm_num_cached_blocks.restype = ctypes.c_int32
_lib.pkv_bm_num_cached_blocks.argtypes = [_vp]
_lib.pkv_bm_add_sequence_cached.restype = ctypes.c_int
_lib.pkv_bm_add_sequence_cached.argtypes = [_vp, ctypes.c_int64, _i64p, ctypes.c_int64, _i64p]
_lib.pkv_bm_build_block_tables.restype = ctypes.c_int
_lib.pkv_bm_build_block_tables.argtypes = [_vp, _i64p, _c_i32, _c_i32, _i32p, _i32p]

EXPORTED = ("pkv_status_string", "reshape_and_cache", "reshape_and_cache_strided",
            "paged_attention_decode_workspace_bytes", "paged_attention_decode",
            "paged_attention_decode_strided", "paged_attention_decode_noalloc",
            "paged_attention_decode_append",
            "paged_attention_decode_append_strided", "paged_kv_gather",
            "copy_blocks",
            "paged_attention_decode_shared_prefix_workspace_bytes",
            "paged_attention_decode_shared_prefix",
            "paged_attention_decode_shared_prefix_append", "pkv_bm_create", "pkv_bm_destroy",
            "pkv_bm_num_free_blocks", "pkv_bm_add_sequence", "pkv_bm_fork",
            "pkv_bm_free_sequence", "pkv_bm_append_tokens", "pkv_bm_get_block_table",
            "pkv_bm_token_slots", "pkv_bm_build_block_tables", "pkv_bm_num_cached_blocks",
            "pkv_bm_add_sequence_cached")


class PagedKVError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_lib.pkv_status_string(status).decode()} (status {status})")


def raw():
    """The loaded ctypes library (for direct C-ABI calls)."""
    return _lib


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.float16:
        return F16
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _check(status: int, where: str):
    if status != 0:
        raise PagedKVError(status, where)


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _row_stride(t, what):
    """Row stride (elements) of a [N, A, D] device tensor whose rows may be spaced
    apart (a view into a wider buffer) but whose [A, D] part is packed."""
    _need(t.is_cuda and t.dim() == 3, f"{what} must be a [N, A, D] device tensor")
    n, a, d = t.shape
    if t.is_contiguous():
        return a * d
    _need((t.stride(2) == 1 or d == 1) and (t.stride(1) == d or a == 1),
          f"{what}: heads and elements of a row must be packed")
    return t.stride(0)


def reshape_and_cache(key, value, key_cache, value_cache, slot_mapping, k_scale=1.0,
                      v_scale=1.0):
    """Write key/value [T, Hk, D] into the caches [NB, Hk, D, BS] at slot_mapping [T] (int64).
    key / value may be row-strided views (e.g. parts of a fused QKV output)."""
    for t in (key_cache, value_cache, slot_mapping):
        _need(t.is_cuda and t.is_contiguous(), "caches and slots must be contiguous device tensors")
    ks, vs = _row_stride(key, "key"), _row_stride(value, "value")
    _need(slot_mapping.dtype == torch.int64, "slot_mapping must be int64")
    T, Hk, D = key.shape
    NB, Hk2, D2, BS = key_cache.shape
    _need(value.shape == key.shape and value_cache.shape == key_cache.shape, "shape mismatch")
    _need((Hk2, D2) == (Hk, D) and slot_mapping.shape == (T,), "shape mismatch")
    _need(key.dtype == value.dtype and key_cache.dtype == value_cache.dtype, "dtype mismatch")
    if ks == Hk * D and vs == Hk * D:
        st = _lib.reshape_and_cache(_ptr(key), _ptr(value), _ptr(key_cache), _ptr(value_cache),
                                    _ptr(slot_mapping), T, Hk, D, BS, NB, _dtype_code(key),
                                    _dtype_code(key_cache), float(k_scale), float(v_scale),
                                    _stream(key))
    else:
        st = _lib.reshape_and_cache_strided(
            _ptr(key), _ptr(value), _ptr(key_cache), _ptr(value_cache), _ptr(slot_mapping), T,
            Hk, D, BS, NB, ks, vs, _dtype_code(key), _dtype_code(key_cache), float(k_scale),
            float(v_scale), _stream(key))
    _check(st, "reshape_and_cache")


def workspace_bytes(num_seqs, num_heads, head_size, max_num_blocks_per_seq,
                    partition_size=0, block_size=BLOCK_SIZE) -> int:
    return int(_lib.paged_attention_decode_workspace_bytes(num_seqs, num_heads, head_size,
                                                            max_num_blocks_per_seq, block_size,
                                                            partition_size))


def alloc_workspace(num_seqs, num_heads, head_size, max_num_blocks_per_seq, device,
                    partition_size=0, block_size=BLOCK_SIZE):
    n = workspace_bytes(num_seqs, num_heads, head_size, max_num_blocks_per_seq, partition_size,
                        block_size)
    return torch.empty(max(n, 4) // 4, dtype=torch.float32, device=device)


def paged_attention_decode(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                           k_scale=1.0, v_scale=1.0, partition_size=0, workspace=None):
    """out, query [S, H, D]; caches [NB, Hk, D, BS]; block_tables [S, MB] int32; context_lens [S]
    int32.  query and out may be row-strided views (e.g. the query part of a fused QKV output)."""
    for t in (key_cache, value_cache, block_tables, context_lens):
        _need(t.is_cuda and t.is_contiguous(), "caches and tables must be contiguous device tensors")
    qs, os_ = _row_stride(query, "query"), _row_stride(out, "out")
    _need(block_tables.dtype == torch.int32 and context_lens.dtype == torch.int32,
          "block_tables and context_lens must be int32")
    S, H, D = query.shape
    NB, Hk, D2, BS = key_cache.shape
    MB = block_tables.shape[1]
    _need(out.shape == query.shape and out.dtype == query.dtype, "out must match query")
    _need(value_cache.shape == key_cache.shape and D2 == D, "cache shape mismatch")
    _need(block_tables.shape[0] == S and context_lens.shape == (S,), "table shape mismatch")
    need = workspace_bytes(S, H, D, MB, partition_size, BS)
    if need and workspace is None:
        workspace = alloc_workspace(S, H, D, MB, query.device, partition_size, BS)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if qs == H * D and os_ == H * D:
        st = _lib.paged_attention_decode(
            _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
            _ptr(context_lens), S, H, Hk, D, BS, MB, NB, float(scale), _dtype_code(query),
            _dtype_code(key_cache), float(k_scale), float(v_scale), int(partition_size),
            _ptr(workspace), ws_bytes, _stream(query))
    else:
        st = _lib.paged_attention_decode_strided(
            _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
            _ptr(context_lens), S, H, Hk, D, BS, MB, NB, qs, os_, float(scale),
            _dtype_code(query), _dtype_code(key_cache), float(k_scale), float(v_scale),
            int(partition_size), _ptr(workspace), ws_bytes, _stream(query))
    _check(st, "paged_attention_decode")
    return out


NOALLOC_SCRATCH_BYTES = 32 << 20      # PKV_NOALLOC_SCRATCH_BYTES


def paged_attention_decode_noalloc(out, query, key_cache, value_cache, block_tables,
                                   context_lens, scale, k_scale=1.0, v_scale=1.0,
                                   partition_size=0):
    """paged_attention_decode with no workspace: partition results go to the
    library's static per-GPU scratch (see the header for its limit and for
    overlapping calls).  Packed tensors only."""
    for t in (out, query, key_cache, value_cache, block_tables, context_lens):
        _need(t.is_cuda and t.is_contiguous(), "tensors must be contiguous device tensors")
    _need(block_tables.dtype == torch.int32 and context_lens.dtype == torch.int32,
          "block_tables and context_lens must be int32")
    S, H, D = query.shape
    NB, Hk, D2, BS = key_cache.shape
    MB = block_tables.shape[1]
    _need(out.shape == query.shape and out.dtype == query.dtype, "out must match query")
    _need(value_cache.shape == key_cache.shape and D2 == D, "cache shape mismatch")
    _need(block_tables.shape[0] == S and context_lens.shape == (S,), "table shape mismatch")
    st = _lib.paged_attention_decode_noalloc(
        _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
        _ptr(context_lens), S, H, Hk, D, BS, MB, NB, float(scale), _dtype_code(query),
        _dtype_code(key_cache), float(k_scale), float(v_scale), int(partition_size),
        _stream(query))
    _check(st, "paged_attention_decode_noalloc")
    return out


def paged_attention_decode_append(out, query, key_new, value_new, key_cache, value_cache,
                                  block_tables, context_lens, scale, k_scale=1.0, v_scale=1.0,
                                  partition_size=0, workspace=None):
    """One decode step: key_new / value_new [S, Hk, D] (query dtype) are stored at each
    sequence's position context_lens[s] - 1, then the decode attends (see the header).
    query, key_new, value_new and out may be row-strided views (a fused QKV output)."""
    for t in (key_cache, value_cache, block_tables, context_lens):
        _need(t.is_cuda and t.is_contiguous(), "caches and tables must be contiguous device tensors")
    qs, os_ = _row_stride(query, "query"), _row_stride(out, "out")
    kns, vns = _row_stride(key_new, "key_new"), _row_stride(value_new, "value_new")
    _need(block_tables.dtype == torch.int32 and context_lens.dtype == torch.int32,
          "block_tables and context_lens must be int32")
    S, H, D = query.shape
    NB, Hk, D2, BS = key_cache.shape
    MB = block_tables.shape[1]
    _need(out.shape == query.shape and out.dtype == query.dtype, "out must match query")
    _need(value_cache.shape == key_cache.shape and D2 == D, "cache shape mismatch")
    _need(block_tables.shape[0] == S and context_lens.shape == (S,), "table shape mismatch")
    _need(key_new.shape == (S, Hk, D) and value_new.shape == key_new.shape and
          key_new.dtype == query.dtype and value_new.dtype == query.dtype,
          "key_new / value_new must be [S, Hk, D] in the query dtype")
    need = workspace_bytes(S, H, D, MB, partition_size, BS)
    if need and workspace is None:
        workspace = alloc_workspace(S, H, D, MB, query.device, partition_size, BS)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if (qs, os_, kns, vns) == (H * D, H * D, Hk * D, Hk * D):
        st = _lib.paged_attention_decode_append(
            _ptr(out), _ptr(query), _ptr(key_new), _ptr(value_new), _ptr(key_cache),
            _ptr(value_cache), _ptr(block_tables), _ptr(context_lens), S, H, Hk, D, BS, MB, NB,
            float(scale), _dtype_code(query), _dtype_code(key_cache), float(k_scale),
            float(v_scale), int(partition_size), _ptr(workspace), ws_bytes, _stream(query))
    else:
        st = _lib.paged_attention_decode_append_strided(
            _ptr(out), _ptr(query), _ptr(key_new), _ptr(value_new), _ptr(key_cache),
            _ptr(value_cache), _ptr(block_tables), _ptr(context_lens), S, H, Hk, D, BS, MB, NB,
            qs, kns, vns, os_, float(scale), _dtype_code(query), _dtype_code(key_cache),
            float(k_scale), float(v_scale), int(partition_size), _ptr(workspace), ws_bytes,
            _stream(query))
    _check(st, "paged_attention_decode_append")
    return out


def shared_prefix_workspace_bytes(num_seqs, num_heads, head_size, max_num_blocks_per_seq,
                                  partition_size=0, block_size=BLOCK_SIZE) -> int:
    return int(_lib.paged_attention_decode_shared_prefix_workspace_bytes(
        num_seqs, num_heads, head_size, max_num_blocks_per_seq, block_size, partition_size))


def alloc_shared_prefix_workspace(num_seqs, num_heads, head_size, max_num_blocks_per_seq, device,
                                  partition_size=0):
    n = shared_prefix_workspace_bytes(num_seqs, num_heads, head_size, max_num_blocks_per_seq,
                                      partition_size)
    return torch.empty(max(n, 4) // 4, dtype=torch.float32, device=device)


def paged_attention_decode_shared_prefix(out, query, key_cache, value_cache, block_tables,
                                         context_lens, group_starts, group_prefix_blocks,
                                         max_group_size, scale, k_scale=1.0, v_scale=1.0,
                                         partition_size=0, workspace=None):
    """As paged_attention_decode, for sequences in groups that share prefix blocks:
    group_starts [G + 1] and group_prefix_blocks [G] are int32 device tensors."""
    for t in (out, query, key_cache, value_cache, block_tables, context_lens, group_starts,
              group_prefix_blocks):
        _need(t.is_cuda and t.is_contiguous(), "tensors must be contiguous device tensors")
    for t in (block_tables, context_lens, group_starts, group_prefix_blocks):
        _need(t.dtype == torch.int32, "index tensors must be int32")
    S, H, D = query.shape
    NB, Hk, D2, BS = key_cache.shape
    MB = block_tables.shape[1]
    G = group_prefix_blocks.shape[0]
    _need(group_starts.shape == (G + 1,), "group_starts must have num_groups + 1 entries")
    _need(out.shape == query.shape and out.dtype == query.dtype, "out must match query")
    _need(value_cache.shape == key_cache.shape and D2 == D, "cache shape mismatch")
    _need(block_tables.shape[0] == S and context_lens.shape == (S,), "table shape mismatch")
    if workspace is None:
        workspace = alloc_shared_prefix_workspace(S, H, D, MB, query.device, partition_size)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = _lib.paged_attention_decode_shared_prefix(
        _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
        _ptr(context_lens), _ptr(group_starts), _ptr(group_prefix_blocks), G,
        int(max_group_size), S, H, Hk, D, BS, MB, NB, float(scale), _dtype_code(query),
        _dtype_code(key_cache), float(k_scale), float(v_scale), int(partition_size),
        _ptr(workspace), ws_bytes, _stream(query))
    _check(st, "paged_attention_decode_shared_prefix")
    return out


def paged_attention_decode_shared_prefix_append(out, query, key_new, value_new, key_cache,
                                                value_cache, block_tables, context_lens,
                                                group_starts, group_prefix_blocks,
                                                max_group_size, scale, k_scale=1.0, v_scale=1.0,
                                                partition_size=0):
    """One decode step of a shared-prefix batch: key_new / value_new [S, Hk, D] (query
    dtype) are stored at each sequence's position context_lens[s] - 1 (not inside its
    group's shared prefix), then the shared-prefix decode attends (grouped heads only:
    2 <= H / Hk <= 16)."""
    for t in (out, query, key_new, value_new, key_cache, value_cache, block_tables,
              context_lens, group_starts, group_prefix_blocks):
        _need(t.is_cuda and t.is_contiguous(), "tensors must be contiguous device tensors")
    for t in (block_tables, context_lens, group_starts, group_prefix_blocks):
        _need(t.dtype == torch.int32, "index tensors must be int32")
    S, H, D = query.shape
    NB, Hk, D2, BS = key_cache.shape
    MB = block_tables.shape[1]
    G = group_prefix_blocks.shape[0]
    _need(group_starts.shape == (G + 1,), "group_starts must have num_groups + 1 entries")
    _need(out.shape == query.shape and out.dtype == query.dtype, "out must match query")
    _need(value_cache.shape == key_cache.shape and D2 == D, "cache shape mismatch")
    _need(block_tables.shape[0] == S and context_lens.shape == (S,), "table shape mismatch")
    _need(key_new.shape == (S, Hk, D) and value_new.shape == key_new.shape and
          key_new.dtype == query.dtype and value_new.dtype == query.dtype,
          "key_new / value_new must be [S, Hk, D] in the query dtype")
    st = _lib.paged_attention_decode_shared_prefix_append(
        _ptr(out), _ptr(query), _ptr(key_new), _ptr(value_new), _ptr(key_cache),
        _ptr(value_cache), _ptr(block_tables), _ptr(context_lens), _ptr(group_starts),
        _ptr(group_prefix_blocks), G, int(max_group_size), S, H, Hk, D, BS, MB, NB, float(scale),
        _dtype_code(query), _dtype_code(key_cache), float(k_scale), float(v_scale),
        int(partition_size), None, 0, _stream(query))
    _check(st, "paged_attention_decode_shared_prefix_append")
    return out


def paged_kv_gather(key_cache, value_cache, block_table_row, context_len):
    """Logical K and V of one sequence, [L, Hk, D] each, read through its block table row."""
    NB, Hk, D, BS = key_cache.shape
    L = int(context_len)
    k_out = torch.empty((L, Hk, D), dtype=key_cache.dtype, device=key_cache.device)
    v_out = torch.empty_like(k_out)
    _need(block_table_row.dtype == torch.int32 and block_table_row.is_cuda, "int32 device table")
    st = _lib.paged_kv_gather(_ptr(k_out), _ptr(v_out), _ptr(key_cache), _ptr(value_cache),
                              _ptr(block_table_row), L, Hk, D, BS, NB, _dtype_code(key_cache),
                              _stream(key_cache))
    _check(st, "paged_kv_gather")
    return k_out, v_out


def copy_blocks(key_caches, value_caches, block_mapping):
    """Copy-on-write block copy: for each row (src, dst) of block_mapping
    ([n, 2] int64, device), block dst of every cache in key_caches /
    value_caches (lists of [NB, Hk, D, 16] device tensors, one per layer)
    becomes a copy of block src."""
    _need(len(key_caches) == len(value_caches), "one value cache per key cache")
    _need(block_mapping.is_cuda and block_mapping.is_contiguous()
          and block_mapping.dtype == torch.int64
          and block_mapping.dim() == 2 and block_mapping.shape[1] == 2,
          "block_mapping must be a contiguous [n, 2] int64 device tensor")
    n_layers = len(key_caches)
    if n_layers == 0:
        return
    shape, dtype = key_caches[0].shape, key_caches[0].dtype
    for t in list(key_caches) + list(value_caches):
        _need(t.is_cuda and t.is_contiguous(), "caches must be contiguous device tensors")
        _need(t.shape == shape and t.dtype == dtype, "all caches must have one shape and dtype")
    NB, Hk, D, BS = shape
    karr = (_vp * n_layers)(*[t.data_ptr() for t in key_caches])
    varr = (_vp * n_layers)(*[t.data_ptr() for t in value_caches])
    st = _lib.copy_blocks(karr, varr, n_layers, _ptr(block_mapping), block_mapping.shape[0], Hk,
                          D, BS, NB, _dtype_code(key_caches[0]), _stream(key_caches[0]))
    _check(st, "copy_blocks")


class BlockManager:
    """Host block manager of the library (free list, block tables, reference
    counts, fork, copy-on-write appends).  Errors raise PagedKVError with the
    status (PKV_ERR_NO_BLOCKS = 9, PKV_ERR_SEQUENCE = 10, ...)."""

    NO_BLOCKS, SEQUENCE = 9, 10

    def __init__(self, num_blocks: int, block_size: int = BLOCK_SIZE):
        h = _vp()
        _check(_lib.pkv_bm_create(num_blocks, block_size, ctypes.byref(h)), "pkv_bm_create")
        self._h = h
        self.block_size = block_size

    def close(self):
        if self._h:
            _lib.pkv_bm_destroy(self._h)
            self._h = _vp()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def num_free(self) -> int:
        return int(_lib.pkv_bm_num_free_blocks(self._h))

    def add_sequence(self, seq_id: int, num_tokens: int):
        _check(_lib.pkv_bm_add_sequence(self._h, seq_id, num_tokens), "pkv_bm_add_sequence")

    def add_sequence_cached(self, seq_id: int, tokens) -> int:
        """New sequence for a prompt of token ids, sharing cached blocks of the same
        leading tokens; returns the number of leading tokens already cached."""
        n = len(tokens)
        buf = (ctypes.c_int64 * max(n, 1))(*[int(t) for t in tokens])
        cached = ctypes.c_int64()
        _check(_lib.pkv_bm_add_sequence_cached(self._h, seq_id, buf, n, ctypes.byref(cached)),
               "pkv_bm_add_sequence_cached")
        return cached.value

    def num_cached(self) -> int:
        return int(_lib.pkv_bm_num_cached_blocks(self._h))

    def fork(self, parent: int, child: int):
        _check(_lib.pkv_bm_fork(self._h, parent, child), "pkv_bm_fork")

    def free_sequence(self, seq_id: int):
        _check(_lib.pkv_bm_free_sequence(self._h, seq_id), "pkv_bm_free_sequence")

    def append_tokens(self, seq_ids):
        """One token per sequence: (slots, copy pairs, number done); on error
        the exception carries .slots / .pairs / .done of the appends made."""
        n = len(seq_ids)
        ids = (ctypes.c_int64 * max(n, 1))(*seq_ids)
        slots = (ctypes.c_int64 * max(n, 1))()
        pairs = (ctypes.c_int64 * max(2 * n, 2))()
        ncopy, ndone = ctypes.c_int32(), ctypes.c_int32()
        st = _lib.pkv_bm_append_tokens(self._h, ids, n, slots, pairs, ctypes.byref(ncopy),
                                       ctypes.byref(ndone))
        out_slots = list(slots[:ndone.value])
        out_pairs = [(pairs[2 * i], pairs[2 * i + 1]) for i in range(ncopy.value)]
        if st != 0:
            e = PagedKVError(st, "pkv_bm_append_tokens")
            e.slots, e.pairs, e.done = out_slots, out_pairs, ndone.value
            raise e
        return out_slots, out_pairs, ndone.value

    def table(self, seq_id: int):
        nb, nt = ctypes.c_int32(), ctypes.c_int64()
        st = _lib.pkv_bm_get_block_table(self._h, seq_id, None, 0, ctypes.byref(nb),
                                         ctypes.byref(nt))
        if st not in (0, 2):                      # 2: no room -- expected with capacity 0
            _check(st, "pkv_bm_get_block_table")
        buf = (ctypes.c_int32 * max(nb.value, 1))()
        _check(_lib.pkv_bm_get_block_table(self._h, seq_id, buf, nb.value, ctypes.byref(nb),
                                           ctypes.byref(nt)), "pkv_bm_get_block_table")
        return list(buf[:nb.value]), nt.value

    def token_slots(self, seq_id: int, first: int, count: int):
        buf = (ctypes.c_int64 * max(count, 1))()
        _check(_lib.pkv_bm_token_slots(self._h, seq_id, first, count, buf), "pkv_bm_token_slots")
        return list(buf[:count])

    def build_block_tables(self, seq_ids, max_blocks_per_seq: int):
        """(block_tables [n, MB] int32, context_lens [n] int32) as numpy arrays."""
        import numpy as np
        n = len(seq_ids)
        bt = np.empty((max(n, 1), max_blocks_per_seq), np.int32)
        lens = np.empty(max(n, 1), np.int32)
        ids = (ctypes.c_int64 * max(n, 1))(*seq_ids)
        _check(_lib.pkv_bm_build_block_tables(
            self._h, ids, n, max_blocks_per_seq, bt.ctypes.data_as(_i32p),
            lens.ctypes.data_as(_i32p)), "pkv_bm_build_block_tables")
        return bt[:n], lens[:n]
