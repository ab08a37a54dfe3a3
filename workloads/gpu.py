"""Put a Workload on the GPU and fill its paged pools through the library.

Used by the GPU tests, bench.py and smoke().  Never imports the oracle.
Pools start as poison (NaN, or the E4M3 NaN code 0x7F) so that any read of a
slot outside a sequence's context shows up in the output.
"""
from __future__ import annotations

import numpy as np
import torch

import paged_kv_cache_139_amd as pkv

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
               "fp8": torch.uint8}


def to_device(a: np.ndarray, fmt: str, device) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if fmt == "bf16":
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a)
    return t.to(device)


def poison_pool(shape, fmt: str, device) -> torch.Tensor:
    if fmt == "fp8":
        return torch.full(shape, 0x7F, dtype=torch.uint8, device=device)
    return torch.full(shape, float("nan"), dtype=TORCH_DTYPE[fmt], device=device)


def to_numpy_storage(t: torch.Tensor, fmt: str) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if fmt == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


class DeviceWorkload:
    """Device copies of a workload's inputs, its pools and its output."""

    def __init__(self, w, device="cuda:0", partition_size: int = 0, shared_prefix: bool = False):
        """shared_prefix: decode() uses the shared-prefix entry point with the
        workload's sharing groups (every other sequence a group of one)."""
        self.w = w
        self.device = torch.device(device)
        self.partition_size = partition_size
        self.shared_prefix = shared_prefix
        shape = (w.NB, w.Hk, w.D, w.BS)
        self.k_cache = poison_pool(shape, w.cache_fmt, self.device)
        self.v_cache = poison_pool(shape, w.cache_fmt, self.device)
        self.query = to_device(w.query, w.q_fmt, self.device)
        self.block_tables = torch.from_numpy(w.block_tables).to(self.device)
        self.context_lens = torch.from_numpy(w.context_lens).to(self.device)
        self.key_new = to_device(w.key_new, w.src_fmt, self.device)
        self.value_new = to_device(w.value_new, w.src_fmt, self.device)
        self.slot_new = torch.from_numpy(w.slot_new).to(self.device)
        self.out = torch.empty_like(self.query)
        if shared_prefix:
            starts, prefix, self.max_group = w.group_arrays()
            self.group_starts = torch.from_numpy(starts).to(self.device)
            self.group_prefix = torch.from_numpy(prefix).to(self.device)
            self.workspace = pkv.alloc_shared_prefix_workspace(w.S, w.H, w.D, w.MB, self.device,
                                                               partition_size)
        else:
            self.workspace = pkv.alloc_workspace(w.S, w.H, w.D, w.MB, self.device,
                                                 partition_size, w.BS)

    def fill(self, chunk_tokens: int = 1 << 16):
        """Bulk-write every token but each sequence's last, in chunks."""
        w = self.w
        T = len(w.slot_bulk)
        for a in range(0, T, chunk_tokens):
            b = min(T, a + chunk_tokens)
            k = to_device(w.key_bulk[a:b], w.src_fmt, self.device)
            v = to_device(w.value_bulk[a:b], w.src_fmt, self.device)
            s = torch.from_numpy(w.slot_bulk[a:b]).to(self.device)
            pkv.reshape_and_cache(k, v, self.k_cache, self.v_cache, s, w.k_scale, w.v_scale)
        return self

    def write_new(self):
        w = self.w
        pkv.reshape_and_cache(self.key_new, self.value_new, self.k_cache, self.v_cache,
                              self.slot_new, w.k_scale, w.v_scale)

    def decode(self, out=None):
        w = self.w
        out = self.out if out is None else out
        if self.shared_prefix:
            pkv.paged_attention_decode_shared_prefix(
                out, self.query, self.k_cache, self.v_cache, self.block_tables,
                self.context_lens, self.group_starts, self.group_prefix, self.max_group,
                w.scale, w.k_scale, w.v_scale, self.partition_size, self.workspace)
        else:
            pkv.paged_attention_decode(out, self.query, self.k_cache, self.v_cache,
                                       self.block_tables, self.context_lens, w.scale, w.k_scale,
                                       w.v_scale, self.partition_size, self.workspace)
        return out

    def decode_append(self, out=None):
        """The decode step in one call: store each sequence's new token, then attend
        (through the shared-prefix call when the workload was set up for it)."""
        w = self.w
        out = self.out if out is None else out
        if self.shared_prefix:
            return pkv.paged_attention_decode_shared_prefix_append(
                out, self.query, self.key_new, self.value_new, self.k_cache, self.v_cache,
                self.block_tables, self.context_lens, self.group_starts, self.group_prefix,
                self.max_group, w.scale, w.k_scale, w.v_scale, self.partition_size)
        return pkv.paged_attention_decode_append(
            out, self.query, self.key_new, self.value_new, self.k_cache, self.v_cache,
            self.block_tables, self.context_lens, w.scale, w.k_scale, w.v_scale,
            self.partition_size, self.workspace)

    def step(self):
        """One pass of the hot path: append the decode token, then attend."""
        self.write_new()
        return self.decode()

    def out_f64(self) -> np.ndarray:
        return self.out.detach().float().cpu().numpy().astype(np.float64)
