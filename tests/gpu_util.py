"""GPU-side helpers for the parity tests and the benchmark (no attention
arithmetic here: uploads and launches through the library only)."""
from __future__ import annotations

import numpy as np
import torch

import paged_kv_cache_varlen_amd as pa
import workloads as W

DEV = "cuda"


def bf16_tensor(bits: np.ndarray, device=DEV) -> torch.Tensor:
    a = np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(a).view(torch.bfloat16).to(device)


def tensor_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def i32(a, device=DEV) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def i64(a, device=DEV) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int64)).to(device)


class Uploaded:
    """A workload on the GPU: pools filled through pa_write_kv."""

    def __init__(self, w: W.Workload, sentinel: bool = True, tables=None,
                 fill_slots=None, new_slots=None, write_new: bool = True):
        self.w = w
        fill = float("nan") if sentinel else 0.0
        self.k_cache, self.v_cache = pa.alloc_pool(w.num_blocks, w.num_kv_heads,
                                                   w.head_dim, fill=fill)
        self.q = bf16_tensor(w.q)
        bt = w.block_tables if tables is None else tables
        self.block_tables = i32(bt)
        self.seq_lens = i32(w.seq_lens)
        self.qsl = i32(w.query_start_loc)
        fs = w.fill_slots if fill_slots is None else fill_slots
        ns = w.new_slots if new_slots is None else new_slots
        self.k_new = bf16_tensor(w.k_new)
        self.v_new = bf16_tensor(w.v_new)
        self.new_slots = i64(ns)
        if len(w.fill_rows):
            step = 1 << 18  # bounded host->device staging
            for s in range(0, len(w.fill_rows), step):
                rows = w.fill_rows[s:s + step]
                pa.write_kv(bf16_tensor(w.k_dense[rows]), bf16_tensor(w.v_dense[rows]),
                            i64(fs[s:s + step]), self.k_cache, self.v_cache)
        if write_new:
            self.write_new()
        self.workspace = pa.alloc_workspace(
            w.num_seqs, w.num_q_tokens, w.num_q_heads, w.num_kv_heads,
            w.head_dim, w.max_query_len, w.max_seq_len)
        self.out = torch.empty_like(self.q)

    def write_new(self):
        pa.write_kv(self.k_new, self.v_new, self.new_slots, self.k_cache,
                    self.v_cache)

    def attend(self, out=None, k_cache=None, v_cache=None, planned=False,
               merge=True):
        w = self.w
        return pa.attend(self.q, self.k_cache if k_cache is None else k_cache,
                         self.v_cache if v_cache is None else v_cache,
                         self.block_tables, self.seq_lens, self.qsl, w.scale,
                         w.max_query_len, w.max_seq_len,
                         num_kv_heads=w.num_kv_heads,
                         out=self.out if out is None else out,
                         workspace=self.workspace, planned=planned, merge=merge)

    def merge(self, out=None):
        w = self.w
        pa.attend_merge(self.out if out is None else out, w.num_seqs,
                        w.num_kv_heads, w.max_query_len, w.max_seq_len,
                        self.workspace)

    def plan(self):
        w = self.w
        pa.attend_plan(self.block_tables, self.seq_lens, self.qsl,
                       w.num_q_tokens, w.num_q_heads, w.num_kv_heads, w.head_dim,
                       w.max_query_len, w.max_seq_len, self.workspace)
