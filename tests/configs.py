"""The five synthetic step configurations for the GPU parity tests, with their
oracle pools and full oracle outputs, each built once per test session.

Building the larger configurations and running the fp64 oracle over every
one of their output rows takes seconds to tens of seconds of host time, and
several test files check the same configuration (bf16 and 8-bit pools,
plain and shared-prefix attention), so the results are memoised here.
Callers must not modify what these functions return.
"""
from __future__ import annotations

import functools

import numpy as np

import oracle
import workloads as W

# one fp32 scale per 8-bit pool (amax / 448 of N(0,1) bf16 data)
FP8_SCALES = (0.011, 0.0107)
SENTINEL8 = 0x7F  # the E4M3 NaN code: an unwritten byte read by mistake shows as NaN


@functools.lru_cache(maxsize=None)
def workload(k: int, shared: bool = True) -> W.Workload:
    return W.make_config(k, shared=shared)


@functools.lru_cache(maxsize=None)
def pool(k: int):
    """The oracle's scatter of configuration k's cached and new tokens into
    NaN-filled bf16 pools (every slot it does not write stays NaN)."""
    w = workload(k)
    kc = np.full(w.pool_elems(), W.BF16_NAN, np.uint16)
    vc = np.full(w.pool_elems(), W.BF16_NAN, np.uint16)
    oracle.write_kv(kc, vc, w.k_dense[w.fill_rows], w.v_dense[w.fill_rows], w.fill_slots)
    oracle.write_kv(kc, vc, w.k_new, w.v_new, w.new_slots)
    return kc, vc


@functools.lru_cache(maxsize=None)
def attend(k: int) -> np.ndarray:
    """The oracle's attention, every output row of configuration k
    ([T][Hq][D] fp64)."""
    w = workload(k)
    kc, vc = pool(k)
    return oracle.attend(w.q, kc, vc, w.block_tables, w.seq_lens, w.query_start_loc,
                         w.num_kv_heads, w.scale)


@functools.lru_cache(maxsize=None)
def pool8(k: int):
    """The oracle's 8-bit scatter of configuration k (FP8_SCALES) into pools
    filled with the NaN code."""
    w = workload(k)
    ks, vs = FP8_SCALES
    kc = np.full(w.pool_elems(), SENTINEL8, np.uint8)
    vc = kc.copy()
    oracle.write_kv_fp8(kc, vc, w.k_dense[w.fill_rows], w.v_dense[w.fill_rows],
                        w.fill_slots, ks, vs)
    oracle.write_kv_fp8(kc, vc, w.k_new, w.v_new, w.new_slots, ks, vs)
    return kc, vc


@functools.lru_cache(maxsize=None)
def attend8(k: int) -> np.ndarray:
    """The oracle's attention over the 8-bit pools of configuration k, every
    output row."""
    w = workload(k)
    kc, vc = pool8(k)
    return oracle.attend_fp8(w.q, kc, vc, *FP8_SCALES, w.block_tables, w.seq_lens,
                             w.query_start_loc, w.num_kv_heads, w.scale)
