"""Seeded synthetic inputs for the paged KV-cache varlen attention path.

This module is the only code that the HIP path's tests/benchmark and the CPU
oracle both consume.  It draws random numbers and builds the per-step metadata
a model runner would hand to the attention backend; it holds none of the
attention arithmetic and none of the pool layout.

What it builds, and where the pages state it:
  * query_start_loc: prefix sum of per-request scheduled token counts
    ("vLLM v1 Deep Dive", Part 3, Step 4c "Mixed batches").
  * block tables: per request an ordered list of physical block ids, any free
    block backing any logical block, ceil(N / block_size) blocks for N tokens
    ("vLLM: An Exhaustive Technical Study" section 2.1; "Inside the vLLM Engine", "A memory
    problem wearing a throughput costume").
  * slot_mapping: per written token, block_id * block_size + offset
    ("vLLM v1 Deep Dive", Aside "KV cache and prefix caching"; "vLLM: An Exhaustive Technical Study"
    section 2.1 "Reaching the kernel").
  * shared prefix blocks held by several block tables with a reference count
    equal to the number of tables that hold them (same Aside; "Deep Dive -
    vLLM", "Block pool, prefix cache, and eviction").

Values are N(0, 1) float32 draws from numpy's default_rng (one generator per
chunk of 2**22 values, keyed by (data seed, tensor, chunk)) rounded to bf16
(round to nearest even) and carried as uint16 bit patterns.  Workload shapes
follow the synthetic configurations described in the design notes (Llama-3-8B
and 70B-class GQA heads, 16-token blocks, decode, mixed chunked-prefill,
shared-prefix and long-context decode steps); the pages' own request traces
are not available, so these stand in for them.
"""
from __future__ import annotations

import os
from collections import deque
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

BLOCK_SIZE = 16
BF16_NAN = np.uint16(0x7FC0)


# ---- bf16 bit helpers ---------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits, round to nearest even (NaN kept quiet)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    out = ((u + rounding) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = BF16_NAN
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


_CHUNK = 1 << 22


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_bf16(key: Tuple[int, ...], shape) -> np.ndarray:
    """N(0,1) float32 draws rounded to bf16, as uint16 bits.

    Chunk i of 2**22 values comes from np.random.default_rng(key + (i,)), so
    the result depends only on the key and the shape, not on the number of
    threads that fill it."""
    n = int(np.prod(shape))
    out = np.empty(n, np.uint16)

    def fill(i):
        s, e = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        rng = np.random.default_rng(tuple(key) + (i,))
        out[s:e] = f32_to_bf16_bits(rng.standard_normal(e - s, dtype=np.float32))

    nchunks = (n + _CHUNK - 1) // _CHUNK
    if nchunks <= 1:
        for i in range(nchunks):
            fill(i)
    else:
        with ThreadPoolExecutor(max_workers=_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


# ---- runner metadata ------------------------------------------------------------

def cdiv(a: int, b: int) -> int:
    return -(-a // b)


def blocks_needed(num_tokens: int, block_size: int = BLOCK_SIZE) -> int:
    """Blocks allocated on demand for num_tokens tokens."""
    return cdiv(num_tokens, block_size)


def query_start_loc(query_lens: Sequence[int]) -> np.ndarray:
    """[0, q0, q0+q1, ...] as int32."""
    out = np.zeros(len(query_lens) + 1, np.int64)
    np.cumsum(np.asarray(query_lens, np.int64), out=out[1:])
    return out.astype(np.int32)


def logits_rows(qsl: np.ndarray) -> np.ndarray:
    """Last flattened row of each request's slice."""
    return np.asarray(qsl[1:], np.int64) - 1


def slots_for(block_row: Sequence[int], positions: np.ndarray,
              block_size: int = BLOCK_SIZE) -> np.ndarray:
    """Physical write slot of each logical position of one request."""
    row = np.asarray(block_row, np.int64)
    positions = np.asarray(positions, np.int64)
    return row[positions // block_size] * block_size + positions % block_size


class BlockPool:
    """Physical block ids with a reference count each (host-side test fixture).

    Free ids wait in a queue filled in a seeded random order, so that block
    tables are "a seeded random permutation of free blocks"; a block held by
    several tables (a shared prefix) counts one reference per table and
    rejoins the queue when its last holder lets it go.  The idea follows
    "Deep Dive - vLLM", section "Block pool, prefix cache, and eviction"."""

    def __init__(self, num_blocks: int, rng: np.random.Generator):
        self.num_blocks = int(num_blocks)
        self.ref_count = np.zeros(self.num_blocks, np.int64)
        self.free_ids = deque(int(i) for i in rng.permutation(self.num_blocks))

    def allocate(self, n: int) -> List[int]:
        """n blocks from the head of the free queue, each held once."""
        if len(self.free_ids) < n:
            raise MemoryError("KV block pool exhausted: %d blocks requested, %d free"
                              % (n, len(self.free_ids)))
        got = [self.free_ids.popleft() for _ in range(n)]
        self.ref_count[got] += 1
        return got

    def share(self, blocks: Sequence[int]) -> List[int]:
        """One more holder for blocks that are already held."""
        ids = np.asarray(list(blocks), np.int64)
        if ids.size and int(self.ref_count[ids].min()) < 1:
            raise ValueError("cannot share a block that nobody holds")
        np.add.at(self.ref_count, ids, 1)
        return [int(b) for b in ids]

    def release(self, blocks: Sequence[int]) -> None:
        """One holder fewer for each block; a block nobody holds any more
        rejoins the free queue."""
        for b in blocks:
            if self.ref_count[b] < 1:
                raise ValueError("block %d is not held" % b)
            self.ref_count[b] -= 1
            if self.ref_count[b] == 0:
                self.free_ids.append(int(b))

    @property
    def refs(self) -> Dict[int, int]:
        """Reference count of every held block."""
        return {int(b): int(self.ref_count[b]) for b in np.flatnonzero(self.ref_count)}

    def used(self) -> int:
        return int(np.count_nonzero(self.ref_count))


# ---- workloads ---------------------------------------------------------------------

@dataclass
class Workload:
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    num_blocks: int
    scale: float
    seq_lens: np.ndarray          # [B] int32, cached + new tokens
    query_lens: np.ndarray        # [B] int32, new tokens this step
    query_start_loc: np.ndarray   # [B+1] int32
    block_tables: np.ndarray      # [B][max_blocks] int32, unused entries -1
    kv_start: np.ndarray          # [B+1] int64 prefix sum of seq_lens
    k_dense: np.ndarray           # [sum L][Hkv][D] uint16 logical K per seq
    v_dense: np.ndarray
    q: np.ndarray                 # [T][Hq][D] uint16
    fill_rows: np.ndarray         # dense rows written to the pool at set-up
    fill_slots: np.ndarray        # their slots (int64)
    new_rows: np.ndarray          # dense rows of this step's tokens [T]
    new_slots: np.ndarray         # their slots [T] int64
    refs: Dict[int, int] = field(default_factory=dict)
    seeds: Dict[str, int] = field(default_factory=dict)
    shared_prefix: int = 0
    block_size: int = BLOCK_SIZE  # tokens per physical block (table entry)

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def num_q_tokens(self) -> int:
        return int(self.query_start_loc[-1])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.num_seqs else 0

    @property
    def max_query_len(self) -> int:
        return int(self.query_lens.max()) if self.num_seqs else 0

    @property
    def k_new(self) -> np.ndarray:
        return self.k_dense[self.new_rows]

    @property
    def v_new(self) -> np.ndarray:
        return self.v_dense[self.new_rows]

    def pool_elems(self) -> int:
        return self.num_blocks * self.num_kv_heads * self.block_size * self.head_dim

    def kv_bytes_read(self) -> int:
        """K+V bytes of the valid tokens that attention reads (logical)."""
        return int(self.seq_lens.astype(np.int64).sum()) * 2 * \
            self.num_kv_heads * self.head_dim * 2

    def describe(self) -> dict:
        return {
            "workload": self.name, "num_seqs": self.num_seqs,
            "num_q_tokens": self.num_q_tokens, "num_q_heads": self.num_q_heads,
            "num_kv_heads": self.num_kv_heads, "head_dim": self.head_dim,
            "block_size": self.block_size, "num_blocks": self.num_blocks,
            "max_seq_len": self.max_seq_len, "max_query_len": self.max_query_len,
            "sum_seq_len": int(self.seq_lens.astype(np.int64).sum()),
            "seeds": dict(self.seeds)}


def make_workload(name: str, seq_lens: Sequence[int], query_lens: Sequence[int],
                  num_q_heads: int, num_kv_heads: int, head_dim: int, seed: int,
                  num_blocks: Optional[int] = None, slack: float = 0.10,
                  shared_prefix: int = 0, shared: bool = True,
                  table_width: Optional[int] = None,
                  block_size: int = BLOCK_SIZE) -> Workload:
    """Build one step's inputs.

    seq_lens include this step's query_lens tokens, which are the last
    positions of each sequence.  With shared_prefix > 0 (a multiple of the
    block size), the first shared_prefix logical tokens of every sequence hold
    the same K/V; with shared=True their blocks are allocated once and held by
    every table (ref_cnt = number of sequences), otherwise every sequence gets
    private copies (the unshared twin).  block_size: tokens per physical
    block (16 by default; the tables, slots and pool size follow it)."""
    seq_lens = np.asarray(seq_lens, np.int32)
    query_lens = np.asarray(query_lens, np.int32)
    B = seq_lens.shape[0]
    assert query_lens.shape == (B,)
    assert np.all(query_lens >= 0) and np.all(query_lens <= seq_lens)
    bs = int(block_size)
    assert shared_prefix % bs == 0
    assert np.all(seq_lens >= shared_prefix)
    seeds = {"data": 1000 + seed, "tables": 3000 + seed}
    rng_tab = np.random.default_rng(seeds["tables"])

    nblk = [blocks_needed(int(L), bs) for L in seq_lens]
    pref_blocks = shared_prefix // bs
    if shared_prefix and shared:
        need = pref_blocks + sum(n - pref_blocks for n in nblk)
    else:
        need = sum(nblk)
    if num_blocks is None:
        num_blocks = max(1, int(np.ceil(need * (1.0 + slack))))
    assert num_blocks >= need, (num_blocks, need)
    width = table_width or max([1] + nblk)
    pool = BlockPool(num_blocks, rng_tab)
    tables = np.full((B, width), -1, np.int32)
    prefix_ids: List[int] = []
    for b in range(B):
        if shared_prefix and shared:
            if b == 0:
                prefix_ids = pool.allocate(pref_blocks)
                own = list(prefix_ids)
            else:
                own = pool.share(prefix_ids)
            own += pool.allocate(nblk[b] - pref_blocks)
        else:
            own = pool.allocate(nblk[b])
        tables[b, :len(own)] = own

    Hkv, D = num_kv_heads, head_dim
    kv_start = np.zeros(B + 1, np.int64)
    np.cumsum(seq_lens.astype(np.int64), out=kv_start[1:])
    total = int(kv_start[-1])
    k_dense = normal_bf16((seeds["data"], 0), (total, Hkv, D))
    v_dense = normal_bf16((seeds["data"], 1), (total, Hkv, D))
    if shared_prefix:
        # every sequence's first shared_prefix tokens carry sequence 0's K/V
        for b in range(1, B):
            s0 = int(kv_start[b])
            k_dense[s0:s0 + shared_prefix] = k_dense[:shared_prefix]
            v_dense[s0:s0 + shared_prefix] = v_dense[:shared_prefix]
    qsl = query_start_loc(query_lens)
    T = int(qsl[-1])
    q = normal_bf16((seeds["data"], 2), (T, num_q_heads, D))

    fill_rows, fill_slots, new_rows, new_slots = [], [], [], []
    for b in range(B):
        s0, L, Q = int(kv_start[b]), int(seq_lens[b]), int(query_lens[b])
        first = 0
        if shared_prefix and shared and b > 0:
            first = shared_prefix  # the shared blocks are written once, by seq 0
        cached = np.arange(first, L - Q, dtype=np.int64)
        fill_rows.append(s0 + cached)
        fill_slots.append(slots_for(tables[b], cached, bs))
        newp = np.arange(L - Q, L, dtype=np.int64)
        new_rows.append(s0 + newp)
        new_slots.append(slots_for(tables[b], newp, bs))
    cat = (lambda xs: np.concatenate(xs) if xs else np.zeros(0, np.int64))
    refs = pool.refs
    return Workload(
        name=name, num_q_heads=num_q_heads, num_kv_heads=Hkv, head_dim=D,
        num_blocks=int(num_blocks), scale=float(np.float32(1.0 / np.sqrt(D))),
        seq_lens=seq_lens, query_lens=query_lens, query_start_loc=qsl,
        block_tables=tables, kv_start=kv_start, k_dense=k_dense,
        v_dense=v_dense, q=q, fill_rows=cat(fill_rows).astype(np.int64),
        fill_slots=cat(fill_slots).astype(np.int64),
        new_rows=cat(new_rows).astype(np.int64),
        new_slots=cat(new_slots).astype(np.int64), refs=refs, seeds=seeds,
        shared_prefix=int(shared_prefix), block_size=bs)


# ---- the five synthetic step configurations ------------------------------------------

CONFIG_NAMES = {
    1: "tiny-decode-4seq-h8-d64",
    2: "llama3-8b-decode-64seq-gqa4-d128",
    3: "llama3-8b-mixed-chunked-prefill-1920+128dec",
    4: "prefix-shared-decode-256seq-2048prefix",
    5: "70b-longctx-decode-16x32768-gqa8-d128",
}


def config_lengths(k: int):
    """(seq_lens, query_lens) of synthetic configuration k (length seed 2000+k)."""
    rng = np.random.default_rng(2000 + k)
    if k == 1:
        L = np.array([56, 17, 100, 33], np.int32)
        return L, np.ones(4, np.int32)
    if k == 2:
        L = rng.integers(128, 4096, size=64, endpoint=True).astype(np.int32)
        return L, np.ones(64, np.int32)
    if k == 3:
        dec = rng.integers(256, 8192, size=128, endpoint=True).astype(np.int32)
        L = np.concatenate([dec, [1536 + 1920]]).astype(np.int32)
        Q = np.concatenate([np.ones(128, np.int32), [1920]]).astype(np.int32)
        return L, Q
    if k == 4:
        suf = rng.integers(64, 512, size=256, endpoint=True).astype(np.int32)
        return (2048 + suf).astype(np.int32), np.ones(256, np.int32)
    if k == 5:
        return np.full(16, 32768, np.int32), np.ones(16, np.int32)
    raise ValueError(k)


def make_prefill_chunk() -> Workload:
    """The prefill request of configuration 3 on its own (1920 new tokens on
    1536 cached, Llama-3-8B heads), for timing the prefill tiles alone."""
    return make_workload("llama3-8b-prefill-chunk-1920-on-1536", [1536 + 1920],
                         [1920], 32, 8, 128, seed=3)


def make_decode_part() -> Workload:
    """The 128 decode requests of configuration 3 on their own (contexts
    U[256, 8192], Llama-3-8B heads), for timing the decode part alone."""
    L, Q = config_lengths(3)
    return make_workload("llama3-8b-decodes-of-mixed-step-128seq", L[:-1], Q[:-1],
                         32, 8, 128, seed=3)


def make_config(k: int, shared: bool = True) -> Workload:
    """Synthetic configuration k in 1..5 (seeds 1000+k data, 2000+k lengths,
    3000+k tables)."""
    L, Q = config_lengths(k)
    if k == 1:
        w = make_workload(CONFIG_NAMES[1], L, Q, 8, 8, 64, seed=k, num_blocks=64)
    elif k == 2:
        w = make_workload(CONFIG_NAMES[2], L, Q, 32, 8, 128, seed=k)
    elif k == 3:
        w = make_workload(CONFIG_NAMES[3], L, Q, 32, 8, 128, seed=k)
    elif k == 4:
        name = CONFIG_NAMES[4] + ("" if shared else "-unshared")
        w = make_workload(name, L, Q, 32, 8, 128, seed=k, shared_prefix=2048,
                          shared=shared)
    elif k == 5:
        w = make_workload(CONFIG_NAMES[5], L, Q, 64, 8, 128, seed=k,
                          num_blocks=32768)
    else:
        raise ValueError(k)
    w.seeds["lengths"] = 2000 + k
    return w
