"""MI355X-native paged KV-cache varlen attention (PagedAttention hot path).

Python binding of libpa.so (include/pa.h).  Argument marshalling only: every
step of the path runs in the library's HIP kernels; torch supplies device
memory and the current stream.  There is no fallback: if libpa.so is missing
or a tensor is not on a GPU, the calls raise.

    k_cache, v_cache = alloc_pool(num_blocks, num_kv_heads, head_dim)
    write_kv(k_new, v_new, slot_mapping, k_cache, v_cache)
    out = attend(q, k_cache, v_cache, block_tables, seq_lens, query_start_loc,
                 scale, max_query_len, max_seq_len)

Sources: "vLLM v1 Deep Dive" (supercharleszhu.github.io), Part 3, Step 4c and the
Aside "KV cache and prefix caching"; "vLLM: An Exhaustive Technical Study"
(anthony-chaudhary.github.io) sections 2.1 and 2.4.
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import _lib
from ._lib import PAError  # noqa: F401

BLOCK_SIZE = 16


def _need_cuda(t: torch.Tensor, name: str) -> None:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)


def _dtype(t: torch.Tensor, dt, name: str) -> None:
    if t.dtype != dt:
        raise TypeError("%s must be %s, got %s" % (name, dt, t.dtype))


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def alloc_pool(num_blocks: int, num_kv_heads: int, head_dim: int,
               device="cuda", fill: Optional[float] = None, block_size: int = BLOCK_SIZE
               ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Two bf16 pools (K, V), each [num_blocks][num_kv_heads][block_size *
    head_dim] in the library's tile layout (block_size 16, or 8 for the
    *_bs calls)."""
    shape = (num_blocks, num_kv_heads, int(block_size) * head_dim)
    if fill is None:
        k = torch.empty(shape, dtype=torch.bfloat16, device=device)
        v = torch.empty(shape, dtype=torch.bfloat16, device=device)
    else:
        k = torch.full(shape, fill, dtype=torch.bfloat16, device=device)
        v = torch.full(shape, fill, dtype=torch.bfloat16, device=device)
    return k, v


def _pool_blocks(cache: torch.Tensor, num_kv_heads: int, head_dim: int,
                 block_size: int = BLOCK_SIZE) -> int:
    per_block = num_kv_heads * int(block_size) * head_dim
    if not cache.is_contiguous() or cache.numel() % per_block:
        raise ValueError("pool must be contiguous with a multiple of "
                         "num_kv_heads*block_size*head_dim elements")
    return cache.numel() // per_block


def _scatter_args(k, v, slot_mapping, k_cache, v_cache, pool_dtype, block_size=BLOCK_SIZE):
    """Checks of a scatter's tensors; returns (T, Hkv, D, num_blocks)."""
    for t, n in ((k, "k"), (v, "v"), (slot_mapping, "slot_mapping"),
                 (k_cache, "k_cache"), (v_cache, "v_cache")):
        _need_cuda(t, n)
    _dtype(k, torch.bfloat16, "k")
    _dtype(v, torch.bfloat16, "v")
    _dtype(slot_mapping, torch.int64, "slot_mapping")
    _dtype(k_cache, pool_dtype, "k_cache")
    _dtype(v_cache, pool_dtype, "v_cache")
    if k.dim() != 3 or v.shape != k.shape:
        raise ValueError("k and v must be [num_tokens][num_kv_heads][head_dim]")
    T, Hkv, D = k.shape
    for t, n in ((k, "k"), (v, "v")):
        if t.stride(2) != 1 or t.stride(1) != D:
            raise ValueError("%s rows must be contiguous [num_kv_heads][head_dim]" % n)
    if not slot_mapping.is_contiguous() or slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be contiguous [num_tokens]")
    nb = _pool_blocks(k_cache, Hkv, D, block_size)
    if _pool_blocks(v_cache, Hkv, D, block_size) != nb:
        raise ValueError("k_cache and v_cache differ in size")
    return T, Hkv, D, nb


def write_kv(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor,
             k_cache: torch.Tensor, v_cache: torch.Tensor,
             block_size: int = BLOCK_SIZE) -> None:
    """Scatter k, v ([T][Hkv][D] bf16, rows may be strided) into their slots
    (pools of block_size-token blocks: 16, or 8 through pa_write_kv_bs)."""
    T, Hkv, D, nb = _scatter_args(k, v, slot_mapping, k_cache, v_cache, torch.bfloat16,
                                  block_size)
    lib = _lib.load()
    args = [_ptr(k), _ptr(v), k.stride(0), v.stride(0), _ptr(slot_mapping), T, Hkv, D,
            _ptr(k_cache), _ptr(v_cache), nb]
    if block_size == BLOCK_SIZE:
        st, name = lib.pa_write_kv(*args, _stream(k)), "pa_write_kv"
    else:
        st, name = lib.pa_write_kv_bs(*args, int(block_size), _stream(k)), "pa_write_kv_bs"
    _lib.check(st, name)


def alloc_pool_fp8(num_blocks: int, num_kv_heads: int, head_dim: int,
                   device="cuda", fill: Optional[int] = None
                   ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Two 8-bit pools (K, V) of E4M3 codes, each uint8
    [num_blocks][num_kv_heads][16 * head_dim] in the library's 8-bit tile
    layout; fill: a code byte, or None for uninitialised memory."""
    shape = (num_blocks, num_kv_heads, BLOCK_SIZE * head_dim)
    if fill is None:
        k = torch.empty(shape, dtype=torch.uint8, device=device)
        v = torch.empty(shape, dtype=torch.uint8, device=device)
    else:
        k = torch.full(shape, fill, dtype=torch.uint8, device=device)
        v = torch.full(shape, fill, dtype=torch.uint8, device=device)
    return k, v


def write_kv_fp8(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor,
                 k_cache: torch.Tensor, v_cache: torch.Tensor, k_scale: float,
                 v_scale: float) -> None:
    """Scatter k, v ([T][Hkv][D] bf16, rows may be strided) into 8-bit pools:
    the E4M3 code of fp32(x) / scale per element."""
    T, Hkv, D, nb = _scatter_args(k, v, slot_mapping, k_cache, v_cache, torch.uint8)
    lib = _lib.load()
    st = lib.pa_write_kv_fp8(_ptr(k), _ptr(v), k.stride(0), v.stride(0),
                             _ptr(slot_mapping), T, Hkv, D, float(k_scale),
                             float(v_scale), _ptr(k_cache), _ptr(v_cache), nb,
                             _stream(k))
    _lib.check(st, "pa_write_kv_fp8")


def workspace_size(num_seqs: int, num_q_tokens: int, num_q_heads: int,
                   num_kv_heads: int, head_dim: int, max_query_len: int,
                   max_seq_len: int, cascade: bool = False) -> int:
    """Workspace bytes of pa_attend (cascade=True: of the shared-prefix calls,
    which add a prefix section)."""
    name = "pa_attend_cascade_workspace_size" if cascade else "pa_attend_workspace_size"
    n = getattr(_lib.load(), name)(num_seqs, num_q_tokens, num_q_heads,
                                   num_kv_heads, head_dim, max_query_len,
                                   max_seq_len)
    if n == 0:
        raise ValueError("invalid arguments for " + name)
    return int(n)


def alloc_workspace(num_seqs, num_q_tokens, num_q_heads, num_kv_heads, head_dim,
                    max_query_len, max_seq_len, device="cuda",
                    cascade: bool = False) -> torch.Tensor:
    n = workspace_size(num_seqs, num_q_tokens, num_q_heads, num_kv_heads,
                       head_dim, max_query_len, max_seq_len, cascade=cascade)
    # torch's caching allocator returns 512-byte aligned blocks
    return torch.empty(n, dtype=torch.uint8, device=device)


def _metadata_args(block_tables, seq_lens, query_start_loc) -> int:
    """Checks of a step's metadata tensors; returns the number of requests."""
    for t, n in ((block_tables, "block_tables"), (seq_lens, "seq_lens"),
                 (query_start_loc, "query_start_loc")):
        _need_cuda(t, n)
        _dtype(t, torch.int32, n)
    if block_tables.dim() != 2 or not block_tables.is_contiguous():
        raise ValueError("block_tables must be contiguous [num_seqs][max_blocks]")
    B = block_tables.shape[0]
    if seq_lens.shape != (B,) or query_start_loc.shape != (B + 1,):
        raise ValueError("seq_lens must be [B] and query_start_loc [B+1]")
    if not (seq_lens.is_contiguous() and query_start_loc.is_contiguous()):
        raise ValueError("seq_lens and query_start_loc must be contiguous")
    return B


def _attend_args(q, k_cache, v_cache, block_tables, seq_lens, query_start_loc,
                 num_kv_heads, out, workspace, max_query_len, max_seq_len,
                 cascade=False, block_size=BLOCK_SIZE):
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _need_cuda(t, n)
    _dtype(q, torch.bfloat16, "q")
    pool_dtype = torch.uint8 if k_cache.dtype == torch.uint8 else torch.bfloat16
    _dtype(k_cache, pool_dtype, "k_cache")
    _dtype(v_cache, pool_dtype, "v_cache")
    B = _metadata_args(block_tables, seq_lens, query_start_loc)
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be contiguous [num_q_tokens][num_q_heads][head_dim]")
    T, Hq, D = q.shape
    if num_kv_heads is None:
        if k_cache.dim() != 3:
            raise ValueError("pass num_kv_heads or a [blocks][kv_heads][16*D] pool")
        num_kv_heads = k_cache.shape[1]
    nb = _pool_blocks(k_cache, num_kv_heads, D, block_size)
    if _pool_blocks(v_cache, num_kv_heads, D, block_size) != nb:
        raise ValueError("k_cache and v_cache differ in size")
    if out is None:
        out = torch.empty_like(q)
    else:
        _need_cuda(out, "out")
        _dtype(out, torch.bfloat16, "out")
        if out.shape != q.shape or not out.is_contiguous():
            raise ValueError("out must be contiguous and shaped like q")
    if workspace is None:
        workspace = alloc_workspace(B, T, Hq, num_kv_heads, D, max_query_len,
                                    max_seq_len, device=q.device, cascade=cascade)
    return T, Hq, D, num_kv_heads, nb, B, out, workspace


def attend(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
           block_tables: torch.Tensor, seq_lens: torch.Tensor,
           query_start_loc: torch.Tensor, scale: float, max_query_len: int,
           max_seq_len: int, num_kv_heads: Optional[int] = None,
           out: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None,
           planned: bool = False, merge: bool = True,
           k_scale: float = 1.0, v_scale: float = 1.0,
           common_prefix_len: Optional[int] = None,
           block_size: int = BLOCK_SIZE) -> torch.Tensor:
    """Paged varlen causal attention of every query row of a mixed batch.

    q [T][Hq][D] bf16; block_tables [B][max_blocks] int32; seq_lens [B] int32;
    query_start_loc [B+1] int32; pools from alloc_pool (bf16) or
    alloc_pool_fp8 (E4M3 codes standing for code * k_scale, code * v_scale).
    Returns out [T][Hq][D] bf16 (written in place when ``out`` is given).
    With planned=True the work plan already in ``workspace`` (from attend_plan
    with the same metadata) is used: the attention kernel is enqueued, then
    (with merge=True, the default) the split-K merge kernel; merge=False
    leaves the merge to a later attend_merge call.

    common_prefix_len (shared-prefix attention): every request's first
    common_prefix_len keys are the same blocks (request 0's table is the one
    read) and every query lies past them; the prefix is then attended once
    for the whole batch and merged with each request's own keys.  Needs a
    workspace from alloc_workspace(..., cascade=True) (allocated here when
    none is given); with planned=True the plan must come from
    attend_plan(..., common_prefix_len=...).

    block_size: 16, or 8 (bf16 pools of 8-token blocks from alloc_pool(...,
    block_size=8), tables of 8-token ids; pa_attend_bs, not planned)."""
    cascade = common_prefix_len is not None
    T, Hq, D, Hkv, nb, B, out, workspace = _attend_args(
        q, k_cache, v_cache, block_tables, seq_lens, query_start_loc,
        num_kv_heads, out, workspace, max_query_len, max_seq_len, cascade, block_size)
    lib = _lib.load()
    if block_size != BLOCK_SIZE:
        if planned or cascade or k_cache.dtype == torch.uint8:
            raise ValueError("block_size != 16: bf16 pools, plain pa_attend_bs only")
        st = lib.pa_attend_bs(_ptr(q), _ptr(k_cache), _ptr(v_cache), nb, int(block_size),
                              _ptr(block_tables), block_tables.shape[1], _ptr(seq_lens),
                              _ptr(query_start_loc), B, T, Hq, Hkv, D, int(max_query_len),
                              int(max_seq_len), float(scale), _ptr(out), _ptr(workspace),
                              workspace.numel(), _stream(q))
        _lib.check(st, "pa_attend_bs")
        return out
    args = [_ptr(q), _ptr(k_cache), _ptr(v_cache), nb, _ptr(block_tables),
            block_tables.shape[1], _ptr(seq_lens), _ptr(query_start_loc), B, T,
            Hq, Hkv, D, int(max_query_len), int(max_seq_len)]
    if cascade and not planned:
        args.append(int(common_prefix_len))
    args.append(float(scale))
    fp8 = k_cache.dtype == torch.uint8
    if fp8:
        args += [float(k_scale), float(v_scale)]
    name = "pa_attend" + ("_planned" if planned else "") + ("_cascade" if cascade else "") \
        + ("_fp8" if fp8 else "")
    st = getattr(lib, name)(*args, _ptr(out), _ptr(workspace), workspace.numel(),
                            _stream(q))
    _lib.check(st, name)
    if planned and merge:
        attend_merge(out, B, Hkv, max_query_len, max_seq_len, workspace,
                     cascade=cascade)
    return out


def attend_merge(out: torch.Tensor, num_seqs: int, num_kv_heads: int,
                 max_query_len: int, max_seq_len: int,
                 workspace: torch.Tensor, cascade: bool = False) -> None:
    """Enqueue the split-K merge after attend(..., planned=True, merge=False)."""
    _need_cuda(out, "out")
    T, Hq, D = out.shape
    name = "pa_attend_merge_cascade" if cascade else "pa_attend_merge"
    st = getattr(_lib.load(), name)(int(num_seqs), T, Hq, int(num_kv_heads), D,
                                    int(max_query_len), int(max_seq_len),
                                    _ptr(out), _ptr(workspace), workspace.numel(),
                                    _stream(out))
    _lib.check(st, name)


def attend_plan(block_tables: torch.Tensor, seq_lens: torch.Tensor,
                query_start_loc: torch.Tensor, num_q_tokens: int,
                num_q_heads: int, num_kv_heads: int, head_dim: int,
                max_query_len: int, max_seq_len: int,
                workspace: torch.Tensor,
                common_prefix_len: Optional[int] = None, fp8: bool = False) -> None:
    """Enqueue only the work plan of pa_attend into ``workspace``; follow
    with attend(..., planned=True) for each layer that shares the metadata
    (with common_prefix_len: a shared-prefix plan, run by
    attend(..., planned=True, common_prefix_len=...); fp8=True: the plan
    pa_attend_fp8 makes for 8-bit pools)."""
    B = _metadata_args(block_tables, seq_lens, query_start_loc)
    _need_cuda(workspace, "workspace")
    lib = _lib.load()
    args = [_ptr(block_tables), block_tables.shape[1], _ptr(seq_lens),
            _ptr(query_start_loc), B, int(num_q_tokens), int(num_q_heads),
            int(num_kv_heads), int(head_dim), int(max_query_len), int(max_seq_len)]
    if common_prefix_len is None:
        name = "pa_attend_plan_fp8" if fp8 else "pa_attend_plan"
    else:
        name = "pa_attend_plan_cascade"
        args.append(int(common_prefix_len))
    st = getattr(lib, name)(*args, _ptr(workspace), workspace.numel(),
                            _stream(workspace))
    _lib.check(st, name)


def write_kv_plan(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor,
                  k_cache: torch.Tensor, v_cache: torch.Tensor,
                  block_tables: torch.Tensor, seq_lens: torch.Tensor,
                  query_start_loc: torch.Tensor, num_q_tokens: int, num_q_heads: int,
                  max_query_len: int, max_seq_len: int, workspace: torch.Tensor,
                  common_prefix_len: Optional[int] = None,
                  k_scale: Optional[float] = None,
                  v_scale: Optional[float] = None) -> None:
    """write_kv (write_kv_fp8 for uint8 pools, with the scales) and
    attend_plan of the same step in one launch."""
    fp8 = k_cache.dtype == torch.uint8
    T, Hkv, D, nb = _scatter_args(k, v, slot_mapping, k_cache, v_cache,
                                  torch.uint8 if fp8 else torch.bfloat16)
    B = _metadata_args(block_tables, seq_lens, query_start_loc)
    _need_cuda(workspace, "workspace")
    if fp8 and (k_scale is None or v_scale is None):
        raise ValueError("8-bit pools need k_scale and v_scale")
    lib = _lib.load()
    scatter = [_ptr(k), _ptr(v), k.stride(0), v.stride(0), _ptr(slot_mapping), T]
    if fp8:
        scatter += [float(k_scale), float(v_scale)]
    plan = [_ptr(k_cache), _ptr(v_cache), nb, _ptr(block_tables), block_tables.shape[1],
            _ptr(seq_lens), _ptr(query_start_loc), B, int(num_q_tokens), int(num_q_heads),
            Hkv, D, int(max_query_len), int(max_seq_len),
            -1 if common_prefix_len is None else int(common_prefix_len),
            _ptr(workspace), workspace.numel(), _stream(k)]
    name = "pa_write_kv_plan_fp8" if fp8 else "pa_write_kv_plan"
    _lib.check(getattr(lib, name)(*scatter, *plan), name)


def validate_cascade(block_tables, seq_lens, query_start_loc,
                     common_prefix_len: int) -> None:
    """Host check of a shared-prefix batch (every query past the prefix, the
    prefix's whole blocks the same in every table); raises PAError.  Takes
    host arrays (numpy or CPU tensors)."""
    import numpy as np
    bt = np.ascontiguousarray(np.asarray(block_tables, dtype=np.int32))
    sl = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    qsl = np.ascontiguousarray(np.asarray(query_start_loc, dtype=np.int32))
    if bt.ndim != 2 or sl.shape != (bt.shape[0],) or qsl.shape != (bt.shape[0] + 1,):
        raise ValueError("block_tables [B][max_blocks], seq_lens [B], query_start_loc [B+1]")
    st = _lib.load().pa_validate_cascade_host(
        bt.ctypes.data, bt.shape[1], sl.ctypes.data, qsl.ctypes.data, bt.shape[0],
        int(common_prefix_len))
    _lib.check(st, "pa_validate_cascade_host")


def copy_blocks(k_cache: torch.Tensor, v_cache: torch.Tensor,
                block_mapping: torch.Tensor, num_kv_heads: int, head_dim: int) -> None:
    """Copy-on-write block copies: block_mapping int64 [n][2] of (src, dst)
    block ids; every kv head of both pools (bf16 or 8-bit) is copied."""
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache"), (block_mapping, "block_mapping")):
        _need_cuda(t, n)
    _dtype(block_mapping, torch.int64, "block_mapping")
    if block_mapping.dim() != 2 or block_mapping.shape[1] != 2 or not block_mapping.is_contiguous():
        raise ValueError("block_mapping must be contiguous [n][2] (src, dst)")
    if k_cache.dtype != v_cache.dtype or k_cache.dtype not in (torch.bfloat16, torch.uint8):
        raise ValueError("pools must both be bf16 or both uint8 (8-bit)")
    nb = _pool_blocks(k_cache, num_kv_heads, head_dim)
    if _pool_blocks(v_cache, num_kv_heads, head_dim) != nb:
        raise ValueError("k_cache and v_cache differ in size")
    st = _lib.load().pa_copy_blocks(_ptr(k_cache), _ptr(v_cache), nb, num_kv_heads,
                                    head_dim, k_cache.element_size(), _ptr(block_mapping),
                                    block_mapping.shape[0], _stream(k_cache))
    _lib.check(st, "pa_copy_blocks")


def expand_block_tables(block_tables: torch.Tensor, block_size: int) -> torch.Tensor:
    """Block tables of block_size-token blocks (a multiple of 16) -> the
    16-token block tables attend() reads (block n = 16-token blocks
    n*R .. n*R+R-1, R = block_size // 16)."""
    _need_cuda(block_tables, "block_tables")
    _dtype(block_tables, torch.int32, "block_tables")
    if block_tables.dim() != 2 or not block_tables.is_contiguous():
        raise ValueError("block_tables must be contiguous [num_seqs][max_blocks]")
    B, M = block_tables.shape
    R = max(1, int(block_size) // BLOCK_SIZE)
    out = torch.empty((B, M * R), dtype=torch.int32, device=block_tables.device)
    st = _lib.load().pa_expand_block_tables(_ptr(block_tables), B, M, int(block_size),
                                            _ptr(out), _stream(block_tables))
    _lib.check(st, "pa_expand_block_tables")
    return out


MLA_BLOCK_SIZE = 64
MLA_DIM = 576
MLA_LATENT = 512


def alloc_mla_cache(num_blocks: int, device="cuda",
                    fill: Optional[float] = None) -> torch.Tensor:
    """A latent cache: bf16 [num_blocks][64 * 576] in the library's layout."""
    shape = (num_blocks, MLA_BLOCK_SIZE * MLA_DIM)
    if fill is None:
        return torch.empty(shape, dtype=torch.bfloat16, device=device)
    return torch.full(shape, fill, dtype=torch.bfloat16, device=device)


def mla_write_kv(kv: torch.Tensor, slot_mapping: torch.Tensor,
                 cache: torch.Tensor) -> None:
    """Scatter kv [T][576] bf16 (rows may be strided) into the latent cache
    at slot_mapping (int64, block * 64 + offset; < 0 skipped)."""
    for t, n in ((kv, "kv"), (slot_mapping, "slot_mapping"), (cache, "cache")):
        _need_cuda(t, n)
    _dtype(kv, torch.bfloat16, "kv")
    _dtype(cache, torch.bfloat16, "cache")
    _dtype(slot_mapping, torch.int64, "slot_mapping")
    if kv.dim() != 2 or kv.shape[1] != MLA_DIM or kv.stride(1) != 1:
        raise ValueError("kv must be [T][576] with unit stride along the dims")
    if not cache.is_contiguous() or cache.numel() % (MLA_BLOCK_SIZE * MLA_DIM):
        raise ValueError("cache must be contiguous [num_blocks][64 * 576]")
    nb = cache.numel() // (MLA_BLOCK_SIZE * MLA_DIM)
    st = _lib.load().pa_mla_write_kv(_ptr(kv), kv.stride(0), _ptr(slot_mapping),
                                     kv.shape[0], _ptr(cache), nb, _stream(kv))
    _lib.check(st, "pa_mla_write_kv")


def mla_workspace(num_q_tokens: int, num_q_heads: int, max_seq_len: int,
                  device="cuda") -> torch.Tensor:
    n = _lib.load().pa_mla_workspace_size(num_q_tokens, num_q_heads, max_seq_len)
    if n == 0:
        raise ValueError("invalid arguments for pa_mla_workspace_size")
    return torch.empty(n, dtype=torch.uint8, device=device)


def mla_decode(q: torch.Tensor, cache: torch.Tensor, block_tables: torch.Tensor,
               seq_lens: torch.Tensor, query_start_loc: torch.Tensor, scale: float,
               max_seq_len: int, out: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """MLA attention of q [T][Hq][576] bf16 over the latent cache (64-token
    block tables) -> out [T][Hq][512] bf16."""
    for t, n in ((q, "q"), (cache, "cache"), (block_tables, "block_tables"),
                 (seq_lens, "seq_lens"), (query_start_loc, "query_start_loc")):
        _need_cuda(t, n)
    _dtype(q, torch.bfloat16, "q")
    _dtype(cache, torch.bfloat16, "cache")
    _dtype(block_tables, torch.int32, "block_tables")
    if q.dim() != 3 or q.shape[2] != MLA_DIM or not q.is_contiguous():
        raise ValueError("q must be contiguous [T][Hq][576]")
    T, Hq, _ = q.shape
    B = block_tables.shape[0]
    nb = cache.numel() // (MLA_BLOCK_SIZE * MLA_DIM)
    if out is None:
        out = torch.empty((T, Hq, MLA_LATENT), dtype=torch.bfloat16, device=q.device)
    if workspace is None:
        workspace = mla_workspace(T, Hq, max_seq_len, device=q.device)
    st = _lib.load().pa_mla_decode(_ptr(q), _ptr(cache), nb, _ptr(block_tables),
                                   block_tables.shape[1], _ptr(seq_lens),
                                   _ptr(query_start_loc), B, T, Hq, int(max_seq_len),
                                   float(scale), _ptr(out), _ptr(workspace),
                                   workspace.numel(), _stream(q))
    _lib.check(st, "pa_mla_decode")
    return out


def gather_kv(k_cache: torch.Tensor, v_cache: torch.Tensor,
              block_tables: torch.Tensor, seq_lens: torch.Tensor,
              kv_start: torch.Tensor, total_rows: int, num_kv_heads: int,
              head_dim: int, block_size: int = BLOCK_SIZE) -> Tuple[torch.Tensor, torch.Tensor]:
    """Logical gather through the block tables: dense [sum L][Hkv][D] K, V
    (pools of block_size-token blocks: 16, or 8 through pa_gather_kv_bs)."""
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache"),
                 (block_tables, "block_tables"), (seq_lens, "seq_lens"),
                 (kv_start, "kv_start")):
        _need_cuda(t, n)
    _dtype(kv_start, torch.int64, "kv_start")
    nb = _pool_blocks(k_cache, num_kv_heads, head_dim, block_size)
    B = block_tables.shape[0]
    ko = torch.empty((total_rows, num_kv_heads, head_dim), dtype=torch.bfloat16,
                     device=k_cache.device)
    vo = torch.empty_like(ko)
    lib = _lib.load()
    if block_size == BLOCK_SIZE:
        st = lib.pa_gather_kv(_ptr(k_cache), _ptr(v_cache), nb, _ptr(block_tables),
                              block_tables.shape[1], _ptr(seq_lens), _ptr(kv_start),
                              B, total_rows, num_kv_heads, head_dim, _ptr(ko),
                              _ptr(vo), _stream(k_cache))
    else:
        st = lib.pa_gather_kv_bs(_ptr(k_cache), _ptr(v_cache), nb, int(block_size),
                                 _ptr(block_tables), block_tables.shape[1], _ptr(seq_lens),
                                 _ptr(kv_start), B, total_rows, num_kv_heads, head_dim,
                                 _ptr(ko), _ptr(vo), _stream(k_cache))
    _lib.check(st, "pa_gather_kv")
    return ko, vo


def validate_metadata(block_tables: torch.Tensor, seq_lens: torch.Tensor,
                      query_start_loc: torch.Tensor, num_q_tokens: int,
                      max_query_len: int, max_seq_len: int, num_blocks: int,
                      slot_mapping: Optional[torch.Tensor] = None) -> None:
    """Synchronous content check of device metadata; raises PAError."""
    B = block_tables.shape[0]
    lib = _lib.load()
    st = lib.pa_validate_metadata(
        _ptr(block_tables), block_tables.shape[1], _ptr(seq_lens),
        _ptr(query_start_loc), B, num_q_tokens, max_query_len, max_seq_len,
        num_blocks, _ptr(slot_mapping),
        0 if slot_mapping is None else slot_mapping.numel())
    _lib.check(st, "pa_validate_metadata")
