"""CPU reference ("oracle") for the paged KV-cache varlen attention path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The product
library (``paged_kv_cache_varlen_amd``) never imports it, and this package
imports nothing from the product: the two share no code.

The arithmetic lives in ``oracle.c`` (plain C, fp64, loops in the order of the
definitions); this module only compiles it with gcc and marshals numpy arrays.
bf16 tensors travel as their uint16 bit patterns.

Sources: "vLLM v1 Deep Dive" (supercharleszhu.github.io), Part 3, Step 4c "Mixed
batches" (query_start_loc) and the Aside "KV cache and prefix caching"
(slot_mapping scatter; block_table + varlen causal attention in one launch);
"vLLM: An Exhaustive Technical Study for Kernel Engineers" (anthony-chaudhary.github.io) sections 2.1 (block
tables, write slot = block number * block_size + offset) and 2.4 (GQA heads
that share a KV head are processed together).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_HDR = os.path.join(_HERE, "oracle.h")
_LIB = os.path.join(_HERE, "liboracle.so")

BLOCK_SIZE = 16

_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so (gcc, -O2, OpenMP)."""
    stale = (not os.path.exists(_LIB)) or max(
        os.path.getmtime(_SRC), os.path.getmtime(_HDR)) > os.path.getmtime(_LIB)
    if force or stale:
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call([
            "gcc", "-O2", "-fopenmp", "-std=c11", "-Wall", "-shared", "-fPIC",
            _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int64
        lib.oracle_k_index.restype = ctypes.c_size_t
        lib.oracle_k_index.argtypes = [I] * 7
        lib.oracle_v_index.restype = ctypes.c_size_t
        lib.oracle_v_index.argtypes = [I] * 7
        lib.oracle_write_kv.restype = None
        lib.oracle_write_kv.argtypes = [P, P, P, P, P, I, I, I, I]
        lib.oracle_gather_kv.restype = None
        lib.oracle_gather_kv.argtypes = [P, P, P, I, P, I, I, I, I, P, P]
        lib.oracle_attend.restype = None
        lib.oracle_attend.argtypes = [P, P, P, P, I, P, P, I, I, I, I, I,
                                      ctypes.c_float, I, P, P, ctypes.c_int]
        lib.oracle_attend_rows.restype = None
        lib.oracle_attend_rows.argtypes = [P, P, P, P, I, P, P, I, I, I, I, I,
                                           ctypes.c_float, I, P, I, P, P,
                                           ctypes.c_int]
        lib.oracle_attend_dense.restype = None
        lib.oracle_attend_dense.argtypes = [P, P, P, P, P, I, I, I, I,
                                            ctypes.c_float, I, P, P]
        lib.oracle_e4m3_decode.restype = ctypes.c_double
        lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3_encode.restype = ctypes.c_uint8
        lib.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        lib.oracle_k8_index.restype = ctypes.c_size_t
        lib.oracle_k8_index.argtypes = [I] * 7
        lib.oracle_v8_index.restype = ctypes.c_size_t
        lib.oracle_v8_index.argtypes = [I] * 7
        lib.oracle_write_kv_fp8.restype = None
        lib.oracle_write_kv_fp8.argtypes = [P, P, P, P, P, I, I, I, I,
                                            ctypes.c_float, ctypes.c_float]
        lib.oracle_attend_fp8.restype = None
        lib.oracle_attend_fp8.argtypes = [P, P, P, ctypes.c_float, ctypes.c_float,
                                          P, I, P, P, I, I, I, I, I,
                                          ctypes.c_float, I, P, I, P, P,
                                          ctypes.c_int]
        lib.oracle_copy_blocks.restype = None
        lib.oracle_copy_blocks.argtypes = [P, P, I, I, P, I]
        lib.oracle_expand_block_tables.restype = None
        lib.oracle_expand_block_tables.argtypes = [P, I, I, I, P]
        lib.oracle_mla_index.restype = ctypes.c_size_t
        lib.oracle_mla_index.argtypes = [I, I, I]
        lib.oracle_mla_write_kv.restype = None
        lib.oracle_mla_write_kv.argtypes = [P, P, P, I]
        lib.oracle_mla_decode.restype = None
        lib.oracle_mla_decode.argtypes = [P, P, P, I, P, P, I, I, ctypes.c_float, P,
                                          ctypes.c_int]
        lib.oracle_abi_version.restype = ctypes.c_int
        _lib = lib
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


# ---- layout ---------------------------------------------------------------

def k_index(n, g, t, d, num_kv_heads, head_dim, block_size=BLOCK_SIZE) -> int:
    """Flat element offset of K(block n, kv head g, slot t, dim d) in a pool."""
    return int(_load().oracle_k_index(n, g, t, d, num_kv_heads, block_size,
                                      head_dim))


def v_index(n, g, t, d, num_kv_heads, head_dim, block_size=BLOCK_SIZE) -> int:
    """Flat element offset of V(block n, kv head g, slot t, dim d) in a pool."""
    return int(_load().oracle_v_index(n, g, t, d, num_kv_heads, block_size,
                                      head_dim))


# ---- scatter / gather -------------------------------------------------------

def write_kv(k_cache: np.ndarray, v_cache: np.ndarray, k: np.ndarray,
             v: np.ndarray, slot_mapping: np.ndarray,
             block_size: int = BLOCK_SIZE) -> None:
    """In-place scatter of k, v ([T][Hkv][D] uint16 bits) into the pools.

    ``k_cache``/``v_cache`` are flat uint16 arrays of
    num_blocks*Hkv*block_size*D elements (any shape, C-contiguous); slot s
    is offset s % block_size of block s // block_size."""
    assert k_cache.dtype == np.uint16 and k_cache.flags.c_contiguous
    assert v_cache.dtype == np.uint16 and v_cache.flags.c_contiguous
    T, Hkv, D = k.shape
    k = _c(k, np.uint16)
    v = _c(v, np.uint16)
    sm = _c(slot_mapping, np.int64)
    assert sm.shape == (T,)
    _load().oracle_write_kv(_p(k_cache), _p(v_cache), _p(k), _p(v), _p(sm), T,
                            Hkv, int(block_size), D)


def gather_kv(k_cache, v_cache, block_tables, seq_lens, num_kv_heads,
              head_dim, block_size=BLOCK_SIZE):
    """Logical gather: dense ([sum L][Hkv][D] uint16) K and V; table entry j
    of a request names the block of its tokens j*block_size ..."""
    bt = _c(block_tables, np.int32)
    sl = _c(seq_lens, np.int32)
    total = int(sl.sum())
    ko = np.empty((total, num_kv_heads, head_dim), np.uint16)
    vo = np.empty_like(ko)
    _load().oracle_gather_kv(_p(k_cache), _p(v_cache), _p(bt), bt.shape[1],
                             _p(sl), sl.shape[0], num_kv_heads, int(block_size),
                             head_dim, _p(ko), _p(vo))
    return ko, vo


# ---- attention ----------------------------------------------------------------

def attend(q, k_cache, v_cache, block_tables, seq_lens, query_start_loc,
           num_kv_heads, scale, nthreads=None, block_size=BLOCK_SIZE) -> np.ndarray:
    """fp64 out [T][Hq][D] of paged varlen causal attention (pools and tables
    of block_size-token blocks)."""
    q = _c(q, np.uint16)
    T, Hq, D = q.shape
    bt = _c(block_tables, np.int32)
    sl = _c(seq_lens, np.int32)
    qsl = _c(query_start_loc, np.int32)
    B = sl.shape[0]
    assert qsl.shape == (B + 1,) and int(qsl[-1]) == T
    nthreads = nthreads or default_threads()
    maxL = max(1, int(sl.max()) if B else 1)
    scratch = np.empty(nthreads * maxL, np.float64)
    out = np.zeros((T, Hq, D), np.float64)
    _load().oracle_attend(_p(q), _p(k_cache), _p(v_cache), _p(bt), bt.shape[1],
                          _p(sl), _p(qsl), B, Hq, num_kv_heads, int(block_size), D,
                          float(scale), maxL, _p(scratch), _p(out),
                          int(nthreads))
    return out


def attend_rows(q, k_cache, v_cache, block_tables, seq_lens, query_start_loc,
                num_kv_heads, scale, rows, nthreads=None,
                block_size=BLOCK_SIZE) -> np.ndarray:
    """fp64 out for selected (token, head) rows only: [len(rows)][D]."""
    q = _c(q, np.uint16)
    T, Hq, D = q.shape
    bt = _c(block_tables, np.int32)
    sl = _c(seq_lens, np.int32)
    qsl = _c(query_start_loc, np.int32)
    rows = _c(rows, np.int64).reshape(-1, 2)
    B = sl.shape[0]
    nthreads = nthreads or default_threads()
    maxL = max(1, int(sl.max()) if B else 1)
    scratch = np.empty(nthreads * maxL, np.float64)
    out = np.zeros((rows.shape[0], D), np.float64)
    _load().oracle_attend_rows(_p(q), _p(k_cache), _p(v_cache), _p(bt),
                               bt.shape[1], _p(sl), _p(qsl), B, Hq,
                               num_kv_heads, int(block_size), D, float(scale), maxL,
                               _p(rows), rows.shape[0], _p(scratch), _p(out),
                               int(nthreads))
    return out


def attend_dense(q, k_dense, v_dense, seq_lens, query_start_loc, scale):
    """Same attention over contiguous per-sequence K/V ([sum L][Hkv][D]) with
    no block tables."""
    q = _c(q, np.uint16)
    T, Hq, D = q.shape
    kd = _c(k_dense, np.uint16)
    vd = _c(v_dense, np.uint16)
    Hkv = kd.shape[1]
    sl = _c(seq_lens, np.int32)
    qsl = _c(query_start_loc, np.int32)
    B = sl.shape[0]
    maxL = max(1, int(sl.max()) if B else 1)
    scratch = np.empty(maxL, np.float64)
    out = np.zeros((T, Hq, D), np.float64)
    _load().oracle_attend_dense(_p(q), _p(kd), _p(vd), _p(sl), _p(qsl), B, Hq,
                                Hkv, D, float(scale), maxL, _p(scratch),
                                _p(out))
    return out


# ---- 8-bit (E4M3) KV cache ------------------------------------------------------

def e4m3_decode(codes) -> np.ndarray:
    """fp64 values of E4M3 codes (uint8 array)."""
    lib = _load()
    c = np.asarray(codes, np.uint8)
    return np.array([lib.oracle_e4m3_decode(int(b)) for b in c.ravel()],
                    np.float64).reshape(c.shape)


def e4m3_encode(values) -> np.ndarray:
    """E4M3 codes (uint8) of fp32 values: nearest, ties to even mantissa;
    |v| >= 448 saturates; NaN -> 0x7f."""
    lib = _load()
    v = np.asarray(values, np.float32)
    return np.array([lib.oracle_e4m3_encode(float(x)) for x in v.ravel()],
                    np.uint8).reshape(v.shape)


def k8_index(n, g, t, d, num_kv_heads, head_dim, block_size=BLOCK_SIZE) -> int:
    """Byte offset of K(block n, kv head g, slot t, dim d) in an 8-bit pool."""
    return int(_load().oracle_k8_index(n, g, t, d, num_kv_heads, block_size,
                                       head_dim))


def v8_index(n, g, t, d, num_kv_heads, head_dim, block_size=BLOCK_SIZE) -> int:
    """Byte offset of V(block n, kv head g, slot t, dim d) in an 8-bit pool."""
    return int(_load().oracle_v8_index(n, g, t, d, num_kv_heads, block_size,
                                       head_dim))


def write_kv_fp8(k_cache: np.ndarray, v_cache: np.ndarray, k: np.ndarray,
                 v: np.ndarray, slot_mapping: np.ndarray, k_scale: float,
                 v_scale: float) -> None:
    """In-place 8-bit scatter: code of fp32(x) / scale for every element of
    k, v ([T][Hkv][D] uint16 bf16 bits) at its slot; flat uint8 pools of
    num_blocks*Hkv*16*D bytes."""
    assert k_cache.dtype == np.uint8 and k_cache.flags.c_contiguous
    assert v_cache.dtype == np.uint8 and v_cache.flags.c_contiguous
    T, Hkv, D = k.shape
    k = _c(k, np.uint16)
    v = _c(v, np.uint16)
    sm = _c(slot_mapping, np.int64)
    assert sm.shape == (T,)
    _load().oracle_write_kv_fp8(_p(k_cache), _p(v_cache), _p(k), _p(v), _p(sm),
                                T, Hkv, BLOCK_SIZE, D, float(k_scale),
                                float(v_scale))


def attend_fp8(q, k_cache, v_cache, k_scale, v_scale, block_tables, seq_lens,
               query_start_loc, num_kv_heads, scale, rows=None,
               nthreads=None) -> np.ndarray:
    """Paged varlen causal attention over 8-bit pools (values decode(code) *
    scale, fp64): out [T][Hq][D], or [len(rows)][D] for selected (token,
    head) rows."""
    q = _c(q, np.uint16)
    T, Hq, D = q.shape
    bt = _c(block_tables, np.int32)
    sl = _c(seq_lens, np.int32)
    qsl = _c(query_start_loc, np.int32)
    B = sl.shape[0]
    assert qsl.shape == (B + 1,) and int(qsl[-1]) == T
    assert k_cache.dtype == np.uint8 and v_cache.dtype == np.uint8
    nthreads = nthreads or default_threads()
    maxL = max(1, int(sl.max()) if B else 1)
    scratch = np.empty(nthreads * maxL, np.float64)
    if rows is None:
        out = np.zeros((T, Hq, D), np.float64)
        rp, nrows = None, T * Hq
    else:
        rows = _c(rows, np.int64).reshape(-1, 2)
        out = np.zeros((rows.shape[0], D), np.float64)
        rp, nrows = _p(rows), rows.shape[0]
    _load().oracle_attend_fp8(_p(q), _p(k_cache), _p(v_cache), float(k_scale),
                              float(v_scale), _p(bt), bt.shape[1], _p(sl),
                              _p(qsl), B, Hq, num_kv_heads, BLOCK_SIZE, D,
                              float(scale), maxL, rp, nrows, _p(scratch),
                              _p(out), int(nthreads))
    return out


# ---- copy-on-write and larger blocks ----------------------------------------------

def copy_blocks(k_cache: np.ndarray, v_cache: np.ndarray, block_bytes: int,
                mapping) -> None:
    """In-place copy-on-write block copies over the pools' bytes (any dtype,
    C-contiguous): mapping [n][2] of (src, dst) block ids, applied in order."""
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    assert k_cache.nbytes == v_cache.nbytes and k_cache.nbytes % block_bytes == 0
    m = _c(mapping, np.int64).reshape(-1, 2)
    _load().oracle_copy_blocks(_p(k_cache), _p(v_cache), int(block_bytes),
                               k_cache.nbytes // int(block_bytes), _p(m), m.shape[0])


def expand_block_tables(block_tables, block_size: int) -> np.ndarray:
    """Tables of block_size-token blocks (a multiple of 16) -> 16-token ids."""
    bt = _c(block_tables, np.int32)
    R = int(block_size) // BLOCK_SIZE
    out = np.empty((bt.shape[0], bt.shape[1] * R), np.int32)
    _load().oracle_expand_block_tables(_p(bt), bt.shape[0], bt.shape[1],
                                       int(block_size), _p(out))
    return out


# ---- MLA latent cache ------------------------------------------------------------

MLA_BLOCK = 64
MLA_DL = 576   # latent (512) + rotary (64) dims cached per token
MLA_DV = 512   # latent dims summed into the output


def mla_index(n, t, d) -> int:
    """Flat element offset of dim d of token t of block n in an MLA cache."""
    return int(_load().oracle_mla_index(n, t, d))


def mla_write_kv(cache: np.ndarray, kv: np.ndarray, slot_mapping) -> None:
    """In-place scatter of kv ([T][576] uint16 bits) into the MLA cache."""
    assert cache.dtype == np.uint16 and cache.flags.c_contiguous
    kv = _c(kv, np.uint16)
    sm = _c(slot_mapping, np.int64)
    assert kv.shape == (sm.shape[0], MLA_DL)
    _load().oracle_mla_write_kv(_p(cache), _p(kv), _p(sm), sm.shape[0])


def mla_decode(q, cache, block_tables, seq_lens, query_start_loc, scale,
               nthreads=None) -> np.ndarray:
    """MLA attention (fp64): q [T][Hq][576] uint16 bits -> [T][Hq][512]."""
    q = _c(q, np.uint16)
    T, Hq, Dl = q.shape
    assert Dl == MLA_DL
    bt = _c(block_tables, np.int32)
    sl = _c(seq_lens, np.int32)
    qsl = _c(query_start_loc, np.int32)
    out = np.zeros((T, Hq, MLA_DV), np.float64)
    _load().oracle_mla_decode(_p(q), _p(cache), _p(bt), bt.shape[1], _p(sl), _p(qsl),
                              sl.shape[0], Hq, float(scale), _p(out),
                              nthreads or default_threads())
    return out
