"""C-ABI checks that need no GPU: libpa.so loads, exports every function
include/pa.h declares, rejects bad arguments before touching the device, and
its host-side metadata validator flags invalid content."""
import ctypes
import os
import re

import numpy as np
import pytest

import workloads as W
from paged_kv_cache_varlen_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        import paged_kv_cache_varlen_amd._build as b
        b.build()
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(_lib.SIGNATURES)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.pa_abi_version() == 1
    assert lib.pa_status_string(0) == b"ok"
    assert lib.pa_status_string(4) == b"workspace too small"


def test_workspace_size(lib):
    a = lib.pa_attend_workspace_size(64, 64, 32, 8, 128, 1, 4096)
    b = lib.pa_attend_workspace_size(64, 64, 32, 8, 128, 1, 8192)
    assert 0 < a < b
    assert lib.pa_attend_workspace_size(64, 64, 32, 8, 96, 1, 4096) == 0   # head_dim
    assert lib.pa_attend_workspace_size(64, 64, 30, 8, 128, 1, 4096) == 0  # Hq % Hkv
    assert lib.pa_attend_workspace_size(64, 64, 64, 2, 128, 1, 4096) == 0  # G > 16
    assert lib.pa_attend_workspace_size(-1, 64, 32, 8, 128, 1, 4096) == 0


FAKE = 1 << 20  # a non-NULL, 256-aligned pointer value: never dereferenced


def attend_args(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, nb=10, bt=FAKE, mb=4, sl=FAKE, qsl=FAKE,
             B=2, T=2, Hq=8, Hkv=2, D=128, mq=1, ms=64, scale=0.1, out=FAKE,
             ws=FAKE, wsb=1 << 30, stream=None)
    a.update(over)
    return [a[k] for k in ("q", "k", "v", "nb", "bt", "mb", "sl", "qsl", "B", "T",
                           "Hq", "Hkv", "D", "mq", "ms", "scale", "out", "ws",
                           "wsb", "stream")]


@pytest.mark.parametrize("over,status", [
    (dict(q=None), _lib.PA_ERR_NULL),
    (dict(out=None), _lib.PA_ERR_NULL),
    (dict(D=96), _lib.PA_ERR_UNSUPPORTED),
    (dict(Hq=6, Hkv=4), _lib.PA_ERR_SHAPE),
    (dict(Hq=64, Hkv=2), _lib.PA_ERR_UNSUPPORTED),
    (dict(T=-1), _lib.PA_ERR_SHAPE),
    (dict(ws=None), _lib.PA_ERR_WORKSPACE),
    (dict(wsb=100), _lib.PA_ERR_WORKSPACE),
    (dict(ws=FAKE + 16), _lib.PA_ERR_WORKSPACE),
    (dict(q=FAKE + 2), _lib.PA_ERR_SHAPE),
    (dict(scale=0.0), _lib.PA_ERR_SHAPE),
    (dict(scale=-0.125), _lib.PA_ERR_SHAPE),
    (dict(scale=float("nan")), _lib.PA_ERR_SHAPE),
    (dict(scale=float("inf")), _lib.PA_ERR_SHAPE),
    (dict(nb=(1 << 31), Hkv=2), _lib.PA_ERR_SHAPE),  # tiles past 2^32
])
def test_attend_rejects_bad_arguments(lib, over, status):
    assert lib.pa_attend(*attend_args(**over)) == status
    assert lib.pa_last_error() != b""


def noalloc_args(**over):
    a = attend_args(**over)
    return a[:17] + a[19:]  # no workspace arguments


@pytest.mark.parametrize("over,status", [
    (dict(q=None), _lib.PA_ERR_NULL),
    (dict(D=96), _lib.PA_ERR_UNSUPPORTED),
    (dict(Hq=6, Hkv=4), _lib.PA_ERR_SHAPE),
    (dict(scale=0.0), _lib.PA_ERR_SHAPE),
    (dict(q=FAKE + 2), _lib.PA_ERR_SHAPE),
    # bounds whose workspace exceeds the static scratch (64 MiB)
    (dict(B=129, T=2048, Hq=32, Hkv=8, mq=1920, ms=8192, mb=512), _lib.PA_ERR_WORKSPACE),
])
def test_attend_noalloc_rejects_bad_arguments(lib, over, status):
    # host checks only: every one of these returns before any device call
    assert lib.pa_attend_noalloc(*noalloc_args(**over)) == status
    assert lib.pa_last_error() != b""


def test_attend_noalloc_scratch_limit(lib):
    # the documented examples: decode batches that fit, a mixed step that does not
    limit = 64 << 20
    assert lib.pa_attend_workspace_size(64, 64, 32, 8, 128, 1, 4096) <= limit
    assert lib.pa_attend_workspace_size(16, 16, 64, 8, 128, 1, 32768) <= limit
    assert lib.pa_attend_workspace_size(129, 2048, 32, 8, 128, 1920, 8192) > limit


@pytest.mark.parametrize("bs,status", [(4, _lib.PA_ERR_UNSUPPORTED),
                                       (32, _lib.PA_ERR_UNSUPPORTED)])
def test_block_size_calls_reject_other_sizes(lib, bs, status):
    a = attend_args()
    assert lib.pa_attend_bs(*(a[:4] + [bs] + a[4:])) == status
    assert lib.pa_write_kv_bs(FAKE, FAKE, 256, 256, FAKE, 4, 2, 128, FAKE, FAKE, 8, bs,
                              None) == status
    assert lib.pa_gather_kv_bs(FAKE, FAKE, 8, bs, FAKE, 4, FAKE, FAKE, 2, 10, 2, 128, FAKE,
                               FAKE, None) == status


def test_block_size_8_argument_checks(lib):
    # the checks of the block-size-16 calls apply unchanged
    a = attend_args(D=96)
    assert lib.pa_attend_bs(*(a[:4] + [8] + a[4:])) == _lib.PA_ERR_UNSUPPORTED
    a = attend_args(wsb=100)
    assert lib.pa_attend_bs(*(a[:4] + [8] + a[4:])) == _lib.PA_ERR_WORKSPACE
    a = attend_args(T=0, q=None, out=None)
    assert lib.pa_attend_bs(*(a[:4] + [8] + a[4:])) == _lib.PA_OK
    assert lib.pa_write_kv_bs(None, FAKE, 256, 256, FAKE, 4, 2, 128, FAKE, FAKE, 8, 8,
                              None) == _lib.PA_ERR_NULL
    assert lib.pa_write_kv_bs(None, None, 256, 256, None, 0, 2, 128, None, None, 8, 8,
                              None) == _lib.PA_OK


def test_attend_empty_batch_is_ok(lib):
    assert lib.pa_attend(*attend_args(T=0, q=None, out=None)) == _lib.PA_OK


@pytest.mark.parametrize("args,status", [
    ((FAKE, FAKE, 256, 256, FAKE, 4, 2, 96, FAKE, FAKE, 8, None), _lib.PA_ERR_UNSUPPORTED),
    ((None, FAKE, 256, 256, FAKE, 4, 2, 128, FAKE, FAKE, 8, None), _lib.PA_ERR_NULL),
    ((FAKE, FAKE, 100, 256, FAKE, 4, 2, 128, FAKE, FAKE, 8, None), _lib.PA_ERR_SHAPE),
    ((FAKE, FAKE, 256, 256, FAKE, -4, 2, 128, FAKE, FAKE, 8, None), _lib.PA_ERR_SHAPE),
    ((FAKE, FAKE, 256, 256, FAKE, 0, 2, 128, None, None, 8, None), _lib.PA_OK),
])
def test_write_kv_argument_checks(lib, args, status):
    assert lib.pa_write_kv(*args) == status


def _w8(k=FAKE, stride=256, T=4, D=128, ks=0.5, vs=0.25, kc=FAKE):
    return (k, FAKE, stride, 256, FAKE, T, 2, D, ks, vs, kc, FAKE, 8, None)


@pytest.mark.parametrize("args,status", [
    (_w8(D=96), _lib.PA_ERR_UNSUPPORTED),
    (_w8(k=None), _lib.PA_ERR_NULL),
    (_w8(stride=100), _lib.PA_ERR_SHAPE),
    (_w8(T=-4), _lib.PA_ERR_SHAPE),
    (_w8(ks=0.0), _lib.PA_ERR_SHAPE),
    (_w8(vs=-1.0), _lib.PA_ERR_SHAPE),
    (_w8(ks=float("nan")), _lib.PA_ERR_SHAPE),
    (_w8(vs=float("inf")), _lib.PA_ERR_SHAPE),
    (_w8(k=FAKE + 8), _lib.PA_ERR_SHAPE),
    (_w8(T=0, k=None, kc=None), _lib.PA_OK),
])
def test_write_kv_fp8_argument_checks(lib, args, status):
    assert lib.pa_write_kv_fp8(*args) == status


def _wp(k=FAKE, D=128, T=4, C=-1, wsb=1 << 30, bt=FAKE, fp8=None):
    """pa_write_kv_plan(_fp8) arguments: 4 new tokens, 2 requests of 8 query
    tokens over 2 kv heads, a workspace of wsb bytes."""
    scatter = [k, FAKE, 256, 256, FAKE, T]
    if fp8 is not None:
        scatter += list(fp8)
    return tuple(scatter + [FAKE, FAKE, 8, bt, 4, FAKE, FAKE, 2, 8, 4, 2, D, 4, 60, C,
                            FAKE, wsb, None])


@pytest.mark.parametrize("args,status", [
    (_wp(D=96), _lib.PA_ERR_UNSUPPORTED),
    (_wp(k=None), _lib.PA_ERR_NULL),
    (_wp(T=-1), _lib.PA_ERR_SHAPE),
    (_wp(bt=None), _lib.PA_ERR_NULL),
    (_wp(wsb=64), _lib.PA_ERR_WORKSPACE),
    (_wp(C=61), _lib.PA_ERR_SHAPE),
])
def test_write_kv_plan_argument_checks(lib, args, status):
    assert lib.pa_write_kv_plan(*args) == status


@pytest.mark.parametrize("args,status", [
    (_wp(fp8=(0.0, 1.0)), _lib.PA_ERR_SHAPE),
    (_wp(fp8=(1.0, float("nan"))), _lib.PA_ERR_SHAPE),
    (_wp(fp8=(1.0, 1.0), D=96), _lib.PA_ERR_UNSUPPORTED),
    (_wp(fp8=(1.0, 1.0), wsb=64), _lib.PA_ERR_WORKSPACE),
])
def test_write_kv_plan_fp8_argument_checks(lib, args, status):
    assert lib.pa_write_kv_plan_fp8(*args) == status


def test_attend_plan_fp8_argument_checks(lib):
    ws = lib.pa_attend_workspace_size(2, 8, 4, 2, 128, 4, 60)
    args = (FAKE, 4, FAKE, FAKE, 2, 8, 4, 2, 128, 4, 60, FAKE)
    assert lib.pa_attend_plan_fp8(*args, ws - 1, None) == _lib.PA_ERR_WORKSPACE
    assert lib.pa_attend_plan_fp8(None, *args[1:], ws, None) == _lib.PA_ERR_NULL
    assert lib.pa_attend_plan_fp8(*args[:8], 96, *args[9:], ws, None) == _lib.PA_ERR_UNSUPPORTED


def test_write_kv_plan_workspace_sizes(lib):
    # a plain plan needs the plain workspace, a shared-prefix plan the larger one
    plain = lib.pa_attend_workspace_size(2, 8, 4, 2, 128, 4, 60)
    casc = lib.pa_attend_cascade_workspace_size(2, 8, 4, 2, 128, 4, 60)
    assert 0 < plain < casc
    assert lib.pa_write_kv_plan(*_wp(C=32, wsb=plain)) == _lib.PA_ERR_WORKSPACE
    assert lib.pa_write_kv_plan(*_wp(C=-1, wsb=plain - 1)) == _lib.PA_ERR_WORKSPACE


def test_gather_argument_checks(lib):
    st = lib.pa_gather_kv(None, FAKE, 8, FAKE, 4, FAKE, FAKE, 2, 10, 2, 64, FAKE,
                          FAKE, None)
    assert st == _lib.PA_ERR_NULL
    st = lib.pa_gather_kv(FAKE, FAKE, 8, FAKE, 4, FAKE, FAKE, 2, 10, 2, 80, FAKE,
                          FAKE, None)
    assert st == _lib.PA_ERR_UNSUPPORTED


# ---- host metadata validator ---------------------------------------------------------

def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def validate(lib, w, bt=None, sl=None, qsl=None, slots=None, mq=None, ms=None,
             nb=None):
    bt = np.ascontiguousarray(w.block_tables if bt is None else bt, np.int32)
    sl = np.ascontiguousarray(w.seq_lens if sl is None else sl, np.int32)
    qsl = np.ascontiguousarray(w.query_start_loc if qsl is None else qsl, np.int32)
    slots = np.ascontiguousarray(w.new_slots if slots is None else slots, np.int64)
    return lib.pa_validate_metadata_host(
        _p(bt), bt.shape[1], _p(sl), _p(qsl), sl.shape[0], int(qsl[-1]),
        w.max_query_len if mq is None else mq, w.max_seq_len if ms is None else ms,
        w.num_blocks if nb is None else nb, _p(slots), slots.shape[0])


@pytest.fixture(scope="module")
def wl():
    return W.make_workload("v", [1, 17, 40, 33, 64, 5], [1, 1, 7, 33, 3, 0], 8, 2,
                           64, seed=0)


def test_validator_accepts_generated_metadata(lib, wl):
    assert validate(lib, wl) == _lib.PA_OK
    allslots = np.concatenate([wl.fill_slots, wl.new_slots])
    assert validate(lib, wl, slots=allslots) == _lib.PA_OK
    for k in (1, 2):
        w = W.make_config(k)
        assert validate(lib, w, slots=np.concatenate([w.fill_slots, w.new_slots])) == 0


def test_validator_rejects_bad_content(lib, wl):
    M = _lib.PA_ERR_METADATA
    bt = wl.block_tables.copy()
    bt[2, 1] = wl.num_blocks
    assert validate(lib, wl, bt=bt) == M
    bt = wl.block_tables.copy()
    bt[4, 0] = -3
    assert validate(lib, wl, bt=bt) == M
    sl = wl.seq_lens.copy()
    sl[3] = 20  # Q = 33 > L
    assert validate(lib, wl, sl=sl) == M
    qsl = wl.query_start_loc.copy()
    qsl[2], qsl[3] = qsl[3], qsl[2]
    assert validate(lib, wl, qsl=qsl) == M
    slots = wl.new_slots.copy()
    slots[1] = slots[0]
    assert validate(lib, wl, slots=slots) == M
    slots = wl.new_slots.copy()
    slots[0] = wl.num_blocks * 16
    assert validate(lib, wl, slots=slots) == M
    assert validate(lib, wl, ms=50) == M   # L = 64 > max_seq_len
    assert validate(lib, wl, mq=3) == M    # Q = 33 > max_query_len
    bt = wl.block_tables[:, :2].copy()     # row too short for L = 64
    assert validate(lib, wl, bt=bt) == M
    assert "request" in lib.pa_last_error().decode()


# ---- shared-prefix (cascade) calls -----------------------------------------------------

def test_cascade_workspace_size(lib):
    plain = lib.pa_attend_workspace_size(256, 256, 32, 8, 128, 1, 2560)
    casc = lib.pa_attend_cascade_workspace_size(256, 256, 32, 8, 128, 1, 2560)
    # the prefix section: up to 8 key ranges per query token, each a float2
    # and a D-float partial per query head, plus its work items
    assert casc >= plain + 256 * 8 * 32 * (128 + 2) * 4
    assert lib.pa_attend_cascade_workspace_size(256, 256, 32, 8, 96, 1, 2560) == 0
    assert lib.pa_attend_cascade_workspace_size(-1, 256, 32, 8, 128, 1, 2560) == 0


def cascade_args(prefix=32, **over):
    a = attend_args(**over)
    return a[:15] + [prefix] + a[15:]


@pytest.mark.parametrize("prefix,over,status", [
    (-1, {}, _lib.PA_ERR_SHAPE),
    (65, {}, _lib.PA_ERR_SHAPE),                     # > max_seq_len
    (32, dict(q=None), _lib.PA_ERR_NULL),
    (32, dict(D=96), _lib.PA_ERR_UNSUPPORTED),
    (32, dict(scale=0.0), _lib.PA_ERR_SHAPE),
    (32, dict(ws=None), _lib.PA_ERR_WORKSPACE),
])
def test_cascade_rejects_bad_arguments(lib, prefix, over, status):
    assert lib.pa_attend_cascade(*cascade_args(prefix, **over)) == status
    assert lib.pa_last_error() != b""


def test_cascade_needs_the_larger_workspace(lib):
    plain = lib.pa_attend_workspace_size(2, 2, 8, 2, 128, 1, 64)
    casc = lib.pa_attend_cascade_workspace_size(2, 2, 8, 2, 128, 1, 64)
    assert casc > plain
    assert lib.pa_attend_cascade(*cascade_args(32, wsb=plain)) == _lib.PA_ERR_WORKSPACE
    assert b"shared-prefix" in lib.pa_last_error()
    a = attend_args(wsb=plain)
    # the planned / merge variants check the same size
    assert lib.pa_attend_planned_cascade(*a) == _lib.PA_ERR_WORKSPACE
    assert lib.pa_attend_merge_cascade(2, 2, 8, 2, 128, 1, 64, FAKE, FAKE, plain,
                                       None) == _lib.PA_ERR_WORKSPACE
    assert lib.pa_attend_plan_cascade(FAKE, 4, FAKE, FAKE, 2, 2, 8, 2, 128, 1, 64, 32,
                                      FAKE, plain, None) == _lib.PA_ERR_WORKSPACE


def test_cascade_fp8_scale_checks(lib):
    a = cascade_args(32)
    args = a[:17] + [0.0, 1.0] + a[17:]  # k_scale 0
    assert lib.pa_attend_cascade_fp8(*args) == _lib.PA_ERR_SHAPE


def test_cascade_empty_batch_is_ok(lib):
    assert lib.pa_attend_cascade(*cascade_args(32, T=0, q=None, out=None)) == _lib.PA_OK


def validate_cascade(lib, w, prefix, bt=None, sl=None, qsl=None):
    bt = np.ascontiguousarray(w.block_tables if bt is None else bt, np.int32)
    sl = np.ascontiguousarray(w.seq_lens if sl is None else sl, np.int32)
    qsl = np.ascontiguousarray(w.query_start_loc if qsl is None else qsl, np.int32)
    return lib.pa_validate_cascade_host(_p(bt), bt.shape[1], _p(sl), _p(qsl),
                                        bt.shape[0], prefix)


def test_cascade_validator(lib):
    M = _lib.PA_ERR_METADATA
    w = W.make_workload("c", [100, 90, 300, 80], [1, 20, 200, 6], 8, 2, 64, seed=1,
                        shared_prefix=64)
    assert validate_cascade(lib, w, 64) == _lib.PA_OK
    assert validate_cascade(lib, w, 70) == _lib.PA_OK   # L - Q >= 70 everywhere
    assert validate_cascade(lib, w, 71) == M            # request 1: L - Q = 70
    assert "request 1" in lib.pa_last_error().decode()
    bt = w.block_tables.copy()
    bt[2, 3] = w.num_blocks - 1                         # differs inside the prefix
    assert validate_cascade(lib, w, 64, bt=bt) == M
    assert validate_cascade(lib, w, 48, bt=bt) == _lib.PA_OK  # block 3 not shared
    u = W.make_workload("u", [100, 90], [1, 20], 8, 2, 64, seed=1, shared_prefix=64,
                        shared=False)                  # private copies: other ids
    assert validate_cascade(lib, u, 64) == M


def test_copy_blocks_argument_checks(lib):
    assert lib.pa_copy_blocks(FAKE, FAKE, 8, 2, 128, 2, FAKE, 0, None) == _lib.PA_OK
    assert lib.pa_copy_blocks(FAKE, FAKE, 8, 2, 128, 3, FAKE, 1, None) == _lib.PA_ERR_SHAPE
    assert lib.pa_copy_blocks(FAKE, FAKE, 8, 2, 96, 2, FAKE, 1, None) == _lib.PA_ERR_UNSUPPORTED
    assert lib.pa_copy_blocks(None, FAKE, 8, 2, 128, 2, FAKE, 1, None) == _lib.PA_ERR_NULL
    assert lib.pa_copy_blocks(FAKE + 8, FAKE, 8, 2, 128, 2, FAKE, 1, None) == _lib.PA_ERR_SHAPE
    assert lib.pa_copy_blocks(FAKE, FAKE, 8, 2, 128, 2, FAKE, -1, None) == _lib.PA_ERR_SHAPE


def test_expand_block_tables_argument_checks(lib):
    assert lib.pa_expand_block_tables(FAKE, 4, 8, 24, FAKE, None) == _lib.PA_ERR_UNSUPPORTED
    assert lib.pa_expand_block_tables(FAKE, 4, 8, 8, FAKE, None) == _lib.PA_ERR_UNSUPPORTED
    assert lib.pa_expand_block_tables(None, 4, 8, 32, FAKE, None) == _lib.PA_ERR_NULL
    assert lib.pa_expand_block_tables(FAKE, 0, 8, 32, FAKE, None) == _lib.PA_OK
    assert lib.pa_expand_block_tables(FAKE, 4, 1 << 30, 64, FAKE, None) == _lib.PA_ERR_SHAPE


# ---- MLA latent decode --------------------------------------------------------------

FAKE = 4096  # a 256-byte-aligned non-NULL address: every call below fails its checks first


def mla_args(**over):
    a = dict(q=FAKE, cache=FAKE, nb=16, bt=FAKE, mbs=4, sl=FAKE, qsl=FAKE, B=2, T=2, Hq=16,
             maxL=256, scale=0.07, out=FAKE, ws=FAKE, wsb=1 << 30, stream=None)
    a.update(over)
    return [a[k] for k in ("q", "cache", "nb", "bt", "mbs", "sl", "qsl", "B", "T", "Hq", "maxL",
                           "scale", "out", "ws", "wsb", "stream")]


def test_mla_workspace_size(lib):
    small = lib.pa_mla_workspace_size(64, 16, 4096)
    assert small > 0 and small % 256 == 0
    # more heads, more partial rows (16 heads: enough for the grouped form's
    # 128 (token, head) rows per slot as well; 48 heads have no grouped form)
    assert lib.pa_mla_workspace_size(64, 128, 4096) >= small
    assert lib.pa_mla_workspace_size(64, 48, 4096) < lib.pa_mla_workspace_size(64, 128, 4096)
    assert lib.pa_mla_workspace_size(64, 24, 4096) == 0      # not a multiple of 16
    assert lib.pa_mla_workspace_size(-1, 16, 4096) == 0
    # past the token limit: no size, and the decode refuses it
    assert lib.pa_mla_workspace_size(1 << 25, 16, 4096) == 0
    assert lib.pa_mla_workspace_size((1 << 25) - 1, 16, 4096) > 0
    # enough for the grouped form too (128 (token, head) rows per slot)
    assert small >= 2 * 256 * 128 * 512 * 2


@pytest.mark.parametrize("over,status", [
    (dict(Hq=24), _lib.PA_ERR_UNSUPPORTED),
    (dict(Hq=144), _lib.PA_ERR_UNSUPPORTED),
    (dict(maxL=(1 << 18) + 1), _lib.PA_ERR_UNSUPPORTED),
    (dict(B=(1 << 17) + 1), _lib.PA_ERR_UNSUPPORTED),
    (dict(nb=(1 << 29) + 1), _lib.PA_ERR_UNSUPPORTED),
    (dict(T=1 << 25), _lib.PA_ERR_UNSUPPORTED),                        # token index bits
    (dict(q=None), _lib.PA_ERR_NULL),
    (dict(scale=0.0), _lib.PA_ERR_SHAPE),
    (dict(q=FAKE + 8), _lib.PA_ERR_SHAPE),                              # 16-byte alignment
    (dict(ws=None), _lib.PA_ERR_WORKSPACE),
    (dict(wsb=256), _lib.PA_ERR_WORKSPACE),
    (dict(ws=FAKE + 16), _lib.PA_ERR_WORKSPACE),                        # 256-byte alignment
    (dict(T=-1), _lib.PA_ERR_SHAPE),
])
def test_mla_decode_rejects_bad_arguments(lib, over, status):
    assert lib.pa_mla_decode(*mla_args(**over)) == status
    assert lib.pa_last_error() != b""


def test_mla_decode_empty_batch_is_ok(lib):
    assert lib.pa_mla_decode(*mla_args(T=0)) == _lib.PA_OK
    assert lib.pa_mla_decode(*mla_args(B=0)) == _lib.PA_OK
