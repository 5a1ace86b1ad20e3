"""GPU parity of pools of 8-token blocks (pa_write_kv_bs, pa_attend_bs,
pa_gather_kv_bs with block_size 8).

Bars: the scatter and the logical gather bit-exact against the oracle's
(block-size-generic) scatter and gather; attention within max-abs 3e-2 and
mean-abs 2e-3 of the fp64 oracle over the same 8-token pools, every output
row; and, because attention over 8-token blocks gathers the same 16-key
steps that 16-token blocks hold, bit-identical outputs to pa_attend over the
same tokens in 16-token blocks and under any permutation of the physical
blocks.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_varlen_amd as pa
import workloads as W
from tests.gpu_util import bf16_tensor, i32, i64, tensor_bits
from tests.test_gpu_parity import check_close

pytestmark = pytest.mark.gpu

CASES = {
    # name: (seq_lens, query_lens, Hq, Hkv, D)
    # decodes of 1..many 8-token blocks, odd block counts, a split request
    "bs8-decode-g4-d128": ([1, 7, 8, 9, 15, 16, 17, 24, 25, 520, 1037, 3000],
                           [1] * 12, 32, 8, 128),
    # chunked-prefill chunks beside decodes, partial last blocks everywhere
    "bs8-mixed-g4-d128": ([1, 17, 40, 33, 64, 5, 16, 700, 1100, 2500],
                          [1, 1, 7, 33, 3, 0, 16, 1, 300, 200], 16, 4, 128),
    "bs8-mixed-g1-d64": ([3, 100, 530, 77, 49], [3, 1, 1, 70, 17], 4, 4, 64),
    "bs8-mixed-g8-d64": ([2, 9, 600, 1025, 265], [2, 1, 2, 1, 37], 16, 2, 64),
    # a chunk split across the 2048-key boundary
    "bs8-split-edge": ([2100, 41], [100, 1], 8, 2, 128),
}


def make(name, seed, block_size=8):
    L, Q, Hq, Hkv, D = CASES[name]
    return W.make_workload(name, L, Q, Hq, Hkv, D, seed=seed, block_size=block_size)


def gpu_pools(w, slots_fill=None, slots_new=None):
    bs = w.block_size
    kc, vc = pa.alloc_pool(w.num_blocks, w.num_kv_heads, w.head_dim, fill=float("nan"),
                           block_size=bs)
    fs = w.fill_slots if slots_fill is None else slots_fill
    ns = w.new_slots if slots_new is None else slots_new
    if len(w.fill_rows):
        pa.write_kv(bf16_tensor(w.k_dense[w.fill_rows]), bf16_tensor(w.v_dense[w.fill_rows]),
                    i64(fs), kc, vc, block_size=bs)
    pa.write_kv(bf16_tensor(w.k_new), bf16_tensor(w.v_new), i64(ns), kc, vc, block_size=bs)
    return kc, vc


def oracle_pools(w, slots_fill=None, slots_new=None):
    bs = w.block_size
    kc = np.full(w.pool_elems(), W.BF16_NAN, np.uint16)
    vc = kc.copy()
    fs = w.fill_slots if slots_fill is None else slots_fill
    ns = w.new_slots if slots_new is None else slots_new
    oracle.write_kv(kc, vc, w.k_dense[w.fill_rows], w.v_dense[w.fill_rows], fs, block_size=bs)
    oracle.write_kv(kc, vc, w.k_new, w.v_new, ns, block_size=bs)
    return kc, vc


def attend(w, kc, vc, tables=None):
    bt = w.block_tables if tables is None else tables
    out = pa.attend(bf16_tensor(w.q), kc, vc, i32(bt), i32(w.seq_lens),
                    i32(w.query_start_loc), w.scale, w.max_query_len, w.max_seq_len,
                    num_kv_heads=w.num_kv_heads, block_size=w.block_size)
    torch.cuda.synchronize()
    return tensor_bits(out)


@pytest.mark.parametrize("name", sorted(CASES))
def test_write_kv_bs8_bit_exact(name):
    w = make(name, seed=1)
    kc, vc = gpu_pools(w)
    torch.cuda.synchronize()
    okc, ovc = oracle_pools(w)
    assert np.array_equal(tensor_bits(kc).ravel(), okc)
    assert np.array_equal(tensor_bits(vc).ravel(), ovc)


def test_write_kv_bs8_strided_rows_and_skips():
    # rows with a stride, skipped (< 0) and out-of-range slots, quads of
    # consecutive slots that start mid-block and cross a block boundary
    rng = np.random.default_rng(5)
    Hkv, D, nb = 2, 128, 6
    slots = np.array([0, 1, 2, 3, 4, 5, 6, 7, 12, 13, 14, 15, 17, -1, 19, 20,
                      8 * nb, 22, 23, 30, 31, 32, 33, 40], np.int64)
    T = len(slots)
    big = rng.integers(0, 1 << 16, (T, Hkv * D + 64), dtype=np.uint16)
    kb, vb = bf16_tensor(big), bf16_tensor(big[::-1].copy())
    k = kb[:, :Hkv * D].view(T, Hkv, D)
    v = vb[:, 64:].view(T, Hkv, D)
    kc, vc = pa.alloc_pool(nb, Hkv, D, fill=float("nan"), block_size=8)
    pa.write_kv(k, v, i64(slots), kc, vc, block_size=8)
    torch.cuda.synchronize()
    okc = np.full(nb * Hkv * 8 * D, W.BF16_NAN, np.uint16)
    ovc = okc.copy()
    oracle.write_kv(okc, ovc, tensor_bits(k), tensor_bits(v), np.where(slots < 8 * nb, slots, -1),
                    block_size=8)
    assert np.array_equal(tensor_bits(kc).ravel(), okc)
    assert np.array_equal(tensor_bits(vc).ravel(), ovc)


@pytest.mark.parametrize("name", ["bs8-mixed-g4-d128", "bs8-mixed-g1-d64"])
def test_gather_kv_bs8_bit_exact(name):
    w = make(name, seed=2)
    kc, vc = gpu_pools(w)
    total = int(w.seq_lens.sum())
    ko, vo = pa.gather_kv(kc, vc, i32(w.block_tables), i32(w.seq_lens), i64(w.kv_start),
                          total, w.num_kv_heads, w.head_dim, block_size=8)
    torch.cuda.synchronize()
    assert np.array_equal(tensor_bits(ko), w.k_dense)
    assert np.array_equal(tensor_bits(vo), w.v_dense)


@pytest.mark.parametrize("name", sorted(CASES))
def test_attend_bs8_parity(name):
    w = make(name, seed=3)
    kc, vc = gpu_pools(w)
    got = attend(w, kc, vc)
    okc, ovc = oracle_pools(w)
    ref = oracle.attend(w.q, okc, ovc, w.block_tables, w.seq_lens, w.query_start_loc,
                        w.num_kv_heads, w.scale, block_size=8)
    check_close(got, ref, name)


@pytest.mark.parametrize("name", sorted(CASES))
def test_attend_bs8_equals_16_token_blocks(name):
    # the same tokens in 16-token blocks through pa_attend: the same bits
    w8, w16 = make(name, seed=4), make(name, seed=4, block_size=16)
    assert np.array_equal(w8.q, w16.q) and np.array_equal(w8.k_dense, w16.k_dense)
    kc8, vc8 = gpu_pools(w8)
    a = attend(w8, kc8, vc8)
    kc16, vc16 = gpu_pools(w16)
    b = attend(w16, kc16, vc16)
    assert np.array_equal(a, b)


def test_attend_bs8_block_permutation_is_bit_identical():
    w = make("bs8-mixed-g4-d128", seed=6)
    kc, vc = gpu_pools(w)
    a = attend(w, kc, vc)
    perm = np.random.default_rng(7).permutation(w.num_blocks)
    bt = w.block_tables.copy()
    bt[bt >= 0] = perm[bt[bt >= 0]]
    rel = lambda s: np.where(s >= 0, perm[s // 8] * 8 + s % 8, s)  # noqa: E731
    kc2, vc2 = gpu_pools(w, rel(w.fill_slots), rel(w.new_slots))
    b = attend(w, kc2, vc2, tables=bt)
    assert np.array_equal(a, b)


def test_attend_bs8_llama3_8b_decode_layer():
    # the 8B decode layer's shapes (64 requests, U[128, 4096]) in 8-token
    # blocks: every output row against the oracle
    L, Q = W.config_lengths(2)
    w = W.make_workload("llama3-8b-decode-64seq-bs8", L, Q, 32, 8, 128, seed=2, block_size=8)
    kc, vc = gpu_pools(w)
    got = attend(w, kc, vc)
    okc, ovc = oracle_pools(w)
    ref = oracle.attend(w.q, okc, ovc, w.block_tables, w.seq_lens, w.query_start_loc,
                        w.num_kv_heads, w.scale, block_size=8)
    check_close(got, ref, "8B decode layer, 8-token blocks")


def test_bs_argument_checks():
    w = make("bs8-mixed-g1-d64", seed=8)
    kc, vc = gpu_pools(w)
    with pytest.raises(pa.PAError):
        pa.write_kv(bf16_tensor(w.k_new), bf16_tensor(w.v_new), i64(w.new_slots), kc, vc,
                    block_size=4)
