"""GPU parity of the 8-bit (E4M3) KV cache path against the CPU oracle.

Bars: the 8-bit scatter bit-exact (every pool byte); attention over 8-bit
pools within the bf16 path's tolerance of the fp64 oracle on the same codes
(the codes stand for exact values, decode(code) * scale, so quantisation
error is common to both sides and not part of the comparison).
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_varlen_amd as pa
import workloads as W
from tests.gpu_util import bf16_tensor, i64
from tests.test_gpu_parity import SMALL, small

pytestmark = pytest.mark.gpu

SENTINEL = 0x7F  # the NaN code: an unwritten byte read by mistake shows as NaN


def u8_bits(t):
    return t.detach().contiguous().view(torch.uint8).cpu().numpy().ravel()


def oracle_pool8(w, k_scale, v_scale, fill=SENTINEL):
    kc = np.full(w.pool_elems(), fill, np.uint8)
    vc = kc.copy()
    if len(w.fill_rows):
        oracle.write_kv_fp8(kc, vc, w.k_dense[w.fill_rows], w.v_dense[w.fill_rows],
                            w.fill_slots, k_scale, v_scale)
    oracle.write_kv_fp8(kc, vc, w.k_new, w.v_new, w.new_slots, k_scale, v_scale)
    return kc, vc


def gpu_pool8(w, k_scale, v_scale, fill=SENTINEL):
    kc, vc = pa.alloc_pool_fp8(w.num_blocks, w.num_kv_heads, w.head_dim, fill=fill)
    if len(w.fill_rows):
        pa.write_kv_fp8(bf16_tensor(w.k_dense[w.fill_rows]), bf16_tensor(w.v_dense[w.fill_rows]),
                        i64(w.fill_slots), kc, vc, k_scale, v_scale)
    pa.write_kv_fp8(bf16_tensor(w.k_new), bf16_tensor(w.v_new), i64(w.new_slots), kc, vc,
                    k_scale, v_scale)
    return kc, vc


@pytest.mark.parametrize("name", ["mixed-g4-d128", "mixed-g1-d64", "mixed-h3-d64",
                                  "mixed-split-edge"])
@pytest.mark.parametrize("scales", [(1.0, 1.0), (0.05, 0.02), (3.0, 0.7)])
def test_write_kv_fp8_bit_exact(name, scales):
    w = small(name, seed=5)
    kc, vc = gpu_pool8(w, *scales)
    torch.cuda.synchronize()
    okc, ovc = oracle_pool8(w, *scales)
    assert np.array_equal(u8_bits(kc), okc)
    assert np.array_equal(u8_bits(vc), ovc)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("scales", [(1.0, 1.0), (0.37, 2.5)])
def test_write_kv_fp8_special_values_and_runs(D, scales):
    # quads of slots 4m..4m+3 of one block (one 16-byte V store), unaligned,
    # block-crossing, with a skipped or out-of-range slot, a partial tail;
    # values: zeros of both signs, infinities, NaN, saturation, exact ties
    # between codes, the subnormal range, random bits
    slots = np.array([32, 33, 34, 35, 49, 50, 51, 52, 60, 61, 62, 63,
                      64, 65, -1, 67, 124, 125, 126, 128, 78, 79, 80, 81,
                      96, 97, 98], np.int64)
    T, Hkv, nblocks = len(slots), 2, 8
    rng = np.random.default_rng(9)
    special = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 448.0, 464.0, 480.0,
                        -1e30, 1.0625, 1.1875, -3.25, 2.0 ** -10, 3 * 2.0 ** -10,
                        2.0 ** -6, 0.009765625, 200.0, -0.3], np.float32)
    vals = rng.standard_normal((T, Hkv, D)).astype(np.float32) * 3
    flat = vals.ravel()
    flat[rng.choice(flat.size, 400, replace=False)] = np.resize(special, 400)
    k = W.f32_to_bf16_bits(vals)
    v = rng.integers(0, 1 << 16, (T, Hkv, D), dtype=np.uint16)  # any bits, NaNs included
    kc, vc = pa.alloc_pool_fp8(nblocks, Hkv, D, fill=SENTINEL)
    pa.write_kv_fp8(bf16_tensor(k), bf16_tensor(v), i64(slots), kc, vc, *scales)
    torch.cuda.synchronize()
    okc = np.full(nblocks * Hkv * 16 * D, SENTINEL, np.uint8)
    ovc = okc.copy()
    oslots = np.where(slots < nblocks * 16, slots, -1)  # out of range: skipped
    oracle.write_kv_fp8(okc, ovc, k, v, oslots, *scales)
    assert np.array_equal(u8_bits(kc), okc)
    assert np.array_equal(u8_bits(vc), ovc)


def test_write_kv_fp8_strided_rows():
    w = small("mixed-g4-d128", seed=2)
    T, Hkv, D = w.k_new.shape
    fused = np.zeros((T, 3, Hkv, D), np.uint16)
    fused[:, 1] = w.k_new
    fused[:, 2] = w.v_new
    ft = bf16_tensor(fused)
    kc, vc = pa.alloc_pool_fp8(w.num_blocks, Hkv, D, fill=SENTINEL)
    pa.write_kv_fp8(ft[:, 1], ft[:, 2], i64(w.new_slots), kc, vc, 0.125, 0.0625)
    torch.cuda.synchronize()
    okc = np.full(w.pool_elems(), SENTINEL, np.uint8)
    ovc = okc.copy()
    oracle.write_kv_fp8(okc, ovc, w.k_new, w.v_new, w.new_slots, 0.125, 0.0625)
    assert np.array_equal(u8_bits(kc), okc)
    assert np.array_equal(u8_bits(vc), ovc)
