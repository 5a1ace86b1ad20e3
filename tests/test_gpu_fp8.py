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
from tests import configs
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


# ---- attention over 8-bit pools -----------------------------------------------------

from tests.test_gpu_parity import check_close, sample_rows, to64  # noqa: E402
from tests.gpu_util import i32, tensor_bits  # noqa: E402


def attend8(w, kc, vc, ks, vs, planned=False, fp8_plan=True):
    bt, sl, qsl = i32(w.block_tables), i32(w.seq_lens), i32(w.query_start_loc)
    q = bf16_tensor(w.q)
    ws = pa.alloc_workspace(w.num_seqs, w.num_q_tokens, w.num_q_heads, w.num_kv_heads,
                            w.head_dim, w.max_query_len, w.max_seq_len)
    if planned:
        pa.attend_plan(bt, sl, qsl, w.num_q_tokens, w.num_q_heads, w.num_kv_heads,
                       w.head_dim, w.max_query_len, w.max_seq_len, ws, fp8=fp8_plan)
    out = pa.attend(q, kc, vc, bt, sl, qsl, w.scale, w.max_query_len, w.max_seq_len,
                    num_kv_heads=w.num_kv_heads, workspace=ws, planned=planned,
                    k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    return tensor_bits(out)


# scales: 1 (codes of N(0,1) data: the 3-bit mantissa, no saturation), the
# usual amax / 448 choice for N(0,1) data, and a pair that saturates often
SCALES = [(1.0, 1.0), (0.011, 0.0107), (0.004, 0.0045)]


@pytest.mark.parametrize("name", sorted(SMALL))
@pytest.mark.parametrize("scales", SCALES)
def test_attend_fp8_small(name, scales):
    w = small(name, seed=3)
    kc, vc = gpu_pool8(w, *scales)
    got = attend8(w, kc, vc, *scales)
    okc, ovc = oracle_pool8(w, *scales)
    ref = oracle.attend_fp8(w.q, okc, ovc, scales[0], scales[1], w.block_tables,
                            w.seq_lens, w.query_start_loc, w.num_kv_heads, w.scale)
    check_close(got, ref, "%s fp8 %s" % (name, scales))


@pytest.mark.parametrize("name", ["mixed-g4-d128", "mixed-g7-d64", "mixed-split-edge"])
def test_attend_fp8_planned_equals_unplanned(name):
    w = small(name, seed=4)
    kc, vc = gpu_pool8(w, 0.02, 0.03)
    a = attend8(w, kc, vc, 0.02, 0.03)
    b = attend8(w, kc, vc, 0.02, 0.03, planned=True)
    assert np.array_equal(a, b)


def test_attend_fp8_block_permutation_is_bit_identical():
    # outputs depend on logical positions only: a random re-placement of the
    # physical blocks gives the same bits
    w = small("mixed-g4-d128", seed=6)
    kc, vc = gpu_pool8(w, 0.015, 0.012)
    a = attend8(w, kc, vc, 0.015, 0.012)
    rng = np.random.default_rng(12)
    perm = rng.permutation(w.num_blocks)
    w2 = small("mixed-g4-d128", seed=6)
    bt = w.block_tables.copy()
    valid = bt >= 0
    bt[valid] = perm[bt[valid]]
    w2.block_tables = bt
    rel = lambda s: np.where(s >= 0, perm[s // 16] * 16 + s % 16, s)  # noqa: E731
    w2.fill_slots = rel(w.fill_slots)
    w2.new_slots = rel(w.new_slots)
    kc2, vc2 = gpu_pool8(w2, 0.015, 0.012)
    b = attend8(w2, kc2, vc2, 0.015, 0.012)
    assert np.array_equal(a, b)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_config_parity_fp8(k):
    # full size: every pool byte against the oracle's 8-bit scatter and every
    # output row against the oracle's attention over the same codes
    w = configs.workload(k)
    ks, vs = configs.FP8_SCALES
    kc, vc = gpu_pool8(w, ks, vs)
    got = attend8(w, kc, vc, ks, vs)
    okc, ovc = configs.pool8(k)
    assert np.array_equal(u8_bits(kc), okc)
    assert np.array_equal(u8_bits(vc), ovc)
    del kc, vc
    torch.cuda.empty_cache()
    check_close(got, configs.attend8(k), "config %d fp8 (all %d rows)" % (k, got.shape[0] * got.shape[1]))


@pytest.mark.parametrize("k", [2])
def test_plain_plan_serves_8bit_pools(k):
    # the 8-bit plan (here a stream plan of 8 units per CU) and the bf16
    # plan (4 per CU) cut the batch differently; both serve 8-bit pools,
    # within the tolerance of the oracle on the same codes, every output row
    w = configs.workload(k)
    scales = configs.FP8_SCALES
    kc, vc = gpu_pool8(w, *scales)
    a = attend8(w, kc, vc, *scales, planned=True, fp8_plan=False)
    b = attend8(w, kc, vc, *scales, planned=True, fp8_plan=True)
    assert not np.array_equal(a, b)  # other splits, other rounding
    ref = configs.attend8(k)
    for bits, what in ((a, "bf16 plan"), (b, "8-bit plan")):
        check_close(bits, ref, what)


# ---- 8-bit decode-only plans (384-key ranges) ---------------------------------------

DEC8 = {
    # name: (seq_lens, query_lens, Hq, Hkv, D); max_query_len <= 16 / G, so
    # these are planned with the 8-bit plan's 384-key decode ranges
    "dec8-g4-edges": ([383, 384, 385, 767, 768, 769, 1151, 1152, 1153, 8191, 8192,
                       8193, 9000, 1, 2, 31, 32, 33], [1] * 18, 32, 8, 128),
    "dec8-g4-q4": ([4, 5, 384, 388, 770, 1155, 2000, 8192, 8196, 7],
                   [4, 1, 4, 3, 2, 4, 1, 4, 2, 4], 32, 8, 128),
    "dec8-g1-q16-d64": ([16, 400, 769, 1536, 8190, 8200, 20],
                        [16, 16, 9, 1, 16, 5, 13], 4, 4, 64),
}


@pytest.mark.parametrize("name", sorted(DEC8))
def test_attend_fp8_decode_plan(name):
    L, Q, Hq, Hkv, D = DEC8[name]
    w = W.make_workload(name, L, Q, Hq, Hkv, D, seed=31)
    scales = (0.02, 0.017)
    kc, vc = gpu_pool8(w, *scales)
    a = attend8(w, kc, vc, *scales)
    b = attend8(w, kc, vc, *scales, planned=True)
    assert np.array_equal(a, b)
    okc, ovc = oracle_pool8(w, *scales)
    ref = oracle.attend_fp8(w.q, okc, ovc, *scales, w.block_tables, w.seq_lens,
                            w.query_start_loc, w.num_kv_heads, w.scale)
    check_close(a, ref, name)


def test_attend_fp8_decode_plan_many_requests():
    # more requests than the plan's workgroup has threads: the two-sweep plan
    # with its bucketed last splits, every output row
    rng = np.random.default_rng(32)
    B = 1100
    L = rng.integers(1, 2400, size=B)
    Q = np.minimum(L, rng.integers(1, 3, size=B))
    w = W.make_workload("dec8-many", L, Q, 16, 2, 128, seed=33)
    scales = (0.011, 0.0107)
    kc, vc = gpu_pool8(w, *scales)
    got = attend8(w, kc, vc, *scales, planned=True)
    okc, ovc = oracle_pool8(w, *scales)
    ref = oracle.attend_fp8(w.q, okc, ovc, *scales, w.block_tables, w.seq_lens,
                            w.query_start_loc, w.num_kv_heads, w.scale)
    check_close(got, ref, "1100 requests fp8")
