"""GPU parity of the MLA latent cache path against the CPU oracle: the
scatter bit-exact (every cache element, unwritten slots keep their NaN
sentinel), the decode within the attention tolerance of the fp64 oracle
(max-abs 3e-2, mean-abs 2e-3) on N(0,1) bf16 inputs."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_varlen_amd as pa
import workloads as W
from tests.gpu_util import bf16_tensor, i32, i64, tensor_bits
from tests.test_gpu_parity import check_close
from tests.test_oracle_mla import mla_batch, oracle_cache

pytestmark = pytest.mark.gpu

BS, DL = oracle.MLA_BLOCK, oracle.MLA_DL


def gpu_cache(m, strided=False):
    cache = pa.alloc_mla_cache(m["nb"], fill=float("nan"))
    kv = bf16_tensor(m["kv"])
    if strided:  # rows inside a wider [T][2 * 576] buffer
        wide = torch.zeros((kv.shape[0], 2 * DL), dtype=torch.bfloat16, device="cuda")
        wide[:, DL:] = kv
        kv = wide[:, DL:]
    pa.mla_write_kv(kv, i64(m["slots"]), cache)
    return cache


@pytest.mark.parametrize("strided", [False, True])
def test_mla_write_kv_bit_exact(strided):
    m = mla_batch([1, 63, 64, 65, 300], [1, 1, 1, 1, 1], 16, seed=1)
    m["slots"] = m["slots"].copy()
    m["slots"][[3, 70]] = -1                      # skipped rows
    cache = gpu_cache(m, strided)
    torch.cuda.synchronize()
    assert np.array_equal(tensor_bits(cache).ravel(), oracle_cache(m))


CASES = {
    # name: (seq_lens, query_lens, Hq, scale)
    "decode-h16": ([1, 17, 64, 65, 200, 256, 257, 700, 1500], [1] * 9, 16, None),
    "decode-h32-peaky": ([90, 513, 1030], [1, 1, 1], 32, 0.0721),
    "spec-decode-h16": ([40, 300, 129], [3, 4, 2], 16, None),
    "decode-h128": ([130, 600], [1, 1], 128, None),
    "long-h16": ([5000, 3], [1, 1], 16, None),
    # chunked prefill through the latent path: chunks of 64 and 96 new tokens
    # (causal over their cached prefix) beside decodes
    "prefill-chunks-h16": ([700, 96, 1200, 5], [64, 96, 1, 1], 16, None),
    # every workgroup shape: 3 .. 8 waves of 16 heads each
    "decode-h48": ([33, 300, 2049], [1, 1, 1], 48, None),
    "spec-decode-h64": ([1000, 64, 65], [2, 1, 4], 64, None),
    "decode-h80": ([500, 1], [1, 1], 80, None),
    "decode-h96": ([129, 4096], [1, 1], 96, None),
    "decode-h112": ([2000, 31, 32], [1, 1, 1], 112, None),
    # grouped form (a batch averaging 4+ query tokens per request; 16, 32 and
    # 64 heads): 128 / Hq consecutive tokens of a request per work item.  A
    # fresh prompt (its first tokens see a handful of keys, so most pieces of
    # their group hold none of them), short last groups, single-token groups,
    # a 1-key request, a long context
    "chunk-h16-fresh": ([200], [200], 16, None),
    "chunk-h32-ragged": ([700, 300, 77], [37, 120, 5], 32, None),
    "chunk-h64-mixed": ([2000, 50, 600, 1], [130, 1, 17, 1], 64, None),
    "chunk-h16-long": ([5000, 64], [100, 64], 16, None),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_mla_decode_parity(name):
    L, Q, Hq, scale = CASES[name]
    scale = float(np.float32(scale or 1 / np.sqrt(DL)))
    print("case", name, flush=True)
    m = mla_batch(L, Q, Hq, seed=len(name))
    cache = gpu_cache(m)
    out = pa.mla_decode(bf16_tensor(m["q"]), cache, i32(m["tables"]), i32(m["L"]),
                        i32(m["qsl"]), scale, int(max(L)))
    torch.cuda.synchronize()
    ref = oracle.mla_decode(m["q"], oracle_cache(m), m["tables"], m["L"], m["qsl"], scale)
    check_close(tensor_bits(out), ref, "mla " + name)


@pytest.mark.parametrize("Q", [[1, 2, 1], [40, 77, 9]])
def test_mla_decode_repeat_bit_identical_and_table_permutation(Q):
    # [1, 2, 1]: one token per work item; [40, 77, 9]: the grouped form
    m = mla_batch([300, 77, 1000], Q, 16, seed=9)
    cache = gpu_cache(m)
    args = (bf16_tensor(m["q"]), cache, i32(m["tables"]), i32(m["L"]), i32(m["qsl"]),
            0.05, 1000)
    a = tensor_bits(pa.mla_decode(*args)).copy()
    b = tensor_bits(pa.mla_decode(*args)).copy()
    assert np.array_equal(a, b)
    # the same tokens in other physical blocks: the same bits
    perm = np.random.default_rng(3).permutation(m["nb"])
    m2 = dict(m)
    t2 = m["tables"].copy()
    t2[t2 >= 0] = perm[t2[t2 >= 0]]
    m2["tables"] = t2
    m2["slots"] = perm[m["slots"] // BS] * BS + m["slots"] % BS
    cache2 = gpu_cache(m2)
    c = tensor_bits(pa.mla_decode(bf16_tensor(m["q"]), cache2, i32(t2), i32(m["L"]),
                                  i32(m["qsl"]), 0.05, 1000))
    assert np.array_equal(a, c)


def per_request_oracle(m, scale, requests):
    """The oracle over each listed request on its own: {token: [Hq][512]}."""
    ref = {}
    cache = oracle_cache(m)
    for b in requests:
        t0, t1 = int(m["qsl"][b]), int(m["qsl"][b + 1])
        o = oracle.mla_decode(m["q"][t0:t1], cache, m["tables"][b:b + 1], m["L"][b:b + 1],
                              np.array([0, t1 - t0], np.int32), scale)
        for i in range(t1 - t0):
            ref[t0 + i] = o[i]
    return ref


def test_mla_many_requests():
    """300 requests (several per lane in the range search), decodes and 2-3
    token queries of 1 .. 900 keys."""
    rng = np.random.default_rng(11)
    Q = rng.choice([1, 1, 1, 2, 3], size=300)
    L = np.maximum(rng.integers(1, 900, size=300), Q)
    m = mla_batch(L, Q, 16, seed=12)
    scale = float(np.float32(1 / np.sqrt(DL)))
    cache = gpu_cache(m)
    out = pa.mla_decode(bf16_tensor(m["q"]), cache, i32(m["tables"]), i32(m["L"]),
                        i32(m["qsl"]), scale, int(L.max()))
    torch.cuda.synchronize()
    ref = oracle.mla_decode(m["q"], oracle_cache(m), m["tables"], m["L"], m["qsl"], scale)
    check_close(tensor_bits(out), ref, "mla 300 requests")


@pytest.mark.parametrize("Hq", [16, 32, 64])
def test_mla_grouped_many_requests(Hq):
    """The grouped form (the batch averages 4+ query tokens per request) over
    150 requests (several per lane in the range search): 1 .. 13 query
    tokens each, so full, short and single-token groups, on 1 .. 600 keys."""
    rng = np.random.default_rng(13 + Hq)
    Q = rng.integers(1, 14, size=150)
    Q[:10] = 1
    L = Q + rng.integers(0, 600, size=150)
    assert Q.sum() >= 4 * len(Q)
    m = mla_batch(L, Q, Hq, seed=14)
    scale = float(np.float32(1 / np.sqrt(DL)))
    cache = gpu_cache(m)
    out = pa.mla_decode(bf16_tensor(m["q"]), cache, i32(m["tables"]), i32(m["L"]),
                        i32(m["qsl"]), scale, int(L.max()))
    torch.cuda.synchronize()
    ref = oracle.mla_decode(m["q"], oracle_cache(m), m["tables"], m["L"], m["qsl"], scale)
    check_close(tensor_bits(out), ref, "mla grouped 150 requests")


def test_mla_out_of_bounds_requests_skipped_and_stale_records_ignored():
    """Requests whose metadata is out of bounds (Q > L: request 1 with L = 0;
    L above max_seq_len: request 4) are skipped: their rows keep what was
    there; the others match the oracle.  Run after a batch of long requests
    on the same workspace, each cut into several pieces, whose records of the
    skipped tokens are stale."""
    scale = float(np.float32(1 / np.sqrt(DL)))
    m = mla_batch([900, 2, 1000, 40, 3000], [1, 1, 2, 1, 1], 32, seed=21)
    T = int(m["qsl"][-1])  # tokens: 0 | 1 | 2, 3 | 4 | 5
    L_gpu = m["L"].copy()
    L_gpu[1] = 0
    ws = pa.mla_workspace(T, 32, 3000)
    big = mla_batch([3000] * T, [1] * T, 32, seed=22)
    pa.mla_decode(bf16_tensor(big["q"]), gpu_cache(big), i32(big["tables"]), i32(big["L"]),
                  i32(big["qsl"]), scale, 3000, workspace=ws)
    sentinel = 0x7FA1
    raw = torch.full((T, 32, 512), sentinel, dtype=torch.int16, device="cuda")
    pa.mla_decode(bf16_tensor(m["q"]), gpu_cache(m), i32(m["tables"]), i32(L_gpu),
                  i32(m["qsl"]), scale, 1000, out=raw.view(torch.bfloat16), workspace=ws)
    torch.cuda.synchronize()
    got = tensor_bits(raw.view(torch.bfloat16))
    ref = per_request_oracle(m, scale, [0, 2, 3])
    for t in (0, 2, 3, 4):
        check_close(got[t], ref[t], "mla in-bounds token %d" % t)
    for t in (1, 5):
        assert (got[t] == sentinel).all(), "row of skipped token %d written" % t


def test_mla_grouped_out_of_bounds_requests_and_stale_records():
    """The same in the grouped form (16 heads, groups of 8 tokens): requests
    1 (L = 0 < Q) and 4 (L above max_seq_len) skipped inside a grouped batch,
    run after a grouped batch on the same workspace whose records (with the
    tokens' places in their groups) are stale."""
    scale = float(np.float32(1 / np.sqrt(DL)))
    m = mla_batch([900, 2, 1000, 40, 3000], [8, 1, 12, 6, 5], 16, seed=23)
    T = int(m["qsl"][-1])  # 32 tokens over 5 requests: grouped
    L_gpu = m["L"].copy()
    L_gpu[1] = 0
    ws = pa.mla_workspace(T, 16, 3000)
    big = mla_batch([3000, 2500], [16, 16], 16, seed=24)
    pa.mla_decode(bf16_tensor(big["q"]), gpu_cache(big), i32(big["tables"]), i32(big["L"]),
                  i32(big["qsl"]), scale, 3000, workspace=ws)
    sentinel = 0x7FA1
    raw = torch.full((T, 16, 512), sentinel, dtype=torch.int16, device="cuda")
    pa.mla_decode(bf16_tensor(m["q"]), gpu_cache(m), i32(m["tables"]), i32(L_gpu),
                  i32(m["qsl"]), scale, 1000, out=raw.view(torch.bfloat16), workspace=ws)
    torch.cuda.synchronize()
    got = tensor_bits(raw.view(torch.bfloat16))
    ref = per_request_oracle(m, scale, [0, 2, 3])
    q = m["qsl"]
    for b in (0, 2, 3):
        for t in range(q[b], q[b + 1]):
            check_close(got[t], ref[t], "mla grouped in-bounds token %d" % t)
    for b in (1, 4):
        for t in range(q[b], q[b + 1]):
            assert (got[t] == sentinel).all(), "row of skipped token %d written" % t


@pytest.mark.parametrize("Hq", [16, 128])
def test_mla_headline_workload_full_parity(Hq):
    """The timed MLA workload: 64 requests of U[128, 4096] keys, one query
    token each, every output row against the oracle."""
    rng = np.random.default_rng(2024)
    L = rng.integers(128, 4096, size=64, endpoint=True).astype(np.int32)
    m = mla_batch(L, np.ones(64, np.int32), Hq, seed=31)
    scale = float(np.float32(1 / np.sqrt(192.0)))
    cache = gpu_cache(m)
    out = pa.mla_decode(bf16_tensor(m["q"]), cache, i32(m["tables"]), i32(m["L"]),
                        i32(m["qsl"]), scale, int(L.max()))
    torch.cuda.synchronize()
    ref = oracle.mla_decode(m["q"], oracle_cache(m), m["tables"], m["L"], m["qsl"], scale)
    check_close(tensor_bits(out), ref, "mla 64 x U[128, 4096] h%d" % Hq)
