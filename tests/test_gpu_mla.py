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


def test_mla_decode_repeat_bit_identical_and_table_permutation():
    m = mla_batch([300, 77, 1000], [1, 2, 1], 16, seed=9)
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
