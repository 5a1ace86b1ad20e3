"""GPU parity of the whole-block operations: copy-on-write block copies and
pools of larger blocks (block tables of 32/64/128-token ids expanded to the
16-token ids attention reads).  Copies and expansions bit-exact against the
oracle; attention over larger-block pools within the attention tolerance of
the fp64 oracle's dense attention over the same logical K/V."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_varlen_amd as pa
import workloads as W
from tests.gpu_util import bf16_tensor, i32, i64, tensor_bits
from tests.test_gpu_parity import check_close

pytestmark = pytest.mark.gpu


def u8_or_bits(t):
    if t.dtype == torch.uint8:
        return t.contiguous().cpu().numpy().ravel()
    return tensor_bits(t).ravel()


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("D", [64, 128])
def test_copy_blocks_bit_exact(fp8, D):
    rng = np.random.default_rng(D + fp8)
    nb, Hkv = 40, 4
    if fp8:
        kh = rng.integers(0, 256, nb * Hkv * 16 * D, dtype=np.uint8)
        vh = rng.integers(0, 256, nb * Hkv * 16 * D, dtype=np.uint8)
        k = torch.from_numpy(kh.copy()).cuda().view(nb, Hkv, 16 * D)
        v = torch.from_numpy(vh.copy()).cuda().view(nb, Hkv, 16 * D)
    else:
        kh = rng.integers(0, 1 << 16, nb * Hkv * 16 * D, dtype=np.uint16)
        vh = rng.integers(0, 1 << 16, nb * Hkv * 16 * D, dtype=np.uint16)
        k = bf16_tensor(kh).view(nb, Hkv, 16 * D)
        v = bf16_tensor(vh).view(nb, Hkv, 16 * D)
    # distinct destinations, none of them a source; invalid pairs skipped
    mapping = np.array([(3, 7), (0, 39), (12, 13), (38, 1), (5, 5), (-1, 2),
                        (6, 40), (20, 21), (20, 22)], np.int64)
    pa.copy_blocks(k, v, i64(mapping), Hkv, D)
    torch.cuda.synchronize()
    oracle.copy_blocks(kh, vh, Hkv * 16 * D * (1 if fp8 else 2), mapping)
    assert np.array_equal(u8_or_bits(k), kh.ravel())
    assert np.array_equal(u8_or_bits(v), vh.ravel())


@pytest.mark.parametrize("bs", [32, 64, 128])
def test_expand_block_tables_bit_exact(bs):
    rng = np.random.default_rng(bs)
    t = rng.integers(0, 5000, (37, 19)).astype(np.int32)
    t[rng.random(t.shape) < 0.2] = -1
    got = pa.expand_block_tables(i32(t), bs).cpu().numpy()
    assert np.array_equal(got, oracle.expand_block_tables(t, bs))


def bs_workload(L, Q, Hq, Hkv, D, bs, seed):
    """One step over a pool of bs-token blocks: tables of bs-token ids, every
    token's slot n * bs + offset, dense K/V and q."""
    rng = np.random.default_rng(seed)
    L = np.asarray(L, np.int32)
    Q = np.asarray(Q, np.int32)
    nblk = [-(-int(x) // bs) for x in L]
    nb = int(np.ceil(sum(nblk) * 1.2)) + 1
    perm = rng.permutation(nb)
    tables = np.full((len(L), max(nblk)), -1, np.int32)
    pos = 0
    for b, n in enumerate(nblk):
        tables[b, :n] = perm[pos:pos + n]
        pos += n
    k = W.normal_bf16((seed, 0), (int(L.sum()), Hkv, D))
    v = W.normal_bf16((seed, 1), (int(L.sum()), Hkv, D))
    q = W.normal_bf16((seed, 2), (int(Q.sum()), Hq, D))
    slots = np.concatenate([W.slots_for(tables[b], np.arange(L[b]), bs)
                            for b in range(len(L))])
    return dict(L=L, Q=Q, qsl=W.query_start_loc(Q), tables=tables, nb=nb, k=k, v=v,
                q=q, slots=slots, scale=float(np.float32(1 / np.sqrt(D))))


@pytest.mark.parametrize("bs", [32, 64])
@pytest.mark.parametrize("Hq,Hkv,D", [(16, 4, 128), (8, 8, 64)])
def test_attend_larger_blocks(bs, Hq, Hkv, D):
    w = bs_workload([1, 40, 700, 95, 1300, 64], [1, 1, 300, 20, 1, 64], Hq, Hkv, D,
                    bs, seed=bs + D)
    R = bs // 16
    kc, vc = pa.alloc_pool(w["nb"] * R, Hkv, D, fill=float("nan"))
    pa.write_kv(bf16_tensor(w["k"]), bf16_tensor(w["v"]), i64(w["slots"]), kc, vc)
    t16 = pa.expand_block_tables(i32(w["tables"]), bs)
    out = pa.attend(bf16_tensor(w["q"]), kc, vc, t16, i32(w["L"]), i32(w["qsl"]),
                    w["scale"], int(w["Q"].max()), int(w["L"].max()), num_kv_heads=Hkv)
    torch.cuda.synchronize()
    ref = oracle.attend_dense(w["q"], w["k"], w["v"], w["L"], w["qsl"], w["scale"])
    check_close(tensor_bits(out), ref, "block size %d" % bs)


def test_copy_on_write_then_write_and_attend():
    # two requests share a prompt of 40 tokens (blocks 3 full + 1 partial);
    # request 1 copies the partial block before writing its next token
    Hq, Hkv, D = 16, 4, 128
    nb = 10
    prompt_k = W.normal_bf16((11, 0), (40, Hkv, D))
    prompt_v = W.normal_bf16((11, 1), (40, Hkv, D))
    new_k = W.normal_bf16((11, 2), (2, Hkv, D))
    new_v = W.normal_bf16((11, 3), (2, Hkv, D))
    q = W.normal_bf16((11, 4), (2, Hq, D))
    shared, own = [7, 2, 9], [7, 2, 4]
    kc, vc = pa.alloc_pool(nb, Hkv, D, fill=float("nan"))
    okc = np.full(nb * Hkv * 16 * D, W.BF16_NAN, np.uint16)
    ovc = okc.copy()
    s_prompt = W.slots_for(shared, np.arange(40))
    pa.write_kv(bf16_tensor(prompt_k), bf16_tensor(prompt_v), i64(s_prompt), kc, vc)
    oracle.write_kv(okc, ovc, prompt_k, prompt_v, s_prompt)
    # copy-on-write of block 9 into block 4, then both requests' new tokens
    pa.copy_blocks(kc, vc, i64(np.array([[9, 4]], np.int64)), Hkv, D)
    oracle.copy_blocks(okc, ovc, Hkv * 16 * D * 2, [(9, 4)])
    s_new = np.array([W.slots_for(shared, [40])[0], W.slots_for(own, [40])[0]])
    pa.write_kv(bf16_tensor(new_k), bf16_tensor(new_v), i64(s_new), kc, vc)
    oracle.write_kv(okc, ovc, new_k, new_v, s_new)
    tables = np.array([shared, own], np.int32)
    L = np.array([41, 41], np.int32)
    qsl = np.array([0, 1, 2], np.int32)
    out = pa.attend(bf16_tensor(q), kc, vc, i32(tables), i32(L), i32(qsl),
                    float(np.float32(1 / np.sqrt(D))), 1, 41, num_kv_heads=Hkv)
    torch.cuda.synchronize()
    assert np.array_equal(tensor_bits(kc).ravel(), okc)
    ref = oracle.attend(q, okc, ovc, tables, L, qsl, Hkv, float(np.float32(1 / np.sqrt(D))))
    check_close(tensor_bits(out), ref, "copy-on-write")
    # each request sees its own token 40: the dense form agrees
    kd = np.concatenate([prompt_k, new_k[:1], prompt_k, new_k[1:]])
    vd = np.concatenate([prompt_v, new_v[:1], prompt_v, new_v[1:]])
    dense = oracle.attend_dense(q, kd, vd, L, qsl, float(np.float32(1 / np.sqrt(D))))
    assert np.max(np.abs(dense - ref)) <= 1e-12
