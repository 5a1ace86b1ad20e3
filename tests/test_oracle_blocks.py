"""Pins of the oracle's whole-block operations against independent code.

Copy-on-write ("vLLM: An Exhaustive Technical Study", section 2.1: a block
held by several requests is duplicated when one of them writes into it) is
checked against numpy slice assignment; the expansion of tables of larger
blocks against tables worked out by hand and, end to end, against the slot
definition (slot = block * block_size + offset): tokens scattered with
block_size-token slots and gathered through the expanded 16-token table come
back as the dense rows exactly.
"""
import numpy as np
import pytest

import oracle
import workloads as W


def test_copy_blocks_matches_numpy_in_order():
    rng = np.random.default_rng(3)
    nb, block_elems = 12, 2 * 16 * 64  # 2 kv heads, D = 64, bf16 bits
    k = rng.integers(0, 1 << 16, nb * block_elems, dtype=np.uint16)
    v = rng.integers(0, 1 << 16, nb * block_elems, dtype=np.uint16)
    mapping = [(3, 7), (7, 1), (0, 0), (-1, 4), (5, 12), (11, 2), (2, 9)]
    kr, vr = k.reshape(nb, block_elems).copy(), v.reshape(nb, block_elems).copy()
    for s, d in mapping:  # numpy, in order, skipping invalid pairs
        if 0 <= s < nb and 0 <= d < nb and s != d:
            kr[d] = kr[s]
            vr[d] = vr[s]
    oracle.copy_blocks(k, v, block_elems * 2, mapping)
    assert np.array_equal(k.reshape(nb, block_elems), kr)
    assert np.array_equal(v.reshape(nb, block_elems), vr)
    # the chained pair (3 -> 7 then 7 -> 1) saw block 3's bytes in block 1
    assert np.array_equal(kr[1], kr[3])


def test_expand_block_tables_by_hand():
    assert oracle.expand_block_tables(np.array([[5, 2, -1]]), 32).tolist() == \
        [[10, 11, 4, 5, -1, -1]]
    assert oracle.expand_block_tables(np.array([[3, 0], [1, -1]]), 64).tolist() == \
        [[12, 13, 14, 15, 0, 1, 2, 3], [4, 5, 6, 7, -1, -1, -1, -1]]
    t = np.array([[4, 9, 0]])
    assert np.array_equal(oracle.expand_block_tables(t, 16), t)


@pytest.mark.parametrize("bs", [32, 64, 128])
def test_larger_blocks_scatter_and_gather_round_trip(bs):
    rng = np.random.default_rng(bs)
    L = np.array([1, 31, 32, 33, 200, 129], np.int32)
    Hkv, D = 2, 64
    nblk = [-(-int(x) // bs) for x in L]
    nb = sum(nblk) + 3
    perm = rng.permutation(nb)
    width = max(nblk)
    tables = np.full((len(L), width), -1, np.int32)
    pos = 0
    for b, n in enumerate(nblk):
        tables[b, :n] = perm[pos:pos + n]
        pos += n
    kv_start = np.concatenate([[0], np.cumsum(L)])
    k_dense = W.normal_bf16((bs, 0), (int(L.sum()), Hkv, D))
    v_dense = W.normal_bf16((bs, 1), (int(L.sum()), Hkv, D))
    slots = np.concatenate([W.slots_for(tables[b], np.arange(L[b]), bs)
                            for b in range(len(L))])
    R = bs // 16
    kc = np.full(nb * R * Hkv * 16 * D, W.BF16_NAN, np.uint16)
    vc = kc.copy()
    oracle.write_kv(kc, vc, k_dense, v_dense, slots)  # 16-token view of the pool
    t16 = oracle.expand_block_tables(tables, bs)
    ko, vo = oracle.gather_kv(kc, vc, t16, L, Hkv, D)
    assert np.array_equal(ko, k_dense) and np.array_equal(vo, v_dense)
    assert kv_start[-1] == ko.shape[0]


def test_copy_on_write_then_write():
    # two requests share their first two blocks; request 1 copies the
    # second (partly filled) block before writing its next token into it:
    # request 0 still reads its own token there, request 1 the new one
    Hkv, D = 2, 64
    nb = 6
    kc = np.full(nb * Hkv * 16 * D, W.BF16_NAN, np.uint16)
    vc = kc.copy()
    prompt = W.normal_bf16((7, 0), (20, Hkv, D))
    vprompt = W.normal_bf16((7, 1), (20, Hkv, D))
    shared = [4, 1]
    oracle.write_kv(kc, vc, prompt, vprompt, W.slots_for(shared, np.arange(20)))
    t0 = W.normal_bf16((7, 2), (1, Hkv, D))
    t1 = W.normal_bf16((7, 3), (1, Hkv, D))
    oracle.write_kv(kc, vc, t0, t0, W.slots_for(shared, np.array([20])))
    own = [4, 5]  # request 1: block 1 copied to block 5 before its write
    oracle.copy_blocks(kc, vc, Hkv * 16 * D * 2, [(1, 5)])
    oracle.write_kv(kc, vc, t1, t1, W.slots_for(own, np.array([20])))
    tables = np.array([shared, own], np.int32)
    ko, _ = oracle.gather_kv(kc, vc, tables, np.array([21, 21], np.int32), Hkv, D)
    assert np.array_equal(ko[:20], prompt) and np.array_equal(ko[21:41], prompt)
    assert np.array_equal(ko[20], t0[0]) and np.array_equal(ko[41], t1[0])
