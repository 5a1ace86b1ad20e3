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


# ---- 8-token blocks ---------------------------------------------------------------------

def _golden_rows(golden_dir, name):
    import os
    with open(os.path.join(golden_dir, name)) as f:
        return [ln for ln in f if ln.strip() and not ln.startswith("#")]


def test_golden_pool_layout_bs8(golden_dir):
    # offsets of the 8-token tile layout worked out by hand
    for row in _golden_rows(golden_dir, "pool_layout_bs8.txt"):
        Hkv, D, n, g, t, d, ko, vo = map(int, row.split())
        assert oracle.k_index(n, g, t, d, Hkv, D, block_size=8) == ko
        assert oracle.v_index(n, g, t, d, Hkv, D, block_size=8) == vo


@pytest.mark.parametrize("D", [64, 128])
def test_pool_layout_bs8_is_a_tile_permutation(D):
    Hkv = 3
    for n, g in [(0, 0), (2, 1), (5, 2)]:
        base = (n * Hkv + g) * 8 * D
        ks = sorted(oracle.k_index(n, g, t, d, Hkv, D, block_size=8) - base
                    for t in range(8) for d in range(D))
        vs = sorted(oracle.v_index(n, g, t, d, Hkv, D, block_size=8) - base
                    for t in range(8) for d in range(D))
        assert ks == list(range(8 * D))
        assert vs == list(range(8 * D))


def _bs8_workload(seed, **kw):
    return W.make_workload("bs8", [1, 8, 9, 16, 17, 40, 100, 333], [1, 1, 9, 3, 1, 40, 7, 20],
                           8, 2, 64, seed=seed, block_size=8, **kw)


def test_bs8_accounting():
    # ceil(L / 8) blocks per request, at most 7 slots of the last one unused
    w = _bs8_workload(1)
    nblk = (w.seq_lens + 7) // 8
    assert np.array_equal((w.block_tables >= 0).sum(axis=1), nblk)
    assert int(nblk.sum()) == 1 + 1 + 2 + 2 + 3 + 5 + 13 + 42
    assert np.all(nblk * 8 - w.seq_lens <= 7)
    assert w.pool_elems() == w.num_blocks * 2 * 8 * 64


def test_bs8_scatter_gather_round_trip():
    w = _bs8_workload(2)
    kc = np.full(w.pool_elems(), W.BF16_NAN, np.uint16)
    vc = kc.copy()
    oracle.write_kv(kc, vc, w.k_dense[w.fill_rows], w.v_dense[w.fill_rows], w.fill_slots,
                    block_size=8)
    oracle.write_kv(kc, vc, w.k_new, w.v_new, w.new_slots, block_size=8)
    kd, vd = oracle.gather_kv(kc, vc, w.block_tables, w.seq_lens, w.num_kv_heads,
                              w.head_dim, block_size=8)
    assert np.array_equal(kd, w.k_dense) and np.array_equal(vd, w.v_dense)
    written = int(w.seq_lens.sum()) * w.num_kv_heads * w.head_dim
    assert int((kc != W.BF16_NAN).sum()) == written


def test_bs8_attention_equals_dense_and_16_token_blocks():
    # the same requests and values in 8-token and in 16-token blocks (and
    # contiguous): one logical order, so the fp64 results are identical
    w8 = _bs8_workload(3)
    w16 = W.make_workload("bs16", w8.seq_lens, w8.query_lens, 8, 2, 64, seed=3)
    assert np.array_equal(w8.k_dense, w16.k_dense) and np.array_equal(w8.q, w16.q)
    outs = []
    for w in (w8, w16):
        kc = np.full(w.pool_elems(), W.BF16_NAN, np.uint16)
        vc = kc.copy()
        oracle.write_kv(kc, vc, w.k_dense[w.fill_rows], w.v_dense[w.fill_rows],
                        w.fill_slots, block_size=w.block_size)
        oracle.write_kv(kc, vc, w.k_new, w.v_new, w.new_slots, block_size=w.block_size)
        outs.append(oracle.attend(w.q, kc, vc, w.block_tables, w.seq_lens,
                                  w.query_start_loc, w.num_kv_heads, w.scale,
                                  block_size=w.block_size))
    dense = oracle.attend_dense(w8.q, w8.k_dense, w8.v_dense, w8.seq_lens,
                                w8.query_start_loc, w8.scale)
    assert np.array_equal(outs[0], outs[1])
    assert np.array_equal(outs[0], dense)
