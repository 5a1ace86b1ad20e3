"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every test here runs on the CPU.  The oracle (oracle/oracle.c) is checked
against: the pages' worked numbers (tests/golden/), the documented pool layout
worked out by hand, closed forms, a numpy brute force, torch's
scaled_dot_product_attention in float64 (a library routine), and exact
invariants (paged == dense under any block permutation, shared == unshared,
chunk row == truncated decode).
"""
import os
from collections import Counter

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.brute import brute_attend


def _read_golden(golden_dir, name):
    rows = []
    with open(os.path.join(golden_dir, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line)
    return rows


def oracle_pool(w, fill=True):
    kc = np.full(w.pool_elems(), W.BF16_NAN, np.uint16)
    vc = np.full(w.pool_elems(), W.BF16_NAN, np.uint16)
    if fill:
        oracle.write_kv(kc, vc, w.k_dense[w.fill_rows], w.v_dense[w.fill_rows],
                        w.fill_slots)
    oracle.write_kv(kc, vc, w.k_new, w.v_new, w.new_slots)
    return kc, vc


def run_oracle(w, kc=None, vc=None, tables=None):
    if kc is None:
        kc, vc = oracle_pool(w)
    bt = w.block_tables if tables is None else tables
    return oracle.attend(w.q, kc, vc, bt, w.seq_lens, w.query_start_loc,
                         w.num_kv_heads, w.scale)


def small_mixed(seed=0, Hq=8, Hkv=2, D=64):
    # decode rows, a chunk on a cached prefix, a pure prefill (Q == L), a
    # sequence with no query this step, ragged block tails.
    L = [1, 17, 40, 33, 64, 5, 16]
    Q = [1, 1, 7, 33, 3, 0, 16]
    return W.make_workload("small-mixed", L, Q, Hq, Hkv, D, seed=seed)


def f64(bits):
    return W.bf16_bits_to_f32(bits).astype(np.float64)


# ---- worked numbers the pages print ---------------------------------------------

def test_golden_block_accounting(golden_dir):
    for row in _read_golden(golden_dir, "block_accounting.txt"):
        n, bs, blocks, full, trailing = map(int, row.split())
        assert W.blocks_needed(n, bs) == blocks
        assert n // bs == full and n % bs == trailing
        # waste is at most one partial block
        assert W.blocks_needed(n, bs) * bs - n <= bs - 1


def test_golden_query_start_loc(golden_dir):
    for row in _read_golden(golden_dir, "query_start_loc.txt"):
        counts, qsl, last = [s.strip() for s in row.split(";")]
        counts = [int(x) for x in counts.split(",")]
        got = W.query_start_loc(counts)
        assert got.tolist() == [int(x) for x in qsl.split(",")]
        if last != "-":
            assert W.logits_rows(got).tolist() == [int(x) for x in last.split(",")]


def test_golden_slot_mapping(golden_dir):
    for row in _read_golden(golden_dir, "slot_mapping.txt"):
        bs, table, pos, slots = [s.strip() for s in row.split(";")]
        table = [int(x) for x in table.split(",")]
        pos = np.array([int(x) for x in pos.split(",")])
        got = W.slots_for(table, pos, int(bs))
        assert got.tolist() == [int(x) for x in slots.split(",")]


def test_golden_pool_layout(golden_dir):
    for row in _read_golden(golden_dir, "pool_layout.txt"):
        Hkv, D, n, g, t, d, ko, vo = map(int, row.split())
        assert oracle.k_index(n, g, t, d, Hkv, D) == ko
        assert oracle.v_index(n, g, t, d, Hkv, D) == vo


@pytest.mark.parametrize("D", [64, 128])
def test_pool_layout_is_a_tile_permutation(D):
    Hkv = 3
    for n, g in [(0, 0), (2, 1), (5, 2)]:
        base = (n * Hkv + g) * 16 * D
        ks = sorted(oracle.k_index(n, g, t, d, Hkv, D) - base
                    for t in range(16) for d in range(D))
        vs = sorted(oracle.v_index(n, g, t, d, Hkv, D) - base
                    for t in range(16) for d in range(D))
        assert ks == list(range(16 * D))
        assert vs == list(range(16 * D))


def test_config_block_accounting():
    # config 1: ceil({56,17,100,33}/16) = {4,2,7,3}: 16 of 64 blocks
    L, _ = W.config_lengths(1)
    assert [W.blocks_needed(int(x)) for x in L] == [4, 2, 7, 3]
    assert sum(W.blocks_needed(int(x)) for x in L) == 16
    assert [W.blocks_needed(int(x)) * 16 - int(x) for x in L] == [8, 15, 12, 15]
    for k in range(1, 6):
        L, Q = W.config_lengths(k)
        waste = np.array([W.blocks_needed(int(x)) * 16 - int(x) for x in L])
        assert waste.min() >= 0 and waste.max() <= 15
        assert np.all(Q <= L)
    L, Q = W.config_lengths(3)
    assert int(Q.sum()) == 2048 and int(Q[-1]) == 1920 and int(L[-1]) == 3456


def test_block_pool_refcounts_and_exhaustion():
    rng = np.random.default_rng(0)
    pool = W.BlockPool(4, rng)
    a = pool.allocate(2)
    b = pool.share(a[:1]) + pool.allocate(2)
    with pytest.raises(MemoryError):
        pool.allocate(1)
    tables = [a, b]
    assert pool.refs == Counter(x for t in tables for x in t)
    pool.release(a)
    assert pool.used() == 3


def test_shared_workload_refcounts():
    w = W.make_workload("shared", [48, 50, 70], [1, 1, 1], 4, 2, 64, seed=3,
                        shared_prefix=32)
    ids = Counter(int(x) for x in w.block_tables.ravel() if x >= 0)
    assert w.refs == dict(ids)
    first = w.block_tables[:, :2]
    assert np.all(first == first[0])
    assert all(w.refs[int(x)] == 3 for x in first[0])


# ---- scatter and gather -------------------------------------------------------------

def test_scatter_gather_round_trip():
    w = small_mixed(seed=1)
    kc, vc = oracle_pool(w)
    kd, vd = oracle.gather_kv(kc, vc, w.block_tables, w.seq_lens,
                              w.num_kv_heads, w.head_dim)
    assert np.array_equal(kd, w.k_dense) and np.array_equal(vd, w.v_dense)
    # every element not written still holds the NaN sentinel
    written = int(w.seq_lens.sum()) * w.num_kv_heads * w.head_dim
    assert int((kc != W.BF16_NAN).sum()) == written
    assert int((vc != W.BF16_NAN).sum()) == written


def test_scatter_skips_negative_slots():
    w = small_mixed(seed=2)
    kc = np.full(w.pool_elems(), W.BF16_NAN, np.uint16)
    vc = kc.copy()
    slots = w.new_slots.copy()
    slots[::2] = -1
    oracle.write_kv(kc, vc, w.k_new, w.v_new, slots)
    n_written = int((slots >= 0).sum())
    assert int((kc != W.BF16_NAN).sum()) == n_written * w.num_kv_heads * w.head_dim
    # written tokens land where the documented layout says
    Hkv, D = w.num_kv_heads, w.head_dim
    for t in np.nonzero(slots >= 0)[0][:5]:
        s = int(slots[t])
        for g in range(Hkv):
            for d in (0, 7, D // 2, D - 1):
                assert kc[oracle.k_index(s // 16, g, s % 16, d, Hkv, D)] == w.k_new[t, g, d]
                assert vc[oracle.v_index(s // 16, g, s % 16, d, Hkv, D)] == w.v_new[t, g, d]


# ---- attention: brute force and a library routine --------------------------------------

@pytest.mark.parametrize("Hq,Hkv,D", [(8, 2, 64), (8, 8, 64), (8, 1, 128), (12, 3, 64)])
def test_oracle_matches_brute_force(Hq, Hkv, D):
    w = small_mixed(seed=4, Hq=Hq, Hkv=Hkv, D=D)
    got = run_oracle(w)
    ref = brute_attend(w.q, w.k_dense, w.v_dense, w.seq_lens, w.query_start_loc,
                       w.scale)
    assert np.max(np.abs(got - ref)) <= 1e-12


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (6, 6)])
def test_oracle_matches_torch_sdpa_float64(Hq, Hkv):
    w = small_mixed(seed=5, Hq=Hq, Hkv=Hkv, D=64)
    got = run_oracle(w)
    for b in range(w.num_seqs):
        t0, t1 = int(w.query_start_loc[b]), int(w.query_start_loc[b + 1])
        if t1 == t0:
            continue
        L = int(w.seq_lens[b])
        s0 = int(w.kv_start[b])
        q = torch.from_numpy(f64(w.q[t0:t1])).permute(1, 0, 2)[None]
        k = torch.from_numpy(f64(w.k_dense[s0:s0 + L])).permute(1, 0, 2)[None]
        v = torch.from_numpy(f64(w.v_dense[s0:s0 + L])).permute(1, 0, 2)[None]
        Q = t1 - t0
        if Q == L:
            # pure prefill: library causal mask, no mask built here
            ref = torch.nn.functional.scaled_dot_product_attention(
                q, k, v, is_causal=True, scale=float(w.scale), enable_gqa=True)
        else:
            allowed = torch.ones(Q, L, dtype=torch.bool).tril(diagonal=L - Q)
            ref = torch.nn.functional.scaled_dot_product_attention(
                q, k, v, attn_mask=allowed, scale=float(w.scale), enable_gqa=True)
        ref = ref[0].permute(1, 0, 2).numpy()
        assert np.max(np.abs(got[t0:t1] - ref)) <= 1e-12, b


# ---- closed forms ------------------------------------------------------------------------

def test_single_key_returns_that_value_exactly():
    w = W.make_workload("L1", [1, 1, 1], [1, 1, 1], 4, 2, 64, seed=6)
    got = run_oracle(w)
    for b in range(3):
        for h in range(4):
            assert np.array_equal(got[b, h], f64(w.v_dense[b, h // 2]))


def test_zero_query_gives_causal_prefix_means():
    w = W.make_workload("zeroq", [40, 9], [12, 9], 4, 2, 64, seed=7)
    w.q[:] = 0
    got = run_oracle(w)
    v = f64(w.v_dense)
    for b in range(2):
        L, Q = int(w.seq_lens[b]), int(w.query_lens[b])
        s0, t0 = int(w.kv_start[b]), int(w.query_start_loc[b])
        for i in range(Q):
            p = L - Q + i
            for h in range(4):
                ref = v[s0:s0 + p + 1, h // 2].mean(axis=0)
                assert np.max(np.abs(got[t0 + i, h] - ref)) <= 1e-12


def test_equal_keys_give_mean_value():
    w = W.make_workload("eqk", [37], [1], 2, 1, 64, seed=8)
    w.k_dense[:] = w.k_dense[0]
    got = run_oracle(w)
    ref = f64(w.v_dense[:, 0]).mean(axis=0)
    assert np.max(np.abs(got[0, 0] - ref)) <= 1e-12


def test_one_hot_keys_select_one_value_exactly():
    # K row j = 64 * e_j, q = 64 * e_target, scale 1: the target's score
    # exceeds every other by 4096, so the other weights are exactly 0 in fp64.
    L, D = 50, 64
    w = W.make_workload("onehot", [L], [1], 1, 1, D, seed=9)
    w.scale = 1.0
    one64 = int(W.f32_to_bf16_bits(np.array([64.0], np.float32))[0])
    w.k_dense[:] = 0
    for j in range(L):
        w.k_dense[j, 0, j] = one64
    target = 29
    w.q[:] = 0
    w.q[0, 0, target] = one64
    got = run_oracle(w)
    assert np.array_equal(got[0, 0], f64(w.v_dense[target, 0]))


# ---- invariants -----------------------------------------------------------------------------

def permute_blocks(w, seed):
    """Same logical sequences on a random relabelling of physical blocks."""
    pi = np.random.default_rng(seed).permutation(w.num_blocks).astype(np.int64)
    bt = w.block_tables.astype(np.int64)
    bt2 = np.where(bt >= 0, pi[np.maximum(bt, 0)], -1).astype(np.int32)
    relabel = (lambda s: pi[s // 16] * 16 + s % 16)
    return bt2, relabel(w.fill_slots), relabel(w.new_slots)


def test_paged_equals_dense_under_block_permutation():
    w = small_mixed(seed=10)
    base = run_oracle(w)
    dense = oracle.attend_dense(w.q, w.k_dense, w.v_dense, w.seq_lens,
                                w.query_start_loc, w.scale)
    assert np.array_equal(base, dense)
    bt2, fs2, ns2 = permute_blocks(w, 11)
    kc = np.full(w.pool_elems(), W.BF16_NAN, np.uint16)
    vc = kc.copy()
    oracle.write_kv(kc, vc, w.k_dense[w.fill_rows], w.v_dense[w.fill_rows], fs2)
    oracle.write_kv(kc, vc, w.k_new, w.v_new, ns2)
    perm = run_oracle(w, kc, vc, bt2)
    assert np.array_equal(perm, base)


def test_shared_prefix_equals_unshared_copy():
    L, Q = [70, 33, 100, 48], [1, 1, 1, 1]
    ws = W.make_workload("s", L, Q, 8, 2, 64, seed=12, shared_prefix=32, shared=True)
    wu = W.make_workload("u", L, Q, 8, 2, 64, seed=12, shared_prefix=32, shared=False)
    assert np.array_equal(ws.k_dense, wu.k_dense)
    assert ws.num_blocks < wu.num_blocks
    assert np.array_equal(run_oracle(ws), run_oracle(wu))


def test_chunk_row_equals_truncated_decode():
    w = W.make_workload("chunk", [45], [20], 8, 2, 64, seed=13)
    got = run_oracle(w)
    L, Q = 45, 20
    for i in (0, 7, 19):
        p = L - Q + i
        one = oracle.attend_dense(w.q[i:i + 1], w.k_dense[:p + 1],
                                  w.v_dense[:p + 1], np.array([p + 1], np.int32),
                                  np.array([0, 1], np.int32), w.scale)
        assert np.array_equal(got[i], one[0])


def test_attend_rows_match_full():
    w = small_mixed(seed=14)
    full = run_oracle(w)
    kc, vc = oracle_pool(w)
    rows = np.array([[0, 0], [3, 5], [w.num_q_tokens - 1, 7], [10, 2]], np.int64)
    got = oracle.attend_rows(w.q, kc, vc, w.block_tables, w.seq_lens,
                             w.query_start_loc, w.num_kv_heads, w.scale, rows)
    for r, (t, h) in enumerate(rows):
        assert np.array_equal(got[r], full[t, h])
