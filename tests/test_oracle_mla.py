"""Pins of the oracle's MLA latent cache and decode against independent code.

The pages: one latent vector per token shared by every query head (512
latent + 64 rotary dims, blocks of 64 tokens), attended MQA-style ("vLLM: An
Exhaustive Technical Study", section 2.4).  Checked against: the layout as a
permutation and by hand, the scatter element by element, a numpy brute force
(matmul, -inf causal mask, exp, row normalisation) on small batches, and
closed forms (one key: the latent itself; zero queries: running means).
"""
import numpy as np
import pytest

import oracle
import workloads as W

BS, DL, DV = oracle.MLA_BLOCK, oracle.MLA_DL, oracle.MLA_DV


def test_layout_is_a_permutation_and_by_hand():
    offs = sorted(oracle.mla_index(0, t, d) for t in range(BS) for d in range(DL))
    assert offs == list(range(BS * DL))
    assert oracle.mla_index(0, 1, 0) == 32            # next token: next 32-dim row
    assert oracle.mla_index(0, 0, 32) == 16 * 32      # next 32-dim chunk
    assert oracle.mla_index(0, 16, 0) == 18 * 16 * 32  # next 16-token tile
    assert oracle.mla_index(0, 17, 545) == ((1 * 18 + 17) * 16 + 1) * 32 + 1
    assert oracle.mla_index(2, 0, 0) == 2 * BS * DL


def mla_batch(L, Q, Hq, seed, nb=None):
    """Requests of lengths L (Q query tokens each, the last ones) over a
    cache of 64-token blocks in a seeded random order; every token written."""
    rng = np.random.default_rng(seed)
    L = np.asarray(L, np.int32)
    Q = np.asarray(Q, np.int32)
    nblk = [-(-int(x) // BS) for x in L]
    nb = nb or sum(nblk) + 2
    perm = rng.permutation(nb)
    tables = np.full((len(L), max(nblk)), -1, np.int32)
    pos = 0
    for b, n in enumerate(nblk):
        tables[b, :n] = perm[pos:pos + n]
        pos += n
    kv = W.normal_bf16((seed, 0), (int(L.sum()), DL))
    q = W.normal_bf16((seed, 1), (int(Q.sum()), Hq, DL))
    slots = np.concatenate([W.slots_for(tables[b], np.arange(L[b]), BS)
                            for b in range(len(L))])
    return dict(L=L, Q=Q, qsl=W.query_start_loc(Q), tables=tables, nb=nb, kv=kv, q=q,
                slots=slots, kv_start=np.concatenate([[0], np.cumsum(L)]))


def oracle_cache(m, fill=W.BF16_NAN):
    cache = np.full(m["nb"] * BS * DL, fill, np.uint16)
    oracle.mla_write_kv(cache, m["kv"], m["slots"])
    return cache


def test_scatter_element_by_element():
    m = mla_batch([70, 5, 130], [1, 1, 1], 16, seed=2)
    cache = oracle_cache(m)
    written = np.zeros(cache.shape, bool)
    for i, s in enumerate(m["slots"]):
        n, t = divmod(int(s), BS)
        for d in range(0, DL, 7):
            assert cache[oracle.mla_index(n, t, d)] == m["kv"][i, d]
        for d in range(DL):
            written[oracle.mla_index(n, t, d)] = True
    assert np.all(cache[~written] == W.BF16_NAN)


def brute(m, Hq, scale):
    """numpy: per request, scores over the dense latent rows with a -inf
    causal mask, exp, normalise, weights times the first 512 dims."""
    kvf = W.bf16_bits_to_f32(m["kv"]).astype(np.float64)
    qf = W.bf16_bits_to_f32(m["q"]).astype(np.float64)
    out = np.zeros((qf.shape[0], Hq, DV))
    for b in range(len(m["L"])):
        L, Q = int(m["L"][b]), int(m["Q"][b])
        t0, s0 = int(m["qsl"][b]), int(m["kv_start"][b])
        K = kvf[s0:s0 + L]
        for i in range(Q):
            p = L - Q + i
            s = scale * (qf[t0 + i] @ K.T)          # [Hq][L]
            s[:, p + 1:] = -np.inf
            w = np.exp(s - s.max(axis=1, keepdims=True))
            out[t0 + i] = (w / w.sum(axis=1, keepdims=True)) @ K[:, :DV]
    return out


@pytest.mark.parametrize("Hq", [16, 32])
def test_decode_matches_numpy_brute_force(Hq):
    m = mla_batch([1, 63, 64, 65, 200], [1, 1, 3, 1, 5], Hq, seed=3 + Hq)
    cache = oracle_cache(m)
    scale = float(np.float32(0.0721))  # the scale travels as fp32
    got = oracle.mla_decode(m["q"], cache, m["tables"], m["L"], m["qsl"], scale)
    assert np.max(np.abs(got - brute(m, Hq, scale))) <= 1e-12


def test_decode_closed_forms():
    # one key: the output is that token's first 512 dims exactly
    m = mla_batch([1, 1], [1, 1], 16, seed=4)
    cache = oracle_cache(m)
    got = oracle.mla_decode(m["q"], cache, m["tables"], m["L"], m["qsl"], 0.3)
    for b in range(2):
        want = W.bf16_bits_to_f32(m["kv"][b, :DV]).astype(np.float64)
        assert np.array_equal(got[b], np.broadcast_to(want, (16, DV)))
    # zero queries: equal weights, each query the mean of the tokens it sees
    m = mla_batch([90], [4], 16, seed=5)
    m["q"][:] = 0
    cache = oracle_cache(m)
    got = oracle.mla_decode(m["q"], cache, m["tables"], m["L"], m["qsl"], 0.3)
    kvf = W.bf16_bits_to_f32(m["kv"]).astype(np.float64)
    for i in range(4):
        p = 90 - 4 + i
        want = kvf[:p + 1, :DV].mean(axis=0)
        assert np.max(np.abs(got[i] - want)) <= 1e-12
