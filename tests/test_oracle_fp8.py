"""Pins of the oracle's 8-bit (E4M3) KV cache against definitions, not itself.

The pages name fp8 E4M3 KV-cache quantisation with one fp32 scale per tensor
("vLLM: An Exhaustive Technical Study for Kernel Engineers", section 2.8,
the KV-cache quantisation axis).  The code points are the OCP E4M3 format:
checked here against values worked out from the format's definition, a numpy
nearest-value search over all finite codes (ties to the even mantissa), the
round trip of every finite code, the 8-bit tile layout worked out by hand,
and the bf16 oracle on pools holding the same values.
"""
import numpy as np
import pytest

import oracle
import workloads as W


def finite_codes():
    return np.array([b for b in range(256) if (b & 0x7F) != 0x7F], np.uint8)


def brute_encode(v):
    """Nearest finite E4M3 value by exhaustive search (numpy, separate code):
    ties go to the code with an even mantissa; |v| >= 448 saturates; NaN is
    0x7f."""
    mags = []
    for b in range(0x7F):  # non-negative finite codes 0x00 .. 0x7e
        e, m = b >> 3, b & 7
        mags.append(m / 8 * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    mags = np.array(mags)
    out = []
    for x in np.asarray(v, np.float32).ravel():
        if np.isnan(x):
            out.append(0x7F)
            continue
        s = 0x80 if np.signbit(x) else 0
        a = abs(float(x))
        if a >= 448.0:
            out.append(s | 0x7E)
            continue
        d = np.abs(mags - a)
        best = np.flatnonzero(d == d.min())
        if len(best) > 1:  # a tie between two neighbours: the even mantissa
            best = [b for b in best if (b & 1) == 0]
        out.append(s | int(best[0]))
    return np.array(out, np.uint8)


def test_decode_values_from_the_format():
    dec = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    assert dec[0x38] == 1.0                      # e = 7, m = 0
    assert dec[0x7E] == 448.0                    # largest finite: 1.75 * 2^8
    assert dec[0x08] == 2.0 ** -6                # smallest normal
    assert dec[0x01] == 2.0 ** -9                # smallest subnormal
    assert dec[0x07] == 7 * 2.0 ** -9            # largest subnormal
    assert dec[0x3C] == 1.5 and dec[0x40] == 2.0
    assert dec[0x00] == 0.0 and not np.signbit(dec[0x00])
    assert dec[0x80] == 0.0 and np.signbit(dec[0x80])
    assert np.isnan(dec[0x7F]) and np.isnan(dec[0xFF])
    assert np.isnan(dec).sum() == 2              # no infinities, two NaNs
    pos = dec[:0x7F]
    assert np.all(np.diff(pos) > 0)              # codes order like values
    assert np.array_equal(dec[0x80:0xFF], -dec[:0x7F])


def test_encode_matches_exhaustive_nearest_search():
    rng = np.random.default_rng(11)
    mags = np.exp(rng.uniform(np.log(2.0 ** -12), np.log(600.0), 20000))
    vals = (mags * rng.choice([-1.0, 1.0], mags.shape)).astype(np.float32)
    fin = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = ((fin[1:] + fin[:-1]) / 2).astype(np.float32)     # exact ties
    specials = np.array([0.0, -0.0, 448.0, 447.99, 464.0, 479.0, 480.0, 1e30,
                         np.inf, -np.inf, np.nan, 2.0 ** -10, 2.0 ** -11,
                         3 * 2.0 ** -10, -2.0 ** -10], np.float32)
    allv = np.concatenate([vals, mids, -mids, fin.astype(np.float32), specials])
    got = oracle.e4m3_encode(allv)
    want = brute_encode(allv)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, [(float(allv[i]), int(got[i]), int(want[i])) for i in bad[:5]]


def test_every_finite_code_round_trips():
    codes = finite_codes()
    assert codes.size == 254
    back = oracle.e4m3_encode(oracle.e4m3_decode(codes).astype(np.float32))
    assert np.array_equal(back, codes)


@pytest.mark.parametrize("D", [64, 128])
def test_8bit_tile_layout_is_a_permutation(D):
    bs = 16
    for idx in (oracle.k8_index, oracle.v8_index):
        offs = sorted(idx(0, 0, t, d, 1, D) for t in range(bs) for d in range(D))
        assert offs == list(range(bs * D))
        # tile (block 3, kv head 1) of a 2-head pool starts at (3*2 + 1) * 16 * D
        assert idx(3, 1, 0, 0, 2, D) == 7 * bs * D


def test_8bit_tile_layout_by_hand():
    # K: 16-byte units [p][q][t]; dims 32c + 8q + j with c = 2p + h sit at
    # unit byte h*8 + j
    D = 128
    assert oracle.k8_index(0, 0, 1, 0, 1, D) == 16           # next token, next unit
    assert oracle.k8_index(0, 0, 0, 32, 1, D) == 8           # chunk 1: second half
    assert oracle.k8_index(0, 0, 0, 8, 1, D) == 16 * 16      # q = 1
    assert oracle.k8_index(0, 0, 0, 64, 1, D) == 64 * 16     # chunk 2: p = 1
    assert oracle.k8_index(0, 0, 5, 45, 1, D) == ((0 * 4 + 1) * 16 + 5) * 16 + 8 + 5
    # V: 16-byte units [p][tg][r]; 4-token runs for (cc, dh) at bytes (2cc+dh)*4
    assert oracle.v8_index(0, 0, 1, 0, 1, D) == 1            # next token of the run
    assert oracle.v8_index(0, 0, 0, 64, 1, D) == 4           # dh = 1
    assert oracle.v8_index(0, 0, 0, 16, 1, D) == 8           # c = 1: cc = 1
    assert oracle.v8_index(0, 0, 4, 0, 1, D) == 16 * 16      # tg = 1
    assert oracle.v8_index(0, 0, 0, 1, 1, D) == 16           # r = 1
    assert oracle.v8_index(0, 0, 0, 32, 1, D) == 64 * 16     # c = 2: p = 1
    assert oracle.v8_index(0, 0, 0, 32, 1, 64) == 4          # D = 64: dh = 1


@pytest.mark.parametrize("k_scale,v_scale", [(1.0, 1.0), (0.03125, 0.5), (0.1, 0.017)])
def test_scatter_stores_nearest_codes_of_the_scaled_values(k_scale, v_scale):
    w = W.make_workload("fp8-scatter", [20, 37], [20, 5], 8, 2, 64, seed=4)
    nb, Hkv, D = w.num_blocks, w.num_kv_heads, w.head_dim
    kc = np.full(nb * Hkv * 16 * D, 0x7F, np.uint8)
    vc = kc.copy()
    oracle.write_kv_fp8(kc, vc, w.k_new, w.v_new, w.new_slots, k_scale, v_scale)
    kf = W.bf16_bits_to_f32(w.k_new)
    vf = W.bf16_bits_to_f32(w.v_new)
    want_k = brute_encode((kf / np.float32(k_scale)).astype(np.float32)).reshape(kf.shape)
    want_v = brute_encode((vf / np.float32(v_scale)).astype(np.float32)).reshape(vf.shape)
    written = np.zeros(kc.shape, bool)
    for i, s in enumerate(w.new_slots):
        n, t = divmod(int(s), 16)
        for g in range(Hkv):
            for d in range(D):
                ko = oracle.k8_index(n, g, t, d, Hkv, D)
                vo = oracle.v8_index(n, g, t, d, Hkv, D)
                assert kc[ko] == want_k[i, g, d] and vc[vo] == want_v[i, g, d]
                written[ko] = True
    assert np.all(kc[~written] == 0x7F)  # everything else untouched


def fp8_pool(w, k_scale, v_scale):
    kc = np.zeros(w.pool_elems(), np.uint8)
    vc = np.zeros(w.pool_elems(), np.uint8)
    oracle.write_kv_fp8(kc, vc, w.k_dense[w.fill_rows], w.v_dense[w.fill_rows],
                        w.fill_slots, k_scale, v_scale)
    oracle.write_kv_fp8(kc, vc, w.k_new, w.v_new, w.new_slots, k_scale, v_scale)
    return kc, vc


def test_fp8_attention_equals_bf16_attention_on_the_same_values():
    # power-of-two scales: every decode(code) * scale is a bf16 value, so a
    # bf16 pool can hold exactly the values the 8-bit pool stands for
    w = W.make_workload("fp8-vs-bf16", [1, 17, 40, 70], [1, 1, 9, 70], 8, 2, 64, seed=6)
    ks, vs = 0.25, 0.0625
    k8, v8 = fp8_pool(w, ks, vs)
    kb = np.zeros(w.pool_elems(), np.uint16)
    vb = np.zeros(w.pool_elems(), np.uint16)
    nb, Hkv, D = w.num_blocks, w.num_kv_heads, w.head_dim
    for n in range(nb):
        for g in range(Hkv):
            for t in range(16):
                for d in range(D):
                    kv = oracle.e4m3_decode(k8[oracle.k8_index(n, g, t, d, Hkv, D)]) * ks
                    vv = oracle.e4m3_decode(v8[oracle.v8_index(n, g, t, d, Hkv, D)]) * vs
                    kb[oracle.k_index(n, g, t, d, Hkv, D)] = W.f32_to_bf16_bits(
                        np.array([kv], np.float32))[0]
                    vb[oracle.v_index(n, g, t, d, Hkv, D)] = W.f32_to_bf16_bits(
                        np.array([vv], np.float32))[0]
    a8 = oracle.attend_fp8(w.q, k8, v8, ks, vs, w.block_tables, w.seq_lens,
                           w.query_start_loc, Hkv, w.scale)
    ab = oracle.attend(w.q, kb, vb, w.block_tables, w.seq_lens, w.query_start_loc,
                       Hkv, w.scale)
    assert np.max(np.abs(a8 - ab)) <= 1e-12


def test_fp8_single_key_returns_its_dequantised_value():
    # L = 1: the output is V[0] = decode(code) * v_scale exactly
    w = W.make_workload("fp8-one-key", [1, 1], [1, 1], 4, 4, 64, seed=7)
    ks, vs = 0.3, 0.07
    k8, v8 = fp8_pool(w, ks, vs)
    out = oracle.attend_fp8(w.q, k8, v8, ks, vs, w.block_tables, w.seq_lens,
                            w.query_start_loc, w.num_kv_heads, w.scale)
    for b in range(2):
        n = int(w.block_tables[b, 0])
        for h in range(w.num_q_heads):
            want = [oracle.e4m3_decode(v8[oracle.v8_index(n, h, 0, d, 4, 64)])
                    * np.float64(np.float32(vs)) for d in range(64)]
            assert np.array_equal(out[b, h], np.array(want))


def test_fp8_rows_match_full():
    w = W.make_workload("fp8-rows", [30, 90], [3, 40], 8, 2, 128, seed=8)
    k8, v8 = fp8_pool(w, 0.05, 0.04)
    full = oracle.attend_fp8(w.q, k8, v8, 0.05, 0.04, w.block_tables, w.seq_lens,
                             w.query_start_loc, w.num_kv_heads, w.scale)
    rows = np.array([[0, 0], [2, 7], [20, 3], [42, 5]], np.int64)
    part = oracle.attend_fp8(w.q, k8, v8, 0.05, 0.04, w.block_tables, w.seq_lens,
                             w.query_start_loc, w.num_kv_heads, w.scale, rows=rows)
    for r, (t, h) in enumerate(rows):
        assert np.array_equal(part[r], full[t, h])
