"""GPU parity of shared-prefix (cascade) attention against the CPU oracle.

The shared-prefix calls compute the same attention as pa_attend (the prefix
attended once for the whole batch, merged with each request's own keys by
log-sum-exp renormalisation), so the bar is pa_attend's: within max-abs 3e-2
and mean-abs 2e-3 of the fp64 oracle's attention on the same pool.  Exact
invariants of the design are checked bit for bit: planned == unplanned, the
unshared twin (private copies of the prefix) == the shared layout, and a
request's rows do not depend on the rest of the batch.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_varlen_amd as pa
import workloads as W
from tests import configs
from tests.gpu_util import Uploaded, bf16_tensor, i32, i64, tensor_bits
from tests.test_gpu_fp8 import gpu_pool8, oracle_pool8
from tests.test_gpu_parity import check_close, oracle_pool, sample_rows, to64

pytestmark = pytest.mark.gpu

CASC = {
    # name: (seq_lens, query_lens, Hq, Hkv, D, shared prefix)
    # decode batch: one 16-token-aligned prefix, suffixes of 1 .. 600 keys
    "casc-decode-g4-d128": ([512 + x for x in (1, 7, 16, 33, 100, 255, 256, 600, 31,
                                               64, 2, 400, 17, 90, 128, 511, 3)],
                            [1] * 17, 32, 8, 128, 512),
    # chunks and decodes together; suffix ranges across the 2048-key split
    "casc-mixed-g4-d128": ([300, 263, 2600, 500, 290, 420, 257],
                           [1, 7, 2300, 100, 3, 16, 1], 16, 4, 128, 256),
    # G = 1: decode tiles of up to 16 tokens
    "casc-g1-d64": ([130, 200, 97, 400, 111], [1, 5, 1, 60, 15], 4, 4, 64, 96),
    # a prefix of 48 keys: 32 are shared, the next 16 stay with each request
    "casc-g8-d64-p48": ([60, 49, 300, 75], [1, 1, 40, 27], 16, 2, 64, 48),
    "casc-g16-d128": ([1100, 1030, 1500], [1, 2, 70], 32, 2, 128, 1024),
    # the most prefix key ranges (8) and a chunk past a long prefix
    "casc-long-prefix": ([4001, 4100, 4300, 4096], [1, 3, 200, 96], 8, 2, 128, 4000),
    # a prefix shorter than 32 keys: nothing shared, plain attention
    "casc-prefix-16": ([40, 17, 90], [1, 1, 30], 8, 8, 64, 16),
    # more requests than the planning workgroup's threads
    "casc-1100-requests": ([64 + (i * 37) % 150 + 1 for i in range(1100)], [1] * 1100,
                           8, 2, 64, 64),
}


def casc(name, seed=0, shared=True):
    L, Q, Hq, Hkv, D, C = CASC[name]
    return W.make_workload(name, L, Q, Hq, Hkv, D, seed=seed, shared_prefix=C,
                           shared=shared), C


def cascade_ws(w):
    return pa.alloc_workspace(w.num_seqs, w.num_q_tokens, w.num_q_heads,
                              w.num_kv_heads, w.head_dim, w.max_query_len,
                              w.max_seq_len, cascade=True)


def run_cascade(u, C, out=None, planned=False, ws=None, k_cache=None, v_cache=None,
                scales=(1.0, 1.0), tables=None, seq_lens=None, qsl=None, q=None,
                max_query_len=None, max_seq_len=None):
    w = u.w
    bt = u.block_tables if tables is None else tables
    sl = u.seq_lens if seq_lens is None else seq_lens
    qs = u.qsl if qsl is None else qsl
    qq = u.q if q is None else q
    mq = w.max_query_len if max_query_len is None else max_query_len
    ms = w.max_seq_len if max_seq_len is None else max_seq_len
    if ws is None:
        ws = pa.alloc_workspace(bt.shape[0], qq.shape[0], w.num_q_heads,
                                w.num_kv_heads, w.head_dim, mq, ms, cascade=True)
    if planned:
        pa.attend_plan(bt, sl, qs, qq.shape[0], w.num_q_heads, w.num_kv_heads,
                       w.head_dim, mq, ms, ws, common_prefix_len=C)
    o = pa.attend(qq, u.k_cache if k_cache is None else k_cache,
                  u.v_cache if v_cache is None else v_cache, bt, sl, qs, w.scale, mq, ms,
                  num_kv_heads=w.num_kv_heads,
                  out=torch.empty_like(qq) if out is None else out, workspace=ws,
                  planned=planned, common_prefix_len=C, k_scale=scales[0],
                  v_scale=scales[1])
    torch.cuda.synchronize()
    return tensor_bits(o).copy()


def oracle_ref(w, rows=None):
    kc, vc = oracle_pool(w)
    if rows is None:
        return oracle.attend(w.q, kc, vc, w.block_tables, w.seq_lens,
                             w.query_start_loc, w.num_kv_heads, w.scale)
    return oracle.attend_rows(w.q, kc, vc, w.block_tables, w.seq_lens,
                              w.query_start_loc, w.num_kv_heads, w.scale, rows)


@pytest.mark.parametrize("name", sorted(CASC))
def test_cascade_parity(name):
    w, C = casc(name, seed=1)
    print("case", name, "prefix", C, flush=True)
    u = Uploaded(w)
    got = run_cascade(u, C)
    check_close(got, oracle_ref(w), name)


@pytest.mark.parametrize("name", ["casc-decode-g4-d128", "casc-mixed-g4-d128",
                                  "casc-g8-d64-p48", "casc-long-prefix"])
@pytest.mark.parametrize("scales", [(1.0, 1.0), (0.011, 0.0107)])
def test_cascade_parity_fp8(name, scales):
    w, C = casc(name, seed=2)
    print("case", name, "prefix", C, "scales", scales, flush=True)
    u = Uploaded(w)
    kc, vc = gpu_pool8(w, *scales)
    got = run_cascade(u, C, k_cache=kc, v_cache=vc, scales=scales)
    okc, ovc = oracle_pool8(w, *scales)
    ref = oracle.attend_fp8(w.q, okc, ovc, scales[0], scales[1], w.block_tables,
                            w.seq_lens, w.query_start_loc, w.num_kv_heads, w.scale)
    check_close(got, ref, "%s fp8 %s" % (name, scales))


@pytest.mark.parametrize("name", ["casc-decode-g4-d128", "casc-mixed-g4-d128",
                                  "casc-1100-requests"])
def test_cascade_planned_equals_unplanned(name):
    w, C = casc(name, seed=3)
    u = Uploaded(w)
    a = run_cascade(u, C)
    ws = cascade_ws(w)
    b1 = run_cascade(u, C, planned=True, ws=ws)
    # the same plan again (one plan, several layers)
    o = pa.attend(u.q, u.k_cache, u.v_cache, u.block_tables, u.seq_lens, u.qsl,
                  w.scale, w.max_query_len, w.max_seq_len, num_kv_heads=w.num_kv_heads,
                  out=torch.empty_like(u.q), workspace=ws, planned=True,
                  common_prefix_len=C)
    torch.cuda.synchronize()
    assert np.array_equal(a, b1)
    assert np.array_equal(a, tensor_bits(o))


def test_cascade_unshared_twin_bit_identical():
    # private copies of the prefix hold the same values: read through request
    # 0's table they give the same bits as the shared blocks
    ws_, C = casc("casc-mixed-g4-d128", seed=4)
    wu, _ = casc("casc-mixed-g4-d128", seed=4, shared=False)
    a = run_cascade(Uploaded(ws_), C)
    b = run_cascade(Uploaded(wu), C)
    assert np.array_equal(a, b)


def test_cascade_rows_independent_of_the_batch():
    # a sub-batch of the same pool (request 0 and every third request): the
    # prefix tiles then group other tokens, and every row keeps its bits
    w, C = casc("casc-decode-g4-d128", seed=5)
    u = Uploaded(w)
    full = run_cascade(u, C)
    keep = [b for b in range(w.num_seqs) if b % 3 == 0]
    qsl = w.query_start_loc
    toks = np.concatenate([np.arange(qsl[b], qsl[b + 1]) for b in keep])
    qlens = [int(qsl[b + 1] - qsl[b]) for b in keep]
    sub = run_cascade(u, C, tables=i32(w.block_tables[keep]),
                      seq_lens=i32(w.seq_lens[keep]), qsl=i32(W.query_start_loc(qlens)),
                      q=bf16_tensor(w.q[toks]))
    assert np.array_equal(sub, full[toks])


def test_cascade_close_to_plain():
    w, C = casc("casc-mixed-g4-d128", seed=6)
    u = Uploaded(w)
    a = to64(run_cascade(u, C))
    b = to64(tensor_bits(u.attend()))
    # two roundings of the same attention: within the bf16 output's rounding
    # plus the fp32 reduction-order difference
    assert np.max(np.abs(a - b)) <= 2e-2


def test_cascade_skips_a_request_inside_the_prefix():
    # request 1 (110 cached tokens, a 40-token chunk) queries inside the
    # 128-key shared prefix: its rows stay untouched, the others are right
    w = W.make_workload("casc-inside", [200, 150, 300, 129], [1, 40, 20, 1], 4, 4, 64,
                        seed=7, shared_prefix=128)
    u = Uploaded(w)
    out = torch.full_like(u.q, 7.0)
    got = run_cascade(u, 128, out=out)
    qsl = w.query_start_loc
    ref = oracle_ref(w)
    for b in range(w.num_seqs):
        t0, t1 = int(qsl[b]), int(qsl[b + 1])
        if b == 1:
            assert np.all(to64(got[t0:t1]) == 7.0)
        else:
            check_close(got[t0:t1], ref[t0:t1], "request %d" % b)


def test_cascade_prefix_longer_than_request0_writes_nothing():
    w, C = casc("casc-g1-d64", seed=8)
    u = Uploaded(w)
    out = torch.full_like(u.q, 7.0)
    got = run_cascade(u, (int(w.seq_lens[0]) + 32) & ~31, out=out)
    assert np.all(to64(got) == 7.0)


def test_plan_kinds_do_not_mix():
    # a shared-prefix plan run by the plain calls (and the reverse) is
    # detected on the device: nothing is written
    w, C = casc("casc-decode-g4-d128", seed=9)
    u = Uploaded(w)
    ws = cascade_ws(w)
    pa.attend_plan(u.block_tables, u.seq_lens, u.qsl, w.num_q_tokens, w.num_q_heads,
                   w.num_kv_heads, w.head_dim, w.max_query_len, w.max_seq_len, ws,
                   common_prefix_len=C)
    out = torch.full_like(u.q, 7.0)
    pa.attend(u.q, u.k_cache, u.v_cache, u.block_tables, u.seq_lens, u.qsl, w.scale,
              w.max_query_len, w.max_seq_len, num_kv_heads=w.num_kv_heads, out=out,
              workspace=ws, planned=True)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
    pa.attend_plan(u.block_tables, u.seq_lens, u.qsl, w.num_q_tokens, w.num_q_heads,
                   w.num_kv_heads, w.head_dim, w.max_query_len, w.max_seq_len, ws)
    pa.attend(u.q, u.k_cache, u.v_cache, u.block_tables, u.seq_lens, u.qsl, w.scale,
              w.max_query_len, w.max_seq_len, num_kv_heads=w.num_kv_heads, out=out,
              workspace=ws, planned=True, common_prefix_len=C)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())


@pytest.mark.timeout(900)
def test_config4_cascade():
    # 256 decodes sharing a 2048-token prefix: every output row against the
    # oracle, and bit-identical to the unshared twin
    w = configs.workload(4)
    C = w.shared_prefix
    u = Uploaded(w)
    got = run_cascade(u, C)
    del u
    torch.cuda.empty_cache()
    check_close(got, configs.attend(4), "config 4 cascade (all rows)")
    wu = configs.workload(4, shared=False)
    gu = run_cascade(Uploaded(wu), C)
    assert np.array_equal(got, gu)


@pytest.mark.timeout(900)
def test_config4_cascade_fp8():
    w = configs.workload(4)
    C = w.shared_prefix
    ks, vs = configs.FP8_SCALES
    u = Uploaded(w)
    kc, vc = gpu_pool8(w, ks, vs)
    got = run_cascade(u, C, k_cache=kc, v_cache=vc, scales=(ks, vs))
    del u, kc, vc
    torch.cuda.empty_cache()
    check_close(got, configs.attend8(4), "config 4 cascade fp8 (all rows)")


def test_cascade_fp8_planned_equals_unplanned():
    w, C = casc("casc-mixed-g4-d128", seed=10)
    u = Uploaded(w)
    kc, vc = gpu_pool8(w, 0.02, 0.03)
    a = run_cascade(u, C, k_cache=kc, v_cache=vc, scales=(0.02, 0.03))
    b = run_cascade(u, C, k_cache=kc, v_cache=vc, scales=(0.02, 0.03), planned=True,
                    ws=cascade_ws(w))
    assert np.array_equal(a, b)


def test_cascade_with_larger_blocks():
    # 32-token blocks: an 8-block (256-token) prefix held by every request,
    # private suffix blocks; the pool read through expanded 16-token tables
    rng = np.random.default_rng(12)
    bs, C, Hq, Hkv, D = 32, 256, 16, 4, 128
    L = np.array([C + 1, C + 40, C + 300, C + 77], np.int32)
    Q = np.array([1, 20, 1, 5], np.int32)
    nb32 = C // bs + sum(-(-(int(x) - C) // bs) for x in L) + 3
    perm = [int(x) for x in rng.permutation(nb32)]
    prefix_ids, pos = perm[:C // bs], C // bs
    tables = np.full((len(L), -(-int(L.max()) // bs)), -1, np.int32)
    for b, x in enumerate(L):
        n = -(-(int(x) - C) // bs)
        tables[b, :C // bs] = prefix_ids
        tables[b, C // bs:C // bs + n] = perm[pos:pos + n]
        pos += n
    kv_start = np.concatenate([[0], np.cumsum(L)])
    kd = W.normal_bf16((12, 0), (int(L.sum()), Hkv, D))
    vd = W.normal_bf16((12, 1), (int(L.sum()), Hkv, D))
    for b in range(1, len(L)):  # every request's first C tokens are request 0's
        kd[kv_start[b]:kv_start[b] + C] = kd[:C]
        vd[kv_start[b]:kv_start[b] + C] = vd[:C]
    rows, slots = [], []
    for b in range(len(L)):
        first = 0 if b == 0 else C  # the shared blocks are written once
        pos_b = np.arange(first, int(L[b]))
        rows.append(kv_start[b] + pos_b)
        slots.append(W.slots_for(tables[b], pos_b, bs))
    rows, slots = np.concatenate(rows), np.concatenate(slots)
    kc, vc = pa.alloc_pool(nb32 * (bs // 16), Hkv, D, fill=float("nan"))
    pa.write_kv(bf16_tensor(kd[rows]), bf16_tensor(vd[rows]), i64(slots), kc, vc)
    t16 = pa.expand_block_tables(i32(tables), bs)
    qsl = W.query_start_loc(Q)
    q = W.normal_bf16((12, 2), (int(Q.sum()), Hq, D))
    scale = float(np.float32(1 / np.sqrt(D)))
    ws = pa.alloc_workspace(len(L), int(Q.sum()), Hq, Hkv, D, int(Q.max()), int(L.max()),
                            cascade=True)
    out = pa.attend(bf16_tensor(q), kc, vc, t16, i32(L), i32(qsl), scale, int(Q.max()),
                    int(L.max()), num_kv_heads=Hkv, workspace=ws, common_prefix_len=C)
    torch.cuda.synchronize()
    ref = oracle.attend_dense(q, kd, vd, L, qsl, scale)
    check_close(tensor_bits(out), ref, "shared prefix over 32-token blocks")
