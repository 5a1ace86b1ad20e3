"""GPU parity of the fused scatter + work plan (pa_write_kv_plan(_fp8)).

The call replaces pa_write_kv (pa_write_kv_fp8) and pa_attend_plan
(pa_attend_plan_cascade) of the same step, so its bars are theirs: every pool
byte equal to the oracle's scatter, and attention over the fused call's plan
bit-identical to pa_attend over the separately written pools (the plan is
the same work list, so the same kernels produce the same bits), which is
itself within the attention tolerance of the fp64 oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_varlen_amd as pa
import workloads as W
from tests.gpu_util import Uploaded, bf16_tensor, i32, i64, tensor_bits
from tests.test_gpu_cascade import casc, cascade_ws, oracle_ref, run_cascade
from tests.test_gpu_fp8 import attend8, gpu_pool8, oracle_pool8, u8_bits
from tests.test_gpu_parity import check_close, oracle_pool, small

pytestmark = pytest.mark.gpu


def fused(u, k_cache, v_cache, ws, common_prefix_len=None, scales=(None, None)):
    w = u.w
    pa.write_kv_plan(u.k_new, u.v_new, u.new_slots, k_cache, v_cache, u.block_tables,
                     u.seq_lens, u.qsl, w.num_q_tokens, w.num_q_heads, w.max_query_len,
                     w.max_seq_len, ws, common_prefix_len=common_prefix_len,
                     k_scale=scales[0], v_scale=scales[1])


@pytest.mark.parametrize("name", ["mixed-g4-d128", "mixed-g1-d64", "mixed-h3-d64",
                                  "mixed-g16-d128", "mixed-split-edge"])
def test_fused_bf16_equals_separate_calls(name):
    w = small(name, seed=21)
    u = Uploaded(w, write_new=False)
    fused(u, u.k_cache, u.v_cache, u.workspace)
    got = tensor_bits(u.attend(out=torch.empty_like(u.q), planned=True)).copy()
    torch.cuda.synchronize()
    kc, vc = oracle_pool(w)
    assert np.array_equal(tensor_bits(u.k_cache).ravel(), kc)
    assert np.array_equal(tensor_bits(u.v_cache).ravel(), vc)
    ref = Uploaded(w)
    want = tensor_bits(ref.attend()).copy()
    assert np.array_equal(got, want)
    check_close(got, oracle.attend(w.q, kc, vc, w.block_tables, w.seq_lens,
                                   w.query_start_loc, w.num_kv_heads, w.scale), name)


@pytest.mark.parametrize("name", ["mixed-g4-d128", "mixed-g1-d64", "mixed-h3-d64"])
def test_fused_fp8_equals_separate_calls(name):
    w = small(name, seed=22)
    scales = (0.011, 0.0107)
    # pools holding every token but the new ones, then the fused call
    kc, vc = pa.alloc_pool_fp8(w.num_blocks, w.num_kv_heads, w.head_dim, fill=0x7F)
    if len(w.fill_rows):
        pa.write_kv_fp8(bf16_tensor(w.k_dense[w.fill_rows]),
                        bf16_tensor(w.v_dense[w.fill_rows]), i64(w.fill_slots), kc, vc,
                        *scales)
    u = Uploaded(w, write_new=False)
    fused(u, kc, vc, u.workspace, scales=scales)
    got = tensor_bits(pa.attend(u.q, kc, vc, u.block_tables, u.seq_lens, u.qsl, w.scale,
                                w.max_query_len, w.max_seq_len,
                                num_kv_heads=w.num_kv_heads, out=torch.empty_like(u.q),
                                workspace=u.workspace, planned=True,
                                k_scale=scales[0], v_scale=scales[1])).copy()
    torch.cuda.synchronize()
    okc, ovc = oracle_pool8(w, *scales)
    assert np.array_equal(u8_bits(kc), okc)
    assert np.array_equal(u8_bits(vc), ovc)
    rk, rv = gpu_pool8(w, *scales)
    assert np.array_equal(got, attend8(w, rk, rv, *scales))


@pytest.mark.parametrize("name", ["casc-decode-g4-d128", "casc-mixed-g4-d128",
                                  "casc-g8-d64-p48"])
def test_fused_shared_prefix_plan(name):
    w, C = casc(name, seed=23)
    u = Uploaded(w, write_new=False)
    ws = cascade_ws(w)
    fused(u, u.k_cache, u.v_cache, ws, common_prefix_len=C)
    got = tensor_bits(pa.attend(u.q, u.k_cache, u.v_cache, u.block_tables, u.seq_lens,
                                u.qsl, w.scale, w.max_query_len, w.max_seq_len,
                                num_kv_heads=w.num_kv_heads, out=torch.empty_like(u.q),
                                workspace=ws, planned=True,
                                common_prefix_len=C)).copy()
    torch.cuda.synchronize()
    kc, vc = oracle_pool(w)
    assert np.array_equal(tensor_bits(u.k_cache).ravel(), kc)
    assert np.array_equal(tensor_bits(u.v_cache).ravel(), vc)
    assert np.array_equal(got, run_cascade(Uploaded(w), C))
    check_close(got, oracle_ref(w), name)


def test_fused_without_new_tokens_is_the_plan():
    w = small("mixed-g4-d128", seed=24)
    u = Uploaded(w)
    none = torch.empty((0, w.num_kv_heads, w.head_dim), dtype=torch.bfloat16,
                       device="cuda")
    pa.write_kv_plan(none, none, i64(np.zeros(0, np.int64)), u.k_cache, u.v_cache,
                     u.block_tables, u.seq_lens, u.qsl, w.num_q_tokens, w.num_q_heads,
                     w.max_query_len, w.max_seq_len, u.workspace)
    got = tensor_bits(u.attend(out=torch.empty_like(u.q), planned=True)).copy()
    want = tensor_bits(Uploaded(w).attend()).copy()
    assert np.array_equal(got, want)


def test_fused_with_nothing_to_plan_is_the_scatter():
    w = small("mixed-g1-d64", seed=25)
    u = Uploaded(w, write_new=False)
    empty_qsl = i32(np.zeros(1, np.int32))
    pa.write_kv_plan(u.k_new, u.v_new, u.new_slots, u.k_cache, u.v_cache,
                     u.block_tables[:0], u.seq_lens[:0], empty_qsl, 0, w.num_q_heads,
                     0, 0, u.workspace)
    torch.cuda.synchronize()
    kc, vc = oracle_pool(w)
    assert np.array_equal(tensor_bits(u.k_cache).ravel(), kc)
    assert np.array_equal(tensor_bits(u.v_cache).ravel(), vc)


def test_fused_plan_serves_several_layers():
    # a forward step: the fused call writes the first layer's
    # new tokens and plans; every other layer reuses the plan
    w = small("mixed-g8-d128", seed=26)
    u = Uploaded(w, write_new=False)
    fused(u, u.k_cache, u.v_cache, u.workspace)
    a = tensor_bits(u.attend(out=torch.empty_like(u.q), planned=True)).copy()
    b = tensor_bits(u.attend(out=torch.empty_like(u.q), planned=True)).copy()
    assert np.array_equal(a, b)
    assert np.array_equal(a, tensor_bits(Uploaded(w).attend()))


def test_binding_rejects_metadata_of_other_types():
    # int32 metadata only: an int64 seq_lens read as int32 would be other lengths
    w = small("mixed-g1-d64", seed=27)
    u = Uploaded(w, write_new=False)
    with pytest.raises(TypeError):
        pa.write_kv_plan(u.k_new, u.v_new, u.new_slots, u.k_cache, u.v_cache,
                         u.block_tables, u.seq_lens.to(torch.int64), u.qsl, w.num_q_tokens,
                         w.num_q_heads, w.max_query_len, w.max_seq_len, u.workspace)
    with pytest.raises(TypeError):
        pa.attend_plan(u.block_tables.to(torch.int64), u.seq_lens, u.qsl, w.num_q_tokens,
                       w.num_q_heads, w.num_kv_heads, w.head_dim, w.max_query_len,
                       w.max_seq_len, u.workspace)


# ---- the plan's work list, read back ------------------------------------------------

def expected_long_split(L, Q, Hq, Hkv, per_cu=4):
    """Key range of the splits of decode requests of more than 8192 keys: the
    shortest of 1024, 2048, 4096 whose units (requests' ranges x kv heads)
    number at most per_cu per CU (4; 8-bit plans 8), else 8192."""
    G = Hq // Hkv
    own = np.asarray(L, np.int64)[(np.asarray(L) > 8192) & (np.asarray(Q) >= 1) &
                                  (np.asarray(Q) <= 16 // G)]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for s in (1024, 2048, 4096):
        if int(((own + s - 1) // s).sum()) * Hkv <= per_cu * cus:
            return s
    return 8192


def RANGES_OFFSET(w):
    """Byte offset of the stream range table: the end of the partial
    accumulators (the layout of pa_attend_workspace_size's sections)."""
    return stream_table_offset(w.num_seqs, w.num_q_tokens, w.num_q_heads, w.num_kv_heads,
                               w.head_dim, w.max_query_len, w.max_seq_len)


def stream_table_offset(B, T, Hq, Hkv, D, max_q, max_l):
    al = lambda x: (x + 255) & ~255
    G = Hq // Hkv
    tq_d, tq_p = 16 // G, 4 * (32 // G)
    sd = -(-max(max_l, 1) // 384)
    sp = -(-max(max_l, 1) // 2048)
    pre_tiles = (T // tq_p + B) if max_q > tq_d else 0
    max_items = max(1, B * (sd + 2) + pre_tiles * sp)
    dec_tok = min(T, B * tq_d)
    pre_tok = T if max_q > tq_d else 0
    max_partials = max(1, dec_tok * (sd + 2) + pre_tok * sp)
    off = 4096 + 4 * 8 * 1024
    off = al(off + 64 * max_items)
    off = al(off + 16 * max_items)
    off = al(off + 8 * max_partials * Hq)
    off = al(off + 4 * max_partials * Hq * D)
    return off


# Internal workspace layout of a plain plan: the plan header at byte 0 (num_work,
# num_items, error, ... as uint32), then 8 decode-queue counters 4 KiB apart
# from byte 4096, then the work items (16 int32 each: seq, tok0, ntok, kind, kv0,
# kv1, split, nsplit, pbase, counter, posbase, pad) from byte 4096 + 32 KiB.
ITEMS_OFFSET = 4096 + 8 * 4096
# Stream positions (of 32 keys each) that stand for a request's start in a
# stream plan: the cost of a wave's switch to the request's first item.
START_PAIRS = 2


def read_plan(w, fp8):
    """Plan w into a workspace filled with 0xff, read the work items back and
    check that every slot in [0, num_items) holds exactly one valid decode item
    and that each request's items cover its keys 0 .. L-1 once, in split
    order.  For a stream plan (header word 9: the number of stream ranges R),
    also check the range table: R equal runs of the decode stream (per
    request in request order, START_PAIRS pairs for its start, then its
    32-key pairs), each a run of consecutive items.
    Returns, per request, the lengths of its key ranges, and R."""
    B, L, Q = w.num_seqs, w.seq_lens, w.query_lens
    bt, sl, qsl = i32(w.block_tables), i32(w.seq_lens), i32(w.query_start_loc)
    ws = pa.alloc_workspace(w.num_seqs, w.num_q_tokens, w.num_q_heads, w.num_kv_heads,
                            w.head_dim, w.max_query_len, w.max_seq_len)
    ws.fill_(0xFF)
    pa.attend_plan(bt, sl, qsl, w.num_q_tokens, w.num_q_heads, w.num_kv_heads,
                   w.head_dim, w.max_query_len, w.max_seq_len, ws, fp8=fp8)
    torch.cuda.synchronize()
    raw = ws.cpu().numpy()
    hdr = raw[:64].view(np.uint32)
    num_work, num_items, err, nranges = int(hdr[0]), int(hdr[1]), int(hdr[2]), int(hdr[9])
    assert err == 0
    assert num_work == (nranges if nranges else num_items) * w.num_kv_heads
    items = raw[ITEMS_OFFSET:ITEMS_OFFSET + 64 * num_items].view(np.int32).reshape(-1, 16)
    seq, tok0, ntok, kind, kv0, kv1, split, nsplit = (items[:, i] for i in range(8))
    assert np.all((seq >= 0) & (seq < B)), "unwritten or foreign slot"
    assert np.all(kind == 0) and np.all(kv1 > kv0)
    qs = w.query_start_loc
    assert np.array_equal(tok0, qs[seq]) and np.array_equal(ntok, Q[seq])
    order = np.lexsort((kv0, seq))
    seq, kv0, kv1, split, nsplit = seq[order], kv0[order], kv1[order], split[order], nsplit[order]
    counts = np.bincount(seq, minlength=B)
    assert np.array_equal(counts, nsplit[np.searchsorted(seq, np.arange(B))])
    first = np.searchsorted(seq, np.arange(B))
    ranges = []
    for b in range(B):
        s0 = first[b]
        r0, r1 = kv0[s0:s0 + counts[b]], kv1[s0:s0 + counts[b]]
        assert r0[0] == 0 and r1[-1] == L[b]
        assert np.array_equal(r0[1:], r1[:-1]), b
        assert np.array_equal(split[s0:s0 + counts[b]], np.arange(counts[b]))
        ranges.append(r1 - r0)
    if nranges:
        # items in request order (the stream's order), the table R + 1 item
        # indices from 0 to num_items, every range the same number of pairs +-1
        assert np.array_equal(order, np.arange(num_items))
        table = raw[RANGES_OFFSET(w):RANGES_OFFSET(w) + 4 * (nranges + 1)].view(np.int32)
        assert table[0] == 0 and table[-1] == num_items and np.all(np.diff(table) >= 1)
        # The stream: every request is START_PAIRS pairs with no keys (its
        # start) followed by its key pairs; range r is positions [s_r,
        # s_(r+1)) of a cut into equal lengths +-1.  A range's length is the
        # key pairs of its items plus the start positions that fall in it.
        pairs = (kv1 - kv0 + 31) // 32
        per_range = np.add.reduceat(pairs, table[:-1])
        span = (L + 31) // 32 + START_PAIRS
        total = int(span.sum())
        q, rem = divmod(total, nranges)
        bounds = np.arange(nranges + 1) * q + np.minimum(np.arange(nranges + 1), rem)
        starts = np.concatenate([[0], np.cumsum(span)[:-1]])
        for k in range(START_PAIRS):
            per_range = per_range + np.bincount(
                np.searchsorted(bounds, starts + k, side="right") - 1, minlength=nranges)
        assert np.array_equal(per_range, np.diff(bounds))
    return ranges, nranges


@pytest.mark.parametrize("B,fp8", [(700, False), (700, True), (1500, False), (1500, True)])
def test_plan_items_partition_every_request(B, fp8):
    # one sweep (<= 1024 requests) and two sweeps, bf16 and 8-bit plans: every
    # slot in [0, num_items) holds exactly one valid item (the workspace is
    # filled with 0xff first, so a slot left unwritten is seen), and the items
    # of each request cover its keys 0 .. L-1 once, in ranges of the plan's
    # split length
    rng = np.random.default_rng(40 + B)
    L = rng.integers(1, 9500, size=B)
    Q = np.minimum(L, rng.integers(1, 3, size=B))
    w = W.make_workload("plan-%d" % B, L, Q, 16, 2, 64, seed=41)
    ranges, nranges = read_plan(w, fp8)
    # 700 requests: one sweep, a stream plan (bf16: 4 units per CU, 8-bit:
    # 8); 1500 (two sweeps): splits of each request's own
    assert (nranges > 0) == (B <= 1024)
    if nranges:
        return
    long_split = expected_long_split(L, Q, w.num_q_heads, w.num_kv_heads, 8 if fp8 else 4)
    for b in range(B):
        span = long_split if L[b] > 8192 else (384 if fp8 else 512)
        assert np.all(ranges[b][:-1] == span), b


@pytest.mark.parametrize("B,Lr,seed", [(12, 12000, 1), (40, 16384, 3), (3, 12000, 4),
                                        (2, 30000, 5)])
def test_long_requests_stream_or_split(B, Lr, seed):
    # decode batches of requests of more than 8192 keys: where the batch fills
    # 4 units per CU with ranges of at least 512 keys it is a stream plan
    # (12 x 12000 and 40 x 16384 keys over 8 kv heads on 256 CUs), otherwise
    # each request is cut into splits of the long length the batch picks
    # (3 x 12000, 2 x 30000: 1024); every output row against the oracle
    rng = np.random.default_rng(seed)
    L = (Lr - rng.integers(0, 200, size=B)).astype(np.int64)
    Q = np.ones(B, np.int64)
    w = W.make_workload("long-%d" % B, L, Q, 8, 8, 64, seed=seed)
    ranges, nranges = read_plan(w, False)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    want = min(4 * cus, 2048) // 8
    # (streamed when the key pairs alone fill the units' minimum ranges)
    assert (nranges > 0) == (int(((L + 31) // 32).sum()) >= want * 16)
    if nranges == 0:
        span = expected_long_split(L, Q, 8, 8)
        for b in range(B):
            assert np.all(ranges[b][:-1] == span) and ranges[b][-1] <= span, b
    out = tensor_bits(Uploaded(w).attend())
    kc, vc = oracle_pool(w)
    ref = oracle.attend(w.q, kc, vc, w.block_tables, w.seq_lens, w.query_start_loc,
                        w.num_kv_heads, w.scale)
    check_close(out, ref, "long requests, %d stream ranges" % nranges)


def test_stream_decision_counts_keys_only():
    # 900 one-key decodes beside one of 1000 keys: with their start positions
    # the stream would fill the units' minimum ranges, with their keys alone
    # it does not, and the keys decide: no stream ranges (per-request
    # splits); every output row against the oracle
    L = np.ones(901, np.int64)
    L[450] = 1000
    Q = np.ones(901, np.int64)
    w = W.make_workload("keys-only", L, Q, 8, 8, 64, seed=24)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    want = min(4 * cus, 2048) // 8
    pairs = (L + 31) // 32
    assert pairs.sum() < want * 16 <= (pairs + START_PAIRS).sum()
    _, nranges = read_plan(w, False)
    assert nranges == 0
    out = tensor_bits(Uploaded(w).attend())
    kc, vc = oracle_pool(w)
    ref = oracle.attend(w.q, kc, vc, w.block_tables, w.seq_lens, w.query_start_loc,
                        w.num_kv_heads, w.scale)
    check_close(out, ref, "one-key decodes beside a long one")


@pytest.mark.parametrize("fp8", [False, True])
def test_stream_plan_requests_of_many_pieces(fp8):
    # a stream plan whose requests meet more than 32 ranges each (the plan's
    # wave emits such a request's pieces, 64 at a time), beside short ones
    # emitted one lane each: 3 requests of about 60000 keys (bf16: ~44
    # pieces, one pass; 8-bit: ~87, two) and 5 of a few hundred; every
    # output row against the oracle
    rng = np.random.default_rng(23)
    L = np.array([60000, 300, 58000, 77, 61111, 500, 900, 33], np.int64)
    Q = np.minimum(L, rng.integers(1, 3, size=len(L)))
    w = W.make_workload("many-pieces", L, Q, 16, 8, 64, seed=23)
    ranges, nranges = read_plan(w, fp8)
    assert nranges > 0 and max(len(r) for r in ranges) > (64 if fp8 else 32)
    if not fp8:
        out = tensor_bits(Uploaded(w).attend())
        kc, vc = oracle_pool(w)
        ref = oracle.attend(w.q, kc, vc, w.block_tables, w.seq_lens, w.query_start_loc,
                            w.num_kv_heads, w.scale)
    else:
        scales = (0.011, 0.0107)
        kc8, vc8 = gpu_pool8(w, *scales)
        out = attend8(w, kc8, vc8, *scales)
        okc, ovc = oracle_pool8(w, *scales)
        ref = oracle.attend_fp8(w.q, okc, ovc, scales[0], scales[1], w.block_tables,
                                w.seq_lens, w.query_start_loc, w.num_kv_heads, w.scale)
    check_close(out, ref, "stream plan, requests of many pieces%s" % (" (8-bit)" if fp8 else ""))


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("Hq,Hkv,D,seed", [(32, 8, 128, 21), (16, 4, 64, 22)])
def test_stream_plan_multi_token_decodes(fp8, Hq, Hkv, D, seed):
    # a stream plan over decodes of 1 to 16/G query tokens (speculative
    # decoding) with lengths from a few blocks to a few thousand keys, so that
    # range boundaries fall inside requests, between them and inside a
    # request's last partial pair; and requests shorter than a range, several
    # in one range.  The read-back checks the range table; every output row
    # against the oracle (8-bit: on the same codes)
    rng = np.random.default_rng(seed)
    B = 220
    L = rng.integers(20, 3000, size=B)
    L[::7] = rng.integers(20, 80, size=len(L[::7]))
    Q = np.minimum(L, rng.integers(1, 16 // (Hq // Hkv) + 1, size=B))
    w = W.make_workload("stream-q", L, Q, Hq, Hkv, D, seed=seed)
    _, nranges = read_plan(w, fp8)
    assert nranges > 0
    if not fp8:
        out = tensor_bits(Uploaded(w).attend())
        kc, vc = oracle_pool(w)
        ref = oracle.attend(w.q, kc, vc, w.block_tables, w.seq_lens, w.query_start_loc,
                            w.num_kv_heads, w.scale)
    else:
        scales = (0.011, 0.0107)
        kc8, vc8 = gpu_pool8(w, *scales)
        out = attend8(w, kc8, vc8, *scales)
        okc, ovc = oracle_pool8(w, *scales)
        ref = oracle.attend_fp8(w.q, okc, ovc, scales[0], scales[1], w.block_tables,
                                w.seq_lens, w.query_start_loc, w.num_kv_heads, w.scale)
    check_close(out, ref, "stream plan, multi-token decodes%s" % (" (8-bit)" if fp8 else ""))
