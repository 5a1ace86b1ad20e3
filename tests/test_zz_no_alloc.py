"""pa_attend_noalloc: attention whose plan and split-K partials live in the
library's static device scratch instead of a caller workspace.

It runs pa_attend's kernels on the same plan, so its outputs must equal
pa_attend's bit for bit (and so lie within the oracle tolerance); checked on
two calls in a row, the second with a smaller batch than the first, so the
scratch still holds the first call's plan and partials when the second runs.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from paged_kv_cache_varlen_amd import _lib
from tests.gpu_util import Uploaded, tensor_bits
from tests.test_gpu_parity import check_close, oracle_pool, small

pytestmark = pytest.mark.gpu


def call_noalloc(lib, u, out):
    w = u.w
    return lib.pa_attend_noalloc(
        u.q.data_ptr(), u.k_cache.data_ptr(), u.v_cache.data_ptr(), w.num_blocks,
        u.block_tables.data_ptr(), u.block_tables.shape[1], u.seq_lens.data_ptr(),
        u.qsl.data_ptr(), w.num_seqs, w.num_q_tokens, w.num_q_heads, w.num_kv_heads,
        w.head_dim, w.max_query_len, w.max_seq_len, w.scale, out.data_ptr(),
        torch.cuda.current_stream().cuda_stream)


def test_noalloc_equals_pa_attend_on_two_calls():
    lib = _lib.load()
    # a decode batch with split requests (many partials), then a smaller
    # mixed batch (a chunked-prefill chunk beside decodes, other heads)
    first = W.make_config(2)
    second = small("mixed-g4-d128", seed=61)
    for w in (first, second):
        u = Uploaded(w)
        ref_bits = tensor_bits(u.attend())  # pa_attend with its own workspace
        out = torch.full_like(u.q, float("nan"))
        st = call_noalloc(lib, u, out)
        assert st == _lib.PA_OK, lib.pa_last_error()
        torch.cuda.synchronize()
        got = tensor_bits(out)
        assert np.array_equal(got, ref_bits), w.name
        kc, vc = oracle_pool(w)
        ref = oracle.attend(w.q, kc, vc, w.block_tables, w.seq_lens, w.query_start_loc,
                            w.num_kv_heads, w.scale)
        check_close(got, ref, "pa_attend_noalloc " + w.name)
        del u
        torch.cuda.empty_cache()


def test_noalloc_rejects_batches_beyond_the_scratch():
    # the mixed chunked-prefill step's bounds need about 310 MiB of workspace:
    # rejected before anything is enqueued, out left as it was
    lib = _lib.load()
    w = small("mixed-g1-d64", seed=62)
    u = Uploaded(w)
    out = torch.full_like(u.q, 5.0)
    st = lib.pa_attend_noalloc(
        u.q.data_ptr(), u.k_cache.data_ptr(), u.v_cache.data_ptr(), w.num_blocks,
        u.block_tables.data_ptr(), u.block_tables.shape[1], u.seq_lens.data_ptr(),
        u.qsl.data_ptr(), 129, 2048, 32, 8, 128, 1920, 8192, w.scale, out.data_ptr(),
        torch.cuda.current_stream().cuda_stream)
    assert st == _lib.PA_ERR_WORKSPACE
    assert b"static scratch" in lib.pa_last_error()
    torch.cuda.synchronize()
    assert bool((out == 5.0).all())
