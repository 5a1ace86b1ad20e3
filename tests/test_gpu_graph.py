"""A step's launches -- the scatter and work plan (one launch), the attention
kernel and the split merge -- hold no host synchronisation, memory fill or
allocation, so a serving loop can capture them in a HIP graph and replay it.
Every replay (with eager work and synchronisations between them) and an eager
step after the replays give the eager step's output bit for bit."""
import numpy as np
import pytest
import torch

import paged_kv_cache_varlen_amd as pa
import workloads as W
from tests.gpu_util import Uploaded, tensor_bits

pytestmark = pytest.mark.gpu


def make_step(w, u, fp8=None):
    ks, vs = (None, None) if fp8 is None else fp8
    scales = {} if fp8 is None else dict(k_scale=ks, v_scale=vs)

    def step():
        pa.write_kv_plan(u.k_new, u.v_new, u.new_slots, u.k_cache, u.v_cache, u.block_tables,
                         u.seq_lens, u.qsl, w.num_q_tokens, w.num_q_heads, w.max_query_len,
                         w.max_seq_len, u.workspace, k_scale=ks, v_scale=vs)
        pa.attend(u.q, u.k_cache, u.v_cache, u.block_tables, u.seq_lens, u.qsl, w.scale,
                  w.max_query_len, w.max_seq_len, num_kv_heads=w.num_kv_heads, out=u.out,
                  workspace=u.workspace, planned=True, merge=False, **scales)
        pa.attend_merge(u.out, w.num_seqs, w.num_kv_heads, w.max_query_len, w.max_seq_len,
                        u.workspace)
    return step


@pytest.mark.parametrize("k", [1, 2, 3])
def test_step_graph_replays_match_eager(k):
    w = W.make_config(k)
    print("config", k, flush=True)
    u = Uploaded(w, sentinel=False)
    step = make_step(w, u)
    step()
    torch.cuda.synchronize()
    ref = tensor_bits(u.out).copy()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.synchronize()
    for r in range(4):
        u.out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(tensor_bits(u.out), ref), "replay %d differs" % r
    u.out.fill_(float("nan"))
    step()
    torch.cuda.synchronize()
    assert np.array_equal(tensor_bits(u.out), ref), "eager step after the replays differs"


@pytest.mark.parametrize("Q", [[1, 1, 1, 1], [40, 3, 77, 9]])
def test_mla_graph_replays_match_eager(Q):
    # the MLA call (decode, then the split merge) in both forms: one token
    # per work item, and groups of tokens
    from tests.gpu_util import bf16_tensor, i32
    from tests.test_gpu_mla import gpu_cache
    from tests.test_oracle_mla import mla_batch
    m = mla_batch([900, 77, 2500, 300], Q, 16, seed=31)
    cache = gpu_cache(m)
    T, L = int(m["qsl"][-1]), m["L"]
    q = bf16_tensor(m["q"])
    out = torch.empty((T, 16, 512), dtype=torch.bfloat16, device="cuda")
    ws = pa.mla_workspace(T, 16, int(L.max()))
    args = (q, cache, i32(m["tables"]), i32(L), i32(m["qsl"]), 0.05, int(L.max()))

    def step():
        pa.mla_decode(*args, out=out, workspace=ws)
    step()
    torch.cuda.synchronize()
    ref = tensor_bits(out).copy()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.synchronize()
    for r in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(tensor_bits(out), ref), "replay %d differs" % r
