#!/usr/bin/env python3
"""Benchmark of one paged-attention layer step on one MI355X.

A step is the whole hot path for one layer over one batch: the scatter of
the step's new K/V rows and the work plan in one launch (pa_write_kv_plan),
then unified varlen paged attention and the split-K merge over every query
row.  Inputs are seeded synthetic tensors already resident in HBM.  Several
copies of the KV pool (one per simulated layer, >= 2 GiB in total) are
cycled so that no step reads K/V left in the caches by the previous one.

Prints one JSON line:
  value    paged-attention KV read GB/s of the headline workload (70B-class
           long-context decode layer: 16 requests x 32768 tokens, 64 q / 8 kv
           heads, head_dim 128, 16-token blocks, a 2.1 GB pool, plus the
           scatter of the step's 16 new tokens) = valid-token K+V bytes per
           step / mean step time; step_ms gives the median and p10/p90 of
           single steps (HIP events between steps);
  roofline the attention kernel against the 8 TB/s HBM peak, its duration
           from HIP events on the launch stream; also against this box's
           measured streaming-read ceiling (measured_ceiling);
  mixed_step  mixed chunked-prefill step (1920-token chunk on 1536 cached
           tokens + 128 decodes): tokens/s per layer;
  prefill_tile  that step's prefill chunk alone: attention TFLOP/s (visible
           query-key pairs x 4 x head_dim x q heads) against the bf16 MFMA
           peak;
  decode_part  that step's 128 decodes alone: attention kernel GB/s against
           the HBM peak;
  decode_8b  the Llama-3-8B decode layer (64 requests, U[128, 4096]) step
           and attention kernel;
  tiny_decode  the 4-request latency case (microseconds per step);
  fp8_kv   the 8-bit (E4M3) KV cache beside bf16 on the 8B decode layer and
           the 70B-class long-context layer: step time, decode tokens/s,
           attention GB/s of code bytes;
  shared_prefix  256 decodes sharing a 2048-token prefix: plain paged
           attention beside shared-prefix (cascade) attention, GB/s of the
           logical and of the unique K/V bytes;
  block_copy  copy-on-write block copies (4096 pairs) on the 8B layer's pool;
  mla_decode  MLA latent decode, 64 requests, 16 and 128 query heads;
  cpu_baseline  the CPU oracle (fp64) on a bounded sample of the headline
           workload, all host threads and one thread; per_config: the same
           for every synthetic configuration.

    python bench.py [--steps K] [--warmup W] [--config 5] [--no-mixed]
                    [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="5",
                    help="workload timed: 1-5, p for the mixed step's prefill "
                         "chunk alone, d for its 128 decodes alone")
    ap.add_argument("--no-mixed", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the streaming-read ceiling probe")
    ap.add_argument("--mla", action="store_true",
                    help="only the MLA latent decode sub-run (one JSON line)")
    ap.add_argument("--no-mla-chunks", action="store_true",
                    help="leave the MLA chunked-prefill batches out (profiles of "
                         "the decode workloads alone)")
    ap.add_argument("--fp8", action="store_true",
                    help="time the workload over 8-bit (E4M3) pools")
    ap.add_argument("--cascade", action="store_true",
                    help="time the workload's shared-prefix attention calls "
                         "(config 4: the 2048-token prefix attended once)")
    ap.add_argument("--min-working-set-gib", type=float, default=2.0)
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run 5 plain 1 GiB device-to-device copies (the "
                         "known-size reference for the HBM byte counters)")
    return ap.parse_args()


def copy_probe():
    """Five 1 GiB torch copies: each reads and writes exactly 2**30 bytes."""
    import torch
    src = torch.ones(2**30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_per_copy": 2**30, "copies": 5}))
    return 0


def kernel_source_hash() -> str:
    """sha256 (first 16 hex) of the attention kernel sources."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_cache_varlen_amd", "csrc")
    for f in ("attend.hip", "pa_device.h", "kv_cache.hip", "kv_scatter.h", "mfma_util.h"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (profiles/hbm_traffic.json), or None when the kernel sources changed
    since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256_16") != kernel_source_hash():
        return None
    k = t.get("kernels", {}).get("%s|%s" % (kernel, workload))
    if not k:
        return None
    return int(k["fetch_bytes"]) + int(k["write_bytes"])


def algorithmic(w):
    """Bytes and flops one attention launch needs at minimum."""
    L = w.seq_lens.astype(np.int64)
    Q = w.query_lens.astype(np.int64)
    kv = int(L.sum()) * 2 * w.num_kv_heads * w.head_dim * 2
    qo = 2 * w.num_q_tokens * w.num_q_heads * w.head_dim * 2
    tables = int(((L + 15) // 16).sum()) * 4
    meta = w.num_seqs * 4 + (w.num_seqs + 1) * 4
    # visible (query, key) pairs per head: query i of a chunk sees L-Q+i+1 keys
    pairs = int((Q * (L - Q) + Q * (Q + 1) // 2).sum())
    flops = 4 * w.head_dim * w.num_q_heads * pairs
    write = 2 * 2 * w.num_q_tokens * w.num_kv_heads * w.head_dim * 2  # read + write
    return {"kv_bytes": kv, "attend_bytes": kv + qo + tables + meta,
            "write_bytes": write, "flops": flops, "pairs_per_head": pairs}


class Runner:
    """Pools for several simulated layers plus the step's inputs, on the GPU."""

    def __init__(self, w, min_ws_gib, fp8=None, cascade=None):
        """fp8: None for bf16 pools, or (k_scale, v_scale) for 8-bit pools
        written by pa_write_kv_fp8.  cascade: None, or the shared prefix
        length for shared-prefix attention (plan, attention and merge of the
        shared-prefix calls)."""
        import torch
        import paged_kv_cache_varlen_amd as pa
        from tests.gpu_util import Uploaded, bf16_tensor, i64
        self.torch, self.pa, self.w, self.fp8 = torch, pa, w, fp8
        self.cascade = cascade
        base = Uploaded(w, sentinel=False)
        if cascade is not None:
            base.workspace = pa.alloc_workspace(
                w.num_seqs, w.num_q_tokens, w.num_q_heads, w.num_kv_heads, w.head_dim,
                w.max_query_len, w.max_seq_len, cascade=True)
        if fp8 is not None:
            k8, v8 = pa.alloc_pool_fp8(w.num_blocks, w.num_kv_heads, w.head_dim, fill=0)
            step = 1 << 18  # bounded host->device staging
            for s0 in range(0, len(w.fill_rows), step):
                rows = w.fill_rows[s0:s0 + step]
                pa.write_kv_fp8(bf16_tensor(w.k_dense[rows]), bf16_tensor(w.v_dense[rows]),
                                i64(w.fill_slots[s0:s0 + step]), k8, v8, *fp8)
            pa.write_kv_fp8(base.k_new, base.v_new, base.new_slots, k8, v8, *fp8)
            base.k_cache, base.v_cache = k8, v8
        pool_bytes = 2 * base.k_cache.numel() * base.k_cache.element_size()
        n = max(1, min(8, int(np.ceil(min_ws_gib * 2**30 / pool_bytes))))
        self.layers = [(base.k_cache, base.v_cache)]
        for _ in range(n - 1):
            self.layers.append((base.k_cache.clone(), base.v_cache.clone()))
        self.u = base
        self.stream = torch.cuda.current_stream()
        self._prepare_calls()

    def _prepare_calls(self):
        """Each layer pool's step as C-ABI calls with their arguments built
        once: the timed loop pays the calls only.  (The binding's checks and
        marshalling are host work a serving loop does once per step, not per
        layer; on a slow host they took as long as the decode step's kernels
        and made the step host-bound.)  Checked once against the binding's
        path, bit for bit."""
        from paged_kv_cache_varlen_amd import _lib
        lib = _lib.load()
        w, u = self.w, self.u
        fp8, casc = self.fp8 is not None, self.cascade is not None
        ks, vs = self.fp8 if fp8 else (1.0, 1.0)
        p = lambda t: t.data_ptr()
        nb, st = int(w.num_blocks), self.stream.cuda_stream
        meta = [p(u.block_tables), int(u.block_tables.shape[1]), p(u.seq_lens), p(u.qsl),
                int(w.num_seqs), int(w.num_q_tokens), int(w.num_q_heads),
                int(w.num_kv_heads), int(w.head_dim), int(w.max_query_len),
                int(w.max_seq_len)]
        ws = [p(u.workspace), int(u.workspace.numel()), st]
        scales = [float(ks), float(vs)] if fp8 else []
        scatter = [p(u.k_new), p(u.v_new), int(u.k_new.stride(0)), int(u.v_new.stride(0)),
                   p(u.new_slots), int(u.k_new.shape[0])] + scales
        sfx = ("_cascade" if casc else "") + ("_fp8" if fp8 else "")
        wp_fn = lib.pa_write_kv_plan_fp8 if fp8 else lib.pa_write_kv_plan
        att_fn = getattr(lib, "pa_attend_planned" + sfx)
        self.calls = []
        for kc, vc in self.layers:
            calls = [(wp_fn, tuple(scatter + [p(kc), p(vc), nb] + meta +
                                   [int(self.cascade) if casc else -1] + ws)),
                     (att_fn, tuple([p(u.q), p(kc), p(vc), nb] + meta + [float(w.scale)] +
                                    scales + [p(u.out)] + ws))]
            merge_fn = lib.pa_attend_merge_cascade if casc else lib.pa_attend_merge
            calls.append((merge_fn, tuple(meta[4:] + [p(u.out)] + ws)))
            self.calls.append(calls)
        # one step through the binding, one through the prepared calls
        torch = self.torch
        self.step_checked(0)
        ref = u.out.clone()
        u.out.fill_(float("nan"))
        self.step(0)
        torch.cuda.synchronize()
        assert torch.equal(ref.view(torch.int16), u.out.view(torch.int16)), \
            "prepared calls differ from the binding's"

    def step_checked(self, i):
        """write_kv + plan + attention (+ merge) through the binding."""
        w, u = self.w, self.u
        kc, vc = self.layers[i % len(self.layers)]
        ks, vs = (None, None) if self.fp8 is None else self.fp8
        self.pa.write_kv_plan(u.k_new, u.v_new, u.new_slots, kc, vc, u.block_tables,
                              u.seq_lens, u.qsl, w.num_q_tokens, w.num_q_heads,
                              w.max_query_len, w.max_seq_len, u.workspace,
                              common_prefix_len=self.cascade, k_scale=ks, v_scale=vs)
        self.attend(kc, vc)
        self.merge()

    def attend(self, kc, vc):
        w, u = self.w, self.u
        scales = {} if self.fp8 is None else dict(k_scale=self.fp8[0], v_scale=self.fp8[1])
        self.pa.attend(u.q, kc, vc, u.block_tables, u.seq_lens, u.qsl, w.scale,
                       w.max_query_len, w.max_seq_len, num_kv_heads=w.num_kv_heads,
                       out=u.out, workspace=u.workspace, planned=True, merge=False,
                       common_prefix_len=self.cascade, **scales)

    def plan(self):
        w, u = self.w, self.u
        self.pa.attend_plan(u.block_tables, u.seq_lens, u.qsl, w.num_q_tokens,
                            w.num_q_heads, w.num_kv_heads, w.head_dim, w.max_query_len,
                            w.max_seq_len, u.workspace, common_prefix_len=self.cascade,
                            fp8=self.fp8 is not None)

    def merge(self):
        w, u = self.w, self.u
        self.pa.attend_merge(u.out, w.num_seqs, w.num_kv_heads, w.max_query_len,
                             w.max_seq_len, u.workspace, cascade=self.cascade is not None)

    def step(self, i):
        """write_kv + plan (one fused launch) + attention + merge for one
        layer, as the prepared C-ABI calls."""
        for fn, args in self.calls[i % len(self.calls)]:
            st = fn(*args)
            if st != 0:
                raise RuntimeError("%s: %s" % (fn.__name__, self.pa._lib.load().pa_last_error()))

    def graph_run(self, steps):
        """Layer 0's step (scatter + plan, attention, merge) captured once as a
        HIP graph (through the binding, on a capture stream) and replayed
        `steps` times back to back: mean ms per replay.  A replay's output is
        checked once against the eager step, bit for bit."""
        torch = self.torch
        self.step_checked(0)
        torch.cuda.synchronize()
        ref = self.u.out.clone()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            self.step_checked(0)
        torch.cuda.synchronize()
        self.u.out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ref.view(torch.int16), self.u.out.view(torch.int16)), \
            "graph replay differs from the eager step"
        for _ in range(10):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            g.replay()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps

    def run(self, steps, warmup):
        """Time `steps` whole steps (nothing but the step's own launches
        between the synchronisations): their mean; then `steps` single steps
        with a HIP event recorded between consecutive steps (median, p10,
        p90); then the attention kernel's launch duration: HIP events on the
        launch stream around runs of back-to-back launches, one per layer
        pool, on one plan (as a forward pass runs the layers).  An event
        record costs a few µs of dispatch gap, so the mean step comes from
        the event-free loop and the kernel's from runs of launches."""
        torch = self.torch
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(i)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record(self.stream)
        for i in range(steps):
            self.step(i)
            ev[i + 1].record(self.stream)
        torch.cuda.synchronize()
        single = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])
        n = len(self.layers)
        runs = max(5, steps // n)
        evs = [(torch.cuda.Event(enable_timing=True),
                torch.cuda.Event(enable_timing=True)) for _ in range(runs)]
        self.plan()
        for r in range(runs):
            evs[r][0].record(self.stream)
            for calls in self.calls:
                fn, args = calls[1]  # the attention kernel alone
                if fn(*args) != 0:
                    raise RuntimeError(self.pa._lib.load().pa_last_error())
            evs[r][1].record(self.stream)
        torch.cuda.synchronize()
        per_launch = np.array([a.elapsed_time(b) for a, b in evs]) / n
        return {"ms_per_step": (t1 - t0) * 1e3 / steps, "step_ms": percentiles(single),
                "attend_ms": float(per_launch.mean()), "attend_pct": percentiles(per_launch)}


def percentiles(x):
    """Median, p10 and p90 of a sample of durations (ms), and its size."""
    x = np.asarray(x, np.float64)
    return {"median": round(float(np.median(x)), 5), "p10": round(float(np.percentile(x, 10)), 5),
            "p90": round(float(np.percentile(x, 90)), 5), "n": int(x.size)}


def host_description():
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    cpu = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    return {"cpu": cpu, "os_cpu_count": os.cpu_count(), "affinity": affinity}


def oracle_sample(w, nthreads, min_s, max_s, seed=0):
    """The CPU oracle (fp64 C, OpenMP over rows) on workload w's own pools,
    over (query token, head) output rows in a seeded random order, in batches
    of 16 rows per thread, until at least min_s (at most max_s) of oracle
    time.  Returns the rows done, the time, and the visible query-key pairs
    and K/V bytes they stand for (a row of a query at position p reads p + 1
    keys; its share of the K/V bytes is (p + 1) * 2 * head_dim * 2 / G, the
    kv head's tokens being read once for its G query heads)."""
    import oracle
    kc = np.zeros(w.pool_elems(), np.uint16)
    vc = np.zeros(w.pool_elems(), np.uint16)
    oracle.write_kv(kc, vc, w.k_dense[w.fill_rows], w.v_dense[w.fill_rows], w.fill_slots)
    oracle.write_kv(kc, vc, w.k_new, w.v_new, w.new_slots)
    T, Hq = w.num_q_tokens, w.num_q_heads
    G = Hq // w.num_kv_heads
    qsl = w.query_start_loc.astype(np.int64)
    seq = np.searchsorted(qsl, np.arange(T), side="right") - 1
    pos = (w.seq_lens[seq].astype(np.int64) - (qsl[seq + 1] - qsl[seq]) +
           (np.arange(T) - qsl[seq]))
    order = np.random.default_rng(seed).permutation(T * Hq)
    batch = min(16 * nthreads, order.size)
    done, spent, pairs = 0, 0.0, 0
    while spent < min_s:
        # (a workload with fewer rows than the time bound needs is passed
        # over again, in the same order)
        idx = np.take(order, np.arange(done, done + batch), mode="wrap")
        rows = np.stack([idx // Hq, idx % Hq], axis=1).astype(np.int64)
        t0 = time.perf_counter()
        oracle.attend_rows(w.q, kc, vc, w.block_tables, w.seq_lens, w.query_start_loc,
                           w.num_kv_heads, w.scale, rows, nthreads=nthreads)
        spent += time.perf_counter() - t0
        done += idx.size
        pairs += int((pos[idx // Hq] + 1).sum())
        if spent >= max_s:
            break
    kv_bytes = pairs * 2 * w.head_dim * 2 / G
    return {"rows": done, "seconds": spent, "pairs": pairs, "kv_bytes": kv_bytes}


def cpu_baseline(w, min_s=10.0, max_s=30.0, min_s1=3.0, max_s1=8.0):
    """The oracle on a bounded sample of the headline workload, all host
    threads and then one thread, scaled to KV GB/s (the value's unit)."""
    import oracle
    threads = oracle.default_threads()
    allt = oracle_sample(w, threads, min_s, max_s)
    one = oracle_sample(w, 1, min_s1, max_s1, seed=1)
    total_rows = w.num_q_tokens * w.num_q_heads
    return dict({"value": round(allt["kv_bytes"] / allt["seconds"] / 1e9, 4), "unit": "GB/s",
                 "cores": threads, "kind": "oracle",
                 "value_1_thread": round(one["kv_bytes"] / one["seconds"] / 1e9, 4),
                 "sample": "%d (query token, head) output rows (%.2f passes over the %d "
                           "rows of the headline workload, in a seeded random order), "
                           "fp64 C oracle with OpenMP over rows, %d threads, %.1f s; one "
                           "thread: %d rows, %.1f s" % (allt["rows"], allt["rows"] / total_rows,
                                                        total_rows, threads, allt["seconds"],
                                                        one["rows"], one["seconds"])},
                **host_description())


def cpu_per_config(workloads, min_s=1.0, max_s=6.0, min_s1=1.0, max_s1=4.0):
    """The oracle on every synthetic configuration: KV GB/s and visible
    query-key pairs per second with all host threads and with one thread,
    on bounded row samples, and the time the whole configuration would take
    at those rates."""
    import oracle
    threads = oracle.default_threads()
    out = {}
    for k, w in workloads:
        G = w.num_q_heads // w.num_kv_heads
        alg = algorithmic(w)
        total_pairs = alg["pairs_per_head"] * w.num_q_heads
        res = {"workload": w.name, "threads": threads}
        for key, n, lo, hi in (("all_threads", threads, min_s, max_s), ("one_thread", 1, min_s1, max_s1)):
            r = oracle_sample(w, n, lo, hi, seed=k)
            rate = r["pairs"] / r["seconds"]
            res[key] = {"kv_gbs": round(r["kv_bytes"] / r["seconds"] / 1e9, 4),
                        "pairs_per_s": round(rate, 1), "rows": r["rows"],
                        "seconds": round(r["seconds"], 2),
                        "full_config_s": round(total_pairs / rate, 2)}
        res["kv_bytes_per_pair"] = round(2 * w.head_dim * 2 / G, 2)
        out[str(k)] = res
    return out


FP8_SCALES = (0.011, 0.0107)  # amax / 448 for N(0,1) bf16 data

_WORKLOADS = {}


def config(W, k):
    """Synthetic configuration k (1-5; "p": the mixed step's prefill chunk
    alone, "d": its 128 decodes alone), built once per run."""
    k = str(k)
    if k not in _WORKLOADS:
        _WORKLOADS[k] = (W.make_prefill_chunk() if k == "p" else
                         W.make_decode_part() if k == "d" else W.make_config(int(k)))
    return _WORKLOADS[k]


def fp8_runs(args, W):
    """8-bit (E4M3) KV cache on the headline decode layer and the 70B-class
    long-context layer: the step's tokens/s and the attention kernel's GB/s of
    code bytes, beside the same workload on bf16 pools."""
    import torch
    out = {"scales": list(FP8_SCALES), "format": "OCP E4M3, one fp32 scale per pool"}
    for key, w in (("decode_8b", config(W, 2)), ("decode_70b_32k", config(W, 5))):
        alg = algorithmic(w)
        res = {"workload": w.name}
        for kind, fp8 in (("bf16", None), ("fp8", FP8_SCALES)):
            r = Runner(w, args.min_working_set_gib, fp8=fp8)
            t = r.run(max(20, args.steps // 4), max(5, args.warmup // 2))
            ms, att = t["ms_per_step"], t["attend_ms"]
            kv = alg["kv_bytes"] / (2 if fp8 else 1)
            res[kind] = {"ms_per_step": round(ms, 5), "step_ms": t["step_ms"],
                         "attend_ms": round(att, 5),
                         "decode_tokens_per_s": round(w.num_q_tokens / (ms * 1e-3), 1),
                         "attend_kv_gbs": round(kv / (att * 1e-3) / 1e9, 2),
                         "hbm_peak_frac": round(kv / (att * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
            del r
            torch.cuda.empty_cache()
        res["step_speedup"] = round(res["bf16"]["ms_per_step"] / res["fp8"]["ms_per_step"], 3)
        out[key] = res
    return out


def unique_kv_bytes(w):
    """K+V bytes of the distinct tokens a shared-prefix batch holds: the
    prefix once, then every request's own tokens."""
    C = int(w.shared_prefix)
    toks = C + int((w.seq_lens.astype(np.int64) - C).sum())
    return toks * 2 * w.num_kv_heads * w.head_dim * 2


def shared_prefix_runs(args, W):
    """The shared-prefix decode layer (256 requests, 2048-token prefix): plain
    paged attention and shared-prefix attention, whole step and attention
    kernel, with the attention's GB/s of logical (per request) and unique
    K/V bytes."""
    import torch
    w = config(W, 4)
    alg = algorithmic(w)
    uniq = unique_kv_bytes(w)
    out = {"workload": w.name, "prefix_tokens": int(w.shared_prefix),
           "logical_kv_bytes": alg["kv_bytes"], "unique_kv_bytes": uniq}
    for kind, casc in (("plain", None), ("cascade", int(w.shared_prefix))):
        r = Runner(w, args.min_working_set_gib, cascade=casc)
        t = r.run(max(20, args.steps // 4), max(5, args.warmup // 2))
        ms, att = t["ms_per_step"], t["attend_ms"]
        out[kind] = {"ms_per_step": round(ms, 5), "step_ms": t["step_ms"],
                     "attend_ms": round(att, 5),
                     "decode_tokens_per_s": round(w.num_q_tokens / (ms * 1e-3), 1),
                     "attend_logical_gbs": round(alg["kv_bytes"] / (att * 1e-3) / 1e9, 2),
                     "attend_unique_gbs": round(uniq / (att * 1e-3) / 1e9, 2)}
        del r
        torch.cuda.empty_cache()
    out["step_speedup"] = round(out["plain"]["ms_per_step"] / out["cascade"]["ms_per_step"], 3)
    return out


def block_copy_run(W):
    """Copy-on-write block copies on the 8B decode layer's pool: 4096 random
    (src, dst) pairs, every kv head of both pools; GB/s of bytes read plus
    written."""
    import torch
    import paged_kv_cache_varlen_amd as pa
    w = config(W, 2)
    kc, vc = pa.alloc_pool(w.num_blocks, w.num_kv_heads, w.head_dim, fill=0.0)
    rng = np.random.default_rng(7)
    ids = rng.permutation(w.num_blocks)[:8192]
    mapping = torch.from_numpy(ids.reshape(2, 4096).T.copy().astype(np.int64)).cuda()
    n = 20
    for _ in range(3):
        pa.copy_blocks(kc, vc, mapping, w.num_kv_heads, w.head_dim)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(n):
        pa.copy_blocks(kc, vc, mapping, w.num_kv_heads, w.head_dim)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / n
    moved = 4096 * 2 * 2 * w.num_kv_heads * 16 * w.head_dim * 2
    # the same bytes as one contiguous device-to-device copy (torch's copy
    # kernel, timed the same way): what read-plus-write traffic reaches on
    # this device, the bound of any copy
    src = torch.empty(moved // 4, dtype=torch.int16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    a.record()
    for _ in range(n):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms_c = a.elapsed_time(b) / n
    gbs, gbs_c = moved / (ms * 1e-3) / 1e9, moved / (ms_c * 1e-3) / 1e9
    return {"pairs": 4096, "block_bytes_per_pool": w.num_kv_heads * 16 * w.head_dim * 2,
            "ms": round(ms, 5), "gbs": round(gbs, 1),
            "hbm_peak_frac": round(gbs / HBM_PEAK_GBS, 4),
            "contiguous_copy": {"ms": round(ms_c, 5), "gbs": round(gbs_c, 1),
                                "hbm_peak_frac": round(gbs_c / HBM_PEAK_GBS, 4)},
            "frac_of_contiguous_copy": round(gbs / gbs_c, 4)}


def mla_case(name, L, Hq, seed):
    """One MLA decode step: requests of lengths L, one query token each, Hq
    heads, a latent cache of 64-token blocks in a seeded random order."""
    rng = np.random.default_rng(seed)
    L = np.asarray(L, np.int32)
    nblk = (L + 63) // 64
    nb = int(nblk.sum() * 1.1) + 1
    perm = rng.permutation(nb)
    tables = np.full((len(L), int(nblk.max())), -1, np.int32)
    pos = 0
    for b, n in enumerate(nblk):
        tables[b, :n] = perm[pos:pos + n]
        pos += int(n)
    return dict(name=name, L=L, Hq=Hq, nb=nb, tables=tables,
                qsl=np.arange(len(L) + 1, dtype=np.int32))


def _mla_time(pa, torch, c, L, qsl, Hq, ncopies, reps):
    """Mean ms of one pa_mla_decode launch (decode + merge) for case c with
    query_start_loc qsl, over back-to-back launches on ncopies cache copies;
    the C-ABI call's arguments are prepared once (the binding's per-call
    checks cost host time comparable to the kernels) and checked once against
    the binding's path bit for bit."""
    from tests.gpu_util import i32
    from paged_kv_cache_varlen_amd import _lib
    T = int(qsl[-1])
    maxL = int(np.max(L))
    caches = [pa.alloc_mla_cache(c["nb"], fill=0.0) for _ in range(ncopies)]
    for cc in caches:
        cc.normal_()
    q = torch.randn((T, Hq, 576), device="cuda").to(torch.bfloat16)
    o = torch.empty((T, Hq, 512), dtype=torch.bfloat16, device="cuda")
    ws = pa.mla_workspace(T, Hq, maxL)
    bt, sl, qs = i32(c["tables"]), i32(np.asarray(L, np.int32)), i32(np.asarray(qsl, np.int32))
    scale = float(1 / np.sqrt(192.0))
    fn = _lib.load().pa_mla_decode
    stream = torch.cuda.current_stream().cuda_stream
    prepared = [(q.data_ptr(), cc.data_ptr(), c["nb"], bt.data_ptr(), int(bt.shape[1]),
                 sl.data_ptr(), qs.data_ptr(), len(L), T, Hq, maxL, scale,
                 o.data_ptr(), ws.data_ptr(), ws.numel(), stream) for cc in caches]

    def run(i):
        if fn(*prepared[i % ncopies]) != 0:
            raise RuntimeError(_lib.load().pa_last_error())
    pa.mla_decode(q, caches[0], bt, sl, qs, scale, maxL, out=o, workspace=ws)
    ref = o.clone()
    o.fill_(float("nan"))
    run(0)
    torch.cuda.synchronize()
    assert torch.equal(ref.view(torch.int16), o.view(torch.int16)), \
        "prepared MLA call differs from the binding's"
    for i in range(3 * ncopies):
        run(i)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        for i in range(ncopies):
            run(i)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / (reps * ncopies)
    del caches
    torch.cuda.empty_cache()
    return ms


# chunked prefill through the latent path: (name, cached + new tokens per
# request, new tokens per request, query heads)
MLA_CHUNKS = (("mla-prefill-chunk-1024-on-1024-h16", [2048], [1024], 16),
              ("mla-prefill-chunk-1024-on-1024-h128", [2048], [1024], 128),
              ("mla-prefill-8x512-on-3584-h16", [4096] * 8, [512] * 8, 16))


def mla_runs(args):
    """MLA latent decode (DeepSeek-V3-shaped: 576 cached values per token,
    512 latent dims out) on 64 requests of U[128, 4096] tokens: 16 query
    heads (one tensor-parallel share of 128) and all 128 heads.  Attention
    kernels (decode + merge) timed with HIP events over back-to-back
    launches on cycled cache copies; GB/s of the latent bytes the step must
    read and TFLOP/s of the scores and weighted sums.  Then chunked-prefill
    batches through the same call (TFLOP/s)."""
    import torch
    import paged_kv_cache_varlen_amd as pa
    rng = np.random.default_rng(2024)
    L = rng.integers(128, 4096, size=64, endpoint=True).astype(np.int32)
    out = {"latent_dims": 576, "out_dims": 512, "block_size": 64}
    for key, Hq in (("h16", 16), ("h128", 128)):
        c = mla_case("deepseek-v3-mla-decode-64seq-%s" % key, L, Hq, seed=7)
        T = len(L)
        cache_bytes = c["nb"] * 64 * 576 * 2
        ncopies = max(1, min(8, int(np.ceil(args.min_working_set_gib * 2**30 / cache_bytes))))
        reps = max(4, args.steps // (4 * ncopies))
        ms = _mla_time(pa, torch, c, L, c["qsl"], Hq, ncopies, reps)
        lat = int(L.sum()) * 576 * 2
        byts = lat + T * Hq * (576 + 512) * 2 + int(((L + 63) // 64).sum()) * 4
        flops = int(L.sum()) * Hq * (576 + 512) * 2
        out[key] = {"workload": c["name"], "num_q_heads": Hq, "ms": round(ms, 5),
                    "latent_gbs": round(lat / (ms * 1e-3) / 1e9, 1),
                    "algorithmic_gbs": round(byts / (ms * 1e-3) / 1e9, 1),
                    "hbm_peak_frac": round(byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
                    "mfma_peak_frac": round(flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                    "decode_tokens_per_s": round(T / (ms * 1e-3), 1)}
    if getattr(args, "no_mla_chunks", False):
        return out
    chunks = {}
    for name, Lc, Qc, Hq in MLA_CHUNKS:
        c = mla_case(name, Lc, Hq, seed=3)
        qsl = np.concatenate([[0], np.cumsum(Qc)]).astype(np.int32)
        ms = _mla_time(pa, torch, c, Lc, qsl, Hq, 1, 10)
        keys = sum(l - qq + 1 + i for l, qq in zip(Lc, Qc) for i in range(qq))
        flops = keys * Hq * (576 + 512) * 2
        chunks[name] = {"num_q_heads": Hq, "query_tokens": int(qsl[-1]), "ms": round(ms, 5),
                        "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
                        "mfma_peak_frac": round(flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
    out["prefill_chunks"] = chunks
    return out


def read_ceiling(torch, gib=4):
    """Measured streaming-read ceiling of this box: the best of a few grid
    sizes of the probe kernel (libpa_probe.so) reading a 4 GiB buffer once
    with 16-byte non-temporal loads; GB/s."""
    import ctypes
    path = os.path.join(ROOT, "paged_kv_cache_varlen_amd", "libpa_probe.so")
    lib = ctypes.CDLL(path)
    lib.pa_probe_stream_read.restype = ctypes.c_int
    lib.pa_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                         ctypes.c_int, ctypes.c_void_p]
    nbytes = gib << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    best = 0.0
    for per_cu in (8, 16, 32):
        def launch():
            rc = lib.pa_probe_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(),
                                          cus * per_cu, stream.cuda_stream)
            assert rc == 0, rc
        for _ in range(2):
            launch()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(5):
            launch()
        b.record(stream)
        torch.cuda.synchronize()
        best = max(best, 5 * nbytes / (a.elapsed_time(b) * 1e-3) / 1e9)
    del buf, sink
    torch.cuda.empty_cache()
    return best


def decode_kernel_name(w, fp8, cascade):
    """The attention kernel a launch over workload w runs (as the trace names it)."""
    G = w.num_q_heads // w.num_kv_heads
    decode = cascade is None and w.max_query_len <= 16 // G
    return ("attend_decode_kernel<%d, %s>" if decode else "attend_mixed_kernel<%d, %s>") % (
        w.head_dim, "true" if fp8 else "false")


def sub_run(args, w, graph=False, **kw):
    """A workload's step and attention kernel, with the kernel's GB/s and
    TFLOP/s of algorithmic bytes and flops; graph: also the step replayed as
    a captured HIP graph (t["graph_ms_per_step"])."""
    import torch
    alg = algorithmic(w)
    r = Runner(w, args.min_working_set_gib, **kw)
    t = r.run(max(20, args.steps // 4), max(5, args.warmup // 2))
    if graph:
        t["graph_ms_per_step"] = r.graph_run(max(50, args.steps))
    del r
    torch.cuda.empty_cache()
    att = t["attend_ms"] * 1e-3
    gbs = alg["attend_bytes"] / att / 1e9
    return alg, t, {"workload": w.name, "ms_per_step": round(t["ms_per_step"], 5),
                    "step_ms": t["step_ms"], "attend_ms": round(t["attend_ms"], 5),
                    "attend_pct": t["attend_pct"], "attend_gbs": round(gbs, 2),
                    "hbm_peak_frac": round(gbs / HBM_PEAK_GBS, 4),
                    "attend_tflops": round(alg["flops"] / att / 1e12, 2)}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the paged-attention path here is a "
              "single-GPU kernel (no multi-GPU sharding is built); use --gpus 1",
              file=sys.stderr)
        return 2
    import torch
    import workloads as W
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_probe:
        return copy_probe()
    if args.mla:
        print(json.dumps({"mla_decode": mla_runs(args)}))
        return 0

    w = config(W, args.config)
    alg = algorithmic(w)
    casc = int(w.shared_prefix) if args.cascade else None
    if args.cascade and not casc:
        print("--cascade needs a workload with a shared prefix (config 4)", file=sys.stderr)
        return 2
    r = Runner(w, args.min_working_set_gib, fp8=FP8_SCALES if args.fp8 else None,
               cascade=casc)
    t = r.run(args.steps, args.warmup)
    ms_step, attend_ms = t["ms_per_step"], t["attend_ms"]
    kernel = decode_kernel_name(w, args.fp8, casc)
    if casc:
        # shared-prefix attention reads the prefix once: its algorithmic
        # bytes are the distinct tokens' K/V (plus the same q, out, metadata)
        alg["attend_bytes"] += unique_kv_bytes(w) - alg["kv_bytes"]
    if args.fp8:
        # 8-bit pools: one byte per K or V element
        alg["attend_bytes"] -= alg["kv_bytes"] // 2
        alg["kv_bytes"] //= 2
    # the line's value: the K/V bytes the step reads (8-bit codes with --fp8)
    kv_gbs = alg["kv_bytes"] / (ms_step * 1e-3) / 1e9
    achieved = alg["attend_bytes"] / (attend_ms * 1e-3) / 1e9
    line = {
        "metric": "paged-attn KV read GB/s (% HBM peak) + mixed-step tokens/s per layer",
        "value": round(kv_gbs, 2),
        "unit": "GB/s",
        "hbm_peak_frac": round(kv_gbs / HBM_PEAK_GBS, 4),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "step_ms": t["step_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3 K/V codes, bf16 q/out" if args.fp8 else "bf16",
        "data": "synthetic (seeded N(0,1) bf16 q/K/V, seeded block tables)",
        "config": dict(W.Workload.describe(w), layers_cycled=len(r.layers),
                       **({"shared_prefix_attention": casc} if casc else {})),
        "decode_tokens_per_s": round(w.num_q_tokens / (ms_step * 1e-3), 1),
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(kernel, w.name + (" shared-prefix" if casc else "")
                                        + (" fp8" if args.fp8 else "")),
            "kernel": kernel,
            "attend_ms": round(attend_ms, 5),
            "attend_pct": t["attend_pct"],
            "algorithmic_bytes": alg["attend_bytes"]},
    }
    if args.config != "p" and not args.no_ceiling:
        ceil = read_ceiling(torch)
        line["roofline"]["measured_ceiling"] = {
            "gbs": round(ceil, 1), "frac": round(achieved / ceil, 4),
            "probe": "one pass over 4 GiB with 16-byte non-temporal loads, best of "
                     "8/16/32 workgroups per CU (libpa_probe.so)"}
    if args.config == "p":
        # the prefill chunk alone is a dense contraction: priced against MFMA
        tflops = alg["flops"] / (attend_ms * 1e-3) / 1e12
        line["roofline"].update({
            "bound": "mfma", "achieved": round(tflops, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "algorithmic_flops": alg["flops"]})
    del r
    torch.cuda.empty_cache()

    if not args.no_mixed and args.config not in ("3", "p", "d"):
        w3 = config(W, 3)
        a3, t3, res = sub_run(args, w3)
        res["tokens_per_s_per_layer"] = round(w3.num_q_tokens / (t3["ms_per_step"] * 1e-3), 1)
        res["kv_read_gbs"] = round(a3["kv_bytes"] / (t3["ms_per_step"] * 1e-3) / 1e9, 2)
        res["traffic"] = measured_traffic(decode_kernel_name(w3, False, None), w3.name)
        line["mixed_step"] = res
        ap, tp, res = sub_run(args, config(W, "p"))
        tflops = ap["flops"] / (tp["attend_ms"] * 1e-3) / 1e12
        line["prefill_tile"] = {
            "workload": res["workload"], "attend_ms": res["attend_ms"],
            "attend_pct": res["attend_pct"], "flops": ap["flops"], "tflops": round(tflops, 2),
            "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
            "mfma_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)}
        _, _, res = sub_run(args, config(W, "d"))
        line["decode_part"] = res
        if args.config != "2":
            w2 = config(W, 2)
            a2, t2, res = sub_run(args, w2)
            res["decode_tokens_per_s"] = round(w2.num_q_tokens / (t2["ms_per_step"] * 1e-3), 1)
            res["kv_read_gbs"] = round(a2["kv_bytes"] / (t2["ms_per_step"] * 1e-3) / 1e9, 2)
            res["traffic"] = measured_traffic(decode_kernel_name(w2, False, None), w2.name)
            line["decode_8b"] = res
        if args.config != "1":
            _, t1, res = sub_run(args, config(W, 1))
            line["tiny_decode"] = {"workload": res["workload"],
                                   "us_per_step": round(t1["ms_per_step"] * 1e3, 2),
                                   "step_us": {k: (round(v * 1e3, 2) if k != "n" else v)
                                               for k, v in t1["step_ms"].items()},
                                   "attend_us": round(t1["attend_ms"] * 1e3, 2)}
        line["fp8_kv"] = fp8_runs(args, W)
        line["shared_prefix"] = shared_prefix_runs(args, W)
        line["block_copy"] = block_copy_run(W)
        line["mla_decode"] = mla_runs(args)

    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w)
        if not args.no_mixed:
            line["cpu_baseline"]["per_config"] = cpu_per_config(
                [(k, config(W, k)) for k in (1, 2, 3, 4, 5)])
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
