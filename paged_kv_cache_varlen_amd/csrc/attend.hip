// Paged varlen causal attention over a mixed batch (chunked-prefill chunks and
// decodes in one launch), gfx950.
//
// What is computed ("vLLM v1 Deep Dive", Part 3, Step 4c and the Aside "KV cache and
// prefix caching"; "vLLM: An Exhaustive Technical Study" sections 2.1 and 2.4): for every
// query token of request b (its Q_b new tokens are the last Q_b of its L_b
// tokens, rows query_start_loc[b]..) and every query head h,
//     out = softmax_j(scale * q.K_j) V_j  over keys j = 0 .. p,  p = L_b - Q_b + i,
// K_j/V_j read from block block_tables[b][j/16], slot j%16, of the kv head
// h / G shared by the G query heads of its group.
//
// Three kernels on one stream, no host synchronisation:
//   plan    one workgroup turns seq_lens / query_start_loc into a work list of
//           (request, query tile, logical key range) items, prefill items
//           first, plus the list of tiles whose key range was split, and
//           zeroes the work-queue head;
//   attend  persistent waves pull (item, kv head) units from the queue.  One
//           wave owns one unit.  The query tile's columns (token x head of
//           the group) are MFMA columns and the 16 keys of a block are MFMA
//           rows, so each K/V tile is read once for all G heads of the group.
//           Scores S^T = K Q^T run on v_mfma_f32_16x16x32_bf16; the online
//           softmax (running max and sum per column) is fp32, reduced across
//           the wave with shuffles; O^T = V^T P^T runs on bf16 MFMA with P
//           taken straight from the score registers.  Units covering a whole
//           causal range write bf16 out; split units write fp32 partials;
//   merge   one wave per (split tile, kv head) combines the partials by
//           log-sum-exp in split order into bf16 out.  (A separate launch:
//           the kernel boundary is what makes partials written on one XCD's
//           L2 visible on another, without device-wide cache flushes.)
//
// Reduction order depends only on (Q_b, L_b), logical key positions and,
// for decode requests of more than 8192 keys, the split length the plan
// chose for the batch's long requests, so results are bitwise independent
// of physical block ids, of shared blocks and of which wave ran which unit,
// and a request of at most 8192 keys (or any prefill chunk) also of the
// rest of the batch.
//
// The kernel template has two instantiations: a decode-only one (batches whose
// max_query_len fits a decode tile; fewer registers, more resident waves) and
// the unified one that serves decode and prefill items of a mixed batch in the
// same launch.
#include <mutex>
#include <type_traits>
#include <utility>
#include <vector>

#include "kv_scatter.h"
#include "mfma_util.h"
#include "pa_device.h"

namespace pa {

namespace {

// block buffers of the decode pipeline (blocks in flight + 1)
constexpr int kDecodeStages = 3;
// In a mixed batch, the first kPrefillWgNum / kPrefillWgDen of the
// workgroups start on prefill tiles and the others on decode units.
constexpr uint32_t kPrefillWgNum = 3;
constexpr uint32_t kPrefillWgDen = 8;
// With shared-prefix units in the queue: kPrefixWgNum / kPrefixWgDen.
constexpr uint32_t kPrefixWgNum = 1;
constexpr uint32_t kPrefixWgDen = 8;

struct AttendParams {
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  int64_t num_blocks;
  const int32_t* bt;
  int32_t bt_stride;
  const int32_t* seq_lens;
  const int32_t* qsl;
  int32_t num_seqs;
  int32_t num_q_tokens;
  int32_t Hq;
  int32_t Hkv;
  int32_t G;
  int32_t max_query_len;
  int32_t max_seq_len;
  float scale_log2;  // scale * k_scale * log2(e): scores live in the exp2 domain
  float v_scale;     // 8-bit pools: the value of a V code is code * v_scale
  uint16_t* out;
  PlanHeader* hdr;
  uint32_t* dec_counters;  // kDecodeShards decode queue heads
  WorkItem* items;
  int4* merge_list;  // per split tile: tok0, ntok, nsplit, pbase
  float2* part_ml;
  float* part_acc;
  int64_t max_items;
  int64_t max_partials;
  // shared-prefix section (null / 0 unless the workspace holds one)
  WorkItem* pitems;
  float2* pre_ml;
  float* pre_acc;
  int64_t max_pre_items;
  int64_t max_pre_partials;
  int32_t prefix_len;  // plan: keys every request shares (0: none)
  int32_t split_decode;  // plan: key range of a decode split (requests <= kLongDecode)
  int32_t long_units;    // plan: decode units wanted (per CU: kLongUnitsPerCu, 8-bit kUnitsPerCu8)
  int32_t* ranges;       // stream plans: first item of each decode range (the workspace's table)
  int32_t min_range_pairs;  // plan: shortest stream range, in 32-key pairs
  int32_t bs_shift;    // log2 of the tokens per block-table entry (4, or 3)
};

// ---------------------------------------------------------------------------
// plan
// ---------------------------------------------------------------------------

// Hash of the sizes a plan's workspace layout depends on; the attention and
// merge kernels run only on a plan made for their own sizes.  (The block
// table stride is not part of it: every item is checked against the stride
// of the launch that reads it.)
__device__ __forceinline__ uint32_t plan_signature(const AttendParams& P) {
  uint32_t h = 2166136261u;
  const int32_t v[10] = {P.num_seqs, P.num_q_tokens, P.Hq, P.Hkv,
                         P.max_query_len, P.max_seq_len, (int32_t)P.max_items,
                         (int32_t)P.max_partials, (int32_t)P.max_pre_items, P.bs_shift};
#pragma unroll
  for (int i = 0; i < 10; ++i) h = (h ^ (uint32_t)v[i]) * 16777619u;
  return h;
}

constexpr int kPlanThreads = 1024;
// Without a shared prefix, a request of at most this many keys is one key
// range whatever its kind and its batch (the shorter of the decode splits).
constexpr int kOneRangeKeys = kSplitDecode8 < kSplitDecode ? kSplitDecode8 : kSplitDecode;
static_assert(kOneRangeKeys <= kSplitPrefill && kOneRangeKeys <= kMinRangeKeys,
              "no split below kOneRangeKeys");
constexpr int kMaxCoop = 64;  // unsplit prefill requests emitted by all threads
constexpr int kLastBuckets = 16;    // queue order of the decode requests' last splits:
constexpr int kLastBucketKeys = 64; // by length, 64-key buckets, longest first

struct SeqCounts {
  int kind;         // -1: nothing to do
  int ntiles;
  int tq;           // tokens per tile
  int splitlen;     // logical tokens per split; 0: unsplit prefill
  int items;
  int partials;
  int split_tiles;  // tiles with more than one split
};

// Queue regions: prefill items, then full-length decode splits, then the
// (shorter) last split of every decode request: longest units first.
// (stream plans: every decode item in the decode region, in request order)
__device__ __forceinline__ int4 scan_lanes(const SeqCounts& c, bool stream = false) {
  const bool dec = c.kind == kKindDecode;
  return make_int4(c.kind == kKindPrefill ? c.items : 0,
                   dec ? (stream ? c.items : c.items - 1) : 0, c.partials, c.split_tiles);
}

// Stream plans.  The decode requests' own keys, in request order and in
// pairs of 32, form one stream cut into R ranges of equal length (+-1 pair);
// each (range, kv head) is one unit of work, and a request's piece in each
// range it meets is one work item.  In the stream every request is preceded
// by kStartPairs pairs that hold no keys: a request starting inside a range
// costs its wave a switch of items (the block pipeline drains and fills
// again), so a range with more request starts gets fewer keys, and every
// wave's unit takes about the same time whatever the mix of lengths
// (measured on the 8B-shaped decode layer, bf16 and 8-bit: 2 pairs best of
// 0 to 4, about 1 us faster than none).  (A range is longer than kStartPairs, so
// each range still holds at least one item.)  A plan is a stream plan when
// it has no shared prefix, max_seq_len is above kOneRangeKeys and the batch
// fills long_units units with ranges of at least min_range_pairs pairs (512
// keys; 8-bit plans 384); otherwise each request is cut into splits of its
// own (seq_counts) and every split is a unit.
// Range r holds q + 1 pairs if r < rem, else q (T = R q + rem).
constexpr int kStartPairs = 2;
struct Stream {
  int T, R, q, rem;  // R = 0: not a stream plan
};
__device__ __forceinline__ int range_start(const Stream& st, int r) {
  return r * st.q + min(r, st.rem);
}
__device__ __forceinline__ int range_of(const Stream& st, int x) {  // x in [0, T)
  const int big = st.rem * (st.q + 1);
  return x < big ? x / (st.q + 1) : st.rem + (x - big) / st.q;
}
// T: stream positions (start positions included), n_req: decode requests
// with keys; whether to stream is decided on the key pairs alone.
__device__ __forceinline__ Stream stream_of(const AttendParams& P, int T, int n_req) {
  const int want = min(P.long_units, kMaxStreamUnits) / P.Hkv;
  // (the pair counts are summed in 32 bits: batches whose bound could pass
  // 2^31 pairs are not streamed)
  const bool ok = P.prefix_len == 0 && P.max_seq_len > kOneRangeKeys &&
                  (int64_t)(P.max_seq_len + 64) * P.num_seqs < ((int64_t)1 << 36) &&
                  want >= 1 &&
                  (int64_t)T - (int64_t)kStartPairs * n_req >= (int64_t)want * P.min_range_pairs;
  return ok ? Stream{T, want, T / want, T % want} : Stream{T, 0, 0, 0};
}
// Own 32-key pairs of a decode request (0 for others).
// A request's length in the stream: kStartPairs, then its key pairs (its
// keys start at stream position gp + kStartPairs).
__device__ __forceinline__ int stream_pairs(const AttendParams& P, int b, const SeqCounts& c) {
  return c.kind == kKindDecode ? ((P.seq_lens[b] - P.prefix_len + 31) >> 5) + kStartPairs : 0;
}
// A decode request's counts in a stream plan (its pairs [gp, gp + np)).
// (with a shared prefix every decode tile merges, as in seq_counts)
__device__ __forceinline__ void stream_counts(const AttendParams& P, const Stream& st, int gp,
                                              int np, SeqCounts& c) {
  const int ns = range_of(st, gp + np - 1) - range_of(st, gp + kStartPairs) + 1;
  const bool part = P.prefix_len > 0 || ns > 1;
  c.items = ns;
  c.partials = part ? c.tq * ns : 0;
  c.split_tiles = part ? 1 : 0;
}

// A request's metadata is usable: its tokens inside [0, T), Q <= L and
// <= max_query_len, L <= max_seq_len, its blocks inside its table row.
__device__ __forceinline__ bool req_ok(const AttendParams& P, int q0, int q1, int L) {
  const int Q = q1 - q0;
  return q0 >= 0 && Q >= 0 && q1 <= P.num_q_tokens && Q <= L && L <= P.max_seq_len &&
         Q <= P.max_query_len && ((L + (1 << P.bs_shift) - 1) >> P.bs_shift) <= P.bt_stride;
}

// split_long: key range of the splits of decode requests with more than
// kLongDecode keys of their own (chosen per plan, pick_split_long).
__device__ SeqCounts seq_counts(const AttendParams& P, int b, int split_long) {
  SeqCounts c{-1, 0, 0, 0, 0, 0, 0};
  const int q0 = P.qsl[b], q1 = P.qsl[b + 1];
  const int Q = q1 - q0, L = P.seq_lens[b];
  if (!req_ok(P, q0, q1, L)) {
    atomicOr(&P.hdr->error, 2u);
    return c;
  }
  if (Q == 0) return c;
  // With a shared prefix of C keys (cascade plan) the request's own items
  // cover keys C .. and every tile merges, since the prefix items add
  // partials to each of its tokens; its queries must all lie past the prefix.
  const int C = P.prefix_len;
  const bool casc = C > 0;
  if (L - Q < C) {
    atomicOr(&P.hdr->error, 2u);
    return c;
  }
  if (Q <= decode_tile_tokens(P.G)) {
    c.kind = kKindDecode;
    c.ntiles = 1;
    c.tq = Q;
    c.splitlen = L - C > kLongDecode ? split_long : P.split_decode;
    const int ns = (L - C + c.splitlen - 1) / c.splitlen;
    const bool part = casc || ns > 1;
    c.items = ns;
    c.partials = part ? Q * ns : 0;
    c.split_tiles = part ? 1 : 0;
    return c;
  }
  c.kind = kKindPrefill;
  c.tq = prefill_tile_tokens(P.G);
  c.ntiles = (Q + c.tq - 1) / c.tq;
  if (!casc && c.ntiles * P.Hkv >= kPrefillUnsplitUnits) {
    c.splitlen = 0;
    c.items = c.ntiles;
    return c;
  }
  c.splitlen = kSplitPrefill;
  for (int t = 0; t < c.ntiles; ++t) {
    const int ntok = min(c.tq, Q - t * c.tq);
    const int pmax1 = L - Q + t * c.tq + ntok;
    const int ns = (pmax1 - C + c.splitlen - 1) / c.splitlen;
    const bool part = casc || ns > 1;
    c.items += ns;
    c.partials += part ? ntok * ns : 0;
    c.split_tiles += part ? 1 : 0;
  }
  return c;
}

// Units of request b at each candidate long split (1024, 2048, 4096, 8192
// keys) if it is a usable decode request with more than kLongDecode keys of
// its own; zeros otherwise.
__device__ __forceinline__ int4 long_units(const AttendParams& P, int b) {
  const int q0 = P.qsl[b], q1 = P.qsl[b + 1], L = P.seq_lens[b];
  const int own = L - P.prefix_len;
  if (!req_ok(P, q0, q1, L) || q1 == q0 || q1 - q0 > decode_tile_tokens(P.G) ||
      L - (q1 - q0) < P.prefix_len || own <= kLongDecode)
    return make_int4(0, 0, 0, 0);
  return make_int4((own + 1023) >> 10, (own + 2047) >> 11, (own + 4095) >> 12,
                   (own + 8191) >> 13);
}
static_assert(kSplitLongMin == 1024 && kSplitLongMax == 8192, "long_units' candidates");

// The long split of a plan from the batch's totals of long_units: the
// shortest candidate whose units (x kv heads) number at most P.long_units.
__device__ __forceinline__ int pick_split_long(const AttendParams& P, int4 tot) {
  const int64_t want = P.long_units;
  const int64_t h = P.Hkv;
  if ((int64_t)tot.x * h <= want) return 1024;
  if ((int64_t)tot.y * h <= want) return 2048;
  if ((int64_t)tot.z * h <= want) return 4096;
  return 8192;
}

// Whether a plan can hold long decode requests at all (max_seq_len bounds
// every request's keys).
__device__ __forceinline__ bool may_have_long(const AttendParams& P) {
  return P.max_seq_len - P.prefix_len > kLongDecode;
}

// Queue bucket of a decode request's last split: longest first, 64 keys a
// bucket.
__device__ __forceinline__ int last_bucket(const AttendParams& P, int b, const SeqCounts& c) {
  const int own = P.seq_lens[b] - P.prefix_len;
  const int rem = own - (c.items - 1) * c.splitlen;  // keys of the last split
  return min(kLastBuckets - 1, max(0, (kLastBucketKeys * kLastBuckets - rem) / kLastBucketKeys));
}

// Four inclusive scans at once over the lanes of a wave.
__device__ __forceinline__ int4 wave_incl_scan4(int4 x) {
  const int lane = threadIdx.x & 63;
  int4 incl = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y0 = __shfl_up(incl.x, off), y1 = __shfl_up(incl.y, off);
    const int y2 = __shfl_up(incl.z, off), y3 = __shfl_up(incl.w, off);
    if (lane >= off) {
      incl.x += y0;
      incl.y += y1;
      incl.z += y2;
      incl.w += y3;
    }
  }
  return incl;
}

// Four exclusive scans at once (one set of barriers); tot receives the sums.
__device__ int4 block_scan4(int4 x, int4* lds, int4* tot) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  constexpr int kWaves = kPlanThreads / 64;
  const int4 incl = wave_incl_scan4(x);
  if (lane == 63) lds[wid] = incl;
  __syncthreads();
  if (wid == 0) {
    const int4 v = lane < kWaves ? lds[lane] : make_int4(0, 0, 0, 0);
    int4 vi = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y0 = __shfl_up(vi.x, off), y1 = __shfl_up(vi.y, off);
      const int y2 = __shfl_up(vi.z, off), y3 = __shfl_up(vi.w, off);
      if (lane >= off) {
        vi.x += y0;
        vi.y += y1;
        vi.z += y2;
        vi.w += y3;
      }
    }
    if (lane < kWaves) lds[lane] = make_int4(vi.x - v.x, vi.y - v.y, vi.z - v.z, vi.w - v.w);
    if (lane == kWaves - 1) lds[kWaves] = vi;
  }
  __syncthreads();
  const int4 base = lds[wid];
  *tot = lds[kWaves];
  __syncthreads();
  return make_int4(incl.x - x.x + base.x, incl.y - x.y + base.y,
                   incl.z - x.z + base.z, incl.w - x.w + base.w);
}

__device__ __forceinline__ void put_item(WorkItem* dst, int idx, int b,
                                         int tok0, int ntok, int kind, int kv0,
                                         int kv1, int split, int nsplit,
                                         int pbase, int counter, int posbase) {
  WorkItem it;
  it.seq = b;
  it.tok0 = tok0;
  it.ntok = ntok;
  it.kind = kind;
  it.kv0 = kv0;
  it.kv1 = kv1;
  it.split = split;
  it.nsplit = nsplit;
  it.pbase = pbase;
  it.counter = counter;
  it.posbase = posbase;
#pragma unroll
  for (int i = 0; i < 5; ++i) it.pad[i] = 0;
  dst[idx] = it;
}

// Items of one request, emitted by one thread (decode requests and prefill
// requests with split key ranges, which have few tiles).
// ibase: first item slot (decode: of the full-length splits); ilast: slot of
// a decode request's last split.
__device__ void emit_seq(const AttendParams& P, int b, const SeqCounts& c,
                         int ibase, int ilast, int pbase, int cbase) {
  const int q0 = P.qsl[b];
  const int Q = P.qsl[b + 1] - q0, L = P.seq_lens[b];
  const int C = P.prefix_len;  // first key of the request's own items
  if (c.kind == kKindDecode) {
    const int ns = c.items;
    const int sl = c.splitlen;
    const bool part = C > 0 || ns > 1;
    for (int s = 0; s < ns; ++s)
      put_item(P.items, s == ns - 1 ? ilast : ibase + s, b, q0, Q, kKindDecode,
               C + s * sl, min(L, C + (s + 1) * sl), s, ns, part ? pbase : -1,
               part ? cbase : -1, L - Q);
    if (part) P.merge_list[cbase] = make_int4(q0, Q, ns, pbase);
    return;
  }
  // prefill (split, or unsplit when the workgroup's list was full): longest
  // tiles (latest tokens) first
  int icur = ibase, pcur = pbase, ccur = cbase;
  for (int t = c.ntiles - 1; t >= 0; --t) {
    const int ntok = min(c.tq, Q - t * c.tq);
    const int pmax1 = L - Q + t * c.tq + ntok;
    const int span = c.splitlen ? c.splitlen : pmax1;
    const int ns = (pmax1 - C + span - 1) / span;
    const bool part = C > 0 || ns > 1;
    const int pb = part ? pcur : -1;
    const int cb = part ? ccur : -1;
    if (part) {
      P.merge_list[ccur] = make_int4(q0 + t * c.tq, ntok, ns, pcur);
      pcur += ntok * ns;
      ccur += 1;
    }
    for (int s = 0; s < ns; ++s)
      put_item(P.items, icur++, b, q0 + t * c.tq, ntok, kKindPrefill, C + s * span,
               min(pmax1, C + (s + 1) * span), s, ns, pb, cb, L - Q + t * c.tq);
  }
}

// The items of decode request b in a stream plan (stream positions [gp, gp +
// np): kStartPairs, then its key pairs), one per range its key pairs meet,
// in key order; the first item of every range that starts inside the
// request's positions goes into the range table.
// Pieces first, first + step, ... of the request (several threads can share
// a request of many pieces); q0 = qsl[b], L = seq_lens[b].
__device__ void emit_pieces(const AttendParams& P, int b, int q0, int L, int Q, int ns,
                            const Stream& st, int gp, int np, int ibase, int pbase, int cbase,
                            int first = 0, int step = 1) {
  const int C = P.prefix_len;  // first key of the request's own items
  const int g1 = gp + kStartPairs;  // stream position of the first key pair
  const int r0 = range_of(st, g1);
  const bool part = C > 0 || ns > 1;
  for (int s = first; s < ns; s += step) {
    const int rs = range_start(st, r0 + s), re = range_start(st, r0 + s + 1);
    const int a = max(g1, rs), e = min(gp + np, re);
    put_item(P.items, ibase + s, b, q0, Q, kKindDecode, C + 32 * (a - g1),
             min(L, C + 32 * (e - g1)), s, ns, part ? pbase : -1, part ? cbase : -1, L - Q);
    if (rs >= gp) P.ranges[r0 + s] = ibase + s;
  }
  if (part && first == 0) P.merge_list[cbase] = make_int4(q0, Q, ns, pbase);
}

// Registers the item bases of request b: emitted now by this thread, or
// queued for the whole workgroup (unsplit prefill: many tiles).
__device__ __forceinline__ void place_seq(const AttendParams& P, int b,
                                          const SeqCounts& c, int ibase,
                                          int ilast, int pbase, int cbase,
                                          int* coop_n, int* coop_b,
                                          int* coop_base) {
  if (c.kind == kKindPrefill && c.splitlen == 0) {
    const int k = atomicAdd(coop_n, 1);
    if (k < kMaxCoop) {
      coop_b[k] = b;
      coop_base[k] = ibase;
      return;
    }
  }
  emit_seq(P, b, c, ibase, ilast, pbase, cbase);
}

// The tiles of an unsplit prefill request b (its first item slot ibase,
// latest tokens first), thread `first` of `step` threads taking every
// step-th tile.
__device__ void emit_tiles_unsplit(const AttendParams& P, int b, int ibase, int first,
                                   int step) {
  const int q0 = P.qsl[b];
  const int Q = P.qsl[b + 1] - q0, L = P.seq_lens[b];
  const int tq = prefill_tile_tokens(P.G);
  const int ntiles = (Q + tq - 1) / tq;
  for (int t = first; t < ntiles; t += step) {
    const int ntok = min(tq, Q - t * tq);
    const int pmax1 = L - Q + t * tq + ntok;
    put_item(P.items, ibase + (ntiles - 1 - t), b, q0 + t * tq, ntok, kKindPrefill, 0,
             pmax1, 0, 1, -1, -1, L - Q + t * tq);
  }
}

// Shared prefix: tiles of tq consecutive tokens of the whole batch x prefix
// key ranges of span keys (a multiple of 32); the partial of (token t,
// range s) sits at slot t * npre + s of the prefix section.  Returns
// (prefix tiles, prefix ranges); (0, 0) without a shared prefix.
__device__ int2 emit_prefix_items(const AttendParams& P, bool fits, int first, int step) {
  int npre = 0, ntp = 0;
  if (P.prefix_len > 0 && fits) {
    const int C = P.prefix_len;
    npre = min(kMaxPrefixSplits, max(1, (C + kPrefixSplitKeys - 1) / kPrefixSplitKeys));
    const int span = ((C + npre - 1) / npre + 31) & ~31;
    npre = (C + span - 1) / span;
    const int tq = prefill_tile_tokens(P.G);
    ntp = (P.num_q_tokens + tq - 1) / tq;
    if ((int64_t)ntp * npre > P.max_pre_items) npre = ntp = 0;  // (not reached)
    for (int i = first; i < ntp * npre; i += step) {
      const int t = i / npre, s = i - t * npre;
      const int tok0 = t * tq;
      put_item(P.pitems, i, 0, tok0, min(tq, P.num_q_tokens - tok0), kKindPrefix,
               s * span, min(C, (s + 1) * span), s, npre, tok0 * npre, -1, C);
    }
  }
  return make_int2(ntp, npre);
}

// The plan's totals into the header (one thread).  total: prefill items,
// full decode splits, partial slots, split tiles; ndec: decode requests
// (one last split each); pre: prefix tiles and ranges.
__device__ void finish_header(const AttendParams& P, bool fits, int4 total, int ndec,
                              int2 pre, const Stream& st) {
  P.hdr->num_prefix_work = (uint32_t)(pre.x * pre.y) * (uint32_t)P.Hkv;
  P.hdr->prefix_splits = (uint32_t)pre.y;
  const int all_items = total.x + total.y + ndec;
  // stream plans: the decode units are (range, kv head) pairs
  const int units = st.R > 0 ? total.x + (int)st.R : all_items;
  if (fits && st.R > 0) P.ranges[st.R] = total.x + total.y;
  P.hdr->num_ranges = fits ? (uint32_t)st.R : 0u;
  P.hdr->num_items = fits ? (uint32_t)all_items : 0u;
  P.hdr->num_work = fits ? (uint32_t)units * (uint32_t)P.Hkv : 0u;
  P.hdr->num_prefill_work = fits ? (uint32_t)total.x * (uint32_t)P.Hkv : 0u;
  P.hdr->num_split_tiles = fits ? (uint32_t)total.w : 0u;
  if (!fits) atomicOr(&P.hdr->error, 1u);
}

// The header fields every plan starts from, the queue heads zeroed; false
// (and an empty plan) if a shared prefix cannot be read.  Threads 0 ..
// kDecodeShards - 1 of the caller take part.
__device__ bool start_plan(const AttendParams& P, int tid) {
  if (tid < kDecodeShards) P.dec_counters[tid * kCounterStride] = 0;
  if (tid == 0) {
    P.hdr->prefill_counter = 0;
    P.hdr->error = 0;
    P.hdr->signature = plan_signature(P);
    P.hdr->num_prefix_work = 0;
    P.hdr->prefix_splits = 0;
    P.hdr->num_ranges = 0;
  }
  // A shared prefix is read through request 0's table: it must hold it, and
  // the prefix section must exist.  Otherwise the plan is empty.
  if (P.prefix_len > 0 &&
      (P.pitems == nullptr || P.prefix_len > P.seq_lens[0] || P.prefix_len > P.max_seq_len)) {
    if (tid == 0) {
      P.hdr->num_items = 0;
      P.hdr->num_work = 0;
      P.hdr->num_prefill_work = 0;
      P.hdr->num_split_tiles = 0;
      P.hdr->error = 2u;
    }
    return false;
  }
  return true;
}

// The plan of a batch of at most 64 requests, built by one wave with request
// b on lane b: the same queue as plan_body's (prefill items, full decode
// splits, the decode requests' last splits longest first, any order within
// a bucket), with wave scans where plan_body needs workgroup barriers.  (For
// larger batches the workgroup's threads are faster than one wave's chunks
// of 64.)  cnt: kLastBuckets ints of LDS.
__device__ void plan_wave(const AttendParams& P, int* cnt) {
  const int lane = threadIdx.x;
  if (!start_plan(P, lane)) return;
  if (lane < kLastBuckets) cnt[lane] = 0;
  int split_long = kSplitLongMin;
  if (may_have_long(P)) {
    const int4 u = lane < P.num_seqs ? long_units(P, lane) : make_int4(0, 0, 0, 0);
    const int4 ui = wave_incl_scan4(u);
    split_long = pick_split_long(P, make_int4(__shfl(ui.x, 63), __shfl(ui.y, 63),
                                              __shfl(ui.z, 63), __shfl(ui.w, 63)));
  }
  SeqCounts c{-1, 0, 0, 0, 0, 0, 0};
  if (lane < P.num_seqs) c = seq_counts(P, lane, split_long);
  // the lane's request metadata, loaded once (the wave's emission of a
  // request of many pieces takes them from its lane)
  const int q0l = lane < P.num_seqs ? P.qsl[lane] : 0;
  const int Ll = lane < P.num_seqs ? P.seq_lens[lane] : 0;
  // stream partition of the decode requests
  const int np = stream_pairs(P, lane, c);
  const int npi = wave_incl_scan4(make_int4(np, 0, 0, 0)).x;
  const Stream st =
      stream_of(P, __shfl(npi, 63), __popcll(__ballot(lane < P.num_seqs && np > 0)));
  const int gp = npi - np;
  if (st.R > 0 && c.kind == kKindDecode) stream_counts(P, st, gp, np, c);
  const int4 x = scan_lanes(c, st.R > 0);
  const int4 incl = wave_incl_scan4(x);
  const int4 total = make_int4(__shfl(incl.x, 63), __shfl(incl.y, 63), __shfl(incl.z, 63),
                               __shfl(incl.w, 63));
  const int4 e = make_int4(incl.x - x.x, incl.y - x.y, incl.z - x.z, incl.w - x.w);
  // queue slot of each decode request's last split (one wave: its LDS
  // operations take effect in program order)
  int bk = -1, rank = 0;
  if (c.kind == kKindDecode && st.R == 0) {
    bk = last_bucket(P, lane, c);
    rank = atomicAdd(&cnt[bk], 1);
  }
  const int n = lane < kLastBuckets ? cnt[lane] : 0;
  const int nincl = wave_incl_scan4(make_int4(n, 0, 0, 0)).x;
  if (lane < kLastBuckets) cnt[lane] = nincl - n;
  const int ndec = __shfl(nincl, 63);
  const bool fits = total.x + total.y + ndec <= P.max_items && total.z <= P.max_partials;
  const bool unsplit = c.kind == kKindPrefill && c.splitlen == 0;
  const bool piece = c.kind == kKindDecode && st.R > 0;
  // (a request of many pieces is emitted by the whole wave, below)
  const bool many = piece && c.items > 32;
  if (fits && piece && !many)
    emit_pieces(P, lane, q0l, Ll, c.tq, c.items, st, gp, np, total.x + e.y, e.z, e.w);
  else if (fits && c.kind >= 0 && !unsplit && !piece)
    emit_seq(P, lane, c, c.kind == kKindPrefill ? e.x : total.x + e.y,
             total.x + total.y + (bk >= 0 ? cnt[bk] : 0) + rank, e.z, e.w);
  // Requests of many pieces: the whole wave emits each one's, one request
  // at a time, lane l taking its pieces l, l + 64, ...  (A lane emits a
  // piece in a few hundred cycles: up to 32 pieces per lane cost less than
  // a wave pass per request; measured on 16 requests of 17 pieces, plan
  // 9.3 -> 6.5 us against one item per lane per pass.)
  uint64_t mm = __ballot(fits && many);
  while (mm) {
    const int b = __builtin_ctzll(mm);
    mm &= mm - 1;
    auto at = [&](int v) { return __builtin_amdgcn_readlane(v, b); };
    emit_pieces(P, b, at(q0l), at(Ll), at(c.tq), at(c.items), st, at(gp), at(np),
                total.x + at(e.y), at(e.z), at(e.w), lane, 64);
  }
  // unsplit prefill requests (many tiles): the whole wave emits each one's
  uint64_t um = __ballot(fits && unsplit);
  while (um) {
    const int b = __builtin_ctzll(um);
    um &= um - 1;
    emit_tiles_unsplit(P, b, __shfl(e.x, b), lane, 64);
  }
  const int2 pre = emit_prefix_items(P, fits, lane, 64);
  if (lane == 0) finish_header(P, fits, total, ndec, pre, st);
}
// Wave 0 of plan_body: the last splits' bucket counts in cnt become each
// bucket's first slot (an exclusive scan); *ndec receives their sum, the
// number of decode requests.
__device__ __forceinline__ void bucket_starts(int* cnt, int* ndec) {
  const int lane = threadIdx.x & 63;
  const int n = lane < kLastBuckets ? cnt[lane] : 0;
  const int incl = wave_incl_scan4(make_int4(n, 0, 0, 0)).x;
  if (lane < kLastBuckets) cnt[lane] = incl - n;
  if (lane == 63) *ndec = incl;
}

// The work plan, run by one workgroup of kPlanThreads threads (one wave of
// it for batches of at most 64 requests).
__device__ void plan_body(const AttendParams& P) {
  __shared__ int4 lds[kPlanThreads / 64 + 1];
  __shared__ int coop_n;
  __shared__ int coop_b[kMaxCoop];
  __shared__ int coop_base[kMaxCoop];
  __shared__ int last_cnt[kLastBuckets];
  __shared__ int ndec_sh;
  const int tid = threadIdx.x;
  if (P.num_seqs <= 64) {
    if (tid < 64) plan_wave(P, last_cnt);
    return;
  }
  if (tid == 0) coop_n = 0;
  if (!start_plan(P, tid)) return;
  // scan lanes: x = prefill items, y = decode items, z = partial slots,
  // w = split tiles.  Prefill items go first, decode items after them.
  int4 total;
  int ndec = 0;  // decode requests: one last split each
  Stream st{0, 0, 0, 0};  // (stream plans: one sweep only)
  int np = 0, gp = 0;
  bool fits;
  if (P.num_seqs <= kPlanThreads) {
    // one sweep: every request handled by one thread
    const int b = tid;
    int split_long = kSplitLongMin;
    if (may_have_long(P)) {
      int4 tl;
      block_scan4(b < P.num_seqs ? long_units(P, b) : make_int4(0, 0, 0, 0), lds, &tl);
      split_long = pick_split_long(P, tl);
    }
    SeqCounts c{-1, 0, 0, 0, 0, 0, 0};
    if (b < P.num_seqs) c = seq_counts(P, b, split_long);
    // stream partition of the decode requests
    np = stream_pairs(P, b, c);
    int4 tp;
    gp = block_scan4(make_int4(np, np > 0 ? 1 : 0, 0, 0), lds, &tp).x;
    st = stream_of(P, tp.x, tp.y);
    if (st.R > 0 && c.kind == kKindDecode) stream_counts(P, st, gp, np, c);
    // The decode requests' last splits (1 .. split keys each) go last in the
    // queue, longest first (16 buckets of 64 keys, any order within one), so
    // that the launch ends on its shortest units.  Where a unit sits in the
    // queue does not change what it computes.
    if (tid < kLastBuckets) last_cnt[tid] = 0;
    const int4 e = block_scan4(scan_lanes(c, st.R > 0), lds, &total);
    int bk = 0, rank = 0;
    if (c.kind == kKindDecode && st.R == 0) {
      bk = last_bucket(P, b, c);
      rank = atomicAdd(&last_cnt[bk], 1);
    }
    __syncthreads();
    if (tid < 64) bucket_starts(last_cnt, &ndec_sh);
    __syncthreads();
    ndec = ndec_sh;
    fits = total.x + total.y + ndec <= P.max_items && total.z <= P.max_partials;
    if (fits && c.kind == kKindDecode && st.R > 0)
      emit_pieces(P, b, P.qsl[b], P.seq_lens[b], c.tq, c.items, st, gp, np, total.x + e.y,
                  e.z, e.w);
    else if (fits && c.kind >= 0)
      place_seq(P, b, c, c.kind == kKindPrefill ? e.x : total.x + e.y,
                total.x + total.y + last_cnt[bk] + rank, e.z, e.w, &coop_n, coop_b,
                coop_base);
  } else {
    // two sweeps over chunks of requests: totals (and the last splits'
    // bucket counts) first, then placement (and before them, if the batch
    // can hold long decode requests, one for their split)
    int split_long = kSplitLongMin;
    if (may_have_long(P)) {
      int4 tl = make_int4(0, 0, 0, 0);
      for (int base = 0; base < P.num_seqs; base += kPlanThreads) {
        const int b = base + tid;
        int4 t;
        block_scan4(b < P.num_seqs ? long_units(P, b) : make_int4(0, 0, 0, 0), lds, &t);
        tl.x += t.x;
        tl.y += t.y;
        tl.z += t.z;
        tl.w += t.w;
      }
      split_long = pick_split_long(P, tl);
    }
    total = make_int4(0, 0, 0, 0);
    if (tid < kLastBuckets) last_cnt[tid] = 0;
    __syncthreads();
    for (int base = 0; base < P.num_seqs; base += kPlanThreads) {
      const int b = base + tid;
      SeqCounts c{-1, 0, 0, 0, 0, 0, 0};
      if (b < P.num_seqs) c = seq_counts(P, b, split_long);
      if (c.kind == kKindDecode) atomicAdd(&last_cnt[last_bucket(P, b, c)], 1);
      int4 t;
      block_scan4(scan_lanes(c), lds, &t);
      total.x += t.x;
      total.y += t.y;
      total.z += t.z;
      total.w += t.w;
    }
    __syncthreads();
    if (tid < 64) bucket_starts(last_cnt, &ndec_sh);  // counts -> first slots
    __syncthreads();
    ndec = ndec_sh;
    fits = total.x + total.y + ndec <= P.max_items && total.z <= P.max_partials;
    int4 carry = make_int4(0, 0, 0, 0);
    for (int base = 0; base < P.num_seqs; base += kPlanThreads) {
      const int b = base + tid;
      SeqCounts c{-1, 0, 0, 0, 0, 0, 0};
      if (b < P.num_seqs) c = seq_counts(P, b, split_long);
      int4 t;
      const int4 e = block_scan4(scan_lanes(c), lds, &t);
      // next free slot of the request's bucket (any order within a bucket)
      const int last = c.kind == kKindDecode ? atomicAdd(&last_cnt[last_bucket(P, b, c)], 1) : 0;
      if (fits && c.kind >= 0)
        place_seq(P, b, c,
                  c.kind == kKindPrefill ? carry.x + e.x : total.x + carry.y + e.y,
                  total.x + total.y + last, carry.z + e.z,
                  carry.w + e.w, &coop_n, coop_b, coop_base);
      carry.x += t.x;
      carry.y += t.y;
      carry.z += t.z;
      carry.w += t.w;
    }
  }
  __syncthreads();
  // unsplit prefill requests: every thread emits some of their tiles
  const int ncoop = min(coop_n, kMaxCoop);
  for (int k = 0; k < ncoop; ++k)
    emit_tiles_unsplit(P, coop_b[k], coop_base[k], tid, kPlanThreads);
  const int2 pre = emit_prefix_items(P, fits, tid, kPlanThreads);
  if (tid == 0) finish_header(P, fits, total, ndec, pre, st);
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(AttendParams P) {
  plan_body(P);
}

// The scatter of a step's new K/V and the work plan in one launch:
// workgroup 0 plans, the others scatter with their first S.per_block threads
// (the rest exit at once).  The two are independent (the plan reads only the
// metadata, the scatter writes only pool slots); both must be complete
// before attention reads the pools, which stream order gives.
template <int D, bool KV8>
__global__ __launch_bounds__(kPlanThreads) void write_plan_kernel(AttendParams P,
                                                                  ScatterArgs S) {
  if (blockIdx.x == 0) {
    plan_body(P);
    return;
  }
  if ((int)threadIdx.x >= S.per_block) return;
  const int64_t gid = (int64_t)(blockIdx.x - 1) * S.per_block + threadIdx.x;
  if constexpr (KV8)
    write_kv8_thread<D>(gid, S.k, S.v, S.k_stride, S.v_stride, S.slots, S.num_tokens,
                        S.Hkv, S.k_scale, S.v_scale, static_cast<uint8_t*>(S.k_cache),
                        static_cast<uint8_t*>(S.v_cache), S.num_slots);
  else
    write_kv_thread<D>(gid, S.k, S.v, S.k_stride, S.v_stride, S.slots, S.num_tokens,
                       S.Hkv, static_cast<uint16_t*>(S.k_cache),
                       static_cast<uint16_t*>(S.v_cache), S.num_slots);
}

// ---------------------------------------------------------------------------
// attend
// ---------------------------------------------------------------------------

__device__ __forceinline__ bf16x8 load16(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// Non-temporal load: decode reads each K/V tile once, so it should not
// displace cached data (the streaming read ceiling is ~10% higher with it).
__device__ __forceinline__ bf16x8 load16_stream(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(p));
}

__device__ __forceinline__ bf16x4 load8(const uint16_t* p) {
  return *reinterpret_cast<const bf16x4*>(p);
}
__device__ __forceinline__ bf16x4 load8_stream(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const bf16x4*>(p));
}

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = (__bf16)0.0f;
  return z;
}

// 8-bit pools: 16-byte loads of E4M3 codes, and their exact conversion to
// bf16 operands (every E4M3 value is a bf16 value; the scale is applied
// outside the MFMAs).
__device__ __forceinline__ u32x4 load16b(const uint8_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x4 load16b_stream(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
// codes in bytes 0..3 of w (lowest first) -> 4 bf16
__device__ __forceinline__ bf16x4 e4m3x4_to_bf16(uint32_t w) {
  const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3);
}
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t w0, uint32_t w1) {
  return __builtin_shufflevector(e4m3x4_to_bf16(w0), e4m3x4_to_bf16(w1), 0, 1, 2, 3, 4,
                                 5, 6, 7);
}


// Query operand and column positions of a unit.  Column c of tile ct is
// token c / G, head c % G of the kv head's group; lane (r, g) holds dims
// 32k + 8g .. +7 of column r for k-step k.
template <int D, int CT>
__device__ __forceinline__ void load_query(const AttendParams& P,
                                           const WorkItem& it, int kvh,
                                           int lane, int posbase,
                                           bf16x8 (&qop)[CT][D / 32],
                                           int (&cpos)[CT]) {
  const int r = lane & 15, g = lane >> 4;
  const int G = P.G;
  const int ncols = it.ntok * G;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int col = ct * 16 + r;
    const int tk = col / G;
    const int hh = col - tk * G;
    const bool valid = col < ncols;
    cpos[ct] = valid ? posbase + tk : -1;
    if (valid) {
      const uint16_t* qp =
          P.q + ((int64_t)(it.tok0 + tk) * P.Hq + kvh * G + hh) * D + 8 * g;
#pragma unroll
      for (int c = 0; c < D / 32; ++c) qop[ct][c] = load16(qp + 32 * c);
    } else {
#pragma unroll
      for (int c = 0; c < D / 32; ++c) qop[ct][c] = zero8();
    }
  }
}


// Online-softmax update of one column tile with N new raw scores per lane
// (q.k; -inf where masked) and c = scale * log2(e).  The running max is kept
// in the exp2 domain; max(s) * c equals max(s * c) exactly since c > 0.
// Returns the bf16 probabilities exp2(s * c - m) (one fused multiply-add
// per score) and the rescale factor of the old state.
template <int N>
__device__ __forceinline__ void softmax_step(const float (&s)[N], float c,
                                             float& mrun, float& lsum,
                                             float& alpha, __bf16 (&p)[N]) {
  float mx = s[0];
#pragma unroll
  for (int i = 1; i < N; ++i) mx = fmaxf(mx, s[i]);
  mx = column_max(mx);
  const float mnew = fmaxf(mrun, mx * c);
  const float muse = (mnew == -INFINITY) ? 0.0f : mnew;
  alpha = __builtin_amdgcn_exp2f(mrun - muse);
  mrun = mnew;
  float psum = 0.0f;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    p[i] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c, -muse));
    psum += (float)p[i];
  }
  lsum = lsum * alpha + psum;
}

// The same update without the probability sum (computed on the matrix core
// by the caller).
template <int N>
__device__ __forceinline__ void softmax_probs(const float (&s)[N], float c,
                                              float& mrun, float& alpha,
                                              __bf16 (&p)[N]) {
  float mx = s[0];
#pragma unroll
  for (int i = 1; i < N; ++i) mx = fmaxf(mx, s[i]);
  mx = column_max(mx);
  const float mnew = fmaxf(mrun, mx * c);
  const float muse = (mnew == -INFINITY) ? 0.0f : mnew;
  alpha = __builtin_amdgcn_exp2f(mrun - muse);
  mrun = mnew;
#pragma unroll
  for (int i = 0; i < N; ++i)
    p[i] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c, -muse));
}

// End of a unit: direct bf16 output, or fp32 partials (running max, sum and
// unnormalised accumulator per column) for the merge kernel.  l[ct] is the
// column's full probability sum (the same in all four lanes of a column).
template <int D, int CT, bool KV8>
__device__ __forceinline__ void finish_unit(const AttendParams& P,
                                            const WorkItem& it, int kvh,
                                            int lane, f32x4 (&acc)[CT][D / 16],
                                            float (&mrun)[CT],
                                            const float (&l)[CT]) {
  constexpr int NT = D / 16;
  const int r = lane & 15, g = lane >> 4;
  const int G = P.G;
  const int ncols = it.ntok * G;
  if (it.pbase < 0) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int col = ct * 16 + r;
      if (col >= ncols) continue;
      const int tk = col / G;
      const int64_t t = it.tok0 + tk;
      const int h = kvh * G + (col - tk * G);
      // 8-bit pools: V codes stand for code * v_scale
      const float inv = (KV8 ? P.v_scale : 1.0f) / l[ct];
      uint16_t* op = P.out + (t * P.Hq + h) * D + 4 * g;
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        bf16x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = (__bf16)(acc[ct][n][i] * inv);
        *reinterpret_cast<bf16x4*>(op + 16 * n) = o;
      }
    }
    return;
  }
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int col = ct * 16 + r;
    if (col >= ncols) continue;
    const int tk = col / G;
    const int h = kvh * G + (col - tk * G);
    const int64_t slot = (int64_t)it.pbase + (int64_t)tk * it.nsplit + it.split;
    // shared-prefix items write the prefix section
    const bool pre = it.kind == kKindPrefix;
    float* ap = (pre ? P.pre_acc : P.part_acc) + (slot * P.Hq + h) * D + 4 * g;
#pragma unroll
    for (int n = 0; n < NT; ++n)
      *reinterpret_cast<f32x4*>(ap + 16 * n) = KV8 ? acc[ct][n] * P.v_scale : acc[ct][n];
    if (g == 0) (pre ? P.pre_ml : P.part_ml)[slot * P.Hq + h] = make_float2(mrun[ct], l[ct]);
  }
}

template <int D>
struct KVBlock {
  bf16x8 k[D / 32];  // K rows in MFMA operand order
  bf16x8 v[D / 32];  // lane's 4 keys at dims d and d + D/2
};

// The same block from 8-bit pools: per lane, unit p of K holds the operands
// of chunks 2p and 2p+1 (8 codes each), unit p of V the 4-key operands of
// chunks 2p + cc at dims d and d + D/2 (one 32-bit word each, (cc, dh) order
// (0,0), (0,1), (1,0), (1,1)).
template <int D>
struct KVBlock8 {
  u32x4 k[D / 64];
  u32x4 v[D / 64];
};

template <int D, bool KV8>
using KVBuf = typename std::conditional<KV8, KVBlock8<D>, KVBlock<D>>::type;

// V operand of k step c for lane (r, g): keys 4g .. 4g+3 at dims 16c + r
// (elements 0-3) and D/2 + 16c + r (4-7), two 8-byte reads of the tile.
template <int D, bool STREAM>
__device__ __forceinline__ bf16x8 load_v(const uint16_t* vp, int c, int lane) {
  const uint16_t* lo = vp + (2 * c) * 256 + lane * 4;
  const bf16x4 a = STREAM ? load8_stream(lo) : load8(lo);
  const bf16x4 b = STREAM ? load8_stream(lo + 256) : load8(lo + 256);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// One (item, kv head) unit on one wave: CT column tiles of 16 (query token x
// head of the group), one block (16 keys) per step with the loads of the next
// NB-1 blocks in flight while the current one is computed.  Scores on
// 16x16x32 MFMA, PV on 16x16x16 MFMA whose B operand is the score registers
// as they stand.  STREAM selects non-temporal K/V loads (decode: every tile is
// read once) or cached loads (prefill: the tiles of a request are re-read by
// all of its query tiles).  Block ids come 64 at a time, one per lane; each
// chunk of 64 blocks runs its own pipeline.
// If `counter` is not null, the next queue entry is claimed from it when the
// load of the unit's last block is issued (its latency then hides behind the
// last blocks and the output stores) and returned; otherwise 0.
// BS8: the pools hold 8-token blocks (block-table entries name 8 tokens), so
// each 16-key step reads two pool tiles: lanes of tokens 0-7 (K) and of key
// groups 0-1 (V) from the first, the others from the second; the operands
// land in the same registers as from one 16-token tile.
__device__ __forceinline__ bool item_ok(const AttendParams& P,
                                        const WorkItem& it) {
  const int maxtok = it.kind == kKindDecode ? decode_tile_tokens(P.G)
                                            : prefill_tile_tokens(P.G);
  bool ok = it.seq >= 0 && it.seq < P.num_seqs && it.tok0 >= 0 &&
            it.ntok >= 1 && it.ntok <= maxtok &&
            it.tok0 + it.ntok <= P.num_q_tokens && it.kv0 >= 0 &&
            (it.kv0 & 31) == 0 && it.kv1 > it.kv0 && it.kv1 <= P.max_seq_len &&
            ((it.kv1 + (1 << P.bs_shift) - 1) >> P.bs_shift) <= P.bt_stride &&
            it.nsplit >= 1 && it.split >= 0 && it.split < it.nsplit;
  if (it.kind == kKindDecode) ok = ok && (it.kv1 - it.kv0) <= kSplitLongMax;
  if (it.nsplit > 1) ok = ok && it.pbase >= 0;
  if (it.pbase >= 0)
    ok = ok && (int64_t)it.pbase + (int64_t)it.ntok * it.nsplit <=
                   (it.kind == kKindPrefix ? P.max_pre_partials : P.max_partials);
  return ok;
}

// One shard of the decode queue as a wave sees it: local unit k is queue
// entry base + stride * k (k < n); a claim returning t hands the wave local
// unit t + first_dynamic, and the claim returning claims - 1 is the shard's
// last in the launch, which resets the counter for the next launch.
struct DecodeQueue {
  uint32_t* counter;
  uint32_t base, stride, n, first_dynamic, claims;
  bool unit_items;  // a unit is one item (plans without stream ranges)
};

// The wave's next unit as run_unit prepares it during the current one: its
// local index k (>= n: none), its item as 16 dwords on lanes 0..15 once
// item_ready, and the physical ids of its first 64 blocks, one per lane,
// once ids_ready.
struct NextUnit {
  uint32_t k;
  int itv;
  int idv;
  bool item_ready;
  bool ids_ready;
};

// Work item idx as 16 dwords, dword i on lane i (0 on lanes 16..63): a vector
// load, ordered with the block loads in flight (a scalar load would be waited
// for by the softmax's cross-lane steps).
__device__ __forceinline__ int load_item_lanes(const WorkItem* items, uint32_t idx, int lane) {
  const int32_t* p = reinterpret_cast<const int32_t*>(items + idx);
  return lane < 16 ? p[lane] : 0;
}

__device__ __forceinline__ WorkItem item_of_lanes(int v) {
  WorkItem it;
  it.seq = __builtin_amdgcn_readlane(v, 0);
  it.tok0 = __builtin_amdgcn_readlane(v, 1);
  it.ntok = __builtin_amdgcn_readlane(v, 2);
  it.kind = __builtin_amdgcn_readlane(v, 3);
  it.kv0 = __builtin_amdgcn_readlane(v, 4);
  it.kv1 = __builtin_amdgcn_readlane(v, 5);
  it.split = __builtin_amdgcn_readlane(v, 6);
  it.nsplit = __builtin_amdgcn_readlane(v, 7);
  it.pbase = __builtin_amdgcn_readlane(v, 8);
  it.counter = __builtin_amdgcn_readlane(v, 9);
  it.posbase = __builtin_amdgcn_readlane(v, 10);
#pragma unroll
  for (int i = 0; i < 5; ++i) it.pad[i] = 0;
  return it;
}

// Physical ids of 16-token blocks c0 .. c0 + 63 of a unit (one per lane,
// lanes past its last block 0), clamped into the pool.
__device__ __forceinline__ int block_ids(const AttendParams& P, const WorkItem& it, int c0,
                                         int lane) {
  const int jb1 = (it.kv1 + kBlock - 1) >> 4;
  int idv = 0;
  if (lane < min(64, jb1 - c0)) idv = P.bt[(int64_t)it.seq * P.bt_stride + c0 + lane];
  return idv < 0 ? 0 : (idv >= P.num_blocks ? (int)(P.num_blocks - 1) : idv);
}

// One decode item (it, kv head kvh) of a wave.  With next_item < 0 it ends
// the wave's unit: exactly one claim on the queue, issued with the loads of
// the item's third block from last, so that its value is back by the time
// that block is computed; otherwise item next_item of the same unit follows.
// Either way the next item, then its first block ids, are loaded while the
// last blocks stream, so that the next call starts on its block loads at
// once (nx: in, the ids of this item if ready; out, the next one).
template <int D, int CT, int NB, bool STREAM, bool KV8, bool BS8 = false>
__device__ __forceinline__ void run_unit(const AttendParams& P,
                                         const WorkItem& it, int kvh,
                                         int lane, const DecodeQueue& Qd,
                                         NextUnit& nx, int next_item) {
  static_assert(!(KV8 && BS8), "8-token blocks: bf16 pools only");
  constexpr int KC = D / 32;
  constexpr int NT = D / 16;
  const int g = lane >> 4;
  const int b = it.seq;
  const int posbase = it.posbase;  // position of the tile's first token

  bf16x8 qop[CT][KC];
  int cpos[CT];
  load_query<D, CT>(P, it, kvh, lane, posbase, qop, cpos);

  f32x4 acc[CT][NT];
  float mrun[CT], lsum[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    mrun[ct] = -INFINITY;
    lsum[ct] = 0.0f;
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[ct][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int jb0 = it.kv0 >> 4;
  const int jb1 = (it.kv1 + kBlock - 1) >> 4;
  const int32_t* btrow = P.bt + (int64_t)b * P.bt_stride;
  const int64_t tile_elems = (int64_t)kBlock * D;
  // 8-bit pools: no prefetch (their waves need the registers for more
  // waves per SIMD, which hide the dequantisation); the claim goes with the
  // last block's loads and is read at the end
  constexpr bool kPrefetch = !KV8;
  const int jclaim = kPrefetch ? max(jb0, jb1 - 3) : jb1 - 1;  // its loads carry the claim
  uint32_t claim = 0;
  bool claimed = next_item >= 0, took = false;
  const bool have_ids = kPrefetch && !BS8 && nx.ids_ready;
  const int ids0 = nx.idv;
  NextUnit next{nx.k, 0, 0, false, false};
  // the next item: the unit's next one, or the claimed unit's (when a unit
  // is one item), loaded at once
  auto take_claim = [&]() {
    if (next_item >= 0) {
      if (kPrefetch) {
        next.itv = load_item_lanes(P.items, (uint32_t)next_item, lane);
        next.item_ready = true;
      }
    } else {
      const uint32_t t = __builtin_amdgcn_readfirstlane(__shfl(claim, 0));
      if (t + 1u == Qd.claims && lane == 0) atomicExch(Qd.counter, 0u);
      next.k = t + Qd.first_dynamic;
      if (kPrefetch && next.k < Qd.n && Qd.unit_items) {
        next.itv = load_item_lanes(P.items, (Qd.base + Qd.stride * next.k) / (uint32_t)P.Hkv,
                                   lane);
        next.item_ready = true;
      }
    }
    took = true;
  };

  for (int c0 = jb0; c0 < jb1; c0 += 64) {
    const int nblk = min(64, jb1 - c0);
    // physical ids of this chunk's blocks, one per lane (8-token blocks: the
    // two of each 16-key step; a second block past the range's keys is not
    // read from the table, the first stands in for it, its keys masked)
    int idv = 0, idv2 = 0;
    if constexpr (BS8) {
      const int j8 = 2 * (c0 + lane);
      const int nb8 = (it.kv1 + 7) >> 3;
      if (lane < nblk) {
        idv = btrow[j8];
        idv2 = j8 + 1 < nb8 ? btrow[j8 + 1] : idv;
      }
      idv2 = idv2 < 0 ? 0 : (idv2 >= P.num_blocks ? (int)(P.num_blocks - 1) : idv2);
      idv = idv < 0 ? 0 : (idv >= P.num_blocks ? (int)(P.num_blocks - 1) : idv);
    } else {
      idv = (have_ids && c0 == jb0) ? ids0 : block_ids(P, it, c0, lane);
    }

    auto issue = [&](KVBuf<D, KV8>& buf, int j) {
      if (!claimed && c0 + j == jclaim) {
        if (lane == 0) claim = atomicAdd(Qd.counter, 1u);
        claimed = true;
      }
      const int id = __builtin_amdgcn_readlane(idv, j);
      const int64_t off = ((int64_t)id * P.Hkv + kvh) * tile_elems;
      if constexpr (BS8) {
        // tiles of 8 * D elements: K chunk q of token t at (q * 8 + t) * 8,
        // V region h (512 bytes in a 16-token tile) at h * 128
        const int id2 = __builtin_amdgcn_readlane(idv2, j);
        const int64_t offa = ((int64_t)id * P.Hkv + kvh) * (8 * D);
        const int64_t offb = ((int64_t)id2 * P.Hkv + kvh) * (8 * D);
        const int r = lane & 15;
        const uint16_t* kp = P.k_cache + (r < 8 ? offa : offb) + g * 64 + (r & 7) * 8;
        const uint16_t* vp = P.v_cache + (g < 2 ? offa : offb) + ((g & 1) * 16 + r) * 4;
#pragma unroll
        for (int c = 0; c < KC; ++c)
          buf.k[c] = STREAM ? load16_stream(kp + c * 256) : load16(kp + c * 256);
#pragma unroll
        for (int c = 0; c < KC; ++c) {
          const bf16x4 a = STREAM ? load8_stream(vp + 2 * c * 128) : load8(vp + 2 * c * 128);
          const bf16x4 b =
              STREAM ? load8_stream(vp + (2 * c + 1) * 128) : load8(vp + (2 * c + 1) * 128);
          buf.v[c] = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
        }
      } else if constexpr (KV8) {
        // tile_elems bytes per tile; unit p of either pool at p KiB + 16 lane
        const uint8_t* kp = reinterpret_cast<const uint8_t*>(P.k_cache) + off;
        const uint8_t* vp = reinterpret_cast<const uint8_t*>(P.v_cache) + off;
#pragma unroll
        for (int u = 0; u < D / 64; ++u)
          buf.k[u] = STREAM ? load16b_stream(kp + u * 1024 + lane * 16)
                            : load16b(kp + u * 1024 + lane * 16);
#pragma unroll
        for (int u = 0; u < D / 64; ++u)
          buf.v[u] = STREAM ? load16b_stream(vp + u * 1024 + lane * 16)
                            : load16b(vp + u * 1024 + lane * 16);
      } else {
        const uint16_t* kp = P.k_cache + off;
        const uint16_t* vp = P.v_cache + off;
#pragma unroll
        for (int c = 0; c < KC; ++c)
          buf.k[c] = STREAM ? load16_stream(kp + c * 512 + lane * 8)
                            : load16(kp + c * 512 + lane * 8);
#pragma unroll
        for (int c = 0; c < KC; ++c) buf.v[c] = load_v<D, STREAM>(vp, c, lane);
      }
    };

    auto compute = [&](KVBuf<D, KV8>& buf8, int j) {
      const int kp0 = (c0 + j) * kBlock;
      KVBlock<D> buf;
      if constexpr (KV8) {
        // keys at or past kv1 may be unwritten pool slots: zero their codes
        // (code 0 is +0) so a 0 weight cannot meet a NaN
        uint32_t keep = 0xffffffffu;
        if (kp0 + kBlock > it.kv1) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (kp0 + 4 * g + i >= it.kv1) keep &= ~(0xffu << (8 * i));
        }
#pragma unroll
        for (int c = 0; c < KC; ++c) {
          const u32x4 ku = buf8.k[c >> 1];
          const u32x4 vu = buf8.v[c >> 1];
          buf.k[c] = (c & 1) ? e4m3x8_to_bf16(ku[2], ku[3]) : e4m3x8_to_bf16(ku[0], ku[1]);
          buf.v[c] = (c & 1) ? e4m3x8_to_bf16(vu[2] & keep, vu[3] & keep)
                             : e4m3x8_to_bf16(vu[0] & keep, vu[1] & keep);
        }
      } else {
        buf = buf8;
      }
      if (!KV8 && kp0 + kBlock > it.kv1) {
        // keys at or past kv1 may be unwritten pool slots: zero their V so a
        // 0 weight cannot meet a NaN
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (kp0 + 4 * g + i >= it.kv1) {
#pragma unroll
            for (int c = 0; c < KC; ++c) {
              buf.v[c][i] = (__bf16)0.0f;
              buf.v[c][i + 4] = (__bf16)0.0f;
            }
          }
        }
      }
      const bool need_mask = kp0 + kBlock - 1 > posbase;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < KC; ++c) sc = mfma32(buf.k[c], qop[ct][c], sc);
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[i] = sc[i];
          if (need_mask && kp0 + 4 * g + i > cpos[ct]) x[i] = -INFINITY;
        }
        float alpha;
        __bf16 p[4];
        softmax_step<4>(x, P.scale_log2, mrun[ct], lsum[ct], alpha, p);
        bf16x4 pop = {p[0], p[1], p[2], p[3]};
        // alpha is exactly 1 where the running max did not move: skip the
        // rescale when that holds for every column of the wave (same bits)
        if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
          for (int n = 0; n < NT; ++n) acc[ct][n] *= alpha;
        }
#pragma unroll
        for (int c = 0; c < KC; ++c) {
          const bf16x4 vlo = __builtin_shufflevector(buf.v[c], buf.v[c], 0, 1, 2, 3);
          const bf16x4 vhi = __builtin_shufflevector(buf.v[c], buf.v[c], 4, 5, 6, 7);
          acc[ct][c] = mfma16(vlo, pop, acc[ct][c]);
          acc[ct][c + KC] = mfma16(vhi, pop, acc[ct][c + KC]);
        }
      }
      if (kPrefetch && c0 + j == jclaim && claimed && !took) take_claim();
    };

    // Ring of NB block buffers, NB-1 blocks in flight while one is computed.
    // Every path into the loop header has the same loads in flight (the
    // prefetch is unconditional, clamped to the last block, and the loop has
    // no early exit), so the compiler's waits stop at the block being
    // computed and never drain the prefetches.  Clamped prefetches past the
    // end re-read the last block (an L2 hit).
    KVBuf<D, KV8> buf[NB];
#pragma unroll
    for (int k = 0; k < NB - 1; ++k) issue(buf[k], min(k, nblk - 1));
    int j = 0;
    for (; j + NB <= nblk; j += NB) {
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        issue(buf[(k + NB - 1) % NB], min(j + k + NB - 1, nblk - 1));
        compute(buf[k], j + k);
      }
    }
#pragma unroll
    for (int k = 0; k < NB - 1; ++k)
      if (j + k < nblk) compute(buf[k], j + k);
  }
  // exactly one claim per call, whatever the loop above did
  if (!claimed) {
    if (lane == 0) claim = atomicAdd(Qd.counter, 1u);
    claimed = true;
  }
  if (kPrefetch && !took) take_claim();
  // the next unit's first block ids go out before this unit's results
  if (kPrefetch && next.item_ready && !BS8) {
    const WorkItem ni = item_of_lanes(next.itv);
    if (item_ok(P, ni) && ni.kind == kKindDecode) {
      next.idv = block_ids(P, ni, ni.kv0 >> 4, lane);
      next.ids_ready = true;
    }
  }
  float l[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    l[ct] = lsum[ct];
    l[ct] += __shfl_xor(l[ct], 16);
    l[ct] += __shfl_xor(l[ct], 32);
  }
  finish_unit<D, CT, KV8>(P, it, kvh, lane, acc, mrun, l);
  if (!took) take_claim();  // (no prefetch: the claim is read after the stores)
  nx = next;
}

// ---- prefill tiles: one workgroup, K/V shared through LDS -------------------

// A prefill tile's kPrefillWaves waves take consecutive token slices of it and
// read the same keys, so its K/V tiles are fetched once per workgroup into an
// LDS ring of key-pair stages (2 blocks), kPairStages - 1 pairs ahead of the
// pair being computed, with direct global-to-LDS loads issued a quarter by
// each wave.  Two blocks per step let PV run on 16x16x32 MFMA: k slot 8g + j
// of the pair is key 4g + j of the first block for j < 4 and key 4g + j - 4
// of the second, matching the score rows the lane holds.
//
// Stage layout (bf16 elements, TILE = 16 * D): K of the first block, V of
// the first, K of the second, V of the second, each a pool tile copied as it
// is (wave w loads tile w with 1 KiB loads).  K operands are 16-byte LDS
// reads; a V operand is two 8-byte reads, one from each block's V tile, into
// adjacent registers.  All are conflict-free.
constexpr int kPairStages = 4;

// Bytes of one K or V pool tile, of a ring stage and of the ring (bf16 or
// 8-bit pools).
template <int D, bool KV8>
constexpr int tile_bytes() {
  return kBlock * D * (KV8 ? 1 : 2);
}
template <int D, bool KV8>
constexpr int pair_stage_bytes() {
  return 4 * tile_bytes<D, KV8>();
}
template <int D, bool KV8>
constexpr int prefill_ring_bytes() {
  return kPairStages * pair_stage_bytes<D, KV8>();
}

__device__ __forceinline__ uint32_t lds_addr(const void* l) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)l);
}

__device__ __forceinline__ const uint16_t* uniform_ptr(const uint16_t* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const uint16_t*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// Global-to-LDS copy of N KiB: load c (c < N) has lane i read 16 bytes at
// base + voff + 1024 c (voff = 16 i) and write them to LDS at
// l + 1024 c + 16 i (bytes); base and l are the same for the whole wave.
// The instruction offset moves the global and the LDS address alike, so
// one M0 value serves all N loads.  Written as inline assembly so that the
// compiler does not track it: it would otherwise wait for every such load
// before any LDS read, draining the pipeline; the ring protocol below
// orders them itself.  The loads read M0 (their LDS base) and an SGPR pair:
// five wait states after they are written cover the hazard rules for both.
// M0 is restored.
template <int N>
__device__ __forceinline__ void load_lds_kib(const uint16_t* base, uint32_t voff,
                                             uint32_t l) {
  static_assert(N == 1 || N == 2 || N == 4, "1, 2 or 4 KiB tiles");
  uint32_t saved;
  if constexpr (N == 1) {
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 4\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(uniform_ptr(base)), "s"(l)
        : "memory");
  } else if constexpr (N == 2) {
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 4\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "global_load_lds_dwordx4 %1, %2 offset:1024\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(uniform_ptr(base)), "s"(l)
        : "memory");
  } else {
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 4\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "global_load_lds_dwordx4 %1, %2 offset:1024\n\t"
        "global_load_lds_dwordx4 %1, %2 offset:2048\n\t"
        "global_load_lds_dwordx4 %1, %2 offset:3072\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(uniform_ptr(base)), "s"(l)
        : "memory");
  }
}
// Global-to-LDS copy of N KiB with a global address per lane: load c has
// lane i read 16 bytes at lane_addr - 512 c + 1024 c and write them to LDS at
// l + 1024 c + 16 i.  (For pools of 8-token blocks: the 16-token tile of a
// stage is gathered from two pool tiles, in which the data of consecutive
// KiB of the stage lie 512 bytes apart.)  M0 is set and restored as in
// load_lds_kib; the addresses are VGPRs, which need no wait states.
template <int N>
__device__ __forceinline__ void load_lds_kib_lanes(uint64_t lane_addr, uint32_t l) {
  static_assert(N == 2 || N == 4, "2 or 4 KiB tiles");
  uint32_t saved;
  const uint64_t a1 = lane_addr - 512;
  if constexpr (N == 2) {
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 4\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "global_load_lds_dwordx4 %2, off offset:1024\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(lane_addr), "v"(a1), "s"(l)
        : "memory");
  } else {
    const uint64_t a2 = lane_addr - 1024, a3 = lane_addr - 1536;
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %5\n\ts_nop 4\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "global_load_lds_dwordx4 %2, off offset:1024\n\t"
        "global_load_lds_dwordx4 %3, off offset:2048\n\t"
        "global_load_lds_dwordx4 %4, off offset:3072\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(lane_addr), "v"(a1), "v"(a2), "v"(a3), "s"(l)
        : "memory");
  }
}

// Wait until at most N of this wave's vector memory loads are outstanding,
// then meet the other waves of the workgroup.  (A compiler-level memory
// barrier as well: LDS reads are not moved across it.)  LDS reads in flight
// are not waited for: the only ones a wave can have here are of the stage
// it computes next, which is not refilled at this barrier (every read of the
// stage that is refilled was consumed, and so waited for, in the previous
// step).
template <int N>
__device__ __forceinline__ void wait_loads_and_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

__device__ __forceinline__ bf16x8 lds16(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// One LDS read of 2 x 8 bytes at addr + 512 O0 and addr + 512 O1 (bytes)
// into one 16-byte operand.  Inline assembly, so the compiler neither pairs
// the halves differently nor tracks the read: the caller waits for it
// (wait_lds_operands) before any use.
template <int O0, int O1>
__device__ __forceinline__ bf16x8 lds_read2st64(uint32_t addr) {
  static_assert(O0 >= 0 && O0 < 256 && O1 >= 0 && O1 < 256, "ds offset range");
  bf16x8 r;
  asm volatile("ds_read2st64_b64 %0, %1 offset0:%2 offset1:%3"
               : "=v"(r)
               : "v"(addr), "n"(O0), "n"(O1));
  return r;
}
// One 16-byte LDS read at addr + O (bytes), untracked like lds_read2st64.
template <int O>
__device__ __forceinline__ u32x4 lds_read_b128(uint32_t addr) {
  static_assert(O >= 0 && O < 65536, "ds offset range");
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(O));
  return r;
}
// The 2 (D/64) raw 8-bit V units of a pair: units p of the first block's V
// tile (at addr + 1 KiB p) and of the second's (SECOND bytes further).
template <int SECOND, int... U>
__device__ __forceinline__ void read_v8_units(uint32_t addr, u32x4* va, u32x4* vb,
                                              std::integer_sequence<int, U...>) {
  ((va[U] = lds_read_b128<U * 1024>(addr)), ...);
  ((vb[U] = lds_read_b128<SECOND + U * 1024>(addr)), ...);
}
template <int SECOND, int... HC>
__device__ __forceinline__ void read_v_regions(uint32_t addr, bf16x8* v,
                                               std::integer_sequence<int, HC...>) {
  ((v[HC] = lds_read2st64<HC, HC + SECOND>(addr)), ...);
}
// Wait for every outstanding LDS read of the wave, then hand the operands
// read by lds_read2st64 on to the compiler (each tied to a real instruction,
// so no use can be scheduled before the wait).
template <typename T, int N>
__device__ __forceinline__ void wait_lds_operands(T (&v)[N]) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(v[0]));
#pragma unroll
  for (int i = 1; i < N; ++i) asm volatile("s_nop 0" : "+v"(v[i]));
}

// Growth of a column's maximum (exp2 domain) below which the running max is
// kept: probabilities then reach at most 2^kRescaleSlack, far inside bf16
// and fp32 range, and the accumulators are rescaled only when some column's
// maximum grows by more than that.
constexpr float kRescaleSlack = 8.0f;

// BS8: pools of 8-token blocks.  A stage still holds 16-token tiles in the
// pool's 16-token layout (the compute below is the same); each is gathered
// from two 8-token pool tiles with per-lane addresses.
template <int D, bool KV8, bool BS8 = false>
__device__ __forceinline__ void run_tile(const AttendParams& P,
                                         const WorkItem& it, int kvh, int lane,
                                         int wslot, uint8_t* ring) {
  static_assert(!(KV8 && BS8), "8-token blocks: bf16 pools only");
  constexpr int KC = D / 32;
  constexpr int NT = D / 16;
  constexpr int CT = kPrefillColTiles;
  constexpr int NS = kPairStages;
  constexpr int TB = tile_bytes<D, KV8>();        // bytes of one K or V tile
  constexpr int SB = pair_stage_bytes<D, KV8>();  // bytes of one stage
  constexpr int LPS = TB / 1024;  // 1 KiB loads per wave per stage
  constexpr int NU = D / 64;      // 8-bit pools: 16-byte units per lane per tile
  const int g = lane >> 4;

  // this wave's token slice of the tile
  const int tw = prefill_wave_tokens(P.G);
  const int wofs = wslot * tw;
  WorkItem wt = it;
  wt.tok0 = it.tok0 + wofs;
  wt.ntok = min(tw, it.ntok - wofs);
  wt.posbase = it.posbase + wofs;
  wt.pbase = it.pbase >= 0 ? it.pbase + wofs * it.nsplit : -1;
  const bool active = wt.ntok > 0;
  const int wlast = active ? wt.posbase + wt.ntok - 1 : -1;  // causal limit

  bf16x8 qop[CT][KC];
  int cpos[CT];
  load_query<D, CT>(P, wt, kvh, lane, wt.posbase, qop, cpos);

  // Per column: reference max mref (exp2 domain; probabilities are
  // exp2(s * c - mref)), the value subtracted (0 while no key was seen), PV
  // accumulators and the column sums of P.
  f32x4 acc[CT][NT], lacc[CT];
  float mref[CT], msub[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    mref[ct] = -INFINITY;
    msub[ct] = 0.0f;
    lacc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[ct][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  bf16x8 ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = (__bf16)1.0f;

  const int jb0 = it.kv0 >> 4;
  const int nblk = ((it.kv1 + kBlock - 1) >> 4) - jb0;
  const int npairs = (nblk + 1) >> 1;
  const int32_t* btrow = P.bt + (int64_t)it.seq * P.bt_stride + (BS8 ? 2 * jb0 : jb0);
  // 8-token blocks of the item's keys, from block 2 * jb0
  const int nblk8 = BS8 ? ((it.kv1 + 7) >> 3) - 2 * jb0 : 0;
  // Wave w loads tile w of every stage: K(first), V(first), K(second),
  // V(second) -- 1 KiB per load, in pool order.
  const uint8_t* pool =
      reinterpret_cast<const uint8_t*>((wslot & 1) ? P.v_cache : P.k_cache);
  const int half = wslot >> 1;

  // physical ids of 64 blocks (32 pairs; 8-token blocks: 16 pairs) from the
  // first block of pair idbase, one per lane, clamped to the item's last
  // block (a clamped copy only fills keys that are masked)
  constexpr int kPairsPerIds = BS8 ? 16 : 32;
  auto load_ids = [&](int pr0) {
    const int jr = BS8 ? min(4 * pr0 + lane, nblk8 - 1) : min(2 * pr0 + lane, nblk - 1);
    const int id = btrow[jr];
    const int idc = id < 0 ? 0 : (id >= P.num_blocks ? (int)(P.num_blocks - 1) : id);
    return (int)((uint32_t)idc * (uint32_t)P.Hkv + (uint32_t)kvh);
  };
  int idbase = 0;
  int idv = load_ids(0);
  // 8-token blocks: this lane's byte offset inside a pool tile of 8 * D and
  // which of the 16-key group's two blocks it reads (K: token lane % 16 of
  // 8-dim chunk lane / 16; V: the 8-byte runs of key group (lane / 8) % 4 at
  // dims lane % 8 * 2 and + 1 of region lane / 32), for the first KiB of the
  // stage tile; each later KiB lies 512 bytes further
  constexpr uint32_t TB8 = TB / 2;
  const bool vwave = (wslot & 1) != 0;
  const uint32_t lane_off8 = vwave ? (uint32_t)((lane >> 5) * 256 + ((lane >> 3) & 1) * 128 +
                                                (lane & 7) * 16)
                                   : (uint32_t)((lane >> 4) * 128 + (lane & 7) * 16);
  const bool second8 = vwave ? ((lane >> 4) & 1) != 0 : ((lane >> 3) & 1) != 0;

  // LDS byte address of this wave's tile in stage 0 (stage s: + s * stage bytes)
  const uint32_t ring_lds = lds_addr(ring) + (uint32_t)(wslot * TB);
  auto issue = [&](int slot, int pr) {
    if (pr >= idbase + kPairsPerIds) {  // pairs are issued in order
      idbase += kPairsPerIds;
      idv = load_ids(idbase);
    }
    if constexpr (BS8) {
      // tile indices id * Hkv + kvh of the 16-key group's two 8-token blocks
      const int e = 4 * (pr - idbase) + 2 * half;
      const uint32_t ta = (uint32_t)__builtin_amdgcn_readlane(idv, e);
      const uint32_t tb = (uint32_t)__builtin_amdgcn_readlane(idv, e + 1);
      const uint64_t addr =
          (uint64_t)(uintptr_t)pool + (uint64_t)(second8 ? tb : ta) * TB8 + lane_off8;
      load_lds_kib_lanes<LPS>(addr, ring_lds + (uint32_t)(slot * SB));
    } else {
      // tile index id * Hkv + kvh (below 2^32 for any pool the device holds)
      const uint32_t tix = (uint32_t)__builtin_amdgcn_readlane(idv, 2 * (pr - idbase) + half);
      const uint16_t* src = reinterpret_cast<const uint16_t*>(pool + (uint64_t)tix * TB);
      load_lds_kib<LPS>(src, (uint32_t)lane * 16, ring_lds + (uint32_t)(slot * SB));
    }
  };

  // Scores of one pair of blocks (stage st): sa for the first block, sb
  // for the second; each K operand feeds the MFMAs of every column tile.
  auto scores = [&](const uint8_t* st, f32x4 (&sa)[CT], f32x4 (&sb)[CT]) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      sa[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      sb[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      bf16x8 ka, kb;
      if constexpr (KV8) {
        // unit c/2 holds the codes of chunks c (even: bytes 0-7) and c + 1
        const u32x4 ua = *reinterpret_cast<const u32x4*>(st + (c >> 1) * 1024 + lane * 16);
        const u32x4 ub =
            *reinterpret_cast<const u32x4*>(st + 2 * TB + (c >> 1) * 1024 + lane * 16);
        ka = (c & 1) ? e4m3x8_to_bf16(ua[2], ua[3]) : e4m3x8_to_bf16(ua[0], ua[1]);
        kb = (c & 1) ? e4m3x8_to_bf16(ub[2], ub[3]) : e4m3x8_to_bf16(ub[0], ub[1]);
      } else {
        ka = lds16(reinterpret_cast<const uint16_t*>(st + c * 1024 + lane * 16));
        kb = lds16(reinterpret_cast<const uint16_t*>(st + 2 * TB + c * 1024 + lane * 16));
      }
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        sa[ct] = mfma32(ka, qop[ct][c], sa[ct]);
        sb[ct] = mfma32(kb, qop[ct][c], sb[ct]);
      }
    }
  };

  // The 2 KC PV operands of pair pr (in stage pr % NS), read in one go: operand
  // hc = 2c + dh holds, for dim dh * D/2 + 16c + lane % 16, keys 4g .. 4g+3
  // of the first block, then the same keys of the second (the rows the score
  // MFMAs left in this lane).  bf16: region hc of a V tile is 512 bytes, and
  // the second block's tile lies 2 tiles further; 8-bit: the reads fetch the
  // lane's raw units, converted in softmax_pv (operand 4p + w from word w of
  // unit p of each block).
  using VRaw = typename std::conditional<KV8, u32x4, bf16x8>::type;
  constexpr int NV = KV8 ? 2 * NU : 2 * KC;
  const uint32_t vbase = lds_addr(ring) + (uint32_t)(TB + lane * (KV8 ? 16 : 8));
  auto read_v = [&](int pr, VRaw (&vraw)[NV]) {
    const uint32_t a = vbase + (uint32_t)((pr % NS) * SB);
    if constexpr (KV8)
      read_v8_units<2 * TB>(a, vraw, vraw + NU, std::make_integer_sequence<int, NU>{});
    else
      read_v_regions<TB / 256>(a, vraw, std::make_integer_sequence<int, 2 * KC>{});
  };

  // Softmax and PV of one pair of blocks from its scores.  MASKED: the pair
  // holds keys past some column's position or past kv1 (the diagonal and
  // the range end); otherwise the step is straight-line code apart from
  // the rare rescale.
  auto softmax_pv = [&](int kp0, const f32x4 (&sa)[CT], const f32x4 (&sb)[CT],
                        VRaw (&vraw)[NV], auto masked) {
    constexpr bool MASKED = decltype(masked)::value;
    float x[CT][8];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[ct][i] = sa[ct][i];
        x[ct][i + 4] = sb[ct][i];
      }
    }
    if (MASKED) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kp0 + 4 * g + i;
          if (key > cpos[ct]) x[ct][i] = -INFINITY;
          if (key + kBlock > cpos[ct]) x[ct][i + 4] = -INFINITY;
        }
      }
    }
    // Each lane checks its own 8 scores of a column against the column's
    // threshold (c > 0, so max(s) * c exceeds it exactly when some lane's
    // local max does); the column max across the four lanes of a column is
    // formed only on the rare step where some column grew.
    float lm[CT];
    bool grow = false;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      float m = x[ct][0];
#pragma unroll
      for (int i = 1; i < 8; ++i) m = fmaxf(m, x[ct][i]);
      lm[ct] = m;
      grow = grow || m * P.scale_log2 > mref[ct] + kRescaleSlack;
    }
    // probabilities against the current reference, recomputed below on the
    // rare step that moves it; the common step is then one straight block
    // from the scores to the PV MFMAs
    bf16x8 pop[CT];
    auto probs = [&]() {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          pop[ct][i] = (__bf16)__builtin_amdgcn_exp2f(
              __builtin_fmaf(x[ct][i], P.scale_log2, -msub[ct]));
      }
    };
    probs();
    // (pin the common-case probabilities here: the compiler would otherwise
    // sink them past the branch)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) asm volatile("s_nop 0" ::"v"(pop[ct]));
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      // (a side effect keeps this a branch: the compiler would otherwise run
      // the rescale on every step with alpha = 1)
      asm volatile("s_nop 0");
      // move the reference to the new max where it grew past the slack;
      // alpha is exactly 1 for the columns that keep theirs
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const float mc = column_max(lm[ct]) * P.scale_log2;
        const float mnew = mc > mref[ct] + kRescaleSlack ? mc : mref[ct];
        const float alpha =
            mnew == mref[ct] ? 1.0f : __builtin_amdgcn_exp2f(mref[ct] - mnew);
        mref[ct] = mnew;
        msub[ct] = mnew == -INFINITY ? 0.0f : mnew;
        lacc[ct] *= alpha;
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[ct][n] *= alpha;
      }
      probs();
    }
    // PV (each accumulator has this one MFMA as its only use in the step,
    // so it is updated in place)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) lacc[ct] = mfma32(ones, pop[ct], lacc[ct]);
    wait_lds_operands(vraw);
    bf16x8 vop[2 * KC];
    if constexpr (KV8) {
#pragma unroll
      for (int u = 0; u < NU; ++u) {
#pragma unroll
        for (int w = 0; w < 4; ++w)
          vop[4 * u + w] = __builtin_shufflevector(e4m3x4_to_bf16(vraw[u][w]),
                                                   e4m3x4_to_bf16(vraw[NU + u][w]), 0, 1,
                                                   2, 3, 4, 5, 6, 7);
      }
    } else {
#pragma unroll
      for (int hc = 0; hc < 2 * KC; ++hc) vop[hc] = vraw[hc];
    }
#pragma unroll
    for (int hc = 0; hc < 2 * KC; ++hc) {
      bf16x8 v = vop[hc];
      if (MASKED) {
        // keys at or past kv1 may be unwritten pool slots: zero their V
        // so a 0 weight cannot meet a NaN
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kp0 + 4 * g + i;
          if (key >= it.kv1) v[i] = (__bf16)0.0f;
          if (key + kBlock >= it.kv1) v[i + 4] = (__bf16)0.0f;
        }
      }
      const int n = (hc & 1) * KC + (hc >> 1);  // dim tile of region hc
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) acc[ct][n] = mfma32(v, pop[ct], acc[ct][n]);
    }
  };

  // Pair pr lives in stage pr % NS.  Every wave issues the same number of
  // loads per stage (the prefetch is unconditional, clamped to the last
  // pair).  Step pr computes the scores of pair pr + 1 and the softmax and
  // PV of pair pr (whose scores the previous step left), so the matrix
  // cores have the next pair's score MFMAs to run while the softmax of this
  // one is on the vector ALUs.  Before step pr a wave waits until only the
  // loads of pairs pr + 2 .. are in flight, so pair pr + 1 has landed; the
  // barrier then makes every wave's tiles visible and guarantees that stage
  // (pr - 1) % NS, refilled next, has been read by all waves (its K at step
  // pr - 2, its V at step pr - 1).
  //
  // The pairs of a wave fall into three runs: pairs every key of which each
  // of its tokens sees (below the diagonal and the range end), then pairs
  // that need the mask, then pairs past its last token (the wave only keeps
  // loading and meeting the others).  One loop per run keeps each loop body
  // a single path, so the accumulators stay in place across iterations.
  static_assert(NS >= 4, "the pipelined steps read two stages and refill a third");
  const int kb = jb0 * kBlock;  // first key of pair 0
  int nmask_end = 0;            // pairs with kp0 <= wlast
  if (wlast >= kb) nmask_end = min(npairs, (wlast - kb) / (2 * kBlock) + 1);
  int nfull = 0;  // pairs with kp0 + 31 <= posbase and kp0 + 32 <= kv1
  {
    const int lim = min(wt.posbase + 1, it.kv1) - kb;  // keys below both limits
    if (lim >= 2 * kBlock) nfull = min(nmask_end, lim / (2 * kBlock));
  }
  auto stage = [&](int pr) { return ring + (pr % NS) * SB; };
#pragma unroll
  for (int s = 0; s < NS - 1; ++s) issue(s, min(s, npairs - 1));
  f32x4 sa[CT], sb[CT];
  wait_loads_and_barrier<LPS * (NS - 2)>();  // pair 0 has landed
  if (nmask_end > 0) scores(stage(0), sa, sb);
  auto step = [&](int pr) {
    wait_loads_and_barrier<LPS * (NS - 3)>();
    issue((pr + NS - 1) % NS, min(pr + NS - 1, npairs - 1));
  };
  // (the scores of pair nmask_end, computed by the last step of a wave's
  // second run, are not used: that stage holds loaded data or a clamped
  // copy, so the read stays inside the ring)
  int pr = 0;
  for (; pr < nfull; ++pr) {
    VRaw vop[NV];
    read_v(pr, vop);  // complete since the previous step's barrier
    step(pr);
    f32x4 na[CT], nb[CT];
    scores(stage(pr + 1), na, nb);
    softmax_pv((jb0 + 2 * pr) * kBlock, sa, sb, vop, std::false_type{});
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      sa[ct] = na[ct];
      sb[ct] = nb[ct];
    }
  }
  for (; pr < nmask_end; ++pr) {
    VRaw vop[NV];
    read_v(pr, vop);  // complete since the previous step's barrier
    step(pr);
    f32x4 na[CT], nb[CT];
    scores(stage(pr + 1), na, nb);
    softmax_pv((jb0 + 2 * pr) * kBlock, sa, sb, vop, std::true_type{});
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      sa[ct] = na[ct];
      sb[ct] = nb[ct];
    }
  }
  for (; pr < npairs; ++pr) step(pr);
  // the ring is free again once every load has landed and every wave is done
  wait_loads_and_barrier<0>();
  if (active) {
    // every row of the all-ones product holds the column sum
    float l[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) l[ct] = lacc[ct][0];
    finish_unit<D, CT, KV8>(P, wt, kvh, lane, acc, mref, l);
  }
}

// A work item read back from the workspace is used only if every index it
// leads to stays inside the buffers this launch was given (a stale or foreign
// workspace then costs outputs, never an out-of-bounds access).

template <int D, bool MIXED, bool KV8, bool BS8 = false>
__device__ __forceinline__ void attend_body(const AttendParams& P,
                                            uint8_t* ring) {
  const int lane = threadIdx.x & 63;
  if (P.hdr->signature != plan_signature(P)) {
    if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(&P.hdr->error, 4u);
    return;
  }
  uint32_t num_work = P.hdr->num_work;
  if ((uint64_t)num_work > (uint64_t)P.max_items * (uint64_t)P.Hkv) num_work = 0;
  uint32_t num_pre = P.hdr->num_prefill_work;
  if (num_pre > num_work) num_pre = num_work;
  // stream plans: the decode units are (range, kv head) pairs over a range
  // table whose entries are item indices in [prefill items, num_items]
  uint32_t num_items = P.hdr->num_items;
  if ((int64_t)num_items > P.max_items) num_items = 0;
  uint32_t nranges = P.hdr->num_ranges;
  const int num_pre_items = (int)(num_pre / (uint32_t)P.Hkv);
  if (nranges > (uint32_t)kMaxStreamUnits || (nranges > 0 && P.ranges == nullptr) ||
      (nranges > 0 && num_pre + nranges * (uint32_t)P.Hkv != num_work)) {
    nranges = 0;
    num_work = num_pre;  // (never: the plan writes them together)
  }
  // shared-prefix units (their own item list) come first in the prefill queue
  uint32_t num_pfx = P.pitems != nullptr ? P.hdr->num_prefix_work : 0u;
  if ((uint64_t)num_pfx > (uint64_t)P.max_pre_items * (uint64_t)P.Hkv) num_pfx = 0;
  const uint32_t Hkv = (uint32_t)P.Hkv;
  constexpr uint32_t kWpg = kAttendThreads / 64;  // waves per workgroup
  const uint32_t wslot = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t ndec = num_work - num_pre;  // decode units follow the prefill ones
  const uint32_t nq = num_pfx + num_pre;     // units of the prefill queue
  auto claim = [&](uint32_t* counter) {
    uint32_t t = 0;
    if (lane == 0) t = atomicAdd(counter, 1u);
    return __builtin_amdgcn_readfirstlane(__shfl(t, 0));
  };

  // Prefill units (tile x kv head) go to whole workgroups, decode units to
  // single waves.  In a mixed batch the first kPrefillWgNum / kPrefillWgDen
  // of the workgroups start on prefill units (workgroup i on unit i, later ones
  // from the prefill queue) and then move their waves to the decode queue;
  // the others start on decode units and, once all of their waves have run
  // out of them, take the prefill units left.  Compute-bound tiles and
  // bandwidth-bound decode thus share every CU, and a prefill-only batch
  // still uses every workgroup.  Every pass of each loop takes one queue
  // entry (one atomic increment), so the loops end; the pass bounds are a
  // second guarantee of that.
  __shared__ uint32_t next_unit[2];
  uint32_t pre_static = 0;
  //
  // The queue counters are left at zero for the next launch on the same
  // plan (one plan serves several layers): each queue is claimed exactly a
  // known number of times per launch -- once per unit processed, plus once
  // per wave (decode queue) or workgroup (prefill queue) entering it by a
  // claim -- so the claim that returns the last value is the last access to
  // that counter in this launch, and it resets the counter.
  const bool mixed = MIXED && nq > 0;
  if (mixed)
    pre_static = min(num_pfx > 0 ? gridDim.x * kPrefixWgNum / kPrefixWgDen
                                 : gridDim.x * kPrefillWgNum / kPrefillWgDen,
                     nq);
  // The decode queue is split into S shards: shard s holds decode units
  // s, s + S, s + 2S, ... (each shard a like share of the longest-first
  // order) and is served by the workgroups b = s (mod S) from a counter of
  // its own, so that claims meet on S addresses instead of one.  Within a
  // shard, units are numbered locally (unit s + S * k is local index k); the
  // shard's decode-first waves start on local units 0 .. dec_static - 1.
  const uint32_t S = min((uint32_t)kDecodeShards, gridDim.x);
  const uint32_t shard = blockIdx.x % S;
  uint32_t* const dctr = P.dec_counters + shard * kCounterStride;
  const uint32_t n_s = ndec > shard ? (ndec - shard + S - 1) / S : 0u;
  const uint32_t wg_s = (gridDim.x - shard + S - 1) / S;  // workgroups of the shard
  const uint32_t pf_s =                                   // of them prefill-first
      pre_static > shard ? min(wg_s, (pre_static - shard + S - 1) / S) : 0u;
  const uint32_t dec_static = (wg_s - pf_s) * kWpg;
  const uint32_t dec_claims = n_s + pf_s * kWpg;
  const uint32_t pre_claims = nq + (gridDim.x - pre_static);
  // one claim on the shard's counter by lane 0 (t: the value it returned)
  auto dec_claimed = [&](uint32_t t) {
    if (t + 1u == dec_claims && lane == 0) atomicExch(dctr, 0u);
    return t + dec_static;
  };
  auto pre_claim = [&]() {  // thread 0 only
    const uint32_t t = atomicAdd(&P.hdr->prefill_counter, 1u);
    if (t + 1u == pre_claims) atomicExch(&P.hdr->prefill_counter, 0u);
    return t + pre_static;
  };
  auto prefill_units = [&](uint32_t u) {
    int k = 0;
    for (uint32_t pass = 0; u < nq && pass <= nq; ++pass) {
      const bool pfx = u < num_pfx;
      const uint32_t w = pfx ? u : u - num_pfx;
      const WorkItem it = pfx ? P.pitems[w / Hkv] : P.items[w / Hkv];
      if (item_ok(P, it) && it.kind == (pfx ? kKindPrefix : kKindPrefill))
        run_tile<D, KV8, BS8>(P, it, (int)(w % Hkv), lane, (int)wslot, ring);
      if (threadIdx.x == 0) next_unit[k] = pre_claim();
      __syncthreads();
      u = __builtin_amdgcn_readfirstlane(next_unit[k]);
      k ^= 1;
    }
  };
  const DecodeQueue dq{dctr, num_pre + shard, S, n_s, dec_static, dec_claims, nranges == 0};
  auto decode_units = [&](uint32_t k) {  // k: local index in the shard
    NextUnit nx{k, 0, 0, false, false};
    for (uint32_t pass = 0; nx.k < n_s && pass <= n_s; ++pass) {
      const uint32_t w = num_pre + shard + S * nx.k;
      if (nranges == 0) {  // the unit is one item
        if (!nx.item_ready) nx.itv = load_item_lanes(P.items, w / Hkv, lane);
        const WorkItem it = item_of_lanes(nx.itv);
        if (item_ok(P, it) && it.kind == kKindDecode) {
          run_unit<D, kDecodeColTiles, kDecodeStages, true, KV8, BS8>(P, it, (int)(w % Hkv),
                                                                       lane, dq, nx, -1);
        } else {
          nx.k = dec_claimed(claim(dctr));
          nx.item_ready = nx.ids_ready = false;
        }
        continue;
      }
      // stream plans: the unit is the items of range r for kv head kvh
      const uint32_t d = w - num_pre;
      const uint32_t r = d / Hkv;
      const int kvh = (int)(d % Hkv);
      int i0 = P.ranges[r], i1 = P.ranges[r + 1];
      if (i0 < num_pre_items || i1 > (int)num_items || i1 <= i0) i1 = i0;  // (never: no items)
      nx.item_ready = nx.ids_ready = false;
      bool done = false;
      for (int i = i0; i < i1; ++i) {
        if (!nx.item_ready) nx.itv = load_item_lanes(P.items, (uint32_t)i, lane);
        const WorkItem it = item_of_lanes(nx.itv);
        const bool last = i + 1 == i1;
        if (item_ok(P, it) && it.kind == kKindDecode) {
          run_unit<D, kDecodeColTiles, kDecodeStages, true, KV8, BS8>(P, it, kvh, lane, dq,
                                                                       nx, last ? -1 : i + 1);
          done = last;
        } else {
          nx.item_ready = nx.ids_ready = false;
        }
      }
      if (!done) {  // the unit's claim, if its last item did not make it
        nx.k = dec_claimed(claim(dctr));
        nx.item_ready = nx.ids_ready = false;
      }
    }
  };
  const uint32_t static_k = (blockIdx.x / S - pf_s) * kWpg + wslot;
  if (!mixed) {
    decode_units(static_k);
    return;
  }
  const bool prefill_first = blockIdx.x < pre_static;
  uint32_t u = blockIdx.x;
  if (!prefill_first) {
    // decode first, then (all waves done) the prefill units left
    decode_units(static_k);
    __syncthreads();
    if (threadIdx.x == 0) next_unit[0] = pre_claim();
    __syncthreads();
    u = __builtin_amdgcn_readfirstlane(next_unit[0]);
  }
  prefill_units(u);
  if (prefill_first) decode_units(dec_claimed(claim(dctr)));
}

// Decode-only batches: registers for the 3-stage pipeline and the next
// item's prefetch (two waves per SIMD for head_dim 128, three for 64; three
// for 128 with 8-bit pools, whose blocks take half the registers and which
// do not prefetch).
template <int D, bool KV8>
__global__ __launch_bounds__(kAttendThreads)
__attribute__((amdgpu_waves_per_eu(D == 64 ? 3 : (KV8 ? 3 : 2), 8)))
void attend_decode_kernel(AttendParams P) {
  attend_body<D, false, KV8>(P, nullptr);
}

// Mixed batches: prefill tiles and decode units in the same launch.
template <int D, bool KV8>
__global__ __launch_bounds__(kAttendThreads)
__attribute__((amdgpu_waves_per_eu(2, 8)))
void attend_mixed_kernel(AttendParams P) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[prefill_ring_bytes<D, KV8>()];
  attend_body<D, true, KV8>(P, ring);
}

// The same two kernels over pools of 8-token blocks (bf16).
template <int D>
__global__ __launch_bounds__(kAttendThreads)
__attribute__((amdgpu_waves_per_eu(D == 64 ? 3 : 2, 8)))
void attend_decode_bs8_kernel(AttendParams P) {
  attend_body<D, false, false, true>(P, nullptr);
}

template <int D>
__global__ __launch_bounds__(kAttendThreads)
__attribute__((amdgpu_waves_per_eu(2, 8)))
void attend_mixed_bs8_kernel(AttendParams P) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[prefill_ring_bytes<D, false>()];
  attend_body<D, true, false, true>(P, ring);
}

// ---------------------------------------------------------------------------
// merge
// ---------------------------------------------------------------------------

// Online log-sum-exp state of one column over the lane's 8 dims: running
// max M (log2 domain), denominator and the two 4-dim numerator halves.
struct MergeState {
  float M, den;
  f32x4 n0, n1;
};

// Folds one partial (running max m, sum l, accumulator a0|a1) into st.
__device__ __forceinline__ void merge_fold(MergeState& st, float m, float l, f32x4 a0,
                                           f32x4 a1) {
  const float mn = fmaxf(st.M, m);
  const float mu = (mn == -INFINITY) ? 0.0f : mn;
  const float c_old = __builtin_amdgcn_exp2f(st.M - mu);
  const float c_new = __builtin_amdgcn_exp2f(m - mu);
  st.den = st.den * c_old + l * c_new;
  st.n0 = st.n0 * c_old + a0 * c_new;
  st.n1 = st.n1 * c_old + a1 * c_new;
  st.M = mn;
}

// W passes per (split tile, kv head), W = the passes one token's G columns
// take (at most 4): the tile's columns of that kv head are dealt to them
// round-robin, 64 / (D/8) at a time (lanes cover (column, 8 dims)).  One
// workgroup per (split tile, kv head, pass): its 4 waves fold consecutive
// quarters of each column's partials (a shared prefix's first, then the
// tile's own splits, in split order, two splits' loads in flight per lane),
// and wave 0 folds the 4 wave states in wave order: a fixed order, so the
// result does not depend on timing, and a long chain of splits is 4 chains
// of a quarter.  Two splits per step keep the kernel at 64 registers, eight
// waves per SIMD, so that a launch of up to 8 workgroups per CU is one
// round (eight splits per step: 121 registers, four waves per SIMD; measured
// 7.1 -> 5.1 us on 2040 (tile, kv head) units, 4.1 -> 3.8 us on the 8B
// decode layer, 7.5 -> 8.3 us on one request of 128 splits).
__host__ __device__ inline uint32_t merge_waves_per_head(int G, int D) {
  const int cpw = 64 / (D / 8);
  const int w = (G + cpw - 1) / cpw;
  return (uint32_t)(w < 1 ? 1 : (w > 4 ? 4 : w));
}
template <int D>
__global__ __launch_bounds__(kAttendThreads)
__attribute__((amdgpu_waves_per_eu(8, 8))) void merge_kernel(AttendParams P) {
  constexpr int LPC = D / 8;      // lanes per column
  constexpr int CPW = 64 / LPC;   // columns per wave pass
  constexpr int SB = 2;           // splits per step
  constexpr int NW = kAttendThreads / 64;
  __shared__ float4 wstate[NW - 1][3][64];  // waves 1..: (M, den), n0, n1 per lane
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int G = P.G;
  const uint32_t W = merge_waves_per_head(G, D);
  const uint32_t per_tile = (uint32_t)P.Hkv * W;
  // the list entry of the workgroup's first unit, loaded beside the header
  // (any entry within the list's capacity may be read; it is used only if
  // the header lists it)
  const uint32_t first_tile = blockIdx.x / per_tile;
  const int4 tile0 = (int64_t)first_tile < P.max_items ? P.merge_list[first_tile]
                                                       : make_int4(-1, 0, 0, 0);
  if (P.hdr->signature != plan_signature(P)) return;
  uint32_t ntiles = P.hdr->num_split_tiles;
  if ((int64_t)ntiles > P.max_items) ntiles = 0;
  // shared-prefix plans: every listed token first combines its npre prefix
  // partials (slots t * npre + s of the prefix section), then its own
  int npre = P.pre_ml != nullptr ? (int)P.hdr->prefix_splits : 0;
  if (npre < 0 || npre > kMaxPrefixSplits ||
      (int64_t)P.num_q_tokens * npre > P.max_pre_partials)
    ntiles = 0;
  const uint32_t nunits = ntiles * per_tile;
  const int cl = lane / LPC;          // column within the pass
  const int d0 = (lane % LPC) * 8;    // first of the lane's 8 dims
  for (uint32_t u = blockIdx.x; u < nunits; u += gridDim.x) {
    // tok0, ntok, nsplit, pbase
    int4 tile = tile0;
    if (u != blockIdx.x) tile = P.merge_list[u / per_tile];
    const int kvh = (int)((u % per_tile) / W);
    const int pass0 = (int)(u % W);
    // same rule as for work items: never follow an entry out of bounds
    // (the same decision in every wave of the workgroup)
    if (tile.x < 0 || tile.y < 1 || tile.x + tile.y > P.num_q_tokens ||
        tile.z < (npre > 0 ? 1 : 2) || tile.w < 0 ||
        (int64_t)tile.w + (int64_t)tile.y * tile.z > P.max_partials)
      continue;
    const int ncols = tile.y * G;
    const int nsplit = tile.z;
    const int nall = npre + nsplit;
    const int s_lo = wave * nall / NW, s_hi = (wave + 1) * nall / NW;
    for (int c0 = pass0 * CPW; c0 < ncols; c0 += (int)W * CPW) {
      const int c = c0 + cl;
      const bool valid = c < ncols;
      const int tk = valid ? c / G : 0;
      const int h = kvh * G + (c - tk * G);
      const int64_t tok = (int64_t)(tile.x + tk);
      const int64_t slot0 = (int64_t)tile.w + (int64_t)tk * nsplit;
      MergeState st{-INFINITY, 0.0f, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      if (valid) {
        for (int s0 = s_lo; s0 < s_hi; s0 += SB) {
          float2 ml[SB];
          f32x4 a0[SB], a1[SB];
#pragma unroll
          for (int k = 0; k < SB; ++k) {
            const int sp = s0 + k;
            if (sp < s_hi) {
              const bool pre = sp < npre;
              const int64_t row = (pre ? tok * npre + sp : slot0 + (sp - npre)) * P.Hq + h;
              ml[k] = (pre ? P.pre_ml : P.part_ml)[row];
              const f32x4* ap = reinterpret_cast<const f32x4*>(
                  (pre ? P.pre_acc : P.part_acc) + row * D + d0);
              a0[k] = ap[0];
              a1[k] = ap[1];
            } else {
              ml[k] = make_float2(-INFINITY, 0.0f);
              a0[k] = f32x4{0.f, 0.f, 0.f, 0.f};
              a1[k] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
          }
#pragma unroll
          for (int k = 0; k < SB; ++k) merge_fold(st, ml[k].x, ml[k].y, a0[k], a1[k]);
        }
      }
      if (wave > 0) {
        wstate[wave - 1][0][lane] = make_float4(st.M, st.den, 0.0f, 0.0f);
        wstate[wave - 1][1][lane] = make_float4(st.n0[0], st.n0[1], st.n0[2], st.n0[3]);
        wstate[wave - 1][2][lane] = make_float4(st.n1[0], st.n1[1], st.n1[2], st.n1[3]);
      }
      __syncthreads();
      if (wave == 0 && valid) {
#pragma unroll
        for (int w = 0; w < NW - 1; ++w) {
          const float4 md = wstate[w][0][lane], x0 = wstate[w][1][lane],
                       x1 = wstate[w][2][lane];
          merge_fold(st, md.x, md.y, f32x4{x0.x, x0.y, x0.z, x0.w},
                     f32x4{x1.x, x1.y, x1.z, x1.w});
        }
        const float inv = 1.0f / st.den;
        bf16x8 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          o[i] = (__bf16)(st.n0[i] * inv);
          o[i + 4] = (__bf16)(st.n1[i] * inv);
        }
        *reinterpret_cast<bf16x8*>(P.out + (tok * P.Hq + h) * D + d0) = o;
      }
      __syncthreads();  // wstate is rewritten by the next pass
    }
  }
}

// Resident workgroups per CU of a kernel (queried once per device).
int resident_wgs(const void* fn, int slot) {
  static std::mutex mu;
  static std::vector<int> cache;  // [device * 16 + slot]
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 1;
  std::lock_guard<std::mutex> lock(mu);
  const size_t idx = (size_t)dev * 16 + slot;
  if (cache.size() <= idx) cache.resize(idx + 1, 0);
  if (cache[idx] == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, kAttendThreads, 0) !=
            hipSuccess ||
        n < 1)
      n = 1;
    cache[idx] = n;
  }
  return cache[idx];
}

}  // namespace

namespace {

AttendParams make_params(const AttendArgs& a) {
  AttendParams P;
  P.q = a.q;
  P.k_cache = a.k_cache;
  P.v_cache = a.v_cache;
  P.num_blocks = a.num_blocks;
  P.bt = a.block_tables;
  P.bt_stride = a.bt_stride;
  P.seq_lens = a.seq_lens;
  P.qsl = a.qsl;
  P.num_seqs = a.num_seqs;
  P.num_q_tokens = (int32_t)a.num_q_tokens;
  P.Hq = a.num_q_heads;
  P.Hkv = a.num_kv_heads;
  P.G = a.num_q_heads / a.num_kv_heads;
  P.max_query_len = a.max_query_len;
  P.max_seq_len = a.max_seq_len;
  // 8-bit pools: a K code stands for code * k_scale, folded into the score
  // scale; V's scale is applied to the outputs
  P.scale_log2 = a.kv8 ? a.scale * a.k_scale * kLog2e : a.scale * kLog2e;
  P.v_scale = a.kv8 ? a.v_scale : 1.0f;
  P.out = a.out;
  char* ws = static_cast<char*>(a.workspace);
  P.hdr = reinterpret_cast<PlanHeader*>(ws);
  P.dec_counters = reinterpret_cast<uint32_t*>(ws + a.ws.counters);
  P.items = reinterpret_cast<WorkItem*>(ws + a.ws.items);
  P.merge_list = reinterpret_cast<int4*>(ws + a.ws.merge_list);
  P.part_ml = reinterpret_cast<float2*>(ws + a.ws.part_ml);
  P.part_acc = reinterpret_cast<float*>(ws + a.ws.part_acc);
  P.max_items = a.ws.max_items;
  P.max_partials = a.ws.max_partials;
  P.pitems = a.cascade ? reinterpret_cast<WorkItem*>(ws + a.ws.pre_items) : nullptr;
  P.pre_ml = a.cascade ? reinterpret_cast<float2*>(ws + a.ws.pre_ml) : nullptr;
  P.pre_acc = a.cascade ? reinterpret_cast<float*>(ws + a.ws.pre_acc) : nullptr;
  P.max_pre_items = a.cascade ? a.ws.max_pre_items : 0;
  P.max_pre_partials = a.cascade ? a.ws.max_pre_partials : 0;
  P.prefix_len = a.cascade ? a.prefix_len : 0;
  P.split_decode = (a.kv8 && !a.cascade && a.max_query_len <= decode_tile_tokens(P.G))
                       ? kSplitDecode8 : kSplitDecode;
  P.bs_shift = a.block_size == 8 ? 3 : 4;
  // units wanted: 4 per CU over bf16 pools (one per SIMD), 8 over 8-bit
  // pools, whose dequantisation needs two waves per SIMD to keep up with
  // the stream (8B decode layer, 8-bit: 49 -> 72 us with 4 units per CU as a
  // stream plan, 51 -> 48 us with 8)
  P.long_units = (a.num_cus > 0 ? a.num_cus : 1) * (a.kv8 ? kUnitsPerCu8 : kLongUnitsPerCu);
  // (a plan of either kind serves either pool type, so every launch reads
  // the table)
  P.ranges = reinterpret_cast<int32_t*>(ws + a.ws.ranges);
  P.min_range_pairs = (a.kv8 ? kMinRangeKeys8 : kMinRangeKeys) / 32;
  return P;
}

}  // namespace

hipError_t launch_plan(const AttendArgs& a, hipStream_t stream) {
  if (a.num_q_tokens == 0 || a.num_seqs == 0) return hipSuccess;
  const AttendParams P = make_params(a);
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, P);
  return hipGetLastError();
}

hipError_t launch_write_plan(const AttendArgs& a, const ScatterArgs& s,
                             hipStream_t stream) {
  if (a.num_q_tokens == 0 || a.num_seqs == 0) return hipErrorInvalidValue;
  if (s.num_tokens == 0) return launch_plan(a, stream);
  const AttendParams P = make_params(a);
  // scatter threads: one per (quad of new tokens, kv head, 16-byte unit).
  // A decode step's scatter is small and its V stores are scattered 1- or
  // 2-byte writes, limited per CU: spread it over every CU (whole waves,
  // at most kPlanThreads per workgroup).
  const int64_t units = a.kv8 ? a.head_dim / 4 : a.head_dim / 8;
  const int64_t threads = ((s.num_tokens + 3) / 4) * s.Hkv * units;
  const int64_t cus = a.num_cus > 0 ? a.num_cus : 1;
  int64_t per = ((threads + cus - 1) / cus + 63) / 64 * 64;
  per = per < 64 ? 64 : (per > kPlanThreads ? kPlanThreads : per);
  ScatterArgs sc = s;
  sc.per_block = (int)per;
  const dim3 grid((unsigned)(1 + (threads + per - 1) / per));
  void (*fn)(AttendParams, ScatterArgs);
  if (a.head_dim == 128)
    fn = a.kv8 ? write_plan_kernel<128, true> : write_plan_kernel<128, false>;
  else
    fn = a.kv8 ? write_plan_kernel<64, true> : write_plan_kernel<64, false>;
  hipLaunchKernelGGL(fn, grid, dim3(kPlanThreads), 0, stream, P, sc);
  return hipGetLastError();
}

hipError_t launch_planned(const AttendArgs& a, hipStream_t stream) {
  if (a.num_q_tokens == 0 || a.num_seqs == 0) return hipSuccess;
  const AttendParams P = make_params(a);
  // (a shared-prefix plan has prefill-kind tiles even in a decode batch)
  const bool decode_only = !a.cascade && a.max_query_len <= decode_tile_tokens(P.G);
  void (*fn)(AttendParams);
  int slot;
  if (a.head_dim == 128) {
    if (a.kv8)
      fn = decode_only ? attend_decode_kernel<128, true> : attend_mixed_kernel<128, true>;
    else
      fn = decode_only ? attend_decode_kernel<128, false> : attend_mixed_kernel<128, false>;
    slot = decode_only ? 0 : 1;
  } else {
    if (a.kv8)
      fn = decode_only ? attend_decode_kernel<64, true> : attend_mixed_kernel<64, true>;
    else
      fn = decode_only ? attend_decode_kernel<64, false> : attend_mixed_kernel<64, false>;
    slot = decode_only ? 2 : 3;
  }
  if (a.kv8) slot += 4;
  if (a.block_size == 8) {  // bf16 pools of 8-token blocks (checked by the caller)
    if (a.head_dim == 128)
      fn = decode_only ? attend_decode_bs8_kernel<128> : attend_mixed_bs8_kernel<128>;
    else
      fn = decode_only ? attend_decode_bs8_kernel<64> : attend_mixed_bs8_kernel<64>;
    slot = 8 + (decode_only ? 0 : 1) + (a.head_dim == 128 ? 0 : 2);
  }
  // Persistent grid: every resident slot of every CU, never more workgroups
  // than the work-unit bound (a decode unit takes one wave, a prefill unit a
  // whole workgroup: bounding a mixed launch by units per wave left a
  // prefill-only batch with about one workgroup per CU).
  const int64_t max_work =
      (a.ws.max_items + (a.cascade ? a.ws.max_pre_items : 0)) * a.num_kv_heads;
  int64_t wgs = (int64_t)a.num_cus * resident_wgs((const void*)fn, slot);
  const int64_t need = decode_only
                           ? (max_work + (kAttendThreads / 64) - 1) / (kAttendThreads / 64)
                           : max_work;
  if (wgs > need) wgs = need;
  if (wgs < 1) wgs = 1;
  hipLaunchKernelGGL(fn, dim3((unsigned)wgs), dim3(kAttendThreads), 0, stream, P);
  return hipGetLastError();
}

// The workspace of pa_attend_noalloc: a file-scope device array, one copy per
// device, allocated with the code object when it is loaded on that device.
// In host code its name stands for a host-side placeholder, not a device
// address: scratch_address() looks up the current device's copy, and only
// that address is ever handed to a kernel.
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

hipError_t scratch_address(void** ptr) {
  static std::mutex mu;
  static std::vector<void*> cache;  // [device]
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)cache.size() <= dev) cache.resize(dev + 1, nullptr);
  if (cache[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr || ((uintptr_t)p & 255)) return hipErrorInvalidSymbol;
    cache[dev] = p;
  }
  *ptr = cache[dev];
  return hipSuccess;
}

hipError_t launch_merge(const AttendArgs& a, hipStream_t stream) {
  if (a.num_q_tokens == 0 || a.num_seqs == 0) return hipSuccess;
  // Without a shared prefix, a request of at most min(decode split, prefill
  // split) keys is one key range, whatever its kind and its batch: a plan
  // for such lengths has no split tile, and nothing is launched.
  if (!a.cascade && a.max_seq_len <= kOneRangeKeys) return hipSuccess;
  const AttendParams P = make_params(a);
  // one workgroup per (split tile, kv head, pass), at most 8 per CU (the
  // workgroups stride over the units); a split tile holds at least one query
  // token of its own, so there are at most num_q_tokens of them
  const int64_t max_tiles =
      a.ws.max_items < a.num_q_tokens ? a.ws.max_items : a.num_q_tokens;
  int64_t mwgs = max_tiles * a.num_kv_heads *
                 merge_waves_per_head(a.num_q_heads / a.num_kv_heads, a.head_dim);
  const int64_t cap = (int64_t)a.num_cus * 8;
  if (mwgs > cap) mwgs = cap;
  if (mwgs < 1) mwgs = 1;
  if (a.head_dim == 128)
    hipLaunchKernelGGL(merge_kernel<128>, dim3((unsigned)mwgs), dim3(kAttendThreads),
                       0, stream, P);
  else
    hipLaunchKernelGGL(merge_kernel<64>, dim3((unsigned)mwgs), dim3(kAttendThreads),
                       0, stream, P);
  return hipGetLastError();
}

}  // namespace pa
