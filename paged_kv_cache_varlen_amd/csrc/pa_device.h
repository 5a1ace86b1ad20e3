// Internal declarations shared by the HIP kernels and the C-ABI host code of
// libpa.so.  gfx950 (CDNA4) only: 64-lane wavefronts, bf16 MFMA.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

constexpr int kBlock = 16;  // tokens per KV block

// Work decomposition of pa_attend (see attend.hip).
// Decode splits: 512 logical tokens.  Requests longer than kLongDecode are
// cut into ranges of 1024, 2048, 4096 or 8192 keys, one length per plan: the
// shortest for which the batch's long-request units number at most
// kLongUnitsPerCu per CU (one per SIMD), else 8192.  Measured on MI355X,
// long ranges streamed as one unbroken pass per SIMD read faster than twice
// as many shorter units in two rounds (16 x 32768 keys, GQA 8: 351 -> 322 us;
// 4 to 32 requests of 32768 keys: 81-84% of 8 TB/s), while half a unit per
// SIMD leaves bandwidth unused.  A short request's split depends on its own
// length only; a long request's also on the batch's other long requests.
constexpr int kSplitDecode = 512;
// 8-bit pools, decode-only batches: their units stream twice as fast, and
// shorter key ranges balance the launch better (measured: 384 keys, 11%
// faster attention on the Llama-3-8B decode layer; mixed batches and bf16
// pools keep 512).
constexpr int kSplitDecode8 = 384;
constexpr int kSplitLongMin = 1024;  // long decode splits: 1024 .. 8192 keys
constexpr int kSplitLongMax = 8192;
constexpr int kLongUnitsPerCu = 4;  // (also the stream units per CU over bf16 pools)
constexpr int kLongDecode = 8192;
// Stream partition of a plan's decode requests (see attend.hip): at most
// kMaxStreamUnits (range, kv head) units, ranges of at least kMinRangeKeys
// keys.
constexpr int kMaxStreamUnits = 2048;
constexpr int kMinRangeKeys = 512;
// 8-bit pools: twice the units (kUnitsPerCu8 per CU), ranges of at least
// 384 keys (a request then still has at most ceil(L / 384) + 1 pieces)
constexpr int kUnitsPerCu8 = 8;
constexpr int kMinRangeKeys8 = 384;
constexpr int kSplitPrefill = 2048;  // logical tokens per prefill split
// A prefill request is split along its keys only if it has fewer than this
// many (query tile x kv head) work units on its own.
constexpr int kPrefillUnsplitUnits = 256;
constexpr int kDecodeColTiles = 1;   // 16 MFMA columns: up to 16/G tokens
constexpr int kPrefillColTiles = 2;  // per wave: 32 MFMA columns, 32/G tokens
constexpr int kPrefillWaves = 4;     // waves sharing one prefill tile's K/V
constexpr int kMaxGroup = 16;        // query heads per kv head
constexpr int kAttendThreads = 256;  // 4 waves per workgroup
// The decode queue is served from kDecodeShards counters, kCounterStride
// words (4 KiB) apart, so that claims spread over several memory channels.
constexpr int kDecodeShards = 8;
constexpr int kCounterStride = 1024;
// Shared-prefix (cascade) plans: the common prefix is cut into at most
// kMaxPrefixSplits key ranges of about kPrefixSplitKeys keys each.
constexpr int kMaxPrefixSplits = 8;
constexpr int kPrefixSplitKeys = 2048;

// kKindPrefix: a tile of consecutive query tokens of the whole batch (any
// requests) against a key range of the common prefix, read through request
// 0's block table, writing partials into the prefix section.
enum ItemKind : int { kKindDecode = 0, kKindPrefill = 1, kKindPrefix = 2 };

// One unit of attention work for all kv heads: a tile of consecutive query
// tokens of one request against one logical key range of that request.
struct WorkItem {
  int32_t seq;      // request index b
  int32_t tok0;     // global index of the tile's first query token
  int32_t ntok;     // tokens in the tile
  int32_t kind;     // ItemKind
  int32_t kv0;      // first logical key (multiple of 32)
  int32_t kv1;      // one past the last logical key
  int32_t split;    // split index of this key range
  int32_t nsplit;   // splits of this tile
  int32_t pbase;    // partial slot of (tile token 0, split 0); -1: the output
                    // is written directly (one split, no shared prefix)
  int32_t counter;  // index of the tile in the merge list; -1 if unsplit
  int32_t posbase;  // logical position of the tile's first query token
  int32_t pad[5];
};
static_assert(sizeof(WorkItem) == 64, "WorkItem is one 64-byte scalar load");

// Workspace header, at offset 0 of the workspace.
struct PlanHeader {
  uint32_t num_work;      // items * num_kv_heads (prefill units first)
  uint32_t num_items;
  uint32_t error;         // bit0: capacity exceeded, bit1: bad request skipped
  uint32_t num_split_tiles;  // entries of the merge list
  uint32_t signature;     // hash of the arguments the plan was made for
  uint32_t prefill_counter;   // prefill queue head (zeroed by the plan)
  uint32_t num_prefill_work;  // prefill items * num_kv_heads
  uint32_t num_prefix_work;   // shared-prefix items * num_kv_heads
  uint32_t prefix_splits;     // key ranges of the shared prefix (0: none)
  uint32_t num_ranges;        // stream ranges of the decode items (0: one unit per item)
};

// Byte offsets of the workspace sections.
struct WorkspaceLayout {
  size_t counters;      // uint32[kDecodeShards * kCounterStride] decode queue heads
  size_t items;         // WorkItem[max_items]
  size_t merge_list;    // int4[max_items]  split tiles: tok0, ntok, nsplit, pbase
  size_t part_ml;       // float2[max_partials * Hq]  (running max, sum)
  size_t part_acc;      // float[max_partials * Hq * D]
  size_t ranges;        // int32[kMaxStreamUnits + 1] first item of each stream range
  size_t total;
  int64_t max_items;
  int64_t max_partials;
  // Shared-prefix section, after the sections above (their offsets are the
  // same with or without it): prefix items and per-(token, prefix split)
  // partials.
  size_t pre_items;     // WorkItem[max_pre_items]
  size_t pre_ml;        // float2[max_pre_partials * Hq]
  size_t pre_acc;       // float[max_pre_partials * Hq * D]
  size_t cascade_total;
  int64_t max_pre_items;
  int64_t max_pre_partials;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Tokens per decode tile / prefill tile for group size G (<= 16).  A
// prefill tile is split between the kPrefillWaves waves of a workgroup, each
// taking prefill_wave_tokens consecutive tokens of it.
inline __host__ __device__ int decode_tile_tokens(int G) {
  return (16 * kDecodeColTiles) / G;
}
inline __host__ __device__ int prefill_wave_tokens(int G) {
  return (16 * kPrefillColTiles) / G;
}
inline __host__ __device__ int prefill_tile_tokens(int G) {
  return kPrefillWaves * prefill_wave_tokens(G);
}

inline WorkspaceLayout workspace_layout(int32_t num_seqs, int64_t num_q_tokens,
                                        int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t head_dim,
                                        int32_t max_query_len,
                                        int32_t max_seq_len) {
  WorkspaceLayout w{};
  const int G = num_q_heads / num_kv_heads;
  const int tq_d = decode_tile_tokens(G);
  const int tq_p = prefill_tile_tokens(G);
  const int64_t L = max_seq_len > 0 ? max_seq_len : 1;
  const int64_t B = num_seqs;
  const int64_t T = num_q_tokens;
  const int64_t sd = cdiv64(L, kSplitDecode8 < kSplitDecode ? kSplitDecode8 : kSplitDecode);
  const int64_t sp = cdiv64(L, kSplitPrefill);
  // decode-kind requests: one tile each; prefill-kind: <= T/tq_p + B tiles.
  int64_t dec_tiles = B;
  int64_t pre_tiles = (max_query_len > tq_d) ? (T / tq_p + B) : 0;
  // (a decode request cut by stream ranges of at least kMinRangeKeys keys
  // has at most ceil(L / 384) + 2 pieces)
  w.max_items = dec_tiles * (sd + 2) + pre_tiles * sp;
  if (w.max_items < 1) w.max_items = 1;
  // partial slots: decode tokens <= min(T, B*tq_d), prefill tokens <= T
  int64_t dec_tok = T < B * tq_d ? T : B * tq_d;
  int64_t pre_tok = (max_query_len > tq_d) ? T : 0;
  w.max_partials = dec_tok * (sd + 2) + pre_tok * sp;
  if (w.max_partials < 1) w.max_partials = 1;
  size_t off = 4096;  // the header, then the counters on their own pages
  w.counters = off;
  off += sizeof(uint32_t) * kDecodeShards * kCounterStride;
  w.items = off;
  off = align256(off + sizeof(WorkItem) * (size_t)w.max_items);
  w.merge_list = off;
  off = align256(off + 16 * (size_t)w.max_items);
  w.part_ml = off;
  off = align256(off + sizeof(float) * 2 * (size_t)w.max_partials * num_q_heads);
  w.part_acc = off;
  off = align256(off + sizeof(float) * (size_t)w.max_partials * num_q_heads *
                           (size_t)head_dim);
  w.ranges = off;
  off = align256(off + sizeof(int32_t) * (size_t)(kMaxStreamUnits + 1));
  w.total = off;
  // prefix tiles span the whole batch: ceil(T / tq_p) tiles x splits
  w.max_pre_items = cdiv64(T, tq_p) * kMaxPrefixSplits;
  if (w.max_pre_items < 1) w.max_pre_items = 1;
  w.max_pre_partials = (T > 0 ? T : 1) * kMaxPrefixSplits;
  w.pre_items = off;
  off = align256(off + sizeof(WorkItem) * (size_t)w.max_pre_items);
  w.pre_ml = off;
  off = align256(off + sizeof(float) * 2 * (size_t)w.max_pre_partials * num_q_heads);
  w.pre_acc = off;
  off = align256(off + sizeof(float) * (size_t)w.max_pre_partials * num_q_heads *
                           (size_t)head_dim);
  w.cascade_total = off;
  return w;
}

// ---- launchers (defined in the .hip files) ---------------------------------

// block_size: tokens per block of the pools, 16 or 8.
hipError_t launch_write_kv(const uint16_t* k, const uint16_t* v,
                           int64_t k_stride, int64_t v_stride,
                           const int64_t* slot_mapping, int64_t num_tokens,
                           int num_kv_heads, int head_dim, uint16_t* k_cache,
                           uint16_t* v_cache, int64_t num_blocks,
                           hipStream_t stream, int block_size = kBlock);

hipError_t launch_write_kv8(const uint16_t* k, const uint16_t* v,
                            int64_t k_stride, int64_t v_stride,
                            const int64_t* slot_mapping, int64_t num_tokens,
                            int num_kv_heads, int head_dim, float k_scale,
                            float v_scale, uint8_t* k_cache, uint8_t* v_cache,
                            int64_t num_blocks, hipStream_t stream);

hipError_t launch_gather_kv(const uint16_t* k_cache, const uint16_t* v_cache,
                            int64_t num_blocks, const int32_t* block_tables,
                            int32_t bt_stride, const int32_t* seq_lens,
                            const int64_t* kv_start, int32_t num_seqs,
                            int64_t total_rows, int num_kv_heads, int head_dim,
                            uint16_t* k_out, uint16_t* v_out,
                            hipStream_t stream, int block_size = kBlock);

// Copy-on-write: copy whole blocks (every kv head) of both pools, for the
// (src, dst) pairs of `mapping`; block_bytes = bytes of one block in a pool.
hipError_t launch_copy_blocks(void* k_cache, void* v_cache, int64_t block_bytes,
                              int64_t num_blocks, const int64_t* mapping,
                              int64_t num_pairs, hipStream_t stream);

// Block tables of R * 16-token blocks -> tables of 16-token block ids.
hipError_t launch_expand_tables(const int32_t* in, int32_t in_stride,
                                int32_t num_seqs, int R, int32_t* out,
                                hipStream_t stream);

struct AttendArgs {
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  int64_t num_blocks;
  const int32_t* block_tables;
  int32_t bt_stride;
  const int32_t* seq_lens;
  const int32_t* qsl;
  int32_t num_seqs;
  int64_t num_q_tokens;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t max_query_len;
  int32_t max_seq_len;
  float scale;
  uint16_t* out;
  void* workspace;
  WorkspaceLayout ws;
  int num_cus;
  bool cascade;    // the workspace holds the shared-prefix section
  int32_t prefix_len;  // plan: keys shared by every request (multiple of 32)
  bool kv8;        // 8-bit pools: E4M3 codes (k_cache, v_cache are uint8)
  float k_scale;   // value of a K code: code * k_scale (8-bit pools)
  float v_scale;   // value of a V code: code * v_scale (8-bit pools)
  int block_size = kBlock;  // tokens per block-table entry: 16, or 8 (bf16 pools)
};

// Work plan into the workspace (one small kernel).
hipError_t launch_plan(const AttendArgs& a, hipStream_t stream);

// The scatter's arguments for the fused scatter + plan launch (the pools as
// bf16 or, with AttendArgs::kv8, as 8-bit codes with their scales).
struct ScatterArgs {
  const uint16_t* k;
  const uint16_t* v;
  int64_t k_stride;     // elements between consecutive tokens of k
  int64_t v_stride;
  const int64_t* slots;
  int64_t num_tokens;
  int Hkv;
  float k_scale;
  float v_scale;
  void* k_cache;
  void* v_cache;
  int64_t num_slots;    // num_blocks * 16
  int per_block;        // scatter threads per workgroup (set by the launcher)
};
// Scatter of the new K/V and the work plan in one launch (a non-empty plan;
// without new tokens, the plan alone).
hipError_t launch_write_plan(const AttendArgs& a, const ScatterArgs& s,
                             hipStream_t stream);
// Attention over the plan in the workspace (one persistent kernel).
hipError_t launch_planned(const AttendArgs& a, hipStream_t stream);

// Bytes of the static device scratch that serves as pa_attend_noalloc's
// workspace (one array per device, held until the process ends).
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
// Device address of the current device's scratch array (looked up once per
// device with hipGetSymbolAddress, then cached).
hipError_t scratch_address(void** ptr);
// Split-K merge of the partials the attention kernel left in the workspace.
hipError_t launch_merge(const AttendArgs& a, hipStream_t stream);

}  // namespace pa
