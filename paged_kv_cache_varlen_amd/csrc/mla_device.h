// Internal declarations of the multi-head latent attention (MLA) kernels
// (mla.hip) shared with the C-ABI host code of libpa.so.  gfx950 only.
#pragma once

#include "pa_device.h"

namespace pa {

constexpr int kMlaBlock = 64;    // tokens per latent-cache block
constexpr int kMlaDim = 576;     // cached dims per token (latent + rotary)
constexpr int kMlaLatent = 512;  // latent dims (the output)

struct MlaParams {
  const uint16_t* q;      // [T][Hq][576]
  const uint16_t* cache;  // [num_blocks][64 * 576]
  int64_t num_blocks;
  const int32_t* bt;
  int32_t bt_stride;
  const int32_t* seq_lens;
  const int32_t* qsl;
  int32_t num_seqs;
  int32_t num_q_tokens;
  int32_t Hq;
  int32_t max_seq_len;
  int32_t grid;        // decode workgroups (equal ranges of the item stream)
  int32_t G;           // query tokens per group (1, or 128 / Hq)
  float scale_log2;
  uint16_t* out;       // [T][Hq][512]
  // [T]: (first range, (2 * pieces + slot flag) << 3 | token's place in its group)
  int2* seg;
  float2* part_ml;     // [2 grid][G Hq]: (running max, sum) of a piece
  uint16_t* part_out;  // [2 grid][G Hq][512]: a piece's normalised output (bf16)
};

// The decode's work is a stream of items over groups of G consecutive query
// tokens of a request (G = 1, or 128 / Hq for 16, 32 and 64 heads when the
// batch's requests have several query tokens: the group's G Hq (token, head)
// rows then fill the 128 MFMA columns of a 32-key stage, as 128 heads of one
// token do).  Per group: qw head items (its ceil(G Hq / SK) query stages and
// the switch to it, costed in key-stage times), then the keys its last token
// sees in stages of SK (16 for 16 and 32 heads with G = 1, else 32).  The
// stream is cut into ranges of R = ceil(items / grid) items, one per
// workgroup; a workgroup's table holds, for each group with key stages in its
// range, the query stages and those key stages: at most R + qs entries (and
// two counts).  grid: 512 for SK = 16 (80 KiB of LDS per workgroup, two per
// compute unit), 256 for SK = 32 (160 KiB, one); more when a range's table
// could exceed its entries, never more than the items there can be.  Only a
// range's first and last group can be cut, so a workgroup leaves at most two
// partial results of G Hq rows (slots 2 rg and 2 rg + 1 of its range rg).
// One workgroup sees every item: no partials (the workspace is then a
// nominal 256 bytes, never touched).
constexpr int mla_stage_keys(int num_q_heads) { return num_q_heads <= 32 ? 16 : 32; }
constexpr int mla_table_entries(int stage_keys) { return stage_keys == 16 ? 1024 : 2048; }
// Head items per group of `rows` (token, head) rows (measured: a switch
// costs about its query stages plus two 16-key stages, or one 32-key stage).
__host__ __device__ constexpr int mla_token_items(int rows, int stage_keys) {
  return (rows + stage_keys - 1) / stage_keys + (stage_keys == 16 ? 2 : 1);
}
// Tokens per group for a batch of num_q_tokens over num_seqs requests: the
// grouped form when the requests average 4 query tokens or more.
inline int mla_group(int32_t num_q_heads, int64_t num_q_tokens, int64_t num_seqs) {
  const bool can = num_q_heads == 16 || num_q_heads == 32 || num_q_heads == 64;
  return can && num_q_tokens >= 4 * num_seqs ? 128 / num_q_heads : 1;
}
constexpr int kMlaMaxSeqs = 1 << 17;        // request index in a table entry: 17 bits
constexpr int64_t kMlaMaxTokens = 1 << 25;  // token index in a table entry: 25 bits
constexpr int64_t kMlaMaxBlocks = 1 << 29;  // block id in a table entry: 29 bits
constexpr int64_t kMlaMaxGrid = 1 << 30;    // decode workgroups of one launch
struct MlaLayout {
  int32_t grid;
  int32_t stage_keys;
  size_t seg;
  size_t part_ml;
  size_t part_out;
  size_t total;
};
inline MlaLayout mla_layout(int64_t num_q_tokens, int32_t num_q_heads,
                            int32_t max_seq_len, int group) {
  MlaLayout m{};
  const int hq = num_q_heads > 0 ? num_q_heads : 16;
  const int sk = group > 1 ? 32 : mla_stage_keys(hq);
  const int rows = group * hq;  // (token, head) rows of a group
  // (a group has at least one token: at most num_q_tokens groups)
  const int64_t most =
      num_q_tokens * (cdiv64(max_seq_len > 0 ? max_seq_len : 1, sk) + mla_token_items(rows, sk));
  // a range of R items has at most R + qs table entries (the table's last
  // two slots hold counts)
  const int64_t qs = cdiv64(rows, sk);
  int64_t grid = cdiv64(most, mla_table_entries(sk) - 2 - qs);
  const int64_t floor = sk == 16 ? 512 : 256;
  if (grid < floor) grid = floor;
  if (grid > most) grid = most > 0 ? most : 1;
  if (grid > kMlaMaxGrid) return m;  // grid 0: more work than one launch takes
  m.grid = (int32_t)grid;
  m.stage_keys = sk;
  if (m.grid == 1) {
    m.total = 256;
    return m;
  }
  const size_t slots = (size_t)2 * m.grid * rows;
  m.seg = 0;
  m.part_ml = align256(sizeof(int2) * (size_t)num_q_tokens);
  m.part_out = align256(m.part_ml + sizeof(float2) * slots);
  m.total = align256(m.part_out + sizeof(uint16_t) * kMlaLatent * slots);
  return m;
}
// Workspace bytes for either form (the form depends on num_seqs, which the
// size query does not take); 0 when either form is more than one launch.
inline size_t mla_workspace_bytes(int64_t num_q_tokens, int32_t num_q_heads,
                                  int32_t max_seq_len) {
  const MlaLayout a = mla_layout(num_q_tokens, num_q_heads, max_seq_len, 1);
  if (a.grid <= 0) return 0;
  const int g = mla_group(num_q_heads, 4, 1);  // the grouped form, where there is one
  if (g == 1) return a.total;
  const MlaLayout b = mla_layout(num_q_tokens, num_q_heads, max_seq_len, g);
  if (b.grid <= 0) return 0;
  return a.total > b.total ? a.total : b.total;
}

hipError_t launch_mla_write_kv(const uint16_t* kv, int64_t stride, const int64_t* slots,
                               int64_t num_tokens, uint16_t* cache, int64_t num_blocks,
                               hipStream_t stream);
// Decode kernel, then (keys split) the merge kernel.
hipError_t launch_mla_decode(const MlaParams& P, hipStream_t stream);

}  // namespace pa
