// Host-side planning of a split-KV decode call: chunk size and launch shape.
// Pure C++; no HIP calls.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace kvs {

// Work lists travel in the kernel arguments up to these sizes (kvs_device.h
// InlineWork); merge counters fill at most kPlanCounterBytes at the start of
// the workspace (kvs_device.h kCounterBytes).
constexpr int kPlanInlineRequests = 256;
constexpr int kPlanInlineSplits = 256;
constexpr int kPlanInlineItems = 1344;
constexpr size_t kPlanCounterBytes = 65536;

struct Plan {
  int chunk = 0;        // tokens per split (multiple of 16)
  int items = 0;        // work items per KV head (sum of splits)
  int max_splits = 0;
  int wave_packs = 1;   // KV-head packs per workgroup (4: one per wave)
  bool needs_merge = false;
  // The partial kernel merges the splits itself (the workgroup that writes a
  // request's last split merges them): the work list is planned on the host
  // and the arrival counters fit their area.  Otherwise a second kernel merges.
  bool fused = false;
  bool fused_pays = false;  // auto mode takes the in-kernel merge (see make_plan)
  size_t counter_bytes = 0; // arrival counters at the start of the workspace (zero between calls)
  size_t o_part_bytes = 0;
  size_t lse_part_bytes = 0;
  size_t sc_part_bytes = 0; // multipliers of row-scaled fp16 partials (0: none)
  size_t meta_bytes = 0;
  size_t workspace_bytes = 0;
};

// Split-count heuristic.  The pages motivate choosing the decode dataflow
// from input length, batch size and the GPU's resources (FlashDecoding++
// explainer, section "hardware-aware heuristic dataflow"), and blame idle
// compute units at small batch (section "problem").  Here: aim for about
// kItemsPerCu work items per compute unit over all KV heads so every CU has
// several chunks to stream; small problems get chunks down to kMinChunk
// tokens (one tile per wave) so that they still spread over many CUs.
constexpr int kItemsPerCu = 8;
// Workgroups that hold two KV heads (pack 2: INT4 at head_dim 128) take
// chunks sized for 10 (item, KV head) pairs per CU, i.e. 5 workgroups per CU
// rather than 4.  Batch-128 INT4 decode, three draws of its lengths, step
// us at the resulting 2048-key chunks against the 2560 of 8 pairs: 138.2 /
// 151.2 / 151.0 against 141.1 / 153.0 / 151.6.  Counting workgroups instead
// (8 per CU, 1280-key chunks) sped the partial kernel but slowed the step
// through the larger merge.
constexpr int kPackedItemsPerCu = 10;
constexpr int kMinChunk = 64;
// The matrix-core decode kernel (one column group per workgroup) takes at
// least two tiles per wave: its second tile's loads overlap the first one's
// products, and half the splits halve the merge's work.  Gemma-shaped single
// decode (8192 keys, head_dim 256): 13.4 against 13.9 us per step, with a
// 512-key window 10.6 against 11.6 us; the vector kernel stays at 64 (a
// 512-key fp32 MHA decode: 9.3 against 10.1 us).
constexpr int kMinMatrixChunk = 128;
constexpr int kChunkQuantum = 64; // 4 waves x 16-token tiles
// Largest chunk: 64 tiles of 16 tokens per wave (a wave keeps the page ids of
// its tiles in one register, one per lane).
constexpr int kMaxChunk = 4096;
// With one KV-head pack per wave (wave_packs = 4) every wave streams the whole
// chunk: chunks are whole tiles, at most 64 of them.
constexpr int kWaveChunkQuantum = 16;
constexpr int kMaxWaveChunk = 1024;

// Whether a plan's work list travels in the kernel arguments (InlineWork).
inline bool plan_inline(int batch, int items, int max_splits) {
  return batch <= kPlanInlineRequests && items <= kPlanInlineItems && max_splits <= kPlanInlineSplits;
}

// Host copies of the device work lists for a plan (see InlineWork /
// InlineMerge): items[x] = (request << 8) | split for the items of one KV
// head in device order (the plan must be inline); merges = (request << 16) |
// splits and the request's first item, for requests with more than one split.
// nq: query rows per request (null: one each); a request's keys start at the
// first key its first query sees.
void list_work(const int32_t *kv_len, const int32_t *nq, int batch, int window, int chunk, uint16_t *items,
               uint32_t *merge_req, uint32_t *merge_first, int *n_merges);

// kv_len: host lengths [batch]; nq: query rows per request or null (one
// each); cols: partial-result columns per KV head over all column groups
// (the group size with one query per request, col_groups * 16 with
// several); col_blocks: partial workgroups per (item, KV head); pack: KV
// heads per workgroup; wave_packs: KV-head packs per workgroup (4: one per
// wave over the whole chunk; 1: the waves split one pack's tiles);
// part_bytes: bytes per element of the split partials o_part (4: fp32, 2:
// fp16); row_scales: each partial row has an fp32 multiplier (sc_part, laid
// out like lse_part).  Returns false if a length is negative.  Workspace
// layout when a request has several splits:
// [counters][o_part][lse_part][sc_part][meta].
// min_chunk: the smallest chunk the heuristic picks with the tiles split
// (kMinChunk or kMinMatrixChunk; the heads split takes kWaveChunkQuantum).
bool make_plan(const int32_t *kv_len, const int32_t *nq, int batch, int window, int num_kv_heads, int cols,
               int col_blocks, int pack, int wave_packs, int head_dim, int part_bytes, bool row_scales,
               int forced_chunk, int num_cus, Plan *out, int min_chunk = kMinChunk);

} // namespace kvs
