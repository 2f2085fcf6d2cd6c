// Host-side planning of a split-KV decode call: chunk size and launch shape.
// Pure C++; no HIP calls.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace kvs {

struct Plan {
  int chunk = 0;        // tokens per split (multiple of 16)
  int items = 0;        // work items per KV head (sum of splits)
  int max_splits = 0;
  bool needs_merge = false;
  size_t o_part_bytes = 0;
  size_t lse_part_bytes = 0;
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
constexpr int kMinChunk = 64;
constexpr int kChunkQuantum = 64; // 4 waves x 16-token tiles
// Largest chunk: 64 tiles of 16 tokens per wave (a wave keeps the page ids of
// its tiles in one register, one per lane).
constexpr int kMaxChunk = 4096;

// Host copies of the device work lists for a plan (see InlineWork /
// InlineMerge): items[x] = (request << 16) | split for the items of one KV
// head in device order; merges = (request << 16) | splits and the request's
// first item, for requests with more than one split.
// nq: query rows per request (null: one each); a request's keys start at the
// first key its first query sees.
void list_work(const int32_t *kv_len, const int32_t *nq, int batch, int window, int chunk, uint32_t *items,
               uint32_t *merge_req, uint32_t *merge_first, int *n_merges);

// kv_len: host lengths [batch]; nq: query rows per request or null (one
// each); cols: partial-result columns per KV head over all column groups
// (the group size with one query per request, col_groups * 16 with
// several); col_blocks: partial workgroups per (item, KV head).  Returns
// false if a length is negative.
bool make_plan(const int32_t *kv_len, const int32_t *nq, int batch, int window, int num_kv_heads, int cols,
               int col_blocks, int head_dim, int forced_chunk, int num_cus, Plan *out);

} // namespace kvs
