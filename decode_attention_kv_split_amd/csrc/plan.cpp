#include "plan.h"

#include <algorithm>

namespace kvs {

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// First key any query of a request sees (its first query sits at L - nq).
static int request_lo(int L, int nq, int window) { return window > 0 ? std::max(0, L - nq + 1 - window) : 0; }

bool make_plan(const int32_t *kv_len, const int32_t *nq, int batch, int window, int num_kv_heads, int cols,
               int col_blocks, int pack, int wave_packs, int head_dim, int part_bytes, bool row_scales,
               int forced_chunk, int num_cus, Plan *out, int min_chunk) {
  Plan pl;
  wave_packs = std::max(1, wave_packs);
  const bool per_wave = wave_packs > 1;
  pl.wave_packs = wave_packs;
  // span of request b: from its first 16-aligned visible tile to its last key
  int64_t total = 0, longest = 0;
  for (int b = 0; b < batch; ++b) {
    const int L = kv_len[b];
    if (L < 0) return false;
    const int lo = request_lo(L, nq ? nq[b] : 1, window);
    total += L - (lo & ~15);
    longest = std::max<int64_t>(longest, L - (lo & ~15));
  }
  int64_t chunk;
  if (forced_chunk > 0) {
    chunk = ((int64_t)forced_chunk + 15) / 16 * 16;
  } else {
    // the same work per workgroup whichever way the waves share it: a
    // workgroup holding wave_packs packs takes chunks wave_packs times shorter
    const int64_t per_cu = pack > 1 ? kPackedItemsPerCu : kItemsPerCu;
    const int64_t target = per_cu * std::max(1, num_cus) * wave_packs;
    const int64_t quantum = per_wave ? kWaveChunkQuantum : kChunkQuantum;
    chunk = (total * num_kv_heads * col_blocks + target - 1) / target;
    // at most kPlanInlineSplits splits per request, so that the work list
    // can still travel in the kernel arguments
    chunk = std::max<int64_t>(chunk, (longest + kPlanInlineSplits - 1) / kPlanInlineSplits);
    chunk = (chunk + quantum - 1) / quantum * quantum;
    chunk = std::max<int64_t>(chunk, per_wave ? kWaveChunkQuantum : min_chunk);
  }
  chunk = std::min<int64_t>(chunk, per_wave ? kMaxWaveChunk : kMaxChunk);
  pl.chunk = (int)chunk;
  int64_t items = 0;
  int max_splits = 0;
  for (int b = 0; b < batch; ++b) {
    const int L = kv_len[b];
    const int lo = request_lo(L, nq ? nq[b] : 1, window);
    const int64_t span = L - (lo & ~15);
    const int64_t n = span <= 0 ? 1 : (span + chunk - 1) / chunk;
    items += n;
    max_splits = std::max<int>(max_splits, (int)n);
  }
  if (items > (int64_t)0x7fffffff) return false;
  pl.items = (int)items;
  pl.max_splits = max_splits;
  pl.needs_merge = max_splits > 1;
  if (pl.needs_merge) {
    const size_t slots = (size_t)items * num_kv_heads * cols;
    // the counter area is always reserved, so a workspace shared by fused and
    // two-kernel calls keeps its counters zero
    pl.counter_bytes = kPlanCounterBytes;
    pl.o_part_bytes = align256(slots * head_dim * part_bytes);
    pl.lse_part_bytes = align256(slots * sizeof(float));
    pl.sc_part_bytes = row_scales ? align256(slots * sizeof(float)) : 0;
    pl.meta_bytes = align256((size_t)batch * 2 * sizeof(int));
    // one counter per (KV head, column block, request) at most (packing two
    // KV heads per workgroup halves it)
    const int64_t counters = (int64_t)num_kv_heads * col_blocks * batch;
    pl.fused = plan_inline(batch, (int)items, max_splits) &&
               counters * (int64_t)sizeof(unsigned) <= (int64_t)kPlanCounterBytes;
    // The merge inside the partial kernel costs every split workgroup a wait
    // for its partial stores and a counter round trip before it exits, and
    // one workgroup folds all splits of a request.  Measured on MI355X it
    // pays only where a second launch is the larger cost: launches of at most
    // one workgroup per CU whose requests have few splits (a 512-key fp32 MHA
    // decode: 9.1 against 10.5 us per step; a 32k-key MHA decode, 2048
    // workgroups: 95 against 88 us; 128 splits of one request: 43 against 17 us).
    const int64_t wgs = items * (int64_t)(num_kv_heads / std::max(1, pack)) * col_blocks / wave_packs;
    pl.fused_pays = pl.fused && wgs <= std::max(1, num_cus) && max_splits <= 8;
  }
  pl.workspace_bytes = pl.counter_bytes + pl.o_part_bytes + pl.lse_part_bytes + pl.sc_part_bytes + pl.meta_bytes;
  *out = pl;
  return true;
}

void list_work(const int32_t *kv_len, const int32_t *nq, int batch, int window, int chunk, uint16_t *items,
               uint32_t *merge_req, uint32_t *merge_first, int *n_merges) {
  int x = 0, m = 0;
  for (int b = 0; b < batch; ++b) {
    const int L = kv_len[b];
    const int lo = request_lo(L, nq ? nq[b] : 1, window);
    const int64_t span = L - (lo & ~15);
    const int n = span <= 0 ? 1 : (int)((span + chunk - 1) / chunk);
    if (n > 1 && merge_req) {
      merge_req[m] = ((uint32_t)b << 16) | (uint32_t)n;
      merge_first[m] = (uint32_t)x;
      ++m;
    }
    for (int s = 0; s < n; ++s) items[x++] = (uint16_t)((b << 8) | s);
  }
  if (n_merges) *n_merges = m;
}

} // namespace kvs
