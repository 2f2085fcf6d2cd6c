#include "plan.h"

#include <algorithm>

namespace kvs {

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// First key any query of a request sees (its first query sits at L - nq).
static int request_lo(int L, int nq, int window) { return window > 0 ? std::max(0, L - nq + 1 - window) : 0; }

bool make_plan(const int32_t *kv_len, const int32_t *nq, int batch, int window, int num_kv_heads, int cols,
               int col_blocks, int head_dim, int forced_chunk, int num_cus, Plan *out) {
  Plan pl;
  // span of request b: from its first 16-aligned visible tile to its last key
  int64_t total = 0;
  for (int b = 0; b < batch; ++b) {
    const int L = kv_len[b];
    if (L < 0) return false;
    const int lo = request_lo(L, nq ? nq[b] : 1, window);
    total += L - (lo & ~15);
  }
  int64_t chunk;
  if (forced_chunk > 0) {
    chunk = ((int64_t)forced_chunk + 15) / 16 * 16;
  } else {
    const int64_t target = (int64_t)kItemsPerCu * std::max(1, num_cus);
    chunk = (total * num_kv_heads * col_blocks + target - 1) / target;
    chunk = (chunk + kChunkQuantum - 1) / kChunkQuantum * kChunkQuantum;
    chunk = std::max<int64_t>(chunk, kMinChunk);
  }
  chunk = std::min<int64_t>(chunk, kMaxChunk);
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
    pl.o_part_bytes = align256(slots * head_dim * sizeof(float));
    pl.lse_part_bytes = align256(slots * sizeof(float));
    pl.meta_bytes = align256((size_t)batch * 2 * sizeof(int));
  }
  pl.workspace_bytes = pl.o_part_bytes + pl.lse_part_bytes + pl.meta_bytes;
  *out = pl;
  return true;
}

void list_work(const int32_t *kv_len, const int32_t *nq, int batch, int window, int chunk, uint32_t *items,
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
    for (int s = 0; s < n; ++s) items[x++] = ((uint32_t)b << 16) | (uint32_t)s;
  }
  if (n_merges) *n_merges = m;
}

} // namespace kvs
