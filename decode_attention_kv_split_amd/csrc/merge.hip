// Merge of split-KV partial results by log-sum-exp, as a second kernel: the
// path for launches whose work list is derived on the device (more requests
// or work items than fit in the kernel arguments) or whose merge counters do
// not fit the workspace's counter area.  Other launches merge inside the
// partial kernel (finish_split in kvs_device.h, the same arithmetic).
//
// Grid: (request, KV-head pack x column group, slice of the head dimension).
// Requests with a single split were already written by the partial kernel
// and exit at once.  Each thread owns four consecutive output dims of one
// query head and a subset of the splits: it issues the LSE and partial loads
// of up to 16 splits at once and folds them with the running-max rescale, so
// a request's merge costs about one memory round trip after its metadata;
// the thread groups that share an output then combine their (max, weight,
// accumulator) states pairwise in LDS.
#include "kvs_device.h"

namespace kvs {
namespace {

__global__ __launch_bounds__(kThreads) void merge_kernel(const Params p, const InlineMerge ml, int D, int slices) {
  __shared__ MergeState s_st[kThreads];
  const int kvg = blockIdx.y / p.col_groups; // KV-head pack
  const int cg = blockIdx.y % p.col_groups;  // column group
  const int slice = blockIdx.z;
  int b, first, nb;
  if (ml.n >= 0) { // requests with several splits, listed by the host
    b = (int)(ml.req[blockIdx.x] >> 16);
    nb = (int)(ml.req[blockIdx.x] & 0xFFFF);
    first = (int)ml.first[blockIdx.x];
  } else {         // one workgroup per request, metadata from the partial kernel
    b = blockIdx.x;
    first = p.meta[2 * b];
    nb = p.meta[2 * b + 1];
  }
  if (nb <= 1) return;
  const int g = p.cols; // columns merged by this workgroup (query heads or (query, head) pairs)
  const int tid = threadIdx.x;
  const size_t slot0 = (size_t)blockIdx.y * p.items + first;
  const int Ds = D / slices;
  const int d0 = slice * Ds;
  const int F = g * Ds / 4;                        // float4 outputs of this workgroup
  const int SG = F >= kThreads ? 1 : kThreads / F; // thread groups splitting the splits
  const size_t cstride = (size_t)g * D / 4;        // four-element units between consecutive splits
  const float *lp = p.lse_part + slot0 * g;
  for (int f0 = 0; f0 < F; f0 += kThreads) {
    const int t = f0 + (SG > 1 ? tid % F : tid);
    const int tg = SG > 1 ? tid / F : 0;       // thread group: which splits this thread folds
    const bool active = t < F && tg < SG;
    const int h = t / (Ds / 4);
    const int d = d0 + 4 * (t % (Ds / 4));
    MergeState st = {-INFINITY, 0.0f, make_float4(0.f, 0.f, 0.f, 0.f)};
    const size_t o4 = slot0 * cstride + ((size_t)h * D + d) / 4;
    if (active) {
      if (p.part_row_scale)
        merge_fold_splits<kMergeBatch, false, true, true>(st, lp + h, g, p.o_part, o4, cstride, tg, SG, nb,
                                                           p.sc_part + slot0 * g + h);
      else if (p.part_f16)
        merge_fold_splits<kMergeBatch, false, true>(st, lp + h, g, p.o_part, o4, cstride, tg, SG, nb);
      else
        merge_fold_splits<kMergeBatch, false, false>(st, lp + h, g, p.o_part, o4, cstride, tg, SG, nb);
    }
    if (SG > 1) merge_groups(st, s_st, F, SG); // one pass (F < kThreads): uniform
    int row, hq;
    if (active && tg == 0 && column_target(p, b, kvg, cg, h, row, hq))
      merge_store(p, st, row, hq, D, d, merge_vscale(p, b, hq / p.group));
  }
}

} // namespace

hipError_t launch_merge(const Params &p, const InlineMerge &ml, int head_dim, int max_splits, hipStream_t stream) {
  const int rows = ml.n >= 0 ? ml.n : p.batch;
  if (rows == 0) return hipSuccess;
  // enough workgroups to spread a small batch: cut the head dimension into up
  // to head_dim / 64 slices while there are fewer than ~256 (request, pack)
  // pairs
  int slices = 1;
  const int packs = p.num_kv_heads / p.pack * p.col_groups;
  while (slices * 64 < head_dim && (int64_t)rows * packs * slices < 256) slices *= 2;
  // then, down to 16-dim slices, until no thread folds more than one batch of
  // splits: each batch is a dependent round trip to memory, and a long request
  // in a small grid would otherwise chain several
  auto folds = [&](int s) { // splits folded one after another by a thread
    const int F = p.cols * (head_dim / s) / 4;
    const int SG = F >= kThreads ? 1 : kThreads / F;
    return ((F + kThreads - 1) / kThreads) * ((max_splits + SG - 1) / SG);
  };
  while (slices * 16 < head_dim && folds(slices) > kMergeBatch) slices *= 2;
  dim3 grid(rows, packs, slices);
  return launch_kernel(Launch{stream}, merge_kernel, grid, p, ml, head_dim, slices);
}

} // namespace kvs
