// Merge of split-KV partial results by log-sum-exp.
//
// For a (request, query head) with splits c = 0..n-1 holding a normalised
// partial output o_c and a log2-domain log-sum-exp l_c:
//   M = max_c l_c,  w_c = 2^(l_c - M),  o = sum_c w_c o_c / sum_c w_c,
//   lse = (M + log2 sum_c w_c) * ln 2,  all l_c = -inf -> o = 0, lse = -inf.
// This is the online-softmax rescale ("Forcing Flash Attention onto TPU",
// section "Flash Attention in JAX": multiply the old accumulator and sum by
// exp(old max - new max)) applied across chunks; the FlashDecoding++
// explainer's asynchronous-softmax section describes this synchronised update
// of per-tile partial softmax results with the previous max and sum.
//
// One workgroup per (request, KV head) merges all query heads of the group;
// requests with a single split were already written by the partial kernel.
#include "kvs_device.h"

namespace kvs {
namespace {

__global__ __launch_bounds__(kThreads) void merge_kernel(const Params p, int D) {
  __shared__ int s_scan[2 * 64];
  __shared__ int s_req[2];
  const int b = blockIdx.x;
  const int kvh = blockIdx.y;
  if (threadIdx.x == 0) {
    s_req[0] = 0;
    s_req[1] = 0;
  }
  scan_requests(p, s_scan, [&](int bb, int first, int nb) {
    if (bb == b) {
      s_req[0] = first;
      s_req[1] = nb;
    }
  });
  __syncthreads();
  const int first = s_req[0];
  const int nb = s_req[1];
  if (nb <= 1) return;
  const int g = p.group;
  const size_t slot0 = (size_t)kvh * p.items + first;
  for (int idx = threadIdx.x; idx < g * D; idx += kThreads) {
    const int h = idx / D;
    const int d = idx - h * D;
    float M = -INFINITY;
    for (int c = 0; c < nb; ++c) M = fmaxf(M, p.lse_part[(slot0 + c) * g + h]);
    float val = 0.0f, lse2 = -INFINITY;
    if (M != -INFINITY) {
      float W = 0.0f, acc = 0.0f;
      for (int c = 0; c < nb; ++c) {
        const float lc = p.lse_part[(slot0 + c) * g + h];
        const float w = (lc == -INFINITY) ? 0.0f : exp2f(lc - M);
        W += w;
        acc += w * p.o_part[((slot0 + c) * g + h) * D + d];
      }
      val = acc / W;
      lse2 = M + __log2f(W);
    }
    const int hq = kvh * g + h;
    const size_t off = ((size_t)b * p.num_qo_heads + hq) * D + d;
    if (p.out_bf16)
      reinterpret_cast<uint16_t *>(p.o)[off] = f32_to_bf16_bits(val);
    else
      reinterpret_cast<float *>(p.o)[off] = val;
    if (d == 0 && p.lse) p.lse[(size_t)b * p.num_qo_heads + hq] = lse2 * kLn2;
  }
}

} // namespace

hipError_t launch_merge(const Params &p, int head_dim, hipStream_t stream) {
  dim3 grid(p.batch, p.num_kv_heads);
  hipLaunchKernelGGL(merge_kernel, grid, dim3(kThreads), 0, stream, p, head_dim);
  return hipGetLastError();
}

} // namespace kvs
