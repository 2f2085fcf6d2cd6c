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
// Grid: (request, KV-head pack, slice of the head dimension).  Requests with a
// single split were already written by the partial kernel and exit at once.
// Each thread owns four consecutive output dims of one query head and a
// subset of the splits: it issues the LSE and partial loads of up to 16
// splits at once and folds them with the same running-max rescale, so a
// request's merge costs about one memory round trip after its metadata; the
// thread groups that share an output then combine their (max, weight,
// accumulator) states in LDS.
#include "kvs_device.h"

namespace kvs {
namespace {

constexpr int kBatch = 16; // splits whose loads are in flight together per thread

struct MergeState {
  float m;   // running max of the split LSEs (log2 domain)
  float w;   // sum of 2^(lse_c - m)
  float4 acc; // sum of 2^(lse_c - m) * o_c
};

__device__ __forceinline__ void fold(MergeState &st, float lc, const float4 &o) {
  // lc = -inf (a split that saw no key) contributes nothing
  if (lc == -INFINITY) return;
  if (lc > st.m) {
    const float r = st.m == -INFINITY ? 0.0f : exp2f(st.m - lc);
    st.w *= r;
    st.acc.x *= r;
    st.acc.y *= r;
    st.acc.z *= r;
    st.acc.w *= r;
    st.m = lc;
  }
  const float e = exp2f(lc - st.m);
  st.w += e;
  st.acc.x += e * o.x;
  st.acc.y += e * o.y;
  st.acc.z += e * o.z;
  st.acc.w += e * o.w;
}

__device__ __forceinline__ void combine(MergeState &a, const MergeState &b) {
  if (b.m == -INFINITY) return;
  const float M = fmaxf(a.m, b.m);
  const float ra = a.m == -INFINITY ? 0.0f : exp2f(a.m - M);
  const float rb = exp2f(b.m - M);
  a.w = a.w * ra + b.w * rb;
  a.acc.x = a.acc.x * ra + b.acc.x * rb;
  a.acc.y = a.acc.y * ra + b.acc.y * rb;
  a.acc.z = a.acc.z * ra + b.acc.z * rb;
  a.acc.w = a.acc.w * ra + b.acc.w * rb;
  a.m = M;
}

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
  const size_t cstride = (size_t)g * D / 4;        // float4 between consecutive splits
  const float4 *op = reinterpret_cast<const float4 *>(p.o_part) + slot0 * cstride;
  const float *lp = p.lse_part + slot0 * g;
  for (int f0 = 0; f0 < F; f0 += kThreads) {
    const int t = f0 + (SG > 1 ? tid % F : tid);
    const int tg = SG > 1 ? tid / F : 0;       // thread group: which splits this thread folds
    const bool active = t < F && tg < SG;
    const int h = t / (Ds / 4);
    const int d = d0 + 4 * (t % (Ds / 4));
    MergeState st = {-INFINITY, 0.0f, make_float4(0.f, 0.f, 0.f, 0.f)};
    if (active) {
      const float4 *src = op + ((size_t)h * D + d) / 4;
      for (int c0 = tg; c0 < nb; c0 += SG * kBatch) {
        float lc[kBatch];
        float4 v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int c = c0 + u * SG;
          lc[u] = c < nb ? lp[(size_t)c * g + h] : -INFINITY;
          v[u] = c < nb ? src[c * cstride] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) fold(st, lc[u], v[u]);
      }
    }
    if (SG > 1) {
      s_st[tid] = st;
      __syncthreads();
      if (tid < F)
        for (int j = 1; j < SG; ++j) combine(st, s_st[tid + j * F]);
    }
    int row, hq;
    if (active && tg == 0 && column_target(p, b, kvg, cg, h, row, hq)) {
      const float inv = st.w > 0.0f ? 1.0f / st.w : 0.0f;
      const float4 o = make_float4(st.acc.x * inv, st.acc.y * inv, st.acc.z * inv, st.acc.w * inv);
      const size_t off = ((size_t)row * p.num_qo_heads + hq) * D + d;
      if (p.out_bf16) {
        *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(p.o) + off) =
            make_uint2(pack_bf16x2(o.x, o.y), pack_bf16x2(o.z, o.w));
      } else {
        *reinterpret_cast<float4 *>(reinterpret_cast<float *>(p.o) + off) = o;
      }
      if (d == 0 && p.lse)
        p.lse[(size_t)row * p.num_qo_heads + hq] = st.m == -INFINITY ? -INFINITY : (st.m + __log2f(st.w)) * kLn2;
    }
  }
}

} // namespace

hipError_t launch_merge(const Params &p, const InlineMerge &ml, int head_dim, hipStream_t stream) {
  const int rows = ml.n >= 0 ? ml.n : p.batch;
  if (rows == 0) return hipSuccess;
  // enough workgroups to spread a small batch: cut the head dimension into up
  // to head_dim / 64 slices while there are fewer than ~256 (request, pack)
  // pairs
  int slices = 1;
  const int packs = p.num_kv_heads / p.pack * p.col_groups;
  while (slices * 64 < head_dim && (int64_t)rows * packs * slices < 256) slices *= 2;
  dim3 grid(rows, packs, slices);
  return launch_kernel(Launch{stream}, merge_kernel, grid, p, ml, head_dim, slices);
}

} // namespace kvs
