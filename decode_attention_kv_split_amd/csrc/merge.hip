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
// A workgroup first turns the split LSEs of every query head of the group
// into normalised weights (LDS), then streams the partial outputs as float4,
// eight splits in flight per thread, with the splits spread over thread
// groups whose sums meet in LDS.
#include "kvs_device.h"

namespace kvs {
namespace {

constexpr int kMergeLds = 8192; // weights kept in LDS (heads x splits)
constexpr int kBatch = 8;       // partial loads in flight per thread

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

__global__ __launch_bounds__(kThreads) void merge_kernel(const Params p, int D, int slices) {
  __shared__ float s_w[kMergeLds];
  __shared__ float s_m[16], s_inv[16], s_lse[16];
  __shared__ float4 s_red[kThreads];
  const int b = blockIdx.x;
  const int kvg = blockIdx.y; // KV-head pack
  const int slice = blockIdx.z;
  const int first = p.meta[2 * b];
  const int nb = p.meta[2 * b + 1];
  if (nb <= 1) return;
  const int g = p.group * p.pack; // query heads merged by this workgroup
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const size_t slot0 = (size_t)kvg * p.items + first;
  const bool in_lds = g * nb <= kMergeLds;

  // ---- weights: one wave per query head ----
  for (int h = wave; h < g; h += kWaves) {
    float M = -INFINITY;
    for (int c = lane; c < nb; c += 64) M = fmaxf(M, p.lse_part[(slot0 + c) * g + h]);
    M = wave_max(M);
    float W = 0.0f;
    for (int c = lane; c < nb; c += 64) {
      const float lc = p.lse_part[(slot0 + c) * g + h];
      const float w = (lc == -INFINITY) ? 0.0f : exp2f(lc - M);
      W += w;
      if (in_lds) s_w[h * nb + c] = w;
    }
    W = wave_sum(W);
    const float inv = W > 0.0f ? 1.0f / W : 0.0f;
    if (in_lds)
      for (int c = lane; c < nb; c += 64) s_w[h * nb + c] *= inv;
    if (lane == 0) {
      s_m[h] = M;
      s_inv[h] = inv;
      s_lse[h] = (M == -INFINITY) ? -INFINITY : (M + __log2f(W)) * kLn2;
    }
  }
  __syncthreads();

  auto weight = [&](int h, int c) -> float {
    if (in_lds) return s_w[h * nb + c];
    const float lc = p.lse_part[(slot0 + c) * g + h];
    return (lc == -INFINITY) ? 0.0f : exp2f(lc - s_m[h]) * s_inv[h];
  };

  // ---- weighted sum of the partial outputs ----
  const int Ds = D / slices;
  const int d0 = slice * Ds;
  const int F = g * Ds / 4;                     // float4 outputs of this workgroup
  const int SG = F >= kThreads ? 1 : kThreads / F; // split groups
  const size_t cstride = (size_t)g * D / 4;      // float4 between consecutive splits
  const float4 *op = reinterpret_cast<const float4 *>(p.o_part) + slot0 * cstride;
  for (int f0 = 0; f0 < F; f0 += kThreads) {
    const int t = f0 + (SG > 1 ? tid % F : tid);
    const int cg = SG > 1 ? tid / F : 0;
    const bool active = t < F && cg < SG;
    const int h = t / (Ds / 4);
    const int d = d0 + 4 * (t % (Ds / 4));
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (active) {
      const float4 *src = op + ((size_t)h * D + d) / 4;
      for (int c0 = cg; c0 < nb; c0 += SG * kBatch) {
        float4 v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int c = c0 + u * SG;
          v[u] = c < nb ? src[c * cstride] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int c = c0 + u * SG;
          const float w = c < nb ? weight(h, c) : 0.0f;
          acc.x += w * v[u].x;
          acc.y += w * v[u].y;
          acc.z += w * v[u].z;
          acc.w += w * v[u].w;
        }
      }
    }
    if (SG > 1) {
      s_red[tid] = acc;
      __syncthreads();
      if (tid < F) {
        for (int j = 1; j < SG; ++j) {
          const float4 o = s_red[tid + j * F];
          acc.x += o.x;
          acc.y += o.y;
          acc.z += o.z;
          acc.w += o.w;
        }
      }
    }
    if (active && cg == 0) {
      const int hq = kvg * g + h;
      const size_t off = ((size_t)b * p.num_qo_heads + hq) * D + d;
      if (p.out_bf16) {
        const uint32_t lo = pack_bf16x2(acc.x, acc.y), hi = pack_bf16x2(acc.z, acc.w);
        *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(p.o) + off) = make_uint2(lo, hi);
      } else {
        *reinterpret_cast<float4 *>(reinterpret_cast<float *>(p.o) + off) = acc;
      }
      if (d == 0 && p.lse) p.lse[(size_t)b * p.num_qo_heads + hq] = s_lse[h];
    }
  }
}

} // namespace

hipError_t launch_merge(const Params &p, int head_dim, hipStream_t stream) {
  // enough workgroups to spread a small batch: cut the head dimension into up
  // to head_dim / 64 slices while there are fewer than ~256 (request, KV head)
  // pairs
  int slices = 1;
  const int packs = p.num_kv_heads / p.pack;
  while (slices * 64 < head_dim && (int64_t)p.batch * packs * slices < 256) slices *= 2;
  dim3 grid(p.batch, packs, slices);
  hipLaunchKernelGGL(merge_kernel, grid, dim3(kThreads), 0, stream, p, head_dim, slices);
  return hipGetLastError();
}

} // namespace kvs
