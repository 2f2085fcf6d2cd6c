// The step before decode attention, for the new tokens of every request:
// QK-norm, rotary embedding, and the append of the new key and value to the
// cache.  One new token per request goes to position p = kv_len[b]; with a
// packed ragged batch of token rows (qo_indptr), row i of request b goes to
// position kv_len[b] + i and is rotated there (the three-kernels section of
// the FlashInfer-from-JAX page: apply_rope over a packed batch).
//
//   QK-norm: an RMSNorm over each head's q and k before their dot product
//     (FlashInfer-from-JAX tutorial page, Gemma 3 section): x / sqrt(mean(x^2)
//     + eps) * w, skipped when no weight is given.
//   Rotary embedding: dimension pair j turns by the angle p * theta^(-2j/d)
//     (the published RoPE definition; the same page's three-kernels section
//     names apply_rope and its Gemma 3 section the per-layer theta, 10,000 for
//     local and 1,000,000 for global layers).  Pairs (j, j + d/2), or
//     (2j, 2j + 1) when interleaved.
//   Append to the growing paged or contiguous cache, fp8 and INT4 included
//     ("Beyond the Memory Wall", section "2. FlashInfer"); an fp8 value is
//     stored as the nearest code of x / scale[b, kv head], saturating at
//     +-448, an INT4 value as the nearest integer to it (ties to even),
//     saturating to [-8, 7], two per byte with element 2i in the low nibble.
//
// Head rows [0, Hq) of a token are its query heads (written to q_out), rows
// [Hq, Hq + Hk) its KV heads (k transformed like q, v copied; both stored).
// A wave takes two consecutive head rows of one token: they share the
// position, so the rotation is computed once per wave.  Lane l holds E = d / 64 elements: indices l + 64 e (pairs
// (j, j + d/2) then sit in one lane for d >= 128 and in lanes l, l ^ 32 for
// d = 64), or E l + e when interleaved (pairs in one lane, or in lanes l, l ^ 1
// for d = 64).  The angle is computed in double precision and reduced modulo
// 2 pi before the single-precision sine and cosine, so large positions keep
// their accuracy.
#include "kvs_device.h"

namespace kvs {
namespace {

struct AppendParams {
  const void *q_in;
  const void *k_in;
  const void *v_in;
  void *q_out;
  void *k_cache;
  void *v_cache;
  const int *page_indptr;
  const int *page_indices;
  const int *kv_len;
  const float *k_scale;
  const float *v_scale;
  const float *q_norm_weight;
  const float *k_norm_weight;
  int batch;
  int num_qo_heads;
  int num_kv_heads;
  int page_size;
  int num_pages; // paged: pages in the pools; contiguous: capacity in tokens
  float norm_eps;
  float rope_theta;
  int interleave;
  int q_f32;   // q_in, k_in, v_in, q_out are fp32 (else bf16)
  int kv_type; // DT_F32, DT_BF16, DT_FP8, DT_INT4
  int n_tok;   // token rows: batch, or qo_indptr[batch]
  const int *qo_indptr; // [batch + 1] token rows of each request; null: one each
};

// The host copy of qo_indptr, passed in the kernel arguments when the batch
// fits, so that a wave finds its token's request without a dependent read.
struct AppendRows {
  int n;                            // entries below (batch + 1); 0: not provided
  int indptr[kInlineRequests + 1];
};

// Request of token row r: the last b with indptr[b] <= r (an empty request's
// indptr[b] equals the next one's, so the search lands on the request that
// holds r).  r is the same in every lane of the wave.
template <typename Ind>
__device__ __forceinline__ int request_of_row(Ind indptr, int batch, int r) {
  int lo = 0, hi = batch; // indptr[lo] <= r < indptr[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (indptr(mid) <= r)
      lo = mid;
    else
      hi = mid;
  }
  return lo;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) { return (uint16_t)(pack_bf16x2(x, 0.0f) & 0xFFFF); }

// OCP fp8 E4M3 code of x, nearest-even, saturating at +-448; NaN -> 0x7F.
__device__ __forceinline__ uint8_t f32_to_fp8_sat(float x) {
  if (__builtin_isnan(x)) return 0x7F;
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fminf(fabsf(x), 448.0f);
  if (a < 0.015625f) {                          // below 2^-6: subnormal quantum 2^-9
    const uint32_t m = (uint32_t)rintf(a * 512.0f); // 0..8; 8 is the smallest normal (code 0x08)
    return (uint8_t)(sign | m);
  }
  const uint32_t u = __float_as_uint(a);
  const uint32_t mant = u & 0x7FFFFFu;
  uint32_t m3 = (mant + 0x7FFFFu + ((mant >> 20) & 1u)) >> 20; // keep 3 fraction bits, ties to even
  uint32_t e = (u >> 23) - 127 + 7;
  if (m3 == 8) {
    m3 = 0;
    e += 1;
  }
  return (uint8_t)(sign | (e << 3) | m3);
}

template <int D>
__device__ __forceinline__ int elem_index(int lane, int e, bool interleave) {
  constexpr int E = D / 64;
  return interleave ? E * lane + e : lane + 64 * e;
}

template <int D>
__device__ __forceinline__ void load_row(const AppendParams &p, const void *base, size_t row, int lane,
                                         float (&x)[D / 64]) {
  constexpr int E = D / 64;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = elem_index<D>(lane, e, p.interleave);
    x[e] = p.q_f32 ? reinterpret_cast<const float *>(base)[row * D + i]
                   : bf16_bits_to_f32(reinterpret_cast<const uint16_t *>(base)[row * D + i]);
  }
}

template <int D>
__device__ __forceinline__ void rms_norm(const AppendParams &p, const float *w, int lane, float (&x)[D / 64]) {
  constexpr int E = D / 64;
  float ss = 0.0f;
#pragma unroll
  for (int e = 0; e < E; ++e) ss = fmaf(x[e], x[e], ss);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
  const float r = 1.0f / sqrtf(ss / (float)D + p.norm_eps);
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] = x[e] * r * w[elem_index<D>(lane, e, p.interleave)];
}

// Angle of pair j at position pos, reduced to [-pi, pi], as (cos, sin).
template <int D>
__device__ __forceinline__ void pair_rotation(double log2_theta, int pos, int j, float &c, float &s) {
  const double w = exp2(-2.0 * (double)j / (double)D * log2_theta);
  double t = (double)pos * w;
  const double two_pi = 6.283185307179586476925286766559;
  t -= two_pi * rint(t / two_pi);
  sincosf((float)t, &s, &c);
}

// The rotations of the pairs this lane touches (they depend on the position
// only, so every head of a request shares them): NP = max(1, E / 2) pairs.
template <int D>
struct Rotation {
  static constexpr int E = D / 64;
  static constexpr int NP = E >= 2 ? E / 2 : 1;
  float c[NP], s[NP];
};

template <int D>
__device__ __forceinline__ void make_rotation(const AppendParams &p, int pos, int lane, Rotation<D> &rot) {
  constexpr int E = D / 64;
  const double lt = log2((double)p.rope_theta);
  if constexpr (E == 1) {
    const int j = p.interleave ? lane >> 1 : (lane & 31);
    pair_rotation<D>(lt, pos, j, rot.c[0], rot.s[0]);
  } else {
#pragma unroll
    for (int k = 0; k < E / 2; ++k) {
      // interleaved: pair (E lane + 2k, +1); rotate-half: pair (lane + 64 k, + D/2)
      const int j = p.interleave ? (E * lane + 2 * k) >> 1 : lane + 64 * k;
      pair_rotation<D>(lt, pos, j, rot.c[k], rot.s[k]);
    }
  }
}

template <int D>
__device__ __forceinline__ void rope(const AppendParams &p, const Rotation<D> &rot, int lane, float (&x)[D / 64]) {
  constexpr int E = D / 64;
  if constexpr (E == 1) {
    // the partner of this lane's element sits in another lane
    const int partner = p.interleave ? (lane ^ 1) : (lane ^ 32);
    const bool first = p.interleave ? (lane & 1) == 0 : lane < 32;
    const float y = __shfl(x[0], partner, 64);
    const float c = rot.c[0], s = rot.s[0];
    // first of the pair: a c - b s; second: a s + b c (a = first, b = second)
    x[0] = first ? x[0] * c - y * s : y * s + x[0] * c;
  } else {
    float out[E];
#pragma unroll
    for (int k = 0; k < E / 2; ++k) {
      const float c = rot.c[k], s = rot.s[k];
      const int a = p.interleave ? 2 * k : k;          // slots of the pair's two elements
      const int b = p.interleave ? 2 * k + 1 : k + E / 2;
      out[a] = x[a] * c - x[b] * s;
      out[b] = x[a] * s + x[b] * c;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = out[e];
  }
}

template <int D>
__device__ __forceinline__ void store_q(const AppendParams &p, size_t row, int lane, const float (&x)[D / 64]) {
  constexpr int E = D / 64;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = elem_index<D>(lane, e, p.interleave);
    if (p.q_f32)
      reinterpret_cast<float *>(p.q_out)[row * D + i] = x[e];
    else
      reinterpret_cast<uint16_t *>(p.q_out)[row * D + i] = f32_to_bf16_rne(x[e]);
  }
}

// INT4 code of x (already divided by its scale): nearest integer, ties to
// even, saturated to [-8, 7]; NaN gives 0.  Returned as the low nibble.
__device__ __forceinline__ uint32_t f32_to_int4_sat(float x) {
  if (__builtin_isnan(x)) return 0u;
  const float r = fminf(fmaxf(rintf(x), -8.0f), 7.0f);
  return (uint32_t)(int)r & 0xFu;
}

template <int D>
__device__ __forceinline__ void store_kv(const AppendParams &p, void *cache, size_t off, float scale, int lane,
                                         const float (&x)[D / 64]) {
  constexpr int E = D / 64;
  if (p.kv_type == DT_INT4) {
    // byte j of the row holds elements 2j (low nibble) and 2j + 1 (high)
    uint8_t *row = reinterpret_cast<uint8_t *>(cache) + off / 2;
    if (p.interleave && E >= 2) { // elements E lane + e: both of a pair in this lane
#pragma unroll
      for (int e = 0; e < E; e += 2)
        row[(E * lane + e) / 2] = (uint8_t)(f32_to_int4_sat(x[e] / scale) | (f32_to_int4_sat(x[e + 1] / scale) << 4));
    } else { // elements lane + 64 e (or lane for E = 1): the pair's other element is in lane ^ 1
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const uint32_t c = f32_to_int4_sat(x[e] / scale);
        const uint32_t other = (uint32_t)__shfl_xor((int)c, 1, 64);
        if ((lane & 1) == 0) row[(elem_index<D>(lane, e, p.interleave)) / 2] = (uint8_t)(c | (other << 4));
      }
    }
    return;
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = elem_index<D>(lane, e, p.interleave);
    if (p.kv_type == DT_F32)
      reinterpret_cast<float *>(cache)[off + i] = x[e];
    else if (p.kv_type == DT_BF16)
      reinterpret_cast<uint16_t *>(cache)[off + i] = f32_to_bf16_rne(x[e]);
    else
      reinterpret_cast<uint8_t *>(cache)[off + i] = f32_to_fp8_sat(x[e] / scale);
  }
}

// Head rows of one request per wave; they share the position and hence the
// rotation, which is computed once.
constexpr int kRowsPerWave = 2;

template <int D>
__global__ __launch_bounds__(kThreads) void append_kernel(const AppendParams p, const AppendRows inl) {
  constexpr int E = D / 64;
  const int lane = threadIdx.x & 63;
  const int rows_per_req = p.num_qo_heads + p.num_kv_heads; // head rows of one token
  const int waves_per_req = (rows_per_req + kRowsPerWave - 1) / kRowsPerWave;
  const int wid = blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wid >= p.n_tok * waves_per_req) return; // whole waves exit
  const int tr = wid / waves_per_req;  // token row (q_in / k_in / v_in / q_out row)
  const int h0 = (wid % waves_per_req) * kRowsPerWave;
  int b = tr, i = 0; // request and index of the token within it
  if (p.qo_indptr) {
    if (inl.n > 0) {
      b = request_of_row([&](int x) { return inl.indptr[x]; }, p.batch, tr);
      i = tr - inl.indptr[b];
    } else {
      b = request_of_row([&](int x) { return p.qo_indptr[x]; }, p.batch, tr);
      i = tr - p.qo_indptr[b];
    }
  }
  const int pos = p.kv_len[b] + i;

  // where the new token goes; a slot its page list does not cover is not written
  bool write_kv = true;
  size_t tok = 0;
  if (p.page_size > 0) {
    const int first = p.page_indptr[b];
    const int npages = p.page_indptr[b + 1] - first;
    const int pi = pos / p.page_size;
    write_kv = pos >= 0 && pi < npages;
    if (write_kv) {
      const int pid = p.page_indices[first + pi];
      write_kv = pid >= 0 && pid < p.num_pages;
      tok = (size_t)pid * p.page_size + pos % p.page_size;
    }
  } else {
    write_kv = pos >= 0 && pos < p.num_pages;
    tok = (size_t)pos;
  }

  // every load of the wave's rows first, so they are in flight together
  float x[kRowsPerWave][E], v[kRowsPerWave][E];
#pragma unroll
  for (int rr = 0; rr < kRowsPerWave; ++rr) {
    const int h = h0 + rr;
    if (h >= rows_per_req) break;
    if (h < p.num_qo_heads) {
      load_row<D>(p, p.q_in, (size_t)tr * p.num_qo_heads + h, lane, x[rr]);
    } else {
      const size_t r = (size_t)tr * p.num_kv_heads + (h - p.num_qo_heads);
      load_row<D>(p, p.k_in, r, lane, x[rr]);
      load_row<D>(p, p.v_in, r, lane, v[rr]);
    }
  }
  Rotation<D> rot;
  if (p.rope_theta > 0.0f) make_rotation<D>(p, pos, lane, rot);

#pragma unroll
  for (int rr = 0; rr < kRowsPerWave; ++rr) {
    const int h = h0 + rr;
    if (h >= rows_per_req) break;
    if (h < p.num_qo_heads) {
      if (p.q_norm_weight) rms_norm<D>(p, p.q_norm_weight, lane, x[rr]);
      if (p.rope_theta > 0.0f) rope<D>(p, rot, lane, x[rr]);
      store_q<D>(p, (size_t)tr * p.num_qo_heads + h, lane, x[rr]);
    } else {
      const int kh = h - p.num_qo_heads;
      if (p.k_norm_weight) rms_norm<D>(p, p.k_norm_weight, lane, x[rr]);
      if (p.rope_theta > 0.0f) rope<D>(p, rot, lane, x[rr]);
      if (write_kv) {
        const size_t r = (size_t)b * p.num_kv_heads + kh; // scales are per (request, KV head)
        const size_t off = (tok * p.num_kv_heads + kh) * D; // in elements
        const bool scaled = p.kv_type == DT_FP8 || p.kv_type == DT_INT4;
        store_kv<D>(p, p.k_cache, off, scaled ? p.k_scale[r] : 1.0f, lane, x[rr]);
        store_kv<D>(p, p.v_cache, off, scaled ? p.v_scale[r] : 1.0f, lane, v[rr]);
      }
    }
  }
}

} // namespace
} // namespace kvs

#include "kvsplit.h"

namespace kvs {

hipError_t launch_append(const kvs_append_args *a, const Launch &l) {
  AppendParams p;
  p.q_in = a->q_in;
  p.k_in = a->k_in;
  p.v_in = a->v_in;
  p.q_out = a->q_out;
  p.k_cache = a->k_cache;
  p.v_cache = a->v_cache;
  p.page_indptr = a->page_indptr;
  p.page_indices = a->page_indices;
  p.kv_len = a->kv_len;
  p.k_scale = a->k_scale;
  p.v_scale = a->v_scale;
  p.q_norm_weight = a->q_norm_weight;
  p.k_norm_weight = a->k_norm_weight;
  p.batch = a->batch;
  p.num_qo_heads = a->num_qo_heads;
  p.num_kv_heads = a->num_kv_heads;
  p.page_size = a->page_size;
  p.num_pages = a->num_pages;
  p.norm_eps = a->norm_eps;
  p.rope_theta = a->rope_theta;
  p.interleave = a->rope_interleave;
  p.q_f32 = a->q_dtype == KVS_F32;
  p.kv_type = a->kv_dtype == KVS_F32 ? DT_F32
              : a->kv_dtype == KVS_BF16 ? DT_BF16
              : a->kv_dtype == KVS_FP8_E4M3 ? DT_FP8
                                            : DT_INT4;
  p.qo_indptr = a->qo_indptr_host ? a->qo_indptr : nullptr;
  p.n_tok = a->qo_indptr_host ? a->qo_indptr_host[a->batch] : a->batch;
  AppendRows inl;
  inl.n = 0;
  if (a->qo_indptr_host && a->batch <= kInlineRequests) {
    for (int b = 0; b <= a->batch; ++b) inl.indptr[b] = a->qo_indptr_host[b];
    inl.n = a->batch + 1;
  }
  if (p.n_tok == 0) return hipSuccess; // no new token anywhere
  const int64_t waves = (int64_t)p.n_tok * ((a->num_qo_heads + a->num_kv_heads + kRowsPerWave - 1) / kRowsPerWave);
  const dim3 grid((unsigned)((waves + kWaves - 1) / kWaves));
  switch (a->head_dim) {
  case 64: return launch_kernel(l, append_kernel<64>, grid, p, inl);
  case 128: return launch_kernel(l, append_kernel<128>, grid, p, inl);
  case 256: return launch_kernel(l, append_kernel<256>, grid, p, inl);
  default: return hipErrorInvalidValue;
  }
}

} // namespace kvs
