// Split-KV partial softmax on the vector ALUs: fp32 KV, small page sizes, and
// any case the matrix-core kernel does not take.
//
// One workgroup (4 waves) owns one chunk of one (request, KV head); wave w
// takes the chunk's 16-token tiles w, w+4, ...  Inside a wave, RL = D * bytes
// / 16 consecutive lanes hold one K/V row (16 bytes each), so one 16-byte load
// per lane covers 64 / RL rows.  Each group of RL lanes is its own online
// softmax stream (running max, sum, accumulator per query head) over the
// tokens it loads; the streams of a wave merge by log-sum-exp with lane
// exchanges at the end, then the four waves merge through LDS.
// Scores and the update follow the tiled online softmax of "Forcing Flash
// Attention onto TPU", section "Flash Attention in JAX", one key at a time.
#include "kvs_device.h"

namespace kvs {
namespace {

template <int KVT>
struct KvType;
template <>
struct KvType<DT_F32> {
  static constexpr int kBytes = 4;
};
template <>
struct KvType<DT_BF16> {
  static constexpr int kBytes = 2;
};
template <>
struct KvType<DT_FP8> {
  static constexpr int kBytes = 1;
};

// 16 bytes -> EPL floats.
template <int KVT>
__device__ __forceinline__ void dequant16(const uint4 w, float *out) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
  if constexpr (KVT == DT_F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(u[i]);
  } else if constexpr (KVT == DT_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(u[i] << 16);
      out[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
    }
  } else {
    typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8(u[i], false);
      const f32x2_t b = __builtin_amdgcn_cvt_pk_f32_fp8(u[i], true);
      out[4 * i + 0] = a[0];
      out[4 * i + 1] = a[1];
      out[4 * i + 2] = b[0];
      out[4 * i + 3] = b[1];
    }
  }
}

template <int D, int KVT, int G>
__global__ __launch_bounds__(kThreads) void partial_valu_kernel(const Params p, const InlineWork w) {
  constexpr int BYTES = KvType<KVT>::kBytes;
  constexpr int EPL = 16 / BYTES;        // elements per lane
  constexpr int RL = D * BYTES / 16;     // lanes per row
  constexpr int RW = 64 / RL;            // rows per wave pass
  constexpr int NPASS = RW >= kTile ? 1 : kTile / RW;
  constexpr int ROWS_USED = RW >= kTile ? kTile : RW;
  constexpr int OSTRIDE = D + 4;
  static_assert(RL >= 1 && RL <= 64, "row must span 1..64 lanes");

  __shared__ int s_scan[2 * 64];
  __shared__ int s_item[4];
  __shared__ float sm_m[kWaves][16];
  __shared__ float sm_l[kWaves][16];
  __shared__ __attribute__((aligned(16))) float sm_o[kWaves * 16 * OSTRIDE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = lane / RL; // row group
  const int lr = lane % RL; // lane within row
  const int item = blockIdx.x;
  const int kvh = blockIdx.y;
  const int g = p.group;
  const int Hk = p.num_kv_heads;

  // ---- which (request, split) is this workgroup? ----
  int b, split, nb, L;
  if (w.n_items > 0) { // planned on the host
    const uint32_t e = w.item[item];
    b = (int)(e >> 8);
    split = (int)(e & 0xFF);
    L = w.req_len[b];
    nb = num_splits(L, 1, p.window, p.chunk);
  } else {
    if (tid == 0) s_item[0] = -1;
    scan_requests(p, s_scan, [&](int bb, int first, int nbb) {
      if (item >= first && item < first + nbb) {
        s_item[0] = bb;
        s_item[1] = item - first;
        s_item[2] = nbb;
        s_item[3] = first;
      }
    });
    __syncthreads();
    b = __builtin_amdgcn_readfirstlane(s_item[0]);
    split = __builtin_amdgcn_readfirstlane(s_item[1]);
    nb = __builtin_amdgcn_readfirstlane(s_item[2]);
    if (b < 0) return; // kv_len on the device disagrees with the planned launch
    if (p.meta && split == 0 && kvh == 0 && tid == 0) {
      p.meta[2 * b] = s_item[3];
      p.meta[2 * b + 1] = nb;
    }
    L = p.kv_len[b];
  }

  const int lo = visible_lo(L, p.window);
  const int a0 = (lo & ~(kTile - 1)) + split * p.chunk;
  const int t_begin = max(lo, a0);
  const int t_end = min(L, a0 + p.chunk);
  const int ntiles = t_end > t_begin ? (t_end - a0 + kTile - 1) / kTile : 0;
  const int my_tiles = ntiles > wave ? (ntiles - wave + kWaves - 1) / kWaves : 0;

  // query slice of every head of the group, prescaled to the log2 domain
  float cscale = p.score_scale;
  if (KVT == DT_FP8) cscale *= p.k_scale[b * Hk + kvh];
  float qv[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const size_t qoff = ((size_t)b * p.num_qo_heads + (size_t)kvh * g + h) * D + lr * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float x = 0.0f;
      if (h < g) {
        x = p.out_bf16 ? bf16_bits_to_f32(reinterpret_cast<const uint16_t *>(p.q)[qoff + e])
                       : reinterpret_cast<const float *>(p.q)[qoff + e];
      }
      qv[h][e] = x * cscale;
    }
  }

  float m_run[G], l_run[G], acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.0f;
  }

  const size_t row_bytes = (size_t)Hk * D * BYTES;
  const char *kbase = reinterpret_cast<const char *>(p.k) + (size_t)kvh * D * BYTES + lr * 16;
  const char *vbase = reinterpret_cast<const char *>(p.v) + (size_t)kvh * D * BYTES + lr * 16;
  const bool paged = p.page_size > 0;
  const int *pages = paged ? p.page_indices + p.page_indptr[b] : nullptr;

  for (int i = 0; i < my_tiles; ++i) {
    const int ts = a0 + (wave + i * kWaves) * kTile;
#pragma unroll
    for (int pass = 0; pass < NPASS; ++pass) {
      const int tok = ts + pass * ROWS_USED + rg;
      const bool valid = rg < ROWS_USED && tok >= t_begin && tok < t_end;
      uint4 kw = make_uint4(0, 0, 0, 0), vw = make_uint4(0, 0, 0, 0);
      if (valid) {
        size_t row;
        if (!paged) {
          row = (size_t)tok;
        } else if (p.page_shift >= 0) {
          row = (size_t)pages[tok >> p.page_shift] * p.page_size + (tok & (p.page_size - 1));
        } else {
          row = (size_t)pages[tok / p.page_size] * p.page_size + (tok % p.page_size);
        }
        kw = *reinterpret_cast<const uint4 *>(kbase + row * row_bytes);
        vw = *reinterpret_cast<const uint4 *>(vbase + row * row_bytes);
      }
      float kf[EPL], vf[EPL];
      dequant16<KVT>(kw, kf);
      dequant16<KVT>(vw, vf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float s = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) s = fmaf(qv[h][e], kf[e], s);
#pragma unroll
        for (int off = 1; off < RL; off <<= 1) s += __shfl_xor(s, off, 64);
        if (p.cap_out > 0.0f) s = tanhf(s) * p.cap_out; // logit soft-cap, log2 units
        if (valid) {
          const float m_new = fmaxf(m_run[h], s);
          const float alpha = __builtin_amdgcn_exp2f(m_run[h] - m_new);
          const float pw = __builtin_amdgcn_exp2f(s - m_new);
          l_run[h] = l_run[h] * alpha + pw;
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(pw, vf[e], acc[h][e] * alpha);
          m_run[h] = m_new;
        }
      }
    }
  }

  // merge the row-group streams of the wave (log-sum-exp, lane exchanges)
#pragma unroll
  for (int off = RL; off < 64; off <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = __shfl_xor(m_run[h], off, 64);
      const float lo_ = __shfl_xor(l_run[h], off, 64);
      const float m_new = fmaxf(m_run[h], mo);
      const float a = (m_run[h] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_run[h] - m_new);
      const float c = (mo == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mo - m_new);
      l_run[h] = l_run[h] * a + lo_ * c;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float ao = __shfl_xor(acc[h][e], off, 64);
        acc[h][e] = acc[h][e] * a + ao * c;
      }
      m_run[h] = m_new;
    }
  }
  if (rg == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (h < g) {
        if (lr == 0) {
          sm_m[wave][h] = m_run[h];
          sm_l[wave][h] = l_run[h];
        }
#pragma unroll
        for (int e = 0; e < EPL; ++e) sm_o[(wave * 16 + h) * OSTRIDE + lr * EPL + e] = acc[h][e];
      }
    }
  }
  __syncthreads();
  merge_waves_and_store<D, OSTRIDE>(p, sm_m, sm_l, sm_o, b, kvh, 0, item, nb);
  finish_split<D>(p, blockIdx.y, b, kvh, 0, 1, item, split, nb, sm_o);
}

template <int D, int KVT>
hipError_t launch_valu_dk(const Params &p, const InlineWork &w, const Launch &l) {
  const dim3 grid(p.items, p.num_kv_heads);
  const int g = p.group;
  if (g == 1) return launch_kernel(l, partial_valu_kernel<D, KVT, 1>, grid, p, w);
  if (g == 2) return launch_kernel(l, partial_valu_kernel<D, KVT, 2>, grid, p, w);
  if (g <= 4) return launch_kernel(l, partial_valu_kernel<D, KVT, 4>, grid, p, w);
  if (g <= 8) return launch_kernel(l, partial_valu_kernel<D, KVT, 8>, grid, p, w);
  if constexpr (KVT != DT_FP8) return launch_kernel(l, partial_valu_kernel<D, KVT, 16>, grid, p, w);
  return hipErrorInvalidValue;
}

} // namespace

// Largest GQA group the vector kernel takes for a KV type.
int valu_max_group(int kv_dtype) { return kv_dtype == DT_FP8 ? 8 : 16; }

hipError_t launch_partial_valu(const Params &p, const InlineWork &w, int head_dim, int kv_dtype, const Launch &l) {
  if (p.part_row_scale) return hipErrorInvalidValue; // this kernel writes fp32 or code partials
  switch (kv_dtype) {
  case DT_F32:
    switch (head_dim) {
    case 64: return launch_valu_dk<64, DT_F32>(p, w, l);
    case 128: return launch_valu_dk<128, DT_F32>(p, w, l);
    case 256: return launch_valu_dk<256, DT_F32>(p, w, l);
    }
    break;
  case DT_BF16:
    switch (head_dim) {
    case 64: return launch_valu_dk<64, DT_BF16>(p, w, l);
    case 128: return launch_valu_dk<128, DT_BF16>(p, w, l);
    case 256: return launch_valu_dk<256, DT_BF16>(p, w, l);
    }
    break;
  case DT_FP8:
    switch (head_dim) {
    case 64: return launch_valu_dk<64, DT_FP8>(p, w, l);
    case 128: return launch_valu_dk<128, DT_FP8>(p, w, l);
    case 256: return launch_valu_dk<256, DT_FP8>(p, w, l);
    }
    break;
  }
  return hipErrorInvalidValue;
}

} // namespace kvs
