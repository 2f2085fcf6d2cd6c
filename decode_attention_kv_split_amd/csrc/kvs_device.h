// Device-side pieces shared by the split-KV decode kernels (gfx950).
//
// Work decomposition.  Request b has nq_b query rows (one in decode; its
// nq_b newest tokens with several) and L_b keys; the keys any of its queries
// sees start at lo_b = max(0, L_b - nq_b + 1 - window) (window > 0) and end
// at L_b.  Tokens are grouped in tiles of 16 aligned to absolute token
// positions; the chunks of a request start at A_b = lo_b rounded down to 16
// and are kv_chunk tokens long (a multiple of 16), so request b has
// n_b = max(1, ceil((L_b - A_b) / kv_chunk)) splits.  Work items of one KV
// head are numbered request by request; grid.x runs over them, grid.y over
// (KV-head pack, column group).  The host passes the item list in the kernel
// arguments when it fits; otherwise both kernels derive (request, split)
// from kv_len on the device.
//
// The workgroup that runs split 0 of KV head 0 of a request records the
// request's first work item and split count in meta[2b], meta[2b+1]; the merge
// kernel reads them instead of scanning the batch again.
//
// Columns.  A workgroup computes up to 16 columns of query rows: with one
// query per request, the gp = g * pack query heads of `pack` adjacent KV
// heads; with several, the (query row, head) pairs cg * 16 .. cg * 16 + 15 of
// one KV head (column c = row * g + head), in column group cg.  Partial
// results of split x of slot (pack kvg, column group cg) live in the
// workspace: o_part[((S * I + x) * cols + h) * D + d] with S = kvg *
// col_groups + cg (fp32, already divided by the chunk's sum and multiplied by
// the V scale) and lse_part[(S * I + x) * cols + h] (log2 domain: chunk max +
// log2(chunk sum), -inf when the chunk saw no key), I = items per KV head.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvs {

constexpr int kTile = 16;        // tokens per tile
constexpr int kWaves = 4;        // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int64_t kMaxWorkgroups = (int64_t{1} << 24) - 1; // per partial launch (kept below 2^32 work-items)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

enum : int { DT_F32 = 0, DT_BF16 = 1, DT_FP8 = 2, DT_INT4 = 3 }; // the kvs_dtype codes

// Where a kernel goes: its stream and, optionally, two events that the
// kernel's own dispatch stamps with its start and end time (no extra marker
// packets on the stream, so timing does not perturb what is timed).
struct Launch {
  hipStream_t stream;
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

template <typename Kernel, typename... Args>
hipError_t launch_kernel(const Launch &l, Kernel kernel, dim3 grid, Args... args) {
  hipExtLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, l.stream, l.start, l.stop, 0, args...);
  return hipGetLastError();
}

struct Params {
  const void *q;
  const void *k;
  const void *v;
  const int *page_indptr;
  const int *page_indices;
  const int *kv_len;
  const float *k_scale;
  const float *v_scale;
  void *o;
  float *lse;
  float *o_part;
  float *lse_part;
  int *meta;       // [batch][2]: first work item and split count of each request
  int batch;
  int num_qo_heads;
  int num_kv_heads;
  int group;
  int pack;       // KV heads per workgroup (partials and merge run per pack)
  int page_size;  // 0: contiguous
  int page_shift; // log2(page_size) when a power of two, else -1
  int window;
  int chunk;
  int items;      // work items per KV head
  const int *qo_indptr; // [batch + 1] query rows of each request; null: one row each
  int col_groups; // groups of 16 (query, head) columns per KV head (1 for one query)
  int col_share;  // column groups one partial workgroup computes together (1 or 2)
  int cols;       // columns per partial slot: group * pack (one query) or 16
  int rows_xcd_order; // multi-row kernels: workgroups in the XCD-balanced order (rows_order)
  float m_init;   // reference max each chunk starts from (log2 units; -inf: none)
  int out_bf16;   // o (and q) stored as bf16
  float score_scale; // sm_scale * log2(e); with a soft cap c: sm_scale / c
  float cap_out;     // soft cap: scores become tanh(score_scale * qk) * cap_out, cap_out = c * log2(e); 0: no cap
};

// Work lists planned on the host from kv_len_host and passed in the kernel
// arguments when they fit, which saves each workgroup a dependent memory read
// before its first K/V load; larger batches derive the same lists from kv_len
// on the device (scan_requests, meta).
constexpr int kInlineRequests = 256;
constexpr int kInlineItems = 448;
constexpr int kInlineMerges = 384;

struct InlineWork {
  int n_items;                   // items per KV head listed below; 0: not provided
  int req_len[kInlineRequests];  // kv_len of each request (the host copy)
  uint32_t item[kInlineItems];   // work item x: (request << 16) | split
};

struct InlineMerge {
  int n;                         // requests listed below; -1: not provided
  uint32_t req[kInlineMerges];   // (request << 16) | number of splits (> 1)
  uint32_t first[kInlineMerges]; // work item of the request's split 0
};

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// float -> bf16 bits, round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  __bf16 h = (__bf16)x;
  return __builtin_bit_cast(uint16_t, h);
}

typedef __attribute__((ext_vector_type(2))) float f32x2_ev;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_ev;

// Two floats -> two bf16 (round to nearest even) in one 32-bit word, low half
// first; a single v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_ev x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2_ev));
}

// Query rows of request b (its new tokens, the last ones of its cache).
__device__ __forceinline__ int req_nq(const Params &p, int b) {
  return p.qo_indptr ? p.qo_indptr[b + 1] - p.qo_indptr[b] : 1;
}

// First key any of a request's nq queries sees: its first query sits at
// position L - nq and sees the last `window` keys up to itself.
__device__ __forceinline__ int request_lo(int L, int nq, int window) {
  return window > 0 ? max(0, L - nq + 1 - window) : 0;
}

__device__ __forceinline__ int visible_lo(int L, int window) { return request_lo(L, 1, window); }

// Number of splits of a request with L keys and nq queries.
__device__ __forceinline__ int num_splits(int L, int nq, int window, int chunk) {
  const int a = request_lo(L, nq, window) & ~(kTile - 1);
  const int span = L - a;
  return span <= 0 ? 1 : (span + chunk - 1) / chunk;
}

// Where column h of (request b, KV-head pack kvg, column group cg) goes:
// output row and query head, or false for a padding column.  One query per
// request: the columns are the pack's query heads.  Several: column
// cg * 16 + h is (query row (cg * 16 + h) / g, head (cg * 16 + h) % g).
__device__ __forceinline__ bool column_target(const Params &p, int b, int kvg, int cg, int h, int &row, int &head) {
  if (!p.qo_indptr) {
    row = b;
    head = kvg * p.cols + h;
    return h < p.cols;
  }
  const int col = cg * 16 + h;
  const int q0 = p.qo_indptr[b];
  if (col >= (p.qo_indptr[b + 1] - q0) * p.group) return false;
  row = q0 + col / p.group;
  head = kvg * p.group + col % p.group;
  return true;
}

// Exclusive scan of per-request split counts over the whole batch, done by one
// 256-thread workgroup.  Calls f(b, first_item, n_b) for every request b whose
// range may interest the caller; returns nothing.  `scratch` holds 2 * 64 ints.
template <typename F>
__device__ __forceinline__ void scan_requests(const Params &p, int *scratch, F &&f) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int base = 0;
  for (int b0 = 0; b0 < p.batch; b0 += kThreads) {
    const int b = b0 + tid;
    const int nb = b < p.batch ? num_splits(p.kv_len[b], req_nq(p, b), p.window, p.chunk) : 0;
    // inclusive wave scan
    int incl = nb;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    if (lane == 63) scratch[wave] = incl;
    __syncthreads();
    int wave_base = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int t = scratch[w];
      wave_base += (w < wave) ? t : 0;
      total += t;
    }
    if (b < p.batch) f(b, base + wave_base + incl - nb, nb);
    base += total;
    __syncthreads();
  }
}

// Merge the per-wave softmax states staged in LDS and write either the final
// output (request with one split) or the split's partial.
//   sm_m[w][h], sm_l[w][h]: running max (log2 domain) and sum of wave w;
//   sm_o[w][h][d]: unnormalised accumulator of wave w (fp32).
template <int D, int OSTRIDE>
__device__ __forceinline__ void merge_waves_and_store(const Params &p, const float (*sm_m)[16],
                                                      const float (*sm_l)[16], const float *sm_o,
                                                      int b, int kvg, int cg, int item, int nb) {
  const int g = p.group;
  for (int idx = threadIdx.x; idx < p.cols * D; idx += kThreads) {
    const int h = idx / D;
    const int d = idx - h * D;
    int row, hq;
    if (!column_target(p, b, kvg, cg, h, row, hq)) continue; // padding column
    const float vscale = p.v_scale ? p.v_scale[b * p.num_kv_heads + hq / g] : 1.0f;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w][h]);
    float val = 0.0f, lse2 = -INFINITY;
    if (M != -INFINITY) {
      float L = 0.0f, acc = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float mw = sm_m[w][h];
        const float a = (mw == -INFINITY) ? 0.0f : exp2f(mw - M);
        L += a * sm_l[w][h];
        acc += a * sm_o[(w * 16 + h) * OSTRIDE + d];
      }
      if (L > 0.0f) { // a finite reference with no visible key leaves L = 0: empty
        val = acc / L * vscale;
        lse2 = M + __log2f(L);
      }
    }
    if (nb == 1) {
      const size_t off = ((size_t)row * p.num_qo_heads + hq) * D + d;
      if (p.out_bf16)
        reinterpret_cast<uint16_t *>(p.o)[off] = f32_to_bf16_bits(val);
      else
        reinterpret_cast<float *>(p.o)[off] = val;
      if (d == 0 && p.lse) p.lse[(size_t)row * p.num_qo_heads + hq] = lse2 * kLn2;
    } else {
      const size_t slot = ((size_t)kvg * p.col_groups + cg) * p.items + item;
      p.o_part[(slot * p.cols + h) * D + d] = val;
      if (d == 0) p.lse_part[slot * p.cols + h] = lse2;
    }
  }
}

} // namespace kvs
