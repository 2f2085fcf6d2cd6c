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
// col_groups + cg (already divided by the chunk's sum) and
// lse_part[(S * I + x) * cols + h] (fp32, log2 domain: chunk max + log2(chunk
// sum), -inf when the chunk saw no key), I = items per KV head.  o_part is
// fp32 for fp32 caches and for the bf16 launches the host keeps in fp32.
// For fp8 and INT4 caches (part_f16) it is fp16 and leaves the V scale to
// the merge: it then holds a weighted average of the decoded codes, which
// lies inside their range (|x| <= 448 for e4m3, <= 8 for INT4), where fp16
// keeps 11 significant bits; half the bytes of fp32.  A bf16 cache's averages
// have no such bound, so the decode, 32-column and 32x32 prefill kernels
// store each partial row scaled by a power of two that puts its
// largest magnitude in [2^14, 2^15) and leave the inverse in
// sc_part[(S * I + x) * cols + h] (part_row_scale); the merge multiplies it
// back (exact).
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
  int wave_packs; // KV-head packs per partial workgroup: 4 (one per wave, each over the
                  // whole chunk) or 1 (the four waves split one pack's tiles)
  int rows_xcd_order; // multi-row kernels: workgroups in the XCD-balanced order (rows_order)
  float m_init;   // reference max each chunk starts from (log2 units; -inf: none)
  int out_bf16;   // o (and q) stored as bf16
  int part_f16;   // split partials o_part are fp16: averages of the stored V codes (fp8, INT4 caches)
                  // or, with part_row_scale, row-scaled averages of bf16 V
  int part_row_scale; // each fp16 partial row is scaled; sc_part holds the multiplier that restores it
  float *sc_part;     // [slots][cols] multipliers (powers of two) of the partial rows (part_row_scale)
  float score_scale; // sm_scale * log2(e); with a soft cap c: sm_scale / c
  float cap_out;     // soft cap: scores become tanh(score_scale * qk) * cap_out, cap_out = c * log2(e); 0: no cap
  // Merge in the partial kernel (null: a second kernel merges): one arrival
  // counter per (partial-launch slot grid.y, request), zero between calls.
  unsigned *counters;
};

// Counters of the merge done inside the partial kernel sit at the start of
// the workspace: at most this many bytes, one uint32 per (grid.y slot,
// request).  They must be zero when a call starts; every call that uses
// them leaves them zero.
constexpr size_t kCounterBytes = 65536;

// Split partials (o_part, lse_part) that the merge inside the partial kernel
// reads back (Params::counters set) are written and read with device-scope
// relaxed atomic accesses: on gfx950 these are the sc1 forms of the plain
// loads and stores, which write through and read at the point where the
// XCDs' L2 caches are coherent.  So a partial written on one XCD is visible
// to the merging workgroup on another once its store has completed, and no
// workgroup needs a device-scope fence (a write-back and invalidate of its
// whole L2, which made every split workgroup pay for the others' traffic).
// Partials for the merge kernel are ordinary (cached, 16-byte) stores: the
// kernel boundary makes them visible.
__device__ __forceinline__ void store_coherent(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_partial(const Params &prm, float *p, float v) {
  if (prm.counters)
    store_coherent(p, v);
  else
    *p = v;
}
// four consecutive floats at p (16-byte aligned)
__device__ __forceinline__ void store_partial4(const Params &prm, float *p, float a, float b, float c, float d) {
  if (prm.counters) {
    store_coherent(p, a);
    store_coherent(p + 1, b);
    store_coherent(p + 2, c);
    store_coherent(p + 3, d);
  } else {
    *reinterpret_cast<float4 *>(p) = make_float4(a, b, c, d);
  }
}
__device__ __forceinline__ float load_partial(const float *p) {
  return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// fp16 partials (Params::part_f16): two values per dword, round to nearest even
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const half2_t h = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, h);
}
__device__ __forceinline__ float2 unpack_f16x2(uint32_t u) {
  const half2_t h = __builtin_bit_cast(half2_t, u);
  return make_float2((float)h.x, (float)h.y);
}
// Split partial dims e .. e + 3 of o_part (e: element index, a multiple of 4),
// in the partials' type (F16: Params::part_f16); written through to the
// coherent level when the partial kernel merges (Params::counters).
template <bool F16>
__device__ __forceinline__ void store_part4(const Params &prm, size_t e, float a, float b, float c, float d) {
  if constexpr (F16) {
    uint32_t *q = reinterpret_cast<uint32_t *>(prm.o_part) + e / 2;
    const uint32_t lo = pack_f16x2(a, b), hi = pack_f16x2(c, d);
    if (prm.counters) {
      __hip_atomic_store(q, lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(q + 1, hi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      *reinterpret_cast<uint2 *>(q) = make_uint2(lo, hi);
    }
  } else {
    store_partial4(prm, prm.o_part + e, a, b, c, d);
  }
}
__device__ __forceinline__ void store_part4(const Params &prm, size_t e, float a, float b, float c, float d) {
  if (prm.part_f16)
    store_part4<true>(prm, e, a, b, c, d);
  else
    store_part4<false>(prm, e, a, b, c, d);
}
// One element e of o_part (store_part4 where four consecutive dims are at hand).
template <bool F16> __device__ __forceinline__ void store_part1(const Params &prm, size_t e, float v) {
  if constexpr (F16) {
    uint16_t *q = reinterpret_cast<uint16_t *>(prm.o_part) + e;
    const uint16_t h = __builtin_bit_cast(uint16_t, (_Float16)v);
    if (prm.counters)
      __hip_atomic_store(q, h, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      *q = h;
  } else {
    store_partial(prm, prm.o_part + e, v);
  }
}
// Row-scaled fp16 partials (Params::part_row_scale): a partial row whose
// largest magnitude is mx is stored times 2^k, which puts mx in [2^14, 2^15)
// (11 significant bits there, no fp16 overflow); the merge multiplies by 2^-k
// (both exact).  k is kept within [-85, 115] so that both factors stay normal
// fp32 numbers.
__device__ __forceinline__ int row_scale_exp(float mx) {
  int ex = 0;
  (void)frexpf(mx, &ex); // mx = f * 2^ex, f in [0.5, 1); 0 gives ex = 0
  return 15 - min(max(ex, -100), 100);
}
// Kernels that know their KV type at compile time: the host sets
// Params::part_f16 by the same rule.
template <int KT> constexpr bool part_f16_of() { return KT == DT_FP8 || KT == DT_INT4; }
// The stored bits of dims 4 i .. 4 i + 3 of o_part (i: index in units of four
// elements): two dwords of fp16 pairs (F16; z, w unused) or four fp32.  The
// merge keeps the raw bits until every load of a batch is issued, and
// converts them afterwards (part_bits_to_float4): converted inside the
// guarded load, the compiler waited for each split's load before issuing
// the next one.
template <bool F16, bool COHERENT>
__device__ __forceinline__ uint4 load_part_bits(const float *o_part, size_t i) {
  if constexpr (F16) {
    const uint32_t *q = reinterpret_cast<const uint32_t *>(o_part) + 2 * i;
    if constexpr (COHERENT) {
      return make_uint4(__hip_atomic_load(const_cast<uint32_t *>(q), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                        __hip_atomic_load(const_cast<uint32_t *>(q + 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                        0u, 0u);
    } else {
      const uint2 u = *reinterpret_cast<const uint2 *>(q);
      return make_uint4(u.x, u.y, 0u, 0u);
    }
  } else if constexpr (COHERENT) {
    const float *o = o_part + 4 * i;
    return make_uint4(__float_as_uint(load_partial(o)), __float_as_uint(load_partial(o + 1)),
                      __float_as_uint(load_partial(o + 2)), __float_as_uint(load_partial(o + 3)));
  } else {
    return reinterpret_cast<const uint4 *>(o_part)[i];
  }
}
// The four values of load_part_bits (all-zero bits are 0 in both forms).
template <bool F16> __device__ __forceinline__ float4 part_bits_to_float4(const uint4 &u) {
  if constexpr (F16) {
    const float2 a = unpack_f16x2(u.x), b = unpack_f16x2(u.y);
    return make_float4(a.x, a.y, b.x, b.y);
  } else {
    return make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w));
  }
}
// The V scale a partial's writer applies to o: none where the merge applies it.
__device__ __forceinline__ bool writer_scales_v(const Params &p, int nb) { return nb == 1 || !p.part_f16; }
// The V scale the merge applies to the merged o of KV head kvh of request b.
__device__ __forceinline__ float merge_vscale(const Params &p, int b, int kvh) {
  return p.part_f16 && p.v_scale ? p.v_scale[b * p.num_kv_heads + kvh] : 1.0f;
}
// Waits until every memory access this thread issued has completed (vmcnt 0;
// on gfx9 stores count there too), and keeps the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void wait_all_vmem() {
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8)); // vmcnt(0), expcnt and lgkmcnt untouched
  __asm__ volatile("" ::: "memory");
}

// Work lists planned on the host from kv_len_host and passed in the kernel
// arguments when they fit, which saves each workgroup a dependent memory read
// before its first K/V load; larger batches derive the same lists from kv_len
// on the device (scan_requests, meta).
// An item is 16 bits, request and split 8 bits each, so the list holds up to
// 1344 items of at most 256 requests with at most 256 splits each.
constexpr int kInlineRequests = 256;
constexpr int kInlineSplits = 256;
constexpr int kInlineItems = 1344;
constexpr int kInlineMerges = 384;

struct InlineWork {
  int n_items;                   // items per KV head listed below; 0: not provided
  int req_len[kInlineRequests];  // kv_len of each request (the host copy)
  uint16_t item[kInlineItems];   // work item x: (request << 8) | split
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
// One thread per column first turns the waves' states into weights
// 2^(m_w - M) * v_scale / L (over sm_m; without v_scale for fp16 partials)
// and the column's lse (into
// sm_l[0]); then every thread combines four dims of one column with them.
// The whole workgroup calls it (one barrier inside); sm_m and sm_l are
// overwritten.
// ROWSC: a split's partial rows are stored row-scaled (part_row_scale) when
// the host asks for it.
template <int D, int OSTRIDE, bool ROWSC = false>
__device__ __forceinline__ void merge_waves_and_store(const Params &p, float (*sm_m)[16], float (*sm_l)[16],
                                                      const float *sm_o, int b, int kvg, int cg, int item, int nb) {
  static_assert(D % 4 == 0 && OSTRIDE % 4 == 0, "float4 rows");
  const int tid = threadIdx.x;
  if (tid < p.cols) { // at most 16 columns
    const int h = tid;
    int row, hq;
    const bool has = column_target(p, b, kvg, cg, h, row, hq);
    const float vscale =
        has && p.v_scale && writer_scales_v(p, nb) ? p.v_scale[b * p.num_kv_heads + hq / p.group] : 1.0f;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w][h]);
    float a[kWaves];
    float L = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = sm_m[w][h];
      a[w] = (mw == -INFINITY) ? 0.0f : exp2f(mw - M);
      L += a[w] * sm_l[w][h];
    }
    // no visible key (M = -inf), or a finite reference with none (L = 0): empty
    const bool live = M != -INFINITY && L > 0.0f;
    const float inv = live ? vscale / L : 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) sm_m[w][h] = a[w] * inv;
    sm_l[0][h] = live ? M + __log2f(L) : -INFINITY;
  }
  __syncthreads();
  for (int idx = tid; idx < p.cols * (D / 4); idx += kThreads) {
    const int h = idx / (D / 4);
    const int d = 4 * (idx - h * (D / 4));
    int row, hq;
    if (!column_target(p, b, kvg, cg, h, row, hq)) continue; // padding column
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float c = sm_m[w][h];
      const float4 x = *reinterpret_cast<const float4 *>(sm_o + (w * 16 + h) * OSTRIDE + d);
      v.x += c * x.x;
      v.y += c * x.y;
      v.z += c * x.z;
      v.w += c * x.w;
    }
    const float lse2 = sm_l[0][h];
    if (nb == 1) {
      const size_t off = ((size_t)row * p.num_qo_heads + hq) * D + d;
      if (p.out_bf16)
        *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(p.o) + off) =
            make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
      else
        *reinterpret_cast<float4 *>(reinterpret_cast<float *>(p.o) + off) = v;
      if (d == 0 && p.lse) p.lse[(size_t)row * p.num_qo_heads + hq] = lse2 * kLn2;
    } else {
      const size_t slot = ((size_t)kvg * p.col_groups + cg) * p.items + item;
      if (ROWSC && p.part_row_scale) {
        // the row's largest magnitude over the D / 4 threads of its column
        // (aligned lanes of one wave, all active: a column is padding or not
        // as a whole)
        float mx = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
#pragma unroll
        for (int off = 1; off < D / 4; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
        const int k = row_scale_exp(mx);
        const float sc = ldexpf(1.0f, k);
        store_part4<true>(p, (slot * p.cols + h) * D + d, v.x * sc, v.y * sc, v.z * sc, v.w * sc);
        if (d == 0) store_partial(p, p.sc_part + slot * p.cols + h, ldexpf(1.0f, -k));
      } else {
        store_part4(p, (slot * p.cols + h) * D + d, v.x, v.y, v.z, v.w);
      }
      if (d == 0) store_partial(p, p.lse_part + slot * p.cols + h, lse2);
    }
  }
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of split partials.  For an output with splits c holding a
// normalised partial o_c and a log2-domain log-sum-exp l_c:
//   M = max_c l_c,  w_c = 2^(l_c - M),  o = sum_c w_c o_c / sum_c w_c,
//   lse = (M + log2 sum_c w_c) * ln 2,  all l_c = -inf -> o = 0, lse = -inf.
// This is the online-softmax rescale ("Forcing Flash Attention onto TPU",
// section "Flash Attention in JAX": multiply the old accumulator and sum by
// exp(old max - new max)) applied across chunks; the FlashDecoding++
// explainer's asynchronous-softmax section describes this synchronised update
// of per-tile partial softmax results with the previous max and sum.

// Splits whose loads are in flight together per thread: 16 in the merge
// kernel; fewer where the merge runs at the end of a partial kernel, whose
// register budget it shares.
constexpr int kMergeBatch = 16;
constexpr int kFusedMergeBatch = 8;

struct MergeState {
  float m;    // running max of the split LSEs (log2 domain)
  float w;    // sum of 2^(lse_c - m)
  float4 acc; // sum of 2^(lse_c - m) * o_c
};

__device__ __forceinline__ void merge_fold(MergeState &st, float lc, const float4 &o) {
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

__device__ __forceinline__ void merge_combine(MergeState &a, const MergeState &b) {
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

// Combine the states of SG thread groups into group 0: group tg = tid / F
// holds a share of the splits of output tid % F.  Pairwise, in about
// log2(SG) rounds through LDS (one combine after another took SG - 1
// dependent LDS round trips).  In round s the groups tg = 0 mod 2s take in
// group tg + s, which writes nothing that round.  The whole workgroup calls
// it with the same F and SG (its barriers are uniform); s_st holds kThreads
// states.
__device__ __forceinline__ void merge_groups(MergeState &st, MergeState *s_st, int F, int SG) {
  const int tid = threadIdx.x;
  const int tg = tid / F;
  s_st[tid] = st;
  __syncthreads();
  for (int s = 1; s < SG; s <<= 1) {
    if (tg % (2 * s) == 0 && tg + s < SG) {
      merge_combine(st, s_st[tid + s * F]);
      s_st[tid] = st;
    }
    __syncthreads();
  }
}

// Fold splits tg, tg + step, ... (< nb) of four outputs: their LSEs at
// lp[c * lstride] and partials at four-element index o4 + c * ostride of
// o_part (load_part_bits; F16: fp16 partials), NB loads of each in flight at a
// time.
// COHERENT: read at the coherent level (the merge inside the partial kernel,
// which may read partials other XCDs wrote in the same launch); otherwise
// plain loads (the merge kernel, after the partial kernel has ended).
// SC: partial rows carry multipliers at sp[c * lstride] (part_row_scale).
template <int NB, bool COHERENT, bool F16, bool SC = false>
__device__ __forceinline__ void merge_fold_splits(MergeState &st, const float *lp, size_t lstride,
                                                  const float *o_part, size_t o4, size_t ostride, int tg, int step,
                                                  int nb, const float *sp = nullptr) {
  for (int c0 = tg; c0 < nb; c0 += step * NB) {
    float lc[NB], sc[NB];
    uint4 raw[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int c = c0 + u * step;
      sc[u] = 1.0f;
      if (c < nb) {
        lc[u] = COHERENT ? load_partial(lp + (size_t)c * lstride) : lp[(size_t)c * lstride];
        raw[u] = load_part_bits<F16, COHERENT>(o_part, o4 + (size_t)c * ostride);
        if constexpr (SC) sc[u] = COHERENT ? load_partial(sp + (size_t)c * lstride) : sp[(size_t)c * lstride];
      } else {
        lc[u] = -INFINITY;
        raw[u] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      float4 v = part_bits_to_float4<F16>(raw[u]);
      if constexpr (SC) v = make_float4(v.x * sc[u], v.y * sc[u], v.z * sc[u], v.w * sc[u]);
      merge_fold(st, lc[u], v);
    }
  }
}

// Final output of one merged float4 (dims d .. d + 3 of query row / head
// (row, hq)), times vs (merge_vscale), and its lse from the thread that holds
// dim 0.
__device__ __forceinline__ void merge_store(const Params &p, const MergeState &st, int row, int hq, int D, int d,
                                            float vs) {
  const float inv = st.w > 0.0f ? vs / st.w : 0.0f;
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

// Merge every split of request b for column groups cg_first .. cg_first +
// ncg - 1 of KV-head pack kvg (its splits are work items first .. first + nb
// - 1) and write the final outputs.  The whole workgroup calls it; s_st holds
// kThreads states of LDS.  When the outputs are fewer than the threads,
// thread groups share the splits of each output and combine through LDS.
// PACK: KV heads per pack (1 with several query rows per request).  ROWSC:
// the kernel may write row-scaled fp16 partials (part_row_scale).
template <int D, int PACK, int NB, bool ROWSC>
__device__ void merge_splits(const Params &p, int b, int kvg, int cg_first, int ncg, int first, int nb,
                             MergeState *s_st) {
  constexpr int D4 = D / 4;
  const int tid = threadIdx.x;
  const int cols = p.cols;
  const int ncg_live = min(ncg, p.col_groups - cg_first);
  const int F = ncg_live * cols * D4;                // float4 outputs
  const int SG = F >= kThreads ? 1 : kThreads / F;  // thread groups over the splits
  const size_t ostride = (size_t)cols * D4;         // four-element units between consecutive splits of one slot
  for (int f0 = 0; f0 < F; f0 += kThreads) {
    const int t = f0 + (SG > 1 ? tid % F : tid);
    const int tg = SG > 1 ? tid / F : 0;
    const int cgi = t / (cols * D4);
    const int h = (t / D4) % cols;
    const int d = 4 * (t % D4);
    int row = 0, hq = 0;
    const bool has = t < F && tg < SG && column_target(p, b, kvg, cg_first + cgi, h, row, hq);
    MergeState st = {-INFINITY, 0.0f, make_float4(0.f, 0.f, 0.f, 0.f)};
    // the column's KV head: uniform in the workgroup with one KV head per pack
    const float vs = merge_vscale(p, b, PACK == 1 ? kvg : kvg * PACK + h / p.group);
    if (has) {
      const size_t slot0 = ((size_t)kvg * p.col_groups + cg_first + cgi) * p.items + first;
      const size_t o4 = (slot0 * cols + h) * D4 + d / 4;
      if (ROWSC && p.part_row_scale)
        merge_fold_splits<NB, true, true, ROWSC>(st, p.lse_part + slot0 * cols + h, cols, p.o_part, o4, ostride, tg,
                                                SG, nb, p.sc_part + slot0 * cols + h);
      else if (p.part_f16)
        merge_fold_splits<NB, true, true>(st, p.lse_part + slot0 * cols + h, cols, p.o_part, o4, ostride, tg, SG, nb);
      else
        merge_fold_splits<NB, true, false>(st, p.lse_part + slot0 * cols + h, cols, p.o_part, o4, ostride, tg, SG,
                                           nb);
    }
    if (SG > 1) merge_groups(st, s_st, F, SG); // one pass only (F < kThreads): uniform
    if (has && tg == 0) merge_store(p, st, row, hq, D, d, vs);
  }
}

// End of a partial workgroup whose request has several splits: count its
// arrival for (grid.y slot `yslot`, request b); the workgroup that brings the
// last split merges them all (merge_splits, for each of its npack KV-head
// packs kvg .. kvg + npack - 1) and resets the counter, so no
// second kernel runs and no workgroup ever waits for another.  Every thread's
// partial stores (store_partial with counters: written through to the device-coherent
// level) have completed before the count, and the merging workgroup reads
// them back with load_partial after it.
// Call with the whole workgroup, after the partial stores; `lds` (at least
// kThreads MergeStates) may be any LDS no thread still reads.  NB: loads in
// flight per thread during the merge (fewer where registers are tight).
template <int D, int PACK = 1, int NB = kFusedMergeBatch, bool ROWSC = false>
__device__ __forceinline__ void finish_split(const Params &p, int yslot, int b, int kvg, int cg_first, int ncg,
                                             int item, int split, int nb, void *lds, int npack = 1) {
  __shared__ int s_last;
  if (nb <= 1 || !p.counters) return; // the same in every thread
  wait_all_vmem(); // this thread's partial stores have completed
  __syncthreads();
  unsigned *ctr = p.counters + (size_t)yslot * p.batch + b;
  if (threadIdx.x == 0) s_last = atomicAdd(ctr, 1u) == (unsigned)(nb - 1);
  __syncthreads();
  if (!s_last) return;
  for (int k = 0; k < npack; ++k) { // KV-head packs kvg .. kvg + npack - 1 (the same in every thread)
    if (k > 0) __syncthreads();     // the previous pack's merge has read its LDS states
    merge_splits<D, PACK, NB, ROWSC>(p, b, kvg + k, cg_first, ncg, item - split, nb, reinterpret_cast<MergeState *>(lds));
  }
  if (threadIdx.x == 0) atomicExch(ctr, 0u); // every split of this call has arrived: ready for the next call
}

} // namespace kvs
