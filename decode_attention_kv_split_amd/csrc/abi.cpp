// C ABI of the split-KV decode-attention library: argument validation on the
// host, planning, and the two launches (partial softmax per chunk, then the
// log-sum-exp merge).  No device memory is allocated and nothing synchronises.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>
#include <vector>

#include "kvsplit.h"
#include "kvs_device.h"
#include "plan.h"

namespace kvs {
hipError_t launch_partial_mfma(const Params &p, const InlineWork &w, int head_dim, int kv_type, const Launch &l);
hipError_t launch_partial_valu(const Params &p, const InlineWork &w, int head_dim, int kv_dtype, const Launch &l);
hipError_t launch_merge(const Params &p, const InlineMerge &ml, int head_dim, int max_splits, hipStream_t stream);
int valu_max_group(int kv_dtype);
int mfma_pack(int head_dim, int group, int num_kv_heads, int kv_type, bool allow_pack);
bool mfma_packable(int head_dim, int group, int num_kv_heads, int kv_type);
int mfma_col_share(int head_dim, int kv_type, int col_groups);
bool mfma_head_dim_ok(int head_dim, int kv_type);
bool rows_merge_in_kernel(int head_dim, int kv_type);
hipError_t launch_append(const kvs_append_args *a, const Launch &l);
} // namespace kvs

static_assert(kvs::kPlanInlineRequests == kvs::kInlineRequests && kvs::kPlanInlineItems == kvs::kInlineItems &&
                  kvs::kPlanInlineSplits == kvs::kInlineSplits,
              "planner and kernels agree on the inline work-list sizes");
static_assert(sizeof(kvs::Params) + sizeof(kvs::InlineWork) <= 4096, "kernel arguments fit 4 KB");
static_assert(kvs::kPlanCounterBytes == kvs::kCounterBytes && kvs::kCounterBytes == KVS_WORKSPACE_COUNTER_BYTES,
              "planner, kernels and header agree on the counter area");

namespace {

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

int log2i(int x) {
  int s = 0;
  while ((1 << s) < x) ++s;
  return s;
}

// Host-only checks shared by plan and decode.  need_ptrs: device pointers must
// be non-null.  Resolves the kernel family into *algo.
kvs_status validate(const kvs_decode_args *a, bool need_ptrs, int *algo) {
  if (!a) return KVS_ERR_INVALID_ARG;
  if (a->batch < 1 || a->num_qo_heads < 1 || a->num_kv_heads < 1) return KVS_ERR_INVALID_ARG;
  if (a->num_qo_heads % a->num_kv_heads) return KVS_ERR_INVALID_ARG;
  if (a->head_dim != 64 && a->head_dim != 128 && a->head_dim != 256) return KVS_ERR_UNSUPPORTED;
  const int group = a->num_qo_heads / a->num_kv_heads;
  if (group > 16) return KVS_ERR_UNSUPPORTED;
  // 16 rows of one KV head must be addressable with 32-bit byte offsets
  if ((int64_t)a->num_kv_heads * a->head_dim * 4 * 16 >= ((int64_t)1 << 31)) return KVS_ERR_UNSUPPORTED;
  const bool pair_ok = (a->q_dtype == KVS_F32 && a->kv_dtype == KVS_F32) ||
                       (a->q_dtype == KVS_BF16 && a->kv_dtype == KVS_BF16) ||
                       (a->q_dtype == KVS_BF16 && a->kv_dtype == KVS_FP8_E4M3) ||
                       (a->q_dtype == KVS_BF16 && a->kv_dtype == KVS_INT4);
  if (a->q_dtype < 0 || a->q_dtype > 2 || a->kv_dtype < 0 || a->kv_dtype > 3) return KVS_ERR_INVALID_ARG;
  if (!pair_ok) return KVS_ERR_UNSUPPORTED;
  const bool scaled = a->kv_dtype == KVS_FP8_E4M3 || a->kv_dtype == KVS_INT4;
  if (a->page_size < 0) return KVS_ERR_INVALID_ARG;
  if (a->page_size == 0 && a->batch != 1) return KVS_ERR_INVALID_ARG;
  if (a->page_size > 0 && !is_pow2(a->page_size)) return KVS_ERR_UNSUPPORTED;
  if (a->page_size > 0 && a->num_pages < 1) return KVS_ERR_INVALID_ARG;
  if (a->num_pages < 0) return KVS_ERR_INVALID_ARG;
  if (!(a->sm_scale > 0.0f) || !std::isfinite(a->sm_scale)) return KVS_ERR_INVALID_ARG;
  if (a->window < -1 || a->window == 0) return KVS_ERR_INVALID_ARG;
  if (a->kv_chunk < 0) return KVS_ERR_INVALID_ARG;
  if (a->num_cus < 0) return KVS_ERR_INVALID_ARG;
  if (!a->kv_len_host) return KVS_ERR_INVALID_ARG;
  if (a->use_unified_max != 0 && a->use_unified_max != 1) return KVS_ERR_INVALID_ARG;
  if (a->use_unified_max && !std::isfinite(a->unified_max)) return KVS_ERR_INVALID_ARG;
  if (!(a->logits_soft_cap >= 0.0f) || !std::isfinite(a->logits_soft_cap)) return KVS_ERR_INVALID_ARG;
  if (a->merge_mode < KVS_MERGE_AUTO || a->merge_mode > KVS_MERGE_KERNEL) return KVS_ERR_INVALID_ARG;
  if (a->wave_split < KVS_WAVES_AUTO || a->wave_split > KVS_WAVES_TILES) return KVS_ERR_INVALID_ARG;
  for (int b = 0; b < a->batch; ++b) {
    const int L = a->kv_len_host[b];
    if (L < 0) return KVS_ERR_INVALID_ARG;
    // the pool (paged) or the rows of the cache (contiguous) must hold L tokens
    const int64_t capacity = a->page_size > 0 ? (int64_t)a->num_pages * a->page_size : (int64_t)a->num_pages;
    if ((int64_t)L > capacity) return KVS_ERR_INVALID_ARG;
  }
  // several queries per request: row offsets start at 0, never decrease, and
  // a request has at most kv_len new tokens
  const bool multi = a->qo_indptr_host != nullptr;
  if (!multi && a->qo_indptr) return KVS_ERR_INVALID_ARG;
  if (multi) {
    if (a->qo_indptr_host[0] != 0) return KVS_ERR_INVALID_ARG;
    for (int b = 0; b < a->batch; ++b) {
      const int n = a->qo_indptr_host[b + 1] - a->qo_indptr_host[b];
      if (n < 0 || n > a->kv_len_host[b]) return KVS_ERR_INVALID_ARG;
    }
  }
  if (need_ptrs) {
    if (!a->q || !a->k || !a->v || !a->kv_len || !a->o) return KVS_ERR_INVALID_ARG;
    // rows of q and o move in 16-byte pieces
    if ((reinterpret_cast<uintptr_t>(a->q) | reinterpret_cast<uintptr_t>(a->o)) & 15) return KVS_ERR_INVALID_ARG;
    if (a->page_size > 0 && (!a->page_indptr || !a->page_indices)) return KVS_ERR_INVALID_ARG;
    if (scaled && (!a->k_scale || !a->v_scale)) return KVS_ERR_INVALID_ARG;
    if (multi && !a->qo_indptr) return KVS_ERR_INVALID_ARG;
  }
  // kernel family (INT4 runs on the matrix-core kernel only)
  const bool mfma_ok = a->kv_dtype != KVS_F32 && a->q_dtype == KVS_BF16 &&
                       (a->page_size == 0 || a->page_size >= 16) &&
                       kvs::mfma_head_dim_ok(a->head_dim, a->kv_dtype);
  const bool valu_ok = a->kv_dtype != KVS_INT4 && !multi && group <= kvs::valu_max_group(a->kv_dtype);
  switch (a->algo) {
  case KVS_ALGO_AUTO:
    if (mfma_ok)
      *algo = a->kv_dtype == KVS_INT4 && !multi &&
                      kvs::mfma_packable(a->head_dim, group, a->num_kv_heads, a->kv_dtype)
                  ? KVS_ALGO_MFMA_PACKED
                  : KVS_ALGO_MFMA;
    else if (valu_ok)
      *algo = KVS_ALGO_VALU;
    else
      return KVS_ERR_UNSUPPORTED;
    break;
  case KVS_ALGO_MFMA:
  case KVS_ALGO_MFMA_PACKED:
    if (!mfma_ok) return KVS_ERR_UNSUPPORTED;
    if (a->algo == KVS_ALGO_MFMA_PACKED && multi) return KVS_ERR_UNSUPPORTED; // columns are (query, head) pairs
    *algo = a->algo;
    break;
  case KVS_ALGO_VALU:
    if (!valu_ok) return KVS_ERR_UNSUPPORTED;
    *algo = KVS_ALGO_VALU;
    break;
  default:
    return KVS_ERR_INVALID_ARG;
  }
  return KVS_OK;
}

// Host-only checks of kvs_append.
kvs_status validate_append(const kvs_append_args *a) {
  if (!a) return KVS_ERR_INVALID_ARG;
  if (a->batch < 1 || a->num_qo_heads < 1 || a->num_kv_heads < 1) return KVS_ERR_INVALID_ARG;
  if (a->num_qo_heads % a->num_kv_heads) return KVS_ERR_INVALID_ARG;
  if (a->head_dim != 64 && a->head_dim != 128 && a->head_dim != 256) return KVS_ERR_UNSUPPORTED;
  if (a->q_dtype < 0 || a->q_dtype > 2 || a->kv_dtype < 0 || a->kv_dtype > 3) return KVS_ERR_INVALID_ARG;
  const bool pair_ok = (a->q_dtype == KVS_F32 && a->kv_dtype == KVS_F32) ||
                       (a->q_dtype == KVS_BF16 && a->kv_dtype == KVS_BF16) ||
                       (a->q_dtype == KVS_BF16 && a->kv_dtype == KVS_FP8_E4M3) ||
                       (a->q_dtype == KVS_BF16 && a->kv_dtype == KVS_INT4);
  if (!pair_ok) return KVS_ERR_UNSUPPORTED;
  // INT4 caches exist at the head sizes the decode kernels read
  if (a->kv_dtype == KVS_INT4 && a->head_dim != 128 && a->head_dim != 256) return KVS_ERR_UNSUPPORTED;
  const bool scaled = a->kv_dtype == KVS_FP8_E4M3 || a->kv_dtype == KVS_INT4;
  if (a->page_size < 0 || a->num_pages < 1) return KVS_ERR_INVALID_ARG;
  if (a->page_size == 0 && a->batch != 1) return KVS_ERR_INVALID_ARG;
  if (a->page_size > 0 && !is_pow2(a->page_size)) return KVS_ERR_UNSUPPORTED;
  if (!(a->norm_eps >= 0.0f) || !std::isfinite(a->norm_eps)) return KVS_ERR_INVALID_ARG;
  if (!(a->rope_theta >= 0.0f) || !std::isfinite(a->rope_theta)) return KVS_ERR_INVALID_ARG;
  if (a->rope_interleave != 0 && a->rope_interleave != 1) return KVS_ERR_INVALID_ARG;
  // token rows: one per request, or a packed ragged batch
  if ((a->qo_indptr == nullptr) != (a->qo_indptr_host == nullptr)) return KVS_ERR_INVALID_ARG;
  int64_t rows = a->batch;
  if (a->qo_indptr_host) {
    if (a->qo_indptr_host[0] != 0) return KVS_ERR_INVALID_ARG;
    for (int b = 0; b < a->batch; ++b)
      if (a->qo_indptr_host[b + 1] < a->qo_indptr_host[b]) return KVS_ERR_INVALID_ARG;
    rows = a->qo_indptr_host[a->batch];
  }
  if (rows * (a->num_qo_heads + a->num_kv_heads) > ((int64_t)1 << 32) / kvs::kThreads * kvs::kWaves)
    return KVS_ERR_UNSUPPORTED; // one launch holds fewer than 2^32 work-items
  if (!a->q_in || !a->k_in || !a->v_in || !a->q_out || !a->k_cache || !a->v_cache || !a->kv_len)
    return KVS_ERR_INVALID_ARG;
  if (a->page_size > 0 && (!a->page_indptr || !a->page_indices)) return KVS_ERR_INVALID_ARG;
  if (scaled && (!a->k_scale || !a->v_scale)) return KVS_ERR_INVALID_ARG;
  return KVS_OK;
}

kvs_status resolve_cus(const kvs_decode_args *a, int *cus) {
  if (a->num_cus > 0) {
    *cus = a->num_cus;
    return KVS_OK;
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return KVS_ERR_HIP;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
    return KVS_ERR_HIP;
  *cus = n;
  return KVS_OK;
}

// Query rows per request and the column groups they need (several queries
// per request only; otherwise nq stays empty and there is one group).
struct Columns {
  std::vector<int32_t> nq;
  int col_groups = 1;
  int col_share = 1;  // groups per partial workgroup
  int col_blocks = 1; // partial workgroups per (item, KV head) along the columns
  int cols = 0;       // partial-result columns per KV head over all groups
  int most = 1;       // query rows of the longest request
};

Columns columns_of(const kvs_decode_args *a) {
  Columns c;
  const int group = a->num_qo_heads / a->num_kv_heads;
  c.cols = group;
  if (!a->qo_indptr_host) return c;
  c.nq.resize(a->batch);
  int most = 0;
  for (int b = 0; b < a->batch; ++b) {
    c.nq[b] = a->qo_indptr_host[b + 1] - a->qo_indptr_host[b];
    most = std::max(most, c.nq[b]);
  }
  c.most = most;
  c.col_groups = std::max(1, (int)(((int64_t)most * group + 15) / 16));
  c.col_share = kvs::mfma_col_share(a->head_dim, a->kv_dtype, c.col_groups);
  c.col_blocks = (c.col_groups + c.col_share - 1) / c.col_share;
  c.cols = c.col_groups * 16;
  return c;
}

// Split partials of fp8 and INT4 caches are fp16 averages of the stored codes
// (the merge applies the V scale); those of fp32 caches are fp32.  Those of
// bf16 caches are fp16 rows scaled by a power of two (the multiplier beside
// each row's LSE) where the decode kernel, the 32-column kernel (one or two
// column groups per workgroup) or the 32x32 prefill kernel (four or more, at
// head_dim 128 or 256) writes them; the shared-tile kernel (several rows at
// head_dim 64) writes them in fp32.
bool part_codes_f16(const kvs_decode_args *a) { return a->kv_dtype == KVS_FP8_E4M3 || a->kv_dtype == KVS_INT4; }
bool part_row_scaled(const kvs_decode_args *a, int algo, const Columns &c) {
  return a->kv_dtype == KVS_BF16 && algo != KVS_ALGO_VALU && (c.col_share <= 2 || a->head_dim >= 128);
}

// KV heads per partial workgroup for the resolved kernel family.

int kv_pack(const kvs_decode_args *a, int algo) {
  if (algo == KVS_ALGO_VALU) return 1;
  return kvs::mfma_pack(a->head_dim, a->num_qo_heads / a->num_kv_heads, a->num_kv_heads, a->kv_dtype,
                        algo == KVS_ALGO_MFMA_PACKED);
}

// Whether one KV-head pack per wave (KVS_WAVES_HEADS) applies: every
// request has one query row and the matrix-core packs come in fours.
bool heads_fit(const kvs_decode_args *a, int algo, const Columns &c) {
  return algo != KVS_ALGO_VALU && !a->qo_indptr_host && c.col_groups == 1 &&
         (a->num_kv_heads / kv_pack(a, algo)) % kvs::kWaves == 0;
}

// Whether the partial kernel merges the splits itself: the plan allows it
// (host work list, counters fit) and the kernel that runs has the merge
// compiled in (the shared-tile kernel for INT4 at head_dim 256 does not).
bool merges_in_partial(const kvs::Plan &pl, const kvs_decode_args *a, const Columns &c) {
  if (!pl.fused || a->merge_mode == KVS_MERGE_KERNEL) return false;
  if (c.col_share >= 4 && !kvs::rows_merge_in_kernel(a->head_dim, a->kv_dtype)) return false;
  return a->merge_mode == KVS_MERGE_IN_PARTIAL || pl.fused_pays;
}

kvs_status plan_call(const kvs_decode_args *a, bool need_ptrs, kvs::Plan *pl, int *algo, int *cus,
                     Columns *cols_out = nullptr) {
  kvs_status st = validate(a, need_ptrs, algo);
  if (st != KVS_OK) return st;
  st = resolve_cus(a, cus);
  if (st != KVS_OK) return st;
  Columns c = columns_of(a);
  const int pack = kv_pack(a, *algo);
  const bool heads = heads_fit(a, *algo, c);
  if (a->wave_split == KVS_WAVES_HEADS && !heads) return KVS_ERR_UNSUPPORTED;
  const int32_t *nq = c.nq.empty() ? nullptr : c.nq.data();
  const bool row_scaled = part_row_scaled(a, *algo, c);
  const int part_bytes = part_codes_f16(a) || row_scaled ? 2 : 4;
  const int min_chunk = *algo != KVS_ALGO_VALU && c.col_share == 1 ? kvs::kMinMatrixChunk : kvs::kMinChunk;
  if (!kvs::make_plan(a->kv_len_host, nq, a->batch, a->window, a->num_kv_heads, c.cols, c.col_blocks, pack,
                      a->wave_split == KVS_WAVES_HEADS ? kvs::kWaves : 1, a->head_dim, part_bytes, row_scaled,
                      a->kv_chunk, *cus, pl, min_chunk))
    return KVS_ERR_INVALID_ARG;
  // Automatic wave split: the tiles split, unless the heads split can keep
  // the tiles plan's chunks (at most 64 tiles per wave) and still give every
  // CU a workgroup.  With the same chunks both write the same split
  // partials, and the heads split then reads whole runs of adjacent head rows
  // (32k-token MHA decode: 81.7 against 84.1 us).  With shorter chunks its
  // extra partials cost more than that (batch-64 bf16: 374 against 365 us).
  const int64_t head_wgs = (int64_t)pl->items * (a->num_kv_heads / pack) / kvs::kWaves;
  if (a->wave_split == KVS_WAVES_AUTO && heads && pl->chunk <= kvs::kMaxWaveChunk &&
      head_wgs >= std::max(1, *cus)) {
    if (!kvs::make_plan(a->kv_len_host, nq, a->batch, a->window, a->num_kv_heads, c.cols, c.col_blocks, pack,
                        kvs::kWaves, a->head_dim, part_bytes, row_scaled, pl->chunk, *cus, pl))
      return KVS_ERR_INVALID_ARG;
  }
  // Row-scaled partials only for launches of more workgroups than CUs: a
  // smaller launch is bound by latency, not by its partials' bytes, and the
  // row reduction in its epilogue costs more than the halved bytes save
  // (Gemma-shaped single decode, 128 splits: 14.4 against 14.05 us per step).
  const int64_t wgs = (int64_t)pl->items * (a->num_kv_heads / pack) * c.col_blocks / pl->wave_packs;
  if (row_scaled && wgs <= std::max(1, *cus)) {
    if (!kvs::make_plan(a->kv_len_host, nq, a->batch, a->window, a->num_kv_heads, c.cols, c.col_blocks, pack,
                        pl->wave_packs, a->head_dim, 4, false, pl->chunk, *cus, pl))
      return KVS_ERR_INVALID_ARG;
  }
  // grid.x (items) x grid.y of kThreads work-items must stay below 2^32 work-items
  // (the merge runs one workgroup per column group)
  if ((int64_t)pl->items * a->num_kv_heads * c.col_groups > kvs::kMaxWorkgroups) return KVS_ERR_UNSUPPORTED;
  if (cols_out) *cols_out = std::move(c);
  return KVS_OK;
}

// Device memory of kvs_decode_noalloc: one file-scope array that every GPU
// the library runs on holds, at its own address, until the process ends.  In
// host code `scratch` names a host-side stand-in, never the device memory:
// the address each device gives for it (hipGetSymbolAddress, with that device
// current) is what kernels receive.
static __device__ __align__(256) char scratch[KVS_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};
bool g_scratch_clear[kMaxDevices] = {}; // its counter area has been zeroed on the device

// Zeroes n 32-bit words (the merge counters at the start of `scratch`).
__global__ void zero_words(unsigned *w, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) w[i] = 0u;
}

// Device address of `scratch` on the current device, looked up once per
// device; null on a HIP error.
void *scratch_address(kvs_status *st) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    *st = KVS_ERR_HIP;
    return nullptr;
  }
  if (dev >= kMaxDevices) {
    *st = KVS_ERR_UNSUPPORTED;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      *st = KVS_ERR_HIP;
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

// Before the first call on a device: zero the counter area of `scratch` with a
// kernel on the caller's stream (ahead of that call's own kernels).  A call
// under graph capture records the zeroing into the graph and leaves the
// device unmarked, so the next eager call zeroes again; calls leave the
// counters zero, so later calls need nothing.
kvs_status clear_scratch_counters(void *ptr, hipStream_t stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return KVS_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_clear[dev]) return KVS_OK;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cap) != hipSuccess) return KVS_ERR_HIP;
  const int words = (int)(KVS_WORKSPACE_COUNTER_BYTES / sizeof(unsigned));
  hipLaunchKernelGGL(zero_words, dim3(words / 256), dim3(256), 0, stream, reinterpret_cast<unsigned *>(ptr), words);
  if (hipGetLastError() != hipSuccess) return KVS_ERR_HIP;
  if (cap == hipStreamCaptureStatusNone) g_scratch_clear[dev] = true;
  return KVS_OK;
}

} // namespace

extern "C" {

kvs_status kvs_decode_plan(const kvs_decode_args *args, kvs_plan_info *out) {
  if (!out) return KVS_ERR_INVALID_ARG;
  kvs::Plan pl;
  int algo = 0, cus = 0;
  const kvs_status st = plan_call(args, false, &pl, &algo, &cus);
  if (st != KVS_OK) return st;
  out->kv_chunk = pl.chunk;
  out->items_per_kv_head = pl.items;
  out->max_splits = pl.max_splits;
  out->needs_merge = pl.needs_merge ? 1 : 0;
  out->algo = algo;
  out->num_cus = cus;
  out->workspace_bytes = pl.workspace_bytes;
  const Columns c = columns_of(args);
  out->col_groups = c.col_groups;
  out->col_share = c.col_share;
  out->merge_in_partial = merges_in_partial(pl, args, c) ? 1 : 0;
  out->wave_packs = pl.wave_packs;
  out->part_format = pl.sc_part_bytes ? KVS_PART_F16_ROWS : part_codes_f16(args) ? KVS_PART_F16_CODES : KVS_PART_F32;
  return KVS_OK;
}

size_t kvs_decode_workspace_bytes(const kvs_decode_args *args) {
  kvs::Plan pl;
  int algo = 0, cus = 0;
  if (plan_call(args, false, &pl, &algo, &cus) != KVS_OK) return 0;
  return pl.workspace_bytes;
}

kvs_status kvs_decode(const kvs_decode_args *a, void *workspace, size_t workspace_bytes, hipStream_t stream) {
  kvs::Plan pl;
  int algo = 0, cus = 0;
  Columns cols;
  kvs_status st = plan_call(a, true, &pl, &algo, &cus, &cols);
  if (st != KVS_OK) return st;
  if (pl.workspace_bytes > 0) {
    if (!workspace || workspace_bytes < pl.workspace_bytes) return KVS_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) & 255) return KVS_ERR_WORKSPACE;
  }
  kvs::Params p{};
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.page_indptr = a->page_indptr;
  p.page_indices = a->page_indices;
  p.kv_len = a->kv_len;
  const bool scaled = a->kv_dtype == KVS_FP8_E4M3 || a->kv_dtype == KVS_INT4;
  p.k_scale = scaled ? a->k_scale : nullptr;
  p.v_scale = scaled ? a->v_scale : nullptr;
  p.o = a->o;
  p.lse = a->lse;
  char *ws = reinterpret_cast<char *>(workspace);
  p.counters = nullptr;
  p.o_part = pl.workspace_bytes ? reinterpret_cast<float *>(ws + pl.counter_bytes) : nullptr;
  p.lse_part = pl.workspace_bytes ? reinterpret_cast<float *>(ws + pl.counter_bytes + pl.o_part_bytes) : nullptr;
  p.sc_part = pl.sc_part_bytes ? reinterpret_cast<float *>(ws + pl.counter_bytes + pl.o_part_bytes +
                                                           pl.lse_part_bytes)
                               : nullptr;
  p.meta = pl.workspace_bytes ? reinterpret_cast<int *>(ws + pl.counter_bytes + pl.o_part_bytes +
                                                        pl.lse_part_bytes + pl.sc_part_bytes)
                              : nullptr;
  p.batch = a->batch;
  p.num_qo_heads = a->num_qo_heads;
  p.num_kv_heads = a->num_kv_heads;
  p.group = a->num_qo_heads / a->num_kv_heads;
  p.pack = kv_pack(a, algo);
  p.qo_indptr = a->qo_indptr_host ? a->qo_indptr : nullptr;
  p.col_groups = cols.col_groups;
  p.col_share = cols.col_share;
  p.cols = a->qo_indptr_host ? 16 : p.group * p.pack;
  p.wave_packs = pl.wave_packs;
  // The chunks of a request differ in work only when its query rows reach
  // over more than one chunk (the early rows stop before the late chunks);
  // only then do the multi-row kernels deal their workgroups to the XCDs by
  // work rather than in launch order, which keeps one chunk per XCD.
  p.rows_xcd_order = cols.most > pl.chunk ? 1 : 0;
  p.page_size = a->page_size;
  p.page_shift = a->page_size > 0 ? log2i(a->page_size) : 0;
  p.window = a->window;
  p.chunk = pl.chunk;
  p.items = pl.items;
  p.out_bf16 = a->q_dtype == KVS_BF16 ? 1 : 0;
  p.part_row_scale = pl.sc_part_bytes ? 1 : 0;
  p.part_f16 = part_codes_f16(a) || p.part_row_scale ? 1 : 0;
  // with a soft cap c the kernels form tanh(sm_scale / c * qk) * c * log2(e)
  const bool capped = a->logits_soft_cap > 0.0f;
  p.score_scale = capped ? a->sm_scale / a->logits_soft_cap : a->sm_scale * kvs::kLog2e;
  p.cap_out = capped ? a->logits_soft_cap * kvs::kLog2e : 0.0f;
  p.m_init = a->use_unified_max ? a->unified_max * kvs::kLog2e : -INFINITY;

  // host-planned work lists, passed inline when they fit
  kvs::InlineWork w;
  w.n_items = 0;
  kvs::InlineMerge ml;
  ml.n = -1;
  if (kvs::plan_inline(a->batch, pl.items, pl.max_splits)) {
    int n_merges = 0; // at most one entry per request, so it fits too
    kvs::list_work(a->kv_len_host, cols.nq.empty() ? nullptr : cols.nq.data(), a->batch, a->window, pl.chunk,
                   w.item, ml.req, ml.first, &n_merges);
    for (int b = 0; b < a->batch; ++b) w.req_len[b] = a->kv_len_host[b];
    w.n_items = pl.items;
    ml.n = n_merges;
    p.meta = nullptr; // the merge kernel reads its list from the arguments
  }
  // the partial kernel merges the splits itself when its work list is the
  // host's (every planned split then arrives) and the counters fit
  if (w.n_items > 0 && merges_in_partial(pl, a, cols)) p.counters = reinterpret_cast<unsigned *>(ws);

  // the partial kernel's dispatch stamps the profiling events itself
  const kvs::Launch lp{stream, reinterpret_cast<hipEvent_t>(a->prof_events[0]),
                       reinterpret_cast<hipEvent_t>(a->prof_events[1])};
  hipError_t e;
  if (algo != KVS_ALGO_VALU)
    e = kvs::launch_partial_mfma(p, w, a->head_dim, a->kv_dtype, lp);
  else
    e = kvs::launch_partial_valu(p, w, a->head_dim, a->kv_dtype, lp);
  if (e != hipSuccess) return KVS_ERR_HIP;
  if (pl.needs_merge && !p.counters) {
    e = kvs::launch_merge(p, ml, a->head_dim, pl.max_splits, stream);
    if (e != hipSuccess) return KVS_ERR_HIP;
  }
  return KVS_OK;
}

kvs_status kvs_decode_noalloc(const kvs_decode_args *a, hipStream_t stream) {
  kvs::Plan pl;
  int algo = 0, cus = 0;
  kvs_status st = plan_call(a, true, &pl, &algo, &cus);
  if (st != KVS_OK) return st;
  if (pl.workspace_bytes > KVS_NOALLOC_SCRATCH_BYTES) return KVS_ERR_TOO_LARGE;
  void *ws = nullptr;
  if (pl.workspace_bytes > 0) {
    st = KVS_OK;
    ws = scratch_address(&st);
    if (!ws) return st;
    st = clear_scratch_counters(ws, stream);
    if (st != KVS_OK) return st;
  }
  // the kernels of kvs_decode, with the fixed array as their workspace: its
  // counter area is zero (above), and every call leaves it zero
  return kvs_decode(a, ws, KVS_NOALLOC_SCRATCH_BYTES, stream);
}

kvs_status kvs_append(const kvs_append_args *args, hipStream_t stream) {
  const kvs_status st = validate_append(args);
  if (st != KVS_OK) return st;
  const kvs::Launch l{stream, reinterpret_cast<hipEvent_t>(args->prof_events[0]),
                      reinterpret_cast<hipEvent_t>(args->prof_events[1])};
  return kvs::launch_append(args, l) == hipSuccess ? KVS_OK : KVS_ERR_HIP;
}

const char *kvs_status_string(int s) {
  switch (s) {
  case KVS_OK: return "ok";
  case KVS_ERR_INVALID_ARG: return "invalid argument";
  case KVS_ERR_UNSUPPORTED: return "unsupported shape or type";
  case KVS_ERR_WORKSPACE: return "workspace missing, too small or not 256-byte aligned";
  case KVS_ERR_HIP: return "HIP runtime or launch error";
  case KVS_ERR_TOO_LARGE: return "call needs more scratch than kvs_decode_noalloc's fixed device array "
                                 "(KVS_NOALLOC_SCRATCH_BYTES); use kvs_decode with a workspace";
  default: return "unknown status";
  }
}

int kvs_abi_version(void) { return KVS_ABI_VERSION; }

} // extern "C"
