/*
 * kvsplit: split-KV single-query decode attention for AMD Instinct MI355X
 * (gfx950), behind a plain C ABI.
 *
 * The operation (one decode step of one attention layer).  For request b,
 * query head h and its KV head kh = h / (num_qo_heads / num_kv_heads):
 *
 *   visible keys   J = { t : lo <= t < L },  L = kv_len[b],
 *                  lo = max(0, L - window) if window > 0 else 0
 *   scores         s_t = sm_scale * <q[b,h,:], K[b,t,kh,:]>      (t in J)
 *   lse[b,h]       = ln sum_{t in J} exp(s_t)                     (natural log)
 *   o[b,h,:]       = sum_{t in J} exp(s_t - lse[b,h]) * V[b,t,kh,:]
 *   J empty        o = 0, lse = -inf
 *
 * Sources, by page and section:
 *   - scaled scores, softmax, weighted sum of V: "Forcing Flash Attention onto
 *     TPU" (Hacker News translation on socker-news), section "standard causal
 *     attention", with one query row and no causal mask;
 *   - one new query against the growing K/V cache, paged KV cache, fp8 KV
 *     cache: "Beyond the Memory Wall" (tiptinker.com), section "2. FlashInfer";
 *   - single-request decode with GQA, a scratch buffer and sentinel values for
 *     optional arguments: the FlashInfer-from-JAX tutorial page (upppp.jp),
 *     section on the three kernels (single_decode);
 *   - local (sliding-window) layers: same page, Gemma 3 section;
 *   - splitting the keys into chunks whose partial softmax results are merged
 *     afterwards: the FlashDecoding++ explainer (abeam.tech), sections
 *     "problem" and "asynchronous softmax and unified max value"; the merge
 *     rescales each chunk by exp(chunk max - global max), the same update as
 *     the online softmax of the TPU page's "Flash Attention in JAX" section.
 *
 * Computation: the visible keys of each (request, KV head) are cut into
 * chunks of kv_chunk tokens; one workgroup computes the partial softmax of a
 * chunk (fp32 running max / sum / accumulator) for all query heads of the
 * group; the chunks of each request are merged by log-sum-exp, by the
 * workgroup that finishes the request's last chunk (or, for work lists
 * derived on the device, by a second kernel).  A request whose keys fit in
 * one chunk is written directly by its workgroup.
 *
 * Threading / streams: every call is asynchronous on the given stream and
 * never synchronises.  The library keeps no pointer after returning and
 * allocates no device memory.  Calls that may run concurrently (different
 * streams) need different workspaces.
 */
#ifndef KVSPLIT_H
#define KVSPLIT_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVS_ABI_VERSION 12

/* Status codes.  Every check of KVS_ERR_INVALID_ARG, KVS_ERR_UNSUPPORTED and
 * KVS_ERR_WORKSPACE runs on the host before any HIP call. */
typedef enum {
  KVS_OK = 0,
  KVS_ERR_INVALID_ARG = -1, /* null pointer, bad size, inconsistent shapes */
  KVS_ERR_UNSUPPORTED = -2, /* valid request the library does not implement */
  KVS_ERR_WORKSPACE = -3,   /* workspace null, too small or misaligned */
  KVS_ERR_HIP = -4,         /* a HIP runtime call or launch failed */
  KVS_ERR_TOO_LARGE = -5    /* kvs_decode_noalloc: the call needs more scratch than
                               KVS_NOALLOC_SCRATCH_BYTES */
} kvs_status;

/* Element types.  q and o share q_dtype; K and V share kv_dtype.
 * Supported (q_dtype, kv_dtype) pairs: (F32, F32), (BF16, BF16), (BF16, FP8_E4M3),
 * (BF16, INT4).
 * FP8_E4M3 is the OCP E4M3 ("fn") format: bias 7, max 448, NaN = S.1111.111.
 * INT4: signed 4-bit integers in [-8, 7] (two's complement), two per byte,
 * element 2i in the low nibble of byte i, so a row of head_dim elements is
 * head_dim / 2 bytes ("Beyond the Memory Wall", section "2. FlashInfer",
 * names FP8 and INT4 KV caches; this packing is the reading taken).  INT4
 * needs head_dim 128 or 256 and the matrix-core kernel (kvs_decode only). */
typedef enum { KVS_F32 = 0, KVS_BF16 = 1, KVS_FP8_E4M3 = 2, KVS_INT4 = 3 } kvs_dtype;

/* Kernel family for the per-chunk partial softmax.  AUTO picks MFMA for bf16,
 * fp8 and INT4 KV with page_size 0 or >= 16 (query group packed into the
 * columns of 16x16 matrix tiles) and VALU otherwise (fp32 KV, small pages:
 * one KV row per 4..64 lanes, fp32 FMA); for INT4 head_dim 128 with one query
 * per request it picks MFMA_PACKED where that applies (a 64-byte INT4 head
 * row is half a 128-byte line).  MFMA_PACKED is the matrix-core kernel with
 * two adjacent KV heads per workgroup when 2 * group <= 16, the head count is
 * even and one head's row is shorter than 256 bytes (fp8 head_dim 128,
 * head_dim 64, INT4 head_dim 128); otherwise it is MFMA. */
typedef enum { KVS_ALGO_AUTO = 0, KVS_ALGO_VALU = 1, KVS_ALGO_MFMA = 2, KVS_ALGO_MFMA_PACKED = 3 } kvs_algo;

typedef struct {
  /* shape */
  int32_t batch;        /* >= 1; must be 1 for a contiguous cache */
  int32_t num_qo_heads; /* >= 1 */
  int32_t num_kv_heads; /* >= 1, divides num_qo_heads; group = Hq / Hk <= 16 */
  int32_t head_dim;     /* 64, 128 or 256 */
  int32_t q_dtype;      /* kvs_dtype of q and o */
  int32_t kv_dtype;     /* kvs_dtype of K and V */
  int32_t page_size;    /* 0: contiguous K, V [kv_len, Hk, head_dim];
                           > 0: paged pools [num_pages, page_size, Hk, head_dim]
                           (INT4: the last axis is head_dim / 2 bytes) */
  int32_t num_pages;    /* paged: number of pages in each pool; contiguous: the
                           cache's capacity in tokens (rows of k and v).  Only
                           the host-side lengths are checked against it
                           (kv_len_host[b] <= capacity); page ids are not */

  /* device inputs (caller-owned, row-major, dense) */
  const void *q;               /* [batch, Hq, head_dim], q_dtype */
  const void *k;               /* cache pool, kv_dtype */
  const void *v;               /* cache pool, kv_dtype, same layout as k */
  const int32_t *page_indptr;  /* paged: [batch + 1]; pages of request b are
                                  page_indices[page_indptr[b] .. page_indptr[b+1]) */
  const int32_t *page_indices; /* paged: page ids, logical order within a request */
  const int32_t *kv_len;       /* [batch] tokens in the cache of each request
                                  (the current token included) */
  const int32_t *kv_len_host;  /* host copy of kv_len, used to plan the launch;
                                  must equal kv_len */
  const float *k_scale;        /* FP8 and INT4 only: [batch, Hk] dequantisation scale
                                  of K (stored code * scale = value) */
  const float *v_scale;        /* FP8 and INT4 only: [batch, Hk] scale of V */

  /* scalars */
  float sm_scale;     /* > 0 and finite, multiplies <q, k> */
  int32_t window;     /* -1: no window; W > 0: attend to the last W keys */
  int32_t kv_chunk;   /* 0: heuristic; > 0: tokens per split, rounded up to a
                         multiple of 16 and capped at 4096 (1024 with
                         KVS_WAVES_HEADS: 64 tiles per wave) */
  int32_t algo;       /* kvs_algo */
  int32_t num_cus;    /* 0: ask the current device; > 0: plan for this many CUs */

  /* device outputs (caller-owned) */
  void *o;    /* [batch, Hq, head_dim], q_dtype, round to nearest even; q and o
                 16-byte aligned (KVS_ERR_INVALID_ARG otherwise) */
  float *lse; /* [batch, Hq] natural-log LSE of the scaled scores, or NULL */

  /* optional profiling: two hipEvent_t (created by the caller) that the
   * partial-softmax kernel's own dispatch stamps with its start and end time,
   * so hipEventElapsedTime gives that kernel's duration; NULL to skip */
  void *prof_events[2];

  /* optional unified max (the FlashDecoding++ explainer, section
   * "asynchronous softmax and unified max value"): with use_unified_max = 1
   * every chunk starts its softmax from the reference max unified_max (a
   * bound on the scaled scores sm_scale * q.k, natural units, finite) instead
   * of from the first tile's max.  A score more than 8 / log2(e) above the
   * reference still moves it (with the usual rescale), and a chunk whose
   * first visible scores lie far below it starts from them, so the result
   * does not depend on the value beyond rounding.  Honoured by the
   * matrix-core kernels; the vector kernel ignores it.  0: off. */
  int32_t use_unified_max;
  float unified_max;

  /* optional: several new query tokens per request (append / prefill
   * attention).  NULL (both): one query per request, the decode step above.
   * Otherwise q, o and lse hold total_q = qo_indptr[batch] rows
   * ([total_q, Hq, head_dim] and [total_q, Hq]); request b's rows are
   * qo_indptr[b] .. qo_indptr[b+1] - 1, its n_b = qo_indptr[b+1] -
   * qo_indptr[b] (0 <= n_b <= kv_len[b]) newest cached tokens.  Row i of the
   * request sits at position p = kv_len[b] - n_b + i and sees the keys
   * max(0, p - window + 1) .. p (window > 0), else 0 .. p: the causal mask of
   * "Forcing Flash Attention onto TPU", section "standard causal
   * attention".  Runs on the matrix-core kernel (bf16 / fp8 / INT4 KV, not
   * KVS_ALGO_MFMA_PACKED).  Each workgroup computes 16 (row, head) columns of
   * one KV head, so K/V are read once per ceil(n_b * group / 16) column
   * groups: efficient for short appends (speculative tokens, small chunks),
   * bandwidth-heavy for long prefill. */
  const int32_t *qo_indptr;      /* device [batch + 1] */
  const int32_t *qo_indptr_host; /* host copy (plans the launch); must equal qo_indptr */

  /* optional logit soft-capping, a score transform the FlashInfer-from-JAX
   * page (Gemma 3 section: what QK-norm replaced) and the "Flashlight"
   * explainer (results: the Softcap variant) name without a formula; the
   * reading is Gemma 2's definition on the scaled score:
   * s -> c * tanh(s / c), for c = logits_soft_cap > 0 (finite).  0: none.
   * Scores then stay inside (-c, c); lse is that of the capped scores.  Both
   * kernels; combines with windows, several query rows and the unified max
   * (give unified_max in capped units, at most c). */
  float logits_soft_cap;

  /* where the splits of a request are merged: KVS_MERGE_AUTO chooses; KVS_MERGE_IN_PARTIAL
   * asks for the merge inside the partial kernel (the workgroup that finishes a
   * request's last split merges them; used when the work list is planned on the
   * host and the counters fit, else the merge kernel runs); KVS_MERGE_KERNEL
   * asks for the second kernel. */
  int32_t merge_mode;

  /* How the four waves of a matrix-core decode workgroup share its work
   * (one query row per request only; other calls always split tiles).
   * KVS_WAVES_HEADS: each wave takes one KV-head pack (pack = 1 or 2 adjacent
   * KV heads) over the whole chunk, so a workgroup holds four packs and reads
   * four adjacent head slices of every token row together; needs
   * (num_kv_heads / pack) % 4 == 0, else KVS_ERR_UNSUPPORTED.  KVS_WAVES_TILES:
   * the waves split the chunk's 16-token tiles of one pack.  KVS_WAVES_AUTO:
   * HEADS where it applies and can keep the chunks TILES would use (at most
   * 1024 tokens) with at least one workgroup per CU, else TILES (shorter
   * chunks would mean more split partials, which cost more than HEADS'
   * reads gain). */
  int32_t wave_split;
} kvs_decode_args;

enum { KVS_MERGE_AUTO = 0, KVS_MERGE_IN_PARTIAL = 1, KVS_MERGE_KERNEL = 2 };
enum { KVS_WAVES_AUTO = 0, KVS_WAVES_HEADS = 1, KVS_WAVES_TILES = 2 };

/* What a call will launch, computed on the host from kv_len_host. */
typedef struct {
  int32_t kv_chunk;          /* tokens per split */
  int32_t items_per_kv_head; /* sum over requests of splits; the partial kernel runs
                                items_per_kv_head * num_kv_heads / (pack * wave_packs)
                                workgroups (one query row per request) */
  int32_t max_splits;        /* largest number of splits of one request */
  int32_t needs_merge;       /* 1 if some request has more than one split */
  int32_t algo;              /* resolved kvs_algo (VALU, MFMA or MFMA_PACKED) */
  int32_t num_cus;           /* CU count the plan was made for */
  size_t workspace_bytes;    /* bytes kvs_decode needs for this plan */
  int32_t col_groups;        /* groups of 16 (query row, head) columns per KV head: 1 unless
                                several queries per request */
  int32_t col_share;         /* column groups one partial workgroup computes: 1 (one query per
                                request), 2, or 4 / 8 (several rows per request on the
                                shared-tile kernel, partial_rows_kernel) */
  int32_t merge_in_partial;  /* 1: the partial kernel merges the splits itself (one launch);
                                0: a second kernel merges them (or nothing needs merging) */
  int32_t wave_packs;        /* KV-head packs per partial workgroup: 4 (one per wave,
                                KVS_WAVES_HEADS) or 1 */
  int32_t part_format;       /* kvs_part_format of the split partials in the workspace */
} kvs_plan_info;

/* How the split partial outputs are stored in the workspace (kvs_decode). */
enum {
  KVS_PART_F32 = 0,      /* fp32 */
  KVS_PART_F16_CODES = 1, /* fp16 averages of the stored fp8 / INT4 codes; the merge applies the V scale */
  KVS_PART_F16_ROWS = 2   /* fp16 rows of a bf16 cache, each times a power of two (multiplier stored) */
};

/* Plan a call without launching anything.  Makes no HIP call when
 * args->num_cus > 0.  Validates the arguments like kvs_decode (except that
 * device pointers may be NULL) and fills *out.  KVS_ERR_UNSUPPORTED when the
 * partial kernel would need more than 2^24 - 1 workgroups (one launch holds
 * fewer than 2^32 work-items): raise kv_chunk. */
kvs_status kvs_decode_plan(const kvs_decode_args *args, kvs_plan_info *out);

/* Workspace bytes kvs_decode needs for these arguments (0 on invalid
 * arguments).  Same HIP-call rule as kvs_decode_plan. */
size_t kvs_decode_workspace_bytes(const kvs_decode_args *args);

/* Bytes at the start of every workspace that hold merge counters. */
#define KVS_WORKSPACE_COUNTER_BYTES ((size_t)65536)

/* Run one decode-attention step asynchronously on `stream`.
 * workspace: device memory, 256-byte aligned, at least
 * kvs_decode_workspace_bytes(args) bytes (0 when no request needs more than
 * one split).  Its first KVS_WORKSPACE_COUNTER_BYTES hold arrival counters:
 * they must be zero before the first call that uses the workspace (allocate
 * it zeroed), and every call leaves them zero.  With the work list planned
 * on the host (batch <= 256, at most 1344 splits per KV head and 256 per
 * request) the workgroup that writes a request's last split merges all of
 * its splits when that pays (merge_mode; one launch, no workgroup waits for
 * another); otherwise a second kernel merges.  The rest of the workspace
 * holds the per-split partial outputs and their log-sum-exp values (fp32),
 * rewritten by every call.  The partial outputs are fp32 for fp32 caches;
 * for fp8 and INT4 caches they are fp16 weighted averages of the stored
 * codes, which lie inside the codes' range (the merge applies the V scale),
 * so fp16 keeps 11 significant bits at half the bytes.  For bf16 caches in
 * launches of more workgroups than CUs, on the decode and 32-column kernels
 * (col_share 1 or 2) and the prefill kernel (head_dim 128 or 256), each partial row
 * is stored in fp16 times a power of two that puts its largest magnitude in
 * [2^14, 2^15), with the inverse multiplier (fp32) beside its log-sum-exp;
 * other bf16 launches write fp32 partials.  kvs_plan_info.part_format names
 * the format of a call.
 * Preconditions that are not checked (they would need a device sync):
 * kv_len equals kv_len_host, page_indptr[b+1] - page_indptr[b] >=
 * ceil(kv_len[b] / page_size), every page id is < num_pages, and all
 * visible K/V values are finite. */
kvs_status kvs_decode(const kvs_decode_args *args, void *workspace, size_t workspace_bytes,
                      hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): kvs_decode
 * with no workspace argument.  The split partials live in one device array
 * of KVS_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends; its address on the current device is looked up
 * once, on the first call there.  The caller still passes every input and
 * output.  The call allocates nothing and runs the kernels of kvs_decode.
 * Returns KVS_ERR_TOO_LARGE (before any HIP call) when
 * kvs_decode_workspace_bytes(args) exceeds KVS_NOALLOC_SCRATCH_BYTES: use
 * kvs_decode with a workspace then.  All calls on one GPU share the array,
 * so calls that may overlap on one GPU (different streams, or host threads
 * racing on one stream) race on it and give wrong results; serialise them. */
#define KVS_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
kvs_status kvs_decode_noalloc(const kvs_decode_args *args, hipStream_t stream);

/* ------------------------------------------------------------------------
 * The step before attention: QK-norm, rotary embedding and KV append for the
 * new tokens of every request (one decode step of one layer, or a packed
 * ragged batch of several new tokens per request).
 *
 * For token row r of request b at position p (one new token per request:
 * r = b and p = kv_len[b], the tokens already cached; with qo_indptr: rows
 * r = qo_indptr[b] + i, i < qo_indptr[b+1] - qo_indptr[b], at p = kv_len[b] + i):
 *   q_out[r,h,:]    = rope(norm(q_in[r,h,:], q_norm_weight), p)     h < Hq
 *   K[b, p, kh, :]  = store(rope(norm(k_in[r,kh,:], k_norm_weight), p))
 *   V[b, p, kh, :]  = store(v_in[r,kh,:])                          kh < Hk
 * norm(x, w) = x / sqrt(mean(x^2) + norm_eps) * w over the head dimension,
 *   skipped when the weight is NULL (QK-norm: the FlashInfer-from-JAX
 *   tutorial page, Gemma 3 section);
 * rope(x, p): dimension pair j (j < head_dim/2) turns by the angle
 *   p * rope_theta^(-2j/head_dim), (x_a, x_b) -> (x_a cos - x_b sin,
 *   x_a sin + x_b cos), with pairs (j, j + head_dim/2), or (2j, 2j + 1) when
 *   rope_interleave = 1; skipped when rope_theta == 0 (apply_rope and the
 *   per-layer theta -- 10,000 local, 1,000,000 global: same page, the
 *   three-kernels and Gemma 3 sections);
 * store: to kv_dtype, nearest even; FP8_E4M3 stores the nearest code of
 *   x / k_scale[b,kh] (v_scale for V), saturating at +-448; INT4 the nearest
 *   integer to x / scale, ties to even, saturated to [-8, 7] (NaN: 0), two
 *   per byte, element 2i in the low nibble ("Beyond the Memory Wall",
 *   section "2. FlashInfer": appending to the growing, paged, fp8 or INT4
 *   cache; the request's existing scale is kept, as the pages give no
 *   running-scale rule).
 * Several new tokens per request follow the packed batch that apply_rope
 * rotates (FlashInfer-from-JAX page, three-kernels section); row i of a
 * request takes the i-th free position after its cached tokens.
 * Angles are formed in double precision; the rest runs in fp32.
 *
 * Layouts as for kvs_decode: q_in, q_out [rows, Hq, d]; k_in, v_in
 * [rows, Hk, d] (rows = batch, or qo_indptr[batch]); the cache
 * [num_pages, page_size, Hk, d] (INT4: d / 2 bytes) or, with page_size 0
 * (batch 1), [num_pages, Hk, d] where num_pages is then the capacity in
 * tokens.  q_out may be q_in (in place).
 * kv_len is read, not changed: the caller raises kv_len and kv_len_host by
 * each request's new rows before the decode call that should see them.
 * Errors: argument checks run on the host before any HIP call, as for
 * kvs_decode.  Not checked (device data): a token whose position p is not
 * covered by its request's page list, or whose page id there is >=
 * num_pages (contiguous: p >= capacity), gets q_out but no cache write.
 * ------------------------------------------------------------------------ */
typedef struct {
  int32_t batch;
  int32_t num_qo_heads;
  int32_t num_kv_heads;
  int32_t head_dim;   /* 64, 128 or 256 */
  int32_t q_dtype;    /* q_in, k_in, v_in, q_out: KVS_F32 or KVS_BF16 */
  int32_t kv_dtype;   /* cache; pairs as for kvs_decode (INT4: head_dim 128 or 256) */
  int32_t page_size;  /* 0: contiguous; else a power of two */
  int32_t num_pages;  /* paged: pages in each pool; contiguous: capacity (tokens) */

  const void *q_in;
  const void *k_in;
  const void *v_in;
  void *q_out;
  void *k_cache;
  void *v_cache;
  const int32_t *page_indptr;  /* paged only, as for kvs_decode */
  const int32_t *page_indices; /* paged only */
  const int32_t *kv_len;       /* device [batch]: position of the new token */
  const float *k_scale;        /* FP8 and INT4 caches only, [batch, Hk] */
  const float *v_scale;
  const float *q_norm_weight;  /* device [head_dim] fp32, or NULL: no q norm */
  const float *k_norm_weight;  /* device [head_dim] fp32, or NULL: no k norm */
  float norm_eps;              /* >= 0 */
  float rope_theta;            /* 0: no rotary embedding; else > 0 */
  int32_t rope_interleave;     /* 0 or 1 */

  /* optional profiling: two hipEvent_t stamped by the kernel's own dispatch
   * with its start and end; NULL to skip */
  void *prof_events[2];

  /* optional: several new tokens per request.  NULL (both): one per request.
   * Otherwise request b's token rows are qo_indptr[b] .. qo_indptr[b+1] - 1
   * (0 rows allowed) and q_in, k_in, v_in, q_out hold qo_indptr[batch] rows. */
  const int32_t *qo_indptr;      /* device [batch + 1] */
  const int32_t *qo_indptr_host; /* host copy (sizes the launch); must equal qo_indptr */
} kvs_append_args;

/* Run the step asynchronously on `stream`.  Allocates nothing. */
kvs_status kvs_append(const kvs_append_args *args, hipStream_t stream);

/* Static description of a status code. */
const char *kvs_status_string(int status);

/* KVS_ABI_VERSION of the built library. */
int kvs_abi_version(void);

/* Measurement helpers (not part of the attention computation).
 * kvs_probe_stream_read streams `bytes` (multiple of 16, 16-byte aligned
 * buffer) from device memory with 16-byte loads: the achievable read
 * bandwidth of the GPU.  `sink`: device buffer of >= 1024 uint32, or NULL.
 * kvs_probe_copy copies `bytes` between two non-overlapping 16-byte aligned
 * device buffers; its known traffic calibrates hardware byte counters.
 * Both are asynchronous on `stream` and return 0 or a hipError_t code. */
int kvs_probe_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream);
int kvs_probe_copy(void *dst, const void *src, size_t bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KVSPLIT_H */
