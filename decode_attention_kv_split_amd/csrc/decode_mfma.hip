// Split-KV partial softmax for bf16 / fp8-e4m3 / INT4 KV on gfx950 matrix cores.
//
// One workgroup (4 waves) owns one chunk of one (request, KV-head pack); wave
// w takes the chunk's 16-token tiles w, w+4, w+8, ...  A pack is PACK
// adjacent KV heads (1 or 2) whose PACK * g query heads fill at most the 16
// columns of a matrix tile; every query head of the pack shares each K/V byte
// the wave loads, and the pack's row segments are contiguous in memory
// (token-major layout), so a wave reads PACK * head_dim * bytes contiguous
// bytes per token.
//
// Per 16-token tile, with lane = 16 * q4 + c16 and DE = PACK * head_dim:
//   * staging: K and V rows of the tile go from HBM into the wave's LDS slot
//     with 16-byte DMA loads in cache-line order (non-temporal); lane
//     (c16, q4) then reads the 16-byte pieces 4*pc + q4 of row c16, which is
//     the operand layout of a matrix whose rows are tokens and whose
//     reduction index runs over the pack's head dimensions.
//   * scores S^T[token][query head] = K . Q^T with v_mfma_f32_16x16x32_bf16
//     (fp8 K converted to bf16 first, exactly; INT4 K as 136 + n, the offset
//     removed afterwards); Q^T is block diagonal, query head c16 only sees
//     the dims of its own KV head.  Lane ends up with tokens 4*q4 + r
//     (r = 0..3) of query head c16.
//   * online softmax per query head in the log2 domain: tile max over the 16
//     tokens (in-lane over r, then across the four quarters with lane
//     swaps); the reference max moves, with a rescale of the running state,
//     only when the tile max exceeds it by more than 8; weights
//     p = exp2(s - reference), running sum.
//   * V^T with tokens 4*q4 + r of one head dimension in lane c16 -- the
//     operand layout the next product needs: bf16 (pack width <= 128) reads
//     it straight from LDS with 16-bit transposing reads; fp8 and INT4 with
//     8-bit ones (4 keys of 2 fp8 dims or 4 INT4 dims per lane), converted
//     exactly to bf16 (fp8) or to 136 + n by byte permutes (INT4); wider bf16
//     tiles are multiplied by an identity (16x16x16).
//   * O^T[dim][query head] += V^T . P^T with v_mfma_f32_16x16x16_bf16; lane
//     keeps four dims per 16-dim slice w (see out_dim) of query
//     head c16, so the running max, sum and rescale of a head never leave its
//     lane; dims of the other KV head of the pack are dropped at the end.
// The first product, the online update and the rescaled accumulation follow
// the tiled online softmax of "Forcing Flash Attention onto TPU", section
// "Flash Attention in JAX"; chunk results are merged by log-sum-exp (FlashDecoding++
// explainer, asynchronous-softmax section: partial softmax per tile, then an
// update with the previous max and sum).
//
// Several query rows per request turn the columns into (query row, head)
// pairs.  Up to two groups of 16 such columns run in this kernel (both on
// each staged tile); from three groups on, the kernels of rows_mfma.hip let
// their four waves share each staged tile instead of splitting the keys.
// The building blocks live in mfma_tiles.h.
#include "mfma_tiles.h"


namespace kvs {
namespace {
using namespace tiles;

// CG: column groups (16 columns each) a wave computes on every staged tile;
// more than one only with several query rows per request and one KV head per
// workgroup.  The groups share the K operand and the V^T products, so K/V
// are read once for all of them.
// HEADS: each wave takes its own KV-head pack (packs 4 y .. 4 y + 3 for
// blockIdx.y = y) over all tiles of the chunk, instead of a quarter of one
// pack's tiles.  The four waves then stream four adjacent head slices of the
// same token rows at the same time, so each 16-token page of the pool is read
// as longer contiguous runs; on MI355X that streamed 6-13% faster (batch-64
// bf16, batch-128 fp8 and INT4, 32k MHA), and each wave's state is already
// its pack's whole chunk, so no cross-wave merge is needed.
template <int D, int PACK, int KT, int NBUF, int CG, bool HEADS>
__global__ __launch_bounds__(kThreads) void partial_mfma_kernel(const Params p, const InlineWork w) {
  static_assert(CG == 1 || PACK == 1, "column groups of (query row, head) pairs take one KV head");
  static_assert(!HEADS || CG == 1, "one pack per wave: one column group");
  constexpr int DE = D * PACK;
  using S = Shape<DE, KT>;
  constexpr int OSTRIDE = D + 4;
  // bf16 caches: split partials stored as row-scaled fp16 when the host asks
  constexpr bool ROWSC = KT == DT_BF16;
  constexpr int kStageBytes = kWaves * NBUF * 2 * S::kTileBytes;
  constexpr int kEpiBytes = 2 * kWaves * 16 * 4 + kWaves * 16 * OSTRIDE * 4;
  constexpr int kSmem = kStageBytes > kEpiBytes ? kStageBytes : kEpiBytes;

  __shared__ int s_scan[2 * 64];
  __shared__ int s_item[4];
  // K/V staging during the main loop; per-wave softmax states afterwards
  __shared__ __attribute__((aligned(16))) char smem[kSmem];
  float(*sm_m)[16] = reinterpret_cast<float(*)[16]>(smem);
  float(*sm_l)[16] = reinterpret_cast<float(*)[16]>(smem + kWaves * 16 * 4);
  float *sm_o = reinterpret_cast<float *>(smem + 2 * kWaves * 16 * 4);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15;
  const int q4 = lane >> 4;
  // Item-major grid: concurrent workgroups read one KV head of many requests'
  // pages spread over the pool, which streamed faster on MI355X than grids
  // that run all heads of an item together (on one XCD or spread over XCDs).
  const int item = blockIdx.x;
  const int col_blocks = (p.col_groups + CG - 1) / CG; // workgroups per (item, KV head pack)
  // KV heads kvg*PACK .. kvg*PACK+PACK-1
  const int kvg = HEADS ? blockIdx.y * kWaves + wave : blockIdx.y / col_blocks;
  const int cg0 = blockIdx.y % col_blocks * CG;        // first column group (several queries per request)
  const int g = p.group;
  const int gp = g * PACK;    // query heads of the pack (<= 16)
  const int Hk = p.num_kv_heads;
  // KV head (within the pack) of this lane's column; (query, head) columns
  // are only run with one KV head per workgroup
  const int my_kv = p.qo_indptr ? 0 : c16 / g;

  // ---- which (request, split) is this workgroup? ----
  int b, split, nb, L;
  if (!locate_item(p, w, item, blockIdx.y == 0, s_scan, s_item, b, split, nb, L)) return;

  // ---- columns: query heads of the pack, or (query row, head) pairs ----
  const int nq = req_nq(p, b);
  if (p.qo_indptr && cg0 * 16 >= nq * g) return; // no column of this workgroup has a query row
  const int lo = request_lo(L, nq, p.window);
  const int a0 = (lo & ~(kTile - 1)) + split * p.chunk; // aligned chunk start
  const int t_begin = max(lo, a0);
  const int t_end = min(L, a0 + p.chunk);
  ColumnSet<DE, KT, CG> cs;
  set_columns(cs, p, b, L, nq, kvg, cg0, gp, t_begin, t_end, c16);
  // keys every column sees (no per-key mask) and keys some column sees
  int all_lo, all_hi, w_lo, w_hi;
  column_ranges(cs, t_begin, t_end, all_lo, all_hi, w_lo, w_hi);
  // Only the tiles holding keys some column sees are streamed: with several
  // rows per request (a causal prefill) the early rows stop long before the
  // chunk does.  With one query per request this is the whole chunk.
  const int ft = w_hi > w_lo ? (w_lo - a0) / kTile : 0; // first tile, counted from the chunk start
  const int ntiles = w_hi > w_lo ? (w_hi - a0 + kTile - 1) / kTile - ft : 0;
  // this wave's tiles: all of them (HEADS; chunks of at most 64 tiles) or
  // every fourth, from the wave's index
  const int my_tiles = HEADS ? min(ntiles, 64) : (ntiles > wave ? (ntiles - wave + kWaves - 1) / kWaves : 0);
  const int t_first = HEADS ? ft : ft + wave;    // tile i of the wave: t_first + i * t_step
  const int t_step = HEADS ? 1 : kWaves;
  load_columns<D>(cs, p, q4, my_kv);

  float cscale = p.score_scale;
  if (KT != DT_BF16) cscale *= p.k_scale[b * Hk + kvg * PACK + min(my_kv, PACK - 1)];
  const float cap_out = p.cap_out;
  const s16x4_t ident = transpose_identity(c16, q4);

  // ---- addressing ----
  const size_t row_bytes = (size_t)Hk * (S::kRowBytes / PACK); // bytes between consecutive tokens
  const bool paged = p.page_size > 0;
  const int *pages = paged ? p.page_indices + p.page_indptr[b] : nullptr;
  const int pshift = p.page_shift;
  const int pmask = p.page_size - 1;

  // Where each of this wave's tiles starts (byte offset of its first row in
  // the K or V pool) and how many of its bytes hold keys of this chunk, one
  // tile per lane (lane i: tile i; a wave owns at most 64 tiles because
  // chunks are capped at 64 * kWaves * kTile tokens).  The main loop takes
  // them with v_readlane and never waits on memory for an address.
  uint32_t voff_lo = 0, voff_hi = 0, vbytes = 0;
  if (lane < my_tiles) {
    const int ts = a0 + (t_first + lane * t_step) * kTile;
    const size_t row0 = paged ? (size_t)pages[ts >> pshift] * p.page_size + (ts & pmask) : (size_t)ts;
    const size_t off = row0 * row_bytes;
    voff_lo = (uint32_t)off;
    voff_hi = (uint32_t)(off >> 32);
    vbytes = (uint32_t)(min(kTile, w_hi - ts) * (int)row_bytes);
  }
  // K/V tiles go from HBM straight into this wave's LDS slots with 16-byte
  // DMA loads in cache-line order (each load covers whole row segments of the
  // pack), non-temporal, then the operand registers are read from LDS.  The
  // loads use a per-tile buffer descriptor built in scalar registers: base =
  // the tile's first row, size = the rows that hold keys of this chunk.  Rows
  // past the chunk end and whole tiles past the wave's last tile (prefetch
  // overrun) fall outside the descriptor and land in LDS as zeros without
  // touching memory, so the prefetch ring needs no branches.
  const char *kpool = reinterpret_cast<const char *>(p.k);
  const char *vpool = reinterpret_cast<const char *>(p.v);
  int dma_voff[S::kDma]; // lane's byte offset within a tile, per DMA load
#pragma unroll
  for (int k = 0; k < S::kDma; ++k) {
    const int r = k * S::kRowsPerDma + lane / S::kPieces;
    const int piece = (lane % S::kPieces) ^ stage_swizzle<DE, KT>(r);
    dma_voff[k] = r * (int)row_bytes + kvg * S::kRowBytes + piece * 16; // < 2^31: checked on the host
  }
  char *wave_stage = smem + wave * NBUF * 2 * S::kTileBytes;
  auto issue = [&](int i, int slot) {
    const int li = min(i, 63);
    const size_t base = ((size_t)__builtin_amdgcn_readlane(voff_hi, li) << 32) | __builtin_amdgcn_readlane(voff_lo, li);
    const int nbytes = i < my_tiles ? (int)__builtin_amdgcn_readlane(vbytes, li) : 0;
    const __amdgpu_buffer_rsrc_t kr =
        __builtin_amdgcn_make_buffer_rsrc((void *)(kpool + base), (short)0, nbytes, kBufferFlags);
    const __amdgpu_buffer_rsrc_t vr =
        __builtin_amdgcn_make_buffer_rsrc((void *)(vpool + base), (short)0, nbytes, kBufferFlags);
    char *kst = wave_stage + slot * 2 * S::kTileBytes;
    char *vst = kst + S::kTileBytes;
#pragma unroll
    for (int k = 0; k < S::kDma; ++k) dma16_to_lds(kr, kst + 1024 * k, dma_voff[k]);
#pragma unroll
    for (int k = 0; k < S::kDma; ++k) dma16_to_lds(vr, vst + 1024 * k, dma_voff[k]);
  };
  // operand registers of a staged tile: lane (c16, q4) takes pieces 4*pc + q4
  // of row c16 (the same pieces the operand layout below expects)
  StageReader<DE, KT> stage; // lane addresses of the tile in slot 0
  stage.init(lds_address(wave_stage), lane);
  auto read_stage = [&](TileRegs<DE, KT> &t, int slot) { stage.read(t, slot * 2 * S::kTileBytes); };

  auto compute = [&](TileRegs<DE, KT> t, int i) {
    const int ts = a0 + (t_first + i * t_step) * kTile;
    zero_v_before(t, ts, w_lo, c16, q4); // rows before the first key any column sees
    tile_update(cs, t, ts, all_lo, all_hi, cscale, cap_out, ident, q4);
  };

  // Ring of NBUF staging slots per wave.  A slot is refilled as soon as its
  // tile has been read into registers, so NBUF tiles are in flight while one
  // is computed.  Loads are issued for every ring position (past the wave's
  // last tile they move no bytes), which keeps the vmcnt arithmetic exact.
  if (my_tiles > 0) {
#pragma unroll
    for (int j = 0; j < NBUF; ++j) issue(j, j);
    const int n_iter = (my_tiles + NBUF - 1) / NBUF * NBUF;
    for (int it = 0; it < n_iter; it += NBUF) {
#pragma unroll
      for (int j = 0; j < NBUF; ++j) {
        const int i = it + j;
        wait_vmem<(NBUF - 1) * 2 * S::kDma>(); // tile i has landed; NBUF - 1 newer tiles may fly
        TileRegs<DE, KT> t;
        read_stage(t, j); // returns with the reads complete
        issue(i + NBUF, j);
        if (i < my_tiles) compute(t, i);
      }
    }
    wait_vmem<0>(); // no DMA may land in the staging area once it is reused
  }
  if constexpr (HEADS) {
    // ---- one pack per wave: the wave's state is its pack's whole chunk.
    // Each lane normalises its own dims into the wave's staging slots (free
    // once its last DMA has landed; no other wave touches them), and the
    // wave then stores whole output rows from there: written straight from
    // the registers, every store instruction covered 16 rows in 64-byte
    // pieces, and that cost batch-64 bf16 about 12% of its time ----
    // dims in NP passes of DP when 16 padded rows of D floats exceed the slots
    constexpr int kStage = NBUF * 2 * S::kTileBytes;
    constexpr int NP = 16 * (D + 4) * 4 <= kStage ? 1 : 2;
    constexpr int DP = D / NP;
    constexpr int WS = DP + 4; // LDS row stride (floats) of a column
    static_assert(16 * WS * 4 <= kStage, "a wave's output fits its staging slots");
    float *wo = reinterpret_cast<float *>(wave_stage);
    float l_tot = cs.l[0] + __shfl_xor(cs.l[0], 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    float voff = 0.0f; // INT4: V entered the product as 136 + n (136 * the weights' sum)
    if constexpr (KT == DT_INT4) {
      float lb_tot = cs.lb[0] + __shfl_xor(cs.lb[0], 16, 64);
      lb_tot += __shfl_xor(lb_tot, 32, 64);
      voff = kInt4Offset * lb_tot;
    }
    const size_t slot = (size_t)kvg * p.items + item; // one column group
    const bool live = l_tot > 0.0f;                   // else no visible key: o = 0, lse = -inf
    const bool row_scaled = ROWSC && p.part_row_scale && nb > 1;
    // row-scaled partials: the largest |acc| of the lane's column over the
    // pack's dims it holds, then over the column's four lane quarters
    float amax = 0.0f;
    if (row_scaled) {
#pragma unroll
      for (int w = 0; w < S::kOTiles; ++w)
        if (out_dim<DE, KT>(w, q4) / D == my_kv)
#pragma unroll
          for (int r = 0; r < 4; ++r) amax = fmaxf(amax, fabsf(cs.acc[0][w][r]));
      amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
      amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
    }
    float inv = 0.0f;
    if (cs.ok[0]) {
      const int hq = cs.head[0];
      const float vscale = p.v_scale && writer_scales_v(p, nb) ? p.v_scale[b * Hk + hq / g] : 1.0f;
      inv = live ? vscale / l_tot : 0.0f;
      int k = 0;
      if (row_scaled) { // the column's partial row is stored times 2^k
        k = row_scale_exp(amax * inv);
        inv = ldexpf(inv, k);
      }
      if (q4 == 0) {
        const float lse2 = live ? cs.m[0] + __log2f(l_tot) : -INFINITY;
        if (nb == 1) {
          if (p.lse) p.lse[(size_t)cs.row[0] * p.num_qo_heads + hq] = lse2 * kLn2;
        } else {
          store_partial(p, p.lse_part + slot * p.cols + c16, lse2);
          if (row_scaled) store_partial(p, p.sc_part + slot * p.cols + c16, ldexpf(1.0f, -k));
        }
      }
    }
    const int gp_live = min(gp, 16);
#pragma unroll
    for (int ps = 0; ps < NP; ++ps) {
      if (ps > 0) { // the previous pass's reads are issued before these writes
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
      if (cs.ok[0]) {
#pragma unroll
        for (int w = 0; w < S::kOTiles; ++w) {
          const int od = out_dim<DE, KT>(w, q4);
          const int d = od % D - ps * DP; // a slice's dims lie in one pass
          if (od / D != my_kv || d < 0 || d >= DP) continue; // the pack's other KV head, or another pass
          float *dst = wo + c16 * WS + d;
          if constexpr (S::kOutStride == 1) {
            *reinterpret_cast<float4 *>(dst) =
                make_float4((cs.acc[0][w][0] - voff) * inv, (cs.acc[0][w][1] - voff) * inv,
                            (cs.acc[0][w][2] - voff) * inv, (cs.acc[0][w][3] - voff) * inv);
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[r * S::kOutStride] = (cs.acc[0][w][r] - voff) * inv;
          }
        }
      }
      // the reads below follow this wave's LDS writes (one wave's LDS
      // accesses complete in order; the fences keep the compiler from
      // moving them)
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      for (int f = lane; f < gp_live * (DP / 4); f += 64) { // float4 f: column f / (DP / 4)
        const int h = f / (DP / 4);
        const int dl = 4 * (f - h * (DP / 4));
        const int d = ps * DP + dl;
        const float4 v = *reinterpret_cast<const float4 *>(wo + h * WS + dl);
        if (nb == 1) {
          const size_t off = ((size_t)b * p.num_qo_heads + kvg * gp + h) * D + d; // bf16 q and o (matrix-core path)
          *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(p.o) + off) =
              make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
        } else if (row_scaled) {
          store_part4<true>(p, (slot * p.cols + h) * D + d, v.x, v.y, v.z, v.w);
        } else {
          store_part4(p, (slot * p.cols + h) * D + d, v.x, v.y, v.z, v.w);
        }
      }
    }
    finish_split<D, PACK, kFusedMergeBatch, ROWSC>(p, blockIdx.y, b, blockIdx.y * kWaves, 0, 1, item, split, nb,
                                                   smem, kWaves);
    return;
  }
  __syncthreads(); // staging area is reused for the per-wave states below

  // ---- per-wave states to LDS (each query head keeps the dims of its KV head),
  // merged over the waves and stored one column group at a time ----
#pragma unroll
  for (int c = 0; c < CG; ++c) {
    if (c > 0) {
      if (!cs.on[c]) break; // the same in every lane of the workgroup
      __syncthreads();       // the previous group's merge has read the states
    }
    float l_tot = cs.l[c] + __shfl_xor(cs.l[c], 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    float lb_tot = 0.0f;
    if constexpr (KT == DT_INT4) {
      lb_tot = cs.lb[c] + __shfl_xor(cs.lb[c], 16, 64);
      lb_tot += __shfl_xor(lb_tot, 32, 64);
    }
    if (cs.ok[c]) {
      if (q4 == 0) {
        sm_m[wave][c16] = l_tot > 0.0f ? cs.m[c] : -INFINITY; // an empty state keeps no reference
        sm_l[wave][c16] = l_tot;
      }
      float *dst = sm_o + (wave * 16 + c16) * OSTRIDE;
      // INT4: V entered the product as 136 + n; remove 136 * (sum of the weights it saw)
      const float voff = kInt4Offset * lb_tot;
#pragma unroll
      for (int w = 0; w < S::kOTiles; ++w) {
        const int od = out_dim<DE, KT>(w, q4);
        if (od / D == my_kv) {
          if constexpr (S::kOutStride == 1) {
            *reinterpret_cast<float4 *>(dst + od % D) =
                make_float4(cs.acc[c][w][0], cs.acc[c][w][1], cs.acc[c][w][2], cs.acc[c][w][3]);
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[od % D + r * S::kOutStride] = cs.acc[c][w][r] - voff;
          }
        }
      }
    }
    __syncthreads();
    merge_waves_and_store<D, OSTRIDE, ROWSC>(p, sm_m, sm_l, sm_o, b, kvg, cg0 + c, item, nb);
  }
  finish_split<D, PACK, kFusedMergeBatch, ROWSC>(p, blockIdx.y, b, kvg, cg0, CG, item, split, nb, smem);
}

} // namespace

template <int D, int PACK, int KT>
static hipError_t launch_mfma_d(const Params &p, const InlineWork &w, const Launch &l) {
  constexpr int NB = Shape<D * PACK, KT>::kNBuf;
  if constexpr (PACK == 1 && D == 128) {
    if (p.col_share == 2) return launch_cols32(p, w, KT, l); // 32x32 tiles, keys split over the waves
  }
  if constexpr (PACK == 1 && D <= 128) {
    if (p.col_share == 2)
      return launch_kernel(l, partial_mfma_kernel<D, 1, KT, NB, 2, false>,
                           dim3(p.items, p.num_kv_heads * ((p.col_groups + 1) / 2)), p, w);
  }
  if (p.col_share != 1) return hipErrorInvalidValue;
  if (p.wave_packs == kWaves) { // one pack per wave (one query row per request)
    if (p.qo_indptr || p.col_groups != 1 || p.num_kv_heads / PACK % kWaves != 0 || p.chunk > 64 * kTile)
      return hipErrorInvalidValue;
    return launch_kernel(l, partial_mfma_kernel<D, PACK, KT, NB, 1, true>,
                         dim3(p.items, p.num_kv_heads / PACK / kWaves), p, w);
  }
  if (p.wave_packs != 1) return hipErrorInvalidValue;
  return launch_kernel(l, partial_mfma_kernel<D, PACK, KT, NB, 1, false>,
                       dim3(p.items, p.num_kv_heads / PACK * p.col_groups), p, w);
}

// KV heads per workgroup.  Two heads per pack would make every staged row at
// least 256 contiguous bytes for fp8 head_dim 128 (128-byte segments stream
// about 12% slower), but a packed tile then fills the LDS budget of two
// staging slots per wave, and on MI355X that lost more than the longer rows
// gained (batch-128 fp8 decode: 311 us unpacked, 407-424 us packed).  So the
// default is one head per workgroup; KVS_ALGO_MFMA_PACKED asks for packs.
// INT4 head_dim 128 is different: one head's row is 64 bytes, half a
// 128-byte line, so unpacked each line reaches the chip once per head (the
// batch-128 INT4 step fetched 2.01x its bytes), and a packed INT4 tile still
// fits three staging slots per wave.
bool mfma_packable(int head_dim, int group, int num_kv_heads, int kv_type) {
  const bool seg_ok = kv_type == DT_INT4 ? head_dim == 128 : head_dim * (kv_type == DT_FP8 ? 1 : 2) < 256;
  return seg_ok && 2 * group <= 16 && num_kv_heads % 2 == 0;
}
int mfma_pack(int head_dim, int group, int num_kv_heads, int kv_type, bool allow_pack) {
  return allow_pack && mfma_packable(head_dim, group, num_kv_heads, kv_type) ? 2 : 1;
}

// Which head sizes the matrix-core kernel takes for a KV type (INT4 rows must
// give each of the four lane quarters a 16-byte piece: head_dim >= 128).
bool mfma_head_dim_ok(int head_dim, int kv_type) {
  if (kv_type == DT_INT4) return head_dim == 128 || head_dim == 256;
  return head_dim == 64 || head_dim == 128 || head_dim == 256;
}

hipError_t launch_partial_mfma(const Params &p, const InlineWork &w, int head_dim, int kv_type, const Launch &l) {
  if (p.col_share >= 4) return launch_partial_rows(p, w, head_dim, kv_type, l);
  const bool pack2 = p.pack == 2;
  if (kv_type == DT_INT4) {
    if (head_dim == 128) return pack2 ? launch_mfma_d<128, 2, DT_INT4>(p, w, l) : launch_mfma_d<128, 1, DT_INT4>(p, w, l);
    if (pack2) return hipErrorInvalidValue;
    if (head_dim == 256) return launch_mfma_d<256, 1, DT_INT4>(p, w, l);
    return hipErrorInvalidValue;
  }
  const bool fp8 = kv_type == DT_FP8;
  switch (head_dim) {
  case 64:
    if (fp8) return pack2 ? launch_mfma_d<64, 2, DT_FP8>(p, w, l) : launch_mfma_d<64, 1, DT_FP8>(p, w, l);
    return pack2 ? launch_mfma_d<64, 2, DT_BF16>(p, w, l) : launch_mfma_d<64, 1, DT_BF16>(p, w, l);
  case 128:
    if (fp8) return pack2 ? launch_mfma_d<128, 2, DT_FP8>(p, w, l) : launch_mfma_d<128, 1, DT_FP8>(p, w, l);
    return pack2 ? launch_mfma_d<128, 2, DT_BF16>(p, w, l) : launch_mfma_d<128, 1, DT_BF16>(p, w, l);
  case 256:
    if (pack2) return hipErrorInvalidValue;
    return fp8 ? launch_mfma_d<256, 1, DT_FP8>(p, w, l) : launch_mfma_d<256, 1, DT_BF16>(p, w, l);
  default: return hipErrorInvalidValue;
  }
}

} // namespace kvs
