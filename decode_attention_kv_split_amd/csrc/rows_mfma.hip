// Partial softmax for several query rows per request (append / prefill
// attention) on gfx950 matrix cores, for plans whose workgroups cover four or
// eight groups of 16 (query row, head) columns of one KV head.  The four
// waves of a workgroup own different columns and share every staged K/V
// block, so the keys are read once for all of them: partial_rows_kernel with
// the 16x16 operand layouts of mfma_tiles.h, and partial_prefill_kernel with
// 32x32 tiles for bf16, fp8 and INT4 at head_dim 128 and bf16 at 256.
#include "mfma_tiles.h"

namespace kvs {
namespace {
using namespace tiles;

// Several query rows per request and many column groups (a long append or a
// prefill): the four waves share every staged K/V tile instead of splitting
// the keys.  Wave w computes column groups cgw + CG * w .. cgw + CG * w + CG - 1
// of one KV head, so a workgroup covers 16 * CG * kWaves columns and reads
// each K/V byte of its chunk once for all of them.  Keys advance in blocks of
// kWaves 16-token tiles: each wave stages one tile of the block into LDS
// (DMA), a barrier publishes the block, every wave runs the block's tiles
// through its column groups, and a second barrier frees the slot for the
// block NBUF further on.  A wave's columns are its own, so it writes its
// results with no merge across waves.
// Whether the shared-tile kernel merges a request's splits itself.
constexpr bool rows_merges_in_kernel(int D, int KT) { return !(D == 256 && KT == DT_INT4); }

template <int D, int KT, int NBUF, int CG>
__global__ __launch_bounds__(kThreads) void partial_rows_kernel(const Params p, const InlineWork w) {
  using S = Shape<D, KT>;
  constexpr int kGroups = kWaves * CG;                   // column groups per workgroup
  constexpr int kBlock = kWaves * kTile;                 // keys per staged block
  constexpr int kSlotBytes = kWaves * 2 * S::kTileBytes; // K and V of a block
  // Tiles two at a time (pair_update) only where one column group per wave
  // leaves the registers for a second tile: with two groups (head_dim <= 128)
  // the pair form reached the register limit and ran slower (a 32k-token MHA
  // cache with 2048 new rows: 359 against 493 TFLOP/s), with one (head_dim
  // 256) it ran faster (8192-row prefill: 162 against 147 TFLOP/s).
  constexpr bool kPairs = CG == 1;

  __shared__ int s_scan[2 * 64];
  __shared__ int s_item[4];
  __shared__ __attribute__((aligned(16))) char smem[NBUF * kSlotBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15;
  const int q4 = lane >> 4;
  const int row_blocks = (p.col_groups + kGroups - 1) / kGroups; // workgroups per (item, KV head)
  const RowsOrder ord = rows_order(row_blocks, p.num_kv_heads, p.rows_xcd_order != 0);
  const int item = ord.item;
  const int kvg = ord.kvg;                                       // KV head
  const int cgw = ord.rb * kGroups;                              // first column group of the workgroup
  const int g = p.group;
  const int Hk = p.num_kv_heads;

  int b, split, nb, L;
  if (!locate_item(p, w, item, kvg == 0 && ord.rb == 0, s_scan, s_item, b, split, nb, L)) return;
  const int nq = req_nq(p, b);
  if (cgw * 16 >= nq * g) return; // no column of this workgroup has a query row (uniform)
  const int lo = request_lo(L, nq, p.window);
  const int a0 = (lo & ~(kTile - 1)) + split * p.chunk; // aligned chunk start
  const int t_begin = max(lo, a0);
  const int t_end = min(L, a0 + p.chunk);
  // keys some column of the workgroup sees: from the first key of its first
  // query row to the position of its last (both grow with the row)
  const int q_first = cgw * 16 / g;
  const int q_last = (min(nq * g, (cgw + kGroups) * 16) - 1) / g;
  const int wg_lo = max(t_begin, p.window > 0 ? max(0, L - nq + q_first - p.window + 1) : 0);
  const int wg_hi = min(t_end, L - nq + q_last + 1);
  const int fb = wg_hi > wg_lo ? (wg_lo - a0) / kBlock : 0; // first block, counted from the chunk start
  const int nblocks = wg_hi > wg_lo ? (wg_hi - a0 + kBlock - 1) / kBlock - fb : 0;
  const int k0 = a0 + fb * kBlock; // first key of block 0

  // ---- this wave's column groups ----
  ColumnSet<D, KT, CG> cs;
  set_columns(cs, p, b, L, nq, kvg, cgw + wave * CG, g, t_begin, t_end, c16);
  int all_lo, all_hi, wv_lo, wv_hi; // keys every / some column of the wave sees
  column_ranges(cs, t_begin, t_end, all_lo, all_hi, wv_lo, wv_hi);
  load_columns<D>(cs, p, q4, 0);
  float cscale = p.score_scale;
  if (KT != DT_BF16) cscale *= p.k_scale[b * Hk + kvg];
  const float cap_out = p.cap_out;
  const s16x4_t ident = transpose_identity(c16, q4);

  // ---- addressing: this wave's tile of block i, one block per lane ----
  // (a block holds kBlock keys and chunks at most 64 * kBlock, so 64 lanes
  // cover every block; tiles holding no key the workgroup sees move no bytes)
  const size_t row_bytes = (size_t)Hk * S::kRowBytes;
  const bool paged = p.page_size > 0;
  const int *pages = paged ? p.page_indices + p.page_indptr[b] : nullptr;
  uint32_t voff_lo = 0, voff_hi = 0, vbytes = 0;
  if (lane < nblocks) {
    const int ts = k0 + lane * kBlock + wave * kTile;
    if (ts < wg_hi && ts + kTile > wg_lo) {
      const size_t row0 =
          paged ? (size_t)pages[ts >> p.page_shift] * p.page_size + (ts & (p.page_size - 1)) : (size_t)ts;
      const size_t off = row0 * row_bytes;
      voff_lo = (uint32_t)off;
      voff_hi = (uint32_t)(off >> 32);
      vbytes = (uint32_t)(min(kTile, wg_hi - ts) * (int)row_bytes);
    }
  }
  const char *kpool = reinterpret_cast<const char *>(p.k);
  const char *vpool = reinterpret_cast<const char *>(p.v);
  int dma_voff[S::kDma]; // lane's byte offset within a tile, per DMA load
#pragma unroll
  for (int k = 0; k < S::kDma; ++k) {
    const int r = k * S::kRowsPerDma + lane / S::kPieces;
    const int piece = (lane % S::kPieces) ^ stage_swizzle<D, KT>(r);
    dma_voff[k] = r * (int)row_bytes + kvg * S::kRowBytes + piece * 16; // < 2^31: checked on the host
  }
  // tile u of slot s sits at smem + (s * kWaves + u) * 2 * kTileBytes (K, then V)
  auto issue = [&](int i, int slot) {
    const int li = min(i, 63);
    const size_t base = ((size_t)__builtin_amdgcn_readlane(voff_hi, li) << 32) | __builtin_amdgcn_readlane(voff_lo, li);
    const int nbytes = i < nblocks ? (int)__builtin_amdgcn_readlane(vbytes, li) : 0;
    const __amdgpu_buffer_rsrc_t kr =
        __builtin_amdgcn_make_buffer_rsrc((void *)(kpool + base), (short)0, nbytes, kBufferFlags);
    const __amdgpu_buffer_rsrc_t vr =
        __builtin_amdgcn_make_buffer_rsrc((void *)(vpool + base), (short)0, nbytes, kBufferFlags);
    char *kst = smem + (slot * kWaves + wave) * 2 * S::kTileBytes;
    char *vst = kst + S::kTileBytes;
#pragma unroll
    for (int k = 0; k < S::kDma; ++k) dma16_to_lds(kr, kst + 1024 * k, dma_voff[k]);
#pragma unroll
    for (int k = 0; k < S::kDma; ++k) dma16_to_lds(vr, vst + 1024 * k, dma_voff[k]);
  };
  StageReader<D, KT> stage; // lane addresses of tile 0 of slot 0
  stage.init(lds_address(smem), lane);
  auto read_stage = [&](TileRegs<D, KT> &t, int slot, int u) {
    stage.read(t, (slot * kWaves + u) * 2 * S::kTileBytes);
  };

  // ---- ring of NBUF block slots shared by the waves ----
  if (nblocks > 0) { // the same in every wave
#pragma unroll
    for (int j = 0; j < NBUF; ++j) issue(j, j);
    const int n_iter = (nblocks + NBUF - 1) / NBUF * NBUF;
    for (int it = 0; it < n_iter; it += NBUF) {
#pragma unroll
      for (int j = 0; j < NBUF; ++j) {
        const int i = it + j;
        wait_vmem<(NBUF - 1) * 2 * S::kDma>(); // this wave's tile of block i has landed
        __syncthreads();                       // ... and every other wave's
        if (i < nblocks) {
          if constexpr (kPairs) {
            // the block's tiles two at a time: one softmax step and one
            // k = 32 product per pair
#pragma unroll
            for (int u = 0; u < kWaves; u += 2) {
              const int tsa = k0 + i * kBlock + u * kTile, tsb = tsa + kTile;
              if (tsa < wv_hi && tsb + kTile > wv_lo) { // the wave's columns see keys of this pair
                TileRegs<D, KT> ta, tb;
                read_stage(ta, j, u);
                read_stage(tb, j, u + 1);
                zero_v_before(ta, tsa, wv_lo, c16, q4);
                zero_v_before(tb, tsb, wv_lo, c16, q4);
                pair_update(cs, ta, tsa, tb, tsb, all_lo, all_hi, cscale, cap_out, ident, q4);
              }
            }
          } else {
#pragma unroll
            for (int u = 0; u < kWaves; ++u) {
              const int ts = k0 + i * kBlock + u * kTile;
              if (ts < wv_hi && ts + kTile > wv_lo) { // the wave's columns see keys of this tile
                TileRegs<D, KT> t;
                read_stage(t, j, u);
                zero_v_before(t, ts, wv_lo, c16, q4);
                tile_update(cs, t, ts, all_lo, all_hi, cscale, cap_out, ident, q4);
              }
            }
          }
        }
        __syncthreads(); // every wave has read slot j
        issue(i + NBUF, j);
      }
    }
    wait_vmem<0>(); // no DMA may land in LDS after the workgroup ends
  }

  // ---- results of this wave's columns: final output, or the split's partial ----
#pragma unroll
  for (int c = 0; c < CG; ++c) {
    if (!cs.on[c]) continue; // the same in every lane of the wave
    float l_tot = cs.l[c] + __shfl_xor(cs.l[c], 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    float lb_tot = 0.0f;
    if constexpr (KT == DT_INT4) {
      lb_tot = cs.lb[c] + __shfl_xor(cs.lb[c], 16, 64);
      lb_tot += __shfl_xor(lb_tot, 32, 64);
    }
    if (!cs.ok[c]) continue;
    const bool live = l_tot > 0.0f; // a finite reference with no visible key leaves l = 0: empty
    const float vscale = p.v_scale && (nb == 1 || !part_f16_of<KT>()) ? p.v_scale[b * Hk + kvg] : 1.0f;
    const float inv = live ? vscale / l_tot : 0.0f;
    const float lse2 = live ? cs.m[c] + __log2f(l_tot) : -INFINITY;
    // INT4: V entered the product as 136 + n; remove 136 * (sum of the weights it saw)
    const float voff = kInt4Offset * lb_tot;
    if (nb == 1) {
      const size_t rowoff = ((size_t)cs.row[c] * p.num_qo_heads + cs.head[c]) * D;
#pragma unroll
      for (int wt = 0; wt < S::kOTiles; ++wt) {
        const int od = out_dim<D, KT>(wt, q4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float val = (cs.acc[c][wt][r] - voff) * inv;
          const size_t off = rowoff + od + r * S::kOutStride;
          if (p.out_bf16)
            reinterpret_cast<uint16_t *>(p.o)[off] = f32_to_bf16_bits(val);
          else
            reinterpret_cast<float *>(p.o)[off] = val;
        }
      }
      if (q4 == 0 && p.lse) p.lse[(size_t)cs.row[c] * p.num_qo_heads + cs.head[c]] = lse2 * kLn2;
    } else {
      const int cg = cgw + wave * CG + c;
      const size_t slot = ((size_t)kvg * p.col_groups + cg) * p.items + item;
      const size_t dst = (slot * p.cols + c16) * D;
#pragma unroll
      for (int wt = 0; wt < S::kOTiles; ++wt) {
        const int od = out_dim<D, KT>(wt, q4);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          store_part1<part_f16_of<KT>()>(p, dst + od + r * S::kOutStride, (cs.acc[c][wt][r] - voff) * inv);
      }
      if (q4 == 0) store_partial(p, p.lse_part + slot * p.cols + c16, lse2);
    }
  }
  // INT4 at head_dim 256 sits at the register limit, and the merge code would
  // cost it half its occupancy: the host leaves its merge to the merge kernel
  if constexpr (rows_merges_in_kernel(D, KT))
    finish_split<D>(p, kvg * row_blocks + ord.rb, b, kvg, cgw, kGroups, item, split, nb, smem);
}

// Four 8-bit transposing reads (ds_read_b64_tr_b8, layout as for
// lds_read_tr8_x8) at four lane addresses, one wait.
__device__ __forceinline__ void lds_read_tr8_x4(uint2 (&v)[4], const uint32_t (&a)[4], uint32_t off) {
  typedef unsigned u32x2v __attribute__((ext_vector_type(2)));
  u32x2v r0, r1, r2, r3;
  __asm__ volatile("ds_read_b64_tr_b8 %0, %4\n\t"
                   "ds_read_b64_tr_b8 %1, %5\n\t"
                   "ds_read_b64_tr_b8 %2, %6\n\t"
                   "ds_read_b64_tr_b8 %3, %7\n\t"
                   "s_waitcnt lgkmcnt(0)"
                   : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
                   : "v"(a[0] + off), "v"(a[1] + off), "v"(a[2] + off), "v"(a[3] + off)
                   : "memory");
  v[0] = __builtin_bit_cast(uint2, r0);
  v[1] = __builtin_bit_cast(uint2, r1);
  v[2] = __builtin_bit_cast(uint2, r2);
  v[3] = __builtin_bit_cast(uint2, r3);
}

// Several query rows per request, bf16, fp8 or INT4 KV at head_dim 128 and
// bf16 at 256, from three groups of 16 columns on (INT4: five): 32x32
// matrix tiles.  Each wave
// owns 32 (query row, head) columns of one KV head (at head_dim 256 a pair of
// waves shares them, each keeping half of the output dims) and the
// workgroup's four waves share every staged block of keys (one part staged
// by each wave, barriers around it, as in partial_rows_kernel).  Per 32-key
// tile and wave:
//   * S^T[key][column] = K . Q^T with v_mfma_f32_32x32x16_bf16 over
//     head_dim / 16 steps of 16 dims: lane (i, h) = (l % 32, l / 32) feeds K row i, dims
//     16 s + 8 h .. + 7, read from LDS; the result holds, in lane (j, h),
//     keys 8 (v / 4) + 4 h + v % 4 (register v) of column j.
//   * online softmax per column over its 32 keys, which sit in lanes j and
//     j + 32: in-lane max over 16 scores, one lane swap.
//   * O^T[dim][column] += V^T . P^T with the same instruction (k = 16 keys),
//     twice per tile: for half t of the tile, lane (j, h) supplies its own
//     registers 8 t .. 8 t + 7 as P^T (keys 16 t + 8 (e / 4) + 4 h + e % 4),
//     and V^T comes straight from LDS with transposing reads in that key
//     order (two reads of four consecutive keys per operand).
// 32-key tiles halve the cross-lane steps per key and run the P.V product
// at the full rate of the 32x32x16 form.
// fp8 KV: K pieces are converted to bf16 for the score product (lane half
// h takes whole 16-byte pieces 2 m + h, dims ordered to match the query's),
// V^T comes from 8-bit transposing reads (eight consecutive rows of a dim
// per lane) and is converted likewise.  So that eight consecutive staged rows
// are exactly the keys of a lane's P^T operand, operand row i of K reads the
// staged row pi(i), pi swapping bits 3 and 2 of the row within each 16; score
// row R then belongs to key pi(R).
// INT4 KV: the same key order; a lane half takes 32 bytes of a K row (64
// dims, nibbles as 136 + n in bf16, even dims then odd, the query permuted to
// match), and one 8-bit transposing read per 64-dim block gives the even and
// odd dims' V^T operands.  The offsets 136 * sum(q) and 136 * sum(p) are taken
// out of the scores and the output.

template <int D, int KT, int NBUF>
__global__ __launch_bounds__(kThreads) void partial_prefill_kernel(const Params p, const InlineWork w) {
  static_assert((D == 128 && (KT == DT_BF16 || KT == DT_FP8 || KT == DT_INT4)) || (D == 256 && KT == DT_BF16),
                "bf16, fp8 or INT4 at head_dim 128, bf16 at 256");
  constexpr bool kFp8 = KT == DT_FP8;
  constexpr bool kInt4 = KT == DT_INT4;
  constexpr bool kPerm = kFp8 || kInt4; // V^T by 8-bit transposing reads: K rows pi-permuted
  using S = Shape<D, KT>;                         // bf16: 16 pieces a row per 128 dims; fp8: 8
  constexpr int kRowBytes = S::kRowBytes;         // one key's K (or V) row of the head
  // head_dim 256: waves 2 c and 2 c + 1 share column set c; both form the
  // scores over all dims (the same softmax state), each keeps the O^T dims
  // 128 w % 2 .. + 127.  Keys are staged 8 rows per wave (32-key blocks) so
  // that two 32 KB block slots still leave two workgroups per CU.
  constexpr bool kSplitD = D == 256;
  // bf16: split partials stored as row-scaled fp16 when the host asks (a
  // row is one wave's, in two lane halves; at head_dim 256 a wave pair's)
  constexpr bool kRowScaled = KT == DT_BF16;
  constexpr int kColWaves = kSplitD ? kWaves / 2 : kWaves; // 32-column sets per workgroup
  constexpr int kPart = kSplitD ? 8 : kTile;      // rows each wave stages per block
  constexpr int kBlock = kWaves * kPart;          // keys staged per block (64 or 32)
  constexpr int kTiles32 = kBlock / 32;           // 32-key tiles per block
  constexpr int kHalf = kBlock * kRowBytes;       // K (or V) bytes of a block
  constexpr int kGroups = kColWaves * 2;          // 16-column groups per workgroup
  constexpr int kDmaP = kPart * kRowBytes / 1024; // 16-byte DMA loads per wave part (K or V)
  constexpr int kSteps = D / 16;                  // 32x32x16 products of S^T per tile
  // head_dim 256: each wave of a pair forms the score product over its own
  // 128 dims and the pair adds the two halves through LDS
  constexpr int kStepsW = kSplitD ? kSteps / 2 : kSteps; // products per wave
  // blocks of the longest chunk (64 tiles per wave, 4096 keys) per lane of the offset table
  constexpr int kLaneBlocks = 64 * kWaves * kTile / kBlock / 64;
  static_assert(kDmaP >= 1 && kLaneBlocks >= 1 && kTiles32 >= 1, "block shape");
  typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

  __shared__ int s_scan[2 * 64];
  __shared__ int s_item[4];
  __shared__ __attribute__((aligned(16))) char smem[NBUF * 2 * kHalf];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j32 = lane & 31; // column of the lane (S^T, O^T) / row (K, V^T operands)
  const int h2 = lane >> 5;  // half of the wave
  const int row_blocks = (p.col_groups + kGroups - 1) / kGroups;
  const RowsOrder ord = rows_order(row_blocks, p.num_kv_heads, p.rows_xcd_order != 0);
  const int item = ord.item;
  const int kvg = ord.kvg;
  const int cgw = ord.rb * kGroups; // first 16-column group of the workgroup
  const int g = p.group;
  const int Hk = p.num_kv_heads;

  int b, split, nb, L;
  if (!locate_item(p, w, item, kvg == 0 && ord.rb == 0, s_scan, s_item, b, split, nb, L)) return;
  const int nq = req_nq(p, b);
  if (cgw * 16 >= nq * g) return; // uniform over the workgroup
  const int lo = request_lo(L, nq, p.window);
  const int a0 = (lo & ~(kTile - 1)) + split * p.chunk;
  const int t_begin = max(lo, a0);
  const int t_end = min(L, a0 + p.chunk);
  // keys some column of the workgroup sees (rows and their keys both grow with the column)
  const int q_first = cgw * 16 / g;
  const int q_last = (min(nq * g, (cgw + kGroups) * 16) - 1) / g;
  const int wg_lo = max(t_begin, p.window > 0 ? max(0, L - nq + q_first - p.window + 1) : 0);
  const int wg_hi = min(t_end, L - nq + q_last + 1);
  const int fb = wg_hi > wg_lo ? (wg_lo - a0) / kBlock : 0;
  const int nblocks = wg_hi > wg_lo ? (wg_hi - a0 + kBlock - 1) / kBlock - fb : 0;
  const int k0 = a0 + fb * kBlock;

  // ---- this lane's column ----
  const int cw = kSplitD ? wave >> 1 : wave; // column set of the wave
  const int dh = kSplitD ? wave & 1 : 0;     // O^T dims 128 dh .. 128 dh + 127 (head_dim 256)
  const int col = cgw * 16 + cw * 32 + j32;
  const bool ok = col < nq * g;
  const bool wave_on = (cgw * 16 + cw * 32) < nq * g; // the same in every lane of the wave
  const int qi = col / g;
  const int qrow = p.qo_indptr[b] + qi;
  const int qhead = kvg * g + col % g;
  const int qpos = L - nq + qi;
  const int c_lo = max(t_begin, p.window > 0 ? max(0, qpos - p.window + 1) : 0);
  const int c_hi = min(t_end, qpos + 1);
  int all_lo = t_begin, all_hi = t_end, wv_lo = t_end, wv_hi = t_begin;
  if (ok) {
    all_lo = c_lo;
    all_hi = c_hi;
    if (c_lo < c_hi) {
      wv_lo = c_lo;
      wv_hi = c_hi;
    }
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    all_lo = max(all_lo, __shfl_xor(all_lo, o, 64));
    all_hi = min(all_hi, __shfl_xor(all_hi, o, 64));
    wv_lo = min(wv_lo, __shfl_xor(wv_lo, o, 64));
    wv_hi = max(wv_hi, __shfl_xor(wv_hi, o, 64));
  }
  all_lo = __builtin_amdgcn_readfirstlane(all_lo);
  all_hi = __builtin_amdgcn_readfirstlane(all_hi);
  wv_lo = __builtin_amdgcn_readfirstlane(wv_lo);
  wv_hi = __builtin_amdgcn_readfirstlane(wv_hi);

  // Q^T operand of step s: dims 16 s + 8 h2 .. + 7 of the column's query
  // (fp8: dims 16 (2 (s / 2) + h2) + 8 (s % 2) .., the order of its K pieces;
  // INT4: the 8 dims of K dword 8 h2 + s, even ones first, as its nibbles)
  bf16x8_t qop[kStepsW];
  float qoff = 0.0f; // INT4: the scores carry 136 * (sum of the column's q)
  {
    const uint16_t *qb = reinterpret_cast<const uint16_t *>(p.q) + ((size_t)qrow * p.num_qo_heads + qhead) * D;
#pragma unroll
    for (int s = 0; s < kStepsW; ++s) {
      const int d0 = kInt4 ? 8 * (8 * h2 + s)
                           : (kFp8 ? 16 * (2 * (s / 2) + h2) + 8 * (s % 2) : 128 * dh + 16 * s + 8 * h2);
      bf16x8_t x = ok ? __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(qb + d0))
                      : __builtin_bit_cast(bf16x8_t, make_uint4(0, 0, 0, 0));
      if constexpr (kInt4) {
        x = __builtin_shufflevector(x, x, 0, 2, 4, 6, 1, 3, 5, 7);
#pragma unroll
        for (int e = 0; e < 8; ++e) qoff += (float)x[e];
      }
      qop[s] = x;
    }
  }
  if constexpr (kInt4) qoff = (qoff + __shfl_xor(qoff, 32, 64)) * kInt4Offset;
  const float cscale = kPerm ? p.score_scale * p.k_scale[b * Hk + kvg] : p.score_scale;
  const float cap_out = p.cap_out;
  float m_run = p.m_init, l_run = 0.0f;
  bool seen = false; // the column has had a visible key (the same in its two lanes)
  float lb_run = 0.0f; // INT4: the same sum of the bf16-rounded weights P.V saw
  // O^T, 32-dim slice sl: register v holds dim 32 sl + 8 (v / 4) + 4 h2 + v % 4
  // (INT4: dim 64 (sl / 2) + 2 (8 (v / 4) + 4 h2 + v % 4) + sl % 2)
  f32x16_t acc[4];
#pragma unroll
  for (int sl = 0; sl < 4; ++sl)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[sl][v] = 0.0f;

  // ---- staging: this wave's kPart-row part of block i; lane l holds the
  // offsets of blocks l + 64 q ----
  const size_t row_bytes = (size_t)Hk * kRowBytes;
  const bool paged = p.page_size > 0;
  const int *pages = paged ? p.page_indices + p.page_indptr[b] : nullptr;
  uint32_t voff_lo[kLaneBlocks], voff_hi[kLaneBlocks], vbytes[kLaneBlocks];
#pragma unroll
  for (int q = 0; q < kLaneBlocks; ++q) {
    voff_lo[q] = voff_hi[q] = vbytes[q] = 0;
    const int bi = lane + 64 * q;
    if (bi < nblocks) {
      const int ts = k0 + bi * kBlock + wave * kPart;
      if (ts < wg_hi && ts + kPart > wg_lo) {
        const size_t row0 =
            paged ? (size_t)pages[ts >> p.page_shift] * p.page_size + (ts & (p.page_size - 1)) : (size_t)ts;
        const size_t off = row0 * row_bytes;
        voff_lo[q] = (uint32_t)off;
        voff_hi[q] = (uint32_t)(off >> 32);
        vbytes[q] = (uint32_t)(min(kPart, wg_hi - ts) * (int)row_bytes);
      }
    }
  }
  const char *kpool = reinterpret_cast<const char *>(p.k);
  const char *vpool = reinterpret_cast<const char *>(p.v);
  // lane i of load k: row k * kRowsPerDma + i / kPieces of the part, position
  // i % kPieces, which holds source piece position ^ swizzle(row) (rows of a
  // block keep the swizzle of their position within the part)
  int dma_voff[kDmaP];
#pragma unroll
  for (int k = 0; k < kDmaP; ++k) {
    const int r = k * S::kRowsPerDma + lane / S::kPieces;
    const int piece = (lane % S::kPieces) ^ stage_swizzle<D, KT>(r);
    dma_voff[k] = r * (int)row_bytes + kvg * kRowBytes + piece * 16;
  }
  auto issue = [&](int i, int slot) {
    const int li = i & 63;
    const int q = min(i >> 6, kLaneBlocks - 1); // uniform
    uint32_t lo = voff_lo[0], hi = voff_hi[0], nb8 = vbytes[0];
#pragma unroll
    for (int c = 1; c < kLaneBlocks; ++c)
      if (q == c) {
        lo = voff_lo[c];
        hi = voff_hi[c];
        nb8 = vbytes[c];
      }
    const size_t base = ((size_t)__builtin_amdgcn_readlane(hi, li) << 32) | __builtin_amdgcn_readlane(lo, li);
    const int nbytes = i < nblocks ? (int)__builtin_amdgcn_readlane(nb8, li) : 0;
    const __amdgpu_buffer_rsrc_t kr =
        __builtin_amdgcn_make_buffer_rsrc((void *)(kpool + base), (short)0, nbytes, kBufferFlags);
    const __amdgpu_buffer_rsrc_t vr =
        __builtin_amdgcn_make_buffer_rsrc((void *)(vpool + base), (short)0, nbytes, kBufferFlags);
    char *kst = smem + slot * 2 * kHalf + wave * kPart * kRowBytes;
#pragma unroll
    for (int k = 0; k < kDmaP; ++k) dma16_to_lds(kr, kst + 1024 * k, dma_voff[k]);
#pragma unroll
    for (int k = 0; k < kDmaP; ++k) dma16_to_lds(vr, kst + kHalf + 1024 * k, dma_voff[k]);
  };
  // Staged row R of a tile was written with the swizzle of its position in
  // its wave's part.
  auto row_swizzle = [](int row) { return stage_swizzle<D, KT>(row % kPart); };
  // K operand: bf16, step s: row j32 of the tile, piece 2 s + h2; fp8: row
  // pi(j32), piece 2 m + h2 for steps 2 m and 2 m + 1.  Eight steps per LDS
  // read block.
  // INT4: pieces 2 h2 and 2 h2 + 1 of row pi(j32) (dwords 8 h2 .. 8 h2 + 7).
  uint32_t k_addr[kStepsW / 8][8];
  const int krow = kPerm ? (j32 & ~12) | ((j32 & 8) >> 1) | ((j32 & 4) << 1) : j32;
  {
    const uint32_t base = lds_address(smem) + krow * kRowBytes;
#pragma unroll
    for (int s = 0; s < kStepsW; ++s) {
      const int piece = kInt4 ? 2 * h2 + (s & 1) : (kFp8 ? s & 3 : (kSplitD ? 8 * dh + s : s)) * 2 + h2;
      k_addr[s / 8][s % 8] = base + (piece ^ row_swizzle(krow)) * 16;
    }
  }
  // fp8 V^T reads (ds_read_b64_tr_b8): lane 16 G + 2 r + c of group G points at
  // staged row 8 (G / 2) + r (+ 16 t), dims 32 sl + 16 (G % 2) + 8 c .. + 7
  // (piece 2 sl + G % 2, bytes 8 c of it); lane i of the group then holds rows
  // 8 (G / 2) + 0..7 of dim 32 sl + 16 (G % 2) + i.
  // INT4 V^T: one 8-bit transposing read per key half t and 64-dim block blk,
  // lane 16 G + 2 r + c at row 16 t + 8 (G / 2) + r, bytes
  // 32 blk + 16 (G % 2) + 8 c .. + 7: lane j of a half-wave holds byte j of
  // the block (dims 2 j, 2 j + 1) for 8 consecutive keys.
  uint32_t vt8_addr[8]; // [4 t + sl]; INT4: [2 t + blk]
  if constexpr (kInt4) {
    const int G = lane >> 4, r = (lane >> 1) & 7, c = lane & 1;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const int row = 16 * t + 8 * (G >> 1) + r;
        const int piece = 2 * blk + (G & 1);
        vt8_addr[2 * t + blk] = lds_address(smem) + kHalf + row * kRowBytes + ((piece ^ row_swizzle(row)) * 16) + c * 8;
      }
  }
  if constexpr (kFp8) {
    const int G = lane >> 4, r = (lane >> 1) & 7, c = lane & 1;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) {
        const int row = 16 * t + 8 * (G >> 1) + r;
        const int piece = 2 * sl + (G & 1);
        vt8_addr[4 * t + sl] = lds_address(smem) + kHalf + row * kRowBytes + ((piece ^ row_swizzle(row)) * 16) + c * 8;
      }
  }
  // V^T operand reads (ds_read_b64_tr_b16): lane l = 16 G + 4 r + c of group G
  // points at key row 8 hh + 4 (G / 2) + r (+ 16 t, an immediate), dims
  // 128 dh + 32 sl + 16 (G % 2) + 4 c .. + 3, i.e. piece
  // 16 dh + 4 sl + 2 (G % 2) + c / 2, bytes (c % 2) * 8 of it; lane i of the
  // group then holds keys 8 hh + 4 (G / 2) + 0..3 of dim
  // 128 dh + 32 sl + 16 (G % 2) + i.  (Rows 16 .. 31 keep the swizzles of
  // rows 0 .. 15: kPart divides 16.)
  uint32_t vt_addr[8]; // [4 hh + sl]
  if constexpr (!kPerm) {
    const int G = lane >> 4, r = (lane >> 2) & 3, c = lane & 3;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) {
        const int row = 8 * hh + 4 * (G >> 1) + r;
        const int piece = 16 * dh + 4 * sl + 2 * (G & 1) + (c >> 1);
        vt_addr[4 * hh + sl] = lds_address(smem) + kHalf + row * kRowBytes + ((piece ^ row_swizzle(row)) * 16) + (c & 1) * 8;
      }
  }

  // one 32-key tile (first key ts) at byte offset `to` of the staged block:
  // the score product (of the wave's dims), then the rest
  auto scores32 = [&](uint32_t to) {
    // ---- S^T = K . Q^T ----
    f32x16_t st;
#pragma unroll
    for (int v = 0; v < 16; ++v) st[v] = 0.0f;
    if constexpr (kInt4) { // dword s of the lane's 32 bytes, as 136 + n (even nibbles, then odd)
      uint4 kr0, kr1;
      lds_read_k2(kr0, kr1, k_addr[0][0] + to, k_addr[0][1] + to);
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const uint32_t x = dword_of(s < 4 ? kr0 : kr1, s & 3);
        const uint32_t ev = int4_even(x), od = int4_odd(x);
        const bf16x8_t kop = __builtin_bit_cast(
            bf16x8_t, make_uint4(offset_bf16_lo(ev), offset_bf16_hi(ev), offset_bf16_lo(od), offset_bf16_hi(od)));
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[s], st, 0, 0, 0);
      }
      // st still carries qoff: taken out in the max and the exponent below
    } else if constexpr (kFp8) {
      bf16x8_t kop[8];
      uint4 kr[4];
      lds_read_x4(kr, k_addr[0], to);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        kop[2 * m] = fp8x8_to_bf16x8(kr[m].x, kr[m].y);
        kop[2 * m + 1] = fp8x8_to_bf16x8(kr[m].z, kr[m].w);
      }
#pragma unroll
      for (int s = 0; s < 8; ++s) st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[s], qop[s], st, 0, 0, 0);
    } else {
#pragma unroll
      for (int hb = 0; hb < kStepsW / 8; ++hb) {
        uint4 kr[8];
        lds_read_x8(kr, k_addr[hb], to);
#pragma unroll
        for (int s = 0; s < 8; ++s)
          st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kr[s]), qop[8 * hb + s], st, 0, 0, 0);
      }
    }
    return st;
  };
  auto finish32 = [&](int ts, uint32_t to, const f32x16_t &st) {
    // V^T operands, read while the products run: vop[t][sl]
    // Keys before wv_lo are seen by no column of the wave; their V rows may
    // hold non-finite values (only visible values are required finite), and
    // 0 * NaN would reach the accumulator, so their operand elements are
    // zeroed (a tile starting there is not whole: its scores are masked).
    const int vt_g = lane >> 4;
    bf16x8_t vop[2][4];
    if constexpr (kInt4) { // operand (t, 2 blk + odd): even or odd nibbles of one read, as 136 + n
      uint2 vn[4];
      lds_read_tr8_x4(vn, *reinterpret_cast<const uint32_t(*)[4]>(&vt8_addr[0]), to);
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
          const uint2 x = vn[2 * t + blk];
          const uint32_t e0 = int4_even(x.x), e1 = int4_even(x.y), o0 = int4_odd(x.x), o1 = int4_odd(x.y);
          vop[t][2 * blk] = __builtin_bit_cast(
              bf16x8_t, make_uint4(offset_bf16_lo(e0), offset_bf16_hi(e0), offset_bf16_lo(e1), offset_bf16_hi(e1)));
          vop[t][2 * blk + 1] = __builtin_bit_cast(
              bf16x8_t, make_uint4(offset_bf16_lo(o0), offset_bf16_hi(o0), offset_bf16_lo(o1), offset_bf16_hi(o1)));
        }
    } else if constexpr (kFp8) {
      uint2 v8[8];
      lds_read_tr8_x8(v8, vt8_addr, to);
      if (ts < wv_lo) { // lane holds rows 16 t + 8 (G / 2) + e, byte e (uniform branch)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          uint32_t lo_keep = 0, hi_keep = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int key = ts + 16 * t + 8 * (vt_g >> 1) + e;
            if (key >= wv_lo) lo_keep |= 0xFFu << (8 * e);
            if (key + 4 >= wv_lo) hi_keep |= 0xFFu << (8 * e);
          }
#pragma unroll
          for (int sl = 0; sl < 4; ++sl) {
            v8[4 * t + sl].x &= lo_keep;
            v8[4 * t + sl].y &= hi_keep;
          }
        }
      }
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int sl = 0; sl < 4; ++sl) vop[t][sl] = fp8x8_to_bf16x8(v8[4 * t + sl].x, v8[4 * t + sl].y);
    } else {
      s16x4_t vt[2][8]; // [t][4 hh + sl]
#pragma unroll
      for (int t = 0; t < 2; ++t) lds_read_tr_x8(vt[t], vt_addr, to + t * 16 * kRowBytes);
      if (ts < wv_lo) { // element e: key 16 t + 8 hh + 4 (G / 2) + e (uniform branch)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (ts + 16 * t + 8 * hh + 4 * (vt_g >> 1) + e < wv_lo) {
#pragma unroll
                for (int sl = 0; sl < 4; ++sl) vt[t][4 * hh + sl][e] = 0;
              }
      }
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int sl = 0; sl < 4; ++sl) {
          const uint2 a = __builtin_bit_cast(uint2, vt[t][sl]), c = __builtin_bit_cast(uint2, vt[t][4 + sl]);
          vop[t][sl] = __builtin_bit_cast(bf16x8_t, make_uint4(a.x, a.y, c.x, c.y));
        }
    }
    // ---- scores: register v holds key ts + 8 (v / 4) + 4 h2 + v % 4 ----
    // Without a soft cap the scale goes into the exponent: the max of the
    // raw scores times the (positive) scale is the max of the scaled ones,
    // and p = exp2(fma(s, scale, -m)) needs no separate multiply.  With a cap
    // the capped scores are formed first and ks is 1.  A zero K scale is
    // raised to the least normal float, so that a masked -inf stays -inf
    // (-inf * 0 would be NaN) while visible scores still contribute nothing.
    const bool capped = cap_out > 0.0f; // uniform
    const float ks = capped ? 1.0f : fmaxf(cscale, __FLT_MIN__);
    float sv[16];
    if (capped) {
#pragma unroll
      for (int v = 0; v < 16; ++v) sv[v] = tanhf((kInt4 ? st[v] - qoff : st[v]) * cscale) * cap_out;
    } else {
#pragma unroll
      for (int v = 0; v < 16; ++v) sv[v] = st[v];
    }
    if (ts < all_lo || ts + 2 * kTile > all_hi) { // some column misses some key (uniform)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = 8 * (v >> 2) + 4 * h2 + (v & 3); // score row; fp8, INT4: key pi(row)
        const int tok = ts + (kPerm ? (row & ~12) | ((row & 8) >> 1) | ((row & 4) << 1) : row);
        if (tok < c_lo || tok >= c_hi) sv[v] = -INFINITY;
      }
    }
    float mx = sv[0];
#pragma unroll
    for (int v = 1; v < 16; ++v) mx = fmaxf(mx, sv[v]);
    mx = xor32_max(mx);
    if constexpr (kInt4) mx -= capped ? 0.0f : qoff; // uncapped INT4 scores still carry qoff
    mx *= ks; // in scaled units
    // lazy rescale (as in the 16x16 kernels): the reference moves only when a
    // score exceeds it by more than kLazy
    const bool empty = !seen; // not l_run == 0: the column's other lane may hold its keys so far
    const bool grow = mx > m_run + kLazy || (empty && mx != -INFINITY && mx < m_run - kDrop);
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float alpha = grow ? (empty ? 0.0f : __builtin_amdgcn_exp2f(m_run - mx)) : 1.0f;
      m_run = grow ? mx : m_run;
      l_run *= alpha;
      if constexpr (kInt4) lb_run *= alpha;
#pragma unroll
      for (int sl = 0; sl < 4; ++sl)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[sl][v] *= alpha;
    }
    seen = seen || mx != -INFINITY;
    // No reference yet (m_run = -inf) means every score of the tile is
    // masked, so any finite offset gives weights of 0 (bf16: one select per
    // tile).  The fp8 and INT4 variants keep a select per weight: the shorter
    // form pushed their register allocation past 256 (one wave per SIMD).
    const bool live = m_run != -INFINITY;
    const float neg_m = live ? -m_run : 0.0f;
    const float bias = kInt4 && !capped ? -m_run - qoff * ks : -m_run; // fp8, INT4 exponent offset
    uint32_t pk[8];
    float sum = 0.0f;
#pragma unroll
    for (int v = 0; v < 16; v += 2) {
      float p0, p1;
      if constexpr (kPerm) {
        p0 = live ? __builtin_amdgcn_exp2f(fmaf(sv[v], ks, bias)) : 0.0f;
        p1 = live ? __builtin_amdgcn_exp2f(fmaf(sv[v + 1], ks, bias)) : 0.0f;
      } else {
        p0 = __builtin_amdgcn_exp2f(fmaf(sv[v], ks, neg_m));
        p1 = __builtin_amdgcn_exp2f(fmaf(sv[v + 1], ks, neg_m));
      }
      sum += p0 + p1;
      pk[v / 2] = pack_bf16x2(p0, p1);
      if constexpr (kInt4) // the weights as the P.V product sees them
        lb_run += __uint_as_float(pk[v / 2] << 16) + __uint_as_float(pk[v / 2] & 0xFFFF0000u);
    }
    l_run += sum;
    // ---- O^T += V^T . P^T, k = 16 keys per product ----
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const bf16x8_t pt = __builtin_bit_cast(bf16x8_t, make_uint4(pk[4 * t], pk[4 * t + 1], pk[4 * t + 2], pk[4 * t + 3]));
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) acc[sl] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[t][sl], pt, acc[sl], 0, 0, 0);
    }
  };

  // ---- ring of NBUF block slots shared by the waves ----
  if (nblocks > 0) {
#pragma unroll
    for (int j = 0; j < NBUF; ++j) issue(j, j);
    const int n_iter = (nblocks + NBUF - 1) / NBUF * NBUF;
    for (int it = 0; it < n_iter; it += NBUF) {
#pragma unroll
      for (int j = 0; j < NBUF; ++j) {
        const int i = it + j;
        wait_vmem<(NBUF - 1) * 2 * kDmaP>();
        __syncthreads();
        if constexpr (kSplitD) {
          // one 32-key tile per block; the pair's two score halves meet in
          // the block's K rows, which no wave reads once its products are
          // formed (the barriers are taken by every wave, whether or not it
          // has keys in this tile)
          static_assert(!kSplitD || kTiles32 == 1, "one tile per block");
          const int ts = k0 + i * kBlock;
          const uint32_t to = j * 2 * kHalf;
          const bool vis = i < nblocks && wave_on && ts < wv_hi && ts + 2 * kTile > wv_lo; // the same in a pair
          f32x16_t st;
          if (vis) st = scores32(to);
          __syncthreads(); // every wave's K reads of this block are done
          float *xs = reinterpret_cast<float *>(smem + to);
          if (vis) {
#pragma unroll
            for (int v = 0; v < 16; ++v) xs[(wave * 16 + v) * 64 + lane] = st[v];
          }
          __syncthreads();
          if (vis) {
#pragma unroll
            for (int v = 0; v < 16; ++v) st[v] += xs[((wave ^ 1) * 16 + v) * 64 + lane];
            finish32(ts, to, st);
          }
        } else if (i < nblocks && wave_on) {
#pragma unroll
          for (int u = 0; u < kTiles32; ++u) {
            const int ts = k0 + i * kBlock + u * 2 * kTile;
            const uint32_t to = j * 2 * kHalf + u * 2 * kTile * kRowBytes;
            if (ts < wv_hi && ts + 2 * kTile > wv_lo) finish32(ts, to, scores32(to));
          }
        }
        __syncthreads();
        issue(i + NBUF, j);
      }
    }
    wait_vmem<0>();
  }

  // head_dim 256, row-scaled partials: the largest magnitude of each row
  // over both waves of its pair (each holds 128 of its dims), exchanged
  // through LDS; every wave takes the barrier (part_row_scale is uniform)
  float pair_amax = 0.0f;
  if constexpr (kRowScaled && kSplitD) {
    __shared__ float s_amax[kWaves][32];
    if (p.part_row_scale) {
      float a = 0.0f;
#pragma unroll
      for (int sl = 0; sl < 4; ++sl)
#pragma unroll
        for (int v = 0; v < 16; ++v) a = fmaxf(a, fabsf(acc[sl][v]));
      a = fmaxf(a, __shfl_xor(a, 32, 64));
      if (h2 == 0) s_amax[wave][j32] = a;
      __syncthreads();
      pair_amax = fmaxf(a, s_amax[wave ^ 1][j32]);
    }
  }

  // ---- this lane's column: final output, or the split's partial ----
  [&] {
  if (!wave_on) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (!ok) return;
  const bool live = l_tot > 0.0f;
  const float vscale = kPerm && writer_scales_v(p, nb) ? p.v_scale[b * Hk + kvg] : 1.0f;
  const float inv = live ? vscale / l_tot : 0.0f;
  const float lse2 = live ? m_run + __log2f(l_tot) : -INFINITY;
  if constexpr (kInt4) {
    // V entered the product as 136 + n: remove 136 * (sum of the weights it
    // saw).  Slices 2 blk and 2 blk + 1 hold the even and odd dims of block
    // blk, so registers 4 q .. 4 q + 3 of the pair are dims
    // 64 blk + 16 q + 8 h2 .. + 7, interleaved.
    const float voff = kInt4Offset * (lb_run + __shfl_xor(lb_run, 32, 64));
    size_t dst = 0;
    uint16_t *orow = nullptr;
    size_t slot = 0;
    if (nb == 1) {
      orow = reinterpret_cast<uint16_t *>(p.o) + ((size_t)qrow * p.num_qo_heads + qhead) * D;
    } else {
      slot = ((size_t)kvg * p.col_groups + col / 16) * p.items + item;
      dst = (slot * p.cols + col % 16) * D;
    }
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float o8[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o8[2 * e] = (acc[2 * blk][4 * q + e] - voff) * inv;
          o8[2 * e + 1] = (acc[2 * blk + 1][4 * q + e] - voff) * inv;
        }
        const int d0 = 64 * blk + 16 * q + 8 * h2;
        if (nb == 1) {
          *reinterpret_cast<uint4 *>(orow + d0) = make_uint4(pack_bf16x2(o8[0], o8[1]), pack_bf16x2(o8[2], o8[3]),
                                                             pack_bf16x2(o8[4], o8[5]), pack_bf16x2(o8[6], o8[7]));
        } else {
          store_part4(p, dst + d0, o8[0], o8[1], o8[2], o8[3]);
          store_part4(p, dst + d0 + 4, o8[4], o8[5], o8[6], o8[7]);
        }
      }
    if (h2 == 0) {
      if (nb == 1) {
        if (p.lse) p.lse[(size_t)qrow * p.num_qo_heads + qhead] = lse2 * kLn2;
      } else {
        store_partial(p, p.lse_part + slot * p.cols + col % 16, lse2);
      }
    }
    return;
  }
  if (nb == 1) {
    uint16_t *orow = reinterpret_cast<uint16_t *>(p.o) + ((size_t)qrow * p.num_qo_heads + qhead) * D;
#pragma unroll
    for (int sl = 0; sl < 4; ++sl)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int d0 = 128 * dh + 32 * sl + 8 * q + 4 * h2;
        *reinterpret_cast<uint2 *>(orow + d0) =
            make_uint2(pack_bf16x2(acc[sl][4 * q] * inv, acc[sl][4 * q + 1] * inv),
                       pack_bf16x2(acc[sl][4 * q + 2] * inv, acc[sl][4 * q + 3] * inv));
      }
    if (h2 == 0 && dh == 0 && p.lse) p.lse[(size_t)qrow * p.num_qo_heads + qhead] = lse2 * kLn2;
  } else {
    const int cg = col / 16;
    const size_t slot = ((size_t)kvg * p.col_groups + cg) * p.items + item;
    const size_t dst = (slot * p.cols + col % 16) * D;
    if constexpr (kRowScaled) {
      if (p.part_row_scale) { // the row is the lane's 64 dims and its other half's (lane ^ 32)
        float amax = pair_amax;  // head_dim 256: both waves of the pair (above)
        if constexpr (!kSplitD) {
#pragma unroll
          for (int sl = 0; sl < 4; ++sl)
#pragma unroll
            for (int v = 0; v < 16; ++v) amax = fmaxf(amax, fabsf(acc[sl][v]));
          amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
        }
        const int k = row_scale_exp(amax * inv);
        const float sc = ldexpf(inv, k);
#pragma unroll
        for (int sl = 0; sl < 4; ++sl)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            store_part4<true>(p, dst + 128 * dh + 32 * sl + 8 * q + 4 * h2, acc[sl][4 * q] * sc,
                              acc[sl][4 * q + 1] * sc, acc[sl][4 * q + 2] * sc, acc[sl][4 * q + 3] * sc);
        if (h2 == 0 && dh == 0) {
          store_partial(p, p.lse_part + slot * p.cols + col % 16, lse2);
          store_partial(p, p.sc_part + slot * p.cols + col % 16, ldexpf(1.0f, -k));
        }
        return;
      }
    }
#pragma unroll
    for (int sl = 0; sl < 4; ++sl)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int d0 = 128 * dh + 32 * sl + 8 * q + 4 * h2;
        store_part4(p, dst + d0, acc[sl][4 * q] * inv, acc[sl][4 * q + 1] * inv, acc[sl][4 * q + 2] * inv,
                       acc[sl][4 * q + 3] * inv);
      }
    if (h2 == 0 && dh == 0) store_partial(p, p.lse_part + slot * p.cols + col % 16, lse2);
  }
  }();
  finish_split<D, 1, kFusedMergeBatch, kRowScaled>(p, kvg * row_blocks + ord.rb, b, kvg, cgw, kGroups, item, split,
                                                    nb, smem);
}

// Two column groups (17 to 32 (query row, head) columns per KV head: a few
// query rows per request, as in speculative decoding) with bf16, fp8 or INT4
// KV at head_dim 128: decode-style work split with 32x32 matrix tiles.  The four
// waves take the chunk's 32-key tiles in turn (wave w: tiles w, w + 4, ...),
// each staging its own tiles through a private ring of LDS slots (no
// workgroup barriers); every wave computes all 32 columns on its tiles with
// the products, key order and softmax of partial_prefill_kernel, and the
// waves' states are merged through LDS at the end.  Against the 16x16 decode
// kernel with two groups, the P.V product runs at the full rate of the
// 32x32x16 form and each key's max and weights are formed once per column.
template <int KT, int NBUF>
__global__ __launch_bounds__(kThreads) void partial_cols32_kernel(const Params p, const InlineWork w) {
  static_assert(KT == DT_BF16 || KT == DT_FP8 || KT == DT_INT4, "bf16, fp8 or INT4 KV");
  constexpr bool kFp8 = KT == DT_FP8;
  constexpr bool kInt4 = KT == DT_INT4;
  constexpr bool kPerm = kFp8 || kInt4;     // V^T by 8-bit transposing reads: K rows pi-permuted
  constexpr int D = 128;
  using S = Shape<D, KT>;                   // fp8: 128-byte rows, 8 pieces; bf16: 256, 16; INT4: 64, 4
  constexpr int kRowBytes = S::kRowBytes;
  constexpr int kT = 32;                    // keys per wave tile
  constexpr int kHalfB = kTile * kRowBytes; // one 16-row half of a K (or V) tile
  constexpr int kTileB = 2 * kHalfB;        // K (or V) bytes of a tile
  constexpr int kSlot = 2 * kTileB;         // K, then V
  constexpr int kDmaH = kHalfB / 1024;      // DMA loads per half
  constexpr int OSTRIDE = D + 4;
  constexpr int kStage = kWaves * NBUF * kSlot;
  constexpr int kEpi = 2 * kWaves * 16 * 4 + kWaves * 16 * OSTRIDE * 4;
  constexpr int kSmem = kStage > kEpi ? kStage : kEpi;
  static_assert(kDmaH >= 1, "half-tile loads");
  typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

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
  const int j32 = lane & 31; // column of the lane (S^T, O^T) / row (K, V^T operands)
  const int h2 = lane >> 5;
  const int item = blockIdx.x;
  const int col_blocks = (p.col_groups + 1) / 2; // workgroups per (item, KV head)
  const int kvg = blockIdx.y / col_blocks;
  const int cg0 = blockIdx.y % col_blocks * 2;   // first of the workgroup's two column groups
  const int g = p.group;
  const int Hk = p.num_kv_heads;

  int b, split, nb, L;
  if (!locate_item(p, w, item, blockIdx.y == 0, s_scan, s_item, b, split, nb, L)) return;
  const int nq = req_nq(p, b);
  if (cg0 * 16 >= nq * g) return; // uniform over the workgroup
  const int lo = request_lo(L, nq, p.window);
  const int a0 = (lo & ~(kTile - 1)) + split * p.chunk;
  const int t_begin = max(lo, a0);
  const int t_end = min(L, a0 + p.chunk);

  // ---- this lane's column and the keys it sees ----
  const int col = cg0 * 16 + j32;
  const bool ok = col < nq * g;
  const int qi = col / g;
  const int qrow = p.qo_indptr[b] + qi;
  const int qhead = kvg * g + col % g;
  const int qpos = L - nq + qi;
  const int c_lo = max(t_begin, p.window > 0 ? max(0, qpos - p.window + 1) : 0);
  const int c_hi = min(t_end, qpos + 1);
  int all_lo = t_begin, all_hi = t_end, w_lo = t_end, w_hi = t_begin;
  if (ok) {
    all_lo = c_lo;
    all_hi = c_hi;
    if (c_lo < c_hi) {
      w_lo = c_lo;
      w_hi = c_hi;
    }
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    all_lo = max(all_lo, __shfl_xor(all_lo, o, 64));
    all_hi = min(all_hi, __shfl_xor(all_hi, o, 64));
    w_lo = min(w_lo, __shfl_xor(w_lo, o, 64));
    w_hi = max(w_hi, __shfl_xor(w_hi, o, 64));
  }
  all_lo = __builtin_amdgcn_readfirstlane(all_lo);
  all_hi = __builtin_amdgcn_readfirstlane(all_hi);
  w_lo = __builtin_amdgcn_readfirstlane(w_lo);
  w_hi = __builtin_amdgcn_readfirstlane(w_hi);
  // 32-key tiles from the (16-aligned) chunk start that hold keys some column sees
  const int ft = w_hi > w_lo ? (w_lo - a0) / kT : 0;
  const int ntiles = w_hi > w_lo ? (w_hi - a0 + kT - 1) / kT - ft : 0;
  const int my_tiles = ntiles > wave ? (ntiles - wave + kWaves - 1) / kWaves : 0;

  // Q^T operand of step s: bf16 dims 16 s + 8 h2 .. + 7; fp8 dims
  // 16 (2 (s / 2) + h2) + 8 (s % 2) .. + 7 (the order of its K pieces);
  // INT4 the 8 dims of K dword 8 h2 + s, even ones first (as its nibbles)
  bf16x8_t qop[8];
  float qoff = 0.0f; // INT4: the scores carry 136 * (sum of the column's q)
  {
    const uint16_t *qb = reinterpret_cast<const uint16_t *>(p.q) + ((size_t)qrow * p.num_qo_heads + qhead) * D;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int d0 = kInt4 ? 8 * (8 * h2 + s) : (kFp8 ? 16 * (2 * (s / 2) + h2) + 8 * (s % 2) : 16 * s + 8 * h2);
      bf16x8_t x = ok ? __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(qb + d0))
                      : __builtin_bit_cast(bf16x8_t, make_uint4(0, 0, 0, 0));
      if constexpr (kInt4) {
        x = __builtin_shufflevector(x, x, 0, 2, 4, 6, 1, 3, 5, 7);
#pragma unroll
        for (int e = 0; e < 8; ++e) qoff += (float)x[e];
      }
      qop[s] = x;
    }
  }
  if constexpr (kInt4) qoff = (qoff + __shfl_xor(qoff, 32, 64)) * kInt4Offset;
  const float cscale = kPerm ? p.score_scale * p.k_scale[b * Hk + kvg] : p.score_scale;
  const float cap_out = p.cap_out;
  const bool capped = cap_out > 0.0f;
  const float ks = capped ? 1.0f : fmaxf(cscale, __FLT_MIN__); // see partial_prefill_kernel
  float m_run = p.m_init, l_run = 0.0f;
  bool seen = false; // the column has had a visible key (the same in its two lanes)
  float lb_run = 0.0f; // INT4: the same sum of the bf16-rounded weights P.V saw
  // O^T, 32-dim slice sl: register v holds dim 32 sl + 8 (v / 4) + 4 h2 + v % 4;
  // INT4: dim 64 (sl / 2) + 2 (8 (v / 4) + 4 h2 + v % 4) + sl % 2
  f32x16_t acc[4];
#pragma unroll
  for (int sl = 0; sl < 4; ++sl)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[sl][v] = 0.0f;

  // ---- staging: lane i holds where the two 16-row halves of this wave's
  // tile i start and how many of their bytes hold keys (a wave owns at most
  // 32 tiles: chunks are capped at 4096 keys) ----
  const size_t row_bytes = (size_t)Hk * kRowBytes;
  const bool paged = p.page_size > 0;
  const int *pages = paged ? p.page_indices + p.page_indptr[b] : nullptr;
  uint32_t voff_lo[2] = {0, 0}, voff_hi[2] = {0, 0}, vbytes[2] = {0, 0};
  if (lane < my_tiles) {
    const int ts = a0 + (ft + wave + lane * kWaves) * kT;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int hs = ts + hh * kTile;
      if (hs < w_hi) {
        const size_t row0 = paged ? (size_t)pages[hs >> p.page_shift] * p.page_size + (hs & (p.page_size - 1)) : (size_t)hs;
        const size_t off = row0 * row_bytes;
        voff_lo[hh] = (uint32_t)off;
        voff_hi[hh] = (uint32_t)(off >> 32);
        vbytes[hh] = (uint32_t)(min(kTile, w_hi - hs) * (int)row_bytes);
      }
    }
  }
  const char *kpool = reinterpret_cast<const char *>(p.k);
  const char *vpool = reinterpret_cast<const char *>(p.v);
  int dma_voff[kDmaH];
#pragma unroll
  for (int k = 0; k < kDmaH; ++k) {
    const int r = k * S::kRowsPerDma + lane / S::kPieces;
    const int piece = (lane % S::kPieces) ^ stage_swizzle<D, KT>(r);
    dma_voff[k] = r * (int)row_bytes + kvg * kRowBytes + piece * 16;
  }
  char *wave_stage = smem + wave * NBUF * kSlot;
  auto issue = [&](int i, int slot) {
    const int li = min(i, 63);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const size_t base =
          ((size_t)__builtin_amdgcn_readlane(voff_hi[hh], li) << 32) | __builtin_amdgcn_readlane(voff_lo[hh], li);
      const int nbytes = i < my_tiles ? (int)__builtin_amdgcn_readlane(vbytes[hh], li) : 0;
      const __amdgpu_buffer_rsrc_t kr =
          __builtin_amdgcn_make_buffer_rsrc((void *)(kpool + base), (short)0, nbytes, kBufferFlags);
      const __amdgpu_buffer_rsrc_t vr =
          __builtin_amdgcn_make_buffer_rsrc((void *)(vpool + base), (short)0, nbytes, kBufferFlags);
      char *kst = wave_stage + slot * kSlot + hh * kHalfB;
#pragma unroll
      for (int k = 0; k < kDmaH; ++k) dma16_to_lds(kr, kst + 1024 * k, dma_voff[k]);
#pragma unroll
      for (int k = 0; k < kDmaH; ++k) dma16_to_lds(vr, kst + kTileB + 1024 * k, dma_voff[k]);
    }
  };
  // Staged row R of a tile carries the swizzle of its position in its half.
  // The operand layouts are partial_prefill_kernel's.  fp8: K row pi(j32)
  // (bits 3 and 2 swapped within each 16), pieces 2 m + h2; V^T by 8-bit
  // transposing reads, lane 16 G + 2 r + c at row 16 t + 8 (G / 2) + r, dims
  // 32 sl + 16 (G % 2) + 8 c .. + 7.  bf16: K row j32, pieces 2 s + h2; V^T
  // by 16-bit transposing reads, lane 16 G + 4 r + c at row
  // 8 hh + 4 (G / 2) + r (+ 16 t), dims 32 sl + 16 (G % 2) + 4 c .. + 3.
  // INT4: K pieces 2 h2 and 2 h2 + 1 of row pi(j32) (dwords 8 h2 .. 8 h2 + 7);
  // V^T by 8-bit transposing reads per key half t and 64-dim block blk,
  // lane 16 G + 2 r + c at row 16 t + 8 (G / 2) + r, bytes
  // 32 blk + 16 (G % 2) + 8 c .. + 7, so lane j of a half-wave holds byte j
  // of the block (dims 2 j, 2 j + 1) for 8 consecutive keys.
  constexpr int kKReads = kFp8 ? 4 : (kInt4 ? 2 : 8);
  const int krow = kPerm ? (j32 & ~12) | ((j32 & 8) >> 1) | ((j32 & 4) << 1) : j32;
  uint32_t k_addr[kKReads], vt_addr[8];
  {
    const uint32_t base = lds_address(wave_stage);
#pragma unroll
    for (int m = 0; m < kKReads; ++m) {
      const int piece = kInt4 ? 2 * h2 + m : 2 * m + h2;
      k_addr[m] = base + krow * kRowBytes + ((piece ^ stage_swizzle<D, KT>(krow % kTile)) * 16);
    }
    const int G = lane >> 4;
    if constexpr (kInt4) {
      const int r = (lane >> 1) & 7, c = lane & 1;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
          const int row = 16 * t + 8 * (G >> 1) + r;
          const int piece = 2 * blk + (G & 1);
          vt_addr[2 * t + blk] =
              base + kTileB + row * kRowBytes + ((piece ^ stage_swizzle<D, KT>(row % kTile)) * 16) + c * 8;
        }
    } else if constexpr (kFp8) {
      const int r = (lane >> 1) & 7, c = lane & 1;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int sl = 0; sl < 4; ++sl) {
          const int row = 16 * t + 8 * (G >> 1) + r;
          const int piece = 2 * sl + (G & 1);
          vt_addr[4 * t + sl] =
              base + kTileB + row * kRowBytes + ((piece ^ stage_swizzle<D, KT>(row % kTile)) * 16) + c * 8;
        }
    } else {
      const int r = (lane >> 2) & 3, c = lane & 3;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int sl = 0; sl < 4; ++sl) {
          const int row = 8 * hh + 4 * (G >> 1) + r;
          const int piece = 4 * sl + 2 * (G & 1) + (c >> 1);
          vt_addr[4 * hh + sl] =
              base + kTileB + row * kRowBytes + ((piece ^ stage_swizzle<D, KT>(row % kTile)) * 16) + (c & 1) * 8;
        }
    }
  }
  const int vt_g = lane >> 4;

  // one staged 32-key tile (first key ts): its raw K pieces and the V^T
  // operands vop[t][sl] of key half t, whose element e holds key
  // 16 t + 8 (G / 2) + e (fp8) or 16 t + 8 (e / 4) + 4 (G / 2) + e % 4 (bf16)
  auto tile32 = [&](const uint4 (&kr)[kKReads], bf16x8_t (&vop)[2][4], int ts) {
    f32x16_t st;
#pragma unroll
    for (int v = 0; v < 16; ++v) st[v] = 0.0f;
    if constexpr (kInt4) { // dword s of the lane's 32 bytes, as 136 + n (even nibbles, then odd)
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const uint32_t x = dword_of(kr[s >> 2], s & 3);
        const uint32_t ev = int4_even(x), od = int4_odd(x);
        const bf16x8_t kop = __builtin_bit_cast(
            bf16x8_t, make_uint4(offset_bf16_lo(ev), offset_bf16_hi(ev), offset_bf16_lo(od), offset_bf16_hi(od)));
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[s], st, 0, 0, 0);
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) st[v] -= qoff;
    } else if constexpr (kFp8) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fp8x8_to_bf16x8(kr[m].x, kr[m].y), qop[2 * m], st, 0, 0, 0);
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fp8x8_to_bf16x8(kr[m].z, kr[m].w), qop[2 * m + 1], st, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int m = 0; m < 8; ++m)
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kr[m]), qop[m], st, 0, 0, 0);
    }
    // keys before w_lo are seen by no column (their values need not be
    // finite): zero their V^T elements; the tile's scores there are masked
    // (every INT4 code is finite)
    if (!kInt4 && ts < w_lo) { // uniform branch
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int key = ts + 16 * t + (kPerm ? 8 * (vt_g >> 1) + e : 8 * (e >> 2) + 4 * (vt_g >> 1) + (e & 3));
          if (key < w_lo) {
#pragma unroll
            for (int sl = 0; sl < 4; ++sl) vop[t][sl][e] = (__bf16)0.0f;
          }
        }
    }
    // ---- scores: register v holds key ts + pi(8 (v / 4) + 4 h2 + v % 4) ----
    float sv[16];
    if (capped) {
#pragma unroll
      for (int v = 0; v < 16; ++v) sv[v] = tanhf(st[v] * cscale) * cap_out;
    } else {
#pragma unroll
      for (int v = 0; v < 16; ++v) sv[v] = st[v];
    }
    if (ts < all_lo || ts + kT > all_hi) { // some column misses some key (uniform)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = 8 * (v >> 2) + 4 * h2 + (v & 3); // score row; fp8 / INT4: key pi(row)
        const int tok = ts + (kPerm ? (row & ~12) | ((row & 8) >> 1) | ((row & 4) << 1) : row);
        if (tok < c_lo || tok >= c_hi) sv[v] = -INFINITY;
      }
    }
    float mx = sv[0];
#pragma unroll
    for (int v = 1; v < 16; ++v) mx = fmaxf(mx, sv[v]);
    mx = xor32_max(mx) * ks;
    const bool empty = !seen; // not l_run == 0: the column's other lane may hold its keys so far
    const bool grow = mx > m_run + kLazy || (empty && mx != -INFINITY && mx < m_run - kDrop);
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float alpha = grow ? (empty ? 0.0f : __builtin_amdgcn_exp2f(m_run - mx)) : 1.0f;
      m_run = grow ? mx : m_run;
      l_run *= alpha;
      if constexpr (kInt4) lb_run *= alpha;
#pragma unroll
      for (int sl = 0; sl < 4; ++sl)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[sl][v] *= alpha;
    }
    seen = seen || mx != -INFINITY;
    const bool live = m_run != -INFINITY;
    uint32_t pk[8];
    float sum = 0.0f;
#pragma unroll
    for (int v = 0; v < 16; v += 2) {
      const float p0 = live ? __builtin_amdgcn_exp2f(fmaf(sv[v], ks, -m_run)) : 0.0f;
      const float p1 = live ? __builtin_amdgcn_exp2f(fmaf(sv[v + 1], ks, -m_run)) : 0.0f;
      sum += p0 + p1;
      pk[v / 2] = pack_bf16x2(p0, p1);
      if constexpr (kInt4) // the weights as the P.V product sees them
        lb_run += __uint_as_float(pk[v / 2] << 16) + __uint_as_float(pk[v / 2] & 0xFFFF0000u);
    }
    l_run += sum;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const bf16x8_t pt = __builtin_bit_cast(bf16x8_t, make_uint4(pk[4 * t], pk[4 * t + 1], pk[4 * t + 2], pk[4 * t + 3]));
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) acc[sl] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[t][sl], pt, acc[sl], 0, 0, 0);
    }
  };

  // ---- ring of NBUF slots per wave, refilled as soon as a tile is in registers ----
  if (my_tiles > 0) {
#pragma unroll
    for (int j = 0; j < NBUF; ++j) issue(j, j);
    const int n_iter = (my_tiles + NBUF - 1) / NBUF * NBUF;
    for (int it = 0; it < n_iter; it += NBUF) {
#pragma unroll
      for (int j = 0; j < NBUF; ++j) {
        const int i = it + j;
        wait_vmem<(NBUF - 1) * 4 * kDmaH>(); // tile i has landed; NBUF - 1 newer tiles may fly
        uint4 kr[kKReads];
        bf16x8_t vop[2][4];
        if constexpr (kInt4) { // operand (t, 2 blk + odd): even or odd nibbles of one read, as 136 + n
          uint2 vn[4];
          lds_read_k2(kr[0], kr[1], k_addr[0] + j * kSlot, k_addr[1] + j * kSlot);
          lds_read_tr8_x4(vn, *reinterpret_cast<const uint32_t(*)[4]>(&vt_addr[0]), j * kSlot);
          issue(i + NBUF, j);
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
              const uint2 x = vn[2 * t + blk];
              const uint32_t e0 = int4_even(x.x), e1 = int4_even(x.y), o0 = int4_odd(x.x), o1 = int4_odd(x.y);
              vop[t][2 * blk] = __builtin_bit_cast(
                  bf16x8_t, make_uint4(offset_bf16_lo(e0), offset_bf16_hi(e0), offset_bf16_lo(e1), offset_bf16_hi(e1)));
              vop[t][2 * blk + 1] = __builtin_bit_cast(
                  bf16x8_t, make_uint4(offset_bf16_lo(o0), offset_bf16_hi(o0), offset_bf16_lo(o1), offset_bf16_hi(o1)));
            }
        } else if constexpr (kFp8) {
          uint2 v8[8];
          lds_read_x4(kr, k_addr, j * kSlot);
          lds_read_tr8_x8(v8, vt_addr, j * kSlot);
          issue(i + NBUF, j);
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int sl = 0; sl < 4; ++sl) vop[t][sl] = fp8x8_to_bf16x8(v8[4 * t + sl].x, v8[4 * t + sl].y);
        } else { // operand (t, sl): two reads of four keys, key halves hh = 0, 1
          s16x4_t vt0[8], vt1[8];
          lds_read_x8(kr, k_addr, j * kSlot);
          lds_read_tr_x8(vt0, vt_addr, j * kSlot);
          lds_read_tr_x8(vt1, vt_addr, j * kSlot + kTile * kRowBytes);
          issue(i + NBUF, j);
#pragma unroll
          for (int sl = 0; sl < 4; ++sl) {
            const uint2 a0v = __builtin_bit_cast(uint2, vt0[sl]), c0v = __builtin_bit_cast(uint2, vt0[4 + sl]);
            const uint2 a1v = __builtin_bit_cast(uint2, vt1[sl]), c1v = __builtin_bit_cast(uint2, vt1[4 + sl]);
            vop[0][sl] = __builtin_bit_cast(bf16x8_t, make_uint4(a0v.x, a0v.y, c0v.x, c0v.y));
            vop[1][sl] = __builtin_bit_cast(bf16x8_t, make_uint4(a1v.x, a1v.y, c1v.x, c1v.y));
          }
        }
        if (i < my_tiles) tile32(kr, vop, a0 + (ft + wave + i * kWaves) * kT);
      }
    }
    wait_vmem<0>(); // no DMA may land in the staging area once it is reused
  }
  __syncthreads(); // staging area is reused for the per-wave states below

  // ---- per-wave states to LDS, merged over the waves, one column group at a time ----
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  // INT4: V entered the product as 136 + n; remove 136 * (sum of the weights it saw)
  const float voff = kInt4 ? kInt4Offset * (lb_run + __shfl_xor(lb_run, 32, 64)) : 0.0f;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    if (c > 0) {
      if ((cg0 + 1) * 16 >= nq * g) break; // the same in every lane of the workgroup
      __syncthreads();                      // the previous group's merge has read the states
    }
    if ((j32 >> 4) == c) {
      const int h = j32 & 15;
      if (h2 == 0) {
        sm_m[wave][h] = l_tot > 0.0f ? m_run : -INFINITY; // an empty state keeps no reference
        sm_l[wave][h] = l_tot;
      }
      float *dst = sm_o + (wave * 16 + h) * OSTRIDE;
      if constexpr (kInt4) {
#pragma unroll
        for (int sl = 0; sl < 4; ++sl)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            dst[64 * (sl >> 1) + 2 * (8 * (v >> 2) + 4 * h2 + (v & 3)) + (sl & 1)] = acc[sl][v] - voff;
      } else {
#pragma unroll
        for (int sl = 0; sl < 4; ++sl)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *reinterpret_cast<float4 *>(dst + 32 * sl + 8 * q + 4 * h2) =
                make_float4(acc[sl][4 * q], acc[sl][4 * q + 1], acc[sl][4 * q + 2], acc[sl][4 * q + 3]);
      }
    }
    __syncthreads();
    // bf16 caches: split partials stored as row-scaled fp16 when the host asks
    merge_waves_and_store<D, OSTRIDE, KT == DT_BF16>(p, sm_m, sm_l, sm_o, b, kvg, cg0 + c, item, nb);
  }
  finish_split<D, 1, kFusedMergeBatch, KT == DT_BF16>(p, blockIdx.y, b, kvg, cg0, 2, item, split, nb, smem);
}

// Column groups one wave of the shared-tile kernel computes: two for
// head_dim <= 128; head_dim 256 keeps one, its accumulators would not fit in
// registers twice.
template <int D>
constexpr int rows_cg() { return D <= 128 ? 2 : 1; }

// Block slots of the shared-tile kernel: about 64 KB of LDS per workgroup
// (two workgroups per CU), two to four slots.
template <int D, int KT>
constexpr int rows_nbuf() {
  constexpr int slot = kWaves * 2 * Shape<D, KT>::kTileBytes;
  return 65536 / slot < 2 ? 2 : (65536 / slot > 4 ? 4 : 65536 / slot);
}

} // namespace

// Column groups from which several query rows per request go to the
// shared-tile kernel.  Below 8 groups some of its waves idle; that pays for
// bf16, whose second read of the keys costs more than the idle waves, from 3
// groups on, but for the compute-heavier fp8 and INT4 tiles only once three
// of the four waves have work (batch-128 fp8, 8 rows of 8 heads = 4 groups:
// 656 us with the chunk-splitting kernel, 980 us shared-tile).  At head_dim
// 256 a workgroup covers 4 groups, one per wave, so fp8 and INT4 there take
// it from 3 groups too (batch-128 fp8 at head_dim 256, 8 rows: 904 us,
// against 2059 us chunk-splitting and 962 us on the 32x32 kernel, whose wave
// pairs convert every K code twice; INT4, 6 and 8 rows: 751 and 781 us
// against 874 and 1128 us chunk-splitting).  INT4 at head_dim 128 keeps 5
// groups on the 32x32 kernel as well (batch-128, 6 and 8 rows: 510 and
// 537 us on the 32-column kernel, 557 and 559 us on the 32x32 one).
constexpr int kRowsMinGroupsBf16 = 3;
constexpr int kRowsMinGroupsQuant = 5;

// Column groups of (query row, head) pairs one partial workgroup computes
// (several query rows per request).  Two: the chunk-splitting kernel runs
// both on each staged tile (head_dim <= 128), halving the K/V reads of short
// appends.  From three groups on: the shared-tile kernel, whose workgroup
// covers 8 groups (head_dim <= 128) or 4 (256) and reads the keys once for
// all of them.
int mfma_col_share(int head_dim, int kv_type, int col_groups) {
  // bf16, fp8 and INT4 at head_dim 128 (bf16 at 256 too) take the 32x32
  // prefill kernel there; bf16 and fp8 at 128 from 3 groups
  const bool tiles32 = head_dim == 128 && (kv_type == DT_BF16 || kv_type == DT_FP8);
  const bool quant_wide = (kv_type == DT_FP8 || kv_type == DT_INT4) && head_dim == 256;
  if (col_groups >= (kv_type == DT_BF16 || tiles32 || quant_wide ? kRowsMinGroupsBf16 : kRowsMinGroupsQuant))
    return kWaves * (head_dim <= 128 ? 2 : 1);
  return col_groups >= 2 && head_dim <= 128 ? 2 : 1;
}

template <int D, int KT>
static hipError_t launch_rows_d(const Params &p, const InlineWork &w, const Launch &l) {
  constexpr int kGroups = kWaves * rows_cg<D>();
  if (p.col_share != kGroups || p.pack != 1) return hipErrorInvalidValue;
  const dim3 grid(p.items, p.num_kv_heads * ((p.col_groups + kGroups - 1) / kGroups));
  if constexpr ((D == 128 && (KT == DT_BF16 || KT == DT_FP8 || KT == DT_INT4)) || (D == 256 && KT == DT_BF16))
    return launch_kernel(l, partial_prefill_kernel<D, KT, KT == DT_INT4 ? 8 : (KT == DT_FP8 ? 4 : 2)>, grid, p, w);
  return launch_kernel(l, partial_rows_kernel<D, KT, rows_nbuf<D, KT>(), rows_cg<D>()>, grid, p, w);
}

hipError_t launch_cols32(const Params &p, const InlineWork &w, int kv_type, const Launch &l) {
  if (p.col_share != 2 || p.pack != 1 || (p.part_row_scale && kv_type != DT_BF16)) return hipErrorInvalidValue;
  const dim3 grid(p.items, p.num_kv_heads * ((p.col_groups + 1) / 2));
  // one 16 KB bf16 slot per wave, two 8 KB fp8 ones, four 4 KB INT4 ones: 64 KB per workgroup
  if (kv_type == DT_FP8) return launch_kernel(l, partial_cols32_kernel<DT_FP8, 2>, grid, p, w);
  if (kv_type == DT_BF16) return launch_kernel(l, partial_cols32_kernel<DT_BF16, 1>, grid, p, w);
  if (kv_type == DT_INT4) return launch_kernel(l, partial_cols32_kernel<DT_INT4, 4>, grid, p, w);
  return hipErrorInvalidValue;
}

bool rows_merge_in_kernel(int head_dim, int kv_type) { return rows_merges_in_kernel(head_dim, kv_type); }

hipError_t launch_partial_rows(const Params &p, const InlineWork &w, int head_dim, int kv_type, const Launch &l) {
  // row-scaled partials: only the 32x32 prefill kernel (bf16 at head_dim 128 and 256) writes them
  if (p.part_row_scale && !(kv_type == DT_BF16 && head_dim >= 128)) return hipErrorInvalidValue;
  if (kv_type == DT_INT4) {
    if (head_dim == 128) return launch_rows_d<128, DT_INT4>(p, w, l);
    if (head_dim == 256) return launch_rows_d<256, DT_INT4>(p, w, l);
    return hipErrorInvalidValue;
  }
  const bool fp8 = kv_type == DT_FP8;
  switch (head_dim) {
  case 64: return fp8 ? launch_rows_d<64, DT_FP8>(p, w, l) : launch_rows_d<64, DT_BF16>(p, w, l);
  case 128: return fp8 ? launch_rows_d<128, DT_FP8>(p, w, l) : launch_rows_d<128, DT_BF16>(p, w, l);
  case 256: return fp8 ? launch_rows_d<256, DT_FP8>(p, w, l) : launch_rows_d<256, DT_BF16>(p, w, l);
  default: return hipErrorInvalidValue;
  }
}

} // namespace kvs
