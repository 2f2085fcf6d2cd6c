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
//     it straight from LDS with transposing reads; otherwise the V tile is
//     multiplied by an identity (bf16, INT4: 16x16x16) or by a 0/1 selection
//     (fp8, 16x16x32 fp8, which also decodes the codes exactly into fp32).
//   * O^T[dim][query head] += V^T . P^T with v_mfma_f32_16x16x16_bf16; lane
//     keeps four consecutive dims per 16-dim slice w (see out_dim) of query
//     head c16, so the running max, sum and rescale of a head never leave its
//     lane; dims of the other KV head of the pack are dropped at the end.
// The first product, the online update and the rescaled accumulation follow
// the tiled online softmax of "Forcing Flash Attention onto TPU", section
// "Flash Attention in JAX"; chunk results are merged by log-sum-exp (FlashDecoding++
// explainer, asynchronous-softmax section: partial softmax per tile, then an
// update with the previous max and sum).
//
// Several query rows per request turn the columns into (query row, head)
// pairs.  Up to two groups of 16 such columns run in the kernel above (both
// on each staged tile); from three groups on, partial_rows_kernel (further
// down) lets its four waves share each staged tile instead of splitting the
// keys, so a workgroup reads the keys once for 128 columns.
#include "kvs_device.h"

namespace kvs {
namespace {

template <int DE, int KT>
struct Shape {
  static_assert(KT == DT_BF16 || KT == DT_FP8 || KT == DT_INT4, "KV type");
  static constexpr int kEpp = KT == DT_BF16 ? 8 : (KT == DT_FP8 ? 16 : 32); // elements per 16-byte piece
  static constexpr int kRowBytes = DE * 16 / kEpp;        // one token's K (or V) row of the pack
  static constexpr int kLaneVec = kRowBytes / 64;          // 16-byte pieces per lane per row
  static constexpr int kKSteps = DE / 32;                  // 16x16x32 products for S^T
  static constexpr int kOTiles = DE / 16;                  // 16-dim slices of O^T
  static constexpr int kOutStride = KT == DT_INT4 ? 2 : 1; // distance between a lane's four O^T dims
  static_assert(kLaneVec >= 1, "row slice must hold at least 16 bytes");
  // LDS staging of a 16-token tile
  static constexpr int kPieces = kRowBytes / 16;           // 16-byte pieces per row
  static constexpr int kRowsPerDma = 1024 / kRowBytes;     // rows one 64-lane x 16-byte load covers
  static constexpr int kDma = kTile * kRowBytes / 1024;    // loads per tile (K or V)
  static constexpr int kTileBytes = kTile * kRowBytes;     // K (or V) bytes of a tile
  static constexpr int kRowsPerBankPeriod = kRowBytes >= 256 ? 1 : 256 / kRowBytes;
  // tiles staged per wave: about 12 KB of K+V in LDS per wave (three
  // workgroups per CU for fp8 head_dim 128), two to eight
  static constexpr int kFit = 12288 / (2 * kTileBytes);
  static constexpr int kNBuf = kFit < 2 ? 2 : (kFit > 8 ? 8 : kFit);
};

// Word 3 of a raw buffer descriptor on CDNA (gfx9 family): 32-bit data format,
// no swizzling; with stride 0 the size field is a byte count and lanes whose
// offset falls outside it read zero.
constexpr int kBufferFlags = 0x00020000;
// Cache policy of the K/V loads: non-temporal.  Every K/V byte is read once
// per call, and streaming loads measured about 10% more HBM bandwidth than
// default-policy loads on MI355X (6.7 vs 6.0 TB/s on a plain read).
constexpr int kKvLoadPolicy = 2;
// Largest rise of a head's running max (log2 units) absorbed without a
// rescale of its state; weights then stay below 2^8.
constexpr float kLazy = 8.0f;
// A starting reference this far (log2 units) above an empty state's first
// tile max is moved down to it.
constexpr float kDrop = 64.0f;

// XOR swizzle of the 16-byte pieces of staged row r: the 16 rows a matrix
// operand reads at the same logical piece land in distinct LDS banks.
template <int DE, int KT>
__device__ __forceinline__ int stage_swizzle(int r) {
  using S = Shape<DE, KT>;
  return (r / S::kRowsPerBankPeriod) & (S::kPieces - 1);
}

// Wait until at most N vector-memory operations of this wave are in flight
// (LDS DMA loads included); nothing else is waited for.  The compiler does
// not order LDS reads after the DMA that fills them, so the staged-tile reads
// follow this explicit wait and a compiler barrier.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
  __asm__ volatile("" ::: "memory");
}

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_address(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)p;
}

// Reads of a staged tile.  Each asm block issues the K and V pieces at one or
// two lane addresses (V sits VOFF bytes after K) and waits for them
// (lgkmcnt 0) before it ends, so the registers are complete when the block
// returns and the slot may be refilled at once.  Written out because the
// compiler's own wait insertion cannot tell, across the main loop's back edge,
// which DMA load filled which slot, and would otherwise drain every load in
// flight there; the explicit vmcnt wait before each read orders DMA and read.
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
template <int VOFF>
__device__ __forceinline__ void lds_read_kv1(uint4 &k0, uint4 &v0, uint32_t a0) {
  u32x4_t rk0, rv0;
  __asm__ volatile("ds_read_b128 %0, %2\n\t"
                   "ds_read_b128 %1, %2 offset:%3\n\t"
                   "s_waitcnt lgkmcnt(0)"
                   : "=&v"(rk0), "=&v"(rv0)
                   : "v"(a0), "i"(VOFF)
                   : "memory");
  k0 = __builtin_bit_cast(uint4, rk0);
  v0 = __builtin_bit_cast(uint4, rv0);
}
template <int VOFF>
__device__ __forceinline__ void lds_read_kv2(uint4 &k0, uint4 &v0, uint4 &k1, uint4 &v1, uint32_t a0, uint32_t a1) {
  u32x4_t rk0, rv0, rk1, rv1;
  __asm__ volatile("ds_read_b128 %0, %4\n\t"
                   "ds_read_b128 %1, %4 offset:%6\n\t"
                   "ds_read_b128 %2, %5\n\t"
                   "ds_read_b128 %3, %5 offset:%6\n\t"
                   "s_waitcnt lgkmcnt(0)"
                   : "=&v"(rk0), "=&v"(rv0), "=&v"(rk1), "=&v"(rv1)
                   : "v"(a0), "v"(a1), "i"(VOFF)
                   : "memory");
  k0 = __builtin_bit_cast(uint4, rk0);
  v0 = __builtin_bit_cast(uint4, rv0);
  k1 = __builtin_bit_cast(uint4, rk1);
  v1 = __builtin_bit_cast(uint4, rv1);
}

// One 16-byte-per-lane DMA load from a buffer into LDS: lane i's bytes land
// at lds + 16 * i.  (Kept out of the kernel body: the host compilation pass
// must not see the LDS address-space cast.)
__device__ __forceinline__ void dma16_to_lds(__amdgpu_buffer_rsrc_t r, char *lds, int voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16, voffset, 0, 0,
                                           kKvLoadPolicy);
}

// bf16 tiles up to 128 pack dims take V^T straight from LDS (transposing
// reads); wider ones, fp8 and INT4 transpose V with a matrix product.  At
// head_dim 256 the transposed slices, read together with K, held registers
// the pair-wise prefill kernel needed (8192-row prefill: 147 against 158
// TFLOP/s); at head_dim 128 they gained (2048 rows on a 32k cache: 499
// against 480 TFLOP/s), decode unchanged.
template <int DE, int KT>
constexpr bool vt_from_lds() { return KT == DT_BF16 && DE <= 128; }

template <int DE, int KT>
struct TileRegs {
  uint4 k[Shape<DE, KT>::kLaneVec];    // K pieces 4 * pc + q4 of row c16
  uint4 v[Shape<DE, KT>::kLaneVec];    // V pieces (fp8, INT4)
  s16x4_t vt[Shape<DE, KT>::kOTiles];  // V^T slices read transposed from LDS (vt_from_lds)
};

// Transposing LDS reads (gfx950 ds_read_b64_tr_b16): within each 16-lane
// group, lane i receives 16-bit element i % 4 of the 8 bytes addressed by
// lane 4 r + i / 4, for r = 0..3.  Four V^T slices per block (two lane
// addresses, each with a second slice 8 bytes further), waited for inside
// the block like the other staged reads.
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void lds_read_vt4(s16x4_t &v0, s16x4_t &v1, s16x4_t &v2, s16x4_t &v3, uint32_t a0,
                                             uint32_t a1) {
  u32x2_t r0, r1, r2, r3;
  __asm__ volatile("ds_read_b64_tr_b16 %0, %4\n\t"
                   "ds_read_b64_tr_b16 %1, %4 offset:8\n\t"
                   "ds_read_b64_tr_b16 %2, %5\n\t"
                   "ds_read_b64_tr_b16 %3, %5 offset:8\n\t"
                   "s_waitcnt lgkmcnt(0)"
                   : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
                   : "v"(a0), "v"(a1)
                   : "memory");
  v0 = __builtin_bit_cast(s16x4_t, r0);
  v1 = __builtin_bit_cast(s16x4_t, r1);
  v2 = __builtin_bit_cast(s16x4_t, r2);
  v3 = __builtin_bit_cast(s16x4_t, r3);
}
// Eight 16-byte reads at eight lane addresses, one wait
__device__ __forceinline__ void lds_read_x8(uint4 (&k)[8], const uint32_t (&a)[8], uint32_t off) {
  u32x4_t r0, r1, r2, r3, r4, r5, r6, r7;
  __asm__ volatile("ds_read_b128 %0, %8\n\t"
                   "ds_read_b128 %1, %9\n\t"
                   "ds_read_b128 %2, %10\n\t"
                   "ds_read_b128 %3, %11\n\t"
                   "ds_read_b128 %4, %12\n\t"
                   "ds_read_b128 %5, %13\n\t"
                   "ds_read_b128 %6, %14\n\t"
                   "ds_read_b128 %7, %15\n\t"
                   "s_waitcnt lgkmcnt(0)"
                   : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6), "=&v"(r7)
                   : "v"(a[0] + off), "v"(a[1] + off), "v"(a[2] + off), "v"(a[3] + off), "v"(a[4] + off),
                     "v"(a[5] + off), "v"(a[6] + off), "v"(a[7] + off)
                   : "memory");
  k[0] = __builtin_bit_cast(uint4, r0);
  k[1] = __builtin_bit_cast(uint4, r1);
  k[2] = __builtin_bit_cast(uint4, r2);
  k[3] = __builtin_bit_cast(uint4, r3);
  k[4] = __builtin_bit_cast(uint4, r4);
  k[5] = __builtin_bit_cast(uint4, r5);
  k[6] = __builtin_bit_cast(uint4, r6);
  k[7] = __builtin_bit_cast(uint4, r7);
}
// Eight transposing reads at eight lane addresses, one wait
__device__ __forceinline__ void lds_read_tr_x8(s16x4_t (&v)[8], const uint32_t (&a)[8], uint32_t off) {
  u32x2_t r0, r1, r2, r3, r4, r5, r6, r7;
  __asm__ volatile("ds_read_b64_tr_b16 %0, %8\n\t"
                   "ds_read_b64_tr_b16 %1, %9\n\t"
                   "ds_read_b64_tr_b16 %2, %10\n\t"
                   "ds_read_b64_tr_b16 %3, %11\n\t"
                   "ds_read_b64_tr_b16 %4, %12\n\t"
                   "ds_read_b64_tr_b16 %5, %13\n\t"
                   "ds_read_b64_tr_b16 %6, %14\n\t"
                   "ds_read_b64_tr_b16 %7, %15\n\t"
                   "s_waitcnt lgkmcnt(0)"
                   : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6), "=&v"(r7)
                   : "v"(a[0] + off), "v"(a[1] + off), "v"(a[2] + off), "v"(a[3] + off), "v"(a[4] + off),
                     "v"(a[5] + off), "v"(a[6] + off), "v"(a[7] + off)
                   : "memory");
  v[0] = __builtin_bit_cast(s16x4_t, r0);
  v[1] = __builtin_bit_cast(s16x4_t, r1);
  v[2] = __builtin_bit_cast(s16x4_t, r2);
  v[3] = __builtin_bit_cast(s16x4_t, r3);
  v[4] = __builtin_bit_cast(s16x4_t, r4);
  v[5] = __builtin_bit_cast(s16x4_t, r5);
  v[6] = __builtin_bit_cast(s16x4_t, r6);
  v[7] = __builtin_bit_cast(s16x4_t, r7);
}
// K pieces only (two per block)
__device__ __forceinline__ void lds_read_k2(uint4 &k0, uint4 &k1, uint32_t a0, uint32_t a1) {
  u32x4_t r0, r1;
  __asm__ volatile("ds_read_b128 %0, %2\n\t"
                   "ds_read_b128 %1, %3\n\t"
                   "s_waitcnt lgkmcnt(0)"
                   : "=&v"(r0), "=&v"(r1)
                   : "v"(a0), "v"(a1)
                   : "memory");
  k0 = __builtin_bit_cast(uint4, r0);
  k1 = __builtin_bit_cast(uint4, r1);
}

// Lane addresses of a staged tile (K rows, then V rows kTileBytes further;
// 16-byte pieces XOR-swizzled per row) and the reads that turn it into the
// operand registers of lane (c16, q4).  K (and fp8 / INT4 V): pieces 4 pc + q4
// of row c16.  bf16 V: V^T slice w straight from LDS with transposing reads;
// lane 16 q4 + 4 r + c points at the four dims of slice w that output rows
// 4 c .. 4 c + 3 hold (out_dim) in token row 4 q4 + r, so lane (i, q4) gets
// keys 4 q4 .. 4 q4 + 3 of dim row i, the A-operand layout of the P.V product.
template <int DE, int KT>
struct StageReader {
  using S = Shape<DE, KT>;
  static constexpr bool kVt = vt_from_lds<DE, KT>();
  static constexpr int kVtAddr = kVt ? S::kOTiles / 2 : 1;
  uint32_t k_addr[S::kLaneVec];
  uint32_t vt_addr[kVtAddr];
  __device__ __forceinline__ void init(uint32_t tile0, int lane) {
    const int c16 = lane & 15, q4 = lane >> 4;
    const int swz = stage_swizzle<DE, KT>(c16);
#pragma unroll
    for (int pc = 0; pc < S::kLaneVec; ++pc)
      k_addr[pc] = tile0 + c16 * S::kRowBytes + ((4 * pc + q4) ^ swz) * 16;
    if constexpr (kVt) {
      const int r = (lane >> 2) & 3, c = lane & 3;
      const int row = 4 * q4 + r;
      const int vswz = stage_swizzle<DE, KT>(row);
#pragma unroll
      for (int h = 0; h < kVtAddr; ++h) {
        // slices 2 h and 2 h + 1: source piece 4 h + c, bytes 0 and 8 of it
        vt_addr[h] = tile0 + S::kTileBytes + row * S::kRowBytes + ((4 * h + c) ^ vswz) * 16;
      }
    }
  }
  // t <- the tile whose K rows start `off` bytes after tile0 (reads complete on return)
  __device__ __forceinline__ void read(TileRegs<DE, KT> &t, uint32_t off) const {
    if constexpr (kVt) {
#pragma unroll
      for (int pc = 0; pc < S::kLaneVec; pc += 2) lds_read_k2(t.k[pc], t.k[pc + 1], k_addr[pc] + off, k_addr[pc + 1] + off);
#pragma unroll
      for (int h = 0; h < kVtAddr; h += 2)
        lds_read_vt4(t.vt[2 * h], t.vt[2 * h + 1], t.vt[2 * h + 2], t.vt[2 * h + 3], vt_addr[h] + off,
                     vt_addr[h + 1] + off);
    } else if constexpr (S::kLaneVec == 1) {
      lds_read_kv1<S::kTileBytes>(t.k[0], t.v[0], k_addr[0] + off);
    } else {
#pragma unroll
      for (int pc = 0; pc < S::kLaneVec; pc += 2)
        lds_read_kv2<S::kTileBytes>(t.k[pc], t.v[pc], t.k[pc + 1], t.v[pc + 1], k_addr[pc] + off,
                                    k_addr[pc + 1] + off);
    }
  }
};

// Max of x over lanes l and l ^ 16 (l ^ 32) with gfx950's lane swaps: swapping
// the odd 16-lane rows of one copy of x with the even rows of another (the
// upper 32 lanes of one with the lower 32 of the other) leaves each lane the
// two values whose max it needs.  VALU instructions, where a lane shuffle
// would go through the LDS unit and wait for it.
__device__ __forceinline__ float xor16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// 8 consecutive fp8 codes (two dwords) -> 8 bf16 (exact).
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
  bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  bf16x8_t r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  return r;
}

// INT4: a dword holds 8 two's-complement nibbles n (element 2i in the low
// nibble of byte i).  n ^ 8 = n + 8 lies in [0, 15], and the bf16 pattern
// 0x43 : (n + 8) is exactly 128 + (n + 8) = n + 136, so one byte permute
// builds two bf16 operands.  The products then carry an offset of 136 per
// element, removed exactly afterwards (scores: 136 * sum of q over the head's
// dims; outputs: 136 * the softmax sum).  kInt4Offset is that 136.
constexpr float kInt4Offset = 136.0f;
__device__ __forceinline__ uint32_t int4_even(uint32_t w) { return (w ^ 0x88888888u) & 0x0F0F0F0Fu; }
__device__ __forceinline__ uint32_t int4_odd(uint32_t w) { return ((w ^ 0x88888888u) >> 4) & 0x0F0F0F0Fu; }
// bytes b0..b3 of x (each in [0, 15]) -> bf16 (128 + b0, 128 + b1), (128 + b2, 128 + b3)
__device__ __forceinline__ uint32_t offset_bf16_lo(uint32_t x) { return __builtin_amdgcn_perm(0x43434343u, x, 0x04010400u); }
__device__ __forceinline__ uint32_t offset_bf16_hi(uint32_t x) { return __builtin_amdgcn_perm(0x43434343u, x, 0x04030402u); }

// Pack dim of element e (0..7) that lane (q4) feeds to the S^T product in
// k-step j (16x16x32: 8 reduction indices per lane).  INT4 feeds the even
// elements of a dword first, then the odd ones.
template <int DE, int KT>
__device__ __forceinline__ int k_elem_dim(int j, int q4, int e) {
  if constexpr (KT == DT_FP8) {
    return 16 * (4 * (j >> 1) + q4) + 8 * (j & 1) + e;
  } else if constexpr (KT == DT_INT4) {
    const int pc = j >> 2, dw = j & 3; // piece 4 pc + q4, dword dw of it
    return 32 * (4 * pc + q4) + 8 * dw + (e < 4 ? 2 * e : 2 * (e - 4) + 1);
  } else {
    return 8 * (4 * j + q4) + e;
  }
}

// First of the four pack dims lane (q4) holds in O^T slice w; the four are
// kOutStride apart.
template <int DE, int KT>
__device__ __forceinline__ int out_dim(int w, int q4) {
  if constexpr (KT == DT_INT4) {
    const int pc = w >> 3, dw = (w & 7) >> 1; // slice w: the even (w even) or odd nibbles of dword dw
    return 32 * (4 * pc + q4) + 8 * dw + (w & 1);
  } else {
    constexpr int per_piece = Shape<DE, KT>::kEpp / 4; // slices per 16-byte piece
    return (4 * (w / per_piece) + q4) * Shape<DE, KT>::kEpp + 4 * (w % per_piece);
  }
}

__device__ __forceinline__ uint32_t dword_of(const uint4 &v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

template <int DE, int KT>
__device__ __forceinline__ bf16x8_t k_operand(const TileRegs<DE, KT> &t, int j) {
  if constexpr (KT == DT_FP8) {
    const uint4 w = t.k[j >> 1];
    return (j & 1) ? fp8x8_to_bf16x8(w.z, w.w) : fp8x8_to_bf16x8(w.x, w.y);
  } else if constexpr (KT == DT_INT4) {
    const uint32_t w = dword_of(t.k[j >> 2], j & 3);
    const uint32_t ev = int4_even(w), od = int4_odd(w);
    return __builtin_bit_cast(bf16x8_t, make_uint4(offset_bf16_lo(ev), offset_bf16_hi(ev), offset_bf16_lo(od),
                                                   offset_bf16_hi(od)));
  } else {
    return __builtin_bit_cast(bf16x8_t, t.k[j]);
  }
}

// Which (request b, split) work item `item` is, with the request's split
// count nb and length L: from the host-planned list, else by a scan of the
// device lengths (which also records each request's first item and split
// count for the merge).  Returns false, the same in every thread, when the
// device lengths disagree with the planned launch.  Every thread calls it.
__device__ __forceinline__ bool locate_item(const Params &p, const InlineWork &w, int item, int *s_scan, int *s_item,
                                            int &b, int &split, int &nb, int &L) {
  if (w.n_items > 0) { // planned on the host
    const uint32_t e = w.item[item];
    b = (int)(e >> 16);
    split = (int)(e & 0xFFFF);
    L = w.req_len[b];
    nb = num_splits(L, req_nq(p, b), p.window, p.chunk);
    return true;
  }
  if (threadIdx.x == 0) s_item[0] = -1;
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
  if (b < 0) return false;
  if (p.meta && split == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
    p.meta[2 * b] = s_item[3];
    p.meta[2 * b + 1] = nb;
  }
  L = p.kv_len[b];
  return true;
}

// Operands of the V transposition for lane (c16, q4): a bf16 identity
// (16x16x16 products) and, for fp8, 0/1 selections of one code per
// 16x16x32 product (the fp8 pattern 0x38 is 1.0).
template <int KT>
__device__ __forceinline__ void transpose_operands(int c16, int q4, s16x4_t &ident, long (&sel)[2]) {
  const short one_bf16 = 0x3F80;
#pragma unroll
  for (int e = 0; e < 4; ++e) ident[e] = (4 * q4 + e == c16) ? one_bf16 : (short)0;
  sel[0] = sel[1] = 0;
  if (KT == DT_FP8) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      uint64_t s = 0;
      if (q4 == (c16 >> 2)) s = (uint64_t)0x38 << (8 * (4 * hh + (c16 & 3)));
      sel[hh] = (long)s;
    }
  }
}

// ---- column groups: per-lane state shared by the two partial kernels ----
// A wave computes CG groups of 16 matrix columns; lane (c16, q4) holds column
// c16 of every group.  A column is a query head of the pack (one query per
// request) or a (query row, head) pair (several rows per request).
template <int DE, int KT, int CG>
struct ColumnSet {
  using S = Shape<DE, KT>;
  bf16x8_t q[CG][S::kKSteps]; // Q^T operand, zero where the column sees no dims
  float qoff[CG];             // INT4: the scores carry 136 * (sum of the column's q)
  bool ok[CG];                // the lane's column holds a (query, head) of the request
  bool on[CG];                // the group holds any (the same in every lane)
  int row[CG], head[CG];      // q / o row and query head of the lane's column
  int lo[CG], hi[CG];         // keys of the chunk the lane's column sees
  float m[CG];                // reference max, log2 domain (the same in the 4 quarters)
  float l[CG];                // partial sum over the lane's tokens
  float lb[CG];               // INT4: the same sum of the bf16-rounded weights P.V saw
  f32x4_t acc[CG][S::kOTiles];
};

// Which (query, head) each lane's column is, and the keys of [t_begin,
// t_end) it sees: up to its query's position, the last `window` of them.
// cg0: the set's first column group; gp: query heads per pack.
template <int DE, int KT, int CG>
__device__ __forceinline__ void set_columns(ColumnSet<DE, KT, CG> &cs, const Params &p, int b, int L, int nq,
                                            int kvg, int cg0, int gp, int t_begin, int t_end, int c16) {
  const int g = p.group;
#pragma unroll
  for (int c = 0; c < CG; ++c) {
    int qi; // query index within the request (0 with one query)
    if (!p.qo_indptr) {
      cs.ok[c] = c16 < gp;
      cs.on[c] = true;
      qi = 0;
      cs.row[c] = b;
      cs.head[c] = kvg * gp + c16;
    } else {
      const int col = (cg0 + c) * 16 + c16;
      cs.ok[c] = col < nq * g;
      cs.on[c] = (cg0 + c) * 16 < nq * g;
      qi = col / g;
      cs.row[c] = p.qo_indptr[b] + qi;
      cs.head[c] = kvg * g + col % g;
    }
    const int qpos = L - nq + qi;
    const int col_lo = p.window > 0 ? max(0, qpos - p.window + 1) : 0;
    cs.lo[c] = max(t_begin, col_lo);
    cs.hi[c] = min(t_end, qpos + 1);
  }
}

// Keys every column of the set sees, [all_lo, all_hi) (tiles inside need no
// per-key mask), and keys some column sees, [any_lo, any_hi); uniform.
template <int DE, int KT, int CG>
__device__ __forceinline__ void column_ranges(const ColumnSet<DE, KT, CG> &cs, int t_begin, int t_end, int &all_lo,
                                              int &all_hi, int &any_lo, int &any_hi) {
  all_lo = t_begin;
  all_hi = t_end;
  any_lo = t_end;
  any_hi = t_begin;
#pragma unroll
  for (int c = 0; c < CG; ++c) {
    if (cs.ok[c]) {
      all_lo = max(all_lo, cs.lo[c]);
      all_hi = min(all_hi, cs.hi[c]);
      if (cs.lo[c] < cs.hi[c]) {
        any_lo = min(any_lo, cs.lo[c]);
        any_hi = max(any_hi, cs.hi[c]);
      }
    }
  }
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) {
    all_lo = max(all_lo, __shfl_xor(all_lo, o, 64));
    all_hi = min(all_hi, __shfl_xor(all_hi, o, 64));
    any_lo = min(any_lo, __shfl_xor(any_lo, o, 64));
    any_hi = max(any_hi, __shfl_xor(any_hi, o, 64));
  }
  all_lo = __builtin_amdgcn_readfirstlane(all_lo);
  all_hi = __builtin_amdgcn_readfirstlane(all_hi);
  any_lo = __builtin_amdgcn_readfirstlane(any_lo);
  any_hi = __builtin_amdgcn_readfirstlane(any_hi);
}

// Q^T operand of each group (block diagonal over the pack: column c16 only
// sees the dims of its own KV head my_kv), its INT4 offset, and an empty
// softmax state starting from the reference max m_init.
template <int D, int DE, int KT, int CG>
__device__ __forceinline__ void load_columns(ColumnSet<DE, KT, CG> &cs, const Params &p, int q4, int my_kv) {
  using S = Shape<DE, KT>;
#pragma unroll
  for (int c = 0; c < CG; ++c) {
    const uint16_t *qb =
        reinterpret_cast<const uint16_t *>(p.q) + ((size_t)cs.row[c] * p.num_qo_heads + cs.head[c]) * D;
#pragma unroll
    for (int j = 0; j < S::kKSteps; ++j) {
      const int kd = k_elem_dim<DE, KT>(j, q4, 0); // the k-step's 8 dims are kd .. kd + 7
      if (cs.ok[c] && kd / D == my_kv) {
        bf16x8_t x = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(qb + (kd % D)));
        if constexpr (KT == DT_INT4) x = __builtin_shufflevector(x, x, 0, 2, 4, 6, 1, 3, 5, 7);
        cs.q[c][j] = x;
      } else {
        cs.q[c][j] = __builtin_bit_cast(bf16x8_t, make_uint4(0, 0, 0, 0));
      }
    }
    cs.qoff[c] = 0.0f;
    if constexpr (KT == DT_INT4) {
#pragma unroll
      for (int j = 0; j < S::kKSteps; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) cs.qoff[c] += (float)cs.q[c][j][e];
      cs.qoff[c] += __shfl_xor(cs.qoff[c], 16, 64);
      cs.qoff[c] += __shfl_xor(cs.qoff[c], 32, 64);
      cs.qoff[c] *= kInt4Offset;
    }
    cs.m[c] = p.m_init;
    cs.l[c] = 0.0f;
    cs.lb[c] = 0.0f;
#pragma unroll
    for (int w = 0; w < S::kOTiles; ++w) cs.acc[c][w] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
}

// Zero the V rows of a staged tile (first key ts) that lie before key lo:
// they hold keys no column of the wave sees, whose weight is 0, and a
// non-finite value there must not reach the P.V product.
template <int DE, int KT>
__device__ __forceinline__ void zero_v_before(TileRegs<DE, KT> &t, int ts, int lo, int c16, int q4) {
  if (ts < lo) {
    if constexpr (vt_from_lds<DE, KT>()) { // V^T: lane (c16, q4) holds keys ts + 4 q4 + e
#pragma unroll
      for (int w = 0; w < Shape<DE, KT>::kOTiles; ++w)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (ts + 4 * q4 + e < lo) t.vt[w][e] = 0;
    } else { // V rows: lane (c16, q4) holds row c16
      const bool ok = ts + c16 >= lo;
#pragma unroll
      for (int k = 0; k < Shape<DE, KT>::kLaneVec; ++k)
        if (!ok) t.v[k] = make_uint4(0, 0, 0, 0);
    }
  }
}

// Scaled scores of one staged 16-token tile (first key ts) for column group c:
// lane (c16, q4) gets keys ts + 4 * q4 + r (r = 0..3) of its column in log2
// units, soft-capped, and -inf where the column does not see the key (only
// tested when the tile is not seen whole by every column).
template <int DE, int KT, int CG>
__device__ __forceinline__ void tile_scores(const ColumnSet<DE, KT, CG> &cs, int c, const TileRegs<DE, KT> &t, int ts,
                                            bool whole, float cscale, float cap_out, int q4, float *sv) {
  using S = Shape<DE, KT>;
  // S^T = K . Q^T
  f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < S::kKSteps; ++j)
    s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_operand<DE, KT>(t, j), cs.q[c][j], s, 0, 0, 0);
  if constexpr (KT == DT_INT4) {
#pragma unroll
    for (int r = 0; r < 4; ++r) s[r] -= cs.qoff[c]; // remove the 136-per-element offset of K
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) sv[r] = s[r] * cscale;
  if (cap_out > 0.0f) { // logit soft-cap: c * tanh(s / c), in log2 units (uniform branch)
#pragma unroll
    for (int r = 0; r < 4; ++r) sv[r] = tanhf(sv[r]) * cap_out;
  }
  if (!whole) { // some column misses some key of the tile (uniform branch)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tok = ts + 4 * q4 + r;
      if (tok < cs.lo[c] || tok >= cs.hi[c]) sv[r] = -INFINITY;
    }
  }
}

// Online-softmax step of column group c over NS new scores per lane: the
// weights, bf16-packed in pairs into pk[NS / 2], and the running state.
template <int NS, int DE, int KT, int CG>
__device__ __forceinline__ void softmax_step(ColumnSet<DE, KT, CG> &cs, int c, const float *sv, uint32_t *pk) {
  using S = Shape<DE, KT>;
  float mx = sv[0];
#pragma unroll
  for (int r = 1; r < NS; ++r) mx = fmaxf(mx, sv[r]);
  mx = xor32_max(xor16_max(mx));
  // Lazy rescale: the reference max m moves (and the state is rescaled by
  // 2^(m - m_new)) only when a score exceeds it by more than kLazy, so
  // weights stay below 2^kLazy and after the first tiles the rescale is
  // almost never needed.  m + log2(l) and acc / l do not depend on which
  // reference is used.
  // m = -inf: any visible key grows it.  A given starting reference (unified
  // max) far above a still-empty state's first scores is moved down to
  // them, so no weight underflows.
  const bool empty = cs.l[c] == 0.0f;
  const bool grow = mx > cs.m[c] + kLazy || (empty && mx != -INFINITY && mx < cs.m[c] - kDrop);
  if (__builtin_amdgcn_ballot_w64(grow) != 0) {
    const float alpha = grow ? (empty ? 0.0f : __builtin_amdgcn_exp2f(cs.m[c] - mx)) : 1.0f;
    cs.m[c] = grow ? mx : cs.m[c];
    cs.l[c] *= alpha;
    if constexpr (KT == DT_INT4) cs.lb[c] *= alpha;
#pragma unroll
    for (int w = 0; w < S::kOTiles; ++w) {
#pragma unroll
      for (int r = 0; r < 4; ++r) cs.acc[c][w][r] *= alpha;
    }
  }
  // no visible key so far for this column: weights 0, state unchanged
  const bool live = cs.m[c] != -INFINITY;
  float pr[NS];
#pragma unroll
  for (int r = 0; r < NS; ++r) pr[r] = live ? __builtin_amdgcn_exp2f(sv[r] - cs.m[c]) : 0.0f;
  float sum = 0.0f;
#pragma unroll
  for (int r = 0; r < NS; r += 4) sum += (pr[r] + pr[r + 1]) + (pr[r + 2] + pr[r + 3]);
  cs.l[c] += sum;
#pragma unroll
  for (int r = 0; r < NS; r += 2) pk[r / 2] = pack_bf16x2(pr[r], pr[r + 1]);
  if constexpr (KT == DT_INT4) {
    float sb = 0.0f; // the weights as the P.V product sees them
#pragma unroll
    for (int r = 0; r < NS / 2; ++r) sb += __uint_as_float(pk[r] << 16) + __uint_as_float(pk[r] & 0xFFFF0000u);
    cs.lb[c] += sb;
  }
}

// V^T slices of a staged tile as bf16 operands: va[w] holds, in lane
// (c16, q4), keys 4 * q4 + r of dimension c16 of the 16-dim slice w.
template <int DE, int KT>
__device__ __forceinline__ void v_slices(const TileRegs<DE, KT> &t, s16x4_t ident, const long (&sel)[2],
                                         s16x4_t *va) {
  using S = Shape<DE, KT>;
  if constexpr (vt_from_lds<DE, KT>()) { // read transposed from LDS already
#pragma unroll
    for (int w = 0; w < S::kOTiles; ++w) va[w] = t.vt[w];
    return;
  }
  // all products first, so the dependent conversions do not wait on each other
  f32x4_t vt[S::kOTiles];
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int w = 0; w < S::kOTiles; ++w) {
    if constexpr (KT == DT_INT4) {
      // even (w even) or odd nibbles of dword (w / 2) % 4 of piece w / 8, as 136 + n
      const uint32_t dw = dword_of(t.v[w >> 3], (w >> 1) & 3);
      const uint32_t nib = (w & 1) ? int4_odd(dw) : int4_even(dw);
      const s16x4_t a = __builtin_bit_cast(s16x4_t, make_uint2(offset_bf16_lo(nib), offset_bf16_hi(nib)));
      vt[w] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, ident, zero, 0, 0, 0);
    } else if constexpr (KT == DT_FP8) {
      const int u = w >> 1, hh = w & 1; // 8-byte group u of the lane slice
      const uint4 wv = t.v[u >> 1];
      const uint32_t lo32 = (u & 1) ? wv.z : wv.x;
      const uint32_t hi32 = (u & 1) ? wv.w : wv.y;
      const long a = (long)(((uint64_t)hi32 << 32) | lo32);
      vt[w] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, sel[hh], zero, 0, 0, 0);
    } else {
      const uint4 wv = t.v[w >> 1];
      const s16x4_t a = __builtin_bit_cast(s16x4_t, (w & 1) ? make_uint2(wv.z, wv.w) : make_uint2(wv.x, wv.y));
      vt[w] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, ident, zero, 0, 0, 0);
    }
  }
#pragma unroll
  for (int w = 0; w < S::kOTiles; ++w)
    va[w] = __builtin_bit_cast(s16x4_t, make_uint2(pack_bf16x2(vt[w][0], vt[w][1]), pack_bf16x2(vt[w][2], vt[w][3])));
}

// One staged 16-token tile (first key ts) through every column group:
// scores, online-softmax step, then O^T += V^T . P^T with the V^T slices
// shared by the groups.  [all_lo, all_hi): keys every column sees.
// ident / sel: the identity and 0/1 selection operands of the V transposition.
template <int DE, int KT, int CG>
__device__ __forceinline__ void tile_update(ColumnSet<DE, KT, CG> &cs, const TileRegs<DE, KT> &t, int ts, int all_lo,
                                            int all_hi, float cscale, float cap_out, s16x4_t ident,
                                            const long (&sel)[2], int q4) {
  using S = Shape<DE, KT>;
  const bool whole = ts >= all_lo && ts + kTile <= all_hi;
  s16x4_t pt[CG]; // P^T operand of each group
#pragma unroll
  for (int c = 0; c < CG; ++c) {
    if (c > 0 && !cs.on[c]) continue; // the same in every lane
    float sv[4];
    tile_scores(cs, c, t, ts, whole, cscale, cap_out, q4, sv);
    uint32_t pk[2];
    softmax_step<4>(cs, c, sv, pk);
    pt[c] = __builtin_bit_cast(s16x4_t, make_uint2(pk[0], pk[1]));
  }
  s16x4_t va[S::kOTiles];
  v_slices(t, ident, sel, va);
#pragma unroll
  for (int c = 0; c < CG; ++c) {
    if (c > 0 && !cs.on[c]) continue;
#pragma unroll
    for (int w = 0; w < S::kOTiles; ++w)
      cs.acc[c][w] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va[w], pt[c], cs.acc[c][w], 0, 0, 0);
  }
}

// Two staged tiles (first keys tsa, tsb) at once: one softmax step over the
// 32 keys and one O^T += V^T . P^T product per 16-dim slice with k = 32
// (v_mfma_f32_16x16x32_bf16, twice the work of the 16x16x16 form per
// instruction).  Lane quarter q4 feeds reduction indices 8 q4 .. 8 q4 + 7 of
// both operands as keys 4 q4 .. 4 q4 + 3 of the first tile, then the same
// keys of the second, so V^T and P^T agree on the key of every index.
template <int DE, int KT, int CG>
__device__ __forceinline__ void pair_update(ColumnSet<DE, KT, CG> &cs, const TileRegs<DE, KT> &ta, int tsa,
                                            const TileRegs<DE, KT> &tb, int tsb, int all_lo, int all_hi,
                                            float cscale, float cap_out, s16x4_t ident, const long (&sel)[2],
                                            int q4) {
  using S = Shape<DE, KT>;
  const bool whole_a = tsa >= all_lo && tsa + kTile <= all_hi;
  const bool whole_b = tsb >= all_lo && tsb + kTile <= all_hi;
  bf16x8_t pt[CG];
#pragma unroll
  for (int c = 0; c < CG; ++c) {
    if (c > 0 && !cs.on[c]) continue; // the same in every lane
    float sv[8];
    tile_scores(cs, c, ta, tsa, whole_a, cscale, cap_out, q4, sv);
    tile_scores(cs, c, tb, tsb, whole_b, cscale, cap_out, q4, sv + 4);
    uint32_t pk[4];
    softmax_step<8>(cs, c, sv, pk);
    pt[c] = __builtin_bit_cast(bf16x8_t, make_uint4(pk[0], pk[1], pk[2], pk[3]));
  }
  s16x4_t va[S::kOTiles], vb[S::kOTiles];
  v_slices(ta, ident, sel, va);
  v_slices(tb, ident, sel, vb);
#pragma unroll
  for (int c = 0; c < CG; ++c) {
    if (c > 0 && !cs.on[c]) continue;
#pragma unroll
    for (int w = 0; w < S::kOTiles; ++w) {
      const uint2 a = __builtin_bit_cast(uint2, va[w]), bv = __builtin_bit_cast(uint2, vb[w]);
      const bf16x8_t v8 = __builtin_bit_cast(bf16x8_t, make_uint4(a.x, a.y, bv.x, bv.y));
      cs.acc[c][w] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v8, pt[c], cs.acc[c][w], 0, 0, 0);
    }
  }
}

// CG: column groups (16 columns each) a wave computes on every staged tile;
// more than one only with several query rows per request and one KV head per
// workgroup.  The groups share the K operand and the V^T products, so K/V
// are read once for all of them.
template <int D, int PACK, int KT, int NBUF, int CG>
__global__ __launch_bounds__(kThreads) void partial_mfma_kernel(const Params p, const InlineWork w) {
  static_assert(CG == 1 || PACK == 1, "column groups of (query row, head) pairs take one KV head");
  constexpr int DE = D * PACK;
  using S = Shape<DE, KT>;
  constexpr int OSTRIDE = D + 4;
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
  const int kvg = blockIdx.y / col_blocks;             // KV heads kvg*PACK .. kvg*PACK+PACK-1
  const int cg0 = blockIdx.y % col_blocks * CG;        // first column group (several queries per request)
  const int g = p.group;
  const int gp = g * PACK;    // query heads of the pack (<= 16)
  const int Hk = p.num_kv_heads;
  // KV head (within the pack) of this lane's column; (query, head) columns
  // are only run with one KV head per workgroup
  const int my_kv = p.qo_indptr ? 0 : c16 / g;

  // ---- which (request, split) is this workgroup? ----
  int b, split, nb, L;
  if (!locate_item(p, w, item, s_scan, s_item, b, split, nb, L)) return;

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
  const int my_tiles = ntiles > wave ? (ntiles - wave + kWaves - 1) / kWaves : 0;
  load_columns<D>(cs, p, q4, my_kv);

  float cscale = p.score_scale;
  if (KT != DT_BF16) cscale *= p.k_scale[b * Hk + kvg * PACK + min(my_kv, PACK - 1)];
  const float cap_out = p.cap_out;
  s16x4_t ident;
  long sel[2];
  transpose_operands<KT>(c16, q4, ident, sel);

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
    const int ts = a0 + (ft + wave + lane * kWaves) * kTile;
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
    const int ts = a0 + (ft + wave + i * kWaves) * kTile;
    zero_v_before(t, ts, w_lo, c16, q4); // rows before the first key any column sees
    tile_update(cs, t, ts, all_lo, all_hi, cscale, cap_out, ident, sel, q4);
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
    merge_waves_and_store<D, OSTRIDE>(p, sm_m, sm_l, sm_o, b, kvg, cg0 + c, item, nb);
  }
}

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
  const int item = blockIdx.x;
  const int row_blocks = (p.col_groups + kGroups - 1) / kGroups; // workgroups per (item, KV head)
  const int kvg = blockIdx.y / row_blocks;                       // KV head
  const int cgw = blockIdx.y % row_blocks * kGroups;             // first column group of the workgroup
  const int g = p.group;
  const int Hk = p.num_kv_heads;

  int b, split, nb, L;
  if (!locate_item(p, w, item, s_scan, s_item, b, split, nb, L)) return;
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
  s16x4_t ident;
  long sel[2];
  transpose_operands<KT>(c16, q4, ident, sel);

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
                pair_update(cs, ta, tsa, tb, tsb, all_lo, all_hi, cscale, cap_out, ident, sel, q4);
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
                tile_update(cs, t, ts, all_lo, all_hi, cscale, cap_out, ident, sel, q4);
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
    const float vscale = p.v_scale ? p.v_scale[b * Hk + kvg] : 1.0f;
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
      float *dst = p.o_part + (slot * p.cols + c16) * D;
#pragma unroll
      for (int wt = 0; wt < S::kOTiles; ++wt) {
        const int od = out_dim<D, KT>(wt, q4);
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[od + r * S::kOutStride] = (cs.acc[c][wt][r] - voff) * inv;
      }
      if (q4 == 0) p.lse_part[slot * p.cols + c16] = lse2;
    }
  }
}

// Several query rows per request, bf16 KV, head_dim 128, from three groups
// of 16 columns on: 32x32 matrix tiles.  Each wave owns 32 (query row, head)
// columns of one KV head and the workgroup's four waves share every staged
// 64-key block (one 16-row part staged by each wave, barriers around it, as
// in partial_rows_kernel).  Per 32-key tile and wave:
//   * S^T[key][column] = K . Q^T with v_mfma_f32_32x32x16_bf16 over 8 steps
//     of 16 dims: lane (i, h) = (l % 32, l / 32) feeds K row i, dims
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
template <int NBUF>
__global__ __launch_bounds__(kThreads) void partial_prefill_kernel(const Params p, const InlineWork w) {
  constexpr int D = 128;
  using S = Shape<D, DT_BF16>;                    // 256-byte rows, 16 pieces
  constexpr int kRowBytes = S::kRowBytes;         // one key's K (or V) row of the head
  constexpr int kBlock = kWaves * kTile;          // 64 keys staged per block
  constexpr int kHalf = kBlock * kRowBytes;       // K (or V) bytes of a block
  constexpr int kGroups = kWaves * 2;             // 16-column groups per workgroup
  typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

  __shared__ int s_scan[2 * 64];
  __shared__ int s_item[4];
  __shared__ __attribute__((aligned(16))) char smem[NBUF * 2 * kHalf];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j32 = lane & 31; // column of the lane (S^T, O^T) / row (K, V^T operands)
  const int h2 = lane >> 5;  // half of the wave
  const int item = blockIdx.x;
  const int row_blocks = (p.col_groups + kGroups - 1) / kGroups;
  const int kvg = blockIdx.y / row_blocks;
  const int cgw = blockIdx.y % row_blocks * kGroups; // first 16-column group of the workgroup
  const int g = p.group;
  const int Hk = p.num_kv_heads;

  int b, split, nb, L;
  if (!locate_item(p, w, item, s_scan, s_item, b, split, nb, L)) return;
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
  const int col = cgw * 16 + wave * 32 + j32;
  const bool ok = col < nq * g;
  const bool wave_on = (cgw * 16 + wave * 32) < nq * g; // the same in every lane of the wave
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

  // Q^T operand: step s holds dims 16 s + 8 h2 .. + 7 of the column's query
  bf16x8_t qop[8];
  {
    const uint16_t *qb = reinterpret_cast<const uint16_t *>(p.q) + ((size_t)qrow * p.num_qo_heads + qhead) * D;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      qop[s] = ok ? __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(qb + 16 * s + 8 * h2))
                  : __builtin_bit_cast(bf16x8_t, make_uint4(0, 0, 0, 0));
  }
  const float cscale = p.score_scale;
  const float cap_out = p.cap_out;
  float m_run = p.m_init, l_run = 0.0f;
  f32x16_t acc[4]; // O^T, 32-dim slice sl: register v holds dim 32 sl + 8 (v / 4) + 4 h2 + v % 4
#pragma unroll
  for (int sl = 0; sl < 4; ++sl)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[sl][v] = 0.0f;

  // ---- staging: this wave's 16-row part of block i, one block per lane ----
  const size_t row_bytes = (size_t)Hk * kRowBytes;
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
  // lane i of load k: row 4 k + i / 16 of the part, position i % 16, which
  // holds source piece position ^ (row % 16) (rows of a block keep the
  // swizzle of their position modulo 16)
  int dma_voff[S::kDma];
#pragma unroll
  for (int k = 0; k < S::kDma; ++k) {
    const int r = k * S::kRowsPerDma + lane / S::kPieces;
    const int piece = (lane % S::kPieces) ^ (r & 15);
    dma_voff[k] = r * (int)row_bytes + kvg * kRowBytes + piece * 16;
  }
  auto issue = [&](int i, int slot) {
    const int li = min(i, 63);
    const size_t base = ((size_t)__builtin_amdgcn_readlane(voff_hi, li) << 32) | __builtin_amdgcn_readlane(voff_lo, li);
    const int nbytes = i < nblocks ? (int)__builtin_amdgcn_readlane(vbytes, li) : 0;
    const __amdgpu_buffer_rsrc_t kr =
        __builtin_amdgcn_make_buffer_rsrc((void *)(kpool + base), (short)0, nbytes, kBufferFlags);
    const __amdgpu_buffer_rsrc_t vr =
        __builtin_amdgcn_make_buffer_rsrc((void *)(vpool + base), (short)0, nbytes, kBufferFlags);
    char *kst = smem + slot * 2 * kHalf + wave * kTile * kRowBytes;
#pragma unroll
    for (int k = 0; k < S::kDma; ++k) dma16_to_lds(kr, kst + 1024 * k, dma_voff[k]);
#pragma unroll
    for (int k = 0; k < S::kDma; ++k) dma16_to_lds(vr, kst + kHalf + 1024 * k, dma_voff[k]);
  };
  // K operand of step s: row j32 of the tile, piece 2 s + h2
  uint32_t k_addr[8];
  {
    const uint32_t base = lds_address(smem) + j32 * kRowBytes;
#pragma unroll
    for (int s = 0; s < 8; ++s) k_addr[s] = base + ((2 * s + h2) ^ (j32 & 15)) * 16;
  }
  // V^T operand reads (ds_read_b64_tr_b16): lane l = 16 G + 4 r + c of group G
  // points at key row 8 hh + 4 (G / 2) + r (+ 16 t, an immediate), dims
  // 32 sl + 16 (G % 2) + 4 c .. + 3, i.e. piece 4 sl + 2 (G % 2) + c / 2, bytes
  // (c % 2) * 8 of it; lane i of the group then holds keys
  // 8 hh + 4 (G / 2) + 0..3 of dim 32 sl + 16 (G % 2) + i.
  uint32_t vt_addr[8]; // [4 hh + sl]
  {
    const int G = lane >> 4, r = (lane >> 2) & 3, c = lane & 3;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) {
        const int row = 8 * hh + 4 * (G >> 1) + r;
        const int piece = 4 * sl + 2 * (G & 1) + (c >> 1);
        vt_addr[4 * hh + sl] = lds_address(smem) + kHalf + row * kRowBytes + ((piece ^ (row & 15)) * 16) + (c & 1) * 8;
      }
  }

  // one 32-key tile (first key ts) at byte offset `to` of the staged block
  auto tile32 = [&](int ts, uint32_t to) {
    // ---- S^T = K . Q^T ----
    uint4 kr[8];
    lds_read_x8(kr, k_addr, to);
    f32x16_t st;
#pragma unroll
    for (int v = 0; v < 16; ++v) st[v] = 0.0f;
#pragma unroll
    for (int s = 0; s < 8; ++s) st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kr[s]), qop[s], st, 0, 0, 0);
    // V^T slices, read while the products run: vt[t][4 hh + sl]
    s16x4_t vt[2][8];
#pragma unroll
    for (int t = 0; t < 2; ++t) lds_read_tr_x8(vt[t], vt_addr, to + t * 16 * kRowBytes);
    // ---- scores: register v holds key ts + 8 (v / 4) + 4 h2 + v % 4 ----
    float sv[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) sv[v] = st[v] * cscale;
    if (cap_out > 0.0f) {
#pragma unroll
      for (int v = 0; v < 16; ++v) sv[v] = tanhf(sv[v]) * cap_out;
    }
    if (ts < all_lo || ts + 2 * kTile > all_hi) { // some column misses some key (uniform)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int tok = ts + 8 * (v >> 2) + 4 * h2 + (v & 3);
        if (tok < c_lo || tok >= c_hi) sv[v] = -INFINITY;
      }
    }
    float mx = sv[0];
#pragma unroll
    for (int v = 1; v < 16; ++v) mx = fmaxf(mx, sv[v]);
    mx = xor32_max(mx);
    // lazy rescale (as in the 16x16 kernels): the reference moves only when a
    // score exceeds it by more than kLazy
    const bool empty = l_run == 0.0f;
    const bool grow = mx > m_run + kLazy || (empty && mx != -INFINITY && mx < m_run - kDrop);
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float alpha = grow ? (empty ? 0.0f : __builtin_amdgcn_exp2f(m_run - mx)) : 1.0f;
      m_run = grow ? mx : m_run;
      l_run *= alpha;
#pragma unroll
      for (int sl = 0; sl < 4; ++sl)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[sl][v] *= alpha;
    }
    const bool live = m_run != -INFINITY;
    uint32_t pk[8];
    float sum = 0.0f;
#pragma unroll
    for (int v = 0; v < 16; v += 2) {
      const float p0 = live ? __builtin_amdgcn_exp2f(sv[v] - m_run) : 0.0f;
      const float p1 = live ? __builtin_amdgcn_exp2f(sv[v + 1] - m_run) : 0.0f;
      sum += p0 + p1;
      pk[v / 2] = pack_bf16x2(p0, p1);
    }
    l_run += sum;
    // ---- O^T += V^T . P^T, k = 16 keys per product ----
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const bf16x8_t pt = __builtin_bit_cast(bf16x8_t, make_uint4(pk[4 * t], pk[4 * t + 1], pk[4 * t + 2], pk[4 * t + 3]));
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) {
        const uint2 a = __builtin_bit_cast(uint2, vt[t][sl]), c = __builtin_bit_cast(uint2, vt[t][4 + sl]);
        const bf16x8_t v8 = __builtin_bit_cast(bf16x8_t, make_uint4(a.x, a.y, c.x, c.y));
        acc[sl] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v8, pt, acc[sl], 0, 0, 0);
      }
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
        wait_vmem<(NBUF - 1) * 2 * S::kDma>();
        __syncthreads();
        if (i < nblocks && wave_on) {
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int ts = k0 + i * kBlock + u * 2 * kTile;
            if (ts < wv_hi && ts + 2 * kTile > wv_lo) tile32(ts, j * 2 * kHalf + u * 2 * kTile * kRowBytes);
          }
        }
        __syncthreads();
        issue(i + NBUF, j);
      }
    }
    wait_vmem<0>();
  }

  // ---- this lane's column: final output, or the split's partial ----
  if (!wave_on) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (!ok) return;
  const bool live = l_tot > 0.0f;
  const float inv = live ? 1.0f / l_tot : 0.0f;
  const float lse2 = live ? m_run + __log2f(l_tot) : -INFINITY;
  if (nb == 1) {
    uint16_t *orow = reinterpret_cast<uint16_t *>(p.o) + ((size_t)qrow * p.num_qo_heads + qhead) * D;
#pragma unroll
    for (int sl = 0; sl < 4; ++sl)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int d0 = 32 * sl + 8 * q + 4 * h2;
        *reinterpret_cast<uint2 *>(orow + d0) =
            make_uint2(pack_bf16x2(acc[sl][4 * q] * inv, acc[sl][4 * q + 1] * inv),
                       pack_bf16x2(acc[sl][4 * q + 2] * inv, acc[sl][4 * q + 3] * inv));
      }
    if (h2 == 0 && p.lse) p.lse[(size_t)qrow * p.num_qo_heads + qhead] = lse2 * kLn2;
  } else {
    const int cg = col / 16;
    const size_t slot = ((size_t)kvg * p.col_groups + cg) * p.items + item;
    float *dst = p.o_part + (slot * p.cols + col % 16) * D;
#pragma unroll
    for (int sl = 0; sl < 4; ++sl)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int d0 = 32 * sl + 8 * q + 4 * h2;
        *reinterpret_cast<float4 *>(dst + d0) =
            make_float4(acc[sl][4 * q] * inv, acc[sl][4 * q + 1] * inv, acc[sl][4 * q + 2] * inv, acc[sl][4 * q + 3] * inv);
      }
    if (h2 == 0) p.lse_part[slot * p.cols + col % 16] = lse2;
  }
}

} // namespace

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

template <int D, int PACK, int KT>
static hipError_t launch_mfma_d(const Params &p, const InlineWork &w, const Launch &l) {
  constexpr int NB = Shape<D * PACK, KT>::kNBuf;
  if constexpr (PACK == 1) {
    constexpr int kGroups = kWaves * rows_cg<D>();
    if (p.col_share == kGroups) {
      const dim3 grid(p.items, p.num_kv_heads * ((p.col_groups + kGroups - 1) / kGroups));
      if constexpr (D == 128 && KT == DT_BF16) return launch_kernel(l, partial_prefill_kernel<2>, grid, p, w);
      return launch_kernel(l, partial_rows_kernel<D, KT, rows_nbuf<D, KT>(), rows_cg<D>()>, grid, p, w);
    }
    if constexpr (D <= 128) {
      if (p.col_share == 2)
        return launch_kernel(l, partial_mfma_kernel<D, 1, KT, NB, 2>,
                             dim3(p.items, p.num_kv_heads * ((p.col_groups + 1) / 2)), p, w);
    }
  }
  if (p.col_share != 1) return hipErrorInvalidValue;
  return launch_kernel(l, partial_mfma_kernel<D, PACK, KT, NB, 1>,
                       dim3(p.items, p.num_kv_heads / PACK * p.col_groups), p, w);
}

// Column groups from which several query rows per request go to the
// shared-tile kernel.  Below 8 groups some of its waves idle; that pays for
// bf16, whose second read of the keys costs more than the idle waves, from 3
// groups on, but for the compute-heavier fp8 and INT4 tiles only once three
// of the four waves have work (batch-128 fp8, 8 rows of 8 heads = 4 groups:
// 656 us with the chunk-splitting kernel, 980 us shared-tile).
constexpr int kRowsMinGroupsBf16 = 3;
constexpr int kRowsMinGroupsQuant = 5;

// Column groups of (query row, head) pairs one partial workgroup computes
// (several query rows per request).  Two: the chunk-splitting kernel runs
// both on each staged tile (head_dim <= 128), halving the K/V reads of short
// appends.  From three groups on: the shared-tile kernel, whose workgroup
// covers 8 groups (head_dim <= 128) or 4 (256) and reads the keys once for
// all of them.
int mfma_col_share(int head_dim, int kv_type, int col_groups) {
  if (col_groups >= (kv_type == DT_BF16 ? kRowsMinGroupsBf16 : kRowsMinGroupsQuant))
    return kWaves * (head_dim <= 128 ? 2 : 1);
  return col_groups >= 2 && head_dim <= 128 ? 2 : 1;
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
