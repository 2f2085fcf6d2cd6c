// Device building blocks of the matrix-core partial kernels (decode_mfma.hip:
// one or two query rows' worth of columns per wave, keys split over the
// waves; rows_mfma.hip: several query rows per request, staged tiles shared
// by the waves): tile shapes and their LDS staging, operand layouts of the
// 16x16 matrix instructions, the per-lane column state, and the per-tile
// online-softmax update.
#pragma once

#include "kvs_device.h"

namespace kvs {
namespace tiles {


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

// XOR swizzle of the 16-byte pieces of staged row r.  gfx950's LDS has 64
// banks of 4 bytes: rows of 256 bytes or more all start in bank 0, rows of
// 128 bytes alternate between the two bank halves, so rows with the same
// u = r / kRowsPerBankPeriod collide.  u -> u ^ ((u & 3) << s) permutes the
// piece index bits, so
//   * the 16 rows a K operand read takes at one logical piece land on 16
//     distinct pieces (conflict-free 16-byte reads), and
//   * four consecutive u, which a transposing V^T read takes at one aligned
//     group of 2^s pieces (four 16-bit rows x four pieces, s = 2; four 8-bit
//     row pairs x two pieces, s = 1), land in four different groups.
// With the plain swizzle u ^ piece the four rows stayed inside one group:
// every 16-bit transposing read of a 256-byte row was a four-way conflict.
template <int DE, int KT>
__device__ __forceinline__ int stage_swizzle(int r) {
  using S = Shape<DE, KT>;
  constexpr int kShift = S::kRowsPerBankPeriod == 1 ? 2 : 1;
  const int u = r / S::kRowsPerBankPeriod;
  return (u ^ ((u & 3) << kShift)) & (S::kPieces - 1);
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

// bf16 tiles up to 128 pack dims take V^T straight from LDS (16-bit
// transposing reads), fp8 and INT4 tiles from 8-bit transposing reads
// (vt_tr8); wider bf16 tiles transpose V with a matrix product.  At
// head_dim 256 the transposed slices, read together with K, held registers
// the pair-wise prefill kernel needed (8192-row prefill: 147 against 158
// TFLOP/s); at head_dim 128 they gained (2048 rows on a 32k cache: 499
// against 480 TFLOP/s), decode unchanged.
template <int DE, int KT>
constexpr bool vt_from_lds() { return KT == DT_BF16 && DE <= 128; }
template <int KT>
constexpr bool vt_tr8() { return KT == DT_FP8 || KT == DT_INT4; }

template <int DE, int KT>
struct TileRegs {
  static constexpr int kTr8Blocks = vt_tr8<KT>() ? Shape<DE, KT>::kRowBytes / 32 : 1;
  uint4 k[Shape<DE, KT>::kLaneVec];    // K pieces 4 * pc + q4 of row c16
  uint4 v[Shape<DE, KT>::kLaneVec];    // V pieces (bf16 beyond 128 pack dims)
  s16x4_t vt[Shape<DE, KT>::kOTiles];  // V^T slices read transposed from LDS (vt_from_lds)
  uint2 vn[kTr8Blocks];                // fp8 / INT4: V codes of 4 keys per 32-byte block (vt_tr8)
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
// Four 16-byte reads at the first four of the lane addresses a, one wait
__device__ __forceinline__ void lds_read_x4(uint4 (&k)[4], const uint32_t *a, uint32_t off) {
  u32x4_t r0, r1, r2, r3;
  __asm__ volatile("ds_read_b128 %0, %4\n\t"
                   "ds_read_b128 %1, %5\n\t"
                   "ds_read_b128 %2, %6\n\t"
                   "ds_read_b128 %3, %7\n\t"
                   "s_waitcnt lgkmcnt(0)"
                   : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
                   : "v"(a[0] + off), "v"(a[1] + off), "v"(a[2] + off), "v"(a[3] + off)
                   : "memory");
  k[0] = __builtin_bit_cast(uint4, r0);
  k[1] = __builtin_bit_cast(uint4, r1);
  k[2] = __builtin_bit_cast(uint4, r2);
  k[3] = __builtin_bit_cast(uint4, r3);
}
// Eight 8-bit transposing reads (gfx950 ds_read_b64_tr_b8) at eight lane
// addresses, one wait: within each 16-lane group, lane i receives byte i % 8
// of the 8 bytes addressed by lane 2 r + i / 8, for r = 0..7.
__device__ __forceinline__ void lds_read_tr8_x8(uint2 (&v)[8], const uint32_t (&a)[8], uint32_t off) {
  u32x2_t r0, r1, r2, r3, r4, r5, r6, r7;
  __asm__ volatile("ds_read_b64_tr_b8 %0, %8\n\t"
                   "ds_read_b64_tr_b8 %1, %9\n\t"
                   "ds_read_b64_tr_b8 %2, %10\n\t"
                   "ds_read_b64_tr_b8 %3, %11\n\t"
                   "ds_read_b64_tr_b8 %4, %12\n\t"
                   "ds_read_b64_tr_b8 %5, %13\n\t"
                   "ds_read_b64_tr_b8 %6, %14\n\t"
                   "ds_read_b64_tr_b8 %7, %15\n\t"
                   "s_waitcnt lgkmcnt(0)"
                   : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6), "=&v"(r7)
                   : "v"(a[0] + off), "v"(a[1] + off), "v"(a[2] + off), "v"(a[3] + off), "v"(a[4] + off),
                     "v"(a[5] + off), "v"(a[6] + off), "v"(a[7] + off)
                   : "memory");
  v[0] = __builtin_bit_cast(uint2, r0);
  v[1] = __builtin_bit_cast(uint2, r1);
  v[2] = __builtin_bit_cast(uint2, r2);
  v[3] = __builtin_bit_cast(uint2, r3);
  v[4] = __builtin_bit_cast(uint2, r4);
  v[5] = __builtin_bit_cast(uint2, r5);
  v[6] = __builtin_bit_cast(uint2, r6);
  v[7] = __builtin_bit_cast(uint2, r7);
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
// fp8 / INT4 tiles: the lane's K pieces and one 8-bit transposing read
// (ds_read_b64_tr_b8, layout as for lds_read_tr8_x8) per 32-byte block of V,
// one wait.
__device__ __forceinline__ void lds_read_k1_tr8x2(uint4 &k0, uint2 (&v)[2], uint32_t ak, uint32_t a0, uint32_t a1) {
  u32x4_t rk;
  u32x2_t r0, r1;
  __asm__ volatile("ds_read_b128 %0, %3\n\t"
                   "ds_read_b64_tr_b8 %1, %4\n\t"
                   "ds_read_b64_tr_b8 %2, %5\n\t"
                   "s_waitcnt lgkmcnt(0)"
                   : "=&v"(rk), "=&v"(r0), "=&v"(r1)
                   : "v"(ak), "v"(a0), "v"(a1)
                   : "memory");
  k0 = __builtin_bit_cast(uint4, rk);
  v[0] = __builtin_bit_cast(uint2, r0);
  v[1] = __builtin_bit_cast(uint2, r1);
}
__device__ __forceinline__ void lds_read_k2_tr8x4(uint4 &k0, uint4 &k1, uint2 (&v)[4], uint32_t ak0, uint32_t ak1,
                                                  uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3) {
  u32x4_t rk0, rk1;
  u32x2_t r0, r1, r2, r3;
  __asm__ volatile("ds_read_b128 %0, %6\n\t"
                   "ds_read_b128 %1, %7\n\t"
                   "ds_read_b64_tr_b8 %2, %8\n\t"
                   "ds_read_b64_tr_b8 %3, %9\n\t"
                   "ds_read_b64_tr_b8 %4, %10\n\t"
                   "ds_read_b64_tr_b8 %5, %11\n\t"
                   "s_waitcnt lgkmcnt(0)"
                   : "=&v"(rk0), "=&v"(rk1), "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
                   : "v"(ak0), "v"(ak1), "v"(a0), "v"(a1), "v"(a2), "v"(a3)
                   : "memory");
  k0 = __builtin_bit_cast(uint4, rk0);
  k1 = __builtin_bit_cast(uint4, rk1);
  v[0] = __builtin_bit_cast(uint2, r0);
  v[1] = __builtin_bit_cast(uint2, r1);
  v[2] = __builtin_bit_cast(uint2, r2);
  v[3] = __builtin_bit_cast(uint2, r3);
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
// fp8 / INT4 V: one 8-bit transposing read per 32-byte block of a row;
// lane 16 q4 + 2 r + h points at token row 4 q4 + r % 4, bytes
// 16 (r / 4) + 8 h .. + 7 of the block, so lane i of quarter q4 gets byte i
// of the block for keys 4 q4 + 0..3 in its low dword and byte 16 + i of the
// same keys in its high dword (fp8: dims i and 16 + i of the block; INT4:
// dims 2 i, 2 i + 1 and 32 + 2 i, 33 + 2 i).
template <int DE, int KT>
struct StageReader {
  using S = Shape<DE, KT>;
  static constexpr bool kVt = vt_from_lds<DE, KT>();
  static constexpr bool kVn = vt_tr8<KT>();
  static constexpr int kVtAddr = kVt ? S::kOTiles / 2 : (kVn ? S::kRowBytes / 32 : 1);
  static_assert(!kVn || (S::kRowBytes >= 64 && S::kRowBytes <= 256), "rows of 64 to 256 bytes");
  uint32_t k_addr[S::kLaneVec];
  uint32_t vt_addr[kVtAddr];
  __device__ __forceinline__ void init(uint32_t tile0, int lane) {
    const int c16 = lane & 15, q4 = lane >> 4;
    const int swz = stage_swizzle<DE, KT>(c16);
#pragma unroll
    for (int pc = 0; pc < S::kLaneVec; ++pc)
      k_addr[pc] = tile0 + c16 * S::kRowBytes + ((4 * pc + q4) ^ swz) * 16;
    if constexpr (kVn) {
      const int r = c16 >> 1, h = c16 & 1;
      const int row = 4 * q4 + (r & 3);
      const int vswz = stage_swizzle<DE, KT>(row);
#pragma unroll
      for (int blk = 0; blk < kVtAddr; ++blk)
        vt_addr[blk] = tile0 + S::kTileBytes + row * S::kRowBytes + (((2 * blk + (r >> 2)) ^ vswz) * 16) + 8 * h;
    }
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
    if constexpr (kVn) {
      if constexpr (S::kLaneVec == 1) {
        uint2 (&vn)[2] = *reinterpret_cast<uint2 (*)[2]>(&t.vn[0]);
        lds_read_k1_tr8x2(t.k[0], vn, k_addr[0] + off, vt_addr[0] + off, vt_addr[1] + off);
      } else {
#pragma unroll
        for (int pc = 0; pc < S::kLaneVec; pc += 2) {
          uint2 (&vn)[4] = *reinterpret_cast<uint2 (*)[4]>(&t.vn[2 * pc]);
          lds_read_k2_tr8x4(t.k[pc], t.k[pc + 1], vn, k_addr[pc] + off, k_addr[pc + 1] + off,
                            vt_addr[2 * pc] + off, vt_addr[2 * pc + 1] + off, vt_addr[2 * pc + 2] + off,
                            vt_addr[2 * pc + 3] + off);
        }
      }
    } else if constexpr (kVt) {
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
    // slice w of 64-dim block w / 4: the even (w even) or odd dims of its
    // first (w % 4 < 2) or second 32 dims; matrix row m is dim 2 m (+ 1)
    return 64 * (w >> 2) + 32 * ((w >> 1) & 1) + (w & 1) + 8 * q4;
  } else if constexpr (KT == DT_FP8) {
    return 16 * w + 4 * q4; // slice w: byte 16 (w % 2) + m of 32-byte block w / 2 is row m
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
// record_meta: this workgroup records the split metadata of its request when
// it holds the request's first split (one workgroup per item may).
__device__ __forceinline__ bool locate_item(const Params &p, const InlineWork &w, int item, bool record_meta,
                                            int *s_scan, int *s_item, int &b, int &split, int &nb, int &L) {
  if (w.n_items > 0) { // planned on the host
    const uint32_t e = w.item[item];
    b = (int)(e >> 8);
    split = (int)(e & 0xFF);
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
  if (p.meta && split == 0 && record_meta && threadIdx.x == 0) {
    p.meta[2 * b] = s_item[3];
    p.meta[2 * b + 1] = nb;
  }
  L = p.kv_len[b];
  return true;
}

// Order of the multi-row kernels' workgroups.  The launch grid is (items,
// KV heads x row blocks); the hardware deals workgroups to the XCDs in turn
// by linear id (x fastest).  Read in launch order, XCD k always gets the
// items congruent to k.  That keeps one chunk per XCD, and it is balanced
// when the items hold equal work; in a causal prefill longer than a chunk the
// early chunks hold far more work than the late ones (a 16384-row prefill in
// 4 chunks: 1.7x the mean on two XCDs).  There (balanced) the linear id is
// mapped to (KV head, item, row block), row block fastest: with a multiple
// of kXcds KV heads each XCD takes whole heads, their items and row blocks in
// turn (the row blocks of one chunk run together and share it in that XCD's
// L2); otherwise consecutive row blocks go to consecutive XCDs.  Either way
// each XCD gets about the same work.
constexpr int kXcds = 8;
struct RowsOrder {
  int kvg, item, rb;
};
__device__ __forceinline__ RowsOrder rows_order(int row_blocks, int num_kv_heads, bool balanced) {
  if (!balanced) return RowsOrder{(int)blockIdx.y / row_blocks, (int)blockIdx.x, (int)blockIdx.y % row_blocks};
  const int nx = gridDim.x;
  const int n = blockIdx.x + nx * blockIdx.y;
  const int total = nx * gridDim.y;
  const int l = num_kv_heads % kXcds == 0 ? (n % kXcds) * (total / kXcds) + n / kXcds : n;
  RowsOrder r;
  r.rb = l % row_blocks;
  r.item = (l / row_blocks) % nx;
  r.kvg = l / (row_blocks * nx);
  return r;
}

// The bf16 identity operand of lane (c16, q4) for the V transposition by a
// 16x16x16 product (bf16 tiles wider than 128 pack dims).
__device__ __forceinline__ s16x4_t transpose_identity(int c16, int q4) {
  const short one_bf16 = 0x3F80;
  s16x4_t ident;
#pragma unroll
  for (int e = 0; e < 4; ++e) ident[e] = (4 * q4 + e == c16) ? one_bf16 : (short)0;
  return ident;
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
  bool seen[CG];              // the column has had a visible key (the same in its 4 lanes)
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
    cs.seen[c] = false;
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
  if constexpr (KT == DT_INT4) return; // every INT4 code is a finite value
  if (ts < lo) {
    if constexpr (vt_tr8<KT>()) { // fp8 V codes: byte e of each dword is key ts + 4 q4 + e
      uint32_t keep = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (ts + 4 * q4 + e >= lo) keep |= 0xFFu << (8 * e);
#pragma unroll
      for (int k = 0; k < TileRegs<DE, KT>::kTr8Blocks; ++k) {
        t.vn[k].x &= keep;
        t.vn[k].y &= keep;
      }
    } else if constexpr (vt_from_lds<DE, KT>()) { // V^T: lane (c16, q4) holds keys ts + 4 q4 + e
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
  // them, so no weight underflows.  Empty means no visible key in the whole
  // column so far: a lane's own l can be 0 while the column's other lanes
  // have keys (a window start inside a tile), and its share of the output
  // dims then already holds their contributions.
  const bool empty = !cs.seen[c];
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
  cs.seen[c] = cs.seen[c] || mx != -INFINITY;
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

// Whether V^T slices come straight from LDS reads (no matrix product), so
// that each slice can be formed where its P.V product uses it.
template <int DE, int KT>
constexpr bool v_direct() { return vt_from_lds<DE, KT>() || vt_tr8<KT>(); }

// Slice w of a directly read V^T (v_direct): in lane (c16, q4), keys
// 4 * q4 + r of matrix row c16 of slice w, as bf16 (INT4: 136 + n).
template <int DE, int KT>
__device__ __forceinline__ s16x4_t v_slice(const TileRegs<DE, KT> &t, int w) {
  if constexpr (vt_from_lds<DE, KT>()) {
    return t.vt[w];
  } else if constexpr (KT == DT_FP8) { // 32-byte block w / 2, dword w % 2
    typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
    const uint32_t x = (w & 1) ? t.vn[w >> 1].y : t.vn[w >> 1].x;
    const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, false);
    const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, true);
    return __builtin_bit_cast(s16x4_t, make_uint2(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)));
  } else { // INT4: 64-dim block w / 4, dword (w / 2) % 2, even (w even) or odd nibbles
    static_assert(KT == DT_INT4, "direct V^T");
    const uint32_t x = ((w >> 1) & 1) ? t.vn[w >> 2].y : t.vn[w >> 2].x;
    const uint32_t nib = (w & 1) ? int4_odd(x) : int4_even(x);
    return __builtin_bit_cast(s16x4_t, make_uint2(offset_bf16_lo(nib), offset_bf16_hi(nib)));
  }
}

// V^T slices of a staged tile as bf16 operands: va[w] holds, in lane
// (c16, q4), keys 4 * q4 + r of matrix row c16 of slice w (the 16 dims
// out_dim describes).
template <int DE, int KT>
__device__ __forceinline__ void v_slices(const TileRegs<DE, KT> &t, s16x4_t ident, s16x4_t *va) {
  using S = Shape<DE, KT>;
  if constexpr (v_direct<DE, KT>()) { // bf16 (16-bit transposing reads), fp8 and INT4 (8-bit ones)
#pragma unroll
    for (int w = 0; w < S::kOTiles; ++w) va[w] = v_slice(t, w);
    return;
  }
  // bf16 beyond 128 pack dims: V times an identity, all products first, so
  // the dependent conversions do not wait on each other
  f32x4_t vt[S::kOTiles];
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int w = 0; w < S::kOTiles; ++w) {
    const uint4 wv = t.v[w >> 1];
    const s16x4_t a = __builtin_bit_cast(s16x4_t, (w & 1) ? make_uint2(wv.z, wv.w) : make_uint2(wv.x, wv.y));
    vt[w] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, ident, zero, 0, 0, 0);
  }
#pragma unroll
  for (int w = 0; w < S::kOTiles; ++w)
    va[w] = __builtin_bit_cast(s16x4_t, make_uint2(pack_bf16x2(vt[w][0], vt[w][1]), pack_bf16x2(vt[w][2], vt[w][3])));
}

// One staged 16-token tile (first key ts) through every column group:
// scores, online-softmax step, then O^T += V^T . P^T with the V^T slices
// shared by the groups.  [all_lo, all_hi): keys every column sees.
// ident: the identity operand of the V transposition (transpose_identity).
template <int DE, int KT, int CG>
__device__ __forceinline__ void tile_update(ColumnSet<DE, KT, CG> &cs, const TileRegs<DE, KT> &t, int ts, int all_lo,
                                            int all_hi, float cscale, float cap_out, s16x4_t ident, int q4) {
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
  v_slices(t, ident, va);
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
                                            float cscale, float cap_out, s16x4_t ident, int q4) {
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
  auto pv = [&](int w, s16x4_t sa, s16x4_t sb) {
    const uint2 a = __builtin_bit_cast(uint2, sa), bv = __builtin_bit_cast(uint2, sb);
    const bf16x8_t v8 = __builtin_bit_cast(bf16x8_t, make_uint4(a.x, a.y, bv.x, bv.y));
#pragma unroll
    for (int c = 0; c < CG; ++c)
      if (c == 0 || cs.on[c]) cs.acc[c][w] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v8, pt[c], cs.acc[c][w], 0, 0, 0);
  };
  if constexpr (v_direct<DE, KT>()) { // each slice formed where its products use it
#pragma unroll
    for (int w = 0; w < S::kOTiles; ++w) pv(w, v_slice(ta, w), v_slice(tb, w));
  } else {
    s16x4_t va[S::kOTiles], vb[S::kOTiles];
    v_slices(ta, ident, va);
    v_slices(tb, ident, vb);
#pragma unroll
    for (int w = 0; w < S::kOTiles; ++w) pv(w, va[w], vb[w]);
  }
}

} // namespace tiles

// Launches the multi-row partial kernels (rows_mfma.hip) for a plan whose
// workgroups cover 4 or 8 column groups (Params::col_share).
hipError_t launch_partial_rows(const Params &p, const InlineWork &w, int head_dim, int kv_type, const Launch &l);
// Launches the 32-column kernel (rows_mfma.hip) for two column groups of
// (query row, head) pairs at head_dim 128 (Params::col_share 2).
hipError_t launch_cols32(const Params &p, const InlineWork &w, int kv_type, const Launch &l);

} // namespace kvs
