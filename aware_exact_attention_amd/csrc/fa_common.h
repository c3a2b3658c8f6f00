// fa_common.h - device-side types and helpers shared by the gfx950 kernels.
#ifndef FA_COMMON_H_
#define FA_COMMON_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>
#include <utility>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Compute units of a gfx950 device (MI355X / MI350X); used to decide whether
// a grid of large workgroups still covers the whole GPU.
constexpr long long kNumCUs = 256;

// v_mfma_f32_32x32x16_bf16.  Lane l supplies row (l % 32) of A and column
// (l % 32) of B, each with eight k-values; lanes l and l+32 together cover
// the 16 k-values, with the same k assignment for A and B, so any fixed
// bijection between (l / 32, element) and k gives A*B.  The accumulator
// element j of lane l is C[8*(j/4) + 4*(l/32) + j%4][l % 32].
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// v_mfma_f32_32x32x16_f16: the same shape and lane layout for fp16 operands.
__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Vector types of a 16-bit element type (__bf16 or _Float16).
template <typename E>
struct Vec;
template <>
struct Vec<__bf16> {
  using v8 = bf16x8;
  using v4 = bf16x4;
};
template <>
struct Vec<_Float16> {
  using v8 = f16x8;
  using v4 = f16x4;
};

// Row index (within a 32x32 accumulator block) held by element j of lane l.
__device__ __forceinline__ int acc_row(int j, int lane) { return 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3); }

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float wave_swap32(float x) { return __shfl_xor(x, 32); }

// Max and sum over lanes l and l^32 (the two halves of a query row in the
// MFMA accumulator layout).
__device__ __forceinline__ float halves_max(float x) { return fmaxf(x, wave_swap32(x)); }
__device__ __forceinline__ float halves_sum(float x) { return x + wave_swap32(x); }

// XOR swizzle of 16-byte units within an LDS row, chosen so that 16
// consecutive rows read at the same logical unit hit 16 distinct 16-byte bank
// groups (and 8 consecutive rows hit 8 distinct groups of a 128-byte window).
//   rows of 16 units (256 B): unit ^ (row % 16)
//   rows of  8 units (128 B): unit ^ ((row ^ row/8) % 8)
template <int UNITS>
__device__ __forceinline__ int swz(int row, int unit) {
  if constexpr (UNITS == 16) return unit ^ (row & 15);
  else return unit ^ ((row ^ (row >> 3)) & 7);
}

// Bytes of one row of a K, V, Q or dO tile in LDS.  Rows in HBM are 2*D
// bytes; at d = 96 the LDS rows are padded to 256 bytes (12 of their 16
// units hold data) so that d = 128's swizzle applies unchanged.
template <int D>
constexpr int lds_row_bytes() {
  return D == 96 ? 256 : 2 * D;
}

// Swizzle of the 16-byte units of one row of a row-major K or V tile in LDS
// (d = 128 and 96: 16 units per 256-byte row; d = 64: 8 units per 128-byte
// row; d = 256: 32 units per 512-byte row, d = 128's table on the low four
// bits of the unit).
// Physical unit = logical unit ^ tile_swz<D>(row).  The tables were chosen so
// that both access patterns of the tiles hit distinct banks, whether the LDS
// serves 16 lanes x 16 bytes or 8 lanes x 16 bytes per cycle:
//  * 128-bit row reads: 32 consecutive rows, one logical unit;
//  * ds_read_b64_tr_b16: per 16-lane group, 4 consecutive rows x 32 bytes.
template <int D>
__device__ __forceinline__ int tile_swz(int row) {
  const int r = row & 15;
  if constexpr (D == 256) {
    return tile_swz<128>(row);
  } else if constexpr (D == 128 || D == 96) {
    const int i = r & 3;  // {0, 6, 10, 12}[i] ^ (r / 4)
    const int p = ((i >> 1) << 3) | ((i & 1) << 2) | (((i ^ (i >> 1)) & 1) << 1);
    return p ^ (r >> 2);
  } else {
    return ((2 * (r & 3)) | ((r >> 2) & 1)) ^ (((r >> 3) & 1) << 1);
  }
}

// Buffer resource over `bytes` bytes at `base`: loads past the end return 0,
// stores past the end are dropped (gfx9 descriptor word 3).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// 16 bytes per lane from a buffer straight into LDS: lane l writes
// lds[16*l .. 16*l+15] (the LDS address is wave-uniform).  The host pass only
// emits the kernel's launch stub, so the builtin is compiled for the device
// alone (its presence in the host pass suppresses the stub).
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, void* lds, int voffset) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, voffset, 0, 0, 0);
#endif
}

// Source byte offset, within HBM rows of 2*D bytes, of the 16 bytes that a
// direct load places at byte p of a row-major LDS tile (rows of
// lds_row_bytes<D>()): LDS unit (row, pu) holds logical unit
// pu ^ tile_swz<D>(row) of that row.  Padding units (d = 96) get an offset
// past every buffer, so their loads read zeros and touch no memory.
template <int D>
__device__ __forceinline__ int swz_src(int p) {
  constexpr int LRS = lds_row_bytes<D>();
  const int row = p / LRS, pu = (p % LRS) / 16;
  const int lu = pu ^ tile_swz<D>(row);
  return lu < D / 8 ? row * (2 * D) + lu * 16 : 0x7fffff00;
}

// Pack two fp32 values into two bf16 (round to nearest even) in one dword.
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  __bf16 a = (__bf16)lo, b = (__bf16)hi;
  unsigned short ua = __builtin_bit_cast(unsigned short, a);
  unsigned short ub = __builtin_bit_cast(unsigned short, b);
  return unsigned(ua) | (unsigned(ub) << 16);
}

// Pack two fp32 values into two 16-bit values of type E (round to nearest
// even) in one dword.
template <typename E>
__device__ __forceinline__ unsigned pack2(float lo, float hi) {
  E a = (E)lo, b = (E)hi;
  unsigned short ua = __builtin_bit_cast(unsigned short, a);
  unsigned short ub = __builtin_bit_cast(unsigned short, b);
  return unsigned(ua) | (unsigned(ub) << 16);
}

// ---------------------------------------------------------------------------
// Dropout bits.  Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC 2011): ten rounds on a 128-bit counter and
// a 64-bit key; a round forms the 64-bit products c0*0xD2511F53 and
// c2*0xCD9E8D57 and returns (hi(c2*M1)^c1^k0, lo(c2*M1), hi(c0*M0)^c3^k1,
// lo(c0*M0)); the key is bumped by 0x9E3779B9 and 0xBB67AE85 between rounds.
//
// Element (b, h, i, j) of P belongs to the 4 x 4 block (i/4, j/4), whose call
// has counter (i/4, j/4, b*H+h, 0) and key (seed lo, seed hi); word i%4, byte
// j%4 (little-endian) is the element's 8-bit draw, and the element is kept
// iff the draw is >= t.  Kept probabilities are scaled by keep_scale.
// ---------------------------------------------------------------------------
struct DropArgs {
  unsigned t;        // 8-bit threshold, 0..255 (0: keep everything)
  float keep_scale;  // 1 / (1 - t/256)
  unsigned k0, k1;   // the seed
};

// Host side: threshold t = round(256 p) clamped to [0, 255], so the
// effective drop probability is t / 256, and keep_scale = 1 / (1 - t/256).
inline DropArgs make_drop_args(float p, unsigned long long seed) {
  double t = std::floor(256.0 * double(p) + 0.5);
  if (t < 0.0) t = 0.0;
  if (t > 255.0) t = 255.0;
  DropArgs d;
  d.t = unsigned(t);
  d.keep_scale = float(1.0 / (1.0 - t / 256.0));
  d.k0 = unsigned(seed & 0xFFFFFFFFull);
  d.k1 = unsigned(seed >> 32);
  return d;
}

__device__ __forceinline__ u32x4 philox4x32_10(unsigned c0, unsigned c1, unsigned c2, unsigned c3, unsigned k0,
                                               unsigned k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const unsigned long long p0 = (unsigned long long)c0 * 0xD2511F53u;
    const unsigned long long p1 = (unsigned long long)c2 * 0xCD9E8D57u;
    const unsigned n0 = unsigned(p1 >> 32) ^ c1 ^ k0;
    const unsigned n2 = unsigned(p0 >> 32) ^ c3 ^ k1;
    c1 = unsigned(p1);
    c3 = unsigned(p0);
    c0 = n0;
    c2 = n2;
  }
  return u32x4{c0, c1, c2, c3};
}

// Keep bits (bit e = element e) of the 4 elements of one row and 4 consecutive
// columns of a 4 x 4 block: query `i`, keys 4*j4 .. 4*j4+3.
__device__ __forceinline__ unsigned keep_row4(const DropArgs& dp, unsigned i, unsigned j4, unsigned bh) {
  const u32x4 w = philox4x32_10(i >> 2, j4, bh, 0u, dp.k0, dp.k1);
  const unsigned s = i & 3u;
  const unsigned word = s == 0 ? w[0] : s == 1 ? w[1] : s == 2 ? w[2] : w[3];
  unsigned bits = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) bits |= unsigned(((word >> (8 * e)) & 0xFFu) >= dp.t) << e;
  return bits;
}

// Keep bits of the 4 elements of one column and 4 consecutive rows of a block:
// queries 4*i4 .. 4*i4+3 (bit e = query 4*i4+e), key `j`.
__device__ __forceinline__ unsigned keep_col4(const DropArgs& dp, unsigned i4, unsigned j, unsigned bh) {
  const u32x4 w = philox4x32_10(i4, j >> 2, bh, 0u, dp.k0, dp.k1);
  const unsigned sh = 8 * (j & 3u);
  unsigned bits = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) bits |= unsigned(((w[e] >> sh) & 0xFFu) >= dp.t) << e;
  return bits;
}

// Keep bits of a whole 4 x 4 block, from one call: bit 4*e + b says whether
// element (row 4*i4 + e, column 4*j4 + b) survives (word e, byte b).
__device__ __forceinline__ unsigned keep_block_rows(const DropArgs& dp, unsigned i4, unsigned j4, unsigned bh) {
  const u32x4 w = philox4x32_10(i4, j4, bh, 0u, dp.k0, dp.k1);
  unsigned bits = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int b = 0; b < 4; ++b) bits |= unsigned(((w[e] >> (8 * b)) & 0xFFu) >= dp.t) << (4 * e + b);
  return bits;
}

// The same block with the bits transposed: bit 4*b + e.
__device__ __forceinline__ unsigned keep_block_cols(const DropArgs& dp, unsigned i4, unsigned j4, unsigned bh) {
  const u32x4 w = philox4x32_10(i4, j4, bh, 0u, dp.k0, dp.k1);
  unsigned bits = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int b = 0; b < 4; ++b) bits |= unsigned(((w[e] >> (8 * b)) & 0xFFu) >= dp.t) << (4 * b + e);
  return bits;
}

// x if bit `bit` of `bits` is set, else +0: the bit is sign-extended into an
// all-ones or all-zeros mask (one bit-field extract, no compare or select).
__device__ __forceinline__ float keep_or_zero(float x, unsigned bits, int bit) {
  const unsigned m = unsigned(int(bits << (31 - bit)) >> 31);
  return __builtin_bit_cast(float, __builtin_bit_cast(unsigned, x) & m);
}

// x as held by lane M of this lane's quad (lanes 4q .. 4q+3): a DPP
// quad_perm broadcast, VALU only.  Every lane of the quad must be active.
template <int M>
__device__ __forceinline__ unsigned quad_bcast(unsigned x) {
  return (unsigned)__builtin_amdgcn_mov_dpp((int)x, M * 0x55, 0xF, 0xF, false);
}

// The four lanes of a quad that need the same four Philox calls make one
// each and share the results: lane t of the quad draws block `blk(t)` (16
// keep bits, laid out so that the 4 bits lane t' needs are bits
// 4*t' .. 4*t'+3) and every lane takes its nibble of each lane's block.
// Returns nibble m (for the block drawn by lane m) at bits 4*m .. 4*m+3.
__device__ __forceinline__ unsigned quad_share_nibbles(unsigned mine, unsigned t) {
  const unsigned sh = 4 * t;
  return ((quad_bcast<0>(mine) >> sh) & 0xFu) | (((quad_bcast<1>(mine) >> sh) & 0xFu) << 4) |
         (((quad_bcast<2>(mine) >> sh) & 0xFu) << 8) | (((quad_bcast<3>(mine) >> sh) & 0xFu) << 12);
}

// Tile-skipping masks (beyond causal), shared by the forward and backward.
// kMaskWindow: key j is visible to query i iff i - left <= j <= i + right (a
// negative bound: no limit on that side).  kMaskBlocks: bm[h][i / 64][j / 64] != 0 keeps the 64 x 64 block,
// with the causal mask on top when CAUSAL; bm_head_stride is 0 when all
// heads share one mask.
enum : int { kMaskDense = 0, kMaskWindow = 1, kMaskBlocks = 2 };
constexpr int kMaskBlock = 64;
constexpr int kMaxMaskTiles = 1024;  // block-sparse: N <= 65536

// Entries of a workgroup's block-sparse tile (or step) list: the index in
// bits 0-13 and, in bits 14 and 15, whether the mask keeps that tile for the
// workgroup's first and second 64-row (or 64-key) block.  A wave then learns
// whether its own block keeps a tile from the list in LDS, with no load from
// the mask inside the sweep.
static_assert(kMaxMaskTiles <= (1 << 14), "list indices fit in 14 bits");
__device__ __forceinline__ unsigned short list_entry(int index, bool first, bool second) {
  return (unsigned short)(index | (int(first) << 14) | (int(second) << 15));
}
__device__ __forceinline__ int list_index(unsigned short e) { return e & 0x3FFF; }
__device__ __forceinline__ bool list_keeps(unsigned short e, int block) { return (e >> (14 + block)) & 1; }
struct MaskArgs {
  int left, right;
  const unsigned char* bm;
  long long bm_head_stride;
  int nb, H;
};

// Whether the window hides key `key` from query `q`.
__device__ __forceinline__ bool window_hides(const MaskArgs& mk, int q, int key) {
  return (mk.left >= 0 && key < q - mk.left) || (mk.right >= 0 && key > q + mk.right);
}

// Calls f(std::integral_constant<int, 0>{}), ..., f(std::integral_constant<int, N-1>{})
// in order, so that every index inside f is a compile-time constant.
template <typename F, int... Is>
__device__ __forceinline__ void static_for_seq(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_seq(f, std::make_integer_sequence<int, N>{});
}

// Map a linear workgroup id to a tile id so that the tiles of one (b, h)
// head are contiguous within one XCD: workgroups are handed to the 8 XCDs
// round-robin, so id w runs on XCD w % 8.  When the grid is not a multiple of
// 8 the identity is used.
__device__ __forceinline__ int xcd_remap(int w, int G) {
  if ((G & 7) != 0) return w;
  return (w & 7) * (G >> 3) + (w >> 3);
}

// Causal grids (BH heads x T blocks, block rank r of a head has T - r units
// of work: key tiles of a query block, or query steps of a key block):
// block w -> (head bh, rank r, 0 = the head's longest).
// When BH is a multiple of the 8 XCDs, XCD x = w % 8 takes the heads
// bh = x (mod 8) -- their K and V stay in that XCD's L2 -- and dispatches
// its blocks longest first over all of those heads, so that the short blocks
// of every head fill in at the end.  (Head by head, each XCD would start a
// new head's long blocks while its other CUs run short ones, and finish
// unevenly.)  Otherwise: xcd_remap order, longest first within a head.
__device__ __forceinline__ void causal_order(int w, int BH, int T, int& bh, int& r) {
  if ((BH & 7) == 0) {
    const int x = w & 7, k = w >> 3, hp = BH >> 3;
    r = k / hp;
    bh = x + 8 * (k - r * hp);
  } else {
    const int t = xcd_remap(w, BH * T);
    bh = t / T;
    r = t - bh * T;
  }
}

}  // namespace fa

#endif  // FA_COMMON_H_
