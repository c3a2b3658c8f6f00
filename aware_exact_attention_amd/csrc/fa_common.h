// fa_common.h - device-side types and helpers shared by the gfx950 kernels.
#ifndef FA_COMMON_H_
#define FA_COMMON_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

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

// Swizzle of the 16-byte units of one row of a row-major K or V tile in LDS
// (d = 128: 16 units per 256-byte row; d = 64: 8 units per 128-byte row).
// Physical unit = logical unit ^ tile_swz<D>(row).  The tables were chosen so
// that both access patterns of the tiles hit distinct banks, whether the LDS
// serves 16 lanes x 16 bytes or 8 lanes x 16 bytes per cycle:
//  * 128-bit row reads: 32 consecutive rows, one logical unit;
//  * ds_read_b64_tr_b16: per 16-lane group, 4 consecutive rows x 32 bytes.
template <int D>
__device__ __forceinline__ int tile_swz(int row) {
  const int r = row & 15;
  if constexpr (D == 128) {
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

// Map a linear workgroup id to a tile id so that the tiles of one (b, h)
// head are contiguous within one XCD: workgroups are handed to the 8 XCDs
// round-robin, so id w runs on XCD w % 8.  When the grid is not a multiple of
// 8 the identity is used.
__device__ __forceinline__ int xcd_remap(int w, int G) {
  if ((G & 7) != 0) return w;
  return (w & 7) * (G >> 3) + (w >> 3);
}

}  // namespace fa

#endif  // FA_COMMON_H_
