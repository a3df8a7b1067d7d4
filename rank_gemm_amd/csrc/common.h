// common.h -- device-side helpers shared by the gfx950 kernels of liblora.so.
//
// Vector types for MFMA operands, bf16 <-> fp32 conversion, and the MFMA
// wrappers.  Lane layouts of the MFMA instructions used here (64-wide wave):
//   v_mfma_f32_16x16x32_bf16: lane l holds A row (l % 16), k = 8*(l / 16) + i,
//       B column (l % 16), same k; accumulator column (l % 16),
//       rows 4*(l / 16) + i, i < 4.
//   v_mfma_f32_16x16x16_bf16: as above with k = 4*(l / 16) + i, i < 4.
//   v_mfma_f32_16x16x4_f32:   A row (l % 16), k = l / 16; B column (l % 16),
//       k = l / 16; accumulator as above.
// ds_read_b64_tr_b16 (measured on gfx950): within each group of 16 lanes, if
// lane i addresses the 4 bf16 values M[i][0..3], lane j receives
// M[4q + j/4][j%4] for q = 0..3.  So when lane i of a group points at row
// r0 + i/4, column c0 + 4 (i%4) of a row-major LDS tile, lane j receives
// rows r0..r0+3 of column c0 + j: an MFMA operand whose contraction index runs
// down the rows, built without a transposed copy.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lora {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf2f(uint16_t h) {
  return __builtin_bit_cast(float, static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16, round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  return static_cast<uint32_t>(f2bf(lo)) | (static_cast<uint32_t>(f2bf(hi)) << 16);
}

__device__ __forceinline__ f32x4 mfma16x16x32(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16x16x16(const u32x2& a, const u32x2& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                   __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16x16x4f32(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

// Buffer offset for a lane that must read zeros: past every valid range.
__device__ __forceinline__ uint32_t off_or_oob(bool in, uint32_t off) { return in ? off : 0x80000000u; }

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// lgkmcnt(0): this wave's LDS reads (and scalar loads) have returned.
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt((63 & 15) | ((63 >> 4) << 14) | (7 << 4) | (0 << 8));
}

// A wave-uniform value kept in a scalar register: stops loop-invariant code
// motion from precomputing one vector offset per load slot.
__device__ __forceinline__ uint32_t sgpr(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

// One transposing LDS read (see the lane layout above); p is an LDS address.
__device__ __forceinline__ u32x2 lds_read_tr16(const void* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p));
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Workgroups are handed to the 8 XCDs round-robin (id % 8).  When the grid
// divides evenly, renumber so that each XCD receives one contiguous range of
// tile ids: neighbouring tiles then share that XCD's L2.
__device__ __forceinline__ int xcd_contiguous_id(int id, int total) {
  if ((total & 7) != 0) return id;
  const int per = total >> 3;
  return (id & 7) * per + (id >> 3);
}

}  // namespace lora
