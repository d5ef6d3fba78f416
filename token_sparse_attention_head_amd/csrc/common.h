// Device helpers shared by the token-sparse attention kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tsa.h"

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define TSA_WAVE 64
#define TSA_LOG2E 1.4426950408889634f

namespace tsa {

// ---- element conversions -------------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Round to nearest even (hardware v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  __bf16 b = static_cast<__bf16>(f);
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// ---- 16-byte global access -----------------------------------------------------------

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
// Streaming variants (non-temporal): data touched once.
__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st16_nt(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// ---- wave helpers ----------------------------------------------------------------------

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Value from lane (l ^ 32).
__device__ __forceinline__ float xor32(float x) {
  return __shfl_xor(x, 32, TSA_WAVE);
}

// ---- MFMA wrappers ---------------------------------------------------------------------
// 32x32 output tiles.  Lane l holds output column (l % 32) and rows
// 8*(r/4) + 4*(l/32) + (r%4) for r = 0..15.  Operand A: lane l supplies row (l % 32);
// operand B: lane l supplies column (l % 32); lanes l < 32 and l >= 32 supply the two
// halves of the contraction slice of one instruction.

__device__ __forceinline__ f32x16 mfma(f32x16 c, bf16x8 a, bf16x8 b) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma(f32x16 c, float a, float b) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Operand fragments of one lane's half of a head-dim row, for the contraction over d.
// The contraction index is permuted so that lane half hf covers d in
// [hf*D/2, (hf+1)*D/2) contiguously; both operands use the same permutation, which
// leaves every dot product unchanged.
template <typename T, int D> struct HalfRow;

template <int D> struct HalfRow<__bf16, D> {
  static constexpr int STEPS = D / 16;          // 32x32x16 instructions per dot product
  static constexpr int VEC16 = D / 16;          // 16-byte vectors in a half row (8 bf16 each)
  bf16x8 f[STEPS];
  __device__ __forceinline__ void load(const __bf16* row_half) {
#pragma unroll
    for (int s = 0; s < STEPS; ++s) f[s] = *reinterpret_cast<const bf16x8*>(row_half + 8 * s);
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int s = 0; s < STEPS; ++s) f[s] = bf16x8{};
  }
  __device__ __forceinline__ bf16x8 step(int s) const { return f[s]; }
};

template <int D> struct HalfRow<float, D> {
  static constexpr int STEPS = D / 2;           // 32x32x2 instructions per dot product
  float f[STEPS];
  __device__ __forceinline__ void load(const float* row_half) {
#pragma unroll
    for (int s = 0; s < STEPS; s += 4) {
      f32x4 v = *reinterpret_cast<const f32x4*>(row_half + s);
      f[s] = v[0]; f[s + 1] = v[1]; f[s + 2] = v[2]; f[s + 3] = v[3];
    }
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int s = 0; s < STEPS; ++s) f[s] = 0.f;
  }
  __device__ __forceinline__ float step(int s) const { return f[s]; }
};

// acc += A . B^T over d, where A and B are half-row fragments (A rows, B columns).
template <typename T, int D>
__device__ __forceinline__ f32x16 dot_tile(f32x16 acc, const HalfRow<T, D>& a, const HalfRow<T, D>& b) {
#pragma unroll
  for (int s = 0; s < HalfRow<T, D>::STEPS; ++s) acc = mfma(acc, a.step(s), b.step(s));
  return acc;
}

// Row of the 32x32 output tile held in accumulator slot r by a lane in half hf.
__device__ __forceinline__ int acc_row(int r, int hf) { return 8 * (r >> 2) + 4 * hf + (r & 3); }

}  // namespace tsa
