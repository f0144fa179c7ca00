// gfx950 (CDNA4) building blocks shared by the attention kernels: vector types, the
// bf16 MFMA, wave-half exchange, exp2 and bf16 packing.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hc {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// D(32x32) += A(32x16) * B(16x32), bf16 inputs, fp32 accumulate.
// Lane l supplies A row (l % 32) and B column (l % 32), 8 consecutive k values each
// for its half (l / 32). Output register r of lane l holds
// D[8*(r/4) + 4*(l/32) + (r%4)][l % 32].
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Reductions across the two halves of the wave (lane l with lane l ^ 32). The swap
// returns this lane's value and its partner's, in an order that depends on the half,
// so only order-free combinations of the pair are formed.
__device__ __forceinline__ float max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Two fp32 -> packed bf16 pair (round to nearest even), lo in bits 0..15.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t x) {
  return __uint_as_float(((uint32_t)x) << 16);
}

// Position of key k (0..63) inside a transposed V tile. The PV product takes its B
// operand straight from the score registers, whose lane half h holds keys
// {8a + 4h + b}; storing key bits (a,h) swapped makes each lane's 8 keys contiguous.
__device__ __forceinline__ int vt_pos(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

// 16-bit element j of a row of 8 bf16 held in 4 dwords.
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);   // a.lo | b.lo << 16
}
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);   // a.hi | b.hi << 16
}

// Workgroup id -> logical index in [0, total) such that the workgroups of one XCD
// (ids x, x + 8, x + 16, ...) take one contiguous block of logical indices.
__device__ __forceinline__ int xcd_block(int bid, int total) {
  const int x = bid & 7, k = bid >> 3;
  const int q = total >> 3, r = total & 7;
  return x * q + min(x, r) + k;
}

}  // namespace hc
