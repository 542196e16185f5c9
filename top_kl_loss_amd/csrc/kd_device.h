// Device helpers shared by the kernel translation units (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kd {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// bf16 <-> fp32.  bf16 values are carried as their 16-bit patterns.
__device__ __forceinline__ float bf16_lo(uint32_t w) {
  return __uint_as_float(w << 16);
}
__device__ __forceinline__ float bf16_hi(uint32_t w) {
  return __uint_as_float(w & 0xffff0000u);
}
// Round to nearest, ties to even (inputs here are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// Two fp32 -> packed bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// Element-type traits: bf16 (stored as uint16_t) or fp32.
template <typename T> struct Elem;
template <> struct Elem<uint16_t> {
  static constexpr int PER16B = 8;
  __device__ static __forceinline__ float to_f(uint16_t v) {
    return __uint_as_float(uint32_t(v) << 16);
  }
  __device__ static __forceinline__ uint16_t from_f(float x) {
    return uint16_t(f32_to_bf16_rne(x));
  }
  // Multiply the 8 values of a 16-byte chunk by s.
  __device__ static __forceinline__ u32x4 scale(u32x4 v, float s) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      r[i] = pack_bf16x2(bf16_lo(v[i]) * s, bf16_hi(v[i]) * s);
    return r;
  }
};
template <> struct Elem<float> {
  static constexpr int PER16B = 4;
  __device__ static __forceinline__ float to_f(float v) { return v; }
  __device__ static __forceinline__ float from_f(float x) { return x; }
  __device__ static __forceinline__ u32x4 scale(u32x4 v, float s) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = __float_as_uint(__uint_as_float(v[i]) * s);
    return r;
  }
};

// Linear workgroup id -> id in an order where consecutive ids run on the
// same XCD (the hardware deals workgroups round-robin over the 8 XCDs of the
// chip), so tiles that share an operand share an L2.
__device__ __forceinline__ int xcd_swizzle(int bid, int n) {
  constexpr int NX = 8;
  const int per = (n + NX - 1) / NX;
  const int tall = n % NX == 0 ? NX : n % NX;
  const int x = bid % NX, local = bid / NX;
  return x < tall ? x * per + local : tall * per + (x - tall) * (per - 1) + local;
}

// Reductions over each aligned group of 8 consecutive lanes, the result in
// all 8 (DPP lane moves: swap neighbours, swap pairs within the quad, then
// mirror within the half row, lane i <- 7 - i).  Every lane of a group ends
// with the same bits (each step adds two values in either order).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float group8_max(float v) {
  v = fmaxf(v, dpp_mov<0xB1>(v));   // quad_perm [1, 0, 3, 2]
  v = fmaxf(v, dpp_mov<0x4E>(v));   // quad_perm [2, 3, 0, 1]
  return fmaxf(v, dpp_mov<0x141>(v));  // row_half_mirror
}
__device__ __forceinline__ float group8_sum(float v) {
  v += dpp_mov<0xB1>(v);
  v += dpp_mov<0x4E>(v);
  return v + dpp_mov<0x141>(v);
}

// Integer forms: the sum over each group of 8 lanes (in all 8), and the
// inclusive prefix sum over it (g = the lane's index in its group; DPP
// row shifts by 1, 2, 4 with out-of-row sources read as 0, and a lane adds
// only what comes from its own group).
template <int CTRL>
__device__ __forceinline__ int dpp_mov_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, true);
}
__device__ __forceinline__ int group8_sum_i(int v) {
  v += dpp_mov_i<0xB1>(v);
  v += dpp_mov_i<0x4E>(v);
  return v + dpp_mov_i<0x141>(v);
}
__device__ __forceinline__ int group8_scan_i(int v, int g) {
  int y = dpp_mov_i<0x111>(v);  // row_shr:1
  if (g >= 1) v += y;
  y = dpp_mov_i<0x112>(v);      // row_shr:2
  if (g >= 2) v += y;
  y = dpp_mov_i<0x114>(v);      // row_shr:4
  if (g >= 4) v += y;
  return v;
}

// Wave-wide (64-lane) reductions through cross-lane shuffles.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace kd
