// Block-level selection helpers (256-thread workgroups): an order-preserving
// 64-bit key for (fp32 value, index) pairs, a workgroup prefix sum, radix
// selection of the r-th smallest key and a bitonic sort in LDS.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace kd {
namespace sel {

// ------------------------------------------------------------------ keys
__device__ __forceinline__ uint32_t key_hi(float v) {
  uint32_t u = __float_as_uint(v);
  if ((u << 1) == 0u) u = 0u;  // -0 -> +0
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ~ord;
}
__device__ __forceinline__ float key_val(uint32_t hi) {
  const uint32_t ord = ~hi;
  return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7fffffffu) : ~ord);
}
__device__ __forceinline__ uint64_t make_key(float v, int id) {
  return (uint64_t(key_hi(v)) << 32) | uint32_t(id);
}

// --------------------------------------------------- block-wide helpers
// (256-thread workgroups)

// Inclusive prefix sum of x over the workgroup in thread order; sc holds
// at least 4 words.
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t x, uint32_t *sc) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) sc[wave] = x;
  __syncthreads();
  uint32_t off = 0;
  for (int w = 0; w < wave; ++w) off += sc[w];
  return x + off;
}

// The r-th smallest (0-based) of n distinct 64-bit keys key_at(0..n-1), by
// most-significant-byte-first radix selection: one 256-bin histogram per
// byte over the keys that match the bytes chosen so far.  Needs r < n.
// hist: 256 words, sc: 8 words, res: one key, all in LDS.
template <class KeyAt>
__device__ __forceinline__ uint64_t block_select(KeyAt key_at, int n, int r, uint32_t *hist, uint32_t *sc,
                                 uint64_t *res) {
  const int tid = threadIdx.x;
  uint64_t prefix = 0, mask = 0;
  for (int shift = 56; shift >= 0; shift -= 8) {
    hist[tid] = 0u;
    __syncthreads();
    for (int i = tid; i < n; i += 256) {
      const uint64_t k = key_at(i);
      if ((k & mask) == prefix) atomicAdd(&hist[uint32_t(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    const uint32_t h = hist[tid];
    const uint32_t incl = block_incl_scan(h, sc);
    const uint32_t excl = incl - h;
    if (excl <= uint32_t(r) && uint32_t(r) < incl) {
      sc[4] = uint32_t(tid);
      sc[5] = uint32_t(r) - excl;
      sc[6] = h;
    }
    __syncthreads();
    const uint32_t b = sc[4], hb = sc[6];
    r = int(sc[5]);
    prefix |= uint64_t(b) << shift;
    mask |= uint64_t(0xffu) << shift;
    __syncthreads();
    if (hb == 1u && shift > 0) {
      // one key left in the chosen bucket: it is the answer
      for (int i = tid; i < n; i += 256) {
        const uint64_t k = key_at(i);
        if ((k & mask) == prefix) *res = k;
      }
      __syncthreads();
      const uint64_t out = *res;
      __syncthreads();
      return out;
    }
  }
  return prefix;
}

// Ascending bitonic sort of n (a power of two) keys in LDS.  The caller
// synchronises before the call; the sorted keys are visible to all threads
// on return.
__device__ __forceinline__ void bitonic_sort(uint64_t *s, int n) {
  for (int k = 2; k <= n; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int t = threadIdx.x; t < n / 2; t += blockDim.x) {
        const int lo = ((t & ~(j - 1)) << 1) | (t & (j - 1)), hi = lo + j;
        const bool up = (lo & k) == 0;
        const uint64_t x = s[lo], y = s[hi];
        if ((x > y) == up) {
          s[lo] = y;
          s[hi] = x;
        }
      }
      __syncthreads();
    }
}

__device__ __forceinline__ int pow2_at_least(int n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

}  // namespace sel
}  // namespace kd
