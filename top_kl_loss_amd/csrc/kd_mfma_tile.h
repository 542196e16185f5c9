// Matrix-core tile machinery shared by the tuned bf16 GEMMs (gfx950).
//
// Workgroup: 512 threads = 8 waves (2 per SIMD) as 2 (M) x 4 (N); tile
// 256 x 256, wave tile 128 x 64 = 4 x 2 blocks of v_mfma_f32_32x32x16_bf16
// with fp32 accumulators.  Two waves per SIMD let the hardware interleave
// one wave's LDS/VMEM/VALU work with the other's MFMAs.  One k-step is 64
// bf16 of the contraction, double-buffered in LDS (2 x 64 KiB).
//
// Every operand tile sits in LDS as rows of 64 contraction elements (128
// bytes), 16-byte chunk c of row r at r*128 + ((c ^ swz(r)) * 16) with
// swz(r) = (r ^ (r >> 3)) & 7, and MFMA fragments are read with
// ds_read_b128.  Operands whose contraction index is contiguous in memory are
// copied HBM -> LDS with buffer_load_dwordx4 ... lds (reads past the buffer
// end return zero); the others are read as 8 x 4 bf16 blocks into registers,
// transposed with v_perm_b32 and written with ds_write_b128.
#pragma once

#include <stdint.h>

#include "kd_device.h"

namespace kd {
namespace tile {

constexpr int NT = 512;
constexpr int BM = 256, BN = 256, BK = 64;
constexpr int WN = 4, WTM = 128, WTN = 64, TM = 4, TN = 2;
constexpr int OP_BYTES = 256 * 128;          // one operand tile per stage
constexpr int STAGE_BYTES = 2 * OP_BYTES;    // A then B
constexpr int LDS_BYTES = 2 * STAGE_BYTES;   // 128 KiB

// Tile shapes with 256 rows of A: 8 waves as (8/WN_) x WN_, each wave
// TM_ x TN_ blocks of 32 x 32.  Square: 256 x 256 (the default above);
// Wide: 256 x 320 for N = d multiple of 320 (d = 2880 = 9 x 320 wastes no
// MFMA work on padding, where 256-wide tiles waste 6.25%).
template <int WN_, int TM_, int TN_>
struct TileCfg {
  static constexpr int WN = WN_, TM = TM_, TN = TN_;
  static constexpr int WTM = TM_ * 32, WTN = TN_ * 32;
  static constexpr int BN = WN_ * WTN;
  static constexpr int LDS = 2 * (256 + BN) * 128;
  static_assert((8 / WN_) * WTM == 256, "256 rows of A");
};
using SquareCfg = TileCfg<4, 4, 2>;
using WideCfg = TileCfg<2, 2, 5>;
static_assert(WideCfg::BN == 320 && WideCfg::LDS <= 160 * 1024, "wide tile");

// Width of the N tile that wastes the least MFMA work on a dimension of n.
inline int best_bn(int n) {
  const int w256 = (n + 255) / 256 * 256 - n, w320 = (n + 319) / 320 * 320 - n;
  return w320 < w256 ? 320 : 256;
}

typedef __attribute__((address_space(3))) void *lds_vptr;

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_res(const void *base,
                                                           uint64_t bytes) {
  const uint32_t n = bytes > 0xffffffffull ? 0xffffffffu : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0,
                                           (int)n, 0x00020000);
}

__device__ __forceinline__ void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ------------------------------------------------------------- operand copy
// K-contiguous operand, element (mn, k) at byte (mn * ld + k) * 2 of `res`,
// ROWS rows copied by NW waves (index w among them), each issuing
// ROWS/8/NW instructions of 1 KiB (8 rows x 128 B) per k-step.
template <int NW, int ROWS = 256>
struct CopyK {
  static constexpr int N = ROWS / 8 / NW;
  static_assert(N * 8 * NW == ROWS, "rows per wave");
  __amdgpu_buffer_rsrc_t res;
  uint32_t off[N];
  int w;
  __device__ __forceinline__ void init(const void *base, uint64_t bytes, int64_t ld,
                                       int mn0, int w_, int lane) {
    res = make_res(base, bytes);
    w = w_;
#pragma unroll
    for (int n = 0; n < N; ++n) {
      const int p = (w * N + n) * 64 + lane;  // 16-byte position in the tile
      const int row = p >> 3, pc = p & 7;
      const int lc = pc ^ swz(row);
      off[n] = (uint32_t)(((int64_t)(mn0 + row) * ld + lc * 8) * 2);
    }
  }
  __device__ __forceinline__ void issue(char *tile, int k0) {
#pragma unroll
    for (int n = 0; n < N; ++n)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(res, (lds_vptr)(tile + (w * N + n) * 1024), 16,
                                               (int)(off[n] + k0 * 2), 0, 0, 0);
  }
};

// MN-contiguous operand, element (mn, k) at base[k * ld + mn], through
// registers: thread t (of 512) owns the 8 (k) x 4 (mn) block (mn block
// t % 64, k block t / 64) of the 256 x 64 tile; it reads 8 rows of 8 bytes,
// transposes them with v_perm_b32 and writes 4 rows of 16 bytes (8
// consecutive k of one mn).  Elements outside mn < mn_lim, k < k_lim are 0.
struct RegMN4 {
  const uint16_t *base;
  int64_t ld;
  int mn, kb, mn_lim, k_lim;
  uint32_t r[8][2];
  __device__ __forceinline__ void init(const uint16_t *b, int64_t ld_, int mn0, int mn_lim_,
                                       int k_lim_, int t) {
    base = b;
    ld = ld_;
    mn = mn0 + (t & 63) * 4;
    kb = (t >> 6) * 8;
    mn_lim = mn_lim_;
    k_lim = k_lim_;
  }
  __device__ __forceinline__ void load(int k0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int k = k0 + kb + e;
      if (k < k_lim && mn < mn_lim) {
        const uint2 v = *reinterpret_cast<const uint2 *>(base + (int64_t)k * ld + mn);
        r[e][0] = v.x;
        r[e][1] = v.y;
      } else {
        r[e][0] = r[e][1] = 0u;
      }
    }
  }
  __device__ __forceinline__ void store(char *tile, int t) {
    const int row0 = (t & 63) * 4, ch = t >> 6;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      u32x4 o;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t lo = r[2 * p][m >> 1], hi = r[2 * p + 1][m >> 1];
        o[p] = (m & 1) ? __builtin_amdgcn_perm(hi, lo, 0x07060302u)
                       : __builtin_amdgcn_perm(hi, lo, 0x05040100u);
      }
      const int row = row0 + m;
      *reinterpret_cast<u32x4 *>(tile + row * 128 + ((ch ^ swz(row)) << 4)) = o;
    }
  }
};

// 8 consecutive k (16 bytes) of tile row `row`, k-group g, half h.
__device__ __forceinline__ u32x4 frag(const char *tile, int row, int g, int h) {
  return *reinterpret_cast<const u32x4 *>(tile + row * 128 + (((2 * g + h) ^ swz(row)) << 4));
}

__device__ __forceinline__ void mfma(f32x16 &acc, u32x4 a, u32x4 b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}

__device__ __forceinline__ int acc_row(int e, int lane) {
  return 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
}

template <int TM_, int TN_>
__device__ __forceinline__ void zero_acc(f32x16 (&acc)[TM_][TN_]) {
#pragma unroll
  for (int i = 0; i < TM_; ++i)
#pragma unroll
    for (int j = 0; j < TN_; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
}

// One k-step on fragments double-buffered in registers: group g+1's
// fragments are read from LDS while group g's MFMAs run.  The scheduling
// barriers pin the order (one MFMA, one fragment read, ...) that keeps the
// matrix pipe fed; the compiler's own order serialises reads and MFMAs.
template <int TM_, int TN_>
__device__ __forceinline__ void kstep(const char *ta, const char *tb, int ar, int br, int h,
                                      f32x16 (&acc)[TM_][TN_]) {
  constexpr int NRD = TM_ + TN_;  // fragment reads per group
  static_assert(TM_ * TN_ >= NRD, "more reads than MFMAs per group");
  u32x4 fa[2][TM_], fb[2][TN_];
#pragma unroll
  for (int i = 0; i < TM_; ++i) fa[0][i] = frag(ta, ar + i * 32, 0, h);
#pragma unroll
  for (int j = 0; j < TN_; ++j) fb[0][j] = frag(tb, br + j * 32, 0, h);
  __builtin_amdgcn_sched_group_barrier(0x100, NRD, 0);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int c = g & 1;
    if (g < 3) {
#pragma unroll
      for (int i = 0; i < TM_; ++i) fa[c ^ 1][i] = frag(ta, ar + i * 32, g + 1, h);
#pragma unroll
      for (int j = 0; j < TN_; ++j) fb[c ^ 1][j] = frag(tb, br + j * 32, g + 1, h);
    }
#pragma unroll
    for (int i = 0; i < TM_; ++i)
#pragma unroll
      for (int j = 0; j < TN_; ++j) mfma(acc[i][j], fa[c][i], fb[c][j]);
    if (g < 3) {
#pragma unroll
      for (int r = 0; r < NRD; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
      }
      if (TM_ * TN_ > NRD) __builtin_amdgcn_sched_group_barrier(0x008, TM_ * TN_ - NRD, 0);
    } else {
      __builtin_amdgcn_sched_group_barrier(0x008, TM_ * TN_, 0);
    }
  }
}

__device__ __forceinline__ int xcd_swizzle(int bid, int n) {
  constexpr int NX = 8;
  const int per = (n + NX - 1) / NX;
  const int tall = n % NX == 0 ? NX : n % NX;
  const int x = bid % NX, local = bid / NX;
  return x < tall ? x * per + local : tall * per + (x - tall) * (per - 1) + local;
}

// Grouped tile order: tiles run in groups of GM consecutive M-tiles, the
// M index fastest, then N, so the ~32 tiles an XCD runs at once form a
// GM x (32/GM) block whose operand slices are shared through its L2.
__device__ __forceinline__ void group_tile(int L, int nm, int nn, int gm_max, int &m, int &n) {
  const int per = gm_max * nn;
  const int first = (L / per) * gm_max;
  const int gm = nm - first < gm_max ? nm - first : gm_max;
  const int r = L % per;
  m = first + r % gm;
  n = r / gm;
}

// Main loop of an NT product (both operands K-contiguous, copied by DMA):
// nk k-steps starting at contraction index kbeg.
// nk k-steps starting at contraction index kbeg; a stage holds RA rows of A
// then RB rows of B (128 bytes each).
template <int RA, int RB, int TM_, int TN_>
__device__ __forceinline__ void nt_loop(CopyK<8, RA> &ca, CopyK<8, RB> &cb, int kbeg, int nk,
                                        char *lds, int ar, int br, int hh,
                                        f32x16 (&acc)[TM_][TN_]) {
  constexpr int OPA = RA * 128, ST = (RA + RB) * 128;
  ca.issue(lds, kbeg);
  cb.issue(lds + OPA, kbeg);
  for (int ks = 0; ks < nk; ++ks) {
    const char *cur = lds + (ks & 1) * ST;
    char *nxt = lds + ((ks + 1) & 1) * ST;
    // the last step re-copies itself into the idle stage (never read)
    const int kn = kbeg + (ks + 1 < nk ? ks + 1 : ks) * BK;
    wait_vm0();
    __syncthreads();
    ca.issue(nxt, kn);
    cb.issue(nxt + OPA, kn);
    kstep(cur, cur + OPA, ar, br, hh, acc);
  }
  wait_vm0();
}

}  // namespace tile
}  // namespace kd
