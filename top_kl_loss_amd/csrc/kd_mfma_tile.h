// Matrix-core tile machinery shared by the tuned bf16 GEMMs (gfx950).
//
// Two families.  The 4-wave tiles (namespace w4, below) run the logits,
// dH and dW products: one wave per SIMD, 128 x 128 (or 96 x 160) wave tiles
// of v_mfma_f32_16x16x32_bf16 with the accumulators in AGPRs.  On this chip
// the GEMMs run power-limited (the shader clock drops under MFMA load), and
// these tiles read fewer LDS bytes per flop and keep the matrix cores busier
// per clock than the 8-wave ones.  The 8-wave tiles (512 threads, 2 waves
// per SIMD as 2 (M) x 4 (N), 256 x 256 tile, wave tile 128 x 64 = 4 x 2
// blocks of v_mfma_f32_32x32x16_bf16) remain for dH without a W^T copy
// (slices smaller than d), whose W operand goes through registers: there
// the second wave per SIMD hides the register-path work.
//
// Every operand tile sits in LDS as rows of 64 contraction elements (128
// bytes), 16-byte chunk c of row r at r*128 + ((c ^ swz(r)) * 16), and MFMA
// fragments are read with ds_read_b128.  Operands whose contraction index is
// contiguous in memory are copied HBM -> LDS with buffer_load_dwordx4 ... lds
// (reads past the buffer end return zero); the others are read as 8 x 4
// bf16 blocks into registers, transposed with v_perm_b32 and written with
// ds_write_b128.
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

// Width (256 or 320) of the N tile that wastes the least MFMA work on a
// dimension of n (d = 2880 = 9 x 320 needs no padding at 320).
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

// Buffer resource over the rows mn0.. of a row-major operand (pitch ld
// elements, `bytes` in the whole buffer): per-tile offsets stay small, so the
// operand itself may exceed the 4 GiB reach of 32-bit buffer offsets; rows at
// or past the buffer's end read as zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_tile_res(const void *base, uint64_t bytes,
                                                                int64_t ld, int mn0) {
  const uint64_t skip = (uint64_t)mn0 * (uint64_t)ld * 2;
  return make_res(reinterpret_cast<const char *>(base) + skip, bytes > skip ? bytes - skip : 0);
}

__device__ __forceinline__ void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ------------------------------------------------------------- operand copy
// K-contiguous operand, element (mn, k) at byte (mn * ld + k) * 2 of the
// buffer (the resource starts at row mn0),
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
    res = make_tile_res(base, bytes, ld, mn0);
    w = w_;
#pragma unroll
    for (int n = 0; n < N; ++n) {
      const int p = (w * N + n) * 64 + lane;  // 16-byte position in the tile
      const int row = p >> 3, pc = p & 7;
      const int lc = pc ^ swz(row);
      off[n] = (uint32_t)(((int64_t)row * ld + lc * 8) * 2);
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

// ------------------------------------------------------------ 4-wave tiles
// Workgroup: 256 threads = 4 waves (one per SIMD) as 2 (M) x 2 (N); tile
// 256 x 256, wave tile 128 x 128 = 8 x 8 blocks of v_mfma_f32_16x16x32_bf16
// with the 256 accumulator registers in AGPRs.  A k-step (64) is two k32
// halves.  Fragments are double-buffered in registers: while one half's 64
// MFMAs run, the other half's 16 fragments are read from LDS (in the order
// the MFMAs use them).  The one barrier per k-step sits between the halves,
// so the MFMAs right after it use fragments already in registers; the copy
// of step ks + 2 is issued during the second half into the stage just
// consumed, which leaves it a whole k-step to land.  Fewer LDS bytes per
// flop than the 8-wave layout, and one wave per SIMD, keep the matrix cores
// busier per joule: the GEMMs here run power-limited.
//
// The MFMAs are inline asm with the accumulator tied ("+a"), which keeps the
// compiler from copying accumulators between AGPRs and keeps the source
// order.  The compiler's hazard checks do not see asm, so two rules stand
// in for them: the first MFMA of every accumulator takes the inline constant
// 0 as srcC, so no VALU write (zeroing) ever precedes an MFMA read of the
// same register (the VALU-write -> MFMA-srcC dependency of the ISA's
// data-dependency table cannot arise; later MFMAs on an accumulator follow
// MFMAs of the same shape, which the hardware orders itself), and
// acc_ready() pads with s_nop before the accumulators are read by VALU
// instructions.  LDS layout as above, with
// swz4(row) = (row & 7) ^ ((row >> 3) & 1), which is the same for rows 16
// apart, so a fragment address is one register plus an immediate.
namespace w4 {

constexpr int NT = 256;

__device__ __forceinline__ int swz4(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// Tile of 2 x 2 waves, each TMB x TNB blocks of 16 x 16: A has 32 TMB rows,
// B 32 TNB rows per stage (128 bytes each).  Every half-step reads
// TMB + TNB = 16 fragments and issues 16 copy instructions per wave.  With
// AIL (A interleaved), wave row wm holds the 16-row blocks i of tile rows
// 32 i + 16 wm .. + 15 instead of 16 TMB wm + 16 i .. + 15, so that any 32
// consecutive tile rows come from both wave rows (an epilogue can stage
// contiguous rows with all four waves).
template <int TMB_, int TNB_, bool AIL_ = false>
struct Shape {
  static constexpr int TMB = TMB_, TNB = TNB_;
  static constexpr bool AIL = AIL_;
  static constexpr int ASTRIDE = AIL ? 4096 : 2048;  // bytes between A blocks
  // first tile row of A block i of wave row wm
  __device__ static __forceinline__ int arow(int wm, int i) {
    return AIL ? 32 * i + 16 * wm : 16 * TMB * wm + 16 * i;
  }
  static constexpr int RA = 32 * TMB, RB = 32 * TNB;  // operand rows per stage
  static constexpr int OPA = RA * 128;                // B starts here
  static constexpr int STB = (RA + RB) * 128;
  static constexpr int LDS = 2 * STB;
  static constexpr int NR = TMB + TNB;
  static_assert(NR == 16, "16 fragment reads and copy instructions per half-step");
  static_assert(TMB * TNB * 4 <= 256, "accumulators fit the AGPRs");
};
using Square = Shape<8, 8>;   // 256 x 256
using SquareI = Shape<8, 8, true>;  // 256 x 256, A blocks interleaved
using Tall = Shape<6, 10>;    // 192 x 320 (N = d multiple of 320)
static_assert(Tall::LDS <= 160 * 1024, "LDS");

// ROWS rows of a K-contiguous operand, element (mn, k) at byte
// (mn * ld + k) * 2 of the buffer (the resource starts at row mn0); wave w
// issues ROWS / 32 instructions of 1 KiB.
template <int ROWS>
struct Copy {
  static constexpr int N = ROWS / 32;
  __amdgpu_buffer_rsrc_t res;
  uint32_t off[N];
  int w;
  __device__ __forceinline__ void init(const void *base, uint64_t bytes, int64_t ld, int mn0,
                                       int w_, int lane) {
    res = make_tile_res(base, bytes, ld, mn0);
    w = w_;
#pragma unroll
    for (int n = 0; n < N; ++n) {
      const int p = (w * N + n) * 64 + lane;
      const int row = p >> 3, pc = p & 7;
      off[n] = (uint32_t)(((int64_t)row * ld + (pc ^ swz4(row)) * 8) * 2);
    }
  }
  __device__ __forceinline__ void issue(char *tile, int k0, int n) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(res, (lds_vptr)(tile + (w * N + n) * 1024), 16,
                                             (int)(off[n] + k0 * 2), 0, 0, 0);
  }
  __device__ __forceinline__ void issue_all(char *tile, int k0) {
#pragma unroll
    for (int n = 0; n < N; ++n) issue(tile, k0, n);
  }
};

__device__ __forceinline__ void mfma(f32x4 &acc, u32x4 a, u32x4 b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_first(f32x4 &acc, u32x4 a, u32x4 b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=a"(acc) : "v"(a), "v"(b));
}

// Byte offsets (within a stage) of this lane's fragments of block 0:
// A rows wm * 16 TMB + (lane & 15), B rows wn * 16 TNB + (lane & 15),
// k-half h chunk 4 h + (lane >> 4); block i adds i * 2048.
template <class S>
struct FragOff {
  int a[2], b[2];
  __device__ __forceinline__ FragOff(int wm, int wn, int lane) {
    const int r = lane & 15, kq = lane >> 4;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = ((4 * h + kq) ^ swz4(r)) << 4;
      a[h] = (S::arow(wm, 0) + r) * 128 + c;
      b[h] = S::OPA + (wn * 16 * S::TNB + r) * 128 + c;
    }
  }
};

template <int STRIDE = 2048>
__device__ __forceinline__ u32x4 rd(const char *stage, int off, int i) {
  return *reinterpret_cast<const u32x4 *>(stage + off + i * STRIDE);
}

// Fragment r of a half in the order the MFMAs use them: A0, B0.., A1...
template <class S>
__device__ __forceinline__ void read_frag(const char *stage, int aoff, int boff, int r,
                                          u32x4 (&fa)[S::TMB], u32x4 (&fb)[S::TNB]) {
  if (r == 0)
    fa[0] = rd<S::ASTRIDE>(stage, aoff, 0);
  else if (r <= S::TNB)
    fb[r - 1] = rd(stage, boff, r - 1);
  else
    fa[r - S::TNB] = rd<S::ASTRIDE>(stage, aoff, r - S::TNB);
}

// The TMB x TNB MFMAs of one k32 half on (fa, fb), spread over 16 slots; in
// slot r, fragment r of the next half is read (and, when CP, copy
// instruction r of the next-but-one k-step is issued).
template <class S, bool FIRST, bool CP>
__device__ __forceinline__ void half_step(f32x4 (&acc)[S::TMB][S::TNB],
                                          const u32x4 (&fa)[S::TMB], const u32x4 (&fb)[S::TNB],
                                          const char *rstage, int aoff, int boff,
                                          u32x4 (&na)[S::TMB], u32x4 (&nb)[S::TNB],
                                          Copy<S::RA> &ca, Copy<S::RB> &cb, char *cstage, int kc) {
  constexpr int NM = S::TMB * S::TNB;
#pragma unroll
  for (int r = 0; r < S::NR; ++r) {
    read_frag<S>(rstage, aoff, boff, r, na, nb);
    if (CP) {
      if (r < Copy<S::RA>::N)
        ca.issue(cstage, kc, r);
      else
        cb.issue(cstage + S::OPA, kc, r - Copy<S::RA>::N);
    }
#pragma unroll
    for (int idx = r * NM / S::NR; idx < (r + 1) * NM / S::NR; ++idx) {
      const int i = idx / S::TNB, j = idx % S::TNB;
      if (FIRST)
        mfma_first(acc[i][j], fa[i], fb[j]);
      else
        mfma(acc[i][j], fa[i], fb[j]);
    }
  }
}

// NT main loop: acc = A[m0.., kbeg + 64 nk) B[n0.., ...)^T, both operands
// K-contiguous and copied by DMA; nk >= 1.  On return every copy has
// landed; callers reusing LDS call __syncthreads first.
template <class S>
__device__ __forceinline__ void nt_loop(Copy<S::RA> &ca, Copy<S::RB> &cb, int kbeg, int nk,
                                        char *lds, int wm, int wn, int lane,
                                        f32x4 (&acc)[S::TMB][S::TNB]) {
  const FragOff<S> fo(wm, wn, lane);
  u32x4 fa0[S::TMB], fb0[S::TNB], fa1[S::TMB], fb1[S::TNB];
  ca.issue_all(lds, kbeg);
  cb.issue_all(lds + S::OPA, kbeg);
  wait_vm0();
  __syncthreads();
#pragma unroll
  for (int r = 0; r < S::NR; ++r) read_frag<S>(lds, fo.a[0], fo.b[0], r, fa0, fb0);
  const int k1 = kbeg + (nk > 1 ? 1 : 0) * BK;
  ca.issue_all(lds + S::STB, k1);
  cb.issue_all(lds + S::STB + S::OPA, k1);
  // k-step 0: the first half sets every accumulator (srcC = 0)
  {
    half_step<S, true, false>(acc, fa0, fb0, lds, fo.a[1], fo.b[1], fa1, fb1, ca, cb, lds, 0);
    wait_vm0();
    __syncthreads();
    const int k2 = kbeg + (nk > 2 ? 2 : nk - 1) * BK;
    half_step<S, false, true>(acc, fa1, fb1, lds + S::STB, fo.a[0], fo.b[0], fa0, fb0, ca, cb,
                              lds, k2);
  }
  for (int ks = 1; ks < nk; ++ks) {
    char *cur = lds + (ks & 1) * S::STB;
    char *nxt = lds + ((ks + 1) & 1) * S::STB;
    half_step<S, false, false>(acc, fa0, fb0, cur, fo.a[1], fo.b[1], fa1, fb1, ca, cb, cur, 0);
    // this stage is fully read and the copy of step ks + 1 has landed
    wait_vm0();
    __syncthreads();
    // the last step re-copies its own k-slice into the idle stage (never read)
    const int k2 = kbeg + (ks + 2 < nk ? ks + 2 : nk - 1) * BK;
    half_step<S, false, true>(acc, fa1, fb1, nxt, fo.a[0], fo.b[0], fa0, fb0, ca, cb, cur, k2);
  }
  wait_vm0();
}

// Wait states between the last MFMA and the first read of its accumulator
// (the compiler's hazard check does not see the asm MFMAs): 4 x s_nop 7 =
// 32, more than the largest XDL-write -> VALU-read requirement of the
// CDNA3/CDNA4 data-dependency table (18-19 wait states, for 16-pass MFMAs;
// the 16x16x32 MFMAs here take fewer passes).  The empty asm statements
// order every accumulator read after the padding.
template <int TMB, int TNB>
__device__ __forceinline__ void acc_ready(f32x4 (&acc)[TMB][TNB]) {
  asm volatile("s_nop 7\n s_nop 7\n s_nop 7\n s_nop 7" ::: "memory");
#pragma unroll
  for (int i = 0; i < TMB; ++i)
#pragma unroll
    for (int j = 0; j < TNB; ++j) asm volatile("" : "+a"(acc[i][j]));
}

// Position of accumulator element e of block (i, j) in the wave tile (rows:
// of a wave row without AIL; with AIL add 16 wm to arow-based positions).
__device__ __forceinline__ int acc_row4(int i, int e, int lane) { return i * 16 + 4 * (lane >> 4) + e; }
__device__ __forceinline__ int acc_col4(int j, int lane) { return j * 16 + (lane & 15); }

}  // namespace w4

}  // namespace tile
}  // namespace kd
