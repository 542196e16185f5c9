// Matrix-core tile machinery shared by the tuned bf16 GEMMs (gfx950).
//
// Workgroups of 4 waves (one per SIMD, namespace w4 below) run the logits,
// dH and dW products: 128 x 128 (or 128 x 160) wave tiles of
// v_mfma_f32_16x16x32_bf16 with the accumulators in AGPRs (those of a
// 128 x 160 wave tile past the 256 AGPRs in VGPRs).  On this chip the
// GEMMs run power-limited (the shader clock drops under MFMA load), and
// these tiles read few LDS bytes per flop and keep the matrix cores busy per
// clock.
//
// Both operands are copied HBM -> LDS with buffer_load_dwordx4 ... lds
// (reads past the buffer end return zero), one k-step (64 contraction
// elements) per stage, double-buffered.  An operand whose contraction index
// is contiguous in memory (K-contiguous) lands as rows of 64 k (128 bytes)
// per mn-row and is read with ds_read_b128; one whose mn index is contiguous
// (MN-contiguous: W in dH, the row-major probabilities in dW) lands as 64
// k-rows of mn-values and is read with gfx950's transposing LDS read
// ds_read_b64_tr_b16, which hands each lane the k-run of one mn-value that
// the MFMA expects.
#pragma once

#include <stdint.h>

#include "kd_device.h"

namespace kd {
namespace tile {

constexpr int BM = 256, BN = 256, BK = 64;

// Width (256 or 320) of the N tile that wastes the least MFMA work on a
// dimension of n (d = 2880 = 9 x 320 needs no padding at 320).
inline int best_bn(int n) {
  const int w256 = (n + 255) / 256 * 256 - n, w320 = (n + 319) / 320 * 320 - n;
  return w320 < w256 ? 320 : 256;
}

typedef __attribute__((address_space(3))) void *lds_vptr;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_res(const void *base,
                                                           uint64_t bytes) {
  const uint32_t n = bytes > 0xffffffffull ? 0xffffffffu : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0,
                                           (int)n, 0x00020000);
}

// Bytes from `skip` to `bytes` (0 when skip >= bytes), capped at 2^32 - 1, with
// 32-bit compares only: the scalar unit has no 64-bit ordered compare, and a
// 64-bit one moves the operands to VGPRs (|bytes - skip| < 2^63 here).
__device__ __forceinline__ uint32_t bytes_left(uint64_t bytes, uint64_t skip) {
  const uint64_t rem = bytes - skip;
  const int32_t hi = (int32_t)(rem >> 32);
  return hi < 0 ? 0u : (hi > 0 ? 0xffffffffu : (uint32_t)rem);
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

// Workgroup barrier for LDS traffic only: this wave's LDS operations
// complete, then s_barrier.  Unlike __syncthreads (whose fence waits for
// every global load in flight), a prefetch into another LDS region keeps
// going.  The "memory" clobber keeps the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
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
// consumed, which leaves it a whole k-step to land.
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
// instructions.
//
// LDS layouts, per stage (A, then B at OPA):
//  K-contiguous: mn-row r holds 64 k in 8 chunks of 16 bytes, chunk c at
//    r * 128 + ((c ^ swz4(r)) * 16), swz4(r) = (r & 7) ^ ((r >> 3) & 1); the
//    swizzle repeats every 16 rows, so a fragment address is one register
//    plus an immediate.  Lane l reads the 8 k of row l % 16 from chunk
//    4 h + l / 16 with ds_read_b128.
//  MN-contiguous: k-row kr holds the tile's mn-values, P = rows / 8 chunks
//    of 16 bytes, chunk c (mn-values 8c ..) at (kr * P + (c ^ 2 mnf(kr))) *
//    16.  ds_read_b64_tr_b16 works on groups of 16 lanes: lane i supplies
//    the address of 4 consecutive 16-bit values ("row" i of a 16 x 4 block)
//    and receives element i % 4 of rows i / 4, i / 4 + 4, i / 4 + 8,
//    i / 4 + 12.  Lane i of group g (= l / 16) therefore points at k-row
//    8 g + i / 4 (+ 4 for the second read), mn-values 4 (i % 4) .. of its
//    16-value block, and gets mn-value i at 4 consecutive k: two reads give
//    the 8 k of an MFMA fragment.  A read touches 16 k-rows (8 per half-wave)
//    of one 32-byte column; mnf spreads them over distinct LDS banks, and
//    depends only on k-row bits 0, 1 and 3, which are fixed per lane, so
//    every read of a lane's block sits at a fixed offset from one register.
namespace w4 {

constexpr int NT = 256;

__device__ __forceinline__ int swz4(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// Swizzle of k-row kr of an MN-contiguous stage with P chunks per k-row
// (P a multiple of 8).  The 8 k-rows a half-wave reads, 8 g + {0..3} (+4)
// for g in {0, 1} (+16), must land their 32-byte columns in 8 distinct
// 32-byte bank groups of the 256-byte bank row, and each group of 16 lanes
// (4 k-rows) in 4 distinct ones of a 128-byte half.  With P / 8 even the
// bank group is the chunk's position in its row: mnf takes the 8 values
// 0..7.  With P / 8 odd consecutive k-rows are 128 bytes out of phase, the
// XOR stays below 4 (the tile's blocks come in aligned fours) and mnf
// varies with k-row bits 0-1 and 3 so that (kr & 1, mnf) is distinct.
template <int P>
__device__ __forceinline__ int mnf(int kr) {
  static_assert(P % 8 == 0, "MN-contiguous stage rows are multiples of 128 bytes");
  if constexpr ((P / 8) % 2 == 0)
    return (kr & 3) | ((kr >> 1) & 4);
  else
    return (kr & 3) ^ ((kr >> 3) & 1);
}

// Tile of 2 x 2 waves, each TMB x TNB blocks of 16 x 16: A has 32 TMB rows,
// B 32 TNB rows per stage (128 bytes each).  Every half-step reads
// TMB + TNB fragments and issues as many copy instructions per wave.  The
// accumulators of the first 64 blocks (i-major) sit in the 256 AGPRs, those
// of the rest (at most 16) in VGPRs.  With
// AIL (A interleaved), wave row wm holds the 16-row blocks i of tile rows
// 32 i + 16 wm .. + 15 instead of 16 TMB wm + 16 i .. + 15, so that any 32
// consecutive tile rows come from both wave rows (an epilogue can stage
// contiguous rows with all four waves).  AMN / BMN: the operand is
// MN-contiguous.
template <int TMB_, int TNB_, bool AIL_ = false, bool AMN_ = false, bool BMN_ = false>
struct Shape {
  static constexpr int TMB = TMB_, TNB = TNB_;
  static constexpr bool AIL = AIL_, AMN = AMN_, BMN = BMN_;
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
  static_assert(TMB * TNB <= 80, "at most 16 accumulator blocks outside the AGPRs");
  static_assert(!(AIL && AMN), "interleaved A blocks are K-contiguous");
  // MN-contiguous stage rows of P = R / 8 chunks, P a multiple of 8: the
  // XOR of 2 mnf then maps a row's chunks onto themselves
  static_assert(!AMN || RA % 64 == 0, "A rows");
  static_assert(!BMN || RB % 64 == 0, "B rows");
};
using Square = Shape<8, 8>;   // 256 x 256
using SquareI = Shape<8, 8, true>;  // 256 x 256, A blocks interleaved
using SquareBMN = Shape<8, 8, false, false, true>;  // dH: B = W
using SquareAMN = Shape<8, 8, false, true, false>;  // dW: A = P~
using WideBMN = Shape<8, 10, false, false, true>;   // dH, 256 x 320 (N = d multiple of 320)
using WideAMN = Shape<8, 10, false, true, false>;   // dW, 256 x 320
static_assert(WideAMN::LDS <= 160 * 1024, "LDS");

// Accumulator block (i, j) of a TNB-wide wave tile sits in AGPRs when its
// i-major index is below 64 (256 AGPRs), else in VGPRs.
template <int TNB>
__device__ __forceinline__ constexpr bool in_agpr(int i, int j) { return i * TNB + j < 64; }

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

// ROWS mn-values (from mn0) of an MN-contiguous operand, element (mn, k) at
// byte (k * ld + mn) * 2 of the buffer: a k-step is 64 k-rows of ROWS * 2
// bytes; wave w issues ROWS / 32 instructions of 1 KiB, lane-permuted so
// that LDS receives the swizzled layout above.  The resource of a step
// starts at its first k-row, so offsets stay small whatever the buffer's
// size; k-rows at or past the buffer's end read as zero (the bytes of a
// k-row past ld belong to the next one: their products land in output
// columns the callers drop).
template <int ROWS>
struct CopyMN {
  static constexpr int N = ROWS / 32, P = ROWS / 8;
  const char *base;
  uint64_t bytes, ldb;
  uint32_t off[N];
  int w;
  __device__ __forceinline__ void init(const void *b, uint64_t total, int64_t ld, int mn0,
                                       int w_, int lane) {
    const uint64_t skip = (uint64_t)mn0 * 2;
    base = reinterpret_cast<const char *>(b) + skip;
    bytes = total > skip ? total - skip : 0;
    ldb = (uint64_t)ld * 2;
    w = w_;
#pragma unroll
    for (int n = 0; n < N; ++n) {
      const int p = (w * N + n) * 64 + lane;  // 16-byte chunk of the stage
      const int kr = p / P, c = (p - kr * P) ^ (2 * mnf<P>(kr));
      off[n] = (uint32_t)(kr * ldb + 16 * c);
    }
  }
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t res(int k0) const {
    const uint64_t skip = (uint64_t)k0 * ldb;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(base + skip), (short)0,
                                             (int)bytes_left(bytes, skip), 0x00020000);
  }
  __device__ __forceinline__ void issue(char *tile, int k0, int n) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(res(k0), (lds_vptr)(tile + (w * N + n) * 1024), 16,
                                             (int)off[n], 0, 0, 0);
  }
  __device__ __forceinline__ void issue_all(char *tile, int k0) {
#pragma unroll
    for (int n = 0; n < N; ++n) issue(tile, k0, n);
  }
};

template <class S>
using CopyA = __type_pack_element<S::AMN ? 1 : 0, Copy<S::RA>, CopyMN<S::RA>>;
template <class S>
using CopyB = __type_pack_element<S::BMN ? 1 : 0, Copy<S::RB>, CopyMN<S::RB>>;

// acc += a b^T (AG: accumulator in AGPRs, else in VGPRs); mfma_first: acc = a b^T.
// A VGPR destination must not share registers with the sources: the
// first MFMA's output is early-clobber (a tied accumulator cannot overlap
// the other, simultaneously live inputs anyway).
template <bool AG>
__device__ __forceinline__ void mfma(f32x4 &acc, u32x4 a, u32x4 b) {
  if constexpr (AG)
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
template <bool AG>
__device__ __forceinline__ void mfma_first(f32x4 &acc, u32x4 a, u32x4 b) {
  if constexpr (AG)
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=a"(acc) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}

// Byte offset, in an MN-contiguous stage of P chunks per k-row, of the 8
// bytes this lane supplies to the first transposing read of 16-value block
// q in k-half 0 (k-row 8 (lane / 16) + (lane % 16) / 4, mn-values
// 16 q + 4 (lane % 4) ..); the second read is 4 k-rows on, k-half 1 32.
template <int P>
__device__ __forceinline__ int mn_off(int q, int lane) {
  const int kr = 8 * (lane >> 4) + ((lane & 15) >> 2);
  return kr * P * 16 + 32 * (q ^ mnf<P>(kr)) + 8 * (lane & 3);
}

// Byte offsets (within a stage) of this lane's fragments.  K-contiguous:
// per k-half h, block 0 (A rows arow(wm, 0) + (lane & 15), B rows
// wn * 16 TNB + (lane & 15), chunk 4 h + (lane >> 4)); block i adds i * the
// block stride.  MN-contiguous: per block, k-half 0 (mn_off).
template <class S>
struct FragOff {
  int a[S::AMN ? S::TMB : 2], b[S::BMN ? S::TNB : 2];
  __device__ __forceinline__ FragOff(int wm, int wn, int lane) {
    const int r = lane & 15, kq = lane >> 4;
    if constexpr (S::AMN) {
#pragma unroll
      for (int i = 0; i < S::TMB; ++i) a[i] = mn_off<S::RA / 8>(wm * S::TMB + i, lane);
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) a[h] = (S::arow(wm, 0) + r) * 128 + (((4 * h + kq) ^ swz4(r)) << 4);
    }
    if constexpr (S::BMN) {
#pragma unroll
      for (int j = 0; j < S::TNB; ++j) b[j] = S::OPA + mn_off<S::RB / 8>(wn * S::TNB + j, lane);
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h)
        b[h] = S::OPA + (wn * 16 * S::TNB + r) * 128 + (((4 * h + kq) ^ swz4(r)) << 4);
    }
  }
};

template <int STRIDE = 2048>
__device__ __forceinline__ u32x4 rd(const char *stage, int off, int i) {
  return *reinterpret_cast<const u32x4 *>(stage + off + i * STRIDE);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 *lds_s16x4;

__device__ __forceinline__ uint2 tr16(const char *p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4)(const_cast<char *>(p)));
  return __builtin_bit_cast(uint2, v);
}

// MN-contiguous fragment of k-half h at lane offset `off`: two transposing
// reads, k 0-3 and 4-7 of the lane's 8.
template <int P>
__device__ __forceinline__ u32x4 rd_mn(const char *stage, int off, int h) {
  const uint2 lo = tr16(stage + off + h * 32 * P * 16);
  const uint2 hi = tr16(stage + off + h * 32 * P * 16 + 4 * P * 16);
  return u32x4{lo.x, lo.y, hi.x, hi.y};
}

template <class S>
__device__ __forceinline__ u32x4 rd_a(const char *stage, const FragOff<S> &fo, int h, int i) {
  if constexpr (S::AMN)
    return rd_mn<S::RA / 8>(stage, fo.a[i], h);
  else
    return rd<S::ASTRIDE>(stage, fo.a[h], i);
}
template <class S>
__device__ __forceinline__ u32x4 rd_b(const char *stage, const FragOff<S> &fo, int h, int j) {
  if constexpr (S::BMN)
    return rd_mn<S::RB / 8>(stage, fo.b[j], h);
  else
    return rd(stage, fo.b[h], j);
}

// Fragment r of k-half h in the order the MFMAs use them: A0, B0.., A1...
template <class S>
__device__ __forceinline__ void read_frag(const char *stage, const FragOff<S> &fo, int h, int r,
                                          u32x4 (&fa)[S::TMB], u32x4 (&fb)[S::TNB]) {
  if (r == 0)
    fa[0] = rd_a<S>(stage, fo, h, 0);
  else if (r <= S::TNB)
    fb[r - 1] = rd_b<S>(stage, fo, h, r - 1);
  else
    fa[r - S::TNB] = rd_a<S>(stage, fo, h, r - S::TNB);
}

// The TMB x TNB MFMAs of one k32 half on (fa, fb), spread over 16 slots; in
// slot r, fragment r of the next half (k-half rh of stage rstage) is read
// (and, when CP, copy instruction r of the next-but-one k-step is issued).
template <class S, bool FIRST, bool CP, class CA, class CB>
__device__ __forceinline__ void half_step(f32x4 (&acc)[S::TMB][S::TNB],
                                          const u32x4 (&fa)[S::TMB], const u32x4 (&fb)[S::TNB],
                                          const char *rstage, const FragOff<S> &fo, int rh,
                                          u32x4 (&na)[S::TMB], u32x4 (&nb)[S::TNB], CA &ca,
                                          CB &cb, char *cstage, int kc) {
  constexpr int NM = S::TMB * S::TNB;
  static_assert(CA::N + CB::N == S::NR, "one copy instruction per slot");
#pragma unroll
  for (int r = 0; r < S::NR; ++r) {
    read_frag<S>(rstage, fo, rh, r, na, nb);
    if (CP) {
      if (r < CA::N)
        ca.issue(cstage, kc, r);
      else
        cb.issue(cstage + S::OPA, kc, r - CA::N);
    }
#pragma unroll
    for (int idx = r * NM / S::NR; idx < (r + 1) * NM / S::NR; ++idx) {
      const int i = idx / S::TNB, j = idx % S::TNB;
      // (both conditions are constants once the loops are unrolled)
      if (in_agpr<S::TNB>(i, j)) {
        if (FIRST)
          mfma_first<true>(acc[i][j], fa[i], fb[j]);
        else
          mfma<true>(acc[i][j], fa[i], fb[j]);
      } else {
        if (FIRST)
          mfma_first<false>(acc[i][j], fa[i], fb[j]);
        else
          mfma<false>(acc[i][j], fa[i], fb[j]);
      }
    }
  }
}

struct NoHook {
  __device__ void operator()() const {}
};

// Main loop on the two stages s0 and s1 (restrict: the compiler then knows
// that the copies into one stage and the fragment reads from the other do
// not overlap, and waits for no copy before a transposing read; the
// explicit waits below order every copy before the reads of its stage).
// The loop body is two k-steps, so each access names its stage statically.
// `hook` runs once the first k-step's operands, and every load the caller
// issued before the loop, have landed: loads it issues complete during the
// first k-step (and are waited for at its end).  `issued`: the caller has
// already issued the first k-step's copies into s0 (all of them, from every
// wave, with the operands of this call).
template <class S, class CA, class CB, class F>
__device__ __forceinline__ void nt_loop_stages(CA &ca, CB &cb, int kbeg, int nk,
                                               char *__restrict__ s0, char *__restrict__ s1,
                                               const FragOff<S> &fo,
                                               f32x4 (&acc)[S::TMB][S::TNB], F &hook,
                                               bool issued) {
  u32x4 fa0[S::TMB], fb0[S::TNB], fa1[S::TMB], fb1[S::TNB];
  if (!issued) {
    ca.issue_all(s0, kbeg);
    cb.issue_all(s0 + S::OPA, kbeg);
  }
  wait_vm0();
  __syncthreads();
  hook();
#pragma unroll
  for (int r = 0; r < S::NR; ++r) read_frag<S>(s0, fo, 0, r, fa0, fb0);
  const int k1 = kbeg + (nk > 1 ? 1 : 0) * BK;
  ca.issue_all(s1, k1);
  cb.issue_all(s1 + S::OPA, k1);
  // the k-step after ks, clamped: the last steps re-copy the final k-slice
  // into the idle stage (never read)
  auto kof = [&](int ks) { return kbeg + (ks < nk ? ks : nk - 1) * BK; };
  // k-step 0 (stage s0): the first half sets every accumulator (srcC = 0)
  half_step<S, true, false>(acc, fa0, fb0, s0, fo, 1, fa1, fb1, ca, cb, s0, 0);
  wait_vm0();
  __syncthreads();
  half_step<S, false, true>(acc, fa1, fb1, s1, fo, 0, fa0, fb0, ca, cb, s0, kof(2));
  for (int ks = 1; ks < nk; ks += 2) {
    // k-step ks on s1 (the copy of ks + 1 into s0 has landed after the wait)
    half_step<S, false, false>(acc, fa0, fb0, s1, fo, 1, fa1, fb1, ca, cb, s1, 0);
    wait_vm0();
    __syncthreads();
    half_step<S, false, true>(acc, fa1, fb1, s0, fo, 0, fa0, fb0, ca, cb, s1, kof(ks + 2));
    if (ks + 1 >= nk) break;
    // k-step ks + 1 on s0
    half_step<S, false, false>(acc, fa0, fb0, s0, fo, 1, fa1, fb1, ca, cb, s0, 0);
    wait_vm0();
    __syncthreads();
    half_step<S, false, true>(acc, fa1, fb1, s1, fo, 0, fa0, fb0, ca, cb, s0, kof(ks + 3));
  }
  wait_vm0();
}

// Main loop: acc = A[m0.., kbeg + 64 nk) B[n0.., ...)^T, operands copied by
// DMA (K- or MN-contiguous as S says); nk >= 1.  On return every copy has
// landed; callers reusing LDS call __syncthreads first.  `hook` and
// `issued`: see nt_loop_stages (the first stage is at lds).
template <class S, class CA, class CB, class F = NoHook>
__device__ __forceinline__ void nt_loop(CA &ca, CB &cb, int kbeg, int nk, char *lds, int wm,
                                        int wn, int lane, f32x4 (&acc)[S::TMB][S::TNB],
                                        F hook = F(), bool issued = false) {
  const FragOff<S> fo(wm, wn, lane);
  // the second stage's offset is hidden from the compiler: with both stages
  // at constant offsets of one array it drops the restrict information
  int st = S::STB;
  asm volatile("" : "+s"(st));
  nt_loop_stages<S>(ca, cb, kbeg, nk, lds, lds + st, fo, acc, hook, issued);
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
    for (int j = 0; j < TNB; ++j) {
      if (in_agpr<TNB>(i, j))
        asm volatile("" : "+a"(acc[i][j]));
      else
        asm volatile("" : "+v"(acc[i][j]));
    }
}

// Position of accumulator element e of block (i, j) in the wave tile (rows:
// of a wave row without AIL; with AIL add 16 wm to arow-based positions).
__device__ __forceinline__ int acc_row4(int i, int e, int lane) { return i * 16 + 4 * (lane >> 4) + e; }
__device__ __forceinline__ int acc_col4(int j, int lane) { return j * 16 + (lane & 15); }

}  // namespace w4

}  // namespace tile
}  // namespace kd
