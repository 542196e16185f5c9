// bf16 matrix-core GEMMs of the fused, chunked top-K KL loss, tuned for
// gfx950 (used when d is a multiple of 64; other shapes and fp32 inputs take
// the generic kernels of kd_gemm.hip, which compute the same thing).
//
//  logits:  Z = H_c W^T      (C x V, K = d)   + softmax-statistics epilogue
//  dH:      dH_c = G W       (C x d, K = V)   split-K over the vocabulary
//  dW:      dW (+)= G^T H_c  (V x d, K = C)   operands P~ and (f H_c)^T
// The logits GEMM stores the slice's probabilities P~ = 2^(z s2 - sh_t) with
// one a-priori shift per row, in bf16, row-major; k_lse_fix applies the
// teacher correction at the ids and defines the per-row gradient factor f_t,
// so that G = f_t P~.  dH = f_t (P~ W) (the factor applied when the split-K
// partials are reduced) and dW = P~^T (f H_c) (k_transpose_h writes
// (f H_c)^T).  The dH GEMM reads W and the dW GEMM reads P~ as stored, their
// mn index contiguous (transposing LDS reads), so neither needs a
// transposed copy.
//
// The tile machinery (4-wave tiles, DMA operand copies, swizzled
// LDS layouts, MFMA schedules) is in kd_mfma_tile.h.
#include <stdint.h>

#include <algorithm>
#include <atomic>

#include "kd_device.h"
#include "kd_internal.h"
#include "kd_mfma_tile.h"

namespace kd {

namespace {

using namespace tile;

// ------------------------------------------------------------ logits GEMM
// A = H_c, B = W (both K-contiguous), 4-wave tiles, one 256 x 256 tile
// (rows m0.., vocabulary segment seg) per call.  Units are base 2
// (s2 = log2(e) / tau).
//  MODE 0, per row and segment: the shift max(z) s2 and the sum of
//    2^(z s2 - shift) (the softmax statistics), z itself at the row's teacher
//    ids inside the segment (the student-logit gather), and, when gradients
//    are wanted, the probabilities with the row's a-priori shift sh_t,
//    P~ = 2^(z s2 - sh_t), stored in bf16, row-major [C, ldp].
//  MODE 1: the same logits, stored only for the rows flagged by k_lse_fix,
//    with their exact maximum as shift (no statistics, no gather).
// The wave tiles interleave their 16-row blocks (w4::SquareI: block i of
// wave row wm holds tile rows 32 i + 16 wm ..), so the epilogue runs in 4
// passes of 64 consecutive tile rows staged by all four waves: pass p stages
// blocks 2p and 2p + 1 of both wave rows, and stage row sr is tile row
// 64 p + sr.  Thread (pr, part) = (tid / 8, tid % 8) takes the two rows
// pr and pr + 32 and the 8-column groups part, part + 8, ... of them, so
// the 8 threads of a row store whole 128-byte lines of P~.  With the stage
// pitch of 260 floats, the 16-byte reads of 16 lanes (two rows, one pitch
// apart) and the 4-byte staging writes of 64 lanes (four rows 4 apart) both
// fall in distinct LDS banks.
//
// The epilogue stages in the LDS above the main loop's first stage, so a
// workgroup that runs several tiles issues the next tile's first k-step
// copies (and loads its rows' first teacher positions) before this tile's
// epilogue, and the next main loop starts on operands already in flight.
constexpr int LG_STAGE_OFF = w4::SquareI::STB;  // epilogue staging: above stage 0
constexpr int LG_PITCH = BN + 4;                // fp32 per staged row
constexpr int LG_LDS = LG_STAGE_OFF + 64 * LG_PITCH * 4;
static_assert(LG_LDS >= w4::SquareI::LDS && LG_LDS <= 160 * 1024, "LDS");

// First sorted position of tile row m0 + tid's teacher ids in segment seg
// (-1: none, or no such row).
__device__ __forceinline__ int first_pos(const SliceArgs &a, int mt, int seg) {
  const int r = mt * BM + (int)threadIdx.x;
  return r < a.C ? a.first[(size_t)r * a.nseg + seg] : -1;
}

// Tile (mt, seg); `issued`: its first k-step's copies are in flight into
// stage 0 and `pos` holds first_pos (MODE 0).  When next_mt >= 0 the next
// tile's first k-step is issued before the epilogue; returns its first_pos.
template <int MODE>
__device__ __forceinline__ int logits_tile(const SliceArgs &a, int mt, int seg, char *lds,
                                           bool issued, int pos, int next_mt, int next_seg) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = mt * BM, n0 = seg * SEG;
  const uint16_t *H = reinterpret_cast<const uint16_t *>(a.H) + a.c0 * a.d;
  const uint16_t *W = reinterpret_cast<const uint16_t *>(a.W);
  using S = w4::SquareI;
  w4::Copy<S::RA> ca;
  w4::Copy<S::RB> cb;
  ca.init(H, (uint64_t)a.C * a.d * 2, a.d, m0, wave, lane);
  cb.init(W, (uint64_t)a.V * a.d * 2, a.d, n0, wave, lane);
  const bool grads = MODE == 1 || a.need_grad;
  const int part = tid & 7, pr = tid >> 3;

  // Teacher ids of tile row m0 + tid inside this segment, fetched during the
  // main loop so that their latency hides under it: the row's first sorted
  // position in the segment is loaded with the first k-step's operands, the
  // next NHIT + 1 sorted ids and NHIT slots once it has landed (no use of
  // them before the loop ends).  After the loop they become up to NHIT
  // (column, slot) pairs; `more` marks rows with further ids.
  constexpr int NHIT = 4;
  if (MODE != 0) pos = -1;
  int id_raw[NHIT + 1], slot_raw[NHIT];
#pragma unroll
  for (int q = 0; q <= NHIT; ++q) id_raw[q] = INT32_MAX;
#pragma unroll
  for (int q = 0; q < NHIT; ++q) slot_raw[q] = 0;
  auto fetch_ids = [&] {
    if (pos >= 0) {
      const int32_t *sid = a.sid + (size_t)(m0 + tid) * a.K;
      const int32_t *sslot = a.sslot + (size_t)(m0 + tid) * a.K;
#pragma unroll
      for (int q = 0; q <= NHIT; ++q)
        if (pos + q < a.K) id_raw[q] = sid[pos + q];
#pragma unroll
      for (int q = 0; q < NHIT; ++q)
        if (pos + q < a.K) slot_raw[q] = sslot[pos + q];
    }
  };
  f32x4 acc[8][8];
  w4::nt_loop<S>(ca, cb, 0, a.d / BK, lds, wm, wn, lane, acc, fetch_ids, issued);
  int hit_col[NHIT], hit_slot[NHIT];
#pragma unroll
  for (int q = 0; q < NHIT; ++q) {
    const bool in = id_raw[q] < n0 + SEG;  // (INT32_MAX past the row's ids)
    hit_col[q] = in ? id_raw[q] - n0 : -1;
    hit_slot[q] = slot_raw[q];
  }
  const bool more = id_raw[NHIT] < n0 + SEG;

  // Shifts of this thread's 8 rows (2 per pass), loaded after the main loop
  // (registers there are full); rows past C store 0 (shift +inf).  MODE 1:
  // only flagged rows are stored (others +inf too).
  float sh[4][2];
#pragma unroll
  for (int pass = 0; pass < 4; ++pass)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int r = m0 + 64 * pass + pr + 32 * q;
      sh[pass][q] = INFINITY;
      if (grads && r < a.C && (MODE == 0 || a.flag[r])) sh[pass][q] = a.shift[r];
    }
  w4::acc_ready(acc);
  // every wave is past its last fragment read: stage 0 may be refilled
  __syncthreads();
  int next_pos = -1;
  if (next_mt >= 0) {
    w4::Copy<S::RA> na;
    w4::Copy<S::RB> nb;
    na.init(H, (uint64_t)a.C * a.d * 2, a.d, next_mt * BM, wave, lane);
    nb.init(W, (uint64_t)a.V * a.d * 2, a.d, next_seg * SEG, wave, lane);
    na.issue_all(lds, 0);
    nb.issue_all(lds + S::OPA, 0);
    if (MODE == 0) next_pos = first_pos(a, next_mt, next_seg);
  }

  constexpr int PITCH = LG_PITCH;
  constexpr int TPR = 8, CPT = BN / TPR;
  float *stage = reinterpret_cast<float *>(lds + LG_STAGE_OFF);
  uint16_t *P = reinterpret_cast<uint16_t *>(a.P);
  const float s2 = a.s2;
  const bool tail = n0 + BN > a.V;
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          stage[(ii * 32 + wm * 16 + 4 * (lane >> 4) + e) * PITCH + wn * 128 +
                w4::acc_col4(j, lane)] = acc[2 * pass + ii][j][e];
    lds_barrier();
    if (tail) {
      // only the vocabulary's last segment has columns past V: -inf there
      // (2^(-inf) = 0 excludes them from the statistics and from P~)
      const int nv = a.V - n0, nx = BN - nv;
      for (int e = tid; e < 64 * nx; e += w4::NT) stage[(e / nx) * PITCH + nv + e % nx] = -INFINITY;
      lds_barrier();
    }
    // Rows one at a time (fewer live registers): z of the row, the
    // statistics, and P~ packed to bf16 pairs of adjacent columns.
    const int r0 = m0 + 64 * pass + pr;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      float v[CPT];
#pragma unroll
      for (int j = 0; j < CPT / 8; ++j)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int col = j * 8 * TPR + part * 8 + 4 * h;
          const f32x4 z = *reinterpret_cast<const f32x4 *>(stage + (pr + 32 * q) * PITCH + col);
#pragma unroll
          for (int u = 0; u < 4; ++u) v[j * 8 + 4 * h + u] = z[u];
        }
      if (MODE == 0) {
        float m4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
        for (int c = 0; c < CPT; ++c) m4[c & 3] = fmaxf(m4[c & 3], v[c]);
        // the segment's maximum, base-2 units (the 8 lanes of a row agree)
        const float mx = group8_max(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]))) * s2;
        // P~ = 2^(z s2 - mx) 2^(mx - sh): one scale per row and segment (the
        // statistics do not depend on the shift, so a forward-only call
        // gets the same bits)
        const float cq = __builtin_amdgcn_exp2f(mx - sh[pass][q]);
        float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
          // 2^(-inf) = 0 covers the excluded columns
          const float pv = __builtin_amdgcn_exp2f(fmaf(v[c], s2, -mx));
          s4[c & 3] += pv;
          v[c] = pv * cq;
        }
        const float sum = group8_sum((s4[0] + s4[1]) + (s4[2] + s4[3]));
        if (part == 0 && r0 + 32 * q < a.C) {
          a.mseg[(size_t)(r0 + 32 * q) * a.nseg + seg] = mx;
          a.sseg[(size_t)(r0 + 32 * q) * a.nseg + seg] = sum;
        }
      } else {
#pragma unroll
        for (int c = 0; c < CPT; ++c) v[c] = __builtin_amdgcn_exp2f(fmaf(v[c], s2, -sh[pass][q]));
      }
      // rows past C (and, in MODE 1, rows not flagged: +inf shift) are not
      // stored
      const int r = r0 + 32 * q;
      if (grads && r < a.C && (MODE == 0 || sh[pass][q] != INFINITY)) {
        uint16_t *dst = P + (size_t)r * a.ldp + n0 + part * 8;
#pragma unroll
        for (int j = 0; j < CPT / 8; ++j)
          *reinterpret_cast<u32x4 *>(dst + j * 8 * TPR) =
              u32x4{pack_bf16x2(v[8 * j], v[8 * j + 1]), pack_bf16x2(v[8 * j + 2], v[8 * j + 3]),
                    pack_bf16x2(v[8 * j + 4], v[8 * j + 5]), pack_bf16x2(v[8 * j + 6], v[8 * j + 7])};
      }
    }
    // Gather z at the teacher ids: thread tid owns tile row tid, staged in
    // pass tid >> 6 at stage row tid & 63.
    if (MODE == 0 && (tid >> 6) == pass) {
      // the row index is hidden from the compiler here so that it computes
      // these pointers anew instead of keeping the prologue's across the
      // main loop
      int r_own = m0 + tid;
      asm volatile("" : "+v"(r_own));
      const int sr_own = tid & 63;
      if (r_own < a.C) {
        float *zg = a.zg + (size_t)r_own * a.K;
#pragma unroll
        for (int q = 0; q < NHIT; ++q)
          if (hit_col[q] >= 0) zg[hit_slot[q]] = stage[sr_own * PITCH + hit_col[q]];
        if (more) {
          const int32_t *sid = a.sid + (size_t)r_own * a.K;
          const int32_t *sslot = a.sslot + (size_t)r_own * a.K;
          for (int p = pos + NHIT; p < a.K; ++p) {
            const int id = sid[p];
            if (id >= n0 + SEG) break;
            zg[sslot[p]] = stage[sr_own * PITCH + (id - n0)];
          }
        }
      }
    }
    lds_barrier();
  }
  return next_pos;
}

// Persistent: gridDim.x = 8 g workgroups, g per XCD (workgroup b runs on
// XCD b % 8).  XCD x owns a contiguous share of the tile order (as
// xcd_swizzle assigns it), and its workgroup s = b / 8 runs tiles s, s + g,
// s + 2 g, ... of that share, so the g tiles an XCD runs at once are
// consecutive in the grouped order.
__global__ __launch_bounds__(w4::NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_fast_logits(SliceArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int nmt = (a.C + BM - 1) / BM;
  const int n = nmt * a.nseg;
  const int g = gridDim.x / 8, x = blockIdx.x % 8;
  const int per = (n + 7) / 8, tall = n % 8 == 0 ? 8 : n % 8;
  const int lo = x < tall ? x * per : tall * per + (x - tall) * (per - 1);
  const int hi = lo + (x < tall ? per : per - 1);
  int L = lo + (int)blockIdx.x / 8;
  if (L >= hi) return;
  int mt, seg;
  group_tile(L, nmt, a.nseg, 4, mt, seg);
  int pos = first_pos(a, mt, seg);
  bool issued = false;
  for (;;) {
    const int Ln = L + g;
    int nmt_, nseg_ = 0;
    if (Ln < hi)
      group_tile(Ln, nmt, a.nseg, 4, nmt_, nseg_);
    else
      nmt_ = -1;
    pos = logits_tile<0>(a, mt, seg, lds, issued, pos, nmt_, nseg_);
    if (Ln >= hi) break;
    L = Ln;
    mt = nmt_;
    seg = nseg_;
    issued = true;
  }
}

// Rows flagged by k_lse_fix: one workgroup per vocabulary segment walks the
// slice's M-tiles and recomputes those holding flagged rows (none: a few
// flag reads and no other work).
__global__ __launch_bounds__(w4::NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_fast_logits_redo(SliceArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int nmt = (a.C + BM - 1) / BM;
  const int seg = xcd_swizzle(blockIdx.x, gridDim.x);
  for (int mt = 0; mt < nmt; ++mt) {
    if (a.tile_flags[mt] == 0) continue;
    logits_tile<1>(a, mt, seg, lds, false, -1, -1, 0);
    __syncthreads();
  }
}

// ---------------------------------------------------------- dH and dW GEMMs
// On 4-wave tiles, both operands copied by DMA:
//  dH partials = P~ W per vocabulary split (f applied by the reduction),
//  A = P~ (K-contiguous), B = W (MN-contiguous: vocabulary rows, hidden
//  contiguous);
//  dW (+)= P~^T (f H_c), A = P~ (MN-contiguous: token rows, vocabulary
//  contiguous), B = (f H_c)^T (K-contiguous);
//  both on 256 x 320 tiles when d is a multiple of 320 (no N padding;
//  d = 2880 = 9 x 320), else 256 x 256.
// A wave's accumulators to out[row * ld + col] (fp32, rows < nrows and
// columns < ncols kept), stored or (ADD) atomically added.  A tile inside
// both bounds (`full`, wave-uniform) takes one row pointer per accumulator
// row and the column blocks at immediate offsets, with no per-element
// checks.
template <class S, bool ADD>
__device__ __forceinline__ void tile_out(float *out, int64_t ld, bool full, int nrows, int ncols,
                                         int m0, int n0, int wm, int wn, int lane,
                                         f32x4 (&acc)[S::TMB][S::TNB]) {
  const int row0 = m0 + wm * 16 * S::TMB + w4::acc_row4(0, 0, lane);
  const int col0 = n0 + wn * 16 * S::TNB + w4::acc_col4(0, lane);
  if (full) {
    float *base = out + (size_t)row0 * ld + col0;
#pragma unroll
    for (int i = 0; i < S::TMB; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float *p = base + (size_t)(16 * i + e) * ld;
#pragma unroll
        for (int j = 0; j < S::TNB; ++j) {
          if (ADD)
            unsafeAtomicAdd(p + 16 * j, acc[i][j][e]);
          else
            p[16 * j] = acc[i][j][e];
        }
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < S::TMB; ++i)
#pragma unroll
    for (int j = 0; j < S::TNB; ++j) {
      const int col = col0 + 16 * j;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = row0 + 16 * i + e;
        if (row < nrows && col < ncols) {
          float *p = out + (size_t)row * ld + col;
          if (ADD)
            unsafeAtomicAdd(p, acc[i][j][e]);
          else
            *p = acc[i][j][e];
        }
      }
    }
}

template <class S>
__global__ __launch_bounds__(w4::NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_fast_dh4(SliceArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int nmt = (a.C + S::RA - 1) / S::RA;
  const int nnt = (a.d + S::RB - 1) / S::RB;
  const int tile = xcd_swizzle(blockIdx.x, gridDim.x);
  const int split = tile / (nnt * nmt);
  int mt, nt;
  // tile order: N fastest within each M-tile (measured faster than groups
  // of 2-4 M-tiles at t32k)
  group_tile(tile % (nnt * nmt), nmt, nnt, 1, mt, nt);
  const int m0 = mt * S::RA, n0 = nt * S::RB;
  const int sbeg = (int)((int64_t)split * a.nseg / a.splits);
  const int send = (int)((int64_t)(split + 1) * a.nseg / a.splits);
  w4::Copy<S::RA> ca;
  w4::CopyMN<S::RB> cb;
  ca.init(a.P, (uint64_t)a.C * a.ldp * 2, a.ldp, m0, wave, lane);
  cb.init(a.W, (uint64_t)a.V * a.d * 2, a.d, n0, wave, lane);
  f32x4 acc[S::TMB][S::TNB];
  w4::nt_loop<S>(ca, cb, sbeg * SEG, (send - sbeg) * (SEG / BK), lds, wm, wn, lane, acc);
  w4::acc_ready(acc);
  float *out = a.dh_part + (size_t)split * a.dh_stride;
  tile_out<S, false>(out, a.d, m0 + S::RA <= a.C && n0 + S::RB <= a.d, a.C, a.d, m0, n0, wm, wn,
                     lane, acc);
}

template <class S>
__global__ __launch_bounds__(w4::NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_fast_dw4(SliceArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int nnt = (a.d + S::RB - 1) / S::RB;
  const int nmt = (a.V + S::RA - 1) / S::RA;
  const int tile = xcd_swizzle(blockIdx.x, gridDim.x);
  int mt, nt;
  // groups of 3 M-tiles (measured faster than 1, 2, 4-9 or 16 at t32k)
  group_tile(tile, nmt, nnt, 3, mt, nt);
  const int m0 = mt * S::RA, n0 = nt * S::RB;
  w4::CopyMN<S::RA> ca;
  w4::Copy<S::RB> cb;
  ca.init(a.P, (uint64_t)a.C * a.ldp * 2, a.ldp, m0, wave, lane);
  cb.init(a.Ht, (uint64_t)a.d * a.ldh * 2, a.ldh, n0, wave, lane);
  f32x4 acc[S::TMB][S::TNB];
  w4::nt_loop<S>(ca, cb, 0, (a.C + BK - 1) / BK, lds, wm, wn, lane, acc);
  w4::acc_ready(acc);
  // exactly one addition per element and dW GEMM, the GEMMs in stream
  // order: the result does not depend on timing
  const bool full = m0 + S::RA <= a.V && n0 + S::RB <= a.d;
  if (a.dw_beta)
    tile_out<S, true>(a.dW, a.d, full, a.V, a.d, m0, n0, wm, wn, lane, acc);
  else
    tile_out<S, false>(a.dW, a.d, full, a.V, a.d, m0, n0, wm, wn, lane, acc);
}

// dst[j * ldd + r] = src[r * d + j] (times rscale[r] when rscale is not
// null, rounded to nearest even) for r < nrows, 0 for nrows <= r < 64
// gridDim.x (bf16, d and ldd multiples of 64, dst 16-byte aligned), over
// 64 (r) x 64 (j) tiles: 16-byte
// loads of the source rows, a transposing read from LDS, 16-byte stores of
// the destination rows.  256 threads.
__device__ __forceinline__ void transpose64(const uint16_t *__restrict__ src, int64_t d, int nrows,
                                            uint16_t *__restrict__ dst, int64_t ldd,
                                            const float *__restrict__ rscale = nullptr) {
  // pitch 66 elements: the column reads of 8 rows 8 apart hit 8 banks
  __shared__ uint16_t t_s[64][66];
  const int r0 = blockIdx.x * 64, j0 = blockIdx.y * 64;
  const int tid = threadIdx.x, ch = tid & 7;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int rr = (tid >> 3) + 32 * h;
    u32x4 v{0u, 0u, 0u, 0u};
    if (r0 + rr < nrows) {
      v = *reinterpret_cast<const u32x4 *>(src + (int64_t)(r0 + rr) * d + j0 + ch * 8);
      if (rscale) v = Elem<uint16_t>::scale(v, rscale[r0 + rr]);
    }
    uint32_t *row = reinterpret_cast<uint32_t *>(&t_s[rr][0]);
#pragma unroll
    for (int q = 0; q < 4; ++q) row[ch * 4 + q] = v[q];
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int jj = (tid >> 3) + 32 * h;
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int ra = ch * 8 + 2 * q;
      o[q] = uint32_t(t_s[ra][jj]) | (uint32_t(t_s[ra + 1][jj]) << 16);
    }
    *reinterpret_cast<u32x4 *>(dst + (int64_t)(j0 + jj) * ldd + r0 + ch * 8) = o;
  }
}

// The slice's columns ht_col .. of (f H)^T [d, ldh], each token row scaled
// by its gradient factor f_t (columns past the slice's C tokens, up to the
// next multiple of 64, zero): dW = P~^T (f H) = G^T H over the group.
__global__ __launch_bounds__(256) void k_transpose_h(SliceArgs a) {
  transpose64(reinterpret_cast<const uint16_t *>(a.H) + a.c0 * a.d, a.d, a.C, a.Ht + a.ht_col,
              a.ldh, a.frow);
}

// Compute units of the current device (cached per device; threads that
// race on the first query store the same value).
int num_cus() {
  static std::atomic<int> cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <typename K>
hipError_t launch(K kern, int grid, const SliceArgs &a, hipStream_t s, int lds, int threads) {
  if (grid <= 0) return hipSuccess;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(threads), lds, s, a);
  return hipGetLastError();
}

}  // namespace

int fast_bn(int d) { return best_bn(d); }

// Splits of the vocabulary contraction of dH.  Each split is one workgroup
// per output tile, run in rounds over the 256 CUs (one workgroup per CU), so
// the time is about ceil(tiles * s / 256) rounds of 1/s of a tile's whole
// contraction, plus the s partial sums written and read back by the
// reduction.  The rates below only weigh the two terms (a tile at ~45% of
// the matrix-core peak of one CU; partials at ~4.5 TB/s).
int fast_dh_splits(int C, int d, int nseg, int bn) {
  constexpr int NCU = 256;
  const int tiles = ((C + BM - 1) / BM) * ((d + bn - 1) / bn);
  const double tile_s = 2.0 * BM * bn * (double)nseg * SEG / 4.4e12;
  const double part_s = (double)C * d * 4.0 / 4.5e12;
  const int smax = nseg < 64 ? nseg : 64;
  int best = 1;
  double best_cost = 1e30;
  for (int sp = 1; sp <= smax; ++sp) {
    const double rounds = (double)((tiles * sp + NCU - 1) / NCU);
    const double cost = rounds * tile_s / sp + (sp + 1) * part_s;
    if (cost < best_cost * (1.0 - 1e-9)) {
      best_cost = cost;
      best = sp;
    }
  }
  return best;
}

hipError_t launch_fast_logits(const SliceArgs &a, hipStream_t s) {
  if (a.d < BK) return hipErrorInvalidValue;  // the main loop needs one k-step
  const int tiles = ((a.C + BM - 1) / BM) * a.nseg;
  // one workgroup per CU (LDS holds one), at most one per tile, 8 | grid
  const int grid = 8 * std::max(1, std::min(num_cus() / 8, (tiles + 7) / 8));
  return launch(k_fast_logits, grid, a, s, LG_LDS, w4::NT);
}

template <class S>
hipError_t launch_dh(const SliceArgs &a, hipStream_t s) {
  const int tiles = ((a.C + S::RA - 1) / S::RA) * ((a.d + S::RB - 1) / S::RB) * a.splits;
  return launch(k_fast_dh4<S>, tiles, a, s, S::LDS, w4::NT);
}

hipError_t launch_fast_dh(const SliceArgs &a, hipStream_t s) {
  if (a.dh_bn == w4::WideBMN::RB) return launch_dh<w4::WideBMN>(a, s);
  return launch_dh<w4::SquareBMN>(a, s);
}

hipError_t launch_transpose_h(const SliceArgs &a, hipStream_t s) {
  if (!a.fast) return hipSuccess;
  const dim3 tg((a.C + 63) / 64, a.d / 64);
  hipLaunchKernelGGL(k_transpose_h, tg, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_flagged_rows(const SliceArgs &a, hipStream_t s) {
  if (!a.fast) return hipSuccess;
  hipError_t e = launch(k_fast_logits_redo, a.nseg, a, s, LG_LDS, w4::NT);
  if (e != hipSuccess) return e;
  return launch_fix_flagged(a, s);
}

template <class S>
hipError_t launch_dw(const SliceArgs &a, hipStream_t s) {
  return launch(k_fast_dw4<S>, ((a.V + S::RA - 1) / S::RA) * ((a.d + S::RB - 1) / S::RB), a, s,
                S::LDS, w4::NT);
}

hipError_t launch_fast_dw(const SliceArgs &a, hipStream_t s) {
  if (a.dw_bn == w4::WideAMN::RB) return launch_dw<w4::WideAMN>(a, s);
  return launch_dw<w4::SquareAMN>(a, s);
}

}  // namespace kd
