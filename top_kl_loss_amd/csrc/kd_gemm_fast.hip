// bf16 matrix-core GEMMs of the fused, chunked top-K KL loss, tuned for
// gfx950 (used when d is a multiple of 64; other shapes and fp32 inputs take
// the generic kernels of kd_gemm.hip, which compute the same thing).
//
//  logits:  Z = H_c W^T      (C x V, K = d)   + softmax-statistics epilogue
//  dH:      dH_c = G W       (C x d, K = V)   split-K over the vocabulary
//  dW:      dW (+)= G^T H_c  (V x d, K = C)   operands G^T and H_c^T
// G is the slice's logit gradient: k_scale_g writes it in bf16 over the P
// buffer and also writes G^T; k_transpose_h writes H_c^T.
//
// The tile machinery (4-wave and 8-wave tiles, DMA operand copies, swizzled
// LDS layouts, MFMA schedules) is in kd_mfma_tile.h.
#include <stdint.h>

#include "kd_device.h"
#include "kd_internal.h"
#include "kd_mfma_tile.h"

namespace kd {

namespace {

using namespace tile;

// ------------------------------------------------------------ logits GEMM
// A = H_c, B = W (both K-contiguous), 4-wave tiles.  Epilogue per row and
// segment: max of z/tau, P = exp(z/tau - max) in bf16, the sum of P, and z
// itself at the row's teacher ids inside the segment (the student-logit
// gather).
__global__ __launch_bounds__(w4::NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_fast_logits(SliceArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int nmt = (a.C + BM - 1) / BM;
  const int tile = xcd_swizzle(blockIdx.x, gridDim.x);
  int mt, seg;
  group_tile(tile, nmt, a.nseg, 4, mt, seg);
  const int m0 = mt * BM, n0 = seg * SEG;
  const uint16_t *H = reinterpret_cast<const uint16_t *>(a.H) + a.c0 * a.d;
  const uint16_t *W = reinterpret_cast<const uint16_t *>(a.W);
  using S = w4::Square;
  w4::Copy<S::RA> ca;
  w4::Copy<S::RB> cb;
  ca.init(H, (uint64_t)a.C * a.d * 2, a.d, m0, wave, lane);
  cb.init(W, (uint64_t)a.V * a.d * 2, a.d, n0, wave, lane);

  // Teacher ids of tile row m0 + tid inside this segment, fetched now so
  // that their latency hides under the main loop: up to NHIT (column, slot)
  // pairs; `more` marks rows with further ids.
  constexpr int NHIT = 4;
  int hit_col[NHIT], hit_slot[NHIT];
  bool more = false;
#pragma unroll
  for (int q = 0; q < NHIT; ++q) hit_col[q] = -1;
  if (m0 + tid < a.C) {
    const int r = m0 + tid;
    const int pos = a.first[(size_t)r * a.nseg + seg];
    if (pos >= 0) {
      const int32_t *sid = a.sid + (size_t)r * a.K;
      const int32_t *sslot = a.sslot + (size_t)r * a.K;
#pragma unroll
      for (int q = 0; q < NHIT; ++q) {
        const int p = pos + q;
        const int id = p < a.K ? sid[p] : INT32_MAX;
        if (id < n0 + SEG) {
          hit_col[q] = id - n0;
          hit_slot[q] = sslot[p];
        }
      }
      if (pos + NHIT < a.K && sid[pos + NHIT] < n0 + SEG) more = true;
    }
  }

  f32x4 acc[8][8];
  w4::nt_loop<S>(ca, cb, 0, a.d / BK, lds, wm, wn, lane, acc);
  w4::acc_ready(acc);
  __syncthreads();

  // Epilogue in 4 passes; pass p stages block-rows 2p and 2p + 1 of both
  // wave rows: 64 tile rows x 256 columns, tile row
  // wm * 128 + (2p + ii) * 16 + r at stage row wm * 32 + ii * 16 + r.  Each
  // row is processed by TPR threads, and each thread takes RPT rows at once
  // (independent work to overlap with one wave per SIMD).
  constexpr int PITCH = BN + 4;
  constexpr int SROWS = 64, TPR = 8, RPT = SROWS * TPR / w4::NT, CPT = BN / TPR;
  float *stage = reinterpret_cast<float *>(lds);
  uint16_t *P = reinterpret_cast<uint16_t *>(a.P);
  const int part = tid % TPR;
  const float s2 = a.inv_tau * LOG2E;
  const bool tail = n0 + BN > a.V;
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          stage[(wm * 32 + ii * 16 + 4 * (lane >> 4) + e) * PITCH + wn * 128 +
                w4::acc_col4(j, lane)] = acc[2 * pass + ii][j][e];
    __syncthreads();
    // Thread `part` of a row owns the 8-column groups part, part + 8, ...,
    // so the row's TPR threads store whole 128-byte lines of P together
    // (contiguous 64-byte runs per thread would split every line).
    // Base-2 units: v = z / tau * log2(e), P = 2^(v - max v); only the
    // vocabulary's last segment has columns past V (excluded).
    float v[RPT][CPT];
    float mx[RPT], sum[RPT];
#pragma unroll
    for (int q = 0; q < RPT; ++q) {
      const int sr = tid / TPR + q * (w4::NT / TPR);
      float m4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
      for (int j = 0; j < CPT / 8; ++j) {
        const int col = j * 8 * TPR + part * 8;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const f32x4 z = *reinterpret_cast<const f32x4 *>(stage + sr * PITCH + col + 4 * h);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int c = j * 8 + 4 * h + u;
            v[q][c] = z[u] * s2;
            if (tail && n0 + col + 4 * h + u >= a.V) v[q][c] = -INFINITY;
            m4[u] = fmaxf(m4[u], v[q][c]);
          }
        }
      }
      mx[q] = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
    }
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1)
#pragma unroll
      for (int q = 0; q < RPT; ++q) mx[q] = fmaxf(mx[q], __shfl_xor(mx[q], o, 64));
#pragma unroll
    for (int q = 0; q < RPT; ++q) {
      float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        // exp2(-inf) = 0 covers the excluded columns
        const float pv = __builtin_amdgcn_exp2f(v[q][c] - mx[q]);
        v[q][c] = pv;
        s4[c & 3] += pv;
      }
      sum[q] = (s4[0] + s4[1]) + (s4[2] + s4[3]);
      mx[q] *= LN2;  // the segment maximum of z / tau
    }
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1)
#pragma unroll
      for (int q = 0; q < RPT; ++q) sum[q] += __shfl_xor(sum[q], o, 64);
#pragma unroll
    for (int q = 0; q < RPT; ++q) {
      const int sr = tid / TPR + q * (w4::NT / TPR);
      const int r = m0 + (sr >> 5) * 128 + (2 * pass + ((sr >> 4) & 1)) * 16 + (sr & 15);
      if (r < a.C) {
        uint16_t *dst = P + (size_t)r * a.ldp + n0 + part * 8;
        if (a.need_grad) {
#pragma unroll
          for (int j = 0; j < CPT / 8; ++j) {
            const int c = j * 8;
            u32x4 w{pack_bf16x2(v[q][c], v[q][c + 1]), pack_bf16x2(v[q][c + 2], v[q][c + 3]),
                    pack_bf16x2(v[q][c + 4], v[q][c + 5]), pack_bf16x2(v[q][c + 6], v[q][c + 7])};
            *reinterpret_cast<u32x4 *>(dst + j * 8 * TPR) = w;
          }
        }
        if (part == 0) {
          a.mseg[(size_t)r * a.nseg + seg] = mx[q];
          a.sseg[(size_t)r * a.nseg + seg] = sum[q];
        }
      }
    }
    // Gather z at the teacher ids: thread tid owns tile row tid, staged in
    // pass (tid & 127) >> 5 at stage row (tid >> 7) * 32 + (tid & 31).
    if (((tid & 127) >> 5) == pass) {
      const int r_own = m0 + tid;
      const int sr_own = (tid >> 7) * 32 + (tid & 31);
      if (r_own < a.C) {
        float *zg = a.zg + (size_t)r_own * a.K;
#pragma unroll
        for (int q = 0; q < NHIT; ++q)
          if (hit_col[q] >= 0) zg[hit_slot[q]] = stage[sr_own * PITCH + hit_col[q]];
        if (more) {
          const int32_t *sid = a.sid + (size_t)r_own * a.K;
          const int32_t *sslot = a.sslot + (size_t)r_own * a.K;
          for (int p = a.first[(size_t)r_own * a.nseg + seg] + NHIT; p < a.K; ++p) {
            const int id = sid[p];
            if (id >= n0 + SEG) break;
            zg[sslot[p]] = stage[sr_own * PITCH + (id - n0)];
          }
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- dH GEMM
// A = G (K-contiguous over the vocabulary; copied by DMA), B = W
// (vocabulary rows, hidden contiguous) transposed through registers: the
// 8-wave path for calls without a W^T copy (slices smaller than d).  With
// the copy, k_fast_dh4 below runs instead.
__global__ __launch_bounds__(NT, 1) void k_fast_dh_reg(SliceArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int nmt = (a.C + BM - 1) / BM;
  const int nnt = (a.d + BN - 1) / BN;
  const int tile = xcd_swizzle(blockIdx.x, gridDim.x);
  const int split = tile / (nnt * nmt);
  int mt, nt;
  group_tile(tile % (nnt * nmt), nmt, nnt, 4, mt, nt);
  const int m0 = mt * BM, n0 = nt * BN;
  const int sbeg = (int)((int64_t)split * a.nseg / a.splits);
  const int send = (int)((int64_t)(split + 1) * a.nseg / a.splits);
  const int kbeg = sbeg * SEG, kend = send * SEG;
  CopyK<8> ca;
  ca.init(a.P, (uint64_t)a.C * a.ldp * 2, a.ldp, m0, wave, lane);
  f32x16 acc[TM][TN];
  zero_acc(acc);
  const int nk = (kend - kbeg) / BK;
  const int ar = wm * WTM + (lane & 31), br = wn * WTN + (lane & 31), hh = lane >> 5;
  RegMN4 rb;
  rb.init(reinterpret_cast<const uint16_t *>(a.W), a.d, n0, a.d, kend < a.V ? kend : a.V, tid);
  ca.issue(lds, kbeg);
  rb.load(kbeg);
  rb.store(lds + OP_BYTES, tid);
  for (int ks = 0; ks < nk; ++ks) {
    const char *cur = lds + (ks & 1) * STAGE_BYTES;
    char *nxt = lds + ((ks + 1) & 1) * STAGE_BYTES;
    const int kn = kbeg + (ks + 1 < nk ? ks + 1 : ks) * BK;
    wait_vm0();
    __syncthreads();
    ca.issue(nxt, kn);
    rb.load(kn);
    kstep(cur, cur + OP_BYTES, ar, br, hh, acc);
    rb.store(nxt + OP_BYTES, tid);
  }
  wait_vm0();

  float *out = a.dh_part + (size_t)split * a.dh_stride;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = n0 + wn * WTN + j * 32 + (lane & 31);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wm * WTM + i * 32 + acc_row(e, lane);
        if (row < a.C && col < a.d) out[(size_t)row * a.d + col] = acc[i][j][e];
      }
    }
}

// ---------------------------------------------------------- dH and dW GEMMs
// On 4-wave tiles, both operands copied by DMA:
//  dH partials = G (W^T)^T per vocabulary split, A = G, B = W^T (the call's
//  W^T copy), 256 x 256 tiles;
//  dW (+)= G^T (H_c^T)^T, A = G^T, B = H_c^T, 192 x 320 tiles when d is a
//  multiple of 320 (no N padding; d = 2880 = 9 x 320), else 256 x 256.
__global__ __launch_bounds__(w4::NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_fast_dh4(SliceArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int nmt = (a.C + BM - 1) / BM;
  const int nnt = (a.d + BN - 1) / BN;
  const int tile = xcd_swizzle(blockIdx.x, gridDim.x);
  const int split = tile / (nnt * nmt);
  int mt, nt;
  group_tile(tile % (nnt * nmt), nmt, nnt, 4, mt, nt);
  const int m0 = mt * BM, n0 = nt * BN;
  const int sbeg = (int)((int64_t)split * a.nseg / a.splits);
  const int send = (int)((int64_t)(split + 1) * a.nseg / a.splits);
  using S = w4::Square;
  w4::Copy<S::RA> ca;
  w4::Copy<S::RB> cb;
  ca.init(a.P, (uint64_t)a.C * a.ldp * 2, a.ldp, m0, wave, lane);
  cb.init(a.Wt, (uint64_t)a.d * a.ldp * 2, a.ldp, n0, wave, lane);
  f32x4 acc[8][8];
  w4::nt_loop<S>(ca, cb, sbeg * SEG, (send - sbeg) * (SEG / BK), lds, wm, wn, lane, acc);
  w4::acc_ready(acc);
  float *out = a.dh_part + (size_t)split * a.dh_stride;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int col = n0 + wn * 128 + w4::acc_col4(j, lane);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = m0 + wm * 128 + w4::acc_row4(i, e, lane);
        if (row < a.C && col < a.d) out[(size_t)row * a.d + col] = acc[i][j][e];
      }
    }
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
  group_tile(tile, nmt, nnt, 4, mt, nt);
  const int m0 = mt * S::RA, n0 = nt * S::RB;
  w4::Copy<S::RA> ca;
  w4::Copy<S::RB> cb;
  ca.init(a.Gt, (uint64_t)a.ldp * a.ldh * 2, a.ldh, m0, wave, lane);
  cb.init(a.Ht, (uint64_t)a.d * a.ldh * 2, a.ldh, n0, wave, lane);
  f32x4 acc[S::TMB][S::TNB];
  w4::nt_loop<S>(ca, cb, 0, (a.C + BK - 1) / BK, lds, wm, wn, lane, acc);
  w4::acc_ready(acc);
#pragma unroll
  for (int i = 0; i < S::TMB; ++i)
#pragma unroll
    for (int j = 0; j < S::TNB; ++j) {
      const int col = n0 + wn * 16 * S::TNB + w4::acc_col4(j, lane);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = m0 + wm * 16 * S::TMB + w4::acc_row4(i, e, lane);
        if (row < a.V && col < a.d) {
          float *p = a.dW + (size_t)row * a.d + col;
          // exactly one addition per element and slice, slices in stream
          // order: the result does not depend on timing
          if (a.dw_beta)
            unsafeAtomicAdd(p, acc[i][j][e]);
          else
            *p = acc[i][j][e];
        }
      }
    }
}

// dst[j * ldd + r] = src[r * d + j] for r < nrows, 0 for nrows <= r < ldd
// (bf16, d and ldd multiples of 64), over 64 (r) x 64 (j) tiles: 16-byte
// loads of the source rows, a transposing read from LDS, 16-byte stores of
// the destination rows.  256 threads.
__device__ __forceinline__ void transpose64(const uint16_t *__restrict__ src, int64_t d, int nrows,
                                            uint16_t *__restrict__ dst, int64_t ldd) {
  // pitch 66 elements: the column reads of 8 rows 8 apart hit 8 banks
  __shared__ uint16_t t_s[64][66];
  const int r0 = blockIdx.x * 64, j0 = blockIdx.y * 64;
  const int tid = threadIdx.x, ch = tid & 7;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int rr = (tid >> 3) + 32 * h;
    u32x4 v{0u, 0u, 0u, 0u};
    if (r0 + rr < nrows) v = *reinterpret_cast<const u32x4 *>(src + (int64_t)(r0 + rr) * d + j0 + ch * 8);
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

// H_c^T [d, ldh] per slice (token columns t >= C zero).
__global__ __launch_bounds__(256) void k_transpose_h(SliceArgs a) {
  transpose64(reinterpret_cast<const uint16_t *>(a.H) + a.c0 * a.d, a.d, a.C, a.Ht, a.ldh);
}

// W^T [d, ldp] once per call (vocabulary columns v >= V zero).
__global__ __launch_bounds__(256) void k_transpose_w(SliceArgs a) {
  transpose64(reinterpret_cast<const uint16_t *>(a.W), a.d, a.V, a.Wt, a.ldp);
}

// G = f[t, seg] * P over one 64-row x 256-column (one segment) tile, written
// in place, and G^T[v, t] through LDS; G^T columns t >= C are zero.
__global__ __launch_bounds__(256) void k_scale_g(SliceArgs a) {
  __shared__ uint16_t g_s[64][256 + 8];
  const int t0 = blockIdx.x * 64, seg = blockIdx.y, v0 = seg * SEG;
  const int tid = threadIdx.x;
  uint16_t *P = reinterpret_cast<uint16_t *>(a.P);
  const int c = tid & 31;            // 16-byte chunk of the 512-byte row
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = (tid >> 5) + 8 * i;
    const int t = t0 + r;
    u32x4 v{0u, 0u, 0u, 0u};
    if (t < a.C) {
      u32x4 *src = reinterpret_cast<u32x4 *>(P + (size_t)t * a.ldp + v0) + c;
      v = Elem<uint16_t>::scale(*src, a.fseg[(size_t)t * a.nseg + seg]);
      __builtin_nontemporal_store(v, src);  // streamed: read once by dH
    }
    *reinterpret_cast<u32x4 *>(&g_s[r][c * 8]) = v;
  }
  __syncthreads();
  // G^T rows v0.. of this tile: 64 tokens = 128 bytes each, written by 8
  // consecutive lanes (16 bytes each) so every store fills whole lines.
  const int q = tid & 7;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int vr = (tid >> 3) + 32 * i;
    u32x4 o;
#pragma unroll
    for (int p = 0; p < 4; ++p)
      o[p] = uint32_t(g_s[q * 8 + 2 * p][vr]) | (uint32_t(g_s[q * 8 + 2 * p + 1][vr]) << 16);
    __builtin_nontemporal_store(o, reinterpret_cast<u32x4 *>(a.Gt + (size_t)(v0 + vr) * a.ldh + t0) + q);
  }
}

template <typename K>
hipError_t launch(K kern, int grid, const SliceArgs &a, hipStream_t s, int lds = LDS_BYTES,
                  int threads = NT) {
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
  return launch(k_fast_logits, ((a.C + BM - 1) / BM) * a.nseg, a, s, w4::Square::LDS, w4::NT);
}

hipError_t launch_fast_dh(const SliceArgs &a, hipStream_t s) {
  const int tiles = ((a.C + BM - 1) / BM) * ((a.d + BN - 1) / BN) * a.splits;
  if (a.Wt) return launch(k_fast_dh4, tiles, a, s, w4::Square::LDS, w4::NT);
  return launch(k_fast_dh_reg, tiles, a, s);
}

hipError_t launch_transpose_h(const SliceArgs &a, hipStream_t s) {
  if (!a.fast) return hipSuccess;
  const dim3 tg(a.ldh / 64, a.d / 64);
  hipLaunchKernelGGL(k_transpose_h, tg, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_transpose_w(const SliceArgs &a, hipStream_t s) {
  if (!a.Wt) return hipSuccess;
  const dim3 g(a.ldp / 64, a.d / 64);
  hipLaunchKernelGGL(k_transpose_w, g, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_scale_g(const SliceArgs &a, hipStream_t s) {
  if (!a.fast) return hipSuccess;
  const dim3 g((a.ldh + 63) / 64, a.nseg);
  hipLaunchKernelGGL(k_scale_g, g, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fast_dw(const SliceArgs &a, hipStream_t s) {
  if (a.dw_bn == w4::Tall::RB) {
    using S = w4::Tall;
    return launch(k_fast_dw4<S>, ((a.V + S::RA - 1) / S::RA) * ((a.d + S::RB - 1) / S::RB), a, s,
                  S::LDS, w4::NT);
  }
  using S = w4::Square;
  return launch(k_fast_dw4<S>, ((a.V + S::RA - 1) / S::RA) * ((a.d + S::RB - 1) / S::RB), a, s,
                S::LDS, w4::NT);
}

}  // namespace kd
