// bf16 matrix-core GEMMs of the fused, chunked top-K KL loss, tuned for
// gfx950 (used when d is a multiple of 64; other shapes and fp32 inputs take
// the generic kernels of kd_gemm.hip, which compute the same thing).
//
//  logits:  Z = H_c W^T        (C x V, K = d)   + softmax-statistics epilogue
//  dH:      dH_c = G W         (C x d, K = V)   split-K over vocabulary
//  dW:      dW (+)= G^T H_c    (V x d, K = C)
// with G[t,v] = f[t, seg(v)] * P[t,v] (see kd_gemm.hip and k_lse_fix).
//
// Workgroup: 256 threads = 4 waves (2 x 2), tile 256 x 256, wave tile
// 128 x 128 = 4 x 4 blocks of v_mfma_f32_32x32x16_bf16, fp32 accumulators.
// One k-step is 64 bf16 of the contraction.  Operands are copied from HBM
// straight into LDS with buffer_load_dwordx4 ... lds (no register staging);
// reads past a buffer's end return zero, which pads row tails.  Two LDS
// stages: the copy of step k+1 runs while step k's MFMAs execute.
//
// LDS layouts of one stage:
//  * K-contiguous operand (rows of 64 k = 128 B): 16-byte chunk c of row r
//    at r*128 + ((c ^ (r & 7)) * 16); fragments are read with ds_read_b128.
//  * MN-contiguous operand (64 k-rows of 256 elements = 512 B): 32-byte unit
//    u of k-row k at k*512 + (u ^ s(k)) * 32 with s(k) = (k & 7) ^ (k & 8 ? 4
//    : 0); fragments are read with ds_read_b64_tr_b16, whose 16-lane groups
//    return lane i the (i mod 4)-th 16-bit element of the rows addressed by
//    lanes 4j + i/4 (j = 0..3), i.e. 4 consecutive k of one column.
#include "kd_device.h"
#include "kd_internal.h"

namespace kd {

namespace {

constexpr int NT = 256;
constexpr int BM = 256, BN = 256, BK = 64;
constexpr int WTM = 128, WTN = 128, TM = 4, TN = 4;
constexpr int OP_BYTES = 256 * 128;          // one operand tile per stage
constexpr int STAGE_BYTES = 2 * OP_BYTES;    // A then B
constexpr int LDS_BYTES = 2 * STAGE_BYTES;   // 128 KiB

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void *lds_vptr;
typedef __attribute__((address_space(3))) s16x4 *lds_s16x4_ptr;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_res(const void *base,
                                                           uint64_t bytes) {
  const uint32_t n = bytes > 0xffffffffull ? 0xffffffffu : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0,
                                           (int)n, 0x00020000);
}

// 64 lanes x 16 bytes from `res` at per-lane byte offsets into LDS at
// `lds_base` (wave-uniform) + lane * 16.
__device__ __forceinline__ void copy16(__amdgpu_buffer_rsrc_t res, char *lds_base,
                                       uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(res, (lds_vptr)lds_base, 16, (int)voff, 0,
                                           0, 0);
}

__device__ __forceinline__ void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ int swz_mn(int k) { return (k & 7) ^ ((k & 8) ? 4 : 0); }

// ------------------------------------------------------------- operand copy
// K-contiguous operand: element (mn, k) at byte (mn * ld + k) * 2 of `res`.
// Per k-step each wave issues 8 copies of 1 KiB (8 rows of 128 B).
struct CopyK {
  __amdgpu_buffer_rsrc_t res;
  uint32_t row_off[8];  // byte offset of this lane's row for copy n
  int lds_off[8];       // wave-uniform LDS offset of copy n (relative)
  __device__ __forceinline__ void init(const void *base, uint64_t bytes, int64_t ld,
                                       int mn0, int wave, int lane) {
    res = make_res(base, bytes);
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const int p = (wave * 8 + n) * 64 + lane;   // 16-byte position in tile
      const int row = p >> 3, pc = p & 7;
      const int lc = pc ^ (row & 7);
      row_off[n] = (uint32_t)(((int64_t)(mn0 + row) * ld + lc * 8) * 2);
      lds_off[n] = (wave * 8 + n) * 1024;
    }
  }
  __device__ __forceinline__ void issue(char *lds_tile, int k0) {
#pragma unroll
    for (int n = 0; n < 8; ++n) copy16(res, lds_tile + lds_off[n], row_off[n] + k0 * 2);
  }
};

// MN-contiguous operand: element (mn, k) at byte (k * ld + mn) * 2 of `res`.
// Per k-step each wave issues 8 copies of 1 KiB (2 k-rows of 512 B).
struct CopyMN {
  __amdgpu_buffer_rsrc_t res;
  uint32_t off[8];
  int lds_off[8];
  int64_t ld;
  __device__ __forceinline__ void init(const void *base, uint64_t bytes, int64_t ld_,
                                       int mn0, int wave, int lane) {
    res = make_res(base, bytes);
    ld = ld_;
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const int kr = 2 * (wave * 8 + n) + (lane >> 5);
      const int c = lane & 31, u = c >> 1, h = c & 1;
      const int lu = u ^ swz_mn(kr);
      off[n] = (uint32_t)(((int64_t)kr * ld + mn0 + (lu * 2 + h) * 8) * 2);
      lds_off[n] = (wave * 8 + n) * 1024;
    }
  }
  __device__ __forceinline__ void issue(char *lds_tile, int k0) {
    const uint32_t kb = (uint32_t)((int64_t)k0 * ld * 2);
#pragma unroll
    for (int n = 0; n < 8; ++n) copy16(res, lds_tile + lds_off[n], off[n] + kb);
  }
};

// --------------------------------------------------------- fragment reads
// 8 consecutive k (16 bytes) of row `row`, k-group g, half h of a
// K-contiguous tile.
__device__ __forceinline__ u32x4 frag_k(const char *tile, int row, int g, int h) {
  const int ch = (2 * g + h) ^ (row & 7);
  return *reinterpret_cast<const u32x4 *>(tile + row * 128 + ch * 16);
}

// 8 consecutive k of column `col` (= col0 + lane % 32) for k-group g of an
// MN-contiguous tile, via two transposing reads.
__device__ __forceinline__ u32x4 frag_mn(const char *tile, int col0, int g, int lane) {
  const int grp = lane >> 4, i = lane & 15;
  const int kb = 16 * g + 8 * (grp >> 1) + (i >> 2);
  const int c = col0 + 16 * (grp & 1) + 4 * (i & 3);
  const int u = c >> 4, w = (c & 15) * 2;
  const char *p0 = tile + kb * 512 + ((u ^ swz_mn(kb)) << 5) + w;
  const char *p1 = tile + (kb + 4) * 512 + ((u ^ swz_mn(kb + 4)) << 5) + w;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(p0));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(p1));
  u32x4 r;
  r[0] = (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
  r[1] = (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
  r[2] = (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
  r[3] = (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
  return r;
}

__device__ __forceinline__ u32x4 scale8(u32x4 v, float s) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = pack_bf16x2(bf16_lo(v[i]) * s, bf16_hi(v[i]) * s);
  return r;
}

__device__ __forceinline__ void mfma(f32x16 &acc, u32x4 a, u32x4 b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}

__device__ __forceinline__ int acc_row(int e, int lane) {
  return 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
}

__device__ __forceinline__ void zero_acc(f32x16 (&acc)[TM][TN]) {
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
}

__device__ __forceinline__ int xcd_swizzle(int bid, int n) {
  constexpr int NX = 8;
  const int per = (n + NX - 1) / NX;
  const int tall = n % NX == 0 ? NX : n % NX;
  const int x = bid % NX, local = bid / NX;
  return x < tall ? x * per + local : tall * per + (x - tall) * (per - 1) + local;
}

// ------------------------------------------------------------ logits GEMM
// A = H_c (K-contiguous), B = W (K-contiguous).  Epilogue as in kd_gemm.hip:
// per row and segment the max of z/tau, P = exp(z/tau - max) in bf16, the
// sum of P, and z at the row's teacher ids inside the segment.
__global__ __launch_bounds__(NT, 1) void k_fast_logits(SliceArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int nmt = (a.C + BM - 1) / BM;
  const int tile = xcd_swizzle(blockIdx.x, gridDim.x);
  const int mt = tile % nmt, seg = tile / nmt;
  const int m0 = mt * BM, n0 = seg * SEG;
  const uint16_t *H = reinterpret_cast<const uint16_t *>(a.H) + a.c0 * a.d;
  const uint16_t *W = reinterpret_cast<const uint16_t *>(a.W);
  CopyK ca, cb;
  ca.init(H, (uint64_t)a.C * a.d * 2, a.d, m0, wave, lane);
  cb.init(W, (uint64_t)a.V * a.d * 2, a.d, n0, wave, lane);

  f32x16 acc[TM][TN];
  zero_acc(acc);
  const int nk = a.d / BK;
  ca.issue(lds, 0);
  cb.issue(lds + OP_BYTES, 0);
  for (int ks = 0; ks < nk; ++ks) {
    char *cur = lds + (ks & 1) * STAGE_BYTES;
    wait_vm0();
    __syncthreads();
    if (ks + 1 < nk) {
      char *nxt = lds + ((ks + 1) & 1) * STAGE_BYTES;
      ca.issue(nxt, (ks + 1) * BK);
      cb.issue(nxt + OP_BYTES, (ks + 1) * BK);
    }
    const char *ta = cur, *tb = cur + OP_BYTES;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x4 fa[TM], fb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) fa[i] = frag_k(ta, wm * WTM + i * 32 + (lane & 31), g, lane >> 5);
#pragma unroll
      for (int j = 0; j < TN; ++j) fb[j] = frag_k(tb, wn * WTN + j * 32 + (lane & 31), g, lane >> 5);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) mfma(acc[i][j], fa[i], fb[j]);
    }
  }
  __syncthreads();

  // Epilogue: stage one block-row per wave-row (64 rows x 256 columns).
  constexpr int PITCH = BN + 4;
  constexpr int SROWS = 64, TPR = NT / SROWS, CPT = BN / TPR;
  float *stage = reinterpret_cast<float *>(lds);
  uint16_t *P = reinterpret_cast<uint16_t *>(a.P);
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        stage[(wm * 32 + acc_row(e, lane)) * PITCH + wn * WTN + tn * 32 + (lane & 31)] =
            acc[tm][tn][e];
    __syncthreads();
    const int sr = tid / TPR, part = tid % TPR;
    const int r = m0 + (sr >> 5) * WTM + tm * 32 + (sr & 31);
    const int cb0 = part * CPT;
    float v[CPT];
    float mx = -INFINITY;
#pragma unroll
    for (int c = 0; c < CPT; c += 4) {
      const f32x4 z = *reinterpret_cast<const f32x4 *>(stage + sr * PITCH + cb0 + c);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool ok = n0 + cb0 + c + u < a.V;
        v[c + u] = ok ? z[u] * a.inv_tau : -INFINITY;
        mx = fmaxf(mx, v[c + u]);
      }
    }
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    float sum = 0.f;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const float p = v[c] == -INFINITY ? 0.f : exp2f((v[c] - mx) * LOG2E);
      v[c] = p;
      sum += p;
    }
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) sum += __shfl_xor(sum, o, 64);
    if (r < a.C) {
      uint16_t *dst = P + (size_t)r * a.ldp + n0 + cb0;
#pragma unroll
      for (int c = 0; c < CPT; c += 8) {
        u32x4 w{pack_bf16x2(v[c], v[c + 1]), pack_bf16x2(v[c + 2], v[c + 3]),
                pack_bf16x2(v[c + 4], v[c + 5]), pack_bf16x2(v[c + 6], v[c + 7])};
        *reinterpret_cast<u32x4 *>(dst + c) = w;
      }
      if (part == 0) {
        a.mseg[(size_t)r * a.nseg + seg] = mx;
        a.sseg[(size_t)r * a.nseg + seg] = sum;
        int pos = a.first[(size_t)r * a.nseg + seg];
        if (pos >= 0) {
          const int32_t *sid = a.sid + (size_t)r * a.K;
          const int32_t *sslot = a.sslot + (size_t)r * a.K;
          for (; pos < a.K; ++pos) {
            const int id = sid[pos];
            if (id >= n0 + SEG) break;
            a.zg[(size_t)r * a.K + sslot[pos]] = stage[sr * PITCH + (id - n0)];
          }
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- dH GEMM
// A = P (K-contiguous over the vocabulary), scaled on the fragment by
// f[t, seg]; B = W (MN-contiguous: vocabulary rows, hidden columns).
__global__ __launch_bounds__(NT, 1) void k_fast_dh(SliceArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int nmt = (a.C + BM - 1) / BM;
  const int nnt = (a.d + BN - 1) / BN;
  const int tile = xcd_swizzle(blockIdx.x, gridDim.x);
  const int nt = tile % nnt;
  const int mt = (tile / nnt) % nmt;
  const int split = tile / (nnt * nmt);
  const int m0 = mt * BM, n0 = nt * BN;
  const int sbeg = (int)((int64_t)split * a.nseg / a.splits);
  const int send = (int)((int64_t)(split + 1) * a.nseg / a.splits);
  const uint16_t *P = reinterpret_cast<const uint16_t *>(a.P);
  const uint16_t *W = reinterpret_cast<const uint16_t *>(a.W);
  CopyK ca;
  CopyMN cb;
  ca.init(P, (uint64_t)a.C * a.ldp * 2, a.ldp, m0, wave, lane);
  cb.init(W, (uint64_t)a.V * a.d * 2, a.d, n0, wave, lane);

  f32x16 acc[TM][TN];
  zero_acc(acc);
  const int kbeg = sbeg * SEG;
  const int nk = (send - sbeg) * (SEG / BK);
  // rows of this lane's A blocks, for the per-(row, segment) scale
  int arow[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) arow[i] = m0 + wm * WTM + i * 32 + (lane & 31);
  float fsc[TM];
  ca.issue(lds, kbeg);
  cb.issue(lds + OP_BYTES, kbeg);
  for (int ks = 0; ks < nk; ++ks) {
    const int k0 = kbeg + ks * BK;
    if ((ks & (SEG / BK - 1)) == 0) {
      const int sg = k0 / SEG;
#pragma unroll
      for (int i = 0; i < TM; ++i)
        fsc[i] = arow[i] < a.C ? a.fseg[(size_t)arow[i] * a.nseg + sg] : 0.f;
    }
    char *cur = lds + (ks & 1) * STAGE_BYTES;
    wait_vm0();
    __syncthreads();
    if (ks + 1 < nk) {
      char *nxt = lds + ((ks + 1) & 1) * STAGE_BYTES;
      ca.issue(nxt, k0 + BK);
      cb.issue(nxt + OP_BYTES, k0 + BK);
    }
    const char *ta = cur, *tb = cur + OP_BYTES;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x4 fa[TM], fb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        fa[i] = scale8(frag_k(ta, wm * WTM + i * 32 + (lane & 31), g, lane >> 5), fsc[i]);
#pragma unroll
      for (int j = 0; j < TN; ++j) fb[j] = frag_mn(tb, wn * WTN + j * 32, g, lane);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) mfma(acc[i][j], fa[i], fb[j]);
    }
  }

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

// ---------------------------------------------------------------- dW GEMM
// A = P^T (MN-contiguous: token rows, vocabulary columns), B = H_c
// (MN-contiguous: token rows, hidden columns) with token row t scaled by
// f[t, seg] while it passes through registers.
__global__ __launch_bounds__(NT, 1) void k_fast_dw(SliceArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int nnt = (a.d + BN - 1) / BN;
  const int tile = xcd_swizzle(blockIdx.x, gridDim.x);
  const int nt = tile % nnt, mt = tile / nnt;
  const int m0 = mt * BM, n0 = nt * BN;
  const int seg = m0 / SEG;
  const uint16_t *P = reinterpret_cast<const uint16_t *>(a.P);
  const uint16_t *H = reinterpret_cast<const uint16_t *>(a.H) + a.c0 * a.d;
  CopyMN ca;
  ca.init(P, (uint64_t)a.C * a.ldp * 2, a.ldp, m0, wave, lane);

  // B through registers: thread covers k-rows kr = tid/32 + 8*n (n < 8),
  // 16-byte chunk c = tid % 32 of the 512-byte row.
  const int bc = tid & 31;
  const int bcol = n0 + bc * 8;
  u32x4 breg[8];
  float bsc[8];
  auto load_b = [&](int k0) {
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const int t = k0 + (tid >> 5) + 8 * n;
      const bool ok = t < a.C && bcol < a.d;
      breg[n] = ok ? *reinterpret_cast<const u32x4 *>(H + (size_t)t * a.d + bcol)
                   : u32x4{0u, 0u, 0u, 0u};
      bsc[n] = t < a.C ? a.fseg[(size_t)t * a.nseg + seg] : 0.f;
    }
  };
  auto store_b = [&](char *tile_b) {
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const int kr = (tid >> 5) + 8 * n;
      const int u = bc >> 1, h = bc & 1;
      *reinterpret_cast<u32x4 *>(tile_b + kr * 512 + ((u ^ swz_mn(kr)) << 5) + h * 16) =
          scale8(breg[n], bsc[n]);
    }
  };

  f32x16 acc[TM][TN];
  zero_acc(acc);
  const int nk = (a.C + BK - 1) / BK;
  ca.issue(lds, 0);
  load_b(0);
  store_b(lds + OP_BYTES);
  for (int ks = 0; ks < nk; ++ks) {
    char *cur = lds + (ks & 1) * STAGE_BYTES;
    wait_vm0();
    __syncthreads();
    const bool more = ks + 1 < nk;
    char *nxt = lds + ((ks + 1) & 1) * STAGE_BYTES;
    if (more) {
      ca.issue(nxt, (ks + 1) * BK);
      load_b((ks + 1) * BK);
    }
    const char *ta = cur, *tb = cur + OP_BYTES;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x4 fa[TM], fb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) fa[i] = frag_mn(ta, wm * WTM + i * 32, g, lane);
#pragma unroll
      for (int j = 0; j < TN; ++j) fb[j] = frag_mn(tb, wn * WTN + j * 32, g, lane);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) mfma(acc[i][j], fa[i], fb[j]);
    }
    if (more) store_b(nxt + OP_BYTES);
  }

#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = n0 + wn * WTN + j * 32 + (lane & 31);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wm * WTM + i * 32 + acc_row(e, lane);
        if (row < a.V && col < a.d) {
          float *p = a.dW + (size_t)row * a.d + col;
          *p = a.dw_beta ? *p + acc[i][j][e] : acc[i][j][e];
        }
      }
    }
}

template <typename K>
hipError_t launch(K kern, int grid, const SliceArgs &a, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NT), LDS_BYTES, s, a);
  return hipGetLastError();
}

}  // namespace

// Splits of the vocabulary contraction of dH: about three full rounds of
// one workgroup per CU.
int fast_dh_splits(int C, int d, int nseg) {
  const int tiles = ((C + BM - 1) / BM) * ((d + BN - 1) / BN);
  int s = (768 + tiles - 1) / tiles;
  if (s < 1) s = 1;
  if (s > nseg) s = nseg;
  return s;
}

hipError_t launch_fast_logits(const SliceArgs &a, hipStream_t s) {
  return launch(k_fast_logits, ((a.C + BM - 1) / BM) * a.nseg, a, s);
}

hipError_t launch_fast_dh(const SliceArgs &a, hipStream_t s) {
  return launch(k_fast_dh, ((a.C + BM - 1) / BM) * ((a.d + BN - 1) / BN) * a.splits, a, s);
}

hipError_t launch_fast_dw(const SliceArgs &a, hipStream_t s) {
  return launch(k_fast_dw, ((a.V + BM - 1) / BM) * ((a.d + BN - 1) / BN), a, s);
}

}  // namespace kd
