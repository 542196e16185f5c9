// The three matrix-core GEMMs of the fused, chunked top-K KL loss on gfx950.
//
//  logits:  Z = H_c W^T        (C x V, K = d)   with a softmax-statistics and
//           teacher-gather epilogue; stores P = 2^(z s2 - shift_seg) (base-2
//           units, s2 = log2(e) / tau)
//  dH:      dH_c = G W         (C x d, K = V)   split-K over vocabulary
//  dW:      dW (+)= G^T H_c    (V x d, K = C)
//
// where G (the logit gradient of the chunk, tau/N * mask * (p - q_scat)) is
// written by k_lse_fix over the buffer the logits GEMM filled with P.  This follows the pages' fused, chunked KL
// ("Making Knowledge Distillation Cheap Enough to Run at Scale", aipuls.nl,
// section "Summary"; "Hugging Face and Multiverse Computing cut KD memory
// costs", agent-gateway.com): only one slice's [C, V] block ever exists.
//
// Structure shared by all three: a 256-thread workgroup computes a BM x BN
// tile with 4 waves (2 x 2); each wave owns (BM/2) x (BN/2) as 32 x 32 MFMA
// blocks.  Operand tiles of one k-step (128 bytes of K per row) are staged
// through LDS, double-buffered, in a [row][k] layout with the 16-byte chunk
// index XOR-swizzled by (row & 7) so that fragment reads are conflict-free.
// Operands whose contraction index is not contiguous in memory are
// transposed in registers (8 x 8 bf16 or 4 x 4 fp32 blocks) on their way
// into LDS.  bf16 uses v_mfma_f32_32x32x16_bf16, fp32 v_mfma_f32_32x32x2_f32;
// accumulation is fp32 in both.
#include "kd_device.h"
#include "kd_internal.h"

namespace kd {

namespace {

constexpr int NTHREADS = 256;
constexpr int ROWB = 128;  // bytes of K per LDS row and k-step

template <int BM_, int BN_>
struct Tile {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int WM = 2, WN = 2;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int TM = WTM / 32, TN = WTN / 32;
  static constexpr int STAGE = (BM + BN) * ROWB;
  static constexpr int LDS = 2 * STAGE;
  static_assert(TM >= 1 && TN >= 1, "tile too small");
};

__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * ROWB + ((chunk ^ (row & 7)) << 4);
}

// ---------------------------------------------------------------- loaders
// Operand element (mn, k) at base[mn * ld + k]: rows of 128 bytes.  With
// SCALED, every element of row mn is multiplied by fs[mn * fld + k0 / SEG]
// (one segment per k-step since SEG is a multiple of the k-step).
template <typename T, int R, bool SCALED>
struct LoadK {
  static constexpr int E = Elem<T>::PER16B;
  static constexpr int N = R * 8 / NTHREADS;
  static_assert(N >= 1, "rows");
  const T *base;
  int64_t ld;
  int mn_lim, k_lim;
  const float *fs;
  int fld;
  u32x4 reg[N];
  float sc[N];

  __device__ __forceinline__ void load(int mn0, int k0, int tid) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int idx = tid + NTHREADS * i;
      const int row = idx >> 3, ch = idx & 7;
      const int mn = mn0 + row, k = k0 + ch * E;
      if (mn < mn_lim && k < k_lim)
        reg[i] = *reinterpret_cast<const u32x4 *>(base + mn * ld + k);
      else
        reg[i] = u32x4{0u, 0u, 0u, 0u};
      if (SCALED) sc[i] = mn < mn_lim ? fs[(int64_t)mn * fld + k0 / SEG] : 0.f;
    }
  }
  __device__ __forceinline__ void store(char *lds, int tid) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int idx = tid + NTHREADS * i;
      const int row = idx >> 3, ch = idx & 7;
      u32x4 v = reg[i];
      if (SCALED) v = Elem<T>::scale(v, sc[i]);
      *reinterpret_cast<u32x4 *>(lds + lds_off(row, ch)) = v;
    }
  }
};

// Operand element (mn, k) at base[k * ld + mn]: E x E blocks (E elements
// per 16 bytes) are read as E rows of 16 bytes along mn and transposed in
// registers into E rows of 16 bytes along k.  With SCALED, row k is
// multiplied by fs[k * fstride] before the transpose.
template <typename T, int R, bool SCALED>
struct LoadMN {
  static constexpr int E = Elem<T>::PER16B;
  static constexpr int NB = (R / E) * 8;  // blocks per tile and k-step
  static constexpr int N = (NB + NTHREADS - 1) / NTHREADS;
  const T *base;
  int64_t ld;
  int mn_lim, k_lim;
  const float *fs;
  int64_t fstride;
  u32x4 reg[N][E];
  float sc[N][E];

  __device__ __forceinline__ void load(int mn0, int k0, int tid) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int b = tid + NTHREADS * i;
      if (NB % NTHREADS == 0 || b < NB) {
        const int mb = b % (R / E), kb = b / (R / E);
        const int mn = mn0 + mb * E;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int k = k0 + kb * E + e;
          if (mn < mn_lim && k < k_lim)
            reg[i][e] = *reinterpret_cast<const u32x4 *>(base + k * ld + mn);
          else
            reg[i][e] = u32x4{0u, 0u, 0u, 0u};
          if (SCALED) sc[i][e] = k < k_lim ? fs[k * fstride] : 0.f;
        }
      }
    }
  }
  __device__ __forceinline__ void store(char *lds, int tid) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int b = tid + NTHREADS * i;
      if (NB % NTHREADS == 0 || b < NB) {
        const int mb = b % (R / E), kb = b / (R / E);
        u32x4 in[E];
#pragma unroll
        for (int e = 0; e < E; ++e)
          in[e] = SCALED ? Elem<T>::scale(reg[i][e], sc[i][e]) : reg[i][e];
        if constexpr (E == 8) {
          // 8 x 8 of 16-bit: out[m].dword[p] = (in[2p].half(m), in[2p+1].half(m))
#pragma unroll
          for (int m = 0; m < 8; ++m) {
            u32x4 o;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              const uint32_t lo = in[2 * p][m >> 1], hi = in[2 * p + 1][m >> 1];
              o[p] = (m & 1) ? ((lo >> 16) | (hi & 0xffff0000u))
                             : ((lo & 0xffffu) | (hi << 16));
            }
            *reinterpret_cast<u32x4 *>(lds + lds_off(mb * 8 + m, kb)) = o;
          }
        } else {
          // 4 x 4 of 32-bit
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            u32x4 o{in[0][m], in[1][m], in[2][m], in[3][m]};
            *reinterpret_cast<u32x4 *>(lds + lds_off(mb * 4 + m, kb)) = o;
          }
        }
      }
    }
  }
};

// ------------------------------------------------------------ MFMA k-step
// Group g of a k-step covers LDS chunks 2g (lanes 0-31) and 2g+1 (lanes
// 32-63).  bf16: one 32x32x16 MFMA per group whose lane l supplies the 8
// k-values of its chunk.  fp32: four 32x32x2 MFMAs per group, MFMA e using
// element e of the chunk; A and B use the same k assignment, so every k of
// the step is summed exactly once.
template <typename T, class TL>
__device__ __forceinline__ void mma_kstep(const char *la, const char *lb,
                                          f32x16 (&acc)[TL::TM][TL::TN],
                                          int wm, int wn, int lane) {
  const int r = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int ch = 2 * g + hi;
    u32x4 a[TL::TM], b[TL::TN];
#pragma unroll
    for (int i = 0; i < TL::TM; ++i)
      a[i] = *reinterpret_cast<const u32x4 *>(la + lds_off(wm * TL::WTM + i * 32 + r, ch));
#pragma unroll
    for (int j = 0; j < TL::TN; ++j)
      b[j] = *reinterpret_cast<const u32x4 *>(lb + lds_off(wn * TL::WTN + j * 32 + r, ch));
#pragma unroll
    for (int i = 0; i < TL::TM; ++i)
#pragma unroll
      for (int j = 0; j < TL::TN; ++j) {
        if constexpr (sizeof(T) == 2) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, a[i]), __builtin_bit_cast(bf16x8, b[j]),
              acc[i][j], 0, 0, 0);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                __uint_as_float(a[i][e]), __uint_as_float(b[j][e]), acc[i][j], 0, 0, 0);
        }
      }
  }
}

// Main loop over k in [kbeg, kend), double-buffered through LDS.
template <typename T, class TL, class LA, class LB>
__device__ __forceinline__ void mainloop(LA &la, LB &lb, int m0, int n0, int kbeg,
                                         int kend, char *lds,
                                         f32x16 (&acc)[TL::TM][TL::TN]) {
  constexpr int KB = ROWB / (int)sizeof(T);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / TL::WN, wn = wave % TL::WN;
#pragma unroll
  for (int i = 0; i < TL::TM; ++i)
#pragma unroll
    for (int j = 0; j < TL::TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  const int nk = (kend - kbeg + KB - 1) / KB;
  if (nk <= 0) return;
  la.load(m0, kbeg, tid);
  lb.load(n0, kbeg, tid);
  la.store(lds, tid);
  lb.store(lds + TL::BM * ROWB, tid);
  __syncthreads();
  for (int ks = 0; ks < nk; ++ks) {
    char *cur = lds + (ks & 1) * TL::STAGE;
    char *nxt = lds + ((ks + 1) & 1) * TL::STAGE;
    const bool more = ks + 1 < nk;
    if (more) {
      la.load(m0, kbeg + (ks + 1) * KB, tid);
      lb.load(n0, kbeg + (ks + 1) * KB, tid);
    }
    mma_kstep<T, TL>(cur, cur + TL::BM * ROWB, acc, wm, wn, lane);
    if (more) {
      la.store(nxt, tid);
      lb.store(nxt + TL::BM * ROWB, tid);
    }
    __syncthreads();
  }
}

// Position of accumulator element e of a 32x32 block for this lane.
__device__ __forceinline__ int acc_row(int e, int lane) {
  return 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
}

// ------------------------------------------------------------ logits GEMM
// Tile (mt, seg): rows m0.. of the slice, vocabulary segment seg.  Epilogue,
// per row: shift = max_v z/tau over the segment, P = exp(z/tau - shift)
// (0 beyond V), sum = sum P, and z itself at every teacher id of the row
// that falls in the segment (the LDS gather of the student logits).
template <typename T>
__global__ __launch_bounds__(NTHREADS) void k_gemm_logits(SliceArgs a) {
  using TL = Tile<G1_BM, G1_BN>;
  static_assert(TL::BN == SEG, "logits tile must be one segment wide");
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int nmt = (a.C + TL::BM - 1) / TL::BM;
  const int tile = xcd_swizzle(blockIdx.x, gridDim.x);
  const int mt = tile % nmt, seg = tile / nmt;
  const int m0 = mt * TL::BM, n0 = seg * SEG;
  const T *H = reinterpret_cast<const T *>(a.H) + a.c0 * a.d;
  const T *W = reinterpret_cast<const T *>(a.W);
  LoadK<T, TL::BM, false> la{H, a.d, a.C, a.d, nullptr, 0};
  LoadK<T, TL::BN, false> lb{W, a.d, a.V, a.d, nullptr, 0};
  f32x16 acc[TL::TM][TL::TN];
  mainloop<T, TL>(la, lb, m0, n0, 0, a.d, lds, acc);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / TL::WN, wn = wave % TL::WN;
  constexpr int PITCH = TL::BN + 4;            // floats per staged row
  constexpr int SROWS = TL::WM * 32;           // staged rows per pass
  constexpr int TPR = NTHREADS / SROWS;        // threads per row
  constexpr int CPT = TL::BN / TPR;            // columns per thread
  static_assert(SROWS * PITCH * 4 <= TL::LDS, "staging does not fit");
  static_assert(CPT % 8 == 0, "columns per thread");
  float *stage = reinterpret_cast<float *>(lds);
  T *P = reinterpret_cast<T *>(a.P);
#pragma unroll
  for (int tm = 0; tm < TL::TM; ++tm) {
#pragma unroll
    for (int tn = 0; tn < TL::TN; ++tn)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        stage[(wm * 32 + acc_row(e, lane)) * PITCH + wn * TL::WTN + tn * 32 + (lane & 31)] =
            acc[tm][tn][e];
    __syncthreads();
    const int sr = tid / TPR, part = tid % TPR;
    const int r = m0 + (sr / 32) * TL::WTM + tm * 32 + (sr % 32);
    const int c0 = part * CPT;
    // base-2 units: shift = max(z) s2, P = 2^(z s2 - shift) with one
    // rounding of the exponent (fma), so P keeps its relative accuracy
    // however large z s2 itself is
    float v[CPT];
    float zmax = -INFINITY;
#pragma unroll
    for (int c = 0; c < CPT; c += 4) {
      const f32x4 z = *reinterpret_cast<const f32x4 *>(stage + sr * PITCH + c0 + c);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool ok = n0 + c0 + c + u < a.V;
        v[c + u] = ok ? z[u] : -INFINITY;
        zmax = fmaxf(zmax, v[c + u]);
      }
    }
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) zmax = fmaxf(zmax, __shfl_xor(zmax, o, 64));
    const float mx = zmax * a.s2;
    float sum = 0.f;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const float p = v[c] == -INFINITY ? 0.f : exp2f(fmaf(v[c], a.s2, -mx));
      v[c] = p;
      sum += p;
    }
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) sum += __shfl_xor(sum, o, 64);
    if (r < a.C) {
      T *dst = P + (size_t)r * a.ldp + n0 + c0;
      if (!a.need_grad) {
        // forward only: the probabilities are not needed
      } else if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int c = 0; c < CPT; c += 8) {
          u32x4 w{pack_bf16x2(v[c], v[c + 1]), pack_bf16x2(v[c + 2], v[c + 3]),
                  pack_bf16x2(v[c + 4], v[c + 5]), pack_bf16x2(v[c + 6], v[c + 7])};
          *reinterpret_cast<u32x4 *>(dst + c) = w;
        }
      } else {
#pragma unroll
        for (int c = 0; c < CPT; c += 4)
          *reinterpret_cast<f32x4 *>(dst + c) = f32x4{v[c], v[c + 1], v[c + 2], v[c + 3]};
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
// Tile (mt, nt, split): dH partial of rows m0.., columns n0.., over the
// vocabulary segments of the split.  A = G, B = W with the vocabulary as
// contraction index (transposed while loading).
template <typename T>
__global__ __launch_bounds__(NTHREADS) void k_gemm_dh(SliceArgs a) {
  using TL = Tile<DH_BM, DH_BN>;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int nmt = (a.C + TL::BM - 1) / TL::BM;
  const int nnt = (a.d + TL::BN - 1) / TL::BN;
  const int tile = xcd_swizzle(blockIdx.x, gridDim.x);
  const int nt = tile % nnt;
  const int mt = (tile / nnt) % nmt;
  const int split = tile / (nnt * nmt);
  const int m0 = mt * TL::BM, n0 = nt * TL::BN;
  const int sbeg = (int)((int64_t)split * a.nseg / a.splits);
  const int send = (int)((int64_t)(split + 1) * a.nseg / a.splits);
  const int kbeg = sbeg * SEG, kend = send * SEG;
  const T *P = reinterpret_cast<const T *>(a.P);
  const T *W = reinterpret_cast<const T *>(a.W);
  LoadK<T, TL::BM, false> la{P, a.ldp, a.C, kend, nullptr, 0};
  LoadMN<T, TL::BN, false> lb{W, a.d, a.d, kend < a.V ? kend : a.V, nullptr, 0};
  f32x16 acc[TL::TM][TL::TN];
  mainloop<T, TL>(la, lb, m0, n0, kbeg, kend, lds, acc);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / TL::WN, wn = wave % TL::WN;
  float *out = a.dh_part + (size_t)split * a.dh_stride;
#pragma unroll
  for (int i = 0; i < TL::TM; ++i)
#pragma unroll
    for (int j = 0; j < TL::TN; ++j) {
      const int col = n0 + wn * TL::WTN + j * 32 + (lane & 31);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wm * TL::WTM + i * 32 + acc_row(e, lane);
        if (row < a.C && col < a.d) out[(size_t)row * a.d + col] = acc[i][j][e];
      }
    }
}

// ---------------------------------------------------------------- dW GEMM
// Tile (mt, nt): dW rows m0.. (vocabulary), columns n0..; contraction over
// the slice's tokens.  A = G^T and B = H_c, both transposed while loading.
template <typename T>
__global__ __launch_bounds__(NTHREADS) void k_gemm_dw(SliceArgs a) {
  using TL = Tile<DW_BM, DW_BN>;
  static_assert(SEG % TL::BM == 0, "dW tile must stay inside a segment");
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int nnt = (a.d + TL::BN - 1) / TL::BN;
  const int tile = xcd_swizzle(blockIdx.x, gridDim.x);
  const int nt = tile % nnt, mt = tile / nnt;
  const int m0 = mt * TL::BM, n0 = nt * TL::BN;
  const T *P = reinterpret_cast<const T *>(a.P);
  const T *H = reinterpret_cast<const T *>(a.H) + a.c0 * a.d;
  LoadMN<T, TL::BM, false> la{P, a.ldp, a.ldp, a.C, nullptr, 0};
  LoadMN<T, TL::BN, false> lb{H, a.d, a.d, a.C, nullptr, 0};
  f32x16 acc[TL::TM][TL::TN];
  mainloop<T, TL>(la, lb, m0, n0, 0, a.C, lds, acc);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / TL::WN, wn = wave % TL::WN;
#pragma unroll
  for (int i = 0; i < TL::TM; ++i)
#pragma unroll
    for (int j = 0; j < TL::TN; ++j) {
      const int col = n0 + wn * TL::WTN + j * 32 + (lane & 31);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wm * TL::WTM + i * 32 + acc_row(e, lane);
        if (row < a.V && col < a.d) {
          float *p = a.dW + (size_t)row * a.d + col;
          *p = a.dw_beta ? *p + acc[i][j][e] : acc[i][j][e];
        }
      }
    }
}

template <typename K>
hipError_t launch(K kern, int grid, int lds_bytes, const SliceArgs &a, hipStream_t s) {
  static_assert(sizeof(SliceArgs) < 4096, "kernel argument size");
  if (grid <= 0) return hipSuccess;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     lds_bytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NTHREADS), lds_bytes, s, a);
  return hipGetLastError();
}

}  // namespace

bool use_fast(bool bf16, int64_t C, int64_t d, int64_t V, int64_t ldp) {
  // Within a tile the buffer offsets are (row < 256) * pitch + k bytes, so
  // pitches (ldp, the slice's token count, d) stay far below 2^31 / 512.
  const int64_t lim = int64_t(1) << 22;
  return bf16 && d % 64 == 0 && d < lim && ldp < lim && C < lim && V < (int64_t(1) << 31);
}

int dh_splits(int C, int d, int nseg, bool fast, int bn) {
  if (fast) return fast_dh_splits(C, d, nseg, bn);
  const int tiles = ((C + DH_BM - 1) / DH_BM) * ((d + DH_BN - 1) / DH_BN);
  int s = (1024 + tiles - 1) / tiles;
  if (s < 1) s = 1;
  if (s > nseg) s = nseg;
  return s;
}

hipError_t launch_gemm_logits(const SliceArgs &a, bool bf16, hipStream_t s) {
  if (a.fast) return launch_fast_logits(a, s);
  using TL = Tile<G1_BM, G1_BN>;
  const int grid = ((a.C + TL::BM - 1) / TL::BM) * a.nseg;
  return bf16 ? launch(k_gemm_logits<uint16_t>, grid, TL::LDS, a, s)
              : launch(k_gemm_logits<float>, grid, TL::LDS, a, s);
}

hipError_t launch_gemm_dh(const SliceArgs &a, bool bf16, hipStream_t s) {
  if (a.fast) return launch_fast_dh(a, s);
  using TL = Tile<DH_BM, DH_BN>;
  const int grid = ((a.C + TL::BM - 1) / TL::BM) * ((a.d + TL::BN - 1) / TL::BN) * a.splits;
  return bf16 ? launch(k_gemm_dh<uint16_t>, grid, TL::LDS, a, s)
              : launch(k_gemm_dh<float>, grid, TL::LDS, a, s);
}

hipError_t launch_gemm_dw(const SliceArgs &a, bool bf16, hipStream_t s) {
  if (a.fast) return launch_fast_dw(a, s);
  using TL = Tile<DW_BM, DW_BN>;
  const int grid = ((a.V + TL::BM - 1) / TL::BM) * ((a.d + TL::BN - 1) / TL::BN);
  return bf16 ? launch(k_gemm_dw<uint16_t>, grid, TL::LDS, a, s)
              : launch(k_gemm_dw<float>, grid, TL::LDS, a, s);
}

}  // namespace kd
