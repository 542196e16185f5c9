// Teacher top-K cache builder: for every token row t, the K largest entries
// of z[t,:] = H[t,:] W^T (the teacher's LM-head logits) with their
// vocabulary ids, sorted by value descending, equal values by id ascending.
// This is the offline step of the method ("Making Knowledge Distillation
// Cheap Enough to Run at Scale", aipuls.nl, section "Summary": the teacher
// runs once and its top-100 logits per position are cached), built so that
// the token-by-vocabulary logit matrix never exists.
//
// Order.  Every entry (value v, id i) is mapped to a 64-bit key whose high
// word decreases as v increases (an order-preserving map of the fp32 bits,
// -0 folded onto +0) and whose low word is i; a smaller key is a better
// entry, and keys are distinct within a row.  The K best entries are the K
// smallest keys.
//
// Tuned path (bf16, d % 64 == 0), per slice of C rows:
//  1. k_tk_gemm<SAMPLE>: logits of ns evenly spaced vocabulary segments
//     (segment 0 included; ns = 32, or more for large K nseg so that about
//     K nseg / ns <= TK_CAP / 2 candidates are expected per row), written to
//     a small [C, ns*256] buffer.
//  2. k_tk_theta: per row, the K-th smallest key among the sampled entries
//     (radix select).  The K sampled entries are real entries of the row, so
//     the row's K-th smallest key is no larger: every top-K entry has a key
//     <= this threshold.  The K sampled entries at or below it are the first
//     candidates of the row.
//  3. k_tk_gemm<FILTER>: the logits of every other segment, on the same
//     MFMA code as step 1; the epilogue appends the entries whose key is <=
//     the row's threshold to the row's candidate list (about K * nseg / ns
//     of them for logits without structure).
//  4. k_tk_select: per row, the exact K smallest candidate keys (radix
//     select, then a sort of those K).
//  5. k_tk_stream: rows whose candidates overflowed TK_CAP slots are
//     recomputed entry by entry and reduced with a streaming top-K.
// Generic path (fp32 or d % 64 != 0): step 5 for every row.
#include <stdint.h>

#include "kd_device.h"
#include "kd_internal.h"
#include "kd_mfma_tile.h"
#include "kd_select.h"

namespace kd {

namespace {

using namespace tile;
using namespace sel;

// Writes the first K keys of top[] (sorted) as the output row t.
__device__ __forceinline__ void write_row(const TkArgs &a, int64_t t, const uint64_t *top) {
  for (int k = threadIdx.x; k < a.K; k += blockDim.x) {
    a.out_idx[t * a.K + k] = int32_t(uint32_t(top[k]));
    a.out_val[t * a.K + k] = key_val(uint32_t(top[k] >> 32));
  }
}

// ------------------------------------------------------------ the GEMM
constexpr int SAMPLE = 0, FILTER = 1;

// Tile (mt, segment) of z = H_c W^T on the 4-wave bf16 main loop.
// SAMPLE: the tile columns are sampled segment nt, stored to zs.  FILTER:
// every non-sampled segment; entries with key <= the row's threshold are
// appended to the row's candidates.
template <int MODE>
__global__ __launch_bounds__(w4::NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_tk_gemm(TkArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int nmt = (a.C + BM - 1) / BM;
  const int tile = xcd_swizzle(blockIdx.x, gridDim.x);
  int mt, nt;
  group_tile(tile, nmt, MODE == SAMPLE ? a.ns : a.nseg, 4, mt, nt);
  const int seg = MODE == SAMPLE ? nt * a.sstride : nt;
  if (MODE == FILTER && seg % a.sstride == 0 && seg / a.sstride < a.ns) return;
  const int m0 = mt * BM, n0 = seg * SEG;
  const uint16_t *H = reinterpret_cast<const uint16_t *>(a.H) + a.c0 * a.d;
  const uint16_t *W = reinterpret_cast<const uint16_t *>(a.W);
  using S = w4::Square;
  w4::Copy<S::RA> ca;
  w4::Copy<S::RB> cb;
  ca.init(H, (uint64_t)a.C * a.d * 2, a.d, m0, wave, lane);
  cb.init(W, (uint64_t)a.V * a.d * 2, a.d, n0, wave, lane);

  // Epilogue layout (as the loss's logits GEMM): 4 passes of 64 tile rows
  // (block-rows 2p, 2p + 1 of both wave rows), 8 threads per row with 32
  // contiguous columns each, 2 rows per thread.
  constexpr int PITCH = BN + 4;
  constexpr int TPR = 8, RPT = 2, CPT = BN / TPR;
  const int part = tid % TPR;
  auto row_of = [&](int pass, int q) {
    const int sr = tid / TPR + q * (w4::NT / TPR);
    return m0 + (sr >> 5) * 128 + (2 * pass + ((sr >> 4) & 1)) * 16 + (sr & 15);
  };
  f32x4 acc[8][8];
  w4::nt_loop<S>(ca, cb, 0, a.d / BK, lds, wm, wn, lane, acc);
  w4::acc_ready(acc);
  __syncthreads();

  float *stage = reinterpret_cast<float *>(lds);
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    // thresholds of this pass's rows (their latency overlaps the staging)
    float th_v[RPT];
    int th_i[RPT];
    if (MODE == FILTER) {
#pragma unroll
      for (int q = 0; q < RPT; ++q) {
        const int r = row_of(pass, q);
        th_v[q] = r < a.C ? a.th_v[r] : INFINITY;
        th_i[q] = r < a.C ? a.th_i[r] : -1;
      }
    }
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          stage[(wm * 32 + ii * 16 + 4 * (lane >> 4) + e) * PITCH + wn * 128 +
                w4::acc_col4(j, lane)] = acc[2 * pass + ii][j][e];
    __syncthreads();
    const int cb0 = part * CPT;
    if (MODE == SAMPLE) {
#pragma unroll
      for (int q = 0; q < RPT; ++q) {
        const int sr = tid / TPR + q * (w4::NT / TPR);
        const int r = row_of(pass, q);
        const float *srow = stage + sr * PITCH + cb0;
        if (r < a.C) {
          float *dst = a.zs + (size_t)r * a.ldzs + nt * SEG + cb0;
#pragma unroll
          for (int c = 0; c < CPT; c += 4)
            *reinterpret_cast<f32x4 *>(dst + c) = *reinterpret_cast<const f32x4 *>(srow + c);
        }
      }
    } else {
      // The thread's two rows in three phases, so that their candidate
      // counters take one atomic round trip together: (1) which of its 32
      // columns pass the row's threshold, their count and its exclusive
      // prefix over the row's 8 threads; (2) one atomic add per row by the
      // row's last thread, reserving the row's slots; (3) the candidates.
      uint32_t mq[RPT];
      int exq[RPT], totq[RPT], bq[RPT];
#pragma unroll
      for (int q = 0; q < RPT; ++q) {
        const int sr = tid / TPR + q * (w4::NT / TPR);
        const float *srow = stage + sr * PITCH + cb0;
        const float tv = th_v[q];
        const int ti = th_i[q];
        uint32_t m = 0u;
#pragma unroll
        for (int c = 0; c < CPT; c += 4) {
          const f32x4 z = *reinterpret_cast<const f32x4 *>(srow + c);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int id = n0 + cb0 + c + u;
            const bool hit = z[u] > tv || (z[u] == tv && id <= ti);
            m |= uint32_t(hit) << (c + u);
          }
        }
        const int lim = a.V - (n0 + cb0);  // columns of this thread below V
        if (lim < CPT) m = lim <= 0 ? 0u : (m & ((1u << lim) - 1u));
        const int n = __popc(m);
        mq[q] = m;
        exq[q] = group8_scan_i(n, part) - n;
        totq[q] = group8_sum_i(n);
      }
#pragma unroll
      for (int q = 0; q < RPT; ++q) {
        const int r = row_of(pass, q);
        bq[q] = 0;
        if (part == TPR - 1 && totq[q] > 0 && r < a.C) bq[q] = atomicAdd(a.cnt + r, totq[q]);
      }
#pragma unroll
      for (int q = 0; q < RPT; ++q) {
        const int sr = tid / TPR + q * (w4::NT / TPR);
        const int r = row_of(pass, q);
        const float *srow = stage + sr * PITCH + cb0;
        const int base = group8_sum_i(bq[q]);  // (only the last thread's is nonzero)
        uint32_t m = mq[q];
        if (m != 0u && r < a.C) {
          int pos = base + exq[q];
          uint64_t *dst = a.cand + (size_t)r * a.cap;
          while (m != 0u) {
            const int i = __builtin_ctz(m);
            m &= m - 1u;
            if (pos < a.cap) dst[pos] = make_key(srow[i], n0 + cb0 + i);
            ++pos;
          }
        }
        if (part == TPR - 1 && r < a.C && totq[q] > 0 && base + totq[q] > a.cap) a.ovf[r] = 1;
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------- row threshold
// One workgroup per row: the K-th smallest key among the sampled entries,
// and those K entries as the row's first candidates.
__global__ __launch_bounds__(256) void k_tk_theta(TkArgs a) {
  extern __shared__ uint32_t hi[];  // ns * SEG
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sc[8];
  __shared__ uint64_t res;
  __shared__ int nc;
  const int r = blockIdx.x, tid = threadIdx.x;
  const int n = a.ns * SEG;
  const int sstride = a.sstride;
  const float *src = a.zs + (size_t)r * a.ldzs;
  auto id_of = [sstride](int i) { return (i / SEG) * sstride * SEG + (i % SEG); };
  // n is a multiple of 256 (ns segments): 16-byte loads, U of a thread's
  // loads in flight before their use
  constexpr int U = 8;
  for (int base = 0; base < n; base += U * 1024) {
    f32x4 zv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = base + (u * 256 + tid) * 4;
      if (i < n) zv[u] = *reinterpret_cast<const f32x4 *>(src + i);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = base + (u * 256 + tid) * 4;
      if (i < n) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          // entries past the vocabulary rank after every real entry
          hi[i + c] = id_of(i + c) < a.V ? key_hi(zv[u][c]) : 0xffffffffu;
        }
      }
    }
  }
  if (tid == 0) nc = 0;
  __syncthreads();
  auto key_at = [&](int i) { return (uint64_t(hi[i]) << 32) | uint32_t(id_of(i)); };
  const uint64_t th = block_select(key_at, n, a.K - 1, hist, sc, &res);
  uint64_t *dst = a.cand + (size_t)r * a.cap;
  for (int i = tid; i < n; i += 256) {
    const uint64_t k = key_at(i);
    if (k <= th) dst[atomicAdd(&nc, 1)] = k;
  }
  if (tid == 0) {
    a.th_v[r] = key_val(uint32_t(th >> 32));
    a.th_i[r] = int32_t(uint32_t(th));
    a.cnt[r] = a.K;
    a.ovf[r] = 0;
  }
}

// ------------------------------------------------------- exact selection
// One workgroup per row: the K smallest candidate keys, sorted.  Rows whose
// candidates overflowed are left to k_tk_stream.
__global__ __launch_bounds__(256) void k_tk_select(TkArgs a) {
  extern __shared__ uint64_t keys[];  // TK_CAP
  __shared__ uint64_t top[256];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sc[8];
  __shared__ uint64_t res;
  __shared__ int nsel;
  const int r = blockIdx.x, tid = threadIdx.x;
  if (a.ovf[r]) return;
  const int cnt = a.cnt[r];
  const int n = cnt < a.cap ? cnt : a.cap;
  const uint64_t *src = a.cand + (size_t)r * a.cap;
  // 16-byte loads, eight in flight per thread
  for (int base = 0; base < n; base += 256 * 16) {
    u32x4 kv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = base + (u * 256 + tid) * 2;
      if (i + 1 < n) kv[u] = *reinterpret_cast<const u32x4 *>(src + i);
      else if (i < n) kv[u] = u32x4{uint32_t(src[i]), uint32_t(src[i] >> 32), 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = base + (u * 256 + tid) * 2;
      if (i < n) keys[i] = uint64_t(kv[u][0]) | (uint64_t(kv[u][1]) << 32);
      if (i + 1 < n) keys[i + 1] = uint64_t(kv[u][2]) | (uint64_t(kv[u][3]) << 32);
    }
  }
  if (tid == 0) nsel = 0;
  __syncthreads();
  const uint64_t th = block_select([&](int i) { return keys[i]; }, n, a.K - 1, hist, sc, &res);
  for (int i = tid; i < n; i += 256)
    if (keys[i] <= th) top[atomicAdd(&nsel, 1)] = keys[i];
  const int P = pow2_at_least(a.K);
  for (int i = a.K + tid; i < P; i += 256) top[i] = ~0ull;
  __syncthreads();
  bitonic_sort(top, P);
  write_row(a, a.c0 + r, top);
}

// ------------------------------------------------- row-streaming top-K
// One workgroup per row: z[t, v] = sum_j H[t,j] W[v,j] in fp32 (fused
// multiply-adds in j order), 256 ids at a time; entries better than the
// current K-th are buffered and merged (sorted) when the buffer fills.
template <typename T>
__global__ __launch_bounds__(256) void k_tk_stream(TkArgs a) {
  extern __shared__ float hs[];  // d
  __shared__ uint64_t arr[TK_STREAM_BUF];
  __shared__ int s_nbuf;
  const int r = blockIdx.x, tid = threadIdx.x;
  if (!a.all_rows && !a.ovf[r]) return;
  constexpr int E = Elem<T>::PER16B;
  const int64_t t = a.c0 + r;
  const T *Hr = reinterpret_cast<const T *>(a.H) + t * a.d;
  for (int j = tid; j < a.d; j += 256) hs[j] = Elem<T>::to_f(Hr[j]);
  if (tid == 0) s_nbuf = 0;
  __syncthreads();
  const T *W = reinterpret_cast<const T *>(a.W);
  int nbest = 0;
  uint64_t thr = ~0ull;
  for (int base = 0; base < a.V; base += 256) {
    const int v = base + tid;
    if (v < a.V) {
      const T *w = W + (size_t)v * a.d;
      float acc = 0.f;
      for (int j = 0; j < a.d; j += E) {
        const u32x4 q = *reinterpret_cast<const u32x4 *>(w + j);
        if constexpr (E == 8) {
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            acc = fmaf(hs[j + 2 * p], bf16_lo(q[p]), acc);
            acc = fmaf(hs[j + 2 * p + 1], bf16_hi(q[p]), acc);
          }
        } else {
#pragma unroll
          for (int p = 0; p < 4; ++p) acc = fmaf(hs[j + p], __uint_as_float(q[p]), acc);
        }
      }
      const uint64_t key = make_key(acc, v);
      if (key < thr) arr[nbest + atomicAdd(&s_nbuf, 1)] = key;
    }
    __syncthreads();
    const int nbuf = s_nbuf;
    __syncthreads();
    if (nbest + nbuf + 256 > TK_STREAM_BUF || base + 256 >= a.V) {
      const int n = nbest + nbuf;
      const int P = pow2_at_least(n);
      for (int i = n + tid; i < P; i += 256) arr[i] = ~0ull;
      if (tid == 0) s_nbuf = 0;
      __syncthreads();
      bitonic_sort(arr, P);
      nbest = n < a.K ? n : a.K;
      thr = nbest == a.K ? arr[a.K - 1] : ~0ull;
    }
  }
  write_row(a, t, arr);
}

template <typename K>
hipError_t launch_dyn(K kern, int grid, int threads, int lds_bytes, const TkArgs &a, hipStream_t s) {
  static_assert(sizeof(TkArgs) < 4096, "kernel argument size");
  if (grid <= 0) return hipSuccess;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(threads), lds_bytes, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tk_sample(const TkArgs &a, hipStream_t s) {
  return launch_dyn(k_tk_gemm<SAMPLE>, ((a.C + BM - 1) / BM) * a.ns, w4::NT, w4::Square::LDS, a, s);
}

hipError_t launch_tk_theta(const TkArgs &a, hipStream_t s) {
  if (a.ns < 1 || a.ns > TK_NSAMPLE_MAX) return hipErrorInvalidValue;
  return launch_dyn(k_tk_theta, a.C, 256, a.ns * SEG * (int)sizeof(uint32_t), a, s);
}

hipError_t launch_tk_filter(const TkArgs &a, hipStream_t s) {
  if (a.ns == a.nseg) return hipSuccess;  // every segment was sampled
  return launch_dyn(k_tk_gemm<FILTER>, ((a.C + BM - 1) / BM) * a.nseg, w4::NT, w4::Square::LDS, a, s);
}

hipError_t launch_tk_select(const TkArgs &a, hipStream_t s) {
  return launch_dyn(k_tk_select, a.C, 256, a.cap * (int)sizeof(uint64_t), a, s);
}

hipError_t launch_tk_stream(const TkArgs &a, bool bf16, hipStream_t s) {
  const int lds = a.d * (int)sizeof(float);
  return bf16 ? launch_dyn(k_tk_stream<uint16_t>, a.C, 256, lds, a, s)
              : launch_dyn(k_tk_stream<float>, a.C, 256, lds, a, s);
}

}  // namespace kd
