// Reverse KL and Jensen-Shannon divergence over the teacher's cached top-K
// support, forward and backward.
//
// Both distributions live on the row's K cached ids: the teacher
// q = softmax(topk_logit / tau) and the student restricted to those ids and
// renormalised, p^ = softmax(z[t, idx] / tau), z = H W^T (the asibiont.com
// article, section "A Concrete Implementation Sketch", distils with a
// divergence between softened distributions; whether the top-K cache keeps
// enough signal is the open question of "Hugging Face and Multiverse
// Computing cut KD memory costs", agent-gateway.com, closing paragraph).
//   reverse KL: D_t = sum_k p^_k (log p^_k - log q_k)
//   JSD:        D_t = 1/2 KL(q || m) + 1/2 KL(p^ || m),  m = (p^ + q) / 2
//   loss = tau^2 / N sum_t mask_t D_t
// With a_k = dD/dp^_k (log(p^/q) + 1, or 1/2 log(p^/m)) the logit gradient
// is G_tk = tau/N mask_t p^_k (a_k - sum_j p^_j a_j) at the K ids only, so
// the whole path is O(T K d) gathers, no dense GEMM:
//   k_div_rows   z at the ids (fp32 dots), the divergence, G (one wave per row)
//   k_div_dh     dH[t] = sum_k G_tk W[idx_tk]          (one wave per row)
//   dW[v] = sum over pairs (t, k) with idx_tk = v of G_tk H[t]: the pairs are
//   sorted by id with a stable radix sort (so each id's pairs keep the order
//   t K + k), split into units of at most DIV_UNIT pairs, summed per unit in
//   order and the units of an id added in order: the result does not depend
//   on timing.
#include <limits.h>

#include "kd_device.h"
#include "kd_internal.h"
#include "kd_topk_kl.h"

namespace kd {

namespace {

constexpr int ROWS = 4;           // rows (one wave each) per 256-thread workgroup
constexpr int KMAX_DIV = 1024;
constexpr int RADIX_BITS = 8;
constexpr int RADIX = 1 << RADIX_BITS;

// dot of one 16-byte chunk of two rows (8 bf16 or 4 fp32 values)
template <typename E>
__device__ __forceinline__ float dot16(u32x4 a, u32x4 b, float acc);
template <>
__device__ __forceinline__ float dot16<uint16_t>(u32x4 a, u32x4 b, float acc) {
#pragma unroll
  for (int e = 0; e < 4; ++e)
    acc = fmaf(bf16_hi(a[e]), bf16_hi(b[e]), fmaf(bf16_lo(a[e]), bf16_lo(b[e]), acc));
  return acc;
}
template <>
__device__ __forceinline__ float dot16<float>(u32x4 a, u32x4 b, float acc) {
#pragma unroll
  for (int e = 0; e < 4; ++e) acc = fmaf(__uint_as_float(a[e]), __uint_as_float(b[e]), acc);
  return acc;
}

// acc[0..n) += g * (the 16-byte chunk as floats)
template <typename E>
__device__ __forceinline__ void axpy16(float g, u32x4 w, float (&acc)[8]);
template <>
__device__ __forceinline__ void axpy16<uint16_t>(float g, u32x4 w, float (&acc)[8]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    acc[2 * e] = fmaf(g, bf16_lo(w[e]), acc[2 * e]);
    acc[2 * e + 1] = fmaf(g, bf16_hi(w[e]), acc[2 * e + 1]);
  }
}
template <>
__device__ __forceinline__ void axpy16<float>(float g, u32x4 w, float (&acc)[8]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) acc[e] = fmaf(g, __uint_as_float(w[e]), acc[e]);
}

// Stores the floats of one chunk (8 for bf16 rows, 4 for fp32) at dst,
// adding to what is there when `add`.
template <typename E>
__device__ __forceinline__ void store_chunk(float *dst, const float (&acc)[8], bool add) {
  constexpr int N = Elem<E>::PER16B;
#pragma unroll
  for (int h = 0; h < N / 4; ++h) {
    f32x4 v{acc[4 * h], acc[4 * h + 1], acc[4 * h + 2], acc[4 * h + 3]};
    f32x4 *p = reinterpret_cast<f32x4 *>(dst) + h;
    if (add) v += *p;
    *p = v;
  }
}

// One wave per token row: teacher log q, student logits at the ids (8 lanes
// per dot), the divergence and the logit gradient at the ids.
template <typename E>
__global__ __launch_bounds__(256) void k_div_rows(DivArgs a) {
  __shared__ float s_u[ROWS][KMAX_DIV];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * ROWS + wave;
  const bool active = t < a.T;
  const int K = a.K;
  const int dq = a.d / Elem<E>::PER16B;  // 16-byte chunks per row
  if (active) {
    const u32x4 *h16 = reinterpret_cast<const u32x4 *>(reinterpret_cast<const E *>(a.H) + t * a.d);
    const int g = lane >> 3, l = lane & 7;
    for (int k0 = 0; k0 < K; k0 += 8) {
      const int k = k0 + g;
      const int id = k < K ? a.topk_idx[t * K + k] : -1;
      const bool ok = id >= 0 && id < a.V;
      float acc = 0.f;
      if (ok) {
        const u32x4 *w16 = reinterpret_cast<const u32x4 *>(reinterpret_cast<const E *>(a.W) +
                                                           (int64_t)id * a.d);
        for (int c = l; c < dq; c += 8) acc = dot16<E>(h16[c], w16[c], acc);
      }
      acc += __shfl_xor(acc, 1, 64);
      acc += __shfl_xor(acc, 2, 64);
      acc += __shfl_xor(acc, 4, 64);
      if (l == 0 && k < K) s_u[wave][k] = ok ? acc * a.inv_tau : -INFINITY;
    }
  }
  __syncthreads();
  if (!active) return;
  const float *lg = a.topk_logit + t * K;
  // teacher: log q with one rounding of logit/tau - max
  float mq = -INFINITY, mu = -INFINITY;
  for (int k = lane; k < K; k += 64) {
    mq = fmaxf(mq, lg[k] * a.inv_tau);
    mu = fmaxf(mu, s_u[wave][k]);
  }
  mq = wave_max(mq);
  mu = wave_max(mu);
  float sq = 0.f, su = 0.f;
  for (int k = lane; k < K; k += 64) {
    sq += expf(fmaf(lg[k], a.inv_tau, -mq));
    su += expf(s_u[wave][k] - mu);
  }
  const float lsq = logf(wave_sum(sq)), lsu = logf(wave_sum(su));
  // per slot: log p^, log q, p^, the divergence term and a = dD/dp^
  constexpr int PER = KMAX_DIV / 64;
  float pp[PER], av[PER];
  float dsum = 0.f, abar = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int k = lane + 64 * i;
    pp[i] = av[i] = 0.f;
    if (k < K) {
      const float lq = fmaf(lg[k], a.inv_tau, -mq) - lsq;
      const float l_p = (s_u[wave][k] - mu) - lsu;
      const float p = expf(l_p);
      float term, ak;
      if (a.kind == KD_DIV_REVERSE_KL) {
        term = p > 0.f ? p * (l_p - lq) : 0.f;
        ak = l_p - lq + 1.f;
      } else {
        const float q = expf(lq);
        // log m = log((p + q) / 2) from the larger log and log1p of the ratio
        const float hi = fmaxf(l_p, lq), lo = fminf(l_p, lq);
        const float lm = hi + log1pf(expf(lo - hi)) - LN2;
        term = 0.5f * (q * (lq - lm) + (p > 0.f ? p * (l_p - lm) : 0.f));
        ak = 0.5f * (l_p - lm);
      }
      pp[i] = p;
      av[i] = ak;
      dsum += term;
      abar += p > 0.f ? p * ak : 0.f;
    }
  }
  dsum = wave_sum(dsum);
  abar = wave_sum(abar);
  const bool valid = a.mask ? (a.mask[t] != 0) : true;
  const float gs = valid ? a.scal->grad_scale : 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int k = lane + 64 * i;
    if (k < K) a.Gk[t * K + k] = (gs != 0.f && pp[i] > 0.f) ? gs * pp[i] * (av[i] - abar) : 0.f;
  }
  if (lane == 0) a.row_loss[t] = valid ? dsum : 0.f;
}

// dH[t] = sum_k G_tk W[idx_tk]: one wave per row, lanes own 16-byte chunks of
// the hidden dimension (each W row read once, coalesced).
template <typename E>
__global__ __launch_bounds__(256) void k_div_dh(DivArgs a) {
  __shared__ float s_g[ROWS][KMAX_DIV];
  __shared__ int32_t s_id[ROWS][KMAX_DIV];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * ROWS + wave;
  const int K = a.K;
  if (t < a.T) {
    for (int k = lane; k < K; k += 64) {
      const int id = a.topk_idx[t * K + k];
      const bool ok = id >= 0 && id < a.V;
      s_g[wave][k] = ok ? a.Gk[t * K + k] : 0.f;
      s_id[wave][k] = ok ? id : 0;
    }
  }
  __syncthreads();
  if (t >= a.T) return;
  constexpr int N = Elem<E>::PER16B;
  const int dq = a.d / N;
  float *out = a.dH + t * a.d;
  for (int c = lane; c < dq; c += 64) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < K; ++k) {
      const float g = s_g[wave][k];
      if (g == 0.f) continue;
      const u32x4 w = reinterpret_cast<const u32x4 *>(reinterpret_cast<const E *>(a.W) +
                                                      (int64_t)s_id[wave][k] * a.d)[c];
      axpy16<E>(g, w, acc);
    }
    store_chunk<E>(out + c * N, acc, false);
  }
}

// ------------------------------------------------------------ radix sort
// Keys (id, or V for an id outside [0, V)) and values (pair index t K + k).
__global__ __launch_bounds__(256) void k_div_keys(DivArgs a) {
  const int64_t n = a.T * a.K;
  for (int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x; p < n; p += (int64_t)gridDim.x * 256) {
    const int id = a.topk_idx[p];
    a.keys[0][p] = (id >= 0 && id < a.V) ? id : a.V;
    a.vals[0][p] = (int32_t)p;
  }
}

// Per block of RADIX_BLOCK keys: the count of each digit, stored digit-major
// (hist[digit * nblk + block]) for the scan.
__global__ __launch_bounds__(256) void k_radix_hist(const int32_t *keys, int64_t n, int shift,
                                                     int32_t *hist, int nblk) {
  __shared__ int32_t h[RADIX];
  h[threadIdx.x] = 0;
  __syncthreads();
  const int64_t b0 = (int64_t)blockIdx.x * RADIX_BLOCK;
  for (int i = threadIdx.x; i < RADIX_BLOCK && b0 + i < n; i += 256)
    atomicAdd(&h[(keys[b0 + i] >> shift) & (RADIX - 1)], 1);
  __syncthreads();
  hist[(int64_t)threadIdx.x * nblk + blockIdx.x] = h[threadIdx.x];
}

// Exclusive scan of n int32 in place by one workgroup of 1024 threads, each
// a contiguous run, total written to *total when not null: for the short
// list of tile sums of scan_excl below.
__global__ __launch_bounds__(1024) void k_scan_excl(int32_t *x, int64_t n, int32_t *total) {
  __shared__ int32_t part[1024];
  const int tid = threadIdx.x;
  const int64_t per = (n + 1023) / 1024;
  const int64_t lo = tid * per, hi = lo + per < n ? lo + per : n;
  int32_t s = 0;
  for (int64_t i = lo; i < hi; ++i) s += x[i];
  part[tid] = s;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int32_t v = tid >= o ? part[tid - o] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int32_t run = part[tid] - s;  // exclusive prefix of this run
  for (int64_t i = lo; i < hi; ++i) {
    const int32_t v = x[i];
    x[i] = run;
    run += v;
  }
  if (total && tid == 1023) *total = part[1023];
}

// Exclusive scan of n int32 in place over tiles of SCAN_TILE: the tiles'
// sums (coalesced loads, one tile per workgroup), an exclusive scan of the
// sums, then each tile scanned with its offset (integer: the result is the
// plain prefix sum).
__global__ __launch_bounds__(256) void k_scan_sums(const int32_t *x, int64_t n, int32_t *bsum) {
  __shared__ int32_t ws[4];
  const int tid = threadIdx.x;
  const int64_t b0 = (int64_t)blockIdx.x * SCAN_TILE;
  int32_t s = 0;
#pragma unroll
  for (int i = 0; i < SCAN_TILE / 256; ++i) {
    const int64_t j = b0 + i * 256 + tid;
    if (j < n) s += x[j];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  if ((tid & 63) == 0) ws[tid >> 6] = s;
  __syncthreads();
  if (tid == 0) bsum[blockIdx.x] = (ws[0] + ws[1]) + (ws[2] + ws[3]);
}

__global__ __launch_bounds__(256) void k_scan_apply(int32_t *x, int64_t n, const int32_t *bsum) {
  constexpr int PER = SCAN_TILE / 256;  // contiguous values per thread
  __shared__ int32_t ws[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t j0 = (int64_t)blockIdx.x * SCAN_TILE + (int64_t)tid * PER;
  int32_t v[PER];
  int32_t s = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    v[i] = j0 + i < n ? x[j0 + i] : 0;
    s += v[i];
  }
  // exclusive prefix of this thread's run within the tile
  int32_t inc = s;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t u = __shfl_up(inc, o, 64);
    if (lane >= o) inc += u;
  }
  if (lane == 63) ws[wave] = inc;
  __syncthreads();
  int32_t run = bsum[blockIdx.x] + inc - s;
  for (int w = 0; w < wave; ++w) run += ws[w];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (j0 + i < n) x[j0 + i] = run;
    run += v[i];
  }
}

hipError_t scan_excl(int32_t *x, int64_t n, int32_t *bsum, hipStream_t s) {
  const int64_t nb = div_scan_blocks(n);
  hipLaunchKernelGGL(k_scan_sums, dim3((unsigned)nb), dim3(256), 0, s, x, n, bsum);
  hipLaunchKernelGGL(k_scan_excl, dim3(1), dim3(1024), 0, s, bsum, nb, (int32_t *)nullptr);
  hipLaunchKernelGGL(k_scan_apply, dim3((unsigned)nb), dim3(256), 0, s, x, n,
                     (const int32_t *)bsum);
  return hipGetLastError();
}

// Stable scatter of one radix pass: each block walks its keys in order, 256
// at a time; a key's position is its digit's offset for the block, plus the
// keys of that digit earlier in the block (earlier rounds, earlier waves,
// lower lanes of its own wave).
__global__ __launch_bounds__(256) void k_radix_scatter(const int32_t *kin, const int32_t *vin,
                                                        int32_t *kout, int32_t *vout, int64_t n,
                                                        int shift, const int32_t *hist, int nblk) {
  __shared__ int32_t base[RADIX];
  __shared__ int32_t wcnt[4][RADIX];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  base[tid] = hist[(int64_t)tid * nblk + blockIdx.x];
  const int64_t b0 = (int64_t)blockIdx.x * RADIX_BLOCK;
  const uint64_t lt = lane ? (~0ull >> (64 - lane)) : 0ull;
  for (int r0 = 0; r0 < RADIX_BLOCK; r0 += 256) {
    const int64_t i = b0 + r0 + tid;
    const bool in = i < n;
    const int32_t key = in ? kin[i] : 0;
    const int dig = (key >> shift) & (RADIX - 1);
#pragma unroll
    for (int w = 0; w < 4; ++w) wcnt[w][tid] = 0;
    __syncthreads();
    // lanes of this wave holding the same digit
    uint64_t same = __ballot(in);
#pragma unroll
    for (int bit = 0; bit < RADIX_BITS; ++bit) {
      const uint64_t b = __ballot((dig >> bit) & 1);
      same &= ((dig >> bit) & 1) ? b : ~b;
    }
    const int rank = __popcll(same & lt);
    if (in && rank == 0) wcnt[wave][dig] = __popcll(same);
    __syncthreads();
    if (in) {
      int off = base[dig] + rank;
      for (int w = 0; w < wave; ++w) off += wcnt[w][dig];
      kout[off] = key;
      vout[off] = vin[i];
    }
    __syncthreads();
    base[tid] += wcnt[0][tid] + wcnt[1][tid] + wcnt[2][tid] + wcnt[3][tid];
    __syncthreads();
  }
}

// seg[v] = first sorted position with key >= v, for v = 0 .. V (seg[V] =
// number of pairs with a valid id); per id the unit count u_v (>= 1) and,
// for ids of more than one unit, the count of partial rows.
__global__ __launch_bounds__(256) void k_div_segments(DivArgs a, const int32_t *keys) {
  const int64_t n = a.T * a.K;
  const int v = blockIdx.x * 256 + threadIdx.x;
  if (v > a.V) return;
  int64_t lo = 0, hi = n;
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if (keys[mid] < v) lo = mid + 1; else hi = mid;
  }
  a.seg[v] = (int32_t)lo;
}

__global__ __launch_bounds__(256) void k_div_units(DivArgs a) {
  const int v = blockIdx.x * 256 + threadIdx.x;
  if (v > a.V) return;
  if (v == a.V) {  // totals land here after the exclusive scans
    a.unit_start[v] = 0;
    a.part_start[v] = 0;
    return;
  }
  const int64_t len = (int64_t)a.seg[v + 1] - a.seg[v];
  const int32_t u = len > DIV_UNIT ? (int32_t)((len + DIV_UNIT - 1) / DIV_UNIT) : 1;
  a.unit_start[v] = u;
  a.part_start[v] = u > 1 ? u : 0;
}

// One wave per unit (a run of at most DIV_UNIT pairs of one id, in sorted
// order): the sum of G H[t] over the run, written to dW[v] when the id has
// one unit (overwritten, or added with accumulate) and to its partial row
// otherwise.  Waves past the last unit exit.
template <typename E>
__global__ __launch_bounds__(256) void k_div_dw(DivArgs a, const int32_t *vals) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * ROWS + wave;
  if (w >= a.unit_start[a.V]) return;
  // the id whose units contain w: last v with unit_start[v] <= w
  int lo = 0, hi = a.V;  // answer in [lo, hi)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.unit_start[mid] <= w) lo = mid; else hi = mid;
  }
  const int v = lo;
  const int j = (int)(w - a.unit_start[v]);
  const int units = a.unit_start[v + 1] - a.unit_start[v];
  const int64_t p0 = (int64_t)a.seg[v] + (int64_t)j * DIV_UNIT;
  const int64_t p1 = p0 + DIV_UNIT < a.seg[v + 1] ? p0 + DIV_UNIT : a.seg[v + 1];
  constexpr int N = Elem<E>::PER16B;
  const int dq = a.d / N;
  float *dst = units == 1 ? a.dW + (int64_t)v * a.d
                          : a.partial + ((int64_t)a.part_start[v] + j) * a.d;
  const bool add = units == 1 && a.accumulate;
  for (int c = lane; c < dq; c += 64) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int64_t p = p0; p < p1; ++p) {
      const int32_t pair = vals[p];
      const float g = a.Gk[pair];
      if (g == 0.f) continue;
      const int64_t t = pair / a.K;
      const u32x4 h = reinterpret_cast<const u32x4 *>(reinterpret_cast<const E *>(a.H) +
                                                      t * a.d)[c];
      axpy16<E>(g, h, acc);
    }
    store_chunk<E>(dst + c * N, acc, add);
  }
}

// Ids of more than one unit: dW[v] (+)= the ordered sum of their partials.
__global__ __launch_bounds__(256) void k_div_dw_reduce(DivArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int v = blockIdx.x * ROWS + wave;
  if (v >= a.V) return;
  const int units = a.unit_start[v + 1] - a.unit_start[v];
  if (units < 2) return;
  const float *src = a.partial + (int64_t)a.part_start[v] * a.d;
  float *dst = a.dW + (int64_t)v * a.d;
  for (int c = lane; c < a.d / 4; c += 64) {
    f32x4 s = reinterpret_cast<const f32x4 *>(src)[c];
    for (int u = 1; u < units; ++u) s += reinterpret_cast<const f32x4 *>(src + (int64_t)u * a.d)[c];
    if (a.accumulate) s += reinterpret_cast<const f32x4 *>(dst)[c];
    reinterpret_cast<f32x4 *>(dst)[c] = s;
  }
}

}  // namespace

int radix_passes(int64_t V) {
  int bits = 0;
  while ((int64_t(1) << bits) <= V) ++bits;  // keys take values 0 .. V
  return (bits + RADIX_BITS - 1) / RADIX_BITS;
}

hipError_t launch_div(const DivArgs &a, hipStream_t s) {
  const int g_rows = (int)((a.T + ROWS - 1) / ROWS);
  const int64_t n = a.T * a.K;
  const bool bf16 = a.bf16;
  if (bf16)
    hipLaunchKernelGGL(k_div_rows<uint16_t>, dim3(g_rows), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_div_rows<float>, dim3(g_rows), dim3(256), 0, s, a);
  if (bf16)
    hipLaunchKernelGGL(k_div_dh<uint16_t>, dim3(g_rows), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_div_dh<float>, dim3(g_rows), dim3(256), 0, s, a);
  // pairs sorted by id (stable), then per-id units
  const int gk = (int)((n + 255) / 256 < 16384 ? (n + 255) / 256 : 16384);
  hipLaunchKernelGGL(k_div_keys, dim3(gk), dim3(256), 0, s, a);
  const int nblk = (int)((n + RADIX_BLOCK - 1) / RADIX_BLOCK);
  const int passes = radix_passes(a.V);
  int cur = 0;
  for (int ps = 0; ps < passes; ++ps) {
    const int shift = ps * RADIX_BITS;
    hipLaunchKernelGGL(k_radix_hist, dim3(nblk), dim3(256), 0, s, a.keys[cur], n, shift, a.hist,
                       nblk);
    if (hipError_t e = scan_excl(a.hist, (int64_t)RADIX * nblk, a.bsum, s)) return e;
    hipLaunchKernelGGL(k_radix_scatter, dim3(nblk), dim3(256), 0, s, a.keys[cur], a.vals[cur],
                       a.keys[cur ^ 1], a.vals[cur ^ 1], n, shift, a.hist, nblk);
    cur ^= 1;
  }
  const int gv = (a.V + 1 + 255) / 256;
  hipLaunchKernelGGL(k_div_segments, dim3(gv), dim3(256), 0, s, a, a.keys[cur]);
  hipLaunchKernelGGL(k_div_units, dim3(gv), dim3(256), 0, s, a);
  if (hipError_t e = scan_excl(a.unit_start, (int64_t)a.V + 1, a.bsum, s)) return e;
  if (hipError_t e = scan_excl(a.part_start, (int64_t)a.V + 1, a.bsum, s)) return e;
  const int64_t max_units = n / DIV_UNIT + a.V;
  const int gw = (int)((max_units + ROWS - 1) / ROWS);
  if (bf16)
    hipLaunchKernelGGL(k_div_dw<uint16_t>, dim3(gw), dim3(256), 0, s, a, a.vals[cur]);
  else
    hipLaunchKernelGGL(k_div_dw<float>, dim3(gw), dim3(256), 0, s, a, a.vals[cur]);
  hipLaunchKernelGGL(k_div_dw_reduce, dim3((a.V + ROWS - 1) / ROWS), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace kd
