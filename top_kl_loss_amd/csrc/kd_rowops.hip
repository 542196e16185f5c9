// Row-wise kernels of the fused, chunked top-K KL loss: valid-token count,
// teacher softmax over the cached top-K, per-row id sort and segment table,
// row logsumexp + per-row KL + teacher correction, split-K reduction of dH
// and the final ordered loss sum.
//
// The method ("Making Knowledge Distillation Cheap Enough to Run at Scale",
// aipuls.nl, section "Summary"; "Hugging Face and Multiverse Computing cut
// KD memory costs", agent-gateway.com) caches the teacher's top-K logits and
// evaluates the KL loss slice by slice.  These kernels are O(T*K + T*V/SEG)
// and run one 64-lane wave per token row.
#include <limits.h>

#include "kd_device.h"
#include "kd_internal.h"

namespace kd {

namespace {

constexpr int KMAX = 1024;
constexpr int ROWS_PER_WG = 4;  // one wave per row

// N = sum(mask), grad scale tau/N and loss scale tau^2/N (zero for N = 0).
// Reading of the reduction: mean over valid tokens, as in the asibiont.com
// article's implementation sketch, with tau^2 scaling of the soft loss.
// grad_loss (device scalar, or null for 1) multiplies the grad scale: the
// upstream gradient of the loss in a backward pass.
__global__ __launch_bounds__(256) void k_valid_count(const uint8_t *mask, int T,
                                                     float tau, const float *grad_loss,
                                                     Scalars *scal) {
  __shared__ int part[4];
  int cnt = 0;
  if (mask) {
    for (int i = threadIdx.x; i < T; i += 256) cnt += mask[i] != 0;
  } else if (threadIdx.x == 0) {
    cnt = T;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = cnt;
  __syncthreads();
  if (threadIdx.x == 0) {
    const int n = part[0] + part[1] + part[2] + part[3];
    scal->n_valid = n;
    const double g = grad_loss ? double(*grad_loss) : 1.0;
    scal->grad_scale = n > 0 ? float(double(tau) / double(n) * g) : 0.f;
    scal->loss_scale = n > 0 ? float(double(tau) * tau / double(n)) : 0.f;
  }
}

// Per slice row: teacher distribution q = softmax(topk_logit / tau) over the
// K cached slots and log q, each from the logits shifted by their maximum
// (one rounding of logit/tau - max, so log q is accurate to its own size);
// the row's ids sorted ascending (with their slots) and, for every
// vocabulary segment, the first sorted position whose id falls in it (-1 if
// none).  Also clears the gathered-logit row.  Ids outside [0, V) are
// replaced by INT_MAX so that no later kernel dereferences them.
__global__ __launch_bounds__(256) void k_prep_rows(SliceArgs a) {
  __shared__ int32_t s_ids[ROWS_PER_WG][KMAX];
  __shared__ int32_t s_sorted[ROWS_PER_WG][KMAX];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = blockIdx.x * ROWS_PER_WG + wave;
  const bool active = r < a.C;
  const int K = a.K;
  const int64_t t = a.c0 + r;
  if (active) {
    const float *lg = a.topk_logit + t * K;
    float mx = -INFINITY;
    for (int k = lane; k < K; k += 64) mx = fmaxf(mx, lg[k] * a.inv_tau);
    mx = wave_max(mx);
    float sum = 0.f;
    for (int k = lane; k < K; k += 64) sum += expf(fmaf(lg[k], a.inv_tau, -mx));
    sum = wave_sum(sum);
    const float lsum = logf(sum);
    for (int k = lane; k < K; k += 64) {
      const float lq = fmaf(lg[k], a.inv_tau, -mx) - lsum;
      a.q[(size_t)r * K + k] = expf(lq);
      a.lq[(size_t)r * K + k] = lq;
      a.zg[(size_t)r * K + k] = 0.f;
      const int id = a.topk_idx[t * K + k];
      s_ids[wave][k] = (id >= 0 && id < a.V) ? id : INT_MAX;
    }
  }
  // Tuned path with gradients: the row's a-priori shift, the largest z s2
  // over its SHIFT_SLOTS best teacher slots (teacher logit descending, equal
  // logits by slot), from fp32 dot products of the bf16 rows of H and W.
  // Each is an actual logit of the row up to rounding, so the shift lies at
  // or below the row maximum; -inf when no slot holds a valid id.  The slots
  // are chosen first (their ids read back from LDS); the dot products then
  // run together, one pass over the hidden dimension whose W loads carry no
  // branch (a slot without a valid id reads row 0 and is ignored), so the
  // scattered rows' round trips to memory overlap instead of following one
  // another.
  if (active && a.fast && a.need_grad) {
    const float *lg = a.topk_logit + t * K;
    const int R = K < SHIFT_SLOTS ? K : SHIFT_SLOTS;
    uint32_t taken = 0;  // bit i: slot lane + 64 i already chosen
    int ids[SHIFT_SLOTS];
#pragma unroll
    for (int rr = 0; rr < SHIFT_SLOTS; ++rr) ids[rr] = -1;
    for (int rr = 0; rr < R; ++rr) {
      float bv = -INFINITY;
      int bk = INT_MAX;
      for (int i = 0, k = lane; k < K; ++i, k += 64)
        if (!((taken >> i) & 1u) && (lg[k] > bv || (lg[k] == bv && k < bk))) {
          bv = lg[k];
          bk = k;
        }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int ok = __shfl_xor(bk, o, 64);
        if (ov > bv || (ov == bv && ok < bk)) {
          bv = ov;
          bk = ok;
        }
      }
      if (bk == INT_MAX) break;
      if ((bk & 63) == lane) taken |= 1u << (bk >> 6);
      const int id = s_ids[wave][bk];  // INT_MAX: not a valid id
#pragma unroll
      for (int s = 0; s < SHIFT_SLOTS; ++s)
        if (s == rr) ids[s] = id == INT_MAX ? -1 : id;
    }
    const int dq = a.d / 8;
    const u32x4 *h16 = reinterpret_cast<const u32x4 *>(
        reinterpret_cast<const uint16_t *>(a.H) + t * a.d);
    const u32x4 *w16[SHIFT_SLOTS];
#pragma unroll
    for (int s = 0; s < SHIFT_SLOTS; ++s)
      w16[s] = reinterpret_cast<const u32x4 *>(reinterpret_cast<const uint16_t *>(a.W) +
                                               (int64_t)(ids[s] < 0 ? 0 : ids[s]) * a.d);
    float acc[SHIFT_SLOTS];
#pragma unroll
    for (int s = 0; s < SHIFT_SLOTS; ++s) acc[s] = 0.f;
#pragma unroll 2
    for (int c = lane; c < dq; c += 64) {
      const u32x4 hv = h16[c];
      u32x4 wv[SHIFT_SLOTS];
#pragma unroll
      for (int s = 0; s < SHIFT_SLOTS; ++s) wv[s] = w16[s][c];
#pragma unroll
      for (int s = 0; s < SHIFT_SLOTS; ++s)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[s] = fmaf(bf16_hi(hv[e]), bf16_hi(wv[s][e]),
                        fmaf(bf16_lo(hv[e]), bf16_lo(wv[s][e]), acc[s]));
    }
    float best = -INFINITY;
#pragma unroll
    for (int s = 0; s < SHIFT_SLOTS; ++s) {
      const float z = wave_sum(acc[s]);
      if (ids[s] >= 0) best = fmaxf(best, z);
    }
    if (lane == 0) {
      a.shift[r] = best * a.s2;
      a.flag[r] = 0;
      if (r % ROW_TILE == 0) a.tile_flags[r / ROW_TILE] = 0;
    }
  }
  __syncthreads();
  if (active) {
    for (int k = lane; k < K; k += 64) {
      const int idk = s_ids[wave][k];
      int rank = 0;
#pragma unroll 8
      for (int j = 0; j < K; ++j) {
        const int idj = s_ids[wave][j];
        rank += (idj < idk) || (idj == idk && j < k);
      }
      s_sorted[wave][rank] = idk;
      a.sid[(size_t)r * K + rank] = idk;
      a.sslot[(size_t)r * K + rank] = k;
    }
  }
  __syncthreads();
  if (active) {
    // first sorted position per segment: -1 everywhere, then, in sorted
    // order, the position where the ids enter a new segment (invalid ids,
    // INT_MAX, sort last and are skipped).  The wait orders this wave's
    // -1 stores before its position stores to the same entries.
    int16_t *fr = a.first + (size_t)r * a.nseg;
    for (int j = lane; j < a.nseg; j += 64) fr[j] = int16_t(-1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    for (int k = lane; k < K; k += 64) {
      const int id = s_sorted[wave][k];
      if (id == INT_MAX) continue;
      const int seg = id / SEG;
      if (k == 0 || s_sorted[wave][k - 1] / SEG != seg) fr[seg] = int16_t(k);
    }
  }
}

// Row statistics from the logits GEMM's per-segment shifts and sums (base-2
// units): M = max_j shift_j and s = sum_j sum_j 2^(shift_j - M), so that
// log2-sum-exp2 of the row is M + log2 s.  Wave-uniform results.
__device__ __forceinline__ void row_stats(const SliceArgs &a, int r, int lane, float &mx,
                                          float &log2s) {
  const float *mrow = a.mseg + (size_t)r * a.nseg;
  const float *srow = a.sseg + (size_t)r * a.nseg;
  // (unrolled so that several iterations' loads are in flight; the sums
  // keep their order)
  mx = -INFINITY;
#pragma unroll 4
  for (int j = lane; j < a.nseg; j += 64) mx = fmaxf(mx, mrow[j]);
  mx = wave_max(mx);
  float s = 0.f;
#pragma unroll 4
  for (int j = lane; j < a.nseg; j += 64) s += srow[j] * exp2f(mrow[j] - mx);
  log2s = log2f(wave_sum(s));
}

// Tuned path: the teacher correction of row r with the row's shift sh: at
// every valid teacher id,
//   P~[r, id] = 2^(z_k s2 - sh) - q_k 2^(M + log2 s - sh),
// from the fp32 logit z_k, rounded once to bf16.
__device__ __forceinline__ void correct_rows_tuned(const SliceArgs &a, int r, int lane, float sh,
                                                   float mx, float log2s) {
  const int K = a.K;
  const int64_t t = a.c0 + r;
  const float *q = a.q + (size_t)r * K;
  const float *zg = a.zg + (size_t)r * K;
  uint16_t *P = reinterpret_cast<uint16_t *>(a.P) + (size_t)r * a.ldp;
  const float corr = exp2f((mx - sh) + log2s);
  for (int k = lane; k < K; k += 64) {
    const int id = a.topk_idx[t * K + k];
    if (id < 0 || id >= a.V) continue;
    const float val = exp2f(fmaf(zg[k], a.s2, -sh)) - q[k] * corr;
    P[id] = uint16_t(f32_to_bf16_rne(val));
  }
}

// Per slice row, after the logits GEMM.  Logits are in base-2 units
// (s2 = log2(e) / tau): shift_j = max over segment j of z s2, sum_j = sum
// over the segment of 2^(z s2 - shift_j).  With M = max_j shift_j and
// s = sum_j sum_j 2^(shift_j - M), log2-sum-exp2 of the row is M + log2 s, so
//  lse   = (M + log2 s) ln 2                      (natural units, z / tau);
//  KL_t  = sum_k q_k (log q_k - (z_k s2 - M) ln 2) + log s  (z_k gathered by
//          the GEMM); every bracket is a difference of nearby values taken
//          with one rounding, so KL_t keeps its accuracy as it tends to 0;
//  P[t, id_k] = 2^(z_k s2 - shift_j) - q_k 2^(M - shift_j + log2 s), from
//          the fp32 logit z_k and rounded once (the teacher correction, so
//          that f_j * P is tau/N (p - q_scat) on segment j);
//  f_j   = tau/N * mask_t * 2^(shift_j - M - log2 s);
//  G[t, v] = f_seg(v) * P[t, v]  written over P (= tau/N mask (p - q_scat)).
// A segment holding teacher ids whose shift lies more than RESHIFT_NATS
// below the row's logsumexp is first re-shifted to RESHIFT_NATS below it.
template <typename T>
__global__ __launch_bounds__(256) void k_lse_fix(SliceArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = blockIdx.x * ROWS_PER_WG + wave;
  if (r >= a.C) return;
  const int nseg = a.nseg, K = a.K;
  const int64_t t = a.c0 + r;
  float *mrow = a.mseg + (size_t)r * nseg;

  float mx, log2s;
  row_stats(a, r, lane, mx, log2s);
  const float lse2 = mx + log2s;  // base 2
  const float lse = lse2 * LN2;

  const float *q = a.q + (size_t)r * K;
  const float *lq = a.lq + (size_t)r * K;
  const float *zg = a.zg + (size_t)r * K;
  float dot = 0.f;
  for (int k = lane; k < K; k += 64) dot += q[k] * (lq[k] - fmaf(zg[k], a.s2, -mx) * LN2);
  dot = wave_sum(dot);
  const bool valid = a.mask ? (a.mask[t] != 0) : true;
  if (lane == 0) {
    a.lse[r] = lse;
    if (a.lse_out) a.lse_out[t] = lse;
    a.row_loss[t] = valid ? (dot + log2s * LN2) : 0.f;
  }
  if (!a.need_grad) return;

  const float gscale = valid ? a.scal->grad_scale : 0.f;
  if (a.fast) {
    // Tuned path: the GEMM stored P~ = 2^(z s2 - sh) with the row's
    // a-priori shift sh, so G = f_t P~ (after the teacher correction) with
    // one factor per row, f_t = tau/N mask 2^(sh - M - log2 s).  A shift
    // more than SHIFT_LIMIT2 below the row maximum (P~ may have overflowed)
    // flags the row: its shift becomes the maximum, and k_fast_logits_redo
    // and k_fix_flagged store it again.
    float sh = a.shift[r];
    const bool flagged = !(mx - sh <= SHIFT_LIMIT2);
    if (flagged) sh = mx;
    if (lane == 0) {
      a.frow[r] = gscale != 0.f ? gscale * exp2f((sh - mx) - log2s) : 0.f;
      if (flagged) {
        a.shift[r] = sh;
        a.flag[r] = 1;
        atomicAdd(&a.tile_flags[r / ROW_TILE], 1);
      }
    }
    if (!flagged && gscale != 0.f) correct_rows_tuned(a, r, lane, sh, mx, log2s);
    return;
  }
  T *P = reinterpret_cast<T *>(a.P) + (size_t)r * a.ldp;
  const int32_t *sid = a.sid + (size_t)r * K;
  constexpr float RESHIFT2 = RESHIFT_NATS * LOG2E;
  if (gscale != 0.f) {
    for (int base = 0; base < K; base += 64) {
      const int pos = base + lane;
      bool need = false;
      int j = 0;
      if (pos < K) {
        const int id = sid[pos];
        if (id < a.V) {
          j = id / SEG;
          const bool first_in_seg = pos == 0 || (sid[pos - 1] / SEG) != j;
          need = first_in_seg && (lse2 - mrow[j] > RESHIFT2);
        }
      }
      uint64_t bal = __ballot(need);
      while (bal) {
        const int src = __ffsll((unsigned long long)bal) - 1;
        bal &= bal - 1;
        const int js = __shfl(j, src, 64);
        const float newm = lse2 - RESHIFT2;
        const float fac = exp2f(mrow[js] - newm);
        for (int c = lane; c < SEG; c += 64) {
          T &e = P[(size_t)js * SEG + c];
          e = Elem<T>::from_f(Elem<T>::to_f(e) * fac);
        }
        __threadfence_block();
        if (lane == 0) mrow[js] = newm;
        __threadfence_block();
      }
    }
    __threadfence_block();
    for (int pos = lane; pos < K; pos += 64) {
      const int id = sid[pos];
      if (id < a.V) {
        const int j = id / SEG;
        const int slot = a.sslot[(size_t)r * K + pos];
        const float mj = mrow[j];
        const float pz = exp2f(fmaf(zg[slot], a.s2, -mj));
        const float corr = q[slot] * exp2f((mx - mj) + log2s);
        P[id] = Elem<T>::from_f(pz - corr);
      }
    }
  }
  float *frow = a.fseg + (size_t)r * nseg;
  for (int j = lane; j < nseg; j += 64)
    frow[j] = gscale != 0.f ? gscale * exp2f((mrow[j] - mx) - log2s) : 0.f;
  __threadfence_block();
  // G row = f_seg * P row, in place: the logit gradient the dH and dW GEMMs
  // consume (all zero for a padding row).
  constexpr int E = Elem<T>::PER16B;
  u32x4 *P16 = reinterpret_cast<u32x4 *>(P);
  const int nchunk = a.ldp / E;
  for (int c = lane; c < nchunk; c += 64) {
    const float f = frow[(c * E) / SEG];
    P16[c] = Elem<T>::scale(P16[c], f);
  }
}

// Tuned path, after k_fast_logits_redo: the teacher correction of the
// flagged rows (shift = row maximum).
__global__ __launch_bounds__(256) void k_fix_flagged(SliceArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = blockIdx.x * ROWS_PER_WG + wave;
  if (r >= a.C || !a.flag[r]) return;
  const bool valid = a.mask ? (a.mask[a.c0 + r] != 0) : true;
  if (!valid || a.scal->grad_scale == 0.f) return;
  float mx, log2s;
  row_stats(a, r, lane, mx, log2s);
  correct_rows_tuned(a, r, lane, a.shift[r], mx, log2s);
}

// dst[i] = src[i] * (*scale) (scale null: 1) in the destination type (bf16
// rounded to nearest even): the gradient handed back to a bf16 or fp32
// parameter.
template <typename T>
__global__ __launch_bounds__(256) void k_grad_cast(const float *src, T *dst, int64_t n,
                                                   const float *scale) {
  const float s = scale ? *scale : 1.f;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * 256)
    dst[i] = Elem<T>::from_f(src[i] * s);
}

// dH rows of the slice = ordered sum of the split-K partials, times the
// row's gradient factor on the tuned path (frow; null on the generic path,
// whose G carries its factors already).
__global__ __launch_bounds__(256) void k_reduce_dh(const float *part, int splits,
                                                   size_t stride, size_t n4, int d4,
                                                   const float *frow, float *out) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  f32x4 acc = reinterpret_cast<const f32x4 *>(part)[i];
  for (int s = 1; s < splits; ++s)
    acc += reinterpret_cast<const f32x4 *>(part + s * stride)[i];
  if (frow) acc *= frow[i / d4];
  reinterpret_cast<f32x4 *>(out)[i] = acc;
}

// loss = tau^2 / N * sum_t row_loss[t], summed in fp64 in a fixed order.
__global__ __launch_bounds__(256) void k_final_loss(const float *row_loss, int T,
                                                    const Scalars *scal,
                                                    float *loss) {
  __shared__ double part[256];
  double s = 0.0;
  for (int i = threadIdx.x; i < T; i += 256) s += row_loss[i];
  part[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const int n = scal->n_valid;
    *loss = n > 0 ? float(double(scal->loss_scale) * part[0]) : 0.f;
  }
}

}  // namespace

hipError_t launch_valid_count(const uint8_t *mask, int T, float tau,
                              const float *grad_loss, Scalars *scal, hipStream_t s) {
  hipLaunchKernelGGL(k_valid_count, dim3(1), dim3(256), 0, s, mask, T, tau, grad_loss, scal);
  return hipGetLastError();
}

hipError_t launch_grad_cast(const float *src, void *dst, bool bf16, int64_t n,
                            const float *scale, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t want = (n + 255) / 256;
  const int g = (int)(want < 8192 ? want : 8192);
  if (bf16)
    hipLaunchKernelGGL(k_grad_cast<uint16_t>, dim3(g), dim3(256), 0, s, src,
                       static_cast<uint16_t *>(dst), n, scale);
  else
    hipLaunchKernelGGL(k_grad_cast<float>, dim3(g), dim3(256), 0, s, src,
                       static_cast<float *>(dst), n, scale);
  return hipGetLastError();
}

hipError_t launch_prep_rows(const SliceArgs &a, hipStream_t s) {
  const int g = (a.C + ROWS_PER_WG - 1) / ROWS_PER_WG;
  hipLaunchKernelGGL(k_prep_rows, dim3(g), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_lse_fix(const SliceArgs &a, bool bf16, hipStream_t s) {
  const int g = (a.C + ROWS_PER_WG - 1) / ROWS_PER_WG;
  if (bf16)
    hipLaunchKernelGGL(k_lse_fix<uint16_t>, dim3(g), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_lse_fix<float>, dim3(g), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_reduce_dh(const SliceArgs &a, hipStream_t s) {
  const size_t n4 = (size_t)a.C * a.d / 4;
  const int g = (int)((n4 + 255) / 256);
  hipLaunchKernelGGL(k_reduce_dh, dim3(g), dim3(256), 0, s, a.dh_part, a.splits,
                     a.dh_stride, n4, a.d / 4, a.fast ? a.frow : nullptr,
                     a.dH + a.c0 * a.d);
  return hipGetLastError();
}

hipError_t launch_final_loss(const float *row_loss, int T, const Scalars *scal,
                             float *loss, hipStream_t s) {
  hipLaunchKernelGGL(k_final_loss, dim3(1), dim3(256), 0, s, row_loss, T, scal, loss);
  return hipGetLastError();
}

}  // namespace kd

namespace kd {
hipError_t launch_fix_flagged(const SliceArgs &a, hipStream_t s) {
  const int g = (a.C + ROWS_PER_WG - 1) / ROWS_PER_WG;
  hipLaunchKernelGGL(k_fix_flagged, dim3(g), dim3(256), 0, s, a);
  return hipGetLastError();
}
}  // namespace kd
