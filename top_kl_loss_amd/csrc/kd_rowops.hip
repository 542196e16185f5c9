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
// K cached slots and c = sum_k q log q; the row's ids sorted ascending (with
// their slots) and, for every vocabulary segment, the first sorted position
// whose id falls in it (-1 if none).  Also clears the gathered-logit row.
// Ids outside [0, V) are replaced by INT_MAX so that no later kernel
// dereferences them.
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
    for (int k = lane; k < K; k += 64) sum += exp2f((lg[k] * a.inv_tau - mx) * LOG2E);
    sum = wave_sum(sum);
    const float lsum = logf(sum);
    float cacc = 0.f;
    for (int k = lane; k < K; k += 64) {
      const float lq = (lg[k] * a.inv_tau - mx) - lsum;
      const float qk = exp2f(lq * LOG2E);
      a.q[(size_t)r * K + k] = qk;
      cacc += qk * lq;
      a.zg[(size_t)r * K + k] = 0.f;
      const int id = a.topk_idx[t * K + k];
      s_ids[wave][k] = (id >= 0 && id < a.V) ? id : INT_MAX;
    }
    cacc = wave_sum(cacc);
    if (lane == 0) a.cterm[r] = cacc;
  }
  __syncthreads();
  if (active) {
    for (int k = lane; k < K; k += 64) {
      const int idk = s_ids[wave][k];
      int rank = 0;
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
    for (int j = lane; j < a.nseg; j += 64) {
      const int lo = j * SEG;
      int L = 0, R = K;
      while (L < R) {
        const int mid = (L + R) >> 1;
        if (s_sorted[wave][mid] < lo) L = mid + 1; else R = mid;
      }
      a.first[(size_t)r * a.nseg + j] =
          int16_t((L < K && s_sorted[wave][L] < lo + SEG) ? L : -1);
    }
  }
}

// Per slice row, after the logits GEMM:
//  lse_t = logsumexp over segments of (shift_j + log sum_j);
//  KL_t  = c_t + lse_t - sum_k q_k z_k / tau      (z_k gathered by the GEMM);
//  P[t, id_k] -= q_k exp(lse_t - shift_j)          (teacher correction, so
//        that f_j * P is exactly tau/N (p - q_scat) on segment j);
//  f_j   = tau/N * mask_t * exp(shift_j - lse_t);
//  G[t, v] = f_seg(v) * P[t, v]  written over P (= tau/N mask (p - q_scat)).
// A segment holding teacher ids whose shift lies more than RESHIFT_NATS
// below lse_t is first re-shifted to lse_t - RESHIFT_NATS.
template <typename T>
__global__ __launch_bounds__(256) void k_lse_fix(SliceArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = blockIdx.x * ROWS_PER_WG + wave;
  if (r >= a.C) return;
  const int nseg = a.nseg, K = a.K;
  const int64_t t = a.c0 + r;
  float *mrow = a.mseg + (size_t)r * nseg;
  const float *srow = a.sseg + (size_t)r * nseg;

  float mx = -INFINITY;
  for (int j = lane; j < nseg; j += 64) mx = fmaxf(mx, mrow[j]);
  mx = wave_max(mx);
  float s = 0.f;
  for (int j = lane; j < nseg; j += 64) s += srow[j] * exp2f((mrow[j] - mx) * LOG2E);
  s = wave_sum(s);
  const float lse = mx + logf(s);

  float dot = 0.f;
  for (int k = lane; k < K; k += 64) dot += a.q[(size_t)r * K + k] * a.zg[(size_t)r * K + k];
  dot = wave_sum(dot);
  const bool valid = a.mask ? (a.mask[t] != 0) : true;
  if (lane == 0) {
    a.lse[r] = lse;
    if (a.lse_out) a.lse_out[t] = lse;
    a.row_loss[t] = valid ? (a.cterm[r] + lse - dot * a.inv_tau) : 0.f;
  }
  if (!a.need_grad) return;

  const float gscale = valid ? a.scal->grad_scale : 0.f;
  T *P = reinterpret_cast<T *>(a.P) + (size_t)r * a.ldp;
  const int32_t *sid = a.sid + (size_t)r * K;
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
          need = first_in_seg && (lse - mrow[j] > RESHIFT_NATS);
        }
      }
      uint64_t bal = __ballot(need);
      while (bal) {
        const int src = __ffsll((unsigned long long)bal) - 1;
        bal &= bal - 1;
        const int js = __shfl(j, src, 64);
        const float newm = lse - RESHIFT_NATS;
        const float fac = exp2f((mrow[js] - newm) * LOG2E);
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
        const float corr = a.q[(size_t)r * K + slot] * exp2f((lse - mrow[j]) * LOG2E);
        P[id] = Elem<T>::from_f(Elem<T>::to_f(P[id]) - corr);
      }
    }
  }
  float *frow = a.fseg + (size_t)r * nseg;
  for (int j = lane; j < nseg; j += 64)
    frow[j] = gscale != 0.f ? gscale * exp2f((mrow[j] - lse) * LOG2E) : 0.f;
  if (a.fast) return;  // k_scale_g forms G (and G^T) on the tuned path
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

// dH rows of the slice = ordered sum of the split-K partials.
__global__ __launch_bounds__(256) void k_reduce_dh(const float *part, int splits,
                                                   size_t stride, size_t n4,
                                                   float *out) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  f32x4 acc = reinterpret_cast<const f32x4 *>(part)[i];
  for (int s = 1; s < splits; ++s)
    acc += reinterpret_cast<const f32x4 *>(part + s * stride)[i];
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
                     a.dh_stride, n4, a.dH + a.c0 * a.d);
  return hipGetLastError();
}

hipError_t launch_final_loss(const float *row_loss, int T, const Scalars *scal,
                             float *loss, hipStream_t s) {
  hipLaunchKernelGGL(k_final_loss, dim3(1), dim3(256), 0, s, row_loss, T, scal, loss);
  return hipGetLastError();
}

}  // namespace kd
