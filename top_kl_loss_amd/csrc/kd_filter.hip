// Entropy-based distillation token filtering over the cached teacher top-K
// (asibiont.com article, sections "Distillation Token Filtering" and "A
// Concrete Implementation Sketch"): tokens whose teacher distribution is
// nearly deterministic carry little signal, so the loss may skip tokens
// whose teacher entropy is at or below a threshold, or keep only a fixed
// fraction of the batch's tokens, those with the highest entropy.  The
// teacher distribution is the one the loss uses: softmax of the K cached
// logits at temperature tau.  The result is a token mask for the loss.
#include <limits.h>

#include "kd_device.h"
#include "kd_internal.h"
#include "kd_select.h"

namespace kd {

namespace {

using namespace sel;

constexpr int ROWS_PER_WG = 4;  // one wave per row

// entropy[t] = -sum_k q_k log q_k, q = softmax(topk_logit[t,:] / tau);
// threshold mode also writes mask_out[t] = mask[t] && entropy[t] > param.
__global__ __launch_bounds__(256) void k_entropy_rows(FilterArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * ROWS_PER_WG + wave;
  if (t >= a.T) return;
  const float *lg = a.topk_logit + t * a.K;
  float mx = -INFINITY;
  for (int k = lane; k < a.K; k += 64) mx = fmaxf(mx, lg[k] * a.inv_tau);
  mx = wave_max(mx);
  float sum = 0.f;
  for (int k = lane; k < a.K; k += 64) sum += exp2f((lg[k] * a.inv_tau - mx) * LOG2E);
  sum = wave_sum(sum);
  const float lsum = logf(sum);
  float h = 0.f;
  for (int k = lane; k < a.K; k += 64) {
    const float lq = (lg[k] * a.inv_tau - mx) - lsum;
    h -= exp2f(lq * LOG2E) * lq;
  }
  h = wave_sum(h);
  if (lane == 0) {
    a.entropy[t] = h;
    if (a.mode == 0) {
      const bool valid = a.mask ? a.mask[t] != 0 : true;
      a.mask_out[t] = (valid && h > a.param) ? 1 : 0;
    }
  }
}

// One workgroup: N = number of valid tokens, n_keep = floor(param * N +
// 1/2), and the n_keep-th smallest key (entropy descending, token index
// ascending) among the valid tokens.
// Up to ENT_LDS_ROWS tokens keep the high words of their keys in LDS for
// the selection's passes; longer batches read them from memory each pass.
constexpr int ENT_LDS_ROWS = 32768;

template <bool IN_LDS>
__global__ __launch_bounds__(256) void k_entropy_select(FilterArgs a) {
  extern __shared__ uint32_t khi[];  // [T] when IN_LDS
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sc[8];
  __shared__ uint64_t res;
  const int tid = threadIdx.x;
  const uint8_t *mask = a.mask;
  const float *ent = a.entropy;
  uint32_t cnt = 0;
  for (int64_t t = tid; t < a.T; t += 256) {
    const bool valid = mask ? (mask[t] != 0) : true;
    cnt += valid;
    if (IN_LDS) khi[t] = valid ? key_hi(ent[t]) : 0xffffffffu;
  }
  const uint32_t n_valid = block_incl_scan(cnt, sc);  // thread 255 holds the total
  __syncthreads();
  if (tid == 255) sc[7] = n_valid;
  __syncthreads();
  const uint32_t N = sc[7];
  const int64_t n_keep = (int64_t)floor(double(a.param) * double(N) + 0.5);
  __syncthreads();
  uint64_t kappa = 0;
  if (n_keep > 0) {
    if (IN_LDS) {
      // padding tokens: high word 0xffffffff, above every valid key
      auto key_at = [](int i) { return (uint64_t(khi[i]) << 32) | uint32_t(i); };
      kappa = block_select(key_at, (int)a.T, (int)(n_keep - 1), hist, sc, &res);
    } else {
      auto key_at = [mask, ent](int i) {
        const bool valid = mask ? mask[i] != 0 : true;
        return valid ? make_key(ent[i], i) : ~0ull;
      };
      kappa = block_select(key_at, (int)a.T, (int)(n_keep - 1), hist, sc, &res);
    }
  }
  if (tid == 0) {
    a.sel[0] = kappa;
    a.sel[1] = (uint64_t)n_keep;
  }
}

// mask_out[t] = mask[t] && key(t) <= kappa (and n_keep > 0).  A padding
// token's key in the selection ranks after every valid key, and padding is
// never kept, so both key forms agree here.
__global__ __launch_bounds__(256) void k_entropy_apply(FilterArgs a) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= a.T) return;
  const bool valid = a.mask ? a.mask[t] != 0 : true;
  const bool keep = valid && a.sel[1] > 0 && make_key(a.entropy[t], (int)t) <= a.sel[0];
  a.mask_out[t] = keep ? 1 : 0;
}

}  // namespace

hipError_t launch_entropy_filter(const FilterArgs &a, hipStream_t s) {
  const int g = (int)((a.T + ROWS_PER_WG - 1) / ROWS_PER_WG);
  hipLaunchKernelGGL(k_entropy_rows, dim3(g), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.mode == 0) return e;
  if (a.T <= ENT_LDS_ROWS) {
    const int lds = (int)(a.T * sizeof(uint32_t));
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(k_entropy_select<true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_entropy_select<true>, dim3(1), dim3(256), lds, s, a);
  } else {
    hipLaunchKernelGGL(k_entropy_select<false>, dim3(1), dim3(256), 0, s, a);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_entropy_apply, dim3((unsigned)((a.T + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace kd
