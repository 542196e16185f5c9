// C ABI of the fused, chunked top-K KL loss: argument checks, workspace
// layout and the slice loop that enqueues the kernels on the caller's
// stream.  The loop follows the pages' description of the loss ("Making
// Knowledge Distillation Cheap Enough to Run at Scale", aipuls.nl, section
// "Summary": successive slices are processed and discarded, so memory is
// bounded by one slice).
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "kd_internal.h"
#include "kd_topk_kl.h"

namespace {

thread_local char g_hip_msg[256] = "";

struct LaunchLog {
  uint32_t mask = 0;
  void *const *start = nullptr;
  void *const *end = nullptr;
  int32_t *kinds = nullptr;
  int32_t capacity = 0;
  int32_t *count = nullptr;
};
thread_local LaunchLog g_log;

// Runs `launch` (which enqueues one kernel of id `kind` on `s`), bracketed by
// the caller's events when the launch log asks for it.
template <class F>
hipError_t logged(int kind, hipStream_t s, F &&launch) {
  const bool rec = g_log.count && ((g_log.mask >> kind) & 1u) &&
                   *g_log.count < g_log.capacity;
  const int i = rec ? *g_log.count : 0;
  if (rec) {
    hipError_t e = hipEventRecord(reinterpret_cast<hipEvent_t>(g_log.start[i]), s);
    if (e != hipSuccess) return e;
  }
  hipError_t e = launch();
  if (rec && e == hipSuccess) {
    e = hipEventRecord(reinterpret_cast<hipEvent_t>(g_log.end[i]), s);
    if (g_log.kinds) g_log.kinds[i] = kind;
    ++*g_log.count;
  }
  return e;
}

struct Layout {
  int C, nseg, ldp, splits;
  int G;  // slices per dW group (tuned path)
  bool fast;
  size_t esize;
  size_t o_scal, o_rowloss, o_q, o_lq, o_zg, o_sid, o_sslot, o_first,
      o_mseg, o_sseg, o_fseg, o_lse, o_P, o_dhp, o_ht, o_shift, o_frow, o_flag,
      o_tflag;
  int dh_bn, dw_bn;
  int ldh;
  size_t total;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// The kernels move rows of H, W, dH and dW 16 bytes at a time.
bool misaligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) != 0; }

int check_sizes(int64_t T, int64_t d, int64_t V, int32_t K, int32_t chunk,
                kd_dtype dtype) {
  if (T < 1 || d < 1 || V < 1 || K < 1 || chunk < 1 || K > V)
    return KD_ERR_INVALID_ARG;
  if (dtype != KD_F32 && dtype != KD_BF16) return KD_ERR_UNSUPPORTED;
  if (d % 8 != 0 || K > KD_MAX_K) return KD_ERR_UNSUPPORTED;
  const int64_t lim = int64_t(1) << 31;
  if (T * d >= lim || V * d >= lim || T * K >= lim || V >= lim - kd::SEG)
    return KD_ERR_UNSUPPORTED;
  return KD_OK;
}

// fwd_only: the regions the forward alone touches (no probabilities, G,
// gradient factors, dH partials or the transposed hidden states): the
// compact layout of the forward entry points (kd_topk_kl_fwd and the
// allocation-free kd_topk_kl_fwd_noalloc).
Layout make_layout(int64_t T, int64_t d, int64_t V, int32_t K, int32_t chunk,
                   kd_dtype dtype, bool fwd_only = false) {
  Layout L{};
  L.C = (int)(chunk < T ? chunk : T);
  L.nseg = (int)((V + kd::SEG - 1) / kd::SEG);
  L.ldp = L.nseg * kd::SEG;
  L.fast = kd::use_fast(dtype == KD_BF16, L.C, d, V, L.ldp);
  // The tuned path keeps the probabilities of G consecutive slices and runs
  // the dW GEMM once per group, over G C tokens: every dW GEMM reads and
  // writes all of dW (V x d fp32), so small slices would otherwise spend
  // more time on that traffic than on the product.  Up to 4 slices, until
  // 2048 tokens (C a multiple of 64, so that the group's transposed hidden
  // states stay 16-byte aligned per slice).
  L.G = 1;
  if (L.fast && L.C % 64 == 0 && L.C < 2048) {
    const int64_t nsl = (T + L.C - 1) / L.C;
    int64_t g = (2048 + L.C - 1) / L.C;
    if (g > 4) g = 4;
    if (g > nsl) g = nsl;
    L.G = (int)g;
  }
  // dH and dW: 256 x 320 tiles when d is a multiple of 320, else 256 x 256
  L.dw_bn = L.fast ? kd::fast_bn((int)d) : 256;
  L.dh_bn = L.dw_bn;
  L.splits = kd::dh_splits(L.C, (int)d, L.nseg, L.fast, L.dh_bn);
  L.esize = dtype == KD_BF16 ? 2 : 4;
  const size_t C = L.C, nseg = L.nseg;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align256(o + bytes); return at; };
  L.o_scal = take(sizeof(kd::Scalars));
  L.o_rowloss = take(sizeof(float) * (size_t)T);
  L.o_q = take(sizeof(float) * C * K);
  L.o_lq = take(sizeof(float) * C * K);
  L.o_zg = take(sizeof(float) * C * K);
  L.o_sid = take(sizeof(int32_t) * C * K);
  L.o_sslot = take(sizeof(int32_t) * C * K);
  L.o_first = take(sizeof(int16_t) * C * nseg);
  L.o_mseg = take(sizeof(float) * C * nseg);
  L.o_sseg = take(sizeof(float) * C * nseg);
  const size_t g = fwd_only ? 0 : 1;  // gradient-only regions
  L.o_fseg = take(g * sizeof(float) * C * nseg);
  L.o_lse = take(sizeof(float) * C);
  L.o_P = take(g * L.esize * (size_t)L.G * C * (size_t)L.ldp);
  L.o_dhp = take(g * sizeof(float) * (size_t)L.splits * C * (size_t)d);
  L.ldh = (int)(((size_t)L.G * C + 63) / 64 * 64);
  L.o_ht = take(g * (L.fast ? sizeof(uint16_t) * (size_t)d * L.ldh : 0));
  L.o_shift = take(g * sizeof(float) * C);
  L.o_frow = take(g * sizeof(float) * C);
  L.o_flag = take(g * sizeof(int32_t) * C);
  L.o_tflag = take(g * sizeof(int32_t) * ((C + kd::ROW_TILE - 1) / kd::ROW_TILE));
  L.total = o;
  return L;
}

// ---- teacher top-K cache builder
int check_tk_sizes(int64_t T, int64_t d, int64_t V, int32_t K, int32_t chunk,
                   kd_dtype dtype) {
  if (T < 1 || d < 1 || V < 1 || K < 1 || chunk < 1 || K > V)
    return KD_ERR_INVALID_ARG;
  if (dtype != KD_F32 && dtype != KD_BF16) return KD_ERR_UNSUPPORTED;
  if (d % 8 != 0 || K > KD_TOPK_MAX_K || d > KD_TOPK_MAX_D) return KD_ERR_UNSUPPORTED;
  const int64_t lim = int64_t(1) << 31;
  if (T * d >= lim || V * d >= lim || T * K >= lim || V >= lim - kd::SEG)
    return KD_ERR_UNSUPPORTED;
  return KD_OK;
}

struct TkLayout {
  int C, nseg, ns, sstride;
  bool fast;
  size_t o_zs, o_thv, o_thi, o_cnt, o_ovf, o_cand, total;
};

TkLayout make_tk_layout(int64_t T, int64_t d, int64_t V, int32_t K, int32_t chunk,
                        kd_dtype dtype) {
  TkLayout L{};
  L.C = (int)(chunk < T ? chunk : T);
  L.nseg = (int)((V + kd::SEG - 1) / kd::SEG);
  L.fast = kd::use_fast(dtype == KD_BF16, L.C, d, V, (int64_t)L.nseg * kd::SEG);
  // sampled segments: enough that about K nseg / ns <= TK_CAP / 2 candidates
  // are expected per row, within [TK_NSAMPLE, TK_NSAMPLE_MAX]
  const int64_t want = ((int64_t)K * L.nseg + kd::TK_CAP / 2 - 1) / (kd::TK_CAP / 2);
  const int ns = (int)std::min<int64_t>(std::max<int64_t>(want, kd::TK_NSAMPLE),
                                        kd::TK_NSAMPLE_MAX);
  if (L.nseg <= ns) {
    L.ns = L.nseg;
    L.sstride = 1;
  } else {
    L.ns = ns;
    L.sstride = L.nseg / ns;
  }
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align256(o + bytes); return at; };
  const size_t C = L.C;
  if (L.fast) {
    L.o_zs = take(sizeof(float) * C * (size_t)L.ns * kd::SEG);
    L.o_thv = take(sizeof(float) * C);
    L.o_thi = take(sizeof(int32_t) * C);
    L.o_cnt = take(sizeof(int32_t) * C);
    L.o_ovf = take(sizeof(int32_t) * C);
    L.o_cand = take(sizeof(uint64_t) * C * (size_t)kd::TK_CAP);
  } else {
    take(1);  // the generic path needs no scratch; keep the size non-zero
  }
  L.total = o;
  return L;
}

int hip_fail(hipError_t e) {
  snprintf(g_hip_msg, sizeof(g_hip_msg), "HIP error: %s", hipGetErrorString(e));
  return KD_ERR_HIP;
}

}  // namespace

extern "C" {

int kd_topk_kl_workspace_size(int64_t T, int64_t d, int64_t V, int32_t K,
                              int32_t chunk, kd_dtype dtype, size_t *bytes_out) {
  if (!bytes_out) return KD_ERR_INVALID_ARG;
  const int st = check_sizes(T, d, V, K, chunk, dtype);
  if (st != KD_OK) return st;
  *bytes_out = make_layout(T, d, V, K, chunk, dtype).total;
  return KD_OK;
}

int kd_topk_kl_fwd_workspace_size(int64_t T, int64_t d, int64_t V, int32_t K,
                                  int32_t chunk, kd_dtype dtype, size_t *bytes_out) {
  if (!bytes_out) return KD_ERR_INVALID_ARG;
  const int st = check_sizes(T, d, V, K, chunk, dtype);
  if (st != KD_OK) return st;
  *bytes_out = make_layout(T, d, V, K, chunk, dtype, /*fwd_only=*/true).total;
  return KD_OK;
}

}  // extern "C"

namespace {

enum LossMode { MODE_FWD_BWD, MODE_FWD, MODE_BWD };

// The slice loop of the three loss entry points.  MODE_FWD skips the
// probability store, G and both backward GEMMs; MODE_BWD skips the loss sum
// and scales G by *grad_loss.
int run_loss(LossMode mode, const void *H, const void *W, kd_dtype dtype,
             const int32_t *topk_idx, const float *topk_logit, const uint8_t *mask,
             int64_t T, int64_t d, int64_t V, int32_t K, float tau, int32_t chunk,
             uint32_t flags, const float *grad_loss, float *loss, float *row_loss,
             float *lse_out, float *dH, float *dW, void *workspace,
             size_t workspace_bytes, void *stream, bool compact = false) {
  if (!(tau > 0.f) || !isfinite(tau)) return KD_ERR_INVALID_ARG;
  if (flags & ~uint32_t(KD_FLAG_ACCUMULATE_DW)) return KD_ERR_INVALID_ARG;
  const int st = check_sizes(T, d, V, K, chunk, dtype);
  if (st != KD_OK) return st;
  const Layout L = make_layout(T, d, V, K, chunk, dtype, compact && mode == MODE_FWD);
  if (!workspace || workspace_bytes < L.total ||
      (reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
    return KD_ERR_WORKSPACE;

  const bool grads = mode != MODE_FWD;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char *ws = static_cast<char *>(workspace);
  const bool bf16 = dtype == KD_BF16;
  kd::Scalars *scal = reinterpret_cast<kd::Scalars *>(ws + L.o_scal);
  float *rl = row_loss ? row_loss : reinterpret_cast<float *>(ws + L.o_rowloss);

  kd::SliceArgs a{};
  a.H = H;
  a.W = W;
  a.topk_idx = topk_idx;
  a.topk_logit = topk_logit;
  a.mask = mask;
  a.scal = scal;
  a.T = (int)T;
  a.d = (int)d;
  a.V = (int)V;
  a.K = K;
  a.nseg = L.nseg;
  a.ldp = L.ldp;
  a.inv_tau = 1.0f / tau;
  a.s2 = a.inv_tau * 1.4426950408889634f;
  a.q = reinterpret_cast<float *>(ws + L.o_q);
  a.lq = reinterpret_cast<float *>(ws + L.o_lq);
  a.zg = reinterpret_cast<float *>(ws + L.o_zg);
  a.sid = reinterpret_cast<int32_t *>(ws + L.o_sid);
  a.sslot = reinterpret_cast<int32_t *>(ws + L.o_sslot);
  a.first = reinterpret_cast<int16_t *>(ws + L.o_first);
  a.mseg = reinterpret_cast<float *>(ws + L.o_mseg);
  a.sseg = reinterpret_cast<float *>(ws + L.o_sseg);
  a.fseg = reinterpret_cast<float *>(ws + L.o_fseg);
  a.lse = reinterpret_cast<float *>(ws + L.o_lse);
  a.P = ws + L.o_P;
  a.dh_part = reinterpret_cast<float *>(ws + L.o_dhp);
  a.Ht = reinterpret_cast<uint16_t *>(ws + L.o_ht);
  a.shift = reinterpret_cast<float *>(ws + L.o_shift);
  a.frow = reinterpret_cast<float *>(ws + L.o_frow);
  a.flag = reinterpret_cast<int32_t *>(ws + L.o_flag);
  a.tile_flags = reinterpret_cast<int32_t *>(ws + L.o_tflag);
  a.ldh = L.ldh;
  a.dh_stride = (size_t)L.C * (size_t)d;
  a.splits = L.splits;
  a.row_loss = rl;
  a.dH = dH;
  a.dW = dW;
  a.fast = L.fast ? 1 : 0;
  a.need_grad = grads ? 1 : 0;
  a.dh_bn = L.dh_bn;
  a.dw_bn = L.dw_bn;
  a.lse_out = lse_out;

  hipError_t e = logged(KD_KERNEL_VALID_COUNT, s, [&] {
    return kd::launch_valid_count(mask, (int)T, tau, mode == MODE_BWD ? grad_loss : nullptr,
                                  scal, s);
  });
  if (e != hipSuccess) return hip_fail(e);
  for (int64_t c0 = 0; c0 < T; c0 += L.C) {
    const int j = (int)((c0 / L.C) % L.G);  // slice within its dW group
    a.c0 = c0;
    a.C = (int)(T - c0 < L.C ? T - c0 : L.C);
    a.P = ws + L.o_P + (size_t)j * L.C * L.ldp * L.esize;
    a.ht_col = j * L.C;
    if ((e = logged(KD_KERNEL_PREP_ROWS, s, [&] { return kd::launch_prep_rows(a, s); })) ||
        (e = logged(KD_KERNEL_GEMM_LOGITS, s, [&] { return kd::launch_gemm_logits(a, bf16, s); })) ||
        (e = logged(KD_KERNEL_LSE_FIX, s, [&] { return kd::launch_lse_fix(a, bf16, s); })))
      return hip_fail(e);
    if (!grads) continue;
    if ((a.fast && (e = logged(KD_KERNEL_FLAGGED_ROWS, s, [&] { return kd::launch_flagged_rows(a, s); }))) ||
        (e = logged(KD_KERNEL_GEMM_DH, s, [&] { return kd::launch_gemm_dh(a, bf16, s); })) ||
        (e = logged(KD_KERNEL_REDUCE_DH, s, [&] { return kd::launch_reduce_dh(a, s); })) ||
        (a.fast && (e = logged(KD_KERNEL_TRANSPOSE_H, s, [&] { return kd::launch_transpose_h(a, s); }))))
      return hip_fail(e);
    if (j == L.G - 1 || c0 + a.C >= T) {
      // dW over the group: its first slice's rows onwards
      kd::SliceArgs b = a;
      b.c0 = c0 - (int64_t)j * L.C;
      b.C = (int)(c0 + a.C - b.c0);
      b.P = ws + L.o_P;
      b.dw_beta = (b.c0 > 0 || (flags & KD_FLAG_ACCUMULATE_DW)) ? 1 : 0;
      e = logged(KD_KERNEL_GEMM_DW, s, [&] { return kd::launch_gemm_dw(b, bf16, s); });
      if (e != hipSuccess) return hip_fail(e);
    }
  }
  if (mode != MODE_BWD) {
    e = logged(KD_KERNEL_FINAL_LOSS, s, [&] {
      return kd::launch_final_loss(rl, (int)T, scal, loss, s);
    });
    if (e != hipSuccess) return hip_fail(e);
  }
  return KD_OK;
}

}  // namespace

extern "C" {

int kd_topk_kl_fwd_bwd(const void *H, const void *W, kd_dtype dtype,
                       const int32_t *topk_idx, const float *topk_logit,
                       const uint8_t *mask, int64_t T, int64_t d, int64_t V,
                       int32_t K, float tau, int32_t chunk, uint32_t flags,
                       float *loss, float *row_loss, float *dH, float *dW,
                       void *workspace, size_t workspace_bytes, void *stream) {
  if (!H || !W || !topk_idx || !topk_logit || !loss || !dH || !dW || misaligned16(H) ||
      misaligned16(W) || misaligned16(dH) || misaligned16(dW))
    return KD_ERR_INVALID_ARG;
  return run_loss(MODE_FWD_BWD, H, W, dtype, topk_idx, topk_logit, mask, T, d, V, K,
                  tau, chunk, flags, nullptr, loss, row_loss, nullptr, dH, dW,
                  workspace, workspace_bytes, stream);
}

int kd_topk_kl_fwd(const void *H, const void *W, kd_dtype dtype,
                   const int32_t *topk_idx, const float *topk_logit,
                   const uint8_t *mask, int64_t T, int64_t d, int64_t V,
                   int32_t K, float tau, int32_t chunk, float *loss,
                   float *row_loss, float *lse, void *workspace,
                   size_t workspace_bytes, void *stream) {
  if (!H || !W || !topk_idx || !topk_logit || !loss || misaligned16(H) || misaligned16(W))
    return KD_ERR_INVALID_ARG;
  // the forward's own (compact) layout: no probabilities, G, gradient
  // factors, dH partials or transposed hidden states
  return run_loss(MODE_FWD, H, W, dtype, topk_idx, topk_logit, mask, T, d, V, K,
                  tau, chunk, 0u, nullptr, loss, row_loss, lse, nullptr, nullptr,
                  workspace, workspace_bytes, stream, /*compact=*/true);
}

}  // extern "C"

namespace {

// Device scratch of kd_topk_kl_fwd_noalloc: one array per GPU, allocated by
// the runtime when the library's code object is loaded and kept until the
// process ends.  Host code never uses the array's name as an address (it is
// a host-side stand-in); each device's address comes from
// hipGetSymbolAddress, taken once per device with that device current.
__device__ __align__(256) unsigned char scratch[KD_NOALLOC_SCRATCH_BYTES];

constexpr int KD_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[KD_MAX_DEVICES] = {};

// The current device's address of `scratch` (nullptr and the HIP error on
// failure).
void *scratch_ptr(hipError_t *err) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess && (dev < 0 || dev >= KD_MAX_DEVICES)) e = hipErrorInvalidDevice;
  if (e != hipSuccess) {
    *err = e;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  *err = hipSuccess;
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int kd_topk_kl_fwd_noalloc(const void *H, const void *W, kd_dtype dtype,
                           const int32_t *topk_idx, const float *topk_logit,
                           const uint8_t *mask, int64_t T, int64_t d, int64_t V,
                           int32_t K, float tau, int32_t chunk, float *loss,
                           float *row_loss, float *lse, void *stream) {
  if (!H || !W || !topk_idx || !topk_logit || !loss || misaligned16(H) || misaligned16(W))
    return KD_ERR_INVALID_ARG;
  if (!(tau > 0.f) || !isfinite(tau)) return KD_ERR_INVALID_ARG;
  const int st = check_sizes(T, d, V, K, chunk, dtype);
  if (st != KD_OK) return st;
  // the size check runs before any HIP call
  if (make_layout(T, d, V, K, chunk, dtype, true).total > KD_NOALLOC_SCRATCH_BYTES)
    return KD_ERR_SCRATCH;
  hipError_t e = hipSuccess;
  void *ws = scratch_ptr(&e);
  if (!ws) return hip_fail(e);
  return run_loss(MODE_FWD, H, W, dtype, topk_idx, topk_logit, mask, T, d, V, K,
                  tau, chunk, 0u, nullptr, loss, row_loss, lse, nullptr, nullptr,
                  ws, KD_NOALLOC_SCRATCH_BYTES, stream, /*compact=*/true);
}

int kd_topk_kl_bwd(const void *H, const void *W, kd_dtype dtype,
                   const int32_t *topk_idx, const float *topk_logit,
                   const uint8_t *mask, int64_t T, int64_t d, int64_t V,
                   int32_t K, float tau, int32_t chunk, uint32_t flags,
                   const float *grad_loss, float *dH, float *dW, void *workspace,
                   size_t workspace_bytes, void *stream) {
  if (!H || !W || !topk_idx || !topk_logit || !dH || !dW || misaligned16(H) || misaligned16(W) ||
      misaligned16(dH) || misaligned16(dW))
    return KD_ERR_INVALID_ARG;
  return run_loss(MODE_BWD, H, W, dtype, topk_idx, topk_logit, mask, T, d, V, K,
                  tau, chunk, flags, grad_loss, nullptr, nullptr, nullptr, dH, dW,
                  workspace, workspace_bytes, stream);
}

int kd_grad_cast(const float *src, void *dst, kd_dtype dst_dtype, int64_t n,
                 const float *scale, void *stream) {
  if (!src || !dst || n < 0) return KD_ERR_INVALID_ARG;
  if (dst_dtype != KD_F32 && dst_dtype != KD_BF16) return KD_ERR_UNSUPPORTED;
  hipError_t e = logged(KD_KERNEL_GRAD_CAST, reinterpret_cast<hipStream_t>(stream), [&] {
    return kd::launch_grad_cast(src, dst, dst_dtype == KD_BF16, n, scale,
                                reinterpret_cast<hipStream_t>(stream));
  });
  return e == hipSuccess ? KD_OK : hip_fail(e);
}

int kd_teacher_topk_workspace_size(int64_t T, int64_t d, int64_t V, int32_t K,
                                   int32_t chunk, kd_dtype dtype, size_t *bytes_out) {
  if (!bytes_out) return KD_ERR_INVALID_ARG;
  const int st = check_tk_sizes(T, d, V, K, chunk, dtype);
  if (st != KD_OK) return st;
  *bytes_out = make_tk_layout(T, d, V, K, chunk, dtype).total;
  return KD_OK;
}

int kd_teacher_topk(const void *H, const void *W, kd_dtype dtype, int64_t T,
                    int64_t d, int64_t V, int32_t K, int32_t chunk,
                    int32_t *topk_idx, float *topk_logit, void *workspace,
                    size_t workspace_bytes, void *stream) {
  if (!H || !W || !topk_idx || !topk_logit || misaligned16(H) || misaligned16(W))
    return KD_ERR_INVALID_ARG;
  const int st = check_tk_sizes(T, d, V, K, chunk, dtype);
  if (st != KD_OK) return st;
  const TkLayout L = make_tk_layout(T, d, V, K, chunk, dtype);
  if (!workspace || workspace_bytes < L.total ||
      (reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
    return KD_ERR_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char *ws = static_cast<char *>(workspace);
  kd::TkArgs a{};
  a.H = H;
  a.W = W;
  a.T = (int)T;
  a.d = (int)d;
  a.V = (int)V;
  a.K = K;
  a.nseg = L.nseg;
  a.ns = L.ns;
  a.sstride = L.sstride;
  a.ldzs = L.ns * kd::SEG;
  a.cap = kd::TK_CAP;
  a.out_idx = topk_idx;
  a.out_val = topk_logit;
  if (L.fast) {
    a.zs = reinterpret_cast<float *>(ws + L.o_zs);
    a.th_v = reinterpret_cast<float *>(ws + L.o_thv);
    a.th_i = reinterpret_cast<int32_t *>(ws + L.o_thi);
    a.cnt = reinterpret_cast<int32_t *>(ws + L.o_cnt);
    a.ovf = reinterpret_cast<int32_t *>(ws + L.o_ovf);
    a.cand = reinterpret_cast<uint64_t *>(ws + L.o_cand);
  }
  a.all_rows = L.fast ? 0 : 1;
  const bool bf16 = dtype == KD_BF16;
  hipError_t e = hipSuccess;
  for (int64_t c0 = 0; c0 < T; c0 += L.C) {
    a.c0 = c0;
    a.C = (int)(T - c0 < L.C ? T - c0 : L.C);
    if (L.fast) {
      if ((e = logged(KD_KERNEL_TK_SAMPLE, s, [&] { return kd::launch_tk_sample(a, s); })) ||
          (e = logged(KD_KERNEL_TK_THETA, s, [&] { return kd::launch_tk_theta(a, s); })) ||
          (e = logged(KD_KERNEL_TK_FILTER, s, [&] { return kd::launch_tk_filter(a, s); })) ||
          (e = logged(KD_KERNEL_TK_SELECT, s, [&] { return kd::launch_tk_select(a, s); })))
        return hip_fail(e);
    }
    e = logged(KD_KERNEL_TK_STREAM, s, [&] { return kd::launch_tk_stream(a, bf16, s); });
    if (e != hipSuccess) return hip_fail(e);
  }
  return KD_OK;
}

}  // extern "C"

namespace {

struct DivLayout {
  size_t o_scal, o_rowloss, o_gk, o_k0, o_k1, o_v0, o_v1, o_hist, o_seg, o_units, o_parts,
      o_partial, o_bsum, total;
};

DivLayout make_div_layout(int64_t T, int64_t d, int64_t V, int32_t K) {
  DivLayout L{};
  const size_t n = (size_t)T * K;
  const size_t nblk = (n + kd::RADIX_BLOCK - 1) / kd::RADIX_BLOCK;
  const size_t pmax = 2 * ((n + kd::DIV_UNIT - 1) / kd::DIV_UNIT);
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align256(o + bytes); return at; };
  L.o_scal = take(sizeof(kd::Scalars));
  L.o_rowloss = take(sizeof(float) * (size_t)T);
  L.o_gk = take(sizeof(float) * n);
  L.o_k0 = take(sizeof(int32_t) * n);
  L.o_k1 = take(sizeof(int32_t) * n);
  L.o_v0 = take(sizeof(int32_t) * n);
  L.o_v1 = take(sizeof(int32_t) * n);
  L.o_hist = take(sizeof(int32_t) * 256 * nblk);
  L.o_seg = take(sizeof(int32_t) * ((size_t)V + 1));
  L.o_units = take(sizeof(int32_t) * ((size_t)V + 1));
  L.o_parts = take(sizeof(int32_t) * ((size_t)V + 1));
  L.o_partial = take(sizeof(float) * pmax * (size_t)d);
  const int64_t nscan = std::max<int64_t>(256 * (int64_t)nblk, V + 1);
  L.o_bsum = take(sizeof(int32_t) * (size_t)kd::div_scan_blocks(nscan));
  L.total = o;
  return L;
}

}  // namespace

extern "C" {

int kd_topk_div_workspace_size(int64_t T, int64_t d, int64_t V, int32_t K, size_t *bytes_out) {
  if (!bytes_out) return KD_ERR_INVALID_ARG;
  const int st = check_sizes(T, d, V, K, 1, KD_BF16);
  if (st != KD_OK) return st;
  *bytes_out = make_div_layout(T, d, V, K).total;
  return KD_OK;
}

int kd_topk_div_fwd_bwd(int32_t kind, const void *H, const void *W, kd_dtype dtype,
                        const int32_t *topk_idx, const float *topk_logit,
                        const uint8_t *mask, int64_t T, int64_t d, int64_t V, int32_t K,
                        float tau, uint32_t flags, float *loss, float *row_loss, float *dH,
                        float *dW, void *workspace, size_t workspace_bytes, void *stream) {
  if (kind != KD_DIV_REVERSE_KL && kind != KD_DIV_JSD) return KD_ERR_INVALID_ARG;
  if (!H || !W || !topk_idx || !topk_logit || !loss || !dH || !dW || misaligned16(H) ||
      misaligned16(W) || misaligned16(dH) || misaligned16(dW))
    return KD_ERR_INVALID_ARG;
  if (!(tau > 0.f) || !isfinite(tau)) return KD_ERR_INVALID_ARG;
  if (flags & ~uint32_t(KD_FLAG_ACCUMULATE_DW)) return KD_ERR_INVALID_ARG;
  const int st = check_sizes(T, d, V, K, 1, dtype);
  if (st != KD_OK) return st;
  const DivLayout L = make_div_layout(T, d, V, K);
  if (!workspace || workspace_bytes < L.total ||
      (reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
    return KD_ERR_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char *ws = static_cast<char *>(workspace);
  kd::Scalars *scal = reinterpret_cast<kd::Scalars *>(ws + L.o_scal);
  float *rl = row_loss ? row_loss : reinterpret_cast<float *>(ws + L.o_rowloss);
  kd::DivArgs a{};
  a.H = H;
  a.W = W;
  a.topk_idx = topk_idx;
  a.topk_logit = topk_logit;
  a.mask = mask;
  a.scal = scal;
  a.T = T;
  a.d = (int)d;
  a.V = (int)V;
  a.K = K;
  a.inv_tau = 1.0f / tau;
  a.kind = kind;
  a.bf16 = dtype == KD_BF16 ? 1 : 0;
  a.accumulate = (flags & KD_FLAG_ACCUMULATE_DW) ? 1 : 0;
  a.Gk = reinterpret_cast<float *>(ws + L.o_gk);
  a.row_loss = rl;
  a.dH = dH;
  a.dW = dW;
  a.keys[0] = reinterpret_cast<int32_t *>(ws + L.o_k0);
  a.keys[1] = reinterpret_cast<int32_t *>(ws + L.o_k1);
  a.vals[0] = reinterpret_cast<int32_t *>(ws + L.o_v0);
  a.vals[1] = reinterpret_cast<int32_t *>(ws + L.o_v1);
  a.hist = reinterpret_cast<int32_t *>(ws + L.o_hist);
  a.seg = reinterpret_cast<int32_t *>(ws + L.o_seg);
  a.unit_start = reinterpret_cast<int32_t *>(ws + L.o_units);
  a.part_start = reinterpret_cast<int32_t *>(ws + L.o_parts);
  a.partial = reinterpret_cast<float *>(ws + L.o_partial);
  a.bsum = reinterpret_cast<int32_t *>(ws + L.o_bsum);
  hipError_t e = logged(KD_KERNEL_VALID_COUNT, s, [&] {
    return kd::launch_valid_count(mask, (int)T, tau, nullptr, scal, s);
  });
  if (e != hipSuccess) return hip_fail(e);
  e = logged(KD_KERNEL_DIVERGENCE, s, [&] { return kd::launch_div(a, s); });
  if (e != hipSuccess) return hip_fail(e);
  e = logged(KD_KERNEL_FINAL_LOSS, s, [&] {
    return kd::launch_final_loss(rl, (int)T, scal, loss, s);
  });
  return e == hipSuccess ? KD_OK : hip_fail(e);
}

int kd_entropy_filter_workspace_size(int64_t T, size_t *bytes_out) {
  if (!bytes_out || T < 1) return KD_ERR_INVALID_ARG;
  if (T >= (int64_t(1) << 31)) return KD_ERR_UNSUPPORTED;
  *bytes_out = align256(sizeof(uint64_t) * 2) + align256(sizeof(float) * (size_t)T);
  return KD_OK;
}

int kd_entropy_filter(const float *topk_logit, const uint8_t *mask, int64_t T,
                      int32_t K, float tau, int32_t mode, float param,
                      uint8_t *mask_out, float *entropy_out, void *workspace,
                      size_t workspace_bytes, void *stream) {
  if (!topk_logit || !mask_out || T < 1 || K < 1) return KD_ERR_INVALID_ARG;
  if (!(tau > 0.f) || !isfinite(tau) || !isfinite(param)) return KD_ERR_INVALID_ARG;
  if (mode != KD_FILTER_ENTROPY_ABOVE && mode != KD_FILTER_TOP_ENTROPY_FRACTION)
    return KD_ERR_INVALID_ARG;
  if (mode == KD_FILTER_TOP_ENTROPY_FRACTION && !(param >= 0.f && param <= 1.f))
    return KD_ERR_INVALID_ARG;
  if (K > KD_MAX_K || T >= (int64_t(1) << 31) || T * K >= (int64_t(1) << 31))
    return KD_ERR_UNSUPPORTED;
  size_t need = 0;
  kd_entropy_filter_workspace_size(T, &need);
  if (!workspace || workspace_bytes < need ||
      (reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
    return KD_ERR_WORKSPACE;
  char *ws = static_cast<char *>(workspace);
  kd::FilterArgs a{};
  a.topk_logit = topk_logit;
  a.mask = mask;
  a.T = T;
  a.K = K;
  a.inv_tau = 1.0f / tau;
  a.mode = mode;
  a.param = param;
  a.sel = reinterpret_cast<uint64_t *>(ws);
  a.entropy = entropy_out ? entropy_out
                          : reinterpret_cast<float *>(ws + align256(sizeof(uint64_t) * 2));
  a.mask_out = mask_out;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const hipError_t e = logged(KD_KERNEL_ENTROPY_FILTER, s,
                              [&] { return kd::launch_entropy_filter(a, s); });
  return e == hipSuccess ? KD_OK : hip_fail(e);
}

int kd_set_launch_log(uint32_t kernel_mask, void *const *start_events,
                      void *const *end_events, int32_t *kinds,
                      int32_t capacity, int32_t *count) {
  if (kernel_mask == 0 || count == nullptr) {
    g_log = LaunchLog{};
    return KD_OK;
  }
  if (!start_events || !end_events || capacity < 0) return KD_ERR_INVALID_ARG;
  g_log.mask = kernel_mask;
  g_log.start = start_events;
  g_log.end = end_events;
  g_log.kinds = kinds;
  g_log.capacity = capacity;
  g_log.count = count;
  return KD_OK;
}

const char *kd_status_string(int status) {
  switch (status) {
    case KD_OK: return "KD_OK: success";
    case KD_ERR_INVALID_ARG:
      return "KD_ERR_INVALID_ARG: null pointer, non-positive size, K > V, "
             "chunk < 1, unknown flag or tau not finite and positive";
    case KD_ERR_WORKSPACE:
      return "KD_ERR_WORKSPACE: workspace missing, smaller than "
             "kd_topk_kl_workspace_size() or not 256-byte aligned";
    case KD_ERR_UNSUPPORTED:
      return "KD_ERR_UNSUPPORTED: d % 8 != 0, K > KD_MAX_K, unknown dtype or "
             "sizes beyond the 32-bit index range";
    case KD_ERR_HIP: return g_hip_msg[0] ? g_hip_msg : "KD_ERR_HIP: HIP error";
    case KD_ERR_SCRATCH:
      return "KD_ERR_SCRATCH: the forward's scratch for these sizes and this "
             "chunk exceeds the fixed KD_NOALLOC_SCRATCH_BYTES of "
             "kd_topk_kl_fwd_noalloc (use a smaller chunk)";
    default: return "unknown kd status";
  }
}

}  // extern "C"
