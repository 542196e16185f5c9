// Internal declarations shared by the launcher and the kernel translation
// units of the fused, chunked top-K KL loss.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kd {

// Width of one vocabulary segment.  The logits GEMM uses it as its N tile,
// so the per-row softmax statistics come in segments of this many
// vocabulary entries; the backward GEMMs align their tiles to it.
constexpr int SEG = 256;

// Generic path: a segment's stored probabilities are shifted by the
// segment's own maximum.  When the row's logsumexp lies more than this far
// (in units of z/tau) above a segment maximum that carries teacher ids, the
// segment is shifted again so that the teacher correction stays finite in
// the stored type.
constexpr float RESHIFT_NATS = 60.0f;

// Tuned path: the probabilities of a row are stored as 2^(z s2 - shift) with
// one a-priori shift per row (the largest student logit among the row's
// SHIFT_SLOTS best teacher slots, a lower bound of the row maximum).  A row
// whose maximum lies more than SHIFT_LIMIT2 (base-2 units) above its shift
// is flagged and its probabilities are recomputed with the exact maximum.
constexpr int SHIFT_SLOTS = 8;
constexpr float SHIFT_LIMIT2 = 64.0f;
constexpr int ROW_TILE = 256;  // rows per M-tile of the tuned logits GEMM

// Device-resident scalars written once per call.
struct Scalars {
  int32_t n_valid;
  float grad_scale;  // tau / N  (0 when N == 0)
  float loss_scale;  // tau^2 / N (0 when N == 0)
  int32_t pad[61];
};

// Everything one slice of `C` token rows needs.  Pointers are device
// pointers.  Row r of the slice is token c0 + r.
struct SliceArgs {
  const void *H;            // [T, d] element type
  const void *W;            // [V, d] element type
  const int32_t *topk_idx;  // [T, K]
  const float *topk_logit;  // [T, K]
  const uint8_t *mask;      // [T] or nullptr
  const Scalars *scal;
  int64_t c0;
  int C;       // rows in this slice
  int T, d, V, K;
  int nseg;    // ceil(V / SEG)
  int ldp;     // nseg * SEG, row pitch of P in elements
  float inv_tau;
  float s2;          // log2(e) / tau: logits in base-2 units (z s2)
  // workspace views (slice-local, row r)
  float *q;          // [Cmax, K] teacher probabilities
  float *lq;         // [Cmax, K] log q, from shifted logits (accurate near 0)
  float *zg;         // [Cmax, K] student logit at each teacher slot
  int32_t *sid;      // [Cmax, K] teacher ids sorted ascending
  int32_t *sslot;    // [Cmax, K] slot of each sorted id
  int16_t *first;    // [Cmax, nseg] first sorted position in segment or -1
  float *mseg;       // [Cmax, nseg] segment max of z s2 (shift, base-2 units)
  float *sseg;       // [Cmax, nseg] segment sum of 2^(z s2 - shift)
  float *fseg;       // [Cmax, nseg] tau/N * mask * exp(shift - lse)
  uint16_t *Ht;      // [d, ldh] bf16 (f H)^T of the dW group's tokens (tuned)
  int ht_col;        // tuned path: column of Ht where this slice's tokens go
  float *shift;      // [Cmax] tuned path: row shift (base-2 units)
  float *frow;       // [Cmax] tuned path: gradient factor f_t of the row
  int32_t *flag;     // [Cmax] tuned path: 1 = row recomputed with its max
  int32_t *tile_flags;  // [ceil(Cmax/ROW_TILE)] flagged rows per M-tile
  int ldh;           // row pitch of Ht: the dW group's tokens rounded up to 64
  float *lse;        // [Cmax] row logsumexp of z/tau
  void *P;           // [Cmax, ldp] shifted probabilities, then (after
                     // k_lse_fix) the logit gradient G (element type); for
                     // the dW GEMM, the group's rows (C of them)
  float *dh_part;    // [splits, Cmax, d] split-K partial sums of dH
  size_t dh_stride;  // elements between two partials (Cmax * d)
  int splits;
  float *row_loss;   // [T] mask * KL_t
  float *dH;         // [T, d]
  float *dW;         // [V, d]
  int dw_beta;       // 0: dW = G^T H, 1: dW += G^T H
  int fast;          // use the tuned bf16 kernels
  int need_grad;     // 0: forward only (no P store, no G)
  int dh_bn, dw_bn;  // tuned path: N-tile width of dH and dW (256 or 320)
  float *lse_out;    // [T] row logsumexp of z/tau, or null
};

// Tile shapes of the three GEMMs (all use 256-thread workgroups).
constexpr int G1_BM = 128, G1_BN = SEG;   // logits:  C x V, K = d
constexpr int DH_BM = 128, DH_BN = 128;   // dH:      C x d, K = V (split)
constexpr int DW_BM = 128, DW_BN = 128;   // dW:      V x d, K = C

// The tuned bf16 kernels (kd_gemm_fast.hip) need d % 64 == 0 (and pitches
// below 2^22 elements, so that offsets inside a 256-row tile fit the 32-bit
// buffer offsets); otherwise the generic kernels (kd_gemm.hip) run.
bool use_fast(bool bf16, int64_t C, int64_t d, int64_t V, int64_t ldp);
int dh_splits(int C, int d, int nseg, bool fast, int bn);
int fast_dh_splits(int C, int d, int nseg, int bn);
// N-tile width (256 or 320) of the tuned dH and dW GEMMs for hidden size d:
// the one that wastes less matrix-core work on padding.
int fast_bn(int d);
hipError_t launch_fast_logits(const SliceArgs &a, hipStream_t s);
hipError_t launch_fast_dh(const SliceArgs &a, hipStream_t s);
hipError_t launch_fast_dw(const SliceArgs &a, hipStream_t s);
// H_c^T for the tuned dW GEMM (no-op on the generic path).
hipError_t launch_transpose_h(const SliceArgs &a, hipStream_t s);
// Tuned path: rows flagged by k_lse_fix (shift too far below the row
// maximum) get their probabilities recomputed with the maximum and their
// teacher correction; no work beyond a flag check when none is flagged.
hipError_t launch_flagged_rows(const SliceArgs &a, hipStream_t s);
// The teacher correction of the flagged rows (part of launch_flagged_rows).
hipError_t launch_fix_flagged(const SliceArgs &a, hipStream_t s);

// Launch wrappers; each returns hipSuccess or the launch error.
hipError_t launch_valid_count(const uint8_t *mask, int T, float tau,
                              const float *grad_loss, Scalars *scal, hipStream_t s);
hipError_t launch_grad_cast(const float *src, void *dst, bool bf16, int64_t n,
                            const float *scale, hipStream_t s);
hipError_t launch_prep_rows(const SliceArgs &a, hipStream_t s);
hipError_t launch_lse_fix(const SliceArgs &a, bool bf16, hipStream_t s);
hipError_t launch_reduce_dh(const SliceArgs &a, hipStream_t s);
hipError_t launch_final_loss(const float *row_loss, int T,
                             const Scalars *scal, float *loss, hipStream_t s);
hipError_t launch_gemm_logits(const SliceArgs &a, bool bf16, hipStream_t s);
hipError_t launch_gemm_dh(const SliceArgs &a, bool bf16, hipStream_t s);
hipError_t launch_gemm_dw(const SliceArgs &a, bool bf16, hipStream_t s);

// ---------------------------------------------------------------------------
// Teacher top-K cache builder (z = H W^T, per row the K largest entries).

// Sampled vocabulary segments per row (evenly spaced, segment 0 included);
// the K-th best entry among them bounds the row's K-th best from below.
// At least TK_NSAMPLE; more for large K nseg, so that a row without
// structure expects about K nseg / ns <= TK_CAP / 2 candidates; at most
// TK_NSAMPLE_MAX (the threshold kernel holds the samples of a row in LDS).
constexpr int TK_NSAMPLE = 32;
constexpr int TK_NSAMPLE_MAX = 128;
// Candidate slots per row; a row with more candidates than this is
// recomputed by the row-streaming kernel.
constexpr int TK_CAP = 8192;
// Merge buffer of the row-streaming kernel (entries, a power of two).
constexpr int TK_STREAM_BUF = 2048;

struct TkArgs {
  const void *H;     // [T, d] element type (teacher hidden states)
  const void *W;     // [V, d] element type (teacher LM head)
  int64_t c0;        // first token of the slice
  int C;             // rows in this slice
  int T, d, V, K;
  int nseg;          // ceil(V / SEG)
  int ns, sstride;   // sampled segments: j * sstride for j < ns
  float *zs;         // [Cmax, ns * SEG] logits of the sampled segments
  int ldzs;          // ns * SEG
  float *th_v;       // [Cmax] value of the row's threshold entry
  int32_t *th_i;     // [Cmax] id of the row's threshold entry
  int32_t *cnt;      // [Cmax] candidates appended
  int32_t *ovf;      // [Cmax] 1 when the candidate slots overflowed
  uint64_t *cand;    // [Cmax, cap] candidate keys
  int cap;
  int32_t *out_idx;  // [T, K]
  float *out_val;    // [T, K]
  int all_rows;      // row-streaming kernel: every row, not only overflows
};

// ---------------------------------------------------------------------------
// Entropy-based token filter over the cached teacher top-K.
struct FilterArgs {
  const float *topk_logit;  // [T, K]
  const uint8_t *mask;      // [T] or null (all valid)
  int64_t T;
  int K;
  float inv_tau;
  int mode;                 // 0: entropy > param; 1: top fraction param
  float param;
  float *entropy;           // [T] teacher entropy (output or workspace)
  uint8_t *mask_out;        // [T]
  uint64_t *sel;            // [2] workspace: selection key, kept count
};
hipError_t launch_entropy_filter(const FilterArgs &a, hipStream_t s);

// ---------------------------------------------------------------------------
// Reverse KL / Jensen-Shannon divergence over the cached top-K support.
constexpr int DIV_UNIT = 1024;     // pairs per unit of the dW reduction
constexpr int RADIX_BLOCK = 4096;  // keys per block of the radix sort
struct DivArgs {
  const void *H;            // [T, d] element type
  const void *W;            // [V, d] element type
  const int32_t *topk_idx;  // [T, K]
  const float *topk_logit;  // [T, K]
  const uint8_t *mask;      // [T] or null
  const Scalars *scal;
  int64_t T;
  int d, V, K;
  float inv_tau;
  int kind;                 // KD_DIV_REVERSE_KL or KD_DIV_JSD
  int bf16;                 // element type of H and W
  int accumulate;           // dW += instead of dW =
  float *Gk;                // [T, K] logit gradient at the ids
  float *row_loss;          // [T] mask * D_t
  float *dH;                // [T, d]
  float *dW;                // [V, d]
  int32_t *keys[2];         // [T K] radix sort keys (ping-pong)
  int32_t *vals[2];         // [T K] pair indices (ping-pong)
  int32_t *hist;            // [256 * blocks] digit counts, then offsets
  int32_t *seg;             // [V + 1] first sorted pair of each id
  int32_t *unit_start;      // [V + 1] units per id, then their first index
  int32_t *part_start;      // [V + 1] partial rows per id, then first row
  float *partial;           // [2 ceil(T K / DIV_UNIT), d] partial dW rows
  int32_t *bsum;            // [div_scan_blocks] tile sums of the scans
};
// Tiles of the exclusive scans of the divergence path (RADIX * blocks and
// V + 1 counts) and the block-sum entries a scan of n values needs.
constexpr int SCAN_TILE = 4096;
inline int64_t div_scan_blocks(int64_t n) { return (n + SCAN_TILE - 1) / SCAN_TILE; }
int radix_passes(int64_t V);
hipError_t launch_div(const DivArgs &a, hipStream_t s);

hipError_t launch_tk_sample(const TkArgs &a, hipStream_t s);
hipError_t launch_tk_theta(const TkArgs &a, hipStream_t s);
hipError_t launch_tk_filter(const TkArgs &a, hipStream_t s);
hipError_t launch_tk_select(const TkArgs &a, hipStream_t s);
hipError_t launch_tk_stream(const TkArgs &a, bool bf16, hipStream_t s);

}  // namespace kd
