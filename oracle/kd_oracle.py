"""Plain fp64 CPU oracle for the fused, chunked top-K KL distillation loss.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
executes this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code with the
HIP library (``top_kl_loss_amd``); both receive their inputs from the seeded
generators in ``synth/``, which hold none of the method's arithmetic.

What is computed, and where the pages say so
--------------------------------------------
Sources are the five web pages about the Multiverse Computing post
"Efficient Knowledge Distillation for LLMs: Offline Top-K Logits and a Fused
Chunked KL Loss"; each function cites the page title and section it follows.

* The teacher is run once and only its top-100 logits per token position are
  kept ("Making Knowledge Distillation Cheap Enough to Run at Scale",
  aipuls.nl summary, section "Summary", second paragraph).  The cache is the
  input ``topk_idx[T,K]`` (int32) / ``topk_logit[T,K]`` (fp32).
* The loss is a KL divergence between the teacher distribution and the
  student's output distribution, computed over successive slices of the
  sequence so that the dense sequence-by-vocabulary matrix never exists at
  once (same page and section; "Hugging Face and Multiverse Computing cut KD
  memory costs", agent-gateway.com, fourth and fifth paragraphs).
* The direction is forward KL, teacher as the target, student
  log-probabilities over the full vocabulary, summed over the vocabulary and
  averaged over the selected (valid) tokens (asibiont.com article, section
  "A Concrete Implementation Sketch").

Readings where the pages are silent (each is listed with its reason in the
design notes of the repository):

* R1  teacher distribution = softmax over the K cached logits at temperature
      tau (renormalised on the top-K support, no tail bucket);
* R2  student distribution = softmax over all V logits at temperature tau;
* R3  loss = tau^2 / N_valid * sum_t mask_t * KL_t, with N_valid = sum mask;
      N_valid = 0 gives loss 0 and zero gradients (never NaN);
* R4  mask: 1 = valid token, 0 = padding; ``mask=None`` means all valid;
* R5  logits are z = H W^T with no bias and no soft-cap;
* R6  the K ids of a row are distinct and lie in [0, V) (caller contract);
* R7  ``chunk`` counts token rows per slice; ``chunk >= T`` is the dense form.

Gradient (derived, not taken from the pages): with p = softmax(z/tau) and
q_scat[t, v] = sum_k q[t,k] [idx[t,k] == v],
    dL/dz[t,v] = (tau / N_valid) * mask_t * (p[t,v] - q_scat[t,v])
because sum_k q[t,k] = 1.  Then dH = G W and dW = G^T H.

Parity status: every function here is pinned by ``tests/test_oracle.py``
(finite differences, closed forms, library special cases, invariances);
the pages print no worked example or loss value, so no pin comes from a
printed number.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "teacher_entropy",
    "entropy_filter_mask",
    "topk_divergence",
    "teacher_distribution",
    "log_softmax_rows",
    "kd_topk_kl",
    "slice_terms",
    "row_lse",
    "rows_loss_and_dh",
    "dw_rows",
    "scattered_teacher",
    "loss_given_lse",
]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def log_softmax_rows(s):
    """Row-wise log-softmax of a 2-D fp64 array (max-shifted logsumexp).

    Student side of R2: the full-vocabulary log-probabilities (asibiont.com,
    "A Concrete Implementation Sketch": the student log-softmax over the
    vocabulary).  Returns (log_p, lse).
    """
    s = _f64(s)
    m = s.max(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(s - m).sum(axis=1))
    return s - lse[:, None], lse


def teacher_distribution(topk_logit, tau):
    """Teacher probabilities over the cached top-K support (reading R1).

    The cache holds the teacher's top-K logits per position (aipuls.nl,
    "Summary"); they are divided by tau and renormalised over the K slots.
    Returns (q, log_q), each [T, K] fp64.
    """
    u = _f64(topk_logit) / float(tau)
    log_q, _ = log_softmax_rows(u)
    return np.exp(log_q), log_q


def scattered_teacher(topk_idx, q, V):
    """Dense [rows, V] fp64 array with q[t,k] added at column topk_idx[t,k]."""
    rows, K = topk_idx.shape
    out = np.zeros((rows, V), dtype=np.float64)
    r = np.repeat(np.arange(rows), K)
    np.add.at(out, (r, np.asarray(topk_idx).reshape(-1)), q.reshape(-1))
    return out


def _mask_vector(mask, T):
    if mask is None:
        return np.ones(T, dtype=np.float64)
    return (np.asarray(mask).reshape(T) != 0).astype(np.float64)


def kd_topk_kl(H, W, topk_idx, topk_logit, mask, tau, chunk=None):
    """Loss and analytic gradients of the chunked top-K KL (readings R1-R7).

    Follows the pages' description of the fused, chunked loss: the token
    rows are processed in successive slices of ``chunk`` rows; for each slice
    the dense logits z = H_c W^T are formed (the sequence-by-vocabulary tensor
    of "Hugging Face and Multiverse Computing cut KD memory costs",
    agent-gateway.com, fourth paragraph, restricted to one slice), the
    student log-softmax is taken over the whole vocabulary, and the forward
    KL against the teacher's top-K distribution is accumulated together with
    its gradient before the slice is discarded (aipuls.nl, "Summary").

    Inputs are upcast exactly to fp64 (bf16 inputs arrive as their exact
    fp32 values).  Returns a dict with fp64 ``loss`` (scalar), ``row_loss``
    [T] (mask_t * KL_t, before the tau^2/N scaling), ``dH`` [T,d], ``dW``
    [V,d], ``lse`` [T] (logsumexp of z/tau) and ``n_valid``.
    """
    H = _f64(H)
    W = _f64(W)
    topk_idx = np.asarray(topk_idx, dtype=np.int64)
    T, d = H.shape
    V = W.shape[0]
    K = topk_idx.shape[1]
    assert W.shape[1] == d and topk_idx.shape == (T, K)
    assert topk_logit.shape == (T, K)
    tau = float(tau)
    m = _mask_vector(mask, T)
    n_valid = float(m.sum())
    # R3: loss scale tau^2/N (and gradient scale tau/N, in slice_terms);
    # N = 0 gives zeros.
    loss_scale = tau * tau / n_valid if n_valid > 0 else 0.0
    chunk = T if chunk is None else max(1, min(int(chunk), T))

    row_loss = np.zeros(T)
    lse_all = np.zeros(T)
    dH = np.zeros((T, d))
    dW = np.zeros((V, d))
    for c0 in range(0, T, chunk):
        c1 = min(T, c0 + chunk)
        rl, lse, dH[c0:c1], dW_part = slice_terms(
            H[c0:c1], W, topk_idx[c0:c1], topk_logit[c0:c1],
            m[c0:c1], tau, n_valid)
        row_loss[c0:c1] = rl
        lse_all[c0:c1] = lse
        dW += dW_part
    loss = loss_scale * row_loss.sum()
    return {
        "loss": loss,
        "row_loss": row_loss,
        "dH": dH,
        "dW": dW,
        "lse": lse_all,
        "n_valid": n_valid,
    }


def slice_terms(H_rows, W, idx_rows, logit_rows, mask_rows, tau, n_valid,
                want_dw=True):
    """One slice of the chunked loss (the body of ``kd_topk_kl``'s loop).

    For the token rows given, with the whole batch's valid-token count
    ``n_valid``: the dense logits z = H_rows W^T of the slice, the student
    log-softmax over the vocabulary, the forward KL against the teacher's
    top-K distribution, and the logit gradient G = tau/N mask (p - q_scat)
    with its two products.  Returns (row_loss = mask*KL [R], lse [R] of z/tau,
    dH rows G W [R, d], the slice's dW contribution G^T H_rows [V, d], or
    None when ``want_dw`` is false), all fp64.  Slices of a batch are
    independent given n_valid, so a full-size batch can be evaluated slice by
    slice with the results summed.
    """
    H_rows = _f64(H_rows)
    W = _f64(W)
    tau = float(tau)
    R = H_rows.shape[0]
    V = W.shape[0]
    m = _mask_vector(mask_rows, R)
    grad_scale = tau / n_valid if n_valid > 0 else 0.0
    q, log_q = teacher_distribution(logit_rows, tau)       # R1
    ids = np.asarray(idx_rows, dtype=np.int64)
    z = H_rows @ W.T                                       # dense slice [R, V]
    log_p, lse = log_softmax_rows(z / tau)                 # R2
    log_p_at = log_p[np.arange(R)[:, None], ids]           # [R, K]
    # forward KL(q || p) on the teacher's support, one value per row
    kl = (q * (log_q - log_p_at)).sum(axis=1)
    # dL/dz = tau/N * mask * (p - q_scat)
    G = np.exp(log_p) - scattered_teacher(ids, q, V)
    G *= (grad_scale * m)[:, None]
    return m * kl, lse, G @ W, (G.T @ H_rows if want_dw else None)


def row_lse(H_rows, W, tau, rows_per_block=256):
    """logsumexp_v(z[t,v]/tau) for the given rows only (reading R2).

    The same student normaliser as ``kd_topk_kl``, evaluated row block by
    row block so that full-size inputs fit in host memory.
    """
    H_rows = _f64(H_rows)
    W = _f64(W)
    out = np.empty(H_rows.shape[0])
    for r0 in range(0, H_rows.shape[0], rows_per_block):
        z = H_rows[r0:r0 + rows_per_block] @ W.T
        _, lse = log_softmax_rows(z / float(tau))
        out[r0:r0 + rows_per_block] = lse
    return out


def rows_loss_and_dh(H_rows, W, idx_rows, logit_rows, mask_rows, tau, n_valid):
    """Per-row KL and dH rows for a sample of token rows.

    A row's KL and its dH row depend only on that row and on N_valid (a
    count of the mask), so sampled rows of a full-size problem can be
    checked one by one.  Returns (row_loss [R] = mask*KL, dH [R,d]).
    """
    rl, _, dH_rows, _ = slice_terms(H_rows, W, idx_rows, logit_rows, mask_rows,
                                    tau, n_valid, want_dw=False)
    return rl, dH_rows


def dw_rows(H, W, topk_idx, topk_logit, mask, tau, lse, v_rows):
    """Selected rows of dW = G^T H, given every token's student lse.

    dW[v] = sum_t G[t,v] H[t] needs column v of G for all T tokens, which
    needs lse_t of every row (from ``row_lse``) but only the logits z[:, v]
    of the selected vocabulary rows.  Returns dW[v_rows] [len(v_rows), d].
    """
    H = _f64(H)
    tau = float(tau)
    T = H.shape[0]
    v_rows = np.asarray(v_rows, dtype=np.int64)
    m = _mask_vector(mask, T)
    n_valid = m.sum()
    grad_scale = tau / n_valid if n_valid > 0 else 0.0
    q, _ = teacher_distribution(topk_logit, tau)
    Wv = _f64(W)[v_rows]                         # [R, d]
    z = H @ Wv.T                                 # [T, R]
    p = np.exp(z / tau - _f64(lse)[:, None])
    ids = np.asarray(topk_idx, dtype=np.int64)
    qs = np.zeros_like(p)
    for j, v in enumerate(v_rows):
        hit = ids == v                           # [T, K]
        qs[:, j] = (q * hit).sum(axis=1)
    G = (p - qs) * (grad_scale * m)[:, None]     # [T, R]
    return G.T @ H


def loss_given_lse(H, W, topk_idx, topk_logit, mask, tau, lse):
    """Total loss and per-row KL from every row's student logsumexp.

    KL_t = sum_k q[t,k] (log q[t,k] - (z[t, idx[t,k]]/tau - lse_t)) needs the
    full-vocabulary normaliser (from ``row_lse``) and only the K student
    logits at the teacher's ids, so a full-size loss can be evaluated without
    the dense logits.  Same readings R1-R6 as ``kd_topk_kl``.
    Returns (loss, row_loss = mask * KL).
    """
    H = _f64(H)
    tau = float(tau)
    T = H.shape[0]
    m = _mask_vector(mask, T)
    n_valid = m.sum()
    q, log_q = teacher_distribution(topk_logit, tau)
    ids = np.asarray(topk_idx, dtype=np.int64)
    z_at = np.empty(ids.shape)
    for r0 in range(0, T, 1024):
        Wg = _f64(W)[ids[r0:r0 + 1024]]                  # [R, K, d]
        z_at[r0:r0 + 1024] = np.einsum("rd,rkd->rk", H[r0:r0 + 1024], Wg)
    log_p_at = z_at / tau - _f64(lse)[:, None]
    kl = (q * (log_q - log_p_at)).sum(axis=1)
    row_loss = m * kl
    loss = tau * tau * row_loss.sum() / n_valid if n_valid > 0 else 0.0
    return loss, row_loss


def teacher_entropy(topk_logit, tau):
    """Entropy -sum_k q_k log q_k of the teacher distribution the loss uses
    (R1: softmax of the K cached logits at temperature tau), fp64.  The
    asibiont.com article, section "Distillation Token Filtering", scores each
    token by the entropy of its teacher distribution; its implementation
    sketch adds 1e-9 inside the log, which this exact form leaves out (q > 0
    for finite logits)."""
    lq, _ = log_softmax_rows(_f64(topk_logit) / float(tau))
    return -(np.exp(lq) * lq).sum(axis=1)


def entropy_filter_mask(topk_logit, mask, tau, mode, param):
    """Token mask of the entropy filter (asibiont.com article, sections
    "Distillation Token Filtering" and "A Concrete Implementation Sketch"):

    * mode "above": a token is kept when it is valid and its teacher entropy
      exceeds param (the sketch combines the padding mask with a strict
      entropy threshold);
    * mode "top_fraction": among the N valid tokens, the n = floor(param*N
      + 1/2) with the highest entropy, equal entropies by lower index (the
      section's alternative of retaining a set share of the batch's most
      uncertain tokens).
    """
    ent = teacher_entropy(topk_logit, tau)
    T = ent.shape[0]
    valid = _mask_vector(mask, T) > 0
    if mode == "above":
        return (valid & (ent > float(param))).astype(np.uint8)
    if mode != "top_fraction":
        raise ValueError(mode)
    n_valid = int(valid.sum())
    n_keep = int(np.floor(float(np.float32(param)) * n_valid + 0.5))
    order = np.lexsort((np.arange(T), -ent))
    kept = [t for t in order if valid[t]][:n_keep]
    out = np.zeros(T, dtype=np.uint8)
    out[kept] = 1
    return out


def topk_divergence(H, W, topk_idx, topk_logit, mask, tau, kind):
    """Reverse KL or Jensen-Shannon divergence over the teacher's top-K
    support, with analytic gradients (readings D1-D3).

    The asibiont.com article (section "A Concrete Implementation Sketch")
    distils with a KL divergence between the softened distributions; the
    question the pages leave open is whether the cached top-K keeps enough
    signal ("Hugging Face and Multiverse Computing cut KD memory costs",
    agent-gateway.com, closing paragraph).  Over the same cache:

    * D1  both distributions live on the row's K cached ids: the teacher
          q = softmax(topk_logit / tau) (as R1) and the student restricted to
          those ids and renormalised, p^ = softmax(z[t, idx] / tau);
    * D2  kind "reverse_kl": D_t = sum_k p^_k (log p^_k - log q_k);
          kind "jsd": with m = (p^ + q) / 2,
          D_t = 1/2 sum_k q_k log(q_k / m_k) + 1/2 sum_k p^_k log(p^_k / m_k);
    * D3  loss = tau^2 / N * sum_t mask_t D_t as R3 (N = 0: zeros).

    Gradient (derived): with u = z[t, idx] / tau and a_k = dD/dp^_k,
    a = log(p^/q) + 1 (reverse KL) or a = 1/2 log(p^/m) (JSD), the softmax
    Jacobian gives dD/du_k = p^_k (a_k - sum_j p^_j a_j); the loss gradient
    tau / N * mask_t * that lands on the K ids only.  Then dH = G W and
    dW = G^T H with G the dense [T, V] gradient (zero off the ids).
    Inputs are upcast exactly to fp64.  Returns loss, row_loss (mask * D_t),
    dH, dW and n_valid.
    """
    if kind not in ("reverse_kl", "jsd"):
        raise ValueError(kind)
    H = _f64(H)
    W = _f64(W)
    ids = np.asarray(topk_idx, dtype=np.int64)
    T, d = H.shape
    V = W.shape[0]
    tau = float(tau)
    m = _mask_vector(mask, T)
    n_valid = float(m.sum())
    q, log_q = teacher_distribution(topk_logit, tau)              # D1, teacher
    z = H @ W.T
    u = np.take_along_axis(z, ids, axis=1) / tau
    log_p, _ = log_softmax_rows(u)                               # D1, student
    p = np.exp(log_p)
    if kind == "reverse_kl":
        div = (p * (log_p - log_q)).sum(axis=1)
        a = log_p - log_q + 1.0
    else:
        log_mid = np.log(0.5 * (p + q))
        div = 0.5 * (q * (log_q - log_mid)).sum(axis=1) + \
            0.5 * (p * (log_p - log_mid)).sum(axis=1)
        a = 0.5 * (log_p - log_mid)
    du = p * (a - (p * a).sum(axis=1, keepdims=True))
    grad_scale = tau / n_valid if n_valid > 0 else 0.0
    loss_scale = tau * tau / n_valid if n_valid > 0 else 0.0
    Gk = du * (grad_scale * m)[:, None]                          # dL/dz at the ids
    G = np.zeros((T, V))
    np.add.at(G, (np.repeat(np.arange(T), ids.shape[1]), ids.reshape(-1)),
              Gk.reshape(-1))
    row_loss = m * div
    return {
        "loss": loss_scale * row_loss.sum(),
        "row_loss": row_loss,
        "dH": G @ W,
        "dW": G.T @ H,
        "n_valid": n_valid,
    }
