"""Helpers for the GPU tests: move synthetic inputs to the device, call the
HIP library through the binding, and compare with the oracle."""
import numpy as np

import top_kl_loss_amd as kd

# Acceptance bars (loss relative error; gradient max relative error per
# tensor = max|g - o| / max|o|; gradient cosine).
TOL = {
    "f32": dict(loss=1e-5, maxrel=1e-4, cos=None),
    "bf16": dict(loss=1e-3, maxrel=2e-2, cos=0.999),
}


def to_device(x, device="cuda"):
    import torch
    if x.dtype == "bf16":
        H = torch.from_numpy(x.H_bits.view(np.int16)).view(torch.bfloat16)
        W = torch.from_numpy(x.W_bits.view(np.int16)).view(torch.bfloat16)
    else:
        H = torch.from_numpy(x.H)
        W = torch.from_numpy(x.W)
    out = dict(H=H.to(device), W=W.to(device),
               topk_idx=torch.from_numpy(x.topk_idx).to(device),
               topk_logit=torch.from_numpy(x.topk_logit).to(device),
               mask=None if x.mask is None else torch.from_numpy(x.mask).to(device))
    return out


def run(dev_inputs, tau, chunk, flags=0, dW=None, sync=True):
    import torch
    loss, rl, dH, dW = kd.kd_topk_kl_fwd_bwd(
        dev_inputs["H"], dev_inputs["W"], dev_inputs["topk_idx"],
        dev_inputs["topk_logit"], dev_inputs["mask"], tau, chunk, flags, dW=dW)
    if sync:
        torch.cuda.synchronize()
    return loss, rl, dH, dW


def to_np(t):
    return t.detach().cpu().numpy().astype(np.float64)


def maxrel(g, o):
    o = np.asarray(o, dtype=np.float64)
    den = np.abs(o).max()
    return float(np.abs(np.asarray(g, np.float64) - o).max() / (den if den > 0 else 1.0))


def cosine(g, o):
    g = np.asarray(g, np.float64).ravel(); o = np.asarray(o, np.float64).ravel()
    ng, no = np.linalg.norm(g), np.linalg.norm(o)
    if ng == 0 and no == 0:
        return 1.0
    return float(g @ o / (ng * no))


def assert_grad_close(g, o, dtype, what):
    tol = TOL[dtype]
    mr = maxrel(g, o)
    assert mr <= tol["maxrel"], f"{what}: max rel {mr:.3e} > {tol['maxrel']}"
    if tol["cos"] is not None:
        c = cosine(g, o)
        assert c >= tol["cos"], f"{what}: cosine {c:.6f} < {tol['cos']}"


def assert_rows_kl(g, o, where):
    """Every row's KL within 1e-3 of its own value (padding rows exactly 0)."""
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    pad = o == 0.0
    assert np.all(g[pad] == 0.0), f"{where}: padding rows carry a loss"
    rel = np.abs(g[~pad] - o[~pad]) / np.abs(o[~pad])
    assert rel.size == 0 or rel.max() <= 1e-3, \
        f"{where}: row KL rel {rel.max():.2e} at row {int(np.argmax(rel))}"


def assert_loss_close(g, o, dtype):
    tol = TOL[dtype]["loss"]
    rel = abs(g - o) / max(abs(o), 1e-30)
    assert rel <= tol or (o == 0 and g == 0), f"loss {g} vs {o}: rel {rel:.3e}"


# ------------------------------------------------------ teacher top-K cache
# fp32 accumulation error of a logit, relative to sum_j |H[t,j] W[v,j]|
# (about 2^-15.6: generous for d up to a few thousand, blocked or sequential)
TOPK_REL_TOL = 2e-5


def check_topk(x, ids, vals, K, exact=False, rows=None):
    """Compare a teacher top-K cache (ids, vals: [len(rows), K]) with the
    fp64 oracle on rows `rows` (default all) of the problem x: ids and
    values exactly, or values within the fp32 rounding tolerance, the order,
    and the id set wherever values closer than the tolerance do not decide."""
    from oracle import teacher_topk as tko
    rows = np.arange(x.H.shape[0]) if rows is None else np.asarray(rows)
    Hs = x.H[rows]
    o_ids, o_vals = tko.teacher_topk_cache(Hs, x.W, K)
    if exact:
        assert np.array_equal(ids, o_ids), "ids differ from the oracle"
        assert np.array_equal(vals, o_vals), "logits differ from the oracle"
        return
    z = tko.teacher_logits(Hs, x.W)
    absz = np.abs(Hs.astype(np.float64)) @ np.abs(x.W.astype(np.float64)).T
    V = z.shape[1]
    for t in range(len(rows)):
        tol = TOPK_REL_TOL * absz[t].max() + 1e-30
        row = ids[t]
        where = f"row {int(rows[t])}"
        assert len(set(row.tolist())) == K and row.min() >= 0 and row.max() < V
        # values are the row's logits at the returned ids
        assert np.abs(vals[t] - z[t, row]).max() <= tol, f"{where}: logit error"
        # order: logit descending, equal logits by id ascending
        dv = np.diff(vals[t])
        assert np.all(dv <= 0), f"{where}: not sorted"
        assert np.all(np.diff(row)[dv == 0] > 0), f"{where}: tie order"
        # the sorted top-K logits agree with the oracle's
        assert np.abs(vals[t] - o_vals[t]).max() <= 2 * tol, f"{where}: top-K values"
        if K < V:
            # no entry left out is better than an entry kept, beyond rounding
            out = np.ones(V, dtype=bool)
            out[row] = False
            assert z[t, row].min() >= z[t, out].max() - 2 * tol, f"{where}: set"
            # entries clearly inside the oracle's top-K are all returned
            zk1 = np.sort(z[t])[::-1][K]
            sure = o_ids[t][o_vals[t] > zk1 + 2 * tol]
            assert set(sure.tolist()) <= set(row.tolist()), f"{where}: missing ids"


# ---------------------------------------------- near-converged loss tolerance
U32 = 2.0 ** -24     # fp32 unit roundoff


def kl_rounding_floor_rows(x):
    """Per-row absolute KL error that fp32 arithmetic alone can cause, for
    the loss bars near KL = 0 (where a relative bar cannot hold).  Twice the
    sum of two first-order terms, plus 8 u:
      * the logits: an fp32 dot product over d terms is off by about
        sqrt(d) * u * max|z|, and KL_t moves by sum_v (p - q_scat) dz / tau
        to first order;
      * the log-probabilities: KL_t = sum_k q_k (log q_k - log p_k) is
        formed from values rounded to u * |log q_k| and u * |log p_k|;
      * the normaliser: log of a sum of exponentials (>= 1 after the shift
        by the maximum), each rounded relative to its size, is off by a few u
        in absolute terms however small KL_t is.
    Computed densely in fp64 from the inputs, for oracle-sized cases."""
    H = np.asarray(x.H, np.float64)
    W = np.asarray(x.W, np.float64)
    z = H @ W.T / x.tau
    zmax = np.abs(z).max(axis=1)
    z -= z.max(axis=1, keepdims=True)
    logp = z - np.log(np.exp(z).sum(axis=1, keepdims=True))
    p = np.exp(logp)
    u = np.asarray(x.topk_logit, np.float64) / x.tau
    u -= u.max(axis=1, keepdims=True)
    logq = u - np.log(np.exp(u).sum(axis=1, keepdims=True))
    q = np.exp(logq)
    qs = np.zeros_like(p)
    np.add.at(qs, (np.repeat(np.arange(x.T), x.K), x.topk_idx.reshape(-1)), q.reshape(-1))
    logp_at = np.take_along_axis(logp, x.topk_idx.astype(np.int64), 1)
    logits = np.abs(p - qs).sum(axis=1) * np.sqrt(x.d) * U32 * zmax
    logs = U32 * (q * (np.abs(logq) + np.abs(logp_at))).sum(axis=1)
    m = np.ones(x.T) if x.mask is None else (x.mask != 0).astype(np.float64)
    return m * (2.0 * (logits + logs) + 8.0 * U32)


def loss_rounding_floor(x, floor_rows):
    """The loss's share of the per-row floors: tau^2 / N * sum_t floor_t."""
    n = x.n_valid
    return x.tau ** 2 * float(floor_rows.sum()) / n if n > 0 else 0.0


def fp32_logit_grad_floor(x, ref):
    """(dH, dW) max relative errors that fp32 logits alone cause near KL = 0:
    the gradients evaluated in fp64 from z = H W^T rounded by a float32
    matrix product (numpy), against the oracle's.  Near the minimum the
    logit gradient is a small difference p - q_scat, and an fp32 logit error
    dz moves p by p dz / tau, so a relative bar meets this floor; the fp32
    near-converged tests add twice it to the 1e-4 bar."""
    z = (np.asarray(x.H, np.float32) @ np.asarray(x.W, np.float32).T).astype(np.float64)
    s = z / x.tau
    s -= s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)
    u = np.asarray(x.topk_logit, np.float64) / x.tau
    q = np.exp(u - u.max(axis=1, keepdims=True))
    q /= q.sum(axis=1, keepdims=True)
    g = p
    np.subtract.at(g, (np.repeat(np.arange(x.T), x.K), x.topk_idx.reshape(-1)), q.reshape(-1))
    m = np.ones(x.T) if x.mask is None else (x.mask != 0).astype(np.float64)
    g *= (x.tau / max(m.sum(), 1.0) * m)[:, None]
    dH = g @ np.asarray(x.W, np.float64)
    dW = g.T @ np.asarray(x.H, np.float64)
    return maxrel(dH, ref["dH"]), maxrel(dW, ref["dW"])
