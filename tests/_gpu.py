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


def assert_loss_close(g, o, dtype):
    tol = TOL[dtype]["loss"]
    rel = abs(g - o) / max(abs(o), 1e-30)
    assert rel <= tol or (o == 0 and g == 0), f"loss {g} vs {o}: rel {rel:.3e}"
