"""GPU parity of the entropy token filter (kd_entropy_filter) against the
fp64 oracle, and of the loss on the filtered tokens.  Entropies are fp32 on
the GPU, so masks are compared exactly except for tokens whose entropy lies
within the rounding tolerance of the decision boundary."""
import sys

import numpy as np
import pytest

import synth
import top_kl_loss_amd as kd
from oracle import kd_oracle as orc
from tests import _gpu as G

pytestmark = pytest.mark.gpu

ENT_TOL = 2e-5   # absolute, entropies are O(log K)


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _logits(case, T, K, scale):
    # teacher logits with a wide spread of entropies: per-row temperature
    rng = np.random.default_rng(1000 * case + 7)
    base = -np.sort(-rng.standard_normal((T, K)), axis=1)
    spread = np.exp(rng.uniform(-1.5, 2.5, size=(T, 1)))
    return np.ascontiguousarray(base * spread * scale, dtype=np.float32)


def _run(lg, mask, tau, mode, param):
    import torch
    tl = torch.from_numpy(lg).cuda()
    tm = None if mask is None else torch.from_numpy(mask).cuda()
    out, ent = kd.kd_entropy_filter(tl, tm, tau, mode, param)
    return out.cpu().numpy(), ent.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("tau", [1.0, 2.0])
def test_entropies_and_threshold_mask(tau):
    T, K = 5000, 100
    lg = _logits(70, T, K, 1.0)
    mask = (np.random.default_rng(71).random(T) > 0.1).astype(np.uint8)
    o_ent = orc.teacher_entropy(lg, tau)
    thr = float(np.median(o_ent))
    _say(f"entropy filter above: T={T} K={K} tau={tau} thr={thr:.4f}")
    out, ent = _run(lg, mask, tau, "above", thr)
    assert np.abs(ent - o_ent).max() <= ENT_TOL
    want = orc.entropy_filter_mask(lg, mask, tau, "above", thr)
    clear = np.abs(o_ent - thr) > ENT_TOL
    assert np.array_equal(out[clear], want[clear])
    assert np.all(out[mask == 0] == 0)


@pytest.mark.parametrize("frac", [0.0, 0.3, 0.75, 1.0])
def test_top_entropy_fraction(frac):
    T, K = 4099, 64
    lg = _logits(72, T, K, 1.0)
    mask = (np.random.default_rng(73).random(T) > 0.15).astype(np.uint8)
    _say(f"entropy filter top_fraction={frac}: T={T} K={K}")
    out, ent = _run(lg, mask, 1.0, "top_fraction", frac)
    want = orc.entropy_filter_mask(lg, mask, 1.0, "top_fraction", frac)
    n_keep = int(want.sum())
    assert int(out.sum()) == n_keep                      # the count is exact
    assert np.all(out[mask == 0] == 0)
    o_ent = orc.teacher_entropy(lg, 1.0)
    kept, dropped = out == 1, (out == 0) & (mask == 1)
    if kept.any() and dropped.any():
        # no dropped token has a higher entropy than a kept one, beyond
        # rounding; tokens clearly inside the oracle's kept set are kept
        assert o_ent[kept].min() >= o_ent[dropped].max() - 2 * ENT_TOL
        bound = np.sort(o_ent[want == 1])[0]
        sure = (want == 1) & (o_ent > bound + 2 * ENT_TOL)
        assert np.all(out[sure] == 1)


def test_top_fraction_ties_go_to_lower_index_and_empty_mask():
    # equal logits in every row: equal entropies, kept by index
    T, K = 1000, 16
    lg = np.zeros((T, K), dtype=np.float32)
    mask = np.ones(T, dtype=np.uint8)
    mask[::3] = 0
    out, _ = _run(lg, mask, 1.0, "top_fraction", 0.4)
    want = orc.entropy_filter_mask(lg, mask, 1.0, "top_fraction", 0.4)
    assert np.array_equal(out, want)
    none, _ = _run(lg, np.zeros(T, np.uint8), 1.0, "top_fraction", 0.5)
    assert none.sum() == 0


def test_loss_on_the_filtered_tokens_matches_the_oracle():
    # the filter's mask fed to the loss: equals the oracle's loss and
    # gradients with the oracle's mask (threshold away from every entropy)
    import torch
    x = synth.make_case("filt", case=74, T=600, d=192, V=3000, K=50,
                        dtype="bf16", tau=1.5, mask_frac=0.05, chunk=256)
    o_ent = orc.teacher_entropy(x.topk_logit, x.tau)
    s = np.sort(o_ent)
    gaps = np.diff(s)
    i = int(np.argmax(gaps[len(s) // 4: 3 * len(s) // 4])) + len(s) // 4
    thr = float((s[i] + s[i + 1]) / 2)
    _say(f"filtered loss: thr={thr:.4f} gap={gaps[i]:.2e}")
    dev = G.to_device(x)
    fmask, _ = kd.kd_entropy_filter(dev["topk_logit"], dev["mask"], x.tau, "above", thr)
    want_mask = orc.entropy_filter_mask(x.topk_logit, x.mask, x.tau, "above", thr)
    assert np.array_equal(fmask.cpu().numpy(), want_mask)
    dev["mask"] = fmask
    loss, rl, dH, dW = G.run(dev, x.tau, x.chunk)
    ref = orc.kd_topk_kl(x.H, x.W, x.topk_idx, x.topk_logit, want_mask, x.tau)
    G.assert_loss_close(float(loss.item()), ref["loss"], x.dtype)
    G.assert_grad_close(G.to_np(dH), ref["dH"], x.dtype, "dH")
    G.assert_grad_close(G.to_np(dW), ref["dW"], x.dtype, "dW")
    del torch


def test_autograd_loss_with_an_entropy_filter():
    import torch
    from top_kl_loss_amd.autograd import topk_kl_loss
    x = synth.make_case("filt_ag", case=75, T=300, d=128, V=2000, K=20,
                        dtype="f32", tau=1.0, chunk=128)
    dev = G.to_device(x)
    H = dev["H"].clone().requires_grad_(True)
    W = dev["W"].clone().requires_grad_(True)
    loss = topk_kl_loss(H, W, dev["topk_idx"], dev["topk_logit"], None, 1.0,
                        128, entropy_filter=("top_fraction", 0.6))
    loss.backward()
    want_mask = orc.entropy_filter_mask(x.topk_logit, None, 1.0, "top_fraction", 0.6)
    assert int(want_mask.sum()) == 180
    ref = orc.kd_topk_kl(x.H, x.W, x.topk_idx, x.topk_logit, want_mask, 1.0)
    G.assert_loss_close(float(loss.item()), ref["loss"], "f32")
    G.assert_grad_close(G.to_np(H.grad), ref["dH"], "f32", "H.grad")
    G.assert_grad_close(G.to_np(W.grad), ref["dW"], "f32", "W.grad")


def test_top_fraction_with_structured_entropies():
    # every 16th token (offset 8) gets the maximal entropy (equal logits):
    # a strongly structured entropy sequence; the selection is still exact
    T, K = 4096, 16
    rng = np.random.default_rng(76)
    lg = np.ascontiguousarray(rng.standard_normal((T, K)) * 3, dtype=np.float32)
    lg[8::16] = 0.0
    out, ent = _run(lg, None, 1.0, "top_fraction", 0.5)
    want = orc.entropy_filter_mask(lg, None, 1.0, "top_fraction", 0.5)
    assert int(out.sum()) == int(want.sum()) == 2048
    assert np.all(out[8::16] == 1)          # the maximal-entropy tokens
    o_ent = orc.teacher_entropy(lg, 1.0)
    assert o_ent[out == 1].min() >= o_ent[out == 0].max() - 2 * ENT_TOL
