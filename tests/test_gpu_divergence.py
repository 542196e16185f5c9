"""GPU parity of the reverse KL and Jensen-Shannon divergences over the
teacher's top-K support (kd_topk_div_fwd_bwd) against the fp64 oracle
(oracle.topk_divergence), at the acceptance bars of the forward KL: fp32
inputs loss rel <= 1e-5 and gradient max rel <= 1e-4; bf16 inputs loss rel
<= 1e-3, gradient cosine >= 0.999 and max rel <= 2e-2."""
import sys

import numpy as np
import pytest

import synth
import top_kl_loss_amd as kd
from oracle import kd_oracle as orc
from tests import _gpu as G

pytestmark = pytest.mark.gpu
KINDS = ("reverse_kl", "jsd")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _run(kind, dev, tau, flags=0, dW=None):
    import torch
    out = kd.kd_topk_div_fwd_bwd(kind, dev["H"], dev["W"], dev["topk_idx"],
                                 dev["topk_logit"], dev["mask"], tau, flags, dW=dW)
    torch.cuda.synchronize()
    return out


def _check(x, kind, dW0=None):
    _say(f"divergence {kind}: {x.name} T={x.T} d={x.d} V={x.V} K={x.K} "
         f"{x.dtype} tau={x.tau}")
    dev = G.to_device(x)
    import torch
    dWin = None
    flags = 0
    if dW0 is not None:
        dWin = torch.from_numpy(dW0).cuda()
        flags = kd.KD_FLAG_ACCUMULATE_DW
    loss, rl, dH, dW = _run(kind, dev, x.tau, flags, dWin)
    ref = orc.topk_divergence(x.H, x.W, x.topk_idx, x.topk_logit, x.mask, x.tau, kind)
    G.assert_loss_close(float(loss.item()), ref["loss"], x.dtype)
    G.assert_grad_close(G.to_np(rl), ref["row_loss"], x.dtype, "row_loss")
    G.assert_grad_close(G.to_np(dH), ref["dH"], x.dtype, "dH")
    want_dW = ref["dW"] if dW0 is None else ref["dW"] + dW0
    G.assert_grad_close(G.to_np(dW), want_dW, x.dtype, "dW")
    if x.mask is not None:
        assert np.all(G.to_np(dH)[x.mask == 0] == 0.0)
        assert np.all(G.to_np(rl)[x.mask == 0] == 0.0)
    return dev, (loss, rl, dH, dW)


@pytest.mark.parametrize("kind", KINDS)
def test_tiny_fp32(kind):
    _check(synth.workload("tiny"), kind)


@pytest.mark.parametrize("kind", KINDS)
def test_bf16_teacher_cache_padding(kind):
    _check(synth.make_case("div_bf16", case=110, T=500, d=256, V=6000, K=50,
                           dtype="bf16", tau=1.5, mask_frac=0.1,
                           cache="teacher"), kind)


@pytest.mark.parametrize("kind", KINDS)
def test_ids_shared_by_many_tokens_and_accumulate(kind):
    # V = 500 ids over 3000 tokens x K = 20: id 7 is in every row (3000 pairs,
    # three reduction units), the others ~115 pairs each; dW accumulated onto
    # a non-zero start; fp32 and a ragged hidden size (d = 72)
    x = synth.make_case("div_shared", case=111, T=3000, d=72, V=500, K=20,
                        dtype="f32", tau=0.8, mask_frac=0.05)
    rng = np.random.default_rng(7)
    idx = np.stack([np.concatenate(([7], rng.permutation(np.delete(np.arange(500), 7))[:19]))
                    for _ in range(x.T)]).astype(np.int32)
    x.topk_idx = idx
    dW0 = rng.standard_normal((x.V, x.d)).astype(np.float32)
    _check(x, kind, dW0=dW0)


@pytest.mark.parametrize("kind", KINDS)
def test_repeatable_and_no_valid_tokens(kind):
    import torch
    x = synth.make_case("div_rep", case=112, T=700, d=128, V=3001, K=37,
                        dtype="bf16", tau=1.0, cache="teacher")
    dev, first = _check(x, kind)
    again = _run(kind, dev, x.tau)
    for a, b in zip(first, again):
        assert torch.equal(a, b)
    dev["mask"] = torch.zeros(x.T, dtype=torch.uint8, device="cuda")
    loss, rl, dH, dW = _run(kind, dev, x.tau)
    assert float(loss.item()) == 0.0
    assert float(dH.abs().max()) == 0.0 and float(dW.abs().max()) == 0.0


def test_autograd_divergences():
    import torch
    from top_kl_loss_amd.autograd import topk_kl_loss
    x = synth.make_case("div_ag", case=113, T=300, d=192, V=2000, K=30,
                        dtype="bf16", tau=1.2, mask_frac=0.1, cache="teacher")
    dev = G.to_device(x)
    for kind in KINDS:
        H = dev["H"].clone().requires_grad_(True)
        W = dev["W"].clone().requires_grad_(True)
        loss = topk_kl_loss(H, W, dev["topk_idx"], dev["topk_logit"], dev["mask"],
                            x.tau, divergence=kind)
        (2.0 * loss).backward()
        ref = orc.topk_divergence(x.H, x.W, x.topk_idx, x.topk_logit, x.mask, x.tau, kind)
        G.assert_loss_close(float(loss.item()), ref["loss"], x.dtype)
        G.assert_grad_close(G.to_np(H.grad.float()), 2.0 * ref["dH"], x.dtype, "H.grad")
        G.assert_grad_close(G.to_np(W.grad.float()), 2.0 * ref["dW"], x.dtype, "W.grad")


@pytest.mark.parametrize("kind", KINDS)
def test_t4k_full_size(kind):
    # the t4k workload (T = 4096, d = 2880, V = 201088, K = 100, bf16): every
    # row's divergence, all of dH and all of dW against the oracle (dense
    # fp64, ~30 s of host time)
    import torch
    x = synth.workload("t4k", teacher_device="cuda")
    _say(f"divergence {kind}: t4k full size")
    dev = G.to_device(x)
    loss, rl, dH, dW = _run(kind, dev, x.tau)
    loss, rl, dH, dW = float(loss.item()), G.to_np(rl), dH.cpu().numpy(), dW.cpu().numpy()
    del dev
    torch.cuda.empty_cache()
    ref = orc.topk_divergence(x.H, x.W, x.topk_idx, x.topk_logit, x.mask, x.tau, kind)
    G.assert_loss_close(loss, ref["loss"], x.dtype)
    G.assert_grad_close(rl, ref["row_loss"], x.dtype, "row_loss")
    G.assert_grad_close(dH, ref["dH"], x.dtype, "dH")
    G.assert_grad_close(dW, ref["dW"], x.dtype, "dW")
    _say(f"  loss {loss:.7f} oracle {ref['loss']:.7f}")
