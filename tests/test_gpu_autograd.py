"""GPU tests of the split entry points (kd_topk_kl_fwd, kd_topk_kl_bwd,
kd_grad_cast) and of the autograd integration, against the fp64 oracle and
against the fused entry point on identical seeded inputs."""
import sys

import numpy as np
import pytest

import synth
import top_kl_loss_amd as kd
from oracle import kd_oracle as orc
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _cases():
    return [
        synth.make_case("ag_f32", case=60, T=300, d=200, V=1000, K=17,
                        dtype="f32", tau=1.7, mask_frac=0.1, chunk=128),
        synth.make_case("ag_bf16", case=61, T=333, d=192, V=3001, K=23,
                        dtype="bf16", tau=2.0, mask_frac=0.1, chunk=128),
    ]


@pytest.mark.parametrize("x", _cases(), ids=lambda x: x.name)
def test_forward_alone_matches_fused_and_oracle(x):
    import torch
    _say(f"fwd: {x.name}")
    dev = G.to_device(x)
    loss, rl, lse = kd.kd_topk_kl_fwd(dev["H"], dev["W"], dev["topk_idx"],
                                      dev["topk_logit"], dev["mask"], x.tau, x.chunk)
    loss2, rl2, _, _ = G.run(dev, x.tau, x.chunk)
    # same kernels up to the row reductions: bitwise equal
    assert torch.equal(loss, loss2) and torch.equal(rl, rl2)
    ref = orc.kd_topk_kl(x.H, x.W, x.topk_idx, x.topk_logit, x.mask, x.tau)
    G.assert_loss_close(float(loss.item()), ref["loss"], x.dtype)
    o_lse = orc.row_lse(x.H, x.W, x.tau)
    tol = 1e-5 if x.dtype == "f32" else 1e-3
    err = np.abs(G.to_np(lse) - o_lse).max() / np.abs(o_lse).max()
    assert err <= tol, f"lse max rel {err:.2e}"


@pytest.mark.parametrize("x", _cases(), ids=lambda x: x.name)
@pytest.mark.parametrize("g", [2.5, 0.0])
def test_backward_alone_scales_by_the_upstream_gradient(x, g):
    import torch
    _say(f"bwd: {x.name} grad_loss={g}")
    dev = G.to_device(x)
    gl = torch.tensor([g], dtype=torch.float32, device="cuda")
    dH, dW = kd.kd_topk_kl_bwd(dev["H"], dev["W"], dev["topk_idx"],
                               dev["topk_logit"], dev["mask"], x.tau, x.chunk,
                               grad_loss=gl)
    if g == 0.0:
        assert float(dH.abs().max()) == 0.0 and float(dW.abs().max()) == 0.0
        return
    _, _, fH, fW = G.run(dev, x.tau, x.chunk)
    # fp32: G is scaled before one fp32 rounding; bf16: G is stored in bf16
    # after the scaling, so the two differ by bf16 rounding of G
    tol = 1e-5 if x.dtype == "f32" else G.TOL["bf16"]["maxrel"]
    for name, a, b in (("dH", dH, fH), ("dW", dW, fW)):
        err = float((a - g * b).abs().max()) / (g * float(b.abs().max()))
        assert err <= tol, f"{name}: {err:.2e} from {g} x fused"
    ref = orc.kd_topk_kl(x.H, x.W, x.topk_idx, x.topk_logit, x.mask, x.tau)
    G.assert_grad_close(G.to_np(dH), g * ref["dH"], x.dtype, "dH")
    G.assert_grad_close(G.to_np(dW), g * ref["dW"], x.dtype, "dW")


def test_grad_cast_rounds_to_bf16_nearest_even():
    import torch
    src = torch.tensor([1.0, 1.00390625, 1.01171875, -3.0, 65504.0, 1e-3],
                       dtype=torch.float32, device="cuda")
    scale = torch.tensor([2.0], dtype=torch.float32, device="cuda")
    out = kd.kd_grad_cast(src, torch.bfloat16, scale)
    want = synth.f32_to_bf16_bits((src * 2).cpu().numpy())
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, want)
    same = kd.kd_grad_cast(src, torch.float32)
    assert torch.equal(same, src)


@pytest.mark.parametrize("recompute", [False, True])
@pytest.mark.parametrize("x", _cases(), ids=lambda x: x.name)
def test_autograd_gradients_match_the_oracle(x, recompute):
    import torch
    from top_kl_loss_amd.autograd import topk_kl_loss
    _say(f"autograd: {x.name} recompute={recompute}")
    dev = G.to_device(x)
    H = dev["H"].clone().requires_grad_(True)
    W = dev["W"].clone().requires_grad_(True)
    loss = topk_kl_loss(H, W, dev["topk_idx"], dev["topk_logit"], dev["mask"],
                        x.tau, x.chunk, recompute=recompute)
    (3.0 * loss).backward()
    assert H.grad.dtype == H.dtype and W.grad.dtype == W.dtype
    ref = orc.kd_topk_kl(x.H, x.W, x.topk_idx, x.topk_logit, x.mask, x.tau)
    G.assert_loss_close(float(loss.item()), ref["loss"], x.dtype)
    G.assert_grad_close(G.to_np(H.grad.float()), 3.0 * ref["dH"], x.dtype, "H.grad")
    G.assert_grad_close(G.to_np(W.grad.float()), 3.0 * ref["dW"], x.dtype, "W.grad")


@pytest.mark.parametrize("x", _cases(), ids=lambda x: x.name)
def test_loss_without_gradients_runs_the_forward_alone(x):
    # under torch.no_grad, or with inputs that need no gradient, the loss is
    # the forward entry point's (bitwise), carries no graph, and the call
    # allocates no gradient buffer (less than dW's size at its peak)
    import torch
    from top_kl_loss_amd.autograd import topk_kl_loss
    _say(f"no-grad loss: {x.name}")
    dev = G.to_device(x)
    want, _, _ = kd.kd_topk_kl_fwd(dev["H"], dev["W"], dev["topk_idx"],
                                   dev["topk_logit"], dev["mask"], x.tau, x.chunk)
    H = dev["H"].clone().requires_grad_(True)
    W = dev["W"].clone().requires_grad_(True)
    torch.cuda.synchronize()
    for ctx, h, w in ((torch.no_grad(), H, W), (torch.enable_grad(), dev["H"], dev["W"])):
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        with ctx:
            loss = topk_kl_loss(h, w, dev["topk_idx"], dev["topk_logit"], dev["mask"],
                                x.tau, x.chunk)
        torch.cuda.synchronize()
        assert loss.dim() == 0 and not loss.requires_grad and loss.grad_fn is None
        assert torch.equal(loss.reshape(1), want)
        assert torch.cuda.max_memory_allocated() - base < x.V * x.d * 4


def test_autograd_through_a_student_head_and_a_training_step():
    # H = X A (a projection in front of the loss): the gradient reaches A by
    # the chain rule, and a few SGD steps on (A, W) lower the loss.
    import torch
    from top_kl_loss_amd.autograd import TopKKLLoss
    x = synth.make_case("ag_train", case=62, T=256, d=128, V=2048, K=16,
                        dtype="f32", tau=1.0, chunk=64)
    dev = G.to_device(x)
    gen = torch.Generator().manual_seed(5)
    X = torch.randn(256, 64, generator=gen).cuda()
    A = (torch.randn(64, 128, generator=gen) / 8).cuda().requires_grad_(True)
    W = dev["W"].clone().requires_grad_(True)
    crit = TopKKLLoss(tau=1.0, chunk=64)
    loss = crit(X @ A, W, dev["topk_idx"], dev["topk_logit"])
    loss.backward()
    H64 = (X.double() @ A.detach().double()).cpu().numpy()
    ref = orc.kd_topk_kl(H64, x.W, x.topk_idx, x.topk_logit, None, 1.0)
    want_A = X.double().cpu().numpy().T @ ref["dH"]
    G.assert_grad_close(G.to_np(A.grad), want_A, "f32", "A.grad")
    G.assert_grad_close(G.to_np(W.grad), ref["dW"], "f32", "W.grad")
    opt = torch.optim.SGD([A, W], lr=0.5)
    losses = []
    for _ in range(5):
        opt.zero_grad()
        loss = crit(X @ A, W, dev["topk_idx"], dev["topk_logit"])
        loss.backward()
        opt.step()
        losses.append(float(loss.item()))
    assert all(b < a for a, b in zip(losses, losses[1:])), losses


def test_training_step_on_one_stream_without_host_synchronisation():
    # torch ops -> loss -> backward -> torch ops, all queued on one side
    # stream: the library calls return while the stream is still busy (no
    # host synchronisation inside), and the results match the oracle
    import torch
    from top_kl_loss_amd.autograd import topk_kl_loss
    x = synth.make_case("ag_stream", case=63, T=384, d=192, V=3000, K=20,
                        dtype="bf16", tau=1.5, mask_frac=0.1, chunk=128)
    dev = G.to_device(x)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    busy = []
    with torch.cuda.stream(s):
        # exact in bf16 (powers of two): the inputs come out of torch kernels
        H = ((dev["H"] * 4.0) * 0.25).requires_grad_(True)
        W = (dev["W"] * 1.0).requires_grad_(True)
        torch.cuda._sleep(100_000_000)     # keeps the stream busy for a while
        loss = topk_kl_loss(H, W, dev["topk_idx"], dev["topk_logit"],
                            dev["mask"], x.tau, x.chunk)
        busy.append(not s.query())
        (loss * 3.0).backward()
        busy.append(not s.query())
        gH = H.grad.float() * 1.0
        gW = W.grad.float() * 1.0
        lv = loss * 1.0
    s.synchronize()
    assert all(busy), busy
    ref = orc.kd_topk_kl(x.H, x.W, x.topk_idx, x.topk_logit, x.mask, x.tau)
    G.assert_loss_close(float(lv.item()), ref["loss"], x.dtype)
    G.assert_grad_close(G.to_np(gH), 3.0 * ref["dH"], x.dtype, "H.grad")
    G.assert_grad_close(G.to_np(gW), 3.0 * ref["dW"], x.dtype, "W.grad")
