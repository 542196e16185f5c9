"""The allocation-free forward, kd_topk_kl_fwd_noalloc, through the C ABI.

Two calls in a row on the same GPU (so the second finds the first's data in
the shared scratch), the second with a smaller input on the other kernel
path; each must give bitwise what kd_topk_kl_fwd gives with a workspace of
its own (the same kernels at the same slice size), and the loss must meet
the oracle's bar."""
import numpy as np
import pytest

import synth
import top_kl_loss_amd as kd
from oracle import kd_oracle as orc
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def _check(x):
    import torch
    print(f"noalloc: {x.name} T={x.T} d={x.d} V={x.V} K={x.K} {x.dtype} "
          f"chunk={x.chunk}", flush=True)
    dev = G.to_device(x)
    want = kd.kd_topk_kl_fwd(dev["H"], dev["W"], dev["topk_idx"],
                             dev["topk_logit"], dev["mask"], x.tau, x.chunk)
    f32 = dict(dtype=torch.float32, device="cuda")
    outs = (torch.full((1,), float("nan"), **f32), torch.full((x.T,), float("nan"), **f32),
            torch.full((x.T,), float("nan"), **f32))
    got = kd.kd_topk_kl_fwd_noalloc(dev["H"], dev["W"], dev["topk_idx"],
                                    dev["topk_logit"], dev["mask"], x.tau,
                                    x.chunk, loss=outs[0], row_loss=outs[1],
                                    lse=outs[2])
    torch.cuda.synchronize()
    for name, g, w in zip(("loss", "row_loss", "lse"), got, want):
        assert g.data_ptr() in [o.data_ptr() for o in outs]
        assert torch.equal(g, w), name
    ref = orc.kd_topk_kl(x.H, x.W, x.topk_idx, x.topk_logit, x.mask, x.tau,
                         chunk=x.chunk)
    G.assert_loss_close(float(got[0].item()), ref["loss"], x.dtype)


def test_noalloc_forward_twice_second_smaller():
    # first: tuned bf16 path, 10% padding, three slices (last one ragged)
    _check(synth.make_case("noalloc_a", case=95, T=4500, d=512, V=50000, K=100,
                           dtype="bf16", tau=1.3, mask_frac=0.1, chunk=2048))
    # second, smaller: generic fp32 path (d % 64 != 0), no padding
    _check(synth.make_case("noalloc_b", case=96, T=300, d=200, V=9000, K=50,
                           dtype="f32", tau=1.0, chunk=128))


def test_noalloc_forward_rejects_a_slice_beyond_the_scratch():
    # T = 32768 rows of V = 201088 at slices of 8192 need ~81 MB of scratch
    with pytest.raises(kd.KdError) as e:
        import torch
        H = torch.zeros(32768, 64, dtype=torch.bfloat16, device="cuda")
        W = torch.zeros(201088, 64, dtype=torch.bfloat16, device="cuda")
        idx = torch.zeros(32768, 100, dtype=torch.int32, device="cuda")
        lg = torch.zeros(32768, 100, dtype=torch.float32, device="cuda")
        kd.kd_topk_kl_fwd_noalloc(H, W, idx, lg, None, 1.0, 8192)
    assert e.value.status == kd.KD_ERR_SCRATCH
