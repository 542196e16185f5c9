"""GPU parity at the full workload sizes, in the launch configurations the
benchmark times.  The oracle cannot afford the dense fp64 forward and
backward at these sizes, so it checks what it can compute one by one:

* the exact total loss and every row's KL where the full-vocabulary
  logsumexp of every row is affordable (T = 4096), plus sampled dW rows;
* sampled rows' KL and dH rows everywhere (each needs only that row and the
  valid-token count);
* identities that hold at any size: sum_v dW[v,:] = 0 (every logit-gradient
  row sums to zero), <dH, H> = <dW, W> (both equal sum G*z), padding rows
  get no gradient, and invariance to the slice size.
"""
import sys

import numpy as np
import pytest

import synth
from oracle import kd_oracle as orc
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _sample_rows(x, extra=()):
    rng = np.random.default_rng(12345)
    rows = set(int(r) for r in rng.choice(x.T, size=10, replace=False))
    rows |= {0, x.T - 1, *extra}
    if x.mask is not None:
        rows |= set(int(r) for r in np.flatnonzero(x.mask == 0)[:2])
    return np.array(sorted(r for r in rows if 0 <= r < x.T))


def _check_rows(x, rl, dH, rows):
    o_rl, o_dh = orc.rows_loss_and_dh(
        x.H[rows], x.W, x.topk_idx[rows], x.topk_logit[rows],
        None if x.mask is None else x.mask[rows], x.tau, x.n_valid)
    g_rl = G.to_np(rl)[rows]
    g_dh = G.to_np(dH[rows])
    G.assert_grad_close(g_rl, o_rl, x.dtype, "sampled row_loss")
    G.assert_grad_close(g_dh, o_dh, x.dtype, "sampled dH rows")
    if x.mask is not None:
        pad = x.mask[rows] == 0
        assert np.all(g_dh[pad] == 0.0) and np.all(g_rl[pad] == 0.0)


def _check_identities(x, dev, dH, dW):
    import torch
    dWd = dW.double()
    colsum = dWd.sum(0).abs()
    colabs = dWd.abs().sum(0)
    ratio = float((colsum / colabs.clamp_min(1e-30)).max())
    assert ratio <= 1e-3, f"sum_v dW not ~0: {ratio:.2e}"
    Hd = dev["H"].double()
    Wd = dev["W"].double()
    a = float((dH.double() * Hd).sum())
    b = float((dWd * Wd).sum())
    scale = float((dH.double() * Hd).abs().sum())
    assert abs(a - b) <= 1e-3 * scale, f"<dH,H>={a} <dW,W>={b}"
    del Hd, Wd, dWd
    torch.cuda.empty_cache()


def test_t4k_exact_loss_all_rows_and_sampled_gradients():
    x = synth.workload("t4k", teacher_device="cuda")
    _say(f"t4k: T={x.T} d={x.d} V={x.V} chunk={x.chunk}")
    dev = G.to_device(x)
    loss, rl, dH, dW = G.run(dev, x.tau, x.chunk)
    lse = orc.row_lse(x.H, x.W, x.tau, rows_per_block=512)
    o_loss, o_rl = orc.loss_given_lse(x.H, x.W, x.topk_idx, x.topk_logit,
                                      x.mask, x.tau, lse)
    G.assert_loss_close(float(loss.item()), o_loss, x.dtype)
    G.assert_grad_close(G.to_np(rl), o_rl, x.dtype, "row_loss (all rows)")
    rows = _sample_rows(x, extra=(1023, 1024, 2047, 2048))
    _check_rows(x, rl, dH, rows)
    vs = np.unique(np.concatenate([x.topk_idx[0, :3], x.topk_idx[4095, :2],
                                   [0, 1, 201087, 100000]]))
    o_dw = orc.dw_rows(x.H, x.W, x.topk_idx, x.topk_logit, x.mask, x.tau,
                       lse, vs)
    G.assert_grad_close(G.to_np(dW[vs]), o_dw, x.dtype, "sampled dW rows")
    _check_identities(x, dev, dH, dW)
    # the forward-only entry point: the same loss bitwise, and every row's
    # logsumexp against the oracle's
    import top_kl_loss_amd as kd
    f_loss, f_rl, f_lse = kd.kd_topk_kl_fwd(dev["H"], dev["W"], dev["topk_idx"],
                                            dev["topk_logit"], dev["mask"],
                                            x.tau, x.chunk)
    assert float(f_loss.item()) == float(loss.item())
    assert np.array_equal(G.to_np(f_rl), G.to_np(rl))
    err = np.abs(G.to_np(f_lse) - lse).max() / np.abs(lse).max()
    assert err <= 1e-5, f"lse max rel {err:.2e}"


def test_t8k_masked_sampled_rows_and_identities():
    x = synth.workload("t8k", teacher_device="cuda")
    assert x.mask is not None and x.T - x.mask.sum() == 410
    _say(f"t8k: T={x.T} masked={x.T - x.n_valid} chunk={x.chunk}")
    dev = G.to_device(x)
    loss, rl, dH, dW = G.run(dev, x.tau, x.chunk)
    rows = _sample_rows(x, extra=(1023, 1024, 8191))
    _check_rows(x, rl, dH, rows)
    # the loss is tau^2/N times the sum of the per-row KL the library reports
    tot = float(rl.double().sum()) * x.tau ** 2 / x.n_valid
    assert abs(float(loss.item()) - tot) <= 1e-5 * abs(tot)
    _check_identities(x, dev, dH, dW)


def test_t32k_bench_configuration():
    # T = 32768 at the slice size bench.py times
    x = synth.workload("t32k", teacher_device="cuda")
    _say(f"t32k: T={x.T} chunk={x.chunk}")
    dev = G.to_device(x)
    loss, rl, dH, dW = G.run(dev, x.tau, x.chunk)
    rows = _sample_rows(x, extra=(x.chunk - 1, x.chunk, 3 * x.chunk + 5))
    _check_rows(x, rl, dH, rows)
    tot = float(rl.double().sum()) * x.tau ** 2 / x.n_valid
    assert abs(float(loss.item()) - tot) <= 1e-5 * abs(tot)
    _check_identities(x, dev, dH, dW)


def test_t32k_slices_past_4_gib_buffers():
    # chunk 16384: the slice's probability / gradient buffer (16384 x 201216
    # bf16 = 6.6 GB) and its transpose exceed the 4 GiB reach of 32-bit
    # buffer offsets; the tiles address them from their own first row.
    # Rows are independent, so the row losses and the loss equal those of the
    # benchmark's slice size bit for bit (which also shows that the tuned
    # kernels ran: the generic ones round differently); the gradients differ
    # only in the order of fp32 partial sums.
    import torch
    x = synth.workload("t32k", teacher_device="cuda")
    dev = G.to_device(x)
    _say(f"t32k: chunk={x.chunk}")
    loss_a, rl_a, dH_a, dW_a = G.run(dev, x.tau, x.chunk)
    _say("t32k: chunk=16384")
    loss_b, rl_b, dH_b, dW_b = G.run(dev, x.tau, 16384)
    assert torch.equal(rl_a, rl_b)
    assert float(loss_a.item()) == float(loss_b.item())
    for name, g, o in (("dH", dH_b, dH_a), ("dW", dW_b, dW_a)):
        err = float((g - o).abs().max()) / float(o.abs().max())
        assert err <= 1e-5, f"chunk 16384: {name} differs by {err:.2e}"
    rows = _sample_rows(x, extra=(16383, 16384, 32767))
    _check_rows(x, rl_b, dH_b, rows)
    del loss_a, rl_a, dH_a, dW_a
    torch.cuda.empty_cache()


def test_t32k_d4096_chunk_sweep():
    # d = 4096, V = 151936, tau = 2, 15% padding; slice sizes 512 ... 4096
    import torch
    x = synth.workload("t32k_d4096", teacher_device="cuda")
    assert x.T - x.mask.sum() == 4915
    dev = G.to_device(x)
    ref = None
    for c in synth.CHUNK_SWEEP["t32k_d4096"]:
        _say(f"t32k_d4096: chunk={c}")
        loss, rl, dH, dW = G.run(dev, x.tau, c)
        if c == 1024:
            rows = _sample_rows(x, extra=(1023, 1024, 30000))
            _check_rows(x, rl, dH, rows)
            _check_identities(x, dev, dH, dW)
        if ref is None:
            ref = (float(loss.item()), rl.clone(), dH.clone(), dW.clone())
        else:
            assert abs(float(loss.item()) - ref[0]) <= 1e-5 * abs(ref[0])
            for name, g, o in (("row_loss", rl, ref[1]), ("dH", dH, ref[2]),
                               ("dW", dW, ref[3])):
                err = float((g - o).abs().max()) / float(o.abs().max())
                assert err <= 2e-3, f"chunk {c}: {name} differs by {err:.2e}"
        del loss, rl, dH, dW
        torch.cuda.empty_cache()


def test_teacher_topk_t32k_bench_configuration():
    # the teacher cache build at the size bench.py --op teacher_topk times:
    # T = 32768 rows of the t32k teacher head, K = 100, chunk 4096
    import torch
    import top_kl_loss_amd as kd
    x = synth.teacher_head("t32k_teacher", case=3, T=32768, d=2880, V=201088)
    _say("teacher top-K: T=32768 d=2880 V=201088 K=100 chunk=4096")
    H = torch.from_numpy(x.H_bits.view(np.int16)).view(torch.bfloat16).cuda()
    W = torch.from_numpy(x.W_bits.view(np.int16)).view(torch.bfloat16).cuda()
    ids, vals = kd.kd_teacher_topk(H, W, 100, 4096)
    ids = ids.cpu().numpy()
    vals = vals.cpu().numpy().astype(np.float64)
    # every row: ids in range and distinct, logits sorted (ties by id)
    assert ids.min() >= 0 and ids.max() < x.V
    srt = np.sort(ids, axis=1)
    assert np.all(np.diff(srt, axis=1) > 0)
    dv = np.diff(vals, axis=1)
    assert np.all(dv <= 0) and np.all(np.diff(ids, axis=1)[dv == 0] > 0)
    # sampled rows (first and last of slices, random) against the oracle
    rng = np.random.default_rng(2024)
    rows = sorted({0, 4095, 4096, 32767, *rng.choice(32768, 8, replace=False).tolist()})
    _say(f"teacher top-K: oracle on rows {rows}")
    G.check_topk(x, ids[rows], vals[rows], 100, rows=rows)
    del H, W
    torch.cuda.empty_cache()
