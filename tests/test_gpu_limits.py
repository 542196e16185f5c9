"""GPU parity at the largest sizes the C ABI accepts.

The library takes T d, V d and T K below 2^31 (every element index of H,
W, the teacher cache and the gradients fits in 31 bits).  At those limits a
byte offset no longer fits in 32 bits: at n d = 2^31 - 128 a bf16 operand
spans 4294967040 bytes, just under 2^32, and its fp32 gradient twice as
many.  These tests run the tuned bf16 path right at the limits, at the
workloads' hidden size d = 2880, and compare with the fp64 oracle:

* the largest vocabulary, V = 745654 (V d = 2^31 - 128): 256 token rows in
  2 slices, uniform teacher ids, which reach the vocabulary's last, partial
  256-wide tile.  The loss and every row's KL (the oracle's logsumexp of
  every row over the whole vocabulary), every dH row, and dW at the rows of
  the first 8 tokens' teacher ids, the vocabulary's last 256 rows and 256
  random rows;
* the most token rows, T = 745654 (T d = 2^31 - 128): V = 300 (two
  segments, the second partial), slices of 65536 (the last one ragged).
  Every row's KL and dH row, the loss and all of dW, the oracle evaluated
  8192 rows at a time;
* the teacher top-K cache builder at the largest vocabulary: 512 rows in 2
  slices, every row's ids distinct, in range and ordered, and 8 rows (the
  first and last of each slice, 4 random) against the oracle.

Host cost of each test: about 40 GB of memory and one to two minutes.
"""
import gc

import numpy as np
import pytest

import synth
from oracle import kd_oracle as orc
from tests import _gpu as G

pytestmark = pytest.mark.gpu

D = 2880
N_MAX = (2 ** 31 - 1) // D        # 745654 rows of d = 2880: 2^31 - 128 elements


def _say(msg):
    print(msg, flush=True)


def _release():
    import torch
    gc.collect()
    torch.cuda.empty_cache()


def test_largest_vocabulary():
    import torch
    x = synth.make_case("v_limit", case=41, T=256, d=D, V=N_MAX, K=100,
                        dtype=synth.BF16, chunk=128, cache="uniform")
    assert x.V * x.d < 2 ** 31 <= (x.V + 1) * x.d
    assert x.topk_idx.max() >= x.V - x.V % 256, "no teacher id in the last tile"
    _say(f"largest vocabulary: T={x.T} d={x.d} V={x.V} chunk={x.chunk}")
    dev = G.to_device(x)
    loss, rl, dH, dW = G.run(dev, x.tau, x.chunk)
    rng = np.random.default_rng(41)
    v_rows = np.unique(np.concatenate([
        x.topk_idx[:8].ravel().astype(np.int64), np.arange(x.V - 256, x.V),
        rng.choice(x.V, 256, replace=False)]))
    g_dW = dW[torch.from_numpy(v_rows).to(dW.device)].cpu().numpy()
    g_loss, g_rl, g_dH = float(loss.item()), G.to_np(rl), dH.cpu().numpy()
    del dev, loss, rl, dH, dW
    _release()

    W64 = np.asarray(x.W, np.float64)
    lse = orc.row_lse(x.H, W64, x.tau, rows_per_block=64)
    o_loss, o_rl = orc.loss_given_lse(x.H, W64, x.topk_idx, x.topk_logit, None,
                                      x.tau, lse)
    G.assert_loss_close(g_loss, o_loss, x.dtype)
    G.assert_rows_kl(g_rl, o_rl, "largest vocabulary")
    for r0 in range(0, x.T, 32):
        r1 = min(x.T, r0 + 32)
        _, o_dH = orc.rows_loss_and_dh(x.H[r0:r1], W64, x.topk_idx[r0:r1],
                                       x.topk_logit[r0:r1], None, x.tau, x.n_valid)
        G.assert_grad_close(g_dH[r0:r1], o_dH, x.dtype, f"dH rows {r0}:{r1}")
    o_dW = orc.dw_rows(x.H, W64, x.topk_idx, x.topk_logit, None, x.tau, lse, v_rows)
    G.assert_grad_close(g_dW, o_dW, x.dtype, f"dW at {len(v_rows)} rows")
    _say(f"largest vocabulary: loss {g_loss:.7f} oracle {o_loss:.7f}")


def test_most_token_rows():
    x = synth.make_case("t_limit", case=42, T=N_MAX, d=D, V=300, K=100,
                        dtype=synth.BF16, chunk=65536, cache="uniform")
    assert x.T * x.d < 2 ** 31 <= (x.T + 1) * x.d
    _say(f"most token rows: T={x.T} d={x.d} V={x.V} chunk={x.chunk}")
    dev = G.to_device(x)
    loss, rl, dH, dW = G.run(dev, x.tau, x.chunk)
    g_loss, g_rl = float(loss.item()), G.to_np(rl)
    g_dH, g_dW = dH.cpu().numpy(), dW.cpu().numpy()
    del dev, loss, rl, dH, dW
    _release()

    W64 = np.asarray(x.W, np.float64)
    o_rl = np.empty(x.T)
    o_dW = np.zeros_like(W64)
    for r0 in range(0, x.T, 8192):
        r1 = min(x.T, r0 + 8192)
        rl, _, dH, dW = orc.slice_terms(x.H[r0:r1], W64, x.topk_idx[r0:r1],
                                        x.topk_logit[r0:r1], None, x.tau, x.n_valid)
        o_rl[r0:r1] = rl
        o_dW += dW
        G.assert_grad_close(g_dH[r0:r1], dH, x.dtype, f"dH rows {r0}:{r1}")
    G.assert_rows_kl(g_rl, o_rl, "most token rows")
    o_loss = x.tau ** 2 * o_rl.sum() / x.n_valid
    G.assert_loss_close(g_loss, o_loss, x.dtype)
    G.assert_grad_close(g_dW, o_dW, x.dtype, "dW")
    _say(f"most token rows: loss {g_loss:.7f} oracle {o_loss:.7f}")


def test_teacher_topk_largest_vocabulary():
    import torch
    import top_kl_loss_amd as kd
    x = synth.teacher_head("v_limit_teacher", case=43, T=512, d=D, V=N_MAX)
    _say(f"teacher top-K, largest vocabulary: T={x.T} d={x.d} V={x.V} chunk=256")
    H = torch.from_numpy(x.H_bits.view(np.int16)).view(torch.bfloat16).cuda()
    W = torch.from_numpy(x.W_bits.view(np.int16)).view(torch.bfloat16).cuda()
    ids, vals = kd.kd_teacher_topk(H, W, 100, 256, sync=True)
    ids = ids.cpu().numpy()
    vals = vals.cpu().numpy().astype(np.float64)
    del H, W
    _release()
    assert ids.min() >= 0 and ids.max() < x.V
    assert np.all(np.diff(np.sort(ids, axis=1), axis=1) > 0)
    dv = np.diff(vals, axis=1)
    assert np.all(dv <= 0) and np.all(np.diff(ids, axis=1)[dv == 0] > 0)
    rng = np.random.default_rng(43)
    rows = sorted({0, 255, 256, 511, *rng.choice(x.T, 4, replace=False).tolist()})
    G.check_topk(x, ids[rows], vals[rows], 100, rows=rows)
