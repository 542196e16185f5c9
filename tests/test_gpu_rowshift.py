"""GPU parity of the tuned path's per-row probability shift and its
fallback.

The tuned bf16 kernels store the probabilities of a row as 2^(z s2 - sh)
with one a-priori shift sh per row: the largest student logit among the
row's best teacher slots, which is at or below the row maximum.  A row
whose maximum lies more than SHIFT_LIMIT2 (64, base 2) above it is
recomputed with the maximum as shift.  These cases make such rows on
purpose: their teacher ids are the student's lowest logits (spread over
about 80 nats), so every shift they get is far below the row maximum.
Everything is compared with the fp64 oracle at the bf16 bars."""
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


def _adversarial(name, case, T, d, V, K, tau, rows, mask_frac=0.0, chunk=256):
    """Student logits z ~ N(0, 12^2); the listed rows get the K ids of
    their lowest student logits as teacher ids (teacher logits kept)."""
    x = synth.make_case(name, case=case, T=T, d=d, V=V, K=K, dtype="bf16",
                        tau=tau, mask_frac=mask_frac, chunk=chunk,
                        cache="self", self_noise=0.1, h_std=12.0)
    z = x.H[rows] @ x.W.T
    low = np.argsort(z, axis=1, kind="stable")[:, :K].astype(np.int32)
    idx = x.topk_idx.copy()
    idx[rows] = low
    x.topk_idx = np.ascontiguousarray(idx)
    return x


def _check(x):
    _say(f"rowshift: {x.name} T={x.T} d={x.d} V={x.V} K={x.K} tau={x.tau} "
         f"chunk={x.chunk}")
    dev = G.to_device(x)
    loss, rl, dH, dW = G.run(dev, x.tau, x.chunk)
    ref = orc.kd_topk_kl(x.H, x.W, x.topk_idx, x.topk_logit, x.mask, x.tau)
    G.assert_loss_close(float(loss.item()), ref["loss"], x.dtype)
    G.assert_grad_close(G.to_np(rl), ref["row_loss"], x.dtype, "row_loss")
    G.assert_grad_close(G.to_np(dH), ref["dH"], x.dtype, "dH")
    G.assert_grad_close(G.to_np(dW), ref["dW"], x.dtype, "dW")
    assert np.isfinite(G.to_np(dH)).all() and np.isfinite(G.to_np(dW)).all()


def test_some_rows_recomputed_with_their_maximum():
    # rows in two of three 256-row tiles of the first slice and one row of
    # the last (ragged) slice; padding among them
    rows = [3, 40, 41, 300, 301, 511, 700, 1000]
    x = _adversarial("rs_some", 70, T=1030, d=256, V=6000, K=50, tau=1.0,
                     rows=rows, mask_frac=0.05, chunk=768)
    if x.mask is not None:
        x.mask[41] = 0               # a flagged padding row: no gradient
    _check(x)


def test_every_row_recomputed_low_temperature():
    # tau = 0.5 doubles the spread in base-2 units; every row is flagged, so
    # every tile of every slice is recomputed
    x = _adversarial("rs_all", 71, T=520, d=128, V=3001, K=20, tau=0.5,
                     rows=list(range(520)), chunk=256)
    _check(x)


def test_teacher_ids_at_the_student_maximum():
    # the opposite extreme: teacher = the student's own top K (shift = the
    # row maximum up to rounding; nothing flagged), ragged vocabulary
    x = synth.make_case("rs_top", case=72, T=333, d=192, V=5003, K=64,
                        dtype="bf16", tau=0.7, chunk=200, cache="self",
                        self_noise=0.3, h_std=12.0)
    _check(x)
