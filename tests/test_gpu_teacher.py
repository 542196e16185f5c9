"""GPU parity of the teacher top-K cache builder (kd_teacher_topk) against
the fp64 oracle (oracle/teacher_topk.py) on identical seeded inputs.

The library accumulates logits in fp32, the oracle in fp64, so values are
compared within a rounding tolerance, and ids wherever the order is not
decided by values closer than that tolerance; integer-valued inputs make
every sum exact, and there ids and values must match the oracle exactly,
ties included."""
import sys

import numpy as np
import pytest

import synth
import top_kl_loss_amd as kd
from oracle import teacher_topk as tko
from tests import _gpu as G

pytestmark = pytest.mark.gpu

def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _to_dev(x):
    import torch
    if x.dtype == "bf16":
        H = torch.from_numpy(x.H_bits.view(np.int16)).view(torch.bfloat16)
        W = torch.from_numpy(x.W_bits.view(np.int16)).view(torch.bfloat16)
    else:
        H, W = torch.from_numpy(x.H), torch.from_numpy(x.W)
    return H.cuda(), W.cuda()


def _run(x, K, chunk, dev=None):
    dev = dev or _to_dev(x)
    ids, vals = kd.kd_teacher_topk(dev[0], dev[1], K, chunk)
    return ids.cpu().numpy(), vals.cpu().numpy().astype(np.float64)


check = G.check_topk


def test_tuned_path_sampled_and_filtered_segments_ragged_slices():
    # V = 40000: 157 segments, 32 sampled; T = 300 in slices 128, 128, 44
    x = synth.teacher_head("tk_main", case=40, T=300, d=192, V=40000)
    _say("teacher: T=300 d=192 V=40000 K=100 chunk=128 bf16")
    ids, vals = _run(x, 100, 128)
    check(x, ids, vals, 100)


@pytest.mark.parametrize("K", [1, 256])
def test_tuned_path_partial_last_segment_and_extreme_k(K):
    # V = 9001: 36 segments, the last one 41 columns wide
    x = synth.teacher_head("tk_partial", case=41, T=64, d=128, V=9001)
    _say(f"teacher: T=64 d=128 V=9001 K={K} chunk=64 bf16")
    ids, vals = _run(x, K, 64)
    check(x, ids, vals, K)


def test_tuned_path_every_segment_sampled():
    x = synth.teacher_head("tk_small_v", case=42, T=100, d=64, V=3000)
    _say("teacher: T=100 d=64 V=3000 K=100 bf16")
    ids, vals = _run(x, 100, 100)
    check(x, ids, vals, 100)


def test_vocabulary_smaller_than_one_segment():
    x = synth.teacher_head("tk_tiny_v", case=43, T=10, d=64, V=200)
    _say("teacher: T=10 d=64 V=200 K=100 bf16")
    ids, vals = _run(x, 100, 4)
    check(x, ids, vals, 100)


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("f32", 40)])
def test_integer_inputs_exact_with_ties(dtype, d):
    # integer entries in [-2, 2]: every logit is an exact integer in fp32,
    # most top-K boundaries fall inside a group of equal logits, and rows 0
    # and 17 are all zero (their cache must be ids 0..K-1)
    x = synth.teacher_head_integer("tk_int", case=44, T=64, d=d, V=20000,
                                   zero_rows=(0, 17), dtype=dtype)
    _say(f"teacher: integer inputs T=64 d={d} V=20000 K=100 {dtype}")
    ids, vals = _run(x, 100, 32)
    check(x, ids, vals, 100, exact=True)
    assert ids[0].tolist() == list(range(100)) and np.all(vals[0] == 0)


def test_rows_that_overflow_their_candidate_slots():
    # Vocabulary ids in the 32 sampled segments (every 4th of 157) use one
    # half of the hidden dimensions, all other ids the other half.  Even
    # rows see logits only on the sampled segments (few candidates); odd
    # rows see all-zero logits there, so their threshold is a zero logit
    # and about 16000 other entries pass it: more than the 8192 slots, and
    # those rows go through the row-streaming kernel.
    V, nseg = 40000, 157
    sampled = [4 * j for j in range(32)]
    x = synth.teacher_head_split("tk_split", case=45, T=48, d=128, V=V,
                                 marked_segments=sampled)
    z = tko.teacher_logits(x.H[1:2], x.W)[0]
    assert (z > 0).sum() > 8192 + 100
    _say("teacher: split head T=48 d=128 V=40000 K=100 bf16")
    ids, vals = _run(x, 100, 48)
    check(x, ids, vals, 100)
    assert nseg == (V + 255) // 256


@pytest.mark.parametrize("dtype,d", [("f32", 96), ("bf16", 72)])
def test_generic_path(dtype, d):
    x = synth.teacher_head("tk_generic", case=46, T=50, d=d, V=5000, dtype=dtype)
    _say(f"teacher: generic path T=50 d={d} V=5000 K=100 {dtype}")
    ids, vals = _run(x, 100, 16)
    check(x, ids, vals, 100)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_hand_worked_example(dtype):
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden",
                           "teacher_topk_hand.json")) as f:
        g = json.load(f)
    H = np.array(g["H"], dtype=np.float32)
    W = np.array(g["W"], dtype=np.float32)
    x = synth.inputs._encode("hand", H, W, dtype)
    for k, exp in g["expected"].items():
        ids, vals = _run(x, int(k), 2)
        assert ids.tolist() == exp["ids"]
        assert vals.tolist() == [[float(v) for v in r] for r in exp["logits"]]


def test_repeated_calls_are_bitwise_identical():
    x = synth.teacher_head("tk_main", case=40, T=300, d=192, V=40000)
    dev = _to_dev(x)
    a = _run(x, 100, 128, dev)
    b = _run(x, 100, 128, dev)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
