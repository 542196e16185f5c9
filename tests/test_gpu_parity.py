"""GPU parity: the HIP library against the fp64 oracle on identical seeded
inputs, element by element at sizes the oracle finishes in seconds (several
tiles, ragged tails, masks, temperatures, edge cases)."""
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


def check_case(x, chunk=None, tau=None, rows=True):
    tau = x.tau if tau is None else tau
    chunk = x.chunk if chunk is None else chunk
    _say(f"case {x.name}: T={x.T} d={x.d} V={x.V} K={x.K} {x.dtype} tau={tau} chunk={chunk}")
    dev = G.to_device(x)
    loss, rl, dH, dW = G.run(dev, tau, chunk)
    ref = orc.kd_topk_kl(x.H, x.W, x.topk_idx, x.topk_logit, x.mask, tau,
                         chunk=chunk)
    G.assert_loss_close(float(loss.item()), ref["loss"], x.dtype)
    if rows:
        G.assert_grad_close(G.to_np(rl), ref["row_loss"], x.dtype, "row_loss")
    G.assert_grad_close(G.to_np(dH), ref["dH"], x.dtype, "dH")
    G.assert_grad_close(G.to_np(dW), ref["dW"], x.dtype, "dW")
    return dev, (loss, rl, dH, dW), ref


def test_tiny_fp32():
    check_case(synth.workload("tiny"))


def test_fp32_ragged_tails_mask_tau():
    # T not a multiple of chunk, d not a multiple of the k-step, V not a
    # multiple of the segment width, K odd, padding rows, tau != 1.
    x = synth.make_case("f32_ragged", case=20, T=300, d=200, V=1000, K=17,
                        dtype="f32", tau=1.7, mask_frac=0.1, chunk=128)
    check_case(x)


def test_bf16_ragged_tails_mask_tau():
    x = synth.make_case("bf16_ragged", case=21, T=333, d=136, V=3001, K=23,
                        dtype="bf16", tau=0.8, mask_frac=0.07, chunk=100)
    check_case(x)


def test_bf16_teacher_cache_tau2():
    x = synth.make_case("bf16_teacher", case=22, T=512, d=256, V=5000, K=100,
                        dtype="bf16", tau=2.0, mask_frac=0.15, chunk=200,
                        cache="teacher", logit_scale=0.5, teacher_device="cuda")
    check_case(x)


def test_bf16_full_vocab_few_rows():
    # The production vocabulary and hidden size (201088 x 2880), 192 rows.
    x = synth.make_case("bf16_fullvocab", case=23, T=192, d=2880, V=201088,
                        K=100, dtype="bf16", tau=1.0, chunk=128,
                        cache="teacher", teacher_device="cuda")
    check_case(x)


def test_fp32_k1_and_k_equals_v():
    x = synth.make_case("k1", case=24, T=130, d=64, V=700, K=1, dtype="f32",
                        tau=1.0, chunk=64)
    check_case(x)
    x = synth.make_case("kv", case=25, T=70, d=32, V=300, K=300, dtype="f32",
                        tau=1.3, chunk=64, mask_frac=0.1)
    check_case(x)


def test_single_row_and_chunk_larger_than_T():
    x = synth.make_case("one", case=26, T=1, d=16, V=513, K=5, dtype="bf16",
                        chunk=4096)
    check_case(x)


def test_all_tokens_masked_gives_zeros():
    x = synth.make_case("allmasked", case=27, T=64, d=32, V=600, K=10,
                        dtype="bf16", chunk=32)
    x.mask = np.zeros(64, dtype=np.uint8)
    dev = G.to_device(x)
    loss, rl, dH, dW = G.run(dev, 1.0, 32)
    assert loss.item() == 0.0
    assert float(rl.abs().max()) == 0.0
    assert float(dH.abs().max()) == 0.0 and float(dW.abs().max()) == 0.0


def test_far_below_max_segments_are_reshifted():
    # One vocabulary entry dominates every row by ~150 nats, so the other
    # segments' maxima lie far below the row's logsumexp while they still
    # hold teacher ids: exercises the re-shift of the teacher correction.
    rng = np.random.default_rng(5)
    x = synth.make_case("reshift", case=28, T=96, d=16, V=1500, K=40,
                        dtype="f32", chunk=64)
    x.W = (rng.standard_normal((1500, 16)) * 0.05).astype(np.float32)
    x.W[3] = 0.0
    x.W[3, 0] = 30.0
    x.H[:, 0] = 5.0
    check_case(x)
    check_case(x, tau=0.5)


def test_repeat_is_bitwise_identical_and_accumulate_adds():
    import torch
    x = synth.make_case("det", case=29, T=400, d=128, V=4000, K=50,
                        dtype="bf16", chunk=128, mask_frac=0.05)
    dev = G.to_device(x)
    a = G.run(dev, 1.0, 128)
    b = G.run(dev, 1.0, 128)
    for u, v in zip(a, b):
        assert torch.equal(u, v)
    dW = a[3].clone()
    c = G.run(dev, 1.0, 128, flags=1, dW=dW)
    # (a + c_1) + c_2 + ... differs from 2 * (c_1 + c_2 + ...) only by fp32
    # rounding of the per-slice additions
    err = float((c[3] - 2 * a[3]).abs().max())
    assert err <= 1e-6 * float(a[3].abs().max())


def test_bf16_tuned_path_ragged_tails():
    # d a multiple of 64 (tuned kernels) but not of the 256-wide tiles, V not
    # a multiple of the segment, chunk not a multiple of the 256-row tile nor
    # of the 64-token k-step of dW (so one dW GEMM per slice), chunk < d, T
    # not a multiple of chunk, padding rows, tau != 1.
    x = synth.make_case("bf16_tuned_ragged", case=30, T=700, d=320, V=3001,
                        K=37, dtype="bf16", tau=1.3, mask_frac=0.1, chunk=300)
    check_case(x)


def test_bf16_tuned_path_reshift_and_small_slices():
    rng = np.random.default_rng(7)
    x = synth.make_case("bf16_tuned_reshift", case=31, T=130, d=64, V=1200,
                        K=40, dtype="bf16", chunk=48)
    W = (rng.standard_normal((1200, 64)) * 0.05).astype(np.float32)
    W[7] = 0.0
    W[7, 0] = 30.0
    H = x.H.copy()
    H[:, 0] = 5.0
    x.W_bits = synth.f32_to_bf16_bits(W)
    x.W = synth.bf16_bits_to_f32(x.W_bits)
    x.H_bits = synth.f32_to_bf16_bits(H)
    x.H = synth.bf16_bits_to_f32(x.H_bits)
    check_case(x)


def test_bf16_tuned_path_dw_groups():
    # chunk a multiple of 64 below 2048 tokens: the probabilities of several
    # slices stay resident and dW runs once per group (4 slices of 128, then
    # 2 of 1024), the last group ending in a ragged slice
    x = synth.make_case("bf16_groups", case=40, T=1000, d=192, V=3001, K=40,
                        dtype="bf16", tau=0.9, mask_frac=0.05, chunk=128)
    check_case(x)
    y = synth.make_case("bf16_groups2", case=41, T=2100, d=64, V=2000, K=30,
                        dtype="bf16", tau=1.0, mask_frac=0.05, chunk=1024)
    check_case(y)


def test_bf16_tuned_path_chunk_above_d():
    # chunk >= d; V and T ragged, padding rows
    x = synth.make_case("bf16_wt", case=32, T=600, d=192, V=3001, K=50,
                        dtype="bf16", tau=1.1, mask_frac=0.05, chunk=256)
    check_case(x)


def test_bf16_tuned_path_wide_tiles():
    # d a multiple of 320: dW runs on 192 x 320 tiles (its P~ operand read
    # with 24-chunk k-rows), dH on 256 x 256 tiles with a ragged N tile whose
    # W columns past d come from the next W row; ragged T, V (192-row tiles),
    # padding rows
    x = synth.make_case("bf16_wide", case=33, T=900, d=640, V=3001, K=64,
                        dtype="bf16", tau=1.2, mask_frac=0.05, chunk=640)
    check_case(x)


def test_bf16_tuned_path_largest_k():
    # K = KD_MAX_K = 1024 teacher slots per row on the tuned path
    x = synth.make_case("bf16_kmax", case=34, T=300, d=128, V=5000, K=1024,
                        dtype="bf16", tau=1.0, mask_frac=0.05, chunk=128)
    check_case(x)


def test_concurrent_calls_on_two_streams():
    # two calls in flight at once on two torch streams, each with its own
    # workspace and outputs, give the results of the same calls made one
    # after the other (bitwise)
    import torch
    import top_kl_loss_amd as kd
    xa = synth.make_case("conc_a", case=35, T=520, d=192, V=4000, K=40,
                         dtype="bf16", tau=1.0, mask_frac=0.05, chunk=256)
    xb = synth.make_case("conc_b", case=36, T=300, d=256, V=3000, K=60,
                         dtype="bf16", tau=2.0, chunk=128)
    da, db = G.to_device(xa), G.to_device(xb)
    ref_a = G.run(da, xa.tau, xa.chunk)
    ref_b = G.run(db, xb.tau, xb.chunk)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    main = torch.cuda.current_stream()
    outs = []
    for s, d, x in ((sa, da, xa), (sb, db, xb)):
        s.wait_stream(main)  # the inputs were written on the main stream
        ws = torch.empty(kd.kd_topk_kl_workspace_size(x.T, x.d, x.V, x.K, x.chunk,
                                                      kd.KD_BF16),
                         dtype=torch.uint8, device="cuda")
        ws.record_stream(s)
        outs.append(kd.kd_topk_kl_fwd_bwd(d["H"], d["W"], d["topk_idx"],
                                          d["topk_logit"], d["mask"], x.tau,
                                          x.chunk, workspace=ws, stream=s))
    torch.cuda.synchronize()
    for got, want in ((outs[0], ref_a), (outs[1], ref_b)):
        for u, v in zip(got, want):
            assert torch.equal(u, v)


def test_misaligned_matrix_is_rejected_before_any_work():
    # a view that starts 2 bytes into its storage: the library moves rows of
    # H and W 16 bytes at a time and rejects such a pointer up front
    import torch
    import top_kl_loss_amd as kd
    x = synth.make_case("misaligned", case=42, T=64, d=64, V=512, K=8,
                        dtype="bf16", chunk=64)
    dev = G.to_device(x)
    flat = torch.empty(x.T * x.d + 1, dtype=torch.bfloat16, device="cuda")
    H = flat[1:].view(x.T, x.d)
    H.copy_(dev["H"])
    assert H.data_ptr() % 16 == 2
    with pytest.raises(kd.KdError) as err:
        kd.kd_topk_kl_fwd_bwd(H, dev["W"], dev["topk_idx"], dev["topk_logit"],
                              None, 1.0, 64)
    assert err.value.status == kd.KD_ERR_INVALID_ARG
    # the same values at an aligned address run and match the oracle
    check_case(x)
