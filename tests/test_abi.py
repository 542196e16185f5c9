"""Host-side tests of the C ABI: the library loads, exports every symbol the
header declares, sizes its workspace, and rejects bad arguments before any
HIP call (so these run without a GPU)."""
import os
import re

import pytest

import top_kl_loss_amd as kd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kd_topk_kl.h")

pytestmark = pytest.mark.skipif(not os.path.exists(kd.LIB_PATH),
                                reason="libkdtopk.so not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(kd_\w+)\s*\(",
                                 src, flags=re.M)))


def test_header_declares_every_exported_entry_point():
    assert declared_functions() == sorted(kd.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    lib = kd.load_library()      # torch's HIP runtime first, then the library
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    for s in range(6):
        assert kd.kd_status_string(s).startswith(
            ["KD_OK", "KD_ERR_INVALID_ARG", "KD_ERR_WORKSPACE",
             "KD_ERR_UNSUPPORTED", "KD_ERR_HIP", "KD_ERR_SCRATCH"][s])
    assert kd.kd_status_string(99) == "unknown kd status"


def test_workspace_size_scales_with_chunk_not_with_T():
    a = kd.kd_topk_kl_workspace_size(32768, 2880, 201088, 100, 1024, kd.KD_BF16)
    b = kd.kd_topk_kl_workspace_size(4096, 2880, 201088, 100, 1024, kd.KD_BF16)
    dense = 8 * 32768 * 201088          # fp32 logits + fp32 gradient
    assert a < dense / 50
    assert a - b < 32768 * 4 * 2        # only O(T) scalars grow with T
    ws = [kd.kd_topk_kl_workspace_size(32768, 2880, 201088, 100, c, kd.KD_BF16)
          for c in (2048, 4096, 8192)]
    # from 2048 tokens on, one slice's probabilities are resident
    assert 1.8 * ws[0] < ws[1] < 2.2 * ws[0] and 1.8 * ws[1] < ws[2] < 2.2 * ws[1]
    # below, the tuned path keeps those of up to 4 slices (until 2048
    # tokens) for one dW GEMM per group: chunk 1024 holds two, about what
    # chunk 2048 holds, and stays near 1 GB at this shape
    assert 0.9 * ws[0] < a < 1.1 * ws[0] and a < 1.1e9
    # chunk is clamped to T
    assert (kd.kd_topk_kl_workspace_size(256, 512, 8192, 100, 64, kd.KD_F32) <
            kd.kd_topk_kl_workspace_size(256, 512, 8192, 100, 10 ** 6, kd.KD_F32)
            == kd.kd_topk_kl_workspace_size(256, 512, 8192, 100, 256, kd.KD_F32))


@pytest.mark.parametrize("args,code", [
    ((0, 512, 8192, 100, 64, kd.KD_F32), kd.KD_ERR_INVALID_ARG),
    ((256, 0, 8192, 100, 64, kd.KD_F32), kd.KD_ERR_INVALID_ARG),
    ((256, 512, 0, 100, 64, kd.KD_F32), kd.KD_ERR_INVALID_ARG),
    ((256, 512, 8192, 0, 64, kd.KD_F32), kd.KD_ERR_INVALID_ARG),
    ((256, 512, 99, 100, 64, kd.KD_F32), kd.KD_ERR_INVALID_ARG),
    ((256, 512, 8192, 100, 0, kd.KD_F32), kd.KD_ERR_INVALID_ARG),
    ((256, 510, 8192, 100, 64, kd.KD_F32), kd.KD_ERR_UNSUPPORTED),
    ((256, 512, 8192, 2000, 64, kd.KD_F32), kd.KD_ERR_UNSUPPORTED),
    ((256, 512, 8192, 100, 64, 7), kd.KD_ERR_UNSUPPORTED),
    ((2 ** 20, 4096, 8192, 100, 64, kd.KD_F32), kd.KD_ERR_UNSUPPORTED),
])
def test_workspace_size_rejects(args, code):
    with pytest.raises(kd.KdError) as e:
        kd.kd_topk_kl_workspace_size(*args)
    assert e.value.status == code


def _call(**kw):
    lib = kd.load_library()
    a = dict(H=256, W=256, dtype=kd.KD_BF16, idx=256, logit=256, mask=None, T=256,
             d=512, V=8192, K=100, tau=1.0, chunk=64, flags=0, loss=256,
             row_loss=None, dH=256, dW=256, ws=256, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return lib.kd_topk_kl_fwd_bwd(
        a["H"], a["W"], a["dtype"], a["idx"], a["logit"], a["mask"], a["T"],
        a["d"], a["V"], a["K"], a["tau"], a["chunk"], a["flags"], a["loss"],
        a["row_loss"], a["dH"], a["dW"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(H=None), kd.KD_ERR_INVALID_ARG),
    (dict(W=None), kd.KD_ERR_INVALID_ARG),
    (dict(idx=None), kd.KD_ERR_INVALID_ARG),
    (dict(logit=None), kd.KD_ERR_INVALID_ARG),
    (dict(loss=None), kd.KD_ERR_INVALID_ARG),
    (dict(dH=None), kd.KD_ERR_INVALID_ARG),
    (dict(dW=None), kd.KD_ERR_INVALID_ARG),
    (dict(tau=0.0), kd.KD_ERR_INVALID_ARG),
    (dict(tau=-1.0), kd.KD_ERR_INVALID_ARG),
    (dict(tau=float("inf")), kd.KD_ERR_INVALID_ARG),
    (dict(tau=float("nan")), kd.KD_ERR_INVALID_ARG),
    (dict(flags=4), kd.KD_ERR_INVALID_ARG),
    (dict(chunk=0), kd.KD_ERR_INVALID_ARG),
    (dict(K=9000), kd.KD_ERR_INVALID_ARG),
    (dict(T=-5), kd.KD_ERR_INVALID_ARG),
    (dict(d=12), kd.KD_ERR_UNSUPPORTED),
    (dict(dtype=3), kd.KD_ERR_UNSUPPORTED),
    (dict(K=1025), kd.KD_ERR_UNSUPPORTED),
    (dict(ws=None), kd.KD_ERR_WORKSPACE),
    (dict(ws_bytes=100), kd.KD_ERR_WORKSPACE),
    (dict(ws=256 + 16), kd.KD_ERR_WORKSPACE),
    # H, W, dH, dW must start on a 16-byte boundary
    (dict(H=256 + 2), kd.KD_ERR_INVALID_ARG),
    (dict(W=256 + 8), kd.KD_ERR_INVALID_ARG),
    (dict(dH=256 + 4), kd.KD_ERR_INVALID_ARG),
    (dict(dW=256 + 12), kd.KD_ERR_INVALID_ARG),
])
def test_fwd_bwd_rejects_before_any_hip_call(kw, code):
    assert _call(**kw) == code


# ------------------------------------------------------ teacher top-K cache
def test_teacher_workspace_is_bounded_by_the_slice():
    a = kd.kd_teacher_topk_workspace_size(32768, 2880, 201088, 100, 4096, kd.KD_BF16)
    b = kd.kd_teacher_topk_workspace_size(8192, 2880, 201088, 100, 4096, kd.KD_BF16)
    assert a == b                         # nothing grows with T
    per_row = 32 * 256 * 4 + 8192 * 8 + 16
    assert 4096 * per_row <= a < 4096 * per_row + 4096
    assert a < 4 * 4096 * 201088 / 8      # far below one fp32 slice of z
    # generic path (fp32, or d % 64 != 0) needs no scratch
    assert kd.kd_teacher_topk_workspace_size(64, 96, 5000, 100, 64, kd.KD_F32) == 256
    assert kd.kd_teacher_topk_workspace_size(64, 72, 5000, 100, 64, kd.KD_BF16) == 256


def test_teacher_samples_grow_with_k_and_vocabulary():
    """The sampled segments per row: 32, or ceil(K nseg / 4096) when larger
    (so that a row expects at most about half of its 8192 candidate slots),
    at most 128; the workspace holds 1 KiB of sampled logits per segment."""
    C = 256
    fixed = 8192 * 8 + 16

    def samples(V, K):
        ws = kd.kd_teacher_topk_workspace_size(C, 2880, V, K, C, kd.KD_BF16)
        ns, rest = divmod(ws - C * fixed, C * 256 * 4)
        assert 0 <= rest < 4096, (V, K, ws)
        return ns

    assert samples(201088, 100) == 32            # K nseg = 78600
    assert samples(201088, 256) == 50            # ceil(256 * 786 / 4096)
    assert samples(745654, 100) == 72            # V d just below 2^31 at d = 2880
    assert samples(745654, 256) == 128           # capped
    assert samples(5000, 100) == 20              # fewer segments than 32: all


@pytest.mark.parametrize("args,code", [
    ((0, 512, 8192, 100, 64, kd.KD_BF16), kd.KD_ERR_INVALID_ARG),
    ((256, 512, 99, 100, 64, kd.KD_BF16), kd.KD_ERR_INVALID_ARG),
    ((256, 512, 8192, 0, 64, kd.KD_BF16), kd.KD_ERR_INVALID_ARG),
    ((256, 512, 8192, 100, 0, kd.KD_BF16), kd.KD_ERR_INVALID_ARG),
    ((256, 510, 8192, 100, 64, kd.KD_BF16), kd.KD_ERR_UNSUPPORTED),
    ((256, 512, 8192, 257, 64, kd.KD_BF16), kd.KD_ERR_UNSUPPORTED),
    ((256, 16392, 8192, 100, 64, kd.KD_BF16), kd.KD_ERR_UNSUPPORTED),
    ((256, 512, 8192, 100, 64, 5), kd.KD_ERR_UNSUPPORTED),
])
def test_teacher_workspace_size_rejects(args, code):
    with pytest.raises(kd.KdError) as e:
        kd.kd_teacher_topk_workspace_size(*args)
    assert e.value.status == code


def _tk_call(**kw):
    lib = kd.load_library()
    a = dict(H=256, W=256, dtype=kd.KD_BF16, T=256, d=512, V=8192, K=100,
             chunk=64, idx=256, logit=256, ws=256, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return lib.kd_teacher_topk(a["H"], a["W"], a["dtype"], a["T"], a["d"],
                               a["V"], a["K"], a["chunk"], a["idx"],
                               a["logit"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(H=256 + 2), kd.KD_ERR_INVALID_ARG),  # 16-byte alignment
    (dict(W=256 + 4), kd.KD_ERR_INVALID_ARG),
    (dict(H=None), kd.KD_ERR_INVALID_ARG),
    (dict(W=None), kd.KD_ERR_INVALID_ARG),
    (dict(idx=None), kd.KD_ERR_INVALID_ARG),
    (dict(logit=None), kd.KD_ERR_INVALID_ARG),
    (dict(K=9000), kd.KD_ERR_INVALID_ARG),
    (dict(chunk=-1), kd.KD_ERR_INVALID_ARG),
    (dict(d=20), kd.KD_ERR_UNSUPPORTED),
    (dict(K=300), kd.KD_ERR_UNSUPPORTED),
    (dict(dtype=2), kd.KD_ERR_UNSUPPORTED),
    (dict(ws=None), kd.KD_ERR_WORKSPACE),
    (dict(ws_bytes=1000), kd.KD_ERR_WORKSPACE),
    (dict(ws=512 + 8), kd.KD_ERR_WORKSPACE),
])
def test_teacher_topk_rejects_before_any_hip_call(kw, code):
    assert _tk_call(**kw) == code


# ------------------------------------------ split forward / backward, cast
def test_forward_workspace_holds_no_probabilities():
    # the forward alone keeps the slice's row statistics, teacher softmax,
    # gathered logits and sorted ids (and T row losses), not the C x V
    # probabilities or any gradient buffer
    T, d, V, K = 32768, 2880, 201088, 100
    nseg = (V + 255) // 256
    for c in (1024, 8192, 32768):
        fused = kd.kd_topk_kl_workspace_size(T, d, V, K, c, kd.KD_BF16)
        fwd = kd.kd_topk_kl_fwd_workspace_size(T, d, V, K, c, kd.KD_BF16)
        per_slice = c * (5 * 4 * K + (2 + 4 + 4) * nseg + 4)   # q lq zg sid sslot, first mseg sseg, lse
        assert per_slice + 4 * T <= fwd <= per_slice + 4 * T + 16 * 256
        assert fwd < fused / 40
    # the size does not depend on the element type (no probabilities)
    assert (kd.kd_topk_kl_fwd_workspace_size(T, d, V, K, 8192, kd.KD_F32) ==
            kd.kd_topk_kl_fwd_workspace_size(T, d, V, K, 8192, kd.KD_BF16))
    with pytest.raises(kd.KdError) as e:
        kd.kd_topk_kl_fwd_workspace_size(T, 12, V, K, 8192, kd.KD_BF16)
    assert e.value.status == kd.KD_ERR_UNSUPPORTED


def test_forward_accepts_its_own_workspace_size_only():
    need = kd.kd_topk_kl_fwd_workspace_size(256, 512, 8192, 100, 64, kd.KD_BF16)
    assert _fwd_call(ws_bytes=need - 1) == kd.KD_ERR_WORKSPACE
    # (a workspace of `need` bytes passes every check; the call itself
    # needs a GPU)


def _fwd_call(**kw):
    lib = kd.load_library()
    a = dict(H=256, W=256, dtype=kd.KD_BF16, idx=256, logit=256, mask=None, T=256,
             d=512, V=8192, K=100, tau=1.0, chunk=64, loss=256, row_loss=None,
             lse=None, ws=256, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return lib.kd_topk_kl_fwd(
        a["H"], a["W"], a["dtype"], a["idx"], a["logit"], a["mask"], a["T"],
        a["d"], a["V"], a["K"], a["tau"], a["chunk"], a["loss"], a["row_loss"],
        a["lse"], a["ws"], a["ws_bytes"], a["stream"])


def _bwd_call(**kw):
    lib = kd.load_library()
    a = dict(H=256, W=256, dtype=kd.KD_BF16, idx=256, logit=256, mask=None, T=256,
             d=512, V=8192, K=100, tau=1.0, chunk=64, flags=0, g=None, dH=256,
             dW=256, ws=256, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return lib.kd_topk_kl_bwd(
        a["H"], a["W"], a["dtype"], a["idx"], a["logit"], a["mask"], a["T"],
        a["d"], a["V"], a["K"], a["tau"], a["chunk"], a["flags"], a["g"],
        a["dH"], a["dW"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(H=256 + 2), kd.KD_ERR_INVALID_ARG),  # 16-byte alignment
    (dict(W=256 + 4), kd.KD_ERR_INVALID_ARG),
    (dict(H=None), kd.KD_ERR_INVALID_ARG),
    (dict(loss=None), kd.KD_ERR_INVALID_ARG),
    (dict(tau=0.0), kd.KD_ERR_INVALID_ARG),
    (dict(K=9000), kd.KD_ERR_INVALID_ARG),
    (dict(d=12), kd.KD_ERR_UNSUPPORTED),
    (dict(ws=None), kd.KD_ERR_WORKSPACE),
    (dict(ws_bytes=100), kd.KD_ERR_WORKSPACE),
])
def test_fwd_rejects_before_any_hip_call(kw, code):
    assert _fwd_call(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(H=256 + 2), kd.KD_ERR_INVALID_ARG),  # 16-byte alignment
    (dict(W=256 + 4), kd.KD_ERR_INVALID_ARG),
    (dict(W=None), kd.KD_ERR_INVALID_ARG),
    (dict(dH=None), kd.KD_ERR_INVALID_ARG),
    (dict(dW=None), kd.KD_ERR_INVALID_ARG),
    (dict(flags=2), kd.KD_ERR_INVALID_ARG),
    (dict(tau=float("nan")), kd.KD_ERR_INVALID_ARG),
    (dict(dtype=9), kd.KD_ERR_UNSUPPORTED),
    (dict(ws=256 + 8), kd.KD_ERR_WORKSPACE),
])
def test_bwd_rejects_before_any_hip_call(kw, code):
    assert _bwd_call(**kw) == code


@pytest.mark.parametrize("args,code", [
    ((None, 1, kd.KD_BF16, 4, None, None), kd.KD_ERR_INVALID_ARG),
    ((1, None, kd.KD_BF16, 4, None, None), kd.KD_ERR_INVALID_ARG),
    ((1, 1, kd.KD_BF16, -1, None, None), kd.KD_ERR_INVALID_ARG),
    ((1, 1, 7, 4, None, None), kd.KD_ERR_UNSUPPORTED),
])
def test_grad_cast_rejects_before_any_hip_call(args, code):
    assert kd.load_library().kd_grad_cast(*args) == code


# ------------------------------------------------------- entropy filter
def _filter_call(**kw):
    lib = kd.load_library()
    a = dict(lg=1, mask=None, T=100, K=10, tau=1.0, mode=0, param=0.5, out=1,
             ent=None, ws=256, ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return lib.kd_entropy_filter(a["lg"], a["mask"], a["T"], a["K"], a["tau"],
                                 a["mode"], a["param"], a["out"], a["ent"],
                                 a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(lg=None), kd.KD_ERR_INVALID_ARG),
    (dict(out=None), kd.KD_ERR_INVALID_ARG),
    (dict(T=0), kd.KD_ERR_INVALID_ARG),
    (dict(K=0), kd.KD_ERR_INVALID_ARG),
    (dict(tau=0.0), kd.KD_ERR_INVALID_ARG),
    (dict(mode=2), kd.KD_ERR_INVALID_ARG),
    (dict(mode=1, param=1.5), kd.KD_ERR_INVALID_ARG),
    (dict(mode=1, param=-0.1), kd.KD_ERR_INVALID_ARG),
    (dict(param=float("nan")), kd.KD_ERR_INVALID_ARG),
    (dict(K=2000), kd.KD_ERR_UNSUPPORTED),
    (dict(ws=None), kd.KD_ERR_WORKSPACE),
    (dict(ws_bytes=8), kd.KD_ERR_WORKSPACE),
])
def test_entropy_filter_rejects_before_any_hip_call(kw, code):
    assert _filter_call(**kw) == code


def test_entropy_filter_workspace_size():
    assert kd.kd_entropy_filter_workspace_size(32768) == 256 + 32768 * 4
    with pytest.raises(kd.KdError):
        kd.kd_entropy_filter_workspace_size(0)


def _fwd_noalloc_call(**kw):
    lib = kd.load_library()
    a = dict(H=256, W=256, dtype=kd.KD_BF16, idx=256, logit=256, mask=None, T=256,
             d=512, V=8192, K=100, tau=1.0, chunk=64, loss=256, row_loss=None,
             lse=None, stream=None)
    a.update(kw)
    return lib.kd_topk_kl_fwd_noalloc(
        a["H"], a["W"], a["dtype"], a["idx"], a["logit"], a["mask"], a["T"],
        a["d"], a["V"], a["K"], a["tau"], a["chunk"], a["loss"], a["row_loss"],
        a["lse"], a["stream"])


def _noalloc_bytes(T, V, K, chunk):
    """The header's bound on the allocation-free forward's scratch."""
    C = min(chunk, T)
    nseg = (V + 255) // 256
    return 4 * T + C * (20 * K + 10 * nseg + 4) + 3072


@pytest.mark.parametrize("kw,code", [
    (dict(H=256 + 2), kd.KD_ERR_INVALID_ARG),  # 16-byte alignment
    (dict(W=256 + 4), kd.KD_ERR_INVALID_ARG),
    (dict(H=None), kd.KD_ERR_INVALID_ARG),
    (dict(loss=None), kd.KD_ERR_INVALID_ARG),
    (dict(tau=-1.0), kd.KD_ERR_INVALID_ARG),
    (dict(T=0), kd.KD_ERR_INVALID_ARG),
    (dict(d=12), kd.KD_ERR_UNSUPPORTED),
    # beyond the fixed scratch: the benchmark's slice of 8192 rows at
    # V = 201088 needs ~81 MB; a 64 MiB scratch takes at most ~6600 rows
    (dict(T=32768, d=2880, V=201088, chunk=8192), kd.KD_ERR_SCRATCH),
    (dict(T=1 << 24, d=64, V=256, K=1, chunk=1), kd.KD_ERR_SCRATCH),
])
def test_fwd_noalloc_rejects_before_any_hip_call(kw, code):
    assert _fwd_noalloc_call(**kw) == code


def test_fwd_noalloc_scratch_bound_covers_the_benchmark_sizes():
    # what the header promises fits: T = 32768, V = 201088, K = 100 at
    # slices up to 4096 rows, and the bound's own arithmetic
    assert _noalloc_bytes(32768, 201088, 100, 1024) < 11 * 10 ** 6
    assert _noalloc_bytes(32768, 201088, 100, 4096) < kd.KD_NOALLOC_SCRATCH_BYTES
    assert _noalloc_bytes(32768, 201088, 100, 8192) > kd.KD_NOALLOC_SCRATCH_BYTES


def _div_call(**kw):
    lib = kd.load_library()
    a = dict(kind=kd.KD_DIV_REVERSE_KL, H=256, W=256, dtype=kd.KD_BF16, idx=256,
             logit=256, mask=None, T=256, d=512, V=8192, K=100, tau=1.0, flags=0,
             loss=256, row_loss=None, dH=256, dW=256, ws=256, ws_bytes=1 << 40,
             stream=None)
    a.update(kw)
    return lib.kd_topk_div_fwd_bwd(
        a["kind"], a["H"], a["W"], a["dtype"], a["idx"], a["logit"], a["mask"],
        a["T"], a["d"], a["V"], a["K"], a["tau"], a["flags"], a["loss"],
        a["row_loss"], a["dH"], a["dW"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(H=256 + 2), kd.KD_ERR_INVALID_ARG),  # 16-byte alignment
    (dict(W=256 + 4), kd.KD_ERR_INVALID_ARG),
    (dict(kind=0), kd.KD_ERR_INVALID_ARG),
    (dict(kind=3), kd.KD_ERR_INVALID_ARG),
    (dict(H=None), kd.KD_ERR_INVALID_ARG),
    (dict(dW=None), kd.KD_ERR_INVALID_ARG),
    (dict(loss=None), kd.KD_ERR_INVALID_ARG),
    (dict(tau=float("inf")), kd.KD_ERR_INVALID_ARG),
    (dict(flags=4), kd.KD_ERR_INVALID_ARG),
    (dict(K=9000), kd.KD_ERR_INVALID_ARG),
    (dict(d=20), kd.KD_ERR_UNSUPPORTED),
    (dict(ws=None), kd.KD_ERR_WORKSPACE),
    (dict(ws_bytes=1000), kd.KD_ERR_WORKSPACE),
])
def test_divergence_rejects_before_any_hip_call(kw, code):
    assert _div_call(**kw) == code


def test_divergence_workspace_is_linear_in_pairs_and_vocabulary():
    a = kd.kd_topk_div_workspace_size(32768, 2880, 201088, 100)
    b = kd.kd_topk_div_workspace_size(16384, 2880, 201088, 100)
    dense = 8 * 32768 * 201088
    assert a < dense / 300                  # ~150 MB against 52.7 GB
    assert 1.5 * b < a < 2.5 * b            # T K pairs dominate
