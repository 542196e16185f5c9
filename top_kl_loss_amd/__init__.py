"""Python binding of libkdtopk.so, the MI355X fused chunked top-K KL loss.

Argument marshalling only: every step of the loss runs in the HIP kernels of
the C library (``include/kd_topk_kl.h``).  PyTorch provides device memory and
streams.  There is no fallback: if the library is missing or cannot be
loaded, every call raises.

The library is loaded after torch, so its dependency on the HIP runtime
resolves (by soname) to the runtime torch has already loaded: one runtime
per process, whose streams and events both sides share.  Every call is
enqueued on a torch stream (by default the current one) without any host
synchronisation, and every temporary buffer is allocated on that stream, so
torch's caching allocator reuses it only after the call's kernels.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "KD_F32", "KD_BF16", "KD_FLAG_ACCUMULATE_DW", "KD_MAX_K", "LIB_PATH",
    "KdError", "load_library", "kd_topk_kl_workspace_size",
    "kd_topk_kl_fwd_bwd", "kd_status_string", "kd_set_launch_log",
    "kd_topk_kl_fwd_workspace_size",
    "EXPORTED_SYMBOLS", "KERNEL_NAMES", "KD_TOPK_MAX_K", "KD_TOPK_MAX_D",
    "kd_teacher_topk_workspace_size", "kd_teacher_topk", "kd_topk_kl_fwd",
    "kd_topk_kl_bwd", "kd_grad_cast", "kd_entropy_filter",
    "kd_entropy_filter_workspace_size", "KD_FILTER_ENTROPY_ABOVE",
    "KD_FILTER_TOP_ENTROPY_FRACTION", "kd_topk_kl_fwd_noalloc",
    "KD_NOALLOC_SCRATCH_BYTES", "KD_ERR_SCRATCH", "KD_DIV_REVERSE_KL",
    "KD_DIV_JSD", "kd_topk_div_workspace_size", "kd_topk_div_fwd_bwd",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkdtopk.so")

KD_F32, KD_BF16 = 0, 1
(KD_OK, KD_ERR_INVALID_ARG, KD_ERR_WORKSPACE, KD_ERR_UNSUPPORTED, KD_ERR_HIP,
 KD_ERR_SCRATCH) = range(6)
KD_FLAG_ACCUMULATE_DW = 1
KD_MAX_K = 1024
KD_TOPK_MAX_K = 256
KD_TOPK_MAX_D = 16384
KD_NOALLOC_SCRATCH_BYTES = 64 << 20
KD_DIV_REVERSE_KL, KD_DIV_JSD = 1, 2
DIVERGENCES = {"reverse_kl": KD_DIV_REVERSE_KL, "jsd": KD_DIV_JSD}
EXPORTED_SYMBOLS = ("kd_topk_kl_workspace_size", "kd_topk_kl_fwd_bwd",
                    "kd_status_string", "kd_set_launch_log",
                    "kd_teacher_topk_workspace_size", "kd_teacher_topk",
                    "kd_topk_kl_fwd", "kd_topk_kl_bwd", "kd_grad_cast",
                    "kd_entropy_filter_workspace_size", "kd_entropy_filter",
                    "kd_topk_kl_fwd_noalloc", "kd_topk_div_workspace_size",
                    "kd_topk_div_fwd_bwd", "kd_topk_kl_fwd_workspace_size")
KD_FILTER_ENTROPY_ABOVE, KD_FILTER_TOP_ENTROPY_FRACTION = 0, 1
# Kernel ids of the launch log (KD_KERNEL_* in the header).
KERNEL_NAMES = ("valid_count", "prep_rows", "gemm_logits", "lse_fix",
                "gemm_dh", "reduce_dh", "gemm_dw", "final_loss", "transpose_h",
                "flagged_rows", "unused_10", "tk_sample", "tk_theta", "tk_filter",
                "tk_select", "tk_stream", "grad_cast", "entropy_filter",
                "divergence")

_lib = None


class KdError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(msg)
        self.status = status


def load_library(path: str = LIB_PATH):
    """Load libkdtopk.so and declare its C signatures (once)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built; run `python -m top_kl_loss_amd.build` "
            "(needs ROCm hipcc)")
    # torch first: its HIP runtime (soname libamdhip64.so.7) is then the one
    # the library's dependency binds to, so torch's streams are valid here.
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    _check_single_runtime()
    c = ctypes
    lib.kd_topk_kl_workspace_size.argtypes = [
        c.c_int64, c.c_int64, c.c_int64, c.c_int32, c.c_int32, c.c_int,
        c.POINTER(c.c_size_t)]
    lib.kd_topk_kl_workspace_size.restype = c.c_int
    lib.kd_topk_kl_fwd_workspace_size.argtypes = [
        c.c_int64, c.c_int64, c.c_int64, c.c_int32, c.c_int32, c.c_int,
        c.POINTER(c.c_size_t)]
    lib.kd_topk_kl_fwd_workspace_size.restype = c.c_int
    lib.kd_topk_kl_fwd_bwd.argtypes = [
        c.c_void_p, c.c_void_p, c.c_int, c.c_void_p, c.c_void_p, c.c_void_p,
        c.c_int64, c.c_int64, c.c_int64, c.c_int32, c.c_float, c.c_int32,
        c.c_uint32, c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p,
        c.c_void_p, c.c_size_t, c.c_void_p]
    lib.kd_topk_kl_fwd_bwd.restype = c.c_int
    lib.kd_teacher_topk_workspace_size.argtypes = [
        c.c_int64, c.c_int64, c.c_int64, c.c_int32, c.c_int32, c.c_int,
        c.POINTER(c.c_size_t)]
    lib.kd_teacher_topk_workspace_size.restype = c.c_int
    lib.kd_teacher_topk.argtypes = [
        c.c_void_p, c.c_void_p, c.c_int, c.c_int64, c.c_int64, c.c_int64,
        c.c_int32, c.c_int32, c.c_void_p, c.c_void_p, c.c_void_p, c.c_size_t,
        c.c_void_p]
    lib.kd_teacher_topk.restype = c.c_int
    lib.kd_topk_kl_fwd.argtypes = [
        c.c_void_p, c.c_void_p, c.c_int, c.c_void_p, c.c_void_p, c.c_void_p,
        c.c_int64, c.c_int64, c.c_int64, c.c_int32, c.c_float, c.c_int32,
        c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p, c.c_size_t, c.c_void_p]
    lib.kd_topk_kl_fwd.restype = c.c_int
    lib.kd_topk_kl_fwd_noalloc.argtypes = [
        c.c_void_p, c.c_void_p, c.c_int, c.c_void_p, c.c_void_p, c.c_void_p,
        c.c_int64, c.c_int64, c.c_int64, c.c_int32, c.c_float, c.c_int32,
        c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p]
    lib.kd_topk_kl_fwd_noalloc.restype = c.c_int
    lib.kd_topk_kl_bwd.argtypes = [
        c.c_void_p, c.c_void_p, c.c_int, c.c_void_p, c.c_void_p, c.c_void_p,
        c.c_int64, c.c_int64, c.c_int64, c.c_int32, c.c_float, c.c_int32,
        c.c_uint32, c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p,
        c.c_size_t, c.c_void_p]
    lib.kd_topk_kl_bwd.restype = c.c_int
    lib.kd_topk_div_workspace_size.argtypes = [
        c.c_int64, c.c_int64, c.c_int64, c.c_int32, c.POINTER(c.c_size_t)]
    lib.kd_topk_div_workspace_size.restype = c.c_int
    lib.kd_topk_div_fwd_bwd.argtypes = [
        c.c_int32, c.c_void_p, c.c_void_p, c.c_int, c.c_void_p, c.c_void_p,
        c.c_void_p, c.c_int64, c.c_int64, c.c_int64, c.c_int32, c.c_float,
        c.c_uint32, c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p,
        c.c_void_p, c.c_size_t, c.c_void_p]
    lib.kd_topk_div_fwd_bwd.restype = c.c_int
    lib.kd_grad_cast.argtypes = [c.c_void_p, c.c_void_p, c.c_int, c.c_int64,
                                 c.c_void_p, c.c_void_p]
    lib.kd_grad_cast.restype = c.c_int
    lib.kd_entropy_filter_workspace_size.argtypes = [c.c_int64, c.POINTER(c.c_size_t)]
    lib.kd_entropy_filter_workspace_size.restype = c.c_int
    lib.kd_entropy_filter.argtypes = [
        c.c_void_p, c.c_void_p, c.c_int64, c.c_int32, c.c_float, c.c_int32,
        c.c_float, c.c_void_p, c.c_void_p, c.c_void_p, c.c_size_t, c.c_void_p]
    lib.kd_entropy_filter.restype = c.c_int
    lib.kd_status_string.argtypes = [c.c_int]
    lib.kd_status_string.restype = c.c_char_p
    lib.kd_set_launch_log.argtypes = [
        c.c_uint32, c.POINTER(c.c_void_p), c.POINTER(c.c_void_p),
        c.POINTER(c.c_int32), c.c_int32, c.POINTER(c.c_int32)]
    lib.kd_set_launch_log.restype = c.c_int
    _lib = lib
    return lib


def _check_single_runtime():
    """Raise if two HIP runtimes are mapped into the process (e.g. the library
    was loaded through ctypes before torch): stream and event handles of one
    are meaningless to the other."""
    try:
        with open("/proc/self/maps") as f:
            paths = {line.split()[-1] for line in f
                     if "libamdhip64" in line.rsplit("/", 1)[-1]}
    except OSError:  # pragma: no cover - not Linux
        return
    real = {os.path.realpath(p) for p in paths}
    if len(real) > 1:
        raise RuntimeError(
            "two HIP runtimes are loaded (" + ", ".join(sorted(real)) + "); "
            "import torch before loading libkdtopk.so")


def kd_status_string(status: int) -> str:
    return load_library().kd_status_string(int(status)).decode()


def _check(status):
    if status != KD_OK:
        raise KdError(status, kd_status_string(status))


def kd_topk_kl_workspace_size(T, d, V, K, chunk, dtype) -> int:
    """Workspace bytes for kd_topk_kl_fwd_bwd (see the C header)."""
    out = ctypes.c_size_t(0)
    _check(load_library().kd_topk_kl_workspace_size(
        int(T), int(d), int(V), int(K), int(chunk), int(dtype),
        ctypes.byref(out)))
    return out.value


def kd_topk_kl_fwd_workspace_size(T, d, V, K, chunk, dtype) -> int:
    """Workspace bytes for kd_topk_kl_fwd (see the C header)."""
    out = ctypes.c_size_t(0)
    _check(load_library().kd_topk_kl_fwd_workspace_size(
        int(T), int(d), int(V), int(K), int(chunk), int(dtype),
        ctypes.byref(out)))
    return out.value


def kd_set_launch_log(kernel_mask, start_events, end_events, kinds, capacity,
                      count):
    """Install (or, with kernel_mask 0, remove) the per-thread launch log:
    raw ctypes arrays of hipEvent_t handles, an int32 kinds array and an
    int32 counter (see the C header)."""
    _check(load_library().kd_set_launch_log(
        int(kernel_mask), start_events, end_events, kinds, int(capacity),
        count))


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return KD_BF16
    if t.dtype == torch.float32:
        return KD_F32
    raise TypeError(f"H/W must be bfloat16 or float32, got {t.dtype}")


def _torch_stream(dev, stream):
    """The torch stream a call runs on: the current stream of ``dev`` (None),
    a ``torch.cuda.Stream``, or a raw hipStream_t handle (int) of the same
    runtime, wrapped as an external stream."""
    import torch
    if stream is None:
        return torch.cuda.current_stream(dev)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=dev)


class _Call:
    """Context of one library call: device and stream guards, so that every
    tensor allocated inside is owned by the call's stream; on exit the
    stream is synchronised only when ``sync`` is set."""

    def __init__(self, dev, stream, sync):
        import torch
        self.dev = dev
        self.ts = _torch_stream(dev, stream)
        self.sync = sync
        self._guards = (torch.cuda.device(dev), torch.cuda.stream(self.ts))

    @property
    def handle(self):
        return self.ts.cuda_stream

    def __enter__(self):
        for g in self._guards:
            g.__enter__()
        return self

    def __exit__(self, *exc):
        for g in reversed(self._guards):
            g.__exit__(*exc)
        if exc[0] is None and self.sync:
            self.ts.synchronize()
        return False


def _loss_inputs(H, W, topk_idx, topk_logit, mask, chunk):
    """Validates the loss inputs; returns (T, d, V, K, chunk, dtype code)."""
    import torch
    T, d = H.shape
    V = W.shape[0]
    K = topk_idx.shape[1]
    chunk = T if chunk is None else int(chunk)
    dt = _dtype_code(H)
    if W.dtype != H.dtype or W.shape[1] != d:
        raise ValueError("W must be [V, d] with H's dtype")
    if topk_idx.dtype != torch.int32 or tuple(topk_idx.shape) != (T, K):
        raise ValueError("topk_idx must be int32 [T, K]")
    if topk_logit.dtype != torch.float32 or tuple(topk_logit.shape) != (T, K):
        raise ValueError("topk_logit must be float32 [T, K]")
    tensors = [H, W, topk_idx, topk_logit]
    if mask is not None:
        if mask.dtype not in (torch.bool, torch.uint8) or mask.numel() != T:
            raise ValueError("mask must be uint8/bool [T]")
        tensors.append(mask)
    dev = H.device
    for t in tensors:
        if not t.is_cuda or t.device != dev or not t.is_contiguous():
            raise ValueError("all inputs must be contiguous tensors on one GPU")
    return T, d, V, K, chunk, dt


def _mask_u8(mask):
    """The mask as uint8 (a bool mask is converted on the call's stream)."""
    import torch
    if mask is None or mask.dtype == torch.uint8:
        return mask
    return mask.to(torch.uint8)


def _workspace(T, d, V, K, chunk, dt, workspace, dev, size=None):
    import torch
    ws_bytes = (size or kd_topk_kl_workspace_size)(T, d, V, K, chunk, dt)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    elif workspace.numel() < ws_bytes:
        raise ValueError("workspace too small")
    return workspace


def _ptr(t):
    return t.data_ptr() if t is not None else None


_STREAM_DOC = """
    ``stream`` is None (torch's current stream on the inputs' device), a
    ``torch.cuda.Stream`` or a raw hipStream_t handle.  The work is enqueued
    there with no host synchronisation, and outputs and temporaries are
    allocated on that stream, so torch work queued on it afterwards sees the
    results; ``sync=True`` also waits for the stream before returning."""


def kd_topk_kl_fwd_bwd(H, W, topk_idx, topk_logit, mask=None, tau=1.0,
                       chunk=None, flags=0, *, dW=None, row_loss=True,
                       workspace=None, stream=None, sync=False):
    """Loss, per-row KL, dH and dW of the top-K KL loss on the GPU.

    H [T,d] and W [V,d] (bf16 or fp32), topk_idx [T,K] int32, topk_logit
    [T,K] fp32 and mask [T] (uint8/bool or None) are CUDA tensors.  Outputs
    are allocated here (``dW`` may be passed in, e.g. with
    KD_FLAG_ACCUMULATE_DW).  Returns (loss[1], row_loss[T] or None, dH, dW).
    """
    import torch
    lib = load_library()
    T, d, V, K, chunk, dt = _loss_inputs(H, W, topk_idx, topk_logit, mask, chunk)
    dev = H.device
    if dW is not None and (dW.shape != (V, d) or dW.dtype != torch.float32
                           or not dW.is_contiguous() or dW.device != dev):
        raise ValueError("dW must be float32 [V, d] on H's device")
    with _Call(dev, stream, sync) as call:
        mask = _mask_u8(mask)
        workspace = _workspace(T, d, V, K, chunk, dt, workspace, dev)
        f32 = dict(dtype=torch.float32, device=dev)
        loss = torch.empty(1, **f32)
        rl = torch.empty(T, **f32) if row_loss else None
        dH = torch.empty(T, d, **f32)
        if dW is None:
            dW = torch.empty(V, d, **f32)
        _check(lib.kd_topk_kl_fwd_bwd(
            H.data_ptr(), W.data_ptr(), dt, topk_idx.data_ptr(),
            topk_logit.data_ptr(), _ptr(mask), T, d, V, K, float(tau), chunk,
            int(flags), loss.data_ptr(), _ptr(rl), dH.data_ptr(),
            dW.data_ptr(), workspace.data_ptr(), workspace.numel(),
            call.handle))
    return loss, rl, dH, dW


kd_topk_kl_fwd_bwd.__doc__ += _STREAM_DOC


def kd_topk_kl_fwd(H, W, topk_idx, topk_logit, mask=None, tau=1.0,
                   chunk=None, *, row_loss=True, lse=True, workspace=None,
                   stream=None, sync=False):
    """The loss alone.  Returns (loss[1], row_loss[T] or None, lse[T] or
    None); arguments as for kd_topk_kl_fwd_bwd."""
    import torch
    lib = load_library()
    T, d, V, K, chunk, dt = _loss_inputs(H, W, topk_idx, topk_logit, mask, chunk)
    dev = H.device
    with _Call(dev, stream, sync) as call:
        mask = _mask_u8(mask)
        workspace = _workspace(T, d, V, K, chunk, dt, workspace, dev,
                               size=kd_topk_kl_fwd_workspace_size)
        f32 = dict(dtype=torch.float32, device=dev)
        loss = torch.empty(1, **f32)
        rl = torch.empty(T, **f32) if row_loss else None
        ls = torch.empty(T, **f32) if lse else None
        _check(lib.kd_topk_kl_fwd(
            H.data_ptr(), W.data_ptr(), dt, topk_idx.data_ptr(),
            topk_logit.data_ptr(), _ptr(mask), T, d, V, K, float(tau), chunk,
            loss.data_ptr(), _ptr(rl), _ptr(ls), workspace.data_ptr(),
            workspace.numel(), call.handle))
    return loss, rl, ls


def kd_topk_kl_fwd_noalloc(H, W, topk_idx, topk_logit, mask=None, tau=1.0,
                           chunk=None, *, loss=None, row_loss=None, lse=None,
                           stream=None, sync=False):
    """kd_topk_kl_fwd without a workspace: the library's fixed per-GPU
    scratch (KD_NOALLOC_SCRATCH_BYTES) holds the intermediates, so the C call
    allocates nothing (for code under graph capture or other callers that
    cannot allocate).  ``loss`` ([1] fp32), ``row_loss`` and ``lse`` ([T]
    fp32) are output tensors to fill; ``loss`` None is allocated here, and
    ``row_loss`` / ``lse`` None are not produced.  A bool mask is converted
    (which allocates); pass uint8 to avoid it.  Calls that overlap on one GPU
    share the scratch and race.  Returns (loss, row_loss, lse)."""
    import torch
    lib = load_library()
    T, d, V, K, chunk, dt = _loss_inputs(H, W, topk_idx, topk_logit, mask, chunk)
    dev = H.device
    for name, t, n in (("loss", loss, 1), ("row_loss", row_loss, T), ("lse", lse, T)):
        if t is not None and (t.dtype != torch.float32 or t.numel() != n
                              or not t.is_contiguous() or t.device != dev):
            raise ValueError(f"{name} must be a contiguous float32 [{n}] tensor on H's device")
    with _Call(dev, stream, sync) as call:
        mask = _mask_u8(mask)
        if loss is None:
            loss = torch.empty(1, dtype=torch.float32, device=dev)
        _check(lib.kd_topk_kl_fwd_noalloc(
            H.data_ptr(), W.data_ptr(), dt, topk_idx.data_ptr(),
            topk_logit.data_ptr(), _ptr(mask), T, d, V, K, float(tau), chunk,
            loss.data_ptr(), _ptr(row_loss), _ptr(lse), call.handle))
    return loss, row_loss, lse


def kd_topk_kl_bwd(H, W, topk_idx, topk_logit, mask=None, tau=1.0,
                   chunk=None, flags=0, grad_loss=None, *, dW=None,
                   workspace=None, stream=None, sync=False):
    """dH and dW (fp32) of grad_loss * loss.  ``grad_loss`` is None (1) or a
    one-element fp32 CUDA tensor.  Returns (dH, dW); other arguments as for
    kd_topk_kl_fwd_bwd."""
    import torch
    lib = load_library()
    T, d, V, K, chunk, dt = _loss_inputs(H, W, topk_idx, topk_logit, mask, chunk)
    dev = H.device
    if grad_loss is not None and (grad_loss.dtype != torch.float32
                                  or grad_loss.numel() != 1
                                  or grad_loss.device != dev):
        raise ValueError("grad_loss must be one float32 value on H's device")
    if dW is not None and (dW.shape != (V, d) or dW.dtype != torch.float32
                           or not dW.is_contiguous() or dW.device != dev):
        raise ValueError("dW must be float32 [V, d] on H's device")
    with _Call(dev, stream, sync) as call:
        mask = _mask_u8(mask)
        if grad_loss is not None:
            grad_loss = grad_loss.contiguous()
        workspace = _workspace(T, d, V, K, chunk, dt, workspace, dev)
        f32 = dict(dtype=torch.float32, device=dev)
        dH = torch.empty(T, d, **f32)
        if dW is None:
            dW = torch.empty(V, d, **f32)
        _check(lib.kd_topk_kl_bwd(
            H.data_ptr(), W.data_ptr(), dt, topk_idx.data_ptr(),
            topk_logit.data_ptr(), _ptr(mask), T, d, V, K, float(tau), chunk,
            int(flags), _ptr(grad_loss), dH.data_ptr(), dW.data_ptr(),
            workspace.data_ptr(), workspace.numel(), call.handle))
    return dH, dW


def kd_topk_div_workspace_size(T, d, V, K) -> int:
    """Workspace bytes for kd_topk_div_fwd_bwd (see the C header)."""
    out = ctypes.c_size_t(0)
    _check(load_library().kd_topk_div_workspace_size(
        int(T), int(d), int(V), int(K), ctypes.byref(out)))
    return out.value


def kd_topk_div_fwd_bwd(kind, H, W, topk_idx, topk_logit, mask=None, tau=1.0,
                        flags=0, *, dW=None, row_loss=True, workspace=None,
                        stream=None, sync=False):
    """Reverse KL ("reverse_kl") or Jensen-Shannon ("jsd") divergence over
    the teacher's top-K support, with dH and dW (see the C header).  Inputs
    as for kd_topk_kl_fwd_bwd; returns (loss[1], row_loss[T] or None, dH,
    dW)."""
    import torch
    lib = load_library()
    code = DIVERGENCES.get(kind, kind)
    if code not in DIVERGENCES.values():
        raise ValueError(f"kind must be one of {sorted(DIVERGENCES)}")
    T, d, V, K, _, dt = _loss_inputs(H, W, topk_idx, topk_logit, mask, None)
    dev = H.device
    if dW is not None and (dW.shape != (V, d) or dW.dtype != torch.float32
                           or not dW.is_contiguous() or dW.device != dev):
        raise ValueError("dW must be float32 [V, d] on H's device")
    with _Call(dev, stream, sync) as call:
        mask = _mask_u8(mask)
        ws_bytes = kd_topk_div_workspace_size(T, d, V, K)
        if workspace is None:
            workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        elif workspace.numel() < ws_bytes:
            raise ValueError("workspace too small")
        f32 = dict(dtype=torch.float32, device=dev)
        loss = torch.empty(1, **f32)
        rl = torch.empty(T, **f32) if row_loss else None
        dH = torch.empty(T, d, **f32)
        if dW is None:
            dW = torch.empty(V, d, **f32)
        _check(lib.kd_topk_div_fwd_bwd(
            int(code), H.data_ptr(), W.data_ptr(), dt, topk_idx.data_ptr(),
            topk_logit.data_ptr(), _ptr(mask), T, d, V, K, float(tau),
            int(flags), loss.data_ptr(), _ptr(rl), dH.data_ptr(),
            dW.data_ptr(), workspace.data_ptr(), workspace.numel(),
            call.handle))
    return loss, rl, dH, dW


def kd_grad_cast(src, dtype, scale=None, *, out=None, stream=None, sync=False):
    """src (fp32 CUDA tensor) times scale (None or a one-element fp32 CUDA
    tensor) as a new tensor of torch dtype ``dtype`` (bfloat16 or float32),
    or into ``out``."""
    import torch
    lib = load_library()
    if src.dtype != torch.float32 or not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous float32 CUDA tensor")
    code = KD_BF16 if dtype == torch.bfloat16 else KD_F32 if dtype == torch.float32 else None
    if code is None:
        raise TypeError(f"unsupported dtype {dtype}")
    if out is not None and (out.dtype != dtype or out.shape != src.shape
                            or not out.is_contiguous()):
        raise ValueError("out must match src's shape and the dtype")
    if scale is not None and (scale.dtype != torch.float32 or scale.numel() != 1):
        raise ValueError("scale must be one float32 value")
    with _Call(src.device, stream, sync) as call:
        if out is None:
            out = torch.empty(src.shape, dtype=dtype, device=src.device)
        _check(lib.kd_grad_cast(src.data_ptr(), out.data_ptr(), code, src.numel(),
                                _ptr(scale), call.handle))
    return out


def kd_teacher_topk_workspace_size(T, d, V, K, chunk, dtype) -> int:
    """Workspace bytes for kd_teacher_topk (see the C header)."""
    out = ctypes.c_size_t(0)
    _check(load_library().kd_teacher_topk_workspace_size(
        int(T), int(d), int(V), int(K), int(chunk), int(dtype),
        ctypes.byref(out)))
    return out.value


def kd_teacher_topk(H, W, K, chunk=None, *, workspace=None, stream=None,
                    sync=False):
    """Teacher top-K cache on the GPU: for each row of z = H W^T, the K
    largest logits (fp32) and their ids (int32), by logit descending and
    equal logits by id ascending.  H [T,d] and W [V,d] are bf16 or fp32
    CUDA tensors.  Returns (ids [T,K], logits [T,K]).  ``stream`` and
    ``sync`` as for kd_topk_kl_fwd_bwd."""
    import torch
    lib = load_library()
    T, d = H.shape
    V = W.shape[0]
    chunk = T if chunk is None else int(chunk)
    dt = _dtype_code(H)
    if W.dtype != H.dtype or W.shape[1] != d:
        raise ValueError("W must be [V, d] with H's dtype")
    dev = H.device
    for t in (H, W):
        if not t.is_cuda or t.device != dev or not t.is_contiguous():
            raise ValueError("H and W must be contiguous tensors on one GPU")
    ws_bytes = kd_teacher_topk_workspace_size(T, d, V, K, chunk, dt)
    with _Call(dev, stream, sync) as call:
        if workspace is None:
            workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        elif workspace.numel() < ws_bytes:
            raise ValueError("workspace too small")
        ids = torch.empty(T, int(K), dtype=torch.int32, device=dev)
        vals = torch.empty(T, int(K), dtype=torch.float32, device=dev)
        _check(lib.kd_teacher_topk(
            H.data_ptr(), W.data_ptr(), dt, T, d, V, int(K), chunk,
            ids.data_ptr(), vals.data_ptr(), workspace.data_ptr(),
            workspace.numel(), call.handle))
    return ids, vals


def kd_entropy_filter_workspace_size(T) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().kd_entropy_filter_workspace_size(int(T), ctypes.byref(out)))
    return out.value


def kd_entropy_filter(topk_logit, mask=None, tau=1.0, mode="above", param=0.5,
                      *, entropy=True, workspace=None, stream=None, sync=False):
    """Token mask from the teacher's entropy over its K cached logits (see
    the C header).  mode "above": keep valid tokens with entropy > param;
    "top_fraction": keep round(param * N) valid tokens of highest entropy.
    Returns (mask_out uint8 [T], entropy fp32 [T] or None)."""
    import torch
    lib = load_library()
    codes = {"above": KD_FILTER_ENTROPY_ABOVE,
             "top_fraction": KD_FILTER_TOP_ENTROPY_FRACTION}
    if mode not in codes:
        raise ValueError(f"mode must be one of {sorted(codes)}")
    T, K = topk_logit.shape
    if topk_logit.dtype != torch.float32 or not topk_logit.is_cuda or \
            not topk_logit.is_contiguous():
        raise ValueError("topk_logit must be a contiguous float32 CUDA tensor")
    dev = topk_logit.device
    if mask is not None and (mask.dtype not in (torch.bool, torch.uint8)
                             or mask.numel() != T or mask.device != dev):
        raise ValueError("mask must be uint8/bool [T] on the logits' device")
    ws_bytes = kd_entropy_filter_workspace_size(T)
    with _Call(dev, stream, sync) as call:
        if mask is not None:
            mask = _mask_u8(mask).contiguous()
        if workspace is None:
            workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        elif workspace.numel() < ws_bytes:
            raise ValueError("workspace too small")
        out = torch.empty(T, dtype=torch.uint8, device=dev)
        ent = torch.empty(T, dtype=torch.float32, device=dev) if entropy else None
        _check(lib.kd_entropy_filter(
            topk_logit.data_ptr(), _ptr(mask), T, K, float(tau), codes[mode],
            float(param), out.data_ptr(), _ptr(ent), workspace.data_ptr(),
            workspace.numel(), call.handle))
    return out, ent
