"""Python binding of libkdtopk.so, the MI355X fused chunked top-K KL loss.

Argument marshalling only: every step of the loss runs in the HIP kernels of
the C library (``include/kd_topk_kl.h``).  PyTorch provides device memory.
There is no fallback: if the library is missing or cannot be loaded, every
call raises.

PyTorch-ROCm carries its own HIP runtime, separate from the one the library
is linked against, so the binding orders the two by host synchronisation:
torch's pending work is finished before the library call, and the library's
stream is synchronised before results are handed back (``sync=True``).
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "KD_F32", "KD_BF16", "KD_FLAG_ACCUMULATE_DW", "KD_MAX_K", "LIB_PATH",
    "KdError", "load_library", "kd_topk_kl_workspace_size",
    "kd_topk_kl_fwd_bwd", "kd_status_string", "kd_set_launch_log",
    "EXPORTED_SYMBOLS", "KERNEL_NAMES", "KD_TOPK_MAX_K", "KD_TOPK_MAX_D",
    "kd_teacher_topk_workspace_size", "kd_teacher_topk", "kd_topk_kl_fwd",
    "kd_topk_kl_bwd", "kd_grad_cast", "kd_entropy_filter",
    "kd_entropy_filter_workspace_size", "KD_FILTER_ENTROPY_ABOVE",
    "KD_FILTER_TOP_ENTROPY_FRACTION",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkdtopk.so")

KD_F32, KD_BF16 = 0, 1
KD_OK, KD_ERR_INVALID_ARG, KD_ERR_WORKSPACE, KD_ERR_UNSUPPORTED, KD_ERR_HIP = range(5)
KD_FLAG_ACCUMULATE_DW = 1
KD_MAX_K = 1024
KD_TOPK_MAX_K = 256
KD_TOPK_MAX_D = 16384
EXPORTED_SYMBOLS = ("kd_topk_kl_workspace_size", "kd_topk_kl_fwd_bwd",
                    "kd_status_string", "kd_set_launch_log",
                    "kd_teacher_topk_workspace_size", "kd_teacher_topk",
                    "kd_topk_kl_fwd", "kd_topk_kl_bwd", "kd_grad_cast",
                    "kd_entropy_filter_workspace_size", "kd_entropy_filter")
KD_FILTER_ENTROPY_ABOVE, KD_FILTER_TOP_ENTROPY_FRACTION = 0, 1
# Kernel ids of the launch log (KD_KERNEL_* in the header).
KERNEL_NAMES = ("valid_count", "prep_rows", "gemm_logits", "lse_fix",
                "gemm_dh", "reduce_dh", "gemm_dw", "final_loss", "transpose_h",
                "scale_g", "transpose_w", "tk_sample", "tk_theta", "tk_filter",
                "tk_select", "tk_stream", "grad_cast", "entropy_filter")

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
    lib = ctypes.CDLL(path)
    c = ctypes
    lib.kd_topk_kl_workspace_size.argtypes = [
        c.c_int64, c.c_int64, c.c_int64, c.c_int32, c.c_int32, c.c_int,
        c.POINTER(c.c_size_t)]
    lib.kd_topk_kl_workspace_size.restype = c.c_int
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
    lib.kd_topk_kl_bwd.argtypes = [
        c.c_void_p, c.c_void_p, c.c_int, c.c_void_p, c.c_void_p, c.c_void_p,
        c.c_int64, c.c_int64, c.c_int64, c.c_int32, c.c_float, c.c_int32,
        c.c_uint32, c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p,
        c.c_size_t, c.c_void_p]
    lib.kd_topk_kl_bwd.restype = c.c_int
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


def _loss_inputs(H, W, topk_idx, topk_logit, mask, chunk):
    """Validates the loss inputs; returns (T, d, V, K, chunk, dtype code,
    mask as uint8 or None)."""
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
        if mask.dtype == torch.bool:
            mask = mask.to(torch.uint8)
        if mask.dtype != torch.uint8 or mask.numel() != T:
            raise ValueError("mask must be uint8/bool [T]")
        tensors.append(mask)
    dev = H.device
    for t in tensors:
        if not t.is_cuda or t.device != dev or not t.is_contiguous():
            raise ValueError("all inputs must be contiguous tensors on one GPU")
    return T, d, V, K, chunk, dt, mask


def _workspace(T, d, V, K, chunk, dt, workspace, dev):
    import torch
    ws_bytes = kd_topk_kl_workspace_size(T, d, V, K, chunk, dt)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    elif workspace.numel() < ws_bytes:
        raise ValueError("workspace too small")
    return workspace


def _enter(dev):
    """Orders the library's work after torch's pending work."""
    import torch
    from . import hip
    torch.cuda.synchronize(dev)          # inputs written by torch are ready
    hip.set_device(dev.index if dev.index is not None else 0)


def _leave(stream, sync):
    if sync:
        from . import hip
        hip.synchronize(stream)


def kd_topk_kl_fwd_bwd(H, W, topk_idx, topk_logit, mask=None, tau=1.0,
                       chunk=None, flags=0, *, dW=None, row_loss=True,
                       workspace=None, stream=None, sync=True):
    """Loss, per-row KL, dH and dW of the top-K KL loss on the GPU.

    H [T,d] and W [V,d] (bf16 or fp32), topk_idx [T,K] int32, topk_logit
    [T,K] fp32 and mask [T] (uint8/bool or None) are CUDA tensors.  Outputs
    are allocated here (``dW`` may be passed in, e.g. with
    KD_FLAG_ACCUMULATE_DW).  Returns (loss[1], row_loss[T] or None, dH, dW).

    ``stream`` is a stream handle of the library's HIP runtime
    (``top_kl_loss_amd.hip.Stream().value``) or None for its null stream.
    With ``sync=False`` the call returns as soon as the work is enqueued;
    the caller must then keep every tensor alive and synchronise the stream
    (``top_kl_loss_amd.hip.synchronize``) before torch touches the results.
    """
    import torch
    lib = load_library()
    T, d, V, K, chunk, dt, mask = _loss_inputs(H, W, topk_idx, topk_logit, mask, chunk)
    dev = H.device
    workspace = _workspace(T, d, V, K, chunk, dt, workspace, dev)
    f32 = dict(dtype=torch.float32, device=dev)
    loss = torch.empty(1, **f32)
    rl = torch.empty(T, **f32) if row_loss else None
    dH = torch.empty(T, d, **f32)
    if dW is None:
        dW = torch.empty(V, d, **f32)
    elif dW.shape != (V, d) or dW.dtype != torch.float32 or not dW.is_contiguous():
        raise ValueError("dW must be float32 [V, d]")
    _enter(dev)
    _check(lib.kd_topk_kl_fwd_bwd(
        H.data_ptr(), W.data_ptr(), dt, topk_idx.data_ptr(),
        topk_logit.data_ptr(), mask.data_ptr() if mask is not None else None,
        T, d, V, K, float(tau), chunk, int(flags), loss.data_ptr(),
        rl.data_ptr() if rl is not None else None, dH.data_ptr(),
        dW.data_ptr(), workspace.data_ptr(), workspace.numel(), stream))
    _leave(stream, sync)
    return loss, rl, dH, dW


def kd_topk_kl_fwd(H, W, topk_idx, topk_logit, mask=None, tau=1.0,
                   chunk=None, *, row_loss=True, lse=True, workspace=None,
                   stream=None, sync=True):
    """The loss alone.  Returns (loss[1], row_loss[T] or None, lse[T] or
    None); arguments as for kd_topk_kl_fwd_bwd."""
    import torch
    lib = load_library()
    T, d, V, K, chunk, dt, mask = _loss_inputs(H, W, topk_idx, topk_logit, mask, chunk)
    dev = H.device
    workspace = _workspace(T, d, V, K, chunk, dt, workspace, dev)
    f32 = dict(dtype=torch.float32, device=dev)
    loss = torch.empty(1, **f32)
    rl = torch.empty(T, **f32) if row_loss else None
    ls = torch.empty(T, **f32) if lse else None
    _enter(dev)
    _check(lib.kd_topk_kl_fwd(
        H.data_ptr(), W.data_ptr(), dt, topk_idx.data_ptr(),
        topk_logit.data_ptr(), mask.data_ptr() if mask is not None else None,
        T, d, V, K, float(tau), chunk, loss.data_ptr(),
        rl.data_ptr() if rl is not None else None,
        ls.data_ptr() if ls is not None else None,
        workspace.data_ptr(), workspace.numel(), stream))
    _leave(stream, sync)
    return loss, rl, ls


def kd_topk_kl_bwd(H, W, topk_idx, topk_logit, mask=None, tau=1.0,
                   chunk=None, flags=0, grad_loss=None, *, dW=None,
                   workspace=None, stream=None, sync=True):
    """dH and dW (fp32) of grad_loss * loss.  ``grad_loss`` is None (1) or a
    one-element fp32 CUDA tensor.  Returns (dH, dW)."""
    import torch
    lib = load_library()
    T, d, V, K, chunk, dt, mask = _loss_inputs(H, W, topk_idx, topk_logit, mask, chunk)
    dev = H.device
    if grad_loss is not None:
        if (grad_loss.dtype != torch.float32 or grad_loss.numel() != 1
                or grad_loss.device != dev):
            raise ValueError("grad_loss must be one float32 value on H's device")
        grad_loss = grad_loss.contiguous()
    workspace = _workspace(T, d, V, K, chunk, dt, workspace, dev)
    f32 = dict(dtype=torch.float32, device=dev)
    dH = torch.empty(T, d, **f32)
    if dW is None:
        dW = torch.empty(V, d, **f32)
    elif dW.shape != (V, d) or dW.dtype != torch.float32 or not dW.is_contiguous():
        raise ValueError("dW must be float32 [V, d]")
    _enter(dev)
    _check(lib.kd_topk_kl_bwd(
        H.data_ptr(), W.data_ptr(), dt, topk_idx.data_ptr(),
        topk_logit.data_ptr(), mask.data_ptr() if mask is not None else None,
        T, d, V, K, float(tau), chunk, int(flags),
        grad_loss.data_ptr() if grad_loss is not None else None,
        dH.data_ptr(), dW.data_ptr(), workspace.data_ptr(), workspace.numel(),
        stream))
    _leave(stream, sync)
    return dH, dW


def kd_grad_cast(src, dtype, scale=None, *, out=None, stream=None, sync=True):
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
    if out is None:
        out = torch.empty(src.shape, dtype=dtype, device=src.device)
    elif out.dtype != dtype or out.shape != src.shape or not out.is_contiguous():
        raise ValueError("out must match src's shape and the dtype")
    if scale is not None and (scale.dtype != torch.float32 or scale.numel() != 1):
        raise ValueError("scale must be one float32 value")
    _enter(src.device)
    _check(lib.kd_grad_cast(src.data_ptr(), out.data_ptr(), code, src.numel(),
                            scale.data_ptr() if scale is not None else None,
                            stream))
    _leave(stream, sync)
    return out


def kd_teacher_topk_workspace_size(T, d, V, K, chunk, dtype) -> int:
    """Workspace bytes for kd_teacher_topk (see the C header)."""
    out = ctypes.c_size_t(0)
    _check(load_library().kd_teacher_topk_workspace_size(
        int(T), int(d), int(V), int(K), int(chunk), int(dtype),
        ctypes.byref(out)))
    return out.value


def kd_teacher_topk(H, W, K, chunk=None, *, workspace=None, stream=None,
                    sync=True):
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
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    elif workspace.numel() < ws_bytes:
        raise ValueError("workspace too small")
    ids = torch.empty(T, int(K), dtype=torch.int32, device=dev)
    vals = torch.empty(T, int(K), dtype=torch.float32, device=dev)
    from . import hip
    torch.cuda.synchronize(dev)
    hip.set_device(dev.index if dev.index is not None else 0)
    _check(lib.kd_teacher_topk(
        H.data_ptr(), W.data_ptr(), dt, T, d, V, int(K), chunk,
        ids.data_ptr(), vals.data_ptr(), workspace.data_ptr(),
        workspace.numel(), stream))
    if sync:
        hip.synchronize(stream)
    return ids, vals


def kd_entropy_filter_workspace_size(T) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().kd_entropy_filter_workspace_size(int(T), ctypes.byref(out)))
    return out.value


def kd_entropy_filter(topk_logit, mask=None, tau=1.0, mode="above", param=0.5,
                      *, entropy=True, workspace=None, stream=None, sync=True):
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
    if mask is not None:
        if mask.dtype == torch.bool:
            mask = mask.to(torch.uint8)
        if mask.dtype != torch.uint8 or mask.numel() != T or mask.device != dev:
            raise ValueError("mask must be uint8/bool [T] on the logits' device")
        mask = mask.contiguous()
    ws_bytes = kd_entropy_filter_workspace_size(T)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    elif workspace.numel() < ws_bytes:
        raise ValueError("workspace too small")
    out = torch.empty(T, dtype=torch.uint8, device=dev)
    ent = torch.empty(T, dtype=torch.float32, device=dev) if entropy else None
    _enter(dev)
    _check(lib.kd_entropy_filter(
        topk_logit.data_ptr(), mask.data_ptr() if mask is not None else None,
        T, K, float(tau), codes[mode], float(param), out.data_ptr(),
        ent.data_ptr() if ent is not None else None, workspace.data_ptr(),
        workspace.numel(), stream))
    _leave(stream, sync)
    return out, ent
