"""Seeded synthetic inputs for the top-K KL loss.

This module only draws and encodes inputs; it holds none of the loss's
arithmetic.  It serves both the oracle and the HIP library: both receive
the very same values (bf16 inputs are rounded here, once, and handed to the
oracle as their exact fp32 values and to the GPU as their bit patterns).

Workloads (the pages quote a 201k vocabulary, 8k and 32k contexts and a
top-100 teacher cache; the hidden size, distributions and masks below are
this repository's choice for synthetic stand-ins):

  tiny         T=256   d=512  V=8192   fp32  tau=1  no mask  chunk=64
               ids: 100 distinct uniform ids per row; logits ~ N(0, 2^2)
               sorted descending, independent of the ids
  t4k          T=4096  d=2880 V=201088 bf16  tau=1  no mask  chunk=1024
  t8k          T=8192  d=2880 V=201088 bf16  tau=1  5% masked chunk=1024
  t32k         T=32768 d=2880 V=201088 bf16  tau=1  no mask  chunk=8192
               (the pages fix no slice size here; 8192 halves the dW
               read-modify-writes of 4096 for 8.1 GB of workspace)
  t32k_d4096   T=32768 d=4096 V=151936 bf16  tau=2  15% masked, teacher
               logits x0.5, chunk sweep {512, 1024, 2048, 4096}

For every workload H ~ N(0,1) and W ~ N(0, 1/d).  For the bf16 workloads
the teacher cache holds the 100 largest entries of z_t = H W_t^T (W_t a
fresh N(0, 1/d) head, computed in fp32 from the rounded H), ids int32 and
logits fp32, sorted descending.  Masks mark exactly round(p*T) positions,
drawn uniformly without replacement, as padding (0); the rest are 1.

Seeds: numpy PCG64 with seed = 1000*case + stream, stream H:0 W:1 W_t:2
mask:3 idx:4 logit:5.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"

WORKLOADS = {
    "tiny": dict(case=0, T=256, d=512, V=8192, K=100, dtype=F32, tau=1.0,
                 mask_frac=0.0, chunk=64, cache="uniform", logit_scale=1.0),
    "t4k": dict(case=1, T=4096, d=2880, V=201088, K=100, dtype=BF16, tau=1.0,
                mask_frac=0.0, chunk=1024, cache="teacher", logit_scale=1.0),
    "t8k": dict(case=2, T=8192, d=2880, V=201088, K=100, dtype=BF16, tau=1.0,
                mask_frac=0.05, chunk=1024, cache="teacher", logit_scale=1.0),
    "t32k": dict(case=3, T=32768, d=2880, V=201088, K=100, dtype=BF16,
                 tau=1.0, mask_frac=0.0, chunk=8192, cache="teacher",
                 logit_scale=1.0),
    "t32k_d4096": dict(case=4, T=32768, d=4096, V=151936, K=100, dtype=BF16,
                       tau=2.0, mask_frac=0.15, chunk=1024, cache="teacher",
                       logit_scale=0.5),
}
CHUNK_SWEEP = {"t32k_d4096": (512, 1024, 2048, 4096)}


def f32_to_bf16_bits(x):
    """Round fp32 to bf16 (round to nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b):
    """Exact fp32 value of bf16 bit patterns."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Inputs:
    """One synthetic problem.  ``H``/``W`` hold exact fp32 values; for bf16
    problems ``H_bits``/``W_bits`` hold the bf16 patterns of the same
    values."""
    name: str
    T: int
    d: int
    V: int
    K: int
    dtype: str
    tau: float
    chunk: int
    H: np.ndarray
    W: np.ndarray
    topk_idx: np.ndarray
    topk_logit: np.ndarray
    mask: Optional[np.ndarray]
    H_bits: Optional[np.ndarray] = None
    W_bits: Optional[np.ndarray] = None

    @property
    def n_valid(self) -> int:
        return self.T if self.mask is None else int(self.mask.sum())


def _rng(case, stream):
    return np.random.Generator(np.random.PCG64(1000 * case + stream))


def _normal(case, stream, shape, std):
    x = _rng(case, stream).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def uniform_cache(case, T, V, K, logit_std=2.0):
    """K distinct uniform ids per row; logits ~ N(0, std^2) sorted
    descending, drawn independently of the ids."""
    rng = _rng(case, 4)
    idx = np.empty((T, K), dtype=np.int32)
    for r0 in range(0, T, 256):
        r1 = min(T, r0 + 256)
        keys = rng.random((r1 - r0, V), dtype=np.float32)
        idx[r0:r1] = np.argpartition(keys, K - 1, axis=1)[:, :K]
    logit = _rng(case, 5).standard_normal((T, K), dtype=np.float32)
    logit *= np.float32(logit_std)
    logit = -np.sort(-logit, axis=1)
    return idx, np.ascontiguousarray(logit)


def teacher_topk(H32, Wt32, K, device=None, rows_per_block=1024):
    """Top-K (ids, values) of z_t = H W_t^T per row, sorted descending.

    ``device`` None runs numpy fp32 on the host; a torch device string runs
    torch fp32 matmul + topk there (only a faster way to draw the same kind
    of input; ties are measure-zero).
    """
    T = H32.shape[0]
    idx = np.empty((T, K), dtype=np.int32)
    val = np.empty((T, K), dtype=np.float32)
    if device is None:
        for r0 in range(0, T, rows_per_block):
            z = H32[r0:r0 + rows_per_block] @ Wt32.T
            part = np.argpartition(-z, K - 1, axis=1)[:, :K]
            pv = np.take_along_axis(z, part, axis=1)
            order = np.lexsort((part, -pv), axis=1)
            idx[r0:r0 + rows_per_block] = np.take_along_axis(part, order, 1)
            val[r0:r0 + rows_per_block] = np.take_along_axis(pv, order, 1)
        return idx, val
    import torch
    Wt = torch.from_numpy(Wt32).to(device)
    for r0 in range(0, T, rows_per_block):
        h = torch.from_numpy(H32[r0:r0 + rows_per_block]).to(device)
        z = h @ Wt.T
        v, i = torch.topk(z, K, dim=1, largest=True, sorted=True)
        idx[r0:r0 + rows_per_block] = i.to(torch.int32).cpu().numpy()
        val[r0:r0 + rows_per_block] = v.cpu().numpy()
    del Wt
    return idx, val


def exact_mask(case, T, frac):
    """uint8 mask with exactly round(frac*T) zeros at uniform positions."""
    n_masked = int(round(frac * T))
    if n_masked == 0:
        return None
    m = np.ones(T, dtype=np.uint8)
    m[_rng(case, 3).choice(T, size=n_masked, replace=False)] = 0
    return m


def make_case(name="custom", *, case, T, d, V, K, dtype, tau=1.0,
              mask_frac=0.0, chunk=None, cache="uniform", logit_scale=1.0,
              teacher_device=None, h_std=1.0, self_noise=0.0):
    """Draw one problem.  ``cache`` is "uniform" (random distinct ids),
    "teacher" (top-K of a random teacher head) or "self" (top-K of the
    student's own logits, plus N(0, self_noise^2) on each logit)."""
    H = _normal(case, 0, (T, d), h_std)
    W = _normal(case, 1, (V, d), 1.0 / np.sqrt(d))
    H_bits = W_bits = None
    if dtype == BF16:
        H_bits = f32_to_bf16_bits(H)
        W_bits = f32_to_bf16_bits(W)
        H = bf16_bits_to_f32(H_bits)
        W = bf16_bits_to_f32(W_bits)
    elif dtype != F32:
        raise ValueError(dtype)
    if cache == "uniform":
        idx, logit = uniform_cache(case, T, V, K)
    elif cache == "teacher":
        Wt = _normal(case, 2, (V, d), 1.0 / np.sqrt(d))
        idx, logit = teacher_topk(H, Wt, K, device=teacher_device)
        del Wt
    elif cache == "self":
        # the student's own top-K logits plus N(0, self_noise^2): a teacher
        # the student already matches up to the noise and the mass outside
        # its top K (the near-converged regime, KL close to 0)
        idx, logit = teacher_topk(H, W, K, device=teacher_device)
        if self_noise:
            logit = logit + _normal(case, 5, logit.shape, self_noise)
            order = np.argsort(-logit, axis=1, kind="stable")
            idx = np.take_along_axis(idx, order, 1)
            logit = np.take_along_axis(logit, order, 1)
    else:
        raise ValueError(cache)
    if logit_scale != 1.0:
        logit = logit * np.float32(logit_scale)
    mask = exact_mask(case, T, mask_frac)
    return Inputs(name=name, T=T, d=d, V=V, K=K, dtype=dtype, tau=float(tau),
                  chunk=int(chunk if chunk is not None else T), H=H, W=W,
                  topk_idx=np.ascontiguousarray(idx, dtype=np.int32),
                  topk_logit=np.ascontiguousarray(logit, dtype=np.float32),
                  mask=mask, H_bits=H_bits, W_bits=W_bits)


def workload(name, teacher_device=None, **overrides):
    """One of the named workloads (see the module docstring)."""
    spec = dict(WORKLOADS[name])
    spec.update(overrides)
    return make_case(name, teacher_device=teacher_device, **spec)


# ------------------------------------------------ teacher top-K cache inputs
@dataclasses.dataclass
class TeacherHead:
    """Teacher hidden states H [T, d] and LM head W [V, d] (exact fp32
    values; bf16 bit patterns too when dtype is bf16)."""
    name: str
    T: int
    d: int
    V: int
    dtype: str
    H: np.ndarray
    W: np.ndarray
    H_bits: Optional[np.ndarray] = None
    W_bits: Optional[np.ndarray] = None


def _encode(name, H, W, dtype):
    H = np.ascontiguousarray(H, dtype=np.float32)
    W = np.ascontiguousarray(W, dtype=np.float32)
    Hb = Wb = None
    if dtype == BF16:
        Hb, Wb = f32_to_bf16_bits(H), f32_to_bf16_bits(W)
        H, W = bf16_bits_to_f32(Hb), bf16_bits_to_f32(Wb)
    elif dtype != F32:
        raise ValueError(dtype)
    return TeacherHead(name=name, T=H.shape[0], d=H.shape[1], V=W.shape[0],
                       dtype=dtype, H=H, W=W, H_bits=Hb, W_bits=Wb)


def teacher_head(name="teacher", *, case, T, d, V, dtype=BF16, h_std=1.0):
    """H ~ N(0, h_std^2) (stream 0) and W ~ N(0, 1/d) (stream 2, the
    teacher head of the loss workloads)."""
    return _encode(name, _normal(case, 0, (T, d), h_std),
                   _normal(case, 2, (V, d), 1.0 / np.sqrt(d)), dtype)


def teacher_head_integer(name="teacher_int", *, case, T, d, V, lo=-2, hi=2,
                         zero_rows=(), dtype=BF16):
    """Integer entries uniform in [lo, hi] (exact in bf16; with small d
    every logit is an exact integer in fp32, so ties are frequent and
    exact).  Rows listed in ``zero_rows`` of H are all zero."""
    H = _rng(case, 0).integers(lo, hi + 1, size=(T, d)).astype(np.float32)
    W = _rng(case, 2).integers(lo, hi + 1, size=(V, d)).astype(np.float32)
    for r in zero_rows:
        H[r] = 0.0
    return _encode(name, H, W, dtype)


def teacher_head_split(name="teacher_split", *, case, T, d, V, marked_segments,
                       seg=256, dtype=BF16):
    """Two families of vocabulary rows: ids in ``marked_segments`` (segment
    width ``seg``) use only the first d/2 hidden dimensions, every other id
    only the last d/2.  Even token rows use only the first half of H, odd
    rows only the second half, so an even row has non-zero logits only on
    the marked segments and an odd row only off them."""
    H = _normal(case, 0, (T, d), 1.0)
    W = _normal(case, 2, (V, d), 1.0 / np.sqrt(d / 2))
    h = d // 2
    marked = np.zeros(V, dtype=bool)
    for s in marked_segments:
        marked[s * seg:(s + 1) * seg] = True
    W[marked, h:] = 0.0
    W[~marked, :h] = 0.0
    H[0::2, h:] = 0.0
    H[1::2, :h] = 0.0
    return _encode(name, H, W, dtype)
