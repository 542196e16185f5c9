"""Plain fp64 CPU oracle for the teacher top-K cache (the offline step).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
executes this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code with the
HIP library (``top_kl_loss_amd``).

What is computed, and where the pages say so
--------------------------------------------
"Making Knowledge Distillation Cheap Enough to Run at Scale" (aipuls.nl),
section "Summary": the teacher model runs once over the data and only its
100 largest logits per token position are kept, with their vocabulary ids;
the student's loss later reads that cache.  The pages do not say how the
cache is built; this oracle is the definition written out:

    z[t, v] = sum_j H[t, j] W[v, j]        (teacher LM-head logits, no bias)
    cache[t] = the K pairs (v, z[t, v]) that come first when the row's
               entries are ordered by z descending, equal z by v ascending

Readings where the pages are silent:

* T1  no temperature is applied in the cache (the loss applies tau to the
      cached logits itself);
* T2  ties in z are broken by the smaller id (any fixed rule would do; this
      one makes the cache a function of the inputs); -0 equals +0;
* T3  the stored logit is z itself, accumulated in fp64 here; the library
      accumulates in fp32, so parity compares values within a rounding
      tolerance and compares the id sets wherever the order is not decided
      by values closer than that tolerance.

Parity status: pinned in ``tests/test_oracle.py`` by a pure-Python brute
force on integer-valued inputs (exact sums, many ties), a hand-worked golden
example (``tests/golden/teacher_topk_hand.json``) and invariances.
"""
from __future__ import annotations

import numpy as np

__all__ = ["teacher_logits", "teacher_topk_cache"]


def teacher_logits(H, W):
    """z = H W^T in fp64 (the teacher's LM-head logits; reading T1)."""
    return np.asarray(H, dtype=np.float64) @ np.asarray(W, dtype=np.float64).T


def teacher_topk_cache(H, W, K, rows_per_block=256):
    """(ids int32 [T, K], logits fp64 [T, K]) of the K best entries of each
    row of z = H W^T: z descending, equal z by id ascending (reading T2).
    ("Making Knowledge Distillation Cheap Enough to Run at Scale",
    aipuls.nl, section "Summary": top-100 logits per position are cached.)
    """
    H = np.asarray(H, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    T, V = H.shape[0], W.shape[0]
    if not 1 <= K <= V:
        raise ValueError("need 1 <= K <= V")
    ids = np.empty((T, K), dtype=np.int32)
    vals = np.empty((T, K), dtype=np.float64)
    col = np.arange(V)
    for r0 in range(0, T, rows_per_block):
        z = teacher_logits(H[r0:r0 + rows_per_block], W)
        for i in range(z.shape[0]):
            # primary key: -z (descending z); secondary: id ascending.
            # -0.0 and +0.0 compare equal, so they tie and go by id.
            order = np.lexsort((col, -z[i]))[:K]
            ids[r0 + i] = order
            vals[r0 + i] = z[i, order]
    return ids, vals
