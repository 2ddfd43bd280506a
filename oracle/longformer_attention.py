"""fp64 CPU oracle for the Longformer combined sliding-window + global
attention forward.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or
executes this module; only the test suite, the smoke check and the CPU
baseline leg of the benchmark do.  It shares no code with the HIP library.

What is computed (plain definition; sparse attention is exact on its
pattern, so the definition is the oracle):

* Sliding window.  Each token attends a fixed-size window of neighbours on
  both sides (segmentfault Longformer summary, "Sliding window";
  ultralytics glossary, "How Longformer attention works": 256 per side in
  the released models).  The one-sided width ``w`` is inclusive: the worked
  mask example on the ultralytics page keeps pairs with |i - j| <= window/2,
  so a row has 2w + 1 window keys.
* Dilation.  The window may have gaps of size d between attended positions
  (segmentfault summary, "Dilated sliding window").  Reading: stride d,
  keys i + k*d for k in [-w, w]; d = 1 is the plain window.
* Causal.  The autoregressive character LM uses the dilated window
  (segmentfault summary, "Implementation").  Reading: k in [-w, 0].
* Global attention is symmetric: a global token attends to every token and
  every token attends to it (segmentfault summary, "Global attention";
  ultralytics glossary, third bullet).  The worked mask example sets row 0
  and column 0 of a boolean mask, i.e. a set union: a global key already
  inside the window is counted once.
* Separate projections: Q_s/K_s/V_s score the sliding-window attention,
  Q_g/K_g/V_g the global attention (segmentfault summary, "Linear
  projections for global attention").  Reading: global rows use
  Q_g K_g^T and V_g over every valid token; local rows use Q_s K_s^T and V_s
  for both their window keys and their global columns.
* Mask values (allenai README, "Usage", run-the-model step): 0 = no
  attention, 1 = local, 2 = global.  Reading: mask-0 tokens are excluded as
  keys everywhere and their own output row is exactly zero.
* Scale: 1/sqrt(D) unless given (the pages are silent).

Parity unpinned (no page fixes them; conventions this oracle and the HIP
path both follow): the projections that score a local row's global columns
(Q_s K_s and V_s), the exactly-zero output row of a mask-0 token, and mask
2 under a causal window (rejected here).

``forward`` gathers each row's key set (window keys by arithmetic plus the
global columns outside the window) and runs a softmax per row in fp64.
``dense_bruteforce`` builds the full n x n boolean pattern the way the
ultralytics worked example does and runs a masked dense softmax; it is an
independent formulation for tiny n.  ``pair_count`` is the number of scored
pairs, the quantity the worked example prints.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

ROW_BLOCK = 128


def _check(q, mask, window, dilation, causal):
    if q.ndim != 4:
        raise ValueError("q must be [B, n, H, D]")
    B, n, H, D = q.shape
    mask = np.asarray(mask)
    if mask.shape != (B, n):
        raise ValueError("mask must be [B, n]")
    if not np.isin(mask, (0, 1, 2)).all():
        raise ValueError("mask values must be 0, 1 or 2")
    if window < 0:
        raise ValueError("window must be >= 0")
    dil = [1] * H if dilation is None else [int(x) for x in dilation]
    if len(dil) != H or min(dil) < 1:
        raise ValueError("dilation must have H entries >= 1")
    if causal and (mask == 2).any():
        # Global attention is described for fine-tuning tasks only; the
        # autoregressive LM uses none.  The combination is left undefined.
        raise ValueError("causal attention with global tokens is undefined")
    return B, n, H, D, mask, dil


def in_window(i, j, w: int, dil: int, causal: bool):
    """Membership j in W(i), elementwise over broadcast integer arrays."""
    d = np.asarray(i) - np.asarray(j)
    ok = (np.abs(d) <= w * dil) & (d % dil == 0)
    if causal:
        ok &= d >= 0
    return ok


def _softmax_rows(e: np.ndarray) -> np.ndarray:
    """Exact fp64 softmax along the last axis; -inf entries get weight 0."""
    mx = e.max(axis=-1, keepdims=True)
    p = np.exp(e - mx)
    return p / p.sum(axis=-1, keepdims=True)


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def local_rows(q, k, v, mask_b, b, h, rows, w, dil, causal, scale):
    """Outputs and key counts for local rows ``rows`` of (b, h).

    Key set S(i) = (W(i) union G) intersect Valid.  Window keys come from
    the index arithmetic i + k*dil; the global columns g are appended only
    when g is not already in W(i).
    """
    n = mask_b.shape[0]
    valid = mask_b != 0
    G = np.flatnonzero(mask_b == 2)
    rows = np.asarray(rows, dtype=np.int64)
    hi = 0 if causal else w
    offs = np.arange(-w, hi + 1, dtype=np.int64) * dil
    J = rows[:, None] + offs[None, :]
    ok = (J >= 0) & (J < n)
    Jc = np.clip(J, 0, n - 1)
    ok &= valid[Jc]
    if G.size:
        Jg = np.broadcast_to(G[None, :], (rows.size, G.size))
        okg = ~in_window(rows[:, None], Jg, w, dil, causal)
        Jc = np.concatenate([Jc, Jg], axis=1)
        ok = np.concatenate([ok, okg], axis=1)
    qi = _f64(q[b, rows, h])  # [r, D]
    kj = _f64(k[b][Jc, h])  # [r, m, D]
    vj = _f64(v[b][Jc, h])
    e = scale * np.einsum("rd,rmd->rm", qi, kj)
    e = np.where(ok, e, -np.inf)
    p = _softmax_rows(e)
    # the sum runs over S(i) only: keys outside it contribute nothing, even
    # where their stored values are not finite
    vj = np.where(ok[:, :, None], vj, 0.0)
    out = np.einsum("rm,rmd->rd", p, vj)
    return out, ok.sum(axis=1)


def global_rows(q_g, k_g, v_g, mask_b, b, h, rows, scale):
    """Global rows attend to every valid token with the global projections."""
    valid = np.flatnonzero(mask_b != 0)
    rows = np.asarray(rows, dtype=np.int64)
    qi = _f64(q_g[b, rows, h])
    kj = _f64(k_g[b][valid, h])
    vj = _f64(v_g[b][valid, h])
    e = scale * (qi @ kj.T)
    p = _softmax_rows(e)
    return p @ vj, np.full(rows.size, valid.size, dtype=np.int64)


def forward(q, k, v, q_g, k_g, v_g, mask, window: int,
            dilation: Optional[Sequence[int]] = None, causal: bool = False,
            scale: Optional[float] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Full forward.  Returns (out fp64 [B, n, H, D], row_nnz int64 [B, H, n]).

    Inputs may be any real arrays (fp32 arrays holding bf16 values are
    widened exactly); all arithmetic is fp64.
    """
    B, n, H, D, mask, dil = _check(q, mask, window, dilation, causal)
    s = 1.0 / math.sqrt(D) if scale is None else float(scale)
    out = np.zeros((B, n, H, D), dtype=np.float64)
    nnz = np.zeros((B, H, n), dtype=np.int64)
    for b in range(B):
        mb = mask[b]
        loc = np.flatnonzero(mb == 1)
        glo = np.flatnonzero(mb == 2)
        for h in range(H):
            for r0 in range(0, loc.size, ROW_BLOCK):
                rows = loc[r0:r0 + ROW_BLOCK]
                o, c = local_rows(q, k, v, mb, b, h, rows, window, dil[h], causal, s)
                out[b, rows, h] = o
                nnz[b, h, rows] = c
            if glo.size:
                o, c = global_rows(q_g, k_g, v_g, mb, b, h, glo, s)
                out[b, glo, h] = o
                nnz[b, h, glo] = c
    return out, nnz


def forward_rows(q, k, v, q_g, k_g, v_g, mask, window: int, b: int, h: int,
                 rows: Iterable[int], dilation: Optional[Sequence[int]] = None,
                 causal: bool = False, scale: Optional[float] = None):
    """The forward restricted to rows ``rows`` of (b, h): for sampled checks
    at sizes where the full oracle is too slow.  Same arithmetic as
    ``forward``."""
    B, n, H, D, mask, dil = _check(q, mask, window, dilation, causal)
    s = 1.0 / math.sqrt(D) if scale is None else float(scale)
    rows = np.asarray(list(rows), dtype=np.int64)
    mb = mask[b]
    out = np.zeros((rows.size, D), dtype=np.float64)
    nnz = np.zeros(rows.size, dtype=np.int64)
    loc = np.flatnonzero(mb[rows] == 1)
    glo = np.flatnonzero(mb[rows] == 2)
    if loc.size:
        o, c = local_rows(q, k, v, mb, b, h, rows[loc], window, dil[h], causal, s)
        out[loc], nnz[loc] = o, c
    if glo.size:
        o, c = global_rows(q_g, k_g, v_g, mb, b, h, rows[glo], s)
        out[glo], nnz[glo] = o, c
    return out, nnz


def pattern(mask_b, window: int, dil: int = 1, causal: bool = False) -> np.ndarray:
    """The n x n boolean attention pattern of one (b, h), built the way the
    ultralytics worked example builds it: the (dilated) window, then whole
    rows and whole columns set for global tokens, then invalid keys and
    padding rows cleared."""
    mask_b = np.asarray(mask_b)
    n = mask_b.shape[0]
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    A = in_window(i, j, window, dil, causal)
    glob = mask_b == 2
    A = A | glob[:, None] | glob[None, :]
    A &= (mask_b != 0)[None, :]
    A &= (mask_b != 0)[:, None]
    return A


def dense_bruteforce(q, k, v, q_g, k_g, v_g, mask, window: int,
                     dilation: Optional[Sequence[int]] = None, causal: bool = False,
                     scale: Optional[float] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Independent dense formulation for tiny n: full score matrices for both
    projection sets, masked by ``pattern``; each row takes the global
    projections if its token is global.  Returns the same as ``forward``."""
    B, n, H, D, mask, dil = _check(q, mask, window, dilation, causal)
    s = 1.0 / math.sqrt(D) if scale is None else float(scale)
    out = np.zeros((B, n, H, D), dtype=np.float64)
    nnz = np.zeros((B, H, n), dtype=np.int64)
    for b in range(B):
        glob = mask[b] == 2
        for h in range(H):
            A = pattern(mask[b], window, dil[h], causal)
            Ss = s * (_f64(q[b, :, h]) @ _f64(k[b, :, h]).T)
            Sg = s * (_f64(q_g[b, :, h]) @ _f64(k_g[b, :, h]).T)
            S = np.where(glob[:, None], Sg, Ss)
            S = np.where(A, S, -np.inf)
            live = A.any(axis=1)
            P = np.zeros_like(S)
            P[live] = _softmax_rows(S[live])
            keep = (mask[b] != 0)[:, None]
            o_s = P @ np.where(keep, _f64(v[b, :, h]), 0.0)
            o_g = P @ np.where(keep, _f64(v_g[b, :, h]), 0.0)
            out[b, :, h] = np.where(glob[:, None], o_g, o_s)
            nnz[b, h] = A.sum(axis=1)
    return out, nnz


def pair_count(mask_b, window: int, dil: int = 1, causal: bool = False) -> int:
    """Number of scored (query, key) pairs of one head: sum over rows of
    |S(i)|, by arithmetic per row (no n x n matrix), so it runs at the
    worked example's sizes."""
    mask_b = np.asarray(mask_b)
    if causal and (mask_b == 2).any():
        raise ValueError("causal attention with global tokens is undefined")
    n = mask_b.shape[0]
    valid = mask_b != 0
    G = np.flatnonzero(mask_b == 2)
    total = 0
    hi = 0 if causal else window
    offs = np.arange(-window, hi + 1, dtype=np.int64) * dil
    for r0 in range(0, n, 1024):
        rows = np.arange(r0, min(n, r0 + 1024), dtype=np.int64)
        kind = mask_b[rows]
        J = rows[:, None] + offs[None, :]
        ok = (J >= 0) & (J < n)
        ok &= valid[np.clip(J, 0, n - 1)]
        cnt = ok.sum(axis=1)
        if G.size:
            cnt = cnt + (~in_window(rows[:, None], G[None, :], window, dil, causal)).sum(axis=1)
        cnt = np.where(kind == 1, cnt, 0)
        cnt = np.where(kind == 2, valid.sum(), cnt)
        total += int(cnt.sum())
    return total
