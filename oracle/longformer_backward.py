"""fp64 CPU oracle for the gradients of the Longformer combined attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or
executes this module; only the test suite uses it.  It shares no code with
the HIP library.

What is computed: the exact gradient of the forward defined in
``longformer_attention`` (same key sets S(i), same projections, same mask
semantics; see that module's header for the readings of the pages) with
respect to all six inputs q, k, v, q_g, k_g, v_g, for an upstream gradient
``dout`` of the output.  The pages motivate the layer for fine-tuning and
pre-training (segmentfault Longformer summary, "Training" and
"Pre-training"; gittoolsai page, the gradient-checkpointing note), which needs this pass, but print no
formula for it; the gradient of softmax attention restricted to a key set
is the chain rule written out.  For one row i with key set S(i), scores
e_j = s <q_i, k_j>, probabilities p = softmax(e) over S(i) and output
o_i = sum_j p_j v_j:

    dv_j += p_j dout_i
    dp_j  = <dout_i, v_j>
    de_j  = p_j (dp_j - sum_m p_m dp_m)          (sum_m p_m dp_m = <dout_i, o_i>)
    dq_i  = s sum_j de_j k_j
    dk_j += s de_j q_i

Local rows take q, k, v (both their window keys and their global columns);
global rows take q_g, k_g, v_g over every valid token; mask-0 rows have no
keys and contribute nothing.  ``row_lse`` is log sum_j exp(e_j) over S(i)
(natural log; -inf for a row with no keys), the row statistic the forward
can save for this pass.

Pinned in tests/test_oracle_backward_pins.py by central finite differences
of the forward oracle, by torch autograd through an independent dense masked
formulation, and by closed-form column sums.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

from .longformer_attention import _check, in_window

ROW_BLOCK = 128


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _local_key_sets(mask_b, rows, w, dil, causal):
    """Key indices [r, m] and membership [r, m] of local rows ``rows``:
    window keys i + k*dil first, then the global columns not in W(i)."""
    n = mask_b.shape[0]
    valid = mask_b != 0
    G = np.flatnonzero(mask_b == 2)
    hi = 0 if causal else w
    offs = np.arange(-w, hi + 1, dtype=np.int64) * dil
    J = rows[:, None] + offs[None, :]
    ok = (J >= 0) & (J < n)
    J = np.clip(J, 0, n - 1)
    ok &= valid[J]
    if G.size:
        Jg = np.broadcast_to(G[None, :], (rows.size, G.size))
        okg = ~in_window(rows[:, None], Jg, w, dil, causal)
        J = np.concatenate([J, Jg], axis=1)
        ok = np.concatenate([ok, okg], axis=1)
    return J, ok


def _softmax_grad(e, ok, dout_r, vj, _plant):
    """p and de for rows of scores e [r, m] (entries outside ok are -inf)."""
    mx = e.max(axis=-1, keepdims=True)
    p = np.exp(e - mx)
    p /= p.sum(axis=-1, keepdims=True)
    p = np.where(ok, p, 0.0)
    dp = np.einsum("rd,rmd->rm", dout_r, vj)
    if _plant == "no_dterm":
        return p, p * dp
    return p, p * (dp - (p * dp).sum(axis=-1, keepdims=True))


def backward(q, k, v, q_g, k_g, v_g, mask, dout, window: int,
             dilation: Optional[Sequence[int]] = None, causal: bool = False,
             scale: Optional[float] = None, heads: Optional[Sequence[int]] = None,
             _plant: str = ""):
    """Gradients (dq, dk, dv, dq_g, dk_g, dv_g), fp64 [B, n, H, D] each.

    ``heads`` restricts the work to those heads (the others stay zero), for
    checks at sizes where all heads would be slow.  ``_plant`` introduces a
    known mistake, for the tests that show the pins catch it.
    """
    B, n, H, D, mask, dil = _check(q, mask, window, dilation, causal)
    s = 1.0 / math.sqrt(D) if scale is None else float(scale)
    grads = [np.zeros((B, n, H, D), dtype=np.float64) for _ in range(6)]
    dq, dk, dv, dqg, dkg, dvg = grads
    hs = range(H) if heads is None else heads
    for b in range(B):
        mb = mask[b]
        loc = np.flatnonzero(mb == 1)
        glo = np.flatnonzero(mb == 2)
        valid = np.flatnonzero(mb != 0)
        for h in hs:
            kb, vb = _f64(k[b, :, h]), _f64(v[b, :, h])
            for r0 in range(0, loc.size, ROW_BLOCK):
                rows = loc[r0:r0 + ROW_BLOCK]
                J, ok = _local_key_sets(mb, rows, window, dil[h], causal)
                qi, doi = _f64(q[b, rows, h]), _f64(dout[b, rows, h])
                kj = np.where(ok[:, :, None], kb[J], 0.0)
                vj = np.where(ok[:, :, None], vb[J], 0.0)
                e = np.where(ok, s * np.einsum("rd,rmd->rm", qi, kj), -np.inf)
                p, de = _softmax_grad(e, ok, doi, vj, _plant)
                dq[b, rows, h] = s * np.einsum("rm,rmd->rd", de, kj)
                sk = 1.0 if _plant == "no_scale_dk" else s
                np.add.at(dk[b, :, h], J[ok], sk * (de[:, :, None] * qi[:, None, :])[ok])
                np.add.at(dv[b, :, h], J[ok], (p[:, :, None] * doi[:, None, :])[ok])
            if glo.size:
                qi, doi = _f64(q_g[b, glo, h]), _f64(dout[b, glo, h])
                kj, vj = _f64(k_g[b, valid, h]), _f64(v_g[b, valid, h])
                e = s * (qi @ kj.T)
                ok = np.ones_like(e, dtype=bool)
                p, de = _softmax_grad(e, ok, doi, np.broadcast_to(vj, (glo.size,) + vj.shape), _plant)
                dqg[b, glo, h] = s * (de @ kj)
                dkg[b, valid, h] += s * (de.T @ qi)
                dvg[b, valid, h] += p.T @ doi
    return tuple(grads)


def row_lse(q, k, q_g, k_g, mask, window: int, dilation: Optional[Sequence[int]] = None,
            causal: bool = False, scale: Optional[float] = None, heads: Optional[Sequence[int]] = None):
    """log sum_{j in S(i)} exp(s <q_i, k_j>) per row, fp64 [B, H, n]; -inf
    for mask-0 rows (empty key set).  ``heads`` restricts the work to those
    heads (the others stay -inf), as in ``backward``."""
    B, n, H, D, mask, dil = _check(q, mask, window, dilation, causal)
    s = 1.0 / math.sqrt(D) if scale is None else float(scale)
    out = np.full((B, H, n), -np.inf)
    hs = range(H) if heads is None else heads
    for b in range(B):
        mb = mask[b]
        loc = np.flatnonzero(mb == 1)
        glo = np.flatnonzero(mb == 2)
        valid = np.flatnonzero(mb != 0)
        for h in hs:
            kb = _f64(k[b, :, h])
            for r0 in range(0, loc.size, ROW_BLOCK):
                rows = loc[r0:r0 + ROW_BLOCK]
                J, ok = _local_key_sets(mb, rows, window, dil[h], causal)
                e = s * np.einsum("rd,rmd->rm", _f64(q[b, rows, h]), kb[J])
                e = np.where(ok, e, -np.inf)
                mx = e.max(axis=-1)
                out[b, h, rows] = mx + np.log(np.exp(e - mx[:, None]).sum(axis=-1))
            if glo.size:
                e = s * (_f64(q_g[b, glo, h]) @ _f64(k_g[b, valid, h]).T)
                mx = e.max(axis=-1)
                out[b, h, glo] = mx + np.log(np.exp(e - mx[:, None]).sum(axis=-1))
    return out
