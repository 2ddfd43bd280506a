"""fp64 CPU oracle for the input projections of the Longformer attention
layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or
executes this module; only the test suite and the benchmark's CPU-baseline
leg do.  It shares no code with the HIP library.

What is computed: the layer's six linear maps of the hidden states, the
sliding-window projections Q_s, K_s, V_s and the separate global-attention
projections Q_g, K_g, V_g (segmentfault Longformer summary, "Linear
projections for global attention"; the global ones start as copies of the
local ones).  Reading: each is a linear layer y = x W^T + b with W stored
[out features, in features] and out features = in features = C = H * D, so
that y, viewed as [B, n, H, D], is the per-head layout the attention takes.
The definition is a matrix product, so the oracle is that product in fp64
(NumPy's matmul as the step).
"""
from __future__ import annotations

import numpy as np


def project(x, w, bias=None):
    """x [M, C], w [P*C, C] (P stacked weights), bias [P*C] or None.
    Returns y [P, M, C] fp64 with y[p] = x @ w[p*C:(p+1)*C].T + bias[p*C:(p+1)*C]."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    M, C = x.shape
    if w.ndim != 2 or w.shape[1] != C or w.shape[0] % C != 0:
        raise ValueError("w must be [P*C, C]")
    P = w.shape[0] // C
    y = np.empty((P, M, C), dtype=np.float64)
    for p in range(P):
        y[p] = x @ w[p * C:(p + 1) * C].T
        if bias is not None:
            y[p] += np.asarray(bias, dtype=np.float64)[p * C:(p + 1) * C]
    return y
