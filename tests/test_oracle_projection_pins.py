"""Pins for the fp64 projection oracle against things other than itself:
torch's linear layer (a library routine with its own weight convention),
an identity and a permutation weight (closed forms that a transposed weight
or a wrong projection offset would fail), linearity, and the global
projections' initial state (copied weights give equal outputs).  CPU only."""
import numpy as np
import torch

import oracle


def test_matches_torch_linear():
    rng = np.random.default_rng(1)
    M, C, P = 37, 16, 3
    x = rng.standard_normal((M, C))
    w = rng.standard_normal((P * C, C))
    b = rng.standard_normal(P * C)
    y = oracle.project(x, w, b)
    for p in range(P):
        ref = torch.nn.functional.linear(torch.from_numpy(x), torch.from_numpy(w[p * C:(p + 1) * C]),
                                         torch.from_numpy(b[p * C:(p + 1) * C])).numpy()
        np.testing.assert_allclose(y[p], ref, rtol=1e-12, atol=1e-12)


def test_identity_and_permutation_weights():
    rng = np.random.default_rng(2)
    M, C = 9, 8
    x = rng.standard_normal((M, C))
    perm = rng.permutation(C)
    eye = np.eye(C)
    pm = eye[perm]  # row j picks input feature perm[j]: y[:, j] = x[:, perm[j]]
    y = oracle.project(x, np.concatenate([eye, pm]), np.concatenate([np.zeros(C), np.arange(C)]))
    np.testing.assert_array_equal(y[0], x)
    np.testing.assert_array_equal(y[1], x[:, perm] + np.arange(C))


def test_linearity_and_copied_global_weights():
    rng = np.random.default_rng(3)
    M, C = 20, 12
    x1, x2 = rng.standard_normal((M, C)), rng.standard_normal((M, C))
    ws = rng.standard_normal((3 * C, C))
    b = rng.standard_normal(3 * C)
    w6 = np.concatenate([ws, ws])  # global projections initialised to the local ones
    y = oracle.project(x1 + x2, w6, np.concatenate([b, b]))
    np.testing.assert_array_equal(y[:3], y[3:])
    y1 = oracle.project(x1, ws, b)
    y2 = oracle.project(x2, ws, None)
    np.testing.assert_allclose(y[:3], y1 + y2, atol=1e-12)
