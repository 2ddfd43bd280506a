"""Pins for the fp64 gradient oracle, against things other than the oracle
itself: central finite differences of the forward oracle, torch autograd
through a dense masked formulation written here from the definition (key
sets built by explicit loops), closed-form column sums, and planted mistakes
that these pins must catch.  CPU only.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import longformer_backward as lbo

NAMES = ("q", "k", "v", "q_g", "k_g", "v_g")


def _case(seed, B, n, H, D, globals_at=(), pad_tail=0):
    rng = np.random.default_rng(seed)
    t = [rng.standard_normal((B, n, H, D)) for _ in range(6)]
    mask = np.ones((B, n), dtype=np.int8)
    for g in globals_at:
        mask[:, g] = 2
    if pad_tail:
        mask[:, n - pad_tail:] = 0
    dout = rng.standard_normal((B, n, H, D))
    return t, mask, dout


def _loss(t, mask, dout, w, dil, causal, scale):
    out, _ = oracle.forward(*t, mask, w, dilation=dil, causal=causal, scale=scale)
    return float((out * dout).sum())


@pytest.mark.parametrize("causal", [False, True])
def test_gradients_match_central_differences(causal):
    """Every element of all six gradients against a central difference of
    the forward oracle: the derivative itself, independent of the chain-rule
    formulas the backward uses."""
    n, H, D, w = 11, 2, 3, 2
    dil = [1, 2]
    g = () if causal else (4,)
    t, mask, dout = _case(1, 1, n, H, D, globals_at=g, pad_tail=2)
    scale = 0.7
    grads = lbo.backward(*t, mask, dout, w, dilation=dil, causal=causal, scale=scale)
    eps = 1e-6
    for ti, gi, name in zip(t, grads, NAMES):
        fd = np.zeros_like(ti)
        for idx in np.ndindex(ti.shape):
            old = ti[idx]
            ti[idx] = old + eps
            lp = _loss(t, mask, dout, w, dil, causal, scale)
            ti[idx] = old - eps
            lm = _loss(t, mask, dout, w, dil, causal, scale)
            ti[idx] = old
            fd[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(gi, fd, rtol=1e-6, atol=1e-7, err_msg=name)


def _dense_torch(t, mask, w, dil, causal, scale):
    """Dense masked attention in torch fp64, built from the definition with
    explicit loops: row i (mask 1) scores j when j is valid and either
    j - i = k*d with -w <= k <= (causal ? 0 : w) or mask[j] == 2; a global
    row scores every valid j with the global projections."""
    q, k, v, qg, kg, vg = t
    B, n, H, D = q.shape
    out = torch.zeros((B, n, H, D), dtype=torch.float64)
    for b in range(B):
        for h in range(H):
            d = dil[h]
            allow = torch.zeros((n, n), dtype=torch.bool)
            allow_g = torch.zeros((n, n), dtype=torch.bool)
            for i in range(n):
                for j in range(n):
                    if mask[b, j] == 0:
                        continue
                    if mask[b, i] == 1:
                        off = j - i
                        in_w = off % d == 0 and -w <= off // d <= (0 if causal else w)
                        allow[i, j] = bool(in_w or mask[b, j] == 2)
                    elif mask[b, i] == 2:
                        allow_g[i, j] = True
            for A, Q, K, V in ((allow, q, k, v), (allow_g, qg, kg, vg)):
                rows = A.any(dim=1)
                e = scale * (Q[b, :, h] @ K[b, :, h].T)
                e = e.masked_fill(~A, float("-inf"))
                p = torch.softmax(e[rows], dim=-1)
                o = out[b, :, h].clone()
                o[rows] = p @ V[b, :, h]
                out[b, :, h] = o
    return out


@pytest.mark.parametrize("seed,causal", [(2, False), (3, False), (4, True)])
def test_gradients_match_torch_autograd_dense(seed, causal):
    n, H, D, w = 14, 2, 4, 3
    dil = [1, 3]
    g = () if causal else (0, 9)
    t, mask, dout = _case(seed, 2, n, H, D, globals_at=g, pad_tail=3)
    mask[1, 5] = 0  # a pad token inside the sequence
    scale = 0.5
    grads = lbo.backward(*t, mask, dout, w, dilation=dil, causal=causal, scale=scale)
    tt = [torch.tensor(x, requires_grad=True) for x in t]
    out = _dense_torch(tt, mask, w, dil, causal, scale)
    (out * torch.from_numpy(dout)).sum().backward()
    for x, gi, name in zip(tt, grads, NAMES):
        np.testing.assert_allclose(gi, x.grad.numpy(), rtol=1e-10, atol=1e-12, err_msg=name)


def test_column_sums_closed_forms():
    """Softmax rows sum to one, so summed over keys: dv collects each scoring
    row's upstream gradient once, and the key gradients cancel (a constant
    shift of every key leaves each row's softmax unchanged)."""
    n, H, D, w = 200, 3, 8, 7
    t, mask, dout = _case(5, 1, n, H, D, globals_at=(0, 57, 120), pad_tail=17)
    dq, dk, dv, dqg, dkg, dvg = lbo.backward(*t, mask, dout, w, dilation=[1, 2, 5])
    loc = mask[0] == 1
    glo = mask[0] == 2
    for h in range(H):
        np.testing.assert_allclose(dv[0, :, h].sum(0), dout[0, loc, h].sum(0), atol=1e-10)
        np.testing.assert_allclose(dvg[0, :, h].sum(0), dout[0, glo, h].sum(0), atol=1e-10)
        np.testing.assert_allclose(dk[0, :, h].sum(0), 0.0, atol=1e-10)
        np.testing.assert_allclose(dkg[0, :, h].sum(0), 0.0, atol=1e-10)
    pad = mask[0] == 0
    for x in (dq, dk, dv, dqg, dkg, dvg):
        assert (x[0, pad] == 0).all()
    assert (dq[0, glo] == 0).all() and (dqg[0, loc] == 0).all()


def test_row_lse_matches_dense_logsumexp():
    n, H, D, w = 30, 2, 4, 3
    t, mask, _ = _case(6, 1, n, H, D, globals_at=(2,), pad_tail=4)
    dil = [1, 2]
    lse = lbo.row_lse(t[0], t[1], t[3], t[4], mask, w, dilation=dil, scale=0.3)
    tt = [torch.from_numpy(x) for x in t]
    for h in range(H):
        for i in range(n):
            if mask[0, i] == 0:
                assert lse[0, h, i] == -np.inf
                continue
            keys = []
            for j in range(n):
                if mask[0, j] == 0:
                    continue
                if mask[0, i] == 2:
                    keys.append(j)
                else:
                    diff = i - j
                    if (diff % dil[h] == 0 and abs(diff) <= w * dil[h]) or mask[0, j] == 2:
                        keys.append(j)
            Q, K = (tt[3], tt[4]) if mask[0, i] == 2 else (tt[0], tt[1])
            e = 0.3 * (K[0, keys, h] @ Q[0, i, h])
            assert abs(lse[0, h, i] - torch.logsumexp(e, 0).item()) < 1e-12


def test_heads_argument_restricts_work():
    t, mask, dout = _case(7, 1, 40, 3, 4, globals_at=(3,))
    full = lbo.backward(*t, mask, dout, 4)
    part = lbo.backward(*t, mask, dout, 4, heads=[1])
    for a, b in zip(full, part):
        np.testing.assert_array_equal(a[:, :, 1], b[:, :, 1])
        assert (b[:, :, [0, 2]] == 0).all()


@pytest.mark.parametrize("plant", ["no_dterm", "no_scale_dk"])
def test_planted_mistakes_are_caught(plant):
    """A dropped softmax-Jacobian term or a missing scale on dk must fail the
    autograd pin."""
    n, H, D, w = 12, 1, 4, 2
    t, mask, dout = _case(8, 1, n, H, D, globals_at=(5,))
    scale = 0.5
    grads = lbo.backward(*t, mask, dout, w, scale=scale, _plant=plant)
    tt = [torch.tensor(x, requires_grad=True) for x in t]
    out = _dense_torch(tt, mask, w, [1], False, scale)
    (out * torch.from_numpy(dout)).sum().backward()
    worst = max(np.abs(gi - x.grad.numpy()).max() for x, gi in zip(tt, grads))
    assert worst > 1e-3
