"""Parity of the HIP input projections (through the C ABI) with the fp64
projection oracle, and of projections followed by the attention forward with
the two oracles chained.

Tolerance: |y - oracle| <= 2^-8 |oracle| + 1e-3 for bf16 (the kernel
accumulates in fp32 and rounds once to nearest even: half a bf16 ulp is at
most 2^-9 relative, fp32 accumulation over C <= 1024 terms adds well under
1e-3) and 2^-10 |oracle| + 1e-3 for f16.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import sparse_long_document_amd as lf
import workloads

pytestmark = pytest.mark.gpu

REL = {torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -10}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lf.library()


def check(seed, M, C, P, dtype, with_bias=True):
    _say(f"[gpu proj] M={M} C={C} P={P} dtype={dtype} bias={with_bias}")
    x, w, b = workloads.projection_problem(seed, M, C, P, dtype)
    d = torch.device("cuda")
    y = lf.project(x.to(d), w.to(d), b.to(d) if with_bias else None)
    torch.cuda.synchronize()
    ref = oracle.project(x.float().numpy(), w.float().numpy(), b.numpy() if with_bias else None)
    got = y.float().cpu().numpy()
    excess = np.abs(got - ref) - (REL[dtype] * np.abs(ref) + 1e-3)
    _say(f"      max abs err {np.abs(got - ref).max():.3e}, worst excess {excess.max():.3e}")
    assert excess.max() <= 0
    return y


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("M,C,P", [(300, 128, 3), (1, 64, 1), (257, 192, 6), (1000, 64, 2)])
def test_projection_small(M, C, P, dtype):
    check(7 + M, M, C, P, dtype)


@pytest.mark.parametrize("M,C,P,dtype", [(2000, 192, 1, torch.bfloat16), (2333, 448, 6, torch.bfloat16),
                                          (2000, 448, 5, torch.bfloat16), (2000, 448, 5, torch.float16),
                                          (4000, 704, 6, torch.bfloat16), (4000, 704, 6, torch.float16),
                                          (6000, 1024, 2, torch.bfloat16), (7000, 960, 2, torch.bfloat16),
                                          (7000, 960, 2, torch.float16)],
                         ids=["s-a", "s-b", "m", "m-f16", "l", "l-f16", "x", "x-ragged", "x-f16"])
def test_projection_tile_configs(M, C, P, dtype):
    """Each tile configuration of the launch (on a 256-CU device the
    chooser takes 128 x 128 tiles for the first two sizes, 128 x 192 for the
    next two, 256 x 288 for the two after and 256 x 256 for the last three),
    with token counts that are not multiples of the token tile and feature
    counts that are not multiples of the feature tile."""
    check(31 + M + C, M, C, P, dtype)


def check_global_only(seed, M, C, P, dtype, bits, mask):
    """lf_attn_project_global_only: projections in ``bits`` at the tokens
    with mask 2 only (zero elsewhere), the others as lf_attn_project, and
    exactly the plain launch's values wherever it computes them."""
    _say(f"[gpu proj global-only] M={M} C={C} P={P} dtype={dtype} bits={bits} globals={(mask == 2).sum()}")
    x, w, b = workloads.projection_problem(seed, M, C, P, dtype)
    d = torch.device("cuda")
    m = torch.from_numpy(mask.astype(np.int8))
    y = lf.project(x.to(d), w.to(d), b.to(d), mask=m.to(d), global_only=bits)
    full = lf.project(x.to(d), w.to(d), b.to(d))
    torch.cuda.synchronize()
    ref = oracle.project(x.float().numpy(), w.float().numpy(), b.numpy())
    g = mask == 2
    for q in bits:
        ref[q][~g] = 0.0
    got = y.float().cpu().numpy()
    excess = np.abs(got - ref) - (REL[dtype] * np.abs(ref) + 1e-3)
    _say(f"      max abs err {np.abs(got - ref).max():.3e}, worst excess {excess.max():.3e}")
    assert excess.max() <= 0
    gt = torch.from_numpy(g).to(d)
    for q in range(P):
        if q in bits:
            assert torch.equal(y[q][gt], full[q][gt]) and not y[q][~gt].any()
        else:
            assert torch.equal(y[q], full[q])


def _mask(rng, M, n_global, others=True):
    m = np.ones(M, dtype=np.int64)
    if others:
        m[rng.random(M) < 0.05] = 0
        m[rng.random(M) < 0.01] = 3  # not a global token
    if n_global:
        m[rng.choice(M, size=n_global, replace=False)] = 2
    return m


@pytest.mark.parametrize("M,C,P,bits,n_global", [(300, 128, 6, (3,), 5), (2000, 448, 5, (3, 4), 9),
                                                 (4000, 704, 6, (3,), 17), (4096, 768, 6, (3,), 1),
                                                 (2333, 448, 6, (3,), 0), (7000, 960, 2, (1,), 13)],
                         ids=["s", "m-two", "l", "longformer-base", "no-global", "x"])
def test_projection_global_only(M, C, P, bits, n_global):
    rng = np.random.default_rng(M + C)
    check_global_only(41 + M, M, C, P, torch.bfloat16, bits, _mask(rng, M, n_global))


def test_projection_global_only_f16_clustered():
    """Global tokens all in one token tile: every other tile of Q_g
    features skips its reduction."""
    M = 2000
    m = np.ones(M, dtype=np.int64)
    m[130:140] = 2
    check_global_only(47, M, 448, 5, torch.float16, (3,), m)


def test_projection_without_bias():
    check(11, 130, 128, 2, torch.bfloat16, with_bias=False)


def test_projection_longformer_base_full():
    """The layer's six projections at the longformer-base size: 4096 tokens,
    768 features (12 heads of 64)."""
    check(3, 4096, 768, 6, torch.bfloat16)


def test_projections_then_attention():
    """Projections feeding the forward, against the oracles chained the same
    way (the oracle's projections rounded to bf16 before its attention)."""
    B, n, H = 1, 600, 4
    C = 64 * H
    x, w, b = workloads.projection_problem(21, B * n, C, 6, torch.bfloat16)
    mask = torch.ones((B, n), dtype=torch.int8)
    mask[0, [0, 333]] = 2
    d = torch.device("cuda")
    y = lf.project(x.to(d), w.to(d), b.to(d))
    t = [y[i].view(B, n, H, 64) for i in range(6)]
    # attention order: q, k, v, q_g, k_g, v_g
    out = lf.forward(*t, mask=mask.to(d), window=50)
    torch.cuda.synchronize()
    yr = oracle.project(x.float().numpy(), w.float().numpy(), b.numpy())
    yr = torch.from_numpy(yr).to(torch.bfloat16).float().numpy()
    ref, _ = oracle.forward(*[yr[i].reshape(B, n, H, 64) for i in range(6)], mask.numpy(), 50)
    err = np.abs(out.float().cpu().numpy() - ref).max()
    _say(f"      chained max abs err {err:.3e}")
    assert err <= 2e-2
