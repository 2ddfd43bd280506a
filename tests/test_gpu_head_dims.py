"""Head dims 32 and 128 of the forward (the kernel source built once per
head dim), through the C ABI, against the fp64 oracle.

The oracle takes any head dim (its scores are plain dot products over D), so
the checks are those of the head-dim-64 suite: every SMALL case element by
element in bf16 and fp32 (and a few in f16), with the same tolerances, and
every row of two heads of the longformer-base layer shape (B1 n4096 H12,
w=256, token 0 global) at each head dim, in the launch configuration the
benchmark times.  row_nnz is bit-exact everywhere.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_long_document_amd as lf
import workloads
from test_gpu_parity import SMALL, TOL, _np, _say, check_full, run_gpu

pytestmark = pytest.mark.gpu

# f16 at the other head dims: a global-row split of each kind, dilation,
# causal, padding
F16_CASES = (5, 8, 10, 13, 21, 23, 24)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lf.library()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("idx", range(len(SMALL)))
@pytest.mark.parametrize("D", [32, 128])
def test_small_head_dim(D, idx, dtype):
    prob = workloads.random_problem(100 + idx, dtype=dtype, name=f"small{idx}_d{D}", D=D, **SMALL[idx])
    check_full(prob)


@pytest.mark.parametrize("idx", F16_CASES)
@pytest.mark.parametrize("D", [32, 128])
def test_small_head_dim_f16(D, idx):
    prob = workloads.random_problem(100 + idx, dtype=torch.float16, name=f"small{idx}_d{D}_f16", D=D,
                                    **SMALL[idx])
    check_full(prob)


@pytest.mark.parametrize("D", [32, 128])
def test_longformer_base_shape_two_heads_full(D):
    """Every row of heads 0 and 11 of the longformer-base shape at head dim
    D, and the pair count of every head (the closed form of the window plus
    the one global token: 2043134 per head)."""
    prob = workloads.longformer_base_n4096_dim(D)
    assert prob.shape == (1, 4096, 12, D)
    out, nnz = run_gpu(prob, validate=False, max_global=1)
    arrs = _np(prob)
    mask = prob.mask.numpy()
    for h in (0, 11):
        ref, rnnz = oracle.forward_rows(*arrs, mask, prob.window, 0, h, range(4096))
        np.testing.assert_array_equal(nnz[0, h], rnnz)
        err = np.abs(out[0, :, h] - ref).max()
        _say(f"      D {D} head {h}: max abs err {err:.3e}")
        assert err <= TOL[torch.bfloat16], (h, err)
    assert (nnz.reshape(12, -1).sum(axis=1) == 2043134).all()


@pytest.mark.parametrize("D", [32, 128])
def test_head_dim_aliased_and_lse(D):
    """Aliased global projections and the log-sum-exp output at head dim D."""
    prob = workloads.random_problem(40 + D, B=1, n=700, H=2, window=50, n_global=6, aliased_global=True,
                                    D=D, name=f"alias_d{D}")
    dev = torch.device("cuda")
    q, k, v = (x.to(dev) for x in (prob.q, prob.k, prob.v))
    mask = prob.mask.to(dev)
    out, lse = lf.forward(q, k, v, mask=mask, window=prob.window, return_lse=True)
    torch.cuda.synchronize()
    arrs = _np(prob)
    ref, _ = oracle.forward(*arrs, prob.mask.numpy(), prob.window)
    assert np.abs(out.float().cpu().numpy() - ref).max() <= TOL[torch.bfloat16]
    # lse bound as in the backward suite: the row sum adds probabilities
    # rounded to bf16 (relative 2^-9 each)
    rl = oracle.row_lse(arrs[0], arrs[1], arrs[3], arrs[4], prob.mask.numpy(), prob.window)
    got = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(rl)
    assert (np.isneginf(got) == ~fin).all()
    assert np.abs(got[fin] - rl[fin]).max() <= 5e-3
