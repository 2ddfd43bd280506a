"""lf_attn_forward_noalloc (the forward for callers that cannot allocate:
its workspace is a static device array of the library) against
lf_attn_forward on the same inputs, through the C ABI.  Both run the same
kernels, which are deterministic, so out and row_nnz must agree bit for bit.
Two calls in a row, the second on a smaller problem (the scratch keeps the
first call's contents), then a problem too large for the scratch, which is
refused before any HIP call."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import sparse_long_document_amd as lf
import workloads

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lf.library()


def _noalloc(prob, max_global):
    B, n, H, D = prob.shape
    d = torch.device("cuda")
    t = [x.to(d) for x in (prob.q, prob.k, prob.v, prob.q_g, prob.k_g, prob.v_g)]
    mask = prob.mask.to(d)
    out = torch.empty_like(t[0])
    nnz = torch.empty((B, H, n), dtype=torch.int32, device=d)
    p, _keep = lf.make_params(B, n, H, D, prob.window, prob.dilation, prob.causal, prob.scale, max_global,
                              prob.q.dtype)
    vp = ctypes.c_void_p
    stream = torch.cuda.current_stream().cuda_stream
    st = lf.library().lf_attn_forward_noalloc(ctypes.byref(p), *[vp(x.data_ptr()) for x in t],
                                              vp(mask.data_ptr()), vp(out.data_ptr()), vp(nnz.data_ptr()),
                                              vp(stream))
    return st, out, nnz, t, mask


CASES = [
    dict(seed=41, B=2, n=1500, H=3, window=40, n_global=5, pad_tail=60, dilation=[1, 2, 1]),
    dict(seed=42, B=1, n=300, H=2, window=16, n_global=2),
]


def test_noalloc_matches_forward_twice_smaller_second():
    for kw in CASES:
        kw = dict(kw)
        seed = kw.pop("seed")
        prob = workloads.random_problem(seed, dtype=torch.bfloat16, name=f"noalloc{seed}", **kw)
        mg = prob.max_global()
        _say(f"[gpu noalloc] {prob.name} shape={prob.shape} globals={mg}")
        st, out, nnz, t, mask = _noalloc(prob, mg)
        assert st == lf.LF_OK, lf.status_str(st)
        ref, rnnz = lf.forward(*t, mask=mask, window=prob.window, dilation=prob.dilation,
                               return_row_nnz=True, validate=False, max_global=mg)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        assert torch.equal(nnz, rnnz)
        # and against the oracle on a few rows, so that agreement is not
        # agreement on a wrong result
        import oracle

        arrs = [x.float().numpy() for x in (prob.q, prob.k, prob.v, prob.q_g, prob.k_g, prob.v_g)]
        rows = [0, 1, prob.shape[1] // 2, prob.shape[1] - 1]
        o = out.float().cpu().numpy()
        for b in range(prob.shape[0]):
            r, rc = oracle.forward_rows(*arrs, prob.mask.numpy(), prob.window, b, 0, rows,
                                        dilation=prob.dilation)
            assert np.abs(o[b, rows, 0] - r).max() <= 2e-2
            assert np.array_equal(nnz.cpu().numpy()[b, 0, rows], rc)


def test_noalloc_refuses_what_does_not_fit():
    # 12 heads x 1024 global tokens x 8 key chunks of partial records: 26.7 MB
    prob = workloads.random_problem(43, B=1, n=4096, H=12, window=8, dtype=torch.bfloat16, name="big")
    st, *_ = _noalloc(prob, 1024)
    assert st == lf.LF_ERR_WORKSPACE
