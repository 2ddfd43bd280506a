"""The forward and the backward under HIP graph capture, through the C ABI.

A captured call must neither allocate nor clear memory (a clear recorded
into a graph is replayed with it, and a buffer taken during capture belongs
to the graph's pool): the binding refuses to create a workspace then, and a
workspace made beforehand with make_workspace is reused by every replay
(each forward leaves its arrival counters back at zero).  Every replay, with
eager work and synchronisations between them, must reproduce the eager
result bit for bit: the kernels are deterministic.
"""
import sys

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


def _problem():
    prob = workloads.random_problem(31, B=2, n=700, H=3, window=48, n_global=3, pad_tail=40,
                                    dilation=[1, 2, 1], name="graph")
    d = torch.device("cuda")
    t = [x.to(d) for x in (prob.q, prob.k, prob.v, prob.q_g, prob.k_g, prob.v_g)]
    return prob, t, prob.mask.to(d)


def test_capture_without_workspace_is_refused():
    prob, t, mask = _problem()
    _say("[gpu graph] refusal on a fresh capture stream")
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with pytest.raises(RuntimeError, match="make_workspace"):
        with torch.cuda.graph(g, stream=s):
            lf.forward(*t, mask=mask, window=prob.window, dilation=prob.dilation, validate=False,
                       max_global=3)
    torch.cuda.synchronize()


def test_forward_and_backward_replays_match_eager():
    prob, t, mask = _problem()
    B, n, H, D = prob.shape
    kw = dict(window=prob.window, dilation=prob.dilation, validate=False, max_global=3)
    dout = workloads.upstream_grad(31, prob.shape, prob.q.dtype).to(t[0].device)
    # eager reference
    out_ref, lse_ref = lf.forward(*t, mask=mask, return_lse=True, **kw)
    g_ref = lf.backward(*t, mask, out_ref, dout, lse_ref, **kw)
    torch.cuda.synchronize()
    # static buffers and workspaces made outside the capture
    ws_f = lf.make_workspace(B, n, H, prob.window, dilation=prob.dilation, max_global=3, dtype=prob.q.dtype)
    ws_b = lf.make_workspace(B, n, H, prob.window, dilation=prob.dilation, max_global=3, dtype=prob.q.dtype,
                             backward=True)
    out = torch.empty_like(t[0])
    lse = torch.empty((B, H, n), dtype=torch.float32, device=t[0].device)
    grads = [torch.empty((B, n, H, D), dtype=torch.float32, device=t[0].device) for _ in range(6)]
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    _say("[gpu graph] capture forward + backward")
    with torch.cuda.graph(g, stream=s):
        lf.forward(*t, mask=mask, out=out, lse=lse, return_lse=True, workspace=ws_f, **kw)
        lf.backward(*t, mask, out, dout, lse, grads=grads, workspace=ws_b, **kw)
    for rep in range(3):
        out.fill_(7.0)
        for x in grads:
            x.fill_(-3.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _say(f"[gpu graph] replay {rep}")
        assert torch.equal(out, out_ref)
        assert torch.equal(lse, lse_ref)
        # dq is written without atomics; the gradients with fp32 atomic adds
        # may differ in the last bits between runs, so those are compared to
        # rounding
        assert torch.equal(grads[0], g_ref[0])
        for a, b in zip(grads[1:], g_ref[1:]):
            torch.testing.assert_close(a, b, rtol=1e-5, atol=1e-6)
        # eager work between replays on the default stream
        lf.forward(*t, mask=mask, **kw)
        torch.cuda.synchronize()
    assert lf.device_status(workspace=ws_f) == 0
    assert lf.device_status(workspace=ws_b) == 0
