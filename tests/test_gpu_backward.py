"""Parity of the HIP backward (through the C ABI) with the fp64 gradient
oracle, and of the forward's saved log-sum-exp with the oracle's.

Tolerances.  lse: |lse - oracle| <= 5e-3 (the row sum adds probabilities
rounded to the element type, relative error at most 2^-9, so the log is off
by at most about 2e-3).  Gradients: for each of the six fp32 results,
max |g - oracle| <= tol * max |oracle| with tol 2e-2 for bf16 and 5e-3 for
f16: the GPU rounds P and dS to the element type before the gradient
products (relative 2^-9 in bf16, 2^-12 in f16 per term) and takes D from the
forward's rounded output, so errors stay a few 2^-9 of the largest entry;
a gradient that is exactly zero keeps fp32 rounding residue below 1e-5.
Small problems are compared with the full oracle; the benchmark workload at
full size on two heads, with closed-form column sums on every head.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import sparse_long_document_amd as lf
import workloads

pytestmark = pytest.mark.gpu

TOL = {torch.bfloat16: 2e-2, torch.float16: 5e-3}
NAMES = ("dq", "dk", "dv", "dq_g", "dk_g", "dv_g")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lf.library()


def run_gpu(prob, dout):
    _say(f"[gpu bwd] {prob.name} shape={prob.shape} w={prob.window} dil={prob.dilation} "
         f"causal={prob.causal} dtype={prob.q.dtype}")
    d = torch.device("cuda")
    t = [x.to(d) for x in (prob.q, prob.k, prob.v, prob.q_g, prob.k_g, prob.v_g)]
    mask = prob.mask.to(d)
    out, lse = lf.forward(*t, mask=mask, window=prob.window, dilation=prob.dilation,
                          causal=prob.causal, scale=prob.scale, return_lse=True)
    grads = lf.backward(*t, mask, out, dout.to(d), lse, window=prob.window, dilation=prob.dilation,
                        causal=prob.causal, scale=prob.scale)
    torch.cuda.synchronize()
    assert lf.device_status(kind="forward") == 0
    assert lf.device_status(kind="backward") == 0
    return lse.cpu().numpy().astype(np.float64), [g.cpu().numpy().astype(np.float64) for g in grads]


def _np(prob):
    return [x.float().numpy() for x in (prob.q, prob.k, prob.v, prob.q_g, prob.k_g, prob.v_g)]


def check(prob, dout, heads=None):
    lse, grads = run_gpu(prob, dout)
    t = _np(prob)
    m = prob.mask.numpy()
    hs = list(range(prob.shape[2])) if heads is None else list(heads)
    ref_lse = oracle.row_lse(t[0], t[1], t[3], t[4], m, prob.window, dilation=prob.dilation,
                             causal=prob.causal, scale=prob.scale, heads=hs)
    fin = np.isfinite(ref_lse[:, hs])
    assert (np.isneginf(lse[:, hs]) == ~fin).all()
    lerr = np.abs(lse[:, hs][fin] - ref_lse[:, hs][fin]).max() if fin.any() else 0.0
    _say(f"      lse max abs err {lerr:.3e}")
    assert lerr <= 5e-3
    ref = oracle.backward(*t, m, dout.float().numpy(), prob.window, dilation=prob.dilation,
                          causal=prob.causal, scale=prob.scale, heads=heads)
    tol = TOL[prob.q.dtype]
    for name, g, r in zip(NAMES, grads, ref):
        g, r = g[:, :, hs], r[:, :, hs]
        big = np.abs(r).max()
        err = np.abs(g - r).max()
        _say(f"      {name}: max abs err {err:.3e} of max {big:.3e}")
        # a gradient that is zero in exact arithmetic (w = 0: out = v, so
        # dp - D vanishes) keeps fp32 rounding residue
        assert err <= max(tol * big, 1e-5), (name, err, big)
    return grads


SMALL = [
    dict(B=1, n=300, H=2, window=40, dilation=[1, 2], global_positions=[0, 137], pad_tail=23),
    dict(B=2, n=517, H=3, window=64, dilation=[1, 2, 3], causal=True, zero_frac=0.02),
    dict(B=1, n=1100, H=1, window=16, n_global=40),
    dict(B=1, n=70, H=1, window=0),
    dict(B=1, n=45, H=2, window=100, n_global=3),
    dict(B=2, n=640, H=2, window=33, n_global=5, pad_tail=100, aliased_global=True),
    dict(B=2, n=900, H=2, window=48, dilation=[1, 3], n_global=2, zero_frac=0.05),
    dict(B=1, n=2100, H=1, window=300, n_global=70, pad_tail=31),
    # whole 128-row tiles of padding: their dq and dk/dv workgroups find no
    # local row or key, skip the block loop and write zeros
    dict(B=2, n=700, H=2, window=40, pad_tail=300, n_global=2),
]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("case", range(len(SMALL)))
def test_backward_small(case, dtype):
    kw = dict(SMALL[case])
    prob = workloads.random_problem(300 + case, dtype=dtype, name=f"bwd_small{case}", **kw)
    dout = workloads.upstream_grad(300 + case, prob.shape, dtype)
    check(prob, dout)


def test_backward_longformer_base_two_heads():
    """The benchmark workload (B1 n4096 H12 w256, token 0 global) at full size:
    heads 0 and 11 against the oracle; every head by closed-form sums."""
    prob = workloads.by_name("longformer_base_n4096")
    dout = workloads.upstream_grad(2, prob.shape, prob.q.dtype)
    grads = check(prob, dout, heads=[0, 11])
    dq, dk, dv, dqg, dkg, dvg = grads
    m = prob.mask.numpy()[0]
    do = dout.float().numpy()[0]
    for h in range(prob.shape[2]):
        sv = dv[0, :, h].sum(0)
        np.testing.assert_allclose(sv, do[m == 1, h].sum(0), atol=2e-2 * np.abs(sv).max() + 1e-3)
        np.testing.assert_allclose(dvg[0, :, h].sum(0), do[m == 2, h].sum(0), atol=2e-2)
        assert np.abs(dk[0, :, h].sum(0)).max() <= 2e-2 * np.abs(dk[0, :, h]).sum(0).max()


def test_backward_rejects_fp32():
    prob = workloads.random_problem(9, 1, 64, 1, 8, dtype=torch.float32)
    d = torch.device("cuda")
    t = [x.to(d) for x in (prob.q, prob.k, prob.v)]
    out, lse = lf.forward(*t, window=8, return_lse=True)
    with pytest.raises(lf.LfError):
        lf.backward(*t, None, None, None, None, out, out, lse, window=8)


def test_backward_too_many_globals_flagged():
    """More mask-2 tokens in a row than max_global: the backward flags its own
    status word (the forward, given the right bound, flags nothing)."""
    prob = workloads.random_problem(13, B=1, n=300, H=1, window=10, n_global=5, name="bwd_toomany")
    d = torch.device("cuda")
    torch.cuda.synchronize()
    s = torch.cuda.Stream()  # fresh stream: fresh workspaces with clear status words
    with torch.cuda.stream(s):
        t = [x.to(d) for x in (prob.q, prob.k, prob.v, prob.q_g, prob.k_g, prob.v_g)]
        mask = prob.mask.to(d)
        out, lse = lf.forward(*t, mask=mask, window=10, return_lse=True, max_global=5)
        dout = workloads.upstream_grad(13, prob.shape, prob.q.dtype).to(d)
        lf.backward(*t, mask, out, dout, lse, window=10, validate=False, max_global=2)
        assert lf.device_status(kind="forward") == 0
        assert lf.device_status(kind="backward") & lf.LF_DEV_TOO_MANY_GLOBALS
    s2 = torch.cuda.Stream()
    with torch.cuda.stream(s2):
        lf.backward(*t, mask, out, dout, lse, window=10, validate=False, max_global=5)
        assert lf.device_status(kind="backward") == 0


@pytest.mark.parametrize("name,head", [("charlm_causal_dilated_n23040", 7), ("led_large_n16384", 3)])
def test_backward_workload_one_head(name, head):
    """The causal dilated char-LM layer (a dilated head) and the LED encoder
    layer (17 globals) at full size: all six gradients of one head against
    the oracle, every element; the closed-form column sums on every head."""
    prob = workloads.by_name(name)
    dout = workloads.upstream_grad(5, prob.shape, prob.q.dtype)
    grads = check(prob, dout, heads=[head])
    dq, dk, dv, dqg, dkg, dvg = grads
    m = prob.mask.numpy()[0]
    if prob.causal:
        m = np.where(m == 2, 1, m)
    do = dout.float().numpy()[0]
    for h in range(prob.shape[2]):
        sv = dv[0, :, h].sum(0)
        np.testing.assert_allclose(sv, do[m == 1, h].sum(0), atol=2e-2 * np.abs(sv).max() + 1e-3)
        assert np.abs(dk[0, :, h].sum(0)).max() <= 2e-2 * np.abs(dk[0, :, h]).sum(0).max()


def test_backward_joins_its_second_stream():
    """With global tokens the global-token work runs on the library's second
    stream, joined back into the caller's before the call returns: work the
    caller enqueues on its stream right after the call must see dq_g and
    dv_g, which only that work writes.  Two calls back to back on a side
    stream, each followed at once by a reduction on that stream; the sums
    are taken again after a device-wide synchronisation, and the gradients
    are compared with single calls on the default stream."""
    d = torch.device("cuda")
    kw = dict(B=1, n=2048, H=4, window=64, n_global=3)
    probs = [workloads.random_problem(410 + i, name=f"bwd_join{i}", **kw) for i in range(2)]
    douts = [workloads.upstream_grad(410 + i, p.shape, p.q.dtype) for i, p in enumerate(probs)]

    def inputs(p):
        return [x.to(d) for x in (p.q, p.k, p.v, p.q_g, p.k_g, p.v_g)], p.mask.to(d)

    def call(p, dout):
        t, mask = inputs(p)
        out, lse = lf.forward(*t, mask=mask, window=p.window, return_lse=True)
        return lf.backward(*t, mask, out, dout.to(d), lse, window=p.window)

    _say("[gpu bwd] two calls back to back on a side stream")
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        res = []
        for p, dout in zip(probs, douts):
            grads = call(p, dout)
            res.append((grads, torch.stack([grads[3].double().sum(), grads[5].double().abs().sum()])))
    torch.cuda.synchronize()
    for grads, sums in res:
        again = torch.stack([grads[3].double().sum(), grads[5].double().abs().sum()])
        assert torch.equal(sums, again), (sums, again)
        assert again[1].item() > 0.0  # dv_g of the global rows is not all zero
    for (grads, _), p, dout in zip(res, probs, douts):
        ref = call(p, dout)
        torch.cuda.synchronize()
        for name, g, r in zip(NAMES, grads, ref):
            g, r = g.double().cpu(), r.double().cpu()
            tol = 1e-5 * max(r.abs().max().item(), 1e-3)  # fp32 atomics add in any order
            assert (g - r).abs().max().item() <= tol, name
