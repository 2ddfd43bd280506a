"""The encoder attention sublayer chained from the C ABI's calls
(lf_attn_project -> lf_attn_forward -> lf_attn_project) against the chained
oracles, stage by stage: the six projections against oracle.project, the
attention on the GPU's (rounded) projections against oracle.forward on the
same values, the output projection on the GPU's attention output against
oracle.project.  Each stage is held to that stage's own bound (projections:
2^-8 |y| + 1e-3 for bf16; attention: 2e-2, row_nnz exact), since each takes
the previous stage's rounded output as exact input.  The LED encoder
workload (16K tokens, 16 heads, 17 global tokens; LED on the gittoolsai
page's news of 2020-12-01, segmentfault summary "Longformer-Encoder-Decoder
(LED)") is checked on every row of two heads."""
import sys

import numpy as np
import pytest
import torch

import oracle
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


def _proj_ok(got, ref):
    return float((np.abs(got - ref) - (2.0 ** -8 * np.abs(ref) + 1e-3)).max()) <= 0


def check_chain(prob, heads=None, rows_per_head=None):
    d = torch.device("cuda")
    B, n, C = prob.shape
    H = prob.H
    _say(f"[gpu encoder] {prob.name} B={B} n={n} C={C} globals={prob.max_global()}")
    y, proj, attn = lf.encoder_attention(prob.x.to(d), prob.w.to(d), prob.bias.to(d), prob.mask.to(d),
                                         prob.window, max_global=prob.max_global(), validate=False,
                                         w_out=prob.w_out.to(d), b_out=prob.b_out.to(d),
                                         return_intermediate=True)
    torch.cuda.synchronize()
    # stage 1: the six projections
    x64 = prob.x.reshape(B * n, C).float().numpy()
    ref_p = oracle.project(x64, prob.w.float().numpy(), prob.bias.numpy()).reshape(6, B, n, C)
    # the chain computes Q_g at the global tokens only and zero elsewhere
    # (lf_attn_project_global_only): the attention reads it nowhere else
    ref_p[3][prob.mask.numpy() != 2] = 0.0
    gp = proj.float().cpu().numpy()
    assert _proj_ok(gp, ref_p), float(np.abs(gp - ref_p).max())
    # stage 2: attention on the GPU's projections
    t = [proj[i].view(B, n, H, 64).cpu() for i in range(6)]
    arrs = [x.float().numpy() for x in t]
    mask = prob.mask.numpy()
    ga = attn.float().cpu().numpy()
    hs = range(H) if heads is None else heads
    worst = 0.0
    for b in range(B):
        for h in hs:
            ref, _rc = oracle.forward_rows(*arrs, mask, prob.window, b, h, range(n))
            worst = max(worst, float(np.abs(ga[b, :, h] - ref).max()))
    _say(f"      attention max abs err {worst:.3e}")
    assert worst <= 2e-2
    # stage 3: the output projection of the GPU's attention output
    ref_y = oracle.project(ga.reshape(B * n, C), prob.w_out.float().numpy(), prob.b_out.numpy())[0]
    gy = y.float().cpu().numpy().reshape(B * n, C)
    assert _proj_ok(gy, ref_y), float(np.abs(gy - ref_y).max())


def test_encoder_chain_small():
    check_chain(workloads.encoder_problem(51, 2, 700, 4, 48, n_global=3, name="enc_small"))


def test_encoder_chain_copied_global_projections():
    # the global projections' initial state: copies of the local ones
    prob = workloads.encoder_problem(52, 1, 500, 2, 32, n_global=4, name="enc_copied", copied_global=True)
    check_chain(prob)
    d = torch.device("cuda")
    _y, proj, _a = lf.encoder_attention(prob.x.to(d), prob.w.to(d), prob.bias.to(d), prob.mask.to(d),
                                        prob.window, w_out=prob.w_out.to(d), b_out=prob.b_out.to(d),
                                        return_intermediate=True)
    assert torch.equal(proj[1:3], proj[4:6])
    g = prob.mask.to(d) == 2
    assert torch.equal(proj[0][g], proj[3][g]) and not proj[3][~g].any()


def test_led_encoder_n16384_two_heads():
    check_chain(workloads.led_encoder_n16384(), heads=[0, 15])
