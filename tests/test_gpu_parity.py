"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Tolerances: max |out - oracle| <= 2e-2 for bf16 inputs, <= 5e-3 for f16
inputs and <= 1e-4 for fp32 inputs (fp32 accumulation on the GPU); row_nnz
(pairs scored per row) bit-exact everywhere.  The f16 bound: the inputs are
exact in both, so the error comes from rounding the probabilities (relative
2^-11) and the output (half an f16 ulp, 2^-10 for |out| < 2) to f16, about
4x below bf16's 2^-8 and 2^-7; 5e-3 keeps bf16's margin.  Small problems are compared element by element with
the full oracle; the five named workloads at full size are checked on
sampled rows that the oracle computes one by one, in the same launch
configuration the benchmark times.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import sparse_long_document_amd as lf
import workloads

pytestmark = pytest.mark.gpu

TOL = {torch.bfloat16: 2e-2, torch.float16: 5e-3, torch.float32: 1e-4}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lf.library()


def _dev(prob):
    d = torch.device("cuda")
    t = [x.to(d) for x in (prob.q, prob.k, prob.v)]
    if prob.aliased_global:
        g = [None, None, None]
    else:
        g = [x.to(d) for x in (prob.q_g, prob.k_g, prob.v_g)]
    return t, g, prob.mask.to(d)


def run_gpu(prob, validate=True, max_global=None):
    _say(f"[gpu] {prob.name} shape={prob.shape} w={prob.window} dil={prob.dilation} "
         f"causal={prob.causal} dtype={prob.q.dtype}")
    t, g, mask = _dev(prob)
    out, nnz = lf.forward(*t, *g, mask=mask, window=prob.window, dilation=prob.dilation,
                          causal=prob.causal, scale=prob.scale, return_row_nnz=True,
                          validate=validate, max_global=max_global)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), nnz.cpu().numpy().astype(np.int64)


def _np(prob):
    return [x.float().numpy() for x in (prob.q, prob.k, prob.v, prob.q_g, prob.k_g, prob.v_g)]


def run_oracle(prob):
    return oracle.forward(*_np(prob), prob.mask.numpy(), prob.window, dilation=prob.dilation,
                          causal=prob.causal, scale=prob.scale)


def check_full(prob):
    out, nnz = run_gpu(prob)
    ref, rnnz = run_oracle(prob)
    np.testing.assert_array_equal(nnz, rnnz)
    err = np.abs(out - ref).max() if out.size else 0.0
    _say(f"      max abs err {err:.3e}")
    assert err <= TOL[prob.q.dtype], err
    pad = np.broadcast_to((prob.mask.numpy() == 0)[:, :, None, None], out.shape)
    assert (out[pad] == 0).all()
    return out, nnz


SMALL = [
    dict(B=1, n=1, H=1, window=0),
    dict(B=1, n=5, H=2, window=2),
    dict(B=1, n=63, H=1, window=7),
    dict(B=1, n=64, H=1, window=64),
    dict(B=1, n=65, H=2, window=31),
    dict(B=1, n=200, H=2, window=16, n_global=3),
    dict(B=2, n=200, H=1, window=100, n_global=1, pad_tail=37),
    dict(B=1, n=333, H=3, window=40, dilation=[1, 2, 3]),
    dict(B=1, n=333, H=3, window=40, dilation=[1, 2, 3], n_global=5),
    dict(B=1, n=300, H=2, window=20, causal=True),
    dict(B=1, n=301, H=3, window=33, causal=True, dilation=[3, 1, 2]),
    dict(B=1, n=257, H=1, window=300),
    dict(B=1, n=190, H=1, window=500, causal=True),
    dict(B=2, n=520, H=2, window=24, n_global=40, zero_frac=0.05),
    dict(B=1, n=1100, H=2, window=64, n_global=70),
    dict(B=1, n=1100, H=1, window=64, n_global=2, pad_tail=300, dilation=[2]),
    dict(B=3, n=130, H=2, window=9, n_global=2, zero_frac=0.3),
    dict(B=1, n=700, H=2, window=64, dilation=[5, 7]),
    dict(B=1, n=96, H=1, window=3, global_positions=[0, 1, 2, 95]),
    # global tokens in the last bytes of the mask, rows not a multiple of 16
    dict(B=2, n=203, H=1, window=20, global_positions=[0, 190, 201, 202]),
    dict(B=1, n=4100, H=1, window=32, global_positions=[5, 4096, 4099]),
    # four global tokens (the vector-unit path), some inside rows' windows, dilated heads
    dict(B=2, n=500, H=2, window=30, dilation=[1, 3], global_positions=[0, 33, 250, 499], pad_tail=20),
    # one dilation for every head, n not a multiple of it (the arithmetic tile decode)
    dict(B=3, n=1001, H=3, window=40, dilation=[3, 3, 3], n_global=2),
    # 32 global tokens, the most the four-wave split takes, over two key chunks
    dict(B=1, n=1500, H=1, window=40, n_global=32),
    # 33 global tokens (the two-parity split), three key chunks, the last ragged
    dict(B=1, n=2100, H=2, window=48, n_global=33, pad_tail=50),
    # the most heads the library takes
    dict(B=1, n=300, H=64, window=20, n_global=2),
    # the most global tokens a batch row may hold (LF_MAX_GLOBAL)
    dict(B=1, n=1100, H=1, window=16, n_global=1024),
]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32], ids=["bf16", "f16", "f32"])
@pytest.mark.parametrize("idx", range(len(SMALL)))
def test_small_full_parity(idx, dtype):
    kw = dict(SMALL[idx])
    prob = workloads.random_problem(100 + idx, dtype=dtype, name=f"small{idx}", **kw)
    check_full(prob)


def test_aliased_global_projections():
    prob = workloads.random_problem(7, B=1, n=400, H=2, window=30, n_global=4,
                                    aliased_global=True, name="aliased")
    check_full(prob)


def test_mask_values_other_than_0_1_2_act_as_0():
    # bytes such as 3, -1, -126 and 127, some right next to global tokens
    # (the kernel finds the global tokens 16 mask bytes at a time)
    prob = workloads.random_problem(13, B=2, n=700, H=2, window=40, global_positions=[0, 5, 130, 131, 600],
                                    name="oddmask")
    rng = np.random.default_rng(3)
    m = prob.mask.clone()
    for b in range(2):
        for g in (5, 130, 600):
            m[b, g - 1] = 3
            m[b, g + 2] = -126
        m[b, rng.integers(0, 700, size=40)] = torch.tensor(rng.choice([3, -1, 127, -126], size=40), dtype=torch.int8)
        m[b, [0, 5, 130, 131, 600]] = 2
    prob.mask = m
    # the binding's validation rejects such bytes; the C ABI reads them as 0,
    # so the reference is the oracle on the mask with those bytes set to 0
    out, nnz = run_gpu(prob, validate=False, max_global=5)
    prob.mask = torch.where((m == 1) | (m == 2), m, torch.zeros_like(m))
    ref, rnnz = run_oracle(prob)
    np.testing.assert_array_equal(nnz, rnnz)
    assert np.abs(out - ref).max() <= TOL[prob.q.dtype]


def test_scale_argument():
    prob = workloads.random_problem(8, B=1, n=300, H=1, window=30, n_global=2, scale=0.3, name="scale")
    check_full(prob)


def test_single_head_fp32_workload_full():
    check_full(workloads.single_head_fp32_n512())


def test_rows_sum_to_one_through_api():
    prob = workloads.random_problem(9, B=1, n=500, H=2, window=50, n_global=3, pad_tail=20, name="ones")
    ones = torch.ones_like(prob.v)
    prob.v = ones
    prob.v_g = ones.clone()
    out, _ = run_gpu(prob)
    live = (prob.mask.numpy() != 0)[:, :, None, None]
    ref = np.broadcast_to(np.where(live, 1.0, 0.0), out.shape)
    assert np.abs(out - ref).max() <= 2e-2


def test_deterministic_and_repeatable():
    prob = workloads.random_problem(10, B=2, n=1500, H=3, window=70, n_global=9, pad_tail=100, name="det")
    a, na = run_gpu(prob)
    small = workloads.random_problem(11, B=1, n=600, H=1, window=10, n_global=2, name="other")
    run_gpu(small)
    b, nb = run_gpu(prob)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(na, nb)


def test_too_many_globals_flagged():
    prob = workloads.random_problem(12, B=1, n=300, H=1, window=10, n_global=5, name="toomany")
    torch.cuda.synchronize()
    # fresh stream => fresh workspace with a clear status word
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        t, g, mask = _dev(prob)
        lf.forward(*t, *g, mask=mask, window=10, validate=False, max_global=2)
        assert lf.device_status(kind="forward") & lf.LF_DEV_TOO_MANY_GLOBALS
    s2 = torch.cuda.Stream()
    with torch.cuda.stream(s2):
        lf.forward(*t, *g, mask=mask, window=10, validate=False, max_global=5)
        assert lf.device_status(kind="forward") == 0


# ---------------------------------------------------------------------------
# Named workloads at full size, sampled rows
# ---------------------------------------------------------------------------

def _sample_rows(n, w, mask_b, rng, extra=()):
    base = {0, 1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, w - 1, w, w + 1,
            n // 2, n - w - 1, n - w, n - 2, n - 1}
    base |= set(int(x) for x in rng.integers(0, n, size=24))
    base |= set(int(x) for x in np.flatnonzero(mask_b == 2)[:20])
    nz = np.flatnonzero(mask_b == 0)
    if nz.size:
        base |= {int(nz[0]) - 2, int(nz[0]) - 1, int(nz[0]), int(nz[-1])}
    base |= set(extra)
    return sorted(x for x in base if 0 <= x < n)


@pytest.mark.parametrize("name", ["longformer_base_n4096", "qa_padded_b2_n4096",
                                  "charlm_causal_dilated_n23040", "led_large_n16384",
                                  "charlm_causal_dilated_n32256"])
def test_workload_sampled_parity(name):
    prob = workloads.by_name(name)
    B, n, H, D = prob.shape
    max_global = prob.max_global()
    out, nnz = run_gpu(prob, validate=False, max_global=max_global)
    arrs = _np(prob)
    mask = prob.mask.numpy()
    rng = np.random.default_rng(0)
    worst = 0.0
    for b in range(B):
        for h in range(H):
            rows = _sample_rows(n, prob.window, mask[b], rng)
            ref, rnnz = oracle.forward_rows(*arrs, mask, prob.window, b, h, rows,
                                            dilation=prob.dilation, causal=prob.causal,
                                            scale=prob.scale)
            np.testing.assert_array_equal(nnz[b, h, rows], rnnz)
            err = np.abs(out[b, rows, h] - ref).max()
            worst = max(worst, err)
            assert err <= TOL[prob.q.dtype], (b, h, err)
    # pair counts of every (b, h) against the oracle's count of the same key
    # sets (exact integers)
    for b in range(B):
        for h in range(H):
            dil = prob.dilation[h] if prob.dilation else 1
            assert int(nnz[b, h].sum()) == oracle.pair_count(mask[b], prob.window, dil, prob.causal), (b, h)
    # pair counts: closed forms where the workload has one
    if name == "longformer_base_n4096":
        assert nnz.sum() == 2043134 * 12
    if name == "charlm_causal_dilated_n23040":
        assert nnz.sum() == 93242880
    if name == "charlm_causal_dilated_n32256":
        # sum over heads and residues r of sum_t (min(t, w) + 1), t < |{r, r+d, ...}|
        assert nnz.sum() == 131065344
    assert (out[np.broadcast_to((mask == 0)[:, :, None, None], out.shape)] == 0).all()
    _say(f"      {name}: worst sampled abs err {worst:.3e}")


def test_longformer_base_f16_two_heads_full():
    """The metric workload's shape and values in f16, every row of two heads."""
    prob = workloads.longformer_base_n4096()
    for name in ("q", "k", "v", "q_g", "k_g", "v_g"):
        setattr(prob, name, getattr(prob, name).to(torch.float16))
    out, nnz = run_gpu(prob, validate=False, max_global=1)
    arrs = _np(prob)
    mask = prob.mask.numpy()
    for h in (0, 7):
        ref, rnnz = oracle.forward_rows(*arrs, mask, prob.window, 0, h, range(4096))
        np.testing.assert_array_equal(nnz[0, h], rnnz)
        err = np.abs(out[0, :, h] - ref).max()
        _say(f"      f16 head {h}: max abs err {err:.3e}")
        assert err <= TOL[torch.float16]


def test_longformer_base_two_heads_full():
    """The metric workload, every row of two heads against the full oracle."""
    prob = workloads.longformer_base_n4096()
    out, nnz = run_gpu(prob, validate=False, max_global=1)
    arrs = _np(prob)
    mask = prob.mask.numpy()
    for h in (0, 11):
        ref, rnnz = oracle.forward_rows(*arrs, mask, prob.window, 0, h, range(4096))
        np.testing.assert_array_equal(nnz[0, h], rnnz)
        err = np.abs(out[0, :, h] - ref).max()
        _say(f"      head {h}: max abs err {err:.3e}")
        assert err <= 2e-2


@pytest.mark.parametrize("name,pairs", [
    ("qa_padded_b2_n4096", [(0, 0), (1, 11)]),
    ("charlm_causal_dilated_n23040", [(0, 0), (0, 7)]),
    ("led_large_n16384", [(0, 0), (0, 15)]),
    ("charlm_causal_dilated_n32256", [(0, 5), (0, 6)]),
])
def test_workload_two_heads_full(name, pairs):
    """Every row of two (batch row, head) pairs of each full-size workload
    against the oracle (the dilated workloads: one undilated and one dilated
    head), in the launch configuration the benchmark times."""
    prob = workloads.by_name(name)
    out, nnz = run_gpu(prob, validate=False, max_global=prob.max_global())
    arrs = _np(prob)
    mask = prob.mask.numpy()
    n = prob.shape[1]
    for b, h in pairs:
        ref, rnnz = oracle.forward_rows(*arrs, mask, prob.window, b, h, range(n), dilation=prob.dilation,
                                        causal=prob.causal, scale=prob.scale)
        np.testing.assert_array_equal(nnz[b, h], rnnz)
        err = np.abs(out[b, :, h] - ref).max()
        _say(f"      {name} (b {b}, h {h}): max abs err {err:.3e}")
        assert err <= TOL[prob.q.dtype], (b, h, err)
