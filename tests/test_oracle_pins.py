"""Pins for the fp64 oracle, against things other than the oracle itself:
the numbers the pages print, closed forms, textbook routines (torch's fp64
scaled-dot-product attention on the CPU), hand-derived key sets, invariants,
and an independent dense formulation on tiny inputs.  CPU only.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import longformer_attention as lfo

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(rng, B, n, H, D=64):
    return rng.standard_normal((B, n, H, D))


def _problem(rng, B, n, H, D=64):
    return [_rand(rng, B, n, H, D) for _ in range(6)]


def _sdpa(q, k, v, mask=None, causal=False, scale=None):
    """torch's reference attention in fp64 on [n, D] operands."""
    Q = torch.from_numpy(q)[None, None]
    K = torch.from_numpy(k)[None, None]
    V = torch.from_numpy(v)[None, None]
    am = None if mask is None else torch.from_numpy(mask)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(
        Q, K, V, attn_mask=am, is_causal=causal, scale=scale)
    return o[0, 0].numpy()


# ---------------------------------------------------------------------------
# Worked example printed on the ultralytics glossary pages
# ---------------------------------------------------------------------------

def _read_worked():
    rows = []
    with open(os.path.join(GOLDEN, "worked_mask_counts.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            n, lf, full = line.split()
            rows.append((int(n), float(lf), float(full)))
    return rows


@pytest.mark.parametrize("case", _read_worked())
def test_worked_example_printed_counts(case):
    """Window 512 (w = 256 per side), token 0 global: the scored-pair counts
    the page prints, in millions at one decimal."""
    n, lf_millions, full_millions = case
    mask = np.ones(n, dtype=np.int8)
    mask[0] = 2
    p = oracle.pair_count(mask, 256)
    assert round(p / 1e6, 1) == lf_millions
    assert round(n * n / 1e6, 1) == full_millions


@pytest.mark.parametrize("n,expect", [(1024, 461054), (2048, 988414), (4096, 2043134)])
def test_worked_example_exact_counts(n, expect):
    """Exact integers of the same example from a closed form.

    Band without globals: every row has 2w+1 window positions, minus the
    positions that fall off either end: sum_{i<w}(w-i) on each side,
    i.e. n(2w+1) - w(w+1).  Global token 0: its own row grows from w+1
    (its window) to n, and every row i > w gains column 0 once
    (n - w - 1 rows).  Total = n(2w+1) - w(w+1) - (w+1) + n + (n-w-1).
    """
    w = 256
    closed = n * (2 * w + 1) - w * (w + 1) - (w + 1) + n + (n - w - 1)
    assert closed == expect
    mask = np.ones(n, dtype=np.int8)
    mask[0] = 2
    assert oracle.pair_count(mask, w) == expect
    # double counting column 0 for the rows whose window holds it would
    # add w more pairs (rows 1..w); the exact count excludes that
    assert expect != closed + w


# ---------------------------------------------------------------------------
# Closed-form pair counts
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,w", [(512, 64), (4096, 256), (16384, 512), (100, 7), (10, 9), (10, 30)])
def test_band_count_closed_form(n, w):
    mask = np.ones(n, dtype=np.int8)
    expect = n * (2 * w + 1) - w * (w + 1) if n > w else n * n
    assert oracle.pair_count(mask, w) == expect


def _causal_count(n_r, w):
    # rows t = 0..n_r-1 of one residue class see min(w, t) + 1 keys
    if n_r - 1 >= w:
        return n_r + w * (w + 1) // 2 + w * (n_r - 1 - w)
    return n_r * (n_r + 1) // 2


def test_causal_dilated_count_closed_form():
    """Character-LM layer shape: n = 23040, causal w = 512, dilation 1 on six
    heads and 2 on two; a dilated head is a plain causal window over each
    residue class {r, r+d, ...}."""
    n, w = 23040, 512
    mask = np.ones(n, dtype=np.int8)
    total = 0
    for dil in [1] * 6 + [2] * 2:
        c = oracle.pair_count(mask, w, dil=dil, causal=True)
        expect = sum(_causal_count(len(range(r, n, dil)), w) for r in range(dil))
        assert c == expect
        total += c
    assert total == 93242880


# ---------------------------------------------------------------------------
# Hand-derived key sets read back through the forward
# ---------------------------------------------------------------------------

def _read_sets():
    cases = []
    cur = None
    with open(os.path.join(GOLDEN, "key_sets_small.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("case"):
                parts = dict(p.split("=") for p in line.split()[2:])
                cur = {
                    "name": line.split()[1],
                    "n": int(parts["n"]), "w": int(parts["w"]),
                    "dil": int(parts["dil"]), "causal": parts["causal"] == "1",
                    "mask": np.array([int(c) for c in parts["mask"]], dtype=np.int8),
                    "rows": {},
                }
                cases.append(cur)
            else:
                head, keys = line.split(":")
                i = int(head.split()[1])
                keys = keys.strip()
                cur["rows"][i] = None if keys == "-" else [int(x) for x in keys.split()]
    return cases


@pytest.mark.parametrize("case", _read_sets(), ids=lambda c: c["name"])
def test_key_sets_readback(case):
    """q = q_g = 0 makes every score equal, so out_i is the mean of the value
    rows over S(i); one-hot value rows (n <= D) read S(i) back exactly."""
    n, D = case["n"], 64
    q = np.zeros((1, n, 1, D))
    v = np.zeros((1, n, 1, D))
    v[0, np.arange(n), 0, np.arange(n)] = 1.0
    k = np.random.default_rng(0).standard_normal((1, n, 1, D))
    out, nnz = oracle.forward(q, k, v, q, k, v, case["mask"][None], case["w"],
                              dilation=[case["dil"]], causal=case["causal"])
    for i, keys in case["rows"].items():
        row = out[0, i, 0]
        if keys is None:
            assert np.all(row == 0) and nnz[0, 0, i] == 0
            continue
        expect = np.zeros(D)
        expect[keys] = 1.0 / len(keys)
        np.testing.assert_allclose(row, expect, rtol=0, atol=1e-15)
        assert nnz[0, 0, i] == len(keys)


# ---------------------------------------------------------------------------
# Textbook special cases (torch fp64 SDPA on the CPU)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,w", [(33, 32), (40, 100)])
def test_full_window_is_dense_attention(n, w):
    rng = np.random.default_rng(1)
    q, k, v, qg, kg, vg = _problem(rng, 1, n, 2)
    mask = np.ones((1, n), dtype=np.int8)
    out, nnz = oracle.forward(q, k, v, qg, kg, vg, mask, w)
    for h in range(2):
        ref = _sdpa(q[0, :, h], k[0, :, h], v[0, :, h])
        np.testing.assert_allclose(out[0, :, h], ref, rtol=0, atol=1e-12)
    assert (nnz == n).all()


def test_full_causal_window_is_causal_attention():
    rng = np.random.default_rng(2)
    n = 50
    q, k, v, qg, kg, vg = _problem(rng, 1, n, 1)
    mask = np.ones((1, n), dtype=np.int8)
    out, nnz = oracle.forward(q, k, v, qg, kg, vg, mask, n + 3, causal=True)
    ref = _sdpa(q[0, :, 0], k[0, :, 0], v[0, :, 0], causal=True)
    np.testing.assert_allclose(out[0, :, 0], ref, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(out[0, 0, 0], v[0, 0, 0])
    np.testing.assert_array_equal(nnz[0, 0], np.arange(1, n + 1))


def test_scale_argument_matches_sdpa_scale():
    rng = np.random.default_rng(3)
    n = 20
    q, k, v, qg, kg, vg = _problem(rng, 1, n, 1)
    mask = np.ones((1, n), dtype=np.int8)
    out, _ = oracle.forward(q, k, v, qg, kg, vg, mask, n, scale=0.3)
    ref = _sdpa(q[0, :, 0], k[0, :, 0], v[0, :, 0], scale=0.3)
    np.testing.assert_allclose(out[0, :, 0], ref, rtol=0, atol=1e-12)


def test_global_init_projections_give_dense_attention():
    """With Q_g/K_g/V_g initialised to Q_s/K_s/V_s (segmentfault summary,
    global projections) and a window covering the whole sequence, every
    row sees every token once, whichever tokens are global.  A global key
    counted twice would shift that row's softmax weights."""
    rng = np.random.default_rng(4)
    n = 48
    q, k, v, _, _, _ = _problem(rng, 1, n, 2)
    mask = np.ones((1, n), dtype=np.int8)
    mask[0, [0, 7, 30]] = 2
    out, nnz = oracle.forward(q, k, v, q, k, v, mask, n)
    for h in range(2):
        ref = _sdpa(q[0, :, h], k[0, :, h], v[0, :, h])
        np.testing.assert_allclose(out[0, :, h], ref, rtol=0, atol=1e-12)
    assert (nnz == n).all()


def test_global_row_is_attention_over_valid_tokens():
    """A global row is plain attention of q_g over all valid (k_g, v_g)."""
    rng = np.random.default_rng(5)
    n = 60
    q, k, v, qg, kg, vg = _problem(rng, 1, n, 1)
    mask = np.ones((1, n), dtype=np.int8)
    mask[0, [3, 40]] = 2
    mask[0, 50:] = 0
    mask[0, 20] = 0
    out, nnz = oracle.forward(q, k, v, qg, kg, vg, mask, 4)
    valid = np.flatnonzero(mask[0] != 0)
    for g in (3, 40):
        ref = _sdpa(qg[0, g:g + 1, 0], kg[0, valid, 0], vg[0, valid, 0])
        np.testing.assert_allclose(out[0, g, 0], ref[0], rtol=0, atol=1e-12)
        assert nnz[0, 0, g] == valid.size


def test_local_row_with_global_column_matches_masked_sdpa():
    """A local row far from the global token: its keys are its window plus
    the global column, scored with the local projections."""
    rng = np.random.default_rng(6)
    n, w = 64, 3
    q, k, v, qg, kg, vg = _problem(rng, 1, n, 1)
    mask = np.ones((1, n), dtype=np.int8)
    mask[0, 0] = 2
    out, nnz = oracle.forward(q, k, v, qg, kg, vg, mask, w)
    i = 30
    keys = [0] + list(range(i - w, i + w + 1))
    ref = _sdpa(q[0, i:i + 1, 0], k[0, keys, 0], v[0, keys, 0])
    np.testing.assert_allclose(out[0, i, 0], ref[0], rtol=0, atol=1e-12)
    assert nnz[0, 0, i] == 2 * w + 2


# ---------------------------------------------------------------------------
# Invariants
# ---------------------------------------------------------------------------

def test_rows_sum_to_one():
    rng = np.random.default_rng(7)
    n = 70
    q, k, _, qg, kg, _ = _problem(rng, 2, n, 3)
    ones = np.ones((2, n, 3, 64))
    mask = np.ones((2, n), dtype=np.int8)
    mask[0, [1, 33]] = 2
    mask[1, 60:] = 0
    out, _ = oracle.forward(q, k, ones, qg, kg, ones, mask, 5, dilation=[1, 2, 3])
    live = (mask != 0)[:, :, None, None]
    np.testing.assert_allclose(out, np.broadcast_to(np.where(live, 1.0, 0.0), out.shape), rtol=0, atol=1e-13)


def test_zero_window_returns_values():
    rng = np.random.default_rng(8)
    q, k, v, qg, kg, vg = _problem(rng, 1, 25, 2)
    mask = np.ones((1, 25), dtype=np.int8)
    out, nnz = oracle.forward(q, k, v, qg, kg, vg, mask, 0, dilation=[1, 4])
    np.testing.assert_array_equal(out, v)
    assert (nnz == 1).all()


@pytest.mark.parametrize("causal", [False, True])
def test_dilated_head_is_window_over_residue_classes(causal):
    rng = np.random.default_rng(9)
    n, w, d = 61, 4, 3
    q, k, v, qg, kg, vg = _problem(rng, 1, n, 1)
    mask = np.ones((1, n), dtype=np.int8)
    mask[0, [5, 17, 40]] = 0
    out, nnz = oracle.forward(q, k, v, qg, kg, vg, mask, w, dilation=[d], causal=causal)
    for r in range(d):
        sl = slice(r, None, d)
        o2, c2 = oracle.forward(q[:, sl], k[:, sl], v[:, sl], qg[:, sl], kg[:, sl],
                                vg[:, sl], mask[:, sl], w, causal=causal)
        np.testing.assert_allclose(out[:, sl], o2, rtol=0, atol=1e-13)
        np.testing.assert_array_equal(nnz[:, :, sl], c2)


def test_padding_does_not_change_real_tokens():
    rng = np.random.default_rng(10)
    n, pad = 45, 19
    q, k, v, qg, kg, vg = _problem(rng, 1, n + pad, 2)
    mask = np.ones((1, n + pad), dtype=np.int8)
    mask[0, [2, 30]] = 2
    mask[0, n:] = 0
    out, nnz = oracle.forward(q, k, v, qg, kg, vg, mask, 6, dilation=[1, 2])
    o2, c2 = oracle.forward(q[:, :n], k[:, :n], v[:, :n], qg[:, :n], kg[:, :n],
                            vg[:, :n], mask[:, :n], 6, dilation=[1, 2])
    np.testing.assert_allclose(out[:, :n], o2, rtol=0, atol=1e-13)
    np.testing.assert_array_equal(nnz[:, :, :n], c2)
    assert (out[:, n:] == 0).all() and (nnz[:, :, n:] == 0).all()


def test_masked_out_positions_do_not_influence_outputs():
    """Non-finite data at mask-0 positions never reaches any output."""
    rng = np.random.default_rng(11)
    n = 40
    q, k, v, qg, kg, vg = _problem(rng, 1, n, 1)
    mask = np.ones((1, n), dtype=np.int8)
    mask[0, 0] = 2
    mask[0, [9, 10, 25]] = 0
    out, _ = oracle.forward(q, k, v, qg, kg, vg, mask, 5)
    for t in (k, v, kg, vg):
        t[0, [9, 10, 25]] = np.nan
    out2, _ = oracle.forward(q, k, v, qg, kg, vg, mask, 5)
    np.testing.assert_array_equal(out, out2)


# ---------------------------------------------------------------------------
# Banded oracle vs independent dense formulation, random tiny problems
# ---------------------------------------------------------------------------

def _random_case(seed):
    rng = np.random.default_rng(1000 + seed)
    n = int(rng.integers(1, 97))
    H = int(rng.integers(1, 4))
    B = int(rng.integers(1, 3))
    w = int(rng.integers(0, n + 1))
    causal = bool(rng.integers(0, 2))
    dil = [int(x) for x in rng.integers(1, 5, size=H)]
    mask = np.ones((B, n), dtype=np.int8)
    for b in range(B):
        mask[b, rng.random(n) < 0.1] = 0
        tail = int(rng.integers(0, max(1, n // 3)))
        if tail:
            mask[b, n - tail:] = 0
        if not causal:
            ng = int(rng.integers(0, 9))
            cand = np.flatnonzero(mask[b])
            if ng and cand.size:
                mask[b, rng.choice(cand, size=min(ng, cand.size), replace=False)] = 2
    D = int(rng.choice([8, 64]))
    t = [rng.standard_normal((B, n, H, D)) for _ in range(6)]
    return t, mask, w, dil, causal


@pytest.mark.parametrize("seed", range(40))
def test_banded_matches_dense_bruteforce(seed):
    t, mask, w, dil, causal = _random_case(seed)
    out, nnz = oracle.forward(*t, mask, w, dilation=dil, causal=causal)
    o2, c2 = oracle.dense_bruteforce(*t, mask, w, dilation=dil, causal=causal)
    np.testing.assert_allclose(out, o2, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(nnz, c2)
    for b in range(mask.shape[0]):
        for h, d in enumerate(dil):
            assert oracle.pair_count(mask[b], w, dil=d, causal=causal) == nnz[b, h].sum()


def test_forward_rows_matches_forward():
    t, mask, w, dil, causal = _random_case(3)
    out, nnz = oracle.forward(*t, mask, w, dilation=dil, causal=causal)
    n = mask.shape[1]
    rows = [0, n // 2, n - 1]
    o, c = oracle.forward_rows(*t, mask, w, 0, 0, rows, dilation=dil, causal=causal)
    np.testing.assert_array_equal(o, out[0, rows, 0])
    np.testing.assert_array_equal(c, nnz[0, 0, rows])


# ---------------------------------------------------------------------------
# Errors for undefined inputs
# ---------------------------------------------------------------------------

def test_rejects_causal_with_globals():
    rng = np.random.default_rng(12)
    t = _problem(rng, 1, 8, 1)
    mask = np.ones((1, 8), dtype=np.int8)
    mask[0, 0] = 2
    with pytest.raises(ValueError):
        oracle.forward(*t, mask, 2, causal=True)


def test_rejects_unknown_mask_values():
    rng = np.random.default_rng(13)
    t = _problem(rng, 1, 8, 1)
    mask = np.ones((1, 8), dtype=np.int8)
    mask[0, 3] = 3
    with pytest.raises(ValueError):
        oracle.forward(*t, mask, 2)


# ---------------------------------------------------------------------------
# Planted mistakes: each plausible slip in the oracle trips a pin above
# ---------------------------------------------------------------------------

def test_planted_window_off_by_one_is_caught(monkeypatch):
    orig = lfo.in_window

    def narrow(i, j, w, dil, causal):  # exclusive bound instead of inclusive
        d = np.asarray(i) - np.asarray(j)
        return orig(i, j, w, dil, causal) & (np.abs(d) < w * dil)

    monkeypatch.setattr(lfo, "in_window", narrow)
    mask = np.ones(1024, dtype=np.int8)
    mask[0] = 2
    assert lfo.pair_count(mask, 256) != 461054


def test_planted_double_count_is_caught(monkeypatch):
    def never(i, j, w, dil, causal):  # every global column appended again
        return np.zeros(np.broadcast(np.asarray(i), np.asarray(j)).shape, dtype=bool)

    monkeypatch.setattr(lfo, "in_window", never)
    mask = np.ones(1024, dtype=np.int8)
    mask[0] = 2
    assert lfo.pair_count(mask, 256) != 461054


def test_planted_causal_sign_is_caught(monkeypatch):
    orig = lfo.in_window

    def flipped(i, j, w, dil, causal):  # keys to the right instead of left
        return orig(j, i, w, dil, causal)

    monkeypatch.setattr(lfo, "in_window", flipped)
    rng = np.random.default_rng(2)
    n = 50
    q, k, v, qg, kg, vg = _problem(rng, 1, n, 1)
    mask = np.ones((1, n), dtype=np.int8)
    # forward gathers the window by offsets, so the flip shows in the dense
    # formulation, which is compared against causal SDPA here
    out, _ = lfo.dense_bruteforce(q, k, v, qg, kg, vg, mask, n + 3, causal=True)
    ref = _sdpa(q[0, :, 0], k[0, :, 0], v[0, :, 0], causal=True)
    assert not np.allclose(out[0, :, 0], ref, atol=1e-6)


def test_planted_transposed_scores_are_caught(monkeypatch):
    orig = lfo._softmax_rows
    seen = {}

    def wrong_axis(e):  # normalise over the wrong axis for square blocks
        if e.ndim == 2 and e.shape[0] == e.shape[1]:
            seen["hit"] = True
            mx = e.max(axis=0, keepdims=True)
            p = np.exp(e - mx)
            return p / p.sum(axis=0, keepdims=True)
        return orig(e)

    monkeypatch.setattr(lfo, "_softmax_rows", wrong_axis)
    rng = np.random.default_rng(1)
    n = 33
    q, k, v, qg, kg, vg = _problem(rng, 1, n, 1)
    mask = np.ones((1, n), dtype=np.int8)
    out, _ = lfo.dense_bruteforce(q, k, v, qg, kg, vg, mask, 32)
    ref = _sdpa(q[0, :, 0], k[0, :, 0], v[0, :, 0])
    assert seen and not np.allclose(out[0, :, 0], ref, atol=1e-6)
