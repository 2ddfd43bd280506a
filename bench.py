"""Benchmark: Longformer sliding-window + global attention forward on one MI355X.

One step = one lf_attn_forward over one batch of seeded synthetic inputs
already resident in HBM (the whole hot path: mask scan, band tiles, global
columns, split global rows and their merge; one kernel launch).

Default workload: the longformer-base layer shape, B=1, n=4096, H=12, D=64,
one-sided window 256, bf16, token 0 global.  Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--no-cpu-baseline] [--no-check] [--no-cold] [--eager]
                  [--pass forward|backward|projections] [--sweep]

The timed value is warm: graph replays of the launch with its inputs
resident.  The line also carries a cold figure (each launch after a 512 MB
write that evicts the caches), the scored pairs of the launch split into
window, global-column and global-row pairs with their exact FLOPs, and the
CPU-baseline leg: the fp64 oracle on whole (batch row, head) pairs of the
workload, timed, whose rows are also compared with the timed output (the
parity field).  Only that leg touches the oracle.

With --sweep it times the longformer-base layer shape at n = 1024 ... 16384
(linear growth in n) and prints one line per length.

--workload longformer_base_n4096_d128 (or _d32) times the same layer shape
with head dim 128 (32) in place of 64.

With --pass projections a step is one lf_attn_project: the six input
projections (Q_s, K_s, V_s, Q_g, K_g, V_g) of the workload's B*n tokens
from C = H*64 hidden features.

With --pass backward a step is one lf_attn_backward (preparation with the
global lists, then the gradient kernel) on the same workload, from the output and
row log-sum-exp of one lf_attn_forward_lse and a seeded upstream gradient.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 matrix
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def band_flops(prob) -> float:
    """Useful band FLOPs of one forward: 4*n*(2w+1)*D*H*B (QK^T and PV over
    the 2w+1 window diagonals); for a causal window the w+1 diagonals that
    exist."""
    B, n, H, D = prob.shape
    keys = prob.window + 1 if prob.causal else 2 * prob.window + 1
    return 4.0 * n * keys * D * H * B


def algorithmic_bytes(prob) -> float:
    """Bytes the method must move once: q, k, v read and out written per
    (token, head); k_g, v_g per (token, head) of batch rows with a global
    token; q_g of global rows; the mask."""
    B, n, H, D = prob.shape
    elt = prob.q.element_size()
    g = (prob.mask == 2).sum(dim=1)
    total = 4.0 * B * n * H * D * elt + B * n
    for b in range(B):
        if int(g[b]) > 0:
            total += 2.0 * n * H * D * elt + int(g[b]) * H * D * elt
    return total


def window_valid_counts(prob, b, h):
    """Per query row of (b, h): the number of valid keys (mask != 0) in its
    window W(i) = {i + k d : -w <= k <= w (causal: <= 0), 0 <= i + k d < n},
    from prefix sums over each residue class.  Host-side accounting of the
    measured work (it splits the kernel's row_nnz into window and global
    pairs); no part of the attention."""
    import numpy as np

    B, n, H, D = prob.shape
    d = prob.dilation[h] if prob.dilation else 1
    w = prob.window
    w_hi = 0 if prob.causal else w
    valid = (prob.mask[b].numpy() != 0).astype(np.int64)
    out = np.zeros(n, dtype=np.int64)
    for r in range(min(d, n)):
        sub = valid[r::d]
        pre = np.concatenate([[0], np.cumsum(sub)])
        t = np.arange(sub.size)
        lo = np.clip(t - w, 0, sub.size)
        hi = np.clip(t + w_hi + 1, 0, sub.size)
        out[r::d] = pre[hi] - pre[lo]
    return out


def pair_accounting(prob, row_nnz):
    """Scored pairs of the measured launch (the kernel's row_nnz, checked
    bit-exact against the oracle by the parity tests) split into window
    pairs of local rows, global columns of local rows and global rows, and
    the exact FLOPs 4 D P of each (QK^T and P V, 2 D each per pair)."""
    import numpy as np

    B, n, H, D = prob.shape
    c = row_nnz.cpu().numpy().astype(np.int64)
    m = prob.mask.numpy()
    if prob.causal:
        m = np.where(m == 2, 1, m)
    win = glob_cols = glob_rows = 0
    for b in range(B):
        loc = m[b] == 1
        gl = m[b] == 2
        for h in range(H):
            wv = window_valid_counts(prob, b, h)
            win += int(wv[loc].sum())
            glob_cols += int((c[b, h][loc] - wv[loc]).sum())
            glob_rows += int(c[b, h][gl].sum())
    total = win + glob_cols + glob_rows
    return {"pairs": total, "pairs_window": win, "pairs_global_columns": glob_cols,
            "pairs_global_rows": glob_rows, "flops_exact": 4.0 * D * total,
            "flops_window": 4.0 * D * win, "flops_global_columns": 4.0 * D * glob_cols,
            "flops_global_rows": 4.0 * D * glob_rows}


class Runner:
    """Prepared arguments for repeated lf_attn_forward calls on torch's
    current stream (ctypes call only, no per-call validation)."""

    def __init__(self, prob, device):
        import torch

        import sparse_long_document_amd as lf

        self.lf = lf
        self.prob = prob
        self.t = [x.to(device).contiguous() for x in (prob.q, prob.k, prob.v, prob.q_g, prob.k_g, prob.v_g)]
        self.mask = prob.mask.to(device).contiguous()
        self.out = torch.empty_like(self.t[0])
        B, n, H, D = prob.shape
        self.row_nnz = torch.empty((B, H, n), dtype=torch.int32, device=device)
        self.max_global = 0 if prob.causal else prob.max_global()
        self.params, self._keep = lf.make_params(B, n, H, D, prob.window, prob.dilation, prob.causal,
                                                 prob.scale, self.max_global, prob.q.dtype)
        lib = lf.library()
        need = lib.lf_attn_workspace_bytes(ctypes.byref(self.params))
        self.stream = torch.cuda.current_stream(device).cuda_stream
        self.ws = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
        st = lib.lf_attn_workspace_init(ctypes.c_void_p(self.ws.data_ptr()), self.ws.numel(),
                                        ctypes.c_void_p(self.stream))
        assert st == 0, st
        vp = ctypes.c_void_p
        self.args = (ctypes.byref(self.params), *[vp(x.data_ptr()) for x in self.t], vp(self.mask.data_ptr()),
                     vp(self.out.data_ptr()), vp(self.row_nnz.data_ptr()), vp(self.ws.data_ptr()),
                     ctypes.c_size_t(self.ws.numel()), vp(self.stream))
        self.fn = lib.lf_attn_forward

    def launch(self):
        st = self.fn(*self.args)
        if st != 0:
            raise RuntimeError(f"lf_attn_forward failed with status {st}")


def backward_bytes(prob) -> float:
    """Bytes the backward must move once: q, k, v, out and dout read and the
    six fp32 gradients written per (token, head); k_g, v_g of batch rows
    with a global token and q_g of the global rows; the row log-sum-exp
    (4 B per row); the mask."""
    B, n, H, D = prob.shape
    elt = prob.q.element_size()
    g = (prob.mask == 2).sum(dim=1)
    total = B * n * H * (5.0 * D * elt + 6.0 * D * 4 + 4) + B * n
    for b in range(B):
        if int(g[b]) > 0:
            total += 2.0 * n * H * D * elt + int(g[b]) * H * D * elt
    return total


def backward_flops(prob) -> float:
    """Useful band FLOPs of one backward: per scored window pair, the score
    recomputed once and the four gradient products dP, dV, dQ, dK, each
    2*D: 2.5 times the forward's count."""
    return 2.5 * band_flops(prob)


class BwdRunner:
    """Prepared arguments for repeated lf_attn_backward calls: out and lse
    from one lf_attn_forward_lse, a seeded upstream gradient."""

    def __init__(self, prob, device):
        import torch

        import sparse_long_document_amd as lf
        import workloads

        self.prob = prob
        self.t = [x.to(device).contiguous() for x in (prob.q, prob.k, prob.v, prob.q_g, prob.k_g, prob.v_g)]
        self.mask = prob.mask.to(device).contiguous()
        self.dout = workloads.upstream_grad(2, prob.shape, prob.q.dtype).to(device)
        self.max_global = 0 if prob.causal else prob.max_global()
        self.out, self.lse = lf.forward(*self.t, mask=self.mask, window=prob.window, dilation=prob.dilation,
                                        causal=prob.causal, scale=prob.scale, return_lse=True,
                                        max_global=self.max_global, validate=False)
        B, n, H, D = prob.shape
        self.grads = [torch.empty((B, n, H, D), dtype=torch.float32, device=device) for _ in range(6)]
        self.params, self._keep = lf.make_params(B, n, H, D, prob.window, prob.dilation, prob.causal,
                                                 prob.scale, self.max_global, prob.q.dtype)
        lib = lf.library()
        need = lib.lf_attn_backward_workspace_bytes(ctypes.byref(self.params))
        self.stream = torch.cuda.current_stream(device).cuda_stream
        self.ws = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
        st = lib.lf_attn_workspace_init(ctypes.c_void_p(self.ws.data_ptr()), self.ws.numel(),
                                        ctypes.c_void_p(self.stream))
        assert st == 0, st
        vp = ctypes.c_void_p
        self.args = (ctypes.byref(self.params), *[vp(x.data_ptr()) for x in self.t], vp(self.mask.data_ptr()),
                     vp(self.out.data_ptr()), vp(self.dout.data_ptr()), vp(self.lse.data_ptr()),
                     *[vp(g.data_ptr()) for g in self.grads], vp(self.ws.data_ptr()),
                     ctypes.c_size_t(self.ws.numel()), vp(self.stream))
        self.fn = lib.lf_attn_backward
        self.out_t = self.grads[0]  # dq: written without atomics, compared across graph replays

    def launch(self):
        st = self.fn(*self.args)
        if st != 0:
            raise RuntimeError(f"lf_attn_backward failed with status {st}")


class ProjRunner:
    """Prepared arguments for repeated lf_attn_project calls: the six
    projections of the workload's tokens."""

    def __init__(self, prob, device, global_only=False):
        import torch

        import sparse_long_document_amd as lf
        import workloads

        B, n, H, D = prob.shape
        self.M, self.C, self.P = B * n, H * D, 6
        self.global_only = global_only
        self.mask = prob.mask.reshape(-1).to(torch.int8).to(device).contiguous()
        x, w, b = workloads.projection_problem(3, self.M, self.C, self.P, prob.q.dtype)
        self.x_cpu, self.w_cpu, self.b_cpu = x, w, b
        self.x, self.w, self.b = x.to(device), w.to(device), b.to(device)
        self.out = torch.empty((self.P, self.M, self.C), dtype=prob.q.dtype, device=device)
        self.out_t = self.out
        self.stream = torch.cuda.current_stream(device).cuda_stream
        vp = ctypes.c_void_p
        self.lib = lf.library()
        self.dt = lf._DTYPES[prob.q.dtype]
        if global_only:  # Q_g (projection 3) at the global tokens only
            self.args = (self.M, self.C, self.P, self.dt, vp(self.x.data_ptr()), vp(self.w.data_ptr()),
                         vp(self.b.data_ptr()), vp(self.mask.data_ptr()), ctypes.c_uint32(1 << 3),
                         vp(self.out.data_ptr()), vp(self.stream))
            self.fn = self.lib.lf_attn_project_global_only
        else:
            self.args = (self.M, self.C, self.P, self.dt, vp(self.x.data_ptr()), vp(self.w.data_ptr()),
                         vp(self.b.data_ptr()), vp(self.out.data_ptr()), vp(self.stream))
            self.fn = self.lib.lf_attn_project

    def launch(self):
        st = self.fn(*self.args)
        if st != 0:
            raise RuntimeError(f"lf_attn_project failed with status {st}")


class EncRunner:
    """The encoder attention sublayer as one step: the six input projections,
    the attention and the output projection (three launches), on the LED
    encoder workload's shape."""

    def __init__(self, prob, device):
        import torch

        import sparse_long_document_amd as lf
        import workloads

        self.lf = lf
        self.enc = workloads.led_encoder_n16384() if prob is None else prob
        e = self.enc
        B, n, C = e.shape
        self.x, self.w, self.bias = e.x.to(device), e.w.to(device), e.bias.to(device)
        self.w_out, self.b_out = e.w_out.to(device), e.b_out.to(device)
        self.mask = e.mask.to(device)
        self.mg = e.max_global()
        self.ws = lf.make_workspace(B, n, e.H, e.window, max_global=self.mg, dtype=e.x.dtype)
        self.out_t = torch.empty((B, n, C), dtype=e.x.dtype, device=device)
        self.args = (None,)  # the stream is torch's current one

    def launch(self):
        y = self.lf.encoder_attention(self.x, self.w, self.bias, self.mask, self.enc.window, max_global=self.mg,
                                      validate=False, w_out=self.w_out, b_out=self.b_out, workspace=self.ws)
        self.out_t.copy_(y)


def report_encoder(args, run, ms, mode, t_wall):
    import torch

    e = run.enc
    B, n, C = e.shape
    H = e.H
    flops_proj = 2.0 * B * n * C * 7 * C  # six input projections and the output projection
    flops_band = 4.0 * B * n * (2 * e.window + 1) * 64 * H
    result = {
        "metric": "LED encoder attention sublayer tokens/s (projections, attention, output projection), bf16",
        "value": B * n / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) hidden states, N(0,1/C) weights, token 0 + 16 random global)",
        "config": {"workload": e.name, "pass": "encoder", "B": B, "n": n, "C": C, "H": H, "w": e.window,
                   "globals_per_row": [int(x) for x in (e.mask == 2).sum(dim=1).tolist()],
                   "timing": mode, "wall_s": round(t_wall, 3)},
        "flops": {"projections": flops_proj, "attention_band": flops_band},
        "mfma_frac": (flops_proj + flops_band) / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
    }
    print(json.dumps(result), flush=True)


def report_projections(args, prob, run, ms, mode, t_wall):
    import numpy as np
    import torch

    flops = 2.0 * run.M * run.C * run.P * run.C
    if run.global_only:  # Q_g only at the global tokens: the FLOPs actually needed
        n_glob = int((run.mask == 2).sum().item())
        flops = 2.0 * run.M * run.C * (run.P - 1) * run.C + 2.0 * n_glob * run.C * run.C
    achieved = flops / (ms * 1e-3) / 1e12
    dname = {torch.bfloat16: "bf16", torch.float16: "f16"}[prob.q.dtype]
    B, n, H, D = prob.shape
    result = {
        "metric": "Longformer input projections tokens/s (six C x C maps, C = H*64), bf16; MFMA util %",
        "value": run.M / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": dname,
        "data": "synthetic (seeded N(0,1) hidden states, N(0,1/C) weights, N(0,0.01) bias)",
        "config": {"workload": args.workload, "pass": "projections", "M": run.M, "C": run.C, "P": run.P,
                   "global_only": "Q_g at global tokens" if run.global_only else None,
                   "timing": mode, "wall_s": round(t_wall, 3)},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None,
                     "kernel": f"lf_proj_*_{dname}", "flops_per_launch": flops},
    }
    if not args.no_cpu_baseline:
        # the CPU-baseline leg: the fp64 oracle on the whole job, timed; its
        # result is also compared with the timed output
        from threadpoolctl import threadpool_info

        import oracle

        xs, ws, bs = run.x_cpu.float().numpy(), run.w_cpu.float().numpy(), run.b_cpu.numpy()
        reps, t0 = 0, time.perf_counter()
        while reps < 3 or time.perf_counter() - t0 < 2.0:
            ref = oracle.project(xs, ws, bs)
            reps += 1
        dt = (time.perf_counter() - t0) / reps
        threads = max([int(t.get("num_threads", 1)) for t in threadpool_info()] or [1])
        result["cpu_baseline"] = {"value": run.M / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
                                  "sample": f"the whole job ({run.M} tokens, six projections), fp64 NumPy "
                                            f"matmul on {threads} BLAS threads, mean of {reps} runs"}
        if not args.no_check:
            got = run.out.float().cpu().numpy()
            if run.global_only:
                ref[3][run.mask.cpu().numpy() != 2] = 0.0
            excess = float((np.abs(got - ref) - (2.0 ** -8 * np.abs(ref) + 1e-3)).max())
            result["parity"] = {"kind": "every row of all six projections vs the fp64 oracle run of the "
                                        "CPU-baseline leg", "max_abs_err": float(np.abs(got - ref).max()),
                                "ok": excess <= 0}
    print(json.dumps(result), flush=True)


def check_backward(prob, run):
    """Closed forms that hold at any size, on every head (no oracle): summed
    over tokens, dv equals the upstream gradient summed over local rows
    (dv_g: over global rows), and dk and dk_g sum to zero (relative to their
    column mass)."""
    import numpy as np

    dq, dk, dv, dqg, dkg, dvg = [g.double().cpu().numpy() for g in run.grads]
    m = prob.mask.numpy()
    do = run.dout.double().cpu().numpy()
    worst = 0.0
    B, n, H, D = prob.shape
    for b in range(B):
        for h in range(H):
            ref = do[b, m[b] == 1, h].sum(0)
            worst = max(worst, np.abs(dv[b, :, h].sum(0) - ref).max() / max(np.abs(ref).max(), 1e-3))
            mass = np.abs(dk[b, :, h]).sum(0).max()
            worst = max(worst, np.abs(dk[b, :, h].sum(0)).max() / max(mass, 1e-30))
            if (m[b] == 2).any():
                refg = do[b, m[b] == 2, h].sum(0)
                worst = max(worst, np.abs(dvg[b, :, h].sum(0) - refg).max() / max(np.abs(refg).max(), 1e-3))
                massg = np.abs(dkg[b, :, h]).sum(0).max()
                worst = max(worst, np.abs(dkg[b, :, h].sum(0)).max() / max(massg, 1e-30))
    return {"kind": "closed-form column sums of dv, dv_g, dk, dk_g, every (b, h)", "max_rel_err": float(worst),
            "tol": 2e-2, "ok": bool(worst <= 2e-2)}


def cpu_baseline_backward(prob, run=None):
    """The CPU-baseline leg of the backward: the fp64 gradient oracle on
    batch row 0 and heads 0 and H-1 at full length (NumPy BLAS on every core
    it finds), scaled to tokens/s of the whole job.  Its six gradients of
    those heads are compared, every element, with the timed run's (tolerance
    2e-2 of each gradient's largest entry, the test suite's bound)."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info
        threads = max([int(t.get("num_threads", 1)) for t in threadpool_info()] or [1])
    except ImportError:  # pragma: no cover
        threads = os.cpu_count() or 1
    t = [x.float().numpy() for x in (prob.q, prob.k, prob.v, prob.q_g, prob.k_g, prob.v_g)]
    dout = run.dout.float().cpu().numpy()
    B, n, H, D = prob.shape
    hs = sorted({0, H - 1})
    t0 = time.perf_counter()
    ref = oracle.backward(*[x[:1] for x in t], prob.mask.numpy()[:1], dout[:1], prob.window,
                          dilation=prob.dilation, causal=prob.causal, scale=prob.scale, heads=hs)
    dt = time.perf_counter() - t0
    out = {"value": B * n * len(hs) / (dt * H * B), "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"batch row 0, heads {hs} of {H}, all {n} tokens ({dt:.1f} s, NumPy BLAS on "
                     f"{threads} threads), scaled to B*H"}
    parity = None
    if run is not None:
        worst = 0.0
        for g, r in zip(run.grads, ref):
            gg = g[:1, :, hs].double().cpu().numpy()
            rr = r[:, :, hs]
            worst = max(worst, float(np.abs(gg - rr).max()) / max(float(np.abs(rr).max()), 1e-3))
        parity = {"kind": f"all six gradients of batch row 0, heads {hs}, every element, vs the oracle run "
                          "of the CPU-baseline leg", "max_rel_err": worst, "tol": 2e-2, "ok": worst <= 2e-2}
    return out, parity


def cpu_baseline(prob, out=None, row_nnz=None, min_s=10.0, max_s=30.0):
    """The CPU-baseline leg: the fp64 oracle as it stands, on a bounded
    sample of the same workload: whole (batch row, head) pairs, all rows
    each, taken in order and cyclically until at least min_s seconds of
    work and three pairs (stopping early at max_s); NumPy's BLAS on every
    host core it finds (its own default).  The time per pair is the median
    over the pairs run, scaled to tokens/s of the full job.  When the timed
    run's out and row_nnz are given, every row of the sampled pairs is
    compared with the oracle's (max |out - oracle| within the parity
    tolerance, row_nnz bit-exact).  Returns (baseline, parity)."""
    import numpy as np
    import torch

    import oracle

    try:
        from threadpoolctl import threadpool_info
        threads = max([int(t.get("num_threads", 1)) for t in threadpool_info()] or [1])
    except ImportError:  # pragma: no cover
        threads = os.cpu_count() or 1
    B, n, H, D = prob.shape
    arrs = [x.float().numpy() for x in (prob.q, prob.k, prob.v, prob.q_g, prob.k_g, prob.v_g)]
    mask = prob.mask.numpy()
    o = out.float().cpu().numpy() if out is not None else None
    c = row_nnz.cpu().numpy() if row_nnz is not None else None
    pairs = [(b, h) for b in range(B) for h in range(H)]
    # head 0 first, then spread over the job
    order = [pairs[(k * 7) % len(pairs)] for k in range(len(pairs))] if len(pairs) % 7 else pairs
    per, t0 = [], time.perf_counter()
    worst, nnz_ok, seen = 0.0, True, []
    while True:
        b, h = order[len(per) % len(order)]
        t1 = time.perf_counter()
        ref, rc = oracle.forward_rows(*arrs, mask, prob.window, b, h, range(n), dilation=prob.dilation,
                                      causal=prob.causal, scale=prob.scale)
        per.append(time.perf_counter() - t1)
        if o is not None and (b, h) not in seen:
            worst = max(worst, float(np.abs(o[b, :, h] - ref).max()))
            nnz_ok &= bool(np.array_equal(c[b, h], rc))
            seen.append((b, h))
        el = time.perf_counter() - t0
        if (el >= min_s and len(per) >= 3) or el + el / len(per) > max_s:
            break
    el = time.perf_counter() - t0
    med = float(np.median(per))
    full = med * len(pairs)  # seconds for the whole job at the sampled rate
    base = {"value": B * n / full, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(per)} (batch row, head) pairs of the {len(pairs)} in the job, all {n} query rows "
                      f"each, {el:.1f} s with NumPy BLAS on {threads} threads (os.cpu_count() = "
                      f"{os.cpu_count()}); value = tokens of the full job / ({len(pairs)} x median seconds "
                      "per pair)"}
    parity = None
    if o is not None:
        tol = {torch.bfloat16: 2e-2, torch.float16: 5e-3}.get(prob.q.dtype, 1e-4)
        parity = {"kind": f"every row of (batch row, head) pairs {seen} vs the oracle run of the CPU-baseline leg",
                  "max_abs_err": worst, "tolerance": tol, "row_nnz_exact": nnz_ok,
                  "ok": bool(worst <= tol and nnz_ok)}
    return base, parity


def time_graph(run, K, eager=False, bwd=False):
    """Time exactly K launches (graph replays of up to 50 launches, or eager
    launches), inputs resident in HBM.  Returns (ms per launch, mode, wall s)."""
    import torch

    mode, graph, per = "eager", None, 1
    if not eager:
        try:
            ref = (run.out_t if bwd else run.out).clone()
            per = max(d for d in range(1, min(K, 50) + 1) if K % d == 0)
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                run.args = run.args[:-1] + (ctypes.c_void_p(s.cuda_stream),)
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(graph, stream=s):
                    for _ in range(per):
                        run.launch()
            torch.cuda.current_stream().wait_stream(s)
            graph.replay()
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            if not torch.equal(ref, run.out_t if bwd else run.out):
                raise RuntimeError("graph replay output differs from the eager launch")
            mode = f"graph({per} launches per replay)"
        except Exception as e:  # fall back to eager timing
            print(f"graph capture unavailable ({e}); timing eager launches", file=sys.stderr)
            graph = None
        # later eager launches go to torch's current stream again
        run.args = run.args[:-1] + (ctypes.c_void_p(torch.cuda.current_stream().cuda_stream),)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record()
    if graph is not None:
        for _ in range(K // per):
            graph.replay()
    else:
        for _ in range(K):
            run.launch()
    end.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    return start.elapsed_time(end) / K, mode, t_wall


def time_cold(run, launches=30, scratch_mb=512):
    """Each launch timed alone (its own event pair on the launch stream)
    right after a 512 MB write that evicts the L2 caches and the 256 MB
    Infinity Cache: inputs come from HBM.  Median ms per launch."""
    import numpy as np
    import torch

    scratch = torch.empty(scratch_mb << 20, dtype=torch.uint8, device=run.out.device if hasattr(run, "out")
                          else run.out_t.device)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    ts = []
    for i in range(launches):
        scratch.fill_(i & 0xFF)
        e0.record()
        run.launch()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    del scratch
    return float(np.median(ts))


def sweep(args):
    """Linear growth in n (ultralytics glossary, "How Longformer attention
    works": the cost grows linearly with the sequence): the longformer-base
    layer shape (H12, w=256, token 0 global) at n = 1024 ... 16384, one JSON
    line per length, then the ratios t(n) / t(n/2)."""
    import torch

    import workloads

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    rows = []
    for n in workloads.SWEEP_N:
        prob = workloads.longformer_base_len(n)
        run = Runner(prob, dev)
        for _ in range(max(1, args.warmup)):
            run.launch()
        torch.cuda.synchronize()
        ms, mode, _ = time_graph(run, args.steps)
        flops = band_flops(prob)
        acct = pair_accounting(prob, run.row_nnz)
        row = {"workload": prob.name, "n": n, "ms_per_launch": ms, "tokens_per_s": n / (ms * 1e-3),
               "mfma_frac_band": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, "timing": mode,
               "pairs": acct["pairs"]}
        if rows:
            row["ratio_to_half_n"] = ms / rows[-1]["ms_per_launch"]
        rows.append(row)
        print(json.dumps(row), flush=True)
        del run
    print(json.dumps({"sweep": "longformer_base_len", "n": [r["n"] for r in rows],
                      "ms": [r["ms_per_launch"] for r in rows],
                      "ratios": [r.get("ratio_to_half_n") for r in rows[1:]]}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="longformer_base_n4096")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-check", action="store_true")
    ap.add_argument("--eager", action="store_true", help="time direct launches instead of a graph replay")
    ap.add_argument("--pass", dest="which", choices=["forward", "backward", "projections", "encoder"],
                    default="forward")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold-cache timing")
    ap.add_argument("--global-only", action="store_true",
                    help="with --pass projections: Q_g at the workload's global tokens only "
                         "(lf_attn_project_global_only)")
    ap.add_argument("--sweep", action="store_true",
                    help="time the longformer-base layer at n = 1024 ... 16384 instead (one line each)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the multi-GPU layout of this "
              "path is a design note, not a measured configuration", file=sys.stderr)
        sys.exit(2)

    import torch

    import sparse_long_document_amd as lf
    import workloads

    if args.sweep:
        return sweep(args)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    bwd = args.which != "forward"  # a runner with out_t, compared across graph replays
    prob = None if args.which == "encoder" else workloads.by_name(args.workload)
    if args.which == "projections":
        run = ProjRunner(prob, dev, global_only=args.global_only)
    else:
        run = {"forward": Runner, "backward": BwdRunner, "encoder": EncRunner}[args.which](prob, dev)
    for _ in range(max(1, args.warmup)):
        run.launch()
    torch.cuda.synchronize()

    K = args.steps
    ms, mode, t_wall = time_graph(run, K, eager=args.eager, bwd=bwd)

    if args.which == "encoder":
        return report_encoder(args, run, ms, mode, t_wall)
    B, n, H, D = prob.shape
    if args.which == "backward":
        return report_backward(args, prob, run, ms, mode, t_wall)
    if args.which == "projections":
        return report_projections(args, prob, run, ms, mode, t_wall)
    flops = band_flops(prob)
    achieved = flops / (ms * 1e-3) / 1e12
    # dense MFMA peak of the element type (f16 and bf16 share one)
    peak = PEAK_F32_TFLOPS if prob.q.dtype == torch.float32 else PEAK_BF16_TFLOPS
    dname = {torch.bfloat16: "bf16", torch.float16: "f16"}.get(prob.q.dtype, "f32")
    khash = lf.kernel_source_hash()
    traffic = None
    try:
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        ent = tr.get(args.workload)
        if ent and ent.get("kernel_hash") == khash:
            traffic = ent["bytes_per_launch"]
    except (OSError, ValueError):
        pass
    result = {
        "metric": "sliding-window attn fwd tokens/s, n=4096 H=12 w=256/side bf16; MFMA util %",
        "value": B * n / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dname,
        "data": "synthetic (seeded N(0,1) q/k/v/q_g/k_g/v_g, mask per workload recipe)",
        "config": {"workload": args.workload, "B": B, "n": n, "H": H, "D": D, "w": prob.window,
                   "causal": prob.causal, "dilation": prob.dilation,
                   "globals_per_row": [int(x) for x in (prob.mask == 2).sum(dim=1).tolist()],
                   "timing": mode, "wall_s": round(t_wall, 3)},
        "mfma_util_band": achieved / peak,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": traffic,
                     "kernel": f"lf_attn_fwd<{dname}>",
                     "flops_per_launch": flops, "algorithmic_bytes": algorithmic_bytes(prob),
                     "kernel_hash": khash},
        "hbm": {"algorithmic_GBs": algorithmic_bytes(prob) / (ms * 1e-3) / 1e9,
                "counted_GBs": None if traffic is None else traffic / (ms * 1e-3) / 1e9,
                "peak_GBs": PEAK_HBM_GBS,
                "counted_frac": None if traffic is None else traffic / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS},
    }
    result["pairs"] = pair_accounting(prob, run.row_nnz)
    result["flops_exact_frac"] = result["pairs"]["flops_exact"] / (ms * 1e-3) / 1e12 / peak
    if not args.no_cold:
        cold = time_cold(run)
        result["cold"] = {"ms_per_launch": cold, "tokens_per_s": B * n / (cold * 1e-3),
                          "mfma_frac_band": flops / (cold * 1e-3) / 1e12 / peak,
                          "algorithmic_GBs": algorithmic_bytes(prob) / (cold * 1e-3) / 1e9,
                          "method": "median of 30 launches, each after a 512 MB write "
                                    "(evicts L2 and Infinity Cache), one event pair per launch"}
    if not args.no_cpu_baseline:
        base, parity = cpu_baseline(prob, None if args.no_check else run.out,
                                    None if args.no_check else run.row_nnz)
        result["cpu_baseline"] = base
        if parity is not None:
            result["parity"] = parity
    print(json.dumps(result), flush=True)


def report_backward(args, prob, run, ms, mode, t_wall):
    import torch

    B, n, H, D = prob.shape
    flops = backward_flops(prob)
    achieved = flops / (ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS
    dname = {torch.bfloat16: "bf16", torch.float16: "f16"}[prob.q.dtype]
    traffic = None
    try:
        with open(TRAFFIC_FILE) as f:
            ent = json.load(f).get(f"{args.workload}:backward")
        import sparse_long_document_amd as lf

        if ent and ent.get("kernel_hash") == lf.backward_source_hash():
            traffic = ent["bytes_per_launch"]
    except (OSError, ValueError):
        pass
    result = {
        "metric": "sliding-window attn bwd tokens/s (all six input gradients), bf16; MFMA util %",
        "value": B * n / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dname,
        "data": "synthetic (seeded N(0,1) inputs and upstream gradient, mask per workload recipe)",
        "config": {"workload": args.workload, "pass": "backward", "B": B, "n": n, "H": H, "D": D,
                   "w": prob.window, "causal": prob.causal, "dilation": prob.dilation,
                   "globals_per_row": [int(x) for x in (prob.mask == 2).sum(dim=1).tolist()],
                   "timing": mode, "wall_s": round(t_wall, 3)},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": traffic,
                     "kernel": f"lf_attn_bwd<{dname}> (whole backward: preparation, band and global-token launches)",
                     "flops_per_launch": flops, "algorithmic_bytes": backward_bytes(prob)},
    }
    if not args.no_check:
        result["closed_forms"] = check_backward(prob, run)
    if not args.no_cpu_baseline:
        base, parity = cpu_baseline_backward(prob, None if args.no_check else run)
        result["cpu_baseline"] = base
        if parity is not None:
            result["parity"] = parity
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
