"""Benchmark: Longformer sliding-window + global attention forward on one MI355X.

One step = one lf_attn_forward over one batch of seeded synthetic inputs
already resident in HBM (the whole hot path: mask scan, band tiles, global
columns, split global rows and their merge; one kernel launch).

Default workload: the longformer-base layer shape, B=1, n=4096, H=12, D=64,
one-sided window 256, bf16, token 0 global.  Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--no-cpu-baseline] [--no-check] [--eager] [--pass backward]

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

    def __init__(self, prob, device):
        import torch

        import sparse_long_document_amd as lf
        import workloads

        B, n, H, D = prob.shape
        self.M, self.C, self.P = B * n, H * D, 6
        x, w, b = workloads.projection_problem(3, self.M, self.C, self.P, prob.q.dtype)
        self.x_cpu, self.w_cpu, self.b_cpu = x, w, b
        self.x, self.w, self.b = x.to(device), w.to(device), b.to(device)
        self.out = torch.empty((self.P, self.M, self.C), dtype=prob.q.dtype, device=device)
        self.out_t = self.out
        self.stream = torch.cuda.current_stream(device).cuda_stream
        vp = ctypes.c_void_p
        self.lib = lf.library()
        self.dt = lf._DTYPES[prob.q.dtype]
        self.args = (self.M, self.C, self.P, self.dt, vp(self.x.data_ptr()), vp(self.w.data_ptr()),
                     vp(self.b.data_ptr()), vp(self.out.data_ptr()), vp(self.stream))
        self.fn = self.lib.lf_attn_project

    def launch(self):
        st = self.fn(*self.args)
        if st != 0:
            raise RuntimeError(f"lf_attn_project failed with status {st}")


def report_projections(args, prob, run, ms, mode, t_wall):
    import numpy as np
    import torch

    import oracle

    flops = 2.0 * run.M * run.C * run.P * run.C
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
                   "timing": mode, "wall_s": round(t_wall, 3)},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None,
                     "kernel": f"lf_proj_{dname}", "flops_per_launch": flops},
    }
    if not args.no_check:
        rows = np.linspace(0, run.M - 1, 64).astype(np.int64)
        ref = oracle.project(run.x_cpu.float().numpy()[rows], run.w_cpu.float().numpy(), run.b_cpu.numpy())
        got = run.out[:, torch.from_numpy(rows).to(run.out.device)].float().cpu().numpy()
        excess = float((np.abs(got - ref) - (2.0 ** -8 * np.abs(ref) + 1e-3)).max())
        result["parity"] = {"kind": "64 sampled rows of all six projections vs the fp64 oracle",
                            "max_abs_err": float(np.abs(got - ref).max()), "ok": excess <= 0}
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_info

        xs, ws, bs = run.x_cpu.float().numpy(), run.w_cpu.float().numpy(), run.b_cpu.numpy()
        reps, t0 = 0, time.perf_counter()
        while reps < 3 or time.perf_counter() - t0 < 2.0:
            oracle.project(xs, ws, bs)
            reps += 1
        dt = (time.perf_counter() - t0) / reps
        threads = max([int(t.get("num_threads", 1)) for t in threadpool_info()] or [1])
        result["cpu_baseline"] = {"value": run.M / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
                                  "sample": f"the whole job ({run.M} tokens, six projections), fp64 NumPy "
                                            f"matmul on {threads} BLAS threads, mean of {reps} runs"}
    print(json.dumps(result), flush=True)


def check_backward(prob, run):
    """Closed forms that hold at any size, on every head: summed over
    tokens, dv equals the upstream gradient summed over local rows (dv_g:
    over global rows), and dk sums to zero (relative to its column mass)."""
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
            refg = do[b, m[b] == 2, h].sum(0)
            if (m[b] == 2).any():
                worst = max(worst, np.abs(dvg[b, :, h].sum(0) - refg).max() / max(np.abs(refg).max(), 1e-3))
            mass = np.abs(dk[b, :, h]).sum(0).max()
            worst = max(worst, np.abs(dk[b, :, h].sum(0)).max() / max(mass, 1e-30))
    return {"kind": "closed-form column sums, every (b, h)", "max_rel_err": float(worst),
            "tol": 2e-2, "ok": bool(worst <= 2e-2)}


def cpu_baseline_backward(prob):
    """The fp64 gradient oracle on one host thread, on one (b, h) of the
    workload at full length, scaled to tokens/s of the whole job."""
    import numpy as np
    import torch

    import oracle
    import workloads

    torch.set_num_threads(1)
    t = [x.float().numpy() for x in (prob.q, prob.k, prob.v, prob.q_g, prob.k_g, prob.v_g)]
    dout = workloads.upstream_grad(2, prob.shape, prob.q.dtype).float().numpy()
    B, n, H, D = prob.shape
    t0 = time.perf_counter()
    hs = list(range(min(H, 2)))
    oracle.backward(*[x[:1] for x in t], prob.mask.numpy()[:1], dout[:1], prob.window,
                    dilation=prob.dilation, causal=prob.causal, scale=prob.scale, heads=hs)
    dt = time.perf_counter() - t0
    return {"value": B * n * len(hs) / (dt * H * B), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"batch row 0, heads 0..{len(hs) - 1} of {H}, all {n} tokens ({dt:.1f} s), "
                      "scaled to B*H"}


def check_parity(prob, out, row_nnz, max_rows=48):
    """Sampled rows of the timed output against the fp64 oracle."""
    import numpy as np
    import torch

    import oracle

    B, n, H, D = prob.shape
    arrs = [x.float().numpy() for x in (prob.q, prob.k, prob.v, prob.q_g, prob.k_g, prob.v_g)]
    mask = prob.mask.numpy()
    o = out.float().cpu().numpy()
    c = row_nnz.cpu().numpy()
    rng = np.random.default_rng(1)
    worst, nnz_ok = 0.0, True
    for b in range(B):
        for h in sorted({0, H // 2, H - 1}):
            rows = sorted(set([0, 1, n - 1, n // 2] + [int(x) for x in rng.integers(0, n, size=max_rows)]
                              + [int(x) for x in np.flatnonzero(mask[b] == 2)[:8]]))
            ref, rc = oracle.forward_rows(*arrs, mask, prob.window, b, h, rows, dilation=prob.dilation,
                                          causal=prob.causal, scale=prob.scale)
            worst = max(worst, float(np.abs(o[b, rows, h] - ref).max()))
            nnz_ok &= bool(np.array_equal(c[b, h, rows], rc))
    tol = {torch.bfloat16: 2e-2, torch.float16: 5e-3}.get(prob.q.dtype, 1e-4)
    return {"max_abs_err_sampled": worst, "tolerance": tol, "row_nnz_exact": nnz_ok,
            "ok": bool(worst <= tol and nnz_ok)}


def cpu_baseline(prob, min_s=10.0, max_s=30.0):
    """The fp64 oracle as it stands, on a bounded sample of the same workload:
    whole (batch row, head) pairs, all rows each, taken in order and
    cyclically until at least min_s seconds of work (stopping early at
    max_s); single BLAS thread; scaled to tokens/s of the full job."""
    import oracle

    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    B, n, H, D = prob.shape
    arrs = [x.float().numpy() for x in (prob.q, prob.k, prob.v, prob.q_g, prob.k_g, prob.v_g)]
    mask = prob.mask.numpy()
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    pairs = [(b, h) for b in range(B) for h in range(H)]
    done, t0 = 0, time.perf_counter()
    try:
        if ctx:
            ctx.__enter__()
        while True:
            b, h = pairs[done % len(pairs)]
            oracle.forward_rows(*arrs, mask, prob.window, b, h, range(n), dilation=prob.dilation,
                                causal=prob.causal, scale=prob.scale)
            done += 1
            el = time.perf_counter() - t0
            if el >= min_s or el + el / done > max_s:
                break
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    el = time.perf_counter() - t0
    full = el / done * len(pairs)  # seconds for the whole job at the sampled rate
    return {"value": B * n / full, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} (batch row, head) pairs of the {len(pairs)} in the job (cycled in order), "
                      f"all {n} query rows each, {el:.1f} s on one thread; value = tokens of the full "
                      f"job / ({len(pairs)} x seconds per pair)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="longformer_base_n4096")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-check", action="store_true")
    ap.add_argument("--eager", action="store_true", help="time direct launches instead of a graph replay")
    ap.add_argument("--pass", dest="which", choices=["forward", "backward", "projections"], default="forward")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the multi-GPU layout of this "
              "path is a design note, not a measured configuration", file=sys.stderr)
        sys.exit(2)

    import torch

    import sparse_long_document_amd as lf
    import workloads

    prob = workloads.by_name(args.workload)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    bwd = args.which != "forward"  # a runner with out_t, compared across graph replays
    run = {"forward": Runner, "backward": BwdRunner, "projections": ProjRunner}[args.which](prob, dev)
    for _ in range(max(1, args.warmup)):
        run.launch()
    torch.cuda.synchronize()

    K = args.steps
    mode = "eager"
    graph = None
    if not args.eager:
        try:
            ref = (run.out_t if bwd else run.out).clone()
            per = max(d for d in range(1, min(K, 50) + 1) if K % d == 0)
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                run.stream = s.cuda_stream
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
            run.args = run.args[:-1] + (ctypes.c_void_p(torch.cuda.current_stream().cuda_stream),)

    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    if graph is not None:
        reps = K // per
        start.record()
        for _ in range(reps):
            graph.replay()
        end.record()
    else:
        start.record()
        for _ in range(K):
            run.launch()
        end.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = start.elapsed_time(end) / K

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
    if not args.no_check:
        result["parity"] = check_parity(prob, run.out, run.row_nnz)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(prob)
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
                     "kernel": f"lf_attn_bwd<{dname}> (whole backward: 2 launches)",
                     "flops_per_launch": flops, "algorithmic_bytes": backward_bytes(prob)},
    }
    if not args.no_check:
        result["parity"] = check_backward(prob, run)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_backward(prob)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
