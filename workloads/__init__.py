"""Seeded synthetic inputs for the Longformer combined attention forward.

This module only draws inputs.  It holds none of the attention arithmetic:
no windows, no scores, no softmax, no counting.  Both sides of every parity
check (the fp64 oracle under ``oracle/`` and the HIP library) receive the
tensors produced here, and nothing else is shared between them.

Recipe (the same for every workload):

* ``numpy.random.Generator(PCG64(seed))``;
* draw q, k, v, q_g, k_g, v_g in that order, each
  ``standard_normal([B, n, H, D], float32)``;
* cast to the workload dtype with round-to-nearest-even (torch ``.to``);
  the oracle consumes the cast values widened to fp64, so both sides see
  bit-identical inputs;
* then draw the mask structure (sequence lengths, global positions) from the
  same generator, after the tensors.

Mask values follow the Longformer attention-mask convention (allenai
longformer README, "Usage", run-the-model step): 0 = no attention,
1 = local (sliding window), 2 = global.

The named workloads are stand-ins for the attention inputs of the pages'
models: a longformer-base layer at 4096 tokens (ultralytics glossary,
"How Longformer attention works"; 256 tokens per side), question answering
with question tokens global and padded documents (allenai README, "Usage"),
the causal dilated character-level LM layer trained up to 23040 tokens
(segmentfault summary, "Training"), and the LED encoder at 16K tokens
(allenai README, LED news item).  No dataset is read.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np
import torch

D_HEAD = 64


@dataclasses.dataclass
class Problem:
    """One attention call's inputs (CPU tensors) and parameters."""

    name: str
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    q_g: torch.Tensor
    k_g: torch.Tensor
    v_g: torch.Tensor
    mask: torch.Tensor  # int8 [B, n] with values in {0, 1, 2}
    window: int  # one-sided
    dilation: Optional[List[int]]  # per head, None = all 1
    causal: bool
    scale: Optional[float]  # None = 1/sqrt(D)
    aliased_global: bool = False  # q_g/k_g/v_g are the same tensors as q/k/v

    @property
    def shape(self):
        return tuple(self.q.shape)

    def max_global(self) -> int:
        return int((self.mask == 2).sum(dim=1).max().item()) if self.mask.numel() else 0

    def describe(self) -> dict:
        B, n, H, D = self.shape
        return {
            "workload": self.name,
            "B": B,
            "n": n,
            "H": H,
            "D": D,
            "w": self.window,
            "dilation": self.dilation,
            "causal": self.causal,
            "dtype": str(self.q.dtype).replace("torch.", ""),
            "globals_per_row": [int(x) for x in (self.mask == 2).sum(dim=1).tolist()],
        }


def _draw(rng: np.random.Generator, shape, dtype: torch.dtype) -> torch.Tensor:
    a = rng.standard_normal(shape, dtype=np.float32)
    return torch.from_numpy(a).to(dtype)


def upstream_grad(seed: int, shape, dtype: torch.dtype) -> torch.Tensor:
    """A seeded upstream gradient of the output, standard normal in ``dtype``
    (its own stream: seed + 1000)."""
    return _draw(np.random.Generator(np.random.PCG64(seed + 1000)), shape, dtype)


def projection_problem(seed: int, M: int, C: int, P: int, dtype: torch.dtype = torch.bfloat16):
    """Hidden states x [M, C] ~ N(0, 1), stacked weights w [P*C, C] ~
    N(0, 1/C) (outputs of unit scale) and an fp32 bias ~ N(0, 0.1^2), all in
    ``dtype`` except the bias."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = _draw(rng, (M, C), dtype)
    w = torch.from_numpy((rng.standard_normal((P * C, C), dtype=np.float32) / np.float32(np.sqrt(C)))).to(dtype)
    bias = torch.from_numpy(rng.standard_normal(P * C, dtype=np.float32) * np.float32(0.1))
    return x, w, bias


def random_problem(
    seed: int,
    B: int,
    n: int,
    H: int,
    window: int,
    dtype: torch.dtype = torch.bfloat16,
    dilation: Optional[List[int]] = None,
    causal: bool = False,
    n_global: int = 0,
    pad_tail: int = 0,
    zero_frac: float = 0.0,
    global_positions: Optional[List[int]] = None,
    aliased_global: bool = False,
    scale: Optional[float] = None,
    D: int = D_HEAD,
    name: str = "random",
) -> Problem:
    """Draw a problem.

    ``n_global`` distinct positions per batch row get mask 2 (or the fixed
    ``global_positions``); the last ``pad_tail`` positions of each row get
    mask 0; ``zero_frac`` scatters additional mask-0 positions.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    shape = (B, n, H, D)
    q = _draw(rng, shape, dtype)
    k = _draw(rng, shape, dtype)
    v = _draw(rng, shape, dtype)
    if aliased_global:
        q_g, k_g, v_g = q, k, v
    else:
        q_g = _draw(rng, shape, dtype)
        k_g = _draw(rng, shape, dtype)
        v_g = _draw(rng, shape, dtype)
    mask = np.ones((B, n), dtype=np.int8)
    for b in range(B):
        if zero_frac > 0:
            z = rng.random(n) < zero_frac
            mask[b, z] = 0
        if pad_tail > 0:
            mask[b, n - pad_tail:] = 0
        if global_positions is not None:
            mask[b, list(global_positions)] = 2
        elif n_global > 0:
            cand = np.flatnonzero(mask[b] != 0)
            if len(cand) > 0:
                pick = rng.choice(cand, size=min(n_global, len(cand)), replace=False)
                mask[b, pick] = 2
    return Problem(
        name=name,
        q=q, k=k, v=v, q_g=q_g, k_g=k_g, v_g=v_g,
        mask=torch.from_numpy(mask),
        window=window,
        dilation=list(dilation) if dilation is not None else None,
        causal=causal,
        scale=scale,
        aliased_global=aliased_global,
    )


# ---------------------------------------------------------------------------
# The five named workloads.  Seed = workload index (1..5).
# ---------------------------------------------------------------------------

WORKLOADS = ("single_head_fp32_n512", "longformer_base_n4096",
             "qa_padded_b2_n4096", "charlm_causal_dilated_n23040",
             "led_large_n16384")


def single_head_fp32_n512() -> Problem:
    """B1 n512 H1 D64, one-sided window 64, fp32, mask all 1, no globals."""
    rng = np.random.Generator(np.random.PCG64(1))
    shape = (1, 512, 1, D_HEAD)
    q = _draw(rng, shape, torch.float32)
    k = _draw(rng, shape, torch.float32)
    v = _draw(rng, shape, torch.float32)
    mask = torch.ones((1, 512), dtype=torch.int8)
    return Problem("single_head_fp32_n512", q, k, v, q, k, v, mask, 64, None,
                   False, 1.0 / 8.0, aliased_global=True)


def longformer_base_n4096() -> Problem:
    """B1 n4096 H12 D64, w=256 per side, bf16, token 0 global, rest local."""
    rng = np.random.Generator(np.random.PCG64(2))
    shape = (1, 4096, 12, D_HEAD)
    t = [_draw(rng, shape, torch.bfloat16) for _ in range(6)]
    mask = torch.ones((1, 4096), dtype=torch.int8)
    mask[0, 0] = 2
    return Problem("longformer_base_n4096", *t, mask, 256, None, False, None)


def qa_padded_b2_n4096() -> Problem:
    """B2 n4096 H12 D64, w=256, bf16; first 64 tokens global; lengths
    U[2500, 4096] with a mask-0 tail (n is already a multiple of 2w=512)."""
    rng = np.random.Generator(np.random.PCG64(3))
    shape = (2, 4096, 12, D_HEAD)
    t = [_draw(rng, shape, torch.bfloat16) for _ in range(6)]
    lengths = rng.integers(2500, 4096, size=2, endpoint=True)
    mask = torch.zeros((2, 4096), dtype=torch.int8)
    for b in range(2):
        L = int(lengths[b])
        mask[b, :L] = 1
        mask[b, :64] = 2
    return Problem("qa_padded_b2_n4096", *t, mask, 256, None, False, None)


def charlm_causal_dilated_n23040() -> Problem:
    """B1 n23040 H8 D64, causal w=512, dilation 1 on heads 0-5 and 2 on
    heads 6-7, bf16, no globals."""
    rng = np.random.Generator(np.random.PCG64(4))
    shape = (1, 23040, 8, D_HEAD)
    t = [_draw(rng, shape, torch.bfloat16) for _ in range(6)]
    mask = torch.ones((1, 23040), dtype=torch.int8)
    return Problem("charlm_causal_dilated_n23040", *t, mask, 512,
                   [1, 1, 1, 1, 1, 1, 2, 2], True, None)


def charlm_causal_dilated_n32256() -> Problem:
    """The char-LM layer at its evaluation length: B1 n32256 H8 D64, causal
    w=512, dilation 1 on heads 0-5 and 2 on heads 6-7, bf16, no globals."""
    rng = np.random.Generator(np.random.PCG64(6))
    shape = (1, 32256, 8, D_HEAD)
    t = [_draw(rng, shape, torch.bfloat16) for _ in range(6)]
    mask = torch.ones((1, 32256), dtype=torch.int8)
    return Problem("charlm_causal_dilated_n32256", *t, mask, 512,
                   [1, 1, 1, 1, 1, 1, 2, 2], True, None)


def led_large_n16384() -> Problem:
    """B1 n16384 H16 D64, w=512, bf16; global at 0 plus 16 distinct random
    positions in 1..n-1."""
    rng = np.random.Generator(np.random.PCG64(5))
    shape = (1, 16384, 16, D_HEAD)
    t = [_draw(rng, shape, torch.bfloat16) for _ in range(6)]
    g = rng.choice(np.arange(1, 16384), size=16, replace=False)
    mask = torch.ones((1, 16384), dtype=torch.int8)
    mask[0, 0] = 2
    mask[0, torch.from_numpy(g.astype(np.int64))] = 2
    return Problem("led_large_n16384", *t, mask, 512, None, False, None)


def longformer_base_n4096_f16() -> Problem:
    """The longformer_base_n4096 problem with its six tensors cast to f16
    (round to nearest even).  Most of its bf16 values are exact in f16; the
    few below f16's normal range (|x| < 2^-14, about a hundred of the 18.9
    million) become subnormals and lose low bits.  Both sides of a parity
    check take the f16 tensors, so that changes nothing there."""
    p = longformer_base_n4096()
    for name in ("q", "k", "v", "q_g", "k_g", "v_g"):
        setattr(p, name, getattr(p, name).to(torch.float16))
    p.name = "longformer_base_n4096_f16"
    return p


@dataclasses.dataclass
class EncoderProblem:
    """Inputs of one encoder attention sublayer: hidden states, the six
    stacked input projections (Q_s, K_s, V_s, Q_g, K_g, V_g) with their
    bias, the output projection with its bias, and the 0/1/2 mask."""

    name: str
    x: torch.Tensor       # [B, n, C]
    w: torch.Tensor       # [6C, C]
    bias: torch.Tensor    # fp32 [6C]
    w_out: torch.Tensor   # [C, C]
    b_out: torch.Tensor   # fp32 [C]
    mask: torch.Tensor    # int8 [B, n]
    H: int
    window: int

    @property
    def shape(self):
        return tuple(self.x.shape)

    def max_global(self) -> int:
        return int((self.mask == 2).sum(dim=1).max().item())


def encoder_problem(seed: int, B: int, n: int, H: int, window: int, n_global: int = 0,
                    dtype: torch.dtype = torch.bfloat16, name: str = "encoder",
                    copied_global: bool = False) -> EncoderProblem:
    """Hidden states x ~ N(0, 1) [B, n, C] (C = 64 H), stacked projection
    weights ~ N(0, 1/C) [6C, C] with an fp32 bias ~ N(0, 0.1^2), an output
    projection of the same kind, global tokens at position 0 and n_global - 1
    further distinct random positions per batch row.  copied_global: the
    global projections start as copies of the local ones (weights and bias),
    their initial state on the pages (segmentfault Longformer summary,
    "Linear projections for global attention")."""
    rng = np.random.Generator(np.random.PCG64(seed))
    C = H * D_HEAD
    x = _draw(rng, (B, n, C), dtype)
    w = rng.standard_normal((6 * C, C), dtype=np.float32) / np.float32(np.sqrt(C))
    bias = rng.standard_normal(6 * C, dtype=np.float32) * np.float32(0.1)
    if copied_global:
        w[3 * C:] = w[:3 * C]
        bias[3 * C:] = bias[:3 * C]
    w_out = rng.standard_normal((C, C), dtype=np.float32) / np.float32(np.sqrt(C))
    b_out = rng.standard_normal(C, dtype=np.float32) * np.float32(0.1)
    mask = torch.ones((B, n), dtype=torch.int8)
    for b in range(B):
        if n_global > 0:
            mask[b, 0] = 2
            if n_global > 1:
                g = rng.choice(np.arange(1, n), size=n_global - 1, replace=False)
                mask[b, torch.from_numpy(g.astype(np.int64))] = 2
    return EncoderProblem(name, x, torch.from_numpy(w).to(dtype), torch.from_numpy(bias),
                          torch.from_numpy(w_out).to(dtype), torch.from_numpy(b_out), mask, H, window)


def led_encoder_n16384() -> EncoderProblem:
    """The LED-large encoder attention sublayer at 16K tokens: B1 n16384 H16
    (C = 1024), w = 512 per side, bf16, token 0 plus 16 random positions
    global (the LED workload's mask recipe).  Seed 7."""
    return encoder_problem(7, 1, 16384, 16, 512, n_global=17, name="led_encoder_n16384")


SWEEP_N = (1024, 2048, 4096, 8192, 16384)


def longformer_base_len(n: int) -> Problem:
    """The longformer-base layer shape at sequence length n (B1 H12 D64,
    w=256 per side, bf16, token 0 global): the inputs of the linear-growth
    sweep.  Seed 1000 + n."""
    rng = np.random.Generator(np.random.PCG64(1000 + n))
    shape = (1, n, 12, D_HEAD)
    t = [_draw(rng, shape, torch.bfloat16) for _ in range(6)]
    mask = torch.ones((1, n), dtype=torch.int8)
    mask[0, 0] = 2
    return Problem(f"longformer_base_len{n}", *t, mask, 256, None, False, None)


HEAD_DIMS = (32, 64, 128)


def longformer_base_n4096_dim(D: int) -> Problem:
    """The longformer-base layer shape (B1 n4096 H12, w=256 per side, bf16,
    token 0 global) with head dim D in place of 64: the head-dim variants.
    Seed 2000 + D."""
    if D == D_HEAD:
        return longformer_base_n4096()
    rng = np.random.Generator(np.random.PCG64(2000 + D))
    shape = (1, 4096, 12, D)
    t = [_draw(rng, shape, torch.bfloat16) for _ in range(6)]
    mask = torch.ones((1, 4096), dtype=torch.int8)
    mask[0, 0] = 2
    return Problem(f"longformer_base_n4096_d{D}", *t, mask, 256, None, False, None)


def by_name(name: str) -> Problem:
    if name.startswith("longformer_base_len"):
        return longformer_base_len(int(name[len("longformer_base_len"):]))
    if name.startswith("longformer_base_n4096_d"):
        return longformer_base_n4096_dim(int(name[len("longformer_base_n4096_d"):]))
    return {
        "single_head_fp32_n512": single_head_fp32_n512,
        "longformer_base_n4096": longformer_base_n4096,
        "longformer_base_n4096_f16": longformer_base_n4096_f16,
        "qa_padded_b2_n4096": qa_padded_b2_n4096,
        "charlm_causal_dilated_n23040": charlm_causal_dilated_n23040,
        "charlm_causal_dilated_n32256": charlm_causal_dilated_n32256,
        "led_large_n16384": led_large_n16384,
    }[name]()


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a bf16/f16/fp32 CPU tensor to a float64 array."""
    return t.detach().to("cpu").to(torch.float64).numpy()
