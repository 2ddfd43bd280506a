"""Longformer combined sliding-window + global attention forward on MI355X.

Thin Python binding over the C ABI of ``include/lf_attn.h`` (library
``liblf_attn.so`` built in-tree by ``sparse_long_document_amd.build``).  It
only marshals arguments: every step of the attention runs in the HIP
kernels.  PyTorch provides device memory and streams.  There is no CPU
fallback: without the built library, or without a GPU, ``forward`` raises.

Entry points (same names as the C ABI where they wrap it):
  * ``forward`` -> ``lf_attn_forward``
  * ``workspace_bytes`` -> ``lf_attn_workspace_bytes``
  * ``device_status`` -> ``lf_attn_device_status``
  * ``pad_to_window_size`` and ``merge_masks``: input helpers for the mask
    conventions of the allenai README ("Usage": pad the sequence to a
    multiple of the attention window; mask 0/1/2) and of the Hugging Face
    ``global_attention_mask`` (ultralytics glossary, "Training and results").
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Sequence

import torch

__all__ = [
    "forward", "backward", "project", "encoder_attention", "workspace_bytes", "make_workspace", "device_status",
    "pad_to_window_size", "merge_masks", "library", "LfError", "LF_MAX_GLOBAL", "LF_MAX_HEADS",
]

# The built library; LF_ATTN_LIBRARY names another build of the same C ABI
# (the test suite's sanitizer build of the host code uses it).
LIB_PATH = os.environ.get("LF_ATTN_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                             "liblf_attn.so")
KERNEL_SOURCES = ("csrc/lf_attn_kernels.hip", "csrc/lf_attn_kernels_f16.hip", "csrc/lf_attn_internal.h")


BACKWARD_SOURCES = ("csrc/lf_attn_bwd.hip", "csrc/lf_attn_bwd_f16.hip", "csrc/lf_attn_internal.h",
                    "csrc/lf_attn_bwd_internal.h")


def kernel_source_hash(sources=KERNEL_SOURCES) -> str:
    """Short digest of the device-code sources (by default the forward's);
    counter measurements are tagged with it so that a later kernel change
    invalidates them."""
    import hashlib

    h = hashlib.sha256()
    base = os.path.dirname(os.path.abspath(__file__))
    for rel in sources:
        with open(os.path.join(base, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def backward_source_hash() -> str:
    """Digest of the backward kernels' sources."""
    return kernel_source_hash(BACKWARD_SOURCES)

LF_OK, LF_ERR_INVALID_ARG, LF_ERR_UNSUPPORTED, LF_ERR_WORKSPACE, LF_ERR_HIP = range(5)
LF_F32, LF_BF16, LF_F16 = 0, 1, 2
_DTYPES = {torch.float32: LF_F32, torch.bfloat16: LF_BF16, torch.float16: LF_F16}
LF_HEAD_DIM = 64
LF_MAX_HEADS = 64
LF_MAX_GLOBAL = 1024
LF_DEV_TOO_MANY_GLOBALS = 1
LF_MAX_PROJ = 6

SYMBOLS = ("lf_attn_workspace_bytes", "lf_attn_workspace_init", "lf_attn_forward",
           "lf_attn_forward_lse", "lf_attn_backward_workspace_bytes", "lf_attn_backward",
           "lf_attn_project", "lf_attn_project_global_only", "lf_attn_forward_noalloc",
           "lf_attn_device_status", "lf_status_str")
LF_NOALLOC_SCRATCH_BYTES = 8 << 20


class LfError(RuntimeError):
    """A non-OK status from the C ABI."""

    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {status_str(code)} (status {code})")


class Params(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("n", ctypes.c_int32), ("H", ctypes.c_int32),
        ("D", ctypes.c_int32), ("window", ctypes.c_int32),
        ("dilation", ctypes.POINTER(ctypes.c_int32)), ("causal", ctypes.c_int32),
        ("scale", ctypes.c_float), ("max_global", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
    ]


_lib = None
_lib_lock = threading.Lock()


def library() -> ctypes.CDLL:
    """Load ``liblf_attn.so``; raise if it has not been built."""
    global _lib
    with _lib_lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with "
                    "`python -m sparse_long_document_amd.build`")
            lib = ctypes.CDLL(LIB_PATH)
            vp, sz = ctypes.c_void_p, ctypes.c_size_t
            lib.lf_attn_workspace_bytes.argtypes = [ctypes.POINTER(Params)]
            lib.lf_attn_workspace_bytes.restype = sz
            lib.lf_attn_workspace_init.argtypes = [vp, sz, vp]
            lib.lf_attn_workspace_init.restype = ctypes.c_int
            lib.lf_attn_forward.argtypes = [ctypes.POINTER(Params), vp, vp, vp, vp, vp, vp,
                                            vp, vp, vp, vp, sz, vp]
            lib.lf_attn_forward.restype = ctypes.c_int
            lib.lf_attn_forward_lse.argtypes = [ctypes.POINTER(Params), vp, vp, vp, vp, vp, vp,
                                                vp, vp, vp, vp, vp, sz, vp]
            lib.lf_attn_forward_lse.restype = ctypes.c_int
            lib.lf_attn_backward_workspace_bytes.argtypes = [ctypes.POINTER(Params)]
            lib.lf_attn_backward_workspace_bytes.restype = sz
            lib.lf_attn_backward.argtypes = [ctypes.POINTER(Params)] + [vp] * 16 + [vp, sz, vp]
            lib.lf_attn_backward.restype = ctypes.c_int
            i32 = ctypes.c_int32
            lib.lf_attn_project.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp]
            lib.lf_attn_project.restype = ctypes.c_int
            lib.lf_attn_project_global_only.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, ctypes.c_uint32, vp, vp]
            lib.lf_attn_project_global_only.restype = ctypes.c_int
            lib.lf_attn_forward_noalloc.argtypes = [ctypes.POINTER(Params), vp, vp, vp, vp, vp, vp,
                                                    vp, vp, vp, vp]
            lib.lf_attn_forward_noalloc.restype = ctypes.c_int
            lib.lf_attn_device_status.argtypes = [vp, vp, ctypes.POINTER(ctypes.c_int32)]
            lib.lf_attn_device_status.restype = ctypes.c_int
            lib.lf_status_str.argtypes = [ctypes.c_int32]
            lib.lf_status_str.restype = ctypes.c_char_p
            _lib = lib
    return _lib


def status_str(code: int) -> str:
    return library().lf_status_str(int(code)).decode()


def make_params(B: int, n: int, H: int, D: int, window: int,
                dilation: Optional[Sequence[int]], causal: bool, scale: Optional[float],
                max_global: int, dtype: torch.dtype):
    """Build the C parameter block.  Returns (params, keepalive)."""
    dil = None
    if dilation is not None:
        dil = (ctypes.c_int32 * len(dilation))(*[int(x) for x in dilation])
    p = Params(
        B=B, n=n, H=H, D=D, window=int(window),
        dilation=ctypes.cast(dil, ctypes.POINTER(ctypes.c_int32)) if dil is not None else None,
        causal=int(bool(causal)), scale=0.0 if scale is None else float(scale),
        max_global=int(max_global),
        dtype=_DTYPES.get(dtype, 99),
    )
    return p, dil


def workspace_bytes(B: int, n: int, H: int, window: int, dilation=None, causal=False,
                    scale=None, max_global: int = 0, dtype=torch.bfloat16, D: int = LF_HEAD_DIM) -> int:
    p, _keep = make_params(B, n, H, D, window, dilation, causal, scale, max_global, dtype)
    return int(library().lf_attn_workspace_bytes(ctypes.byref(p)))


_ws_cache = {}
_bwd_ws = {}
_ws_lock = threading.Lock()


def _capturing() -> bool:
    try:
        return bool(torch.cuda.is_current_stream_capturing())
    except Exception:  # pragma: no cover - older torch
        return False


_CAPTURE_MSG = ("{what} would allocate and clear a workspace inside a HIP graph capture (the clear "
                "would be recorded into the graph and the buffer would come from the graph's memory "
                "pool): create one beforehand with make_workspace(...) and pass it as workspace=")


def _workspace(nbytes: int, device: torch.device, stream: int, layout) -> torch.Tensor:
    """A zero-initialised workspace of at least nbytes, cached per
    (device, stream): calls on one stream are ordered, so they may share it.
    Each call leaves its arrival counters at zero, but where they sit depends
    on (B, H), so a change of layout re-initialises the buffer.  Under graph
    capture nothing is allocated or cleared: the cached buffer must already
    fit, else this raises."""
    key = (device.index, stream)
    with _ws_lock:
        ws, last = _ws_cache.get(key, (None, None))
        if ws is None or ws.numel() < nbytes or last != layout:
            if _capturing():
                raise RuntimeError(_CAPTURE_MSG.format(what="forward"))
            if ws is None or ws.numel() < nbytes:
                ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
            st = library().lf_attn_workspace_init(ctypes.c_void_p(ws.data_ptr()),
                                                  ctypes.c_size_t(ws.numel()),
                                                  ctypes.c_void_p(stream))
            if st != LF_OK:
                raise LfError(st, "lf_attn_workspace_init")
            _ws_cache[key] = (ws, layout)
        return ws


def make_workspace(B: int, n: int, H: int, window: int, dilation=None, causal=False, scale=None,
                   max_global: int = 0, dtype=torch.bfloat16, device=None, backward: bool = False,
                   D: int = LF_HEAD_DIM) -> torch.Tensor:
    """Allocate a workspace for ``forward`` (or, with backward=True, for
    ``backward``) on the current stream and zero it (``lf_attn_workspace_init``),
    outside any graph capture.  Pass it as ``workspace=`` to calls with the
    same B and H, for instance inside ``torch.cuda.graph``: each forward call
    leaves its arrival counters back at zero, so replays may reuse it."""
    if _capturing():
        raise RuntimeError("make_workspace must be called outside a graph capture")
    device = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    p, _keep = make_params(B, n, H, D, window, dilation, causal, scale, max_global, dtype)
    lib = library()
    need = int((lib.lf_attn_backward_workspace_bytes if backward else lib.lf_attn_workspace_bytes)(
        ctypes.byref(p)))
    if need == 0:
        raise LfError(LF_ERR_INVALID_ARG, "workspace size")
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    stream = torch.cuda.current_stream(device).cuda_stream
    st = lib.lf_attn_workspace_init(ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(ws.numel()),
                                    ctypes.c_void_p(stream))
    if st != LF_OK:
        raise LfError(st, "lf_attn_workspace_init")
    return ws


def _given_workspace(ws: torch.Tensor, need: int, device: torch.device) -> torch.Tensor:
    if not isinstance(ws, torch.Tensor) or ws.dtype != torch.uint8 or ws.device != device:
        raise ValueError("workspace must be a uint8 tensor on the inputs' device (see make_workspace)")
    if not ws.is_contiguous() or ws.numel() < need:
        raise ValueError(f"workspace holds {ws.numel()} bytes, {need} needed")
    return ws


def _check_tensor(name, t, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (this library has no CPU path)")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
            q_g: Optional[torch.Tensor] = None, k_g: Optional[torch.Tensor] = None,
            v_g: Optional[torch.Tensor] = None, mask: Optional[torch.Tensor] = None,
            window: int = 256, dilation: Optional[Sequence[int]] = None,
            causal: bool = False, scale: Optional[float] = None,
            max_global: Optional[int] = None, return_row_nnz: bool = False,
            validate: bool = True, out: Optional[torch.Tensor] = None,
            row_nnz: Optional[torch.Tensor] = None, return_lse: bool = False,
            lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Longformer attention forward (``lf_attn_forward``).

    q, k, v, q_g, k_g, v_g: [B, n, H, 64] bf16, f16 or fp32 GPU tensors, contiguous
    (q_g/k_g/v_g default to q/k/v).  mask: [B, n] int8 (other integer dtypes
    are converted) with 0 = no attention, 1 = local, 2 = global; None means
    all local.  window: one-sided w.  dilation: per-head stride.  Returns
    out, then row_nnz int32 [B, H, n] and lse fp32 [B, H, n] if asked
    (``lf_attn_forward_lse``: each row's natural log-sum-exp, what
    ``backward`` takes).

    validate=True checks mask contents on the host (one device sync) and
    derives max_global from the mask; validate=False trusts the caller
    (max_global then defaults to the library limit unless given).
    workspace: a buffer from ``make_workspace`` (needed under graph capture);
    by default one is cached per (device, stream).
    """
    if q.dim() != 4:
        raise ValueError("q must be [B, n, H, D]")
    B, n, H, D = q.shape
    device = q.device
    if device.type != "cuda":
        raise ValueError("q must be a GPU tensor (this library has no CPU path)")
    dtype = q.dtype
    q_g = q if q_g is None else q_g
    k_g = k if k_g is None else k_g
    v_g = v if v_g is None else v_g
    for name, t in (("q", q), ("k", k), ("v", v), ("q_g", q_g), ("k_g", k_g), ("v_g", v_g)):
        _check_tensor(name, t, (B, n, H, D), dtype, device)
    mask, max_global = _prep_mask(mask, B, n, device, causal, max_global, validate)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_tensor("out", out, (B, n, H, D), dtype, device)
    if return_row_nnz and row_nnz is None:
        row_nnz = torch.empty((B, H, n), dtype=torch.int32, device=device)
    if row_nnz is not None:
        _check_tensor("row_nnz", row_nnz, (B, H, n), torch.int32, device)
    if return_lse and lse is None:
        lse = torch.empty((B, H, n), dtype=torch.float32, device=device)
    if lse is not None:
        _check_tensor("lse", lse, (B, H, n), torch.float32, device)

    p, _keep = make_params(B, n, H, D, window, dilation, causal, scale, max_global, dtype)
    lib = library()
    need = int(lib.lf_attn_workspace_bytes(ctypes.byref(p)))
    if need == 0:
        raise LfError(LF_ERR_INVALID_ARG, "lf_attn_workspace_bytes")
    stream = torch.cuda.current_stream(device).cuda_stream
    if workspace is not None:
        ws = _given_workspace(workspace, need, device)
    else:
        ws = _workspace(need, device, stream, (B, H))
    vp = ctypes.c_void_p
    args = [ctypes.byref(p), vp(q.data_ptr()), vp(k.data_ptr()), vp(v.data_ptr()),
            vp(q_g.data_ptr()), vp(k_g.data_ptr()), vp(v_g.data_ptr()), vp(mask.data_ptr()),
            vp(out.data_ptr()), vp(row_nnz.data_ptr() if row_nnz is not None else None)]
    tail = [vp(ws.data_ptr()), ctypes.c_size_t(ws.numel()), vp(stream)]
    if lse is not None:
        st = lib.lf_attn_forward_lse(*args, vp(lse.data_ptr()), *tail)
        if st != LF_OK:
            raise LfError(st, "lf_attn_forward_lse")
    else:
        st = lib.lf_attn_forward(*args, *tail)
        if st != LF_OK:
            raise LfError(st, "lf_attn_forward")
    res = (out,) + ((row_nnz,) if return_row_nnz else ()) + ((lse,) if return_lse else ())
    return res if len(res) > 1 else out


def project(x: torch.Tensor, w: torch.Tensor, bias: Optional[torch.Tensor] = None,
            out: Optional[torch.Tensor] = None, mask: Optional[torch.Tensor] = None,
            global_only: Sequence[int] = ()) -> torch.Tensor:
    """The layer's input projections (``lf_attn_project``): x [M, C] (or
    [B, n, C]) bf16/f16, w [P*C, C] stacked weights in the [out, in] layout,
    bias fp32 [P*C] or None.  Returns out [P, M, C] (or [P, B, n, C]);
    out[p].view(B, n, H, 64) is one attention input.  The four buffers must
    start on 16-byte boundaries (freshly allocated tensors do; an offset
    view may not), else the call raises with LF_ERR_UNSUPPORTED.

    With ``global_only`` (projection indices) and ``mask`` (the attention's
    [B, n] mask, or [M]), those projections are computed at the tokens with
    mask 2 only and are zero elsewhere (``lf_attn_project_global_only``);
    with the weights stacked Q_s, K_s, V_s, Q_g, K_g, V_g, global_only=(3,)
    leaves the attention's inputs unchanged where it reads them."""
    shape = x.shape
    if x.dim() == 3:
        x = x.reshape(-1, shape[-1])
    if x.dim() != 2:
        raise ValueError("x must be [M, C] or [B, n, C]")
    M, C = x.shape
    if x.device.type != "cuda":
        raise ValueError("x must be a GPU tensor (this library has no CPU path)")
    if w.dim() != 2 or w.shape[1] != C or w.shape[0] % C != 0:
        raise ValueError("w must be [P*C, C]")
    P = w.shape[0] // C
    _check_tensor("x", x, (M, C), x.dtype, x.device)
    _check_tensor("w", w, (P * C, C), x.dtype, x.device)
    if bias is not None:
        _check_tensor("bias", bias, (P * C,), torch.float32, x.device)
    if out is None:
        out = torch.empty((P, M, C), dtype=x.dtype, device=x.device)
    _check_tensor("out", out, (P, M, C), x.dtype, x.device)
    vp = ctypes.c_void_p
    stream = torch.cuda.current_stream(x.device).cuda_stream
    bits = 0
    for q in global_only:
        if not 0 <= int(q) < P:
            raise ValueError(f"global_only index {q} outside 0..{P - 1}")
        bits |= 1 << int(q)
    if bits:
        if mask is None:
            raise ValueError("global_only needs the mask")
        m8 = mask.reshape(-1)
        if m8.numel() != M:
            raise ValueError("mask must hold one value per token")
        m8 = m8.to(device=x.device, dtype=torch.int8).contiguous()
        st = library().lf_attn_project_global_only(
            M, C, P, _DTYPES.get(x.dtype, 99), vp(x.data_ptr()), vp(w.data_ptr()),
            vp(bias.data_ptr() if bias is not None else None), vp(m8.data_ptr()), ctypes.c_uint32(bits),
            vp(out.data_ptr()), vp(stream))
        if st != LF_OK:
            raise LfError(st, "lf_attn_project_global_only")
        return out.view((P,) + tuple(shape[:-1]) + (C,))
    st = library().lf_attn_project(M, C, P, _DTYPES.get(x.dtype, 99), vp(x.data_ptr()), vp(w.data_ptr()),
                                   vp(bias.data_ptr() if bias is not None else None), vp(out.data_ptr()),
                                   vp(stream))
    if st != LF_OK:
        raise LfError(st, "lf_attn_project")
    return out.view((P,) + tuple(shape[:-1]) + (C,))


def encoder_attention(x: torch.Tensor, w: torch.Tensor, bias: Optional[torch.Tensor], mask: Optional[torch.Tensor],
                      window: int, dilation: Optional[Sequence[int]] = None, scale: Optional[float] = None,
                      max_global: Optional[int] = None, validate: bool = True,
                      w_out: Optional[torch.Tensor] = None, b_out: Optional[torch.Tensor] = None,
                      return_intermediate: bool = False, workspace: Optional[torch.Tensor] = None):
    """The attention sublayer of a Longformer/LED encoder layer as a chain
    of the C ABI's calls on the current stream: ``lf_attn_project`` (the six
    input projections Q_s, K_s, V_s, Q_g, K_g, V_g of x [B, n, C] in one
    launch, w [6C, C] stacked in that order, bias fp32 [6C] or None; with a
    mask, ``lf_attn_project_global_only`` with Q_g at the global tokens
    only, zero elsewhere), then
    ``lf_attn_forward`` on the six [B, n, H, 64] views of its output (H =
    C / 64), then, when w_out [C, C] is given, the output projection with
    ``lf_attn_project`` (P = 1, bias b_out fp32 [C] or None).  Returns
    [B, n, C] (and, with return_intermediate, the projections [6, B, n, C]
    and the attention output [B, n, H, 64]).  workspace: the attention's,
    from make_workspace (needed under graph capture)."""
    if x.dim() != 3:
        raise ValueError("x must be [B, n, C]")
    B, n, C = x.shape
    if C % LF_HEAD_DIM != 0:
        raise ValueError("C must be a multiple of 64")
    H = C // LF_HEAD_DIM
    if w.shape != (6 * C, C):
        raise ValueError("w must be [6C, C]: Q_s, K_s, V_s, Q_g, K_g, V_g stacked")
    # Q_g is read at the global rows only: computed there, zero elsewhere
    proj = project(x, w, bias, mask=mask, global_only=(3,)) if mask is not None else project(x, w, bias)
    heads = [proj[i].view(B, n, H, LF_HEAD_DIM) for i in range(6)]
    attn = forward(*heads, mask=mask, window=window, dilation=dilation, scale=scale, max_global=max_global,
                   validate=validate, workspace=workspace)
    y = attn.view(B, n, C)
    if w_out is not None:
        y = project(y, w_out, b_out)[0]
    return (y, proj, attn) if return_intermediate else y


def _prep_mask(mask, B, n, device, causal, max_global, validate):
    """Mask as contiguous int8 [B, n] on the device, and the max_global bound
    (derived from the mask when validating)."""
    if mask is None:
        mask = torch.ones((B, n), dtype=torch.int8, device=device)
    elif mask.dtype != torch.int8:
        mask = mask.to(torch.int8)
    mask = mask.contiguous()
    _check_tensor("mask", mask, (B, n), torch.int8, device)
    if validate:
        bad = ~((mask == 0) | (mask == 1) | (mask == 2))
        if bool(bad.any()):
            raise ValueError("mask values must be 0, 1 or 2")
        g = int((mask == 2).sum(dim=1).max().item())
        if causal and g > 0:
            raise ValueError("causal attention with global tokens is undefined")
        if max_global is None:
            max_global = g
        elif g > max_global:
            raise ValueError(f"mask has {g} global tokens in a row, max_global={max_global}")
        if max_global > LF_MAX_GLOBAL:
            raise ValueError(f"at most {LF_MAX_GLOBAL} global tokens per row are supported")
    if max_global is None:
        max_global = 0 if causal else min(n, LF_MAX_GLOBAL)
    return mask, max_global


def backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
             q_g: Optional[torch.Tensor], k_g: Optional[torch.Tensor], v_g: Optional[torch.Tensor],
             mask: Optional[torch.Tensor], out: torch.Tensor, dout: torch.Tensor, lse: torch.Tensor,
             window: int = 256, dilation: Optional[Sequence[int]] = None, causal: bool = False,
             scale: Optional[float] = None, max_global: Optional[int] = None,
             validate: bool = True, grads: Optional[Sequence[torch.Tensor]] = None,
             workspace: Optional[torch.Tensor] = None):
    """Gradients of the forward (``lf_attn_backward``): returns fp32
    (dq, dk, dv, dq_g, dk_g, dv_g), each [B, n, H, 64].  q..v_g, out and dout
    are bf16 or f16; out and lse are what ``forward(..., return_lse=True)``
    returned for the same inputs.  When q_g/k_g/v_g are None (aliasing
    q/k/v) the gradient of a shared tensor is the sum of its two results.
    ``grads`` may supply the six output tensors; ``workspace`` a buffer from
    ``make_workspace(..., backward=True)`` (needed under graph capture)."""
    if q.dim() != 4:
        raise ValueError("q must be [B, n, H, D]")
    B, n, H, D = q.shape
    device = q.device
    if device.type != "cuda":
        raise ValueError("q must be a GPU tensor (this library has no CPU path)")
    dtype = q.dtype
    q_g = q if q_g is None else q_g
    k_g = k if k_g is None else k_g
    v_g = v if v_g is None else v_g
    for name, t in (("q", q), ("k", k), ("v", v), ("q_g", q_g), ("k_g", k_g), ("v_g", v_g),
                    ("out", out), ("dout", dout)):
        _check_tensor(name, t, (B, n, H, D), dtype, device)
    _check_tensor("lse", lse, (B, H, n), torch.float32, device)
    mask, max_global = _prep_mask(mask, B, n, device, causal, max_global, validate)
    if grads is None:
        grads = [torch.empty((B, n, H, D), dtype=torch.float32, device=device) for _ in range(6)]
    for name, t in zip(("dq", "dk", "dv", "dq_g", "dk_g", "dv_g"), grads):
        _check_tensor(name, t, (B, n, H, D), torch.float32, device)
    p, _keep = make_params(B, n, H, D, window, dilation, causal, scale, max_global, dtype)
    lib = library()
    need = int(lib.lf_attn_backward_workspace_bytes(ctypes.byref(p)))
    if need == 0:
        raise LfError(LF_ERR_INVALID_ARG, "lf_attn_backward_workspace_bytes")
    stream = torch.cuda.current_stream(device).cuda_stream
    key = (device.index, stream)
    with _ws_lock:
        ws = _bwd_ws.get(key) if workspace is None else _given_workspace(workspace, need, device)
        if ws is None or ws.numel() < need:
            if _capturing():
                raise RuntimeError(_CAPTURE_MSG.format(what="backward"))
            ws = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
            st = lib.lf_attn_workspace_init(ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(ws.numel()),
                                            ctypes.c_void_p(stream))
            if st != LF_OK:
                raise LfError(st, "lf_attn_workspace_init")
            _bwd_ws[key] = ws
    vp = ctypes.c_void_p
    st = lib.lf_attn_backward(
        ctypes.byref(p), *[vp(t.data_ptr()) for t in (q, k, v, q_g, k_g, v_g, mask, out, dout, lse)],
        *[vp(t.data_ptr()) for t in grads], vp(ws.data_ptr()), ctypes.c_size_t(ws.numel()), vp(stream))
    if st != LF_OK:
        raise LfError(st, "lf_attn_backward")
    return tuple(grads)


def device_status(device: Optional[torch.device] = None, kind: str = "any",
                  workspace: Optional[torch.Tensor] = None) -> int:
    """Synchronise and read a device status word (``lf_attn_device_status``);
    0 = nothing flagged.  kind="forward" or "backward" reads the workspace
    that ``forward`` or ``backward`` used on the current stream, "any" the OR
    of both; ``workspace`` reads that buffer instead.  The words are sticky:
    a flag stays set until the workspace is re-initialised."""
    device = torch.device("cuda", torch.cuda.current_device()) if device is None else device
    stream = torch.cuda.current_stream(device).cuda_stream
    if kind not in ("any", "forward", "backward"):
        raise ValueError("kind must be 'any', 'forward' or 'backward'")
    bufs = []
    if workspace is not None:
        bufs.append(workspace)
    else:
        key = (device.index, stream)
        if kind in ("any", "forward"):
            bufs.append(_ws_cache.get(key, (None, None))[0])
        if kind in ("any", "backward"):
            bufs.append(_bwd_ws.get(key))
    word = 0
    for ws in bufs:
        if ws is None:
            continue
        val = ctypes.c_int32(0)
        st = library().lf_attn_device_status(ctypes.c_void_p(ws.data_ptr()), ctypes.c_void_p(stream),
                                             ctypes.byref(val))
        if st != LF_OK:
            raise LfError(st, "lf_attn_device_status")
        word |= int(val.value)
    return word


def pad_to_window_size(x: torch.Tensor, mask: torch.Tensor, attention_window: int, pad_value=0):
    """Pad dim 1 of ``x`` (ids [B, n] or tensors [B, n, ...]) and of ``mask``
    ([B, n]) up to a multiple of ``attention_window`` (the two-sided window,
    2w).  Padding tokens get ``pad_value`` in x and 0 (no attention) in the
    mask, as the allenai README's usage step prescribes before the model
    call.  Returns (x, mask); unchanged if already a multiple."""
    if attention_window <= 0:
        raise ValueError("attention_window must be positive")
    n = x.shape[1]
    if mask.shape[:2] != x.shape[:2]:
        raise ValueError("x and mask disagree on [B, n]")
    pad = (-n) % attention_window
    if pad == 0:
        return x, mask
    xs = list(x.shape)
    xs[1] = pad
    x = torch.cat([x, torch.full(xs, pad_value, dtype=x.dtype, device=x.device)], dim=1)
    ms = list(mask.shape)
    ms[1] = pad
    mask = torch.cat([mask, torch.zeros(ms, dtype=mask.dtype, device=mask.device)], dim=1)
    return x, mask


def merge_masks(attention_mask: torch.Tensor, global_attention_mask: torch.Tensor) -> torch.Tensor:
    """Turn a 0/1 attention mask plus a 0/1 global-attention mask into the
    0/1/2 mask (int8): padding stays 0, attended tokens are 1, attended
    global tokens are 2."""
    if attention_mask.shape != global_attention_mask.shape:
        raise ValueError("mask shapes differ")
    a = (attention_mask != 0).to(torch.int8)
    g = (global_attention_mask != 0).to(torch.int8)
    return a * (1 + g)
