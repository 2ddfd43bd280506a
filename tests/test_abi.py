"""The C-ABI library without a GPU: it loads, exports every entry point the
header declares, and rejects every invalid argument before any HIP call.
Also the pure-torch input helpers of the binding."""
import ctypes
import os
import re

import pytest
import torch

import sparse_long_document_amd as lf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lf_attn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(lf.LIB_PATH), reason="library not built")

FAKE = 0x7F0000000000  # never dereferenced: validation fails first


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lf_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert set(names) == set(lf.SYMBOLS)
    lib = lf.library()
    for name in names:
        assert hasattr(lib, name), name


def test_header_constants_match_binding():
    text = open(HEADER).read()
    for name, val in (("LF_HEAD_DIM", lf.LF_HEAD_DIM), ("LF_MAX_HEADS", lf.LF_MAX_HEADS),
                      ("LF_MAX_GLOBAL", lf.LF_MAX_GLOBAL)):
        m = re.search(rf"#define {name} (\d+)", text)
        assert m and int(m.group(1)) == val


def test_status_strings():
    assert lf.status_str(0) == "ok"
    for code in range(1, 5):
        assert lf.status_str(code) != "unknown status"
    assert lf.status_str(77) == "unknown status"


def _params(**kw):
    base = dict(B=1, n=4096, H=12, D=64, window=256, dilation=None, causal=False,
                scale=None, max_global=1, dtype=torch.bfloat16)
    base.update(kw)
    return lf.make_params(**base)


def _forward(p, ptrs=None, ws_bytes=1 << 30, row_nnz=None):
    lib = lf.library()
    vp = ctypes.c_void_p
    base = dict(q=FAKE, k=FAKE + (1 << 32), v=FAKE + (2 << 32), qg=None, kg=None, vg=None,
                mask=FAKE + (3 << 32), out=FAKE + (4 << 32), ws=FAKE + (5 << 32))
    base.update(ptrs or {})
    ptrs = base
    return lib.lf_attn_forward(ctypes.byref(p), vp(ptrs["q"]), vp(ptrs["k"]), vp(ptrs["v"]),
                               vp(ptrs["qg"]), vp(ptrs["kg"]), vp(ptrs["vg"]), vp(ptrs["mask"]),
                               vp(ptrs["out"]), vp(row_nnz), vp(ptrs["ws"]),
                               ctypes.c_size_t(ws_bytes), vp(None))


def test_workspace_bytes_layout():
    # 256-byte status block, B*H counters padded to 256, then the partial
    # records of the global rows: B*H*max_global*ceil(n/512) records of 68
    # floats (the split count of the shorter key chunk)
    p, _k = _params(B=2, n=4096, H=12, max_global=64)
    got = lf.library().lf_attn_workspace_bytes(ctypes.byref(p))
    rec = 2 * 12 * 64 * 8 * 68 * 4
    assert got == 256 + 256 + rec
    p, _k = _params(causal=True, max_global=0)
    assert lf.library().lf_attn_workspace_bytes(ctypes.byref(p)) == 512


@pytest.mark.parametrize("D", [32, 64, 128])
def test_workspace_bytes_per_head_dim(D):
    # a partial record holds (m, l, count, pad) and the D outputs
    p, _k = _params(B=1, n=1000, H=3, D=D, max_global=5)
    rec = 1 * 3 * 5 * 2 * (4 + D) * 4
    assert lf.library().lf_attn_workspace_bytes(ctypes.byref(p)) == 256 + 256 + (rec + 255) // 256 * 256


@pytest.mark.parametrize("D", [32, 128])
def test_backward_takes_head_dim_64_only(D):
    # the forward takes these head dims; the gradient kernels do not
    p, _k = _params(D=D)
    assert lf.library().lf_attn_workspace_bytes(ctypes.byref(p)) > 0
    assert lf.library().lf_attn_backward_workspace_bytes(ctypes.byref(p)) == 0
    assert _backward(p) == lf.LF_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), lf.LF_ERR_INVALID_ARG),
    (dict(n=0), lf.LF_ERR_INVALID_ARG),
    (dict(H=0), lf.LF_ERR_INVALID_ARG),
    (dict(window=-1), lf.LF_ERR_INVALID_ARG),
    (dict(dilation=[1] * 11 + [0]), lf.LF_ERR_INVALID_ARG),
    (dict(scale=float("nan")), lf.LF_ERR_INVALID_ARG),
    (dict(scale=float("inf")), lf.LF_ERR_INVALID_ARG),
    (dict(scale=-0.5), lf.LF_ERR_INVALID_ARG),
    (dict(max_global=-1), lf.LF_ERR_INVALID_ARG),
    (dict(D=16), lf.LF_ERR_UNSUPPORTED),
    (dict(D=48), lf.LF_ERR_UNSUPPORTED),
    (dict(D=96), lf.LF_ERR_UNSUPPORTED),
    (dict(D=256), lf.LF_ERR_UNSUPPORTED),
    (dict(D=1), lf.LF_ERR_UNSUPPORTED),
    (dict(dtype=torch.float64), lf.LF_ERR_UNSUPPORTED),
    (dict(H=65, dilation=None), lf.LF_ERR_UNSUPPORTED),
    (dict(max_global=2000), lf.LF_ERR_UNSUPPORTED),
    (dict(n=(1 << 24) + 1), lf.LF_ERR_UNSUPPORTED),
    (dict(n=1 << 20, H=16, dilation=None), lf.LF_ERR_UNSUPPORTED),  # one batch row of q is 2 GiB
])
def test_invalid_params_rejected_before_hip(kw, code):
    p, _k = _params(**kw)
    assert _forward(p) == code
    assert lf.library().lf_attn_workspace_bytes(ctypes.byref(p)) == 0


def test_causal_flag_must_be_boolean():
    p, _k = _params()
    p.causal = 2
    assert _forward(p) == lf.LF_ERR_INVALID_ARG


def test_null_params_and_pointers():
    lib = lf.library()
    vp = ctypes.c_void_p
    assert lib.lf_attn_forward(None, *([vp(FAKE)] * 8), vp(None), vp(FAKE), ctypes.c_size_t(1 << 30),
                               vp(None)) == lf.LF_ERR_INVALID_ARG
    p, _k = _params()
    for name in ("q", "k", "v", "mask", "out"):
        assert _forward(p, {name: None}) == lf.LF_ERR_INVALID_ARG, name


def test_output_aliasing_rejected():
    p, _k = _params()
    assert _forward(p, {"out": FAKE}) == lf.LF_ERR_INVALID_ARG  # out == q
    assert _forward(p, {"out": FAKE + 100}) == lf.LF_ERR_INVALID_ARG  # overlaps q
    assert _forward(p, {"qg": FAKE + (4 << 32)}) == lf.LF_ERR_INVALID_ARG  # q_g == out
    assert _forward(p, row_nnz=FAKE + (4 << 32) + 64) == lf.LF_ERR_INVALID_ARG


def test_workspace_errors():
    p, _k = _params(B=2, max_global=64)
    need = lf.library().lf_attn_workspace_bytes(ctypes.byref(p))
    assert _forward(p, {"ws": None}) == lf.LF_ERR_WORKSPACE
    assert _forward(p, ws_bytes=need - 1) == lf.LF_ERR_WORKSPACE
    lib = lf.library()
    assert lib.lf_attn_workspace_init(None, 4096, None) == lf.LF_ERR_WORKSPACE
    assert lib.lf_attn_workspace_init(ctypes.c_void_p(FAKE), 16, None) == lf.LF_ERR_WORKSPACE
    assert lib.lf_attn_device_status(None, None, None) == lf.LF_ERR_INVALID_ARG


def test_workspace_overlapping_any_buffer_rejected():
    # the kernel writes tickets and partial records into the workspace, so it
    # may overlap none of the six inputs, the mask, out, row_nnz or lse
    p, _k = _params(B=2, max_global=64)
    tb = 2 * 4096 * 12 * 64 * 2
    for name, addr in (("q", FAKE), ("k", FAKE + (1 << 32)), ("v", FAKE + (2 << 32)),
                       ("mask", FAKE + (3 << 32)), ("out", FAKE + (4 << 32))):
        assert _forward(p, {"ws": addr + 64}) == lf.LF_ERR_INVALID_ARG, name
    for name in ("qg", "kg", "vg"):
        other = FAKE + (7 << 32)
        assert _forward(p, {name: other, "ws": other + tb - 256}) == lf.LF_ERR_INVALID_ARG, name
    nnz = FAKE + (8 << 32)
    assert _forward(p, {"ws": nnz + 16}, row_nnz=nnz) == lf.LF_ERR_INVALID_ARG


def test_forward_refuses_cpu_tensors():
    x = torch.zeros(1, 8, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        lf.forward(x, x, x, window=2)


def test_pad_to_window_size():
    ids = torch.arange(10).reshape(1, 10)
    mask = torch.ones(1, 10, dtype=torch.int8)
    mask[0, 0] = 2
    ids2, mask2 = lf.pad_to_window_size(ids, mask, 8, pad_value=1)
    assert ids2.shape == (1, 16) and mask2.shape == (1, 16)
    assert ids2[0, 10:].eq(1).all() and mask2[0, 10:].eq(0).all()
    assert torch.equal(ids2[:, :10], ids) and torch.equal(mask2[:, :10], mask)
    x = torch.randn(2, 16, 3, 64)
    m = torch.ones(2, 16, dtype=torch.int8)
    x3, m3 = lf.pad_to_window_size(x, m, 8)
    assert x3 is x and m3 is m


def test_merge_masks():
    a = torch.tensor([[1, 1, 1, 0]])
    g = torch.tensor([[1, 0, 0, 1]])
    assert lf.merge_masks(a, g).tolist() == [[2, 1, 1, 0]]
    assert lf.merge_masks(a, g).dtype == torch.int8


# ---------------------------------------------------------------------------
# lf_attn_forward_lse and lf_attn_backward: argument checks (no HIP call)
# ---------------------------------------------------------------------------

def _backward(p, ptrs=None, ws_bytes=1 << 30):
    lib = lf.library()
    vp = ctypes.c_void_p
    names = ("q", "k", "v", "qg", "kg", "vg", "mask", "out", "dout", "lse",
             "dq", "dk", "dv", "dqg", "dkg", "dvg", "ws")
    base = {nm: FAKE + (i << 32) for i, nm in enumerate(names)}
    base.update(qg=None, kg=None, vg=None)
    base.update(ptrs or {})
    return lib.lf_attn_backward(ctypes.byref(p), *[vp(base[nm]) for nm in names],
                                ctypes.c_size_t(ws_bytes), vp(None))


def test_backward_workspace_bytes_layout():
    # status block, B counts, B lists of max_global entries, two fp32 per
    # row (<dout, out> and the log2-domain lse)
    p, _k = _params(B=2, n=4096, H=12, max_global=64)
    got = lf.library().lf_attn_backward_workspace_bytes(ctypes.byref(p))
    assert got == 256 + 256 + 512 + 2 * 2 * 12 * 4096 * 4
    p, _k = _params(B=0)
    assert lf.library().lf_attn_backward_workspace_bytes(ctypes.byref(p)) == 0


def test_backward_argument_errors():
    p, _k = _params()
    for name in ("q", "k", "v", "mask", "out", "dout", "lse", "dq", "dk", "dv", "dqg", "dkg", "dvg"):
        assert _backward(p, {name: None}) == lf.LF_ERR_INVALID_ARG, name
    assert _backward(p, {"dk": FAKE + (10 << 32)}) == lf.LF_ERR_INVALID_ARG  # dk == dq
    assert _backward(p, {"dq": FAKE + 64}) == lf.LF_ERR_INVALID_ARG  # dq overlaps q
    assert _backward(p, {"ws": None}) == lf.LF_ERR_WORKSPACE
    need = lf.library().lf_attn_backward_workspace_bytes(ctypes.byref(p))
    assert _backward(p, ws_bytes=need - 1) == lf.LF_ERR_WORKSPACE
    p32, _k = _params(dtype=torch.float32)
    assert _backward(p32) == lf.LF_ERR_UNSUPPORTED


def test_forward_lse_requires_lse():
    p, _k = _params()
    lib = lf.library()
    vp = ctypes.c_void_p
    args = [vp(FAKE), vp(FAKE + (1 << 32)), vp(FAKE + (2 << 32)), vp(None), vp(None), vp(None),
            vp(FAKE + (3 << 32)), vp(FAKE + (4 << 32)), vp(None)]
    ws = [vp(FAKE + (5 << 32)), ctypes.c_size_t(1 << 30), vp(None)]
    assert lib.lf_attn_forward_lse(ctypes.byref(p), *args, vp(None), *ws) == lf.LF_ERR_INVALID_ARG
    # lse overlapping the output
    assert lib.lf_attn_forward_lse(ctypes.byref(p), *args, vp(FAKE + (4 << 32) + 256), *ws) \
        == lf.LF_ERR_INVALID_ARG


def test_project_argument_errors():
    lib = lf.library()
    vp = ctypes.c_void_p
    BF16 = lf._DTYPES[torch.bfloat16]

    def call(M=4096, C=768, P=6, dtype=BF16, x=FAKE, w=FAKE + (1 << 32), bias=FAKE + (2 << 32),
             out=FAKE + (3 << 32)):
        return lib.lf_attn_project(M, C, P, dtype, vp(x), vp(w), vp(bias), vp(out), vp(None))

    for kw in (dict(M=0), dict(C=0), dict(P=0), dict(x=None), dict(w=None), dict(out=None),
               dict(out=FAKE + 4096)):  # out overlapping x
        assert call(**kw) == lf.LF_ERR_INVALID_ARG, kw
    for kw in (dict(dtype=99), dict(C=96), dict(P=7),
               dict(M=1 << 20, C=1024),  # x larger than 2^31 - 1 bytes
               dict(x=FAKE + 8), dict(w=FAKE + (1 << 32) + 2), dict(out=FAKE + (3 << 32) + 4),
               dict(bias=FAKE + (2 << 32) + 8)):  # bases not 16-byte aligned
        assert call(**kw) == lf.LF_ERR_UNSUPPORTED, kw


def test_project_global_only_argument_errors():
    lib = lf.library()
    vp = ctypes.c_void_p
    BF16 = lf._DTYPES[torch.bfloat16]

    def call(P=6, bits=1 << 3, mask=FAKE + (4 << 32), out=FAKE + (3 << 32)):
        return lib.lf_attn_project_global_only(4096, 768, P, BF16, vp(FAKE), vp(FAKE + (1 << 32)),
                                               vp(FAKE + (2 << 32)), vp(mask), ctypes.c_uint32(bits), vp(out),
                                               vp(None))

    assert call(bits=1 << 6) == lf.LF_ERR_INVALID_ARG  # a projection beyond P
    assert call(P=3, bits=1 << 3) == lf.LF_ERR_INVALID_ARG
    assert call(mask=None) == lf.LF_ERR_INVALID_ARG
    assert call(mask=FAKE + (3 << 32) + 4096) == lf.LF_ERR_INVALID_ARG  # mask inside out
    assert call(P=7) == lf.LF_ERR_UNSUPPORTED
