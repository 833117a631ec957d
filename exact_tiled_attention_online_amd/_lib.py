"""ctypes binding of libfa.so: the C entry points under the same names, plus
torch-tensor conveniences that only marshal arguments.

Every step of the computation runs in the library's HIP kernels; this module
allocates outputs with torch and passes device pointers and the current HIP
stream.  If the library has not been built, loading fails loudly: there is no
fallback implementation.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_OK, FA_ERR_INVALID, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE, FA_ERR_HIP, FA_ERR_SCRATCH = 0, -1, -2, -3, -4, -5
FA_SPLITKV_NOALLOC_MAX_BYTES = 32 * 1024 * 1024
FA_BF16, FA_FP32 = 0, 1
FA_LAYOUT_BHND, FA_LAYOUT_BNHD = 0, 1
FA_DQ_HANDOFF, FA_DQ_RECOMPUTE, FA_DQ_ATOMIC = 0, 1, 2

EXPORTS = ("fa_fwd", "fa_bwd", "fa_bwd_workspace_bytes", "fa_bwd_workspace_size", "fa_bwd_dq_method",
           "fa_bwd_preprocess", "fa_bwd_dkdv",
           "fa_bwd_dq", "fa_fwd_fp8", "fa_fwd_splitkv_workspace_bytes", "fa_fwd_splitkv",
           "fa_fwd_splitkv_fp8_workspace_bytes", "fa_fwd_splitkv_fp8", "fa_fwd_dropout", "fa_bwd_dropout",
           "fa_fwd_splitkv_noalloc", "fa_fwd_strided", "fa_bwd_strided",
           "fa_strerror")

_lib = None


class FAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {fa_strerror(status)} (status {status})")


def load():
    """Load libfa.so once and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    _lib = _open(LIB_PATH)
    return _lib


_variants = {}


@contextlib.contextmanager
def using_library(path):
    """Route every entry point of this module to another build of the library
    (the checking variants libfa_debug_sync.so and libfa_tile_alt.so) for the
    duration of the block: tests run the same calls against both builds."""
    global _lib
    prev = load()
    if path not in _variants:
        _variants[path] = _open(path)
    _lib = _variants[path]
    try:
        yield _lib
    finally:
        _lib = prev


def _open(path):
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m exact_tiled_attention_online_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, vp, i, i]
    lib.fa_fwd.restype = i
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, vp, sz, vp, i, i]
    lib.fa_bwd.restype = i
    lib.fa_bwd_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.fa_bwd_workspace_bytes.restype = sz
    lib.fa_bwd_workspace_size.argtypes = [i, i, i, i, i, i, i]
    lib.fa_bwd_workspace_size.restype = sz
    lib.fa_bwd_dq_method.argtypes = [i, i, i, i, i, i, sz, i]
    lib.fa_bwd_dq_method.restype = i
    lib.fa_bwd_preprocess.argtypes = [vp, vp, vp, i, i, i, i, f, vp, sz, vp, i, i]
    lib.fa_bwd_preprocess.restype = i
    lib.fa_bwd_dkdv.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, vp, sz, vp, i, i]
    lib.fa_bwd_dkdv.restype = i
    lib.fa_bwd_dq.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, vp, sz, vp, i, i]
    lib.fa_bwd_dq.restype = i
    lib.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, f, f, f, vp, i]
    lib.fa_fwd_fp8.restype = i
    lib.fa_fwd_splitkv_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.fa_fwd_splitkv_workspace_bytes.restype = sz
    lib.fa_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, sz, vp, i, i]
    lib.fa_fwd_splitkv.restype = i
    lib.fa_fwd_splitkv_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, i, i]
    lib.fa_fwd_splitkv_noalloc.restype = i
    lib.fa_fwd_splitkv_fp8_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.fa_fwd_splitkv_fp8_workspace_bytes.restype = sz
    lib.fa_fwd_splitkv_fp8.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, f, f, f, i, vp, sz, vp, i]
    lib.fa_fwd_splitkv_fp8.restype = i
    u64, u32 = ctypes.c_ulonglong, ctypes.c_uint
    lib.fa_fwd_dropout.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, u64, u32, vp, i]
    lib.fa_fwd_dropout.restype = i
    lib.fa_bwd_dropout.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, u64, u32, vp, sz,
                                   vp, i]
    lib.fa_bwd_dropout.restype = i
    pll = ctypes.POINTER(ctypes.c_longlong)
    lib.fa_fwd_strided.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, pll, vp, i]
    lib.fa_fwd_strided.restype = i
    lib.fa_bwd_strided.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, pll, vp, sz, vp, i]
    lib.fa_bwd_strided.restype = i
    lib.fa_strerror.argtypes = [i]
    lib.fa_strerror.restype = ctypes.c_char_p
    return lib


# ---- the C entry points, same names, raw integer pointers ------------------

def fa_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, stream, dtype, layout) -> int:
    return load().fa_fwd(q, k, v, o, lse, B, H, N, d, int(causal), float(scale), stream, dtype, layout)


def fa_bwd(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, causal, scale, workspace, workspace_bytes,
           stream, dtype, layout) -> int:
    return load().fa_bwd(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, int(causal), float(scale),
                         workspace, workspace_bytes, stream, dtype, layout)


def fa_bwd_workspace_bytes(B, H, N, d, dtype) -> int:
    return load().fa_bwd_workspace_bytes(B, H, N, d, dtype)


def fa_bwd_workspace_size(B, H, N, d, causal, dtype, dq_method) -> int:
    return load().fa_bwd_workspace_size(B, H, N, d, int(causal), dtype, dq_method)


def fa_bwd_dq_method(B, H, N, d, causal, dtype, workspace_bytes, dropout) -> int:
    return load().fa_bwd_dq_method(B, H, N, d, int(causal), dtype, workspace_bytes, int(dropout))


def fa_bwd_preprocess(o, dO, lse, B, H, N, d, scale, workspace, workspace_bytes, stream, dtype,
                      layout) -> int:
    return load().fa_bwd_preprocess(o, dO, lse, B, H, N, d, float(scale), workspace, workspace_bytes,
                                    stream, dtype, layout)


def fa_bwd_dkdv(q, k, v, dO, lse, dk, dv, B, H, N, d, causal, scale, workspace, workspace_bytes,
                stream, dtype, layout) -> int:
    return load().fa_bwd_dkdv(q, k, v, dO, lse, dk, dv, B, H, N, d, int(causal), float(scale),
                              workspace, workspace_bytes, stream, dtype, layout)


def fa_bwd_dq(q, k, v, dO, lse, dq, B, H, N, d, causal, scale, workspace, workspace_bytes,
              stream, dtype, layout) -> int:
    return load().fa_bwd_dq(q, k, v, dO, lse, dq, B, H, N, d, int(causal), float(scale),
                            workspace, workspace_bytes, stream, dtype, layout)


def fa_fwd_fp8(q, k, v, o, lse, B, H, N, d, causal, scale, descale_q, descale_k, descale_v, stream,
               layout) -> int:
    return load().fa_fwd_fp8(q, k, v, o, lse, B, H, N, d, int(causal), float(scale), float(descale_q),
                             float(descale_k), float(descale_v), stream, layout)


def fa_fwd_splitkv_workspace_bytes(B, H, Nq, Nk, d, num_splits) -> int:
    return load().fa_fwd_splitkv_workspace_bytes(B, H, Nq, Nk, d, num_splits)


def fa_fwd_splitkv(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, num_splits, workspace, workspace_bytes,
                   stream, dtype, layout) -> int:
    return load().fa_fwd_splitkv(q, k, v, o, lse, B, H, Nq, Nk, d, int(causal), float(scale), num_splits,
                                 workspace, workspace_bytes, stream, dtype, layout)


def fa_fwd_splitkv_noalloc(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, num_splits, stream, dtype,
                           layout) -> int:
    return load().fa_fwd_splitkv_noalloc(q, k, v, o, lse, B, H, Nq, Nk, d, int(causal), float(scale), num_splits,
                                         stream, dtype, layout)


def fa_fwd_splitkv_fp8_workspace_bytes(B, H, Nq, Nk, d, num_splits) -> int:
    return load().fa_fwd_splitkv_fp8_workspace_bytes(B, H, Nq, Nk, d, num_splits)


def fa_fwd_splitkv_fp8(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, descale_q, descale_k, descale_v,
                       num_splits, workspace, workspace_bytes, stream, layout) -> int:
    return load().fa_fwd_splitkv_fp8(q, k, v, o, lse, B, H, Nq, Nk, d, int(causal), float(scale),
                                     float(descale_q), float(descale_k), float(descale_v), num_splits, workspace,
                                     workspace_bytes, stream, layout)


def fa_fwd_dropout(q, k, v, o, lse, B, H, N, d, causal, scale, drop_t, seed, offset, stream, layout) -> int:
    return load().fa_fwd_dropout(q, k, v, o, lse, B, H, N, d, int(causal), float(scale), int(drop_t),
                                 _check_uint(seed, 64, "seed"), _check_uint(offset, 32, "offset"), stream, layout)


def fa_bwd_dropout(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, causal, scale, drop_t, seed, offset, workspace,
                   workspace_bytes, stream, layout) -> int:
    return load().fa_bwd_dropout(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, int(causal), float(scale),
                                 int(drop_t), _check_uint(seed, 64, "seed"), _check_uint(offset, 32, "offset"),
                                 workspace, workspace_bytes, stream, layout)


def _strides_arg(strides):
    """A host array of element strides for the strided calls (None: NULL)."""
    if strides is None:
        return None
    vals = [int(x) for x in strides]
    return (ctypes.c_longlong * len(vals))(*vals)


def fa_fwd_strided(q, k, v, o, lse, B, H, N, d, causal, scale, strides, stream, dtype) -> int:
    """strides: 12 integers, (batch, head, row) element strides of q, k, v, o."""
    if strides is not None and len(strides) != 12:
        raise ValueError("fa_fwd_strided takes 12 strides (3 each for q, k, v, o)")
    return load().fa_fwd_strided(q, k, v, o, lse, B, H, N, d, int(causal), float(scale), _strides_arg(strides),
                                 stream, dtype)


def fa_bwd_strided(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, causal, scale, strides, workspace,
                   workspace_bytes, stream, dtype) -> int:
    """strides: 24 integers, (batch, head, row) element strides of q, k, v,
    o, dO, dq, dk, dv."""
    if strides is not None and len(strides) != 24:
        raise ValueError("fa_bwd_strided takes 24 strides (3 each for q, k, v, o, dO, dq, dk, dv)")
    return load().fa_bwd_strided(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, int(causal), float(scale),
                                 _strides_arg(strides), workspace, workspace_bytes, stream, dtype)


def fa_strerror(status: int) -> str:
    return load().fa_strerror(status).decode()


# ---- torch conveniences ------------------------------------------------------

def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float32:
        return FA_FP32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _check(ts, shape):
    for t in ts:
        if not t.is_cuda or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
            raise ValueError("expected contiguous device tensors of one shape")
        if t.dtype != ts[0].dtype:
            raise ValueError("q, k, v (and o, dO) must share one dtype")
        if t.device != ts[0].device:
            raise ValueError("all tensors must be on one device")


def _check_buf(t, shape, dtype, device, name):
    """A caller-supplied output or statistics buffer: the kernels write (or
    read) exactly `shape` elements of `dtype` through its pointer."""
    if (t.device != device or t.dtype != dtype or not t.is_contiguous()
            or tuple(t.shape) != tuple(shape)):
        raise ValueError(f"{name}: expected a contiguous {dtype} tensor of shape {tuple(shape)} on {device}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")
    return t


def _check_ws(ws, device):
    """The workspace is passed as (pointer, byte count): a contiguous uint8
    device tensor, so that numel() is its size in bytes."""
    import torch
    if ws.device != device or ws.dtype != torch.uint8 or not ws.is_contiguous():
        raise ValueError("workspace: expected a contiguous uint8 tensor on the inputs' device")
    return ws


def _check_uint(x, bits, name):
    x = int(x)
    if not 0 <= x < (1 << bits):
        raise ValueError(f"{name} = {x} is outside [0, 2^{bits})")
    return x


def _dims(q, layout):
    """(B, H, N, d) of a tensor in the named layout."""
    if layout == FA_LAYOUT_BHND:
        B, H, N, d = q.shape
    elif layout == FA_LAYOUT_BNHD:
        B, N, H, d = q.shape
    else:
        raise ValueError(f"unknown layout {layout}")
    return B, H, N, d


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check_kv_heads(q, k, layout, what="k, v"):
    """The key/value cache of a split forward must have q's batch, heads and
    head dim (the kernels address K and V rows with q's (B, H, d)); only the
    row count may differ."""
    B, H, _, d = _dims(q, layout)
    Bk, Hk, _, dk = _dims(k, layout)
    if (Bk, Hk, dk) != (B, H, d):
        raise ValueError(f"{what}: expected batch, heads and head dim {(B, H, d)} as q, got {(Bk, Hk, dk)}")


def forward(q, k, v, causal: bool, scale: float, out=None, lse=None, stream=None,
            layout: int = FA_LAYOUT_BHND):
    """O, LSE = attention forward on device tensors (bf16 or fp32) of shape
    [B,H,N,d] (layout FA_LAYOUT_BHND) or [B,N,H,d] (FA_LAYOUT_BNHD); LSE is
    always [B,H,N] float32."""
    import torch
    B, H, N, d = _dims(q, layout)
    _check((q, k, v), q.shape)
    o = torch.empty_like(q) if out is None else _check_buf(out, q.shape, q.dtype, q.device, "out")
    l = (torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None
         else _check_buf(lse, (B, H, N), torch.float32, q.device, "lse"))
    st = fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), l.data_ptr(),
                B, H, N, d, causal, scale, _stream(stream), _dtype_code(q), layout)
    if st != FA_OK:
        raise FAError(st, "fa_fwd")
    return o, l


def workspace(q, layout: int = FA_LAYOUT_BHND, causal: bool = False, method: int = FA_DQ_HANDOFF):
    """A device byte buffer for fa_bwd on q's shape and dtype, sized for the dQ
    method `method` (the library takes the hand-off whenever the buffer holds
    it).  The hand-off buffer of a non-causal backward also serves a causal one.
    Never smaller than fa_bwd_workspace_bytes (which, with FA_DQ_MODE=atomic,
    holds the atomic method's accumulator)."""
    import torch
    B, H, N, d = _dims(q, layout)
    code = _dtype_code(q)
    n = max(fa_bwd_workspace_size(B, H, N, d, causal, code, method), fa_bwd_workspace_bytes(B, H, N, d, code))
    return torch.empty(max(n, 256), dtype=torch.uint8, device=q.device)


def backward(q, k, v, o, do, lse, causal: bool, scale: float, ws=None, grads=None, stream=None,
             layout: int = FA_LAYOUT_BHND, method: int = FA_DQ_HANDOFF):
    """dQ, dK, dV of attention on device tensors in the named layout, given O
    and LSE from forward.  Without `ws`, a workspace for `method` is allocated
    (FA_DQ_RECOMPUTE: the smallest one)."""
    import torch
    B, H, N, d = _dims(q, layout)
    _check((q, k, v, o, do), q.shape)
    _check_buf(lse, (B, H, N), torch.float32, q.device, "lse")
    ws = workspace(q, layout, causal, method) if ws is None else _check_ws(ws, q.device)
    if grads is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    else:
        dq, dk, dv = (_check_buf(g, q.shape, q.dtype, q.device, n) for g, n in zip(grads, ("dq", "dk", "dv")))
    st = fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, causal, scale,
                ws.data_ptr(), ws.numel(), _stream(stream), _dtype_code(q), layout)
    if st != FA_OK:
        raise FAError(st, "fa_bwd")
    return dq, dk, dv


def _view(t, shape, dtype, device, name):
    """(stride_b, stride_h, stride_n) in elements of a [B,H,N,d] device view
    whose rows are contiguous (any other strides: slices of a packed buffer,
    permuted dimensions, padding between rows).  A dimension of one entry
    reports stride 0 (its stride never enters an address)."""
    if not t.is_cuda or t.device != device or t.dtype != dtype or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected a {dtype} view of shape {tuple(shape)} on {device}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")
    if shape[3] > 1 and t.stride(3) != 1:
        raise ValueError(f"{name}: the head dim must be contiguous (stride 1), got strides {t.stride()}")
    return tuple(0 if shape[i] == 1 else t.stride(i) for i in range(3))


def forward_strided(q, k, v, causal: bool, scale: float, out=None, lse=None, stream=None):
    """O, LSE of attention on [B,H,N,d] views with any strides whose rows are
    contiguous, e.g. q, k, v = qkv.view(B, N, 3, H, d).permute(2, 0, 3, 1, 4)
    for a packed projection, with no copy.  O is a new contiguous [B,H,N,d]
    tensor unless `out` (any such view) is given; LSE is [B,H,N] float32."""
    import torch
    B, H, N, d = q.shape
    shape, dt, dev = (B, H, N, d), q.dtype, q.device
    st = []
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        st += _view(t, shape, dt, dev, n)
    o = torch.empty(shape, dtype=dt, device=dev) if out is None else out
    st += _view(o, shape, dt, dev, "out")
    l = (torch.empty((B, H, N), dtype=torch.float32, device=dev) if lse is None
         else _check_buf(lse, (B, H, N), torch.float32, dev, "lse"))
    r = fa_fwd_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), l.data_ptr(), B, H, N, d, causal,
                       scale, st, _stream(stream), _dtype_code(q))
    if r != FA_OK:
        raise FAError(r, "fa_fwd_strided")
    return o, l


def backward_strided(q, k, v, o, do, lse, causal: bool, scale: float, ws=None, grads=None, stream=None,
                     method: int = FA_DQ_HANDOFF):
    """dQ, dK, dV on [B,H,N,d] views with any strides whose rows are
    contiguous (as forward_strided).  `grads` may be three such views (for
    example slices of one packed gradient buffer); otherwise new contiguous
    [B,H,N,d] tensors are returned."""
    import torch
    B, H, N, d = q.shape
    shape, dt, dev = (B, H, N, d), q.dtype, q.device
    if grads is None:
        grads = tuple(torch.empty(shape, dtype=dt, device=dev) for _ in range(3))
    dq, dk, dv = grads
    st = []
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (do, "do"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
        st += _view(t, shape, dt, dev, n)
    _check_buf(lse, (B, H, N), torch.float32, dev, "lse")
    ws = workspace(q, FA_LAYOUT_BHND, causal, method) if ws is None else _check_ws(ws, dev)
    r = fa_bwd_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                       dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, causal, scale, st,
                       ws.data_ptr(), ws.numel(), _stream(stream), _dtype_code(q))
    if r != FA_OK:
        raise FAError(r, "fa_bwd_strided")
    return dq, dk, dv


def forward_splitkv(q, k, v, causal: bool, scale: float, num_splits: int = 0, out=None, lse=None, ws=None,
                    stream=None, layout: int = FA_LAYOUT_BHND):
    """O, LSE for q [B,H,Nq,d] against k, v [B,H,Nk,d] (bf16 device tensors;
    [B,Nq,H,d] / [B,Nk,H,d] with FA_LAYOUT_BNHD) through the split-key-range
    forward.  With ``causal`` the queries are the last Nq positions."""
    import torch
    B, H, Nq, d = _dims(q, layout)
    Nk = _dims(k, layout)[2]
    _check((q,), q.shape)
    _check((k, v), k.shape)
    if k.dtype != q.dtype or k.device != q.device:
        raise ValueError("q, k, v must share one dtype and device")
    _check_kv_heads(q, k, layout)
    o = torch.empty_like(q) if out is None else _check_buf(out, q.shape, q.dtype, q.device, "out")
    l = (torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if lse is None
         else _check_buf(lse, (B, H, Nq), torch.float32, q.device, "lse"))
    if ws is None:
        n = fa_fwd_splitkv_workspace_bytes(B, H, Nq, Nk, d, num_splits)
        ws = torch.empty(max(n, 256), dtype=torch.uint8, device=q.device)
    else:
        _check_ws(ws, q.device)
    st = fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), l.data_ptr(), B, H, Nq, Nk,
                        d, causal, scale, num_splits, ws.data_ptr(), ws.numel(), _stream(stream),
                        _dtype_code(q), layout)
    if st != FA_OK:
        raise FAError(st, "fa_fwd_splitkv")
    return o, l


def forward_fp8(q8, k8, v8, descale_q: float, descale_k: float, descale_v: float, causal: bool, scale: float,
                out=None, lse=None, stream=None, layout: int = FA_LAYOUT_BHND):
    """O (bf16), LSE for e4m3fn codes q8, k8, v8 (uint8 device tensors of one
    shape, [B,H,N,d] or [B,N,H,d]) standing for descale * code."""
    import torch
    B, H, N, d = _dims(q8, layout)
    _check((q8, k8, v8), q8.shape)
    if q8.dtype != torch.uint8:
        raise TypeError("FP8 inputs are passed as uint8 e4m3fn codes")
    o = (torch.empty(q8.shape, dtype=torch.bfloat16, device=q8.device) if out is None
         else _check_buf(out, q8.shape, torch.bfloat16, q8.device, "out"))
    l = (torch.empty((B, H, N), dtype=torch.float32, device=q8.device) if lse is None
         else _check_buf(lse, (B, H, N), torch.float32, q8.device, "lse"))
    st = fa_fwd_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), o.data_ptr(), l.data_ptr(), B, H, N, d, causal,
                    scale, descale_q, descale_k, descale_v, _stream(stream), layout)
    if st != FA_OK:
        raise FAError(st, "fa_fwd_fp8")
    return o, l


def forward_splitkv_fp8(q8, k8, v8, descale_q: float, descale_k: float, descale_v: float, causal: bool,
                        scale: float, num_splits: int = 0, out=None, lse=None, ws=None, stream=None,
                        layout: int = FA_LAYOUT_BHND):
    """O (bf16), LSE for e4m3fn codes q8 [B,H,Nq,d] against k8, v8 [B,H,Nk,d]
    (uint8 device tensors; [B,Nq,H,d] / [B,Nk,H,d] with FA_LAYOUT_BNHD)
    through the split-key-range FP8 forward."""
    import torch
    B, H, Nq, d = _dims(q8, layout)
    Nk = _dims(k8, layout)[2]
    _check((q8,), q8.shape)
    _check((k8, v8), k8.shape)
    if q8.dtype != torch.uint8 or k8.dtype != torch.uint8:
        raise TypeError("FP8 inputs are passed as uint8 e4m3fn codes")
    if k8.device != q8.device:
        raise ValueError("q8, k8, v8 must share one device")
    _check_kv_heads(q8, k8, layout, "k8, v8")
    o = (torch.empty(q8.shape, dtype=torch.bfloat16, device=q8.device) if out is None
         else _check_buf(out, q8.shape, torch.bfloat16, q8.device, "out"))
    l = (torch.empty((B, H, Nq), dtype=torch.float32, device=q8.device) if lse is None
         else _check_buf(lse, (B, H, Nq), torch.float32, q8.device, "lse"))
    if ws is None:
        n = fa_fwd_splitkv_fp8_workspace_bytes(B, H, Nq, Nk, d, num_splits)
        ws = torch.empty(max(n, 256), dtype=torch.uint8, device=q8.device)
    else:
        _check_ws(ws, q8.device)
    st = fa_fwd_splitkv_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), o.data_ptr(), l.data_ptr(), B, H, Nq,
                            Nk, d, causal, scale, descale_q, descale_k, descale_v, num_splits, ws.data_ptr(),
                            ws.numel(), _stream(stream), layout)
    if st != FA_OK:
        raise FAError(st, "fa_fwd_splitkv_fp8")
    return o, l


def drop_threshold(p: float) -> int:
    """The integer threshold t of the dropout entry points for a drop
    probability p: t = round(256 p), so that t / 256 is the probability
    actually used (0 <= p < 255.5 / 256)."""
    t = int(round(256.0 * float(p)))
    if not 0 <= t <= 255:
        raise ValueError(f"drop probability {p} outside [0, 255/256]")
    return t


def forward_dropout(q, k, v, causal: bool, scale: float, p_drop: float, seed: int, offset: int = 0, out=None,
                    lse=None, stream=None, layout: int = FA_LAYOUT_BHND):
    """O, LSE of attention with dropout (drop probability round(256 p)/256,
    mask from (seed, offset)) on bf16 device tensors in the named layout."""
    import torch
    B, H, N, d = _dims(q, layout)
    _check((q, k, v), q.shape)
    o = torch.empty_like(q) if out is None else _check_buf(out, q.shape, q.dtype, q.device, "out")
    l = (torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None
         else _check_buf(lse, (B, H, N), torch.float32, q.device, "lse"))
    st = fa_fwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), l.data_ptr(), B, H, N, d, causal,
                        scale, drop_threshold(p_drop), seed, offset, _stream(stream), layout)
    if st != FA_OK:
        raise FAError(st, "fa_fwd_dropout")
    return o, l


def backward_dropout(q, k, v, o, do, lse, causal: bool, scale: float, p_drop: float, seed: int, offset: int = 0,
                     ws=None, grads=None, stream=None, layout: int = FA_LAYOUT_BHND, method: int = FA_DQ_HANDOFF):
    """dQ, dK, dV for the O, LSE of forward_dropout with the same arguments."""
    import torch
    B, H, N, d = _dims(q, layout)
    _check((q, k, v, o, do), q.shape)
    _check_buf(lse, (B, H, N), torch.float32, q.device, "lse")
    ws = workspace(q, layout, causal, method) if ws is None else _check_ws(ws, q.device)
    if grads is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    else:
        dq, dk, dv = (_check_buf(g, q.shape, q.dtype, q.device, n) for g, n in zip(grads, ("dq", "dk", "dv")))
    st = fa_bwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, causal, scale,
                        drop_threshold(p_drop), seed, offset, ws.data_ptr(), ws.numel(), _stream(stream), layout)
    if st != FA_OK:
        raise FAError(st, "fa_bwd_dropout")
    return dq, dk, dv
