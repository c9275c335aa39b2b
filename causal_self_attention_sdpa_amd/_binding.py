"""ctypes marshalling for libgattn.so.  No computation happens here."""
from __future__ import annotations

import ctypes
import math
import os

PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(PKG, "libgattn.so")

F32 = 0
BF16 = 1
F16 = 2
_STATUS = {0: "GATTN_OK", 1: "GATTN_ERR_INVALID_ARG", 2: "GATTN_ERR_UNSUPPORTED",
           3: "GATTN_ERR_WORKSPACE", 4: "GATTN_ERR_HIP"}

_lib = None


class GattnError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what} failed: {_STATUS.get(status, status)}")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Loads libgattn.so (building it first only if it has never been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build
        _build.build()
    # torch's HIP runtime must be in the process before libgattn.so: the library
    # asks for libamdhip64.so.7, which then resolves to torch's copy (same
    # soname).  Loaded the other way round, the library would bring in the
    # system runtime and torch a second one of its own, and torch's streams and
    # allocations would not be valid in the runtime the library launches on.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.gattn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
    lib.gattn_fwd.restype = i
    lib.gattn_bwd_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.gattn_bwd_workspace_bytes.restype = sz
    lib.gattn_bwd.argtypes = [vp] * 9 + [i, i, i, i, f, i, vp, sz, vp]
    lib.gattn_bwd.restype = i
    lib.gattn_bwd_noalloc.argtypes = [vp] * 9 + [i, i, i, i, f, i, vp]
    lib.gattn_bwd_noalloc.restype = i
    lib.gattn_bwd_noalloc_max_bytes.argtypes = []
    lib.gattn_bwd_noalloc_max_bytes.restype = sz
    lib.gattn_bwd_preprocess.argtypes = [vp, vp, vp, i, i, i, i, i, vp, sz, vp]
    lib.gattn_bwd_preprocess.restype = i
    lib.gattn_bwd_dq.argtypes = [vp] * 7 + [i, i, i, i, f, i, vp, sz, vp]
    lib.gattn_bwd_dq.restype = i
    lib.gattn_bwd_dkdv.argtypes = [vp] * 6 + [i, i, i, i, f, i, vp, sz, vp]
    lib.gattn_bwd_dkdv.restype = i
    lib.gattn_fwd_strided.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, vp, vp]
    lib.gattn_fwd_strided.restype = i
    lib.gattn_bwd_strided.argtypes = [vp] * 9 + [i, i, i, i, f, i, vp, sz, vp, vp, vp, vp]
    lib.gattn_bwd_strided.restype = i
    lib.gattn_fwd_decode_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.gattn_fwd_decode_workspace_bytes.restype = sz
    lib.gattn_fwd_decode.argtypes = [vp] * 5 + [i, i, i, i, i, f, i, vp, vp, vp, vp, sz, vp]
    lib.gattn_fwd_decode.restype = i
    u64, u32 = ctypes.c_uint64, ctypes.c_uint32
    lib.gattn_fwd_dropout.argtypes = [vp] * 5 + [i, i, i, i, f, i, f, u64, u32, vp, vp, vp, vp]
    lib.gattn_fwd_dropout.restype = i
    lib.gattn_bwd_dropout.argtypes = ([vp] * 9 + [i, i, i, i, f, i, f, u64, u32, vp, vp, sz]
                                      + [vp, vp, vp, vp])
    lib.gattn_dropout_keep_bytes.argtypes = [i, i, i]
    lib.gattn_dropout_keep_bytes.restype = sz
    lib.gattn_bwd_dropout.restype = i
    lib.gattn_bwd_dropout_workspace_bytes.argtypes = [i, i, i, i, i, f]
    lib.gattn_bwd_dropout_workspace_bytes.restype = sz
    lib.gattn_dropout_mask.argtypes = [vp, i, i, i, f, u64, u32, vp]
    lib.gattn_dropout_mask.restype = i
    lib.gattn_probe_mfma_bf16.argtypes = [vp, i, i, vp]
    lib.gattn_probe_mfma_bf16.restype = i
    lib.gattn_probe_issue.argtypes = [vp, i, i, i, i, i, vp]
    lib.gattn_probe_issue.restype = i
    lib.gattn_status_string.argtypes = [i]
    lib.gattn_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def gattn_status_string(status: int) -> str:
    return load_library().gattn_status_string(int(status)).decode()


def _check(status: int, what: str) -> None:
    if status != 0:
        raise GattnError(status, what)


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.float16:
        return F16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(t, name: str, shape=None, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _on(stream, *tensors):
    """The stream a call launches on: the given one, else the current stream of
    the device that holds the call's tensors (all of them on one device, and a
    given stream on that device too)."""
    torch = _torch()
    devs = {t.device for t in tensors if t is not None}
    if len(devs) != 1:
        raise ValueError("the tensors of one call must be on one device, got "
                         f"{sorted(map(str, devs))}")
    dev = devs.pop()
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    elif stream.device != dev:
        raise ValueError(f"stream is on {stream.device}, the tensors on {dev}")
    return ctypes.c_void_p(stream.cuda_stream)


def _shape4(q):
    if q.dim() != 4:
        raise ValueError("expected (B, H, T, hs) tensors")
    return tuple(int(x) for x in q.shape)


def gattn_bwd_workspace_bytes(B: int, H: int, T: int, hs: int, dtype: int) -> int:
    return int(load_library().gattn_bwd_workspace_bytes(B, H, T, hs, dtype))


def gattn_fwd(q, k, v, o, lse, scale: float, stream=None) -> None:
    """o, lse (lse may be None) <- causal attention of q, k, v on the stream."""
    lib = load_library()
    B, H, T, hs = _shape4(q)
    dt = _dtype_code(q)
    args = [_dev(x, n, q.shape, q.dtype) for x, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"))]
    lp = None if lse is None else _dev(lse, "lse", (B, H, T), _torch().float32)
    st = _on(stream, q, k, v, o, lse)
    _check(lib.gattn_fwd(*args, lp, B, H, T, hs, float(scale), dt, st), "gattn_fwd")


def gattn_bwd(q, k, v, o, dO, lse, dq, dk, dv, scale: float, workspace, stream=None) -> None:
    lib = load_library()
    B, H, T, hs = _shape4(q)
    dt = _dtype_code(q)
    ptrs = [_dev(x, n, q.shape, q.dtype) for x, n in
            ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dO, "dO"))]
    lp = _dev(lse, "lse", (B, H, T), _torch().float32)
    outs = [_dev(x, n, q.shape, q.dtype) for x, n in ((dq, "dq"), (dk, "dk"), (dv, "dv"))]
    ws = _dev(workspace, "workspace")
    nbytes = workspace.numel() * workspace.element_size()
    st = _on(stream, q, k, v, o, dO, lse, dq, dk, dv, workspace)
    _check(lib.gattn_bwd(*ptrs, lp, *outs, B, H, T, hs, float(scale), dt, ws, nbytes,
                         st), "gattn_bwd")


def gattn_bwd_noalloc(q, k, v, o, dO, lse, dq, dk, dv, scale: float, stream=None) -> None:
    """gattn_bwd with the library's static device scratch instead of a workspace."""
    lib = load_library()
    B, H, T, hs = _shape4(q)
    dt = _dtype_code(q)
    ptrs = [_dev(x, n, q.shape, q.dtype) for x, n in
            ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dO, "dO"))]
    lp = _dev(lse, "lse", (B, H, T), _torch().float32)
    outs = [_dev(x, n, q.shape, q.dtype) for x, n in ((dq, "dq"), (dk, "dk"), (dv, "dv"))]
    st = _on(stream, q, k, v, o, dO, lse, dq, dk, dv)
    with _torch().cuda.device(q.device):  # the scratch used is the current device's
        _check(lib.gattn_bwd_noalloc(*ptrs, lp, *outs, B, H, T, hs, float(scale), dt, st),
               "gattn_bwd_noalloc")


def gattn_bwd_noalloc_max_bytes() -> int:
    return int(load_library().gattn_bwd_noalloc_max_bytes())


def gattn_bwd_preprocess(o, dO, lse, workspace, stream=None) -> None:
    lib = load_library()
    B, H, T, hs = _shape4(o)
    st = _on(stream, o, dO, lse, workspace)
    _check(lib.gattn_bwd_preprocess(_dev(o, "o"), _dev(dO, "dO", o.shape, o.dtype),
                                    _dev(lse, "lse", (B, H, T), _torch().float32), B, H, T, hs,
                                    _dtype_code(o), _dev(workspace, "workspace"),
                                    workspace.numel() * workspace.element_size(), st),
           "gattn_bwd_preprocess")


def gattn_bwd_dq(q, k, v, o, dO, lse, dq, scale: float, workspace, stream=None) -> None:
    lib = load_library()
    B, H, T, hs = _shape4(q)
    ptrs = [_dev(x, n, q.shape, q.dtype) for x, n in
            ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dO, "dO"))]
    lp = _dev(lse, "lse", (B, H, T), _torch().float32)
    st = _on(stream, q, k, v, o, dO, lse, dq, workspace)
    _check(lib.gattn_bwd_dq(*ptrs, lp, _dev(dq, "dq", q.shape, q.dtype), B, H, T, hs,
                            float(scale), _dtype_code(q), _dev(workspace, "workspace"),
                            workspace.numel() * workspace.element_size(), st),
           "gattn_bwd_dq")


def gattn_bwd_dkdv(q, k, v, dO, dk, dv, scale: float, workspace, stream=None) -> None:
    lib = load_library()
    B, H, T, hs = _shape4(q)
    ptrs = [_dev(x, n, q.shape, q.dtype) for x, n in ((q, "q"), (k, "k"), (v, "v"), (dO, "dO"))]
    outs = [_dev(x, n, q.shape, q.dtype) for x, n in ((dk, "dk"), (dv, "dv"))]
    st = _on(stream, q, k, v, dO, dk, dv, workspace)
    _check(lib.gattn_bwd_dkdv(*ptrs, *outs, B, H, T, hs, float(scale), _dtype_code(q),
                              _dev(workspace, "workspace"),
                              workspace.numel() * workspace.element_size(), st),
           "gattn_bwd_dkdv")


def _view(t, name: str, shape, dtype):
    """Pointer and {batch, head, row} element strides of a (B, H, T, hs) view
    whose last dimension is contiguous."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.shape[3] != 1 and t.stride(3) != 1:
        raise ValueError(f"{name}: the head dimension must be contiguous")
    # The stride of a dimension of size 1 addresses nothing and torch leaves it
    # arbitrary (0 for a view built from a broadcast array); pass canonical
    # values so that views of one layout compare equal: the contiguous strides
    # for a contiguous tensor (the library's contiguous kernels then run),
    # else 0 for a batch or head dimension of size 1 and hs for one row.
    B, H, T, hs = (int(x) for x in t.shape)
    if t.is_contiguous():
        st = (H * T * hs, T * hs, hs)
    else:
        st = tuple(int(x) for x in t.stride()[:3])
        st = (0 if B == 1 else st[0], 0 if H == 1 else st[1], hs if T == 1 else st[2])
    return ctypes.c_void_p(t.data_ptr()), st


def _strides_arg(views, group: str):
    st = {v[1] for v in views}
    if len(st) != 1:
        raise ValueError(f"{group} must share one set of strides, got {sorted(st)}")
    return (ctypes.c_int64 * 3)(*st.pop())


def gattn_fwd_strided(q, k, v, o, lse, scale: float, stream=None) -> None:
    """As gattn_fwd for (B, H, T, hs) views with any strides (hs contiguous):
    q, k, v share one stride set, o has its own; lse is contiguous (B, H, T)."""
    lib = load_library()
    B, H, T, hs = _shape4(q)
    dt = _dtype_code(q)
    qkv = [_view(x, n, q.shape, q.dtype) for x, n in ((q, "q"), (k, "k"), (v, "v"))]
    ov = _view(o, "o", q.shape, q.dtype)
    lp = None if lse is None else _dev(lse, "lse", (B, H, T), _torch().float32)
    st = _on(stream, q, k, v, o, lse)
    _check(lib.gattn_fwd_strided(*(p for p, _ in qkv), ov[0], lp, B, H, T, hs, float(scale), dt,
                                 _strides_arg(qkv, "q, k, v"), _strides_arg([ov], "o"),
                                 st), "gattn_fwd_strided")


def gattn_bwd_strided(q, k, v, o, dO, lse, dq, dk, dv, scale: float, workspace,
                      stream=None) -> None:
    """As gattn_bwd for strided (B, H, T, hs) views: q, k, v share one stride
    set, o and dO another, dq, dk, dv a third."""
    lib = load_library()
    B, H, T, hs = _shape4(q)
    dt = _dtype_code(q)
    qkv = [_view(x, n, q.shape, q.dtype) for x, n in ((q, "q"), (k, "k"), (v, "v"))]
    od = [_view(x, n, q.shape, q.dtype) for x, n in ((o, "o"), (dO, "dO"))]
    gr = [_view(x, n, q.shape, q.dtype) for x, n in ((dq, "dq"), (dk, "dk"), (dv, "dv"))]
    lp = _dev(lse, "lse", (B, H, T), _torch().float32)
    ws = _dev(workspace, "workspace")
    nbytes = workspace.numel() * workspace.element_size()
    st = _on(stream, q, k, v, o, dO, lse, dq, dk, dv, workspace)
    _check(lib.gattn_bwd_strided(*(p for p, _ in qkv), *(p for p, _ in od), lp,
                                 *(p for p, _ in gr), B, H, T, hs, float(scale), dt, ws, nbytes,
                                 _strides_arg(qkv, "q, k, v"), _strides_arg(od, "o, dO"),
                                 _strides_arg(gr, "dq, dk, dv"), st),
           "gattn_bwd_strided")


def gattn_fwd_decode_workspace_bytes(B: int, H: int, Tq: int, Tk: int, hs: int,
                                     dtype: int) -> int:
    return int(load_library().gattn_fwd_decode_workspace_bytes(B, H, Tq, Tk, hs, dtype))


def gattn_fwd_decode(q, k, v, o, lse, scale: float, workspace=None, stream=None) -> None:
    """Forward of the newest Tq tokens: q, o (B, H, Tq, hs) and k, v (B, H, Tk,
    hs) views (hs contiguous; k and v share strides, e.g. the first Tk rows of
    a key/value cache), Tk >= Tq; query i sees keys j <= Tk - Tq + i.  lse
    (B, H, Tq) contiguous or None.  The 16-bit path needs a workspace of
    gattn_fwd_decode_workspace_bytes() bytes (allocated here if None)."""
    lib = load_library()
    B, H, Tq, hs = _shape4(q)
    Tk = int(k.shape[2])
    dt = _dtype_code(q)
    qv = _view(q, "q", q.shape, q.dtype)
    kvv = [_view(x, n, (B, H, Tk, hs), q.dtype) for x, n in ((k, "k"), (v, "v"))]
    ov = _view(o, "o", q.shape, q.dtype)
    lp = None if lse is None else _dev(lse, "lse", (B, H, Tq), _torch().float32)
    need = gattn_fwd_decode_workspace_bytes(B, H, Tq, Tk, hs, dt)
    if workspace is None and need > 0:
        workspace = _torch().empty(need, dtype=_torch().uint8, device=q.device)
    ws = None if workspace is None else _dev(workspace, "workspace")
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _on(stream, q, k, v, o, lse, workspace)
    _check(lib.gattn_fwd_decode(qv[0], kvv[0][0], kvv[1][0], ov[0], lp, B, H, Tq, Tk, hs,
                                float(scale), dt, _strides_arg([qv], "q"),
                                _strides_arg(kvv, "k, v"), _strides_arg([ov], "o"), ws, nbytes,
                                st), "gattn_fwd_decode")


def attention_decode(q, k, v, scale=None, need_lse: bool = False, workspace=None, stream=None):
    """Returns (o, lse) of the newest Tq tokens q (B, H, Tq, hs) against k, v
    (B, H, Tk, hs) views; lse is None unless asked for."""
    torch = _torch()
    B, H, Tq, hs = _shape4(q)
    o = torch.empty((B, H, Tq, hs), dtype=q.dtype, device=q.device)
    lse = torch.empty((B, H, Tq), dtype=torch.float32, device=q.device) if need_lse else None
    gattn_fwd_decode(q, k, v, o, lse, _default_scale(hs, scale), workspace, stream)
    return o, lse


def gattn_dropout_keep_bytes(B: int, H: int, T: int) -> int:
    return int(load_library().gattn_dropout_keep_bytes(B, H, T))


def _keep_arg(keep, B, H, T):
    if keep is None:
        return None
    need = gattn_dropout_keep_bytes(B, H, T)
    if keep.dtype != _torch().uint8 or not keep.is_contiguous() or keep.numel() < need:
        raise ValueError(f"keep: a contiguous uint8 device tensor of at least {need} bytes")
    return _dev(keep, "keep")


def gattn_fwd_dropout(q, k, v, o, lse, scale: float, p: float, seed: int, offset: int,
                      stream=None, keep=None) -> None:
    """As gattn_fwd_strided with attention dropout of probability p; the
    mask is drawn from (seed, offset) as the C header defines.  keep: None or
    a uint8 tensor of gattn_dropout_keep_bytes() bytes the 16-bit kernels
    store the keep decisions in, for gattn_bwd_dropout."""
    lib = load_library()
    B, H, T, hs = _shape4(q)
    dt = _dtype_code(q)
    qkv = [_view(x, n, q.shape, q.dtype) for x, n in ((q, "q"), (k, "k"), (v, "v"))]
    ov = _view(o, "o", q.shape, q.dtype)
    lp = None if lse is None else _dev(lse, "lse", (B, H, T), _torch().float32)
    st = _on(stream, q, k, v, o, lse, keep)
    _check(lib.gattn_fwd_dropout(*(x for x, _ in qkv), ov[0], lp, B, H, T, hs, float(scale), dt,
                                 float(p), int(seed), int(offset), _keep_arg(keep, B, H, T),
                                 _strides_arg(qkv, "q, k, v"), _strides_arg([ov], "o"),
                                 st), "gattn_fwd_dropout")


def gattn_bwd_dropout_workspace_bytes(B: int, H: int, T: int, hs: int, dtype: int,
                                      p: float) -> int:
    return int(load_library().gattn_bwd_dropout_workspace_bytes(B, H, T, hs, dtype, float(p)))


def gattn_bwd_dropout(q, k, v, o, dO, lse, dq, dk, dv, scale: float, p: float, seed: int,
                      offset: int, workspace, stream=None, keep=None) -> None:
    """Backward of gattn_fwd_dropout (same p, seed, offset); strided views as
    gattn_bwd_strided; keep: None or the keep tensor that forward filled."""
    lib = load_library()
    B, H, T, hs = _shape4(q)
    dt = _dtype_code(q)
    qkv = [_view(x, n, q.shape, q.dtype) for x, n in ((q, "q"), (k, "k"), (v, "v"))]
    od = [_view(x, n, q.shape, q.dtype) for x, n in ((o, "o"), (dO, "dO"))]
    gr = [_view(x, n, q.shape, q.dtype) for x, n in ((dq, "dq"), (dk, "dk"), (dv, "dv"))]
    lp = _dev(lse, "lse", (B, H, T), _torch().float32)
    ws = _dev(workspace, "workspace")
    nbytes = workspace.numel() * workspace.element_size()
    st = _on(stream, q, k, v, o, dO, lse, dq, dk, dv, workspace, keep)
    _check(lib.gattn_bwd_dropout(*(x for x, _ in qkv), *(x for x, _ in od), lp,
                                 *(x for x, _ in gr), B, H, T, hs, float(scale), dt, float(p),
                                 int(seed), int(offset), _keep_arg(keep, B, H, T), ws, nbytes,
                                 _strides_arg(qkv, "q, k, v"), _strides_arg(od, "o, dO"),
                                 _strides_arg(gr, "dq, dk, dv"), st),
           "gattn_bwd_dropout")


def gattn_dropout_mask(keep, B: int, H: int, T: int, p: float, seed: int, offset: int,
                       stream=None) -> None:
    """Writes the keep decisions (uint8, 1 = kept) into keep (B, H, T, T)."""
    torch = _torch()
    kp = _dev(keep, "keep", (B, H, T, T), torch.uint8)
    st = _on(stream, keep)
    _check(load_library().gattn_dropout_mask(kp, B, H, T, float(p), int(seed), int(offset),
                                             st), "gattn_dropout_mask")


def attention_forward_dropout(q, k, v, p: float, seed: int, offset: int = 0, scale=None,
                              need_lse: bool = True, stream=None, return_keep: bool = False):
    """Returns (o, lse) with attention dropout; lse is None if not needed.
    return_keep: also return the keep-decision bits the forward stored
    (uint8 tensor, for attention_backward_dropout), as (o, lse, keep)."""
    torch = _torch()
    B, H, T, hs = _shape4(q)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device) if need_lse else None
    keep = None
    if return_keep:
        keep = torch.empty(gattn_dropout_keep_bytes(B, H, T), dtype=torch.uint8, device=q.device)
    gattn_fwd_dropout(q, k, v, o, lse, _default_scale(hs, scale), p, seed, offset, stream, keep)
    return (o, lse, keep) if return_keep else (o, lse)


def attention_backward_dropout(q, k, v, o, dO, lse, p: float, seed: int, offset: int = 0,
                               scale=None, workspace=None, stream=None, keep=None):
    """Returns (dq, dk, dv) of attention_forward_dropout with the same p, seed,
    offset (and its keep bits if it returned them); allocates the workspace
    unless one is given."""
    torch = _torch()
    B, H, T, hs = _shape4(q)
    if workspace is None:
        n = (gattn_bwd_workspace_bytes(B, H, T, hs, _dtype_code(q)) if keep is not None
             else gattn_bwd_dropout_workspace_bytes(B, H, T, hs, _dtype_code(q), p))
        workspace = torch.empty(n, dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    gattn_bwd_dropout(q, k, v, o, dO, lse, dq, dk, dv, _default_scale(hs, scale), p, seed,
                      offset, workspace, stream, keep)
    return dq, dk, dv


def _qkv_views(qkv, n_head: int):
    """(B, H, T, hs) views of q, k, v inside a (B, T, 3C) projection output."""
    B, T, C3 = (int(x) for x in qkv.shape)
    if C3 % (3 * n_head):
        raise ValueError("last dimension must be 3 * n_head * hs")
    hs = C3 // (3 * n_head)
    v4 = qkv.view(B, T, 3, n_head, hs)
    return tuple(v4[:, :, j].transpose(1, 2) for j in range(3))


def attention_forward_qkv(qkv, n_head: int, scale=None, need_lse: bool = True, stream=None):
    """Causal attention of a GPT block straight from the fused projection
    output qkv (B, T, 3C), contiguous: returns y (B, T, C) (heads side by side,
    the layout the output projection reads) and lse (B, H, T) or None."""
    torch = _torch()
    if not qkv.is_contiguous():
        raise ValueError("qkv must be contiguous (B, T, 3C)")
    q, k, v = _qkv_views(qkv, n_head)
    B, H, T, hs = _shape4(q)
    y = torch.empty((B, T, H * hs), dtype=qkv.dtype, device=qkv.device)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=qkv.device) if need_lse else None
    gattn_fwd_strided(q, k, v, y.view(B, T, H, hs).transpose(1, 2), lse,
                      _default_scale(hs, scale), stream)
    return y, lse


def attention_backward_qkv(qkv, y, dy, lse, n_head: int, scale=None, workspace=None,
                           stream=None):
    """Gradient of attention_forward_qkv: from y and dy (B, T, C), returns
    dqkv (B, T, 3C), the gradient of the fused projection output."""
    torch = _torch()
    if not (qkv.is_contiguous() and y.is_contiguous() and dy.is_contiguous()):
        raise ValueError("qkv, y and dy must be contiguous")
    q, k, v = _qkv_views(qkv, n_head)
    B, H, T, hs = _shape4(q)
    if workspace is None:
        n = gattn_bwd_workspace_bytes(B, H, T, hs, _dtype_code(q))
        workspace = torch.empty(n, dtype=torch.uint8, device=qkv.device)
    dqkv = torch.empty_like(qkv)
    dq, dk, dv = _qkv_views(dqkv, n_head)
    o4 = y.view(B, T, H, hs).transpose(1, 2)
    do4 = dy.view(B, T, H, hs).transpose(1, 2)
    gattn_bwd_strided(q, k, v, o4, do4, lse, dq, dk, dv, _default_scale(hs, scale), workspace,
                      stream)
    return dqkv


def _default_scale(hs: int, scale):
    return 1.0 / math.sqrt(hs) if scale is None else float(scale)


def attention_forward(q, k, v, scale=None, need_lse: bool = True, stream=None):
    """Returns (o, lse) for (B, H, T, hs) device tensors; lse is None if not needed."""
    torch = _torch()
    B, H, T, hs = _shape4(q)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device) if need_lse else None
    gattn_fwd(q, k, v, o, lse, _default_scale(hs, scale), stream)
    return o, lse


def attention_backward(q, k, v, o, dO, lse, scale=None, workspace=None, stream=None):
    """Returns (dq, dk, dv); allocates the workspace unless one is given."""
    torch = _torch()
    B, H, T, hs = _shape4(q)
    if workspace is None:
        n = gattn_bwd_workspace_bytes(B, H, T, hs, _dtype_code(q))
        workspace = torch.empty(n, dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    gattn_bwd(q, k, v, o, dO, lse, dq, dk, dv, _default_scale(hs, scale), workspace, stream)
    return dq, dk, dv
