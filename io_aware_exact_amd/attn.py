"""Python binding of the C ABI in include/attn.h (ctypes; marshalling only).

Every step of the computation runs in the HIP kernels of ``libattn.so``.
PyTorch provides device memory and the current stream.  There is no fallback:
if the library is missing or a tensor is not on a GPU, the call raises.

Each call runs on q's device and that device's current stream.  Every other
tensor (outputs and workspace included) must be on the same device, and
outputs given by the caller must have exactly the shape the call writes.
"""

from __future__ import annotations

import ctypes
import math
import os

import torch

ATTN_OK = 0
ATTN_EINVAL = -1
ATTN_EUNSUPPORTED = -2
ATTN_EHIP = -3
ATTN_EWORKSPACE = -4

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")

# name -> (restype, argtypes), in the order of include/attn.h
_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_S = ctypes.c_size_t
SIGNATURES = {
    "attn_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P]),
    "attn_fwd_split_workspace_bytes": (_S, [_I, _I, _I, _I, _I, _I, _I]),
    "attn_fwd_split": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _P, _S, _P]),
    "attn_fwd_f32": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P]),
    "attn_decode_workspace_bytes": (_S, [_I, _I, _I, _I]),
    "attn_decode_splits": (_I, [_I, _I, _I, _I, _I]),
    "attn_decode": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P, _S, _P]),
    "attn_decode_gqa": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P, _S, _P]),
    "attn_decode_noalloc": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P]),
    "attn_decode_noalloc_max_bytes": (_S, []),
    "attn_bwd_workspace_bytes": (_S, [_I, _I, _I]),
    "attn_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P, _S, _P]),
    "attn_last_kernel": (ctypes.c_char_p, []),
    "attn_status_string": (ctypes.c_char_p, [_I]),
}

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"attn status {status}: {detail}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libattn.so (built in-tree) and declare its signatures."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build the HIP extension first "
                "(python -m io_aware_exact_amd.build, or __graft_entry__.build())")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(status: int) -> None:
    if status == ATTN_OK:
        return
    detail = lib().attn_status_string(status).decode()
    if status in (ATTN_EINVAL, ATTN_EWORKSPACE):
        raise ValueError(f"attn status {status}: {detail}")
    if status == ATTN_EUNSUPPORTED:
        raise NotImplementedError(f"attn status {status}: {detail}")
    raise AttnError(status, detail)


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _dev(t: torch.Tensor, name: str, dtype, device=None, shape=None) -> int:
    """Device pointer of ``t`` after checking its type, place, dtype, layout
    and (when given) its device and exact shape."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (the attention path has no CPU fallback)")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}; the call's tensors are on {device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _gpu(q) -> torch.device:
    """The device every tensor of the call must be on (q's)."""
    _dev(q, "q", None)
    return q.device


def _shape4(q, k, v):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, T, d]")
    B, H, Tq, d = q.shape
    if k.shape[0] != B or k.shape[1] != H or k.shape[3] != d or v.shape != k.shape:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    return B, H, Tq, k.shape[2], d


def _qkvo(q, k, v, o, dtype, dev):
    return [_dev(q, "q", dtype, dev), _dev(k, "k", dtype, dev), _dev(v, "v", dtype, dev),
            _dev(o, "o", dtype, dev, q.shape)]


def _lse_ptr(lse, shape, dev):
    return None if lse is None else _dev(lse, "lse", torch.float32, dev, shape)


def _ws_ptr(workspace, dev):
    if workspace is None:
        return None, 0
    return _dev(workspace, "workspace", None, dev), workspace.numel() * workspace.element_size()


def attn_fwd(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None,
             return_lse: bool = True):
    """bf16 attention forward; q [B,H,Tq,d], k/v [B,H,Tkv,d] -> (o, lse)."""
    B, H, Tq, Tkv, d = _shape4(q, k, v)
    dev = _gpu(q)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else out
    if return_lse and lse is None:
        lse = torch.empty((B, H, Tq), dtype=torch.float32, device=dev)
    lp = _lse_ptr(lse, (B, H, Tq), dev) if return_lse else None
    ptrs = _qkvo(q, k, v, o, torch.bfloat16, dev)
    with torch.cuda.device(dev):
        st = lib().attn_fwd(*ptrs, lp, B, H, Tq, Tkv, d, int(bool(causal)), scale, _stream(dev))
    _check(st)
    return (o, lse) if return_lse else o


def attn_fwd_split_workspace_bytes(B: int, H: int, Tq: int, Tkv: int, d: int, causal: bool,
                                   kv_chunk: int = 0) -> int:
    return int(lib().attn_fwd_split_workspace_bytes(B, H, Tq, Tkv, d, int(bool(causal)), int(kv_chunk)))


def _workspace(workspace, need: int, device):
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    return _ws_ptr(workspace, device)


def attn_fwd_split(q, k, v, causal: bool = False, scale: float | None = None, kv_chunk: int = 0, workspace=None,
                   out=None, lse=None, return_lse: bool = True):
    """bf16 forward with long query tiles split over the key axis (see
    include/attn.h); ``workspace`` (a GPU tensor) is allocated when needed and
    not given."""
    B, H, Tq, Tkv, d = _shape4(q, k, v)
    dev = _gpu(q)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else out
    if return_lse and lse is None:
        lse = torch.empty((B, H, Tq), dtype=torch.float32, device=dev)
    lp = _lse_ptr(lse, (B, H, Tq), dev) if return_lse else None
    ptrs = _qkvo(q, k, v, o, torch.bfloat16, dev)
    wp, wbytes = _workspace(workspace, attn_fwd_split_workspace_bytes(B, H, Tq, Tkv, d, causal, kv_chunk), dev)
    with torch.cuda.device(dev):
        st = lib().attn_fwd_split(*ptrs, lp, B, H, Tq, Tkv, d, int(bool(causal)), scale, int(kv_chunk), wp, wbytes,
                                  _stream(dev))
    _check(st)
    return (o, lse) if return_lse else o


def attn_fwd_f32(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None,
                 return_lse: bool = True):
    """fp32 attention forward (exact path); same contract as attn_fwd."""
    B, H, Tq, Tkv, d = _shape4(q, k, v)
    dev = _gpu(q)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else out
    if return_lse and lse is None:
        lse = torch.empty((B, H, Tq), dtype=torch.float32, device=dev)
    lp = _lse_ptr(lse, (B, H, Tq), dev) if return_lse else None
    ptrs = _qkvo(q, k, v, o, torch.float32, dev)
    with torch.cuda.device(dev):
        st = lib().attn_fwd_f32(*ptrs, lp, B, H, Tq, Tkv, d, int(bool(causal)), scale, _stream(dev))
    _check(st)
    return (o, lse) if return_lse else o


def attn_decode_workspace_bytes(B: int, H: int, d: int, num_splits: int) -> int:
    return int(lib().attn_decode_workspace_bytes(B, H, d, num_splits))


def _shape_gqa(q, k, v):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, T, d]")
    B, Hq, Tq, d = q.shape
    Hkv = k.shape[1]
    if k.shape[0] != B or k.shape[3] != d or v.shape != k.shape:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if Tq != 1:
        raise ValueError("decode takes exactly one query per (batch, head)")
    return B, Hq, Hkv, k.shape[2], d


def attn_decode_splits(B: int, Hq: int, Hkv: int, Tkv: int, d: int) -> int:
    return int(lib().attn_decode_splits(B, Hq, Hkv, Tkv, d))


def _resolve_splits(num_splits: int, B: int, Hq: int, Hkv: int, Tkv: int, d: int) -> int:
    """The partition count the library will use (0 = its automatic choice)."""
    n = int(num_splits)
    if n == 0:
        n = attn_decode_splits(B, Hq, Hkv, Tkv, d)
    return max(1, min(n, Tkv))


def attn_decode(q, k, v, scale: float | None = None, num_splits: int = 16, workspace=None, out=None, lse=None,
                return_lse: bool = True):
    """One query per (batch, head): q [B,H,1,d], k/v [B,H,Tkv,d] -> (o, lse [B,H]).

    ``num_splits`` = 0 lets the library choose (attn_decode_splits);
    ``workspace`` (a uint8 GPU tensor) is allocated when not given.
    """
    B, H, Hkv, Tkv, d = _shape_gqa(q, k, v)
    if Hkv != H:
        raise ValueError(f"attn_decode needs as many key/value heads as query heads ({Hkv} != {H}); "
                         "use attn_decode_gqa")
    dev = _gpu(q)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else out
    if return_lse and lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    lp = _lse_ptr(lse, (B, H), dev) if return_lse else None
    ptrs = _qkvo(q, k, v, o, torch.bfloat16, dev)
    splits = _resolve_splits(num_splits, B, H, H, Tkv, d)
    wp, wbytes = _workspace(workspace, attn_decode_workspace_bytes(B, H, d, splits), dev)
    with torch.cuda.device(dev):
        st = lib().attn_decode(*ptrs, lp, B, H, Tkv, d, scale, int(num_splits), wp, wbytes, _stream(dev))
    _check(st)
    return (o, lse) if return_lse else o


def attn_decode_gqa(q, k, v, scale: float | None = None, num_splits: int = 16, workspace=None, out=None,
                    lse=None, return_lse: bool = True):
    """Grouped-query decode: q [B,Hq,1,d], k/v [B,Hkv,Tkv,d] with Hq % Hkv == 0
    -> (o [B,Hq,1,d], lse [B,Hq]); query head h reads key/value head h // (Hq/Hkv)."""
    B, Hq, Hkv, Tkv, d = _shape_gqa(q, k, v)
    dev = _gpu(q)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else out
    if return_lse and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    lp = _lse_ptr(lse, (B, Hq), dev) if return_lse else None
    ptrs = _qkvo(q, k, v, o, torch.bfloat16, dev)
    splits = _resolve_splits(num_splits, B, Hq, Hkv, Tkv, d)
    wp, wbytes = _workspace(workspace, attn_decode_workspace_bytes(B, Hq, d, splits), dev)
    with torch.cuda.device(dev):
        st = lib().attn_decode_gqa(*ptrs, lp, B, Hq, Hkv, Tkv, d, scale, int(num_splits), wp, wbytes, _stream(dev))
    _check(st)
    return (o, lse) if return_lse else o


def attn_decode_noalloc_max_bytes() -> int:
    return int(lib().attn_decode_noalloc_max_bytes())


def attn_decode_noalloc(q, k, v, o, lse=None, scale: float | None = None, num_splits: int = 16):
    """attn_decode_gqa writing its partials to the library's per-device
    scratch instead of a workspace: nothing is allocated, here or in the
    library, so the caller passes the outputs ``o`` [B,Hq,1,d] and
    (optionally) ``lse`` [B,Hq].  Calls on one device must not overlap."""
    B, Hq, Hkv, Tkv, d = _shape_gqa(q, k, v)
    dev = _gpu(q)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    lp = _lse_ptr(lse, (B, Hq), dev)
    ptrs = _qkvo(q, k, v, o, torch.bfloat16, dev)
    with torch.cuda.device(dev):
        st = lib().attn_decode_noalloc(*ptrs, lp, B, Hq, Hkv, Tkv, d, scale, int(num_splits), _stream(dev))
    _check(st)
    return o, lse


def attn_bwd_workspace_bytes(B: int, H: int, Tq: int) -> int:
    return int(lib().attn_bwd_workspace_bytes(B, H, Tq))


def _bwd_ptrs(q, k, v, o, lse, dout, dq, dk, dv, dev):
    B, H, Tq = q.shape[:3]
    bf, f32 = torch.bfloat16, torch.float32
    return [_dev(q, "q", bf, dev), _dev(k, "k", bf, dev), _dev(v, "v", bf, dev), _dev(o, "o", bf, dev, q.shape),
            _dev(dout, "dout", bf, dev, q.shape), _dev(lse, "lse", f32, dev, (B, H, Tq)),
            _dev(dq, "dq", f32, dev, q.shape), _dev(dk, "dk", f32, dev, k.shape), _dev(dv, "dv", f32, dev, v.shape)]


def attn_bwd(q, k, v, o, lse, dout, causal: bool = False, scale: float | None = None, workspace=None,
             dq=None, dk=None, dv=None):
    """Backward of attn_fwd: (dq, dk, dv) fp32 from the forward's inputs, its
    output ``o`` and LSE, and the upstream gradient ``dout`` (bf16)."""
    B, H, Tq, Tkv, d = _shape4(q, k, v)
    dev = _gpu(q)
    if lse is None:
        raise ValueError("lse [B, H, Tq] is required")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dq = torch.empty(q.shape, dtype=torch.float32, device=dev) if dq is None else dq
    dk = torch.empty(k.shape, dtype=torch.float32, device=dev) if dk is None else dk
    dv = torch.empty(v.shape, dtype=torch.float32, device=dev) if dv is None else dv
    ptrs = _bwd_ptrs(q, k, v, o, lse, dout, dq, dk, dv, dev)
    wp, wbytes = _workspace(workspace, attn_bwd_workspace_bytes(B, H, Tq), dev)
    with torch.cuda.device(dev):
        st = lib().attn_bwd(*ptrs, B, H, Tq, Tkv, d, int(bool(causal)), scale, wp, wbytes, _stream(dev))
    _check(st)
    return dq, dk, dv


def _prepared(fn, args, dev):
    """A zero-argument callable running fn(*args); it refuses to run while
    another device than ``dev`` is current, since the library launches on the
    current device."""
    index = dev.index

    def call():
        if torch.cuda.current_device() != index:
            raise RuntimeError(f"prepared call for {dev} run while cuda:{torch.cuda.current_device()} is current")
        _check(fn(*args))

    return call


def prepared_bwd(q, k, v, o, lse, dout, dq, dk, dv, causal: bool, workspace, scale: float | None = None):
    """Zero-argument callable enqueuing attn_bwd; see prepared_fwd."""
    B, H, Tq, Tkv, d = _shape4(q, k, v)
    dev = _gpu(q)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    ptrs = _bwd_ptrs(q, k, v, o, lse, dout, dq, dk, dv, dev)
    wp, wb = _ws_ptr(workspace, dev)
    args = (*ptrs, B, H, Tq, Tkv, d, int(bool(causal)), scale, wp, wb, _stream(dev))
    return _prepared(lib().attn_bwd, args, dev)


def attn_last_kernel() -> str:
    return lib().attn_last_kernel().decode()


def attn_status_string(status: int) -> str:
    return lib().attn_status_string(int(status)).decode()


def prepared_fwd(q, k, v, o, lse, causal: bool, scale: float | None = None, f32: bool = False,
                 kv_chunk: int | None = None, workspace=None):
    """A zero-argument callable that enqueues attn_fwd (or attn_fwd_f32, or
    attn_fwd_split when ``kv_chunk`` is given) with these tensors, on the
    stream current on q's device now; argument checks happen once here, so
    repeated launches (benchmark loops) cost only the C call.  Run it while
    q's device is current."""
    B, H, Tq, Tkv, d = _shape4(q, k, v)
    dev = _gpu(q)
    dt = torch.float32 if f32 else torch.bfloat16
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    ptrs = _qkvo(q, k, v, o, dt, dev)
    lp = _lse_ptr(lse, (B, H, Tq), dev)
    stream = _stream(dev)
    if kv_chunk is not None:
        if f32:
            raise ValueError("the split forward is bf16")
        wp, wb = _ws_ptr(workspace, dev)
        fn = lib().attn_fwd_split
        args = (*ptrs, lp, B, H, Tq, Tkv, d, int(bool(causal)), scale, int(kv_chunk), wp, wb, stream)
    else:
        fn = lib().attn_fwd_f32 if f32 else lib().attn_fwd
        args = (*ptrs, lp, B, H, Tq, Tkv, d, int(bool(causal)), scale, stream)
    return _prepared(fn, args, dev)


def prepared_decode(q, k, v, o, lse, num_splits: int, workspace, scale: float | None = None):
    """Zero-argument callable enqueuing attn_decode (or attn_decode_gqa when k
    and v have fewer heads than q); see prepared_fwd."""
    B, Hq, Hkv, Tkv, d = _shape_gqa(q, k, v)
    dev = _gpu(q)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    ptrs = _qkvo(q, k, v, o, torch.bfloat16, dev)
    lp = _lse_ptr(lse, (B, Hq), dev)
    wp, wb = _ws_ptr(workspace, dev)
    if Hkv == Hq:
        fn = lib().attn_decode
        args = (*ptrs, lp, B, Hq, Tkv, d, scale, int(num_splits), wp, wb, _stream(dev))
    else:
        fn = lib().attn_decode_gqa
        args = (*ptrs, lp, B, Hq, Hkv, Tkv, d, scale, int(num_splits), wp, wb, _stream(dev))
    return _prepared(fn, args, dev)
