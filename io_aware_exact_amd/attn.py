"""Python binding of the C ABI in include/attn.h (ctypes; marshalling only).

Every step of the computation runs in the HIP kernels of ``libattn.so``.
PyTorch provides device memory and the current stream.  There is no fallback:
if the library is missing or a tensor is not on a GPU, the call raises.
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


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dev(t: torch.Tensor, name: str, dtype) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (the attention path has no CPU fallback)")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _shape4(q, k, v):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, T, d]")
    B, H, Tq, d = q.shape
    if k.shape[0] != B or k.shape[1] != H or k.shape[3] != d or v.shape != k.shape:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    return B, H, Tq, k.shape[2], d


def attn_fwd(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None,
             return_lse: bool = True):
    """bf16 attention forward; q [B,H,Tq,d], k/v [B,H,Tkv,d] -> (o, lse)."""
    B, H, Tq, Tkv, d = _shape4(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else out
    if return_lse and lse is None:
        lse = torch.empty((B, H, Tq), dtype=torch.float32, device=q.device)
    lp = _dev(lse, "lse", torch.float32) if return_lse else None
    st = lib().attn_fwd(_dev(q, "q", torch.bfloat16), _dev(k, "k", torch.bfloat16), _dev(v, "v", torch.bfloat16),
                        _dev(o, "o", torch.bfloat16), lp, B, H, Tq, Tkv, d, int(bool(causal)), scale, _stream())
    _check(st)
    return (o, lse) if return_lse else o


def attn_fwd_split_workspace_bytes(B: int, H: int, Tq: int, Tkv: int, d: int, causal: bool,
                                   kv_chunk: int = 0) -> int:
    return int(lib().attn_fwd_split_workspace_bytes(B, H, Tq, Tkv, d, int(bool(causal)), int(kv_chunk)))


def attn_fwd_split(q, k, v, causal: bool = False, scale: float | None = None, kv_chunk: int = 0, workspace=None,
                   out=None, lse=None, return_lse: bool = True):
    """bf16 forward with long query tiles split over the key axis (see
    include/attn.h); ``workspace`` (a GPU tensor) is allocated when needed and
    not given."""
    B, H, Tq, Tkv, d = _shape4(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else out
    if return_lse and lse is None:
        lse = torch.empty((B, H, Tq), dtype=torch.float32, device=q.device)
    lp = _dev(lse, "lse", torch.float32) if return_lse else None
    wp, wbytes = _workspace(workspace, attn_fwd_split_workspace_bytes(B, H, Tq, Tkv, d, causal, kv_chunk),
                            q.device)
    st = lib().attn_fwd_split(_dev(q, "q", torch.bfloat16), _dev(k, "k", torch.bfloat16),
                              _dev(v, "v", torch.bfloat16), _dev(o, "o", torch.bfloat16), lp, B, H, Tq, Tkv, d,
                              int(bool(causal)), scale, int(kv_chunk), wp, wbytes, _stream())
    _check(st)
    return (o, lse) if return_lse else o


def attn_fwd_f32(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None,
                 return_lse: bool = True):
    """fp32 attention forward (exact path); same contract as attn_fwd."""
    B, H, Tq, Tkv, d = _shape4(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else out
    if return_lse and lse is None:
        lse = torch.empty((B, H, Tq), dtype=torch.float32, device=q.device)
    lp = _dev(lse, "lse", torch.float32) if return_lse else None
    st = lib().attn_fwd_f32(_dev(q, "q", torch.float32), _dev(k, "k", torch.float32), _dev(v, "v", torch.float32),
                            _dev(o, "o", torch.float32), lp, B, H, Tq, Tkv, d, int(bool(causal)), scale, _stream())
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


def _workspace(workspace, need: int, device):
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    if workspace is None:
        return None, 0
    return _dev(workspace, "workspace", workspace.dtype), workspace.numel() * workspace.element_size()


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
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else out
    if return_lse and lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    lp = _dev(lse, "lse", torch.float32) if return_lse else None
    splits = _resolve_splits(num_splits, B, H, H, Tkv, d)
    wp, wbytes = _workspace(workspace, attn_decode_workspace_bytes(B, H, d, splits), q.device)
    st = lib().attn_decode(_dev(q, "q", torch.bfloat16), _dev(k, "k", torch.bfloat16), _dev(v, "v", torch.bfloat16),
                           _dev(o, "o", torch.bfloat16), lp, B, H, Tkv, d, scale, int(num_splits), wp, wbytes,
                           _stream())
    _check(st)
    return (o, lse) if return_lse else o


def attn_decode_gqa(q, k, v, scale: float | None = None, num_splits: int = 16, workspace=None, out=None,
                    lse=None, return_lse: bool = True):
    """Grouped-query decode: q [B,Hq,1,d], k/v [B,Hkv,Tkv,d] with Hq % Hkv == 0
    -> (o [B,Hq,1,d], lse [B,Hq]); query head h reads key/value head h // (Hq/Hkv)."""
    B, Hq, Hkv, Tkv, d = _shape_gqa(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else out
    if return_lse and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    lp = _dev(lse, "lse", torch.float32) if return_lse else None
    splits = _resolve_splits(num_splits, B, Hq, Hkv, Tkv, d)
    wp, wbytes = _workspace(workspace, attn_decode_workspace_bytes(B, Hq, d, splits), q.device)
    st = lib().attn_decode_gqa(_dev(q, "q", torch.bfloat16), _dev(k, "k", torch.bfloat16),
                               _dev(v, "v", torch.bfloat16), _dev(o, "o", torch.bfloat16), lp, B, Hq, Hkv, Tkv, d,
                               scale, int(num_splits), wp, wbytes, _stream())
    _check(st)
    return (o, lse) if return_lse else o


def attn_bwd_workspace_bytes(B: int, H: int, Tq: int) -> int:
    return int(lib().attn_bwd_workspace_bytes(B, H, Tq))


def attn_bwd(q, k, v, o, lse, dout, causal: bool = False, scale: float | None = None, workspace=None,
             dq=None, dk=None, dv=None):
    """Backward of attn_fwd: (dq, dk, dv) fp32 from the forward's inputs, its
    output ``o`` and LSE, and the upstream gradient ``dout`` (bf16)."""
    B, H, Tq, Tkv, d = _shape4(q, k, v)
    if o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("o and dout must have q's shape")
    if lse is None or tuple(lse.shape) != (B, H, Tq):
        raise ValueError("lse [B, H, Tq] is required")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dq = torch.empty(q.shape, dtype=torch.float32, device=q.device) if dq is None else dq
    dk = torch.empty(k.shape, dtype=torch.float32, device=q.device) if dk is None else dk
    dv = torch.empty(v.shape, dtype=torch.float32, device=q.device) if dv is None else dv
    wp, wbytes = _workspace(workspace, attn_bwd_workspace_bytes(B, H, Tq), q.device)
    st = lib().attn_bwd(_dev(q, "q", torch.bfloat16), _dev(k, "k", torch.bfloat16), _dev(v, "v", torch.bfloat16),
                        _dev(o, "o", torch.bfloat16), _dev(dout, "dout", torch.bfloat16),
                        _dev(lse, "lse", torch.float32), _dev(dq, "dq", torch.float32),
                        _dev(dk, "dk", torch.float32), _dev(dv, "dv", torch.float32), B, H, Tq, Tkv, d,
                        int(bool(causal)), scale, wp, wbytes, _stream())
    _check(st)
    return dq, dk, dv


def prepared_bwd(q, k, v, o, lse, dout, dq, dk, dv, causal: bool, workspace, scale: float | None = None):
    """Zero-argument callable enqueuing attn_bwd; see prepared_fwd."""
    B, H, Tq, Tkv, d = _shape4(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    ptrs = [_dev(t, n, torch.bfloat16) for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout"))]
    f32 = [_dev(t, n, torch.float32) for t, n in ((lse, "lse"), (dq, "dq"), (dk, "dk"), (dv, "dv"))]
    wp, wb = _dev(workspace, "workspace", workspace.dtype), workspace.numel() * workspace.element_size()
    fn = lib().attn_bwd
    args = (*ptrs, *f32, B, H, Tq, Tkv, d, int(bool(causal)), scale, wp, wb, _stream())

    def call():
        _check(fn(*args))

    return call


def attn_last_kernel() -> str:
    return lib().attn_last_kernel().decode()


def attn_status_string(status: int) -> str:
    return lib().attn_status_string(int(status)).decode()


def prepared_fwd(q, k, v, o, lse, causal: bool, scale: float | None = None, f32: bool = False,
                 kv_chunk: int | None = None, workspace=None):
    """A zero-argument callable that enqueues attn_fwd (or attn_fwd_f32, or
    attn_fwd_split when ``kv_chunk`` is given) on the current stream with these
    tensors; argument checks happen once here, so repeated launches
    (benchmark loops) cost only the C call."""
    B, H, Tq, Tkv, d = _shape4(q, k, v)
    dt = torch.float32 if f32 else torch.bfloat16
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    ptrs = [_dev(t, n, dt) for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"))]
    lp = None if lse is None else _dev(lse, "lse", torch.float32)
    stream = _stream()
    if kv_chunk is not None:
        if f32:
            raise ValueError("the split forward is bf16")
        wp, wb = (None, 0) if workspace is None else (_dev(workspace, "workspace", workspace.dtype),
                                                      workspace.numel() * workspace.element_size())
        fn = lib().attn_fwd_split
        args = (*ptrs, lp, B, H, Tq, Tkv, d, int(bool(causal)), scale, int(kv_chunk), wp, wb, stream)
    else:
        fn = lib().attn_fwd_f32 if f32 else lib().attn_fwd
        args = (*ptrs, lp, B, H, Tq, Tkv, d, int(bool(causal)), scale, stream)

    def call():
        _check(fn(*args))

    return call


def prepared_decode(q, k, v, o, lse, num_splits: int, workspace, scale: float | None = None):
    """Zero-argument callable enqueuing attn_decode (or attn_decode_gqa when k
    and v have fewer heads than q); see prepared_fwd."""
    B, Hq, Hkv, Tkv, d = _shape_gqa(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    ptrs = [_dev(t, n, torch.bfloat16) for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"))]
    lp = None if lse is None else _dev(lse, "lse", torch.float32)
    wp, wb = (None, 0) if workspace is None else (_dev(workspace, "workspace", workspace.dtype),
                                                  workspace.numel() * workspace.element_size())
    if Hkv == Hq:
        fn = lib().attn_decode
        args = (*ptrs, lp, B, Hq, Tkv, d, scale, int(num_splits), wp, wb, _stream())
    else:
        fn = lib().attn_decode_gqa
        args = (*ptrs, lp, B, Hq, Hkv, Tkv, d, scale, int(num_splits), wp, wb, _stream())

    def call():
        _check(fn(*args))

    return call
