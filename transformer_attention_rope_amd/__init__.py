"""Python binding of libnc_attn.so, the MI355X (gfx950) attention-block forward.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/nc_attn.h``. Tensors must be
contiguous CUDA (HIP) tensors in bfloat16 or float32; work is enqueued on the
current torch stream of the tensors' device. There is no CPU fallback: if the
library is not built, or a tensor is not on the GPU, the call raises.

    rope_qknorm(q, k, rope_base=1e4, pos_offset=0)          -> (q', k')
    qkv_rope_qknorm(x, w_q, w_k, w_v, H=..., Hkv=...)        -> (q', k', v)
    attn_fwd(q, k, v, window=..., rope_base=1e4, pos_offset=0) -> o
    attn_fwd_lse(q, k, v, window=...) -> (o, lse)
    attn_fwd_normed(q', k', v, window=...) -> o      (q', k' already rotated, normalised)
    attn_bwd(q, k, v, o, dout, lse, window=...) -> (dq, dk, dv)
    attn_prep(k, ...) -> workspace;  attn_core(q, v, workspace, window=...) -> o
    attn_prefill(q, k, v, k_cache, v_cache, window=..., pos_offset=0, rope_base=1e4) -> o
    attn_decode(q, k_new, v_new, k_cache, v_cache, seqlens, window=..., rope_base=1e4) -> o
    attn_decode_shared(q, k_new, v_new, k_prompt, v_prompt, k_cache, v_cache, seqlens, window=...) -> o
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "NcError", "lib", "library_path", "rope_qknorm", "attn_fwd", "attn_fwd_lse", "attn_bwd",
    "attn_bwd_workspace_bytes", "attn_fwd_noalloc", "attn_fwd_normed", "attn_fwd_normed_workspace_bytes",
    "qkv_rope_qknorm", "qkv_rope_qknorm_workspace_bytes", "attn_prefill", "attn_decode",
    "attn_decode_shared", "attn_decode_shared_workspace_bytes",
    "attn_prep", "attn_core", "decode_workspace",
    "attn_fwd_workspace_bytes", "attn_prefill_workspace_bytes", "attn_decode_workspace_bytes",
    "rope_qknorm_workspace_bytes",
    "NC_OK", "NC_ERR_INVALID", "NC_ERR_UNSUPPORTED", "NC_ERR_HIP", "NC_BF16", "NC_F32",
]

NC_OK, NC_ERR_INVALID, NC_ERR_UNSUPPORTED, NC_ERR_HIP = 0, 1, 2, 3
NC_BF16, NC_F32 = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libnc_attn.so"
_lib = None

_vp, _i, _d, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_double, ctypes.c_size_t
_SIGS = {
    "nc_abi_version": (_i, []),
    "nc_status_string": (ctypes.c_char_p, [_i]),
    "nc_last_error": (ctypes.c_char_p, []),
    "nc_rope_qknorm_workspace_bytes": (_sz, [_i, _i, _i]),
    "nc_rope_qknorm": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _d, _i, _i, _vp, _sz, _vp]),
    "nc_attn_fwd_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "nc_attn_fwd": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _d, _i, _i, _vp, _sz, _vp]),
    "nc_attn_fwd_lse": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _d, _i, _i, _vp, _sz,
                             _vp]),
    "nc_attn_bwd_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "nc_qkv_rope_qknorm_workspace_bytes": (_sz, [_i, _i, _i]),
    "nc_qkv_rope_qknorm": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _d, _i, _i, _vp,
                                _sz, _vp]),
    "nc_attn_fwd_normed_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "nc_attn_fwd_normed": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp, _sz, _vp]),
    "nc_attn_fwd_noalloc": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _d, _i, _i, _vp]),
    "nc_attn_bwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _d, _i, _i,
                         _vp, _sz, _vp]),
    "nc_attn_prep": (_i, [_vp, _i, _i, _i, _i, _d, _i, _i, _vp, _sz, _vp]),
    "nc_attn_core": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp, _sz, _vp]),
    "nc_attn_prefill_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "nc_attn_prefill": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _d, _i, _i,
                             _vp, _sz, _vp]),
    "nc_attn_decode_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "nc_attn_decode_shared_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "nc_attn_decode_shared": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i,
                                   _i, _d, _i, _vp, _sz, _vp]),
    "nc_attn_decode": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _d, _i,
                            _vp, _sz, _vp]),
}


class NcError(RuntimeError):
    """A non-OK status from the C ABI, with the library's detail message."""

    def __init__(self, status: int, message: str):
        self.status = status
        super().__init__(f"{_status_name(status)}: {message}")


def _status_name(s):
    return {0: "NC_OK", 1: "NC_ERR_INVALID", 2: "NC_ERR_UNSUPPORTED", 3: "NC_ERR_HIP"}.get(s, str(s))


def library_path() -> str:
    """The in-tree libnc_attn.so, or the build named by NC_ATTN_LIBRARY (another
    build of the same sources, such as a host-sanitizer build of the ABI layer)."""
    return os.environ.get("NC_ATTN_LIBRARY") or os.path.join(_HERE, _LIB_NAME)


def lib() -> ctypes.CDLL:
    """Load the in-tree shared library (built by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build the HIP library first "
                "(python -c 'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(path)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _call(name, *args):
    L = lib()
    st = getattr(L, name)(*args)
    if st != NC_OK:
        raise NcError(st, L.nc_last_error().decode(errors="replace"))


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return NC_BF16
    if t.dtype == torch.float32:
        return NC_F32
    raise TypeError(f"unsupported dtype {t.dtype}: use torch.bfloat16 or torch.float32")


def _gpu(t: torch.Tensor, name: str, ndim: int, dtype=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU (got {t.device}); there is no CPU path")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def rope_qknorm_workspace_bytes(T: int, D: int, pos_offset: int = 0) -> int:
    return int(lib().nc_rope_qknorm_workspace_bytes(T, D, pos_offset))


def attn_fwd_workspace_bytes(B, T, H, Hkv, D, pos_offset=0, dtype=torch.bfloat16) -> int:
    dt = NC_F32 if dtype == torch.float32 else NC_BF16
    return int(lib().nc_attn_fwd_workspace_bytes(B, T, H, Hkv, D, pos_offset, dt))

def attn_prefill_workspace_bytes(B, T, Tmax, H, Hkv, D, dtype=torch.bfloat16) -> int:
    dt = NC_F32 if dtype == torch.float32 else NC_BF16
    return int(lib().nc_attn_prefill_workspace_bytes(B, T, Tmax, H, Hkv, D, dt))


def attn_decode_workspace_bytes(B, Tmax, H, Hkv, D, window) -> int:
    return int(lib().nc_attn_decode_workspace_bytes(B, Tmax, H, Hkv, D, window))


def attn_decode_shared_workspace_bytes(B, Lp, Tgen, H, Hkv, D, window) -> int:
    return int(lib().nc_attn_decode_shared_workspace_bytes(B, Lp, Tgen, H, Hkv, D, window))


def _ve_pair(ve, ve_gate, like, name):
    """Checks the optional value-embedding pair against the values `like`."""
    if (ve is None) != (ve_gate is None):
        raise ValueError(f"{name}: ve and ve_gate must both be given or both be None")
    if ve is None:
        return None, None
    ve = _gpu(ve, "ve", like.dim(), like.dtype)
    ve_gate = _gpu(ve_gate, "ve_gate", like.dim() - 1, like.dtype)
    if ve.shape != like.shape or tuple(ve_gate.shape) != tuple(like.shape[:-1]):
        raise ValueError(f"{name}: ve must have the values' shape and ve_gate that shape without D")
    return ve, ve_gate


def _workspace(nbytes: int, device, workspace):
    if nbytes == 0:
        return None
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError(f"workspace holds fewer than the {nbytes} bytes required")
        return workspace
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def decode_workspace(B, Tmax, H, Hkv, D, window, device="cuda"):
    """A decode workspace for these sizes, reusable by later calls on one stream."""
    n = attn_decode_workspace_bytes(B, Tmax, H, Hkv, D, window)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def rope_qknorm(q, k, *, rope_base: float = 10000.0, pos_offset: int = 0, q_out=None, k_out=None):
    """norm(rope(q)), norm(rope(k)); q (B,T,H,D), k (B,T,Hkv,D). Outputs may be q / k."""
    q = _gpu(q, "q", 4)
    k = _gpu(k, "k", 4, q.dtype)
    B, T, H, D = q.shape
    Hkv = k.shape[2]
    if k.shape[0] != B or k.shape[1] != T or k.shape[3] != D:
        raise ValueError(f"k shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    q_out = torch.empty_like(q) if q_out is None else _gpu(q_out, "q_out", 4, q.dtype)
    k_out = torch.empty_like(k) if k_out is None else _gpu(k_out, "k_out", 4, q.dtype)
    if q_out.shape != q.shape or k_out.shape != k.shape:
        raise ValueError("output shapes must match the inputs")
    ws = _workspace(rope_qknorm_workspace_bytes(T, D, pos_offset), q.device, None)
    _call("nc_rope_qknorm", _ptr(q), _ptr(k), _ptr(q_out), _ptr(k_out), B, T, H, Hkv, D,
          float(rope_base), int(pos_offset), _dt(q), _ptr(ws), 0 if ws is None else ws.numel(),
          _stream(q))
    return q_out, k_out


def qkv_rope_qknorm_workspace_bytes(T, D, dtype=torch.bfloat16) -> int:
    dt = NC_F32 if dtype == torch.float32 else NC_BF16
    return int(lib().nc_qkv_rope_qknorm_workspace_bytes(T, D, dt))


def qkv_rope_qknorm(x, w_q, w_k, w_v, *, H: int, Hkv: int, rope_base: float = 10000.0,
                    pos_offset: int = 0, q_out=None, k_out=None, v_out=None, workspace=None):
    """x (B,T,C) and bias-free weights w_q (H*D,C), w_k, w_v (Hkv*D,C) ->
    (norm(rope(x w_q^T)) (B,T,H,D), norm(rope(x w_k^T)) (B,T,Hkv,D), x w_v^T (B,T,Hkv,D))."""
    x = _gpu(x, "x", 3)
    w_q = _gpu(w_q, "w_q", 2, x.dtype)
    w_k = _gpu(w_k, "w_k", 2, x.dtype)
    w_v = _gpu(w_v, "w_v", 2, x.dtype)
    B, T, C = x.shape
    if w_q.shape[0] % H != 0:
        raise ValueError("w_q rows must be H * D")
    D = w_q.shape[0] // H
    if (tuple(w_q.shape) != (H * D, C) or tuple(w_k.shape) != (Hkv * D, C)
            or tuple(w_v.shape) != (Hkv * D, C)):
        raise ValueError("projection weight shapes are inconsistent")
    q_out = (torch.empty((B, T, H, D), dtype=x.dtype, device=x.device) if q_out is None
             else _gpu(q_out, "q_out", 4, x.dtype))
    k_out = (torch.empty((B, T, Hkv, D), dtype=x.dtype, device=x.device) if k_out is None
             else _gpu(k_out, "k_out", 4, x.dtype))
    v_out = (torch.empty((B, T, Hkv, D), dtype=x.dtype, device=x.device) if v_out is None
             else _gpu(v_out, "v_out", 4, x.dtype))
    if (tuple(q_out.shape) != (B, T, H, D) or tuple(k_out.shape) != (B, T, Hkv, D)
            or tuple(v_out.shape) != (B, T, Hkv, D)):
        raise ValueError("output shapes are inconsistent")
    ws = _workspace(qkv_rope_qknorm_workspace_bytes(T, D, x.dtype), x.device, workspace)
    _call("nc_qkv_rope_qknorm", _ptr(x), _ptr(w_q), _ptr(w_k), _ptr(w_v), _ptr(q_out), _ptr(k_out),
          _ptr(v_out), B, T, C, H, Hkv, D, float(rope_base), int(pos_offset), _dt(x), _ptr(ws),
          ws.numel() * ws.element_size(), _stream(x))
    return q_out, k_out, v_out


def attn_fwd(q, k, v, *, window: int, rope_base: float = 10000.0, pos_offset: int = 0,
             out=None, workspace=None):
    """Prefill attention from raw q (B,T,H,D), k, v (B,T,Hkv,D) -> o (B,T,H,D)."""
    q = _gpu(q, "q", 4)
    k = _gpu(k, "k", 4, q.dtype)
    v = _gpu(v, "v", 4, q.dtype)
    B, T, H, D = q.shape
    Hkv = k.shape[2]
    if tuple(k.shape) != (B, T, Hkv, D) or tuple(v.shape) != (B, T, Hkv, D):
        raise ValueError(f"k {tuple(k.shape)} / v {tuple(v.shape)} do not match q {tuple(q.shape)}")
    o = torch.empty_like(q) if out is None else _gpu(out, "out", 4, q.dtype)
    if o.shape != q.shape:
        raise ValueError("out must have q's shape")
    need = attn_fwd_workspace_bytes(B, T, H, Hkv, D, pos_offset, q.dtype)
    ws = _workspace(need, q.device, workspace)
    _call("nc_attn_fwd", _ptr(q), _ptr(k), _ptr(v), _ptr(o), B, T, H, Hkv, D, int(window),
          float(rope_base), int(pos_offset), _dt(q), _ptr(ws),
          0 if ws is None else ws.numel() * ws.element_size(), _stream(q))
    return o


def attn_fwd_normed(q, k, v, *, window: int, out=None, workspace=None):
    """Attention from q' (B,T,H,D) and k' (B,T,Hkv,D) that are already rotated and
    normalised (e.g. qkv_rope_qknorm's outputs), and v -> o (B,T,H,D)."""
    q = _gpu(q, "q", 4)
    k = _gpu(k, "k", 4, q.dtype)
    v = _gpu(v, "v", 4, q.dtype)
    B, T, H, D = q.shape
    Hkv = k.shape[2]
    if tuple(k.shape) != (B, T, Hkv, D) or tuple(v.shape) != (B, T, Hkv, D):
        raise ValueError(f"k {tuple(k.shape)} / v {tuple(v.shape)} do not match q {tuple(q.shape)}")
    o = torch.empty_like(q) if out is None else _gpu(out, "out", 4, q.dtype)
    if o.shape != q.shape:
        raise ValueError("out must have q's shape")
    dt = _dt(q)
    ws = _workspace(int(lib().nc_attn_fwd_normed_workspace_bytes(B, T, H, Hkv, D, dt)), q.device, workspace)
    _call("nc_attn_fwd_normed", _ptr(q), _ptr(k), _ptr(v), _ptr(o), B, T, H, Hkv, D, int(window), dt,
          _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(q))
    return o


def attn_fwd_lse(q, k, v, *, window: int, rope_base: float = 10000.0, pos_offset: int = 0,
                 out=None, lse=None, workspace=None):
    """attn_fwd that also returns the row log-sum-exp lse (B,T,H) float32,
    ln sum_j exp(q'.k'_j/sqrt(D)) over the visible keys (the backward's input)."""
    q = _gpu(q, "q", 4)
    k = _gpu(k, "k", 4, q.dtype)
    v = _gpu(v, "v", 4, q.dtype)
    B, T, H, D = q.shape
    Hkv = k.shape[2]
    if tuple(k.shape) != (B, T, Hkv, D) or tuple(v.shape) != (B, T, Hkv, D):
        raise ValueError(f"k {tuple(k.shape)} / v {tuple(v.shape)} do not match q {tuple(q.shape)}")
    o = torch.empty_like(q) if out is None else _gpu(out, "out", 4, q.dtype)
    if o.shape != q.shape:
        raise ValueError("out must have q's shape")
    lse = (torch.empty((B, T, H), dtype=torch.float32, device=q.device) if lse is None
           else _gpu(lse, "lse", 3, torch.float32))
    if tuple(lse.shape) != (B, T, H):
        raise ValueError("lse must be (B, T, H)")
    ws = _workspace(attn_fwd_workspace_bytes(B, T, H, Hkv, D, pos_offset, q.dtype), q.device, workspace)
    _call("nc_attn_fwd_lse", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, T, H, Hkv, D, int(window),
          float(rope_base), int(pos_offset), _dt(q), _ptr(ws),
          0 if ws is None else ws.numel() * ws.element_size(), _stream(q))
    return o, lse


def attn_fwd_noalloc(q, k, v, *, window: int, out, rope_base: float = 10000.0, pos_offset: int = 0):
    """attn_fwd into the caller's `out` with the library's static scratch as its
    workspace: the C entry point allocates nothing (q, k, v, out on the current
    device). Calls overlapping on one GPU race on the shared scratch."""
    q = _gpu(q, "q", 4)
    k = _gpu(k, "k", 4, q.dtype)
    v = _gpu(v, "v", 4, q.dtype)
    o = _gpu(out, "out", 4, q.dtype)
    B, T, H, D = q.shape
    Hkv = k.shape[2]
    if tuple(k.shape) != (B, T, Hkv, D) or tuple(v.shape) != (B, T, Hkv, D) or o.shape != q.shape:
        raise ValueError("attn_fwd_noalloc tensor shapes are inconsistent")
    with torch.cuda.device(q.device):
        _call("nc_attn_fwd_noalloc", _ptr(q), _ptr(k), _ptr(v), _ptr(o), B, T, H, Hkv, D, int(window),
              float(rope_base), int(pos_offset), _dt(q), _stream(q))
    return o


def attn_fwd_normed_workspace_bytes(B, T, H, Hkv, D, dtype=torch.bfloat16) -> int:
    dt = NC_F32 if dtype == torch.float32 else NC_BF16
    return int(lib().nc_attn_fwd_normed_workspace_bytes(B, T, H, Hkv, D, dt))


def attn_bwd_workspace_bytes(B, T, H, Hkv, D, dtype=torch.bfloat16) -> int:
    dt = NC_F32 if dtype == torch.float32 else NC_BF16
    return int(lib().nc_attn_bwd_workspace_bytes(B, T, H, Hkv, D, dt))


def attn_bwd(q, k, v, o, dout, lse, *, window: int, rope_base: float = 10000.0, pos_offset: int = 0,
             dq=None, dk=None, dv=None, workspace=None):
    """Gradients (dq, dk, dv) of attn_fwd with respect to its raw q, k, v, from
    the forward's output o, dL/do and its row log-sum-exp lse (attn_fwd_lse)."""
    q = _gpu(q, "q", 4)
    k = _gpu(k, "k", 4, q.dtype)
    v = _gpu(v, "v", 4, q.dtype)
    o = _gpu(o, "o", 4, q.dtype)
    dout = _gpu(dout, "dout", 4, q.dtype)
    lse = _gpu(lse, "lse", 3, torch.float32)
    B, T, H, D = q.shape
    Hkv = k.shape[2]
    if (tuple(k.shape) != (B, T, Hkv, D) or tuple(v.shape) != (B, T, Hkv, D) or o.shape != q.shape
            or dout.shape != q.shape or tuple(lse.shape) != (B, T, H)):
        raise ValueError("backward tensor shapes are inconsistent")
    dq = torch.empty_like(q) if dq is None else _gpu(dq, "dq", 4, q.dtype)
    dk = torch.empty_like(k) if dk is None else _gpu(dk, "dk", 4, q.dtype)
    dv = torch.empty_like(v) if dv is None else _gpu(dv, "dv", 4, q.dtype)
    if dq.shape != q.shape or dk.shape != k.shape or dv.shape != v.shape:
        raise ValueError("gradient shapes must match q, k, v")
    ws = _workspace(attn_bwd_workspace_bytes(B, T, H, Hkv, D, q.dtype), q.device, workspace)
    _call("nc_attn_bwd", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
          _ptr(dv), B, T, H, Hkv, D, int(window), float(rope_base), int(pos_offset), _dt(q), _ptr(ws),
          ws.numel() * ws.element_size(), _stream(q))
    return dq, dk, dv


def attn_prep(k, *, rope_base: float = 10000.0, pos_offset: int = 0, H=None, workspace=None):
    """First stage of attn_fwd: k' = norm(rope(k)) and the q-side (cos, sin) table,
    into a workspace (returned) for attn_core. k (B,T,Hkv,D)."""
    k = _gpu(k, "k", 4)
    B, T, Hkv, D = k.shape
    need = attn_fwd_workspace_bytes(B, T, Hkv if H is None else H, Hkv, D, pos_offset, k.dtype)
    ws = _workspace(need, k.device, workspace)
    _call("nc_attn_prep", _ptr(k), B, T, Hkv, D, float(rope_base), int(pos_offset), _dt(k),
          _ptr(ws), ws.numel() * ws.element_size(), _stream(k))
    return ws


def attn_core(q, v, workspace, *, window: int, out=None):
    """Second stage of attn_fwd: attention from raw q (B,T,H,D), v (B,T,Hkv,D) and the
    workspace filled by attn_prep for the same B, T, Hkv, D and dtype (sized by
    attn_fwd_workspace_bytes for this H: partial rows may be written after k')."""
    q = _gpu(q, "q", 4)
    v = _gpu(v, "v", 4, q.dtype)
    B, T, H, D = q.shape
    Hkv = v.shape[2]
    if tuple(v.shape) != (B, T, Hkv, D):
        raise ValueError(f"v {tuple(v.shape)} does not match q {tuple(q.shape)}")
    o = torch.empty_like(q) if out is None else _gpu(out, "out", 4, q.dtype)
    if o.shape != q.shape:
        raise ValueError("out must have q's shape")
    _call("nc_attn_core", _ptr(q), _ptr(v), _ptr(o), B, T, H, Hkv, D, int(window), _dt(q),
          _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(q))
    return o


def attn_prefill(q, k, v, k_cache, v_cache, *, window: int, pos_offset: int = 0,
                 rope_base: float = 10000.0, ve=None, ve_gate=None, out=None, workspace=None):
    """Prefill of a chunk at positions pos_offset.. into the caches (in place):
    rows pos_offset .. pos_offset+T-1 receive norm(rope(k)) and v (v + ve_gate * ve
    with the optional value embedding ve (B,T,Hkv,D), ve_gate (B,T,Hkv)), then the
    chunk's queries attend to cache rows within the window. q (B,T,H,D);
    k, v (B,T,Hkv,D); caches (B,Tmax,Hkv,D) -> o (B,T,H,D)."""
    q = _gpu(q, "q", 4)
    k = _gpu(k, "k", 4, q.dtype)
    v = _gpu(v, "v", 4, q.dtype)
    k_cache = _gpu(k_cache, "k_cache", 4, q.dtype)
    v_cache = _gpu(v_cache, "v_cache", 4, q.dtype)
    B, T, H, D = q.shape
    Hkv = k.shape[2]
    Tmax = k_cache.shape[1]
    if (tuple(k.shape) != (B, T, Hkv, D) or tuple(v.shape) != (B, T, Hkv, D)
            or tuple(k_cache.shape) != (B, Tmax, Hkv, D) or tuple(v_cache.shape) != (B, Tmax, Hkv, D)):
        raise ValueError("prefill tensor shapes are inconsistent")
    o = torch.empty_like(q) if out is None else _gpu(out, "out", 4, q.dtype)
    if o.shape != q.shape:
        raise ValueError("out must have q's shape")
    ws = _workspace(attn_prefill_workspace_bytes(B, T, Tmax, H, Hkv, D, q.dtype), q.device, workspace)
    ve, ve_gate = _ve_pair(ve, ve_gate, v, "attn_prefill")
    _call("nc_attn_prefill", _ptr(q), _ptr(k), _ptr(v), _ptr(ve), _ptr(ve_gate), _ptr(k_cache),
          _ptr(v_cache), _ptr(o),
          B, T, Tmax, H, Hkv, D, int(window), float(rope_base), int(pos_offset), _dt(q),
          _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(q))
    return o


def attn_decode(q, k_new, v_new, k_cache, v_cache, seqlens, *, window: int,
                rope_base: float = 10000.0, ve=None, ve_gate=None, out=None, workspace=None):
    """One decode step: appends norm(rope(k_new)) and v_new at index seqlens-1 of the
    caches (in place), then attends. q (B,H,D); k_new, v_new (B,Hkv,D);
    caches (B,Tmax,Hkv,D); seqlens (B,) int32 on the GPU -> o (B,H,D)."""
    q = _gpu(q, "q", 3)
    k_new = _gpu(k_new, "k_new", 3, q.dtype)
    v_new = _gpu(v_new, "v_new", 3, q.dtype)
    k_cache = _gpu(k_cache, "k_cache", 4, q.dtype)
    v_cache = _gpu(v_cache, "v_cache", 4, q.dtype)
    seqlens = _gpu(seqlens, "seqlens", 1, torch.int32)
    B, H, D = q.shape
    Hkv = k_new.shape[1]
    Tmax = k_cache.shape[1]
    if (tuple(k_new.shape) != (B, Hkv, D) or tuple(v_new.shape) != (B, Hkv, D)
            or tuple(k_cache.shape) != (B, Tmax, Hkv, D) or tuple(v_cache.shape) != (B, Tmax, Hkv, D)
            or tuple(seqlens.shape) != (B,)):
        raise ValueError("decode tensor shapes are inconsistent")
    o = torch.empty_like(q) if out is None else _gpu(out, "out", 3, q.dtype)
    need = attn_decode_workspace_bytes(B, Tmax, H, Hkv, D, window)
    ws = _workspace(need, q.device, workspace)
    ve, ve_gate = _ve_pair(ve, ve_gate, v_new, "attn_decode")
    _call("nc_attn_decode", _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(ve), _ptr(ve_gate),
          _ptr(k_cache), _ptr(v_cache),
          _ptr(seqlens), _ptr(o), B, Tmax, H, Hkv, D, int(window), float(rope_base), _dt(q),
          _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(q))
    return o


def attn_decode_shared(q, k_new, v_new, k_prompt, v_prompt, k_cache, v_cache, seqlens, *,
                       window: int, rope_base: float = 10000.0, ve=None, ve_gate=None, out=None,
                       workspace=None):
    """One decode step of B samples continuing one prompt: prompt positions from the
    shared (Lp,Hkv,D) caches, the samples' own positions Lp.. from their
    (B,Tgen,Hkv,D) caches, whose row L-1-Lp receives the new token (in place).
    q (B,H,D); k_new, v_new (B,Hkv,D); seqlens (B,) int32 on the GPU -> o (B,H,D)."""
    q = _gpu(q, "q", 3)
    k_new = _gpu(k_new, "k_new", 3, q.dtype)
    v_new = _gpu(v_new, "v_new", 3, q.dtype)
    k_prompt = _gpu(k_prompt, "k_prompt", 3, q.dtype)
    v_prompt = _gpu(v_prompt, "v_prompt", 3, q.dtype)
    k_cache = _gpu(k_cache, "k_cache", 4, q.dtype)
    v_cache = _gpu(v_cache, "v_cache", 4, q.dtype)
    seqlens = _gpu(seqlens, "seqlens", 1, torch.int32)
    B, H, D = q.shape
    Hkv = k_new.shape[1]
    Lp, Tgen = k_prompt.shape[0], k_cache.shape[1]
    if (tuple(k_new.shape) != (B, Hkv, D) or tuple(v_new.shape) != (B, Hkv, D)
            or tuple(k_prompt.shape) != (Lp, Hkv, D) or tuple(v_prompt.shape) != (Lp, Hkv, D)
            or tuple(k_cache.shape) != (B, Tgen, Hkv, D) or tuple(v_cache.shape) != (B, Tgen, Hkv, D)
            or tuple(seqlens.shape) != (B,)):
        raise ValueError("shared decode tensor shapes are inconsistent")
    o = torch.empty_like(q) if out is None else _gpu(out, "out", 3, q.dtype)
    need = attn_decode_shared_workspace_bytes(B, Lp, Tgen, H, Hkv, D, window)
    ws = _workspace(need, q.device, workspace)
    ve, ve_gate = _ve_pair(ve, ve_gate, v_new, "attn_decode_shared")
    _call("nc_attn_decode_shared", _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(ve), _ptr(ve_gate),
          _ptr(k_prompt), _ptr(v_prompt),
          Lp, _ptr(k_cache), _ptr(v_cache), _ptr(seqlens), _ptr(o), B, Tgen, H, Hkv, D, int(window),
          float(rope_base), _dt(q), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
          _stream(q))
    return o
