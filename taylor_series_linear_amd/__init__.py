"""Python binding of libtaylor_attn.so (causal Taylor-series linear attention on MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/taylor_attn.h. Torch supplies
device memory and the current stream. There is no CPU fallback: if the
library is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtaylor_attn.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "taylor_attn.h")

TAYLOR_OK = 0
TAYLOR_ERR_NULL_PTR = 1
TAYLOR_ERR_BAD_SHAPE = 2
TAYLOR_ERR_UNSUPPORTED = 3
TAYLOR_ERR_BAD_SCALE = 4
TAYLOR_ERR_WORKSPACE = 5
TAYLOR_ERR_HIP = 6
TAYLOR_F32 = 0
TAYLOR_BF16 = 1

_lib = None


class Ext(ctypes.Structure):
    """taylor_attn_ext: decay and query/key preprocessing options."""
    _fields_ = [("gamma", ctypes.c_float), ("qk_norm", ctypes.c_int), ("q_scale", ctypes.c_float),
                ("k_scale", ctypes.c_float), ("q_head_scale", ctypes.c_void_p)]


class TaylorError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"taylor_attn status {status}: {msg}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libtaylor_attn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m taylor_series_linear_amd.build`")
    # torch ships its own HIP runtime (same soname, libamdhip64.so.7). Load it
    # first so the library binds to that one instance; two runtimes in one
    # process do not share devices, streams or allocations.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    fp = ctypes.POINTER(ctypes.c_float)
    L.taylor_feature_dim.argtypes = [i32, i32]
    L.taylor_feature_dim.restype = i64
    L.taylor_is_supported.argtypes = [i32, i32, i32]
    L.taylor_is_supported.restype = i32
    L.taylor_last_error.argtypes = []
    L.taylor_last_error.restype = ctypes.c_char_p
    L.taylor_feature_map.argtypes = [vp, i32, i64, i32, i32, f32, i32, vp, vp]
    L.taylor_feature_map.restype = i32
    L.taylor_attn_prefill_workspace.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    L.taylor_attn_prefill_workspace.restype = sz
    L.taylor_attn_prefill.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32,
                                      vp, vp, vp, i32, vp, vp, vp, sz, vp]
    L.taylor_attn_prefill.restype = i32
    L.taylor_attn_prefill_noalloc.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32,
                                              vp, vp, vp, i32, vp, vp, vp]
    L.taylor_attn_prefill_noalloc.restype = i32
    L.taylor_attn_decode.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, f32,
                                     vp, vp, vp, i32, vp]
    L.taylor_attn_decode.restype = i32
    L.taylor_attn_prefill_decayed_workspace.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    L.taylor_attn_prefill_decayed_workspace.restype = sz
    L.taylor_attn_prefill_decayed.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, f32,
                                              vp, vp, vp, i32, vp, vp, vp, sz, vp]
    L.taylor_attn_prefill_decayed.restype = i32
    L.taylor_attn_decode_decayed.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, f32,
                                             vp, vp, vp, i32, vp]
    L.taylor_attn_decode_decayed.restype = i32
    ep = ctypes.POINTER(Ext)
    L.taylor_attn_prefill_ext_workspace.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    L.taylor_attn_prefill_ext_workspace.restype = sz
    L.taylor_attn_prefill_ext.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, ep,
                                          vp, vp, vp, i32, vp, vp, vp, sz, vp]
    L.taylor_attn_prefill_ext.restype = i32
    L.taylor_attn_decode_ext.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, ep,
                                         vp, vp, vp, i32, vp]
    L.taylor_attn_decode_ext.restype = i32
    del fp
    _lib = L
    return L


def header_functions() -> list[str]:
    """Names of the functions include/taylor_attn.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(taylor_[a-z_]+)\s*\(", text)))


def check(status: int) -> None:
    if status == TAYLOR_OK:
        return
    msg = lib().taylor_last_error().decode()
    if status in (TAYLOR_ERR_BAD_SHAPE, TAYLOR_ERR_BAD_SCALE, TAYLOR_ERR_NULL_PTR):
        raise ValueError(f"taylor_attn status {status}: {msg}")
    if status == TAYLOR_ERR_UNSUPPORTED:
        raise NotImplementedError(f"taylor_attn status {status}: {msg}")
    raise TaylorError(status, msg)


def feature_dim(d: int, n_terms: int) -> int:
    return int(lib().taylor_feature_dim(d, n_terms))


def is_supported(d: int, dv: int, n_terms: int) -> bool:
    return bool(lib().taylor_is_supported(d, dv, n_terms))


# ---------------------------------------------------------------------------
# torch-facing wrappers
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dt(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return TAYLOR_F32
    if t.dtype == torch.bfloat16:
        return TAYLOR_BF16
    raise NotImplementedError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def feature_map(x, n_terms: int, a: float | None = None):
    """phi(x) for x [..., d] -> float32 [..., F]; with `a`, sqrt(alpha_m) is folded in."""
    torch = _torch()
    _need(x, "x")
    d = x.shape[-1]
    F = feature_dim(d, n_terms)
    rows = x.numel() // d if d else 0
    phi = torch.empty(x.shape[:-1] + (max(F, 0),), dtype=torch.float32, device=x.device)
    check(lib().taylor_feature_map(_ptr(x), _dt(x), rows, d, n_terms,
                                   float(a) if a is not None else 0.0, 1 if a is not None else 0,
                                   _ptr(phi), _stream()))
    return phi


def prefill_workspace_bytes(B, H, N, d, dv, n_terms, in_dtype, decayed: bool = False) -> int:
    code = TAYLOR_BF16 if str(in_dtype).endswith("bfloat16") or in_dtype == TAYLOR_BF16 else TAYLOR_F32
    fn = lib().taylor_attn_prefill_decayed_workspace if decayed else lib().taylor_attn_prefill_workspace
    r = fn(B, H, N, d, dv, n_terms, code)
    if r == ctypes.c_size_t(-1).value:
        raise ValueError(lib().taylor_last_error().decode())
    return int(r)


def _ext(gamma, qk_norm, q_scale, k_scale, q_head_scale, H):
    """The options struct, or None when every option is at its default."""
    if gamma is None and not qk_norm and q_scale == 1.0 and k_scale == 1.0 and q_head_scale is None:
        return None
    hp = None
    if q_head_scale is not None:
        _need(q_head_scale, "q_head_scale")
        if q_head_scale.dtype != _torch().float32 or q_head_scale.dim() != 1 or q_head_scale.numel() != H:
            raise ValueError(f"q_head_scale must be a float32 tensor [H] = [{H}]")
        hp = q_head_scale.data_ptr()
    return Ext(1.0 if gamma is None else float(gamma), 1 if qk_norm else 0, float(q_scale), float(k_scale), hp)


def prefill(q, k, v, n_terms: int, a: float, S0=None, z0=None, *, out_dtype=None,
            want_output: bool = True, return_state: bool = False, S=None, z=None,
            workspace=None, gamma: float | None = None, qk_norm: bool = False, q_scale: float = 1.0,
            k_scale: float = 1.0, q_head_scale=None):
    """Causal prefill. q, k [B, H, N, d], v [B, H, N, dv] (float32 or bfloat16, same dtype).

    Returns o [B, H, N, dv] (out_dtype, default q.dtype) or None, and with
    return_state=True also the final state (S [B, H, F, dv], z [B, H, F], float32).
    S / z may be passed to write the state into given buffers (they may be S0 / z0).
    With ``gamma`` (0 < gamma <= 1) the state decays by gamma before every
    write; ``qk_norm``, ``q_scale``, ``k_scale`` and ``q_head_scale`` (a float32
    tensor [H]) preprocess q and k rows inside the kernels
    (taylor_attn_prefill_ext).
    """
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n)
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k and v must share a dtype")
    B, H, N, d = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != q.shape[:3]:
        raise ValueError("shape mismatch between q, k and v")
    F = feature_dim(d, n_terms)
    out_dtype = q.dtype if out_dtype is None else out_dtype
    o = torch.empty((B, H, N, dv), dtype=out_dtype, device=q.device) if want_output else None
    if return_state and S is None:
        S = torch.empty((B, H, F, dv), dtype=torch.float32, device=q.device)
        z = torch.empty((B, H, F), dtype=torch.float32, device=q.device)
    for t, n in ((S0, "S0"), (z0, "z0"), (S, "S"), (z, "z")):
        if t is not None:
            _need(t, n)
            if t.dtype != torch.float32:
                raise ValueError(f"{n} must be float32")
    ext = _ext(gamma, qk_norm, q_scale, k_scale, q_head_scale, H)
    ws_bytes = prefill_workspace_bytes(B, H, N, d, dv, n_terms, q.dtype, decayed=ext is not None)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    od = TAYLOR_F32 if o is None else _dt(o)
    if ext is None:
        check(lib().taylor_attn_prefill(
            _ptr(q), _ptr(k), _ptr(v), _dt(q), B, H, N, d, dv, n_terms, float(a),
            _ptr(S0), _ptr(z0), _ptr(o), od, _ptr(S), _ptr(z), _ptr(workspace), ws_len, _stream()))
    else:
        check(lib().taylor_attn_prefill_ext(
            _ptr(q), _ptr(k), _ptr(v), _dt(q), B, H, N, d, dv, n_terms, float(a), ctypes.byref(ext),
            _ptr(S0), _ptr(z0), _ptr(o), od, _ptr(S), _ptr(z), _ptr(workspace), ws_len, _stream()))
    if return_state or S is not None:
        return o, S, z
    return o


def decode(q, k, v, S, z, n_terms: int, a: float, *, out_dtype=None, o=None, gamma: float | None = None,
           qk_norm: bool = False, q_scale: float = 1.0, k_scale: float = 1.0, q_head_scale=None):
    """One decode step: q, k [B, H, d], v [B, H, dv]; S, z updated in place. Returns o [B, H, dv].

    With ``gamma`` the state decays by gamma before the write; the other
    options preprocess q and k as for prefill (taylor_attn_decode_ext)."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (S, "S"), (z, "z")):
        _need(t, n)
    B, H, d = q.shape
    dv = v.shape[-1]
    if o is None:
        o = torch.empty((B, H, dv), dtype=q.dtype if out_dtype is None else out_dtype, device=q.device)
    ext = _ext(gamma, qk_norm, q_scale, k_scale, q_head_scale, H)
    if ext is None:
        check(lib().taylor_attn_decode(_ptr(q), _ptr(k), _ptr(v), _dt(q), B, H, d, dv, n_terms,
                                       float(a), _ptr(S), _ptr(z), _ptr(o), _dt(o), _stream()))
    else:
        check(lib().taylor_attn_decode_ext(_ptr(q), _ptr(k), _ptr(v), _dt(q), B, H, d, dv, n_terms,
                                           float(a), ctypes.byref(ext), _ptr(S), _ptr(z), _ptr(o), _dt(o),
                                           _stream()))
    return o
