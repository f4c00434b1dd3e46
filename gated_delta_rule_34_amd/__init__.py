"""Python binding of the gfx950 gated delta rule library (``libgdn.so``).

Argument marshalling only: each function checks tensor dtypes, shapes and
devices, allocates outputs and workspace with torch (device memory is torch's
business), and calls the C entry point of the same name on torch's current
stream.  All computation happens in the HIP kernels; there is no fallback.
If the library is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "lib_path", "load", "status_string",
    "gdn_chunk_fwd", "gdn_chunk_intra", "gdn_chunk_walk", "gdn2_chunk_fwd", "gdn_recurrent_step",
    "gdn2_recurrent_step", "gdn_chunk_bwd", "gdn_chunk_bwd_workspace", "gdn_chunk_fwd_varlen",
    "gdn2_chunk_fwd_varlen", "gdn2_chunk_fwd_varlen_workspace",
    "gdn_chunk_fwd_workspace", "gdn2_chunk_fwd_workspace", "gdn_prologue", "gdn_gated_rmsnorm",
    "gdn2_chunk_bwd", "gdn2_chunk_bwd_workspace", "gdn2_chunk_fwd_noalloc", "gdn2_chunk_fwd_noalloc_max_bytes",
    "clock_probe",
    "GDN_F32", "GDN_BF16", "BT",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libgdn.so")

GDN_F32, GDN_BF16 = 0, 1
BT = 64
_lib = None

_vp = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float
_sz = ctypes.c_size_t


def load():
    """Load libgdn.so and declare its C signatures (raises if not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(lib_path):
        raise RuntimeError(f"{lib_path} is not built; run `python gated_delta_rule_34_amd/build.py`")
    lib = ctypes.CDLL(lib_path)
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_status_string.argtypes = [_i]
    lib.gdn_chunk_fwd_workspace.restype = _sz
    lib.gdn_chunk_fwd_workspace.argtypes = [_i] * 6
    lib.gdn2_chunk_fwd_workspace.restype = _sz
    lib.gdn2_chunk_fwd_workspace.argtypes = [_i] * 6
    lib.gdn_chunk_fwd.restype = _i
    lib.gdn_chunk_fwd.argtypes = [_vp] * 8 + [_i] * 6 + [_f, _vp, _sz, _vp]
    lib.gdn_chunk_intra.restype = _i
    lib.gdn_chunk_intra.argtypes = [_vp] * 5 + [_i] * 5 + [_vp]
    lib.gdn_chunk_walk.restype = _i
    lib.gdn_chunk_walk.argtypes = [_vp] * 9 + [_i] * 6 + [_f, _vp]
    lib.gdn2_chunk_fwd.restype = _i
    lib.gdn2_chunk_fwd.argtypes = [_vp] * 9 + [_i] * 6 + [_f, _vp, _sz, _vp]
    lib.gdn_recurrent_step.restype = _i
    lib.gdn_recurrent_step.argtypes = [_vp] * 7 + [_i] * 5 + [_f, _vp]
    lib.gdn_chunk_fwd_varlen.restype = _i
    lib.gdn_chunk_fwd_varlen.argtypes = [_vp] * 9 + [_i] * 6 + [_f, _vp]
    lib.gdn2_chunk_fwd_varlen_workspace.restype = _sz
    lib.gdn2_chunk_fwd_varlen_workspace.argtypes = [_i] * 6
    lib.gdn2_chunk_fwd_varlen.restype = _i
    lib.gdn2_chunk_fwd_varlen.argtypes = [_vp] * 10 + [_i] * 6 + [_f, _vp, _sz, _vp]
    lib.gdn_chunk_bwd_workspace.restype = _sz
    lib.gdn_chunk_bwd_workspace.argtypes = [_i] * 6
    lib.gdn_chunk_bwd.restype = _i
    lib.gdn_chunk_bwd.argtypes = [_vp] * 14 + [_i] * 6 + [_f, _vp, _sz, _vp]
    lib.gdn2_recurrent_step.restype = _i
    lib.gdn2_recurrent_step.argtypes = [_vp] * 8 + [_i] * 5 + [_f, _vp]
    lib.gdn2_chunk_bwd_workspace.restype = _sz
    lib.gdn2_chunk_bwd_workspace.argtypes = [_i] * 6
    lib.gdn2_chunk_bwd.restype = _i
    lib.gdn2_chunk_bwd.argtypes = [_vp] * 16 + [_i] * 6 + [_f, _vp, _sz, _vp]
    lib.gdn_prologue.restype = _i
    lib.gdn_prologue.argtypes = [_vp] * 17 + [_i] * 5 + [_vp]
    lib.gdn2_chunk_fwd_noalloc.restype = _i
    lib.gdn2_chunk_fwd_noalloc.argtypes = [_vp] * 9 + [_i] * 6 + [_f, _vp]
    lib.gdn2_chunk_fwd_noalloc_max_bytes.restype = _sz
    lib.gdn2_chunk_fwd_noalloc_max_bytes.argtypes = []
    lib.gdn_clock_probe.restype = _i
    lib.gdn_clock_probe.argtypes = [_vp, _i, _i, _vp]
    lib.gdn_gated_rmsnorm.restype = _i
    lib.gdn_gated_rmsnorm.argtypes = [_vp] * 4 + [ctypes.c_longlong, _i, _f, _vp]
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load().gdn_status_string(code).decode()


def _check(code: int, what: str):
    if code != 0:
        raise RuntimeError(f"{what} failed: {status_string(code)} (status {code})")


def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float32:
        return GDN_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, shape, dtype, device):
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name}: expected device {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _workspace(nbytes, device):
    torch = _torch()
    ws = torch.empty(max(int(nbytes), 256) + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    return ws, ws[off:off + max(int(nbytes), 256)]


def gdn_chunk_fwd_workspace(B, T, H, Dk, Dv, dtype_code):
    return int(load().gdn_chunk_fwd_workspace(B, T, H, Dk, Dv, dtype_code))


def gdn2_chunk_fwd_workspace(B, T, H, Dk, Dv, dtype_code):
    return int(load().gdn2_chunk_fwd_workspace(B, T, H, Dk, Dv, dtype_code))


def gdn_chunk_fwd(q, k, v, g, beta, h0=None, scale=None, output_final_state=True, workspace=None,
                  out=None, final_state=None):
    """Chunked Gated DeltaNet forward.  q, k [B,T,H,Dk], v [B,T,H,Dv] (bf16 or fp32),
    g, beta [B,T,H] fp32, h0 [B,H,Dk,Dv] fp32 or None.  Returns (o fp32, ht or None)."""
    torch = _torch()
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    dt = _dtype_code(q)
    _need(q, "q", (B, T, H, Dk), q.dtype, dev)
    _need(k, "k", (B, T, H, Dk), q.dtype, dev)
    _need(v, "v", (B, T, H, Dv), q.dtype, dev)
    _need(g, "g", (B, T, H), torch.float32, dev)
    _need(beta, "beta", (B, T, H), torch.float32, dev)
    if h0 is not None:
        _need(h0, "h0", (B, H, Dk, Dv), torch.float32, dev)
    if scale is None:
        scale = Dk ** -0.5
    o = out if out is not None else torch.empty((B, T, H, Dv), dtype=torch.float32, device=dev)
    _need(o, "out", (B, T, H, Dv), torch.float32, dev)
    ht = None
    if output_final_state:
        ht = final_state if final_state is not None else torch.empty((B, H, Dk, Dv), dtype=torch.float32,
                                                                     device=dev)
        _need(ht, "final_state", (B, H, Dk, Dv), torch.float32, dev)
    lib = load()
    need = lib.gdn_chunk_fwd_workspace(B, T, H, Dk, Dv, dt)
    if need == 0:
        _check(2, "gdn_chunk_fwd_workspace")
    if workspace is None:
        _, ws = _workspace(need, dev)
    else:
        ws = workspace
    _check(lib.gdn_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(o), _ptr(ht),
                             B, T, H, Dk, Dv, dt, float(scale), _ptr(ws), ws.numel() * ws.element_size(),
                             _stream(dev)), "gdn_chunk_fwd")
    return o, ht


def gdn_chunk_fwd_varlen(q, k, v, g, beta, cu_seqlens, h0=None, scale=None, output_final_state=True):
    """Chunked forward over packed variable-length sequences.  q, k [total_T,H,Dk] and
    v [total_T,H,Dv] bf16 (a leading batch dim of 1 is accepted), g, beta [total_T,H]
    fp32, cu_seqlens int32 [N+1] on the device, h0 [N,H,Dk,Dv] fp32 or None.
    Returns (o [total_T,H,Dv] fp32, ht [N,H,Dk,Dv] or None)."""
    torch = _torch()
    if q.dim() == 4:
        q, k, v, g, beta = q[0], k[0], v[0], g[0], beta[0]
    total_T, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    N = cu_seqlens.numel() - 1
    dt = _dtype_code(q)
    _need(q, "q", (total_T, H, Dk), q.dtype, dev)
    _need(k, "k", (total_T, H, Dk), q.dtype, dev)
    _need(v, "v", (total_T, H, Dv), q.dtype, dev)
    _need(g, "g", (total_T, H), torch.float32, dev)
    _need(beta, "beta", (total_T, H), torch.float32, dev)
    _need(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    if h0 is not None:
        _need(h0, "h0", (N, H, Dk, Dv), torch.float32, dev)
    if scale is None:
        scale = Dk ** -0.5
    o = torch.empty((total_T, H, Dv), dtype=torch.float32, device=dev)
    ht = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=dev) if output_final_state else None
    _check(load().gdn_chunk_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), _ptr(h0),
                                       _ptr(o), _ptr(ht), N, total_T, H, Dk, Dv, dt, float(scale), _stream(dev)),
           "gdn_chunk_fwd_varlen")
    return o, ht


def gdn2_chunk_fwd_varlen_workspace(N, total_T, H, Dk, Dv, dtype_code):
    return load().gdn2_chunk_fwd_varlen_workspace(N, total_T, H, Dk, Dv, dtype_code)


def gdn2_chunk_fwd_varlen(q, k, v, log_alpha, b, w, cu_seqlens, h0=None, scale=None, output_final_state=True,
                          workspace=None):
    """Gated DeltaNet-2 forward over packed variable-length sequences.  q, k, b
    [total_T,H,Dk] and v, w [total_T,H,Dv] bf16 (a leading batch dim of 1 is accepted),
    log_alpha [total_T,H,Dk] fp32, cu_seqlens int32 [N+1] on the device, h0 [N,H,Dk,Dv]
    fp32 or None.  Returns (o [total_T,H,Dv] fp32, ht [N,H,Dk,Dv] or None)."""
    torch = _torch()
    if q.dim() == 4:
        q, k, v, log_alpha, b, w = q[0], k[0], v[0], log_alpha[0], b[0], w[0]
    total_T, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    N = cu_seqlens.numel() - 1
    dt = _dtype_code(q)
    for t, name, d in ((q, "q", Dk), (k, "k", Dk), (v, "v", Dv), (b, "b", Dk), (w, "w", Dv)):
        _need(t, name, (total_T, H, d), q.dtype, dev)
    _need(log_alpha, "log_alpha", (total_T, H, Dk), torch.float32, dev)
    _need(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    if h0 is not None:
        _need(h0, "h0", (N, H, Dk, Dv), torch.float32, dev)
    if scale is None:
        scale = Dk ** -0.5
    o = torch.empty((total_T, H, Dv), dtype=torch.float32, device=dev)
    ht = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=dev) if output_final_state else None
    lib = load()
    need = lib.gdn2_chunk_fwd_varlen_workspace(N, total_T, H, Dk, Dv, dt)
    if need == 0:
        _check(2, "gdn2_chunk_fwd_varlen_workspace")
    ws = workspace if workspace is not None else _workspace(need, dev)[1]
    _check(lib.gdn2_chunk_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w),
                                     _ptr(cu_seqlens), _ptr(h0), _ptr(o), _ptr(ht), N, total_T, H, Dk, Dv, dt,
                                     float(scale), _ptr(ws), ws.numel() * ws.element_size(), _stream(dev)),
           "gdn2_chunk_fwd_varlen")
    return o, ht


def gdn_chunk_bwd_workspace(B, T, H, Dk, Dv, dtype_code):
    return int(load().gdn_chunk_bwd_workspace(B, T, H, Dk, Dv, dtype_code))


def gdn_chunk_bwd(q, k, v, g, beta, h0, do, dht=None, scale=None, workspace=None):
    """Backward of gdn_chunk_fwd: gradients of sum(do * o) + sum(dht * ht).
    Inputs as gdn_chunk_fwd (h0 may be None), do [B,T,H,Dv] fp32, dht [B,H,Dk,Dv]
    fp32 or None.  Returns (dq, dk, dv, dg, dbeta, dh0) fp32; dh0 is None when h0 is."""
    torch = _torch()
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    dt = _dtype_code(q)
    _need(q, "q", (B, T, H, Dk), q.dtype, dev)
    _need(k, "k", (B, T, H, Dk), q.dtype, dev)
    _need(v, "v", (B, T, H, Dv), q.dtype, dev)
    _need(g, "g", (B, T, H), torch.float32, dev)
    _need(beta, "beta", (B, T, H), torch.float32, dev)
    _need(do, "do", (B, T, H, Dv), torch.float32, dev)
    if h0 is not None:
        _need(h0, "h0", (B, H, Dk, Dv), torch.float32, dev)
    if dht is not None:
        _need(dht, "dht", (B, H, Dk, Dv), torch.float32, dev)
    if scale is None:
        scale = Dk ** -0.5
    f32 = dict(dtype=torch.float32, device=dev)
    dq = torch.empty((B, T, H, Dk), **f32)
    dk = torch.empty((B, T, H, Dk), **f32)
    dv = torch.empty((B, T, H, Dv), **f32)
    dg = torch.empty((B, T, H), **f32)
    dbeta = torch.empty((B, T, H), **f32)
    dh0 = torch.empty((B, H, Dk, Dv), **f32) if h0 is not None else None
    lib = load()
    need = lib.gdn_chunk_bwd_workspace(B, T, H, Dk, Dv, dt)
    if need == 0:
        _check(2, "gdn_chunk_bwd_workspace")
    ws = workspace if workspace is not None else _workspace(need, dev)[1]
    _check(lib.gdn_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(do), _ptr(dht),
                             _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dbeta), _ptr(dh0), B, T, H, Dk, Dv, dt,
                             float(scale), _ptr(ws), ws.numel() * ws.element_size(), _stream(dev)), "gdn_chunk_bwd")
    return dq, dk, dv, dg, dbeta, dh0


def gdn2_chunk_bwd_workspace(B, T, H, Dk, Dv, dtype_code):
    return int(load().gdn2_chunk_bwd_workspace(B, T, H, Dk, Dv, dtype_code))


def gdn2_chunk_bwd(q, k, v, log_alpha, b, w, h0, do, dht=None, scale=None, workspace=None):
    """Backward of gdn2_chunk_fwd.  Inputs as gdn2_chunk_fwd (h0 may be None), do
    [B,T,H,Dv] fp32, dht [B,H,Dk,Dv] fp32 or None.  Returns (dq, dk, dv, dlog_alpha,
    db, dw, dh0) in fp32 (dh0 None when h0 is None)."""
    torch = _torch()
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    dt = _dtype_code(q)
    _need(q, "q", (B, T, H, Dk), q.dtype, dev)
    _need(k, "k", (B, T, H, Dk), q.dtype, dev)
    _need(v, "v", (B, T, H, Dv), q.dtype, dev)
    _need(log_alpha, "log_alpha", (B, T, H, Dk), torch.float32, dev)
    _need(b, "b", (B, T, H, Dk), q.dtype, dev)
    _need(w, "w", (B, T, H, Dv), q.dtype, dev)
    _need(do, "do", (B, T, H, Dv), torch.float32, dev)
    if h0 is not None:
        _need(h0, "h0", (B, H, Dk, Dv), torch.float32, dev)
    if dht is not None:
        _need(dht, "dht", (B, H, Dk, Dv), torch.float32, dev)
    if scale is None:
        scale = Dk ** -0.5
    f32 = torch.float32
    dq = torch.empty((B, T, H, Dk), dtype=f32, device=dev)
    dk = torch.empty((B, T, H, Dk), dtype=f32, device=dev)
    dla = torch.empty((B, T, H, Dk), dtype=f32, device=dev)
    db = torch.empty((B, T, H, Dk), dtype=f32, device=dev)
    dv = torch.empty((B, T, H, Dv), dtype=f32, device=dev)
    dw = torch.empty((B, T, H, Dv), dtype=f32, device=dev)
    dh0 = torch.empty((B, H, Dk, Dv), dtype=f32, device=dev) if h0 is not None else None
    nbytes = gdn2_chunk_bwd_workspace(B, T, H, Dk, Dv, dt)
    if workspace is None:
        _hold, ws = _workspace(nbytes, dev)
    else:
        ws = workspace
    _check(load().gdn2_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w), _ptr(h0), _ptr(do),
                                 _ptr(dht), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dla), _ptr(db), _ptr(dw), _ptr(dh0),
                                 B, T, H, Dk, Dv, dt, float(scale), _ptr(ws), ws.numel(), _stream(dev)),
           "gdn2_chunk_bwd")
    return dq, dk, dv, dla, db, dw, dh0


def gdn_chunk_intra(k, g, beta, G2_out=None, Tinv_out=None):
    """State-independent chunk stage: returns (G2 [B,H,NT,64], Tinv [B,H,NT,64,64]) fp32,
    Tinv = (I + A)^-1 - I per chunk.  Preallocated outputs may be passed in."""
    torch = _torch()
    B, T, H, Dk = k.shape
    dev = k.device
    dt = _dtype_code(k)
    _need(k, "k", (B, T, H, Dk), k.dtype, dev)
    _need(g, "g", (B, T, H), torch.float32, dev)
    _need(beta, "beta", (B, T, H), torch.float32, dev)
    NT = (T + BT - 1) // BT
    G2 = G2_out if G2_out is not None else torch.empty((B, H, NT, BT), dtype=torch.float32, device=dev)
    Tinv = Tinv_out if Tinv_out is not None else torch.empty((B, H, NT, BT, BT), dtype=torch.float32, device=dev)
    _need(G2, "G2_out", (B, H, NT, BT), torch.float32, dev)
    _need(Tinv, "Tinv_out", (B, H, NT, BT, BT), torch.float32, dev)
    _check(load().gdn_chunk_intra(_ptr(k), _ptr(g), _ptr(beta), _ptr(G2), _ptr(Tinv), B, T, H, Dk, dt,
                                  _stream(dev)), "gdn_chunk_intra")
    return G2, Tinv


def gdn_chunk_walk(q, k, v, beta, G2, Tinv, h0=None, scale=None, output_final_state=True, out=None,
                   final_state=None):
    """Sequential stage of the chunked forward on the outputs of gdn_chunk_intra.
    Returns (o fp32, ht or None)."""
    torch = _torch()
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    dt = _dtype_code(q)
    NT = (T + BT - 1) // BT
    _need(q, "q", (B, T, H, Dk), q.dtype, dev)
    _need(k, "k", (B, T, H, Dk), q.dtype, dev)
    _need(v, "v", (B, T, H, Dv), q.dtype, dev)
    _need(beta, "beta", (B, T, H), torch.float32, dev)
    _need(G2, "G2", (B, H, NT, BT), torch.float32, dev)
    _need(Tinv, "Tinv", (B, H, NT, BT, BT), torch.float32, dev)
    if h0 is not None:
        _need(h0, "h0", (B, H, Dk, Dv), torch.float32, dev)
    if scale is None:
        scale = Dk ** -0.5
    o = out if out is not None else torch.empty((B, T, H, Dv), dtype=torch.float32, device=dev)
    _need(o, "out", (B, T, H, Dv), torch.float32, dev)
    ht = None
    if output_final_state:
        ht = final_state if final_state is not None else torch.empty((B, H, Dk, Dv), dtype=torch.float32,
                                                                     device=dev)
        _need(ht, "final_state", (B, H, Dk, Dv), torch.float32, dev)
    _check(load().gdn_chunk_walk(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(G2), _ptr(Tinv), _ptr(h0), _ptr(o),
                                 _ptr(ht), B, T, H, Dk, Dv, dt, float(scale), _stream(dev)), "gdn_chunk_walk")
    return o, ht


def gdn2_chunk_fwd(q, k, v, log_alpha, b, w, h0=None, scale=None, output_final_state=True, workspace=None,
                   out=None, final_state=None):
    """Chunked Gated DeltaNet-2 forward.  log_alpha [B,T,H,Dk] fp32; b [B,T,H,Dk] and
    w [B,T,H,Dv] in the dtype of q.  Returns (o fp32, ht or None)."""
    torch = _torch()
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    dt = _dtype_code(q)
    _need(q, "q", (B, T, H, Dk), q.dtype, dev)
    _need(k, "k", (B, T, H, Dk), q.dtype, dev)
    _need(v, "v", (B, T, H, Dv), q.dtype, dev)
    _need(log_alpha, "log_alpha", (B, T, H, Dk), torch.float32, dev)
    _need(b, "b", (B, T, H, Dk), q.dtype, dev)
    _need(w, "w", (B, T, H, Dv), q.dtype, dev)
    if h0 is not None:
        _need(h0, "h0", (B, H, Dk, Dv), torch.float32, dev)
    if scale is None:
        scale = Dk ** -0.5
    o = out if out is not None else torch.empty((B, T, H, Dv), dtype=torch.float32, device=dev)
    _need(o, "out", (B, T, H, Dv), torch.float32, dev)
    ht = None
    if output_final_state:
        ht = final_state if final_state is not None else torch.empty((B, H, Dk, Dv), dtype=torch.float32,
                                                                     device=dev)
        _need(ht, "final_state", (B, H, Dk, Dv), torch.float32, dev)
    lib = load()
    need = lib.gdn2_chunk_fwd_workspace(B, T, H, Dk, Dv, dt)
    if need == 0:
        _check(2, "gdn2_chunk_fwd_workspace")
    if workspace is None:
        _, ws = _workspace(need, dev)
    else:
        ws = workspace
    _check(lib.gdn2_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w), _ptr(h0), _ptr(o),
                              _ptr(ht), B, T, H, Dk, Dv, dt, float(scale), _ptr(ws),
                              ws.numel() * ws.element_size(), _stream(dev)), "gdn2_chunk_fwd")
    return o, ht


def gdn2_chunk_fwd_noalloc_max_bytes() -> int:
    """Size of the library's fixed device workspace used by gdn2_chunk_fwd_noalloc."""
    return int(load().gdn2_chunk_fwd_noalloc_max_bytes())


def gdn2_chunk_fwd_noalloc(q, k, v, log_alpha, b, w, h0=None, scale=None, out=None, final_state=None):
    """gdn2_chunk_fwd through the entry point that takes its workspace from the
    library's fixed device array instead of an argument.  `out` (and
    `final_state`, when the final state is wanted) should be preallocated by
    callers that cannot allocate; otherwise they are allocated here with torch
    (the C entry point itself allocates nothing).  Returns (o, ht or None)."""
    torch = _torch()
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    dt = _dtype_code(q)
    _need(q, "q", (B, T, H, Dk), q.dtype, dev)
    _need(k, "k", (B, T, H, Dk), q.dtype, dev)
    _need(v, "v", (B, T, H, Dv), q.dtype, dev)
    _need(log_alpha, "log_alpha", (B, T, H, Dk), torch.float32, dev)
    _need(b, "b", (B, T, H, Dk), q.dtype, dev)
    _need(w, "w", (B, T, H, Dv), q.dtype, dev)
    if h0 is not None:
        _need(h0, "h0", (B, H, Dk, Dv), torch.float32, dev)
    if scale is None:
        scale = Dk ** -0.5
    o = out if out is not None else torch.empty((B, T, H, Dv), dtype=torch.float32, device=dev)
    _need(o, "out", (B, T, H, Dv), torch.float32, dev)
    ht = final_state
    if ht is not None:
        _need(ht, "final_state", (B, H, Dk, Dv), torch.float32, dev)
    _check(load().gdn2_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w), _ptr(h0),
                                         _ptr(o), _ptr(ht), B, T, H, Dk, Dv, dt, float(scale), _stream(dev)),
           "gdn2_chunk_fwd_noalloc")
    return o, ht


def gdn_recurrent_step(q, k, v, g, beta, S, scale=None, out=None):
    """One decode token: q, k [B,H,Dk], v [B,H,Dv], g, beta [B,H] fp32, S [B,H,Dk,Dv] fp32
    updated in place.  Returns o [B,H,Dv] fp32."""
    torch = _torch()
    B, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    dt = _dtype_code(q)
    _need(q, "q", (B, H, Dk), q.dtype, dev)
    _need(k, "k", (B, H, Dk), q.dtype, dev)
    _need(v, "v", (B, H, Dv), q.dtype, dev)
    _need(g, "g", (B, H), torch.float32, dev)
    _need(beta, "beta", (B, H), torch.float32, dev)
    _need(S, "S", (B, H, Dk, Dv), torch.float32, dev)
    if scale is None:
        scale = Dk ** -0.5
    o = out if out is not None else torch.empty((B, H, Dv), dtype=torch.float32, device=dev)
    _need(o, "out", (B, H, Dv), torch.float32, dev)
    _check(load().gdn_recurrent_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S), _ptr(o),
                                     B, H, Dk, Dv, dt, float(scale), _stream(dev)), "gdn_recurrent_step")
    return o


def gdn2_recurrent_step(q, k, v, log_alpha, b, w, S, scale=None, out=None):
    """One GDN-2 decode token: q, k, b [B,H,Dk] and v, w [B,H,Dv] in the path dtype,
    log_alpha [B,H,Dk] fp32, S [B,H,Dk,Dv] fp32 updated in place.  Returns o [B,H,Dv] fp32."""
    torch = _torch()
    B, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    dt = _dtype_code(q)
    _need(q, "q", (B, H, Dk), q.dtype, dev)
    _need(k, "k", (B, H, Dk), q.dtype, dev)
    _need(v, "v", (B, H, Dv), q.dtype, dev)
    _need(log_alpha, "log_alpha", (B, H, Dk), torch.float32, dev)
    _need(b, "b", (B, H, Dk), q.dtype, dev)
    _need(w, "w", (B, H, Dv), q.dtype, dev)
    _need(S, "S", (B, H, Dk, Dv), torch.float32, dev)
    if scale is None:
        scale = Dk ** -0.5
    o = out if out is not None else torch.empty((B, H, Dv), dtype=torch.float32, device=dev)
    _need(o, "out", (B, H, Dv), torch.float32, dev)
    _check(load().gdn2_recurrent_step(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w), _ptr(S),
                                      _ptr(o), B, H, Dk, Dv, dt, float(scale), _stream(dev)), "gdn2_recurrent_step")
    return o


def gdn_prologue(xq, xk, xv, a, b, wq, wk, wv, A_log, dt_bias, conv_state=None, update_conv_state=False):
    """Short convolution, SiLU, q/k L2 norm and gates in one pass.  xq, xk [B,T,H,Dk] and
    xv [B,T,H,Dv] bf16; a, b [B,T,H] fp32; wq, wk [H*Dk,4], wv [H*Dv,4], A_log, dt_bias [H]
    fp32; conv_state [B,3,H*(2Dk+Dv)] fp32 or None.  Returns (q, k, v bf16, g, beta fp32,
    new conv state or None); with update_conv_state the new state overwrites conv_state."""
    torch = _torch()
    B, T, H, Dk = xq.shape
    Dv = xv.shape[-1]
    dev = xq.device
    bf, f32 = torch.bfloat16, torch.float32
    _need(xq, "xq", (B, T, H, Dk), bf, dev)
    _need(xk, "xk", (B, T, H, Dk), bf, dev)
    _need(xv, "xv", (B, T, H, Dv), bf, dev)
    _need(a, "a", (B, T, H), f32, dev)
    _need(b, "b", (B, T, H), f32, dev)
    _need(wq, "wq", (H * Dk, 4), f32, dev)
    _need(wk, "wk", (H * Dk, 4), f32, dev)
    _need(wv, "wv", (H * Dv, 4), f32, dev)
    _need(A_log, "A_log", (H,), f32, dev)
    _need(dt_bias, "dt_bias", (H,), f32, dev)
    C = H * (2 * Dk + Dv)
    if conv_state is not None:
        _need(conv_state, "conv_state", (B, 3, C), f32, dev)
    if update_conv_state:
        if conv_state is None:
            raise ValueError("update_conv_state needs conv_state")
        new_state = conv_state
    else:
        new_state = torch.empty((B, 3, C), dtype=f32, device=dev)
    q = torch.empty((B, T, H, Dk), dtype=bf, device=dev)
    k = torch.empty((B, T, H, Dk), dtype=bf, device=dev)
    v = torch.empty((B, T, H, Dv), dtype=bf, device=dev)
    g = torch.empty((B, T, H), dtype=f32, device=dev)
    beta = torch.empty((B, T, H), dtype=f32, device=dev)
    _check(load().gdn_prologue(_ptr(xq), _ptr(xk), _ptr(xv), _ptr(a), _ptr(b), _ptr(wq), _ptr(wk), _ptr(wv),
                               _ptr(A_log), _ptr(dt_bias), _ptr(conv_state), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                               _ptr(beta), _ptr(new_state), B, T, H, Dk, Dv, _stream(dev)), "gdn_prologue")
    return q, k, v, g, beta, new_state


def gdn_gated_rmsnorm(o, z, weight, eps=1e-5, out=None):
    """y = o / sqrt(mean(o^2) + eps) * weight * SiLU(z) over the last axis.  o [..., Dv]
    fp32, z [..., Dv] bf16, weight [Dv] fp32.  Returns y [..., Dv] bf16."""
    torch = _torch()
    Dv = o.shape[-1]
    dev = o.device
    _need(o, "o", tuple(o.shape), torch.float32, dev)
    _need(z, "z", tuple(o.shape), torch.bfloat16, dev)
    _need(weight, "weight", (Dv,), torch.float32, dev)
    y = out if out is not None else torch.empty(o.shape, dtype=torch.bfloat16, device=dev)
    _need(y, "out", tuple(o.shape), torch.bfloat16, dev)
    rows = o.numel() // Dv
    _check(load().gdn_gated_rmsnorm(_ptr(o), _ptr(z), _ptr(weight), _ptr(y), rows, Dv, float(eps), _stream(dev)),
           "gdn_gated_rmsnorm")
    return y


def clock_probe(nblocks=256, spin_us=2000, device="cuda"):
    """Enqueue the clock probe (measurement aid) on torch's current stream and
    return a device tensor [nblocks, 2] int64 of (shader cycles, 100 MHz ticks);
    read it after the stream has run: clock_MHz = 100 * cycles / ticks."""
    torch = _torch()
    out = torch.zeros((nblocks, 2), dtype=torch.int64, device=device)
    _check(load().gdn_clock_probe(_ptr(out), int(nblocks), int(spin_us), _stream(out.device)), "gdn_clock_probe")
    return out
