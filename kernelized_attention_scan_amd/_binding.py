"""ctypes binding of liblinattn.so (the C ABI declared in include/linattn.h).

Argument marshalling only: tensor checks, raw device pointers, the caller's
current HIP stream, and a workspace tensor from torch's allocator.  Every step
of the computation runs in the library's HIP kernels; there is no fallback.
If the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

import torch

(LA_OK, LA_ERR_INVALID_ARG, LA_ERR_UNSUPPORTED, LA_ERR_WORKSPACE, LA_ERR_HIP,
 LA_ERR_EXCHANGE) = range(6)
MAP_IDENTITY, MAP_ELU1, MAP_PERFORMER = 0, 1, 2
LA_F32, LA_BF16 = 0, 1
LD_CHANNEL, LD_POSITION, LD_BOTH = 0, 1, 2
_LAYOUTS = {"channel": LD_CHANNEL, "position": LD_POSITION, "both": LD_BOTH}

_MAPS = {"identity": MAP_IDENTITY, "elu1": MAP_ELU1, "performer": MAP_PERFORMER}
_DTYPES = {torch.float32: LA_F32, torch.bfloat16: LA_BF16}

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                        "liblinattn.so")

# Exported symbols, in the order include/linattn.h declares them.
SYMBOLS = ("la_featmap", "la_forward_workspace_bytes", "la_forward",
           "la_forward_state", "la_forward_train", "la_backward",
           "la_backward_workspace_bytes",
           "la_forward_gated", "la_forward_gated_train", "la_backward_gated",
           "la_backward_gated_workspace_bytes",
           "la_forward_gated_workspace_bytes",
           "la_forward_noalloc",
           "la_decode_step", "la_decode_step_gated", "la_workspace_check",
           "la_set_exchange_spin_limit", "la_status_str", "la_last_error")

_lock = threading.Lock()
_lib = None
# Zero-initialised workspaces, one per (device, stream): the library keeps the
# synchronisation area at their start zero between calls, so a workspace is
# zeroed once when it is allocated and then reused by every call on that
# stream.
_workspaces = {}


class LinAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load liblinattn.so once; raise if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build the HIP library first "
                "(python -m kernelized_attention_scan_amd.build)")
        lib = ctypes.CDLL(path)
        vp, i32, i64, sz = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                            ctypes.c_size_t)
        lib.la_featmap.argtypes = [vp, vp, vp, i64, i32, i32, i32, i32, i32, vp]
        lib.la_featmap.restype = i32
        lib.la_forward_workspace_bytes.argtypes = [i32, i32, i64, i32, i32,
                                                   i32, i32, i32]
        lib.la_forward_workspace_bytes.restype = sz
        lib.la_forward.argtypes = [vp, vp, vp, vp, i32, i32, i64, i32, i32,
                                   i32, vp, vp, i32, i32, vp, vp]
        lib.la_forward.restype = i32
        lib.la_forward_state.argtypes = [vp, vp, vp, vp, i32, i32, i64, i32,
                                         i32, i32, vp, vp, i32, i32, vp, vp,
                                         vp, vp]
        lib.la_forward_state.restype = i32
        lib.la_forward_train.argtypes = [vp, vp, vp, vp, vp, i32, i32, i64,
                                         i32, i32, i32, vp, vp, i32, vp, vp]
        lib.la_forward_train.restype = i32
        lib.la_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32,
                                    i32, i64, i32, i32, i32, vp, vp, i32, vp,
                                    vp]
        lib.la_backward.restype = i32
        lib.la_backward_workspace_bytes.argtypes = [i32, i32, i64, i32, i32,
                                                    i32, i32]
        lib.la_backward_workspace_bytes.restype = sz
        lib.la_forward_gated.argtypes = [vp, vp, vp, vp, i32, i32, i64, i32,
                                         i32, i32, vp, vp, i32, i32, i32, vp,
                                         vp, vp, vp]
        lib.la_forward_gated.restype = i32
        lib.la_forward_gated_train.argtypes = [vp, vp, vp, vp, vp, i32, i32,
                                               i64, i32, i32, i32, vp, vp,
                                               i32, i32, vp, vp]
        lib.la_forward_gated_train.restype = i32
        lib.la_backward_gated.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                          i32, i32, i64, i32, i32, i32, vp,
                                          vp, i32, i32, vp, vp]
        lib.la_backward_gated.restype = i32
        lib.la_backward_gated_workspace_bytes.argtypes = [i32, i32, i64, i32,
                                                          i32, i32, i32]
        lib.la_backward_gated_workspace_bytes.restype = sz
        lib.la_forward_gated_workspace_bytes.argtypes = [
            i32, i32, i64, i32, i32, i32, i32, i32, i32]
        lib.la_forward_gated_workspace_bytes.restype = sz
        lib.la_decode_step_gated.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32,
                                             i32, i32, i32, vp, vp, i32, i32,
                                             vp]
        lib.la_decode_step_gated.restype = i32
        lib.la_forward_noalloc.argtypes = [vp, vp, vp, vp, i32, i32, i64, i32,
                                           i32, i32, vp, vp, i32, i32, vp]
        lib.la_forward_noalloc.restype = i32
        lib.la_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32,
                                       i32, i32, vp, vp, i32, vp]
        lib.la_decode_step.restype = i32
        lib.la_workspace_check.argtypes = [vp, vp]
        lib.la_workspace_check.restype = i32
        lib.la_set_exchange_spin_limit.argtypes = [ctypes.c_uint]
        lib.la_set_exchange_spin_limit.restype = None
        lib.la_status_str.argtypes = [i32]
        lib.la_status_str.restype = ctypes.c_char_p
        lib.la_last_error.argtypes = []
        lib.la_last_error.restype = ctypes.c_char_p
        _lib = lib
        return lib


def _check(status: int, what: str) -> None:
    if status != LA_OK:
        lib = load_library()
        msg = lib.la_last_error().decode()
        name = lib.la_status_str(status).decode()
        raise LinAttnError(status, f"{what}: {name}: {msg}")


def _map_code(feature_map) -> int:
    if isinstance(feature_map, int):
        return feature_map
    try:
        return _MAPS[feature_map]
    except KeyError:
        raise ValueError(f"unknown feature map {feature_map!r}") from None


def _dtype_code(t: torch.dtype) -> int:
    try:
        return _DTYPES[t]
    except KeyError:
        raise TypeError(f"unsupported storage dtype {t}") from None


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, name: str) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _check_out(out: torch.Tensor, shape, dtype) -> None:
    """A caller-supplied out must have the expected shape and dtype (one of
    another size would be written past its end)."""
    if tuple(out.shape) != tuple(shape):
        raise ValueError(f"out has shape {tuple(out.shape)}, expected "
                         f"{tuple(shape)}")
    if out.dtype != dtype:
        raise TypeError(f"out has dtype {out.dtype}, expected {dtype}")


def _check_omega(omega: Optional[torch.Tensor], mapk: int, d: int) -> int:
    """omega must be fp32 [d, m] for the Performer map; returns m (0 when
    the map needs no omega)."""
    if mapk != MAP_PERFORMER:
        return 0
    if omega is None:
        raise ValueError("the performer map needs omega [d, m]")
    if omega.dtype != torch.float32:
        raise TypeError("omega must be float32")
    if omega.dim() != 2 or omega.shape[0] != d:
        raise ValueError(f"omega must be [d={d}, m], got {tuple(omega.shape)}")
    return int(omega.shape[1])


def _check_decay(decay: Optional[torch.Tensor], H: int) -> None:
    if decay is None:
        return
    if decay.dtype != torch.float32:
        raise TypeError("decay must be float32")
    if decay.dim() != 1 or decay.shape[0] != H:
        raise ValueError(f"decay must be [H={H}], got {tuple(decay.shape)}")


def _on_gpu(ref: torch.Tensor, *named) -> None:
    """Every given tensor is a contiguous GPU tensor on ref's device."""
    for t, name in named:
        if t is None:
            continue
        _dev(t, name)
        if t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, expected {ref.device}")


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _workspace(need: int, device) -> torch.Tensor:
    key = (device.index, torch.cuda.current_stream(device).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < need:
        ws = torch.zeros(need, dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def new_workspace(B: int, H: int, n: int, d: int, d_feat: int,
                  feature_map="elu1", dtype=torch.bfloat16, causal: bool = True,
                  device="cuda") -> torch.Tensor:
    """A zero-initialised workspace for forward() with these sizes (its
    synchronisation area must be zero before the first call; calls keep it
    so)."""
    need = forward_workspace_bytes(B, H, n, d, d_feat, feature_map, dtype,
                                   causal)
    return torch.zeros(max(need, 1), dtype=torch.uint8, device=device)


def forward_workspace_bytes(B: int, H: int, n: int, d: int, d_feat: int,
                            feature_map="elu1", dtype=torch.bfloat16,
                            causal: bool = True) -> int:
    """Device workspace la_forward needs (0 if none or if rejected)."""
    return int(load_library().la_forward_workspace_bytes(
        B, H, n, d, d_feat, _map_code(feature_map), _dtype_code(dtype),
        int(bool(causal))))


def gated_workspace_bytes(B: int, H: int, n: int, d: int, d_feat: int,
                          feature_map="elu1", layout="position",
                          dtype=torch.bfloat16, causal: bool = True) -> int:
    """Device workspace la_forward_gated needs for this decay layout (0 if
    none or if rejected)."""
    return int(load_library().la_forward_gated_workspace_bytes(
        B, H, n, d, d_feat, _map_code(feature_map), _layout_code(layout),
        _dtype_code(dtype), int(bool(causal))))


def featmap(x: torch.Tensor, feature_map="elu1", omega=None,
            out_dtype: Optional[torch.dtype] = None,
            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """phi row by row over the last axis: [..., d] -> [..., d_feat]."""
    lib = load_library()
    mapk = _map_code(feature_map)
    d = x.shape[-1]
    m = _check_omega(omega, mapk, d) or d
    out_dtype = out_dtype or x.dtype
    _dtype_code(x.dtype)
    _dtype_code(out_dtype)
    if out is not None:
        _check_out(out, x.shape[:-1] + (m,), out.dtype)
        _dtype_code(out.dtype)
    _on_gpu(x, (x, "x"), (out, "out"), (omega, "omega"))
    if out is None:
        out = torch.empty(x.shape[:-1] + (m,), dtype=out_dtype, device=x.device)
    st = lib.la_featmap(_ptr(x), _ptr(out), _ptr(omega), x.numel() // d, d, m,
                        mapk, _dtype_code(x.dtype), _dtype_code(out.dtype),
                        _stream(x.device))
    _check(st, "la_featmap")
    return out


def forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
            feature_map="elu1", omega: Optional[torch.Tensor] = None,
            decay: Optional[torch.Tensor] = None, causal: bool = True,
            out: Optional[torch.Tensor] = None,
            workspace: Optional[torch.Tensor] = None,
            mu_out: Optional[torch.Tensor] = None,
            nu_out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Kernelized linear attention over q, k [B,H,n,d_qk], v [B,H,n,d].

    workspace: optional uint8 device tensor from new_workspace(); by default a
    cached zero-initialised one per (device, stream) is used.
    mu_out [B,H,d_feat,d], nu_out [B,H,d_feat] (fp32, both or neither):
    receive the state after the last position (la_forward_state), the state
    decode_step continues from."""
    lib = load_library()
    if q.dim() != 4 or v.dim() != 4 or q.shape != k.shape:
        raise ValueError("q, k must be [B,H,n,d_qk] and v [B,H,n,d]")
    B, H, n, d = v.shape
    if q.shape[:3] != v.shape[:3]:
        raise ValueError("q, k, v disagree on B, H, n")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    _dtype_code(v.dtype)
    mapk = _map_code(feature_map)
    if mapk != MAP_IDENTITY and q.shape[-1] != d:
        raise ValueError("q, k must have width d for elu1 and performer")
    d_feat = _check_omega(omega, mapk, d) or q.shape[-1]
    _check_decay(decay, H)
    if out is not None:
        _check_out(out, v.shape, v.dtype)
    if (mu_out is None) != (nu_out is None):
        raise ValueError("mu_out and nu_out go together")
    if mu_out is not None:
        if mu_out.dtype != torch.float32 or nu_out.dtype != torch.float32:
            raise TypeError("mu_out and nu_out must be float32")
        if mu_out.shape != (B, H, d_feat, d) or nu_out.shape != (B, H, d_feat):
            raise ValueError("mu_out must be [B,H,d_feat,d] and nu_out "
                             "[B,H,d_feat]")
    if workspace is not None and workspace.dtype != torch.uint8:
        raise TypeError("workspace must be a uint8 tensor")
    _on_gpu(v, (q, "q"), (k, "k"), (v, "v"), (out, "out"), (omega, "omega"),
            (decay, "decay"), (workspace, "workspace"), (mu_out, "mu_out"),
            (nu_out, "nu_out"))
    if out is None:
        out = torch.empty_like(v)
    dt = _dtype_code(v.dtype)
    need = lib.la_forward_workspace_bytes(B, H, n, d, d_feat, mapk, dt,
                                          int(bool(causal)))
    if need and workspace is None:
        workspace = _workspace(need, v.device)
    if need and workspace.numel() < need:
        raise ValueError(f"workspace of {workspace.numel()} bytes is smaller "
                         f"than the {need} bytes required")
    if mu_out is None:
        st = lib.la_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, n, d,
                            d_feat, mapk, _ptr(omega), _ptr(decay),
                            int(bool(causal)), dt,
                            _ptr(workspace) if need else None,
                            _stream(v.device))
        _check(st, "la_forward")
        return out
    st = lib.la_forward_state(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, n,
                              d, d_feat, mapk, _ptr(omega), _ptr(decay),
                              int(bool(causal)), dt,
                              _ptr(workspace) if need else None, _ptr(mu_out),
                              _ptr(nu_out), _stream(v.device))
    _check(st, "la_forward_state")
    return out


def decode_step(mu: torch.Tensor, nu: torch.Tensor, q: torch.Tensor,
                k: torch.Tensor, v: torch.Tensor, feature_map="elu1",
                omega: Optional[torch.Tensor] = None,
                decay: Optional[torch.Tensor] = None,
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One decode step; mu [S,H,d_feat,d] and nu [S,H,d_feat] are updated in
    place.  Returns out [S,H,d]."""
    lib = load_library()
    if v.dim() != 3 or mu.dim() != 4:
        raise ValueError("v must be [S,H,d] and mu [S,H,d_feat,d]")
    if mu.dtype != torch.float32 or nu.dtype != torch.float32:
        raise TypeError("mu and nu must be float32")
    S, H, d = v.shape
    d_feat = mu.shape[2]
    if mu.shape != (S, H, d_feat, d) or nu.shape != (S, H, d_feat):
        raise ValueError("mu must be [S,H,d_feat,d] and nu [S,H,d_feat]")
    mapk = _map_code(feature_map)
    m = _check_omega(omega, mapk, d)
    if mapk == MAP_PERFORMER and m != d_feat:
        raise ValueError(f"omega has {m} features, mu has d_feat={d_feat}")
    if mapk == MAP_ELU1 and d_feat != d:
        raise ValueError("elu1 keeps the width: mu must be [S,H,d,d]")
    dqk = d_feat if mapk == MAP_IDENTITY else d
    if q.shape != (S, H, dqk) or k.shape != (S, H, dqk):
        raise ValueError(f"q, k must be [S={S}, H={H}, {dqk}], got "
                         f"{tuple(q.shape)}, {tuple(k.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    _dtype_code(v.dtype)
    _check_decay(decay, H)
    if out is not None:
        _check_out(out, v.shape, v.dtype)
    _on_gpu(v, (mu, "mu"), (nu, "nu"), (q, "q"), (k, "k"), (v, "v"),
            (out, "out"), (omega, "omega"), (decay, "decay"))
    if out is None:
        out = torch.empty_like(v)
    st = lib.la_decode_step(_ptr(mu), _ptr(nu), _ptr(q), _ptr(k), _ptr(v),
                            _ptr(out), S, H, d, d_feat, mapk,
                            _ptr(omega), _ptr(decay), _dtype_code(v.dtype),
                            _stream(v.device))
    _check(st, "la_decode_step")
    return out


def workspace_check(workspace: torch.Tensor) -> None:
    """Raise LinAttnError(LA_ERR_EXCHANGE) if a segment exchange failed in a
    call that used this workspace since the last check (and clear that
    status).  Synchronises with the current stream."""
    lib = load_library()
    _on_gpu(workspace, (workspace, "workspace"))
    _check(lib.la_workspace_check(_ptr(workspace), _stream(workspace.device)),
           "la_workspace_check")


def cached_workspace(device="cuda") -> Optional[torch.Tensor]:
    """The workspace forward() uses on the current stream of `device` when no
    workspace is passed (None until a call needed one)."""
    device = torch.device(device)
    if device.index is None:
        device = torch.device(device.type, torch.cuda.current_device())
    return _workspaces.get((device.index,
                            torch.cuda.current_stream(device).cuda_stream))


def set_exchange_spin_limit(spins: int) -> None:
    """Diagnostics: polls an exchange wait makes before giving up (0 restores
    the default)."""
    load_library().la_set_exchange_spin_limit(int(spins))


def forward_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                    feature_map="elu1", omega: Optional[torch.Tensor] = None,
                    decay: Optional[torch.Tensor] = None, causal: bool = True,
                    out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """forward() through la_forward_noalloc: no workspace, the library's
    static per-GPU scratch instead (calls overlapping on one GPU race).
    `out` must be given by a caller that cannot allocate."""
    lib = load_library()
    if q.dim() != 4 or v.dim() != 4 or q.shape != k.shape:
        raise ValueError("q, k must be [B,H,n,d_qk] and v [B,H,n,d]")
    B, H, n, d = v.shape
    if q.shape[:3] != v.shape[:3]:
        raise ValueError("q, k, v disagree on B, H, n")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    dt = _dtype_code(v.dtype)
    mapk = _map_code(feature_map)
    if mapk != MAP_IDENTITY and q.shape[-1] != d:
        raise ValueError("q, k must have width d for elu1 and performer")
    d_feat = _check_omega(omega, mapk, d) or q.shape[-1]
    _check_decay(decay, H)
    if out is not None:
        _check_out(out, v.shape, v.dtype)
    _on_gpu(v, (q, "q"), (k, "k"), (v, "v"), (out, "out"), (omega, "omega"),
            (decay, "decay"))
    if out is None:
        out = torch.empty_like(v)
    st = lib.la_forward_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, n,
                                d, d_feat, mapk, _ptr(omega), _ptr(decay),
                                int(bool(causal)), dt, _stream(v.device))
    _check(st, "la_forward_noalloc")
    return out


def _layout_code(layout) -> int:
    if isinstance(layout, int):
        return layout
    try:
        return _LAYOUTS[layout]
    except KeyError:
        raise ValueError(f"unknown decay layout {layout!r}") from None


def forward_gated(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                  log_decay: torch.Tensor, layout="position",
                  feature_map="elu1", omega: Optional[torch.Tensor] = None,
                  causal: bool = True, out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None,
                  mu_out: Optional[torch.Tensor] = None,
                  nu_out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """forward() with a decay exp(log_decay) per position and/or state row
    (la_forward_gated): log_decay is fp32 [B, H, n] for layout "position",
    [H, d_feat] for "channel" and [B, H, n, d_feat] for "both"."""
    lib = load_library()
    if q.dim() != 4 or v.dim() != 4 or q.shape != k.shape:
        raise ValueError("q, k must be [B,H,n,d_qk] and v [B,H,n,d]")
    B, H, n, d = v.shape
    if q.shape[:3] != v.shape[:3]:
        raise ValueError("q, k, v disagree on B, H, n")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    dt = _dtype_code(v.dtype)
    mapk = _map_code(feature_map)
    if mapk != MAP_IDENTITY and q.shape[-1] != d:
        raise ValueError("q, k must have width d for elu1 and performer")
    d_feat = _check_omega(omega, mapk, d) or q.shape[-1]
    lay = _layout_code(layout)
    want = {LD_CHANNEL: (H, d_feat), LD_POSITION: (B, H, n),
            LD_BOTH: (B, H, n, d_feat)}[lay]
    if log_decay.dtype != torch.float32:
        raise TypeError("log_decay must be float32")
    if tuple(log_decay.shape) != want:
        raise ValueError(f"log_decay must be {want}, got "
                         f"{tuple(log_decay.shape)}")
    if out is not None:
        _check_out(out, v.shape, v.dtype)
    if (mu_out is None) != (nu_out is None):
        raise ValueError("mu_out and nu_out go together")
    if mu_out is not None:
        if mu_out.dtype != torch.float32 or nu_out.dtype != torch.float32:
            raise TypeError("mu_out and nu_out must be float32")
        if mu_out.shape != (B, H, d_feat, d) or nu_out.shape != (B, H, d_feat):
            raise ValueError("mu_out must be [B,H,d_feat,d] and nu_out "
                             "[B,H,d_feat]")
    if workspace is not None and workspace.dtype != torch.uint8:
        raise TypeError("workspace must be a uint8 tensor")
    _on_gpu(v, (q, "q"), (k, "k"), (v, "v"), (out, "out"), (omega, "omega"),
            (log_decay, "log_decay"), (workspace, "workspace"),
            (mu_out, "mu_out"), (nu_out, "nu_out"))
    if out is None:
        out = torch.empty_like(v)
    need = lib.la_forward_gated_workspace_bytes(B, H, n, d, d_feat, mapk, lay,
                                                dt, int(bool(causal)))
    if need and workspace is None:
        workspace = _workspace(need, v.device)
    if need and workspace.numel() < need:
        raise ValueError(f"workspace of {workspace.numel()} bytes is smaller "
                         f"than the {need} bytes required")
    st = lib.la_forward_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, n,
                              d, d_feat, mapk, _ptr(omega), _ptr(log_decay),
                              lay, int(bool(causal)), dt,
                              _ptr(workspace) if need else None, _ptr(mu_out),
                              _ptr(nu_out), _stream(v.device))
    _check(st, "la_forward_gated")
    return out


def decode_step_gated(mu: torch.Tensor, nu: torch.Tensor, q: torch.Tensor,
                      k: torch.Tensor, v: torch.Tensor,
                      log_decay: torch.Tensor, layout="channel",
                      feature_map="elu1", omega: Optional[torch.Tensor] = None,
                      out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """decode_step() with a decay exp(log_decay) per state row and/or per
    unit: log_decay [H, d_feat] ("channel"), [S, H] ("position") or
    [S, H, d_feat] ("both")."""
    lib = load_library()
    if v.dim() != 3 or mu.dim() != 4:
        raise ValueError("v must be [S,H,d] and mu [S,H,d_feat,d]")
    if mu.dtype != torch.float32 or nu.dtype != torch.float32:
        raise TypeError("mu and nu must be float32")
    S, H, d = v.shape
    d_feat = mu.shape[2]
    if mu.shape != (S, H, d_feat, d) or nu.shape != (S, H, d_feat):
        raise ValueError("mu must be [S,H,d_feat,d] and nu [S,H,d_feat]")
    mapk = _map_code(feature_map)
    m = _check_omega(omega, mapk, d)
    if mapk == MAP_PERFORMER and m != d_feat:
        raise ValueError(f"omega has {m} features, mu has d_feat={d_feat}")
    if mapk == MAP_ELU1 and d_feat != d:
        raise ValueError("elu1 keeps the width: mu must be [S,H,d,d]")
    dqk = d_feat if mapk == MAP_IDENTITY else d
    if q.shape != (S, H, dqk) or k.shape != (S, H, dqk):
        raise ValueError(f"q, k must be [S={S}, H={H}, {dqk}]")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    _dtype_code(v.dtype)
    lay = _layout_code(layout)
    want = {LD_CHANNEL: (H, d_feat), LD_POSITION: (S, H),
            LD_BOTH: (S, H, d_feat)}[lay]
    if log_decay.dtype != torch.float32:
        raise TypeError("log_decay must be float32")
    if tuple(log_decay.shape) != want:
        raise ValueError(f"log_decay must be {want}, got "
                         f"{tuple(log_decay.shape)}")
    if out is not None:
        _check_out(out, v.shape, v.dtype)
    _on_gpu(v, (mu, "mu"), (nu, "nu"), (q, "q"), (k, "k"), (v, "v"),
            (out, "out"), (omega, "omega"), (log_decay, "log_decay"))
    if out is None:
        out = torch.empty_like(v)
    st = lib.la_decode_step_gated(_ptr(mu), _ptr(nu), _ptr(q), _ptr(k),
                                  _ptr(v), _ptr(out), S, H, d, d_feat, mapk,
                                  _ptr(omega), _ptr(log_decay), lay,
                                  _dtype_code(v.dtype), _stream(v.device))
    _check(st, "la_decode_step_gated")
    return out


def forward_train(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                  feature_map="elu1", decay: Optional[torch.Tensor] = None,
                  out: Optional[torch.Tensor] = None,
                  den: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None,
                  omega: Optional[torch.Tensor] = None,
                  log_decay: Optional[torch.Tensor] = None):
    """The causal forward for training (la_forward_train): returns (out,
    den), den [B,H,n] fp32 being each row's denominator, which backward()
    takes.  omega: fp32 [d, m] for the performer map.  log_decay: fp32
    [B, H, n], a decay exp(log_decay) per position in place of decay
    (la_forward_gated_train)."""
    lib = load_library()
    if q.dim() != 4 or v.dim() != 4 or q.shape != k.shape:
        raise ValueError("q, k must be [B,H,n,d_qk] and v [B,H,n,d]")
    B, H, n, d = v.shape
    if q.shape[:3] != v.shape[:3]:
        raise ValueError("q, k, v disagree on B, H, n")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    dt = _dtype_code(v.dtype)
    mapk = _map_code(feature_map)
    if mapk != MAP_IDENTITY and q.shape[-1] != d:
        raise ValueError("q, k must have width d for elu1 and performer")
    d_feat = _check_omega(omega, mapk, d) or q.shape[-1]
    _check_decay(decay, H)
    _check_position_decay(log_decay, decay, B, H, n)
    if out is not None:
        _check_out(out, v.shape, v.dtype)
    if den is not None and (den.dtype != torch.float32 or
                            tuple(den.shape) != (B, H, n)):
        raise ValueError("den must be float32 [B, H, n]")
    _on_gpu(v, (q, "q"), (k, "k"), (v, "v"), (out, "out"), (den, "den"),
            (decay, "decay"), (workspace, "workspace"), (omega, "omega"),
            (log_decay, "log_decay"))
    if out is None:
        out = torch.empty_like(v)
    if den is None:
        den = torch.empty((B, H, n), dtype=torch.float32, device=v.device)
    need = lib.la_forward_workspace_bytes(B, H, n, d, d_feat, mapk, dt, 1)
    if need and workspace is None:
        workspace = _workspace(need, v.device)
    if need and workspace.numel() < need:
        raise ValueError("workspace too small")
    if log_decay is not None:
        st = lib.la_forward_gated_train(
            _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(den), B, H, n, d,
            d_feat, mapk, _ptr(omega), _ptr(log_decay), LD_POSITION, dt,
            _ptr(workspace) if need else None, _stream(v.device))
        _check(st, "la_forward_gated_train")
        return out, den
    st = lib.la_forward_train(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(den),
                              B, H, n, d, d_feat, mapk, _ptr(omega),
                              _ptr(decay), dt,
                              _ptr(workspace) if need else None,
                              _stream(v.device))
    _check(st, "la_forward_train")
    return out, den


def _check_position_decay(log_decay, decay, B, H, n):
    """A decay per position: fp32 [B, H, n], not together with decay."""
    if log_decay is None:
        return
    if decay is not None:
        raise ValueError("pass decay or log_decay, not both")
    if log_decay.dtype != torch.float32:
        raise TypeError("log_decay must be float32")
    if tuple(log_decay.shape) != (B, H, n) or not log_decay.is_contiguous():
        raise ValueError(f"log_decay must be contiguous [B, H, n] = "
                         f"{(B, H, n)}, got {tuple(log_decay.shape)}")


def backward_workspace_bytes(B: int, H: int, n: int, d: int,
                             feature_map="elu1",
                             dtype: torch.dtype = torch.bfloat16,
                             d_feat: Optional[int] = None,
                             gated: bool = False) -> int:
    """Device workspace la_backward needs (la_backward_workspace_bytes), or
    with gated la_backward_gated (la_backward_gated_workspace_bytes); d_feat
    defaults to d (the performer map's m otherwise)."""
    lib = load_library()
    fn = (lib.la_backward_gated_workspace_bytes if gated
          else lib.la_backward_workspace_bytes)
    return int(fn(B, H, n, d, d if d_feat is None else d_feat,
                  _map_code(feature_map), _dtype_code(dtype)))


# backward()'s workspaces when none is passed: one per (device, stream),
# grown as needed (no initial contents are needed)
_bwd_workspaces = {}


def backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
             out: torch.Tensor, den: torch.Tensor, dout: torch.Tensor,
             feature_map="elu1", decay: Optional[torch.Tensor] = None,
             dq: Optional[torch.Tensor] = None,
             dk: Optional[torch.Tensor] = None,
             dv: Optional[torch.Tensor] = None,
             workspace: Optional[torch.Tensor] = None,
             omega: Optional[torch.Tensor] = None,
             log_decay: Optional[torch.Tensor] = None):
    """Gradients (dq, dk, dv) of sum(out * dout) for the causal forward
    (la_backward); out and den as forward_train() returned them.  omega:
    fp32 [d, m] for the performer map (not differentiated).  log_decay: fp32
    [B, H, n], the forward's decay per position (la_backward_gated; not
    differentiated).
    workspace: optional uint8 device tensor of at least
    backward_workspace_bytes(...) bytes; by default one cached per (device,
    stream) is used."""
    lib = load_library()
    if q.dim() != 4 or v.dim() != 4 or q.shape != k.shape:
        raise ValueError("q, k must be [B,H,n,d] and v [B,H,n,d]")
    B, H, n, d = v.shape
    if q.shape != v.shape:
        raise ValueError("la_backward needs q, k, v of one shape")
    for t, nm in ((out, "out"), (dout, "dout")):
        if t.shape != v.shape or t.dtype != v.dtype:
            raise ValueError(f"{nm} must match v in shape and dtype")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    if den.dtype != torch.float32 or tuple(den.shape) != (B, H, n):
        raise ValueError("den must be float32 [B, H, n]")
    dt = _dtype_code(v.dtype)
    mapk = _map_code(feature_map)
    d_feat = _check_omega(omega, mapk, d) or d
    _check_decay(decay, H)
    _check_position_decay(log_decay, decay, B, H, n)
    for t, nm in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        if t is not None:
            _check_out(t, v.shape, v.dtype)
    gated = log_decay is not None
    need = int((lib.la_backward_gated_workspace_bytes if gated
                else lib.la_backward_workspace_bytes)(B, H, n, d, d_feat,
                                                      mapk, dt))
    if workspace is not None and (workspace.dtype != torch.uint8
                                  or not workspace.is_contiguous()
                                  or workspace.numel() < need):
        raise ValueError(f"workspace must be a contiguous uint8 tensor of "
                         f"at least {need} bytes")
    _on_gpu(v, (q, "q"), (k, "k"), (v, "v"), (out, "out"), (den, "den"),
            (dout, "dout"), (decay, "decay"), (dq, "dq"), (dk, "dk"),
            (dv, "dv"), (workspace, "workspace"), (omega, "omega"),
            (log_decay, "log_decay"))
    if workspace is None and need > 0:
        key = (v.device.index, torch.cuda.current_stream(v.device).cuda_stream)
        workspace = _bwd_workspaces.get(key)
        if workspace is None or workspace.numel() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=v.device)
            _bwd_workspaces[key] = workspace
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if gated:
        st = lib.la_backward_gated(
            _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(den), _ptr(dout),
            _ptr(dq), _ptr(dk), _ptr(dv), B, H, n, d, d_feat, mapk,
            _ptr(omega), _ptr(log_decay), LD_POSITION, dt, _ptr(workspace),
            _stream(v.device))
        _check(st, "la_backward_gated")
        return dq, dk, dv
    st = lib.la_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(den),
                         _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), B, H, n, d,
                         d_feat, mapk, _ptr(omega), _ptr(decay), dt,
                         _ptr(workspace), _stream(v.device))
    _check(st, "la_backward")
    return dq, dk, dv


class _LinearAttention(torch.autograd.Function):
    """forward_train() forward, backward() gradients (no arithmetic here)."""

    @staticmethod
    def forward(ctx, q, k, v, feature_map, decay, omega, log_decay):
        out, den = forward_train(q.contiguous(), k.contiguous(),
                                 v.contiguous(), feature_map, decay=decay,
                                 omega=omega, log_decay=log_decay)
        ctx.save_for_backward(q, k, v, out, den)
        ctx.feature_map = feature_map
        ctx.decay = decay
        ctx.omega = omega
        ctx.log_decay = log_decay
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, out, den = ctx.saved_tensors
        dq, dk, dv = backward(q.contiguous(), k.contiguous(), v.contiguous(),
                              out, den, dout.contiguous(), ctx.feature_map,
                              decay=ctx.decay, omega=ctx.omega,
                              log_decay=ctx.log_decay)
        return dq, dk, dv, None, None, None, None


def linear_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                     feature_map="elu1",
                     decay: Optional[torch.Tensor] = None,
                     omega: Optional[torch.Tensor] = None,
                     log_decay: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Causal kernelized linear attention as a differentiable torch op:
    la_forward_train forward, la_backward gradients for q, k and v (decay,
    log_decay and omega are not differentiated).  elu1 or identity features
    with d_feat == d, or the performer map with omega fp32 [d, m];
    log_decay fp32 [B, H, n] (a decay per position: la_forward_gated_train
    and la_backward_gated, elu1 or identity) in place of decay."""
    return _LinearAttention.apply(q, k, v, feature_map, decay, omega,
                                  log_decay)
