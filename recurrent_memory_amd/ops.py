"""Thin ctypes binding of ``libdeltarule.so`` (see include/deltarule.h).

Argument marshalling only: shapes and dtypes of torch device tensors are
checked, outputs are allocated with torch when not supplied, and the call is
enqueued on the current HIP stream.  Every step of the computation runs in the
library's gfx950 kernels; there is no fallback.  If the library is missing the
import-time loader raises.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdeltarule.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "deltarule.h")

ABI_VERSION = 5   # DR_ABI_VERSION of the header this binding follows
VARIANTS = {"deltanet": 0, "gdn": 1, "kda": 2, "gdn2": 3, "fg2": 4}
# forms whose beta is one value per key channel (the erase gate, or the step sizes)
_CHANNEL_BETA = ("gdn2", "fg2")
DTYPES = {torch.float32: 0, torch.bfloat16: 1}
STATUS = {0: "DR_OK", 1: "DR_E_NULLPTR", 2: "DR_E_SHAPE", 3: "DR_E_UNSUPPORTED",
          4: "DR_E_ALIGN", 5: "DR_E_DEVICE", 6: "DR_E_LAUNCH", 7: "DR_E_ALIAS",
          8: "DR_E_WORKSPACE"}


class DrDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("variant", ctypes.c_int32), ("dtype", ctypes.c_int32), ("H_k", ctypes.c_int32)]


class DeltaRuleError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load (once) and type the C ABI.  Raises if the library was not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m recurrent_memory_amd.build`")
    lib = ctypes.CDLL(path)
    vp = ctypes.c_void_p
    sz = ctypes.c_size_t
    for name in ("delta_fwd_workspace_bytes", "delta_bwd_workspace_bytes",
                 "delta_ttt_pre_workspace_bytes"):
        getattr(lib, name).argtypes = [ctypes.POINTER(DrDesc), ctypes.POINTER(sz)]
        getattr(lib, name).restype = ctypes.c_int
    lib.delta_fwd.argtypes = [ctypes.POINTER(DrDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.delta_fwd.restype = ctypes.c_int
    lib.delta_fwd_noalloc.argtypes = [ctypes.POINTER(DrDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.delta_fwd_noalloc.restype = ctypes.c_int
    lib.delta_decode.argtypes = [ctypes.POINTER(DrDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.delta_decode.restype = ctypes.c_int
    lib.delta_bwd.argtypes = [ctypes.POINTER(DrDesc)] + [vp] * 17 + [sz, vp]
    lib.delta_bwd.restype = ctypes.c_int
    lib.delta_efla_beta.argtypes = [ctypes.POINTER(DrDesc), vp, vp, vp, vp]
    lib.delta_efla_beta.restype = ctypes.c_int
    lib.delta_ttt_pre.argtypes = [ctypes.POINTER(DrDesc)] + [vp] * 13 + [sz, vp]
    lib.delta_ttt_pre.restype = ctypes.c_int
    lib.dr_status_str.argtypes = [ctypes.c_int]
    lib.dr_status_str.restype = ctypes.c_char_p
    lib.dr_abi_version.argtypes = []
    lib.dr_abi_version.restype = ctypes.c_int
    if lib.dr_abi_version() != ABI_VERSION:
        raise ImportError(f"{path} has ABI version {lib.dr_abi_version()}, the binding expects "
                          f"{ABI_VERSION}: rebuild it")
    _lib = lib
    return lib


def header_functions(path: str = HEADER):
    """Names of the functions declared in the public header."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(name, t, shape, dtype, device):
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: expected dtype {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name}: expected device {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _raise(status: int):
    lib = load_library()
    raise DeltaRuleError(status, lib.dr_status_str(status).decode())


def workspace_bytes(entry: str, desc: "DrDesc") -> int:
    """Device workspace a call needs (``entry`` is "fwd", "bwd" or "ttt_pre")."""
    lib = load_library()
    n = ctypes.c_size_t(0)
    st = getattr(lib, f"delta_{entry}_workspace_bytes")(ctypes.byref(desc), ctypes.byref(n))
    if st != 0:
        _raise(st)
    return n.value


def _workspace(entry: str, desc: "DrDesc", device, workspace: Optional[torch.Tensor], stream=None):
    """(pointer, bytes) of the call's workspace: the caller's tensor when given,
    otherwise a fresh uint8 tensor from torch's allocator (None when no
    workspace is needed).  Returns the tensor too, to keep it alive.  A fresh
    tensor is marked as used on ``stream``, so torch does not hand its memory
    to another allocation before the call's kernels have finished."""
    need = workspace_bytes(entry, desc)
    if need == 0:
        return None, 0, None
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
        if stream is not None:
            workspace.record_stream(stream)
    if workspace.device != device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the call's device")
    nbytes = workspace.numel() * workspace.element_size()
    return ctypes.c_void_p(workspace.data_ptr()), nbytes, workspace


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def delta_fwd(variant: str, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
              beta: torch.Tensor, wgate: Optional[torch.Tensor] = None,
              g: Optional[torch.Tensor] = None, S0: Optional[torch.Tensor] = None,
              o: Optional[torch.Tensor] = None, S_T: Optional[torch.Tensor] = None,
              want_state: bool = True, chunk: int = 64, stream=None,
              workspace: Optional[torch.Tensor] = None
              ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunkwise forward; tensors as in include/deltarule.h ([B, T, H, d] per token).

    q and k may have fewer heads than v (H_k dividing H: grouped value heads).
    Returns (o, S_T).  ``S_T`` is allocated when ``want_state`` and not given;
    passing ``S_T=S0`` updates the state in place.  ``workspace`` (a uint8
    device tensor of at least ``workspace_bytes("fwd", desc)`` bytes) is
    allocated with torch when needed and not given.
    """
    lib = load_library()
    var = VARIANTS[variant]
    B, T, Hk, dk = q.shape
    H, dv = v.shape[2], v.shape[-1]
    dt, dev = q.dtype, q.device
    if dt not in DTYPES:
        raise ValueError(f"unsupported dtype {dt}")
    _check("q", q, (B, T, Hk, dk), dt, dev)
    _check("k", k, (B, T, Hk, dk), dt, dev)
    _check("v", v, (B, T, H, dv), dt, dev)
    _check("beta", beta, (B, T, H, dk) if variant in _CHANNEL_BETA else (B, T, H), dt, dev)
    if variant == "gdn2":
        _check("wgate", wgate, (B, T, H, dv), dt, dev)
    elif wgate is not None:
        raise ValueError("only gdn2 takes a write gate")
    if variant == "deltanet":
        if g is not None:
            raise ValueError("deltanet takes no decay")
    else:
        _check("g", g, (B, T, H) if variant == "gdn" else (B, T, H, dk), dt, dev)
    if S0 is not None:
        _check("S0", S0, (B, H, dv, dk), torch.float32, dev)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    _check("o", o, (B, T, H, dv), dt, dev)
    if S_T is None and want_state:
        S_T = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
    if S_T is not None:
        _check("S_T", S_T, (B, H, dv, dk), torch.float32, dev)
    desc = DrDesc(B, T, H, dk, dv, chunk, var, DTYPES[dt], Hk)
    wp, wn, _keep = _workspace("fwd", desc, dev, workspace, stream)
    st = lib.delta_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(wgate),
                       _ptr(g), _ptr(S0), _ptr(o), _ptr(S_T), wp, wn, _stream(stream))
    if st != 0:
        _raise(st)
    return o, S_T


def delta_fwd_noalloc(variant: str, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                      beta: torch.Tensor, o: torch.Tensor, wgate: Optional[torch.Tensor] = None,
                      g: Optional[torch.Tensor] = None, S0: Optional[torch.Tensor] = None,
                      S_T: Optional[torch.Tensor] = None, chunk: int = 64, stream=None) -> None:
    """delta_fwd through the entry point that allocates nothing (the library's
    built-in scratch replaces the workspace).  Outputs o (and S_T, if given)
    must be supplied; this wrapper allocates nothing either."""
    lib = load_library()
    var = VARIANTS[variant]
    B, T, Hk, dk = q.shape
    H, dv = v.shape[2], v.shape[-1]
    dt, dev = q.dtype, q.device
    if dt not in DTYPES:
        raise ValueError(f"unsupported dtype {dt}")
    _check("q", q, (B, T, Hk, dk), dt, dev)
    _check("k", k, (B, T, Hk, dk), dt, dev)
    _check("v", v, (B, T, H, dv), dt, dev)
    _check("beta", beta, (B, T, H, dk) if variant in _CHANNEL_BETA else (B, T, H), dt, dev)
    if variant == "gdn2":
        _check("wgate", wgate, (B, T, H, dv), dt, dev)
    if variant != "deltanet":
        _check("g", g, (B, T, H) if variant == "gdn" else (B, T, H, dk), dt, dev)
    if S0 is not None:
        _check("S0", S0, (B, H, dv, dk), torch.float32, dev)
    _check("o", o, (B, T, H, dv), dt, dev)
    if S_T is not None:
        _check("S_T", S_T, (B, H, dv, dk), torch.float32, dev)
    desc = DrDesc(B, T, H, dk, dv, chunk, var, DTYPES[dt], Hk)
    st = lib.delta_fwd_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(wgate),
                               _ptr(g), _ptr(S0), _ptr(o), _ptr(S_T), _stream(stream))
    if st != 0:
        _raise(st)


def delta_decode(variant: str, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                 beta: torch.Tensor, S: torch.Tensor, wgate: Optional[torch.Tensor] = None,
                 g: Optional[torch.Tensor] = None, o: Optional[torch.Tensor] = None,
                 stream=None) -> torch.Tensor:
    """One decode step; q, k [B, H_k, dk], v [B, H, dv]; S [B, H, dv, dk] fp32 updated in place."""
    lib = load_library()
    var = VARIANTS[variant]
    B, Hk, dk = q.shape
    H, dv = v.shape[1], v.shape[-1]
    dt, dev = q.dtype, q.device
    if dt not in DTYPES:
        raise ValueError(f"unsupported dtype {dt}")
    _check("q", q, (B, Hk, dk), dt, dev)
    _check("k", k, (B, Hk, dk), dt, dev)
    _check("v", v, (B, H, dv), dt, dev)
    _check("beta", beta, (B, H, dk) if variant in _CHANNEL_BETA else (B, H), dt, dev)
    if variant == "gdn2":
        _check("wgate", wgate, (B, H, dv), dt, dev)
    elif wgate is not None:
        raise ValueError("only gdn2 takes a write gate")
    if variant == "deltanet":
        if g is not None:
            raise ValueError("deltanet takes no decay")
    else:
        _check("g", g, (B, H) if variant == "gdn" else (B, H, dk), dt, dev)
    _check("S", S, (B, H, dv, dk), torch.float32, dev)
    if o is None:
        o = torch.empty((B, H, dv), dtype=dt, device=dev)
    _check("o", o, (B, H, dv), dt, dev)
    desc = DrDesc(B, 1, H, dk, dv, 64, var, DTYPES[dt], Hk)
    st = lib.delta_decode(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(wgate),
                          _ptr(g), _ptr(S), _ptr(o), _stream(stream))
    if st != 0:
        _raise(st)
    return o


def efla_beta(variant: str, k: torch.Tensor, beta: torch.Tensor,
              out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Exact-flow step sizes (1 - exp(-beta |k|^2)) / |k|^2.

    k [B, T, H_k, dk] with beta [B, T, H], or the decode layout k [B, H_k, dk]
    with beta [B, H].  ``out`` may be ``beta`` itself (in place).
    """
    lib = load_library()
    var = VARIANTS[variant]
    if k.dim() == 3:
        B, Hk, dk = k.shape
        T, H = 1, beta.shape[1]
        bshape = (B, H)
    else:
        B, T, Hk, dk = k.shape
        H = beta.shape[2]
        bshape = (B, T, H)
    dt, dev = k.dtype, k.device
    if dt not in DTYPES:
        raise ValueError(f"unsupported dtype {dt}")
    _check("beta", beta, bshape, dt, dev)
    if out is None:
        out = torch.empty_like(beta)
    _check("out", out, bshape, dt, dev)
    desc = DrDesc(B, T, H, dk, 64, 64, var, DTYPES[dt], Hk)
    st = lib.delta_efla_beta(ctypes.byref(desc), _ptr(k), _ptr(beta), _ptr(out), _stream(stream))
    if st != 0:
        _raise(st)
    return out


def delta_bwd(variant: str, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
              beta: torch.Tensor, dO: torch.Tensor, g: Optional[torch.Tensor] = None,
              S0: Optional[torch.Tensor] = None, dS_T: Optional[torch.Tensor] = None,
              wgate: Optional[torch.Tensor] = None, want_dS0: bool = True, chunk: int = 64,
              stream=None, workspace: Optional[torch.Tensor] = None,
              out: Optional[dict] = None) -> dict:
    """Gradients of delta_fwd: dict of dq, dk, dv, dbeta (gdn2: the erase gate's),
    dwgate (gdn2 only), dg (None for deltanet) in the input dtype and dS0 (fp32,
    None unless wanted).  ``out`` may supply any of these tensors; the rest are
    allocated."""
    lib = load_library()
    var = VARIANTS[variant]
    B, T, Hk, dk = q.shape
    H, dv = v.shape[2], v.shape[-1]
    dt, dev = q.dtype, q.device
    if dt not in DTYPES:
        raise ValueError(f"unsupported dtype {dt}")
    bshape = (B, T, H, dk) if variant in _CHANNEL_BETA else (B, T, H)
    for name, t, shape in (("q", q, (B, T, Hk, dk)), ("k", k, (B, T, Hk, dk)), ("v", v, (B, T, H, dv)),
                           ("beta", beta, bshape), ("dO", dO, (B, T, H, dv))):
        _check(name, t, shape, dt, dev)
    if variant == "gdn2":
        _check("wgate", wgate, (B, T, H, dv), dt, dev)
    elif wgate is not None:
        raise ValueError("only gdn2 takes a write gate")
    gshape = None if variant == "deltanet" else ((B, T, H) if variant == "gdn" else (B, T, H, dk))
    if gshape is not None:
        _check("g", g, gshape, dt, dev)
    elif g is not None:
        raise ValueError("deltanet takes no decay")
    for name, t in (("S0", S0), ("dS_T", dS_T)):
        if t is not None:
            _check(name, t, (B, H, dv, dk), torch.float32, dev)
    given = dict(out or {})
    out = {"dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v),
           "dbeta": torch.empty_like(beta),
           "dwgate": torch.empty_like(wgate) if variant == "gdn2" else None,
           "dg": None if gshape is None else torch.empty(gshape, dtype=dt, device=dev),
           "dS0": torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev) if want_dS0 else None}
    for name, t in given.items():
        if name not in out or out[name] is None:
            raise ValueError(f"{name} is not an output of this call")
        _check(name, t, tuple(out[name].shape), out[name].dtype, dev)
        out[name] = t
    desc = DrDesc(B, T, H, dk, dv, chunk, var, DTYPES[dt], Hk)
    wp, wn, _keep = _workspace("bwd", desc, dev, workspace, stream)
    st = lib.delta_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(wgate), _ptr(g),
                       _ptr(S0), _ptr(dO), _ptr(dS_T), _ptr(out["dq"]), _ptr(out["dk"]),
                       _ptr(out["dv"]), _ptr(out["dbeta"]), _ptr(out["dwgate"]), _ptr(out["dg"]),
                       _ptr(out["dS0"]), wp, wn, _stream(stream))
    if st != 0:
        _raise(st)
    return out


def ttt_pre(variant: str, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, beta1: torch.Tensor,
            beta2: torch.Tensor, g1: Optional[torch.Tensor] = None, g2: Optional[torch.Tensor] = None,
            A0: Optional[torch.Tensor] = None, B0: Optional[torch.Tensor] = None,
            o: Optional[torch.Tensor] = None, A_T: Optional[torch.Tensor] = None,
            B_T: Optional[torch.Tensor] = None, want_state: bool = True, stream=None,
            workspace: Optional[torch.Tensor] = None
            ) -> Tuple[torch.Tensor, Optional[torch.Tensor], Optional[torch.Tensor]]:
    """DeltaTTT-pre (two delta-rule memory layers; include/deltarule.h, delta_ttt_pre).

    q, k [B, T, H, dk]; v [B, T, H, dv]; beta1, beta2 (and g1, g2 for "gdn")
    [B, T, H]; A0 [B, H, dv, dk], B0 [B, H, dv, dv] fp32 or None.  Returns
    (o, A_T, B_T); passing ``A_T=A0`` / ``B_T=B0`` updates the states in place.
    """
    if variant not in ("deltanet", "gdn"):
        raise ValueError("DeltaTTT-pre takes the deltanet or gdn form")
    lib = load_library()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dt, dev = q.dtype, q.device
    if dt not in DTYPES:
        raise ValueError(f"unsupported dtype {dt}")
    for name, t, shape in (("q", q, (B, T, H, dk)), ("k", k, (B, T, H, dk)), ("v", v, (B, T, H, dv)),
                           ("beta1", beta1, (B, T, H)), ("beta2", beta2, (B, T, H))):
        _check(name, t, shape, dt, dev)
    for name, t in (("g1", g1), ("g2", g2)):
        if variant == "gdn":
            _check(name, t, (B, T, H), dt, dev)
        elif t is not None:
            raise ValueError("deltanet takes no decay")
    if A0 is not None:
        _check("A0", A0, (B, H, dv, dk), torch.float32, dev)
    if B0 is not None:
        _check("B0", B0, (B, H, dv, dv), torch.float32, dev)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    _check("o", o, (B, T, H, dv), dt, dev)
    if want_state:
        if A_T is None:
            A_T = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
        if B_T is None:
            B_T = torch.empty((B, H, dv, dv), dtype=torch.float32, device=dev)
    if A_T is not None:
        _check("A_T", A_T, (B, H, dv, dk), torch.float32, dev)
    if B_T is not None:
        _check("B_T", B_T, (B, H, dv, dv), torch.float32, dev)
    desc = DrDesc(B, T, H, dk, dv, 64, VARIANTS[variant], DTYPES[dt], H)
    wp, wn, _keep = _workspace("ttt_pre", desc, dev, workspace, stream)
    st = lib.delta_ttt_pre(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(beta1), _ptr(g1),
                           _ptr(beta2), _ptr(g2), _ptr(A0), _ptr(B0), _ptr(o), _ptr(A_T), _ptr(B_T),
                           wp, wn, _stream(stream))
    if st != 0:
        _raise(st)
    return o, A_T, B_T
