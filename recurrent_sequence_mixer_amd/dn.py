"""Python binding of libdn.so (include/dn.h): argument marshalling only.

Every step of the computation runs in the library's HIP kernels.  Tensors
are torch tensors on the GPU; torch provides device memory and the current
stream.  If the library is missing the binding raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# The library; DN_LIBRARY names another build of it (the checking builds next
# to it: libdn_debug.so with LDS poisoning, libdn_hostasan.so with the host
# code under AddressSanitizer).
LIB_PATH = os.environ.get("DN_LIBRARY") or os.path.join(_HERE, "libdn.so")
DEBUG_LIB_PATH = os.path.join(_HERE, "libdn_debug.so")
HOSTASAN_LIB_PATH = os.path.join(_HERE, "libdn_hostasan.so")

DN_OK = 0
STATUS = {0: "DN_OK", -1: "DN_ERR_NULL", -2: "DN_ERR_SHAPE", -3: "DN_ERR_DTYPE", -4: "DN_ERR_GAIN",
          -5: "DN_ERR_WORKSPACE", -6: "DN_ERR_UNSUPPORTED", -7: "DN_ERR_HIP", -8: "DN_ERR_ALIAS"}
GAIN = {"kla": 0, "gdn": 1, "pgdn": 2, "kdn": 3, "explicit": 4, "kdn_iso": 5}
DECAY = {"scalar": 0, "channel": 1}
IO = {torch.float32: 0, torch.bfloat16: 1}

# Symbols declared in include/dn.h.
EXPORTS = ("dn_chunk_fwd", "dn_chunk_fwd_long", "dn_chunk_fwd_long_workspace", "dn_decode_step",
           "dn_gain_prep", "dn_status_string", "dn_version", "dn_workspace_bytes",
           "dn_chunk_fwd_noalloc", "dn_chunk_bwd", "dn_chunk_bwd_workspace")


class DnDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("T", ctypes.c_int32),
                ("dk", ctypes.c_int32), ("dv", ctypes.c_int32), ("C", ctypes.c_int32),
                ("io", ctypes.c_int32), ("gain", ctypes.c_int32), ("decay", ctypes.c_int32),
                ("eps", ctypes.c_float), ("x", ctypes.c_float), ("mu_info", ctypes.c_float)]


class DnGates(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("alpha", "eta", "alphaP", "betaP", "mu_log", "omega", "r", "w")]


class DnGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("dq", "dk", "dv", "dalpha", "deta", "dalphaP", "dbetaP", "dmu_log", "dw", "dS0",
                 "daux0", "domega", "dr")]


class DnError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {STATUS.get(status, status)} ({status_string(status)})")
        self.status = status


_lib = None


def use_library(path: str) -> None:
    """Load another build of the library (same ABI) for the calls that follow."""
    global _lib, LIB_PATH
    LIB_PATH = path
    _lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m recurrent_sequence_mixer_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, ip = ctypes.c_void_p, ctypes.c_int
        L.dn_workspace_bytes.argtypes = [ctypes.POINTER(DnDesc)]
        L.dn_workspace_bytes.restype = ctypes.c_size_t
        L.dn_chunk_fwd.argtypes = [ctypes.POINTER(DnDesc), vp, vp, vp, ctypes.POINTER(DnGates),
                                   vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.dn_chunk_fwd.restype = ip
        L.dn_chunk_fwd_noalloc.argtypes = [ctypes.POINTER(DnDesc), vp, vp, vp,
                                           ctypes.POINTER(DnGates), vp, vp, vp, vp, vp, vp]
        L.dn_chunk_fwd_noalloc.restype = ip
        L.dn_chunk_fwd_long.argtypes = [ctypes.POINTER(DnDesc), ip, vp, vp, vp, ctypes.POINTER(DnGates),
                                        vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.dn_chunk_fwd_long.restype = ip
        L.dn_chunk_fwd_long_workspace.argtypes = [ctypes.POINTER(DnDesc), ip]
        L.dn_chunk_fwd_long_workspace.restype = ctypes.c_size_t
        L.dn_decode_step.argtypes = [ctypes.POINTER(DnDesc), vp, vp, vp, ctypes.POINTER(DnGates),
                                     vp, vp, vp, vp]
        L.dn_decode_step.restype = ip
        L.dn_gain_prep.argtypes = [ctypes.POINTER(DnDesc), vp, ctypes.POINTER(DnGates), vp,
                                   vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.dn_gain_prep.restype = ip
        L.dn_chunk_bwd_workspace.argtypes = [ctypes.POINTER(DnDesc)]
        L.dn_chunk_bwd_workspace.restype = ctypes.c_size_t
        L.dn_chunk_bwd.argtypes = [ctypes.POINTER(DnDesc), vp, vp, vp, ctypes.POINTER(DnGates), vp, vp,
                                   vp, vp, vp, ctypes.POINTER(DnGrads), vp, ctypes.c_size_t, vp]
        L.dn_chunk_bwd.restype = ip
        L.dn_status_string.argtypes = [ip]
        L.dn_status_string.restype = ctypes.c_char_p
        L.dn_version.argtypes = []
        L.dn_version.restype = ip
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().dn_status_string(status).decode()


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libdn must be contiguous")
    return t.data_ptr()


def make_desc(B, H, T, dk, dv, io, gain="kla", decay="scalar", eps=1e-6, x=1.5, mu_info=1.0,
              C=64) -> DnDesc:
    return DnDesc(B, H, T, dk, dv, C, IO[io] if isinstance(io, torch.dtype) else io,
                  GAIN[gain] if isinstance(gain, str) else gain,
                  DECAY[decay] if isinstance(decay, str) else decay, eps, x, mu_info)


def make_gates(g: Dict[str, torch.Tensor]) -> DnGates:
    return DnGates(*[_ptr(g.get(n)) for n in
                     ("alpha", "eta", "alphaP", "betaP", "mu_log", "omega", "r", "w")])


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _check(status: int, what: str):
    if status != DN_OK:
        raise DnError(status, what)


def workspace_bytes(desc: DnDesc) -> int:
    """dn_workspace_bytes: device workspace a chunked forward or gain scan of
    this shape needs (0: none)."""
    return lib().dn_workspace_bytes(ctypes.byref(desc))


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]):
    """(pointer, size) of the caller's workspace tensor, or of a fresh one."""
    if nbytes == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty((nbytes,), dtype=torch.uint8, device=device)
    if workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace of {workspace.numel() * workspace.element_size()} bytes, "
                         f"{nbytes} needed")
    return _ptr(workspace), workspace.numel() * workspace.element_size()


def chunk_fwd(q, k, v, gates: Dict[str, torch.Tensor], *, gain="kla", decay=None, eps=1e-6,
              x=1.5, mu_info=1.0, S0=None, aux0=None, out=None, S_final=None, aux_final=None,
              want_state=True, workspace=None, stream=None):
    """Chunked forward: returns (o, S_final, aux_final).

    q, k [B, H, T, dk], v [B, H, T, dv] (fp32 or bf16, same dtype); gates as
    in include/dn.h.  Output buffers may be passed in (S_final may be S0 for
    an in-place resume).  `workspace`: a device tensor of at least
    workspace_bytes(desc) bytes, allocated here with torch when not given
    and the shape needs one.
    """
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    if decay is None:
        decay = "channel" if gates["alpha"].dim() == 4 else "scalar"
    desc = make_desc(B, H, T, dk, dv, q.dtype, gain, decay, eps, x, mu_info)
    o = out if out is not None else torch.empty((B, H, T, dv), dtype=v.dtype, device=v.device)
    if want_state and S_final is None:
        S_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=v.device)
    has_aux = gain in ("pgdn", "kdn", "kdn_iso")
    if has_aux and want_state and aux_final is None:
        aux_final = torch.empty((B, H) if gain == "kdn_iso" else (B, H, dk), dtype=torch.float32,
                                device=v.device)
    ws, nbytes = _workspace(workspace_bytes(desc), v.device, workspace)
    gt = make_gates(gates)
    st = lib().dn_chunk_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), ctypes.byref(gt),
                            _ptr(S0), _ptr(aux0), _ptr(o), _ptr(S_final), _ptr(aux_final),
                            ws, nbytes, _stream(stream))
    _check(st, "dn_chunk_fwd")
    return o, S_final, aux_final


def chunk_fwd_long(q, k, v, gates: Dict[str, torch.Tensor], nseg: int, *, gain="kla", decay=None,
                   eps=1e-6, x=1.5, mu_info=1.0, S0=None, aux0=None, out=None, S_final=None,
                   aux_final=None, want_state=True, stream=None):
    """Chunked forward by nseg parallel segments per head (bf16; every gain and
    decay):
    returns (o, S_final, aux_final).  The workspace is allocated here with
    torch and passed to the library.  nseg: B H nseg d_v / 64 near the number
    of compute units works best (16 for B1 H8 d128)."""
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    if decay is None:
        decay = "channel" if gates["alpha"].dim() == 4 else "scalar"
    desc = make_desc(B, H, T, dk, dv, q.dtype, gain, decay, eps, x, mu_info)
    o = out if out is not None else torch.empty((B, H, T, dv), dtype=v.dtype, device=v.device)
    if want_state and S_final is None:
        S_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=v.device)
    has_aux = gain in ("pgdn", "kdn", "kdn_iso")
    if has_aux and want_state and aux_final is None:
        aux_final = torch.empty((B, H) if gain == "kdn_iso" else (B, H, dk), dtype=torch.float32,
                                device=v.device)
    nbytes = lib().dn_chunk_fwd_long_workspace(ctypes.byref(desc), nseg)
    ws = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=v.device)
    gt = make_gates(gates)
    st = lib().dn_chunk_fwd_long(ctypes.byref(desc), nseg, _ptr(q), _ptr(k), _ptr(v),
                                 ctypes.byref(gt), _ptr(S0), _ptr(aux0), _ptr(o), _ptr(S_final),
                                 _ptr(aux_final), _ptr(ws), nbytes, _stream(stream))
    _check(st, "dn_chunk_fwd_long")
    return o, S_final, aux_final


def decode_step(q, k, v, gates: Dict[str, torch.Tensor], S, aux=None, *, gain="kla", decay=None,
                eps=1e-6, x=1.5, mu_info=1.0, out=None, stream=None):
    """One token for N sequences: q, k [N, H, dk], v [N, H, dv]; S [N, H, dk, dv]
    (and aux [N, H, dk] for pgdn/kdn, [N, H] for kdn_iso) updated in place.
    Returns o [N, H, dv]."""
    N, H, dk = k.shape
    dv = v.shape[-1]
    if decay is None:
        decay = "channel" if gates["alpha"].dim() == 3 else "scalar"
    desc = make_desc(N, H, 1, dk, dv, q.dtype, gain, decay, eps, x, mu_info)
    o = out if out is not None else torch.empty((N, H, dv), dtype=v.dtype, device=v.device)
    gt = make_gates(gates)
    st = lib().dn_decode_step(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), ctypes.byref(gt),
                              _ptr(S), _ptr(aux), _ptr(o), _stream(stream))
    _check(st, "dn_decode_step")
    return o


def gain_prep(k, gates: Dict[str, torch.Tensor], *, gain="kla", decay=None, eps=1e-6, x=1.5,
              mu_info=1.0, aux0=None, C=64, workspace=None, stream=None):
    """Write-gain scans: returns (w, g, aux_chunk, aux_final)."""
    B, H, T, dk = k.shape
    if decay is None:
        decay = "channel" if gates["alpha"].dim() == 4 else "scalar"
    desc = make_desc(B, H, T, dk, dk, k.dtype, gain, decay, eps, x, mu_info, C)
    dev = k.device
    w = torch.empty((B, H, T, dk), dtype=torch.float32, device=dev)
    g = torch.empty((B, H, T, dk) if decay == "channel" else (B, H, T), dtype=torch.float32,
                    device=dev)
    has_aux = gain in ("pgdn", "kdn", "kdn_iso")
    nch = (T + C - 1) // C
    per = () if gain == "kdn_iso" else (dk,)
    aux_chunk = torch.empty((B, H, nch) + per, dtype=torch.float32, device=dev) if has_aux else None
    aux_final = torch.empty((B, H) + per, dtype=torch.float32, device=dev) if has_aux else None
    ws, nbytes = _workspace(workspace_bytes(desc), dev, workspace)
    gt = make_gates(gates)
    st = lib().dn_gain_prep(ctypes.byref(desc), _ptr(k), ctypes.byref(gt), _ptr(aux0), _ptr(w),
                            _ptr(g), _ptr(aux_chunk), _ptr(aux_final), ws, nbytes,
                            _stream(stream))
    _check(st, "dn_gain_prep")
    return w, g, aux_chunk, aux_final


def chunk_bwd(q, k, v, gates: Dict[str, torch.Tensor], dO, *, gain="kla", decay=None, eps=1e-6,
              x=1.5, mu_info=1.0, S0=None, aux0=None, dS_T=None, daux_T=None, workspace=None,
              stream=None) -> Dict[str, Optional[torch.Tensor]]:
    """Chunked backward (dn_chunk_bwd): the gradients of
    sum <dO, o> + <dS_T, S_T> + <daux_T, aux_T> with respect to the inputs of
    chunk_fwd, as fp32 tensors in a dict (q, k, v, alpha, S0 and the gain's
    gates; aux0 for the gains with a statistic)."""
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    if decay is None:
        decay = "channel" if gates["alpha"].dim() == 4 else "scalar"
    desc = make_desc(B, H, T, dk, dv, q.dtype, gain, decay, eps, x, mu_info)
    dev = v.device
    f32 = lambda *shape: torch.empty(shape, dtype=torch.float32, device=dev)
    g = {"q": f32(B, H, T, dk), "k": f32(B, H, T, dk), "v": f32(B, H, T, dv),
         "alpha": f32(*gates["alpha"].shape), "S0": f32(B, H, dk, dv)}
    if gain in ("kla", "gdn", "pgdn"):
        g["eta"] = f32(B, H, T)
    if gain == "pgdn":
        g |= {"alphaP": f32(B, H, T), "betaP": f32(B, H, T), "mu_log": f32(H), "aux0": f32(B, H, dk)}
    if gain == "kdn":
        g |= {"omega": f32(B, H, T, dk), "r": f32(B, H, T), "aux0": f32(B, H, dk)}
    if gain == "kdn_iso":
        g |= {"omega": f32(B, H, T), "r": f32(B, H, T), "aux0": f32(B, H)}
    if gain == "explicit":
        g["w"] = f32(B, H, T, dk)
    grads = DnGrads(_ptr(g["q"]), _ptr(g["k"]), _ptr(g["v"]), _ptr(g["alpha"]), _ptr(g.get("eta")),
                    _ptr(g.get("alphaP")), _ptr(g.get("betaP")), _ptr(g.get("mu_log")), _ptr(g.get("w")),
                    _ptr(g["S0"]), _ptr(g.get("aux0")), _ptr(g.get("omega")), _ptr(g.get("r")))
    nbytes = lib().dn_chunk_bwd_workspace(ctypes.byref(desc))
    ws, nbytes = _workspace(nbytes, dev, workspace)
    gt = make_gates(gates)
    st = lib().dn_chunk_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), ctypes.byref(gt), _ptr(S0),
                            _ptr(aux0), _ptr(dO), _ptr(dS_T), _ptr(daux_T), ctypes.byref(grads), ws,
                            nbytes, _stream(stream))
    _check(st, "dn_chunk_bwd")
    return g


def to_device(arrays, io_dtype: torch.dtype, device="cuda"):
    """numpy inputs of recurrent_sequence_mixer_amd.workloads -> device tensors.

    Arrays holding io-dtype data (q, k, v, per-channel alpha/omega, w) are
    converted to io_dtype exactly (their values are representable); scalar
    gates, mu_log, S0 and aux stay fp32.
    """
    out = {}
    for name, a in arrays.items():
        t = torch.from_numpy(a)
        # per-channel gates are io dtype; isotropic KDN's omega is a per-token scalar
        io_like = name in ("q", "k", "v", "w") or (name in ("alpha", "omega") and a.ndim == 4)
        out[name] = t.to(device=device, dtype=io_dtype if io_like else torch.float32).contiguous()
    return out

