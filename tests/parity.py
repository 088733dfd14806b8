"""Helpers shared by the GPU parity tests: the error measure, and running the
HIP path and the oracle on the same seeded inputs."""
import numpy as np
import torch

from oracle.recurrence import run_workload

# Tolerances on the maximum relative error, per (batch, head) slice:
#   max |gpu - oracle| / max |oracle|   over o (T x d_v) and over S_T (d_k x d_v).
TOL = {"f32": 1e-4, "bf16": 2e-2}


def max_rel_err(gpu, ref):
    """Worst (b, h) slice of max|gpu - ref| / max|ref|; arrays [n, ...]."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    n = ref.shape[0]
    g = gpu.reshape(n, -1)
    r = ref.reshape(n, -1)
    scale = np.abs(r).max(axis=1)
    scale = np.where(scale == 0, 1.0, scale)
    err = np.abs(g - r).max(axis=1) / scale
    if not np.all(np.isfinite(g)):
        return float("inf")
    return float(err.max())


def gpu_chunk(wl, inp, **kw):
    """Run dn_chunk_fwd on a workload's inputs; returns numpy (o, S_T, aux_T)."""
    from recurrent_sequence_mixer_amd import dn
    io = torch.float32 if wl.io == "f32" else torch.bfloat16
    t = dn.to_device(inp, io)
    gates = {n: t[n] for n in ("alpha", "eta", "alphaP", "betaP", "mu_log", "omega", "r", "w")
             if n in t}
    o, S, aux = dn.chunk_fwd(t["q"], t["k"], t["v"], gates, gain=wl.gain, eps=wl.eps, x=wl.x,
                             mu_info=wl.mu_info, S0=t.get("S0"), aux0=t.get("aux0"), **kw)
    torch.cuda.synchronize()
    to_np = lambda x: None if x is None else x.float().cpu().numpy()
    return to_np(o), to_np(S), to_np(aux)


def flat_heads(a, heads=None):
    a = np.asarray(a)
    f = a.reshape((a.shape[0] * a.shape[1],) + a.shape[2:])
    return f if heads is None else f[np.asarray(heads)]


def oracle_chunk(wl, inp, heads=None):
    o, S, aux, _ = run_workload(wl, inp, heads=heads, aux0=None if "aux0" not in inp
                                else flat_heads(inp["aux0"], heads))
    return o, S, aux


def gpu_chunk_long(wl, inp, nseg, in_place=True):
    """Run dn_chunk_fwd_long on a workload's bf16 inputs; returns numpy
    (o, S_T, aux_T).  With in_place, S_T and aux_T overwrite S0 and aux0."""
    from recurrent_sequence_mixer_amd import dn
    t = dn.to_device(inp, torch.bfloat16)
    gates = {n: t[n] for n in ("alpha", "eta", "alphaP", "betaP", "mu_log", "omega", "r", "w")
             if n in t}
    S0, aux0 = t.get("S0"), t.get("aux0")
    kw = dict(S_final=S0, aux_final=aux0) if in_place else {}
    o, S, aux = dn.chunk_fwd_long(t["q"], t["k"], t["v"], gates, nseg, gain=wl.gain, eps=wl.eps,
                                  x=wl.x, mu_info=wl.mu_info, S0=S0, aux0=aux0, **kw)
    torch.cuda.synchronize()
    to_np = lambda x: None if x is None else x.float().cpu().numpy()
    return to_np(o), to_np(S), to_np(aux)
