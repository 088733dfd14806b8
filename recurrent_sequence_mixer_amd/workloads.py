"""Seeded synthetic inputs for the gated delta-rule forward engine.

This module only draws and rounds input tensors; it holds none of the
recurrence's arithmetic.  Both the fp64 oracle (through the tests) and the
HIP path consume exactly the arrays produced here, so the two sides see
bit-identical inputs.

Conventions (shared with the C ABI):
  * q, k, v, o: [B, H, T, d] row-major, d contiguous.
  * per-token scalar gates (eta, scalar alpha, alphaP, betaP, r): fp32 [B, H, T].
  * per-channel gates (alpha, omega of diagonal KDN): io dtype [B, H, T, dk];
    isotropic KDN draws omega per token, fp32 [B, H, T].
  * per-head PGDN log-centre mu_log: fp32 [H].
  * state S: fp32 [B, H, dk, dv]; auxiliary state (PGDN A, KDN p): fp32 [B, H, dk];
    isotropic KDN b: fp32 [B, H].

Distributions follow the workloads the pages evaluate, stated per config
below.  Values are drawn in fp64 with numpy's PCG64 generator, rounded to
fp32, and (for bf16 workloads) rounded again to bf16 with round-to-nearest-
even.  Every array is returned as a float32 numpy array whose values are
exactly representable in the io dtype, so widening them to fp64 is exact.
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass, field, replace
from typing import Dict, Optional

import numpy as np

GAINS = ("kla", "gdn", "pgdn", "kdn", "kdn_iso", "explicit")
DECAYS = ("scalar", "channel")


@dataclass(frozen=True)
class Workload:
    """One synthetic forward workload (sizes, gain variant and draw recipe)."""

    name: str
    gain: str
    decay: str
    io: str  # "f32" or "bf16"
    B: int
    H: int
    T: int
    dk: int
    dv: int
    C: int = 64
    eps: float = 1e-6  # KLA stabiliser
    x: float = 1.5  # PGDN bound of the write scale, B in [1/x, x]
    mu_log: float = math.log(4.0)  # PGDN per-head log-centre
    # PGDN: head h gets mu_log + mu_spread (2 h / (H - 1) - 1), so that the
    # per-head indexing of the centre is exercised (0: the same for all heads)
    mu_spread: float = 0.0
    mu_info: float = 1.0  # KDN information scaling (1 = strict reverse-KL update)
    alpha_mean: float = 3.0  # decay alpha = sigmoid(N(alpha_mean, 1)); lower is stronger decay
    keys: str = "scaled"  # "scaled": N(0,1) rows times U[0.25, 4]; "unit": L2-normalised
    s0: str = "normal"  # "zero" or "normal" (N(0, 0.01), i.e. std 0.1)
    seed: int = 0

    def replace(self, **kw) -> "Workload":
        return replace(self, **kw)

    @property
    def tokens(self) -> int:
        return self.B * self.T

    @property
    def head_tokens(self) -> int:
        return self.B * self.H * self.T


@dataclass(frozen=True)
class DecodeWorkload:
    """Batched token-by-token decode: N sequences x H heads, `steps` steps."""

    name: str
    N: int
    H: int
    dk: int
    dv: int
    steps: int
    gain: str = "kla"
    eps: float = 1e-6
    seed: int = 4


# The five workloads of the engine.  Sizes and distributions are those the
# forward engine is specified on; seeds are the workload index.
WORKLOADS: Dict[int, object] = {
    0: Workload("kla_f32_B1H1T256d64", "kla", "scalar", "f32", 1, 1, 256, 64, 64,
                s0="zero", seed=0),
    1: Workload("kla_bf16_B8H16T4096d128", "kla", "scalar", "bf16", 8, 16, 4096, 128, 128,
                seed=1),
    2: Workload("pgdn_bf16_B8H16T4096d128", "pgdn", "scalar", "bf16", 8, 16, 4096, 128, 128,
                keys="unit", seed=2),
    3: Workload("kdn_diag_bf16_B4H16T8192d128", "kdn", "channel", "bf16", 4, 16, 8192, 128, 128,
                seed=3),
    4: DecodeWorkload("decode_kla_N512H16d128x256", 512, 16, 128, 128, 256, seed=4),
}


def _sigmoid(z: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-z))


def _softplus(z: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, z)


def round_f32(a: np.ndarray) -> np.ndarray:
    return np.asarray(a, dtype=np.float64).astype(np.float32)


def round_bf16(a: np.ndarray) -> np.ndarray:
    """fp64 -> fp32 -> bf16 (round to nearest, ties to even), kept as fp32."""
    f = np.ascontiguousarray(round_f32(a))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)
    out = u.astype(np.uint32).view(np.float32)
    # keep NaN as NaN (inputs here are finite; this is only a guard)
    return np.where(np.isnan(f), f, out)


def round_io(a: np.ndarray, io: str) -> np.ndarray:
    if io == "f32":
        return round_f32(a)
    if io == "bf16":
        return round_bf16(a)
    raise ValueError(f"unknown io dtype {io!r}")


def _l2_rows(a: np.ndarray) -> np.ndarray:
    return a / np.linalg.norm(a, axis=-1, keepdims=True)


def generate(wl: Workload) -> Dict[str, np.ndarray]:
    """Draw the inputs of a forward workload.

    Fixed draw order: q, k, k_scale, v, eta, alpha, [alphaP, betaP], [omega, r], S0.
    q is L2-normalised per row in fp64 before rounding (the caller's job: the
    engine reads S^T q with q as given).  k rows are N(0,1) times a per-row
    Uniform[0.25, 4] scale, or L2-normalised when wl.keys == "unit".
    """
    rng = np.random.Generator(np.random.PCG64(wl.seed))
    B, H, T, dk, dv = wl.B, wl.H, wl.T, wl.dk, wl.dv
    shp = (B, H, T)
    q = _l2_rows(rng.standard_normal(shp + (dk,)))
    k = rng.standard_normal(shp + (dk,))
    k_scale = rng.uniform(0.25, 4.0, size=shp + (1,))
    k = _l2_rows(k) if wl.keys == "unit" else k * k_scale
    v = rng.standard_normal(shp + (dv,))
    eta = _sigmoid(rng.standard_normal(shp))
    if wl.decay == "scalar":
        alpha = round_f32(_sigmoid(rng.normal(wl.alpha_mean, 1.0, size=shp)))
    else:
        alpha = round_io(_sigmoid(rng.normal(wl.alpha_mean, 1.0, size=shp + (dk,))), wl.io)
    out = {
        "q": round_io(q, wl.io),
        "k": round_io(k, wl.io),
        "v": round_io(v, wl.io),
        "eta": round_f32(eta),
        "alpha": alpha,
    }
    if wl.gain == "pgdn":
        out["alphaP"] = round_f32(_sigmoid(rng.normal(2.0, 1.0, size=shp)))
        out["betaP"] = round_f32(_sigmoid(rng.normal(2.0, 1.0, size=shp)))
        spread = np.linspace(-1.0, 1.0, H) if H > 1 else np.zeros(1)
        out["mu_log"] = round_f32(wl.mu_log + wl.mu_spread * spread)
    if wl.gain == "kdn":
        out["omega"] = round_io(_softplus(rng.normal(-3.0, 1.0, size=shp + (dk,))), wl.io)
        out["r"] = round_f32(_softplus(rng.standard_normal(shp)))
    if wl.gain == "kdn_iso":
        out["omega"] = round_f32(_softplus(rng.normal(-3.0, 1.0, size=shp)))
        out["r"] = round_f32(_softplus(rng.standard_normal(shp)))
    if wl.s0 == "zero":
        out["S0"] = np.zeros((B, H, dk, dv), np.float32)
    else:
        out["S0"] = round_f32(rng.normal(0.0, 0.1, size=(B, H, dk, dv)))
    return out


def generate_decode_state(wl: DecodeWorkload) -> np.ndarray:
    """Initial decode states N(0, 0.01) (std 0.1), fp32 [N, H, dk, dv]."""
    rng = np.random.Generator(np.random.PCG64(wl.seed))
    return round_f32(rng.normal(0.0, 0.1, size=(wl.N, wl.H, wl.dk, wl.dv)))


def generate_decode_step(wl: DecodeWorkload, step: int) -> Dict[str, np.ndarray]:
    """Fresh per-step decode inputs (q, k, v bf16; eta, scalar alpha fp32).

    Each step has its own PCG64 stream (seed, step) so that any step can be
    regenerated alone; draw order q, k, k_scale, v, eta, alpha as for the
    forward workloads.
    """
    rng = np.random.Generator(np.random.PCG64([wl.seed, step + 1]))
    shp = (wl.N, wl.H)
    q = _l2_rows(rng.standard_normal(shp + (wl.dk,)))
    k = rng.standard_normal(shp + (wl.dk,)) * rng.uniform(0.25, 4.0, size=shp + (1,))
    v = rng.standard_normal(shp + (wl.dv,))
    eta = _sigmoid(rng.standard_normal(shp))
    alpha = _sigmoid(rng.normal(3.0, 1.0, size=shp))
    return {
        "q": round_bf16(q),
        "k": round_bf16(k),
        "v": round_bf16(v),
        "eta": round_f32(eta),
        "alpha": round_f32(alpha),
    }


def sha256(arrays: Dict[str, np.ndarray]) -> Dict[str, str]:
    return {n: hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()[:16]
            for n, a in sorted(arrays.items())}


def small(wl: Workload, **kw) -> Workload:
    """A reduced copy of a workload for parity tests (same recipe)."""
    return wl.replace(**kw)
