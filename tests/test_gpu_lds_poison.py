"""The checking build libdn_debug.so (-DDN_DEBUG: every kernel's LDS starts as
NaN) against the fp64 oracle: a result that depends on LDS no thread wrote
turns into NaN and fails.  One case per kernel and mode (both chunked-forward
kernels and their modes, the segmented schedule with its statistic and
combine kernels, decode, the gain scans, the backward, padded heads).  The
module switches the binding to the debug library and back."""
import numpy as np
import pytest
import torch

from oracle.backward import backward
from oracle.recurrence import run_workload
from parity import TOL, flat_heads, gpu_chunk, gpu_chunk_long, max_rel_err, oracle_chunk
from recurrent_sequence_mixer_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def debug_library():
    import os
    from recurrent_sequence_mixer_amd import dn
    if not os.path.exists(dn.DEBUG_LIB_PATH):
        pytest.fail("libdn_debug.so is not built (__graft_entry__.build() builds it)")
    release = dn.LIB_PATH
    dn.use_library(dn.DEBUG_LIB_PATH)
    try:
        yield dn
    finally:
        dn.use_library(release)


def _check_fwd(wl, inp, o, S, aux):
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
    o_ref, S_ref, aux_ref = oracle_chunk(wl, inp)
    eo, es = max_rel_err(flat_heads(o), o_ref), max_rel_err(flat_heads(S), S_ref)
    print(f"poisoned {wl.name} {wl.dk}x{wl.dv} T={wl.T}: o {eo:.2e} S {es:.2e}", flush=True)
    assert eo <= TOL[wl.io] and es <= TOL[wl.io]
    if aux_ref is not None:
        assert max_rel_err(flat_heads(aux), aux_ref) <= (1e-5 if wl.io == "f32" else 1e-3)


@pytest.mark.parametrize("gain,decay,keys,io,dk,dv", [
    ("kla", "scalar", "scaled", "bf16", 128, 128), ("pgdn", "scalar", "unit", "bf16", 128, 128),
    ("explicit", "scalar", "unit", "bf16", 64, 64), ("kdn", "channel", "scaled", "bf16", 128, 128),
    ("kdn_iso", "channel", "scaled", "bf16", 128, 64), ("gdn", "channel", "unit", "bf16", 128, 128),
    ("kdn", "scalar", "scaled", "bf16", 64, 128), ("kla", "scalar", "scaled", "f32", 64, 64),
    ("kla", "scalar", "scaled", "bf16", 120, 120), ("kla", "channel", "scaled", "bf16", 128, 128),
    ("explicit", "channel", "unit", "bf16", 64, 128)])
def test_poisoned_chunk_fwd(debug_library, gain, decay, keys, io, dk, dv):
    wl = W.Workload(f"poison_{gain}_{decay}", gain, decay, io, 2, 2, 150, dk, dv, keys=keys, seed=990)
    inp = W.generate(wl)
    if gain == "explicit":
        inp["w"] = W.round_io(np.random.default_rng(991).standard_normal((2, 2, 150, dk)) * 0.05, io)
    o, S, aux = gpu_chunk(wl, inp)
    _check_fwd(wl, inp, o, S, aux)


@pytest.mark.parametrize("gain,io", [("kdn", "bf16"), ("gdn", "f32")])
def test_poisoned_token_pass(debug_library, gain, io):
    """Head 0's decay leaves the chunk form's range in chunk 0 (2^-220 over
    tokens 10..31): the tokenwise pass recomputes it."""
    d = 128 if io == "bf16" else 64
    wl = W.Workload(f"poison_oor_{gain}", gain, "channel", io, 1, 2, 200, d, d,
                    keys="scaled" if gain == "kdn" else "unit", seed=993)
    inp = W.generate(wl)
    inp["alpha"][0, 0, 10:32, 4] = np.float32(2.0 ** -10)
    o, S, aux = gpu_chunk(wl, inp)
    _check_fwd(wl, inp, o, S, aux)


@pytest.mark.parametrize("gain,decay,keys", [("kla", "scalar", "scaled"), ("pgdn", "scalar", "unit"),
                                             ("kdn_iso", "channel", "scaled")])
def test_poisoned_segmented(debug_library, gain, decay, keys):
    wl = W.Workload(f"poison_long_{gain}", gain, decay, "bf16", 1, 2, 1024, 128, 128, keys=keys, seed=992)
    inp = W.generate(wl)
    o, S, aux = gpu_chunk_long(wl, inp, 4, in_place=False)
    _check_fwd(wl, inp, o, S, aux)


@pytest.mark.parametrize("gain,decay", [("kla", "scalar"), ("kdn", "channel"), ("kdn_iso", "channel")])
def test_poisoned_decode(debug_library, gain, decay):
    dn = debug_library
    wl = W.Workload("poison_dec", gain, decay, "bf16", 4, 2, 6, 128, 128, seed=993)
    inp = W.generate(wl)
    t = dn.to_device(inp, torch.bfloat16)
    S = t["S0"].clone()
    aux = {"kdn": torch.ones((4, 2, 128), device="cuda"), "kdn_iso": torch.ones((4, 2), device="cuda")}.get(gain)
    outs = []
    for s in range(wl.T):
        gates = {n: t[n][:, :, s].contiguous() for n in ("alpha", "eta", "omega", "r") if n in t}
        outs.append(dn.decode_step(t["q"][:, :, s].contiguous(), t["k"][:, :, s].contiguous(),
                                   t["v"][:, :, s].contiguous(), gates, S, aux, gain=gain, eps=wl.eps,
                                   mu_info=wl.mu_info))
    torch.cuda.synchronize()
    o = torch.stack(outs, dim=2).float().cpu().numpy()
    o_ref, S_ref, _, _ = run_workload(wl, inp)
    eo, es = max_rel_err(flat_heads(o), o_ref), max_rel_err(flat_heads(S.cpu().numpy()), S_ref)
    print(f"poisoned decode {gain}: o {eo:.2e} S {es:.2e}", flush=True)
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


@pytest.mark.parametrize("gain,decay", [("pgdn", "scalar"), ("kdn_iso", "channel")])
def test_poisoned_gain_prep(debug_library, gain, decay):
    dn = debug_library
    keys = "unit" if gain == "pgdn" else "scaled"
    wl = W.Workload("poison_gp", gain, decay, "bf16", 2, 2, 256, 128, 128, keys=keys, seed=994)
    inp = W.generate(wl)
    t = dn.to_device(inp, torch.bfloat16)
    gates = {n: t[n] for n in ("alpha", "eta", "alphaP", "betaP", "mu_log", "omega", "r") if n in t}
    w, _, _, aux_final = dn.gain_prep(t["k"], gates, gain=gain, eps=wl.eps, x=wl.x, mu_info=wl.mu_info)
    torch.cuda.synchronize()
    _, _, aux_ref, tr = run_workload(wl, inp, record=True)
    assert max_rel_err(flat_heads(w.cpu().numpy()), tr["w"]) <= 1e-5
    assert max_rel_err(flat_heads(aux_final.cpu().numpy()), aux_ref) <= 1e-5


@pytest.mark.parametrize("gain,decay,keys", [("kla", "scalar", "scaled"), ("kdn", "channel", "scaled"),
                                             ("pgdn", "scalar", "unit")])
def test_poisoned_backward(debug_library, gain, decay, keys):
    dn = debug_library
    wl = W.Workload("poison_bwd", gain, decay, "bf16", 1, 2, 150, 128, 128, keys=keys, seed=995)
    inp = W.generate(wl)
    rng = np.random.default_rng(996)
    dO = W.round_io(rng.standard_normal((1, 2, 150, 128)), "bf16")
    t = dn.to_device(inp, torch.bfloat16)
    gates = {n: t[n] for n in ("alpha", "eta", "alphaP", "betaP", "mu_log", "omega", "r") if n in t}
    g = dn.chunk_bwd(t["q"], t["k"], t["v"], gates, torch.from_numpy(dO).cuda().to(torch.bfloat16),
                     gain=gain, decay=decay, eps=wl.eps, x=wl.x, mu_info=wl.mu_info, S0=t["S0"])
    torch.cuda.synchronize()
    fh = flat_heads
    H = wl.H
    mu = None if "mu_log" not in inp else np.asarray(inp["mu_log"], np.float64)[np.arange(wl.B * H) % H]
    ref = backward(fh(inp["q"]), fh(inp["k"]), fh(inp["v"]), gain, fh(inp["alpha"]), fh(dO),
                   eta=None if "eta" not in inp else fh(inp["eta"]), eps=wl.eps,
                   alphaP=None if "alphaP" not in inp else fh(inp["alphaP"]),
                   betaP=None if "betaP" not in inp else fh(inp["betaP"]), mu_log=mu, x=wl.x,
                   omega=None if "omega" not in inp else fh(inp["omega"]),
                   r=None if "r" not in inp else fh(inp["r"]), mu_info=wl.mu_info, S0=fh(inp["S0"]))
    for n in ("q", "k", "v", "alpha", "S0"):
        e = max_rel_err(fh(g[n].cpu().numpy()), ref[n])
        print(f"poisoned backward {gain} d{n} {e:.1e}", flush=True)
        assert e <= TOL["bf16"], (n, e)
