"""dn_chunk_fwd_noalloc (the chunked forward with the library's own device
scratch array instead of a caller workspace) against dn_chunk_fwd on the
same inputs: two calls in a row, the second with a smaller input, each
shape one that runs by segments (so the scratch array is used)."""
import ctypes

import numpy as np
import pytest
import torch

from parity import TOL, max_rel_err
from recurrent_sequence_mixer_amd import workloads as W

pytestmark = pytest.mark.gpu


def _run(wl, noalloc):
    from recurrent_sequence_mixer_amd import dn
    inp = W.generate(wl)
    t = dn.to_device(inp, torch.bfloat16)
    gates = {n: t[n] for n in ("alpha", "eta", "alphaP", "betaP", "mu_log", "omega", "r") if n in t}
    desc = dn.make_desc(wl.B, wl.H, wl.T, wl.dk, wl.dv, torch.bfloat16, wl.gain, wl.decay, wl.eps,
                        wl.x, wl.mu_info)
    assert dn.workspace_bytes(desc) > 0  # the shape runs by segments
    o = torch.empty_like(t["v"])
    S = torch.empty_like(t["S0"])
    aux = torch.empty((wl.B, wl.H, wl.dk), device="cuda") if wl.gain in ("pgdn", "kdn") else None
    if noalloc:
        # the outputs start as NaN: every element must be written
        o.fill_(float("nan"))
        S.fill_(float("nan"))
        gt = dn.make_gates(gates)
        p = lambda x: None if x is None else x.data_ptr()
        st = dn.lib().dn_chunk_fwd_noalloc(ctypes.byref(desc), p(t["q"]), p(t["k"]), p(t["v"]),
                                           ctypes.byref(gt), p(t["S0"]), None, p(o), p(S), p(aux),
                                           torch.cuda.current_stream().cuda_stream)
        assert st == 0, dn.status_string(st)
    else:
        dn.chunk_fwd(t["q"], t["k"], t["v"], gates, gain=wl.gain, eps=wl.eps, x=wl.x,
                     mu_info=wl.mu_info, S0=t["S0"], out=o, S_final=S, aux_final=aux)
    torch.cuda.synchronize()
    return [x.float().cpu().numpy() for x in (o, S) + ((aux,) if aux is not None else ())]


def test_noalloc_matches_chunk_fwd_two_calls():
    big = W.Workload("pgdn_noalloc", "pgdn", "scalar", "bf16", 1, 8, 32768, 128, 128, keys="unit",
                     seed=61)
    small = W.Workload("kla_noalloc", "kla", "scalar", "bf16", 1, 4, 16384, 128, 128, seed=62)
    for wl in (big, small):
        print(f"dn_chunk_fwd_noalloc {wl.name} B{wl.B} H{wl.H} T{wl.T}", flush=True)
        ref = _run(wl, False)
        got = _run(wl, True)
        for name, g, r in zip(("o", "S", "aux"), got, ref):
            err = max_rel_err(g.reshape(r.shape[0], -1)[None], r.reshape(r.shape[0], -1)[None])
            print(f"   {name}: max rel err {err:.2e}, identical {np.array_equal(g, r)}", flush=True)
            assert np.all(np.isfinite(g))
            assert err <= TOL["bf16"]
            # the same kernels on the same inputs
            np.testing.assert_array_equal(g, r)
