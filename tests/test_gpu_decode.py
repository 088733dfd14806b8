"""GPU parity of the batched decode step and of the standalone gain scans
against the fp64 oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

from oracle.recurrence import forward, run_workload
from parity import TOL, flat_heads, gpu_chunk, max_rel_err
from recurrent_sequence_mixer_amd import workloads as W

pytestmark = pytest.mark.gpu


def _dn():
    from recurrent_sequence_mixer_amd import dn
    return dn


def test_workload0_as_decode_steps_f32():
    """Workload 0 (KLA fp32) token by token through dn_decode_step, 256 steps."""
    dn = _dn()
    wl = W.WORKLOADS[0]
    inp = W.generate(wl)
    t = dn.to_device(inp, torch.float32)
    S = t["S0"].clone()  # N = B = 1 sequence, H = 1 head
    outs = []
    for s in range(wl.T):
        step = lambda name: t[name][:, :, s].contiguous()
        o = dn.decode_step(step("q"), step("k"), step("v"), {"alpha": step("alpha"), "eta": step("eta")},
                           S, gain="kla", eps=wl.eps)
        outs.append(o)
    torch.cuda.synchronize()
    o = torch.stack(outs, dim=2).cpu().numpy()
    o_ref, S_ref, _, _ = run_workload(wl, inp)
    eo, es = max_rel_err(flat_heads(o), o_ref), max_rel_err(flat_heads(S.cpu().numpy()), S_ref)
    print(f"decode f32: o {eo:.2e} S {es:.2e}")
    assert eo <= TOL["f32"] and es <= TOL["f32"]


@pytest.mark.parametrize("gain,decay", [("kla", "scalar"), ("gdn", "scalar"), ("pgdn", "scalar"),
                                        ("kdn", "channel"), ("kdn", "scalar"), ("kla", "channel"),
                                        ("kdn_iso", "channel"), ("kdn_iso", "scalar")])
@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (64, 128)])
def test_decode_gains(gain, decay, io, dk, dv):
    """A short prefill-free decode (12 steps) over 6 sequences x 3 heads."""
    dn = _dn()
    keys = "unit" if gain in ("gdn", "pgdn") else "scaled"
    wl = W.Workload("dec", gain, decay, io, 6, 3, 12, dk, dv, keys=keys, seed=21)
    inp = W.generate(wl)
    dt = torch.float32 if io == "f32" else torch.bfloat16
    t = dn.to_device(inp, dt)
    S = t["S0"].clone()
    aux = torch.ones((6, 3, dk), device="cuda") if gain in ("pgdn", "kdn") else None
    if gain == "kdn_iso":
        aux = torch.ones((6, 3), device="cuda")
    outs = []
    for s in range(wl.T):
        gates = {n: t[n][:, :, s].contiguous() for n in ("alpha", "eta", "alphaP", "betaP", "omega", "r")
                 if n in t}
        if "mu_log" in t:
            gates["mu_log"] = t["mu_log"]
        outs.append(dn.decode_step(t["q"][:, :, s].contiguous(), t["k"][:, :, s].contiguous(),
                                   t["v"][:, :, s].contiguous(), gates, S, aux, gain=gain, eps=wl.eps,
                                   x=wl.x, mu_info=wl.mu_info))
    torch.cuda.synchronize()
    o = torch.stack(outs, dim=2).float().cpu().numpy()
    o_ref, S_ref, aux_ref, _ = run_workload(wl, inp)
    eo, es = max_rel_err(flat_heads(o), o_ref), max_rel_err(flat_heads(S.cpu().numpy()), S_ref)
    tol = TOL[io]
    print(f"decode {gain}/{decay}/{io} {dk}x{dv}: o {eo:.2e} S {es:.2e}")
    assert eo <= tol and es <= tol
    if aux is not None:
        assert max_rel_err(flat_heads(aux.cpu().numpy()), aux_ref) <= 1e-5


@pytest.mark.parametrize("gain,decay,keys,dk,dv", [("kla", "scalar", "scaled", 128, 256),
                                                  ("kdn", "channel", "scaled", 128, 512),
                                                  ("pgdn", "scalar", "unit", 64, 192),
                                                  ("kdn_iso", "channel", "scaled", 128, 384),
                                                  ("gdn", "scalar", "unit", 64, 2048)])
def test_decode_value_expansion(gain, decay, keys, dk, dv):
    """Wider value heads d_v = v_expand d_k (Kalman Delta Networks: value
    expansion up to 16): one workgroup walks the head's value slices, its
    gain (and statistic update) formed once; 10 steps over 3 x 2 heads."""
    dn = _dn()
    wl = W.Workload("dec_vexp", gain, decay, "bf16", 3, 2, 10, dk, dv, keys=keys, seed=580 + dv)
    inp = W.generate(wl)
    t = dn.to_device(inp, torch.bfloat16)
    S = t["S0"].clone()
    aux = torch.ones((3, 2, dk), device="cuda") if gain in ("pgdn", "kdn") else None
    if gain == "kdn_iso":
        aux = torch.ones((3, 2), device="cuda")
    outs = []
    for s in range(wl.T):
        gates = {n: t[n][:, :, s].contiguous() for n in ("alpha", "eta", "alphaP", "betaP", "omega", "r")
                 if n in t}
        if "mu_log" in t:
            gates["mu_log"] = t["mu_log"]
        outs.append(dn.decode_step(t["q"][:, :, s].contiguous(), t["k"][:, :, s].contiguous(),
                                   t["v"][:, :, s].contiguous(), gates, S, aux, gain=gain, eps=wl.eps,
                                   x=wl.x, mu_info=wl.mu_info))
    torch.cuda.synchronize()
    o = torch.stack(outs, dim=2).float().cpu().numpy()
    o_ref, S_ref, aux_ref, _ = run_workload(wl, inp)
    eo, es = max_rel_err(flat_heads(o), o_ref), max_rel_err(flat_heads(S.cpu().numpy()), S_ref)
    print(f"decode {gain} {dk}x{dv}: o {eo:.2e} S {es:.2e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]
    if aux is not None:
        assert max_rel_err(flat_heads(aux.cpu().numpy()), aux_ref) <= 1e-5


def test_decode_full_size_sampled():
    """Workload 4 at its full size (512 sequences x 16 heads) over all 256
    steps, every step on the whole batch; sampled heads against the oracle,
    o over all 256 steps and the final state."""
    dn = _dn()
    wl = W.WORKLOADS[4]
    S0 = W.generate_decode_state(wl)
    S = torch.from_numpy(S0).cuda()
    heads = [0, 4097, 8191]
    sel = lambda a: a.reshape((wl.N * wl.H,) + a.shape[2:])[heads]
    picked = {n: [] for n in ("q", "k", "v", "eta", "alpha")}
    outs = []
    for s in range(wl.steps):
        st = W.generate_decode_step(wl, s)
        for n in picked:
            picked[n].append(sel(st[n]))
        t = dn.to_device(st, torch.bfloat16)
        o = dn.decode_step(t["q"], t["k"], t["v"], {"alpha": t["alpha"], "eta": t["eta"]}, S,
                           gain="kla", eps=wl.eps)
        outs.append(o.reshape(wl.N * wl.H, wl.dv)[heads].float())
        if s % 64 == 63:
            print(f"decode full size: {s + 1} of {wl.steps} steps", flush=True)
    torch.cuda.synchronize()
    stack = lambda name: np.stack(picked[name], axis=1)
    o_ref, S_ref, _, _ = forward(stack("q"), stack("k"), stack("v"), "kla", stack("alpha"),
                                 eta=stack("eta"), eps=wl.eps, S0=sel(S0))
    o = torch.stack(outs, dim=1).cpu().numpy()
    eo, es = max_rel_err(o, o_ref), max_rel_err(sel(S.cpu().numpy()), S_ref)
    print(f"decode full size, {wl.steps} steps: o {eo:.2e} S {es:.2e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


@pytest.mark.parametrize("decay", ["scalar", "channel"])
def test_decode_pgdn_distinct_centre_per_head(decay):
    """PGDN decode with a different centre mu_h per head (N = 4, H = 3)."""
    dn = _dn()
    wl = W.Workload("dec_pgdn_mu", "pgdn", decay, "bf16", 4, 3, 10, 128, 128, keys="unit",
                    mu_spread=1.5, seed=540)
    inp = W.generate(wl)
    t = dn.to_device(inp, torch.bfloat16)
    S = t["S0"].clone()
    aux = torch.ones((4, 3, 128), device="cuda")
    outs = []
    for s in range(wl.T):
        gates = {n: t[n][:, :, s].contiguous() for n in ("alpha", "eta", "alphaP", "betaP")}
        gates["mu_log"] = t["mu_log"]
        outs.append(dn.decode_step(t["q"][:, :, s].contiguous(), t["k"][:, :, s].contiguous(),
                                   t["v"][:, :, s].contiguous(), gates, S, aux, gain="pgdn", x=wl.x))
    torch.cuda.synchronize()
    o = torch.stack(outs, dim=2).float().cpu().numpy()
    o_ref, S_ref, aux_ref, _ = run_workload(wl, inp)
    eo, es = max_rel_err(flat_heads(o), o_ref), max_rel_err(flat_heads(S.cpu().numpy()), S_ref)
    ea = max_rel_err(flat_heads(aux.cpu().numpy()), aux_ref)
    print(f"decode pgdn per-head mu ({decay}): o {eo:.2e} S {es:.2e} aux {ea:.2e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"] and ea <= 1e-5


def test_prefill_then_decode_equals_one_pass():
    """dn_chunk_fwd over a prefix, then dn_decode_step token by token, against
    the oracle over the whole sequence."""
    dn = _dn()
    wl = W.Workload("kdn_pd", "kdn", "channel", "bf16", 2, 2, 140, 128, 128, seed=9)
    inp = W.generate(wl)
    t = dn.to_device(inp, torch.bfloat16)
    P = 100
    pre = {n: t[n][:, :, :P].contiguous() for n in ("alpha", "omega", "r")}
    o_pre, S, aux = dn.chunk_fwd(t["q"][:, :, :P].contiguous(), t["k"][:, :, :P].contiguous(),
                                 t["v"][:, :, :P].contiguous(), pre, gain="kdn", mu_info=wl.mu_info,
                                 S0=t["S0"])
    outs = [o_pre]
    for s in range(P, wl.T):
        g = {n: t[n][:, :, s].contiguous() for n in ("alpha", "omega", "r")}
        outs.append(dn.decode_step(t["q"][:, :, s].contiguous(), t["k"][:, :, s].contiguous(),
                                   t["v"][:, :, s].contiguous(), g, S, aux, gain="kdn",
                                   mu_info=wl.mu_info)[:, :, None])
    torch.cuda.synchronize()
    o = torch.cat(outs, dim=2).float().cpu().numpy()
    o_ref, S_ref, aux_ref, _ = run_workload(wl, inp)
    assert max_rel_err(flat_heads(o), o_ref) <= TOL["bf16"]
    assert max_rel_err(flat_heads(S.cpu().numpy()), S_ref) <= TOL["bf16"]


@pytest.mark.parametrize("decay", ["channel", "scalar"])
def test_kdn_iso_prefill_decode_and_resume(decay):
    """Isotropic KDN: dn_chunk_fwd over a prefix (ragged), a second
    dn_chunk_fwd resuming from its (S, b), then dn_decode_step token by
    token, against one oracle pass (the head's variance b is handed over
    between the chunk kernel and the decode kernel)."""
    dn = _dn()
    wl = W.Workload("iso_pd", "kdn_iso", decay, "bf16", 2, 2, 170, 128, 128, seed=13)
    inp = W.generate(wl)
    t = dn.to_device(inp, torch.bfloat16)
    P1, P2 = 70, 150
    names = ("alpha", "omega", "r")
    part = lambda a, b: {n: t[n][:, :, a:b].contiguous() for n in names}
    seq = lambda n, a, b: t[n][:, :, a:b].contiguous()
    kw = dict(gain="kdn_iso", mu_info=wl.mu_info)
    o1, S, b = dn.chunk_fwd(seq("q", 0, P1), seq("k", 0, P1), seq("v", 0, P1), part(0, P1),
                            S0=t["S0"], **kw)
    b2 = torch.empty_like(b)
    o2, _, _ = dn.chunk_fwd(seq("q", P1, P2), seq("k", P1, P2), seq("v", P1, P2), part(P1, P2),
                            S0=S, aux0=b, S_final=S, aux_final=b2, **kw)
    outs = [o1, o2]
    for s in range(P2, wl.T):
        g = {n: t[n][:, :, s].contiguous() for n in names}
        outs.append(dn.decode_step(t["q"][:, :, s].contiguous(), t["k"][:, :, s].contiguous(),
                                   t["v"][:, :, s].contiguous(), g, S, b2, **kw)[:, :, None])
    torch.cuda.synchronize()
    o = torch.cat(outs, dim=2).float().cpu().numpy()
    o_ref, S_ref, b_ref, _ = run_workload(wl, inp)
    eo = max_rel_err(flat_heads(o), o_ref)
    es = max_rel_err(flat_heads(S.cpu().numpy()), S_ref)
    eb = max_rel_err(flat_heads(b2.cpu().numpy()), b_ref)
    print(f"iso prefill/resume/decode {decay}: o {eo:.2e} S {es:.2e} b {eb:.2e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"] and eb <= 1e-3


@pytest.mark.parametrize("T", [150, 320])
@pytest.mark.parametrize("gain,decay,io", [("kla", "scalar", "bf16"), ("pgdn", "scalar", "bf16"),
                                           ("kdn", "channel", "bf16"), ("kdn", "channel", "f32"),
                                           ("gdn", "channel", "f32"), ("kdn_iso", "channel", "bf16"),
                                           ("kdn_iso", "scalar", "f32"), ("kdn", "scalar", "bf16"),
                                           ("pgdn", "channel", "bf16"), ("kdn_iso", "scalar", "bf16"),
                                           ("kdn", "channel", "f32_128"), ("pgdn", "scalar", "f32_128")])
def test_gain_prep_per_token(gain, decay, io, T):
    """dn_gain_prep's per-token write vectors, chunk-start aux and in-chunk
    cumulative log-decay against the oracle's trace.  T = 320 (whole chunks)
    scans every chunk in parallel (for the gains with a statistic from the
    chunk summaries and carry, bf16), T = 150 one head at a time; a
    non-default aux0 and, for PGDN, a different centre per head."""
    dn = _dn()
    keys = "unit" if gain in ("gdn", "pgdn") else "scaled"
    d = 64 if io == "f32" else 128  # f32_128: fp32 io at d_k = 128
    io = "f32" if io == "f32_128" else io
    wl = W.Workload("gp", gain, decay, io, 2, 3, T, d, d, keys=keys, mu_spread=1.0, seed=31)
    inp = W.generate(wl)
    rng = np.random.default_rng(32)
    if gain in ("pgdn", "kdn", "kdn_iso"):
        shape = (2, 3) if gain == "kdn_iso" else (2, 3, wl.dk)
        inp["aux0"] = rng.uniform(0.5, 2.0, size=shape).astype(np.float32)
    t = dn.to_device(inp, torch.float32 if io == "f32" else torch.bfloat16)
    gates = {n: t[n] for n in ("alpha", "eta", "alphaP", "betaP", "mu_log", "omega", "r") if n in t}
    w, g, aux_chunk, aux_final = dn.gain_prep(t["k"], gates, gain=gain, eps=wl.eps, x=wl.x,
                                              mu_info=wl.mu_info, aux0=t.get("aux0"))
    torch.cuda.synchronize()
    _, _, aux_ref, tr = run_workload(wl, inp, record=True, aux0=None if "aux0" not in inp
                                     else flat_heads(inp["aux0"]))
    ew = max_rel_err(flat_heads(w.cpu().numpy()), tr["w"])
    print(f"gain_prep {gain}: w {ew:.2e}")
    assert ew <= 1e-5
    alpha = flat_heads(inp["alpha"]).astype(np.float64)
    T = wl.T
    G = np.zeros_like(alpha)
    for c0 in range(0, T, 64):
        G[:, c0:c0 + 64] = np.cumsum(np.log(alpha[:, c0:c0 + 64]), axis=1)
    np.testing.assert_allclose(flat_heads(g.cpu().numpy()), G, rtol=1e-5, atol=1e-5)
    if aux_ref is not None:
        assert max_rel_err(flat_heads(aux_final.cpu().numpy()), aux_ref) <= 1e-5
        key = "A" if gain == "pgdn" else "p"
        ac = flat_heads(aux_chunk.cpu().numpy())
        np.testing.assert_array_equal(ac[:, 0], flat_heads(inp["aux0"]))
        for ci, c0 in enumerate(range(64, T, 64)):
            assert max_rel_err(ac[:, ci + 1], tr[key][:, c0 - 1]) <= 1e-5
