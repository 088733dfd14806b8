"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs.

Bar: max relative error per (b, h) slice of o and of S_T within 1e-4 for
fp32 io and 2e-2 for bf16 io (fp32 accumulation and state).  Small cases are
compared element by element over every head; the full-size workloads run in
the launch configuration the benchmark times and are compared on sampled
heads, each evaluated in full by the oracle.
"""
import math

import numpy as np
import pytest
import torch

from parity import TOL, flat_heads, gpu_chunk, gpu_chunk_long, max_rel_err, oracle_chunk
from recurrent_sequence_mixer_amd import workloads as W

pytestmark = pytest.mark.gpu


def _check(wl, inp, heads=None, o_gpu=None, S_gpu=None, aux_gpu=None, tol=None):
    tol = TOL[wl.io] if tol is None else tol
    o_ref, S_ref, aux_ref = oracle_chunk(wl, inp, heads)
    eo = max_rel_err(flat_heads(o_gpu, heads), o_ref)
    es = max_rel_err(flat_heads(S_gpu, heads), S_ref)
    print(f"{wl.name} T={wl.T}: o {eo:.2e} S {es:.2e} (tol {tol:g})", flush=True)
    assert eo <= tol and es <= tol
    if aux_ref is not None and aux_gpu is not None:
        ea = max_rel_err(flat_heads(aux_gpu, heads), aux_ref)
        print(f"   aux {ea:.2e}", flush=True)
        assert ea <= (1e-5 if wl.io == "f32" else 1e-3)
    return eo, es


# ---------------------------------------------------------------- fp32 (workload 0)

def test_kla_f32_workload0():
    wl = W.WORKLOADS[0]
    inp = W.generate(wl)
    o, S, _ = gpu_chunk(wl, inp)
    _check(wl, inp, None, o, S)


@pytest.mark.parametrize("T", [1, 17, 63, 64, 65, 130, 200])
@pytest.mark.parametrize("gain", ["kla", "gdn", "pgdn", "kdn", "kdn_iso"])
def test_f32_gains_ragged(gain, T):
    decay = "channel" if gain in ("kdn", "kdn_iso") else "scalar"
    keys = "unit" if gain in ("gdn", "pgdn") else "scaled"
    wl = W.Workload(f"{gain}_f32", gain, decay, "f32", 2, 3, T, 64, 64, keys=keys, seed=10 + T)
    inp = W.generate(wl)
    o, S, aux = gpu_chunk(wl, inp)
    _check(wl, inp, None, o, S, aux)


# fp32 io at d_k = 128: dn_chunk_fwd runs the tokenwise kernel over every
# head (no chunk kernel is built for fp32 operand tiles of that width);
# d_v = 64 / 128 / 256, ragged lengths
@pytest.mark.parametrize("T", [1, 150])
@pytest.mark.parametrize("gain,decay,keys,dv", [("kla", "scalar", "scaled", 128), ("pgdn", "scalar", "unit", 64),
                                                ("kdn", "channel", "scaled", 128),
                                                ("kdn_iso", "channel", "scaled", 256),
                                                ("gdn", "channel", "unit", 128), ("explicit", "scalar", "unit", 64)])
def test_f32_dk128(gain, decay, keys, dv, T):
    wl = W.Workload(f"{gain}_{decay}_f32_dk128", gain, decay, "f32", 2, 2, T, 128, dv, keys=keys,
                    seed=800 + T + dv)
    inp = W.generate(wl)
    if gain == "explicit":
        inp["w"] = np.random.default_rng(801).standard_normal((2, 2, T, 128)).astype(np.float32) * 0.05
    if gain in ("pgdn", "kdn"):
        inp["aux0"] = np.random.default_rng(802).uniform(0.5, 2.0, (2, 2, 128)).astype(np.float32)
    o, S, aux = gpu_chunk(wl, inp)
    _check(wl, inp, None, o, S, aux)


def test_f32_dk128_empty_sequence():
    """T = 0 on the tokenwise path: S_final = S0, aux_final = aux0."""
    from recurrent_sequence_mixer_amd import dn
    B, H, d = 1, 2, 128
    S0 = torch.randn(B, H, d, d, device="cuda")
    aux0 = torch.rand(B, H, d, device="cuda") + 0.5
    z = torch.empty(B, H, 0, d, device="cuda")
    gates = {"alpha": torch.empty(B, H, 0, d, device="cuda"), "omega": z, "r": torch.empty(B, H, 0, device="cuda")}
    o, S, aux = dn.chunk_fwd(z, z, z, gates, gain="kdn", S0=S0, aux0=aux0)
    torch.cuda.synchronize()
    assert torch.equal(S, S0) and torch.equal(aux, aux0)


# ---------------------------------------------------------------- bf16, small

@pytest.mark.parametrize("T", [1, 63, 65, 200, 333])
@pytest.mark.parametrize("gain,decay,keys", [("kla", "scalar", "scaled"), ("gdn", "scalar", "unit"),
                                             ("pgdn", "scalar", "unit"), ("kdn", "channel", "scaled"),
                                             ("kla", "channel", "scaled"), ("kdn", "scalar", "scaled"),
                                             ("pgdn", "channel", "unit"), ("kdn_iso", "channel", "scaled"),
                                             ("kdn_iso", "scalar", "scaled")])
def test_bf16_gains_ragged(gain, decay, keys, T):
    wl = W.Workload(f"{gain}_{decay}_bf16", gain, decay, "bf16", 2, 2, T, 128, 128, keys=keys,
                    seed=100 + T)
    inp = W.generate(wl)
    o, S, aux = gpu_chunk(wl, inp)
    _check(wl, inp, None, o, S, aux)


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64)])
def test_bf16_other_head_dims(dk, dv):
    wl = W.Workload("kla_dims", "kla", "scalar", "bf16", 2, 2, 150, dk, dv, seed=7)
    inp = W.generate(wl)
    o, S, _ = gpu_chunk(wl, inp)
    _check(wl, inp, None, o, S)


# wider value heads, d_v = v_expand d_k (2 and 4): more 64-column value slices
# per head on the same kernels
@pytest.mark.parametrize("gain,decay,keys,io,dk,dv", [
    ("kla", "scalar", "scaled", "bf16", 128, 256), ("kla", "scalar", "scaled", "bf16", 128, 512),
    ("pgdn", "scalar", "unit", "bf16", 128, 256), ("kdn", "channel", "scaled", "bf16", 128, 256),
    ("kdn_iso", "channel", "scaled", "bf16", 128, 256), ("kla", "channel", "scaled", "bf16", 64, 256),
    ("kla", "scalar", "scaled", "f32", 64, 256)])
def test_value_expansion(gain, decay, keys, io, dk, dv):
    wl = W.Workload(f"{gain}_{decay}_{io}_dv{dv}", gain, decay, io, 1, 2, 150, dk, dv, keys=keys,
                    seed=400 + dv)
    inp = W.generate(wl)
    o, S, aux = gpu_chunk(wl, inp)
    _check(wl, inp, None, o, S, aux)


# d_k = 64 changes the work split of the per-channel scans: the PGDN
# statistic and the KDN channel-decay variance both run in eight 8-token
# segments per channel; ragged lengths cover the partial last chunk
@pytest.mark.parametrize("T", [37, 200])
@pytest.mark.parametrize("dv", [64, 128])
@pytest.mark.parametrize("gain,decay,keys", [("gdn", "scalar", "unit"), ("pgdn", "scalar", "unit"),
                                             ("kdn", "channel", "scaled"), ("kdn_iso", "channel", "scaled")])
def test_bf16_gains_dk64(gain, decay, keys, dv, T):
    wl = W.Workload(f"{gain}_{decay}_bf16_dk64", gain, decay, "bf16", 2, 2, T, 64, dv, keys=keys,
                    seed=300 + T + dv)
    inp = W.generate(wl)
    o, S, aux = gpu_chunk(wl, inp)
    _check(wl, inp, None, o, S, aux)


# KLA, GDN (KDA) and explicit write vectors with per-channel decay: the fused
# kernel's decay-scaled mode without a variance, both head widths, ragged
# lengths, a nonzero S0 (the workload's)
@pytest.mark.parametrize("T", [1, 63, 65, 200, 333])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128)])
@pytest.mark.parametrize("gain,keys", [("kla", "scaled"), ("gdn", "unit"), ("explicit", "unit")])
def test_bf16_channel_decay_gains(gain, keys, dk, dv, T):
    wl = W.Workload(f"{gain}_channel_bf16", gain, "channel", "bf16", 2, 2, T, dk, dv, keys=keys,
                    seed=700 + T + dk)
    inp = W.generate(wl)
    if gain == "explicit":
        inp["w"] = W.round_io(np.random.default_rng(wl.seed + 1).standard_normal((2, 2, T, dk)) * 0.05,
                              "bf16")
    o, S, aux = gpu_chunk(wl, inp)
    _check(wl, inp, None, o, S, aux)


# ---------------------------------------------------------------- full size workloads

@pytest.mark.parametrize("idx", [1, 2, 3])
def test_full_size_sampled_heads(idx):
    wl = W.WORKLOADS[idx]
    inp = W.generate(wl)
    o, S, aux = gpu_chunk(wl, inp)
    nheads = wl.B * wl.H
    heads = [0, nheads // 3, nheads - 1]
    _check(wl, inp, heads, o, S, aux)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))


@pytest.mark.parametrize("gain,keys", [("gdn", "unit"), ("kla", "scaled")])
def test_channel_decay_full_size_sampled_heads(gain, keys):
    """KDA (GDN with per-channel decay) and KLA with per-channel decay at the
    KLA workload's shape B8 H16 T4096 d128 (the bench's kda and kla_channel
    lines), sampled heads."""
    wl = W.WORKLOADS[1].replace(name=f"{gain}_channel_full", gain=gain, decay="channel", keys=keys)
    inp = W.generate(wl)
    o, S, aux = gpu_chunk(wl, inp)
    nheads = wl.B * wl.H
    _check(wl, inp, [0, nheads // 2, nheads - 1], o, S, aux)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))


def test_kdn_iso_full_size_sampled_heads():
    """Isotropic KDN (Kalman Delta Networks §2.7) at the diagonal-KDN shape
    B4 H16 T8192 d128 with per-channel decay, sampled heads."""
    wl = W.WORKLOADS[3].replace(name="kdn_iso_bf16_B4H16T8192d128", gain="kdn_iso")
    inp = W.generate(wl)
    o, S, aux = gpu_chunk(wl, inp)
    heads = [0, 21, 63]
    _check(wl, inp, heads, o, S, aux)


@pytest.mark.parametrize("T", [131072, 131071])
def test_long_prefill_batch1_sampled_head(T):
    """Batch-1 long prefill (B1 H8 d128, KLA bf16; the pages' long-context
    prefill length) through dn_chunk_fwd: at T = 131072 the call picks 16
    segments per head on its workspace; T = 131071 is not whole chunks, so
    one launch walks 2048 chunks per head and a ragged tail.  One head is
    compared in full with the oracle."""
    from recurrent_sequence_mixer_amd import dn
    wl = W.Workload("kla_long_B1H8d128", "kla", "scalar", "bf16", 1, 8, T, 128, 128, seed=51)
    desc = dn.make_desc(1, 8, T, 128, 128, torch.bfloat16, "kla")
    assert (dn.workspace_bytes(desc) > 0) == (T % 64 == 0)
    inp = W.generate(wl)
    o, S, _ = gpu_chunk(wl, inp)
    _check(wl, inp, [5], o, S)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))


@pytest.mark.parametrize("gain,keys,nseg", [("kla", "scaled", 1), ("kla", "scaled", 4), ("kla", "scaled", 8),
                                            ("gdn", "unit", 4)])
def test_chunk_fwd_long_segments(gain, keys, nseg):
    """dn_chunk_fwd_long: segments in parallel, chained by their transfer
    matrices (S_out = A S_in + B per segment), against the oracle over every
    head, from a nonzero S0."""
    from recurrent_sequence_mixer_amd import dn
    wl = W.Workload(f"{gain}_long_small", gain, "scalar", "bf16", 1, 2, 2048, 128, 128, keys=keys,
                    seed=60 + nseg)
    inp = W.generate(wl)
    t = dn.to_device(inp, torch.bfloat16)
    gates = {n: t[n] for n in ("alpha", "eta")}
    # the state in place (S_final is S0)
    S = t["S0"].clone()
    o, _, _ = dn.chunk_fwd_long(t["q"], t["k"], t["v"], gates, nseg, gain=gain, eps=wl.eps, S0=S,
                             S_final=S)
    torch.cuda.synchronize()
    _check(wl, inp, None, o.float().cpu().numpy(), S.cpu().numpy())


def test_chunk_fwd_long_segments_carry_state():
    """No decay and a small step (alpha = 1, eta = 0.1, unit keys): a segment
    keeps much of its entering state, so the transfer matrices carry it; the
    norm of A_s is checked to be far from 0 through the state it hands on."""
    from oracle.recurrence import run_workload
    from recurrent_sequence_mixer_amd import dn
    wl = W.Workload("gdn_long_carry", "gdn", "scalar", "bf16", 1, 2, 2048, 128, 128, keys="unit",
                    seed=71)
    inp = W.generate(wl)
    inp["alpha"] = np.ones_like(inp["alpha"])
    inp["eta"] = np.full_like(inp["eta"], np.float32(0.1))
    t = dn.to_device(inp, torch.bfloat16)
    o, S, _ = dn.chunk_fwd_long(t["q"], t["k"], t["v"], {"alpha": t["alpha"], "eta": t["eta"]}, 4,
                             gain="gdn", S0=t["S0"])
    torch.cuda.synchronize()
    _check(wl, inp, None, o.float().cpu().numpy(), S.cpu().numpy())
    # the state entering the last segment still matters: rerunning that segment
    # from zero instead changes its outputs by a sizeable fraction
    last = slice(1536, 2048)
    part = {n: (a[:, :, last] if n not in ("S0",) else np.zeros_like(a)) for n, a in inp.items()}
    o_zero, _, _, _ = run_workload(wl.replace(T=512), part)
    o_ref, _, _, _ = run_workload(wl, inp)
    diff = np.abs(o_zero - o_ref[:, 1536:]).max() / np.abs(o_ref[:, 1536:]).max()
    print(f"carried state: last segment from zero differs by {diff:.2f}")
    assert diff > 0.1


def test_chunk_fwd_long_full_size_sampled_head():
    """Batch-1 long prefill B1 H8 T131072 d128 by 16 segments of 8192 tokens
    (256 workgroups per pass instead of 16); one head against the oracle."""
    from recurrent_sequence_mixer_amd import dn
    wl = W.Workload("kla_long_B1H8T131072d128", "kla", "scalar", "bf16", 1, 8, 131072, 128, 128,
                    seed=51)
    inp = W.generate(wl)
    t = dn.to_device(inp, torch.bfloat16)
    o, S, _ = dn.chunk_fwd_long(t["q"], t["k"], t["v"], {"alpha": t["alpha"], "eta": t["eta"]}, 16,
                             gain="kla", eps=wl.eps, S0=t["S0"])
    torch.cuda.synchronize()
    _check(wl, inp, [5], o.float().cpu().numpy(), S.cpu().numpy())


@pytest.mark.parametrize("gain,decay,keys,T,nseg,d", [
    ("pgdn", "scalar", "unit", 2048, 4, 128),      # 512-token segments: two 256-token pieces
    ("pgdn", "scalar", "unit", 1536, 8, 128),      # 192-token segments: three 64-token pieces
    ("kdn", "channel", "scaled", 2048, 8, 128),    # one 256-token piece per segment
    ("kdn", "channel", "scaled", 1536, 8, 128),
    ("kdn", "channel", "scaled", 1024, 2, 64),
    ("kdn_iso", "channel", "scaled", 2048, 4, 128),
    ("kdn_iso", "channel", "scaled", 1280, 10, 64),  # 128-token segments
    ("kdn_iso", "channel", "scaled", 8320, 2, 128),  # 130 pieces of 64 tokens: three scan rounds
    ("pgdn", "scalar", "unit", 8320, 5, 128),        # 65 pieces of 128 tokens
    ("pgdn", "scalar", "unit", 1024, 4, 64),
    # per-channel decay: PKDA (PGDN, generic chunk kernel), KLA, GDN
    ("pgdn", "channel", "unit", 1024, 4, 128),
    ("kla", "channel", "scaled", 1024, 4, 128),
    ("gdn", "channel", "unit", 1024, 2, 64),
    # KDN and isotropic KDN with scalar decay (generic kernel; alpha per token)
    ("kdn", "scalar", "scaled", 1024, 4, 128),
    ("kdn_iso", "scalar", "scaled", 1024, 4, 64),
])
def test_chunk_fwd_long_statistic_gains(gain, decay, keys, T, nseg, d):
    """dn_chunk_fwd_long with a gain statistic (PGDN's A_t, KDN's p_t and b_t):
    the statistic entering every segment comes from the composed per-token
    maps; o, S_T and aux_T (both in place) against one oracle pass, from a
    nonzero S0 and a non-default aux0."""
    wl = W.Workload(f"{gain}_long_small", gain, decay, "bf16", 1, 2, T, d, d, keys=keys,
                    seed=80 + nseg)
    inp = W.generate(wl)
    rng = np.random.default_rng(wl.seed)
    shape = (1, 2) if gain == "kdn_iso" else (1, 2, d)
    if gain in ("pgdn", "kdn", "kdn_iso"):
        inp["aux0"] = rng.uniform(0.5, 2.0, size=shape).astype(np.float32)
    o, S, aux = gpu_chunk_long(wl, inp, nseg)
    _check(wl, inp, None, o, S, aux)


@pytest.mark.parametrize("gain,decay,keys", [("kla", "scalar", "scaled"), ("pgdn", "scalar", "unit"),
                                             ("kdn", "channel", "scaled")])
def test_chunk_fwd_long_batch_of_two(gain, decay, keys):
    """B = 2, H = 3 through dn_chunk_fwd_long: the [B, H nseg] segment view
    across batches, and the combine's workgroup mapping when the slices of
    the heads do not divide evenly over the XCDs."""
    wl = W.Workload(f"{gain}_long_b2", gain, decay, "bf16", 2, 3, 1024, 128, 128, keys=keys, seed=90)
    inp = W.generate(wl)
    if gain != "kla":
        rng = np.random.default_rng(91)
        inp["aux0"] = rng.uniform(0.5, 2.0, size=(2, 3, 128)).astype(np.float32)
    o, S, aux = gpu_chunk_long(wl, inp, 4)
    _check(wl, inp, None, o, S, aux)


@pytest.mark.parametrize("gain,decay,keys", [("kla", "scalar", "scaled"), ("pgdn", "scalar", "unit"),
                                             ("kdn", "channel", "scaled")])
def test_chunk_fwd_long_then_resume(gain, decay, keys):
    """T not a multiple of nseg C: the first 1024 tokens by 4 segments, the
    last 101 with dn_chunk_fwd from the segmented call's S_final and
    aux_final, against one oracle pass over all 1125 tokens."""
    from recurrent_sequence_mixer_amd import dn
    wl = W.Workload(f"{gain}_long_resume", gain, decay, "bf16", 1, 2, 1125, 128, 128, keys=keys,
                    seed=95)
    inp = W.generate(wl)
    t = dn.to_device(inp, torch.bfloat16)
    names = ("alpha", "eta", "alphaP", "betaP", "omega", "r")
    part = lambda x, sl: x[:, :, sl].contiguous()
    gates = lambda sl: {n: part(t[n], sl) for n in names if n in t} | (
        {"mu_log": t["mu_log"]} if "mu_log" in t else {})
    kw = dict(gain=gain, eps=wl.eps, x=wl.x, mu_info=wl.mu_info)
    head, tail = slice(0, 1024), slice(1024, None)
    o1, S, aux = dn.chunk_fwd_long(part(t["q"], head), part(t["k"], head), part(t["v"], head),
                                   gates(head), 4, S0=t["S0"], **kw)
    o2, S, aux = dn.chunk_fwd(part(t["q"], tail), part(t["k"], tail), part(t["v"], tail), gates(tail),
                              S0=S, aux0=aux, **kw)
    torch.cuda.synchronize()
    o = torch.cat([o1, o2], dim=2).float().cpu().numpy()
    _check(wl, inp, None, o, S.cpu().numpy(), None if aux is None else aux.cpu().numpy())


@pytest.mark.parametrize("gain", ["kla", "pgdn", "kdn_iso"])
def test_chunk_fwd_long_empty_sequence(gain):
    """T = 0 through dn_chunk_fwd_long: S_final is S0 and aux_final is aux0
    (q, k, v, o point at one-token buffers; no token is read or written)."""
    import ctypes
    from recurrent_sequence_mixer_amd import dn
    decay = "channel" if gain == "kdn_iso" else "scalar"
    desc = dn.make_desc(1, 2, 0, 128, 128, torch.bfloat16, gain, decay, 1e-6, 1.5, 1.0)
    dev = "cuda"
    q, k, v, o = (torch.ones((1, 2, 1, 128), dtype=torch.bfloat16, device=dev) for _ in range(4))
    alpha = torch.ones((1, 2, 1, 128) if decay == "channel" else (1, 2, 1), device=dev,
                       dtype=torch.bfloat16 if decay == "channel" else torch.float32)
    one = torch.ones((1, 2, 1), device=dev)
    gates = {"alpha": alpha, "eta": one}
    if gain == "pgdn":
        gates |= {"alphaP": one, "betaP": one, "mu_log": torch.zeros(2, device=dev)}
    if gain == "kdn_iso":
        gates |= {"omega": one, "r": one}
    g = torch.Generator(device="cpu").manual_seed(9)
    S0 = torch.randn((1, 2, 128, 128), generator=g).to(dev)
    aux0 = (torch.rand((1, 2) if gain == "kdn_iso" else (1, 2, 128), generator=g) + 0.5).to(dev)
    S = torch.full_like(S0, float("nan"))
    aux = torch.full_like(aux0, float("nan"))
    nbytes = dn.lib().dn_chunk_fwd_long_workspace(ctypes.byref(desc), 4)
    ws = torch.empty((nbytes,), dtype=torch.uint8, device=dev)
    gt = dn.make_gates(gates)
    st = dn.lib().dn_chunk_fwd_long(ctypes.byref(desc), 4, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                    ctypes.byref(gt), S0.data_ptr(), aux0.data_ptr(), o.data_ptr(),
                                    S.data_ptr(), aux.data_ptr(), ws.data_ptr(), nbytes,
                                    torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    assert torch.equal(S, S0)
    if gain != "kla":
        assert torch.equal(aux, aux0)
    assert torch.equal(o, torch.ones_like(o))


def test_chunk_fwd_long_pgdn_full_size_sampled_head():
    """PGDN batch-1 prefill B1 H8 T32768 d128 by 16 segments of 2048 tokens,
    one head against the oracle."""
    wl = W.Workload("pgdn_long_B1H8T32768d128", "pgdn", "scalar", "bf16", 1, 8, 32768, 128, 128,
                    keys="unit", seed=52)
    inp = W.generate(wl)
    o, S, aux = gpu_chunk_long(wl, inp, 16, in_place=False)
    _check(wl, inp, [3], o, S, aux)


@pytest.mark.parametrize("decay,dk,T", [("scalar", 128, 333), ("scalar", 64, 200), ("channel", 128, 150)])
def test_pgdn_distinct_centre_per_head(decay, dk, T):
    """PGDN with a different centre mu_h for every head (Preconditioned
    DeltaNet §2.4: mu is per head): B2 H3, so heads of both batch rows use
    their own entry of mu_log.  Scalar decay runs the producer / consumer
    kernel, channel decay (PKDA) the generic one."""
    wl = W.Workload("pgdn_mu_heads", "pgdn", decay, "bf16", 2, 3, T, dk, dk, keys="unit",
                    mu_spread=1.5, seed=500 + T)
    inp = W.generate(wl)
    assert len(set(inp["mu_log"].tolist())) == 3
    o, S, aux = gpu_chunk(wl, inp)
    _check(wl, inp, None, o, S, aux)


@pytest.mark.parametrize("decay,nseg", [("scalar", 4), ("channel", 2)])
def test_chunk_fwd_long_pgdn_distinct_centre_per_head(decay, nseg):
    """dn_chunk_fwd_long, PGDN with a different mu_h per head (B2 H3): the
    centre is repeated into the [H nseg] segment view, head by head."""
    wl = W.Workload("pgdn_long_mu_heads", "pgdn", decay, "bf16", 2, 3, 1024, 128, 128, keys="unit",
                    mu_spread=1.5, seed=520 + nseg)
    inp = W.generate(wl)
    rng = np.random.default_rng(wl.seed)
    inp["aux0"] = rng.uniform(0.5, 2.0, size=(2, 3, 128)).astype(np.float32)
    o, S, aux = gpu_chunk_long(wl, inp, nseg)
    _check(wl, inp, None, o, S, aux)


def test_kla_zero_key_rows():
    """KLA with some all-zero keys (Kaczmarz Linear Attention §2.4: with
    eps > 0 a zero key writes nothing): the column scale eta / eps (about
    1e6) multiplies a zero key in the chunk kernel; o and S must still match."""
    wl = W.Workload("kla_zero_keys", "kla", "scalar", "bf16", 2, 2, 200, 128, 128, seed=530)
    inp = W.generate(wl)
    rng = np.random.default_rng(531)
    zero = rng.random((2, 2, 200)) < 0.15
    zero[:, :, 63] = zero[:, :, 64] = zero[:, :, 0] = True  # chunk edges and the first token
    inp["k"][zero] = 0.0
    o, S, _ = gpu_chunk(wl, inp)
    _check(wl, inp, None, o, S)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
    # f32 io (the generic kernel) as well
    wl = wl.replace(io="f32", dk=64, dv=64)
    inp = W.generate(wl)
    inp["k"][zero] = 0.0
    o, S, _ = gpu_chunk(wl, inp)
    _check(wl, inp, None, o, S)


@pytest.mark.parametrize("gain,keys,io,dk", [("kdn", "scaled", "bf16", 128), ("kdn_iso", "scaled", "bf16", 128),
                                           ("kdn", "scaled", "bf16", 64), ("pgdn", "unit", "bf16", 128),
                                           ("kla", "scaled", "bf16", 128), ("gdn", "unit", "f32", 64)])
def test_strong_channel_decay_in_range(gain, keys, io, dk):
    """Per-channel decay alpha = sigmoid(N(-1, 1)) (about 2 bits of decay per
    token; within a chunk the state decays by 2^-128 or more): every factor
    of the chunk form stays in range, o and S match the oracle.  KDN and
    isotropic KDN run the producer / consumer kernel, PKDA (PGDN), KLA and
    fp32 GDN the generic one."""
    wl = W.Workload(f"{gain}_strong_decay", gain, "channel", io, 2, 2, 333, dk, dk, keys=keys,
                    alpha_mean=-1.0, seed=550 + dk)
    inp = W.generate(wl)
    o, S, aux = gpu_chunk(wl, inp)
    _check(wl, inp, None, o, S, aux)


def test_strong_channel_decay_long_segments():
    """The same strong decay through dn_chunk_fwd_long (4 segments)."""
    wl = W.Workload("kdn_strong_decay_long", "kdn", "channel", "bf16", 1, 2, 1024, 128, 128,
                    alpha_mean=-1.0, seed=560)
    inp = W.generate(wl)
    o, S, aux = gpu_chunk_long(wl, inp, 4)
    _check(wl, inp, None, o, S, aux)


# Per-channel decay beyond the range of the chunk form: a channel that
# decays by 2^-240 or more within half a chunk (alpha = 2^-10 over 24-32
# tokens) has operand factors beyond fp32 range when referred to a point
# inside the chunk.  The chunked kernels flag such a head and the tokenwise
# pass recomputes it; every output, the final state and the statistic match
# the oracle, for the flagged heads and the others alike.
@pytest.mark.parametrize("gain,keys,io", [
    ("kdn", "scaled", "bf16"), ("kdn_iso", "scaled", "bf16"), ("pgdn", "unit", "bf16"),
    ("gdn", "unit", "bf16"), ("kla", "scaled", "bf16"), ("explicit", "unit", "bf16"),
    ("kdn", "scaled", "f32"), ("kdn_iso", "scaled", "f32"), ("gdn", "unit", "f32")])
def test_channel_decay_beyond_range_exact(gain, keys, io):
    d = 128 if io == "bf16" else 64
    wl = W.Workload(f"{gain}_decay_oor_{io}", gain, "channel", io, 1, 3, 448, d, d, keys=keys,
                    seed=570)
    inp = W.generate(wl)
    if gain == "explicit":
        inp["w"] = W.round_io(np.random.default_rng(571).standard_normal((1, 3, 448, d)) * 0.05, io)
    inp["alpha"][0, 0, 320:352, 3] = np.float32(2.0 ** -10)  # head 0: first half of chunk 5
    inp["alpha"][0, 2, 40:64, 7] = np.float32(2.0 ** -10)    # head 2: second half of chunk 0
    o, S, aux = gpu_chunk(wl, inp)
    _check(wl, inp, None, o, S, aux)


def test_channel_decay_beyond_range_in_place():
    """The same with S_final = S0 (an in-place resume): the flagged head's S0
    is left as it was by the chunked pass, for the tokenwise pass to start from."""
    from recurrent_sequence_mixer_amd import dn
    wl = W.Workload("kdn_decay_oor_in_place", "kdn", "channel", "bf16", 1, 2, 448, 128, 128, seed=573)
    inp = W.generate(wl)
    inp["alpha"][0, 1, 100:128, 5] = np.float32(2.0 ** -10)  # head 1: second half of chunk 1
    t = dn.to_device(inp, torch.bfloat16)
    gates = {n: t[n] for n in ("alpha", "omega", "r") if n in t}
    S = t["S0"].clone()
    o, _, aux = dn.chunk_fwd(t["q"], t["k"], t["v"], gates, gain="kdn", mu_info=wl.mu_info, S0=S,
                             aux0=t.get("aux0"), S_final=S)
    torch.cuda.synchronize()
    _check(wl, inp, None, o.float().cpu().numpy(), S.cpu().numpy(), aux.cpu().numpy())


@pytest.mark.parametrize("gain,keys", [("kdn", "scaled"), ("gdn", "unit"), ("kdn_iso", "scaled")])
def test_channel_decay_beyond_range_long(gain, keys):
    """dn_chunk_fwd_long (4 segments, S and the statistic in place) with one
    out-of-range chunk in the third segment of head 0: the combine leaves that
    head's S0 alone and the tokenwise pass starts from it and from the
    statistic entering segment 0."""
    wl = W.Workload(f"{gain}_decay_oor_long", gain, "channel", "bf16", 1, 2, 1024, 128, 128, keys=keys,
                    seed=574)
    inp = W.generate(wl)
    rng = np.random.default_rng(575)
    shape = (1, 2) if gain == "kdn_iso" else (1, 2, 128)
    if gain in ("kdn", "kdn_iso"):
        inp["aux0"] = rng.uniform(0.5, 2.0, size=shape).astype(np.float32)
    inp["alpha"][0, 0, 576:608, 9] = np.float32(2.0 ** -10)  # chunk 9, first half
    o, S, aux = gpu_chunk_long(wl, inp, 4, in_place=True)
    _check(wl, inp, None, o, S, aux)


def test_channel_decay_beyond_range_auto_segments():
    """A few-head shape that dn_chunk_fwd runs by segments on its own (B1 H2
    T8192 d64: 16 segments), with one out-of-range chunk in head 1."""
    wl = W.Workload("gdn_decay_oor_auto", "gdn", "channel", "bf16", 1, 2, 8192, 64, 64, keys="unit",
                    seed=576)
    inp = W.generate(wl)
    inp["alpha"][0, 1, 5000:5024, 11] = np.float32(2.0 ** -10)  # second half of chunk 78
    o, S, aux = gpu_chunk(wl, inp)
    _check(wl, inp, None, o, S, aux)


def test_kdn_mu_dk_and_kla_key_norm_only():
    """The pages' other gain settings on the same kernels: diagonal KDN with
    information scaling mu = d_k (Kalman Delta Networks §2.5), and KLA's
    key-norm-only step 1 / ||k||^2 (eta = 1, eps = 0; Kaczmarz Linear
    Attention ablation)."""
    wl = W.Workload("kdn_mu128", "kdn", "channel", "bf16", 2, 2, 200, 128, 128, mu_info=128.0,
                    seed=41)
    inp = W.generate(wl)
    o, S, aux = gpu_chunk(wl, inp)
    _check(wl, inp, None, o, S, aux)
    wl = W.Workload("kla_keynorm", "kla", "scalar", "bf16", 2, 2, 200, 128, 128, eps=0.0, seed=42)
    inp = W.generate(wl)
    inp["eta"] = np.ones_like(inp["eta"])
    o, S, _ = gpu_chunk(wl, inp)
    _check(wl, inp, None, o, S)


# ---------------------------------------------------------------- edge cases

def test_empty_sequence_copies_state():
    wl = W.Workload("kdn_empty", "kdn", "channel", "bf16", 1, 2, 0, 128, 128, seed=3)
    inp = W.generate(wl.replace(T=5))
    inp = {k: (v[:, :, :0] if v.ndim >= 3 and k not in ("S0",) else v) for k, v in inp.items()}
    inp["aux0"] = np.random.default_rng(0).uniform(0.5, 2, size=(1, 2, 128)).astype(np.float32)
    o, S, aux = gpu_chunk(wl, inp)
    np.testing.assert_array_equal(S, inp["S0"])
    np.testing.assert_array_equal(aux, inp["aux0"])


def test_resume_equals_single_call():
    """chunk_fwd(T1) -> (S, aux) -> chunk_fwd(T2) against one oracle pass."""
    from recurrent_sequence_mixer_amd import dn
    wl = W.Workload("pgdn_resume", "pgdn", "scalar", "bf16", 2, 2, 300, 128, 128, keys="unit", seed=5)
    inp = W.generate(wl)
    t = dn.to_device(inp, torch.bfloat16)
    T1 = 130
    part = lambda x, s: x[:, :, s].contiguous()
    g = lambda s: {n: part(t[n], s) for n in ("alpha", "eta", "alphaP", "betaP")} | {"mu_log": t["mu_log"]}
    kw = dict(gain="pgdn", x=wl.x)
    S = t["S0"].clone()
    aux_a = torch.ones((2, 2, 128), device="cuda")
    aux_b = torch.empty_like(aux_a)
    o1, _, _ = dn.chunk_fwd(part(t["q"], slice(0, T1)), part(t["k"], slice(0, T1)),
                            part(t["v"], slice(0, T1)), g(slice(0, T1)), S0=S, aux0=aux_a,
                            S_final=S, aux_final=aux_b, **kw)  # state in place
    o2, _, _ = dn.chunk_fwd(part(t["q"], slice(T1, None)), part(t["k"], slice(T1, None)),
                            part(t["v"], slice(T1, None)), g(slice(T1, None)), S0=S, aux0=aux_b,
                            S_final=S, aux_final=aux_a, **kw)
    torch.cuda.synchronize()
    o = torch.cat([o1, o2], dim=2).float().cpu().numpy()
    _check(wl, inp, None, o, S.cpu().numpy(), aux_a.cpu().numpy())


def test_deterministic_run_to_run():
    wl = W.WORKLOADS[3].replace(B=1, H=4, T=700)
    inp = W.generate(wl)
    a = gpu_chunk(wl, inp)
    b = gpu_chunk(wl, inp)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_explicit_gain_reads_out_ridge_solution():
    """Exact ATK write keys (Sherman-Morrison, Preconditioned DeltaNet §2.2)
    with no decay: the readout is the ridge solution at every step."""
    from oracle import kalman
    from recurrent_sequence_mixer_amd import dn
    T, d, lam = 150, 64, 2.0
    rng = np.random.default_rng(11)
    K = rng.standard_normal((T, d)).astype(np.float32)
    V = rng.standard_normal((T, d)).astype(np.float32)
    Qr = rng.standard_normal((T, d)).astype(np.float32)
    Wv, _ = kalman.atk_write_vectors(K.astype(np.float64), lam)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()[None, None]
    o, S, _ = dn.chunk_fwd(dev(Qr), dev(K), dev(V), {"alpha": torch.ones((1, 1, T), device="cuda"),
                                                    "w": dev(Wv)}, gain="explicit")
    torch.cuda.synchronize()
    S_ridge = kalman.ridge(K.astype(np.float64), V.astype(np.float64), lam)
    err = np.abs(S.cpu().numpy()[0, 0] - S_ridge).max() / np.abs(S_ridge).max()
    print(f"ridge S err {err:.2e}")
    assert err < 1e-4
    o = o.cpu().numpy()[0, 0]
    for t in (0, 63, 64, 149):
        ref = kalman.ridge(K[:t + 1].astype(np.float64), V[:t + 1].astype(np.float64), lam).T @ Qr[t]
        assert np.abs(o[t] - ref).max() <= 1e-4 * np.abs(ref).max() + 1e-5
