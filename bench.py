"""Benchmark of the gated delta-rule forward engine on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step = one dn_chunk_fwd call (the fused chunked forward: gains, intra-chunk
products, triangular solve, output and state propagation) over the KLA bf16
workload B=8, H=16, T=4096, d_k=d_v=128, C=64, inputs resident in HBM.
`value` is tokens/s (B*T tokens per call).  The same line also reports the
PGDN, diagonal-KDN and isotropic-KDN forwards, batch-1 long prefills and the
batched decode step (HBM GB/s), the roofline of the chunked-forward kernel,
the parity of sampled heads of the timed run against the fp64 oracle, and the
oracle timed on the host CPU over the same inputs.

Every timed loop is bracketed by two one-element fill launches, so that the
dispatches between such a pair in a `rocprofv3 --kernel-trace` of this script
are exactly the timed launches (no settle or warm-up launches).
"""
import argparse
import ctypes
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 matrix (256 CU x 2.4 GHz x 4096 flop/clk)
METRIC = "delta-rule fwd tokens/s + %MFMA peak (T=4096,d=128); decode GB/s vs HBM peak"
KERNEL_SOURCES = ("recurrent_sequence_mixer_amd/csrc/chunk_fwd_ws.hip",
                  "recurrent_sequence_mixer_amd/csrc/common.hpp",
                  "recurrent_sequence_mixer_amd/csrc/gains.hpp")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "chunk_fwd_kla_B8H16T4096d128_traffic.txt")
GATES = ("alpha", "eta", "alphaP", "betaP", "mu_log", "omega", "r", "w")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class Region:
    """Delimiters of the timed loops in a kernel trace: a one-element fill
    launch right before and right after each timed loop (on the same stream),
    so that the dispatches between a pair of fills in a `rocprofv3
    --kernel-trace` of this script are exactly the timed launches (no settle
    or warm-up launches)."""

    def __init__(self):
        import torch
        self.flag = torch.zeros(1, device="cuda")

    def resume(self):
        self.flag.fill_(1.0)

    def pause(self):
        self.flag.fill_(0.0)


REGION = None


def chunk_bytes(wl):
    """Algorithmic HBM bytes of one chunked forward: every input read once,
    every output written once (q, k, v, o, gates, S0, S_T, aux)."""
    es = 2 if wl.io == "bf16" else 4
    ht = wl.B * wl.H * wl.T
    per_ht = es * (2 * wl.dk + 2 * wl.dv)  # q, k, v, o
    if wl.decay == "scalar":
        per_ht += 4  # alpha
    else:
        per_ht += es * wl.dk
    per_ht += {"kla": 4, "gdn": 4, "pgdn": 12, "kdn": 4 + es * wl.dk, "kdn_iso": 8,
               "explicit": es * wl.dk}[wl.gain]
    state = 2 * wl.B * wl.H * wl.dk * wl.dv * 4
    aux = 2 * wl.B * wl.H * wl.dk * 4 if wl.gain in ("pgdn", "kdn") else 0
    if wl.gain == "kdn_iso":
        aux = 2 * wl.B * wl.H * 4
    return ht * per_ht + state + aux


def chunk_flops(wl):
    """Counted flops of the chunk form per head-token (dense C x C products and
    a forward-substitution solve): 6 dk dv + 4 C dk + 3 C dv."""
    return wl.B * wl.H * wl.T * (6 * wl.dk * wl.dv + 4 * wl.C * wl.dk + 3 * wl.C * wl.dv)


def decode_bytes(dwl):
    """Per step: read + write S, read q, k, v (bf16) and eta, alpha, write o."""
    nh = dwl.N * dwl.H
    return nh * (2 * dwl.dk * dwl.dv * 4 + 2 * (2 * dwl.dk + dwl.dv) + 8 + 2 * dwl.dv)


def settle(call, seconds):
    """Run `call` untimed for about `seconds` of wall time before the warm-up
    steps.  Under sustained load the GPU's clocks ramp up over the first tens
    of milliseconds (back-to-back launches of the chunk kernel go from
    0.25 ms to a steady 0.17-0.18 ms); this puts the W warm-up and the K timed
    steps at that steady state.  Synchronises every few calls so that the
    queue stays short."""
    import torch
    end = time.time() + seconds
    while time.time() < end:
        for _ in range(8):
            call()
        torch.cuda.synchronize()


def prepare_chunk(wl):
    """Inputs on the device, output buffers and the workspace of a chunked
    forward; returns (inputs numpy, tensors, call)."""
    import torch
    from recurrent_sequence_mixer_amd import dn
    from recurrent_sequence_mixer_amd import workloads as W
    t0 = time.time()
    inp = W.generate(wl)
    t = dn.to_device(inp, torch.bfloat16 if wl.io == "bf16" else torch.float32)
    log(f"[bench] {wl.name}: inputs ready in {time.time() - t0:.1f}s")
    gates = {n: t[n] for n in GATES if n in t}
    o = torch.empty_like(t["v"])
    S = torch.empty_like(t["S0"])
    aux = torch.empty((wl.B, wl.H, wl.dk), device="cuda") if wl.gain in ("pgdn", "kdn") else None
    if wl.gain == "kdn_iso":
        aux = torch.empty((wl.B, wl.H), device="cuda")
    desc = dn.make_desc(wl.B, wl.H, wl.T, wl.dk, wl.dv, t["q"].dtype, wl.gain, wl.decay, wl.eps,
                        wl.x, wl.mu_info)
    nbytes = dn.workspace_bytes(desc)
    ws = torch.empty((nbytes,), dtype=torch.uint8, device="cuda") if nbytes else None
    call = lambda: dn.chunk_fwd(t["q"], t["k"], t["v"], gates, gain=wl.gain, eps=wl.eps, x=wl.x,
                                mu_info=wl.mu_info, S0=t["S0"], out=o, S_final=S, aux_final=aux,
                                workspace=ws)
    return inp, {"o": o, "S": S, "aux": aux, "ws_bytes": nbytes}, call


def time_calls(call, steps, warmup, settle_s, per_step=False):
    """Settle, warm up, then time `steps` calls between HIP events on torch's
    current stream (the stream the library launches on).  Returns (ms per
    call, sorted per-call ms or None)."""
    import torch
    settle(call, settle_s)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    each = None
    if per_step:
        per = []
        for _ in range(steps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            call()
            b.record()
            per.append((a, b))
        torch.cuda.synchronize()
        each = sorted(x.elapsed_time(y) for x, y in per)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    REGION.resume()
    ev0.record()
    for _ in range(steps):
        call()
    ev1.record()
    torch.cuda.synchronize()
    REGION.pause()
    return ev0.elapsed_time(ev1) / steps, each


def parity_sample(wl, inp, out, heads):
    """Max relative error (per head, worst of the sampled heads) of o and S_T
    of the timed run against the fp64 oracle on the same inputs."""
    from oracle.recurrence import run_workload
    o_ref, S_ref, _, _ = run_workload(wl, inp, heads=heads)
    flat = lambda x: x.reshape((wl.B * wl.H,) + tuple(x.shape[2:]))[heads].float().cpu().numpy()
    rel = lambda g, r: float(max(np.abs(g[i] - r[i]).max() / np.abs(r[i]).max() for i in range(len(heads))))
    return {"heads": list(heads), "o": rel(flat(out["o"]), o_ref), "S": rel(flat(out["S"]), S_ref)}


def time_decode(dwl, steps_timed, settle_s=0.0):
    import torch
    from recurrent_sequence_mixer_amd import dn
    from recurrent_sequence_mixer_amd import workloads as W
    t0 = time.time()
    S = torch.from_numpy(W.generate_decode_state(dwl)).cuda()
    ins = []
    for s in range(dwl.steps):
        st = dn.to_device(W.generate_decode_step(dwl, s), torch.bfloat16)
        ins.append((st["q"], st["k"], st["v"], {"alpha": st["alpha"], "eta": st["eta"]}))
    log(f"[bench] decode: {dwl.steps} steps of inputs ready in {time.time() - t0:.1f}s")
    o = torch.empty((dwl.N, dwl.H, dwl.dv), dtype=torch.bfloat16, device="cuda")
    Sw = S.clone()  # scratch state for the untimed steps
    q0, k0, v0, g0 = ins[0]
    settle(lambda: dn.decode_step(q0, k0, v0, g0, Sw, gain="kla", eps=dwl.eps, out=o), settle_s)
    for s in range(3):  # warm-up steps on a scratch copy of the state
        q, k, v, g = ins[s]
        dn.decode_step(q, k, v, g, S.clone(), gain="kla", eps=dwl.eps, out=o)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    REGION.resume()
    ev0.record()
    for s in range(steps_timed):
        q, k, v, g = ins[s % dwl.steps]
        dn.decode_step(q, k, v, g, S, gain="kla", eps=dwl.eps, out=o)
    ev1.record()
    torch.cuda.synchronize()
    REGION.pause()
    return ev0.elapsed_time(ev1) / steps_timed


def kernel_source_hash():
    """sha256[:16] of the chunk kernel's code: its sources with comments and
    blank lines removed, so that an edit of the comments alone keeps the
    counters that were taken on the same code."""
    import re
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel)) as f:
            text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
        for line in text.splitlines():
            code = line.split("//", 1)[0].rstrip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the chunked-forward kernel from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary, or None when the kernel
    sources changed since the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != kernel_source_hash():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def calib_copy(mib):
    """A plain device copy of known size, for scaling HBM byte counters."""
    import torch
    n = mib * 1024 * 1024 // 4
    src = torch.ones(n, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] calibration copy: {mib} MiB read + {mib} MiB written, 3 launches")


def host_info():
    import torch
    cpu = platform.processor()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": cpu, "host_cores": len(os.sched_getaffinity(0)), "numpy": np.__version__,
            "torch": torch.__version__, "hip": torch.version.hip,
            "gpu": torch.cuda.get_device_name(0), "python": platform.python_version()}


_ORACLE_JOB = {}


def _oracle_heads(heads):
    """One worker's share of the CPU baseline: the oracle over some heads (a
    checksum comes back, not the outputs)."""
    from oracle.recurrence import run_workload
    o, _, _, _ = run_workload(_ORACLE_JOB["wl"], _ORACLE_JOB["inp"], heads=heads)
    return float(o[..., 0].sum())


def cpu_baseline(wl, inp, heads, T):
    """The fp64 oracle, as it is, on a bounded sample of the timed workload's
    own inputs (`heads` heads x the first `T` tokens), its heads spread over a
    process pool of the host's cores."""
    import multiprocessing as mp
    T = min(T, wl.T)
    heads = min(heads, wl.B * wl.H)
    _ORACLE_JOB["wl"] = wl.replace(T=T)
    _ORACLE_JOB["inp"] = inp  # shared with the forked workers
    nproc = max(1, min(len(os.sched_getaffinity(0)), heads))
    shares = [list(range(i, heads, nproc)) for i in range(nproc)]
    t0 = time.time()
    with mp.get_context("fork").Pool(nproc) as pool:
        pool.map(_oracle_heads, shares)
    wall = time.time() - t0
    head_tok_s = heads * T / wall
    return {
        "value": head_tok_s / wl.H,  # workload tokens/s: every token passes H heads
        "unit": "tokens/s",
        "cores": nproc,
        "kind": "oracle",
        "sample": f"{wl.name}: the timed inputs' first {heads} heads (of {wl.B * wl.H}) x {T} tokens "
                  f"(of {wl.T}) over {nproc} processes, {wall:.1f}s wall; value scaled to workload "
                  f"tokens/s ({wl.H} heads per token)",
    }


def extra_chunk(wl, steps, warmup, settle_s):
    _, out, call = prepare_chunk(wl)
    ms, _ = time_calls(call, steps, warmup, settle_s)
    b = chunk_bytes(wl)
    log(f"[bench] {wl.name}: {ms:.3f} ms/step")
    return {"workload": wl.name, "ms": ms, "tokens_per_s": wl.tokens / (ms * 1e-3),
            "hbm_gbs": b / (ms * 1e-3) / 1e9, "hbm_frac": b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "mfma_frac": chunk_flops(wl) / (ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS,
            "workspace_bytes": out["ws_bytes"]}


def bwd_bytes(wl):
    """Least HBM bytes of one chunked backward: q, k, v, dO and the gates read
    once, every gradient (fp32) written once, S0 / dS_T read and dS0 written."""
    es = 2 if wl.io == "bf16" else 4
    nht = wl.B * wl.H * wl.T
    per_ht = 2 * wl.dk * es + 2 * wl.dv * es + 8  # q, k, v, dO; eta, alpha
    per_ht += 2 * wl.dk * 4 + wl.dv * 4 + 8       # dq, dk, dv; deta, dalpha
    return nht * per_ht + 3 * wl.B * wl.H * wl.dk * wl.dv * 4


def extra_bwd(wl, steps, warmup, settle_s):
    """The chunked backward (dn_chunk_bwd) of a KLA workload."""
    import numpy as np
    import torch
    from recurrent_sequence_mixer_amd import dn
    from recurrent_sequence_mixer_amd import workloads as W
    inp = W.generate(wl)
    io = torch.bfloat16 if wl.io == "bf16" else torch.float32
    t = dn.to_device(inp, io)
    gates = {n: t[n] for n in GATES if n in t}
    rng = np.random.default_rng(wl.seed + 1)
    dO = torch.from_numpy(W.round_io(rng.standard_normal((wl.B, wl.H, wl.T, wl.dv)), wl.io)).cuda().to(io)
    dS_T = torch.from_numpy(rng.standard_normal((wl.B, wl.H, wl.dk, wl.dv)).astype(np.float32)).cuda()
    desc = dn.make_desc(wl.B, wl.H, wl.T, wl.dk, wl.dv, io, wl.gain, wl.decay, wl.eps, wl.x, wl.mu_info)
    nbytes = dn.lib().dn_chunk_bwd_workspace(ctypes.byref(desc))
    ws = torch.empty((nbytes,), dtype=torch.uint8, device="cuda")
    call = lambda: dn.chunk_bwd(t["q"], t["k"], t["v"], gates, dO, gain=wl.gain, eps=wl.eps, S0=t["S0"],
                                dS_T=dS_T, workspace=ws)
    ms, _ = time_calls(call, steps, warmup, settle_s)
    b = bwd_bytes(wl)
    log(f"[bench] backward {wl.name}: {ms:.3f} ms/step")
    return {"workload": wl.name, "ms": ms, "tokens_per_s": wl.tokens / (ms * 1e-3),
            "hbm_gbs": b / (ms * 1e-3) / 1e9, "hbm_frac": b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "workspace_bytes": nbytes}


def main():
    global REGION
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-extra", action="store_true", help="only the headline workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-steps", type=int, default=256)
    ap.add_argument("--settle-s", type=float, default=0.3,
                    help="untimed run of each workload before its warm-up steps (GPU clock ramp)")
    ap.add_argument("--cpu-heads", type=int, default=128, help="oracle sample: heads")
    ap.add_argument("--cpu-tokens", type=int, default=4096, help="oracle sample: tokens per head")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a device copy of this size (byte-counter calibration)")
    ap.add_argument("--only", default=None,
                    help="time only these extras (comma list of pgdn, kdn, kdn_iso, kda, kla_channel, long, bwd, "
                         "decode) "
                         "after the headline")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the forward engine shards "
              "(batch, head) pairs with no exchange, so multi-GPU runs are not part of this build.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from recurrent_sequence_mixer_amd import workloads as W
    torch.cuda.set_device(0)
    REGION = Region()

    wl = W.WORKLOADS[1]
    inp, out1, call = prepare_chunk(wl)
    ms, each = time_calls(call, args.steps, args.warmup, args.settle_s, per_step=True)
    bytes_ = chunk_bytes(wl)
    flops = chunk_flops(wl)
    achieved = bytes_ / (ms * 1e-3) / 1e9
    log(f"[bench] {wl.name}: {ms:.3f} ms/step")
    nh = wl.B * wl.H
    parity = parity_sample(wl, inp, out1, [0, nh // 2 + 3, nh - 1])
    log(f"[bench] parity of the timed run (sampled heads): {parity}")
    out = {
        "metric": METRIC,
        "value": wl.tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "gain": wl.gain, "B": wl.B, "H": wl.H, "T": wl.T,
                   "dk": wl.dk, "dv": wl.dv, "C": wl.C},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(),
                     "kernel": "chunk_fwd_ws_kernel<128,KLA>",
                     "bytes_per_launch": bytes_},
        "mfma": {"counted_tflops": flops / (ms * 1e-3) / 1e12,
                 "frac_of_bf16_peak": flops / (ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS,
                 "counted_flops_per_launch": flops},
        "step_ms_p10_p50_p90": [each[len(each) // 10], each[len(each) // 2], each[9 * len(each) // 10]],
        "settle_s": args.settle_s,
        "parity": parity,
        "inputs_sha256": W.sha256(inp),
        "host": host_info(),
    }
    if not args.no_extra:
        extra = {}
        only = None if args.only is None else set(args.only.split(","))
        want = lambda key: only is None or key in only
        half = max(5, args.steps // 2)
        # isotropic KDN (Kalman Delta Networks §2.7) at the diagonal-KDN shape
        iso = W.WORKLOADS[3].replace(name="kdn_iso_bf16_B4H16T8192d128", gain="kdn_iso")
        # GDN with per-channel decay (KDA) and KLA with per-channel decay at the
        # KLA shape B8 H16 T4096 d128
        kda = W.WORKLOADS[1].replace(name="kda_bf16_B8H16T4096d128", gain="gdn", decay="channel",
                                     keys="unit")
        kla_ch = W.WORKLOADS[1].replace(name="kla_channel_bf16_B8H16T4096d128", decay="channel")
        for key, w2 in (("pgdn", W.WORKLOADS[2]), ("kdn", W.WORKLOADS[3]), ("kdn_iso", iso),
                        ("kda", kda), ("kla_channel", kla_ch)):
            if want(key):
                extra[key] = extra_chunk(w2, half, args.warmup, args.settle_s)
        if want("long"):
            # batch-1 long prefills (dn_chunk_fwd picks 16 segments per head for
            # these shapes): KLA at the pages' 131072-token length, PGDN and
            # diagonal KDN at B1 H8 T32768 (Preconditioned DeltaNet Fig. 4:
            # batch 1, 8 heads, head dim 128)
            longs = (("long_prefill", W.Workload("kla_long_B1H8T131072d128", "kla", "scalar", "bf16", 1,
                                                 8, 131072, 128, 128, seed=51)),
                     ("long_prefill_pgdn", W.Workload("pgdn_long_B1H8T32768d128", "pgdn", "scalar",
                                                      "bf16", 1, 8, 32768, 128, 128, keys="unit",
                                                      seed=52)),
                     ("long_prefill_kdn", W.Workload("kdn_long_B1H8T32768d128", "kdn", "channel", "bf16",
                                                     1, 8, 32768, 128, 128, seed=53)))
            for key, w2 in longs:
                extra[key] = extra_chunk(w2, half, args.warmup, args.settle_s)
        if want("bwd"):
            # the chunked backward at the headline shape and at the pages' operator
            # shape (Preconditioned DeltaNet Fig. 4: batch 1, 8 heads, head dim 128)
            long_op = W.Workload("kla_B1H8T32768d128", "kla", "scalar", "bf16", 1, 8, 32768, 128, 128, seed=55)
            for key, w2 in (("bwd_kla", W.WORKLOADS[1]),
                            ("bwd_kla_B1H8", W.Workload("kla_bwd_B1H8T4096d128", "kla", "scalar", "bf16",
                                                        1, 8, 4096, 128, 128, seed=54)),
                            ("bwd_kla_B1H8T32768", long_op)):
                extra[key] = extra_bwd(w2, 3, 1, 0.0)
            # and the forward of the longest operator shape, for forward + backward
            extra["fwd_kla_B1H8T32768"] = extra_chunk(long_op, 5, 1, 0.0)
        if want("decode"):
            dwl = W.WORKLOADS[4]
            dms = time_decode(dwl, args.decode_steps, args.settle_s)
            gbs = decode_bytes(dwl) / (dms * 1e-3) / 1e9
            extra["decode"] = {"workload": dwl.name, "ms_per_step": dms,
                               "seq_tokens_per_s": dwl.N / (dms * 1e-3), "hbm_gbs": gbs,
                               "hbm_frac": gbs / HBM_PEAK_GBS, "bytes_per_step": decode_bytes(dwl)}
            log(f"[bench] decode: {dms:.3f} ms/step, {gbs:.0f} GB/s")
        out["extra"] = extra
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, inp, args.cpu_heads, args.cpu_tokens)
        log(f"[bench] cpu baseline: {out['cpu_baseline']}")
    if args.calib_copy_mib:
        calib_copy(args.calib_copy_mib)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
