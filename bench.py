"""Benchmark of the gated delta-rule forward engine on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step = one dn_chunk_fwd call (the fused chunked forward: gains, intra-chunk
products, triangular solve, output and state propagation) over the KLA bf16
workload B=8, H=16, T=4096, d_k=d_v=128, C=64, inputs resident in HBM.
`value` is tokens/s (B*T tokens per call).  The same line also reports the
PGDN, diagonal-KDN and isotropic-KDN forwards and the batched decode step (HBM GB/s), the
roofline of the chunked-forward kernel, and the fp64 oracle timed on a
bounded sample on the host CPU.
"""
import argparse
import hashlib
import json
import os
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


def log(msg):
    print(msg, file=sys.stderr, flush=True)


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


def time_chunk_long(wl, nseg, steps, warmup, settle_s=0.0):
    """dn_chunk_fwd_long (segments in parallel) on a workload; ms per call."""
    import torch
    from recurrent_sequence_mixer_amd import dn
    from recurrent_sequence_mixer_amd import workloads as W
    inp = W.generate(wl)
    t = dn.to_device(inp, torch.bfloat16)
    o = torch.empty_like(t["v"])
    S = torch.empty_like(t["S0"])
    gates = {n: t[n] for n in ("alpha", "eta", "alphaP", "betaP", "mu_log", "omega", "r", "w")
             if n in t}
    aux = torch.empty((wl.B, wl.H, wl.dk), device="cuda") if wl.gain in ("pgdn", "kdn") else None
    if wl.gain == "kdn_iso":
        aux = torch.empty((wl.B, wl.H), device="cuda")
    call = lambda: dn.chunk_fwd_long(t["q"], t["k"], t["v"], gates, nseg, gain=wl.gain, eps=wl.eps,
                                     x=wl.x, mu_info=wl.mu_info, S0=t["S0"], aux0=t.get("aux0"),
                                     out=o, S_final=S, aux_final=aux)
    settle(call, settle_s)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(steps):
        call()
    ev1.record()
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / steps


def time_chunk(wl, steps, warmup, settle_s=0.0):
    import torch
    from recurrent_sequence_mixer_amd import dn
    from recurrent_sequence_mixer_amd import workloads as W
    t0 = time.time()
    inp = W.generate(wl)
    t = dn.to_device(inp, torch.bfloat16 if wl.io == "bf16" else torch.float32)
    log(f"[bench] {wl.name}: inputs ready in {time.time() - t0:.1f}s")
    gates = {n: t[n] for n in ("alpha", "eta", "alphaP", "betaP", "mu_log", "omega", "r") if n in t}
    o = torch.empty_like(t["v"])
    S = torch.empty_like(t["S0"])
    aux = torch.empty((wl.B, wl.H, wl.dk), device="cuda") if wl.gain in ("pgdn", "kdn") else None
    if wl.gain == "kdn_iso":
        aux = torch.empty((wl.B, wl.H), device="cuda")
    call = lambda: dn.chunk_fwd(t["q"], t["k"], t["v"], gates, gain=wl.gain, eps=wl.eps, x=wl.x,
                                mu_info=wl.mu_info, S0=t["S0"], out=o, S_final=S, aux_final=aux)
    settle(call, settle_s)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    # dn launches on torch's current stream, so these events bracket exactly its kernels
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    per = []
    for _ in range(steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        call()
        b.record()
        per.append((a, b))
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(steps):
        call()
    ev1.record()
    torch.cuda.synchronize()
    total_ms = ev0.elapsed_time(ev1)
    each = sorted(x.elapsed_time(y) for x, y in per)
    return total_ms / steps, each


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
    ev0.record()
    for s in range(steps_timed):
        q, k, v, g = ins[s % dwl.steps]
        dn.decode_step(q, k, v, g, S, gain="kla", eps=dwl.eps, out=o)
    ev1.record()
    torch.cuda.synchronize()
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


_ORACLE_JOB = {}


def _oracle_heads(heads):
    """One worker's share of the CPU baseline: the oracle over some heads (a
    checksum comes back, not the outputs)."""
    from oracle.recurrence import run_workload
    o, _, _, _ = run_workload(_ORACLE_JOB["wl"], _ORACLE_JOB["inp"], heads=heads)
    return float(o[..., 0].sum())


def cpu_baseline(wl, heads=2, T=1024):
    """The fp64 oracle, as it is, on a bounded sample (`heads` heads x `T`
    tokens), its heads spread over a process pool of the host's cores."""
    import multiprocessing as mp
    from recurrent_sequence_mixer_amd import workloads as W
    sample = wl.replace(B=1, H=heads, T=T)
    _ORACLE_JOB["wl"] = sample
    _ORACLE_JOB["inp"] = W.generate(sample)  # shared with the forked workers
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
        "sample": f"{wl.name}: {heads} heads x {T} tokens (of {wl.B * wl.H} x {wl.T}) over {nproc} "
                  f"processes, {wall:.1f}s wall; value scaled to workload tokens/s ({wl.H} heads per token)",
    }


def main():
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
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the forward engine shards "
              "(batch, head) pairs with no exchange, so multi-GPU runs are not part of this build.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from recurrent_sequence_mixer_amd import workloads as W
    torch.cuda.set_device(0)

    wl = W.WORKLOADS[1]
    ms, each = time_chunk(wl, args.steps, args.warmup, args.settle_s)
    bytes_ = chunk_bytes(wl)
    flops = chunk_flops(wl)
    achieved = bytes_ / (ms * 1e-3) / 1e9
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
    }
    log(f"[bench] {wl.name}: {ms:.3f} ms/step")
    if not args.no_extra:
        extra = {}
        # isotropic KDN (Kalman Delta Networks §2.7) at the diagonal-KDN shape
        iso = W.WORKLOADS[3].replace(name="kdn_iso_bf16_B4H16T8192d128", gain="kdn_iso")
        # batch-1 long prefill at the pages' 131072-token length (8 heads: 16 workgroups)
        longp = W.Workload("kla_long_B1H8T131072d128", "kla", "scalar", "bf16", 1, 8, 131072, 128,
                           128, seed=51)
        for w2 in (W.WORKLOADS[2], W.WORKLOADS[3], iso, longp):
            ms2, _ = time_chunk(w2, max(5, args.steps // 2), args.warmup, args.settle_s)
            b2 = chunk_bytes(w2)
            key = "long_prefill" if w2 is longp else w2.gain
            extra[key] = {"workload": w2.name, "ms": ms2, "tokens_per_s": w2.tokens / (ms2 * 1e-3),
                              "hbm_gbs": b2 / (ms2 * 1e-3) / 1e9,
                              "hbm_frac": b2 / (ms2 * 1e-3) / 1e9 / HBM_PEAK_GBS,
                              "mfma_frac": chunk_flops(w2) / (ms2 * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS}
            log(f"[bench] {w2.name}: {ms2:.3f} ms/step")
        # the same long prefill by 16 segments of 8192 tokens in parallel (dn_chunk_fwd_long)
        ms3 = time_chunk_long(longp, 16, max(5, args.steps // 2), args.warmup, args.settle_s)
        extra["long_prefill_segments"] = {"workload": longp.name, "nseg": 16, "ms": ms3,
                                          "tokens_per_s": longp.tokens / (ms3 * 1e-3),
                                          "hbm_frac": chunk_bytes(longp) / (ms3 * 1e-3) / 1e9 / HBM_PEAK_GBS}
        log(f"[bench] {longp.name} by 16 segments: {ms3:.3f} ms/step")
        # PGDN batch-1 prefill (Preconditioned DeltaNet Fig. 4: batch 1, 8 heads,
        # head dim 128): one pass (16 workgroups) and 16 segments of 2048 tokens
        longpg = W.Workload("pgdn_long_B1H8T32768d128", "pgdn", "scalar", "bf16", 1, 8, 32768, 128,
                            128, keys="unit", seed=52)
        ms4, _ = time_chunk(longpg, max(5, args.steps // 2), args.warmup, args.settle_s)
        ms5 = time_chunk_long(longpg, 16, max(5, args.steps // 2), args.warmup, args.settle_s)
        extra["long_prefill_pgdn"] = {"workload": longpg.name, "ms_one_pass": ms4, "nseg": 16,
                                      "ms_segments": ms5,
                                      "tokens_per_s_segments": longpg.tokens / (ms5 * 1e-3)}
        log(f"[bench] {longpg.name}: one pass {ms4:.3f} ms, by 16 segments {ms5:.3f} ms")
        # diagonal KDN with per-channel decay at the same batch-1 shape
        longkd = W.Workload("kdn_long_B1H8T32768d128", "kdn", "channel", "bf16", 1, 8, 32768, 128,
                            128, seed=53)
        ms6, _ = time_chunk(longkd, max(5, args.steps // 4), args.warmup, args.settle_s)
        ms7 = time_chunk_long(longkd, 16, max(5, args.steps // 2), args.warmup, args.settle_s)
        extra["long_prefill_kdn"] = {"workload": longkd.name, "ms_one_pass": ms6, "nseg": 16,
                                     "ms_segments": ms7,
                                     "tokens_per_s_segments": longkd.tokens / (ms7 * 1e-3)}
        log(f"[bench] {longkd.name}: one pass {ms6:.3f} ms, by 16 segments {ms7:.3f} ms")
        dwl = W.WORKLOADS[4]
        dms = time_decode(dwl, args.decode_steps, args.settle_s)
        gbs = decode_bytes(dwl) / (dms * 1e-3) / 1e9
        extra["decode"] = {"workload": dwl.name, "ms_per_step": dms,
                           "seq_tokens_per_s": dwl.N / (dms * 1e-3), "hbm_gbs": gbs,
                           "hbm_frac": gbs / HBM_PEAK_GBS, "bytes_per_step": decode_bytes(dwl)}
        log(f"[bench] decode: {dms:.3f} ms/step, {gbs:.0f} GB/s")
        out["extra"] = extra
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_heads, args.cpu_tokens)
        log(f"[bench] cpu baseline: {out['cpu_baseline']}")
    if args.calib_copy_mib:
        calib_copy(args.calib_copy_mib)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
