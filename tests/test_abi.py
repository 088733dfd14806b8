"""The C-ABI library: it loads, exports what include/dn.h declares, and rejects
invalid arguments on the host before launching anything.

These run without a GPU: every call here fails validation, so no HIP call is
made (the pointers are never dereferenced).
"""
import ctypes
import os
import re
import subprocess
import sys

import pytest

from recurrent_sequence_mixer_amd import dn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(dn.LIB_PATH),
                                reason="libdn.so not built (run __graft_entry__.build())")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dn_[a-z_]+)\s*\(", text)))


def test_exports_match_header():
    decl = declared_functions()
    assert decl == sorted(dn.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", dn.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = sorted({ln.split()[-1] for ln in out.splitlines() if " T dn_" in ln})
    assert exported == decl
    L = dn.lib()
    for name in decl:
        assert hasattr(L, name)


def test_version_and_status_strings():
    assert dn.lib().dn_version() == 1
    for code in dn.STATUS:
        assert dn.status_string(code)
    assert dn.status_string(12345) == "unknown status"


FAKE = 1 << 40  # a host integer that is never dereferenced


def _gates(**kw):
    g = dict(alpha=FAKE, eta=FAKE + (1 << 30), alphaP=None, betaP=None, mu_log=None, omega=None,
             r=None, w=None)
    g.update(kw)
    return dn.DnGates(*[g[n] for n in ("alpha", "eta", "alphaP", "betaP", "mu_log", "omega", "r", "w")])


def _chunk(desc, gates=None, q=FAKE + (2 << 30), k=FAKE + (3 << 30), v=FAKE + (4 << 30),
           o=FAKE + (5 << 30), S0=None, aux0=None, S_final=None, aux_final=None, ws=None,
           nbytes=0):
    gates = gates or _gates()
    return dn.lib().dn_chunk_fwd(ctypes.byref(desc), q, k, v, ctypes.byref(gates), S0, aux0, o,
                                 S_final, aux_final, ws, nbytes, None)


def _desc(**kw):
    base = dict(B=2, H=3, T=100, dk=128, dv=128, io=1, gain="kla", decay="scalar")
    base.update(kw)
    return dn.make_desc(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(dk=100), -2), (dict(dk=136), -2), (dict(dk=0), -2), (dict(dv=36), -2), (dict(dv=200), -2), (dict(dv=4096), -2), (dict(B=0), -2), (dict(H=0), -2), (dict(T=-1), -2),
    (dict(B=300, H=300), -2), (dict(io=7), -3), (dict(gain=9), -4), (dict(decay=3), -4),
    (dict(eps=-1.0), -4), (dict(gain="pgdn", x=0.5), -4), (dict(gain="kdn", mu_info=0.0), -4),
    (dict(gain="kdn_iso", mu_info=-1.0), -4), (dict(gain=6), -4),
])
def test_chunk_fwd_rejects_bad_descriptor(kw, status):
    assert _chunk(_desc(**kw)) == status


def test_chunk_fwd_rejects_bad_chunk_length():
    d = _desc()
    d.C = 32
    assert _chunk(d) == -2


def test_chunk_fwd_rejects_missing_pointers():
    assert _chunk(_desc(), q=None) == -1
    assert _chunk(_desc(), o=None) == -1
    assert _chunk(_desc(), gates=_gates(alpha=None)) == -1
    assert _chunk(_desc(), gates=_gates(eta=None)) == -1
    assert _chunk(_desc(gain="pgdn")) == -1  # alphaP, betaP, mu_log missing
    assert _chunk(_desc(gain="kdn")) == -1  # omega, r missing
    assert _chunk(_desc(gain="kdn_iso")) == -1  # omega, r missing
    assert _chunk(_desc(gain="explicit")) == -1  # w missing
    assert dn.lib().dn_chunk_fwd(None, FAKE, FAKE, FAKE, None, None, None, FAKE, None, None,
                                 None, 0, None) == -1


def test_chunk_fwd_rejects_overlaps():
    d = _desc(B=1, H=1, T=64, dk=128, dv=128)
    qbytes = 64 * 128 * 2
    q = FAKE + (2 << 30)
    # output overlapping an input
    assert _chunk(d, q=q, o=q + qbytes // 2) == -8
    # S_final overlapping S0 without being the same buffer
    S0 = FAKE + (8 << 30)
    assert _chunk(d, S0=S0, S_final=S0 + 4) == -8
    # S_final overlapping the output
    assert _chunk(d, S_final=FAKE + (5 << 30)) == -8


def test_decode_rejects_bad_arguments():
    L = dn.lib()
    g = _gates()
    f = lambda desc, S=FAKE + (9 << 30), aux=None: L.dn_decode_step(
        ctypes.byref(desc), FAKE + (2 << 30), FAKE + (3 << 30), FAKE + (4 << 30), ctypes.byref(g),
        S, aux, FAKE + (5 << 30), None)
    assert f(_desc(T=2)) == -2
    assert f(_desc(T=1), S=None) == -1
    assert f(_desc(T=1, gain="pgdn")) == -1
    assert f(_desc(T=1, dk=50)) == -2  # head widths are multiples of 8
    assert f(_desc(T=1, dv=100)) == -2
    assert f(_desc(T=1, dv=200)) == -2  # wide value heads are multiples of 64 columns
    assert f(_desc(T=1, dv=4096)) == -2


def test_gain_prep_rejects_bad_arguments():
    L = dn.lib()
    g = _gates()
    d = _desc()
    gp = lambda desc, k, w, ws=None, nbytes=0, gates=g: L.dn_gain_prep(
        ctypes.byref(desc), k, ctypes.byref(gates), None, w, None, None, None, ws, nbytes, None)
    assert gp(d, FAKE, None) == -1
    assert gp(_desc(dk=81), FAKE, FAKE + (7 << 30)) == -2
    # w_out overlapping k
    assert gp(d, FAKE + (3 << 30), FAKE + (3 << 30)) == -8
    # PGDN over whole chunks scans them in parallel and needs its workspace
    dp = _desc(B=2, H=3, T=1024, gain="pgdn")
    gpg = _gates(alphaP=FAKE + (6 << 30), betaP=FAKE + (7 << 30), mu_log=FAKE + (8 << 30))
    need = L.dn_workspace_bytes(ctypes.byref(dp))
    assert need > 0
    assert gp(dp, FAKE + (3 << 30), FAKE + (12 << 30), gates=gpg) == -5
    assert gp(dp, FAKE + (3 << 30), FAKE + (12 << 30), FAKE + (20 << 30), need - 1, gates=gpg) == -5
    # workspace overlapping w_out
    assert gp(dp, FAKE + (3 << 30), FAKE + (12 << 30), FAKE + (12 << 30) + 64, need, gates=gpg) == -8


def test_workspace_bytes_layouts():
    """dn_workspace_bytes follows the layouts the header states."""
    L = dn.lib()
    ws = lambda **kw: L.dn_workspace_bytes(ctypes.byref(_desc(**kw)))
    # many heads: one pass, nothing; gains without a statistic scan by chunks with none
    assert ws(B=8, H=16, T=4096) == 0
    assert ws(B=2, H=3, T=1024) == 0  # few heads but a short sequence: one pass is cheaper
    assert ws(B=8, H=16, T=4096, io=0, dk=64, dv=64, gain="pgdn") == 0  # fp32: serial scan
    assert ws(B=8, H=16, T=100, gain="pgdn") == 0  # not whole chunks: serial scan
    # per-channel decay, one pass: an int per head, the out-of-range flags of
    # the tokenwise pass
    assert ws(B=8, H=16, T=4096, decay="channel") == 8 * 16 * 4
    assert ws(B=8, H=16, T=4096, gain="gdn", decay="channel", io=0, dk=64, dv=64) == 8 * 16 * 4
    # the chunk-parallel gain scan: summaries [B, H, dk, T / C, 3], the
    # statistic entering every chunk [B, H, T / C, dk] and PGDN's centre per
    # chunk [H T / C], each on a 256-byte boundary
    summ, aux_in, mu = 6 * 128 * 16 * 3 * 4, 6 * 16 * 128 * 4, 3 * 16 * 4
    r256 = lambda x: (x + 255) // 256 * 256
    assert ws(B=2, H=3, T=1024, gain="pgdn") == r256(r256(summ) + aux_in) + mu
    assert ws(B=2, H=3, T=1024, gain="kdn_iso", decay="channel") == r256(r256(6 * 16 * 3 * 4) + 6 * 16 * 4) + mu
    # a batch-1 long prefill: 16 segments of 8192 tokens, dn_chunk_fwd_long's layout
    d = _desc(B=1, H=8, T=131072)
    assert ws(B=1, H=8, T=131072) == L.dn_chunk_fwd_long_workspace(ctypes.byref(d), 16) == \
        128 * 128 * (128 + 2 * 128) * 4
    dp = _desc(B=1, H=8, T=32768, gain="pgdn")
    long16 = L.dn_chunk_fwd_long_workspace(ctypes.byref(dp), 16)
    prep = r256(r256(8 * 128 * 512 * 3 * 4) + 8 * 512 * 128 * 4) + 8 * 512 * 4
    assert ws(B=1, H=8, T=32768, gain="pgdn") == max(long16, prep)
    assert ws(B=0, H=8, T=32768) == 0  # invalid descriptor


def test_chunk_fwd_rejects_missing_workspace():
    """A shape that runs by segments needs its workspace (DN_ERR_WORKSPACE),
    which may not overlap another buffer (DN_ERR_ALIAS)."""
    L = dn.lib()
    d = _desc(B=1, H=8, T=131072)
    need = L.dn_workspace_bytes(ctypes.byref(d))
    assert _chunk(d) == -5
    assert _chunk(d, ws=FAKE + (20 << 30), nbytes=need - 256) == -5
    assert _chunk(d, ws=FAKE + (5 << 30), nbytes=need) == -8  # the output's range
    assert _chunk(d, ws=FAKE + (2 << 30) + 4096, nbytes=need) == -8  # inside q


def test_chunk_fwd_long_rejects_bad_arguments():
    L = dn.lib()
    g = _gates()
    q, k, v, o = FAKE + (2 << 30), FAKE + (3 << 30), FAKE + (4 << 30), FAKE + (5 << 30)
    ws = FAKE + (20 << 30)

    def f(desc, nseg=4, ws=ws, nbytes=None, o=o):
        if nbytes is None:
            nbytes = L.dn_chunk_fwd_long_workspace(ctypes.byref(desc), nseg)
        return L.dn_chunk_fwd_long(ctypes.byref(desc), nseg, q, k, v, ctypes.byref(g), None, None, o,
                                   None, None, ws, nbytes, None)
    d = _desc(B=1, H=2, T=1024)
    # fp32 A [B H nseg, dk, dk], then B and S_in [B H nseg, dk, dv]
    assert L.dn_chunk_fwd_long_workspace(ctypes.byref(d), 4) == 8 * 128 * (128 + 2 * 128) * 4
    assert L.dn_chunk_fwd_long_workspace(ctypes.byref(d), 0) == 0
    assert f(_desc(B=1, H=2, T=1024, io=0, dk=64, dv=64)) == -6  # fp32: not built
    # the statistic's part: aux_in [B H nseg, dk] and mu_seg [H nseg] on
    # 256-byte boundaries, then 3 floats per channel for each 256-token piece
    dp = _desc(B=1, H=2, T=1024, gain="pgdn")
    base = 8 * 128 * (128 + 2 * 128) * 4
    assert L.dn_chunk_fwd_long_workspace(ctypes.byref(dp), 4) == base + 4096 + 256 + 2 * 4 * 3 * 128 * 4
    assert L.dn_chunk_fwd_long_workspace(ctypes.byref(d), 3) == 0  # does not divide T
    # isotropic KDN: one statistic per head (aux_in 8 floats, mu_seg 8 floats, 2 x 4 pieces x 3)
    # then (per-channel decay) the out-of-range flags, an int per segment
    di = _desc(B=1, H=2, T=1024, gain="kdn_iso", decay="channel")
    assert L.dn_chunk_fwd_long_workspace(ctypes.byref(di), 4) == base + 256 + 256 + 256 + 2 * 4 * 4
    # 192-token segments: 64-token pieces, 3 per segment
    assert L.dn_chunk_fwd_long_workspace(ctypes.byref(_desc(B=1, H=2, T=1536, gain="pgdn")), 8) == \
        16 * 128 * (128 + 2 * 128) * 4 + 16 * 128 * 4 + 256 + 2 * 24 * 3 * 128 * 4
    assert f(d, nseg=0) == -2
    assert f(d, nseg=3) == -2  # does not divide T
    assert f(d, nseg=32) == -2  # segments of 32 tokens: not whole chunks
    assert f(d, ws=None) == -5
    assert f(d, nbytes=1024) == -5
    assert f(d, ws=o) == -8  # workspace overlapping the output

    # PGDN: aux0 / aux_final [B, H, dk] fp32 join the alias checks
    def fa(aux0, aux_final, S0=None, S_final=None):
        nbytes = L.dn_chunk_fwd_long_workspace(ctypes.byref(dp), 4)
        gp = _gates(alphaP=FAKE + (6 << 30), betaP=FAKE + (7 << 30), mu_log=FAKE + (8 << 30))
        return L.dn_chunk_fwd_long(ctypes.byref(dp), 4, q, k, v, ctypes.byref(gp), S0, aux0, o,
                                   S_final, aux_final, ws, nbytes, None)
    aux = FAKE + (9 << 30)
    assert fa(aux, aux + 256) == -8      # aux_final overlapping aux0 other than exactly
    assert fa(aux, o) == -8              # aux_final overlapping the output
    assert fa(aux, ws + 64) == -8        # aux_final inside the workspace
    assert fa(ws + 64, None) == -8       # aux0 inside the workspace
    assert fa(aux, FAKE + (10 << 30), S_final=FAKE + (10 << 30) + 512) == -8  # aux_final in S_final


def test_noalloc_rejects_workspace_beyond_scratch():
    """dn_chunk_fwd_noalloc: a shape whose workspace exceeds the library's
    scratch array (48 MiB) returns DN_ERR_WORKSPACE before any HIP call; an
    invalid descriptor is reported as by dn_chunk_fwd."""
    L = dn.lib()
    d = _desc(B=1, H=1, T=1 << 22, gain="pgdn")
    assert L.dn_workspace_bytes(ctypes.byref(d)) > (48 << 20)
    gp = _gates(alphaP=FAKE + (6 << 30), betaP=FAKE + (7 << 30), mu_log=FAKE + (8 << 30))
    call = lambda desc: L.dn_chunk_fwd_noalloc(ctypes.byref(desc), FAKE + (2 << 30), FAKE + (3 << 30),
                                               FAKE + (4 << 30), ctypes.byref(gp), None, None,
                                               FAKE + (5 << 30), None, None, None)
    assert call(d) == -5
    assert call(_desc(dk=100)) == -2


def test_chunk_bwd_rejects_bad_arguments():
    """dn_chunk_bwd: unsupported combinations, missing pointers and
    gradients, the workspace, and overlaps are refused before any launch."""
    L = dn.lib()
    q, k, v, dO = FAKE + (2 << 30), FAKE + (3 << 30), FAKE + (4 << 30), FAKE + (5 << 30)
    outs = [FAKE + ((10 + i) << 30) for i in range(13)]
    ws = FAKE + (30 << 30)

    def call(desc, gates=None, grads=None, ws_=ws, nbytes=None):
        gates = gates or _gates()
        grads = grads or dn.DnGrads(*outs)
        if nbytes is None:
            nbytes = L.dn_chunk_bwd_workspace(ctypes.byref(desc))
        return L.dn_chunk_bwd(ctypes.byref(desc), q, k, v, ctypes.byref(gates), None, None, dO, None, None,
                              ctypes.byref(grads), ws_, nbytes, None)
    d = _desc(B=2, H=3, T=100)
    assert call(_desc(io=0, dk=128)) == -6
    assert L.dn_chunk_bwd_workspace(ctypes.byref(_desc(io=0, dk=128))) == 0
    assert call(d, grads=dn.DnGrads(None, *outs[1:])) == -1  # dq missing
    assert call(_desc(gain="pgdn")) == -1  # PGDN gates missing
    gk = _gates(omega=FAKE + (6 << 30), r=FAKE + (7 << 30))
    assert call(_desc(gain="kdn", decay="channel"), gates=gk,
                grads=dn.DnGrads(*outs[:11], None, outs[12])) == -1  # KDN domega missing
    assert call(_desc(gain="kdn_iso"), gates=gk, grads=dn.DnGrads(*outs[:12], None)) == -1  # dr missing
    assert call(d, ws_=None) == -5
    assert call(d, nbytes=1024) == -5
    assert call(d, grads=dn.DnGrads(q, *outs[1:])) == -8  # dq on top of q
    assert call(d, ws_=outs[0]) == -8  # workspace on top of dq
    # the workspace: w, S_ck, E, dw, dG (each on a 256-byte boundary); with
    # bf16 io and scalar decay but for the KDN gains (the split path) also
    # dS_out and Z of every chunk
    r256 = lambda x: (x + 255) // 256 * 256
    bht, nch = 2 * 3 * 100, 2
    size = r256(r256(r256(r256(bht * 128 * 4) + 6 * nch * 128 * 128 * 4) + bht * 128 * 4) + bht * 128 * 4) + bht * 4
    dsck, zck = 6 * nch * 128 * 128 * 4, 6 * nch * 64 * 128 * 4
    split = r256(r256(r256(size) + dsck) + zck)
    assert L.dn_chunk_bwd_workspace(ctypes.byref(d)) == split
    dp = _desc(B=2, H=3, T=100, gain="pgdn")
    assert L.dn_chunk_bwd_workspace(ctypes.byref(dp)) == split + 6 * nch * 128 * 4
    # channel decay: dG per (token, channel); KDN / KDN_ISO: the statistic per chunk
    sizec = r256(r256(r256(r256(bht * 128 * 4) + 6 * nch * 128 * 128 * 4) + bht * 128 * 4) + bht * 128 * 4) + bht * 128 * 4
    dc = _desc(B=2, H=3, T=100, decay="channel")
    assert L.dn_chunk_bwd_workspace(ctypes.byref(dc)) == sizec
    dk_ = _desc(B=2, H=3, T=100, decay="channel", gain="kdn")
    assert L.dn_chunk_bwd_workspace(ctypes.byref(dk_)) == r256(sizec) + 6 * nch * 128 * 4
    di = _desc(B=2, H=3, T=100, gain="kdn_iso")
    assert L.dn_chunk_bwd_workspace(ctypes.byref(di)) == r256(r256(size) + 6 * nch * 4)


def test_bench_refuses_more_than_one_gpu():
    """bench.py runs on one GPU; --gpus N > 1 exits with a message before any GPU work."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_narrow_heads_workspace_and_limits():
    """Head widths no kernel is built for (multiples of 8 up to 128) run on
    padded copies in the workspace: dn_workspace_bytes sizes them, the
    unpaddable combination (isotropic KDN with channel decay) and fp32 keys
    wider than 64 are refused, the backward and the segmented call refuse
    them, and dn_gain_prep takes C = 32."""
    L = dn.lib()
    r256 = lambda x: (x + 255) // 256 * 256
    d = _desc(B=2, H=3, T=100, dk=120, dv=120)
    bht, bh = 2 * 3 * 100, 6
    # q, k, v, o padded (bf16), S0 and S_final padded (fp32); KLA has no other tensor
    want = 4 * r256(bht * 128 * 2) + 2 * r256(bh * 128 * 128 * 4)
    assert L.dn_workspace_bytes(ctypes.byref(d)) == want
    assert L.dn_workspace_bytes(ctypes.byref(_desc(dk=120, dv=120, gain="kdn_iso", decay="channel"))) == 0
    gk = _gates(omega=FAKE + (6 << 30), r=FAKE + (7 << 30))
    assert _chunk(_desc(dk=120, dv=120, gain="kdn_iso", decay="channel"), gates=gk) == -6
    # fp32 io wider than 64 key channels: the tokenwise kernel, no workspace
    # beyond the padded copies (nothing is launched here)
    assert L.dn_workspace_bytes(ctypes.byref(_desc(io=0, dk=128, dv=64))) == 0
    assert L.dn_workspace_bytes(ctypes.byref(_desc(io=0, dk=128, dv=64, decay="channel"))) == 0
    # (padded q, k; v, o; S0, S_final)
    assert L.dn_workspace_bytes(ctypes.byref(_desc(io=0, dk=120, dv=64))) == \
        2 * r256(bht * 128 * 4) + 2 * r256(bht * 64 * 4) + 2 * r256(bh * 128 * 64 * 4)
    assert L.dn_chunk_bwd_workspace(ctypes.byref(d)) == 0
    assert L.dn_chunk_fwd_long_workspace(ctypes.byref(_desc(B=1, H=1, T=4096, dk=120, dv=120)), 4) == 0
    # workspace missing or short for the padded copies
    assert _chunk(d) == -5
    assert _chunk(d, ws=FAKE + (30 << 30), nbytes=want - 256) == -5
    # C = 32: the gain scans only
    d32 = _desc(B=2, H=3, T=128, C=32, gain="pgdn")
    assert L.dn_workspace_bytes(ctypes.byref(d32)) > 0
    gp = _gates(alphaP=FAKE + (6 << 30), betaP=FAKE + (7 << 30), mu_log=FAKE + (8 << 30))
    assert _chunk(d32, gates=gp) == -2
    assert _desc(C=16).C == 16 and L.dn_workspace_bytes(ctypes.byref(_desc(C=16))) == 0
