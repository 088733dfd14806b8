"""MI355X forward engine for the gated delta-rule recurrence.

    S_t = D_t S_{t-1} + w_t (v_t - (D_t S_{t-1})^T k_t)^T,   o_t = S_t^T q_t

with the write vector w_t given by one of the gains KLA, GDN, PGDN,
diagonal KDN or an explicit per-token vector.  The compute runs in
hand-written HIP kernels for gfx950 behind the C ABI of include/dn.h
(libdn.so); `recurrent_sequence_mixer_amd.dn` is the thin Python binding.
"""

__all__ = ["dn", "workloads"]
