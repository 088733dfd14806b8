/*
 * dn.h — C ABI of the MI355X (gfx950) forward engine for the gated
 * delta-rule recurrence (library libdn.so).
 *
 * The recurrence, per batch row b and head h, token t = 0 .. T-1
 * (Kalman Delta Networks reading notes §1.1, unified family; Kaczmarz Linear
 * Attention reading notes §2.1 and Algorithm 1; Preconditioned DeltaNet
 * reading notes §2.4-2.5, Eq. 9, transposed to this orientation):
 *
 *     S_dec = D_t S_{t-1}                 D_t = alpha_t I  or  diag(alpha_t)
 *     e_t   = v_t - S_dec^T k_t           residual from the decayed state
 *     S_t   = S_dec + w_t e_t^T           rank-1 write with write vector w_t
 *     o_t   = S_t^T q_t                   readout after the write
 *
 * S is d_k x d_v (key channels are rows).  The write vector w_t (the write key
 * including its gain) depends on the gain:
 *
 *   DN_GAIN_KLA       w = eta / (||k||^2 + eps) * k
 *                     (Kaczmarz Linear Attention §2.1, boxed formula)
 *   DN_GAIN_GDN       w = eta * k            (same page §1.1)
 *   DN_GAIN_PGDN      A_t = alphaP A_{t-1} + betaP (k*k);  r = log A_t - mu_h;
 *                     s = r / (1 + |r|);  B = exp(-log(x) s);  w = eta B * k
 *                     (Preconditioned DeltaNet §2.4, Eq. 9)
 *   DN_GAIN_KDN       p_hat = alpha^2 p_{t-1} + omega;  z = sum p_hat k^2;
 *                     w = p_hat * k / (r + z);  u = (mu_info / r) k^2;
 *                     p_t = p_hat / (1 + u p_hat)
 *                     (Kalman Delta Networks §2.4 Eqs. 23-30 and §2.5)
 *   DN_GAIN_EXPLICIT  w_t read from gates->w (e.g. the exact ATK write key of
 *                     Preconditioned DeltaNet §2.2)
 *   DN_GAIN_KDN_ISO   one variance b per head: a = mean_i alpha_i^2 (alpha^2
 *                     for scalar decay);  b_hat = a b_{t-1} + omega;
 *                     n = ||k||^2;  w = b_hat / (r + b_hat n) * k;
 *                     b_t = b_hat / (1 + u b_hat),  u = mu_info n / (dk r)
 *                     (Kalman Delta Networks §2.7, Eq. 40; omega and r are
 *                     scalars per token)
 *
 * q is used as given: normalising it (Kaczmarz Linear Attention §2.1 reads
 * S^T q / ||q||) is the caller's job.
 *
 * LAYOUT.  All tensors are dense and row-major with the last index
 * contiguous:
 *   q, k, o       [B, H, T, dk] / [B, H, T, dv]   io dtype
 *   v             [B, H, T, dv]                   io dtype
 *   alpha         scalar decay: fp32 [B, H, T];  channel decay: io [B, H, T, dk]
 *   eta           fp32 [B, H, T]   (KLA eta, GDN/PGDN beta; unused by KDN)
 *   alphaP, betaP fp32 [B, H, T]   (PGDN statistic gates)
 *   mu_log        fp32 [H]         (PGDN per-head log-centre)
 *   omega         io   [B, H, T, dk] (KDN process noise);
 *                 KDN_ISO: fp32 [B, H, T]
 *   r             fp32 [B, H, T]   (KDN / KDN_ISO observation noise, > 0)
 *   w             io   [B, H, T, dk] (EXPLICIT write vectors)
 *   S0, S_final   fp32 [B, H, dk, dv]
 *   aux0, aux_final fp32 [B, H, dk] (PGDN statistic A; KDN variance p);
 *                 KDN_ISO: fp32 [B, H] (the variance b of each head)
 *
 * OWNERSHIP.  Every pointer except the descriptor and the gate table (host
 * structs, read before the call returns) is a device pointer owned by the
 * caller, 16-byte aligned (as hipMalloc and tensor allocators return them:
 * the kernels move rows in 16-byte vectors).  The library allocates no device memory, never synchronises, and
 * enqueues all work on `stream` (a hipStream_t; NULL = the null stream) -
 * except that dn_chunk_bwd may run one pass on a second stream of its own,
 * ordered after the work already on `stream` and before the rest of the
 * call's work there by two events (see dn_chunk_bwd).
 *
 * ERRORS.  Arguments are validated on the host before anything is launched;
 * on a negative status nothing has been enqueued.  DN_ERR_HIP reports a
 * failed launch.  NaN/Inf in the data are not checked and propagate.
 * Preconditions on values (not checked): alpha in (0, 1]; PGDN A_0 > 0 and
 * alphaP, betaP >= 0; KDN and KDN_ISO r > 0, omega >= 0, p_0 and b_0 > 0.
 * RANGE OF CHANNEL DECAY (checked on the device).  The chunked forward refers
 * the decay factors of each key channel to the middle of its chunk of 64
 * tokens (token 31), which stays within fp32 range while each half chunk's
 * decay of a channel is at least 2^-96 (a geometric-mean alpha of at least
 * 1/8 over its 32 tokens).  A head whose decay goes beyond in some chunk is
 * flagged on the device and recomputed by a tokenwise pass over its whole
 * sequence, which has no such bound: dn_chunk_fwd and dn_chunk_fwd_long
 * return the token recurrence's results for any alpha in (0, 1], at the cost
 * of that head's sequential pass (about a microsecond per token) when it
 * happens.  dn_chunk_bwd keeps the bound (the gradients of such a head are
 * NaN).  dn_decode_step has no bound; scalar decay has none in any call.
 *
 * Thread safety: all entry points are reentrant; there is no mutable global
 * state.
 */
#ifndef DN_H
#define DN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DN_VERSION 1

typedef enum dn_status {
  DN_OK = 0,
  DN_ERR_NULL = -1,        /* a required pointer is NULL                      */
  DN_ERR_SHAPE = -2,       /* B, H, T, dk, dv or C outside the supported set  */
  DN_ERR_DTYPE = -3,       /* unknown io dtype                                 */
  DN_ERR_GAIN = -4,        /* unknown gain / decay, or invalid gain parameter  */
  DN_ERR_WORKSPACE = -5,   /* workspace missing or smaller than required       */
  DN_ERR_UNSUPPORTED = -6, /* valid but not built (e.g. the backward in fp32 io with dk = 128) */
  DN_ERR_HIP = -7,         /* a kernel launch failed                           */
  DN_ERR_ALIAS = -8        /* forbidden overlap between buffers                */
} dn_status;

typedef enum dn_dtype { DN_F32 = 0, DN_BF16 = 1 } dn_dtype;

typedef enum dn_gain {
  DN_GAIN_KLA = 0,
  DN_GAIN_GDN = 1,
  DN_GAIN_PGDN = 2,
  DN_GAIN_KDN = 3,
  DN_GAIN_EXPLICIT = 4,
  DN_GAIN_KDN_ISO = 5
} dn_gain;

typedef enum dn_decay { DN_DECAY_SCALAR = 0, DN_DECAY_CHANNEL = 1 } dn_decay;

/* Problem descriptor (host struct).
 *   B, H >= 1, B H <= 65535; T >= 0 (T = 0: S_final = S0, aux_final = aux0,
 *   o untouched);
 *   dk a multiple of 8 up to 128; dv a multiple of 8 up to 128, or any
 *   multiple of 64 up to 2048 (d_v = v_expand d_k).  The kernels are built
 *   for dk in {64, 128} and dv a multiple of 64; other widths (the 120-wide
 *   heads of Preconditioned DeltaNet §3.1, for example) run on them: the
 *   chunked calls on zero-padded copies in the workspace (key channels with
 *   k = q = w = 0 and decay 1, value columns with v = 0, the outputs cropped
 *   back; isotropic KDN's mu rescaled so that mu ||k||^2 / (d_k r) keeps its
 *   value), the decode step masked in place.  Isotropic KDN with channel
 *   decay at such a d_k (the mean of alpha^2 over the channels has no padded
 *   form), the backward and the segmented call at such widths return
 *   DN_ERR_UNSUPPORTED.  fp32 io with dk > 64: dn_chunk_fwd evaluates the
 *   token recurrence per head (exact; a sequential pass over T, about a
 *   microsecond per token) and needs no workspace for it; dn_gain_prep and
 *   dn_decode_step run their usual kernels; dn_chunk_bwd returns
 *   DN_ERR_UNSUPPORTED;
 *   C = 64, the chunk length of the chunked forward and backward; dn_gain_prep
 *   also takes C = 32 (its per-chunk outputs and parallel scan pieces: the
 *   memory chunk of 32 or 64 tokens of Kalman Delta Networks Appendix D);
 *   io: dn_dtype of q, k, v, o and of per-channel gates;
 *   gain: dn_gain; decay: dn_decay (KDN requires DN_DECAY_CHANNEL or SCALAR);
 *   eps >= 0 (KLA), x >= 1 (PGDN bound: B in [1/x, x];
 *   x = 1 is the GDN write), mu_info > 0 (KDN,
 *   KDN_ISO). */
typedef struct dn_desc {
  int32_t B, H, T, dk, dv, C;
  int32_t io;
  int32_t gain;
  int32_t decay;
  float eps;
  float x;
  float mu_info;
} dn_desc;

/* Gate table (host struct of device pointers); unused entries may be NULL. */
typedef struct dn_gates {
  const void* alpha;   /* required                                   */
  const float* eta;    /* KLA, GDN, PGDN                             */
  const float* alphaP; /* PGDN                                       */
  const float* betaP;  /* PGDN                                       */
  const float* mu_log; /* PGDN                                       */
  const void* omega;   /* KDN (io, per channel), KDN_ISO (fp32)      */
  const float* r;      /* KDN, KDN_ISO                               */
  const void* w;       /* EXPLICIT                                   */
} dn_gates;

/* Device workspace, in bytes, that dn_chunk_fwd and dn_gain_prep need for
 * this descriptor: the larger of the two needs, 0 when neither call needs
 * any, and 0 for an invalid descriptor.  It depends on the descriptor only
 * (not on pointers or data), so one query serves every call of that shape.
 *   dn_chunk_fwd: shapes with too few (batch, head, 64-column value slice)
 *     workgroups to fill the device's compute units and a long sequence
 *     (bf16 io, T a multiple of C) run by segments of each head, as
 *     dn_chunk_fwd_long does, on dn_chunk_fwd_long's workspace layout for
 *     the chosen segment count (e.g. B1 H8 T131072 d128: 16 segments, about
 *     26 MB); other shapes with per-channel decay need an int per head (the
 *     flags of RANGE OF CHANNEL DECAY); every other shape needs none.
 *   dn_gain_prep: the gains with a statistic (PGDN, KDN, KDN_ISO), bf16 io
 *     and T a multiple of C (at least two chunks) scan every chunk in
 *     parallel; the workspace holds the chunks' piece summaries, the
 *     statistic entering every chunk and PGDN's centre repeated per chunk.
 *   Head widths no kernel is built for: the padded call's own workspace,
 *   then the padded copies of the inputs and outputs (each on a 256-byte
 *   boundary).
 *   C = 32 is valid for dn_gain_prep only: the size is then its need. */
size_t dn_workspace_bytes(const dn_desc* desc);

/* Chunked forward over a whole sequence batch (Kaczmarz Linear Attention
 * §2.5 Eqs. 7-9 and Preconditioned DeltaNet §2.6 Eq. 6 give the chunk form;
 * results equal the token recurrence above up to rounding).
 *   S0        initial state, NULL = zeros.
 *   aux0      PGDN A_0 / KDN p_0 / KDN_ISO b_0, NULL = ones; ignored by
 *             other gains.
 *   o         output [B, H, T, dv], io dtype (round to nearest even).
 *   S_final   final state, nullable.  May alias S0 exactly (in-place resume).
 *   aux_final final A_T / p_T / b_T, nullable.  Must not overlap aux0 (every value
 *             slice of a head reads aux0 while one of them writes aux_final).
 *   ws        device workspace of ws_bytes >= dn_workspace_bytes(desc) bytes,
 *             owned by the caller; may be NULL when that size is 0.  It holds
 *             nothing between calls and may not overlap any other buffer.
 *             DN_ERR_WORKSPACE when it is missing or too small.
 * No other buffers may overlap (DN_ERR_ALIAS is returned for the overlaps
 * the host can see from the pointer ranges).  With T = 0 the tensors q, k, v,
 * o and the gate table may be NULL.  One launch on `stream` (a
 * segmented schedule: three, five with a statistic; per-channel decay adds
 * the tokenwise pass, which returns at once for heads in range); nothing is
 * allocated. */
int dn_chunk_fwd(const dn_desc* desc, const void* q, const void* k, const void* v,
                 const dn_gates* gates, const float* S0, const float* aux0, void* o,
                 float* S_final, float* aux_final, void* ws, size_t ws_bytes, void* stream);

/* dn_chunk_fwd for callers that cannot allocate device memory (code under
 * stream capture into a graph, tight serving loops, harnesses that forbid
 * allocation): the same computation, with the workspace taken from a
 * device array inside the library instead of an argument.
 *   The array holds DN_NOALLOC_SCRATCH_BYTES (48 MiB) on every device the
 *   library runs on, from the first call on that device until the process
 *   ends.  A descriptor whose dn_workspace_bytes exceeds it returns
 *   DN_ERR_WORKSPACE before anything is launched.  The call itself allocates
 *   nothing (no hipMalloc, no allocating library routine).
 *   Every call on one device shares that device's array: calls that overlap
 *   in time on one device (other streams, other host threads) race on it and
 *   must be serialised by the caller.  Nothing is kept between calls.
 * Arguments, errors and results as for dn_chunk_fwd. */
#define DN_NOALLOC_SCRATCH_BYTES ((size_t)48 << 20)
int dn_chunk_fwd_noalloc(const dn_desc* desc, const void* q, const void* k, const void* v,
                         const dn_gates* gates, const float* S0, const float* aux0, void* o,
                         float* S_final, float* aux_final, void* stream);

/* Chunked forward of long sequences by segments, for shapes with few heads
 * (e.g. batch-1 prefill): each head's T tokens are cut into nseg segments
 * of T / nseg tokens, which run in parallel.  Over a segment the recurrence
 * is affine in its entering state, S_out = A S_in + B (the affine memory
 * scan of Kalman Delta Networks §2.6, Eq. 39, taken per segment), so the
 * call (1) forms every segment's end state B from S_in = 0 and, in the same
 * launch, its transfer matrix A from S_in = I with v = 0, (2) chains
 * S_in(s + 1) = A_s S_in(s) + B_s from S0, and (3) reruns every segment from
 * its S_in, writing o.  For PGDN and KDN the gain statistic (A_t, p_t, b_t)
 * does not depend on S: a first step (0) composes its per-token maps (affine
 * for PGDN, Moebius for KDN, the associative gain scan of §2.6) over pieces
 * of each segment in parallel and chains them from aux0, giving the
 * statistic entering every segment and aux_final.  Results equal
 * dn_chunk_fwd's up to rounding.
 *   Built for io = DN_BF16 with every gain and decay (DN_ERR_UNSUPPORTED for
 *   fp32).  nseg >= 1 must divide T into segments of a multiple of C = 64
 *   tokens, and B H nseg <= 65535 (DN_ERR_SHAPE).  Any other T: run the
 *   longest such prefix here and the remaining tokens with dn_chunk_fwd,
 *   its S0 and aux0 being this call's S_final and aux_final.
 *   q, k, v, gates, S0 (nullable: zeros), aux0 (nullable: ones), o, S_final
 *   (nullable) and aux_final (nullable) are laid out as for dn_chunk_fwd;
 *   aux0 and aux_final are ignored for the gains without a statistic.
 *   S_final may be S0 exactly, and aux_final aux0 exactly (in-place resume).
 *   q, k, v and o are required also when T = 0.
 *   workspace: device memory of at least dn_chunk_fwd_long_workspace(desc,
 *   nseg) bytes, owned by the caller: fp32 A [B, H nseg, dk, dk], then B and
 *   S_in [B, H nseg, dk, dv] each, for PGDN and KDN the segments' entering
 *   statistics and the piece summaries, and with per-channel decay an int
 *   per segment (RANGE OF CHANNEL DECAY).  It may not overlap any other
 *   buffer (DN_ERR_WORKSPACE when too small, DN_ERR_ALIAS on overlap).
 *   dn_chunk_fwd_long_workspace returns that size in bytes, or 0 for an
 *   invalid descriptor, nseg < 1, or segments that are not whole chunks.
 *   Three launches on `stream` (five with a statistic; one more with
 *   per-channel decay); nothing is allocated.  Choosing nseg: the last launch runs B H nseg d_v / 64
 *   workgroups of one chunk step at a time each; filling the device's
 *   compute units once (256 on MI355X) is best, e.g. nseg = 16 for B1 H8
 *   d128 (measured at T = 32768 and 131072: 32 and 64 segments are slower,
 *   the combine's serial chain growing with nseg). */
size_t dn_chunk_fwd_long_workspace(const dn_desc* desc, int nseg);
int dn_chunk_fwd_long(const dn_desc* desc, int nseg, const void* q, const void* k, const void* v,
                      const dn_gates* gates, const float* S0, const float* aux0, void* o,
                      float* S_final, float* aux_final, void* workspace, size_t workspace_bytes,
                      void* stream);

/* One token for N = desc->B independent sequences (desc->T must be 1), the
 * tokenwise step of Kaczmarz Linear Attention Algorithm 1 (and its PGDN/KDN
 * analogues).  S [N, H, dk, dv] and aux [N, H, dk] (PGDN, KDN; [N, H] for
 * KDN_ISO; NULL otherwise) are updated in place; o [N, H, dv] receives S_t^T q_t.
 * q, k, v, gates are laid out as for dn_chunk_fwd with T = 1. */
int dn_decode_step(const dn_desc* desc, const void* q, const void* k, const void* v,
                   const dn_gates* gates, float* S, float* aux, void* o, void* stream);

/* The write-gain scans alone, for inspection and testing: the write vector
 * w_t of every token as the chunked forward applies it (KLA / GDN:
 * Kaczmarz Linear Attention §2.1 and §1.1; PGDN: Preconditioned DeltaNet
 * §2.4, Eq. 9; KDN: Kalman Delta Networks §2.4, Eqs. 23-30, with the
 * information scaling of §2.5; KDN_ISO: §2.7, Eq. 40; EXPLICIT: w copied),
 * the in-chunk cumulative log-decay and the statistic entering each chunk.
 * Whole chunks (T a multiple of C, at least two) are scanned in parallel:
 * for the gains with a statistic (bf16 io) the statistic entering every
 * chunk comes first from chunk summaries of the per-token maps and a carry
 * across chunks (the gain scan of Kalman Delta Networks §6 and Appendix D:
 * summaries, carry, replay; the chunked statistic recursion of
 * Preconditioned DeltaNet §2.6), then every chunk replays its tokens.
 *   w_out     fp32 [B, H, T, dk]: write vectors w_t (required).
 *   g_out     fp32 cumulative log-decay within each chunk of C tokens
 *             (G_t = sum of log alpha from the chunk start through t):
 *             [B, H, T] (scalar decay) or [B, H, T, dk] (channel); nullable.
 *   aux_chunk fp32 [B, H, ceil(T/C), dk]: PGDN A / KDN p entering each
 *             chunk ([B, H, ceil(T/C)]: KDN_ISO b); nullable (ignored by
 *             gains without state).
 *   aux_final fp32 [B, H, dk]: A_T / p_T ([B, H]: KDN_ISO b_T); nullable.
 *   aux0      as for dn_chunk_fwd.
 *   ws        device workspace of ws_bytes >= dn_workspace_bytes(desc)
 *             bytes (may be NULL when that is 0); DN_ERR_WORKSPACE when
 *             missing or too small.
 * Outputs may not overlap inputs, each other or the workspace
 * (DN_ERR_ALIAS).  One to three launches on `stream`. */
int dn_gain_prep(const dn_desc* desc, const void* k, const dn_gates* gates, const float* aux0,
                 float* w_out, float* g_out, float* aux_chunk, float* aux_final, void* ws,
                 size_t ws_bytes, void* stream);

/* Gradients of the chunked forward (the backward pass of training: the
 * recurrence differentiated, Preconditioned DeltaNet §2.5), for the loss
 *     L = sum_t <dO_t, o_t> + <dS_T, S_T> + <daux_T, aux_T>
 * with respect to every input of dn_chunk_fwd.  Every gradient is fp32, laid
 * out like its input; dq, dk, dv, dalpha required, the gates' by gain. */
typedef struct dn_grads {
  float* dq;      /* [B, H, T, dk]                                  */
  float* dk;      /* [B, H, T, dk] (through the residual and the gain) */
  float* dv;      /* [B, H, T, dv]                                  */
  float* dalpha;  /* [B, H, T] (scalar decay), [B, H, T, dk] (channel) */
  float* deta;    /* KLA, GDN, PGDN: [B, H, T]                      */
  float* dalphaP; /* PGDN: [B, H, T]                                */
  float* dbetaP;  /* PGDN: [B, H, T]                                */
  float* dmu_log; /* PGDN: [H], summed over the batch rows          */
  float* dw;      /* EXPLICIT: [B, H, T, dk]                        */
  float* dS0;     /* [B, H, dk, dv], nullable                       */
  float* daux0;   /* PGDN dL/dA_0, KDN dL/dp_0 [B, H, dk]; KDN_ISO dL/db_0
                     [B, H]; nullable                               */
  float* domega;  /* KDN: [B, H, T, dk]; KDN_ISO: [B, H, T]         */
  float* dr;      /* KDN, KDN_ISO: [B, H, T]                        */
} dn_grads;

/* Chunked backward.  Per chunk of C tokens it evaluates the derivative of
 * the chunk form (Kaczmarz Linear Attention §2.5 Eqs. 7-9; Preconditioned
 * DeltaNet §2.6 Eq. 6): with (I + L) E = V - diag(g) K S_in, O = diag(g) Q
 * S_in + M E and S_out = g_n S_in + W~^T E, the chunk takes dO and dS_out
 * and gives dE = M^T dO + W~ dS_out, dR from (I + L)^T dR = dE, dV = dR,
 * dS_in = g_n dS_out + (gQ)^T dO - (gK)^T dR, dL = -dR E^T, dM = dO E^T, and
 * from them the gradients of k, q, w and the decay (per key channel for
 * channel decay, the decay then applied inside the products); the chunks are
 * walked from the last, after a forward sweep that keeps the state entering
 * each chunk and the residuals E.  With bf16 io and scalar decay, for KLA,
 * GDN, PGDN and explicit w with dv a multiple of 64, the chunked forward's
 * kernel runs that sweep without output; what of dR does not depend on dS
 * (dR = P + Z dS_out, Z = (I + L)^-T W~, P = (I + L)^-T M^T dO) is solved
 * for every chunk at once, so that the reverse walk carries only dS; and
 * when the forward sweep fills at most half of the compute units (B H dv/64
 * <= 128) it runs on a second stream of the library (one per device,
 * created at its first use), forked from `stream` by an event after the work
 * already queued there and joined back by another before the gradients that
 * read its checkpoints.  With few heads and at least 16 chunks (when a
 * chunk-step cost model finds it cheaper) both serial passes run by segments: the forward sweep as
 * dn_chunk_fwd_long's schedule, and the reverse walk as every segment's
 * affine map (dS_in = A dS_out + B) formed in parallel, the maps chained from
 * dS_T, and every segment walked again from its own dS_out.  The write gain is then differentiated token by token
 * backwards (KLA, GDN: Kaczmarz Linear Attention §2.1; PGDN: Preconditioned
 * DeltaNet §2.4, Eq. 9, through the statistic A_t, its centre mu and its
 * gates; KDN: Kalman Delta Networks §2.4, Eqs. 23-30 and §2.5, through the
 * variance p_t, omega and r; KDN_ISO: §2.7, Eq. 40 - the gain scan of
 * Appendix D run backwards).
 *   Every gain and both decays; io bf16 (dk 64 or 128) or fp32 (dk 64);
 *   other shapes return DN_ERR_UNSUPPORTED.  Results equal the gradients of
 *   the token recurrence up to rounding (fp32 accumulation; k, q and w enter
 *   the products in the io dtype, with channel decay scaled by their decay
 *   relative to the chunk's token 31 first; with bf16 io the fp32 operands
 *   enter as pairs of bf16, within 2^-16, and where the chunked forward's
 *   kernel writes the checkpoints they carry its rounding, as its o and
 *   S_final do).  Channel decay has the range of
 *   the chunked forward (RANGE OF CHANNEL DECAY): beyond it the gradients
 *   of the head are NaN.
 *   q, k, v, gates, S0 (nullable: zeros), aux0 (nullable: ones): as for
 *   dn_chunk_fwd.  dO [B, H, T, dv] io dtype; dS_T [B, H, dk, dv] and
 *   daux_T (PGDN / KDN [B, H, dk], KDN_ISO [B, H]) fp32, nullable (zero).
 *   ws: device workspace of at least dn_chunk_bwd_workspace(desc) bytes
 *   (the write vectors [B, H, T, dk], fp32 or, with bf16 io and scalar
 *   decay, bf16; fp32: the state entering every chunk
 *   [B, H, ceil(T/C), dk, dv], the residuals [B, H, T, dv], the write vectors'
 *   gradient [B, H, T, dk], the decay's per token ([B, H, T], channel decay
 *   [B, H, T, dk]), on the bf16 scalar-decay path above dS_out of every chunk
 *   [B, H, ceil(T/C), dv, dk] and Z of every chunk [B, H, ceil(T/C), C, dk]
 *   (bf16 pairs, 4 bytes each), with segments their maps and entering dS
 *   and the forward schedule's workspace, and for the gains with a statistic the
 *   statistic entering every chunk; 2.15 GB at B8 H16 T4096 d128 with bf16
 *   io and scalar decay).  No gradient
 *   buffer may overlap an input, another gradient or the workspace
 *   (DN_ERR_ALIAS).  dmu_log is summed over the batch rows with atomic
 *   additions: its last bits may vary from run to run, as may those of dq,
 *   dk, dw and dalpha (summed over value-column slices, or on the bf16
 *   scalar-decay path through shared-memory atomic additions; there, for
 *   KLA and GDN, the kernel that forms dk also runs the gain's and the
 *   decay's backward, and the write vectors' and decay's gradients in the
 *   workspace are left unwritten). */
size_t dn_chunk_bwd_workspace(const dn_desc* desc);
int dn_chunk_bwd(const dn_desc* desc, const void* q, const void* k, const void* v,
                 const dn_gates* gates, const float* S0, const float* aux0, const void* dO,
                 const float* dS_T, const float* daux_T, const dn_grads* grads, void* ws,
                 size_t ws_bytes, void* stream);

/* Static text for a status code. */
const char* dn_status_string(int status);

/* DN_VERSION of the library. */
int dn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DN_H */
