// Host side of libdn.so: argument validation, aliasing checks and kernel
// dispatch for the C ABI declared in include/dn.h.  Validation happens before
// anything is enqueued; every entry point returns a dn_status.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "dn.h"
#include "launch.hpp"

#define DN_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

// key width: a multiple of 8 up to 128 (the kernels are built for 64 and
// 128; other widths run on them zero-padded, see pad.hip)
bool valid_dim(int d) { return d >= 8 && d <= 128 && d % 8 == 0; }
// value width: a multiple of 8 up to 128, or d_v = v_expand d_k, a multiple of
// 64 up to 2048 (the kernels walk 64- or 128-column value slices)
bool valid_dv(int d) { return d >= 8 && d <= 2048 && d % 8 == 0 && (d <= 128 || d % 64 == 0); }
// the widths the kernels are built for
bool kernel_dims(const dn_desc* d) { return (d->dk == 64 || d->dk == 128) && d->dv % 64 == 0; }
// the kernel widths a head of other widths runs at.  Isotropic KDN divides
// by d_k (u = mu ||k||^2 / (d_k r)): mu is scaled so that the padded call
// computes the same u.
dn_desc padded_desc(const dn_desc* d) {
  dn_desc p = *d;
  p.dk = d->dk <= 64 ? 64 : 128;
  p.dv = (d->dv + 63) / 64 * 64;
  if (d->gain == DN_GAIN_KDN_ISO) p.mu_info = d->mu_info * static_cast<float>(p.dk) / d->dk;
  return p;
}
// Padding keeps every gain except isotropic KDN with channel decay, whose
// mean of alpha^2 over the channels no padded decay value preserves.
bool paddable(const dn_desc* d) {
  return kernel_dims(d) || !(d->gain == DN_GAIN_KDN_ISO && d->decay == DN_DECAY_CHANNEL);
}

size_t io_size(int io) { return io == DN_BF16 ? 2 : 4; }

struct Range {
  const void* p;
  size_t bytes;
};

bool overlap(Range a, Range b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Common descriptor checks.  `chunked` = the call walks chunks of C tokens.
int check_desc(const dn_desc* d, bool chunked) {
  if (!d) return DN_ERR_NULL;
  if (d->B < 1 || d->H < 1 || d->T < 0) return DN_ERR_SHAPE;
  if (!valid_dim(d->dk) || !valid_dv(d->dv)) return DN_ERR_SHAPE;
  if (chunked && d->C != 64) return DN_ERR_SHAPE;
  if (static_cast<long long>(d->B) * d->H > 65535) return DN_ERR_SHAPE;
  if (static_cast<long long>(d->B) * d->H * d->T * (d->dk > d->dv ? d->dk : d->dv) >
      (1LL << 40))
    return DN_ERR_SHAPE;
  if (d->io != DN_F32 && d->io != DN_BF16) return DN_ERR_DTYPE;
  if (d->gain < DN_GAIN_KLA || d->gain > DN_GAIN_KDN_ISO) return DN_ERR_GAIN;
  if (d->decay != DN_DECAY_SCALAR && d->decay != DN_DECAY_CHANNEL) return DN_ERR_GAIN;
  if (d->gain == DN_GAIN_KLA && !(d->eps >= 0.f && std::isfinite(d->eps))) return DN_ERR_GAIN;
  if (d->gain == DN_GAIN_PGDN && !(d->x >= 1.f && std::isfinite(d->x))) return DN_ERR_GAIN;
  if ((d->gain == DN_GAIN_KDN || d->gain == DN_GAIN_KDN_ISO) &&
      !(d->mu_info > 0.f && std::isfinite(d->mu_info)))
    return DN_ERR_GAIN;
  return DN_OK;
}

int check_gates(const dn_desc* d, const dn_gates* g) {
  if (!g || !g->alpha) return DN_ERR_NULL;
  switch (d->gain) {
    case DN_GAIN_KLA:
    case DN_GAIN_GDN:
      if (!g->eta) return DN_ERR_NULL;
      break;
    case DN_GAIN_PGDN:
      if (!g->eta || !g->alphaP || !g->betaP || !g->mu_log) return DN_ERR_NULL;
      break;
    case DN_GAIN_KDN:
    case DN_GAIN_KDN_ISO:
      if (!g->omega || !g->r) return DN_ERR_NULL;
      break;
    default:
      if (!g->w) return DN_ERR_NULL;
  }
  return DN_OK;
}

dn::GateArgs gate_args(const dn_desc* d, const dn_gates* g) {
  dn::GateArgs a;
  a.alpha = g->alpha;
  a.eta = g->eta;
  a.alphaP = g->alphaP;
  a.betaP = g->betaP;
  a.mu_log = g->mu_log;
  a.omega = g->omega;
  a.r = g->r;
  a.w = g->w;
  a.eps = d->eps;
  a.log2x = d->gain == DN_GAIN_PGDN ? std::log2(d->x) : 0.f;
  a.mu_info = d->mu_info;
  return a;
}

// Byte ranges of every input a call reads, for the aliasing checks.
int gate_ranges(const dn_desc* d, const dn_gates* g, Range* out) {
  const size_t bht = static_cast<size_t>(d->B) * d->H * d->T;
  const size_t es = io_size(d->io);
  int n = 0;
  out[n++] = {g->alpha, d->decay == DN_DECAY_CHANNEL ? bht * d->dk * es : bht * 4};
  out[n++] = {g->eta, bht * 4};
  out[n++] = {g->alphaP, bht * 4};
  out[n++] = {g->betaP, bht * 4};
  out[n++] = {g->mu_log, static_cast<size_t>(d->H) * 4};
  out[n++] = {g->omega, d->gain == DN_GAIN_KDN_ISO ? bht * 4 : bht * d->dk * es};
  out[n++] = {g->r, bht * 4};
  out[n++] = {g->w, bht * d->dk * es};
  return n;
}

int hip_status(hipError_t e) { return e == hipSuccess ? DN_OK : DN_ERR_HIP; }

// Gains that carry an auxiliary state between tokens, and its size per head.
bool has_aux_state(const dn_desc* d) {
  return d->gain == DN_GAIN_PGDN || d->gain == DN_GAIN_KDN || d->gain == DN_GAIN_KDN_ISO;
}
size_t aux_per_head(const dn_desc* d) { return d->gain == DN_GAIN_KDN_ISO ? 1 : d->dk; }

}  // namespace

DN_EXPORT int dn_version(void) { return DN_VERSION; }

DN_EXPORT const char* dn_status_string(int s) {
  switch (s) {
    case DN_OK: return "ok";
    case DN_ERR_NULL: return "a required pointer is NULL";
    case DN_ERR_SHAPE: return "unsupported shape (B, H, T, dk, dv or C)";
    case DN_ERR_DTYPE: return "unknown io dtype";
    case DN_ERR_GAIN: return "unknown gain or decay, or invalid gain parameter";
    case DN_ERR_UNSUPPORTED: return "combination not built (fp32 io chunked forward needs dk = 64)";
    case DN_ERR_HIP: return "kernel launch failed";
    case DN_ERR_WORKSPACE: return "workspace missing or smaller than required";
    case DN_ERR_ALIAS: return "forbidden overlap between buffers";
    default: return "unknown status";
  }
}

// Workspace of dn_chunk_fwd_long, fp32: A [B, H nseg, dk, dk], then B and S_in
// [B, H nseg, dk, dv]; for the gains with a statistic (PGDN, KDN) then
// aux_in [B, H nseg, aph], mu_seg [H nseg] and the piece summaries
// [B, H, T / lsub, 3, aph]; with per-channel decay then the out-of-range
// flags [B, H nseg] (int), each of these starting on a 256-byte boundary.
struct LongLayout {
  size_t a, b, s, aux_in, mu_seg, summ, oor, total;
  int lsub;
};

static size_t round256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Per-channel decay: one int per head (of the [B, H nseg] view) that the
// chunked kernels set when the head's decay leaves the range of the chunk form
static size_t oor_bytes(const dn_desc* d, int nseg) {
  return d->decay == DN_DECAY_CHANNEL ? static_cast<size_t>(d->B) * d->H * nseg * sizeof(int) : 0;
}

static LongLayout long_layout(const dn_desc* d, int nseg) {
  LongLayout L{};
  const size_t heads = static_cast<size_t>(d->B) * d->H * nseg;
  const int ts = d->T / nseg;
  L.lsub = ts % 256 == 0 ? 256 : ts % 128 == 0 ? 128 : 64;
  L.a = 0;
  L.b = heads * d->dk * d->dk * sizeof(float);
  L.s = L.b + heads * d->dk * d->dv * sizeof(float);
  L.total = L.s + heads * d->dk * d->dv * sizeof(float);
  if (has_aux_state(d)) {
    const size_t aph = aux_per_head(d);
    L.aux_in = round256(L.total);
    L.mu_seg = round256(L.aux_in + heads * aph * sizeof(float));
    L.summ = round256(L.mu_seg + static_cast<size_t>(d->H) * nseg * sizeof(float));
    L.total = L.summ + static_cast<size_t>(d->B) * d->H * (d->T / L.lsub) * 3 * aph * sizeof(float);
  }
  if (oor_bytes(d, nseg) > 0) {
    L.oor = round256(L.total);
    L.total = L.oor + oor_bytes(d, nseg);
  }
  return L;
}

// The tokenwise pass over the heads whose per-channel decay the chunked
// kernels flagged (oor: nflag ints per head); aux0 is the statistic entering
// the sequence, aux_seg the head stride of its array in units of one head's
// statistic.  A head not flagged costs a read of its flags.
static int run_token_pass(const dn_desc* d, const void* q, const void* k, const void* v,
                          const dn_gates* g, const float* S0, const float* aux0, int aux_seg,
                          void* o, float* S_final, float* aux_final, const int* oor, int nflag,
                          hipStream_t s) {
  const bool has_aux = has_aux_state(d);
  dn::TokenArgs t;
  t.B = d->B;
  t.H = d->H;
  t.T = d->T;
  t.dk = d->dk;
  t.dv = d->dv;
  t.q = q;
  t.k = k;
  t.v = v;
  t.g = gate_args(d, g);
  t.S0 = S0;
  t.aux0 = has_aux ? aux0 : nullptr;
  t.aux_seg = aux_seg;
  t.o = o;
  t.S_final = S_final;
  t.aux_final = has_aux ? aux_final : nullptr;
  t.flags = oor;
  t.nflag = nflag;
  return hip_status(dn::launch_token_fwd(t, d->io == DN_BF16, d->gain, d->decay == DN_DECAY_CHANNEL, s));
}

static bool long_shape_ok(const dn_desc* d, int nseg) {
  return kernel_dims(d) && nseg >= 1 && d->T % nseg == 0 && (d->T / nseg) % d->C == 0;
}

// Aliasing checks of a run that works on copies in the workspace (by
// segments, or padded) against its workspace range.
static int check_long_aliases(const dn_desc* d, const dn_gates* g, const void* q, const void* k,
                              const void* v, const float* S0, const float* aux0, void* o,
                              float* S_final, float* aux_final, const void* ws, size_t ws_used) {
  const bool has_aux = has_aux_state(d);
  const size_t bht = static_cast<size_t>(d->B) * d->H * d->T;
  const size_t sbytes = static_cast<size_t>(d->B) * d->H * d->dk * d->dv * 4;
  const size_t abytes = static_cast<size_t>(d->B) * d->H * aux_per_head(d) * 4;
  const size_t es = io_size(d->io);
  Range in[16];
  int n = gate_ranges(d, g, in);
  in[n++] = {q, bht * d->dk * es};
  in[n++] = {k, bht * d->dk * es};
  in[n++] = {v, bht * d->dv * es};
  in[n++] = {S0, S0 ? sbytes : 0};
  in[n++] = {has_aux ? aux0 : nullptr, abytes};
  const Range ro{o, bht * d->dv * es}, rs{S_final, S_final ? sbytes : 0},
      ra{has_aux ? aux_final : nullptr, abytes}, rw{ws, ws_used};
  for (int i = 0; i < n; ++i) {
    // S_final may be S0 exactly and aux_final aux0 (in-place resume): the
    // combine and chain kernels read and write each element from one thread
    const bool s_in_place = in[i].p == S0 && S_final == S0;
    const bool a_in_place = has_aux && in[i].p == aux0 && aux_final == aux0;
    if (overlap(ro, in[i]) || (!s_in_place && overlap(rs, in[i])) ||
        (!a_in_place && overlap(ra, in[i])) || overlap(rw, in[i]))
      return DN_ERR_ALIAS;
  }
  if (overlap(ro, rs) || overlap(ro, ra) || overlap(rs, ra) || overlap(ro, rw) ||
      overlap(rs, rw) || overlap(ra, rw))
    return DN_ERR_ALIAS;
  return DN_OK;
}

// The segmented forward (already validated): steps (0) to (3) of
// dn_chunk_fwd_long on `ws`, laid out by long_layout(d, nseg).
// S_ck / E_ck (nullable, with o null): step (3) writes the state entering
// every chunk [B, H, T / C, dk, dv] and the residuals [B, H, T, dv] instead
// of o (the checkpoints of dn_chunk_bwd).
static int run_long(const dn_desc* d, int nseg, const void* q, const void* k, const void* v,
                    const dn_gates* g, const float* S0, const float* aux0, void* o, float* S_final,
                    float* aux_final, void* ws, const LongLayout& lay, hipStream_t s,
                    float* S_ck = nullptr, float* E_ck = nullptr) {
  const bool has_aux = has_aux_state(d);
  // the [B, H, T, d] tensors read as [B, H nseg, T / nseg, d]: segment s of
  // head h is head h nseg + s of the view (and likewise the per-token gates)
  const int Hs = d->H * nseg, Ts = d->T / nseg;
  char* wbase = static_cast<char*>(ws);
  float* wA = reinterpret_cast<float*>(wbase + lay.a);
  float* wB = reinterpret_cast<float*>(wbase + lay.b);
  float* wS = reinterpret_cast<float*>(wbase + lay.s);
  dn::ChunkArgs a;
  a.B = d->B;
  a.H = Hs;
  a.T = Ts;
  a.dk = d->dk;
  a.dv = d->dv;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = gate_args(d, g);
  a.S0 = nullptr;
  a.aux0 = nullptr;
  a.o = nullptr;
  a.S_final = wB;
  a.aux_final = nullptr;
  hipError_t e;
  if (has_aux) {
    // (0) the gain statistic entering every segment (and after the last)
    dn::StatArgs sa;
    sa.B = d->B;
    sa.H = d->H;
    sa.T = d->T;
    sa.dk = d->dk;
    sa.nseg = nseg;
    sa.lsub = lay.lsub;
    sa.gain = d->gain;
    sa.channel = d->decay == DN_DECAY_CHANNEL;
    sa.k = k;
    sa.g = a.g;
    sa.aux0 = aux0;
    sa.summ = reinterpret_cast<float*>(wbase + lay.summ);
    sa.aux_in = reinterpret_cast<float*>(wbase + lay.aux_in);
    sa.aux_final = aux_final;
    sa.mu_seg = reinterpret_cast<float*>(wbase + lay.mu_seg);
    if ((e = dn::launch_segment_stats(sa, s)) != hipSuccess) return DN_ERR_HIP;
    a.aux0 = sa.aux_in;
    if (d->gain == DN_GAIN_PGDN) a.g.mu_log = sa.mu_seg;
  }
  const auto launch = [&]() {
    return dn::launch_chunk_fwd(a, 1, d->gain, d->decay == DN_DECAY_CHANNEL, s);
  };
  // per-channel decay: the segments whose decay leaves the chunk form's range
  int* const oor = lay.oor ? reinterpret_cast<int*>(wbase + lay.oor) : nullptr;
  // (1) in one launch: the end states B_s from S_in = 0 (the value slices) and
  // the transfer matrices A_s from S_in = I with v = 0 (d_k more slices)
  a.xcols = d->dk;
  a.S_final_x = wA;
  a.oor = oor;
  if ((e = launch()) != hipSuccess) return DN_ERR_HIP;
  a.xcols = 0;
  a.S_final_x = nullptr;
  a.oor = nullptr;
  // (2) the entering state of every segment, and the final state
  dn::CombineArgs c;
  c.B = d->B;
  c.H = d->H;
  c.nseg = nseg;
  c.dk = d->dk;
  c.dv = d->dv;
  c.A = wA;
  c.Bs = wB;
  c.S0 = S0;
  c.S_in = wS;
  c.S_final = S_final;
  c.oor = oor;
  if ((e = dn::launch_segment_combine(c, s)) != hipSuccess) return DN_ERR_HIP;
  // (3) every segment from its entering state, writing o (or the
  // checkpoints: the view's [B, H nseg, T / (nseg C), ...] layouts are the
  // sequence's [B, H, T / C, ...])
  a.S0 = wS;
  a.S_final = nullptr;
  a.o = o;
  a.S_ck = S_ck;
  a.E_ck = E_ck;
  if ((e = launch()) != hipSuccess) return DN_ERR_HIP;
  // (4) per-channel decay: the flagged heads token by token, from S0 and the
  // statistic entering segment 0
  if (!oor) return DN_OK;
  return run_token_pass(d, q, k, v, g, S0, has_aux ? a.aux0 : nullptr, nseg, o, S_final, aux_final,
                        oor, nseg, s);
}

// Schedule of dn_chunk_fwd: one pass (nseg = 1), or nseg segments per head
// run as by dn_chunk_fwd_long when the shape has too few workgroups to fill
// the device.  A pass of the chunk kernel costs one chunk step per round of
// CU_COUNT workgroups; by segments, the first launch runs the value and the
// d_k / 64 transfer slices of every segment, the last one the value slices,
// each over T / nseg tokens, and the combine chains nseg steps of about 1.2
// chunk steps each.  The cheapest nseg (a power of two that cuts T into whole
// chunks) is taken when it saves at least a fifth of the single pass; the
// extra launches count as a few chunk steps.
constexpr int CU_COUNT = 256;        // compute units of an MI355X
constexpr double SEG_LAUNCHES = 6.;  // the segmented schedule's extra launches, in chunk steps

static double rounds(long long wgs) { return static_cast<double>((wgs + CU_COUNT - 1) / CU_COUNT); }

static int auto_nseg(const dn_desc* d) {
  if (d->io != DN_BF16 || d->T <= 0 || d->T % d->C != 0) return 1;
  const long long wg = static_cast<long long>(d->B) * d->H * (d->dv / 64);
  const long long nch = d->T / d->C;
  const double one = rounds(wg) * static_cast<double>(nch);
  double best = one;
  int pick = 1;
  for (int nseg = 2; nseg <= nch && static_cast<long long>(d->B) * d->H * nseg <= 65535; nseg *= 2) {
    if (nch % nseg != 0) break;
    const double cost = (rounds(wg * nseg * (d->dv + d->dk) / d->dv) + rounds(wg * nseg)) *
                            static_cast<double>(nch / nseg) +
                        1.2 * nseg + SEG_LAUNCHES;
    if (cost < best) {
      best = cost;
      pick = nseg;
    }
  }
  return best <= 0.8 * one ? pick : 1;
}

// Workspace of dn_gain_prep: for the gains with a statistic, bf16 io and T a
// multiple of C (at least two chunks), the chunk-parallel scan's piece summaries
// [B, H, aph, T / C, 3], the statistic entering every chunk [B, H, T / C, aph]
// (used when the caller passes no aux_chunk) and PGDN's centre repeated per
// chunk [H T / C], each on a 256-byte boundary.
struct PrepLayout {
  size_t summ, aux_in, mu_seg, total;
};

// chunks scanned in parallel: whole chunks, at least two; with a statistic
// only for bf16 io (the summary kernels read bf16 k and gates)
static bool prep_by_chunks(const dn_desc* d) {
  return d->T >= 2 * d->C && d->T % d->C == 0 && (!has_aux_state(d) || d->io == DN_BF16);
}
static bool prep_parallel(const dn_desc* d) { return has_aux_state(d) && prep_by_chunks(d); }

static PrepLayout prep_layout(const dn_desc* d) {
  PrepLayout L{};
  if (!prep_parallel(d)) return L;
  const size_t nch = d->T / d->C, aph = aux_per_head(d), bh = static_cast<size_t>(d->B) * d->H;
  L.summ = 0;
  L.aux_in = round256(bh * aph * nch * 3 * sizeof(float));
  L.mu_seg = round256(L.aux_in + bh * nch * aph * sizeof(float));
  L.total = L.mu_seg + static_cast<size_t>(d->H) * nch * sizeof(float);
  return L;
}

// Heads of widths no kernel is built for (padded_desc): the call runs at the
// padded widths on copies in the workspace.  After the padded call's own
// workspace come the padded inputs and outputs, each on a 256-byte boundary
// (a region of 0 bytes where the gain or decay has no such tensor).
struct PadLayout {
  size_t inner;                     // the padded call's workspace, at offset 0
  size_t q, k, v, o, al, om, w;     // io tensors [B, H, T, d]
  size_t s0, sf;                    // S0, S_final [B, H, dk, dv]
  size_t a0, af;                    // per-channel aux0 / aux_final [B, H, dk]
  size_t wo, go, ac;                // dn_gain_prep: w_out, g_out, aux_chunk
  size_t total;
};

static bool per_channel_aux(const dn_desc* d) { return d->gain == DN_GAIN_PGDN || d->gain == DN_GAIN_KDN; }

static size_t chunk_ws_bytes(const dn_desc* d);

// prep: the layout of dn_gain_prep, else of dn_chunk_fwd
static PadLayout pad_layout(const dn_desc* d, bool prep) {
  const dn_desc p = padded_desc(d);
  const size_t bh = static_cast<size_t>(d->B) * d->H, bht = bh * d->T, es = io_size(d->io);
  const size_t nch = (static_cast<size_t>(d->T) + d->C - 1) / d->C;
  const bool chan = d->decay == DN_DECAY_CHANNEL, pca = per_channel_aux(d);
  PadLayout L{};
  L.inner = prep ? prep_layout(&p).total : chunk_ws_bytes(&p);
  size_t off = round256(L.inner);
  auto take = [&](bool on, size_t bytes) {
    const size_t at = off;
    if (on) off = round256(off + bytes);
    return at;
  };
  L.q = take(!prep, bht * p.dk * es);
  L.k = take(true, bht * p.dk * es);
  L.v = take(!prep, bht * p.dv * es);
  L.o = take(!prep, bht * p.dv * es);
  L.al = take(chan, bht * p.dk * es);
  L.om = take(d->gain == DN_GAIN_KDN, bht * p.dk * es);
  L.w = take(d->gain == DN_GAIN_EXPLICIT, bht * p.dk * es);
  L.s0 = take(!prep, bh * p.dk * p.dv * 4);
  L.sf = take(!prep, bh * p.dk * p.dv * 4);
  L.a0 = take(pca, bh * p.dk * 4);
  L.af = take(pca, bh * p.dk * 4);
  L.wo = take(prep, bht * p.dk * 4);
  L.go = take(prep && chan, bht * p.dk * 4);
  L.ac = take(prep && pca, bh * nch * p.dk * 4);
  L.total = off;
  return L;
}

static size_t chunk_ws_bytes(const dn_desc* d) {
  if (!kernel_dims(d)) return pad_layout(d, false).total;
  if (d->io == DN_F32 && d->dk == 128) return 0;  // the tokenwise kernel: no workspace
  const int nseg = auto_nseg(d);
  return nseg > 1 ? long_layout(d, nseg).total : oor_bytes(d, 1);
}

static size_t prep_ws_bytes(const dn_desc* d) {
  return kernel_dims(d) ? prep_layout(d).total : pad_layout(d, true).total;
}

DN_EXPORT size_t dn_workspace_bytes(const dn_desc* d) {
  if (check_desc(d, false) != DN_OK || (d->C != 64 && d->C != 32) || !paddable(d)) return 0;
  // dn_chunk_fwd needs C = 64; dn_gain_prep takes either chunk length
  const size_t a = d->C == 64 ? chunk_ws_bytes(d) : 0, b = prep_ws_bytes(d);
  return a > b ? a : b;
}

DN_EXPORT size_t dn_chunk_fwd_long_workspace(const dn_desc* d, int nseg) {
  if (check_desc(d, true) != DN_OK || !long_shape_ok(d, nseg)) return 0;
  return long_layout(d, nseg).total;
}

DN_EXPORT int dn_chunk_fwd_long(const dn_desc* d, int nseg, const void* q, const void* k,
                                const void* v, const dn_gates* g, const float* S0,
                                const float* aux0, void* o, float* S_final, float* aux_final,
                                void* ws, size_t ws_bytes, void* stream) {
  int st = check_desc(d, true);
  if (st != DN_OK) return st;
  if (d->io != DN_BF16) return DN_ERR_UNSUPPORTED;
  if (!long_shape_ok(d, nseg)) return DN_ERR_SHAPE;
  if (static_cast<long long>(d->B) * d->H * nseg > 65535) return DN_ERR_SHAPE;
  if ((st = check_gates(d, g)) != DN_OK) return st;
  if (!q || !k || !v || !o) return DN_ERR_NULL;
  const LongLayout lay = long_layout(d, nseg);
  if (!ws || ws_bytes < lay.total) return DN_ERR_WORKSPACE;
  if ((st = check_long_aliases(d, g, q, k, v, S0, aux0, o, S_final, aux_final, ws, lay.total)) !=
      DN_OK)
    return st;
  return run_long(d, nseg, q, k, v, g, S0, aux0, o, S_final, aux_final, ws, lay,
                  static_cast<hipStream_t>(stream));
}

// Copies [outer][rs][cs] -> [outer][rd][cd] (padding with `fill`, or
// cropping); false once a launch failed.
struct Reshaper {
  hipStream_t s;
  bool ok = true;
  void operator()(const void* src, void* dst, long outer, int rs, int cs, int rd, int cd, int esize,
                  uint32_t fill = 0) {
    ok = ok && dn::launch_reshape3(src, dst, outer, rs, cs, rd, cd, esize, fill, s) == hipSuccess;
  }
};

constexpr uint32_t ONE_F32 = 0x3F800000u, ONE_BF16 = 0x3F80u;

// dn_chunk_fwd of a head whose widths no kernel is built for, on validated
// arguments: the inputs padded into the workspace (key channels with k = q =
// w = 0, decay 1, omega 0, statistic 1; value columns with v = 0), the call
// at the padded widths, the outputs cropped back.
static int run_padded_fwd(const dn_desc* d, const PadLayout& L, const void* q, const void* k,
                          const void* v, const dn_gates* g, const float* S0, const float* aux0,
                          void* o, float* S_final, float* aux_final, void* ws, hipStream_t s) {
  const dn_desc p = padded_desc(d);
  char* wb = static_cast<char*>(ws);
  const long bh = static_cast<long>(d->B) * d->H, bht = bh * d->T;
  const int es = static_cast<int>(io_size(d->io));
  const uint32_t one_io = d->io == DN_BF16 ? ONE_BF16 : ONE_F32;
  const bool pca = per_channel_aux(d);
  Reshaper copy{s};
  dn_gates gp = g ? *g : dn_gates{};
  if (d->T > 0) {
    copy(q, wb + L.q, bht, 1, d->dk, 1, p.dk, es);
    copy(k, wb + L.k, bht, 1, d->dk, 1, p.dk, es);
    copy(v, wb + L.v, bht, 1, d->dv, 1, p.dv, es);
    if (d->decay == DN_DECAY_CHANNEL) {
      copy(g->alpha, wb + L.al, bht, 1, d->dk, 1, p.dk, es, one_io);
      gp.alpha = reinterpret_cast<const float*>(wb + L.al);
    }
    if (d->gain == DN_GAIN_KDN) {
      copy(g->omega, wb + L.om, bht, 1, d->dk, 1, p.dk, es);
      gp.omega = wb + L.om;
    }
    if (d->gain == DN_GAIN_EXPLICIT) {
      copy(g->w, wb + L.w, bht, 1, d->dk, 1, p.dk, es);
      gp.w = wb + L.w;
    }
  }
  float* S0p = nullptr;
  if (S0) {
    S0p = reinterpret_cast<float*>(wb + L.s0);
    copy(S0, S0p, bh, d->dk, d->dv, p.dk, p.dv, 4);
  }
  const float* aux0p = aux0;
  if (pca && aux0) {
    aux0p = reinterpret_cast<const float*>(wb + L.a0);
    copy(aux0, wb + L.a0, bh, 1, d->dk, 1, p.dk, 4, ONE_F32);
  }
  float* Sfp = S_final ? reinterpret_cast<float*>(wb + L.sf) : nullptr;
  float* afp = pca ? (aux_final ? reinterpret_cast<float*>(wb + L.af) : nullptr) : aux_final;
  if (!copy.ok) return DN_ERR_HIP;
  const int st = dn_chunk_fwd(&p, wb + L.q, wb + L.k, wb + L.v, &gp, S0p, aux0p, wb + L.o, Sfp, afp,
                              ws, L.inner, s);
  if (st != DN_OK) return st;
  if (d->T > 0) copy(wb + L.o, o, bht, 1, p.dv, 1, d->dv, es);
  if (S_final) copy(Sfp, S_final, bh, p.dk, p.dv, d->dk, d->dv, 4);
  if (pca && aux_final) copy(afp, aux_final, bh, 1, p.dk, 1, d->dk, 4);
  return copy.ok ? DN_OK : DN_ERR_HIP;
}

DN_EXPORT int dn_chunk_fwd(const dn_desc* d, const void* q, const void* k, const void* v,
                           const dn_gates* g, const float* S0, const float* aux0, void* o,
                           float* S_final, float* aux_final, void* ws, size_t ws_bytes,
                           void* stream) {
  int st = check_desc(d, true);
  if (st != DN_OK) return st;
  if (d->T > 0) {
    if ((st = check_gates(d, g)) != DN_OK) return st;
    if (!q || !k || !v || !o) return DN_ERR_NULL;
  }
  if (!paddable(d)) return DN_ERR_UNSUPPORTED;
  const size_t need = chunk_ws_bytes(d);
  if (need > 0 && (!ws || ws_bytes < need)) return DN_ERR_WORKSPACE;

  const size_t bht = static_cast<size_t>(d->B) * d->H * d->T;
  const size_t es = io_size(d->io);
  const size_t sbytes = static_cast<size_t>(d->B) * d->H * d->dk * d->dv * 4;
  const size_t abytes = static_cast<size_t>(d->B) * d->H * aux_per_head(d) * 4;
  const bool has_aux = has_aux_state(d);
  Range in[16];
  const dn_gates nog{};
  int n = gate_ranges(d, g ? g : &nog, in);
  in[n++] = {q, bht * d->dk * es};
  in[n++] = {k, bht * d->dk * es};
  in[n++] = {v, bht * d->dv * es};
  in[n++] = {S0, S0 ? sbytes : 0};
  in[n++] = {has_aux ? aux0 : nullptr, abytes};
  const Range ro{o, bht * d->dv * es}, rs{S_final, S_final ? sbytes : 0},
      ra{has_aux ? aux_final : nullptr, abytes};
  for (int i = 0; i < n; ++i) {
    if (overlap(ro, in[i])) return DN_ERR_ALIAS;
    // S may be updated in place: each workgroup reads and writes only its own
    // value columns.  aux may not: every value slice of a head reads aux0.
    const bool s_in_place = in[i].p == S0 && S_final == S0;
    if (!s_in_place && overlap(rs, in[i])) return DN_ERR_ALIAS;
    if (overlap(ra, in[i])) return DN_ERR_ALIAS;
  }
  if (overlap(ro, rs) || overlap(ro, ra) || overlap(rs, ra)) return DN_ERR_ALIAS;

  // widths no kernel is built for: padded copies in the workspace
  if (!kernel_dims(d)) {
    const PadLayout L = pad_layout(d, false);
    if ((st = check_long_aliases(d, g, q, k, v, S0, aux0, o, S_final, aux_final, ws, L.total)) !=
        DN_OK)
      return st;
    return run_padded_fwd(d, L, q, k, v, g, S0, aux0, o, S_final, aux_final, ws,
                          static_cast<hipStream_t>(stream));
  }

  // few heads: the same forward by segments, on the workspace
  const int nseg = auto_nseg(d);
  if (nseg > 1) {
    const LongLayout lay = long_layout(d, nseg);
    if ((st = check_long_aliases(d, g, q, k, v, S0, aux0, o, S_final, aux_final, ws, lay.total)) !=
        DN_OK)
      return st;
    return run_long(d, nseg, q, k, v, g, S0, aux0, o, S_final, aux_final, ws, lay,
                    static_cast<hipStream_t>(stream));
  }

  // fp32 io at d_k = 128: no chunk kernel is built for it (its fp32 operand
  // tiles would exceed the LDS); the tokenwise kernel runs every head
  if (d->io == DN_F32 && d->dk == 128)
    return run_token_pass(d, q, k, v, g ? g : &nog, S0, aux0, 1, o, S_final, aux_final, nullptr, 0,
                          static_cast<hipStream_t>(stream));
  // per-channel decay: the out-of-range flags in the workspace
  int* const oor = need > 0 ? static_cast<int*>(ws) : nullptr;
  if (oor && (st = check_long_aliases(d, g ? g : &nog, q, k, v, S0, aux0, o, S_final, aux_final, ws,
                                      need)) != DN_OK)
    return st;
  dn::ChunkArgs a;
  a.B = d->B;
  a.H = d->H;
  a.T = d->T;
  a.dk = d->dk;
  a.dv = d->dv;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = gate_args(d, g ? g : &nog);
  a.S0 = S0;
  a.aux0 = has_aux ? aux0 : nullptr;
  a.o = o;
  a.S_final = S_final;
  a.aux_final = has_aux ? aux_final : nullptr;
  a.xcols = 0;
  a.S_final_x = nullptr;
  a.oor = oor;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (dn::launch_chunk_fwd(a, d->io == DN_BF16, d->gain, d->decay == DN_DECAY_CHANNEL, s) !=
      hipSuccess)
    return DN_ERR_HIP;
  // heads whose decay left the range of the chunk form, token by token
  if (!oor || d->T == 0) return DN_OK;
  return run_token_pass(d, q, k, v, g, S0, aux0, 1, o, S_final, aux_final, oor, 1, s);
}

DN_EXPORT int dn_decode_step(const dn_desc* d, const void* q, const void* k, const void* v,
                             const dn_gates* g, float* S, float* aux, void* o, void* stream) {
  int st = check_desc(d, false);
  if (st != DN_OK) return st;
  if (d->T != 1) return DN_ERR_SHAPE;
  if ((st = check_gates(d, g)) != DN_OK) return st;
  const bool has_aux = has_aux_state(d);
  if (!q || !k || !v || !o || !S || (has_aux && !aux)) return DN_ERR_NULL;

  const size_t bh = static_cast<size_t>(d->B) * d->H;
  const size_t es = io_size(d->io);
  Range in[16];
  int n = gate_ranges(d, g, in);
  in[n++] = {q, bh * d->dk * es};
  in[n++] = {k, bh * d->dk * es};
  in[n++] = {v, bh * d->dv * es};
  const Range ro{o, bh * d->dv * es}, rs{S, bh * d->dk * d->dv * 4},
      ra{has_aux ? aux : nullptr, bh * aux_per_head(d) * 4};
  for (int i = 0; i < n; ++i)
    if (overlap(ro, in[i]) || overlap(rs, in[i]) || overlap(ra, in[i])) return DN_ERR_ALIAS;
  if (overlap(ro, rs) || overlap(ro, ra) || overlap(rs, ra)) return DN_ERR_ALIAS;

  dn::DecodeArgs a;
  a.N = d->B;
  a.H = d->H;
  a.dk = d->dk;
  a.dv = d->dv;
  a.q = q;
  a.k = k;
  a.v = v;
  const dn::GateArgs ga = gate_args(d, g);
  a.alpha = ga.alpha;
  a.eta = ga.eta;
  a.alphaP = ga.alphaP;
  a.betaP = ga.betaP;
  a.mu_log = ga.mu_log;
  a.omega = ga.omega;
  a.r = ga.r;
  a.w = ga.w;
  a.eps = ga.eps;
  a.log2x = ga.log2x;
  a.mu_info = ga.mu_info;
  a.S = S;
  a.aux = has_aux ? aux : nullptr;
  a.o = o;
  return hip_status(dn::launch_decode(a, d->io == DN_BF16, d->gain, d->decay == DN_DECAY_CHANNEL,
                                      static_cast<hipStream_t>(stream)));
}

// The gain scans of dn_gain_prep on validated arguments; ws holds at least
// prep_layout(d).total bytes when that is not zero.  w_bf16: w_out receives
// the write vectors in bf16 (RNE) instead of fp32.
static int run_gain_prep(const dn_desc* d, const void* k, const dn_gates* g, const float* aux0,
                         float* w_out, float* g_out, float* aux_chunk, float* aux_final, void* ws,
                         hipStream_t s, bool w_bf16 = false) {
  const bool has_aux = has_aux_state(d);
  const size_t nch = (static_cast<size_t>(d->T) + d->C - 1) / d->C;
  const PrepLayout lay = prep_layout(d);
  dn::GainPrepArgs a;
  a.B = d->B;
  a.H = d->H;
  a.T = d->T;
  a.dk = d->dk;
  a.k = k;
  a.g = gate_args(d, g);
  a.aux0 = has_aux ? aux0 : nullptr;
  a.w_out = w_out;
  a.w_bf16 = w_bf16 ? reinterpret_cast<uint16_t*>(w_out) : nullptr;
  a.g_out = g_out;
  a.aux_chunk = has_aux ? aux_chunk : nullptr;
  a.aux_final = has_aux ? aux_final : nullptr;
  a.C = d->C;
  // Whole chunks: every chunk is scanned by its own workgroup, as a head of
  // the [B, H nch, C] view of the [B, H, T] tensors.  The gains with a
  // statistic first get the statistic entering every chunk from the
  // composed per-token maps of the chunks (the associative gain scan of
  // Kalman Delta Networks §2.6; the chunked statistic recursion of
  // Preconditioned DeltaNet §2.6), written where aux_chunk goes.
  if (prep_by_chunks(d)) {
    if (has_aux) {
      char* wbase = static_cast<char*>(ws);
      dn::StatArgs sa;
      sa.B = d->B;
      sa.H = d->H;
      sa.T = d->T;
      sa.dk = d->dk;
      sa.nseg = static_cast<int>(nch);
      sa.lsub = d->C;
      sa.gain = d->gain;
      sa.channel = d->decay == DN_DECAY_CHANNEL;
      sa.k = k;
      sa.g = a.g;
      sa.aux0 = aux0;
      sa.summ = reinterpret_cast<float*>(wbase + lay.summ);
      sa.aux_in = aux_chunk ? aux_chunk : reinterpret_cast<float*>(wbase + lay.aux_in);
      sa.aux_final = aux_final;
      sa.mu_seg = reinterpret_cast<float*>(wbase + lay.mu_seg);
      if (dn::launch_segment_stats(sa, s) != hipSuccess) return DN_ERR_HIP;
      a.aux0 = sa.aux_in;
      if (d->gain == DN_GAIN_PGDN) a.g.mu_log = sa.mu_seg;
    }
    a.H = static_cast<int>(d->H * nch);
    a.T = d->C;
    a.aux_chunk = nullptr;
    a.aux_final = nullptr;
  }
  return hip_status(dn::launch_gain_prep(a, d->io == DN_BF16, d->gain,
                                         d->decay == DN_DECAY_CHANNEL, s));
}

// dn_gain_prep of a head whose key width no kernel is built for, on validated
// arguments: the inputs padded into the workspace as for run_padded_fwd, the
// scans at the padded width, the outputs cropped back.
static int run_padded_prep(const dn_desc* d, const PadLayout& L, const void* k, const dn_gates* g,
                           const float* aux0, float* w_out, float* g_out, float* aux_chunk,
                           float* aux_final, void* ws, hipStream_t s) {
  const dn_desc p = padded_desc(d);
  char* wb = static_cast<char*>(ws);
  const long bh = static_cast<long>(d->B) * d->H, bht = bh * d->T;
  const long nch = (d->T + d->C - 1) / d->C;
  const int es = static_cast<int>(io_size(d->io));
  const uint32_t one_io = d->io == DN_BF16 ? ONE_BF16 : ONE_F32;
  const bool pca = per_channel_aux(d), chan = d->decay == DN_DECAY_CHANNEL;
  Reshaper copy{s};
  dn_gates gp = *g;
  copy(k, wb + L.k, bht, 1, d->dk, 1, p.dk, es);
  if (chan) {
    copy(g->alpha, wb + L.al, bht, 1, d->dk, 1, p.dk, es, one_io);
    gp.alpha = reinterpret_cast<const float*>(wb + L.al);
  }
  if (d->gain == DN_GAIN_KDN) {
    copy(g->omega, wb + L.om, bht, 1, d->dk, 1, p.dk, es);
    gp.omega = wb + L.om;
  }
  if (d->gain == DN_GAIN_EXPLICIT) {
    copy(g->w, wb + L.w, bht, 1, d->dk, 1, p.dk, es);
    gp.w = wb + L.w;
  }
  const float* aux0p = aux0;
  if (pca && aux0) {
    aux0p = reinterpret_cast<const float*>(wb + L.a0);
    copy(aux0, wb + L.a0, bh, 1, d->dk, 1, p.dk, 4, ONE_F32);
  }
  float* wop = reinterpret_cast<float*>(wb + L.wo);
  float* gop = chan ? (g_out ? reinterpret_cast<float*>(wb + L.go) : nullptr) : g_out;
  float* acp = pca ? (aux_chunk ? reinterpret_cast<float*>(wb + L.ac) : nullptr) : aux_chunk;
  float* afp = pca ? (aux_final ? reinterpret_cast<float*>(wb + L.af) : nullptr) : aux_final;
  if (!copy.ok) return DN_ERR_HIP;
  const int st = run_gain_prep(&p, wb + L.k, &gp, aux0p, wop, gop, acp, afp, ws, s);
  if (st != DN_OK) return st;
  copy(wop, w_out, bht, 1, p.dk, 1, d->dk, 4);
  if (chan && g_out) copy(gop, g_out, bht, 1, p.dk, 1, d->dk, 4);
  if (pca && aux_chunk) copy(acp, aux_chunk, bh * nch, 1, p.dk, 1, d->dk, 4);
  if (pca && aux_final) copy(afp, aux_final, bh, 1, p.dk, 1, d->dk, 4);
  return copy.ok ? DN_OK : DN_ERR_HIP;
}

DN_EXPORT int dn_gain_prep(const dn_desc* d, const void* k, const dn_gates* g, const float* aux0,
                           float* w_out, float* g_out, float* aux_chunk, float* aux_final, void* ws,
                           size_t ws_bytes, void* stream) {
  int st = check_desc(d, false);
  if (st != DN_OK) return st;
  if (d->C != 64 && d->C != 32) return DN_ERR_SHAPE;
  if (!paddable(d)) return DN_ERR_UNSUPPORTED;
  if ((st = check_gates(d, g)) != DN_OK) return st;
  if (!k || !w_out) return DN_ERR_NULL;
  const size_t need = prep_ws_bytes(d);
  if (need > 0 && (!ws || ws_bytes < need)) return DN_ERR_WORKSPACE;
  const bool has_aux = has_aux_state(d);
  const size_t bht = static_cast<size_t>(d->B) * d->H * d->T;
  const size_t es = io_size(d->io);
  const size_t nch = (static_cast<size_t>(d->T) + d->C - 1) / d->C;
  const size_t aph = aux_per_head(d);
  Range in[16];
  int n = gate_ranges(d, g, in);
  in[n++] = {k, bht * d->dk * es};
  in[n++] = {has_aux ? aux0 : nullptr, static_cast<size_t>(d->B) * d->H * aph * 4};
  Range outs[5] = {{w_out, bht * d->dk * 4},
                   {g_out, g_out ? bht * (d->decay == DN_DECAY_CHANNEL ? d->dk : 1) * 4 : 0},
                   {has_aux ? aux_chunk : nullptr, static_cast<size_t>(d->B) * d->H * nch * aph * 4},
                   {has_aux ? aux_final : nullptr, static_cast<size_t>(d->B) * d->H * aph * 4},
                   {need > 0 ? ws : nullptr, need}};
  for (int j = 0; j < 5; ++j) {
    for (int i = 0; i < n; ++i)
      if (overlap(outs[j], in[i])) return DN_ERR_ALIAS;
    for (int i = j + 1; i < 5; ++i)
      if (overlap(outs[j], outs[i])) return DN_ERR_ALIAS;
  }
  if (!kernel_dims(d))
    return run_padded_prep(d, pad_layout(d, true), k, g, aux0, w_out, g_out, aux_chunk, aux_final, ws,
                           static_cast<hipStream_t>(stream));
  return run_gain_prep(d, k, g, aux0, w_out, g_out, aux_chunk, aux_final, ws,
                       static_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------------------
// dn_chunk_fwd_noalloc: dn_chunk_fwd with the workspace in a file-scope
// device array, for callers that cannot allocate.  Every device the library
// runs on holds its own copy of the array until the process ends.  The host
// name `scratch` is not a device address: its device address is looked up
// once per device (hipGetSymbolAddress, with that device current) and only
// that address is passed on.  No segmented step accumulates into the
// workspace (every region is written before it is read), so nothing needs
// clearing between calls.
static __device__ __align__(256) unsigned char scratch[DN_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
void* scratch_ptr[MAX_DEVICES];  // device address of `scratch` per device, once looked up

// The current device's address of `scratch`, or nullptr on a HIP error.
void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    scratch_ptr[dev] = p;
  }
  return scratch_ptr[dev];
}
}  // namespace

DN_EXPORT int dn_chunk_fwd_noalloc(const dn_desc* d, const void* q, const void* k, const void* v,
                                   const dn_gates* g, const float* S0, const float* aux0, void* o,
                                   float* S_final, float* aux_final, void* stream) {
  const int st = check_desc(d, true);
  if (st != DN_OK) return st;
  const size_t need = chunk_ws_bytes(d);
  if (need > DN_NOALLOC_SCRATCH_BYTES) return DN_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0 && !(ws = scratch_address())) return DN_ERR_HIP;
  return dn_chunk_fwd(d, q, k, v, g, S0, aux0, o, S_final, aux_final, ws, need, stream);
}

// ---------------------------------------------------------------------------
// A second stream per device for the backward: on the split path the
// forward checkpoint pass (state entering every chunk, residuals) and the
// Z/P solves plus the serial dS sweep depend on none of each other's results,
// and with few heads each occupies only a few compute units, so then the
// checkpoint pass runs on this stream between two events (fork: after the
// work already queued on the caller's stream; join: before the tile kernel).
// Created once per device at its first use, at the default priority; the
// lock orders the event records of concurrent callers on one device.
namespace {
struct SideStream {
  std::mutex mu;
  bool tried = false;
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
SideStream side_streams[MAX_DEVICES];

// The current device's side stream, locked through `lk`; nullptr if the
// device's stream or events could not be created (the caller then runs
// everything on its own stream).
SideStream* side_stream(std::unique_lock<std::mutex>& lk) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
  SideStream& ss = side_streams[dev];
  lk = std::unique_lock<std::mutex>(ss.mu);
  if (!ss.tried) {
    ss.tried = true;
    if (hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&ss.join, hipEventDisableTiming) != hipSuccess)
      ss.s = nullptr;
  }
  return ss.s ? &ss : nullptr;
}
}  // namespace

// ---------------------------------------------------------------------------
// Chunked backward.  Workspace, each part on a 256-byte boundary: w
// [B, H, T, dk] (fp32, bf16 with bf16 io and scalar decay), S_ck [B, H, nch,
// dk, dv], E [B, H, T, dv], dw_acc [B, H, T, dk], dG ([B, H, T]; channel decay
// [B, H, T, dk]), on the split path dS_ck [B, H, nch, dv, dk] and Z_ck
// [B, H, nch, 64, dk] (split bf16 pairs, 4 bytes each) and with a segmented
// sweep its segment maps A [B, H nseg, dk, dk], B and the chained dS_out
// [B, H nseg, dk, dv], then for the
// gains with a statistic the statistic entering every chunk ([B, H, nch, dk];
// KDN_ISO [B, H, nch]), and the workspace of the gain scans (as for
// dn_gain_prep); fp32 where not said.
struct BwdLayout {
  size_t w, sck, e, dw, dg, dsck, zck, sega, segb, segin, ckl, aux, prep, total;
};

// The split backward: bf16 io, scalar decay, the gains the forward chunk
// kernel runs with a write vector per token (KLA, GDN, PGDN, explicit w), dv
// in 64-column slices.  That kernel writes the checkpoints (the state
// entering every chunk and the residuals E) in a pass without output; the
// serial sweep carries only dS, and one workgroup per chunk forms the
// per-(token, key) gradients.
static bool bwd_split(const dn_desc* d) {
  return d->io == DN_BF16 && d->decay == DN_DECAY_SCALAR && d->gain != DN_GAIN_KDN &&
         d->gain != DN_GAIN_KDN_ISO && d->dv % 64 == 0;
}

// Segments of the split path's serial sweep.  With few heads its
// workgroups (one per head and 64 value columns) leave most compute units
// idle while they walk every chunk in turn; then the chunks are cut into
// nseg segments whose affine maps dS_in = A dS_out + B are formed in
// parallel, chained, and each segment is swept again from its own dS_out.
// Cost in chunk steps: the map pass (value and identity columns) and the
// second pass each take a chunk step per segment chunk and round of
// CU_COUNT workgroups, a link of the chain about 0.6 of a step.  nseg: the
// cheapest power of two with at least four chunks per segment, taken when it
// saves at least a fifth of the plain sweep; 1 below 16 chunks.
static int bwd_nseg(const dn_desc* d) {
  if (!bwd_split(d)) return 1;
  const long long bh = static_cast<long long>(d->B) * d->H;
  const long long nch = (static_cast<long long>(d->T) + 63) / 64;
  if (nch < 16) return 1;
  const long long wv = bh * (d->dv / 64), wm = bh * ((d->dv + d->dk) / 64);
  const double one = rounds(wv) * static_cast<double>(nch);
  double best = one;
  int pick = 1;
  for (int nseg = 2; 4 * nseg <= nch && bh * nseg <= 65535; nseg *= 2) {
    const double len = static_cast<double>((nch + nseg - 1) / nseg);
    const double cost = (rounds(wm * nseg) + rounds(wv * nseg)) * len + 0.6 * nseg;
    if (cost < best) {
      best = cost;
      pick = nseg;
    }
  }
  return best <= 0.8 * one ? pick : 1;
}

// Segments of the split path's checkpoint pass: the forward's own schedule
// (auto_nseg), run as by dn_chunk_fwd_long with the checkpoints written by
// its last step.
static int bwd_ck_nseg(const dn_desc* d) { return bwd_split(d) && d->C == 64 ? auto_nseg(d) : 1; }

static BwdLayout bwd_layout(const dn_desc* d) {
  BwdLayout L{};
  const size_t bh = static_cast<size_t>(d->B) * d->H, bht = bh * d->T;
  const size_t nch = (static_cast<size_t>(d->T) + d->C - 1) / d->C;
  const size_t gdim = d->decay == DN_DECAY_CHANNEL ? d->dk : 1;
  L.w = 0;
  L.sck = round256(L.w + bht * d->dk * 4);
  L.e = round256(L.sck + bh * nch * d->dk * d->dv * 4);
  L.dw = round256(L.e + bht * d->dv * 4);
  L.dg = round256(L.dw + bht * d->dk * 4);
  L.dsck = round256(L.dg + bht * gdim * 4);
  L.zck = round256(L.dsck + (bwd_split(d) ? bh * nch * d->dk * d->dv * 4 : 0));
  const int nseg = bwd_nseg(d);
  const size_t ns = nseg > 1 ? bh * nseg : 0;
  L.sega = round256(L.zck + (bwd_split(d) ? bh * nch * 64 * d->dk * 4 : 0));
  L.segb = round256(L.sega + ns * d->dk * d->dk * 4);
  L.segin = round256(L.segb + ns * d->dk * d->dv * 4);
  const int cks = bwd_ck_nseg(d);
  L.ckl = round256(L.segin + ns * d->dk * d->dv * 4);
  L.aux = round256(L.ckl + (cks > 1 ? long_layout(d, cks).total : 0));
  L.prep = round256(L.aux + (has_aux_state(d) ? bh * nch * aux_per_head(d) * 4 : 0));
  L.total = L.prep + prep_layout(d).total;
  return L;
}

// every gain and decay; io bf16 with dk 64 or 128, fp32 with dk 64; dv a
// multiple of the value slice (16 columns with channel decay, 32 with scalar)
static int bwd_supported(const dn_desc* d) {
  if (!kernel_dims(d)) return DN_ERR_UNSUPPORTED;
  if (d->io == DN_F32 && d->dk != 64) return DN_ERR_UNSUPPORTED;
  if (d->dv % (d->decay == DN_DECAY_CHANNEL ? 16 : 32) != 0) return DN_ERR_UNSUPPORTED;
  return DN_OK;
}

DN_EXPORT size_t dn_chunk_bwd_workspace(const dn_desc* d) {
  if (check_desc(d, true) != DN_OK || bwd_supported(d) != DN_OK) return 0;
  return bwd_layout(d).total;
}

DN_EXPORT int dn_chunk_bwd(const dn_desc* d, const void* q, const void* k, const void* v,
                           const dn_gates* g, const float* S0, const float* aux0, const void* dO,
                           const float* dS_T, const float* daux_T, const dn_grads* gr, void* ws,
                           size_t ws_bytes, void* stream) {
  int st = check_desc(d, true);
  if (st != DN_OK) return st;
  if ((st = bwd_supported(d)) != DN_OK) return st;
  if (!gr) return DN_ERR_NULL;
  const bool pg = d->gain == DN_GAIN_PGDN;
  const bool kd = d->gain == DN_GAIN_KDN || d->gain == DN_GAIN_KDN_ISO;
  const bool has_aux = has_aux_state(d);
  const bool has_eta = d->gain == DN_GAIN_KLA || d->gain == DN_GAIN_GDN || pg;
  const bool chan = d->decay == DN_DECAY_CHANNEL;
  if (d->T > 0) {
    if ((st = check_gates(d, g)) != DN_OK) return st;
    if (!q || !k || !v || !dO || !gr->dq || !gr->dk || !gr->dv || !gr->dalpha) return DN_ERR_NULL;
    if (has_eta && !gr->deta) return DN_ERR_NULL;
    if (pg && (!gr->dalphaP || !gr->dbetaP || !gr->dmu_log)) return DN_ERR_NULL;
    if (kd && (!gr->domega || !gr->dr)) return DN_ERR_NULL;
    if (d->gain == DN_GAIN_EXPLICIT && !gr->dw) return DN_ERR_NULL;
  }
  const BwdLayout lay = bwd_layout(d);
  if (d->T > 0 && (!ws || ws_bytes < lay.total)) return DN_ERR_WORKSPACE;

  const size_t bh = static_cast<size_t>(d->B) * d->H, bht = bh * d->T;
  const size_t es = io_size(d->io);
  const size_t sbytes = bh * d->dk * d->dv * 4;
  const size_t abytes = has_aux ? bh * aux_per_head(d) * 4 : 0;
  Range in[20];
  const dn_gates nog{};
  int n = gate_ranges(d, g ? g : &nog, in);
  in[n++] = {q, bht * d->dk * es};
  in[n++] = {k, bht * d->dk * es};
  in[n++] = {v, bht * d->dv * es};
  in[n++] = {dO, bht * d->dv * es};
  in[n++] = {S0, S0 ? sbytes : 0};
  in[n++] = {has_aux ? aux0 : nullptr, abytes};
  in[n++] = {dS_T, dS_T ? sbytes : 0};
  in[n++] = {has_aux ? daux_T : nullptr, abytes};
  const size_t omega_bytes = d->gain == DN_GAIN_KDN_ISO ? bht * 4 : bht * d->dk * 4;
  constexpr int NOUT = 14;
  const Range outs[NOUT] = {{gr->dq, bht * d->dk * 4},
                            {gr->dk, bht * d->dk * 4},
                            {gr->dv, bht * d->dv * 4},
                            {gr->dalpha, bht * (chan ? d->dk : 1) * 4},
                            {has_eta ? gr->deta : nullptr, bht * 4},
                            {pg ? gr->dalphaP : nullptr, bht * 4},
                            {pg ? gr->dbetaP : nullptr, bht * 4},
                            {pg ? gr->dmu_log : nullptr, static_cast<size_t>(d->H) * 4},
                            {d->gain == DN_GAIN_EXPLICIT ? gr->dw : nullptr, bht * d->dk * 4},
                            {gr->dS0, gr->dS0 ? sbytes : 0},
                            {has_aux ? gr->daux0 : nullptr, abytes},
                            {kd ? gr->domega : nullptr, omega_bytes},
                            {kd ? gr->dr : nullptr, bht * 4},
                            {d->T > 0 ? ws : nullptr, lay.total}};
  for (int j = 0; j < NOUT; ++j) {
    for (int i = 0; i < n; ++i)
      if (overlap(outs[j], in[i])) return DN_ERR_ALIAS;
    for (int i = j + 1; i < NOUT; ++i)
      if (overlap(outs[j], outs[i])) return DN_ERR_ALIAS;
  }

  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (d->T == 0) {
    // no token: dS0 = dS_T, dA_0 = daux_T
    if (gr->dS0) {
      if (dS_T) {
        if (hipMemcpyAsync(gr->dS0, dS_T, sbytes, hipMemcpyDeviceToDevice, s) != hipSuccess) return DN_ERR_HIP;
      } else if (dn::launch_zero(gr->dS0, sbytes / 4, s) != hipSuccess) {
        return DN_ERR_HIP;
      }
    }
    if (has_aux && gr->daux0) {
      if (daux_T) {
        if (hipMemcpyAsync(gr->daux0, daux_T, abytes, hipMemcpyDeviceToDevice, s) != hipSuccess)
          return DN_ERR_HIP;
      } else if (dn::launch_zero(gr->daux0, abytes / 4, s) != hipSuccess) {
        return DN_ERR_HIP;
      }
    }
    if (pg && gr->dmu_log && dn::launch_zero(gr->dmu_log, d->H, s) != hipSuccess) return DN_ERR_HIP;
    return DN_OK;
  }
  char* wb = static_cast<char*>(ws);
  float* w_ws = reinterpret_cast<float*>(wb + lay.w);
  float* dw_acc = reinterpret_cast<float*>(wb + lay.dw);
  float* dG = reinterpret_cast<float*>(wb + lay.dg);
  float* aux_chunk = has_aux ? reinterpret_cast<float*>(wb + lay.aux) : nullptr;
  // the accumulated gradients start at zero (the split path writes dq, dk,
  // dw_acc and dG once each instead)
  const bool split = bwd_split(d);
  if ((!split && (dn::launch_zero(gr->dq, bht * d->dk, s) != hipSuccess ||
                  dn::launch_zero(gr->dk, bht * d->dk, s) != hipSuccess ||
                  dn::launch_zero(dw_acc, bht * d->dk, s) != hipSuccess ||
                  dn::launch_zero(dG, bht * (chan ? d->dk : 1), s) != hipSuccess)) ||
      (pg && dn::launch_zero(gr->dmu_log, d->H, s) != hipSuccess))
    return DN_ERR_HIP;
  const dn::GateArgs ga = gate_args(d, g);
  // the write vectors (and the statistic entering every chunk), chunks in
  // parallel where T is whole chunks; bf16 with bf16 io and scalar decay (the
  // state kernel rounds them to bf16 as it stages them; with per-channel
  // decay it first scales them by the decay, so they stay fp32)
  if ((st = run_gain_prep(d, k, g, has_aux ? aux0 : nullptr, w_ws, nullptr, aux_chunk, nullptr,
                          wb + lay.prep, s, d->io == DN_BF16 && !chan)) != DN_OK)
    return st;
  // the memory recurrence backwards, chunk by chunk
  dn::BwdArgs b;
  b.B = d->B;
  b.H = d->H;
  b.T = d->T;
  b.dk = d->dk;
  b.dv = d->dv;
  b.q = q;
  b.k = k;
  b.v = v;
  b.g = ga;
  b.w = w_ws;
  b.S0 = S0;
  b.dO = dO;
  b.dS_T = dS_T;
  b.S_ck = reinterpret_cast<float*>(wb + lay.sck);
  b.E = reinterpret_cast<float*>(wb + lay.e);
  b.dq_out = gr->dq;
  b.dk_out = gr->dk;
  b.dv_out = gr->dv;
  b.dw_acc = dw_acc;
  b.dG = dG;
  b.dS0 = gr->dS0;
  // the split path: the forward chunk kernel writes the checkpoints, then the
  // serial sweep and the per-chunk tile kernel
  if (split) {
    dn::ChunkArgs ca{};
    ca.B = d->B;
    ca.H = d->H;
    ca.T = d->T;
    ca.dk = d->dk;
    ca.dv = d->dv;
    ca.q = q;
    ca.k = k;
    ca.v = v;
    ca.g = ga;
    ca.S0 = S0;
    ca.aux0 = pg ? aux0 : nullptr;
    ca.S_ck = b.S_ck;
    ca.E_ck = b.E;
    // the checkpoint pass on the side stream, after everything queued so far,
    // when its workgroups (one per head and 64 value columns) fill at most
    // half of the compute units (otherwise both sides fill the device and
    // gain nothing from running together: measured 2.53 against 2.50 ms at
    // B8 H16 T4096 d128, against 0.42 for 0.52 ms at B1 H8)
    std::unique_lock<std::mutex> lk;
    SideStream* ss = 2 * static_cast<long>(bh) * (d->dv / 64) <= CU_COUNT ? side_stream(lk) : nullptr;
    if (ss && (hipEventRecord(ss->fork, s) != hipSuccess || hipStreamWaitEvent(ss->s, ss->fork, 0) != hipSuccess))
      return DN_ERR_HIP;
    // (by segments, as the forward with few heads, when that is cheaper)
    const int cks = bwd_ck_nseg(d);
    if (cks > 1) {
      if ((st = run_long(d, cks, q, k, v, g, S0, pg ? aux0 : nullptr, nullptr, nullptr, nullptr, wb + lay.ckl,
                         long_layout(d, cks), ss ? ss->s : s, b.S_ck, b.E)) != DN_OK)
        return st;
    } else if (dn::launch_chunk_fwd_bf16_scalar(ca, d->gain, ss ? ss->s : s) != hipSuccess) {
      return DN_ERR_HIP;
    }
    if (ss && hipEventRecord(ss->join, ss->s) != hipSuccess) return DN_ERR_HIP;
    b.ck_given = 1;
    b.dS_ck = reinterpret_cast<float*>(wb + lay.dsck);
    b.Z_ck = reinterpret_cast<uint32_t*>(wb + lay.zck);
    b.nseg = bwd_nseg(d);
    if (b.nseg > 1) {
      b.segA = reinterpret_cast<float*>(wb + lay.sega);
      b.segB = reinterpret_cast<float*>(wb + lay.segb);
      b.seg_in = reinterpret_cast<float*>(wb + lay.segin);
    }
    // meanwhile Z, P and the dS sweep on the caller's stream; the tile kernel
    // reads the checkpoints
    if (dn::launch_chunk_bwd_split(b, s, 1) != hipSuccess) return DN_ERR_HIP;
    if (ss && hipStreamWaitEvent(s, ss->join, 0) != hipSuccess) return DN_ERR_HIP;
    // KLA and GDN: the tile kernel also runs the write gain's and the decay's
    // backward (no per-token statistic; dk, deta and dalpha final there)
    const bool fuse = d->gain == DN_GAIN_KLA || d->gain == DN_GAIN_GDN;
    if (fuse) {
      b.fuse_gain = d->gain == DN_GAIN_KLA ? dn::FUSE_KLA : dn::FUSE_GDN;
      b.deta = gr->deta;
      b.dalpha = gr->dalpha;
    }
    if (dn::launch_chunk_bwd_split(b, s, 2) != hipSuccess) return DN_ERR_HIP;
    if (fuse) return DN_OK;
  } else if (dn::launch_chunk_bwd_state(b, d->io == DN_BF16, chan, s) != hipSuccess) {
    return DN_ERR_HIP;
  }
  // the write gains and the decay backwards
  dn::GainBwdArgs gb;
  gb.B = d->B;
  gb.H = d->H;
  gb.T = d->T;
  gb.dk = d->dk;
  gb.k = k;
  gb.g = ga;
  gb.aux_chunk = aux_chunk;
  gb.daux_T = has_aux ? daux_T : nullptr;
  gb.dw_acc = dw_acc;
  gb.dG = dG;
  gb.dk_out = gr->dk;
  gb.dalpha = gr->dalpha;
  gb.deta = has_eta ? gr->deta : nullptr;
  gb.dalphaP = pg ? gr->dalphaP : nullptr;
  gb.dbetaP = pg ? gr->dbetaP : nullptr;
  gb.dmu_log = pg ? gr->dmu_log : nullptr;
  gb.dw_out = d->gain == DN_GAIN_EXPLICIT ? gr->dw : nullptr;
  gb.domega = kd ? gr->domega : nullptr;
  gb.dr = kd ? gr->dr : nullptr;
  gb.daux0 = has_aux ? gr->daux0 : nullptr;
  if (!has_aux && d->T % d->C == 0) {
    // no statistic carried between chunks: every chunk is independent (a head
    // of the [B, H nch, C] view)
    gb.H = static_cast<int>(d->H * (d->T / d->C));
    gb.T = d->C;
  }
  return hip_status(dn::launch_gain_bwd(gb, d->io == DN_BF16, d->gain, chan, s));
}
