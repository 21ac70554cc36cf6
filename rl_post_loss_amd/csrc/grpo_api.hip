// libgrpo C ABI: argument validation, workspace layout and kernel launches.
// The declarations, with the meaning, layout, ownership and error behaviour of
// every argument, are in include/grpo.h.

#include <math.h>
#include <string.h>

#include <mutex>

#include <hip/hip_runtime.h>

#include "../../include/grpo.h"
#include "grpo_internal.hpp"

namespace grpo {
hipError_t launch_prep(const PrepArgs& a, hipStream_t stream);
hipError_t launch_zero(void* ws, size_t bytes, hipStream_t stream);
hipError_t launch_reduce(const ReduceArgs& a, hipStream_t stream);
hipError_t launch_token(const TokenArgs& a, hipStream_t stream);
hipError_t launch_final(const FinalArgs& a, hipStream_t stream);
hipError_t launch_rows(const RowArgs& a, const RowLaunch& l, hipStream_t s);
hipError_t launch_seq(const SeqArgs& a, hipStream_t stream);
hipError_t launch_real(const RealArgs& a, hipStream_t stream);
hipError_t launch_token_advantages(const TokAdvArgs& a, hipStream_t s);
hipError_t launch_scale(const ScaleArgs& a, hipStream_t s);
hipError_t launch_gdpo(const GdpoArgs& a, hipStream_t s);
hipError_t launch_copy_offsets(const int64_t* host, int64_t n, int64_t* dev, hipStream_t s);
bool resident_fits(int64_t V, int esize);
}  // namespace grpo

using namespace grpo;

namespace {

hipEvent_t g_ev_start = nullptr;
hipEvent_t g_ev_stop = nullptr;

// Largest element count we accept for one tensor: keeps every byte offset
// far inside int64 and every row index inside the kernels' arithmetic.
constexpr int64_t kMaxElems = int64_t(1) << 50;
// Largest grid dimension: the row kernels launch a block per row (B*T rows),
// the token-advantage output pass a block per 256 slots at most.
constexpr int64_t kMaxGridBlocks = (int64_t(1) << 31) - 1;

bool mul_ok(int64_t a, int64_t b, int64_t limit, int64_t* out) {
  if (a <= 0 || b <= 0) return false;
  if (a > limit / b) return false;
  *out = a * b;
  return true;
}

// Validated group description.  For CSR groups the host offsets are checked
// here and copied into the workspace by the caller of check_groups.
grpo_status check_groups(const grpo_groups* g, int64_t B) {
  if (!g) return GRPO_ERR_NULL;
  const bool uniform = g->samples_per_prompt > 0;
  const bool csr = g->group_boundaries != nullptr;
  if (uniform == csr) return GRPO_ERR_GROUPS;
  if (g->leave_one_out != 0 && g->leave_one_out != 1) return GRPO_ERR_GROUPS;
  if (g->scale_by_std != 0 && g->scale_by_std != 1) return GRPO_ERR_GROUPS;
  if (!(g->std_eps > 0.0) || !isfinite(g->std_eps)) return GRPO_ERR_GROUPS;
  if (g->clip_advantages != 0 && g->clip_advantages != 1) return GRPO_ERR_GROUPS;
  if (g->clip_advantages &&
      !(isfinite(g->adv_clip_low) && isfinite(g->adv_clip_high) && g->adv_clip_low <= g->adv_clip_high))
    return GRPO_ERR_GROUPS;
  if (uniform) {
    if (g->samples_per_prompt < 2 || B % g->samples_per_prompt != 0) return GRPO_ERR_GROUPS;
    return GRPO_OK;
  }
  if (g->num_groups < 1) return GRPO_ERR_GROUPS;
  const int64_t* o = g->group_boundaries;
  if (o[0] != 0 || o[g->num_groups] != B) return GRPO_ERR_GROUPS;
  for (int32_t k = 0; k < g->num_groups; ++k)
    if (o[k + 1] - o[k] < 2) return GRPO_ERR_GROUPS;
  return GRPO_OK;
}

grpo_status check_cfg(const grpo_cfg* c, bool has_ref, bool has_gen) {
  if (!c) return GRPO_ERR_NULL;
  if (!(c->eps_low >= 0.0 && c->eps_low < 1.0)) return GRPO_ERR_CONFIG;
  if (!(c->eps_high >= 0.0) || !isfinite(c->eps_high)) return GRPO_ERR_CONFIG;
  if (!(c->beta >= 0.0) || !isfinite(c->beta)) return GRPO_ERR_CONFIG;
  if (c->beta > 0.0 && !has_ref) return GRPO_ERR_CONFIG;
  if (c->reduction < GRPO_TOKEN_MEAN || c->reduction > GRPO_SEQUENCE_MEAN_LIVE) return GRPO_ERR_CONFIG;
  if (c->reduction == GRPO_LENGTH_ALPHA && !(c->alpha >= 0.0 && c->alpha <= 1.0))
    return GRPO_ERR_CONFIG;
  if (c->reduction == GRPO_FIXED_CONSTANT && !(c->norm_constant > 0.0 && isfinite(c->norm_constant)))
    return GRPO_ERR_CONFIG;
  if (c->pg_loss < GRPO_PG_CLIP || c->pg_loss > GRPO_PG_REAL) return GRPO_ERR_CONFIG;
  // sequence-level ratios exclude the token-level reduction; REAL takes its
  // KL term as the global token mean and no off-policy weights
  if (c->pg_loss == GRPO_PG_GSPO && c->reduction == GRPO_TOKEN_MEAN) return GRPO_ERR_CONFIG;
  if (c->pg_loss == GRPO_PG_REAL &&
      (c->reduction != GRPO_TOKEN_MEAN || has_gen || !(c->real_tau > 0.0 && isfinite(c->real_tau))))
    return GRPO_ERR_CONFIG;
  if (c->kl_estimator < GRPO_KL_K3 || c->kl_estimator > GRPO_KL_K2) return GRPO_ERR_CONFIG;
  // dual clip: 0 (off) or a finite c > 1, with the clipped surrogate only
  if (c->dual_clip_c != 0.0 &&
      !(c->pg_loss == GRPO_PG_CLIP && c->dual_clip_c > 1.0 && isfinite(c->dual_clip_c)))
    return GRPO_ERR_CONFIG;
  if (c->pg_loss == GRPO_PG_SAPO &&
      !(c->sapo_tau_pos > 0.0 && isfinite(c->sapo_tau_pos) && c->sapo_tau_neg > 0.0 &&
        isfinite(c->sapo_tau_neg)))
    return GRPO_ERR_CONFIG;
  for (double v : {c->kl_input_clamp, c->kl_output_clamp})
    if (v != 0.0 && !(v > 0.0 && isfinite(v))) return GRPO_ERR_CONFIG;
  if (c->tis_type < GRPO_TIS_NONE || c->tis_type > GRPO_TIS_SEQ_MASK) return GRPO_ERR_CONFIG;
  if (c->tis_type == GRPO_TIS_SEQ_MASK &&
      (c->pg_loss == GRPO_PG_GSPO || c->pg_loss == GRPO_PG_REAL))
    return GRPO_ERR_CONFIG;
  if (c->tis_type != GRPO_TIS_NONE &&
      !(has_gen && c->tis_ratio_max > 0.0 && isfinite(c->tis_ratio_max) &&
        c->tis_ratio_min >= 0.0 && c->tis_ratio_min <= c->tis_ratio_max))
    return GRPO_ERR_CONFIG;
  return GRPO_OK;
}

// The advantages come from exactly one source: rewards with their groups,
// or the caller's token advantages (then neither rewards nor groups).
grpo_status check_advantage_source(const float* rewards, const float* token_advantages,
                                   const grpo_groups* groups, int64_t B) {
  if (token_advantages) return (rewards || groups) ? GRPO_ERR_CONFIG : GRPO_OK;
  if (!rewards) return GRPO_ERR_NULL;
  return check_groups(groups, B);
}

// CSR group count of a (possibly absent) group description, 0 for uniform.
int32_t group_count_csr(const grpo_groups* g) {
  return (!g || g->samples_per_prompt > 0) ? 0 : g->num_groups;
}

bool is_sequence_level(const grpo_cfg* c) {
  return c->pg_loss == GRPO_PG_GSPO || c->pg_loss == GRPO_PG_REAL;
}

// Number of reward groups of a validated group description.
int64_t group_count(const grpo_groups* g, int64_t B) {
  return g->samples_per_prompt > 0 ? B / g->samples_per_prompt : int64_t(g->num_groups);
}

// Objective parameters for the kernels (float32, as they compute).
Objective make_objective(const grpo_cfg* c, bool has_gen) {
  Objective o{};
  o.lo = float(1.0 - c->eps_low);
  o.hi = float(1.0 + c->eps_high);
  o.beta = float(c->beta);
  o.pg = c->pg_loss;
  o.kl = c->kl_estimator;
  o.dual_c = float(c->dual_clip_c);
  o.tau_pos = float(c->sapo_tau_pos);
  o.tau_neg = float(c->sapo_tau_neg);
  o.kl_in = float(c->kl_input_clamp);
  o.kl_out = float(c->kl_output_clamp);
  o.has_is = has_gen ? 1 : 0;
  o.tis = (c->tis_type == GRPO_TIS_TIS || c->tis_type == GRPO_TIS_ICEPOP) ? 1 : 0;
  o.tis_lo = float(c->tis_ratio_min);
  o.tis_hi = float(c->tis_ratio_max);
  o.seq = is_sequence_level(c) ? 1 : 0;
  o.seq_mask = c->tis_type == GRPO_TIS_SEQ_MASK ? 1 : 0;
  o.general = (o.pg != GRPO_PG_CLIP || o.kl != GRPO_KL_K3 || c->dual_clip_c != 0.0 ||
               c->kl_input_clamp != 0.0 || c->kl_output_clamp != 0.0 || has_gen)
                  ? 1
                  : 0;
  return o;
}

struct Ws {
  WsLayout l;
  char* base;
  WsHeader* hdr() const { return reinterpret_cast<WsHeader*>(base + l.hdr); }
  template <typename T> T* at(size_t off) const { return reinterpret_cast<T*>(base + off); }
};

grpo_status check_ws(void* ws, size_t ws_bytes, int64_t B, int64_t T, int32_t num_groups, Ws* out) {
  if (!ws) return GRPO_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % kAlign != 0) return GRPO_ERR_WORKSPACE;
  const size_t need = grpo_workspace_bytes(B, T, num_groups);
  if (need == 0) return GRPO_ERR_SHAPE;
  if (ws_bytes < need) return GRPO_ERR_WORKSPACE;
  out->l = ws_layout(B, T, num_groups);
  out->base = static_cast<char*>(ws);
  return GRPO_OK;
}

// The device view of a group specification; CSR offsets are copied into the
// workspace (the one host array of the boundary).  No groups: a zero spec.
grpo_status copy_offsets(const Ws& w, const grpo_groups* g, hipStream_t s, GroupSpec* out) {
  *out = GroupSpec{};
  if (!g) return GRPO_OK;
  out->spp = g->samples_per_prompt;
  out->num_groups = g->samples_per_prompt > 0 ? 0 : g->num_groups;
  if (out->num_groups > 0) {
    int64_t* dev = w.at<int64_t>(w.l.offsets);
    if (launch_copy_offsets(g->group_boundaries, int64_t(out->num_groups) + 1, dev, s) != hipSuccess)
      return GRPO_ERR_HIP;
    out->offsets = dev;
  }
  out->leave_one_out = g->leave_one_out;
  out->scale_by_std = g->scale_by_std;
  out->std_eps = g->std_eps;
  out->clip = g->clip_advantages;
  out->clip_lo = g->adv_clip_low;
  out->clip_hi = g->adv_clip_high;
  return GRPO_OK;
}

// Prep launch shared by every entry point: copies CSR offsets, then counts,
// advantages and (optionally) weights.
grpo_status run_prep(const Ws& w, const float* rewards, const uint8_t* mask, int64_t B, int64_t T,
                     const grpo_groups* g, const grpo_cfg* cfg, bool want_weights,
                     const grpo_outputs* out, float* adv_out, hipStream_t s,
                     const float* old = nullptr, const float* gen = nullptr,
                     bool weights_kernel = true) {
  PrepArgs a{};
  a.iw_mode = kIwNone;
  if (cfg && gen) {
    if (cfg->tis_type == GRPO_TIS_SEQ_MASK) a.iw_mode = kIwSeqMask;
    else if (cfg->pg_loss == GRPO_PG_GSPO) a.iw_mode = kIwMean;
  }
  a.old = old;
  a.gen = gen;
  if (cfg) a.obj = make_objective(cfg, gen != nullptr);
  a.seq_lo = cfg ? cfg->tis_ratio_min : 0.0;
  a.seq_hi = cfg ? cfg->tis_ratio_max : 0.0;
  a.iwseq = w.at<double>(w.l.iwseq);
  a.useq = want_weights ? w.at<float>(w.l.useq) : nullptr;
  a.mask = mask;
  a.rewards = g ? rewards : nullptr;  // no groups: the caller gives token advantages
  a.B = B;
  a.T = T;
  a.spp = g ? g->samples_per_prompt : 0;
  a.num_groups = (!g || g->samples_per_prompt > 0) ? 0 : g->num_groups;
  a.offsets = nullptr;
  if (a.num_groups > 0) {
    int64_t* dev = w.at<int64_t>(w.l.offsets);
    if (launch_copy_offsets(g->group_boundaries, int64_t(a.num_groups) + 1, dev, s) != hipSuccess)
      return GRPO_ERR_HIP;
    a.offsets = dev;
  }
  if (g) {
    a.leave_one_out = g->leave_one_out;
    a.scale_by_std = g->scale_by_std;
    a.std_eps = g->std_eps;
    a.clip = g->clip_advantages;
    a.clip_lo = g->adv_clip_low;
    a.clip_hi = g->adv_clip_high;
  }
  a.reduction = cfg ? cfg->reduction : GRPO_TOKEN_MEAN;
  a.alpha = cfg ? cfg->alpha : 0.0;
  a.norm_constant = cfg ? cfg->norm_constant : 0.0;
  a.want_weights = want_weights ? 1 : 0;
  a.weights_kernel = weights_kernel ? 1 : 0;
  a.hdr = w.hdr();
  a.L = w.at<int32_t>(w.l.L);
  a.A = w.at<float>(w.l.A);
  a.w = w.at<double>(w.l.w);
  a.adv_out = adv_out ? adv_out : (out ? out->advantages : nullptr);
  a.seq_weight_out = out ? out->seq_weight : nullptr;
  a.seq_tokens_out = out ? out->seq_tokens : nullptr;
  return launch_prep(a, s) == hipSuccess ? GRPO_OK : GRPO_ERR_HIP;
}

grpo_status run_final(const Ws& w, int64_t B, double beta, const grpo_outputs* out,
                      hipStream_t s, int64_t real_groups = 0, bool count_tokens = false,
                      bool fault_words = false) {
  FinalArgs f{};
  f.L = count_tokens ? w.at<int32_t>(w.l.L) : nullptr;
  f.fault = fault_words ? w.at<uint32_t>(w.l.fault) : nullptr;
  f.B = B;
  f.beta = beta;
  f.gloss = real_groups > 0 ? w.at<double>(w.l.gloss) : nullptr;
  f.num_groups = real_groups;
  f.hdr = w.hdr();
  f.w = w.at<double>(w.l.w);
  f.P = w.at<double>(w.l.P);
  f.K = w.at<double>(w.l.K);
  f.C = w.at<int64_t>(w.l.C);
  f.scalars = out->scalars;
  f.counts = out->counts;
  f.status = out->status;
  return launch_final(f, s) == hipSuccess ? GRPO_OK : GRPO_ERR_HIP;
}

int fdtype_size(int32_t dt) {
  return dt == GRPO_F32 ? 4 : ((dt == GRPO_BF16 || dt == GRPO_F16) ? 2 : 0);
}

// Supported (logits, gradient) storage pairs: a float32 gradient from any
// logits; a bf16 gradient from f32 or bf16 logits; an f16 gradient from f16.
bool dtype_pair_ok(int32_t x, int32_t g) {
  if (g == GRPO_F32) return true;
  if (g == GRPO_BF16) return x == GRPO_F32 || x == GRPO_BF16;
  return g == GRPO_F16 && x == GRPO_F16;
}

bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + bn && b0 < a0 + an;
}

#ifndef GRPO_RESIDENT
#define GRPO_RESIDENT 1    // use the resident-row kernel where it fits
#endif

#ifndef GRPO_NT_LARGE
#define GRPO_NT_LARGE 1024  // threads per row for rows above 64 KB (fused kernel)
#endif
#ifndef GRPO_NT_SPLIT
#define GRPO_NT_SPLIT 256   // threads per row above 4 KB for the forward-only and
                            // gradient-only kernels (several rows per CU, measured best;
                            // the gradient-only pass over aligned rows above 64 KB is
                            // grpo_rows.hip's flat map instead)
#endif
#ifndef GRPO_NT_BWD_MID
#define GRPO_NT_BWD_MID 1024  // the gradient-only kernel on rows of 32-64 KB (measured at
                              // V = 32,000 bf16: 1024 threads 5% faster than 256; it does no
                              // reduction, so the thread count changes no result bit)
#endif

// Threads per row.  The fused kernel gives a long row a whole block; the
// split kernels (one pass each) run better with several rows per CU.
int choose_nt(int64_t V, int esize, int mode) {
  const int64_t bytes = V * esize;
  if (bytes <= 4096) return 64;
  if (mode == 2 && bytes > 32768 && bytes <= 65536) return GRPO_NT_BWD_MID;
  if (mode != 0) return GRPO_NT_SPLIT;
  if (bytes <= 65536) return 256;
  return GRPO_NT_LARGE;
}

// Sequence phase of GSPO / REAL: per-sequence s_i (and the GSPO loss and
// coefficient), then for REAL the group kernel.  `fill` (logits path) also
// writes the token losses and per-sequence totals over the row pass's KL.
grpo_status run_sequence_phase(const Ws& w, const grpo_cfg* cfg, const grpo_groups* g,
                               const float* logp, const float* old, const float* gen,
                               const uint8_t* mask, int64_t B, int64_t T,
                               const float* grad_scale, bool fill, const grpo_outputs* out,
                               hipStream_t s) {
  SeqArgs q{};
  q.B = B;
  q.T = T;
  q.pg = cfg->pg_loss;
  q.lo = 1.0 - cfg->eps_low;
  q.hi = 1.0 + cfg->eps_high;
  q.obj = make_objective(cfg, gen != nullptr);
  q.logp = logp;
  q.old = old;
  q.gen = gen;
  q.mask = mask;
  q.grad_scale = grad_scale;
  q.stash = fill ? w.at<RowStash>(w.l.stash) : nullptr;
  q.fill = fill ? 1 : 0;
  q.hdr = w.hdr();
  q.L = w.at<int32_t>(w.l.L);
  q.A = w.at<float>(w.l.A);
  q.w = w.at<double>(w.l.w);
  q.iwseq = (gen && cfg->pg_loss == GRPO_PG_GSPO) ? w.at<double>(w.l.iwseq) : nullptr;
  q.tok_kl = w.at<float>(w.l.tok_kl);
  q.slogr = w.at<double>(w.l.slogr);
  q.useq = w.at<float>(w.l.useq);
  q.lseq = w.at<double>(w.l.lseq);
  q.cseq = w.at<int32_t>(w.l.cseq);
  q.tok_loss = w.at<float>(w.l.tok_loss);
  q.flags = w.at<uint8_t>(w.l.flags);
  q.P = w.at<double>(w.l.P);
  q.K = w.at<double>(w.l.K);
  q.C = w.at<int64_t>(w.l.C);
  q.seq_logratio = out->seq_logratio;
  q.seq_policy = out->seq_policy;
  q.seq_kl = out->seq_kl;
  q.out_loss = out->tok_loss;
  if (launch_seq(q, s) != hipSuccess) return GRPO_ERR_HIP;
  if (cfg->pg_loss != GRPO_PG_REAL) return GRPO_OK;
  RealArgs r{};
  r.B = B;
  r.spp = g->samples_per_prompt;
  r.num_groups = g->samples_per_prompt > 0 ? 0 : g->num_groups;
  r.offsets = r.num_groups > 0 ? w.at<int64_t>(w.l.offsets) : nullptr;
  r.tau = cfg->real_tau;
  r.grad_scale = grad_scale;
  r.L = q.L;
  r.A = q.A;
  r.slogr = q.slogr;
  r.useq = q.useq;
  r.gloss = w.at<double>(w.l.gloss);
  return launch_real(r, s) == hipSuccess ? GRPO_OK : GRPO_ERR_HIP;
}

// Workspace of grpo_loss_fwd_bwd_noalloc, for callers that cannot allocate:
// one array per GPU, held until the process ends.  In host code `scratch`
// names a host-side stand-in, never the device memory: host code uses only
// the per-device address hipGetSymbolAddress returns for it.
static __device__ __align__(256) unsigned char scratch[GRPO_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of `scratch` on the device that runs `stream` (the current
// device for the null stream), looked up once per device with that device
// current.
grpo_status scratch_for_stream(hipStream_t stream, void** out) {
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return GRPO_ERR_HIP;
  int dev = cur;
  if (stream) {
    hipDevice_t d = 0;
    if (hipStreamGetDevice(stream, &d) != hipSuccess) return GRPO_ERR_HIP;
    dev = int(d);
  }
  if (dev < 0 || dev >= kMaxScratchDevices) return GRPO_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return GRPO_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return GRPO_ERR_HIP;
    if (e != hipSuccess || !p) return GRPO_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return GRPO_OK;
}

}  // namespace

extern "C" {

int grpo_abi_version(void) { return GRPO_ABI_VERSION; }

const char* grpo_status_str(int status) {
  switch (status) {
    case GRPO_OK: return "ok";
    case GRPO_ERR_NULL: return "a required pointer is NULL";
    case GRPO_ERR_SHAPE: return "invalid or overflowing sizes or row stride";
    case GRPO_ERR_DTYPE: return "unknown dtype";
    case GRPO_ERR_GROUPS: return "invalid group specification";
    case GRPO_ERR_CONFIG: return "invalid loss configuration";
    case GRPO_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case GRPO_ERR_ALIAS: return "gradient output overlaps an input without being exactly in place";
    case GRPO_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

size_t grpo_workspace_bytes(int64_t B, int64_t T, int32_t num_groups) {
  int64_t rows;
  if (!mul_ok(B, T, kMaxElems, &rows)) return 0;
  if (num_groups < 0 || num_groups > B) return 0;
  return ws_layout(B, T, num_groups).total;
}

grpo_status grpo_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (!ws || reinterpret_cast<uintptr_t>(ws) % kAlign != 0) return GRPO_ERR_WORKSPACE;
  return launch_zero(ws, ws_bytes, static_cast<hipStream_t>(stream)) == hipSuccess ? GRPO_OK
                                                                                    : GRPO_ERR_HIP;
}

void grpo_set_timing_events(void* start, void* stop) {
  g_ev_start = static_cast<hipEvent_t>(start);
  g_ev_stop = static_cast<hipEvent_t>(stop);
}

grpo_status grpo_advantages(const float* rewards, int64_t B, const grpo_groups* groups,
                            float* adv_out, void* ws, size_t ws_bytes, void* stream) {
  if (!rewards || !adv_out || !groups) return GRPO_ERR_NULL;
  if (B <= 0 || B > (int64_t(1) << 31) - 1) return GRPO_ERR_SHAPE;
  grpo_status st = check_groups(groups, B);
  if (st != GRPO_OK) return st;
  const int32_t ng = groups->samples_per_prompt > 0 ? 0 : groups->num_groups;
  Ws w;
  st = check_ws(ws, ws_bytes, B, 1, ng, &w);
  if (st != GRPO_OK) return st;
  return run_prep(w, rewards, nullptr, B, 0, groups, nullptr, false, nullptr, adv_out,
                  static_cast<hipStream_t>(stream));
}

grpo_status grpo_token_loss(const float* logp, const float* old_logp, const float* ref_logp,
                            const float* gen_logp, const uint8_t* mask, const float* rewards,
                            const float* token_advantages, int64_t B, int64_t T,
                            const grpo_groups* groups, const grpo_cfg* cfg, float* dlogp_out,
                            const float* grad_scale, const grpo_outputs* out, void* ws,
                            size_t ws_bytes, void* stream) {
  if (!logp || !old_logp || !out || !out->scalars) return GRPO_ERR_NULL;
  int64_t rows;
  if (!mul_ok(B, T, kMaxElems, &rows) || B > (int64_t(1) << 31) - 1) return GRPO_ERR_SHAPE;
  grpo_status st = check_advantage_source(rewards, token_advantages, groups, B);
  if (st != GRPO_OK) return st;
  st = check_cfg(cfg, ref_logp != nullptr, gen_logp != nullptr);
  if (st != GRPO_OK) return st;
  if (token_advantages && is_sequence_level(cfg)) return GRPO_ERR_CONFIG;
  const int32_t ng = group_count_csr(groups);
  Ws w;
  st = check_ws(ws, ws_bytes, B, T, ng, &w);
  if (st != GRPO_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // token-level objectives: the token kernel forms the weights itself (no
  // weights kernel), and where no weight needs N and no sequence statistic
  // is needed beforehand, the counts and advantages too (no prep kernel);
  // the sequence-level losses need everything before their sequence phase
  const bool seqlv = is_sequence_level(cfg);
  const bool seq_stat = gen_logp != nullptr && cfg->tis_type == GRPO_TIS_SEQ_MASK;
  // weights needing a batch count (N, or the live sequences) take the prep
  // kernel's counts (mode 1); the others are formed by the token kernel alone
  const bool needs_count =
      cfg->reduction == GRPO_TOKEN_MEAN || cfg->reduction == GRPO_SEQUENCE_MEAN_LIVE;
  const int weights_mode = seqlv ? 0 : ((!needs_count && !seq_stat) ? 2 : 1);
  GroupSpec grp{};
  if (weights_mode == 2) {
    st = copy_offsets(w, groups, s, &grp);
  } else {
    st = run_prep(w, rewards, mask, B, T, groups, cfg, true, out, nullptr, s, old_logp, gen_logp,
                  seqlv);
  }
  if (st != GRPO_OK) return st;
  if (seqlv) {
    st = run_sequence_phase(w, cfg, groups, logp, old_logp, gen_logp, mask, B, T, grad_scale,
                            false, out, s);
    if (st != GRPO_OK) return st;
  }
  TokenArgs a{};
  a.logp = logp;
  a.old = old_logp;
  a.ref = ref_logp;
  a.gen = gen_logp;
  a.adv_tok = token_advantages;
  a.mask = mask;
  a.B = B;
  a.T = T;
  a.obj = make_objective(cfg, gen_logp != nullptr);
  a.grad_scale = grad_scale;
  a.dlogp = dlogp_out;
  a.hdr = w.hdr();
  a.A = w.at<float>(w.l.A);
  a.w = w.at<double>(w.l.w);
  a.P = w.at<double>(w.l.P);
  a.K = w.at<double>(w.l.K);
  a.C = w.at<int64_t>(w.l.C);
  a.iwseq = cfg->tis_type == GRPO_TIS_SEQ_MASK ? w.at<double>(w.l.iwseq) : nullptr;
  a.useq = w.at<float>(w.l.useq);
  a.lseq = w.at<double>(w.l.lseq);
  a.cseq = w.at<int32_t>(w.l.cseq);
  a.seq_policy = out->seq_policy;
  a.seq_kl = out->seq_kl;
  a.out_loss = out->tok_loss;
  a.out_kl = out->tok_kl;
  a.weights_mode = weights_mode;
  a.L = w.at<int32_t>(w.l.L);
  a.reduction = cfg->reduction;
  a.alpha = cfg->alpha;
  a.norm_constant = cfg->norm_constant;
  a.w_out = w.at<double>(w.l.w);
  a.seq_weight_out = out->seq_weight;
  a.rewards = groups ? rewards : nullptr;
  a.grp = grp;
  a.adv_out = out->advantages;
  a.seq_tokens_out = out->seq_tokens;
  a.fault = w.at<uint32_t>(w.l.fault);
  const bool timed = g_ev_start && g_ev_stop;
  if (timed && hipEventRecord(g_ev_start, s) != hipSuccess) return GRPO_ERR_HIP;
  if (launch_token(a, s) != hipSuccess) return GRPO_ERR_HIP;
  if (timed && hipEventRecord(g_ev_stop, s) != hipSuccess) return GRPO_ERR_HIP;
  return run_final(w, B, cfg->beta, out, s,
                   cfg->pg_loss == GRPO_PG_REAL ? group_count(groups, B) : 0, !seqlv,
                   weights_mode == 2);
}

static grpo_status logits_common_checks(const void* policy, int32_t logits_dtype,
                                        int64_t row_stride, const void* action_ids,
                                        int32_t ids_dtype, int64_t B, int64_t T, int64_t V,
                                        void* grad_out, int32_t grad_dtype,
                                        int64_t grad_row_stride, int64_t* rows) {
  if (!policy || !action_ids) return GRPO_ERR_NULL;
  if (fdtype_size(logits_dtype) == 0 || (ids_dtype != GRPO_I64 && ids_dtype != GRPO_I32))
    return GRPO_ERR_DTYPE;
  if (grad_out && (fdtype_size(grad_dtype) == 0 || !dtype_pair_ok(logits_dtype, grad_dtype)))
    return GRPO_ERR_DTYPE;
  int64_t tmp;
  if (!mul_ok(B, T, kMaxElems, rows) || B > (int64_t(1) << 31) - 1) return GRPO_ERR_SHAPE;
  if (V <= 0 || row_stride < V || !mul_ok(*rows, row_stride, kMaxElems, &tmp))
    return GRPO_ERR_SHAPE;
  if (V > (int64_t(1) << 40)) return GRPO_ERR_SHAPE;
  if (*rows > kMaxGridBlocks) return GRPO_ERR_SHAPE;
  if (grad_out && (grad_row_stride < V || !mul_ok(*rows, grad_row_stride, kMaxElems, &tmp)))
    return GRPO_ERR_SHAPE;
  return GRPO_OK;
}

static grpo_status check_alias(const void* policy, const void* ref, int32_t logits_dtype,
                               int64_t row_stride, int64_t rows, int64_t V, const void* grad_out,
                               int32_t grad_dtype, int64_t grad_row_stride) {
  if (!grad_out) return GRPO_OK;
  const size_t xs = size_t((rows - 1) * row_stride + V) * size_t(fdtype_size(logits_dtype));
  const size_t gs = size_t((rows - 1) * grad_row_stride + V) * size_t(fdtype_size(grad_dtype));
  if (grad_out == policy) {
    if (grad_dtype != logits_dtype || grad_row_stride != row_stride) return GRPO_ERR_ALIAS;
  } else if (overlaps(grad_out, gs, policy, xs)) {
    return GRPO_ERR_ALIAS;
  }
  if (ref && ref != policy && overlaps(grad_out, gs, ref, xs)) return GRPO_ERR_ALIAS;
  return GRPO_OK;
}

static bool rows_vectorizable(const void* x, const void* y, int64_t ld, int32_t xdt, const void* g,
                              int64_t ldg, int32_t gdt) {
  const uintptr_t m = 15;
  if ((reinterpret_cast<uintptr_t>(x) & m) || (reinterpret_cast<uintptr_t>(y) & m)) return false;
  if ((ld * fdtype_size(xdt)) & 15) return false;
  if (g && ((reinterpret_cast<uintptr_t>(g) & m) || ((ldg * fdtype_size(gdt)) & 15))) return false;
  return true;
}

// Both logits entry points: validates everything, then (ws == NULL) takes
// the library's scratch array as the workspace, then launches.
static grpo_status loss_fwd_bwd(const void* policy_logits, const void* ref_logits,
                                int32_t logits_dtype, int64_t row_stride, const void* action_ids,
                                int32_t ids_dtype, const float* old_logps, const float* gen_logps,
                                const uint8_t* mask, const float* rewards,
                                const float* token_advantages, int64_t B, int64_t T, int64_t V,
                                const grpo_groups* groups, const grpo_cfg* cfg, void* grad_out,
                                int32_t grad_dtype, int64_t grad_row_stride,
                                const float* grad_scale, const grpo_outputs* out, void* ws,
                                size_t ws_bytes, bool use_scratch, void* stream) {
  if (!old_logps || !out || !out->scalars) return GRPO_ERR_NULL;
  int64_t rows = 0;
  grpo_status st = logits_common_checks(policy_logits, logits_dtype, row_stride, action_ids,
                                        ids_dtype, B, T, V, grad_out, grad_dtype,
                                        grad_row_stride, &rows);
  if (st != GRPO_OK) return st;
  st = check_advantage_source(rewards, token_advantages, groups, B);
  if (st != GRPO_OK) return st;
  st = check_cfg(cfg, ref_logits != nullptr, gen_logps != nullptr);
  if (st != GRPO_OK) return st;
  if (token_advantages && is_sequence_level(cfg)) return GRPO_ERR_CONFIG;
  st = check_alias(policy_logits, ref_logits, logits_dtype, row_stride, rows, V, grad_out,
                   grad_dtype, grad_row_stride);
  if (st != GRPO_OK) return st;
  const int32_t ng = group_count_csr(groups);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (use_scratch) {
    // every argument is valid: refuse sizes beyond the scratch array before
    // touching the device, then take this device's copy of it
    const size_t need = grpo_workspace_bytes(B, T, ng);
    if (need == 0) return GRPO_ERR_SHAPE;
    if (need > GRPO_NOALLOC_SCRATCH_BYTES) return GRPO_ERR_WORKSPACE;
    st = scratch_for_stream(s, &ws);
    if (st != GRPO_OK) return st;
    ws_bytes = GRPO_NOALLOC_SCRATCH_BYTES;
  }
  Ws w;
  st = check_ws(ws, ws_bytes, B, T, ng, &w);
  if (st != GRPO_OK) return st;

  st = run_prep(w, rewards, mask, B, T, groups, cfg, true, out, nullptr, s, old_logps, gen_logps);
  if (st != GRPO_OK) return st;
  const bool seqlv = is_sequence_level(cfg);

  RowArgs a{};
  a.x = policy_logits;
  a.y = ref_logits;
  a.ld = row_stride;
  a.ids = action_ids;
  a.ids_i32 = ids_dtype == GRPO_I32 ? 1 : 0;
  a.old = old_logps;
  a.gen = gen_logps;
  a.adv_tok = token_advantages;
  a.mask = mask;
  a.T = T;
  a.V = V;
  a.rows = rows;
  a.obj = make_objective(cfg, gen_logps != nullptr);
  a.grad_scale = grad_scale;
  a.g = seqlv ? nullptr : grad_out;
  a.ldg = (grad_out && !seqlv) ? grad_row_stride : 0;
  a.hdr = w.hdr();
  a.A = w.at<float>(w.l.A);
  a.w = w.at<double>(w.l.w);
  a.tok_loss = w.at<float>(w.l.tok_loss);
  a.tok_kl = w.at<float>(w.l.tok_kl);
  a.flags = w.at<uint8_t>(w.l.flags);
  a.stash = w.at<RowStash>(w.l.stash);
  a.tok_logp = seqlv ? w.at<float>(w.l.tok_logp) : nullptr;
  a.iwseq = cfg->tis_type == GRPO_TIS_SEQ_MASK ? w.at<double>(w.l.iwseq) : nullptr;
  a.useq = w.at<float>(w.l.useq);
  a.out_logp = out->tok_logp;
  a.out_loss = out->tok_loss;
  a.out_kl = out->tok_kl;
  RowLaunch l{};
  l.mode = (grad_out && !seqlv) ? 0 : 1;
  l.tin = logits_dtype;
  l.tg = grad_out ? grad_dtype : logits_dtype;
  l.nt = choose_nt(V, fdtype_size(logits_dtype), l.mode);
  l.vec = rows_vectorizable(policy_logits, ref_logits, row_stride, logits_dtype, grad_out,
                            grad_row_stride, grad_dtype);
  // rows above 4 KB that fit one block's registers keep the policy row
  // resident between the passes (fused mode); longer rows stream
  l.resident = GRPO_RESIDENT && l.mode == 0 && l.vec && V * fdtype_size(logits_dtype) > 4096 &&
               resident_fits(V, fdtype_size(logits_dtype));
  const bool timed = g_ev_start && g_ev_stop;
  if (timed && hipEventRecord(g_ev_start, s) != hipSuccess) return GRPO_ERR_HIP;
  if (launch_rows(a, l, s) != hipSuccess) return GRPO_ERR_HIP;

  if (seqlv) {
    // the sequence phase needs every log-prob of a sequence; the gradient
    // pass then re-reads the policy rows
    st = run_sequence_phase(w, cfg, groups, a.tok_logp, old_logps, gen_logps, mask, B, T,
                            grad_scale, true, out, s);
    if (st != GRPO_OK) return st;
    if (grad_out) {
      RowArgs b = a;
      b.y = nullptr;
      b.g = grad_out;
      b.ldg = grad_row_stride;
      b.grad_scale = nullptr;  // the row and sequence passes folded it in
      RowLaunch lb = l;
      lb.mode = 2;
      lb.nt = choose_nt(V, fdtype_size(logits_dtype), lb.mode);
      lb.resident = 0;
      if (launch_rows(b, lb, s) != hipSuccess) return GRPO_ERR_HIP;
    }
    if (timed && hipEventRecord(g_ev_stop, s) != hipSuccess) return GRPO_ERR_HIP;
    return run_final(w, B, cfg->beta, out, s,
                     cfg->pg_loss == GRPO_PG_REAL ? group_count(groups, B) : 0);
  }
  if (timed && hipEventRecord(g_ev_stop, s) != hipSuccess) return GRPO_ERR_HIP;

  ReduceArgs r{};
  r.B = B;
  r.T = T;
  r.hdr = w.hdr();
  r.tok_loss = a.tok_loss;
  r.tok_kl = a.tok_kl;
  r.flags = a.flags;
  r.w = a.w;
  r.P = w.at<double>(w.l.P);
  r.K = w.at<double>(w.l.K);
  r.C = w.at<int64_t>(w.l.C);
  r.seq_policy = out->seq_policy;
  r.seq_kl = out->seq_kl;
  if (launch_reduce(r, s) != hipSuccess) return GRPO_ERR_HIP;
  return run_final(w, B, cfg->beta, out, s);
}

grpo_status grpo_loss_fwd_bwd(const void* policy_logits, const void* ref_logits,
                              int32_t logits_dtype, int64_t row_stride, const void* action_ids,
                              int32_t ids_dtype, const float* old_logps, const float* gen_logps,
                              const uint8_t* mask, const float* rewards,
                              const float* token_advantages, int64_t B, int64_t T,
                              int64_t V, const grpo_groups* groups, const grpo_cfg* cfg, void* grad_out,
                              int32_t grad_dtype, int64_t grad_row_stride,
                              const float* grad_scale, const grpo_outputs* out, void* ws,
                              size_t ws_bytes, void* stream) {
  return loss_fwd_bwd(policy_logits, ref_logits, logits_dtype, row_stride, action_ids, ids_dtype,
                      old_logps, gen_logps, mask, rewards, token_advantages, B, T, V, groups, cfg,
                      grad_out, grad_dtype, grad_row_stride, grad_scale, out, ws, ws_bytes, false,
                      stream);
}

grpo_status grpo_loss_fwd_bwd_noalloc(const void* policy_logits, const void* ref_logits,
                                      int32_t logits_dtype, int64_t row_stride,
                                      const void* action_ids, int32_t ids_dtype,
                                      const float* old_logps, const float* gen_logps,
                                      const uint8_t* mask, const float* rewards,
                                      const float* token_advantages, int64_t B, int64_t T,
                                      int64_t V, const grpo_groups* groups, const grpo_cfg* cfg,
                                      void* grad_out, int32_t grad_dtype, int64_t grad_row_stride,
                                      const float* grad_scale, const grpo_outputs* out,
                                      void* stream) {
  return loss_fwd_bwd(policy_logits, ref_logits, logits_dtype, row_stride, action_ids, ids_dtype,
                      old_logps, gen_logps, mask, rewards, token_advantages, B, T, V, groups, cfg,
                      grad_out, grad_dtype, grad_row_stride, grad_scale, out, nullptr, 0, true,
                      stream);
}

grpo_status grpo_loss_bwd(const void* policy_logits, int32_t logits_dtype, int64_t row_stride,
                          const void* action_ids, int32_t ids_dtype, const uint8_t* mask,
                          int64_t B, int64_t T, int64_t V, void* grad_out, int32_t grad_dtype,
                          int64_t grad_row_stride, const float* grad_scale, void* ws,
                          size_t ws_bytes, void* stream) {
  if (!grad_out) return GRPO_ERR_NULL;
  int64_t rows = 0;
  grpo_status st = logits_common_checks(policy_logits, logits_dtype, row_stride, action_ids,
                                        ids_dtype, B, T, V, grad_out, grad_dtype,
                                        grad_row_stride, &rows);
  if (st != GRPO_OK) return st;
  st = check_alias(policy_logits, nullptr, logits_dtype, row_stride, rows, V, grad_out,
                   grad_dtype, grad_row_stride);
  if (st != GRPO_OK) return st;
  Ws w;
  st = check_ws(ws, ws_bytes, B, T, 0, &w);  // the stash offset does not depend on groups
  if (st != GRPO_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  RowArgs a{};
  a.x = policy_logits;
  a.y = nullptr;
  a.ld = row_stride;
  a.ids = action_ids;
  a.ids_i32 = ids_dtype == GRPO_I32 ? 1 : 0;
  a.mask = mask;
  a.T = T;
  a.V = V;
  a.rows = rows;
  a.grad_scale = grad_scale;
  a.g = grad_out;
  a.ldg = grad_row_stride;
  a.hdr = w.hdr();
  a.stash = w.at<RowStash>(w.l.stash);
  a.useq = w.at<float>(w.l.useq);
  RowLaunch l{};
  l.mode = 2;
  l.tin = logits_dtype;
  l.tg = grad_dtype;
  l.nt = choose_nt(V, fdtype_size(logits_dtype), l.mode);
  l.vec = rows_vectorizable(policy_logits, nullptr, row_stride, logits_dtype, grad_out,
                            grad_row_stride, grad_dtype);
  const bool timed = g_ev_start && g_ev_stop;
  if (timed && hipEventRecord(g_ev_start, s) != hipSuccess) return GRPO_ERR_HIP;
  if (launch_rows(a, l, s) != hipSuccess) return GRPO_ERR_HIP;
  if (timed && hipEventRecord(g_ev_stop, s) != hipSuccess) return GRPO_ERR_HIP;
  return GRPO_OK;
}

grpo_status grpo_token_advantages(int32_t estimator, const float* rewards, const float* old_logp,
                                  const float* ref_logp, const uint8_t* mask, int64_t B, int64_t T,
                                  const grpo_groups* groups, double kl_coef, double gamma,
                                  int32_t normalize, float* adv_out, uint32_t* status, void* ws,
                                  size_t ws_bytes, void* stream) {
  if (!rewards || !adv_out) return GRPO_ERR_NULL;
  int64_t rows;
  if (!mul_ok(B, T, kMaxElems, &rows) || B > (int64_t(1) << 31) - 1) return GRPO_ERR_SHAPE;
  if ((rows + 255) / 256 > kMaxGridBlocks) return GRPO_ERR_SHAPE;
  if (estimator != GRPO_ADV_REINFORCE_PP && estimator != GRPO_ADV_REINFORCE_PP_BASELINE)
    return GRPO_ERR_CONFIG;
  if (!(kl_coef >= 0.0 && isfinite(kl_coef)) || !(gamma > 0.0 && gamma <= 1.0))
    return GRPO_ERR_CONFIG;
  if (normalize != 0 && normalize != 1) return GRPO_ERR_CONFIG;
  if (estimator == GRPO_ADV_REINFORCE_PP && kl_coef != 0.0 && (!old_logp || !ref_logp))
    return GRPO_ERR_NULL;
  if (groups) {
    grpo_status st = check_groups(groups, B);
    if (st != GRPO_OK) return st;
  }
  if (estimator == GRPO_ADV_REINFORCE_PP_BASELINE) {
    // the inclusive group mean without std division
    if (!groups) return GRPO_ERR_NULL;
    if (groups->leave_one_out || groups->scale_by_std) return GRPO_ERR_GROUPS;
  }
  const int32_t ng = group_count_csr(groups);
  Ws w;
  grpo_status st = check_ws(ws, ws_bytes, B, T, ng, &w);
  if (st != GRPO_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  TokAdvArgs a{};
  a.estimator = estimator;
  a.rewards = rewards;
  a.old = old_logp;
  a.ref = ref_logp;
  a.mask = mask;
  a.B = B;
  a.T = T;
  a.spp = groups ? groups->samples_per_prompt : 0;
  a.num_groups = ng;
  if (ng > 0) {
    int64_t* dev = w.at<int64_t>(w.l.offsets);
    if (launch_copy_offsets(groups->group_boundaries, int64_t(ng) + 1, dev, s) != hipSuccess)
      return GRPO_ERR_HIP;
    a.offsets = dev;
  }
  a.kl_coef = kl_coef;
  a.gamma = gamma;
  a.normalize = normalize;
  a.clip = groups ? groups->clip_advantages : 0;
  a.clip_lo = groups ? groups->adv_clip_low : 0.0;
  a.clip_hi = groups ? groups->adv_clip_high : 0.0;
  a.hdr = w.hdr();
  a.L = w.at<int32_t>(w.l.L);
  a.mean = w.at<double>(w.l.P);
  a.M2 = w.at<double>(w.l.K);
  a.V = w.at<double>(w.l.stash);  // the row stash (16 bytes per slot) holds one double per slot
  a.out = adv_out;
  a.status = status;
  const bool timed = g_ev_start && g_ev_stop;
  if (timed && hipEventRecord(g_ev_start, s) != hipSuccess) return GRPO_ERR_HIP;
  if (launch_token_advantages(a, s) != hipSuccess) return GRPO_ERR_HIP;
  if (timed && hipEventRecord(g_ev_stop, s) != hipSuccess) return GRPO_ERR_HIP;
  return GRPO_OK;
}

grpo_status grpo_gdpo_advantages(const float* rewards, int32_t num_components, int64_t B,
                                 const grpo_groups* groups, float* adv_out, void* ws,
                                 size_t ws_bytes, void* stream) {
  if (!rewards || !adv_out) return GRPO_ERR_NULL;
  if (B <= 0 || B > (int64_t(1) << 31) - 1) return GRPO_ERR_SHAPE;
  if (num_components < 2) return GRPO_ERR_CONFIG;
  int64_t tmp;
  if (!mul_ok(B, num_components, kMaxElems, &tmp)) return GRPO_ERR_SHAPE;
  grpo_status st = check_groups(groups, B);
  if (st != GRPO_OK) return st;
  const int32_t ng = group_count_csr(groups);
  Ws w;
  st = check_ws(ws, ws_bytes, B, 1, ng, &w);
  if (st != GRPO_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  GdpoArgs a{};
  a.rewards = rewards;
  a.C = num_components;
  a.B = B;
  a.spp = groups->samples_per_prompt;
  a.num_groups = ng;
  if (ng > 0) {
    int64_t* dev = w.at<int64_t>(w.l.offsets);
    if (launch_copy_offsets(groups->group_boundaries, int64_t(ng) + 1, dev, s) != hipSuccess)
      return GRPO_ERR_HIP;
    a.offsets = dev;
  }
  a.leave_one_out = groups->leave_one_out;
  a.scale_by_std = groups->scale_by_std;
  a.std_eps = groups->std_eps;
  a.clip = groups->clip_advantages;
  a.clip_lo = groups->adv_clip_low;
  a.clip_hi = groups->adv_clip_high;
  a.total = w.at<double>(w.l.P);
  a.out = adv_out;
  return launch_gdpo(a, s) == hipSuccess ? GRPO_OK : GRPO_ERR_HIP;
}

grpo_status grpo_scale_grad(void* grad, int32_t grad_dtype, int64_t rows, int64_t V,
                            int64_t row_stride, const float* scale, void* stream) {
  if (!grad || !scale) return GRPO_ERR_NULL;
  if (fdtype_size(grad_dtype) == 0) return GRPO_ERR_DTYPE;
  int64_t tmp;
  if (rows <= 0 || V <= 0 || row_stride < V || !mul_ok(rows, row_stride, kMaxElems, &tmp))
    return GRPO_ERR_SHAPE;
  ScaleArgs a{};
  a.g = grad;
  a.dtype = grad_dtype;
  a.rows = rows;
  a.V = V;
  a.ld = row_stride;
  a.scale = scale;
  return launch_scale(a, static_cast<hipStream_t>(stream)) == hipSuccess ? GRPO_OK : GRPO_ERR_HIP;
}

}  // extern "C"
