// Host/device shared definitions of libgrpo: workspace layout and kernel
// argument blocks.  Internal to the library.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace grpo {

constexpr size_t kAlign = 256;

inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Workspace header (first 256 bytes).  Every call writes what it later reads:
// the prep kernel clears `status`, the weights kernel writes `num_tokens`.
struct WsHeader {
  uint32_t status;        // GRPO_FAULT_* bits gathered during the call
  uint32_t pad0;
  int64_t num_tokens;     // N
  double mu, sd;          // moments of the global masked normalization
};

// Per-row state handed from the forward pass to the gradient pass.
struct RowStash {
  float G;     // d loss / d logp of the row known after the row pass (0: masked,
               // bad id, or no gradient); the sequence-level policy part is
               // added from the per-sequence coefficient
  float c;     // base-2 log-normaliser: p_v = 2^(x_v * log2e - c)
  float omp;   // 1 - p_a, computed without cancellation
  float act;   // 1: an active row with a valid action id; 0 otherwise
};

struct WsLayout {
  size_t hdr, L, A, w, P, K, C, slogr, useq, lseq, cseq, iwseq, gloss, fault, offsets, tok_loss,
      tok_kl, tok_logp, flags, stash, total;
};

// The token-advantage estimators keep one binary64 value per slot in the stash.
static_assert(sizeof(RowStash) >= sizeof(double), "stash slot too small for a double");

inline WsLayout ws_layout(int64_t B, int64_t T, int32_t num_groups) {
  WsLayout l{};
  size_t o = 0;
  const size_t rows = size_t(B) * size_t(T);
  l.hdr = o; o = align_up(o + sizeof(WsHeader));
  l.L = o; o = align_up(o + size_t(B) * 4);
  l.A = o; o = align_up(o + size_t(B) * 4);
  l.w = o; o = align_up(o + size_t(B) * 8);
  l.P = o; o = align_up(o + size_t(B) * 8);
  l.K = o; o = align_up(o + size_t(B) * 8);
  l.C = o; o = align_up(o + size_t(B) * 8);
  l.slogr = o; o = align_up(o + size_t(B) * 8);   // s_i (sequence-level losses)
  l.useq = o; o = align_up(o + size_t(B) * 4);    // per-sequence gradient coefficient
  l.lseq = o; o = align_up(o + size_t(B) * 8);    // GSPO sequence loss l_i
  l.cseq = o; o = align_up(o + size_t(B) * 4);    // GSPO sequence clipped flag
  l.iwseq = o; o = align_up(o + size_t(B) * 8);   // seq-mask keep flag or GSPO mean weight
  l.gloss = o; o = align_up(o + size_t(B) * 8);   // REAL group losses (<= B groups)
  l.fault = o; o = align_up(o + size_t(B) * 4);   // per-sequence fault bits (token kernel)
  l.tok_loss = o; o = align_up(o + rows * 4);
  l.tok_kl = o; o = align_up(o + rows * 4);
  l.tok_logp = o; o = align_up(o + rows * 4);
  l.flags = o; o = align_up(o + rows);
  l.stash = o; o = align_up(o + rows * sizeof(RowStash));
  // last, so that every other offset is independent of the group count
  l.offsets = o; o = align_up(o + size_t(num_groups > 0 ? num_groups + 1 : 1) * 8);
  l.total = o;
  return l;
}

// Per-token objective parameters, in the precision the kernels compute in.
// `general` is 0 exactly for the clipped surrogate with k3, no dual clip and
// no KL clamps, which takes a shorter code path.
struct Objective {
  float lo, hi;       // clip band [1 - eps_low, 1 + eps_high]
  float beta;         // KL coefficient
  int32_t pg;         // grpo_pg_loss
  int32_t kl;         // grpo_kl_estimator
  int32_t general;
  float dual_c;       // dual-clip bound; 0: off
  float tau_pos, tau_neg;
  float kl_in, kl_out;  // clamps; 0: off
  int32_t has_is;     // off-policy weight exp(old - gen) on the policy term
  int32_t tis;        // truncate that weight to [tis_lo, tis_hi] (tis, icepop)
  float tis_lo, tis_hi;
  int32_t seq;        // 1: sequence-level policy loss (GSPO, REAL): the row and
                      // token passes compute the KL part only
  int32_t seq_mask;   // 1: the weight is multiplied by the sequence's keep flag
};

// Importance-weight statistics per sequence, computed by the prep kernel.
enum IwMode { kIwNone = 0, kIwSeqMask = 1, kIwMean = 2 };

// Device view of a group specification (grpo_groups).
struct GroupSpec {
  int32_t spp;              // uniform group size, or 0 for CSR
  int32_t num_groups;
  const int64_t* offsets;   // device copy of the CSR offsets (num_groups + 1)
  int32_t leave_one_out, scale_by_std;
  double std_eps;
  int32_t clip;             // clamp the advantages to [clip_lo, clip_hi]
  double clip_lo, clip_hi;
};

// Group / advantage / weight preparation.
struct PrepArgs {
  const uint8_t* mask;      // [B, T] or null (all active)
  const float* rewards;     // [B]
  int64_t B, T;             // T == 0: advantages only
  int32_t spp;              // uniform group size, or 0 for CSR
  int32_t num_groups;
  const int64_t* offsets;   // device copy of the CSR offsets (num_groups + 1)
  int32_t leave_one_out, scale_by_std;
  double std_eps;
  int32_t clip;             // clamp the advantages to [clip_lo, clip_hi]
  double clip_lo, clip_hi;
  int32_t reduction;
  double alpha;
  double norm_constant;     // GRPO_FIXED_CONSTANT
  int32_t want_weights;     // 0: advantages only
  int32_t weights_kernel;   // with want_weights: also launch the weights kernel
  // per-sequence importance-weight statistic (IwMode) over the active tokens
  int32_t iw_mode;
  const float* old;
  const float* gen;
  Objective obj;            // token-weight truncation (kIwMean)
  double seq_lo, seq_hi;    // sequence-ratio bounds (kIwSeqMask)
  // workspace
  WsHeader* hdr;
  int32_t* L;
  float* A;
  double* w;
  double* iwseq;            // kIwSeqMask: keep flag (0 or 1); kIwMean: mean token weight
  float* useq;              // cleared to 0 (token-level losses) when non-null
  // outputs (nullable)
  float* adv_out;
  float* seq_weight_out;
  int32_t* seq_tokens_out;
};

// Forward/backward over vocabulary rows.
struct RowArgs {
  const void* x;            // policy logits
  const void* y;            // reference logits (null when beta == 0)
  int64_t ld;               // row stride of x and y, elements
  const void* ids;
  int32_t ids_i32;
  const float* old;
  const float* gen;         // generating policy's log-probs, or null
  const float* adv_tok;     // [B, T] token advantages, or null (per-sequence A)
  const uint8_t* mask;
  int64_t T, V, rows;
  Objective obj;
  const float* grad_scale;  // null = 1
  void* g;                  // gradient out (null in forward-only mode)
  int64_t ldg;
  // workspace
  WsHeader* hdr;
  const float* A;
  const double* w;
  float* tok_loss;
  float* tok_kl;
  uint8_t* flags;
  RowStash* stash;
  float* tok_logp;          // workspace copy of logp (sequence-level losses), or null
  const double* iwseq;      // seq-mask keep flags, or null
  const float* useq;        // backward: per-sequence gradient coefficient
  // per-token outputs (nullable)
  float* out_logp;
  float* out_loss;
  float* out_kl;
};

// Row-kernel instantiation choice.
struct RowLaunch {
  int mode;      // 0 fused forward+backward, 1 forward only, 2 backward only
  int tin;       // logits storage (grpo_fdtype)
  int tg;        // gradient storage (grpo_fdtype)
  int nt;        // threads per row: 64, 256, 512 or 1024
  int vec;       // every row is 16-byte aligned: 16-byte chunks
  int resident;  // fused mode with the policy row held in registers
};

// Per-sequence reduction (stage 1).
struct ReduceArgs {
  int64_t B, T;
  WsHeader* hdr;
  const float* tok_loss;
  const float* tok_kl;
  const uint8_t* flags;
  const double* w;
  double* P;
  double* K;
  int64_t* C;
  // outputs
  float* seq_policy;
  float* seq_kl;
};

// Sequence phase of the sequence-level losses (one block per sequence):
// s_i, and for GSPO the sequence loss, clip flag and gradient coefficient.
struct SeqArgs {
  int64_t B, T;
  int32_t pg;               // GRPO_PG_GSPO or GRPO_PG_REAL
  double lo, hi;            // GSPO clip band (binary64)
  Objective obj;            // token-weight settings (has_is, tis bounds)
  const float* logp;        // [B, T]: the caller's log-probs or the row pass's copy
  const float* old;
  const float* gen;         // or null
  const uint8_t* mask;      // or null
  const float* grad_scale;  // or null
  const RowStash* stash;    // logits path: skips slots with an out-of-range id; else null
  int32_t fill;             // 1: also write token losses, clip flags and P, K, C
  // workspace
  WsHeader* hdr;
  const int32_t* L;
  const float* A;
  const double* w;
  const double* iwseq;      // GSPO mean token weight (null without gen)
  const float* tok_kl;      // fill: the row pass's KL values
  double* slogr;
  float* useq;
  double* lseq;
  int32_t* cseq;
  float* tok_loss;
  uint8_t* flags;
  double* P;
  double* K;
  int64_t* C;
  // outputs (nullable)
  float* seq_logratio;
  float* seq_policy;
  float* seq_kl;
  float* out_loss;
};

// REAL group phase (one block over all groups).
struct RealArgs {
  int64_t B;
  int32_t spp;              // uniform group size, or 0 for CSR
  int32_t num_groups;
  const int64_t* offsets;   // device CSR offsets (num_groups + 1) or null
  double tau;
  const float* grad_scale;
  const int32_t* L;
  const float* A;
  const double* slogr;
  float* useq;
  double* gloss;
};

// Token-level advantage estimators (REINFORCE++, -baseline) and the global
// masked normalization, in passes over the sequences.
struct TokAdvArgs {
  int32_t estimator;        // grpo_adv_estimator
  const float* rewards;
  const float* old;         // or null (no KL shaping)
  const float* ref;         // or null (no KL shaping)
  const uint8_t* mask;
  int64_t B, T;
  int32_t spp, num_groups;
  const int64_t* offsets;
  double kl_coef, gamma;
  int32_t normalize;
  int32_t clip;
  double clip_lo, clip_hi;
  WsHeader* hdr;
  // per sequence: active slots, mean and sum of squared deviations of its
  // raw advantages (the moments the global normalization merges)
  int32_t* L;
  double* mean;
  double* M2;
  double* V;                // [B, T] raw REINFORCE++ returns (normalizing only)
  float* out;               // [B, T]
  uint32_t* status;         // or null
};

// In-place scaling of gradient rows by a device scalar.
struct ScaleArgs {
  void* g;
  int32_t dtype;            // grpo_fdtype
  int64_t rows, V, ld;      // ld: row stride, elements
  const float* scale;       // device scalar; 1 skips the work
};

// GDPO multi-reward advantages (one block).
struct GdpoArgs {
  const float* rewards;     // [C, B]
  int32_t C;
  int64_t B;
  int32_t spp, num_groups;
  const int64_t* offsets;
  int32_t leave_one_out, scale_by_std;
  double std_eps;
  int32_t clip;
  double clip_lo, clip_hi;
  double* total;            // [B] workspace
  float* out;               // [B]
};

// Scalar reduction (stage 2).
struct FinalArgs {
  int64_t B;
  double beta;
  WsHeader* hdr;
  const double* w;
  const double* P;
  const double* K;
  const int64_t* C;
  const double* gloss;      // REAL: group losses; null otherwise
  int64_t num_groups;       // REAL: number of groups
  const int32_t* L;         // non-null: form N (and its fault bit) from these counts
  const uint32_t* fault;    // non-null: the call's fault bits are the OR of these
  float* scalars;
  int64_t* counts;
  uint32_t* status;
};

// Logprob-level token loss.
struct TokenArgs {
  const float* logp;
  const float* old;
  const float* ref;         // null when beta == 0
  const float* gen;         // null: no off-policy weight
  const float* adv_tok;     // [B, T] token advantages, or null (per-sequence A)
  const uint8_t* mask;
  int64_t B, T;
  Objective obj;
  const float* grad_scale;
  float* dlogp;
  // workspace
  WsHeader* hdr;
  const float* A;
  const double* w;
  double* P;
  double* K;
  int64_t* C;
  const double* iwseq;      // seq-mask keep flags, or null
  const float* useq;        // sequence-level: per-sequence gradient coefficient
  const double* lseq;       // GSPO: sequence loss
  const int32_t* cseq;      // GSPO: sequence clipped flag
  // outputs
  float* seq_policy;
  float* seq_kl;
  float* out_loss;
  float* out_kl;
  // token-level objectives: each block forms its own w_i (weights mode 1:
  // from the prep kernel's counts; mode 2: from its own count of the mask,
  // with its own group advantage); the scalar kernel then forms N
  int32_t weights_mode;     // 0: w from the workspace
  int32_t* L;
  int32_t reduction;
  double alpha, norm_constant;
  double* w_out;
  float* seq_weight_out;
  // weights mode 2
  const float* rewards;     // null with token advantages
  GroupSpec grp;
  float* adv_out;
  int32_t* seq_tokens_out;
  uint32_t* fault;
};

}  // namespace grpo
