// Per-row building blocks shared by the vocabulary-row kernels: element
// access, the per-thread online base-2 log-sum-exp, finishing a row's
// log-prob and the per-token epilogue.  See grpo_rows.hip for the numerics.
#pragma once

#include "../../include/grpo.h"
#include "grpo_device.hpp"
#include "grpo_internal.hpp"
#include "grpo_objective.hpp"

namespace grpo {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

enum RowMode { kFused = 0, kForward = 1, kBackward = 2 };

// --- launch order to work order across the XCDs ----------------------------
#ifndef GRPO_XCD_ROWS
#define GRPO_XCD_ROWS 16  // row kernels: runs of 16 consecutive rows (row blocks) per XCD
#endif
#ifndef GRPO_XCD_FLAT
#define GRPO_XCD_FLAT 64  // the flat gradient pass: runs of 64 consecutive 4 KB blocks (256 KB) per XCD
#endif
// (xcd_runs() in grpo_device.hpp; the launch order is remapped on the device)


// --- element access ---------------------------------------------------------
// In<T, VEC>::N values per chunk; a chunk is one 16-byte load when VEC.
template <typename T, bool VEC> struct In;

template <> struct In<uint16_t, true> {  // bf16, 8 per 16 bytes
  static constexpr int N = 8;
  typedef u32x4 raw_t;
  __device__ static raw_t load(const void* row, int64_t c) {
    return reinterpret_cast<const raw_t*>(row)[c];
  }
  __device__ static raw_t load_nt(const void* row, int64_t c) {
    return __builtin_nontemporal_load(reinterpret_cast<const raw_t*>(row) + c);
  }
  __device__ static void cvt(raw_t r, float (&f)[N]) {
    f[0] = bf16lo(r.x); f[1] = bf16hi(r.x); f[2] = bf16lo(r.y); f[3] = bf16hi(r.y);
    f[4] = bf16lo(r.z); f[5] = bf16hi(r.z); f[6] = bf16lo(r.w); f[7] = bf16hi(r.w);
  }
};

template <> struct In<float, true> {  // f32, 4 per 16 bytes
  static constexpr int N = 4;
  typedef f32x4 raw_t;
  __device__ static raw_t load(const void* row, int64_t c) {
    return reinterpret_cast<const raw_t*>(row)[c];
  }
  __device__ static raw_t load_nt(const void* row, int64_t c) {
    return __builtin_nontemporal_load(reinterpret_cast<const raw_t*>(row) + c);
  }
  __device__ static void cvt(raw_t r, float (&f)[N]) {
    f[0] = r.x; f[1] = r.y; f[2] = r.z; f[3] = r.w;
  }
};

template <> struct In<_Float16, true> {  // f16, 8 per 16 bytes
  static constexpr int N = 8;
  typedef u32x4 raw_t;
  __device__ static raw_t load(const void* row, int64_t c) {
    return reinterpret_cast<const raw_t*>(row)[c];
  }
  __device__ static raw_t load_nt(const void* row, int64_t c) {
    return __builtin_nontemporal_load(reinterpret_cast<const raw_t*>(row) + c);
  }
  __device__ static void cvt(raw_t r, float (&f)[N]) {
    const f2 a = f16x2_to_f32(r.x), b = f16x2_to_f32(r.y), c = f16x2_to_f32(r.z),
             d = f16x2_to_f32(r.w);
    f[0] = a.x; f[1] = a.y; f[2] = b.x; f[3] = b.y;
    f[4] = c.x; f[5] = c.y; f[6] = d.x; f[7] = d.y;
  }
};

template <> struct In<_Float16, false> {
  static constexpr int N = 1;
  typedef uint16_t raw_t;
  __device__ static raw_t load(const void* row, int64_t c) {
    return reinterpret_cast<const uint16_t*>(row)[c];
  }
  __device__ static raw_t load_nt(const void* row, int64_t c) { return load(row, c); }
  __device__ static void cvt(raw_t r, float (&f)[N]) { f[0] = f16_to_f32(r); }
};

template <> struct In<uint16_t, false> {
  static constexpr int N = 1;
  typedef uint16_t raw_t;
  __device__ static raw_t load(const void* row, int64_t c) {
    return reinterpret_cast<const uint16_t*>(row)[c];
  }
  __device__ static raw_t load_nt(const void* row, int64_t c) { return load(row, c); }
  __device__ static void cvt(raw_t r, float (&f)[N]) { f[0] = bf16_to_f32(r); }
};

template <> struct In<float, false> {
  static constexpr int N = 1;
  typedef float raw_t;
  __device__ static raw_t load(const void* row, int64_t c) {
    return reinterpret_cast<const float*>(row)[c];
  }
  __device__ static raw_t load_nt(const void* row, int64_t c) { return load(row, c); }
  __device__ static void cvt(raw_t r, float (&f)[N]) { f[0] = r; }
};

__device__ __forceinline__ float load_one(const void* row, int64_t v, uint16_t*) {
  return bf16_to_f32(reinterpret_cast<const uint16_t*>(row)[v]);
}
__device__ __forceinline__ float load_one(const void* row, int64_t v, float*) {
  return reinterpret_cast<const float*>(row)[v];
}
__device__ __forceinline__ float load_one(const void* row, int64_t v, _Float16*) {
  return f16_to_f32(reinterpret_cast<const uint16_t*>(row)[v]);
}

// Store N gradient values of type TG at chunk c (N consecutive elements).
template <typename TG, int N> struct Out;

template <int N> struct Out<uint16_t, N> {
  __device__ static void store(void* row, int64_t c, const float (&g)[N]) {
    if constexpr (N == 8) {
      u32x4 v = {pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3]), pack_bf16x2(g[4], g[5]),
                 pack_bf16x2(g[6], g[7])};
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(row) + c);
    } else if constexpr (N == 4) {
      u32x2 v = {pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3])};
      __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(row) + c);
    } else {
      reinterpret_cast<uint16_t*>(row)[c] = f32_to_bf16(g[0]);
    }
  }
  __device__ static void zero(void* row, int64_t c) {
    if constexpr (N == 8) {
      u32x4 v = {0u, 0u, 0u, 0u};
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(row) + c);
    } else if constexpr (N == 4) {
      u32x2 v = {0u, 0u};
      __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(row) + c);
    } else {
      reinterpret_cast<uint16_t*>(row)[c] = 0;
    }
  }
};

template <int N> struct Out<_Float16, N> {
  __device__ static void store(void* row, int64_t c, const float (&g)[N]) {
    if constexpr (N == 8) {
      u32x4 v = {pack_f16x2(g[0], g[1]), pack_f16x2(g[2], g[3]), pack_f16x2(g[4], g[5]),
                 pack_f16x2(g[6], g[7])};
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(row) + c);
    } else if constexpr (N == 4) {
      u32x2 v = {pack_f16x2(g[0], g[1]), pack_f16x2(g[2], g[3])};
      __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(row) + c);
    } else {
      reinterpret_cast<uint16_t*>(row)[c] = f32_to_f16(g[0]);
    }
  }
  __device__ static void zero(void* row, int64_t c) { Out<uint16_t, N>::zero(row, c); }
};

template <int N> struct Out<float, N> {
  __device__ static void store(void* row, int64_t c, const float (&g)[N]) {
    if constexpr (N == 8) {
      f32x4 a = {g[0], g[1], g[2], g[3]}, b = {g[4], g[5], g[6], g[7]};
      f32x4* p = reinterpret_cast<f32x4*>(row) + 2 * c;
      __builtin_nontemporal_store(a, p);
      __builtin_nontemporal_store(b, p + 1);
    } else if constexpr (N == 4) {
      f32x4 a = {g[0], g[1], g[2], g[3]};
      __builtin_nontemporal_store(a, reinterpret_cast<f32x4*>(row) + c);
    } else {
      reinterpret_cast<float*>(row)[c] = g[0];
    }
  }
  __device__ static void zero(void* row, int64_t c) {
    if constexpr (N == 8) {
      f32x4 z = {0.f, 0.f, 0.f, 0.f};
      f32x4* p = reinterpret_cast<f32x4*>(row) + 2 * c;
      __builtin_nontemporal_store(z, p);
      __builtin_nontemporal_store(z, p + 1);
    } else if constexpr (N == 4) {
      f32x4 z = {0.f, 0.f, 0.f, 0.f};
      __builtin_nontemporal_store(z, reinterpret_cast<f32x4*>(row) + c);
    } else {
      reinterpret_cast<float*>(row)[c] = 0.0f;
    }
  }
};

__device__ __forceinline__ void store_one(void* row, int64_t v, float g, uint16_t*) {
  reinterpret_cast<uint16_t*>(row)[v] = f32_to_bf16(g);
}
__device__ __forceinline__ void store_one(void* row, int64_t v, float g, float*) {
  reinterpret_cast<float*>(row)[v] = g;
}
__device__ __forceinline__ void store_one(void* row, int64_t v, float g, _Float16*) {
  reinterpret_cast<uint16_t*>(row)[v] = f32_to_f16(g);
}

// --- per-thread online log-sum-exp over one chunk -----------------------------
template <int N>
__device__ __forceinline__ void lse_add(Lse& s, const float (&f)[N]) {
  // the running maximum without a branch: when it does not grow, mL is
  // recomputed to the same rounded value and the sum is scaled by 2^0 = 1
  // exactly, so the bits equal those of a conditional rescale
  float vm = s.m;
#pragma unroll
  for (int j = 0; j < N; ++j) vm = fmaxf(vm, f[j]);
  const float nmL = vm * kLog2e;
  s.s = s.s * fast_exp2(s.mL - nmL);
  s.m = vm;
  s.mL = nmL;
  float e[N];
#pragma unroll
  for (int j = 0; j < N; ++j) e[j] = fast_exp2(fmaf(f[j], kLog2e, -s.mL));
  // pairwise sum: shorter dependency chain, smaller rounding error
#pragma unroll
  for (int w = 1; w < N; w *= 2)
#pragma unroll
    for (int j = 0; j + w < N; j += 2 * w) e[j] = e[j] + e[j + w];
  s.s = s.s + e[0];
}

// If this chunk holds the taken token, capture its value and drop it from the
// chunk (it is added back when the row is finished).
template <int N>
__device__ __forceinline__ void take_out(float (&f)[N], int ja, float& out) {
#pragma unroll
  for (int j = 0; j < N; ++j)
    if (j == ja) {
      out = f[j];
      f[j] = -INFINITY;
    }
}

struct RowLogp {
  float logp;  // log softmax at a
  float c;     // base-2 normaliser for the gradient pass
  float omp;   // 1 - p_a
  float am;    // x_a - M (exact for bf16 inputs)
  float resid; // M * log2e - ML (exact)
  float S;     // sum of 2^(x_v*log2e - ML) over the row
  bool conf;   // p_a >= 1/2: logp came from log1p
};

__device__ RowLogp finish_row(Lse s, float xa) {
  RowLogp r;
  const float M = fmaxf(s.m, xa);
  const float ML = M * kLog2e;
  const float Sx = s.s * fast_exp2(s.mL - ML);
  const float ea = fast_exp2(fmaf(xa, kLog2e, -ML));
  const float S = Sx + ea;
  r.resid = fmaf(M, kLog2e, -ML);
  r.am = xa - M;
  r.S = S;
  r.conf = ea >= Sx;
  if (r.conf) {
    r.logp = -log1pf(Sx / ea);
  } else {
    r.logp = r.am - (logf(S) - r.resid * kLn2);
  }
  r.c = ML + log2f(S);
  r.omp = Sx / S;
  return r;
}

// d = logp_ref - logp.  Away from confident tokens the two log-probs are not
// rounded separately first: d = (am_y - am_x) + (r_y - r_x) ln 2 - log(S_y / S_x),
// which keeps d accurate to about 1e-7 absolute at any vocabulary size.  For
// identical rows every term is exactly zero.
__device__ float row_log_ratio(const RowLogp& px, const RowLogp& py) {
  if (px.conf || py.conf) return py.logp - px.logp;
  return (py.am - px.am) + (py.resid - px.resid) * kLn2 - logf(py.S / px.S);
}

// Per-token epilogue, run by one lane of the row: log-probs, ratio, k3, the
// clipped surrogate and G = d loss / d logp ("GRPO Loss", Accuracy; ms-swift
// REAL blog, background: the clip indicator times A * e^s; dockyard_rl,
// Reference-KL penalty for k3).  Writes the per-token values and returns
// what the gradient pass needs.
struct RowGrad {
  float G, c2, omp;
};

__device__ __forceinline__ RowGrad row_epilogue(const RowArgs& a, int64_t row, Lse sx, Lse sy,
                                                float xa, float ya, bool has_ref, float old,
                                                float gen, float adv, float wgt, float gs,
                                                float keep) {
  const RowLogp px = finish_row(sx, xa);
  const float d = has_ref ? row_log_ratio(px, finish_row(sy, ya)) : 0.0f;
  const TokObj t = token_objective<true>(a.obj, px.logp, old, d, adv, gen, keep);
  const float G = wgt * gs * t.g;
  if (!(isfinite(t.loss) && isfinite(t.kl) && isfinite(G))) atomicOr(&a.hdr->status, GRPO_FAULT_NONFINITE);
  a.tok_loss[row] = t.loss;
  a.tok_kl[row] = t.kl;
  a.flags[row] = t.clipped ? 1 : 0;
  if (a.tok_logp) a.tok_logp[row] = px.logp;
  if (a.out_logp) a.out_logp[row] = px.logp;
  if (a.out_loss) a.out_loss[row] = t.loss;
  if (a.out_kl) a.out_kl[row] = t.kl;
  return RowGrad{G, px.c, px.omp};
}

// A row that contributes nothing (masked, or an out-of-range id): zero
// per-token values and stash; run by one lane.
__device__ __forceinline__ void row_inactive(const RowArgs& a, int64_t row, bool bad) {
  a.tok_loss[row] = 0.0f;
  a.tok_kl[row] = 0.0f;
  a.flags[row] = 0;
  a.stash[row] = RowStash{0.0f, 0.0f, 0.0f, 0.0f};
  if (a.tok_logp) a.tok_logp[row] = 0.0f;
  if (a.out_logp) a.out_logp[row] = 0.0f;
  if (a.out_loss) a.out_loss[row] = 0.0f;
  if (a.out_kl) a.out_kl[row] = 0.0f;
  if (bad) atomicOr(&a.hdr->status, GRPO_FAULT_BAD_ACTION);
}

__device__ __forceinline__ int64_t load_action(const RowArgs& a, int64_t row) {
  return a.ids_i32 ? int64_t(static_cast<const int32_t*>(a.ids)[row])
                   : static_cast<const int64_t*>(a.ids)[row];
}

}  // namespace grpo
