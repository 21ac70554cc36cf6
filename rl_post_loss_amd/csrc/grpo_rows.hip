// Vocabulary-row kernels: the bandwidth-bound part of the GRPO loss.
//
// One group of NT threads owns one row (i, t) of [B, T, V] logits:
//   pass 1  streams the policy row x and the reference row y once, keeping a
//           running base-2 log-sum-exp per thread (online normaliser, as in
//           the grpo.cpp README's fused logits kernel, CUDA section) and
//           picking out x_a, y_a on the way;
//   epilogue (one lane) forms logp, logp_ref, the ratio, k3, the clipped
//           surrogate and the per-token gradient weight G ("GRPO Loss",
//           Accuracy; ms-swift REAL blog, background: clip indicator times
//           A * e^s; dockyard_rl, Reference-KL penalty);
//   pass 2  re-reads x and writes g_v = G * (onehot(a)_v - softmax(x)_v)
//           ("GRPO Loss", Entry Point: the gradient lands in policy_logits).
// Pass 2 walks the row backwards, so the bytes pass 1 read last are the
// first ones re-read, while they are still in L2 / the memory-side cache.
//
// Numerics (all float32): every thread accumulates
//   S_t = sum 2^(fma(x_v, log2e, -mL_t)),  mL_t = fl(m_t * log2e),
// leaving out the taken token a.  Merging threads rescales by 2^(mL - mL').
// The lane that finishes the row adds x_a back; with M the row maximum,
// ML = fl(M * log2e) and r = M*log2e - ML (exact, from one fma):
//   S = S_excl + e_a,  e_a = 2^(fma(x_a, log2e, -ML))
//   logp = -log1p(S_excl / e_a)                       if e_a >= S_excl
//        = (x_a - M) - (log S - r ln 2)               otherwise
//   1 - p_a = S_excl / S                              (no cancellation)
//   p_v = 2^(fma(x_v, log2e, -c)),  c = ML + log2 S
// The policy and reference rows go through the same code, so identical rows
// give bit-identical log-probs and d = 0 exactly.

#include "../../include/grpo.h"
#include "grpo_device.hpp"
#include "grpo_internal.hpp"

namespace grpo {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

enum RowMode { kFused = 0, kForward = 1, kBackward = 2 };

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

// --- per-thread online log-sum-exp over one chunk -----------------------------
template <int N>
__device__ __forceinline__ void lse_add(Lse& s, const float (&f)[N]) {
  float vm = f[0];
#pragma unroll
  for (int j = 1; j < N; ++j) vm = fmaxf(vm, f[j]);
  if (vm > s.m) {
    const float nmL = vm * kLog2e;
    s.s = s.s * fast_exp2(s.mL - nmL);
    s.m = vm;
    s.mL = nmL;
  }
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

// --- the row kernel ----------------------------------------------------------
// NT threads per row; BLOCK = max(NT, 256) threads per block, BLOCK / NT rows
// per block.  U chunks of x (and y) are loaded before any is used.
template <typename TI, typename TG, int NT, int MODE, bool VEC, int U>
__global__ __launch_bounds__(NT < 256 ? 256 : NT) void grpo_rows_kernel(RowArgs a) {
  constexpr int BLOCK = NT < 256 ? 256 : NT;
  constexpr int RPB = BLOCK / NT;  // rows per block
  constexpr int NW = NT / kWave;   // waves per row (1 when NT == 64)
  typedef In<TI, VEC> IN;
  constexpr int N = IN::N;
  constexpr bool kPass1 = MODE != kBackward;
  constexpr bool kPass2 = MODE != kForward;

  __shared__ Lse sh_lse[2][NW > 1 ? NW : 1];
  __shared__ float sh_xa[2];
  __shared__ float sh_bcast[4];

  const int lid = threadIdx.x % NT;
  const int64_t row = int64_t(blockIdx.x) * RPB + threadIdx.x / NT;
  if (row >= a.rows) return;  // only possible when RPB > 1 (no block barriers then)

  const int64_t V = a.V;
  const int64_t nvec = V / N;           // whole chunks
  const int64_t tail0 = nvec * N;       // first element of the scalar tail
  const void* xrow = static_cast<const char*>(a.x) + row * a.ld * int64_t(sizeof(TI));
  void* grow = kPass2 ? static_cast<char*>(a.g) + row * a.ldg * int64_t(sizeof(TG)) : nullptr;

  // ---- row status --------------------------------------------------------
  float G = 0.0f, c2 = 0.0f, omp = 0.0f;
  int64_t aid = 0;
  if constexpr (kPass1) {
    const bool active = a.mask == nullptr || a.mask[row] != 0;
    if (active)
      aid = a.ids_i32 ? int64_t(static_cast<const int32_t*>(a.ids)[row])
                      : static_cast<const int64_t*>(a.ids)[row];
    const bool bad = active && (aid < 0 || aid >= V);
    if (!active || bad) {
      if (lid == 0) {
        a.tok_loss[row] = 0.0f;
        a.tok_kl[row] = 0.0f;
        a.flags[row] = 0;
        a.stash[row] = RowStash{0.0f, 0.0f, 0.0f, 0.0f};
        if (a.out_logp) a.out_logp[row] = 0.0f;
        if (a.out_loss) a.out_loss[row] = 0.0f;
        if (a.out_kl) a.out_kl[row] = 0.0f;
        if (bad) atomicOr(&a.hdr->status, GRPO_FAULT_BAD_ACTION);
      }
      if constexpr (kPass2) {
        for (int64_t c = lid; c < nvec; c += NT) Out<TG, N>::zero(grow, c);
        for (int64_t v = tail0 + lid; v < V; v += NT) store_one(grow, v, 0.0f, (TG*)nullptr);
      }
      return;
    }

    // taken token's chunk and lane inside the chunk
    const int64_t ca = aid / N;
    const int ja = int(aid - ca * N);
    const bool has_ref = a.y != nullptr;
    const void* yrow = has_ref ? static_cast<const char*>(a.y) + row * a.ld * int64_t(sizeof(TI))
                               : nullptr;

    // per-token side inputs, loaded early by the finishing lane
    float old = 0.0f, adv = 0.0f, wgt = 0.0f, gs = 1.0f;
    if (lid == 0) {
      old = a.old[row];
      const int64_t i = row / a.T;
      adv = a.A[i];
      wgt = float(a.w[i]);
      if (a.grad_scale) gs = *a.grad_scale;
    }

    // ---- pass 1 ----------------------------------------------------------
    Lse sx = lse_init(), sy = lse_init();
    float xa = 0.0f, ya = 0.0f;
    bool own = false;
    int64_t c = lid;
    for (; c + (U - 1) * NT < nvec; c += U * NT) {
      typename IN::raw_t rx[U], ry[U];
#pragma unroll
      for (int u = 0; u < U; ++u) rx[u] = IN::load(xrow, c + u * NT);
      if (has_ref) {
#pragma unroll
        for (int u = 0; u < U; ++u) ry[u] = IN::load_nt(yrow, c + u * NT);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float fx[N], fy[N];
        IN::cvt(rx[u], fx);
        if (has_ref) IN::cvt(ry[u], fy);
        if (c + u * NT == ca) {
          own = true;
          take_out(fx, ja, xa);
          if (has_ref) take_out(fy, ja, ya);
        }
        lse_add(sx, fx);
        if (has_ref) lse_add(sy, fy);
      }
    }
    for (; c < nvec; c += NT) {
      float fx[N], fy[N];
      IN::cvt(IN::load(xrow, c), fx);
      if (has_ref) IN::cvt(IN::load_nt(yrow, c), fy);
      if (c == ca) {
        own = true;
        take_out(fx, ja, xa);
        if (has_ref) take_out(fy, ja, ya);
      }
      lse_add(sx, fx);
      if (has_ref) lse_add(sy, fy);
    }
    for (int64_t v = tail0 + lid; v < V; v += NT) {
      float fx[1] = {load_one(xrow, v, (TI*)nullptr)};
      float fy[1] = {has_ref ? load_one(yrow, v, (TI*)nullptr) : 0.0f};
      if (v == aid) {
        own = true;
        take_out(fx, 0, xa);
        if (has_ref) take_out(fy, 0, ya);
      }
      lse_add(sx, fx);
      if (has_ref) lse_add(sy, fy);
    }

    // ---- reduce the row ----------------------------------------------------
    sx = wave_lse<kWave>(sx);
    if (has_ref) sy = wave_lse<kWave>(sy);
    if constexpr (NW > 1) {
      const int wv = lid / kWave;
      if (lid % kWave == 0) {
        sh_lse[0][wv] = sx;
        sh_lse[1][wv] = sy;
      }
      if (own) {
        sh_xa[0] = xa;
        sh_xa[1] = ya;
      }
      __syncthreads();
      if (lid == 0) {
        sx = sh_lse[0][0];
        sy = sh_lse[1][0];
        for (int k = 1; k < NW; ++k) {
          sx = lse_merge(sx, sh_lse[0][k]);
          if (has_ref) sy = lse_merge(sy, sh_lse[1][k]);
        }
        xa = sh_xa[0];
        ya = sh_xa[1];
      }
    } else {
      // the owner lane of the taken token inside this wave
      const int owner = ca < nvec ? int(ca % NT) : int((aid - tail0) % NT);
      xa = __shfl(xa, owner);
      ya = __shfl(ya, owner);
    }

    // ---- per-token epilogue -------------------------------------------------
    if (lid == 0) {
      const RowLogp px = finish_row(sx, xa);
      float d = 0.0f;
      if (has_ref) d = row_log_ratio(px, finish_row(sy, ya));
      const float rho = expf(px.logp - old);
      const float k3 = expm1f(d) - d;
      const bool clipped = (adv > 0.0f && rho > a.hi) || (adv < 0.0f && rho < a.lo);
      const float unc = rho * adv;
      const float clp = fminf(fmaxf(rho, a.lo), a.hi) * adv;
      const float tl = -fminf(unc, clp);
      const float dloss = clipped ? 0.0f : -adv * rho;
      const float dkl = -expm1f(d);
      G = wgt * gs * (dloss + a.beta * dkl);
      if (!(isfinite(tl) && isfinite(k3) && isfinite(G)))
        atomicOr(&a.hdr->status, GRPO_FAULT_NONFINITE);
      a.tok_loss[row] = tl;
      a.tok_kl[row] = k3;
      a.flags[row] = clipped ? 1 : 0;
      if (a.out_logp) a.out_logp[row] = px.logp;
      if (a.out_loss) a.out_loss[row] = tl;
      if (a.out_kl) a.out_kl[row] = k3;
      c2 = px.c;
      omp = px.omp;
      if constexpr (!kPass2) a.stash[row] = RowStash{G, c2, omp, 0.0f};
    }
    if constexpr (!kPass2) return;
    // broadcast G, c2, omp to the row's threads
    if constexpr (NW > 1) {
      if (lid == 0) {
        sh_bcast[0] = G;
        sh_bcast[1] = c2;
        sh_bcast[2] = omp;
      }
      __syncthreads();
      G = sh_bcast[0];
      c2 = sh_bcast[1];
      omp = sh_bcast[2];
    } else {
      G = __shfl(G, 0);
      c2 = __shfl(c2, 0);
      omp = __shfl(omp, 0);
    }
  } else {
    // backward only: per-row state from the forward pass
    const RowStash st = a.stash[row];
    G = st.G * (a.grad_scale ? *a.grad_scale : 1.0f);
    c2 = st.c;
    omp = st.omp;
    if (G != 0.0f)
      aid = a.ids_i32 ? int64_t(static_cast<const int32_t*>(a.ids)[row])
                      : static_cast<const int64_t*>(a.ids)[row];
  }

  if constexpr (kPass2) {
    // ---- pass 2: g_v = G * (onehot(a)_v - p_v) -----------------------------
    if (G == 0.0f) {
      for (int64_t c = lid; c < nvec; c += NT) Out<TG, N>::zero(grow, c);
      for (int64_t v = tail0 + lid; v < V; v += NT) store_one(grow, v, 0.0f, (TG*)nullptr);
      return;
    }
    const int64_t ca = aid / N;
    const int ja = int(aid - ca * N);
    const float ga = G * omp;
    const float mG = -G;
    // tail first (it was read last)
    for (int64_t v = tail0 + lid; v < V; v += NT) {
      const float xv = load_one(xrow, v, (TI*)nullptr);
      const float gv = (v == aid) ? ga : mG * fast_exp2(fmaf(xv, kLog2e, -c2));
      store_one(grow, v, gv, (TG*)nullptr);
    }
    if (lid < nvec) {
      const int64_t last = lid + ((nvec - 1 - lid) / NT) * NT;  // this thread's last chunk
      int64_t c = last;
      for (; c - (U - 1) * NT >= 0; c -= U * NT) {
        typename IN::raw_t rx[U];
#pragma unroll
        for (int u = 0; u < U; ++u) rx[u] = IN::load(xrow, c - u * NT);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float f[N], g[N];
          IN::cvt(rx[u], f);
#pragma unroll
          for (int j = 0; j < N; ++j) g[j] = mG * fast_exp2(fmaf(f[j], kLog2e, -c2));
          if (c - u * NT == ca) {
#pragma unroll
            for (int j = 0; j < N; ++j)
              if (j == ja) g[j] = ga;
          }
          Out<TG, N>::store(grow, c - u * NT, g);
        }
      }
      for (; c >= 0; c -= NT) {
        float f[N], g[N];
        IN::cvt(IN::load(xrow, c), f);
#pragma unroll
        for (int j = 0; j < N; ++j) g[j] = mG * fast_exp2(fmaf(f[j], kLog2e, -c2));
        if (c == ca) {
#pragma unroll
          for (int j = 0; j < N; ++j)
            if (j == ja) g[j] = ga;
        }
        Out<TG, N>::store(grow, c, g);
      }
    }
  }
}

// --- launch ------------------------------------------------------------------
template <typename TI, typename TG, int NT, int MODE, bool VEC>
static hipError_t launch_t(const RowArgs& a, hipStream_t stream) {
  constexpr int BLOCK = NT < 256 ? 256 : NT;
  constexpr int RPB = BLOCK / NT;
  constexpr int U = VEC ? 4 : 8;
  const int64_t blocks = (a.rows + RPB - 1) / RPB;
  hipLaunchKernelGGL((grpo_rows_kernel<TI, TG, NT, MODE, VEC, U>), dim3(unsigned(blocks)),
                     dim3(BLOCK), 0, stream, a);
  return hipGetLastError();
}

template <typename TI, typename TG, int MODE, bool VEC>
static hipError_t launch_nt(const RowArgs& a, int nt, hipStream_t s) {
  switch (nt) {
    case 64: return launch_t<TI, TG, 64, MODE, VEC>(a, s);
    case 256: return launch_t<TI, TG, 256, MODE, VEC>(a, s);
    case 512: return launch_t<TI, TG, 512, MODE, VEC>(a, s);
    case 1024: return launch_t<TI, TG, 1024, MODE, VEC>(a, s);
  }
  return hipErrorInvalidValue;
}

template <typename TI, typename TG, int MODE>
static hipError_t launch_vec(const RowArgs& a, const RowLaunch& l, hipStream_t s) {
  return l.vec ? launch_nt<TI, TG, MODE, true>(a, l.nt, s) : launch_nt<TI, TG, MODE, false>(a, l.nt, s);
}

template <int MODE>
static hipError_t launch_types(const RowArgs& a, const RowLaunch& l, hipStream_t s) {
  if (l.tin_bf16) {
    return l.tg_bf16 ? launch_vec<uint16_t, uint16_t, MODE>(a, l, s)
                     : launch_vec<uint16_t, float, MODE>(a, l, s);
  }
  return l.tg_bf16 ? launch_vec<float, uint16_t, MODE>(a, l, s)
                   : launch_vec<float, float, MODE>(a, l, s);
}

hipError_t launch_rows(const RowArgs& a, const RowLaunch& l, hipStream_t s) {
  switch (l.mode) {
    case kFused: return launch_types<kFused>(a, l, s);
    case kForward: return launch_types<kForward>(a, l, s);
    case kBackward: return launch_types<kBackward>(a, l, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace grpo
