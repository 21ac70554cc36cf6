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
// first ones re-read, while they are still in L2 / the memory-side cache;
// with a whole block per row (1024 threads, one block per CU) the row's first
// GRPO_HOLD_CHUNKS x 1024 chunks, re-read last, are kept in LDS instead.
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

#include "grpo_rowcore.hpp"

// Tuning knobs (compile-time; the defaults are the measured best).
#ifndef GRPO_PASS2_REVERSE
#define GRPO_PASS2_REVERSE 1   // gradient pass walks each thread's chunks backwards
#endif
#ifndef GRPO_UNROLL
#define GRPO_UNROLL 6          // 16-byte chunks of x (and of y) in flight per thread: at 8
                               // the fused 1024-thread kernel spilled (128 VGPRs) and the
                               // 256-thread forward-only kernel fit three waves per SIMD
                               // instead of four (V = 151,936: 11.87 -> 11.60 ms fused;
                               // GSPO at V = 32,000: 1.84 -> 1.74 ms)
#endif
#ifndef GRPO_HOLD_CHUNKS
#define GRPO_HOLD_CHUNKS 8     // fused 1024-thread rows: chunks per thread kept in LDS from
                               // pass 1 to pass 2, the row's first ones, which pass 2 re-reads
                               // last (128 KB per block; none -> 6 took V = 151,936 from 11.69
                               // to 11.04 ms; with the XCD-aware row order 8 beats 6 by
                               // 0.3-0.8%: 10.47 -> 10.44 ms, CSR V = 128,256 8.72 -> 8.67 ms)
#endif
#ifndef GRPO_Y_NONTEMPORAL
#define GRPO_Y_NONTEMPORAL 1   // the reference row is read once: non-temporal loads
#endif
#ifndef GRPO_PASS1_PIPELINE
#define GRPO_PASS1_PIPELINE 1  // pass 1 in two register stages: the next stage's loads are
                               // in flight while the current one is summed
#endif
#ifndef GRPO_LOAD_PRIO
#define GRPO_LOAD_PRIO 0       // wave priority while a stage's loads are issued (s_setprio)
#endif

namespace grpo {

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
  // the row's first kHoldN chunks stay in LDS between the passes (thread lid
  // keeps its own chunks lid + k NT at index lid + k NT, so no barrier)
  constexpr int64_t kHoldN = (MODE == kFused && VEC && NT == 1024) ? int64_t(GRPO_HOLD_CHUNKS) * NT : 0;
  extern __shared__ __align__(16) unsigned char grpo_rows_hold[];
  typename IN::raw_t* const hold = reinterpret_cast<typename IN::raw_t*>(grpo_rows_hold);

  const int lid = threadIdx.x % NT;
  const int64_t row = int64_t(xcd_runs(blockIdx.x, gridDim.x, GRPO_XCD_ROWS)) * RPB + threadIdx.x / NT;
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
    if (active) aid = load_action(a, row);
    const bool bad = active && (aid < 0 || aid >= V);
    if (!active || bad) {
      if (lid == 0) row_inactive(a, row, bad);
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
    float old = 0.0f, gen = 0.0f, adv = 0.0f, wgt = 0.0f, gs = 1.0f, keep = 1.0f;
    if (lid == 0) {
      old = a.old[row];
      if (a.gen) gen = a.gen[row];
      const int64_t i = row / a.T;
      adv = a.adv_tok ? a.adv_tok[row] : a.A[i];
      wgt = float(a.w[i]);
      if (a.grad_scale) gs = *a.grad_scale;
      if (a.iwseq) keep = float(a.iwseq[i]);
    }

    // ---- pass 1 ----------------------------------------------------------
    Lse sx = lse_init(), sy = lse_init();
    float xa = 0.0f, ya = 0.0f;
    bool own = false;
    typedef typename IN::raw_t raw_t;
    // one chunk of x (and y) into the running sums; the owner of the taken
    // token's chunk lifts it out first
    auto consume = [&](const raw_t* px, const raw_t* py, int u, int64_t cc) {
      if constexpr (kHoldN > 0) {
        if (cc < kHoldN) hold[cc] = px[u];
      }
      float fx[N], fy[N];
      IN::cvt(px[u], fx);
      if (has_ref) IN::cvt(py[u], fy);
      if (cc == ca) {
        own = true;
        take_out(fx, ja, xa);
        if (has_ref) take_out(fy, ja, ya);
      }
      lse_add(sx, fx);
      if (has_ref) lse_add(sy, fy);
    };
    int64_t c = lid;
#if GRPO_PASS1_PIPELINE
    // stages of P chunks each for x and y, in two register sets: while one
    // stage is summed the next one's loads are in flight
    constexpr int P = U / 2;
    if (c + (P - 1) * NT < nvec) {
      raw_t ax[P], ay[P], bx[P], by[P];
      auto load_stage = [&](raw_t* dx, raw_t* dy, int64_t c0) {
        if constexpr (GRPO_LOAD_PRIO > 0) __builtin_amdgcn_s_setprio(GRPO_LOAD_PRIO);
#pragma unroll
        for (int u = 0; u < P; ++u) dx[u] = IN::load(xrow, c0 + u * NT);
        if (has_ref) {
#pragma unroll
          for (int u = 0; u < P; ++u)
            dy[u] = GRPO_Y_NONTEMPORAL ? IN::load_nt(yrow, c0 + u * NT) : IN::load(yrow, c0 + u * NT);
        }
        if constexpr (GRPO_LOAD_PRIO > 0) __builtin_amdgcn_s_setprio(0);
      };
      auto sum_stage = [&](const raw_t* dx, const raw_t* dy, int64_t c0) {
#pragma unroll
        for (int u = 0; u < P; ++u) consume(dx, dy, u, c0 + u * NT);
      };
      load_stage(ax, ay, c);
      while (true) {
        int64_t cn = c + P * NT;
        if (cn + (P - 1) * NT >= nvec) {
          sum_stage(ax, ay, c);
          c = cn;
          break;
        }
        load_stage(bx, by, cn);
        sum_stage(ax, ay, c);
        c = cn;
        cn = c + P * NT;
        if (cn + (P - 1) * NT >= nvec) {
          sum_stage(bx, by, c);
          c = cn;
          break;
        }
        load_stage(ax, ay, cn);
        sum_stage(bx, by, c);
        c = cn;
      }
    }
#else
    for (; c + (U - 1) * NT < nvec; c += U * NT) {
      raw_t rx[U], ry[U];
#pragma unroll
      for (int u = 0; u < U; ++u) rx[u] = IN::load(xrow, c + u * NT);
      if (has_ref) {
#pragma unroll
        for (int u = 0; u < U; ++u)
          ry[u] = GRPO_Y_NONTEMPORAL ? IN::load_nt(yrow, c + u * NT) : IN::load(yrow, c + u * NT);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) consume(rx, ry, u, c + u * NT);
    }
#endif
    for (; c < nvec; c += NT) {
      float fx[N], fy[N];
      const raw_t rxc = IN::load(xrow, c);
      if constexpr (kHoldN > 0) {
        if (c < kHoldN) hold[c] = rxc;
      }
      IN::cvt(rxc, fx);
      if (has_ref) IN::cvt(GRPO_Y_NONTEMPORAL ? IN::load_nt(yrow, c) : IN::load(yrow, c), fy);
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
      xa = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(xa), owner));
      ya = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ya), owner));
    }

    // ---- per-token epilogue -------------------------------------------------
    if (lid == 0) {
      const RowGrad rg = row_epilogue(a, row, sx, sy, xa, ya, has_ref, old, gen, adv, wgt, gs,
                                      keep);
      G = rg.G;
      c2 = rg.c2;
      omp = rg.omp;
      if constexpr (!kPass2) a.stash[row] = RowStash{G, c2, omp, 1.0f};
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
      G = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(G), 0));
      c2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(c2), 0));
      omp = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(omp), 0));
    }
  } else {
    // backward only: per-row state from the forward pass, plus the policy
    // part of the sequence-level losses (0 for the token-level ones)
    const RowStash st = a.stash[row];
    G = st.act != 0.0f ? (st.G + a.useq[row / a.T]) * (a.grad_scale ? *a.grad_scale : 1.0f)
                       : 0.0f;
    c2 = st.c;
    omp = st.omp;
    if (G != 0.0f) aid = load_action(a, row);
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
      // this thread's chunks are lid, lid + NT, ..., last
      const int64_t last = lid + ((nvec - 1 - lid) / NT) * NT;
      constexpr int64_t step = GRPO_PASS2_REVERSE ? -int64_t(NT) : int64_t(NT);
      int64_t c = GRPO_PASS2_REVERSE ? last : lid;
      auto more = [&](int64_t cc) { return GRPO_PASS2_REVERSE ? cc >= 0 : cc <= last; };
      for (; more(c + (U - 1) * step); c += U * step) {
        typename IN::raw_t rx[U];
        if constexpr (GRPO_LOAD_PRIO > 0) __builtin_amdgcn_s_setprio(GRPO_LOAD_PRIO);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t cc = c + u * step;
          if constexpr (kHoldN > 0) {
            if (cc < kHoldN)
              rx[u] = hold[cc];
            else
              rx[u] = IN::load(xrow, cc);
          } else {
            rx[u] = IN::load(xrow, cc);
          }
        }
        if constexpr (GRPO_LOAD_PRIO > 0) __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float f[N], g[N];
          IN::cvt(rx[u], f);
#pragma unroll
          for (int j = 0; j < N; ++j) g[j] = mG * fast_exp2(fmaf(f[j], kLog2e, -c2));
          Out<TG, N>::store(grow, c + u * step, g);
        }
      }
      for (; more(c); c += step) {
        float f[N], g[N];
        typename IN::raw_t r;
        if constexpr (kHoldN > 0) {
          if (c < kHoldN)
            r = hold[c];
          else
            r = IN::load(xrow, c);
        } else {
          r = IN::load(xrow, c);
        }
        IN::cvt(r, f);
#pragma unroll
        for (int j = 0; j < N; ++j) g[j] = mG * fast_exp2(fmaf(f[j], kLog2e, -c2));
        Out<TG, N>::store(grow, c, g);
      }
      // the taken token's element: its chunk went out with -G p_a there; the
      // owner overwrites that one element (a later store of the same thread
      // to the same address lands after the first)
      if (ca < nvec && lid == ca % NT) store_one(grow, aid, ga, (TG*)nullptr);
    }
  }
}

// --- gradient-only pass as a flat map ------------------------------------------
// The gradient pass needs no reduction: g_v = G (onehot(a)_v - p_v) with the
// row's G, c and 1 - p_a from the forward pass's stash.  Here every block of
// kFlatThreads threads writes kFlatThreads 16-byte chunks (4 KB) of one row
// (row = block / blocks per row), so a launch is millions of short blocks
// with a small address footprint each.  Measured on MI355X at V = 151,936
// bf16: the gradient pass takes 6.0 ms instead of 7.3 (a row-per-block walk
// over the same bytes).  Two chunks per thread measured slower, and so did
// loading the policy chunk before the row's G is known once a third of the
// rows are masked (their policy rows are never read).  The values are those
// of grpo_rows_kernel's pass 2, bit for bit (the same expressions per
// element).  Rows up to 64 KB keep the row kernel at 1024 threads: there the
// two measured alike.
constexpr int kFlatThreads = 256;
constexpr int kFlatChunks = 1;
constexpr int64_t kFlatMinRowBytes = 65536;  // rows longer than this take the flat map

template <typename TI, typename TG>
__global__ __launch_bounds__(kFlatThreads) void grpo_grad_flat_kernel(RowArgs a, uint32_t bpr) {
  typedef In<TI, true> IN;
  constexpr int N = IN::N;
  typedef typename IN::raw_t raw_t;
  const uint32_t b = xcd_runs(blockIdx.x, gridDim.x, GRPO_XCD_FLAT);
  const uint32_t row32 = b / bpr;
  const int64_t row = row32;
  const uint32_t seg = b - row32 * bpr;
  const int64_t V = a.V;
  const int64_t nvec = V / N;
  const int64_t tail0 = nvec * N;
  const void* xrow = static_cast<const char*>(a.x) + row * a.ld * int64_t(sizeof(TI));
  void* grow = static_cast<char*>(a.g) + row * a.ldg * int64_t(sizeof(TG));
  const int64_t c0 = int64_t(seg) * (kFlatThreads * kFlatChunks) + threadIdx.x;
  const bool last = seg == bpr - 1;
  const RowStash st = a.stash[row];
  const float G = st.act != 0.0f
                      ? (st.G + a.useq[row / a.T]) * (a.grad_scale ? *a.grad_scale : 1.0f)
                      : 0.0f;
  if (G == 0.0f) {
#pragma unroll
    for (int u = 0; u < kFlatChunks; ++u)
      if (c0 + u * kFlatThreads < nvec) Out<TG, N>::zero(grow, c0 + u * kFlatThreads);
    if (last)
      for (int64_t v = tail0 + threadIdx.x; v < V; v += kFlatThreads) store_one(grow, v, 0.0f, (TG*)nullptr);
    return;
  }
  raw_t rx[kFlatChunks];
#pragma unroll
  for (int u = 0; u < kFlatChunks; ++u)
    if (c0 + u * kFlatThreads < nvec) rx[u] = IN::load(xrow, c0 + u * kFlatThreads);
  const int64_t aid = load_action(a, row);
  const int64_t ca = aid / N;
  const int ja = int(aid - ca * N);
  const float c2 = st.c;
  const float ga = G * st.omp;
  const float mG = -G;
#pragma unroll
  for (int u = 0; u < kFlatChunks; ++u) {
    const int64_t c = c0 + u * kFlatThreads;
    if (c < nvec) {
      float f[N], g[N];
      IN::cvt(rx[u], f);
#pragma unroll
      for (int j = 0; j < N; ++j) g[j] = mG * fast_exp2(fmaf(f[j], kLog2e, -c2));
      Out<TG, N>::store(grow, c, g);
      // the taken token's element, over the value just stored (same thread,
      // same address: the later store lands last)
      if (c == ca) store_one(grow, aid, ga, (TG*)nullptr);
    }
  }
  if (last) {
    for (int64_t v = tail0 + threadIdx.x; v < V; v += kFlatThreads) {
      const float xv = load_one(xrow, v, (TI*)nullptr);
      store_one(grow, v, (v == aid) ? ga : mG * fast_exp2(fmaf(xv, kLog2e, -c2)), (TG*)nullptr);
    }
  }
}

// Blocks per row of the flat gradient pass, or 0 when the grid would not fit
// a 32-bit block index (such launches use the row kernel).
static uint32_t flat_blocks_per_row(const RowArgs& a, int n) {
  const int64_t nvec = a.V / n;
  const int64_t per = int64_t(kFlatThreads) * kFlatChunks;
  const int64_t bpr = nvec > 0 ? (nvec + per - 1) / per : 1;
  if (a.rows <= 0 || bpr * a.rows > int64_t(INT32_MAX)) return 0;
  return uint32_t(bpr);
}

template <typename TI, typename TG>
static hipError_t launch_flat(const RowArgs& a, uint32_t bpr, hipStream_t s) {
  hipLaunchKernelGGL((grpo_grad_flat_kernel<TI, TG>), dim3(unsigned(int64_t(bpr) * a.rows)),
                     dim3(kFlatThreads), 0, s, a, bpr);
  return hipGetLastError();
}

// The gradient-only pass over 16-byte-aligned rows above kFlatMinRowBytes:
// the flat map.  Returns hipErrorNotSupported when it does not apply (the
// caller runs the row kernel).
static hipError_t launch_grad_flat(const RowArgs& a, const RowLaunch& l, hipStream_t s) {
  const int n = l.tin == GRPO_F32 ? 4 : 8;
  if (!l.vec || a.rows <= 0 || a.V * int64_t(16 / n) <= kFlatMinRowBytes) return hipErrorNotSupported;
  const uint32_t bpr = flat_blocks_per_row(a, n);
  if (bpr == 0) return hipErrorNotSupported;
  if (l.tin == GRPO_BF16)
    return l.tg == GRPO_BF16 ? launch_flat<uint16_t, uint16_t>(a, bpr, s)
                             : launch_flat<uint16_t, float>(a, bpr, s);
  if (l.tin == GRPO_F16)
    return l.tg == GRPO_F16 ? launch_flat<_Float16, _Float16>(a, bpr, s)
                            : launch_flat<_Float16, float>(a, bpr, s);
  return l.tg == GRPO_BF16 ? launch_flat<float, uint16_t>(a, bpr, s)
                           : launch_flat<float, float>(a, bpr, s);
}

// --- launch ------------------------------------------------------------------
template <typename TI, typename TG, int NT, int MODE, bool VEC>
static hipError_t launch_t(const RowArgs& a, hipStream_t stream) {
  constexpr int BLOCK = NT < 256 ? 256 : NT;
  constexpr int RPB = BLOCK / NT;
  constexpr int U = VEC ? GRPO_UNROLL : 8;
  const int64_t blocks = (a.rows + RPB - 1) / RPB;
  constexpr size_t kHoldBytes = (MODE == kFused && VEC && NT == 1024) ? size_t(GRPO_HOLD_CHUNKS) * NT * 16 : 0;
  hipLaunchKernelGGL((grpo_rows_kernel<TI, TG, NT, MODE, VEC, U>), dim3(unsigned(blocks)),
                     dim3(BLOCK), kHoldBytes, stream, a);
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

// Storage pairs (logits -> gradient): f32 -> f32 | bf16, bf16 -> bf16 | f32,
// f16 -> f16 | f32 (the entry points reject the others).
template <int MODE>
static hipError_t launch_types(const RowArgs& a, const RowLaunch& l, hipStream_t s) {
  if (l.tin == GRPO_BF16)
    return l.tg == GRPO_BF16 ? launch_vec<uint16_t, uint16_t, MODE>(a, l, s)
                             : launch_vec<uint16_t, float, MODE>(a, l, s);
  if (l.tin == GRPO_F16)
    return l.tg == GRPO_F16 ? launch_vec<_Float16, _Float16, MODE>(a, l, s)
                            : launch_vec<_Float16, float, MODE>(a, l, s);
  return l.tg == GRPO_BF16 ? launch_vec<float, uint16_t, MODE>(a, l, s)
                           : launch_vec<float, float, MODE>(a, l, s);
}

hipError_t launch_rows_resident(const RowArgs& a, const RowLaunch& l, hipStream_t s);

hipError_t launch_rows(const RowArgs& a, const RowLaunch& l, hipStream_t s) {
  if (l.resident && l.mode == kFused && l.vec) return launch_rows_resident(a, l, s);
  switch (l.mode) {
    case kFused: return launch_types<kFused>(a, l, s);
    case kForward: return launch_types<kForward>(a, l, s);
    case kBackward:
      {
        const hipError_t e = launch_grad_flat(a, l, s);
        if (e != hipErrorNotSupported) return e;
      }
      return launch_types<kBackward>(a, l, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace grpo
