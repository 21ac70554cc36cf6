// Resident-row variant of the fused vocabulary kernel.
//
// Same arithmetic as grpo_rows.hip (shared through grpo_rowcore.hpp), but the
// policy row is loaded once into registers and kept there: pass 1 consumes
// it for the log-sum-exp and the gradient pass recomputes the softmax from
// the registers instead of re-reading HBM.  Per active row that is
// V * (2 b_x + b_g) bytes instead of V * (3 b_x + b_g).  A block of NT
// threads owns one row; thread `lid` holds the 16-byte chunks
// lid, lid + NT, ..., lid + (K-1) NT.  With NT = 512 and K = 16 a block
// holds up to 16 x 16 B x 512 = 128 KB, a 65,536-entry bf16 row.
//
// The x chunks are issued first, interleaved with the first UY reference
// chunks; each reference slot is refilled as soon as it has been consumed,
// so the reference row streams through a short ring of registers while the
// held policy chunks arrive.

#include "grpo_rowcore.hpp"

namespace grpo {

// YFIRST: stream the whole reference row (UY chunks at a time) while the held
// policy chunks arrive, then run the policy log-sum-exp over the registers;
// otherwise walk both rows chunk by chunk with a UY-deep reference ring.
template <typename TI, typename TG, int NT, int K, int UY, bool YFIRST>
__global__ __launch_bounds__(NT) void grpo_rows_resident_kernel(RowArgs a) {
  typedef In<TI, true> IN;
  constexpr int N = IN::N;
  constexpr int NW = NT / kWave;
  static_assert(NW > 1 && NT % kWave == 0, "one block per row, whole waves");

  __shared__ Lse sh_lse[2][NW];
  __shared__ float sh_xa[2];
  __shared__ float sh_bcast[4];

  const int lid = threadIdx.x;
  const int64_t row = xcd_runs(blockIdx.x, gridDim.x, GRPO_XCD_ROWS);
  const int64_t V = a.V;
  const int64_t nvec = V / N;
  const int64_t tail0 = nvec * N;
  const void* xrow = static_cast<const char*>(a.x) + row * a.ld * int64_t(sizeof(TI));
  void* grow = static_cast<char*>(a.g) + row * a.ldg * int64_t(sizeof(TG));

  const bool active = a.mask == nullptr || a.mask[row] != 0;
  const int64_t aid = active ? load_action(a, row) : 0;
  const bool bad = active && (aid < 0 || aid >= V);
  // chunks of this thread: lid + k NT for k < kt (kt is 0 or K-1 or K)
  const int kt = lid < nvec ? int((nvec - 1 - lid) / NT) + 1 : 0;
  typedef typename IN::raw_t raw_t;
  const raw_t* xp = reinterpret_cast<const raw_t*>(xrow) + lid;
  if (!active || bad) {
    if (lid == 0) row_inactive(a, row, bad);
#pragma unroll
    for (int k = 0; k < K; ++k)
      if (k < kt) Out<TG, N>::zero(grow, lid + k * NT);
    for (int64_t v = tail0 + lid; v < V; v += NT) store_one(grow, v, 0.0f, (TG*)nullptr);
    return;
  }

  // the taken token sits in chunk ca = ka NT + la, value ja (uniform per row);
  // a token in the scalar tail has ka >= K and is handled there
  const int64_t ca = aid / N;
  const int ja = int(aid - ca * N);
  const int ka = int(ca / NT);
  const bool mine = lid == int(ca % NT);
  const bool has_ref = a.y != nullptr;
  const void* yrow = has_ref ? static_cast<const char*>(a.y) + row * a.ld * int64_t(sizeof(TI))
                             : nullptr;
  const raw_t* yp = reinterpret_cast<const raw_t*>(yrow) + lid;

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

  // ---- issue the loads -----------------------------------------------------
  raw_t xr[K];
  Lse sx = lse_init(), sy = lse_init();
  float xa = 0.0f, ya = 0.0f;
  bool own = false;
  if constexpr (YFIRST) {
#pragma unroll
  for (int k = 0; k < K; ++k)
    if (k < kt) xr[k] = xp[k * NT];
  if (has_ref) {
    // the reference row streams through UY-deep groups while x arrives
    for (int k0 = 0; k0 < kt; k0 += UY) {
      raw_t yb[UY];
#pragma unroll
      for (int u = 0; u < UY; ++u)
        if (k0 + u < kt) yb[u] = __builtin_nontemporal_load(yp + (k0 + u) * NT);
#pragma unroll
      for (int u = 0; u < UY; ++u) {
        if (k0 + u < kt) {
          float fy[N];
          IN::cvt(yb[u], fy);
          if (k0 + u == ka && mine) take_out(fy, ja, ya);
          lse_add(sy, fy);
        }
      }
    }
  }
#pragma unroll
  for (int k = 0; k < K; ++k) {
    if (k < kt) {
      float fx[N];
      IN::cvt(xr[k], fx);
      if (k == ka && mine) {
        own = true;
        take_out(fx, ja, xa);
      }
      lse_add(sx, fx);
    }
  }
  } else {
  raw_t yb[UY];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    if (k < kt) xr[k] = xp[k * NT];
    if (k < UY && has_ref && k < kt) yb[k] = __builtin_nontemporal_load(yp + k * NT);
  }

  // ---- pass 1 over the held chunks --------------------------------------------
#pragma unroll
  for (int k = 0; k < K; ++k) {
    if (k < kt) {
      float fx[N], fy[N];
      IN::cvt(xr[k], fx);
      if (has_ref) IN::cvt(yb[k % UY], fy);
      if (k == ka && mine) {
        own = true;
        take_out(fx, ja, xa);
        if (has_ref) take_out(fy, ja, ya);
      }
      lse_add(sx, fx);
      if (has_ref) lse_add(sy, fy);
    }
    if (k + UY < K && has_ref && k + UY < kt) yb[k % UY] = __builtin_nontemporal_load(yp + (k + UY) * NT);
  }
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

  // ---- reduce the row (fixed butterfly, then fixed wave order) ----------------
  sx = wave_lse<kWave>(sx);
  if (has_ref) sy = wave_lse<kWave>(sy);
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
    const RowGrad rg = row_epilogue(a, row, sx, sy, sh_xa[0], sh_xa[1], has_ref, old, gen, adv, wgt, gs,
                                    keep);
    sh_bcast[0] = rg.G;
    sh_bcast[1] = rg.c2;
    sh_bcast[2] = rg.omp;
  }
  __syncthreads();
  const float G = sh_bcast[0];
  const float c2 = sh_bcast[1];
  const float omp = sh_bcast[2];

  // ---- pass 2 from the registers ----------------------------------------------
  if (G == 0.0f) {
#pragma unroll
    for (int k = 0; k < K; ++k)
      if (k < kt) Out<TG, N>::zero(grow, lid + k * NT);
    for (int64_t v = tail0 + lid; v < V; v += NT) store_one(grow, v, 0.0f, (TG*)nullptr);
    return;
  }
  const float ga = G * omp;
  const float mG = -G;
  for (int64_t v = tail0 + lid; v < V; v += NT) {
    const float xv = load_one(xrow, v, (TI*)nullptr);
    store_one(grow, v, (v == aid) ? ga : mG * fast_exp2(fmaf(xv, kLog2e, -c2)), (TG*)nullptr);
  }
#pragma unroll
  for (int k = 0; k < K; ++k) {
    if (k < kt) {
      float f[N], g[N];
      IN::cvt(xr[k], f);
#pragma unroll
      for (int j = 0; j < N; ++j) g[j] = mG * fast_exp2(fmaf(f[j], kLog2e, -c2));
      Out<TG, N>::store(grow, lid + k * NT, g);
    }
  }
  // the taken token's element, over the value its chunk carried (same
  // thread, same address: the later store lands last)
  if (mine && ca < nvec) store_one(grow, aid, ga, (TG*)nullptr);
}

// Launch shapes, measured on MI355X (bf16 rows): how many rows are in flight
// per CU matters as much as how many waves.  Rows of up to 1,024 chunks:
// 256-thread blocks.  Rows of up to 4,096 chunks (64 KB of bf16): 512 threads
// x 8 chunks, held to two blocks per CU by a 64 KB LDS reservation each
// (measured at 4,000 chunks: two rows in flight per CU beat three or four by
// 3-4%; one 1024-thread row per CU is a third slower, its serial epilogue
// idles the CU).  Rows of up to 8,192 chunks (128 KB): 512 threads x 12 or 16
// chunks, two blocks per CU by their registers.  Longer rows take the
// streaming kernel: a 1024-thread resident block per CU leaves the policy
// row's log-sum-exp and the gradient exponentials without memory traffic to
// overlap (V = 100,000 and 128,256 with every row active: 13.6 and 15.7 ms
// against 11.5 and 13.8 for the streaming kernel).  Rows of 8 chunks or more
// per thread stream the reference row first, shorter ones walk both rows
// together.
constexpr unsigned kResCapLds = 65536;  // a third block would need more than the CU's 160 KB

template <typename TI, typename TG, int NT, int K>
static hipError_t launch_res(const RowArgs& a, unsigned lds, hipStream_t s) {
  constexpr bool kYFirst = K >= 8;
  constexpr int kUY = 4;  // reference chunks in flight per thread (8 measured no better at V = 32,000)
  hipLaunchKernelGGL((grpo_rows_resident_kernel<TI, TG, NT, K, kUY, kYFirst>), dim3(unsigned(a.rows)),
                     dim3(NT), lds, s, a);
  return hipGetLastError();
}

template <typename TI, typename TG>
static hipError_t launch_res_types(const RowArgs& a, int64_t nvec, hipStream_t s) {
  if (nvec <= 256 * 4) return launch_res<TI, TG, 256, 4>(a, 0, s);
  if (nvec <= 512 * 8) return launch_res<TI, TG, 512, 8>(a, kResCapLds, s);
  if (nvec <= 512 * 12) return launch_res<TI, TG, 512, 12>(a, 0, s);
  if (nvec <= 512 * 16) return launch_res<TI, TG, 512, 16>(a, 0, s);
  return hipErrorInvalidValue;
}

// esize: bytes per logit (2 or 4); a 16-byte chunk holds 16 / esize logits.
// Up to 8,192 chunks (128 KB; a 65,536-entry bf16 row) stay resident.
bool resident_fits(int64_t V, int esize) {
  const int64_t nvec = V / (16 / esize);
  return nvec <= int64_t(8192);
}

hipError_t launch_rows_resident(const RowArgs& a, const RowLaunch& l, hipStream_t s) {
  const int64_t nvec = a.V / (l.tin == GRPO_F32 ? 4 : 8);
  if (l.tin == GRPO_BF16)
    return l.tg == GRPO_BF16 ? launch_res_types<uint16_t, uint16_t>(a, nvec, s)
                             : launch_res_types<uint16_t, float>(a, nvec, s);
  if (l.tin == GRPO_F16)
    return l.tg == GRPO_F16 ? launch_res_types<_Float16, _Float16>(a, nvec, s)
                            : launch_res_types<_Float16, float>(a, nvec, s);
  return l.tg == GRPO_BF16 ? launch_res_types<float, uint16_t>(a, nvec, s)
                           : launch_res_types<float, float>(a, nvec, s);
}

}  // namespace grpo
