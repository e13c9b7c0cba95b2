// LayerNorm forward and backward (replicated, not partitioned).
//
// One wave owns one row and keeps it in registers (CPL 16-byte vectors per
// lane), so each row is read once: statistics by wave shuffles, no LDS and no
// barriers.  The gamma/beta gradients are deterministic column sums over
// row slabs (partials in the workspace, then a fixed-order final pass).
#include "common.h"
#include "slab_sum.h"

namespace mp {

int colsum(mp_dtype dt, int64_t rows, int64_t cols, const void* dy, float* out, void* ws, hipStream_t s);
size_t colsum_workspace(int64_t rows, int64_t cols);

// The 16-byte vector at element offset `elem` of a bf16 / fp32 array, raw.
template <bool BF16>
__device__ __forceinline__ uint4 ld_vec(const void* base, int64_t elem) {
  return *reinterpret_cast<const uint4*>(static_cast<const char*>(base) + elem * (BF16 ? 2 : 4));
}

// Every load of a row (and of gamma / beta) is issued unconditionally, at a
// clamped index, all before the first use, and kept raw (16 bytes) until
// used; values past the row's end are selected away.  With the loads inside
// a per-lane `if`, the compiler waited for each one before the next branch,
// so a wave made one memory round trip per 16-byte vector.
template <bool BF16, int CPL>
__global__ __launch_bounds__(256) void layernorm_fwd_kernel(int64_t T, int64_t K, const void* __restrict__ x,
                                                            const void* __restrict__ gamma,
                                                            const void* __restrict__ beta, float eps,
                                                            void* __restrict__ y, float* __restrict__ mean_out,
                                                            float* __restrict__ rstd_out) {
  using V = Vec16<BF16>;
  constexpr int E = V::N;
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= T) return;
  const int64_t nvec = K / E;
  uint4 rx[CPL], rg[CPL], rb[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int64_t vi = lane + 64 * c, vs = vi < nvec ? vi : 0;
    rx[c] = ld_vec<BF16>(x, row * K + vs * E);
    rg[c] = ld_vec<BF16>(gamma, vs * E);
    rb[c] = ld_vec<BF16>(beta, vs * E);
  }
  float sum = 0.0f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const bool ok = lane + 64 * c < nvec;
    float f[E];
    V::unpack(rx[c], f);
#pragma unroll
    for (int i = 0; i < E; ++i) sum += ok ? f[i] : 0.0f;
  }
  const float mean = wave_sum(sum) / static_cast<float>(K);
  float sq = 0.0f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const bool ok = lane + 64 * c < nvec;
    float f[E];
    V::unpack(rx[c], f);
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const float dlt = ok ? f[i] - mean : 0.0f;
      sq += dlt * dlt;
    }
  }
  const float rstd = rsqrtf(wave_sum(sq) / static_cast<float>(K) + eps);
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int64_t vi = lane + 64 * c;
    float f[E], g[E], b[E], o[E];
    V::unpack(rx[c], f);
    V::unpack(rg[c], g);
    V::unpack(rb[c], b);
#pragma unroll
    for (int i = 0; i < E; ++i) o[i] = (f[i] - mean) * rstd * g[i] + b[i];
    if (vi < nvec) V::store(y, row * K + vi * E, o);
  }
  if (lane == 0) {
    if (mean_out) mean_out[row] = mean;
    if (rstd_out) rstd_out[row] = rstd;
  }
}

// dx = dres + rstd * (g - mean(g) - xhat * mean(g * xhat)), g = dy * gamma.
// Loads at clamped indices, with no per-lane branch around them, as in the
// forward.
template <bool BF16, int CPL>
__global__ __launch_bounds__(256) void layernorm_bwd_dx_kernel(int64_t T, int64_t K, const void* __restrict__ x,
                                                               const void* __restrict__ gamma,
                                                               const float* __restrict__ mean_in,
                                                               const float* __restrict__ rstd_in,
                                                               const void* __restrict__ dy,
                                                               const void* __restrict__ dres, void* __restrict__ dx) {
  using V = Vec16<BF16>;
  constexpr int E = V::N;
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= T) return;
  const int64_t nvec = K / E;
  const float mean = mean_in[row];
  const float rstd = rstd_in[row];
  float xh[CPL][E], g[CPL][E];
  float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int64_t vi = lane + 64 * c, vs = vi < nvec ? vi : 0;
    const bool ok = vi < nvec;
    float gm[E];
    V::load(x, row * K + vs * E, xh[c]);
    V::load(dy, row * K + vs * E, g[c]);
    V::load(gamma, vs * E, gm);
#pragma unroll
    for (int i = 0; i < E; ++i) {
      xh[c][i] = (xh[c][i] - mean) * rstd;
      g[c][i] = ok ? g[c][i] * gm[i] : 0.0f;
      s1 += g[c][i];
      s2 += g[c][i] * xh[c][i];
    }
  }
  const float inv_k = 1.0f / static_cast<float>(K);
  const float m1 = wave_sum(s1) * inv_k;
  const float m2 = wave_sum(s2) * inv_k;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int64_t vi = lane + 64 * c;
    float o[E], r[E];
    if (dres != nullptr) {
      V::load(dres, row * K + (vi < nvec ? vi : 0) * E, r);
    } else {
#pragma unroll
      for (int i = 0; i < E; ++i) r[i] = 0.0f;
    }
#pragma unroll
    for (int i = 0; i < E; ++i) o[i] = r[i] + rstd * (g[c][i] - m1 - xh[c][i] * m2);
    if (vi < nvec) V::store(dx, row * K + vi * E, o);
  }
}

// Partial sums of dy * xhat (dgamma) and dy (dbeta) over row slabs:
// partial[slab, 0:K] and partial[slab, K:2K].  Same block shape as colsum.
template <bool BF16>
__global__ __launch_bounds__(256) void layernorm_bwd_param_kernel(int64_t T, int64_t K, const void* __restrict__ x,
                                                                  const float* __restrict__ mean_in,
                                                                  const float* __restrict__ rstd_in,
                                                                  const void* __restrict__ dy, int64_t slab_rows,
                                                                  float* __restrict__ partial) {
  using V = Vec16<BF16>;
  constexpr int E = V::N;
  __shared__ float red[8][32 * E * 2];
  const int cv = threadIdx.x & 31;
  const int rl = threadIdx.x >> 5;
  const int64_t c0 = (static_cast<int64_t>(blockIdx.x) * 32 + cv) * E;
  const int64_t r_begin = static_cast<int64_t>(blockIdx.y) * slab_rows;
  const int64_t r_end = r_begin + slab_rows < T ? r_begin + slab_rows : T;
  float ag[E], ab[E];
#pragma unroll
  for (int i = 0; i < E; ++i) ag[i] = ab[i] = 0.0f;
  if (c0 < K) {
    float xv[E], dv[E];
    for (int64_t r = r_begin + rl; r < r_end; r += 8) {
      V::load(x, r * K + c0, xv);
      V::load(dy, r * K + c0, dv);
      const float mu = mean_in[r], rs = rstd_in[r];
#pragma unroll
      for (int i = 0; i < E; ++i) {
        ag[i] += dv[i] * ((xv[i] - mu) * rs);
        ab[i] += dv[i];
      }
    }
  }
#pragma unroll
  for (int i = 0; i < E; ++i) {
    red[rl][cv * E + i] = ag[i];
    red[rl][32 * E + cv * E + i] = ab[i];
  }
  __syncthreads();
  if (rl == 0 && c0 < K) {
    float* pg = partial + static_cast<int64_t>(blockIdx.y) * 2 * K;
#pragma unroll
    for (int i = 0; i < E; ++i) {
      float tg = red[0][cv * E + i], tb = red[0][32 * E + cv * E + i];
#pragma unroll
      for (int l = 1; l < 8; ++l) {
        tg += red[l][cv * E + i];
        tb += red[l][32 * E + cv * E + i];
      }
      pg[c0 + i] = tg;
      pg[K + c0 + i] = tb;
    }
  }
}

// Sums the slab partials of dgamma (columns [0, K)), dbeta ([K, 2K)) and,
// with partial rows 3K wide, a third vector ([2K, 3K)) in the fixed order of
// slab_sum.h.
__global__ __launch_bounds__(SLAB_THREADS) void layernorm_param_final_kernel(const float* __restrict__ partial,
                                                                             int64_t slabs, int64_t K, int64_t w,
                                                                             float* __restrict__ dgamma,
                                                                             float* __restrict__ dbeta,
                                                                             float* __restrict__ dthird) {
  __shared__ float red[SLAB_GROUPS][SLAB_COLS];
  const int64_t c = static_cast<int64_t>(blockIdx.x) * SLAB_COLS + threadIdx.x % SLAB_COLS;
  const float v = slab_column_sum(partial, slabs, w, c, red);
  if (threadIdx.x >= SLAB_COLS || c >= w) return;
  if (c < K) {
    if (dgamma) dgamma[c] = v;
  } else if (c < 2 * K) {
    if (dbeta) dbeta[c - K] = v;
  } else if (dthird) {
    dthird[c - 2 * K] = v;
  }
}

// dgamma[c] = sum_s partial[s, c], dbeta[c] = sum_s partial[s, K + c] in a
// fixed order (shared with the fused reduce + LayerNorm backward); with
// `dthird`, partial rows are 3K wide and dthird[c] = sum_s partial[s, 2K + c].
void layernorm_param_final(const float* partial, int64_t slabs, int64_t K, float* dgamma, float* dbeta,
                           hipStream_t s, float* dthird = nullptr) {
  const int64_t w = (dthird != nullptr ? 3 : 2) * K;
  layernorm_param_final_kernel<<<static_cast<unsigned>(ceil_div(w, SLAB_COLS)), SLAB_THREADS, 0, s>>>(
      partial, slabs, K, w, dgamma, dbeta, dthird);
}

static void ln_slabs(int64_t T, int64_t& slab_rows, int64_t& slabs) {
  slab_rows = T / 256;
  if (slab_rows < 64) slab_rows = 64;
  slab_rows = align_up(static_cast<size_t>(slab_rows), 8);
  slabs = T > 0 ? ceil_div(T, slab_rows) : 0;
}

template <bool BF16, template <bool, int> class Launcher, typename... Args>
static int dispatch_cpl(int64_t nvec, Args... args) {
  const int64_t cpl = ceil_div(nvec, 64);
  if (cpl <= 1) return Launcher<BF16, 1>::run(args...);
  if (cpl <= 2) return Launcher<BF16, 2>::run(args...);
  if (cpl <= 3) return Launcher<BF16, 3>::run(args...);
  if (cpl <= 4) return Launcher<BF16, 4>::run(args...);
  if (cpl <= 6) return Launcher<BF16, 6>::run(args...);
  if (cpl <= 8) return Launcher<BF16, 8>::run(args...);
  if (cpl <= 12) return Launcher<BF16, 12>::run(args...);
  return Launcher<BF16, 16>::run(args...);
}

template <bool BF16, int CPL>
struct LnFwd {
  static int run(int64_t T, int64_t K, const void* x, const void* g, const void* b, float eps, void* y, float* mean,
                 float* rstd, hipStream_t s) {
    layernorm_fwd_kernel<BF16, CPL><<<static_cast<unsigned>(ceil_div(T, 4)), 256, 0, s>>>(T, K, x, g, b, eps, y, mean,
                                                                                         rstd);
    return check_launch("mp_layernorm");
  }
};

template <bool BF16, int CPL>
struct LnBwd {
  static int run(int64_t T, int64_t K, const void* x, const void* g, const float* mean, const float* rstd,
                 const void* dy, const void* dres, void* dx, hipStream_t s) {
    layernorm_bwd_dx_kernel<BF16, CPL><<<static_cast<unsigned>(ceil_div(T, 4)), 256, 0, s>>>(T, K, x, g, mean, rstd,
                                                                                            dy, dres, dx);
    return check_launch("mp_layernorm_bwd");
  }
};

}  // namespace mp

using namespace mp;

extern "C" int mp_layernorm(mp_dtype dtype, int64_t T, int64_t K, const void* x, const void* gamma, const void* beta,
                            float eps, void* y, float* mean, float* rstd, hipStream_t s) {
  MP_REQUIRE(dtype_ok(dtype), MP_ERR_DTYPE, "mp_layernorm: bad dtype");
  MP_REQUIRE(T >= 0 && K > 0 && K % vec_elems(dtype) == 0, MP_ERR_SHAPE, "mp_layernorm: bad shape");
  MP_REQUIRE(K / vec_elems(dtype) <= 64 * 16, MP_ERR_UNSUPPORTED, "mp_layernorm: K=%lld too large (max %lld)",
             (long long)K, (long long)(64 * 16 * vec_elems(dtype)));
  MP_REQUIRE(eps > 0.0f, MP_ERR_ARG, "mp_layernorm: eps must be positive");
  MP_REQUIRE_PTR(x);
  MP_REQUIRE_PTR(gamma);
  MP_REQUIRE_PTR(beta);
  MP_REQUIRE_PTR(y);
  MP_REQUIRE_ALIGN(x);
  MP_REQUIRE_ALIGN(gamma);
  MP_REQUIRE_ALIGN(beta);
  MP_REQUIRE_ALIGN(y);
  if (T == 0) return MP_OK;
  const int64_t nvec = K / vec_elems(dtype);
  if (dtype == MP_BF16) return dispatch_cpl<true, LnFwd>(nvec, T, K, x, gamma, beta, eps, y, mean, rstd, s);
  return dispatch_cpl<false, LnFwd>(nvec, T, K, x, gamma, beta, eps, y, mean, rstd, s);
}

extern "C" size_t mp_layernorm_bwd_workspace(int64_t T, int64_t K) {
  if (T < 0 || K <= 0) return 0;
  int64_t slab_rows, slabs;
  ln_slabs(T, slab_rows, slabs);
  return align_up(static_cast<size_t>(slabs * 2 * K) * sizeof(float), 256);
}

extern "C" int mp_layernorm_bwd(mp_dtype dtype, int64_t T, int64_t K, const void* x, const void* gamma,
                                const float* mean, const float* rstd, const void* dy, const void* dres, void* dx,
                                float* dgamma, float* dbeta, void* ws, size_t ws_bytes, hipStream_t s) {
  MP_REQUIRE(dtype_ok(dtype), MP_ERR_DTYPE, "mp_layernorm_bwd: bad dtype");
  MP_REQUIRE(T >= 0 && K > 0 && K % vec_elems(dtype) == 0, MP_ERR_SHAPE, "mp_layernorm_bwd: bad shape");
  MP_REQUIRE(K / vec_elems(dtype) <= 64 * 16, MP_ERR_UNSUPPORTED, "mp_layernorm_bwd: K too large");
  MP_REQUIRE_PTR(x);
  MP_REQUIRE_PTR(gamma);
  MP_REQUIRE_PTR(mean);
  MP_REQUIRE_PTR(rstd);
  MP_REQUIRE_PTR(dy);
  MP_REQUIRE_PTR(dx);
  MP_REQUIRE_ALIGN(x);
  MP_REQUIRE_ALIGN(gamma);
  MP_REQUIRE_ALIGN(dy);
  MP_REQUIRE_ALIGN(dx);
  MP_REQUIRE_OPT_ALIGN(dres);
  const bool params = dgamma != nullptr || dbeta != nullptr;
  const size_t need = params ? mp_layernorm_bwd_workspace(T, K) : 0;
  MP_REQUIRE(need == 0 || (ws != nullptr && ws_bytes >= need), MP_ERR_WORKSPACE,
             "mp_layernorm_bwd: workspace needs %zu bytes", need);
  const int64_t nvec = K / vec_elems(dtype);
  if (T > 0) {
    const int rc = dtype == MP_BF16 ? dispatch_cpl<true, LnBwd>(nvec, T, K, x, gamma, mean, rstd, dy, dres, dx, s)
                                    : dispatch_cpl<false, LnBwd>(nvec, T, K, x, gamma, mean, rstd, dy, dres, dx, s);
    if (rc) return rc;
  }
  if (!params) return MP_OK;
  int64_t slab_rows, slabs;
  ln_slabs(T, slab_rows, slabs);
  if (slabs > 0) {
    const dim3 grid(static_cast<unsigned>(ceil_div(nvec, 32)), static_cast<unsigned>(slabs));
    if (dtype == MP_BF16)
      layernorm_bwd_param_kernel<true><<<grid, 256, 0, s>>>(T, K, x, mean, rstd, dy, slab_rows, static_cast<float*>(ws));
    else
      layernorm_bwd_param_kernel<false><<<grid, 256, 0, s>>>(T, K, x, mean, rstd, dy, slab_rows, static_cast<float*>(ws));
  }
  layernorm_param_final(static_cast<const float*>(ws), slabs, K, dgamma, dbeta, s);
  return check_launch("mp_layernorm_bwd");
}
