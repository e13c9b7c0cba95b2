// Shard reduce fused with the LayerNorm that follows it.
//
// In the layer each all-reduce (here: the local N-way shard reduce) feeds a
// LayerNorm: forward, H1 = X + Drop(sum_j P_j + b_o) is normalised by LN2;
// backward, the summed input gradient of a block goes straight into that
// block's LayerNorm backward.  Doing both in one pass per row keeps the sum
// in registers: the forward writes H1 (still needed as the residual and for
// the LN2 backward) and LN2(H1) without re-reading H1; the backward never
// writes the summed gradient at all.
//
// A block walks a few rows; thread t owns the 16-byte vector t of each row
// (one vector per thread keeps registers low and many waves in flight), and
// the row statistics are block sums in a fixed order.  The sum over the
// partials runs in the fixed order j = 0..N-1, exactly as in the unfused
// reduce, and the statistics are taken from the stored (rounded) H1.  The
// backward's dgamma/dbeta are per-block partial column sums over a fixed
// range of rows, summed in a fixed order by the final pass shared with
// mp_layernorm_bwd.
#include "common.h"

namespace mp {

void layernorm_param_final(const float* partial, int64_t slabs, int64_t K, float* dgamma, float* dbeta,
                           hipStream_t s, float* dthird = nullptr);

struct PartPtrs {
  const void* p[MP_MAX_SHARDS];
};

__device__ __forceinline__ float round_to_bf16(float x) {
  return __uint_as_float(static_cast<uint32_t>(f32_to_bf16(x)) << 16);
}

// Raw 16-byte vector at element `elem`, and its values as floats.
template <bool BF16>
__device__ __forceinline__ uint4 ld_raw(const void* base, int64_t elem) {
  return *reinterpret_cast<const uint4*>(static_cast<const char*>(base) + elem * (BF16 ? 2 : 4));
}
// Shard partials are read exactly once: streaming loads keep them from
// displacing the operands of the GEMM that runs next.
template <bool BF16>
__device__ __forceinline__ uint4 ld_part(const void* base, int64_t elem) {
  return load_stream16(static_cast<const char*>(base) + elem * (BF16 ? 2 : 4));
}
template <bool BF16>
__device__ __forceinline__ void raw_to_f(const uint4& v, float* f) {
  if constexpr (BF16) {
    unpack8(v, f);
  } else {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  }
}

// One row's inputs for one thread, loaded a row ahead of their use.
template <int NMAX>
struct RowIn {
  uint4 p[NMAX];  // the partials' vectors
  uint4 a, b;     // forward: residual; backward: x and dres
};

template <bool BF16, int NMAX>
__device__ __forceinline__ void load_row(RowIn<NMAX>& in, const PartPtrs& parts, int n, int64_t e0, const void* a,
                                         const void* b) {
#pragma unroll
  for (int j = 0; j < NMAX; ++j)
    if (j < n) in.p[j] = ld_part<BF16>(parts.p[j], e0);
  if (a != nullptr) in.a = ld_raw<BF16>(a, e0);
  if (b != nullptr) in.b = ld_raw<BF16>(b, e0);
}

// Sum of the partials in the fixed order j = 0..n-1.
template <bool BF16, int NMAX>
__device__ __forceinline__ void sum_row(const RowIn<NMAX>& in, int n, float* acc) {
  constexpr int E = Vec16<BF16>::N;
  raw_to_f<BF16>(in.p[0], acc);
#pragma unroll
  for (int j = 1; j < NMAX; ++j)
    if (j < n) {
      float t[E];
      raw_to_f<BF16>(in.p[j], t);
#pragma unroll
      for (int i = 0; i < E; ++i) acc[i] += t[i];
    }
}

// Block-wide sum of one value per thread for NW waves: wave sums, then the
// NW wave totals in wave order (fixed order).  `red` holds NW floats and is
// reused only after a barrier the caller places between uses.
template <int NW>
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float t = red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) t += red[w];
  return t;
}

// Two independent block sums behind one barrier (each summed exactly as
// block_sum does, so the results are the same bits).
template <int NW>
__device__ __forceinline__ void block_sum2(float& a, float& b, float* red_a, float* red_b) {
  a = wave_sum(a);
  b = wave_sum(b);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    red_a[wave] = a;
    red_b[wave] = b;
  }
  __syncthreads();
  float ta = red_a[0], tb = red_b[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    ta += red_a[w];
    tb += red_b[w];
  }
  a = ta;
  b = tb;
}

// out = residual + Drop(sum_j parts[j] + bias); y = LN(out) * gamma + beta.
// Block = NW waves; thread t owns the 16-byte vector t of every row, and the
// block walks rows [blockIdx.x * RPB, +RPB).  The loads of row r+1 are issued
// before row r's reductions, so each thread keeps two rows in flight.
template <bool BF16, int NMAX, int NW>
__global__ __launch_bounds__(64 * NW) void reduce_ln_fwd_kernel(PartPtrs parts, int n_parts, int64_t T, int64_t K,
                                                                int64_t rpb, const void* __restrict__ bias,
                                                                const void* __restrict__ residual, DropoutParams dp,
                                                                void* __restrict__ out, uint8_t* __restrict__ mask,
                                                                const void* __restrict__ gamma,
                                                                const void* __restrict__ beta, float eps,
                                                                void* __restrict__ y, float* __restrict__ mean_out,
                                                                float* __restrict__ rstd_out) {
  using V = Vec16<BF16>;
  constexpr int E = V::N;
  __shared__ float red[4][NW];
  const int64_t vi = threadIdx.x;
  const bool act = vi < K / E;
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * rpb;
  const int64_t r1 = r0 + rpb < T ? r0 + rpb : T;
  float bv[E], gv[E], be[E];
  if (act) {
    if (bias != nullptr) V::load(bias, vi * E, bv);
    else
#pragma unroll
      for (int i = 0; i < E; ++i) bv[i] = 0.0f;
    V::load(gamma, vi * E, gv);
    V::load(beta, vi * E, be);
  }
  const float inv_k = 1.0f / static_cast<float>(K);
  // The next row's inputs are loaded before the current row's reductions,
  // except in 16-wave blocks, whose 128-register cap does not hold two rows
  // of up to 16 + 2 vectors (they spilled).
  constexpr bool PF = NW < 16;
  RowIn<NMAX> nxt;
  if (PF && act && r0 < r1) load_row<BF16, NMAX>(nxt, parts, n_parts, r0 * K + vi * E, residual, nullptr);
  int slot = 0;
  for (int64_t row = r0; row < r1; ++row, slot ^= 2) {
    const int64_t e0 = row * K + vi * E;
    RowIn<NMAX> cur;
    if constexpr (PF) {
      cur = nxt;
      if (act && row + 1 < r1) load_row<BF16, NMAX>(nxt, parts, n_parts, e0 + K, residual, nullptr);
    } else {
      if (act) load_row<BF16, NMAX>(cur, parts, n_parts, e0, residual, nullptr);
    }
    float h[E];
    float sum = 0.0f;
    uint8_t keep[E];
#pragma unroll
    for (int i = 0; i < E; ++i) keep[i] = 0;
    if (act) {
      sum_row<BF16, NMAX>(cur, n_parts, h);
#pragma unroll
      for (int i = 0; i < E; ++i) h[i] += bv[i];
      apply_dropout<E>(dp, dp.index_base + static_cast<uint64_t>(e0), h, keep);
      if (residual != nullptr) {
        float tmp[E];
        raw_to_f<BF16>(cur.a, tmp);
#pragma unroll
        for (int i = 0; i < E; ++i) h[i] += tmp[i];
      }
      if constexpr (BF16) {
#pragma unroll
        for (int i = 0; i < E; ++i) h[i] = round_to_bf16(h[i]);
      }
      V::store(out, e0, h);
#pragma unroll
      for (int i = 0; i < E; ++i) sum += h[i];
    }
    if (mask != nullptr) store_keep_bits<E>(mask, e0, keep, act);
    // red[slot], red[slot + 1] alternate with the next row's pair, so one
    // barrier per reduction suffices.
    const float mean = block_sum<NW>(sum, red[slot]) * inv_k;
    float sq = 0.0f;
    if (act) {
#pragma unroll
      for (int i = 0; i < E; ++i) {
        const float dlt = h[i] - mean;
        sq += dlt * dlt;
      }
    }
    const float rstd = rsqrtf(block_sum<NW>(sq, red[slot + 1]) * inv_k + eps);
    if (act) {
      float o[E];
#pragma unroll
      for (int i = 0; i < E; ++i) o[i] = (h[i] - mean) * rstd * gv[i] + be[i];
      V::store(y, e0, o);
    }
    if (threadIdx.x == 0) {
      if (mean_out) mean_out[row] = mean;
      if (rstd_out) rstd_out[row] = rstd;
    }
  }
}

// dy = sum_j parts[j]; dx = dres + rstd * (g - mean(g) - xhat * mean(g * xhat)),
// g = dy * gamma.  Same block layout as the forward; the block's column sums
// of dy * xhat and dy go to partial[blockIdx.x, 0:K] and [.., K:2K].  With
// `ddrop`, the dropout of the branch below this residual join is applied to
// dx as stored, from the keep bits its forward saved (ddrop = Drop(dx), the
// input gradient of that branch's bias + dropout), and its column sums go to
// [.., 2K:3K] (partial rows 3K wide).
template <bool BF16, int NMAX, int NW>
__global__ __launch_bounds__(64 * NW) void reduce_ln_bwd_kernel(PartPtrs parts, int n_parts, int64_t T, int64_t K,
                                                                int64_t rpb, const void* __restrict__ x,
                                                                const void* __restrict__ gamma,
                                                                const float* __restrict__ mean_in,
                                                                const float* __restrict__ rstd_in,
                                                                const void* __restrict__ dres, void* __restrict__ dx,
                                                                float* __restrict__ partial,
                                                                const uint8_t* __restrict__ keep_bits, float dscale,
                                                                void* __restrict__ ddrop) {
  using V = Vec16<BF16>;
  constexpr int E = V::N;
  __shared__ float red[4][NW];
  const int64_t vi = threadIdx.x;
  const bool act = vi < K / E;
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * rpb;
  const int64_t r1 = r0 + rpb < T ? r0 + rpb : T;
  float gm[E], pg[E], pb[E], pd[E];
#pragma unroll
  for (int i = 0; i < E; ++i) pg[i] = pb[i] = pd[i] = 0.0f;
  if (act) V::load(gamma, vi * E, gm);
  const float inv_k = 1.0f / static_cast<float>(K);
  constexpr bool PF = NW < 16;  // prefetch of the next row, as in the forward
  RowIn<NMAX> nxt;
  if (PF && act && r0 < r1) load_row<BF16, NMAX>(nxt, parts, n_parts, r0 * K + vi * E, x, dres);
  int slot = 0;
  for (int64_t row = r0; row < r1; ++row, slot ^= 2) {
    const int64_t e0 = row * K + vi * E;
    RowIn<NMAX> cur;
    if constexpr (PF) {
      cur = nxt;
      if (act && row + 1 < r1) load_row<BF16, NMAX>(nxt, parts, n_parts, e0 + K, x, dres);
    } else {
      if (act) load_row<BF16, NMAX>(cur, parts, n_parts, e0, x, dres);
    }
    const float mean = mean_in[row];
    const float rstd = rstd_in[row];
    float g[E], xh[E];
    float s1 = 0.0f, s2 = 0.0f;
    if (act) {
      sum_row<BF16, NMAX>(cur, n_parts, g);
      raw_to_f<BF16>(cur.a, xh);
#pragma unroll
      for (int i = 0; i < E; ++i) {
        if constexpr (BF16) g[i] = round_to_bf16(g[i]);  // the unfused path reads the sum back as bf16
        xh[i] = (xh[i] - mean) * rstd;
        pg[i] += g[i] * xh[i];
        pb[i] += g[i];
        g[i] *= gm[i];  // from here on g = dy * gamma
        s1 += g[i];
        s2 += g[i] * xh[i];
      }
    }
    block_sum2<NW>(s1, s2, red[slot], red[slot + 1]);
    const float m1 = s1 * inv_k, m2 = s2 * inv_k;
    if (act) {
      float o[E], r[E];
      if (dres != nullptr) {
        raw_to_f<BF16>(cur.b, r);
      } else {
#pragma unroll
        for (int i = 0; i < E; ++i) r[i] = 0.0f;
      }
#pragma unroll
      for (int i = 0; i < E; ++i) o[i] = r[i] + rstd * (g[i] - m1 - xh[i] * m2);
      V::store(dx, e0, o);
      if (ddrop != nullptr) {
        // Dropout (saved keep bits) of dx as stored (bf16-rounded), rounded
        // again on store: the values a separate pass over dx produces.
        const uint32_t k = load_keep_bits<E>(keep_bits, e0);
#pragma unroll
        for (int i = 0; i < E; ++i) {
          if constexpr (BF16) o[i] = round_to_bf16(o[i]);
          o[i] = ((k >> i) & 1u) ? o[i] * dscale : 0.0f;
        }
        V::store(ddrop, e0, o);
#pragma unroll
        for (int i = 0; i < E; ++i) pd[i] += BF16 ? round_to_bf16(o[i]) : o[i];
      }
    }
  }
  if (partial == nullptr || !act) return;
  const int64_t w = (ddrop != nullptr ? 3 : 2) * K;
  float* pw = partial + static_cast<int64_t>(blockIdx.x) * w + vi * E;
#pragma unroll
  for (int i = 0; i < E; i += 4) {
    *reinterpret_cast<float4*>(pw + i) = make_float4(pg[i], pg[i + 1], pg[i + 2], pg[i + 3]);
    *reinterpret_cast<float4*>(pw + K + i) = make_float4(pb[i], pb[i + 1], pb[i + 2], pb[i + 3]);
    if (ddrop != nullptr)
      *reinterpret_cast<float4*>(pw + 2 * K + i) = make_float4(pd[i], pd[i + 1], pd[i + 2], pd[i + 3]);
  }
}

// Rows per block: the forward uses few (parallelism); the backward more, so
// the per-block dgamma/dbeta partials stay small next to the main traffic.
static int64_t fwd_rows_per_block(int64_t T) { return T >= 4096 ? 4 : 2; }
static int64_t bwd_rows_per_block(int64_t T) {
  const int64_t r = ceil_div(T, 512);
  return r < 1 ? 1 : (r > 32 ? 32 : r);
}

template <bool BF16, int NMAX, int NW>
static void launch_fwd_n(const PartPtrs& parts, int n, int64_t T, int64_t K, const void* bias, const void* residual,
                         const DropoutParams& dp, void* out, uint8_t* mask, const void* gamma, const void* beta,
                         float eps, void* y, float* mean, float* rstd, hipStream_t s) {
  const int64_t rpb = fwd_rows_per_block(T);
  reduce_ln_fwd_kernel<BF16, NMAX, NW><<<static_cast<unsigned>(ceil_div(T, rpb)), 64 * NW, 0, s>>>(
      parts, n, T, K, rpb, bias, residual, dp, out, mask, gamma, beta, eps, y, mean, rstd);
}

template <bool BF16, int NMAX, int NW>
static void launch_bwd_n(const PartPtrs& parts, int n, int64_t T, int64_t K, const void* x, const void* gamma,
                         const float* mean, const float* rstd, const void* dres, void* dx, float* partial,
                         const uint8_t* keep_bits, float dscale, void* ddrop, hipStream_t s) {
  const int64_t rpb = bwd_rows_per_block(T);
  reduce_ln_bwd_kernel<BF16, NMAX, NW><<<static_cast<unsigned>(ceil_div(T, rpb)), 64 * NW, 0, s>>>(
      parts, n, T, K, rpb, x, gamma, mean, rstd, dres, dx, partial, keep_bits, dscale, ddrop);
}

// Dispatch on the partial count (NMAX) and the waves per block (one thread
// per 16-byte vector of a row).
template <bool BF16, int NMAX, bool FWD, typename... Args>
static void by_waves(int64_t nw, Args... a) {
#define MP_NW_CASE(W)                                      \
  if (nw <= W) {                                           \
    if constexpr (FWD) launch_fwd_n<BF16, NMAX, W>(a...);  \
    else launch_bwd_n<BF16, NMAX, W>(a...);                \
    return;                                                \
  }
  MP_NW_CASE(1)
  MP_NW_CASE(2)
  MP_NW_CASE(4)
  MP_NW_CASE(6)
  MP_NW_CASE(8)
  MP_NW_CASE(16)
#undef MP_NW_CASE
}

// bf16 (the hot path): N <= 2, <= 8 or <= 16; fp32: one bound for all N.
template <bool BF16, bool FWD, typename... Args>
static void by_n(int n, int64_t nw, Args... a) {
  if constexpr (BF16) {
    if (n <= 2) by_waves<BF16, 2, FWD>(nw, a...);
    else if (n <= 8) by_waves<BF16, 8, FWD>(nw, a...);
    else by_waves<BF16, 16, FWD>(nw, a...);
  } else {
    by_waves<BF16, 16, FWD>(nw, a...);
  }
}

static int gather_parts(int N, const void* const* partials, PartPtrs& arr, const char* fn) {
  MP_REQUIRE(N >= 1 && N <= MP_MAX_SHARDS, MP_ERR_SHAPE, "%s: N=%d not in [1, %d]", fn, N, MP_MAX_SHARDS);
  MP_REQUIRE_PTR(partials);
  for (int j = 0; j < N; ++j) {
    MP_REQUIRE(partials[j] != nullptr, MP_ERR_NULL, "%s: partials[%d] is NULL", fn, j);
    MP_REQUIRE((reinterpret_cast<uintptr_t>(partials[j]) & 15u) == 0, MP_ERR_ALIGN,
               "%s: partials[%d] is not 16-byte aligned", fn, j);
    arr.p[j] = partials[j];
  }
  return MP_OK;
}

}  // namespace mp

using namespace mp;

extern "C" int mp_shard_reduce_layernorm(mp_dtype dtype, int N, int64_t rows, int64_t cols,
                                         const void* const* partials, const void* bias, const void* residual, float p,
                                         uint64_t seed, uint64_t offset, uint64_t index_base, void* out,
                                         uint8_t* mask_out, const void* gamma, const void* beta, float eps, void* y,
                                         float* mean, float* rstd, hipStream_t s) {
  static const char* fn = "mp_shard_reduce_layernorm";
  MP_REQUIRE(dtype_ok(dtype), MP_ERR_DTYPE, "%s: bad dtype %d", fn, static_cast<int>(dtype));
  MP_REQUIRE(rows >= 0 && cols > 0 && cols % vec_elems(dtype) == 0, MP_ERR_SHAPE, "%s: bad shape %lld x %lld", fn,
             (long long)rows, (long long)cols);
  MP_REQUIRE(cols / vec_elems(dtype) <= 64 * 16, MP_ERR_UNSUPPORTED, "%s: cols=%lld too large", fn, (long long)cols);
  MP_REQUIRE(p >= 0.0f && p < 1.0f, MP_ERR_ARG, "%s: dropout probability %g not in [0, 1)", fn, p);
  MP_REQUIRE(index_base % 4 == 0, MP_ERR_ARG, "%s: index_base must be a multiple of 4", fn);
  MP_REQUIRE(eps > 0.0f, MP_ERR_ARG, "%s: eps must be positive", fn);
  PartPtrs arr{};
  if (int rc = gather_parts(N, partials, arr, fn)) return rc;
  MP_REQUIRE_PTR(out);
  MP_REQUIRE_PTR(gamma);
  MP_REQUIRE_PTR(beta);
  MP_REQUIRE_PTR(y);
  MP_REQUIRE_ALIGN(out);
  MP_REQUIRE_ALIGN(gamma);
  MP_REQUIRE_ALIGN(beta);
  MP_REQUIRE_ALIGN(y);
  MP_REQUIRE_OPT_ALIGN(bias);
  MP_REQUIRE_OPT_ALIGN(residual);
  MP_REQUIRE(mask_out == nullptr || cols % 8 == 0, MP_ERR_SHAPE, "%s: mask_out needs cols %% 8 == 0", fn);
  if (rows == 0) return MP_OK;
  const DropoutParams dp = make_dropout(p, seed, offset, index_base);
  const int64_t nw = ceil_div(cols / vec_elems(dtype), 64);
  if (dtype == MP_BF16)
    by_n<true, true>(N, nw, arr, N, rows, cols, bias, residual, dp, out, mask_out, gamma, beta, eps, y, mean, rstd, s);
  else
    by_n<false, true>(N, nw, arr, N, rows, cols, bias, residual, dp, out, mask_out, gamma, beta, eps, y, mean, rstd,
                      s);
  return check_launch(fn);
}

extern "C" size_t mp_shard_reduce_layernorm_bwd_workspace(int64_t rows, int64_t cols) {
  if (rows <= 0 || cols <= 0) return 0;
  const int64_t blocks = ceil_div(rows, bwd_rows_per_block(rows));
  return align_up(static_cast<size_t>(blocks * 3 * cols) * sizeof(float), 256);
}

static int reduce_ln_bwd(const char* fn, mp_dtype dtype, int N, int64_t rows, int64_t cols,
                         const void* const* partials, const void* x, const void* gamma, const float* mean,
                         const float* rstd, const void* dres, void* dx, float* dgamma, float* dbeta,
                         const uint8_t* keep_bits, float dscale, void* ddrop, float* dbias, void* ws,
                         size_t ws_bytes, hipStream_t s) {
  MP_REQUIRE(dtype_ok(dtype), MP_ERR_DTYPE, "%s: bad dtype %d", fn, static_cast<int>(dtype));
  MP_REQUIRE(rows >= 0 && cols > 0 && cols % vec_elems(dtype) == 0, MP_ERR_SHAPE, "%s: bad shape %lld x %lld", fn,
             (long long)rows, (long long)cols);
  MP_REQUIRE(cols / vec_elems(dtype) <= 64 * 16, MP_ERR_UNSUPPORTED, "%s: cols=%lld too large", fn, (long long)cols);
  PartPtrs arr{};
  if (int rc = gather_parts(N, partials, arr, fn)) return rc;
  MP_REQUIRE_PTR(x);
  MP_REQUIRE_PTR(gamma);
  MP_REQUIRE_PTR(mean);
  MP_REQUIRE_PTR(rstd);
  MP_REQUIRE_PTR(dx);
  MP_REQUIRE_ALIGN(x);
  MP_REQUIRE_ALIGN(gamma);
  MP_REQUIRE_ALIGN(dx);
  MP_REQUIRE_OPT_ALIGN(dres);
  MP_REQUIRE_OPT_ALIGN(ddrop);
  MP_REQUIRE(dbias == nullptr || ddrop != nullptr, MP_ERR_NULL, "%s: dbias needs ddrop", fn);
  const bool params = dgamma != nullptr || dbeta != nullptr || dbias != nullptr;
  const size_t need = params ? mp_shard_reduce_layernorm_bwd_workspace(rows, cols) : 0;
  MP_REQUIRE(need == 0 || (ws != nullptr && ws_bytes >= need), MP_ERR_WORKSPACE, "%s: workspace needs %zu bytes",
             fn, need);
  MP_REQUIRE(need == 0 || (reinterpret_cast<uintptr_t>(ws) & 15u) == 0, MP_ERR_ALIGN, "%s: ws not 16-byte aligned",
             fn);
  if (rows == 0) return MP_OK;
  float* partial = params ? static_cast<float*>(ws) : nullptr;
  const int64_t nw = ceil_div(cols / vec_elems(dtype), 64);
  if (dtype == MP_BF16)
    by_n<true, false>(N, nw, arr, N, rows, cols, x, gamma, mean, rstd, dres, dx, partial, keep_bits, dscale, ddrop,
                      s);
  else
    by_n<false, false>(N, nw, arr, N, rows, cols, x, gamma, mean, rstd, dres, dx, partial, keep_bits, dscale, ddrop,
                       s);
  if (params) {
    const int64_t blocks = ceil_div(rows, bwd_rows_per_block(rows));
    layernorm_param_final(partial, blocks, cols, dgamma, dbeta, s, ddrop != nullptr ? dbias : nullptr);
  }
  return check_launch(fn);
}

extern "C" int mp_shard_reduce_layernorm_bwd(mp_dtype dtype, int N, int64_t rows, int64_t cols,
                                             const void* const* partials, const void* x, const void* gamma,
                                             const float* mean, const float* rstd, const void* dres, void* dx,
                                             float* dgamma, float* dbeta, void* ws, size_t ws_bytes, hipStream_t s) {
  return reduce_ln_bwd("mp_shard_reduce_layernorm_bwd", dtype, N, rows, cols, partials, x, gamma, mean, rstd, dres,
                       dx, dgamma, dbeta, nullptr, 1.0f, nullptr, nullptr, ws, ws_bytes, s);
}

extern "C" int mp_shard_reduce_layernorm_bwd_dropout(mp_dtype dtype, int N, int64_t rows, int64_t cols,
                                                     const void* const* partials, const void* x, const void* gamma,
                                                     const float* mean, const float* rstd, const void* dres,
                                                     void* dx, float* dgamma, float* dbeta, float p,
                                                     const uint8_t* keep_bits, void* ddrop, float* dbias, void* ws,
                                                     size_t ws_bytes, hipStream_t s) {
  static const char* fn = "mp_shard_reduce_layernorm_bwd_dropout";
  MP_REQUIRE(p >= 0.0f && p < 1.0f, MP_ERR_ARG, "%s: dropout probability %g not in [0, 1)", fn, p);
  MP_REQUIRE_PTR(keep_bits);
  MP_REQUIRE_PTR(ddrop);
  return reduce_ln_bwd(fn, dtype, N, rows, cols, partials, x, gamma, mean, rstd, dres, dx, dgamma, dbeta, keep_bits,
                       1.0f / (1.0f - p), ddrop, dbias, ws, ws_bytes, s);
}
