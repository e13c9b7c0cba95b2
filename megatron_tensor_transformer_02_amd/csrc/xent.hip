// Vocab-parallel cross-entropy: per-shard row statistics (one pass over the
// fp32 logits shard), the cross-shard combine and the logits gradient.
//
// The statistics pass is HBM-bound: one wave owns one row, streams it with
// 16-byte loads (a round of them in flight per lane) and keeps an online
// (max, scaled exp-sum) pair per lane, folded across the wave with shuffles.
#include "common.h"
#include "gemm.h"

namespace mp {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Merges (m2, s2) into (m, s): both are (max, sum of exp2(x*log2e - max*log2e)).
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;  // both empty
  s = s * exp2_fast((m - mn) * kLog2e) + s2 * exp2_fast((m2 - mn) * kLog2e);
  m = mn;
}

// One wave per row.  A lane owns float4s lane, lane+64, ... of its row and
// loads them in rounds of UNROLL, all issued before any is used (lanes past
// the row's end read -inf, which leaves the pair unchanged), so a row takes
// ceil(Vi/4/64/UNROLL) dependent memory round trips.
template <int UNROLL>
__global__ __launch_bounds__(256) void xent_triples_kernel(int64_t T, int64_t Vi, int64_t v_start,
                                                           const float* __restrict__ Z,
                                                           const int32_t* __restrict__ labels,
                                                           float* __restrict__ triples) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= T) return;
  const float* zr = Z + row * Vi;
  float m = -INFINITY, s = 0.0f;
  const int64_t nv = Vi >> 2;  // Vi is a multiple of 4
  for (int64_t i0 = lane; i0 < nv; i0 += 64 * UNROLL) {
    float4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t i = i0 + 64 * u;
      v[u] = i < nv ? load_nt4(zr + 4 * i) : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    }
    float lm = m;
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) lm = fmaxf(lm, fmaxf(fmaxf(v[u].x, v[u].y), fmaxf(v[u].z, v[u].w)));
    const float ml = lm * kLog2e;
    float acc = (m == -INFINITY) ? 0.0f : s * exp2_fast(m * kLog2e - ml);
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      acc += exp2_fast(fmaf(v[u].x, kLog2e, -ml));
      acc += exp2_fast(fmaf(v[u].y, kLog2e, -ml));
      acc += exp2_fast(fmaf(v[u].z, kLog2e, -ml));
      acc += exp2_fast(fmaf(v[u].w, kLog2e, -ml));
    }
    m = lm;
    s = acc;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64);
    const float s2 = __shfl_xor(s, o, 64);
    lse_merge(m, s, m2, s2);
  }
  if (lane == 0) {
    const int64_t col = static_cast<int64_t>(labels[row]) - v_start;
    const float tgt = (col >= 0 && col < Vi) ? zr[col] : 0.0f;
    triples[row * 3 + 0] = m;
    triples[row * 3 + 1] = s;
    triples[row * 3 + 2] = tgt;
  }
}

// The fused logits GEMM's per-slot row statistics folded into the shard's
// triple (max, exp-sum, target logit): one wave per row, lane l merges slots
// l, l+64, ... in order, then a fixed butterfly merges the lanes.
__global__ __launch_bounds__(256) void lse_fold_kernel(int64_t T, int P, const float* __restrict__ part,
                                                       float* __restrict__ triples) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* pp = part + t * P * 3;
  float m = -INFINITY, s = 0.0f, tg = 0.0f;
  for (int k = lane; k < P; k += 64) {
    lse_merge(m, s, pp[3 * k], pp[3 * k + 1]);
    tg += pp[3 * k + 2];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64);
    const float s2 = __shfl_xor(s, o, 64);
    lse_merge(m, s, m2, s2);
    tg += __shfl_xor(tg, o, 64);
  }
  if (lane == 0) {
    triples[t * 3 + 0] = m;
    triples[t * 3 + 1] = s;
    triples[t * 3 + 2] = tg;
  }
}

struct TripleArray {
  const float* p[MP_MAX_SHARDS];
};

__global__ __launch_bounds__(256) void xent_combine_kernel(int n_shards, int64_t T, TripleArray tr,
                                                           float* __restrict__ loss, float* __restrict__ stats) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= T) return;
  float big_m = -INFINITY;
  for (int j = 0; j < n_shards; ++j) big_m = fmaxf(big_m, tr.p[j][t * 3]);
  float big_s = 0.0f, tgt = 0.0f;
  for (int j = 0; j < n_shards; ++j) {
    big_s += tr.p[j][t * 3 + 1] * expf(tr.p[j][t * 3] - big_m);
    tgt += tr.p[j][t * 3 + 2];
  }
  loss[t] = logf(big_s) + big_m - tgt;
  if (stats != nullptr) {
    stats[t * 2] = big_m;
    stats[t * 2 + 1] = big_s;
  }
}

// Mean of loss[T] by one block: strided per-thread sums, then a fixed-order
// tree in LDS (deterministic).
__global__ __launch_bounds__(1024) void mean_kernel(int64_t T, const float* __restrict__ loss,
                                                    float* __restrict__ mean) {
  __shared__ float red[1024];
  float acc = 0.0f;
  for (int64_t t = threadIdx.x; t < T; t += 1024) acc += loss[t];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if (static_cast<int>(threadIdx.x) < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) mean[0] = T > 0 ? red[0] / static_cast<float>(T) : 0.0f;
}

// dZ = g * (exp(z - M) / S - onehot), one float4 per thread.
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void xent_bwd_kernel(int64_t T, int64_t Vi, int64_t v_start,
                                                       const float* __restrict__ Z,
                                                       const int32_t* __restrict__ labels,
                                                       const float* __restrict__ stats, float g,
                                                       void* __restrict__ dZ) {
  const int64_t nv_row = Vi >> 2;
  const int64_t v = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (v >= T * nv_row) return;
  const int64_t t = v / nv_row;
  const int64_t c0 = (v - t * nv_row) * 4;
  const float big_m = stats[t * 2];
  const float gs = g / stats[t * 2 + 1];
  const int64_t lc = static_cast<int64_t>(labels[t]) - v_start - c0;
  const float4 z = load_nt4(Z + 4 * v);
  float r[4] = {z.x, z.y, z.z, z.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] = gs * exp2_fast((r[i] - big_m) * kLog2e);
    if (lc == i) r[i] -= g;
  }
  if constexpr (OUT_BF16) {
    uint2 o;
    o.x = pack_bf16x2(r[0], r[1]);
    o.y = pack_bf16x2(r[2], r[3]);
    reinterpret_cast<uint2*>(dZ)[v] = o;
  } else {
    store_nt4(static_cast<float*>(dZ) + 4 * v, r[0], r[1], r[2], r[3]);
  }
}

}  // namespace mp

using namespace mp;

extern "C" int mp_vocab_parallel_xent(int64_t T, int64_t Vi, int64_t v_start, const float* Z_i, const int32_t* labels,
                                      float* triples, hipStream_t s) {
  MP_REQUIRE(T >= 0 && Vi > 0 && v_start >= 0, MP_ERR_SHAPE, "mp_vocab_parallel_xent: bad shape");
  MP_REQUIRE(Vi % 4 == 0, MP_ERR_SHAPE, "mp_vocab_parallel_xent: Vi=%lld not a multiple of 4", (long long)Vi);
  MP_REQUIRE_PTR(Z_i);
  MP_REQUIRE_PTR(labels);
  MP_REQUIRE_PTR(triples);
  MP_REQUIRE_ALIGN(Z_i);
  if (T == 0) return MP_OK;
  if (int rc = debug_check_range("mp_vocab_parallel_xent", "labels", labels, T, 0, INT32_MAX + 1LL, s)) return rc;
#ifndef MP_XENT_UNROLL
#define MP_XENT_UNROLL 25
#endif
  xent_triples_kernel<MP_XENT_UNROLL><<<static_cast<unsigned>(ceil_div(T, 4)), 256, 0, s>>>(T, Vi, v_start, Z_i,
                                                                                           labels, triples);
  return check_launch("mp_vocab_parallel_xent");
}

extern "C" size_t mp_vocab_parallel_logits_xent_workspace(int64_t T, int64_t K, int64_t Vi) {
  if (T <= 0 || K <= 0 || Vi <= 0) return 0;
  return align_up(static_cast<size_t>(T) * gemm_lse_slots(T, Vi, K) * 3 * sizeof(float), 256);
}

extern "C" int mp_vocab_parallel_logits_xent(mp_dtype dtype, int64_t T, int64_t K, int64_t Vi, int64_t v_start,
                                             const void* H, const void* E_i, const int32_t* labels, float* triples,
                                             void* ws, size_t ws_bytes, hipStream_t s) {
  static const char* fn = "mp_vocab_parallel_logits_xent";
  MP_REQUIRE(dtype == MP_BF16, MP_ERR_DTYPE, "%s: the fused logits GEMM runs in bf16 only", fn);
  MP_REQUIRE(T >= 0 && K > 0 && Vi > 0 && v_start >= 0, MP_ERR_SHAPE, "%s: bad shape", fn);
  MP_REQUIRE(K % 8 == 0, MP_ERR_SHAPE, "%s: K=%lld must be a multiple of 8", fn, (long long)K);
  MP_REQUIRE_PTR(H);
  MP_REQUIRE_PTR(E_i);
  MP_REQUIRE_PTR(labels);
  MP_REQUIRE_PTR(triples);
  MP_REQUIRE_ALIGN(H);
  MP_REQUIRE_ALIGN(E_i);
  const size_t need = mp_vocab_parallel_logits_xent_workspace(T, K, Vi);
  MP_REQUIRE(need == 0 || (ws != nullptr && ws_bytes >= need), MP_ERR_WORKSPACE, "%s: workspace needs %zu bytes", fn,
             need);
  MP_REQUIRE_OPT_ALIGN(ws);
  if (T == 0) return MP_OK;
  if (int rc = debug_check_range(fn, "labels", labels, T, 0, INT32_MAX + 1LL, s)) return rc;
  float* part = static_cast<float*>(ws);
  if (int rc = gemm_logits_lse(T, Vi, K, H, E_i, labels, v_start, part, s)) return rc;
  lse_fold_kernel<<<static_cast<unsigned>(ceil_div(T, 4)), 256, 0, s>>>(T, gemm_lse_slots(T, Vi, K), part, triples);
  return check_launch(fn);
}

extern "C" int mp_vocab_xent_combine(int N, int64_t T, const float* const* triples, float* loss, float* stats,
                                     float* mean_loss, hipStream_t s) {
  MP_REQUIRE(N >= 1 && N <= MP_MAX_SHARDS, MP_ERR_SHAPE, "mp_vocab_xent_combine: N=%d not in [1, %d]", N,
             MP_MAX_SHARDS);
  MP_REQUIRE(T >= 0, MP_ERR_SHAPE, "mp_vocab_xent_combine: bad T");
  MP_REQUIRE_PTR(triples);
  MP_REQUIRE_PTR(loss);
  TripleArray arr{};
  for (int j = 0; j < N; ++j) {
    MP_REQUIRE(triples[j] != nullptr, MP_ERR_NULL, "mp_vocab_xent_combine: triples[%d] is NULL", j);
    arr.p[j] = triples[j];
  }
  if (T > 0)
    xent_combine_kernel<<<static_cast<unsigned>(ceil_div(T, 256)), 256, 0, s>>>(N, T, arr, loss, stats);
  if (mean_loss != nullptr) mean_kernel<<<1, 1024, 0, s>>>(T, loss, mean_loss);
  return check_launch("mp_vocab_xent_combine");
}

extern "C" int mp_vocab_parallel_xent_bwd(int64_t T, int64_t Vi, int64_t v_start, const float* Z_i,
                                          const int32_t* labels, const float* stats, float g, mp_dtype out_dtype,
                                          void* dZ_i, hipStream_t s) {
  MP_REQUIRE(dtype_ok(out_dtype), MP_ERR_DTYPE, "mp_vocab_parallel_xent_bwd: bad dtype");
  MP_REQUIRE(T >= 0 && Vi > 0 && v_start >= 0 && Vi % 4 == 0, MP_ERR_SHAPE, "mp_vocab_parallel_xent_bwd: bad shape");
  MP_REQUIRE(out_dtype == MP_F32 || Vi % 8 == 0, MP_ERR_SHAPE, "mp_vocab_parallel_xent_bwd: bf16 needs Vi %% 8 == 0");
  MP_REQUIRE_PTR(Z_i);
  MP_REQUIRE_PTR(labels);
  MP_REQUIRE_PTR(stats);
  MP_REQUIRE_PTR(dZ_i);
  MP_REQUIRE_ALIGN(Z_i);
  MP_REQUIRE_ALIGN(dZ_i);
  MP_REQUIRE(out_dtype == MP_F32 || static_cast<const void*>(Z_i) != dZ_i, MP_ERR_ARG,
             "mp_vocab_parallel_xent_bwd: in-place only for fp32 output");
  if (T == 0) return MP_OK;
  if (int rc = debug_check_range("mp_vocab_parallel_xent_bwd", "labels", labels, T, 0, INT32_MAX + 1LL, s)) return rc;
  const int64_t nvec = T * (Vi / 4);
  const unsigned grid = static_cast<unsigned>(ceil_div(nvec, 256));
  if (out_dtype == MP_BF16)
    xent_bwd_kernel<true><<<grid, 256, 0, s>>>(T, Vi, v_start, Z_i, labels, stats, g, dZ_i);
  else
    xent_bwd_kernel<false><<<grid, 256, 0, s>>>(T, Vi, v_start, Z_i, labels, stats, g, dZ_i);
  return check_launch("mp_vocab_parallel_xent_bwd");
}
