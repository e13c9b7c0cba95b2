// HBM-bound element-wise calls: the shard reduce (stand-in for the
// all-reduce, with bias, shared-seed dropout and residual fused), the
// standalone shared-seed dropout, the vocab-parallel embedding lookup and the
// deterministic bias gradient (column sums).
//
// Every thread moves whole 16-byte vectors (8 bf16 or 4 fp32), so a wave reads
// 1 KiB contiguous per load instruction.
#include "common.h"
#include "slab_sum.h"

namespace mp {

struct PtrArray {
  const void* p[MP_MAX_SHARDS];
};

// out = residual + Drop(sum_j parts[j] + bias), one 16-byte vector per thread.
// NMAX is a compile-time bound on N so all partial loads are issued before
// the fp32 sum consumes them (summation order j = 0..N-1 is fixed).
template <bool BF16, int NMAX>
__global__ __launch_bounds__(256) void shard_reduce_kernel(PtrArray parts, int n_parts, int64_t nvec,
                                                           int64_t cols, const void* __restrict__ bias,
                                                           const void* __restrict__ residual, DropoutParams dp,
                                                           void* __restrict__ out, uint8_t* __restrict__ mask) {
  using V = Vec16<BF16>;
  constexpr int E = V::N;
  const int64_t v = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const bool live = v < nvec;
  if (!live && (E == 8 || mask == nullptr)) return;  // fp32 lanes stay for the mask-bit exchange
  const int64_t e0 = v * E;
  uint8_t keep[E];
#pragma unroll
  for (int i = 0; i < E; ++i) keep[i] = 0;
  if (live) {
    float part[NMAX][E];
#pragma unroll
    for (int j = 0; j < NMAX; ++j)
      if (j < n_parts) V::load_stream(parts.p[j], e0, part[j]);
    float acc[E];
#pragma unroll
    for (int i = 0; i < E; ++i) acc[i] = part[0][i];
#pragma unroll
    for (int j = 1; j < NMAX; ++j)
      if (j < n_parts) {
#pragma unroll
        for (int i = 0; i < E; ++i) acc[i] += part[j][i];
      }
    float tmp[E];
    if (bias != nullptr) {
      V::load(bias, e0 % cols, tmp);
#pragma unroll
      for (int i = 0; i < E; ++i) acc[i] += tmp[i];
    }
    apply_dropout<E>(dp, dp.index_base + static_cast<uint64_t>(e0), acc, keep);
    if (residual != nullptr) {
      V::load(residual, e0, tmp);
#pragma unroll
      for (int i = 0; i < E; ++i) acc[i] += tmp[i];
    }
    V::store(out, e0, acc);
  }
  if (mask != nullptr) store_keep_bits<E>(mask, e0, keep, live);
}

// Dropout backward from saved keep bits over a slab of rows, one column vector
// per thread (block: 32 column vectors x 8 row lanes, as the column sums):
// dx = dy * keep * scale, and with SUM the slab's column sums of dx as stored
// go to partial[slab, :] (the bias gradient's first stage).
template <bool BF16, bool SUM>
__global__ __launch_bounds__(256) void dropout_mask_bwd_kernel(const void* __restrict__ dy,
                                                               const uint8_t* __restrict__ bits, float scale,
                                                               int64_t rows, int64_t cols, int64_t slab_rows,
                                                               void* __restrict__ dx, float* __restrict__ partial) {
  using V = Vec16<BF16>;
  constexpr int E = V::N;
  __shared__ float red[SUM ? 8 : 1][SUM ? 32 * E : 1];
  const int cv = threadIdx.x & 31;
  const int rl = threadIdx.x >> 5;
  // Blocks are dealt to the 8 XCDs round-robin by their linear id; each XCD
  // instead gets a contiguous run of (column block, slab) pairs, so the four
  // column-neighbour blocks that read one 128-byte line of keep bits (32
  // vectors x 8 bits each) share its L2 instead of fetching it four times.
  // Runs cover whole groups of four when the block count is a multiple of 32
  // and a slab's column blocks a multiple of 4; otherwise the plain order.
  const unsigned gx = gridDim.x, nb = gx * gridDim.y, hw = blockIdx.x + gx * blockIdx.y;
  const unsigned lid = (nb % 32 == 0 && gx % 4 == 0) ? (hw % 8) * (nb / 8) + hw / 8 : hw;
  const unsigned bx = lid % gx, by = lid / gx;
  const int64_t c0 = (static_cast<int64_t>(bx) * 32 + cv) * E;
  const int64_t r_begin = static_cast<int64_t>(by) * slab_rows;
  const int64_t r_end = r_begin + slab_rows < rows ? r_begin + slab_rows : rows;
  float acc[E];
#pragma unroll
  for (int i = 0; i < E; ++i) acc[i] = 0.0f;
  if (c0 < cols) {
    for (int64_t r = r_begin + rl; r < r_end; r += 8) {
      const int64_t e0 = r * cols + c0;
      float v[E];
      V::load_stream(dy, e0, v);
      const uint32_t k = load_keep_bits<E>(bits, e0);
#pragma unroll
      for (int i = 0; i < E; ++i) v[i] = ((k >> i) & 1u) ? v[i] * scale : 0.0f;
      V::store(dx, e0, v);
      if constexpr (SUM) {
#pragma unroll
        for (int i = 0; i < E; ++i) acc[i] += BF16 ? __uint_as_float(static_cast<uint32_t>(f32_to_bf16(v[i])) << 16)
                                                   : v[i];
      }
    }
  }
  if constexpr (SUM) {
#pragma unroll
    for (int i = 0; i < E; ++i) red[rl][cv * E + i] = acc[i];
    __syncthreads();
    if (rl == 0 && c0 < cols) {
#pragma unroll
      for (int i = 0; i < E; ++i) {
        float t = red[0][cv * E + i];
#pragma unroll
        for (int l = 1; l < 8; ++l) t += red[l][cv * E + i];
        partial[static_cast<int64_t>(by) * cols + c0 + i] = t;
      }
    }
  }
}

template <bool BF16>
static int launch_reduce(int n_parts, const PtrArray& parts, int64_t nvec, int64_t cols, const void* bias,
                         const void* residual, const DropoutParams& dp, void* out, uint8_t* mask, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(ceil_div(nvec, 256)));
  if (n_parts == 1)
    shard_reduce_kernel<BF16, 1><<<grid, 256, 0, s>>>(parts, n_parts, nvec, cols, bias, residual, dp, out, mask);
  else if (n_parts == 2)
    shard_reduce_kernel<BF16, 2><<<grid, 256, 0, s>>>(parts, n_parts, nvec, cols, bias, residual, dp, out, mask);
  else if (n_parts <= 4)
    shard_reduce_kernel<BF16, 4><<<grid, 256, 0, s>>>(parts, n_parts, nvec, cols, bias, residual, dp, out, mask);
  else if (n_parts <= 8)
    shard_reduce_kernel<BF16, 8><<<grid, 256, 0, s>>>(parts, n_parts, nvec, cols, bias, residual, dp, out, mask);
  else
    shard_reduce_kernel<BF16, 16><<<grid, 256, 0, s>>>(parts, n_parts, nvec, cols, bias, residual, dp, out, mask);
  return check_launch("shard_reduce");
}

static int validate_dropout(float p, uint64_t index_base, const char* fn) {
  MP_REQUIRE(p >= 0.0f && p < 1.0f, MP_ERR_ARG, "%s: dropout probability %g not in [0, 1)", fn, p);
  MP_REQUIRE(index_base % 4 == 0, MP_ERR_ARG, "%s: index_base must be a multiple of 4", fn);
  return MP_OK;
}

// Column-sum stage 1: partial[slab, c] = sum of rows in the slab, fixed order.
// Block: 32 column vectors x 8 row lanes; the 8 lanes are reduced through LDS
// in lane order.
template <bool BF16>
__global__ __launch_bounds__(256) void colsum_partial_kernel(const void* __restrict__ dy, int64_t rows, int64_t cols,
                                                             int64_t slab_rows, float* __restrict__ partial) {
  using V = Vec16<BF16>;
  constexpr int E = V::N;
  __shared__ float red[8][32 * E];
  const int cv = threadIdx.x & 31;
  const int rl = threadIdx.x >> 5;
  const int64_t c0 = (static_cast<int64_t>(blockIdx.x) * 32 + cv) * E;
  const int64_t r_begin = static_cast<int64_t>(blockIdx.y) * slab_rows;
  const int64_t r_end = r_begin + slab_rows < rows ? r_begin + slab_rows : rows;
  float acc[E];
#pragma unroll
  for (int i = 0; i < E; ++i) acc[i] = 0.0f;
  if (c0 < cols) {
    float tmp[E];
    for (int64_t r = r_begin + rl; r < r_end; r += 8) {
      V::load(dy, r * cols + c0, tmp);
#pragma unroll
      for (int i = 0; i < E; ++i) acc[i] += tmp[i];
    }
  }
#pragma unroll
  for (int i = 0; i < E; ++i) red[rl][cv * E + i] = acc[i];
  __syncthreads();
  if (rl == 0 && c0 < cols) {
#pragma unroll
    for (int i = 0; i < E; ++i) {
      float t = red[0][cv * E + i];
#pragma unroll
      for (int l = 1; l < 8; ++l) t += red[l][cv * E + i];
      partial[static_cast<int64_t>(blockIdx.y) * cols + c0 + i] = t;
    }
  }
}

// Column-sum stage 2: out[c] = sum over slabs (fixed order, slab_sum.h).
__global__ __launch_bounds__(SLAB_THREADS) void colsum_final_kernel(const float* __restrict__ partial, int64_t slabs,
                                                                    int64_t cols, float* __restrict__ out) {
  __shared__ float red[SLAB_GROUPS][SLAB_COLS];
  const int64_t c = static_cast<int64_t>(blockIdx.x) * SLAB_COLS + threadIdx.x % SLAB_COLS;
  const float v = slab_column_sum(partial, slabs, cols, c, red);
  if (threadIdx.x < SLAB_COLS && c < cols) out[c] = v;
}

static void colsum_plan(int64_t rows, int64_t& slab_rows, int64_t& slabs) {
  slab_rows = rows / 256;
  if (slab_rows < 64) slab_rows = 64;
  slab_rows = align_up(static_cast<size_t>(slab_rows), 8);
  slabs = rows > 0 ? ceil_div(rows, slab_rows) : 0;
}

size_t colsum_workspace(int64_t rows, int64_t cols) {
  int64_t slab_rows, slabs;
  colsum_plan(rows, slab_rows, slabs);
  return align_up(static_cast<size_t>(slabs * cols) * sizeof(float), 256);
}

// Deterministic column sums of a [rows, cols] matrix (cols a multiple of the
// vector width) into out[cols]; `ws` holds colsum_workspace(rows, cols) bytes.
int colsum(mp_dtype dt, int64_t rows, int64_t cols, const void* dy, float* out, void* ws, hipStream_t s) {
  int64_t slab_rows, slabs;
  colsum_plan(rows, slab_rows, slabs);
  const int64_t E = vec_elems(dt);
  if (slabs > 0) {
    const dim3 grid(static_cast<unsigned>(ceil_div(cols / E, 32)), static_cast<unsigned>(slabs));
    if (dt == MP_BF16)
      colsum_partial_kernel<true><<<grid, 256, 0, s>>>(dy, rows, cols, slab_rows, static_cast<float*>(ws));
    else
      colsum_partial_kernel<false><<<grid, 256, 0, s>>>(dy, rows, cols, slab_rows, static_cast<float*>(ws));
  }
  colsum_final_kernel<<<static_cast<unsigned>(ceil_div(cols, SLAB_COLS)), SLAB_THREADS, 0, s>>>(
      static_cast<const float*>(ws), slabs, cols, out);
  return check_launch("colsum");
}

// Embedding backward (the lookup's adjoint, a deterministic scatter-add):
// block b owns shard rows [16b, 16b+16).  Tokens are taken in chunks of
// 8192; a chunk's tokens whose row falls in the block's range are compacted
// into LDS in token order (per-thread counts and an exclusive scan), then each
// of the block's rows adds its tokens' gradient rows in that order, one
// 16-byte vector of columns per thread.  No atomics: the sums are fixed-order.
template <bool BF16>
__global__ __launch_bounds__(256) void embedding_bwd_kernel(int64_t T, int64_t Vi, int64_t v_start, int64_t K,
                                                            const int32_t* __restrict__ ids,
                                                            const void* __restrict__ dout, float* __restrict__ dE,
                                                            int accumulate) {
  using V = Vec16<BF16>;
  constexpr int E = V::N, R = 16, CH = 8192, TPT = CH / 256;
  __shared__ int list[CH];  // (token within the chunk) * R + (row within the block)
  __shared__ int offs[257];
  const int tid = threadIdx.x;
  const int64_t v0 = static_cast<int64_t>(blockIdx.x) * R;
  const int rows = static_cast<int>(Vi - v0 < R ? Vi - v0 : R);
  const int64_t nvec = K / E;
  for (int64_t c0 = 0; c0 < T || c0 == 0; c0 += CH) {  // T = 0 still writes the zero rows
    int n = 0;
#pragma unroll 4
    for (int u = 0; u < TPT; ++u) {
      const int64_t t = c0 + tid * TPT + u;
      if (t < T) {
        const int64_t v = static_cast<int64_t>(ids[t]) - v_start - v0;
        n += (v >= 0 && v < rows) ? 1 : 0;
      }
    }
    offs[tid] = n;
    __syncthreads();
    if (tid == 0) {
      int acc = 0;
      for (int i = 0; i < 256; ++i) {
        const int x = offs[i];
        offs[i] = acc;
        acc += x;
      }
      offs[256] = acc;
    }
    __syncthreads();
    int pos = offs[tid];
    for (int u = 0; u < TPT; ++u) {
      const int64_t t = c0 + tid * TPT + u;
      if (t < T) {
        const int64_t v = static_cast<int64_t>(ids[t]) - v_start - v0;
        if (v >= 0 && v < rows) list[pos++] = (tid * TPT + u) * R + static_cast<int>(v);
      }
    }
    __syncthreads();
    const int L = offs[256];
    for (int r = 0; r < rows; ++r) {
      float* drow = dE + (v0 + r) * K;
      for (int64_t cv = tid; cv < nvec; cv += 256) {
        float acc[E];
        if (c0 == 0 && !accumulate) {
#pragma unroll
          for (int i = 0; i < E; ++i) acc[i] = 0.0f;
        } else {
#pragma unroll
          for (int i = 0; i < E; i += 4) {
            const float4 f = *reinterpret_cast<const float4*>(drow + cv * E + i);
            acc[i] = f.x; acc[i + 1] = f.y; acc[i + 2] = f.z; acc[i + 3] = f.w;
          }
        }
        for (int e = 0; e < L; ++e) {
          const int x = list[e];
          if ((x & (R - 1)) != r) continue;
          float g[E];
          V::load(dout, (c0 + (x >> 4)) * K + cv * E, g);
#pragma unroll
          for (int i = 0; i < E; ++i) acc[i] += g[i];
        }
#pragma unroll
        for (int i = 0; i < E; i += 4)
          *reinterpret_cast<float4*>(drow + cv * E + i) = make_float4(acc[i], acc[i + 1], acc[i + 2], acc[i + 3]);
      }
    }
    __syncthreads();  // the next chunk reuses list and offs
  }
}

// All-gather stand-in: out rows [j*rows, (j+1)*rows) = slices[j], one 16-byte
// vector per thread (a slice may be out's own rows: then it copies onto itself).
__global__ __launch_bounds__(256) void gather_rows_kernel(PtrArray slices, int n, int64_t vec_per_slice,
                                                          uint4* __restrict__ out) {
  const int64_t v = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (v >= n * vec_per_slice) return;
  const int64_t j = v / vec_per_slice;
  out[v] = static_cast<const uint4*>(slices.p[j])[v - j * vec_per_slice];
}

// Vocab-parallel embedding: one 16-byte vector of one token's row per thread.
__global__ __launch_bounds__(256) void embedding_kernel(int64_t nvec, int64_t vec_per_row, int64_t Vi, int64_t v_start,
                                                        const int32_t* __restrict__ ids, const uint4* __restrict__ emb,
                                                        uint4* __restrict__ out) {
  const int64_t v = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (v >= nvec) return;
  const int64_t t = v / vec_per_row;
  const int64_t c = v - t * vec_per_row;
  const int64_t row = static_cast<int64_t>(ids[t]) - v_start;
  uint4 val = make_uint4(0, 0, 0, 0);
  if (row >= 0 && row < Vi) val = emb[row * vec_per_row + c];
  out[v] = val;
}

}  // namespace mp

using namespace mp;

extern "C" int mp_shard_reduce(mp_dtype dtype, int N, int64_t rows, int64_t cols, const void* const* partials,
                               const void* bias, const void* residual, float p, uint64_t seed, uint64_t offset,
                               uint64_t index_base, void* out, uint8_t* mask_out, hipStream_t s) {
  MP_REQUIRE(dtype_ok(dtype), MP_ERR_DTYPE, "mp_shard_reduce: bad dtype %d", static_cast<int>(dtype));
  MP_REQUIRE(N >= 1 && N <= MP_MAX_SHARDS, MP_ERR_SHAPE, "mp_shard_reduce: N=%d not in [1, %d]", N, MP_MAX_SHARDS);
  MP_REQUIRE(rows >= 0 && cols > 0, MP_ERR_SHAPE, "mp_shard_reduce: bad shape %lld x %lld", (long long)rows,
             (long long)cols);
  MP_REQUIRE(cols % vec_elems(dtype) == 0, MP_ERR_SHAPE, "mp_shard_reduce: cols %lld not a multiple of %lld",
             (long long)cols, (long long)vec_elems(dtype));
  MP_REQUIRE_PTR(partials);
  MP_REQUIRE_PTR(out);
  MP_REQUIRE_ALIGN(out);
  MP_REQUIRE_OPT_ALIGN(bias);
  MP_REQUIRE_OPT_ALIGN(residual);
  if (int rc = validate_dropout(p, index_base, "mp_shard_reduce")) return rc;
  PtrArray arr{};
  for (int j = 0; j < N; ++j) {
    MP_REQUIRE(partials[j] != nullptr, MP_ERR_NULL, "mp_shard_reduce: partials[%d] is NULL", j);
    MP_REQUIRE((reinterpret_cast<uintptr_t>(partials[j]) & 15u) == 0, MP_ERR_ALIGN,
               "mp_shard_reduce: partials[%d] is not 16-byte aligned", j);
    arr.p[j] = partials[j];
  }
  if (rows == 0) return MP_OK;
  const DropoutParams dp = make_dropout(p, seed, offset, index_base);
  const int64_t nvec = rows * cols / vec_elems(dtype);
  return dtype == MP_BF16 ? launch_reduce<true>(N, arr, nvec, cols, bias, residual, dp, out, mask_out, s)
                          : launch_reduce<false>(N, arr, nvec, cols, bias, residual, dp, out, mask_out, s);
}

extern "C" int mp_shared_seed_dropout(mp_dtype dtype, int64_t n, const void* x, void* y, uint8_t* mask_out, float p,
                                      uint64_t seed, uint64_t offset, uint64_t index_base, hipStream_t s) {
  MP_REQUIRE(dtype_ok(dtype), MP_ERR_DTYPE, "mp_shared_seed_dropout: bad dtype %d", static_cast<int>(dtype));
  MP_REQUIRE(n >= 0 && n % vec_elems(dtype) == 0, MP_ERR_SHAPE,
             "mp_shared_seed_dropout: n=%lld must be a non-negative multiple of %lld", (long long)n,
             (long long)vec_elems(dtype));
  MP_REQUIRE_PTR(x);
  MP_REQUIRE_PTR(y);
  MP_REQUIRE_ALIGN(x);
  MP_REQUIRE_ALIGN(y);
  if (int rc = validate_dropout(p, index_base, "mp_shared_seed_dropout")) return rc;
  if (n == 0) return MP_OK;
  PtrArray arr{};
  arr.p[0] = x;
  const DropoutParams dp = make_dropout(p, seed, offset, index_base);
  const int64_t nvec = n / vec_elems(dtype);
  return dtype == MP_BF16 ? launch_reduce<true>(1, arr, nvec, n, nullptr, nullptr, dp, y, mask_out, s)
                          : launch_reduce<false>(1, arr, nvec, n, nullptr, nullptr, dp, y, mask_out, s);
}

extern "C" size_t mp_dropout_mask_bwd_workspace(int64_t rows, int64_t cols) {
  if (rows < 0 || cols <= 0) return 0;
  return colsum_workspace(rows, cols);
}

extern "C" int mp_dropout_mask_bwd(mp_dtype dtype, int64_t rows, int64_t cols, const void* dy,
                                   const uint8_t* keep_bits, float p, void* dx, float* dbias, void* ws,
                                   size_t ws_bytes, hipStream_t s) {
  static const char* fn = "mp_dropout_mask_bwd";
  MP_REQUIRE(dtype_ok(dtype), MP_ERR_DTYPE, "%s: bad dtype %d", fn, static_cast<int>(dtype));
  MP_REQUIRE(rows >= 0 && cols > 0 && cols % vec_elems(dtype) == 0, MP_ERR_SHAPE, "%s: bad shape %lld x %lld", fn,
             (long long)rows, (long long)cols);
  MP_REQUIRE(p >= 0.0f && p < 1.0f, MP_ERR_ARG, "%s: dropout probability %g not in [0, 1)", fn, p);
  MP_REQUIRE(rows == 0 || (dy != nullptr && dx != nullptr && keep_bits != nullptr), MP_ERR_NULL,
             "%s: dy, dx and keep_bits must be non-NULL", fn);
  MP_REQUIRE_OPT_ALIGN(dy);
  MP_REQUIRE_OPT_ALIGN(dx);
  const size_t need = dbias != nullptr ? colsum_workspace(rows, cols) : 0;
  MP_REQUIRE(need == 0 || (ws != nullptr && ws_bytes >= need), MP_ERR_WORKSPACE, "%s: workspace needs %zu bytes", fn,
             need);
  MP_REQUIRE_OPT_ALIGN(ws);
  int64_t slab_rows, slabs;
  colsum_plan(rows, slab_rows, slabs);
  const float scale = 1.0f / (1.0f - p);
  float* partial = static_cast<float*>(ws);
  if (slabs > 0) {
    const dim3 grid(static_cast<unsigned>(ceil_div(cols / vec_elems(dtype), 32)), static_cast<unsigned>(slabs));
    if (dtype == MP_BF16) {
      if (dbias) dropout_mask_bwd_kernel<true, true><<<grid, 256, 0, s>>>(dy, keep_bits, scale, rows, cols, slab_rows, dx, partial);
      else dropout_mask_bwd_kernel<true, false><<<grid, 256, 0, s>>>(dy, keep_bits, scale, rows, cols, slab_rows, dx, partial);
    } else {
      if (dbias) dropout_mask_bwd_kernel<false, true><<<grid, 256, 0, s>>>(dy, keep_bits, scale, rows, cols, slab_rows, dx, partial);
      else dropout_mask_bwd_kernel<false, false><<<grid, 256, 0, s>>>(dy, keep_bits, scale, rows, cols, slab_rows, dx, partial);
    }
  }
  if (dbias != nullptr)
    colsum_final_kernel<<<static_cast<unsigned>(ceil_div(cols, SLAB_COLS)), SLAB_THREADS, 0, s>>>(partial, slabs,
                                                                                                 cols, dbias);
  return check_launch(fn);
}

extern "C" size_t mp_bias_grad_workspace(int64_t rows, int64_t cols) {
  if (rows < 0 || cols <= 0) return 0;
  return colsum_workspace(rows, cols);
}

extern "C" int mp_bias_grad(mp_dtype dtype, int64_t rows, int64_t cols, const void* dy, float* db, void* ws,
                            size_t ws_bytes, hipStream_t s) {
  MP_REQUIRE(dtype_ok(dtype), MP_ERR_DTYPE, "mp_bias_grad: bad dtype %d", static_cast<int>(dtype));
  MP_REQUIRE(rows >= 0 && cols > 0 && cols % vec_elems(dtype) == 0, MP_ERR_SHAPE, "mp_bias_grad: bad shape");
  MP_REQUIRE_PTR(db);
  MP_REQUIRE(rows == 0 || dy != nullptr, MP_ERR_NULL, "mp_bias_grad: dy is NULL");
  MP_REQUIRE_OPT_ALIGN(dy);
  const size_t need = colsum_workspace(rows, cols);
  MP_REQUIRE(need == 0 || (ws != nullptr && ws_bytes >= need), MP_ERR_WORKSPACE,
             "mp_bias_grad: workspace needs %zu bytes", need);
  MP_REQUIRE_OPT_ALIGN(ws);
  return colsum(dtype, rows, cols, dy, db, ws, s);
}

extern "C" int mp_vocab_parallel_embedding_bwd(mp_dtype dtype, int64_t T, int64_t Vi, int64_t v_start, int64_t K,
                                               const int32_t* ids, const void* dOut, float* dE_i, int accumulate,
                                               hipStream_t s) {
  static const char* fn = "mp_vocab_parallel_embedding_bwd";
  MP_REQUIRE(dtype_ok(dtype), MP_ERR_DTYPE, "%s: bad dtype %d", fn, static_cast<int>(dtype));
  MP_REQUIRE(T >= 0 && Vi > 0 && v_start >= 0 && K > 0, MP_ERR_SHAPE, "%s: bad shape", fn);
  MP_REQUIRE(K % 8 == 0, MP_ERR_SHAPE, "%s: K=%lld must be a multiple of 8", fn, (long long)K);
  MP_REQUIRE(T == 0 || (ids != nullptr && dOut != nullptr), MP_ERR_NULL, "%s: ids and dOut must be non-NULL", fn);
  MP_REQUIRE_PTR(dE_i);
  MP_REQUIRE_OPT_ALIGN(dOut);
  MP_REQUIRE_ALIGN(dE_i);
  if (int rc = debug_check_range(fn, "ids", ids, T, 0, INT32_MAX + 1LL, s)) return rc;
  const unsigned grid = static_cast<unsigned>(ceil_div(Vi, 16));
  if (dtype == MP_BF16)
    embedding_bwd_kernel<true><<<grid, 256, 0, s>>>(T, Vi, v_start, K, ids, dOut, dE_i, accumulate);
  else
    embedding_bwd_kernel<false><<<grid, 256, 0, s>>>(T, Vi, v_start, K, ids, dOut, dE_i, accumulate);
  return check_launch(fn);
}

extern "C" int mp_all_gather_rows(mp_dtype dtype, int N, int64_t rows, int64_t cols, const void* const* slices,
                                  void* out, hipStream_t s) {
  static const char* fn = "mp_all_gather_rows";
  MP_REQUIRE(dtype_ok(dtype), MP_ERR_DTYPE, "%s: bad dtype %d", fn, static_cast<int>(dtype));
  MP_REQUIRE(N >= 1 && N <= MP_MAX_SHARDS, MP_ERR_SHAPE, "%s: N=%d not in [1, %d]", fn, N, MP_MAX_SHARDS);
  MP_REQUIRE(rows >= 0 && cols > 0 && cols % vec_elems(dtype) == 0, MP_ERR_SHAPE, "%s: bad shape %lld x %lld", fn,
             (long long)rows, (long long)cols);
  MP_REQUIRE_PTR(slices);
  MP_REQUIRE_PTR(out);
  MP_REQUIRE_ALIGN(out);
  PtrArray arr{};
  for (int j = 0; j < N; ++j) {
    MP_REQUIRE(slices[j] != nullptr, MP_ERR_NULL, "%s: slices[%d] is NULL", fn, j);
    MP_REQUIRE((reinterpret_cast<uintptr_t>(slices[j]) & 15u) == 0, MP_ERR_ALIGN,
               "%s: slices[%d] is not 16-byte aligned", fn, j);
    arr.p[j] = slices[j];
  }
  if (rows == 0) return MP_OK;
  const int64_t vps = rows * cols / vec_elems(dtype);
  gather_rows_kernel<<<static_cast<unsigned>(ceil_div(N * vps, 256)), 256, 0, s>>>(arr, N, vps,
                                                                                  static_cast<uint4*>(out));
  return check_launch(fn);
}

extern "C" int mp_vocab_parallel_embedding(mp_dtype dtype, int64_t T, int64_t Vi, int64_t v_start, int64_t K,
                                           const int32_t* ids, const void* E_i, void* out_partial, hipStream_t s) {
  MP_REQUIRE(dtype_ok(dtype), MP_ERR_DTYPE, "mp_vocab_parallel_embedding: bad dtype %d", static_cast<int>(dtype));
  MP_REQUIRE(T >= 0 && Vi > 0 && K > 0 && v_start >= 0, MP_ERR_SHAPE, "mp_vocab_parallel_embedding: bad shape");
  MP_REQUIRE(K % vec_elems(dtype) == 0, MP_ERR_SHAPE, "mp_vocab_parallel_embedding: K=%lld not a multiple of %lld",
             (long long)K, (long long)vec_elems(dtype));
  MP_REQUIRE_PTR(ids);
  MP_REQUIRE_PTR(E_i);
  MP_REQUIRE_PTR(out_partial);
  MP_REQUIRE_ALIGN(E_i);
  MP_REQUIRE_ALIGN(out_partial);
  if (T == 0) return MP_OK;
  if (int rc = debug_check_range("mp_vocab_parallel_embedding", "ids", ids, T, 0, INT32_MAX + 1LL, s)) return rc;
  const int64_t vpr = K / vec_elems(dtype);
  const int64_t nvec = T * vpr;
  embedding_kernel<<<static_cast<unsigned>(ceil_div(nvec, 256)), 256, 0, s>>>(
      nvec, vpr, Vi, v_start, ids, static_cast<const uint4*>(E_i), static_cast<uint4*>(out_partial));
  return check_launch("mp_vocab_parallel_embedding");
}
