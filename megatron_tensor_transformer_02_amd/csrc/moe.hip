// One expert-parallel shard of a MoE layer, with every dynamic shape kept on
// the device (no host synchronisation):
//
//  1. count   -- per token, how many of its top-k picks hit each local expert;
//  2. scan    -- per expert, exclusive prefix of those counts over tokens
//                (deterministic; gives each pick its rank inside its expert);
//  3. offsets -- exclusive scan over experts of the row counts, and of their
//                256-row tile counts (the grouped GEMMs' schedule);
//  4. scatter -- perm_picks[row] = t*topk + k in (expert, token, slot) order,
//                plus the inverse map pick -> row;
//  5. grouped gate/up GEMM -- A rows are gathered straight from X through the
//                permutation (no permuted copy of X), each wave's B rows
//                interleave gate and up rows of the same output columns so
//                the SwiGLU epilogue is local: act = silu(gate) * up;
//  6. grouped down GEMM  -- y = act * W_d^T for each expert's rows;
//  7. unpermute -- out[t] = sum_k w[t,k] * y[row(t,k)], fp32, k ascending.
//
// The grouped GEMMs launch a worst-case grid; a workgroup finds its expert
// and tile from the device-side schedule and exits if it has none.
#include "mfma.h"

namespace mp {

constexpr int MOE_BM = 256, MOE_BN = 256;

struct MoeArgs {
  int64_t T, Hd, Fe;
  int topk, E_loc, e_start;
  int64_t r_cap;           // capacity of the permuted rows (T * topk)
  const uint16_t* X;       // [T, Hd]
  const int32_t* ids;      // [T, topk]
  const float* w;          // [T, topk]
  const uint16_t* W_gu;    // [E_loc, 2*Fe, Hd]
  const uint16_t* W_d;     // [E_loc, Hd, Fe]
  uint16_t* out;           // [T, Hd]
  int32_t* perm;           // [r_cap]
  int32_t* offsets;        // [E_loc + 1]
  int32_t* tile_start;     // [E_loc + 1]
  int32_t* counts;         // [E_loc]
  int32_t* cnt;            // [T, E_loc] per-token counts, then per-token ranks
  int32_t* pick_row;       // [T * topk]
  uint16_t* act;           // [r_cap, Fe]
  uint16_t* yperm;         // [r_cap, Hd]
  int tiles_n;
};

__global__ __launch_bounds__(256) void moe_count_kernel(const MoeArgs a) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= a.T) return;
  int32_t* c = a.cnt + t * a.E_loc;
  for (int e = 0; e < a.E_loc; ++e) c[e] = 0;
  for (int k = 0; k < a.topk; ++k) {
    const int e = a.ids[t * a.topk + k] - a.e_start;
    if (e >= 0 && e < a.E_loc) c[e] += 1;
  }
}

// One block per local expert: exclusive scan of cnt[:, e] over tokens, in
// place, in chunks of 1024 tokens (wave prefix sums + an LDS pass over the
// 16 wave totals).
__global__ __launch_bounds__(1024) void moe_scan_kernel(const MoeArgs a) {
  __shared__ int wsum[16];
  __shared__ int carry_s;
  const int e = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) carry_s = 0;
  __syncthreads();
  for (int64_t base = 0; base < a.T; base += 1024) {
    const int64_t t = base + tid;
    const int v = t < a.T ? a.cnt[t * a.E_loc + e] : 0;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int n = __shfl_up(incl, o, 64);
      if (lane >= o) incl += n;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int before = carry_s;
    for (int w2 = 0; w2 < wave; ++w2) before += wsum[w2];
    if (t < a.T) a.cnt[t * a.E_loc + e] = before + incl - v;
    __syncthreads();
    if (tid == 1023) carry_s = before + incl;
    __syncthreads();
  }
  if (tid == 0) a.counts[e] = carry_s;
}

__global__ void moe_offsets_kernel(const MoeArgs a) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  int off = 0, tiles = 0;
  for (int e = 0; e < a.E_loc; ++e) {
    a.offsets[e] = off;
    a.tile_start[e] = tiles;
    off += a.counts[e];
    tiles += (a.counts[e] + MOE_BM - 1) / MOE_BM;
  }
  a.offsets[a.E_loc] = off;
  a.tile_start[a.E_loc] = tiles;
}

__global__ __launch_bounds__(256) void moe_scatter_kernel(const MoeArgs a) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= a.T) return;
  for (int k = 0; k < a.topk; ++k) {
    const int e = a.ids[t * a.topk + k] - a.e_start;
    int32_t row = -1;
    if (e >= 0 && e < a.E_loc) {
      int dup = 0;  // earlier slots of this token on the same expert
      for (int k2 = 0; k2 < k; ++k2) dup += (a.ids[t * a.topk + k2] - a.e_start) == e;
      row = a.offsets[e] + a.cnt[t * a.E_loc + e] + dup;
      a.perm[row] = static_cast<int32_t>(t * a.topk + k);
    }
    a.pick_row[t * a.topk + k] = row;
  }
}

// Grouped GEMM.  MODE 0: act[rows of e, :] = SwiGLU(X[tokens] W_gu[e]^T);
// MODE 1: yperm[rows of e, :] = act[rows of e] W_d[e]^T.  256x256x64 tiles,
// 4 waves in a 2x2 grid, LDS double buffering as in the dense GEMM.
template <int MODE>
__global__ __launch_bounds__(256) void moe_gemm_kernel(const MoeArgs a) {
  constexpr int BM = MOE_BM, BN = MOE_BN, WM = BM / 2, WN = BN / 2, TM = WM / 32, TN = WN / 32;
  constexpr int A_SLOTS = BM * 8, B_SLOTS = BN * 8, NR = BM * 8 / 256;
  __shared__ uint4 lds[2][A_SLOTS + B_SLOTS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
  const int frow = lane & 31, fgrp = lane >> 5;

  // Device-side schedule: real tiles = tile_start[E_loc] * tiles_n.
  const int n_real = a.tile_start[a.E_loc] * a.tiles_n;
  const int wg = blockIdx.x;
  if (wg >= n_real) return;
  const int per = n_real >> 3, rem = n_real & 7, xcd = wg & 7, idx = wg >> 3;
  const int lid = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + idx;
  const int mtg = lid / a.tiles_n, nt = lid - mtg * a.tiles_n;
  int e = 0;
  while (e + 1 < a.E_loc && a.tile_start[e + 1] <= mtg) ++e;
  const int64_t row0 = a.offsets[e] + static_cast<int64_t>(mtg - a.tile_start[e]) * BM;
  const int64_t row_end = a.offsets[e + 1];
  const int64_t K = MODE == 0 ? a.Hd : a.Fe;

  // Per-thread row offsets (elements) of the A and B rows this thread loads.
  int64_t aoff[NR], boff[NR];
  bool aok[NR], bok[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int r = (tid + 256 * i) >> 3;
    const int64_t grow = row0 + r;
    aok[i] = grow < row_end;
    if constexpr (MODE == 0) {
      aoff[i] = aok[i] ? static_cast<int64_t>(a.perm[grow] / a.topk) * a.Hd : 0;
      // Wave column block wn holds WN/2 gate rows then the WN/2 up rows of the
      // same output columns.
      const int wcol = r / WN, within = r % WN;
      const int64_t j = static_cast<int64_t>(nt) * (BN / 2) + wcol * (WN / 2) + (within % (WN / 2));
      bok[i] = j < a.Fe;
      boff[i] = ((within < WN / 2) ? j : a.Fe + j) * a.Hd;
    } else {
      aoff[i] = grow * a.Fe;
      const int64_t n = static_cast<int64_t>(nt) * BN + r;
      bok[i] = n < a.Hd;
      boff[i] = n * a.Fe;
    }
  }
  const BufRes ra = MODE == 0 ? make_bufres(a.X, a.T * a.Hd * 2) : make_bufres(a.act, a.r_cap * a.Fe * 2);
  const BufRes rb = MODE == 0 ? make_bufres(a.W_gu + static_cast<int64_t>(e) * 2 * a.Fe * a.Hd, 2 * a.Fe * a.Hd * 2)
                              : make_bufres(a.W_d + static_cast<int64_t>(e) * a.Hd * a.Fe, a.Hd * a.Fe * 2);

  uint4 ra_reg[NR], rb_reg[NR];
  auto load = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int64_t gk = k0 + ((tid + 256 * i) & 7) * 8;
      const bool kin = gk < K;
      ra_reg[i] = buf_load16(ra, (aok[i] && kin) ? static_cast<uint32_t>((aoff[i] + gk) * 2) : kBufOOB);
      rb_reg[i] = buf_load16(rb, (bok[i] && kin) ? static_cast<uint32_t>((boff[i] + gk) * 2) : kBufOOB);
    }
  };
  auto store = [&](uint4* tile) {
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int id2 = tid + 256 * i;
      tile[lds_slot(id2 >> 3, id2 & 7)] = ra_reg[i];
      tile[A_SLOTS + lds_slot(id2 >> 3, id2 & 7)] = rb_reg[i];
    }
  };

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nk = static_cast<int>((K + 63) / 64);
  load(0);
  store(lds[0]);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) load(static_cast<int64_t>(kt + 1) * 64);
    const uint4* ta = lds[cur];
    const uint4* tb = lds[cur] + A_SLOTS;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int ch = 2 * ks + fgrp;
      uint4 af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = ta[lds_slot(wm * WM + i * 32 + frow, ch)];
#pragma unroll
      for (int j = 0; j < TN; ++j) bfr[j] = tb[lds_slot(wn * WN + j * 32 + frow, ch)];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma_32x32x16(af[i], bfr[j], acc[i][j]);
    }
    if (more) store(lds[cur ^ 1]);
    __syncthreads();
  }

  // LDS-staged epilogue (see the dense GEMM): one 32-row strip at a time.
  constexpr int SP = WN + 4;
  float* strip = reinterpret_cast<float*>(&lds[0][0]) + wave * 32 * SP;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) strip[mfma_row(r, lane) * SP + j * 32 + frow] = acc[i][j][r];
    __syncthreads();
    constexpr int VPR = MODE == 0 ? WN / 16 : WN / 8;  // output vectors of 8 per strip row
#pragma unroll 1
    for (int v = lane; v < 32 * VPR; v += 64) {
      const int row = v / VPR, c8 = (v - row * VPR) * 8;
      const int64_t grow = row0 + wm * WM + i * 32 + row;
      if (grow >= row_end) continue;
      const float4 g0 = *reinterpret_cast<const float4*>(strip + row * SP + c8);
      const float4 g1 = *reinterpret_cast<const float4*>(strip + row * SP + c8 + 4);
      float val[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
      if constexpr (MODE == 0) {
        const int64_t jcol = static_cast<int64_t>(nt) * (BN / 2) + wn * (WN / 2) + c8;
        if (jcol >= a.Fe) continue;
        const float4 u0 = *reinterpret_cast<const float4*>(strip + row * SP + WN / 2 + c8);
        const float4 u1 = *reinterpret_cast<const float4*>(strip + row * SP + WN / 2 + c8 + 4);
        const float up[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
        for (int q = 0; q < 8; ++q) val[q] = val[q] / (1.0f + expf(-val[q])) * up[q];
        *reinterpret_cast<uint4*>(a.act + grow * a.Fe + jcol) = pack8(val);
      } else {
        const int64_t n = static_cast<int64_t>(nt) * BN + wn * WN + c8;
        if (n >= a.Hd) continue;
        *reinterpret_cast<uint4*>(a.yperm + grow * a.Hd + n) = pack8(val);
      }
    }
    __syncthreads();
  }
}

// out[t, 8c..8c+7] = sum_k w[t,k] * yperm[row(t,k), 8c..8c+7] (k ascending).
__global__ __launch_bounds__(256) void moe_unpermute_kernel(const MoeArgs a) {
  const int64_t vpr = a.Hd / 8;
  const int64_t v = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (v >= a.T * vpr) return;
  const int64_t t = v / vpr, c = (v - t * vpr) * 8;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int k = 0; k < a.topk; ++k) {
    const int32_t row = a.pick_row[t * a.topk + k];
    if (row < 0) continue;
    const float wk = a.w[t * a.topk + k];
    float y[8];
    unpack8(*reinterpret_cast<const uint4*>(a.yperm + static_cast<int64_t>(row) * a.Hd + c), y);
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] += wk * y[q];
  }
  *reinterpret_cast<uint4*>(a.out + t * a.Hd + c) = pack8(acc);
}

struct MoeLayout {
  size_t cnt, pick_row, perm, offsets, tile_start, counts, act, yperm, total;
};

static MoeLayout moe_layout(int64_t T, int64_t Hd, int64_t Fe, int topk, int E_loc) {
  MoeLayout L{};
  const int64_t r_cap = T * topk;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align_up(bytes, 256);
    return at;
  };
  L.cnt = take(static_cast<size_t>(T * E_loc) * 4);
  L.pick_row = take(static_cast<size_t>(T * topk) * 4);
  L.perm = take(static_cast<size_t>(r_cap) * 4);
  L.offsets = take(static_cast<size_t>(E_loc + 1) * 4);
  L.tile_start = take(static_cast<size_t>(E_loc + 1) * 4);
  L.counts = take(static_cast<size_t>(E_loc) * 4);
  L.act = take(static_cast<size_t>(r_cap * Fe) * 2);
  L.yperm = take(static_cast<size_t>(r_cap * Hd) * 2);
  L.total = off;
  return L;
}

}  // namespace mp

using namespace mp;

extern "C" size_t mp_grouped_expert_gemm_workspace(int64_t T, int64_t Hd, int64_t Fe, int topk, int E_loc) {
  if (T < 0 || Hd <= 0 || Fe <= 0 || topk <= 0 || E_loc <= 0) return 0;
  return moe_layout(T, Hd, Fe, topk, E_loc).total;
}

extern "C" int mp_grouped_expert_gemm(int64_t T, int64_t Hd, int64_t Fe, int topk, int E_loc, int e_start,
                                      const void* X, const int32_t* topk_ids, const float* topk_w, const void* W_gu,
                                      const void* W_d, void* out, int32_t* perm_picks, int32_t* expert_offsets,
                                      void* ws, size_t ws_bytes, hipStream_t s) {
  static const char* fn = "mp_grouped_expert_gemm";
  MP_REQUIRE(T >= 0 && Hd > 0 && Fe > 0 && topk > 0 && E_loc > 0 && e_start >= 0, MP_ERR_SHAPE, "%s: bad shape", fn);
  MP_REQUIRE(Hd % 8 == 0 && Fe % 8 == 0, MP_ERR_SHAPE, "%s: Hd and Fe must be multiples of 8", fn);
  MP_REQUIRE(T * Hd * 2 < 0x7fffffffLL && 2 * Fe * Hd * 2 < 0x7fffffffLL && T * topk * Fe * 2 < 0x7fffffffLL,
             MP_ERR_UNSUPPORTED, "%s: an operand exceeds 2 GiB", fn);
  MP_REQUIRE_PTR(X);
  MP_REQUIRE_PTR(topk_ids);
  MP_REQUIRE_PTR(topk_w);
  MP_REQUIRE_PTR(W_gu);
  MP_REQUIRE_PTR(W_d);
  MP_REQUIRE_PTR(out);
  MP_REQUIRE_ALIGN(X);
  MP_REQUIRE_ALIGN(W_gu);
  MP_REQUIRE_ALIGN(W_d);
  MP_REQUIRE_ALIGN(out);
  const MoeLayout L = moe_layout(T, Hd, Fe, topk, E_loc);
  MP_REQUIRE(ws != nullptr && ws_bytes >= L.total, MP_ERR_WORKSPACE, "%s: workspace needs %zu bytes", fn, L.total);
  MP_REQUIRE_ALIGN(ws);
  if (T == 0) return MP_OK;
  char* w = static_cast<char*>(ws);
  MoeArgs a{};
  a.T = T;
  a.Hd = Hd;
  a.Fe = Fe;
  a.topk = topk;
  a.E_loc = E_loc;
  a.e_start = e_start;
  a.r_cap = T * topk;
  a.X = static_cast<const uint16_t*>(X);
  a.ids = topk_ids;
  a.w = topk_w;
  a.W_gu = static_cast<const uint16_t*>(W_gu);
  a.W_d = static_cast<const uint16_t*>(W_d);
  a.out = static_cast<uint16_t*>(out);
  a.cnt = reinterpret_cast<int32_t*>(w + L.cnt);
  a.pick_row = reinterpret_cast<int32_t*>(w + L.pick_row);
  a.perm = perm_picks != nullptr ? perm_picks : reinterpret_cast<int32_t*>(w + L.perm);
  a.offsets = expert_offsets != nullptr ? expert_offsets : reinterpret_cast<int32_t*>(w + L.offsets);
  a.tile_start = reinterpret_cast<int32_t*>(w + L.tile_start);
  a.counts = reinterpret_cast<int32_t*>(w + L.counts);
  a.act = reinterpret_cast<uint16_t*>(w + L.act);
  a.yperm = reinterpret_cast<uint16_t*>(w + L.yperm);
  const unsigned tgrid = static_cast<unsigned>(ceil_div(T, 256));
  moe_count_kernel<<<tgrid, 256, 0, s>>>(a);
  moe_scan_kernel<<<static_cast<unsigned>(E_loc), 1024, 0, s>>>(a);
  moe_offsets_kernel<<<1, 64, 0, s>>>(a);
  moe_scatter_kernel<<<tgrid, 256, 0, s>>>(a);
  const int64_t max_mtiles = ceil_div(a.r_cap, MOE_BM) + E_loc;
  a.tiles_n = static_cast<int>(ceil_div(Fe, MOE_BN / 2));
  moe_gemm_kernel<0><<<static_cast<unsigned>(max_mtiles * a.tiles_n), 256, 0, s>>>(a);
  a.tiles_n = static_cast<int>(ceil_div(Hd, MOE_BN));
  moe_gemm_kernel<1><<<static_cast<unsigned>(max_mtiles * a.tiles_n), 256, 0, s>>>(a);
  moe_unpermute_kernel<<<static_cast<unsigned>(ceil_div(T * (Hd / 8), 256)), 256, 0, s>>>(a);
  return check_launch(fn);
}
