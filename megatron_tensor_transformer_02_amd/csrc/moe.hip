// One expert-parallel shard of a MoE layer, with every dynamic shape kept on
// the device (no host synchronisation):
//
//  1. routing -- per expert, each pick's rank among the expert's picks in
//                (token, slot) order (deterministic), the row counts and their
//                exclusive scan over experts (offsets), the 256-row and 64-row
//                tile lists (the grouped GEMMs' schedule), and
//                perm_picks[row] = t*topk + k in (expert, token, slot) order
//                with the inverse map pick -> row: two kernels over blocks of
//                256 tokens, or count / scan / offsets / scatter kernels for
//                larger shards;
//  2. grouped gate/up GEMM -- A rows are gathered straight from X through the
//                permutation (no permuted copy of X), each wave's B rows
//                interleave gate and up rows of the same output columns so
//                the SwiGLU epilogue is local: act = silu(gate) * up;
//  3. grouped down GEMM  -- y = act * W_d^T for each expert's rows;
//  4. unpermute -- out[t] = sum_k w[t,k] * y[row(t,k)], fp32, k ascending.
//
// The grouped GEMMs launch a worst-case grid; a workgroup finds its expert
// and tile from the device-side schedule and exits if it has none.  Experts
// with few rows run on 64-row tiles in launches of their own, split over k
// with a fixed-order reduce.
#include "gemm.h"
#include "mfma.h"

namespace mp {

constexpr int MOE_BM = 256, MOE_BN = 256;
// Tiles per band of the grouped GEMMs' tile order: one round of workgroups
// (the 256-row kernel's 128 KiB of LDS fit once on each of 256 CUs).
#ifndef MP_MOE_BAND
#define MP_MOE_BAND 256
#endif
constexpr int MOE_BAND = MP_MOE_BAND;
static_assert(MOE_BAND % 8 == 0, "bands start on the first XCD");
// bf16 forward: an expert with fewer rows than this is "sparse" and runs on
// 64-row tiles (a 256-row tile would spend most of its MFMA work on padding).
constexpr int MOE_BM_SPARSE = 64, MOE_SPARSE_ROWS = 192;
// Most 64-row tiles a sparse expert (at most MOE_SPARSE_ROWS - 1 rows) needs:
// the bound the sparse launches' grids are sized by, derived from the same
// constants the offsets kernel counts tiles with.
constexpr int MOE_MAX_STILES = (MOE_SPARSE_ROWS - 1 + MOE_BM_SPARSE - 1) / MOE_BM_SPARSE;
static_assert(MOE_MAX_STILES * MOE_BM_SPARSE >= MOE_SPARSE_ROWS - 1 &&
                  (MOE_MAX_STILES - 1) * MOE_BM_SPARSE < MOE_SPARSE_ROWS - 1,
              "MOE_MAX_STILES is ceil((MOE_SPARSE_ROWS - 1) / MOE_BM_SPARSE)");

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
  int32_t* tile_start;     // [E_loc + 1]: 256-row tiles of every expert
  int32_t* tile_start_d;   // [E_loc + 1]: 256-row tiles of the dense experts only
  int32_t* tile_start_s;   // [E_loc + 1]: 64-row tiles of the sparse experts only
  int32_t* counts;         // [E_loc]
  int32_t* cnt;            // [T, E_loc] per-token counts, then per-token ranks
  int32_t* pick_row;       // [T * topk]
  uint16_t* act;           // [r_cap, Fe]
  uint16_t* yperm;         // [r_cap, Hd]
  int tiles_n;
  int w_on_act;            // routing weight applied to the activation (memory-efficient form)
  // MXFP8 operands: E4M3 codes and E8M0 scales (4 * ceil(K / 128) bytes per row).
  const uint8_t* xq;       // [T, Hd]
  const uint8_t* xs;       // [T, swh]
  const uint8_t* gq;       // [E_loc, 2*Fe, Hd]
  const uint8_t* gs;       // [E_loc, 2*Fe, swh]
  const uint8_t* dq;       // [E_loc, Hd, Fe]
  const uint8_t* ds;       // [E_loc, Hd, swf]
  const uint8_t* aq;       // [r_cap, Fe]
  const uint8_t* as;       // [r_cap, swf]
  int64_t swh, swf;
  // Training: the forward keeps each permuted row's gate and up
  // pre-activations; the backward's operands and outputs.
  uint16_t* gu_save;       // [r_cap, 2*Fe]: gate in [0, Fe), up in [Fe, 2*Fe)
  const uint16_t* dout;    // [T, Hd]
  uint16_t* dy;            // [r_cap, Hd]
  uint16_t* xp;            // [r_cap, Hd]
  float* dw;               // [T, topk]
  float* wperm;            // [r_cap]: each permuted row's routing weight (weighted-activation form)
  float* dwp;              // [r_cap, Fe/8]: parts of each row's routing-weight gradient
  // Split-K sparse launches: k-range split s covers [s * k_per, (s+1) * k_per)
  // (2-byte units, a multiple of 64); its fp32 sums of sparse tile slot row q
  // (64-row tile mtg of the sparse list, row r: q = 64 * mtg + r) go to
  // part[(s * part_rows + q) * width + column], width 2*Fe (gate/up, gate
  // columns first) or Hd (down).
  float* part;
  int64_t part_rows, k_per;
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
  int off = 0, tiles = 0, dense = 0, sparse = 0;
  for (int e = 0; e < a.E_loc; ++e) {
    const int c = a.counts[e];
    a.offsets[e] = off;
    a.tile_start[e] = tiles;
    off += c;
    tiles += (c + MOE_BM - 1) / MOE_BM;
    if (a.tile_start_d != nullptr) {
      a.tile_start_d[e] = dense;
      a.tile_start_s[e] = sparse;
      if (c < MOE_SPARSE_ROWS) sparse += (c + MOE_BM_SPARSE - 1) / MOE_BM_SPARSE;
      else dense += (c + MOE_BM - 1) / MOE_BM;
    }
  }
  a.offsets[a.E_loc] = off;
  a.tile_start[a.E_loc] = tiles;
  if (a.tile_start_d != nullptr) {
    a.tile_start_d[a.E_loc] = dense;
    a.tile_start_s[a.E_loc] = sparse;
  }
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

// Two-kernel routing (T <= MOE_ROUTE_TOKENS, E_loc <= MOE_ROUTE_EXPERTS),
// with the results of the four kernels above.  Blocks of 256 tokens:
//  1. each block counts its tokens' picks per local expert in LDS (one
//     column per thread), scans every expert's column in token order, and
//     gives each pick its rank among the block's picks of that expert (in
//     (token, slot) order), kept in pick_row; the block's totals go to
//     cnt[block, expert];
//  2. each block sums the totals of the blocks before it (its base per
//     expert) and of all blocks (the expert's row count), scans those over
//     experts (offsets; block 0 writes offsets, counts and tile starts) and
//     places every local pick at row offset + base + rank.
constexpr int MOE_ROUTE_TOKENS = 65536, MOE_ROUTE_EXPERTS = 64;

__global__ __launch_bounds__(256) void moe_route_rank_kernel(const MoeArgs a) {
  __shared__ int sc[MOE_ROUTE_EXPERTS][257];  // padded: a wave's 4-value runs fall in distinct banks
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + tid;
  for (int e = 0; e < a.E_loc; ++e) sc[e][tid] = 0;
  // A token's picks are loaded 8 at a time before any is used (every load
  // issued: indexes clamped in range, values past the token's picks unused).
  const int64_t tc = t < a.T ? t : a.T - 1;
  const int64_t plast = a.T * a.topk - 1;
  int le[8];  // local expert of picks k0 .. k0+7 of this token, or -1
  for (int k0 = 0; k0 < a.topk; k0 += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u) le[u] = a.ids[min(tc * a.topk + k0 + u, plast)];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = le[u] - a.e_start;
      if (t < a.T && k0 + u < a.topk && e >= 0 && e < a.E_loc) sc[e][tid] += 1;
    }
  }
  __syncthreads();
  // Exclusive scan of each expert's 256 counts: wave w takes experts w, w+4,
  // ...; lane l sums values 4l .. 4l+3, the wave scans the lane sums.
  for (int e = wave; e < a.E_loc; e += 4) {
    int v[4], sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = sc[e][4 * lane + i];
      sum += v[i];
    }
    int incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int n = __shfl_up(incl, o, 64);
      if (lane >= o) incl += n;
    }
    int run = incl - sum;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sc[e][4 * lane + i] = run;
      run += v[i];
    }
    if (lane == 63) a.cnt[static_cast<int64_t>(blockIdx.x) * a.E_loc + e] = incl;
  }
  __syncthreads();
  if (t >= a.T) return;
  for (int k0 = 0; k0 < a.topk; k0 += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u) le[u] = a.ids[min(t * a.topk + k0 + u, plast)];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = le[u] - a.e_start;
      if (k0 + u < a.topk && e >= 0 && e < a.E_loc)
        a.pick_row[t * a.topk + k0 + u] = sc[e][tid]++;  // a token's repeats in slot order
    }
  }
}

__global__ __launch_bounds__(256) void moe_route_place_kernel(const MoeArgs a) {
  __shared__ int base[MOE_ROUTE_EXPERTS], off[MOE_ROUTE_EXPERTS], tot[MOE_ROUTE_EXPERTS];
  const int tid = threadIdx.x;
  const int b = blockIdx.x, nb = gridDim.x;
  if (tid < a.E_loc) {
    int before = 0, all = 0;
    for (int b0 = 0; b0 < nb; b0 += 8) {  // 8 blocks' totals loaded before any is used
      int c[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) c[u] = a.cnt[static_cast<int64_t>(min(b0 + u, nb - 1)) * a.E_loc + tid];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int cu = b0 + u < nb ? c[u] : 0;
        before += b0 + u < b ? cu : 0;
        all += cu;
      }
    }
    base[tid] = before;
    tot[tid] = all;
  }
  __syncthreads();
  if (tid == 0) {
    int o = 0, tiles = 0, dense = 0, sparse = 0;
    for (int e = 0; e < a.E_loc; ++e) {
      const int c = tot[e];
      off[e] = o;
      if (b == 0) {
        a.offsets[e] = o;
        a.counts[e] = c;
        a.tile_start[e] = tiles;
        if (a.tile_start_d != nullptr) {
          a.tile_start_d[e] = dense;
          a.tile_start_s[e] = sparse;
        }
      }
      o += c;
      tiles += (c + MOE_BM - 1) / MOE_BM;
      if (c < MOE_SPARSE_ROWS) sparse += (c + MOE_BM_SPARSE - 1) / MOE_BM_SPARSE;
      else dense += (c + MOE_BM - 1) / MOE_BM;
    }
    if (b == 0) {
      a.offsets[a.E_loc] = o;
      a.tile_start[a.E_loc] = tiles;
      if (a.tile_start_d != nullptr) {
        a.tile_start_d[a.E_loc] = dense;
        a.tile_start_s[a.E_loc] = sparse;
      }
    }
  }
  __syncthreads();
  const int64_t t = static_cast<int64_t>(b) * 256 + tid;
  if (t >= a.T) return;
  const int64_t plast = a.T * a.topk - 1;
  for (int k0 = 0; k0 < a.topk; k0 += 8) {
    int id[8], rk[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t p = min(t * a.topk + k0 + u, plast);
      id[u] = a.ids[p];
      rk[u] = a.pick_row[p];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (k0 + u >= a.topk) break;
      const int64_t p = t * a.topk + k0 + u;
      const int e = id[u] - a.e_start;
      int32_t row = -1;
      if (e >= 0 && e < a.E_loc) {
        row = off[e] + base[e] + rk[u];
        a.perm[row] = static_cast<int32_t>(p);
      }
      a.pick_row[p] = row;
    }
  }
}

static void launch_routing(const MoeArgs& a, hipStream_t s) {
  if (a.T <= MOE_ROUTE_TOKENS && a.E_loc <= MOE_ROUTE_EXPERTS) {
    const unsigned nb = static_cast<unsigned>(ceil_div(a.T, 256));
    moe_route_rank_kernel<<<nb, 256, 0, s>>>(a);
    moe_route_place_kernel<<<nb, 256, 0, s>>>(a);
    return;
  }
  const unsigned tgrid = static_cast<unsigned>(ceil_div(a.T, 256));
  moe_count_kernel<<<tgrid, 256, 0, s>>>(a);
  moe_scan_kernel<<<static_cast<unsigned>(a.E_loc), 1024, 0, s>>>(a);
  moe_offsets_kernel<<<1, 64, 0, s>>>(a);
  moe_scatter_kernel<<<tgrid, 256, 0, s>>>(a);
}

// Direct global -> LDS loader for a 256-row x 64-k operand tile whose rows
// are gathered: the byte offset of every row this lane fetches (one per copy)
// is computed once per tile, so a row may come from anywhere in the operand
// (a token of X picked by the routing, or a gate/up row of W_gu).  The slot
// layout is that of DmaTile: copy q of wave w fills slots (q*NWV + w)*64 + l
// with tile row q*NWV*8 + w*8 + l/8, chunk (l%8) ^ swz(row).  An absent row,
// a dead copy and a chunk past the k-range get an offset beyond the resource
// in the per-lane (vector) offset, so they are fetched as zeros without
// touching memory; every live address lies inside the operand.
template <int R, int NT>
struct GatherDma {
  static constexpr int NWV = NT / 64, NI = R * 8 / NT;
  static_assert(NWV == 8 && (R * 8) % NT == 0, "8 waves, whole copies");
  static constexpr uint32_t kOOB = 0x80000000u;
  i32x4_t desc;
  uint32_t voff[NI];
  int wave, kc;  // kc: first k-value of this lane's chunk

  // row_off(r) returns the element offset of tile row r from `base`, or -1
  // for a row that must read as zeros.
  template <typename F>
  __device__ __forceinline__ void init(const uint16_t* base, int64_t elems, int tid, F row_off) {
    const int lane = tid & 63;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    desc = make_desc(base, elems * 2);
#pragma unroll
    for (int q = 0; q < NI; ++q) {
      const int r = q * NWV * 8 + wave * 8 + (lane >> 3);
      const int c = (lane & 7) ^ lds_swz(r);
      kc = c * 8;
      const int64_t o = row_off(r);
      voff[q] = o < 0 ? kOOB : static_cast<uint32_t>((o + c * 8) * 2);
    }
  }

  // Fills `tile` with k-values [k0, k0+64); `live` false fills zeros, and
  // chunks at k >= kend read as zeros (kend % 8 == 0).
  __device__ __forceinline__ void issue(uint4* tile, int64_t k0, int64_t kend, bool live) const {
    const uint32_t lb = __builtin_amdgcn_readfirstlane(lds_addr(tile)) + wave * 1024;
    const bool ok = live && k0 + kc < kend;
    const uint32_t so = live ? static_cast<uint32_t>(k0 * 2) : 0u;
#pragma unroll
    for (int q = 0; q < NI; ++q) {
      const uint32_t v = ok ? voff[q] : kOOB;
      const uint32_t m0v = lb + q * NWV * 1024;
      asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds" ::"v"(v), "s"(desc),
                   "s"(m0v), "s"(so)
                   : "memory", "m0");
    }
  }
};

// ------------------------------------------------------------------ MXFP8
// OCP MX: 32-value blocks share an E8M0 exponent floor(log2 max|x|) - 8 (8 is
// E4M3's largest exponent), clamped to [-127, 127], -127 for blocks below
// 2^-126; values become E4M3 codes of x / 2^exponent.

// E4M3 codes of four values (|v| < 2^9), value i in byte i: nearest, ties to
// the even code, saturating at 448 (0x7E); the sign bit is kept, so a value
// rounding to zero gives +-0, and below 2^-6 the grid is the multiples of
// 2^-9.  gfx950's v_cvt_pk_fp8_f32 converts to the OCP E4M3 format with that
// rounding; its out-of-range results are not the saturated code, so values
// are clamped to +-448 first.  Checked against a bit-level encoder of the
// format over every f32 of magnitude below 2^9, both signs: identical codes.
__device__ __forceinline__ uint32_t e4m3x4(float v0, float v1, float v2, float v3) {
  const int w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(v0, -448.0f, 448.0f),
                                                __builtin_amdgcn_fmed3f(v1, -448.0f, 448.0f), 0, false);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(v2, -448.0f, 448.0f),
                                                               __builtin_amdgcn_fmed3f(v3, -448.0f, 448.0f), w, true));
}

// One 32-value MX block held by four consecutive lanes (aligned to 4), eight
// values each: the block's shared exponent se (E8M0 byte se + 127) is the
// largest one that keeps the block's maximum magnitude finite in E4M3 (the
// maximum's exponent minus 8, at least -127), and each value becomes the
// E4M3 code of value * 2^-se (exact scaling).  Returns the eight codes
// (value i in byte i % 4 of word i / 4).  All four lanes must be active.
__device__ __forceinline__ uint2 mx_block8(const float* f, int& se) {
  float mx = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) mx = fmaxf(mx, fabsf(f[i]));
  mx = fmaxf(mx, __shfl_xor(mx, 1, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 2, 64));
  const int e8 = static_cast<int>(__float_as_uint(mx) >> 23);
  se = e8 == 0 ? -127 : max(e8 - 135, -127);
  const float inv = __uint_as_float(static_cast<uint32_t>(127 - se) << 23);  // 2^-se
  return make_uint2(e4m3x4(f[0] * inv, f[1] * inv, f[2] * inv, f[3] * inv),
                    e4m3x4(f[4] * inv, f[5] * inv, f[6] * inv, f[7] * inv));
}

// Rows of x (bf16, row stride ld) to codes q [rows, K] and scales sc
// [rows, sw] (bytes past the last block set to 127); four lanes per block,
// eight values each.
__global__ __launch_bounds__(256) void mx_quantize_kernel(const uint16_t* __restrict__ x, int64_t ld, int64_t rows,
                                                          int64_t K, uint8_t* __restrict__ q,
                                                          uint8_t* __restrict__ sc, int64_t sw) {
  const int64_t v = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t gpr = K / 8;  // a multiple of 4: the four lanes of a block share a row
  const int64_t r = v / gpr;
  if (r >= rows) return;
  const int64_t c = (v - r * gpr) * 8;
  float f[8];
  unpack8(*reinterpret_cast<const uint4*>(x + r * ld + c), f);
  int se;
  *reinterpret_cast<uint2*>(q + r * K + c) = mx_block8(f, se);
  if ((c & 31) == 0) sc[r * sw + c / 32] = static_cast<uint8_t>(se + 127);
  if (c == 0)
    for (int64_t bk = K / 32; bk < sw; ++bk) sc[r * sw + bk] = 127;
}

// Grouped GEMM.  MODE 0: act[rows of e, :] = SwiGLU(X[tokens] W_gu[e]^T);
// MODE 1: yperm[rows of e, :] = act[rows of e] W_d[e]^T.  256x256x64 tiles on
// 8 waves in a 2x4 grid (two per SIMD), each wave owning 128x64 of the tile;
// the same software pipeline as the dense GEMM: both operands stream into two
// LDS buffers by direct loads issued two k-tiles ahead, fragments are
// double-buffered in registers, and the barrier sits inside the last k-step.
// MX: both operands are MXFP8 (E4M3 codes, k-tiles of 128 codes = the same
// 128-byte LDS rows), two scaled 32x32x64 MFMA steps per k-tile, each row's
// four block exponents of a k-tile read as one dword per fragment row.
template <int MODE, bool MX, bool SAVE = false, int BMT = MOE_BM, bool SPLIT = false>
__global__ __launch_bounds__(512) void moe_gemm_kernel(const MoeArgs a) {
  constexpr int BM = BMT, BN = MOE_BN, NT = 512, WC = 4, WM = BM / 2, WN = BN / WC;
  constexpr int TM = WM / 32, TN = WN / 32, A_SLOTS = BM * 8, B_SLOTS = BN * 8;
  static_assert(TN == 2, "the SwiGLU epilogue pairs the gate and up 32-column tiles of a wave");
  // MXFP8: each k-tile buffer also holds the k-tile's exponent dword of every
  // A row (256) and B row (256), 2 KiB, loaded with the tile.
  constexpr int S_SLOTS = MX ? 128 : 0;
  static_assert(!MX || (BM == 256 && BN == 256), "the exponent region covers 256 + 256 rows");
  static_assert(!SPLIT || (!MX && !SAVE && BM == MOE_BM_SPARSE), "split-K runs the bf16 sparse launches");
  __shared__ uint4 lds[2][A_SLOTS + B_SLOTS + S_SLOTS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave / WC, wn = wave % WC;

  // Device-side schedule: real tiles = ts[E_loc] * tiles_n.  MXFP8 runs every
  // expert on 256-row tiles; bf16 splits them into dense experts (256-row
  // tiles) and sparse ones (64-row tiles, a launch of their own).
  const int32_t* ts = MX ? a.tile_start : (BM == MOE_BM ? a.tile_start_d : a.tile_start_s);
  const int n_real = ts[a.E_loc] * a.tiles_n;
  const int wg = blockIdx.x;
  if (wg >= n_real) return;
  // Workgroups are dealt round-robin to the 8 XCDs and start in dispatch
  // order, 256 at a time (one per CU).  The tile list is cut into bands of
  // MOE_BAND consecutive tiles taken in that order, and inside a band each
  // XCD takes a contiguous run: in every round all XCDs work on neighbouring
  // tiles (mostly one expert, whose weight panels they then share through the
  // last-level cache), the workgroups of one XCD on two or three m-tiles
  // (their token rows shared in its L2).
  const int b0 = wg - wg % MOE_BAND, nb = min(MOE_BAND, n_real - b0), w = wg - b0;
  const int per = nb >> 3, rem = nb & 7, xcd = w & 7, idx = w >> 3;
  const int lid = b0 + (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + idx;
  const int mtg = lid / a.tiles_n, nt = lid - mtg * a.tiles_n;
  int e = 0;
  while (e + 1 < a.E_loc && ts[e + 1] <= mtg) ++e;
  const int64_t row0 = a.offsets[e] + static_cast<int64_t>(mtg - ts[e]) * BM;
  const int64_t row_end = a.offsets[e + 1];
  const int64_t K = MODE == 0 ? a.Hd : a.Fe;
  // The loaders count 2-byte units: bf16 values, or pairs of E4M3 codes.
  const int64_t KU = MX ? K / 2 : K;
  auto base16 = [](const uint8_t* q, const uint16_t* h, int64_t off) -> const uint16_t* {
    return MX ? reinterpret_cast<const uint16_t*>(q + off) : h + off;
  };

  // Gate/up weight row (within expert e) of B tile row r, or -1: wave column
  // block c holds WN/2 gate rows, then the WN/2 up rows of the same output
  // columns.
  auto gu_row = [&](int r) -> int64_t {
    const int wcol = r / WN, within = r % WN;
    const int64_t j = static_cast<int64_t>(nt) * (BN / 2) + wcol * (WN / 2) + (within % (WN / 2));
    if (j >= a.Fe) return -1;
    return (within < WN / 2) ? j : a.Fe + j;
  };
  const int64_t n0 = static_cast<int64_t>(nt) * BN;
  GatherDma<BM, NT> da;
  GatherDma<BN, NT> db;
  if constexpr (MODE == 0) {
    da.init(base16(a.xq, a.X, 0), a.T * KU, tid, [&](int r) -> int64_t {
      const int64_t grow = row0 + r;
      return grow < row_end ? static_cast<int64_t>(a.perm[grow] / a.topk) * KU : -1;
    });
    db.init(base16(a.gq, a.W_gu, static_cast<int64_t>(e) * 2 * a.Fe * a.Hd), 2 * a.Fe * KU, tid,
            [&](int r) -> int64_t {
              const int64_t w = gu_row(r);
              return w < 0 ? -1 : w * KU;
            });
  } else {
    da.init(base16(a.aq, a.act, row0 * a.Fe), (row_end - row0) * KU, tid,
            [&](int r) -> int64_t { return row0 + r < row_end ? static_cast<int64_t>(r) * KU : -1; });
    db.init(base16(a.dq, a.W_d, static_cast<int64_t>(e) * a.Hd * a.Fe + n0 * a.Fe), (a.Hd - n0) * KU, tid,
            [&](int r) -> int64_t { return n0 + r < a.Hd ? static_cast<int64_t>(r) * KU : -1; });
  }
  constexpr int NI = GatherDma<BM, NT>::NI + GatherDma<BN, NT>::NI;
  // This workgroup's k-range (all of K, or split blockIdx.y's share).
  const int64_t kb = SPLIT ? static_cast<int64_t>(blockIdx.y) * a.k_per : 0;
  const int64_t ke = SPLIT ? min(KU, kb + a.k_per) : KU;
  const int nk = ke > kb ? static_cast<int>((ke - kb + 63) / 64) : 0;
  auto fill = [&](uint4* buf, int t) {
    const int64_t k0 = kb + 64 * static_cast<int64_t>(t);
    da.issue(buf, k0, ke, t < nk);
    db.issue(buf + A_SLOTS, k0, ke, t < nk);
  };

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int ar0 = wm * WM, br0 = wn * WN;
  if constexpr (MX) {
    // Exponents travel with their k-tile: the dword of k-tile t of each A and
    // B row goes global -> LDS by the same direct loads as the codes (wave w
    // fills dwords w*64 .. +63 of the buffer's exponent region: A rows, then
    // B rows), so they are complete at the same barrier and are read from LDS
    // like the fragments, never waited for as separate loads.  A row with no
    // data (past the expert's rows, or a gate/up row past Fe) reads zeros:
    // its codes are zeros too, so its products are 0 whatever the scale.
    i32x4_t sdesc;
    uint32_t svoff;
    {
      const int r = (wave & 3) * 64 + lane;
      int64_t off = -1;
      if (wave < 4) {
        const int64_t grow = row0 + r;
        if (grow < row_end)
          off = MODE == 0 ? static_cast<int64_t>(a.perm[grow] / a.topk) * a.swh : grow * a.swf;
        sdesc = MODE == 0 ? make_desc(a.xs, a.T * a.swh) : make_desc(a.as, a.r_cap * a.swf);
      } else {
        if constexpr (MODE == 0) {
          const int64_t w = gu_row(r);
          if (w >= 0) off = (static_cast<int64_t>(e) * 2 * a.Fe + w) * a.swh;
          sdesc = make_desc(a.gs, static_cast<int64_t>(a.E_loc) * 2 * a.Fe * a.swh);
        } else {
          if (n0 + r < a.Hd) off = (static_cast<int64_t>(e) * a.Hd + n0 + r) * a.swf;
          sdesc = make_desc(a.ds, static_cast<int64_t>(a.E_loc) * a.Hd * a.swf);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sdesc[i] = __builtin_amdgcn_readfirstlane(sdesc[i]);
      svoff = off < 0 ? 0x80000000u : static_cast<uint32_t>(off);
    }
    auto sfill = [&](uint4* buf, int t) {
      const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr(buf + A_SLOTS + B_SLOTS) + wave * 256);
      const uint32_t so = __builtin_amdgcn_readfirstlane(t < nk ? static_cast<uint32_t>(4 * t) : 0x80000000u);
      asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, %3 offen lds" ::"v"(svoff), "s"(sdesc),
                   "s"(m0v), "s"(so)
                   : "memory", "m0");
    };
    // Lane l < 32 supplies block 0 of each 64-code step, lane l + 32 block 1:
    // shifting the k-tile's dword by a byte for the upper lanes makes byte 0
    // (step 0) and byte 2 (step 1) the right exponents for every lane.
    const int shift = 8 * (lane >> 5);
    uint32_t sa[TM], sb[TN];
    auto read_scales = [&](const uint4* buf, uint32_t* ra, uint32_t* rb) {
      const uint32_t* sd = reinterpret_cast<const uint32_t*>(buf + A_SLOTS + B_SLOTS);
#pragma unroll
      for (int i = 0; i < TM; ++i) ra[i] = sd[ar0 + 32 * i + (lane & 31)];
#pragma unroll
      for (int j = 0; j < TN; ++j) rb[j] = sd[256 + br0 + 32 * j + (lane & 31)];
    };
    fill(lds[0], 0);
    sfill(lds[0], 0);
    fill(lds[1], 1);
    sfill(lds[1], 1);
    wait_vm_lds();
    __syncthreads();
    read_scales(lds[0], sa, sb);
#pragma unroll
    for (int i = 0; i < TM; ++i) sa[i] >>= shift;
#pragma unroll
    for (int j = 0; j < TN; ++j) sb[j] >>= shift;
    // Software pipeline in registers: a fragment is reloaded as soon as its
    // last MFMA of the step is issued (step 0's A fragments become step 1's,
    // step 1's become the next k-tile's step 0), and the barrier sits after
    // the first half of step 1, when every read of the k-tile has returned.
    constexpr int H = TM / 2;
    uint4 fa0[TM], fa1[TM], fb0[TN], fb1[TN];
    auto load_a = [&](const uint4* t, int i, int step) {
      fa0[i] = lds_frag<true>(t, ar0 + 32 * i, 2 * step, lane);
      fa1[i] = lds_frag<true>(t, ar0 + 32 * i, 2 * step + 1, lane);
    };
    auto load_b = [&](const uint4* t, int j, int step) {
      fb0[j] = lds_frag<true>(t + A_SLOTS, br0 + 32 * j, 2 * step, lane);
      fb1[j] = lds_frag<true>(t + A_SLOTS, br0 + 32 * j, 2 * step + 1, lane);
    };
#pragma unroll
    for (int i = 0; i < TM; ++i) load_a(lds[0], i, 0);
#pragma unroll
    for (int j = 0; j < TN; ++j) load_b(lds[0], j, 0);
    for (int kt = 0; kt < nk; ++kt) {
      uint4* cur = lds[kt & 1];
      const uint4* nxt = lds[(kt & 1) ^ 1];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = mfma_mx_32x32x64<0>(fa0[i], fa1[i], fb0[j], fb1[j], sa[i], sb[j], acc[i][j]);
        load_a(cur, i, 1);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) load_b(cur, j, 1);
#pragma unroll
      for (int i = 0; i < H; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = mfma_mx_32x32x64<2>(fa0[i], fa1[i], fb0[j], fb1[j], sa[i], sb[j], acc[i][j]);
      wait_vm_lds();  // k-tile kt+1 and its exponents have landed; reads of kt retired
      __syncthreads();
      uint32_t na[TM], nb[TN];  // the next k-tile's exponents, read under this step's MFMAs
      read_scales(nxt, na, nb);
      fill(cur, kt + 2);
      sfill(cur, kt + 2);
#pragma unroll
      for (int i = 0; i < H; ++i) load_a(nxt, i, 0);
#pragma unroll
      for (int i = H; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = mfma_mx_32x32x64<2>(fa0[i], fa1[i], fb0[j], fb1[j], sa[i], sb[j], acc[i][j]);
        load_a(nxt, i, 0);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) load_b(nxt, j, 0);
#pragma unroll
      for (int i = 0; i < TM; ++i) sa[i] = na[i] >> shift;
#pragma unroll
      for (int j = 0; j < TN; ++j) sb[j] = nb[j] >> shift;
    }
  } else {
  fill(lds[0], 0);
  fill(lds[1], 1);
  wait_vmcnt<NI>();
  __syncthreads();

  constexpr int NR = TM + TN, NM = TM * TN, H = TM / 2;  // H = 0 for 64-row tiles: all after the barrier
  uint4 fa[2][TM], fb[2][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) fa[0][i] = lds_frag<true>(lds[0], ar0 + 32 * i, 0, lane);
#pragma unroll
  for (int j = 0; j < TN; ++j) fb[0][j] = lds_frag<true>(lds[0] + A_SLOTS, br0 + 32 * j, 0, lane);

  for (int kt = 0; kt < nk; ++kt) {
    uint4* cur = lds[kt & 1];
    const uint4* ta = cur;
    const uint4* tb = cur + A_SLOTS;
    const uint4* na = lds[(kt & 1) ^ 1];
#pragma unroll
    for (int ks = 0; ks < 3; ++ks) {
      const int c = ks & 1, n = c ^ 1;
#pragma unroll
      for (int i = 0; i < TM; ++i) fa[n][i] = lds_frag<true>(ta, ar0 + 32 * i, ks + 1, lane);
#pragma unroll
      for (int j = 0; j < TN; ++j) fb[n][j] = lds_frag<true>(tb, br0 + 32 * j, ks + 1, lane);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma_32x32x16(fa[c][i], fb[c][j], acc[i][j]);
      sched_mfma_interleave<0, NM, 0x100, NR, 0>();
    }
#pragma unroll
    for (int i = 0; i < H; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = mfma_32x32x16(fa[1][i], fb[1][j], acc[i][j]);
    wait_vm_lds();  // k-tile kt+1 has landed (this wave's share); reads of kt retired
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[0][i] = lds_frag<true>(na, ar0 + 32 * i, 0, lane);
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[0][j] = lds_frag<true>(na + A_SLOTS, br0 + 32 * j, 0, lane);
    fill(cur, kt + 2);
#pragma unroll
    for (int i = H; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = mfma_32x32x16(fa[1][i], fb[1][j], acc[i][j]);
  }
  }
  wait_vm_lds();  // the trailing (all-zero) loads write LDS the epilogue reuses
  __syncthreads();

  if constexpr (SPLIT) {
    // fp32 sums of this k-range straight from the accumulators (lane l holds
    // column l % 32 of each 32x32 tile: 128 contiguous bytes per tile row);
    // the reduce applies the epilogue.
    const int64_t width = MODE == 0 ? 2 * a.Fe : a.Hd;
    float* P = a.part + (static_cast<int64_t>(blockIdx.y) * a.part_rows + static_cast<int64_t>(mtg) * BM) * width;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      int64_t col;
      if constexpr (MODE == 0) {
        const int64_t jcol = static_cast<int64_t>(nt) * (BN / 2) + wn * (WN / 2) + (lane & 31);
        col = jcol < a.Fe ? jcol + j * a.Fe : -1;
      } else {
        const int64_t n = n0 + wn * WN + j * 32 + (lane & 31);
        col = n < a.Hd ? n : -1;
      }
      if (col < 0) continue;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rr = wm * WM + i * 32 + mfma_row(r, lane);
          if (row0 + rr < row_end) P[rr * width + col] = acc[i][j][r];
        }
    }
    return;
  }

  // Epilogue through a wave-private LDS strip, one 32-row strip at a time (as
  // in the dense GEMM; no barrier needed).  MODE 0: lane l holds the gate and
  // the up value of the same output column (l % 32) in its two accumulator
  // tiles, so SwiGLU is applied in registers and the strip is 32 columns wide.
  constexpr int SC = MODE == 0 ? WN / 2 : WN;  // strip columns
  constexpr int SP = SC + 4;                   // padded strip row (floats)
  constexpr int VPR = SC / 8, NV = 32 * VPR / 64;
  static_assert((32 * VPR) % 64 == 0, "strip vectors must cover the wave evenly");
  // SAVE (MODE 0): two more passes through the strip first store the gate and
  // the up pre-activations of the same outputs (for the backward).
  constexpr int NPASS = MODE == 0 && SAVE ? 3 : 1;
  float* strip = reinterpret_cast<float*>(&lds[0][0]) + wave * 32 * SP;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
  for (int pass = 0; pass < NPASS; ++pass) {
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int srow = mfma_row(r, lane) * SP + (lane & 31);
      if constexpr (MODE == 0) {
        // silu(g) = g / (1 + e^-g): e^-g by the hardware exp2, the division
        // by v_rcp_f32 (about 1 ulp each, far below the bf16 output's
        // resolution); large |g| still gives g or -0.
        const float g = acc[i][0][r];
        if (pass + 1 < NPASS) {
          strip[srow] = pass == 0 ? g : acc[i][1][r];
        } else {
          const float e = __builtin_amdgcn_exp2f(-1.4426950408889634f * g);
          strip[srow] = g * __builtin_amdgcn_rcpf(1.0f + e) * acc[i][1][r];
        }
      } else {
        strip[srow] = acc[i][0][r];
        strip[srow + 32] = acc[i][1][r];
      }
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int it = 0; it < NV; ++it) {
      const int v = lane + 64 * it;
      const int row = v / VPR, c8 = (v - row * VPR) * 8;
      const int64_t grow = row0 + wm * WM + i * 32 + row;
      const float4 lo = *reinterpret_cast<const float4*>(strip + row * SP + c8);
      const float4 hi = *reinterpret_cast<const float4*>(strip + row * SP + c8 + 4);
      float val[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      if (grow >= row_end) continue;
      if constexpr (MODE == 0) {
        const int64_t jcol = static_cast<int64_t>(nt) * (BN / 2) + wn * (WN / 2) + c8;
        if (jcol >= a.Fe) continue;
        if (pass + 1 < NPASS) {
          *reinterpret_cast<uint4*>(a.gu_save + grow * 2 * a.Fe + pass * a.Fe + jcol) = pack8(val);
          continue;
        }
        if (a.w_on_act) {  // the row's routing weight, before the bf16 rounding
          const float wr = a.w[a.perm[grow]];
#pragma unroll
          for (int q = 0; q < 8; ++q) val[q] *= wr;
        }
        if constexpr (MX) {
          // The activation is rounded to bf16, then quantised: the wave's 32
          // columns are one MX block of the row (Fe is a multiple of 32), held
          // by the row's four consecutive lanes.  The lane of the block's
          // first 8 values writes its exponent, and, for the row's last
          // block, the padding bytes of the row's scale record.
          float f[8];
          unpack8(pack8(val), f);
          int se;
          *reinterpret_cast<uint2*>(const_cast<uint8_t*>(a.aq) + grow * a.Fe + jcol) = mx_block8(f, se);
          if (c8 == 0) {
            uint8_t* srow = const_cast<uint8_t*>(a.as) + grow * a.swf;
            srow[jcol / 32] = static_cast<uint8_t>(se + 127);
            if (jcol + 32 == a.Fe)
              for (int64_t bk = a.Fe / 32; bk < a.swf; ++bk) srow[bk] = 127;
          }
        } else {
          *reinterpret_cast<uint4*>(a.act + grow * a.Fe + jcol) = pack8(val);
        }
      } else {
        const int64_t n = static_cast<int64_t>(nt) * BN + wn * WN + c8;
        if (n >= a.Hd) continue;
        *reinterpret_cast<uint4*>(a.yperm + grow * a.Hd + n) = pack8(val);
      }
    }
  }
  }
}

__device__ __forceinline__ void unpack_f32x8(const float* p, float* f) {
  const float4 lo = *reinterpret_cast<const float4*>(p), hi = *reinterpret_cast<const float4*>(p + 4);
  f[0] = lo.x; f[1] = lo.y; f[2] = lo.z; f[3] = lo.w;
  f[4] = hi.x; f[5] = hi.y; f[6] = hi.z; f[7] = hi.w;
}

// Reduce of the split-K sparse launches: the row's fp32 sums over the splits
// in split order, then the epilogue the unsplit kernel applies.  MODE 0:
// act = silu(gate) * up (times the routing weight with w_on_act), bf16, and
// with SAVE the gate and up sums as bf16 pre-activations; MODE 1: yperm in
// bf16.  Thread: 8 columns of one slot row; slots without a row exit.
template <int MODE, bool SAVE>
__global__ __launch_bounds__(256) void moe_splitk_reduce_kernel(const MoeArgs a, int splits) {
  constexpr int SB = MOE_BM_SPARSE;
  const int64_t nc = MODE == 0 ? a.Fe : a.Hd, width = MODE == 0 ? 2 * a.Fe : a.Hd, vpr = nc / 8;
  const int64_t v = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t q = v / vpr;
  if (q >= a.part_rows) return;
  const int64_t c = (v - q * vpr) * 8;
  const int32_t* ts = a.tile_start_s;
  const int mtg = static_cast<int>(q / SB);
  if (mtg >= ts[a.E_loc]) return;
  int e = 0;
  while (e + 1 < a.E_loc && ts[e + 1] <= mtg) ++e;
  const int64_t grow = a.offsets[e] + static_cast<int64_t>(mtg - ts[e]) * SB + (q - static_cast<int64_t>(mtg) * SB);
  if (grow >= a.offsets[e + 1]) return;
  float x[8], u[8];
  for (int sp = 0; sp < splits; ++sp) {
    const float* p = a.part + (static_cast<int64_t>(sp) * a.part_rows + q) * width + c;
    float px[8], pu[8];
    unpack_f32x8(p, px);
    if constexpr (MODE == 0) unpack_f32x8(p + a.Fe, pu);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[i] = sp == 0 ? px[i] : x[i] + px[i];
      if constexpr (MODE == 0) u[i] = sp == 0 ? pu[i] : u[i] + pu[i];
    }
  }
  if constexpr (MODE == 0) {
    if constexpr (SAVE) {
      *reinterpret_cast<uint4*>(a.gu_save + grow * 2 * a.Fe + c) = pack8(x);
      *reinterpret_cast<uint4*>(a.gu_save + grow * 2 * a.Fe + a.Fe + c) = pack8(u);
    }
    // The same SwiGLU evaluation as the grouped GEMM's epilogue.
    float val[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float ex = __builtin_amdgcn_exp2f(-1.4426950408889634f * x[i]);
      val[i] = x[i] * __builtin_amdgcn_rcpf(1.0f + ex) * u[i];
    }
    if (a.w_on_act) {
      const float wr = a.w[a.perm[grow]];
#pragma unroll
      for (int i = 0; i < 8; ++i) val[i] *= wr;
    }
    *reinterpret_cast<uint4*>(a.act + grow * a.Fe + c) = pack8(val);
  } else {
    *reinterpret_cast<uint4*>(a.yperm + grow * a.Hd + c) = pack8(x);
  }
}

// out[t, 8c..8c+7] = sum_k w[t,k] * yperm[row(t,k), 8c..8c+7] (k ascending;
// w = 1 when the weights were applied to the activation).  A token's row is
// split over tpt = ceil(Hd / 32) threads, thread i owning chunks i, i + tpt,
// i + 2 tpt, i + 3 tpt of 8 columns (consecutive threads, consecutive
// chunks), so the token's pick rows and weights are loaded once for four
// chunks.  With KMAX > 0 (topk <= KMAX) every pick's row index, weight and
// row chunks are loaded before the sum, so the loads of one token overlap;
// the sum keeps the k order.
#ifndef MP_UNPERM_CH
#define MP_UNPERM_CH 4
#endif
constexpr int UNPERM_CH = MP_UNPERM_CH;
template <int KMAX>
__global__ __launch_bounds__(256) void moe_unpermute_kernel(const MoeArgs a) {
  const int64_t vpr = a.Hd / 8, tpt = (vpr + UNPERM_CH - 1) / UNPERM_CH;
  const int64_t v = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (v >= a.T * tpt) return;
  const int64_t t = v / tpt, i = v - t * tpt;
  float acc[UNPERM_CH][8] = {};
  if constexpr (KMAX > 0) {
    int32_t rows[KMAX];
    float wk[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      rows[k] = k < a.topk ? a.pick_row[t * a.topk + k] : -1;
      wk[k] = k < a.topk && !a.w_on_act ? a.w[t * a.topk + k] : 1.0f;
    }
    uint4 yv[UNPERM_CH][KMAX];
#pragma unroll
    for (int j = 0; j < UNPERM_CH; ++j) {
      const int64_t ch = i + j * tpt;
#pragma unroll
      for (int k = 0; k < KMAX; ++k)
        yv[j][k] = rows[k] >= 0 && ch < vpr
                       ? *reinterpret_cast<const uint4*>(a.yperm + static_cast<int64_t>(rows[k]) * a.Hd + ch * 8)
                       : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < UNPERM_CH; ++j)
#pragma unroll
      for (int k = 0; k < KMAX; ++k) {
        if (rows[k] < 0) continue;
        float y[8];
        unpack8(yv[j][k], y);
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[j][q] += wk[k] * y[q];
      }
  } else {
    for (int k = 0; k < a.topk; ++k) {
      const int32_t row = a.pick_row[t * a.topk + k];
      if (row < 0) continue;
      const float wk = a.w_on_act ? 1.0f : a.w[t * a.topk + k];
#pragma unroll
      for (int j = 0; j < UNPERM_CH; ++j) {
        const int64_t ch = i + j * tpt;
        if (ch >= vpr) break;
        float y[8];
        unpack8(*reinterpret_cast<const uint4*>(a.yperm + static_cast<int64_t>(row) * a.Hd + ch * 8), y);
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[j][q] += wk * y[q];
      }
    }
  }
#pragma unroll
  for (int j = 0; j < UNPERM_CH; ++j) {
    const int64_t ch = i + j * tpt;
    if (ch < vpr) *reinterpret_cast<uint4*>(a.out + t * a.Hd + ch * 8) = pack8(acc[j]);
  }
}

// Backward, one wave per permuted row r < R: with pick p = perm[r] of token
// t = p / topk, dy[r] = w[p] * dout[t] (bf16), xp[r] = X[t] (the gathered
// input rows of the gate/up weight gradient) and dw[p] = dout[t] . yperm[r]
// in fp32 (each lane sums its columns in order, then a fixed shuffle tree).
// W_ON_ACT (the weighted-activation form): the unpermute was unweighted, so
// dy[r] = dout[t]; the row's weight goes to wperm[r] for the d act GEMM, and
// dw comes from the activation side there (no expert output is read).
template <bool W_ON_ACT>
__global__ __launch_bounds__(256) void moe_bwd_rows_kernel(const MoeArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (r >= a.offsets[a.E_loc]) return;
  const int32_t p = a.perm[r];
  const int64_t t = p / a.topk;
  const float wv = a.w[p];
  if constexpr (W_ON_ACT) {
    if (lane == 0) a.wperm[r] = wv;
    for (int64_t c = lane * 8; c < a.Hd; c += 512) {
      *reinterpret_cast<uint4*>(a.dy + r * a.Hd + c) = *reinterpret_cast<const uint4*>(a.dout + t * a.Hd + c);
      *reinterpret_cast<uint4*>(a.xp + r * a.Hd + c) = *reinterpret_cast<const uint4*>(a.X + t * a.Hd + c);
    }
    return;
  }
  const uint16_t* go = a.dout + t * a.Hd;
  const uint16_t* yr = a.yperm + r * a.Hd;
  const uint16_t* xr = a.X + t * a.Hd;
  float dot = 0.0f;
  for (int64_t c = lane * 8; c < a.Hd; c += 512) {
    float gv[8], yv[8];
    unpack8(*reinterpret_cast<const uint4*>(go + c), gv);
    unpack8(*reinterpret_cast<const uint4*>(yr + c), yv);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      dot += gv[q] * yv[q];
      gv[q] *= wv;
    }
    *reinterpret_cast<uint4*>(a.dy + r * a.Hd + c) = pack8(gv);
    *reinterpret_cast<uint4*>(a.xp + r * a.Hd + c) = *reinterpret_cast<const uint4*>(xr + c);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) dot += __shfl_xor(dot, o, 64);
  if (lane == 0) a.dw[p] = dot;
}

// n fp32 zeros (a kernel rather than a memset, so the call stays capturable).
__global__ __launch_bounds__(256) void moe_zero_f32_kernel(float* p, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

// Weighted-activation form: dw[perm[r]] = sum of row r's Fe/8 parts from the
// d act GEMM's epilogue (one wave per row; lane order, then a fixed tree).
__global__ __launch_bounds__(256) void moe_bwd_dw_rows_kernel(const MoeArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (r >= a.offsets[a.E_loc]) return;
  const int64_t np = a.Fe / 8;
  float acc = 0.0f;
  for (int64_t c = lane; c < np; c += 64) acc += a.dwp[r * np + c];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if (lane == 0) a.dw[a.perm[r]] = acc;
}

// The routing-weight gradient of picks held by other shards is zero.
__global__ __launch_bounds__(256) void moe_bwd_dw_zero_kernel(const MoeArgs a) {
  const int64_t p = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (p < a.T * a.topk && a.pick_row[p] < 0) a.dw[p] = 0.0f;
}

static void launch_unpermute(const MoeArgs& a, hipStream_t s) {
  const unsigned grid = static_cast<unsigned>(ceil_div(a.T * ceil_div(a.Hd / 8, UNPERM_CH), 256));
  if (a.topk <= 8) moe_unpermute_kernel<8><<<grid, 256, 0, s>>>(a);
  else moe_unpermute_kernel<0><<<grid, 256, 0, s>>>(a);
}

struct MoeLayout {
  size_t cnt, pick_row, perm, offsets, tile_start, tile_start_d, tile_start_s, counts, act, yperm, xq, xs, aq, as,
      part, total;
};

static int64_t mx_scale_width(int64_t K) { return 4 * ceil_div(K, 128); }

// k-range splits of a bf16 sparse launch (64-row tiles) over a reduction of
// K values.  A sparse shard has one tile-row per expert, so its launches have
// few workgroups, each streaming a slice of the experts' weights; every split
// adds a full set of them.  Each split keeps at least 8 k-tiles.
#ifndef MP_MOE_SPARSE_KSPLIT
#define MP_MOE_SPARSE_KSPLIT 2
#endif
static int sparse_splits(int64_t K) {
  const int64_t nk = ceil_div(K, 64);
  return static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(MP_MOE_SPARSE_KSPLIT, nk / 8)));
}
// Slot rows of the sparse tiles (MOE_MAX_STILES per expert).
static int64_t sparse_slot_rows(int E_loc) { return static_cast<int64_t>(MOE_MAX_STILES) * E_loc * MOE_BM_SPARSE; }

// With mx, the quantised token rows and activations follow the bf16 buffers.
static MoeLayout moe_layout(int64_t T, int64_t Hd, int64_t Fe, int topk, int E_loc, bool mx = false) {
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
  L.tile_start_d = take(static_cast<size_t>(E_loc + 1) * 4);
  L.tile_start_s = take(static_cast<size_t>(E_loc + 1) * 4);
  L.counts = take(static_cast<size_t>(E_loc) * 4);
  L.act = take(mx ? 0 : static_cast<size_t>(r_cap * Fe) * 2);  // MXFP8 keeps only the quantised activation
  L.yperm = take(static_cast<size_t>(r_cap * Hd) * 2);
  // fp32 partial sums of the split sparse launches (one launch at a time).
  const int64_t part_w = mx ? 0
                            : std::max<int64_t>(sparse_splits(Hd) > 1 ? sparse_splits(Hd) * 2 * Fe : 0,
                                                sparse_splits(Fe) > 1 ? sparse_splits(Fe) * Hd : 0);
  L.part = take(static_cast<size_t>(part_w * sparse_slot_rows(E_loc)) * 4);
  if (mx) {
    L.xq = take(static_cast<size_t>(T * Hd));
    L.xs = take(static_cast<size_t>(T * mx_scale_width(Hd)));
    L.aq = take(static_cast<size_t>(r_cap * Fe));
    L.as = take(static_cast<size_t>(r_cap * mx_scale_width(Fe)));
  }
  L.total = off;
  return L;
}

}  // namespace mp

using namespace mp;

extern "C" size_t mp_grouped_expert_gemm_workspace(int64_t T, int64_t Hd, int64_t Fe, int topk, int E_loc) {
  if (T < 0 || Hd <= 0 || Fe <= 0 || topk <= 0 || E_loc <= 0) return 0;
  return moe_layout(T, Hd, Fe, topk, E_loc).total;
}

static int grouped_expert_gemm(const char* fn, bool w_on_act, int64_t T, int64_t Hd, int64_t Fe, int topk,
                               int E_loc, int e_start, const void* X, const int32_t* topk_ids, const float* topk_w,
                               const void* W_gu, const void* W_d, void* out, int32_t* perm_picks,
                               int32_t* expert_offsets, void* ws, size_t ws_bytes, hipStream_t s,
                               void* gu_save = nullptr) {
  MP_REQUIRE(T >= 0 && Hd > 0 && Fe > 0 && topk > 0 && E_loc > 0 && e_start >= 0, MP_ERR_SHAPE, "%s: bad shape", fn);
  MP_REQUIRE(Hd % 8 == 0 && Fe % 8 == 0, MP_ERR_SHAPE, "%s: Hd and Fe must be multiples of 8", fn);
  MP_REQUIRE(T * Hd * 2 < 0x7fffffffLL && 2 * Fe * Hd * 2 < 0x7fffffffLL && T * topk * Fe * 2 < 0x7fffffffLL,
             MP_ERR_UNSUPPORTED, "%s: an operand exceeds 2 GiB", fn);
  if (T == 0) return MP_OK;  // no tokens: nothing is read or written
  MP_REQUIRE_PTR(X);
  MP_REQUIRE_PTR(topk_ids);
  MP_REQUIRE_PTR(topk_w);
  MP_REQUIRE_PTR(W_gu);
  MP_REQUIRE_PTR(W_d);
  MP_REQUIRE_PTR(out);
  if (int rc = debug_check_range(fn, "topk_ids", topk_ids, T * topk, 0, INT32_MAX + 1LL, s)) return rc;
  MP_REQUIRE_ALIGN(X);
  MP_REQUIRE_ALIGN(W_gu);
  MP_REQUIRE_ALIGN(W_d);
  MP_REQUIRE_ALIGN(out);
  const MoeLayout L = moe_layout(T, Hd, Fe, topk, E_loc);
  MP_REQUIRE(ws != nullptr && ws_bytes >= L.total, MP_ERR_WORKSPACE, "%s: workspace needs %zu bytes", fn, L.total);
  MP_REQUIRE_ALIGN(ws);
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
  a.tile_start_d = reinterpret_cast<int32_t*>(w + L.tile_start_d);
  a.tile_start_s = reinterpret_cast<int32_t*>(w + L.tile_start_s);
  a.counts = reinterpret_cast<int32_t*>(w + L.counts);
  a.act = reinterpret_cast<uint16_t*>(w + L.act);
  a.yperm = reinterpret_cast<uint16_t*>(w + L.yperm);
  a.w_on_act = w_on_act ? 1 : 0;
  a.gu_save = static_cast<uint16_t*>(gu_save);
  a.part = reinterpret_cast<float*>(w + L.part);
  a.part_rows = sparse_slot_rows(E_loc);
  launch_routing(a, s);
  // Dense experts' 256-row tiles and sparse experts' 64-row tiles (each
  // sparse expert has at most MOE_MAX_STILES); the two launches cover
  // disjoint rows.
  const int64_t max_mtiles = ceil_div(a.r_cap, MOE_BM) + E_loc,
                max_stiles = static_cast<int64_t>(MOE_MAX_STILES) * E_loc;
  constexpr int SB = MOE_BM_SPARSE;
  a.tiles_n = static_cast<int>(ceil_div(Fe, MOE_BN / 2));
  const unsigned gd0 = static_cast<unsigned>(max_mtiles * a.tiles_n), gs0 = static_cast<unsigned>(max_stiles * a.tiles_n);
  // A split sparse launch writes fp32 partial sums; its reduce (one thread per
  // 8 columns of every sparse slot row) applies the epilogue.
  auto split_launch = [&](auto gemm, auto reduce, unsigned grid, int64_t K, int64_t nc) {
    const int ks = sparse_splits(K);
    a.k_per = ceil_div(ceil_div(K, 64), ks) * 64;
    gemm<<<dim3(grid, static_cast<unsigned>(ks)), 512, 0, s>>>(a);
    reduce<<<static_cast<unsigned>(ceil_div(a.part_rows * (nc / 8), 256)), 256, 0, s>>>(a, ks);
  };
  if (gu_save != nullptr) moe_gemm_kernel<0, false, true><<<gd0, 512, 0, s>>>(a);
  else moe_gemm_kernel<0, false><<<gd0, 512, 0, s>>>(a);
  if (sparse_splits(Hd) > 1) {
    if (gu_save != nullptr)
      split_launch(moe_gemm_kernel<0, false, false, SB, true>, moe_splitk_reduce_kernel<0, true>, gs0, Hd, Fe);
    else
      split_launch(moe_gemm_kernel<0, false, false, SB, true>, moe_splitk_reduce_kernel<0, false>, gs0, Hd, Fe);
  } else if (gu_save != nullptr) {
    moe_gemm_kernel<0, false, true, SB><<<gs0, 512, 0, s>>>(a);
  } else {
    moe_gemm_kernel<0, false, false, SB><<<gs0, 512, 0, s>>>(a);
  }
  a.tiles_n = static_cast<int>(ceil_div(Hd, MOE_BN));
  const unsigned gd1 = static_cast<unsigned>(max_mtiles * a.tiles_n), gs1 = static_cast<unsigned>(max_stiles * a.tiles_n);
  moe_gemm_kernel<1, false><<<gd1, 512, 0, s>>>(a);
  if (sparse_splits(Fe) > 1)
    split_launch(moe_gemm_kernel<1, false, false, SB, true>, moe_splitk_reduce_kernel<1, false>, gs1, Fe, Hd);
  else
    moe_gemm_kernel<1, false, false, SB><<<gs1, 512, 0, s>>>(a);
  launch_unpermute(a, s);
  return check_launch(fn);
}

extern "C" int mp_grouped_expert_gemm(int64_t T, int64_t Hd, int64_t Fe, int topk, int E_loc, int e_start,
                                      const void* X, const int32_t* topk_ids, const float* topk_w, const void* W_gu,
                                      const void* W_d, void* out, int32_t* perm_picks, int32_t* expert_offsets,
                                      void* ws, size_t ws_bytes, hipStream_t s) {
  return grouped_expert_gemm("mp_grouped_expert_gemm", false, T, Hd, Fe, topk, E_loc, e_start, X, topk_ids, topk_w,
                             W_gu, W_d, out, perm_picks, expert_offsets, ws, ws_bytes, s);
}

extern "C" int mp_grouped_expert_gemm_weighted_act(int64_t T, int64_t Hd, int64_t Fe, int topk, int E_loc,
                                                   int e_start, const void* X, const int32_t* topk_ids,
                                                   const float* topk_w, const void* W_gu, const void* W_d, void* out,
                                                   int32_t* perm_picks, int32_t* expert_offsets, void* ws,
                                                   size_t ws_bytes, hipStream_t s) {
  return grouped_expert_gemm("mp_grouped_expert_gemm_weighted_act", true, T, Hd, Fe, topk, E_loc, e_start, X,
                             topk_ids, topk_w, W_gu, W_d, out, perm_picks, expert_offsets, ws, ws_bytes, s);
}

// ------------------------------------------------------------------ backward

static int fwd_train(const char* fn, bool w_on_act, int64_t T, int64_t Hd, int64_t Fe, int topk, int E_loc,
                     int e_start, const void* X, const int32_t* topk_ids, const float* topk_w, const void* W_gu,
                     const void* W_d, void* out, void* gu_save, void* ws, size_t ws_bytes, hipStream_t s) {
  if (T != 0) {
    MP_REQUIRE_PTR(gu_save);
    MP_REQUIRE_ALIGN(gu_save);
  }
  return grouped_expert_gemm(fn, w_on_act, T, Hd, Fe, topk, E_loc, e_start, X, topk_ids, topk_w, W_gu, W_d, out,
                             nullptr, nullptr, ws, ws_bytes, s, gu_save);
}

extern "C" int mp_grouped_expert_gemm_fwd_train(int64_t T, int64_t Hd, int64_t Fe, int topk, int E_loc, int e_start,
                                                const void* X, const int32_t* topk_ids, const float* topk_w,
                                                const void* W_gu, const void* W_d, void* out, void* gu_save,
                                                void* ws, size_t ws_bytes, hipStream_t s) {
  return fwd_train("mp_grouped_expert_gemm_fwd_train", false, T, Hd, Fe, topk, E_loc, e_start, X, topk_ids, topk_w,
                   W_gu, W_d, out, gu_save, ws, ws_bytes, s);
}

extern "C" int mp_grouped_expert_gemm_weighted_act_fwd_train(int64_t T, int64_t Hd, int64_t Fe, int topk,
                                                             int E_loc, int e_start, const void* X,
                                                             const int32_t* topk_ids, const float* topk_w,
                                                             const void* W_gu, const void* W_d, void* out,
                                                             void* gu_save, void* ws, size_t ws_bytes,
                                                             hipStream_t s) {
  return fwd_train("mp_grouped_expert_gemm_weighted_act_fwd_train", true, T, Hd, Fe, topk, E_loc, e_start, X,
                   topk_ids, topk_w, W_gu, W_d, out, gu_save, ws, ws_bytes, s);
}

struct MoeBwdLayout {
  size_t xp, dy, dgu, wperm, dwp, total;
};

static MoeBwdLayout moe_bwd_layout(int64_t T, int64_t Hd, int64_t Fe, int topk) {
  MoeBwdLayout L{};
  const int64_t r_cap = T * topk;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align_up(bytes, 256);
    return at;
  };
  L.xp = take(static_cast<size_t>(r_cap * Hd) * 2);
  L.dy = take(static_cast<size_t>(r_cap * Hd) * 2);
  L.dgu = take(static_cast<size_t>(r_cap * 2 * Fe) * 2);
  L.wperm = take(static_cast<size_t>(r_cap) * 4);
  L.dwp = take(static_cast<size_t>(r_cap * (Fe / 8)) * 4);
  L.total = off;
  return L;
}

extern "C" size_t mp_grouped_expert_gemm_bwd_workspace(int64_t T, int64_t Hd, int64_t Fe, int topk, int E_loc) {
  if (T < 0 || Hd <= 0 || Fe <= 0 || topk <= 0 || E_loc <= 0) return 0;
  return moe_bwd_layout(T, Hd, Fe, topk).total;
}

static int grouped_expert_gemm_bwd(const char* fn, bool w_on_act, int64_t T, int64_t Hd, int64_t Fe, int topk,
                                   int E_loc, const void* X, const float* topk_w, const void* W_gu, const void* W_d,
                                   const void* dOut, const void* gu_save, const void* fwd_ws, size_t fwd_ws_bytes,
                                   void* dX, float* dW_gu, float* dW_d, float* dtopk_w, void* ws, size_t ws_bytes,
                                   hipStream_t s) {
  MP_REQUIRE(T >= 0 && Hd > 0 && Fe > 0 && topk > 0 && E_loc > 0, MP_ERR_SHAPE, "%s: bad shape", fn);
  MP_REQUIRE(Hd % 8 == 0 && Fe % 8 == 0, MP_ERR_SHAPE, "%s: Hd and Fe must be multiples of 8", fn);
  MP_REQUIRE(T * Hd * 2 < 0x7fffffffLL && 2 * Fe * Hd * 2 < 0x7fffffffLL && T * topk * Hd * 2 < 0x7fffffffLL &&
                 T * topk * 2 * Fe * 2 < 0x7fffffffLL,
             MP_ERR_UNSUPPORTED, "%s: an operand exceeds 2 GiB", fn);
  MP_REQUIRE_PTR(dW_gu);
  MP_REQUIRE_PTR(dW_d);
  MP_REQUIRE_ALIGN(dW_gu);
  MP_REQUIRE_ALIGN(dW_d);
  if (T == 0) {
    // No tokens: every expert's weight gradient is zero; the token-sized
    // buffers are empty and may be NULL.
    const int64_t n = static_cast<int64_t>(E_loc) * 2 * Fe * Hd, m = static_cast<int64_t>(E_loc) * Hd * Fe;
    moe_zero_f32_kernel<<<static_cast<unsigned>(ceil_div(n, 256)), 256, 0, s>>>(dW_gu, n);
    moe_zero_f32_kernel<<<static_cast<unsigned>(ceil_div(m, 256)), 256, 0, s>>>(dW_d, m);
    return check_launch(fn);
  }
  MP_REQUIRE_PTR(X);
  MP_REQUIRE_PTR(topk_w);
  MP_REQUIRE_PTR(W_gu);
  MP_REQUIRE_PTR(W_d);
  MP_REQUIRE_PTR(dOut);
  MP_REQUIRE_PTR(gu_save);
  MP_REQUIRE_PTR(dX);
  MP_REQUIRE_PTR(dtopk_w);
  MP_REQUIRE_ALIGN(X);
  MP_REQUIRE_ALIGN(W_gu);
  MP_REQUIRE_ALIGN(W_d);
  MP_REQUIRE_ALIGN(dOut);
  MP_REQUIRE_ALIGN(gu_save);
  MP_REQUIRE_ALIGN(dX);
  const MoeLayout F = moe_layout(T, Hd, Fe, topk, E_loc);
  MP_REQUIRE(fwd_ws != nullptr && fwd_ws_bytes >= F.total, MP_ERR_WORKSPACE,
             "%s: the forward's workspace holds %zu bytes", fn, F.total);
  MP_REQUIRE_ALIGN(fwd_ws);
  const MoeBwdLayout L = moe_bwd_layout(T, Hd, Fe, topk);
  MP_REQUIRE(ws != nullptr && ws_bytes >= L.total, MP_ERR_WORKSPACE, "%s: workspace needs %zu bytes", fn, L.total);
  MP_REQUIRE_ALIGN(ws);
  char* fw = static_cast<char*>(const_cast<void*>(fwd_ws));
  char* w = static_cast<char*>(ws);
  MoeArgs a{};
  a.T = T;
  a.Hd = Hd;
  a.Fe = Fe;
  a.topk = topk;
  a.E_loc = E_loc;
  a.r_cap = T * topk;
  a.X = static_cast<const uint16_t*>(X);
  a.w = topk_w;
  a.pick_row = reinterpret_cast<int32_t*>(fw + F.pick_row);
  a.perm = reinterpret_cast<int32_t*>(fw + F.perm);
  a.offsets = reinterpret_cast<int32_t*>(fw + F.offsets);
  a.tile_start = reinterpret_cast<int32_t*>(fw + F.tile_start);
  a.act = reinterpret_cast<uint16_t*>(fw + F.act);
  a.yperm = reinterpret_cast<uint16_t*>(fw + F.yperm);
  a.dout = static_cast<const uint16_t*>(dOut);
  a.dy = reinterpret_cast<uint16_t*>(w + L.dy);
  a.xp = reinterpret_cast<uint16_t*>(w + L.xp);
  a.dw = dtopk_w;
  a.wperm = reinterpret_cast<float*>(w + L.wperm);
  a.dwp = reinterpret_cast<float*>(w + L.dwp);
  uint16_t* dgu = reinterpret_cast<uint16_t*>(w + L.dgu);
  const int64_t max_mtiles = ceil_div(a.r_cap, MOE_BM) + E_loc;
  const unsigned rgrid = static_cast<unsigned>(ceil_div(a.r_cap, 4));
  moe_bwd_dw_zero_kernel<<<static_cast<unsigned>(ceil_div(T * topk, 256)), 256, 0, s>>>(a);
  if (w_on_act) moe_bwd_rows_kernel<true><<<rgrid, 256, 0, s>>>(a);
  else moe_bwd_rows_kernel<false><<<rgrid, 256, 0, s>>>(a);
  // d act -> (d gate, d up) through the SwiGLU derivative, per expert (in the
  // weighted-activation form, via d act_w, with the weight's gradient parts).
  if (int rc = gemm_grouped_m(EPI_SWIGLU_BWD, E_loc, a.offsets, a.tile_start, max_mtiles, Fe, Hd, a.dy, Hd, W_d, Fe,
                              Hd * Fe, dgu, 2 * Fe, gu_save, s, w_on_act ? a.wperm : nullptr,
                              w_on_act ? a.dwp : nullptr))
    return rc;
  if (w_on_act) moe_bwd_dw_rows_kernel<<<rgrid, 256, 0, s>>>(a);
  // dW_d[e] = dy_e^T act_e.
  if (int rc = gemm_grouped_k(E_loc, a.offsets, a.r_cap, Hd, Fe, a.dy, Hd, a.act, Fe, dW_d, Fe, Hd * Fe, s)) return rc;
  // d x_perm = [d gate, d up] W_gu,e, into dy's buffer (dy is consumed).
  if (int rc = gemm_grouped_m(EPI_STORE, E_loc, a.offsets, a.tile_start, max_mtiles, Hd, 2 * Fe, dgu, 2 * Fe, W_gu,
                              Hd, 2 * Fe * Hd, a.dy, Hd, nullptr, s))
    return rc;
  // dX[t] = sum over t's local picks of d x_perm rows (k ascending).
  MoeArgs u = a;
  u.yperm = a.dy;
  u.w_on_act = 1;
  u.out = static_cast<uint16_t*>(dX);
  launch_unpermute(u, s);
  // dW_gu[e] = [d gate, d up]_e^T x_perm,e.
  if (int rc = gemm_grouped_k(E_loc, a.offsets, a.r_cap, 2 * Fe, Hd, dgu, 2 * Fe, a.xp, Hd, dW_gu, Hd, 2 * Fe * Hd, s))
    return rc;
  return check_launch(fn);
}

extern "C" int mp_grouped_expert_gemm_bwd(int64_t T, int64_t Hd, int64_t Fe, int topk, int E_loc, const void* X,
                                          const float* topk_w, const void* W_gu, const void* W_d, const void* dOut,
                                          const void* gu_save, const void* fwd_ws, size_t fwd_ws_bytes, void* dX,
                                          float* dW_gu, float* dW_d, float* dtopk_w, void* ws, size_t ws_bytes,
                                          hipStream_t s) {
  return grouped_expert_gemm_bwd("mp_grouped_expert_gemm_bwd", false, T, Hd, Fe, topk, E_loc, X, topk_w, W_gu, W_d,
                                 dOut, gu_save, fwd_ws, fwd_ws_bytes, dX, dW_gu, dW_d, dtopk_w, ws, ws_bytes, s);
}

extern "C" int mp_grouped_expert_gemm_weighted_act_bwd(int64_t T, int64_t Hd, int64_t Fe, int topk, int E_loc,
                                                       const void* X, const float* topk_w, const void* W_gu,
                                                       const void* W_d, const void* dOut, const void* gu_save,
                                                       const void* fwd_ws, size_t fwd_ws_bytes, void* dX,
                                                       float* dW_gu, float* dW_d, float* dtopk_w, void* ws,
                                                       size_t ws_bytes, hipStream_t s) {
  return grouped_expert_gemm_bwd("mp_grouped_expert_gemm_weighted_act_bwd", true, T, Hd, Fe, topk, E_loc, X, topk_w,
                                 W_gu, W_d, dOut, gu_save, fwd_ws, fwd_ws_bytes, dX, dW_gu, dW_d, dtopk_w, ws,
                                 ws_bytes, s);
}

// ------------------------------------------------------------------ MXFP8

extern "C" int mp_mxfp8_quantize(int64_t rows, int64_t K, const void* x, int64_t ld, uint8_t* q, uint8_t* scales,
                                 hipStream_t s) {
  static const char* fn = "mp_mxfp8_quantize";
  MP_REQUIRE(rows >= 0 && K > 0 && K % 32 == 0, MP_ERR_SHAPE, "%s: K=%lld must be a positive multiple of 32", fn,
             (long long)K);
  MP_REQUIRE(ld >= K && ld % 8 == 0, MP_ERR_SHAPE, "%s: ld=%lld must be >= K and a multiple of 8", fn, (long long)ld);
  if (rows == 0) return MP_OK;
  MP_REQUIRE_PTR(x);
  MP_REQUIRE_PTR(q);
  MP_REQUIRE_PTR(scales);
  MP_REQUIRE_ALIGN(x);
  MP_REQUIRE(reinterpret_cast<uintptr_t>(q) % 8 == 0, MP_ERR_ALIGN, "%s: q must be 8-byte aligned", fn);
  const int64_t groups = rows * (K / 8);
  mx_quantize_kernel<<<static_cast<unsigned>(ceil_div(groups, 256)), 256, 0, s>>>(
      static_cast<const uint16_t*>(x), ld, rows, K, q, scales, mx_scale_width(K));
  return check_launch(fn);
}

extern "C" size_t mp_grouped_expert_gemm_mxfp8_workspace(int64_t T, int64_t Hd, int64_t Fe, int topk, int E_loc) {
  if (T < 0 || Hd <= 0 || Fe <= 0 || topk <= 0 || E_loc <= 0) return 0;
  return moe_layout(T, Hd, Fe, topk, E_loc, true).total;
}

extern "C" int mp_grouped_expert_gemm_mxfp8(int64_t T, int64_t Hd, int64_t Fe, int topk, int E_loc, int e_start,
                                            const void* X, const int32_t* topk_ids, const float* topk_w,
                                            const uint8_t* W_gu_q, const uint8_t* W_gu_s, const uint8_t* W_d_q,
                                            const uint8_t* W_d_s, void* out, int32_t* perm_picks,
                                            int32_t* expert_offsets, void* ws, size_t ws_bytes, hipStream_t s) {
  static const char* fn = "mp_grouped_expert_gemm_mxfp8";
  MP_REQUIRE(T >= 0 && Hd > 0 && Fe > 0 && topk > 0 && E_loc > 0 && e_start >= 0, MP_ERR_SHAPE, "%s: bad shape", fn);
  MP_REQUIRE(Hd % 32 == 0 && Fe % 32 == 0, MP_ERR_SHAPE, "%s: Hd and Fe must be multiples of 32 (MX blocks)", fn);
  MP_REQUIRE(T * Hd * 2 < 0x7fffffffLL && 2 * Fe * Hd < 0x7fffffffLL && T * topk * Fe * 2 < 0x7fffffffLL,
             MP_ERR_UNSUPPORTED, "%s: an operand exceeds 2 GiB", fn);
  if (T == 0) return MP_OK;  // no tokens: nothing is read or written
  MP_REQUIRE_PTR(X);
  MP_REQUIRE_PTR(topk_ids);
  MP_REQUIRE_PTR(topk_w);
  MP_REQUIRE_PTR(W_gu_q);
  MP_REQUIRE_PTR(W_gu_s);
  MP_REQUIRE_PTR(W_d_q);
  MP_REQUIRE_PTR(W_d_s);
  MP_REQUIRE_PTR(out);
  if (int rc = debug_check_range(fn, "topk_ids", topk_ids, T * topk, 0, INT32_MAX + 1LL, s)) return rc;
  MP_REQUIRE_ALIGN(X);
  MP_REQUIRE_ALIGN(W_gu_q);
  MP_REQUIRE_ALIGN(W_d_q);
  MP_REQUIRE_ALIGN(out);
  MP_REQUIRE(reinterpret_cast<uintptr_t>(W_gu_s) % 4 == 0 && reinterpret_cast<uintptr_t>(W_d_s) % 4 == 0,
             MP_ERR_ALIGN, "%s: scale arrays must be 4-byte aligned", fn);
  const MoeLayout L = moe_layout(T, Hd, Fe, topk, E_loc, true);
  MP_REQUIRE(ws != nullptr && ws_bytes >= L.total, MP_ERR_WORKSPACE, "%s: workspace needs %zu bytes", fn, L.total);
  MP_REQUIRE_ALIGN(ws);
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
  a.out = static_cast<uint16_t*>(out);
  a.cnt = reinterpret_cast<int32_t*>(w + L.cnt);
  a.pick_row = reinterpret_cast<int32_t*>(w + L.pick_row);
  a.perm = perm_picks != nullptr ? perm_picks : reinterpret_cast<int32_t*>(w + L.perm);
  a.offsets = expert_offsets != nullptr ? expert_offsets : reinterpret_cast<int32_t*>(w + L.offsets);
  a.tile_start = reinterpret_cast<int32_t*>(w + L.tile_start);
  a.counts = reinterpret_cast<int32_t*>(w + L.counts);
  a.act = nullptr;  // the gate/up GEMM writes the quantised activation only
  a.yperm = reinterpret_cast<uint16_t*>(w + L.yperm);
  a.swh = mx_scale_width(Hd);
  a.swf = mx_scale_width(Fe);
  uint8_t* xq = reinterpret_cast<uint8_t*>(w + L.xq);
  uint8_t* xs = reinterpret_cast<uint8_t*>(w + L.xs);
  uint8_t* aq = reinterpret_cast<uint8_t*>(w + L.aq);
  uint8_t* as = reinterpret_cast<uint8_t*>(w + L.as);
  a.xq = xq;
  a.xs = xs;
  a.gq = W_gu_q;
  a.gs = W_gu_s;
  a.dq = W_d_q;
  a.ds = W_d_s;
  a.aq = aq;
  a.as = as;
  launch_routing(a, s);
  // Token rows quantised once along the hidden dimension (the expert GEMMs'
  // reduction dimension); the weights arrive quantised.
  mx_quantize_kernel<<<static_cast<unsigned>(ceil_div(T * (Hd / 8), 256)), 256, 0, s>>>(a.X, Hd, T, Hd, xq, xs,
                                                                                          a.swh);
  const int64_t max_mtiles = ceil_div(a.r_cap, MOE_BM) + E_loc;
  a.tiles_n = static_cast<int>(ceil_div(Fe, MOE_BN / 2));
  // The gate/up GEMM quantises the bf16-rounded activation along Fe in its
  // epilogue (aq, as), the down GEMM's A operand.
  moe_gemm_kernel<0, true><<<static_cast<unsigned>(max_mtiles * a.tiles_n), 512, 0, s>>>(a);
  a.tiles_n = static_cast<int>(ceil_div(Hd, MOE_BN));
  moe_gemm_kernel<1, true><<<static_cast<unsigned>(max_mtiles * a.tiles_n), 512, 0, s>>>(a);
  launch_unpermute(a, s);
  return check_launch(fn);
}
