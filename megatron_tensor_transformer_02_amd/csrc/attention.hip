// Head-partitioned causal self-attention of one tensor-parallel rank: the
// fused QKV GEMM over the rank's heads, then attention per (batch, head)
// (heads are independent, so a rank's heads need no communication).
//
// Forward (flash-style, one pass over the keys): a wave owns 16 queries and
// computes S^T = K Q^T with 16x16x32 bf16 MFMAs, so lane l holds scores of
// query l % 16 only (4 of every 16 keys; the four lanes l % 16 + 16j share
// the query), and the online softmax needs two lane exchanges for the
// running max.  The probabilities of keys {32t + 4g .. +3, 32t+16+4g .. +3}
// (g = lane / 16) are, as they stand, the B operand of O^T += V^T P^T for
// the 32-key step t; the V^T fragments come from the plain V row tile
// through two LDS transpose reads (4 consecutive keys each) in that same key
// order, so P never leaves registers and no transposed tile is stored.
// Sixteen rows per wave keep the register footprint small enough for two or
// more waves per SIMD and give short sequences with few heads enough waves.
//
// Every kernel streams 64-row tiles through two LDS buffers: direct global ->
// LDS loads fill the other buffer while the current one is multiplied (no
// staging registers, no LDS stores; one wait and one barrier per tile).
//
// Backward (P recomputed from the saved log-sum-exp, no atomics):
//  * dQ kernel -- lanes own queries: rowsum(dO * O) (also left for the next
//    kernel), S^T, dP^T = V dO^T, dS^T, dQ^T += K^T dS^T;
//  * dK/dV kernel -- lanes own keys: S = Q K^T, dP = dO V^T, dS,
//    dV^T += dO^T P, dK^T += Q^T dS.
// With few (batch, head) pairs and at most 4096 keys the order turns round:
// rowsum(dO * O) by a small kernel, then the dK/dV kernel, which also writes
// dS^T (bf16, 64 x 64 tiles) to the workspace, then a dQ kernel that forms
// dQ^T = K^T dS^T from the stored tiles without recomputing S and dP.
// The QKV GEMM's input and weight gradients then run on the GEMM family.
#include "gemm.h"
#include "mfma.h"

namespace mp {

constexpr float kLog2eA = 1.4426950408889634f;

struct AttnArgs {
  const uint16_t* qkv;   // [B*L, 3*h*D]
  uint16_t* ctx;         // [B*L, h*D]
  float* lse;            // [B, h, L]
  const uint16_t* dctx;  // [B*L, h*D]        (backward)
  const float* dvec;     // [B, h, L] rowsum(dO * O), written by the dQ kernel
  uint16_t* dqkv;        // [B*L, 3*h*D]      (backward)
  uint16_t* dst;         // [B, h, L keys, L queries] dS^T (backward, stored-dS form) or null
  int B, L, h, causal;
  int nblk;              // query (or key) blocks per (batch, head)
  float scale;           // 1/sqrt(D)
  float scale_log2;      // log2(e)/sqrt(D)
};

// 8 consecutive bf16 of `p` (16-byte aligned) or zeros.
__device__ __forceinline__ uint4 ld16_or_zero(const uint16_t* p, bool ok) {
  return ok ? *reinterpret_cast<const uint4*>(p) : make_uint4(0, 0, 0, 0);
}

// A 64-row x D-column tile of a [L, ld] bf16 matrix (a head slice), held in
// D/64 LDS sub-tiles of the GEMM tile format (64 rows x 64 columns, rows of
// eight swizzled 16-byte chunks) and filled by direct global -> LDS loads (no
// registers, no LDS stores): `issue` starts the copy of rows r0..r0+63,
// which lands asynchronously; wait_vm_lds() and a barrier make it visible.
// The resource covers rows [0, L) of the head slice, so rows >= L arrive as
// zeros.
template <int D, int NT>
struct RowTileDma {
  DmaTile<64, true, NT> part;
  __device__ __forceinline__ void init(const uint16_t* base, int64_t ld, int L, int tid) {
    part.init(base, ld, 0, L, D, tid);
  }
  __device__ __forceinline__ void issue(uint4* lds, int r0) const {
#pragma unroll
    for (int hf = 0; hf < D / 64; ++hf) part.issue_rows(lds + hf * 512, r0, 64 * hf);
  }
};

// 64 consecutive floats [q0, q0 + 64) of a per-row vector copied into LDS by
// one wave's direct loads (lane l fills lds[l]); entries past the vector's
// end arrive as zeros.  No compiler-visible load stays in the tile loop, so
// the compiler places no wait there that would also wait for the tiles.
struct VecDma {
  i32x4_t desc;
  __device__ __forceinline__ void init(const float* base, int64_t n) {
    desc = make_desc(base, n * 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) desc[i] = __builtin_amdgcn_readfirstlane(desc[i]);
  }
  __device__ __forceinline__ void issue(float* lds, int q0, int lane) const {
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr(lds));
    const uint32_t so = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(q0) * 4u);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, %3 offen lds" ::"v"(lane * 4), "s"(desc),
                 "s"(m0v), "s"(so)
                 : "memory", "m0");
  }
};

// Column group of k-group g (lane / 16) in a 32-column step: 8 * kgrp(g),
// kgrp = (0, 3, 1, 2).  The MFMA sums over the step's 32 columns in any
// order, so both operands only have to agree on it.  A 16-byte LDS read
// serves lanes {0-3, 12-15, 20-27} (and the matching sets) in one cycle
// (measured on gfx950), which pairs rows of k-groups 0 and 1 (and 2 and 3)
// whose swizzles differ by an odd-weight value; chunks whose indexes differ
// by 3 then fall in distinct banks, where the plain order (chunks 0, 1)
// put every such pair in the same banks: 4 conflict cycles per read.
__device__ __forceinline__ int kgrp(int g) { return (0x2130 >> (4 * g)) & 3; }

// Row fragment (A or B operand) of a row tile: row r0 + lane%16, columns
// 32*st + 8*kgrp(lane/16) .. +7.
__device__ __forceinline__ uint4 row_frag(const uint4* tile, int r0, int st, int lane) {
  const int c = 32 * st + 8 * kgrp(lane >> 4);
  return tile[(c >> 6) * 512 + lds_slot(r0 + (lane & 15), (c & 63) >> 3)];
}

// Byte address of element (r, d) of a row tile.
__device__ __forceinline__ const char* tile_elem(const uint4* tile, int r, int d) {
  return reinterpret_cast<const char*>(tile + (d >> 6) * 512 + lds_slot(r, (d & 63) >> 3)) + (d & 7) * 2;
}

// Transposed A-operand fragment from a row tile: operand row = tile column
// d0 + lane%16; its 8 k-slots are tile rows {32t + 4g .. +3} and
// {32t + 16 + 4g .. +3} (g = lane / 16): two transpose reads of 4 rows.
__device__ __forceinline__ uint4 tr_frag(const uint4* tile, int d0, int t, int lane) {
  const int grp = lane >> 4, i = lane & 15;
  const int r = 32 * t + 4 * grp + (i >> 2);
  const int d = d0 + 4 * (i & 3);
  const uint2 lo = lds_read_tr16(tile_elem(tile, r, d));
  const uint2 hi = lds_read_tr16(tile_elem(tile, r + 16, d));
  return make_uint4(lo.x, lo.y, hi.x, hi.y);
}

// B operand for the 32-row step t from two 16-row results (rows 4g + r):
// rows {32t + 4g + r} from x0 and {32t + 16 + 4g + r} from x1, as bf16.
__device__ __forceinline__ uint4 pack_pair(const f32x4_t& x0, const f32x4_t& x1) {
  return make_uint4(pack_bf16x2(x0[0], x0[1]), pack_bf16x2(x0[2], x0[3]), pack_bf16x2(x1[0], x1[1]),
                    pack_bf16x2(x1[2], x1[3]));
}

// Max over the four lanes that share lane % 16.
__device__ __forceinline__ float max4(float v) {
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  return fmaxf(v, __shfl_xor(v, 32, 64));
}
__device__ __forceinline__ float sum4(float v) {
  v += __shfl_xor(v, 16, 64);
  return v + __shfl_xor(v, 32, 64);
}

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void attn_fwd_kernel(const AttnArgs a) {
  constexpr int NT = 64 * NW, BQ = 16 * NW, DB = D / 16, KS = D / 32, TS = D / 64 * 512;
  __shared__ uint4 lds_k[2][TS];
  __shared__ uint4 lds_v[2][TS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, qc = lane & 15, g = lane >> 4;
  const int nbh = a.B * a.h;
  const int bh = blockIdx.x % nbh;
  const int qb = a.nblk - 1 - static_cast<int>(blockIdx.x / nbh);  // heavy (late) query blocks first
  const int b = bh / a.h, hh = bh % a.h;
  const int64_t S3 = 3LL * a.h * D, HD = static_cast<int64_t>(a.h) * D;
  const uint16_t* base = a.qkv + static_cast<int64_t>(b) * a.L * S3;
  const int q0 = qb * BQ, qw0 = q0 + wave * 16, qi = qw0 + qc;
  const bool qvalid = qi < a.L;

  uint4 qf[KS];  // Q^T as the B operand: query qi, d = 32 st + 8 kgrp(g) .. +7
#pragma unroll
  for (int st = 0; st < KS; ++st) qf[st] = ld16_or_zero(base + static_cast<int64_t>(qi) * S3 + hh * D + 32 * st + 8 * kgrp(g), qvalid);

  RowTileDma<D, NT> tk, tv;
  tk.init(base + HD + hh * D, S3, a.L, tid);
  tv.init(base + 2 * HD + hh * D, S3, a.L, tid);

  float m = -INFINITY, l = 0.0f;
  f32x4_t o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  const int kv_end = a.causal ? min(a.L, q0 + BQ) : a.L;
  const int nkb = (kv_end + 63) / 64;
  tk.issue(lds_k[0], 0);
  tv.issue(lds_v[0], 0);
  wait_compiler_loads();  // the Q fragments
  wait_vm_lds();
  __syncthreads();
  for (int it = 0; it < nkb; ++it) {
    const int kv0 = it * 64, cur = it & 1;
    const bool more = it + 1 < nkb;
    if (more) {  // the other buffer's reads retired before the last barrier
      tk.issue(lds_k[cur ^ 1], kv0 + 64);
      tv.issue(lds_v[cur ^ 1], kv0 + 64);
    }
    if (!(a.causal && kv0 > qw0 + 15)) {  // else every key of the tile is in this wave's future
      const uint4* kt_ = lds_k[cur];
      const uint4* vt_ = lds_v[cur];
      f32x4_t s[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        s[kb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int st = 0; st < KS; ++st) s[kb] = mfma_16x16x32(row_frag(kt_, 16 * kb, st, lane), qf[st], s[kb]);
      }
      // Keys of this lane: kv0 + 16 kb + 4 g + r.
      if (kv0 + 63 >= a.L || (a.causal && kv0 + 63 > qw0)) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = kv0 + 16 * kb + 4 * g + r;
            if (key >= a.L || (a.causal && key > qi)) s[kb][r] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = max4(mx);
      const float mn = fmaxf(m, mx);
      const float ms = mn == -INFINITY ? 0.0f : mn;
      const float alpha = exp2_fast((m - ms) * a.scale_log2);
      const float msc = ms * a.scale_log2;
      float ps = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          s[kb][r] = exp2_fast(fmaf(s[kb][r], a.scale_log2, -msc));
          ps += s[kb][r];
        }
      l = l * alpha + ps;
      const uint4 pb0 = pack_pair(s[0], s[1]), pb1 = pack_pair(s[2], s[3]);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        o[db] *= alpha;
        o[db] = mfma_16x16x32(tr_frag(vt_, 16 * db, 0, lane), pb0, o[db]);
        o[db] = mfma_16x16x32(tr_frag(vt_, 16 * db, 1, lane), pb1, o[db]);
      }
      m = mn;
    }
    wait_vm_lds();  // this wave's copies of the next tile landed; its reads of this one retired
    __syncthreads();
  }
  const float lt = sum4(l);
  if (!qvalid) return;
  const float inv = 1.0f / lt;
  uint16_t* crow = a.ctx + (static_cast<int64_t>(b) * a.L + qi) * HD + hh * D;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    uint2 v;
    v.x = pack_bf16x2(o[db][0] * inv, o[db][1] * inv);
    v.y = pack_bf16x2(o[db][2] * inv, o[db][3] * inv);
    *reinterpret_cast<uint2*>(crow + 16 * db + 4 * g) = v;
  }
  if (g == 0) a.lse[(static_cast<int64_t>(b) * a.h + hh) * a.L + qi] = m * a.scale + logf(lt);
}

// Causal forward for few (batch, head) pairs: a block holds 4 query tiles of
// 16 rows x 2 waves (8 waves, two per SIMD, one block per CU), and the two
// waves of a query tile take alternate 64-key tiles (wave (qt, p) the tiles of
// parity p): each step multiplies a whole tile per wave, with four
// independent S^T chains and one max / rescale per 64 keys, and the heaviest
// block runs ceil(n/2) steps for its n key tiles.  Both tiles of a step are
// in LDS together.  At the end the two waves' (running max, exp-sum, O) are
// merged through LDS, rescaled to the common max.
template <int D>
__global__ __launch_bounds__(512) void attn_fwd_par_kernel(const AttnArgs a) {
  constexpr int NT = 512, BQ = 64, DB = D / 16, KS = D / 32, TS = D / 64 * 512;
  __shared__ uint4 lds[2][4][TS];  // [buffer][K even, K odd, V even, V odd]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, qt = wave & 3, par = wave >> 2;
  const int qc = lane & 15, g = lane >> 4;
  const int nbh = a.B * a.h;
  const int bh = blockIdx.x % nbh;
  const int qb = a.nblk - 1 - static_cast<int>(blockIdx.x / nbh);  // heavy (late) query blocks first
  const int b = bh / a.h, hh = bh % a.h;
  const int64_t S3 = 3LL * a.h * D, HD = static_cast<int64_t>(a.h) * D;
  const uint16_t* base = a.qkv + static_cast<int64_t>(b) * a.L * S3;
  const int q0 = qb * BQ, qw0 = q0 + qt * 16, qi = qw0 + qc;
  const bool qvalid = qi < a.L;

  RowTileDma<D, NT> tk, tv;
  tk.init(base + HD + hh * D, S3, a.L, tid);
  tv.init(base + 2 * HD + hh * D, S3, a.L, tid);
  auto fetch = [&](int buf, int kt0) {  // key tiles kt0 and kt0 + 1
    tk.issue(lds[buf][0], 64 * kt0);
    tk.issue(lds[buf][1], 64 * kt0 + 64);
    tv.issue(lds[buf][2], 64 * kt0);
    tv.issue(lds[buf][3], 64 * kt0 + 64);
  };
  fetch(0, 0);

  uint4 qf[KS];  // Q^T as the B operand: query qi, d = 32 st + 8 kgrp(g) .. +7
#pragma unroll
  for (int st = 0; st < KS; ++st) qf[st] = ld16_or_zero(base + static_cast<int64_t>(qi) * S3 + hh * D + 32 * st + 8 * kgrp(g), qvalid);

  float m = -INFINITY, l = 0.0f;
  f32x4_t o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  const int nkb = (min(a.L, q0 + BQ) + 63) / 64, nit = (nkb + 1) / 2;
  wait_compiler_loads();  // the Q fragments
  wait_vm_lds();
  __syncthreads();
  for (int it = 0; it < nit; ++it) {
    const int cur = it & 1;
    if (it + 1 < nit) fetch(cur ^ 1, 2 * it + 2);  // the other buffer's reads retired before the last barrier
    const int kv0 = 128 * it + 64 * par;  // this wave's tile
    if (kv0 < a.L && kv0 <= qw0 + 15) {
      const uint4* kt_ = lds[cur][par];
      const uint4* vt_ = lds[cur][2 + par];
      f32x4_t s[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) s[kb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int st = 0; st < KS; ++st) {
        uint4 kfr[4];  // the step's four K fragments in flight together
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) kfr[kb] = row_frag(kt_, 16 * kb, st, lane);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) s[kb] = mfma_16x16x32(kfr[kb], qf[st], s[kb]);
      }
      // Keys of this lane: kv0 + 16 kb + 4 g + r.
      if (kv0 + 63 >= a.L || kv0 + 63 > qw0) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = kv0 + 16 * kb + 4 * g + r;
            if (key >= a.L || key > qi) s[kb][r] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = max4(mx);
      const float mn = fmaxf(m, mx);
      const float ms = mn == -INFINITY ? 0.0f : mn;
      const float alpha = exp2_fast((m - ms) * a.scale_log2);
      const float msc = ms * a.scale_log2;
      float ps = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          s[kb][r] = exp2_fast(fmaf(s[kb][r], a.scale_log2, -msc));
          ps += s[kb][r];
        }
      l = l * alpha + ps;
      const uint4 pb0 = pack_pair(s[0], s[1]), pb1 = pack_pair(s[2], s[3]);
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
#pragma unroll
      for (int d4 = 0; d4 < DB; d4 += 4) {  // V^T fragments four at a time, in flight together
        uint4 v0[4], v1[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v0[j] = tr_frag(vt_, 16 * (d4 + j), 0, lane);
          v1[j] = tr_frag(vt_, 16 * (d4 + j), 1, lane);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          o[d4 + j] = mfma_16x16x32(v0[j], pb0, o[d4 + j]);
          o[d4 + j] = mfma_16x16x32(v1[j], pb1, o[d4 + j]);
        }
      }
      m = mn;
    }
    wait_vm_lds();  // this wave's copies of the next tiles landed; its reads of these retired
    __syncthreads();
  }
  // The parity-1 wave leaves (m, l, O) in LDS, laid out [tile][value][lane]
  // (conflict-free); the parity-0 wave rescales both to the common max.
  constexpr int MS = 4 * DB + 2;
  float* mrg = reinterpret_cast<float*>(&lds[0][0][0]) + qt * MS * 64 + lane;
  if (par == 1) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) mrg[(4 * db + r) * 64] = o[db][r];
    mrg[(4 * DB) * 64] = m;
    mrg[(4 * DB + 1) * 64] = l;
  }
  __syncthreads();
  if (par == 1) return;
  {
    const float m1 = mrg[(4 * DB) * 64], l1 = mrg[(4 * DB + 1) * 64];
    const float mn = fmaxf(m, m1);
    const float ms = mn == -INFINITY ? 0.0f : mn;
    const float a0 = exp2_fast((m - ms) * a.scale_log2), a1 = exp2_fast((m1 - ms) * a.scale_log2);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) o[db][r] = o[db][r] * a0 + mrg[(4 * db + r) * 64] * a1;
    l = l * a0 + l1 * a1;
    m = mn;
  }
  const float lt = sum4(l);
  if (!qvalid) return;
  const float inv = 1.0f / lt;
  uint16_t* crow = a.ctx + (static_cast<int64_t>(b) * a.L + qi) * HD + hh * D;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    uint2 v;
    v.x = pack_bf16x2(o[db][0] * inv, o[db][1] * inv);
    v.y = pack_bf16x2(o[db][2] * inv, o[db][3] * inv);
    *reinterpret_cast<uint2*>(crow + 16 * db + 4 * g) = v;
  }
  if (g == 0) a.lse[(static_cast<int64_t>(b) * a.h + hh) * a.L + qi] = m * a.scale + logf(lt);
}

// Forward with the keys of each query tile split between two waves: a block
// holds 4 query tiles of 16 rows x 2 key halves (8 waves, two per SIMD).
// Wave (qt, hf) multiplies keys 32*hf .. 32*hf+31 of every 64-key tile, so
// each wave's dependent chain per tile (S^T, softmax, O^T) is half as long and
// a second wave per SIMD covers its latency.  At the end the two halves'
// (running max, exp-sum, O) are merged through LDS, rescaled to the common
// max as the online softmax does between tiles.
template <int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) void attn_fwd_split_kernel(
    const AttnArgs a) {  // <= 128 VGPRs: two blocks per CU
  constexpr int NT = 512, BQ = 64, DB = D / 16, KS = D / 32, TS = D / 64 * 512;
  __shared__ uint4 lds[4][TS];  // K tiles in [0], [1]; V tiles in [2], [3]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, qt = wave & 3, hf = wave >> 2;
  const int qc = lane & 15, g = lane >> 4;
  const int nbh = a.B * a.h;
  const int bh = blockIdx.x % nbh;
  const int qb = a.nblk - 1 - static_cast<int>(blockIdx.x / nbh);  // heavy (late) query blocks first
  const int b = bh / a.h, hh = bh % a.h;
  const int64_t S3 = 3LL * a.h * D, HD = static_cast<int64_t>(a.h) * D;
  const uint16_t* base = a.qkv + static_cast<int64_t>(b) * a.L * S3;
  const int q0 = qb * BQ, qw0 = q0 + qt * 16, qi = qw0 + qc;
  const bool qvalid = qi < a.L;

  uint4 qf[KS];  // Q^T as the B operand: query qi, d = 32 st + 8 kgrp(g) .. +7
#pragma unroll
  for (int st = 0; st < KS; ++st) qf[st] = ld16_or_zero(base + static_cast<int64_t>(qi) * S3 + hh * D + 32 * st + 8 * kgrp(g), qvalid);

  RowTileDma<D, NT> tk, tv;
  tk.init(base + HD + hh * D, S3, a.L, tid);
  tv.init(base + 2 * HD + hh * D, S3, a.L, tid);

  float m = -INFINITY, l = 0.0f;
  f32x4_t o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  const int kv_end = a.causal ? min(a.L, q0 + BQ) : a.L;
  const int nkb = (kv_end + 63) / 64;
  tk.issue(lds[0], 0);
  tv.issue(lds[2], 0);
  wait_compiler_loads();  // the Q fragments
  wait_vm_lds();
  __syncthreads();
  for (int it = 0; it < nkb; ++it) {
    const int kv0 = it * 64, cur = it & 1;
    const bool more = it + 1 < nkb;
    if (more) {  // the other buffer's reads retired before the last barrier
      tk.issue(lds[cur ^ 1], kv0 + 64);
      tv.issue(lds[2 + (cur ^ 1)], kv0 + 64);
    }
    const int k0h = kv0 + 32 * hf;  // this wave's 32 keys
    if (k0h < a.L && !(a.causal && k0h > qw0 + 15)) {
      const uint4* kt_ = lds[cur];
      const uint4* vt_ = lds[2 + cur];
      f32x4_t s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int st = 0; st < KS; ++st) s[kb] = mfma_16x16x32(row_frag(kt_, 32 * hf + 16 * kb, st, lane), qf[st], s[kb]);
      }
      // Keys of this lane: k0h + 16 kb + 4 g + r.
      if (k0h + 31 >= a.L || (a.causal && k0h + 31 > qw0)) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = k0h + 16 * kb + 4 * g + r;
            if (key >= a.L || (a.causal && key > qi)) s[kb][r] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = max4(mx);
      const float mn = fmaxf(m, mx);
      const float ms = mn == -INFINITY ? 0.0f : mn;
      const float alpha = exp2_fast((m - ms) * a.scale_log2);
      const float msc = ms * a.scale_log2;
      float ps = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          s[kb][r] = exp2_fast(fmaf(s[kb][r], a.scale_log2, -msc));
          ps += s[kb][r];
        }
      l = l * alpha + ps;
      const uint4 pb = pack_pair(s[0], s[1]);
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
      // V^T fragments four at a time: their transpose reads are in flight
      // together instead of one before each MFMA.
#pragma unroll
      for (int d4 = 0; d4 < DB; d4 += 4) {
        uint4 vf[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) vf[j] = tr_frag(vt_, 16 * (d4 + j), hf, lane);
#pragma unroll
        for (int j = 0; j < 4; ++j) o[d4 + j] = mfma_16x16x32(vf[j], pb, o[d4 + j]);
      }
      m = mn;
    }
    wait_vm_lds();  // this wave's copies of the next tile landed; its reads of this one retired
    __syncthreads();
  }
  // Merge the key halves: the second half's wave leaves (m, l, O) in LDS,
  // laid out [tile][value][lane] (conflict-free), the first half's wave
  // rescales both to the common max and finishes.
  constexpr int MS = 4 * DB + 2;
  float* mrg = reinterpret_cast<float*>(&lds[0][0]) + qt * MS * 64 + lane;
  if (hf == 1) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) mrg[(4 * db + r) * 64] = o[db][r];
    mrg[(4 * DB) * 64] = m;
    mrg[(4 * DB + 1) * 64] = l;
  }
  __syncthreads();
  if (hf == 1) return;
  {
    const float m1 = mrg[(4 * DB) * 64], l1 = mrg[(4 * DB + 1) * 64];
    const float mn = fmaxf(m, m1);
    const float ms = mn == -INFINITY ? 0.0f : mn;
    const float a0 = exp2_fast((m - ms) * a.scale_log2), a1 = exp2_fast((m1 - ms) * a.scale_log2);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) o[db][r] = o[db][r] * a0 + mrg[(4 * db + r) * 64] * a1;
    l = l * a0 + l1 * a1;
    m = mn;
  }
  const float lt = sum4(l);
  if (!qvalid) return;
  const float inv = 1.0f / lt;
  uint16_t* crow = a.ctx + (static_cast<int64_t>(b) * a.L + qi) * HD + hh * D;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    uint2 v;
    v.x = pack_bf16x2(o[db][0] * inv, o[db][1] * inv);
    v.y = pack_bf16x2(o[db][2] * inv, o[db][3] * inv);
    *reinterpret_cast<uint2*>(crow + 16 * db + 4 * g) = v;
  }
  if (g == 0) a.lse[(static_cast<int64_t>(b) * a.h + hh) * a.L + qi] = m * a.scale + logf(lt);
}

// Backward kernels.  NH = 1: each wave owns 16 rows (queries for dQ, keys
// for dK/dV) and walks every visible 64-row tile of the other side.  NH = 2
// (few (batch, head) pairs): two waves share each 16-row group and take one
// 32-row half of every tile each, which halves the dependent chain per wave
// and puts two waves on each SIMD; the halves' fp32 sums are added through
// LDS at the end (half 0 + half 1, a fixed order).

// Adds the NV fp32 vectors of the half-1 wave of each group to those of the
// half-0 wave through `buf` (NG * NV * 64 vectors); every thread of the block
// must call it.
template <int NV, int NG>
__device__ __forceinline__ void merge_halves(f32x4_t* x, f32x4_t* buf, int grp, int half, int lane) {
  if (half == 1) {
#pragma unroll
    for (int v = 0; v < NV; ++v) buf[(grp * NV + v) * 64 + lane] = x[v];
  }
  __syncthreads();
  if (half == 0) {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const f32x4_t y = buf[(grp * NV + v) * 64 + lane];
#pragma unroll
      for (int r = 0; r < 4; ++r) x[v][r] += y[r];
    }
  }
}

// dvec[b, h, l] = rowsum(dO * O) of query row l: D/8 lanes per row, one
// 16-byte chunk of dO and of O each, then a fixed-order butterfly.
template <int D>
__global__ __launch_bounds__(256) void attn_dvec_kernel(const AttnArgs a) {
  constexpr int LPR = D / 8, RPB = 256 / LPR;  // lanes per (token, head) row, rows per block
  const int64_t T = static_cast<int64_t>(a.B) * a.L, HD = static_cast<int64_t>(a.h) * D;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * RPB + threadIdx.x / LPR;
  const int c = threadIdx.x % LPR;
  const bool ok = idx < T * a.h;
  const int64_t t = ok ? idx / a.h : 0;
  const int hh = ok ? static_cast<int>(idx - t * a.h) : 0;
  float x[8], y[8];
  unpack8(ld16_or_zero(a.ctx + t * HD + hh * D + 8 * c, ok), x);
  unpack8(ld16_or_zero(a.dctx + t * HD + hh * D + 8 * c, ok), y);
  float acc = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc = fmaf(x[e], y[e], acc);
#pragma unroll
  for (int o = LPR / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if (ok && c == 0) {
    const int64_t b = t / a.L, l = t - b * a.L;
    const_cast<float*>(a.dvec)[(b * a.h + hh) * a.L + l] = acc;
  }
}

// dQ from the stored dS^T (the dK/dV kernel of this form writes it): per
// 64-query block, dQ^T += K^T dS^T over the visible 64-key tiles, with no
// recomputation of S and dP.  Waves (grp, half): 16 queries, keys 32*half ..
// +31 of each tile; both operands are transposed LDS reads of row tiles (K
// rows; dS^T rows are keys, columns queries).  The halves' sums are added
// through LDS at the end.  Each tile costs a fixed chain (barrier, LDS reads,
// products) of about a microsecond; a deeper tile ring and 4-wave blocks
// with a third of the LDS reads both measured slower.
template <int D>
__global__ __launch_bounds__(512) void attn_bwd_dq_ds_kernel(const AttnArgs a) {
  constexpr int NT = 512, NG = 4, BQ = 64, DB = D / 16, TS = D / 64 * 512;
  __shared__ uint4 lds_k[2][TS];
  __shared__ uint4 lds_s[2][512];  // one 64 x 64 tile of dS^T
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, qc = lane & 15;
  const int grp = wave % NG, half = wave / NG;
  const int nbh = a.B * a.h;
  const int bh = blockIdx.x % nbh;
  const int qb = a.nblk - 1 - static_cast<int>(blockIdx.x / nbh);  // heavy (late) query blocks first
  const int b = bh / a.h, hh = bh % a.h;
  const int64_t S3 = 3LL * a.h * D;
  const uint16_t* base = a.qkv + static_cast<int64_t>(b) * a.L * S3;
  const int q0 = qb * BQ, qi = q0 + grp * 16 + qc;

  RowTileDma<D, NT> tk;
  RowTileDma<64, NT> ts_;  // dS^T tile (key tile, query tile qb): keys as rows, queries as columns
  tk.init(base + static_cast<int64_t>(a.h) * D + hh * D, S3, a.L, tid);
  const int nt = (a.L + 63) / 64;
  ts_.init(a.dst + static_cast<int64_t>(bh) * nt * nt * 4096, 64, nt * nt * 64, tid);
  f32x4_t dq[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dq[db] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  const int kv_end = a.causal ? min(a.L, q0 + BQ) : a.L;
  const int nkb = (kv_end + 63) / 64;
  tk.issue(lds_k[0], 0);
  ts_.issue(lds_s[0], 64 * qb);
  wait_vm_lds();
  __syncthreads();
  for (int it = 0; it < nkb; ++it) {
    const int kv0 = it * 64, cur = it & 1;
    if (it + 1 < nkb) {  // the other buffer's reads retired before the last barrier
      tk.issue(lds_k[cur ^ 1], kv0 + 64);
      ts_.issue(lds_s[cur ^ 1], 64 * ((it + 1) * nt + qb));
    }
    if (!(a.causal && kv0 + 32 * half > q0 + grp * 16 + 15)) {  // else dS is zero for these keys
      const uint4 d = tr_frag(lds_s[cur], 16 * grp, half, lane);
#pragma unroll
      for (int d4 = 0; d4 < DB; d4 += 4) {  // K^T fragments four at a time, in flight together
        uint4 fk[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) fk[j] = tr_frag(lds_k[cur], 16 * (d4 + j), half, lane);
#pragma unroll
        for (int j = 0; j < 4; ++j) dq[d4 + j] = mfma_16x16x32(fk[j], d, dq[d4 + j]);
      }
    }
    wait_vm_lds();  // this wave's copies of the next tiles landed; its reads of these retired
    __syncthreads();
  }
  static_assert(NG * DB * 64 * 16 <= sizeof(lds_k), "merge buffer exceeds the tile buffers");
  merge_halves<DB, NG>(dq, reinterpret_cast<f32x4_t*>(&lds_k[0][0]), grp, half, lane);
  if (half != 0 || qi >= a.L) return;
  uint16_t* row = a.dqkv + (static_cast<int64_t>(b) * a.L + qi) * S3 + hh * D;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    uint2 v;
    v.x = pack_bf16x2(dq[db][0] * a.scale, dq[db][1] * a.scale);
    v.y = pack_bf16x2(dq[db][2] * a.scale, dq[db][3] * a.scale);
    *reinterpret_cast<uint2*>(row + 16 * db + 4 * (lane >> 4)) = v;
  }
}

// WPE: at least this many waves per SIMD (a register cap: 4 keeps two 8-wave
// blocks on a CU, which pays when every block carries the same work).
template <int D, int NW, int NH, int WPE = 1>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(WPE))) void attn_bwd_dq_kernel(
    const AttnArgs a) {
  constexpr int NT = 64 * NW, NG = NW / NH, BQ = 16 * NG, DB = D / 16, KS = D / 32, TS = D / 64 * 512;
  constexpr int SUB = 4 / NH;  // 16-key sub-blocks per wave per tile
  static_assert(NH == 1 || NH == 2, "one or two waves per row group");
  __shared__ uint4 lds_k[2][TS];
  __shared__ uint4 lds_v[2][TS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, qc = lane & 15, g = lane >> 4;
  const int grp = wave % NG, half = wave / NG;
  const int nbh = a.B * a.h;
  const int bh = blockIdx.x % nbh;
  const int qb = a.nblk - 1 - static_cast<int>(blockIdx.x / nbh);
  const int b = bh / a.h, hh = bh % a.h;
  const int64_t S3 = 3LL * a.h * D, HD = static_cast<int64_t>(a.h) * D;
  const uint16_t* base = a.qkv + static_cast<int64_t>(b) * a.L * S3;
  const int q0 = qb * BQ, qw0 = q0 + grp * 16, qi = qw0 + qc;
  const bool qvalid = qi < a.L;
  const int64_t trow = static_cast<int64_t>(b) * a.L + qi;

  // The first K and V tiles are in flight while the rows below load.
  RowTileDma<D, NT> tk, tv;
  tk.init(base + HD + hh * D, S3, a.L, tid);
  tv.init(base + 2 * HD + hh * D, S3, a.L, tid);
  tk.issue(lds_k[0], 0);
  tv.issue(lds_v[0], 0);

  const int64_t sidx = (static_cast<int64_t>(b) * a.h + hh) * a.L + qi;
  const float lse2 = qvalid ? a.lse[sidx] * kLog2eA : 0.0f;  // loaded before the dvec store below
  uint4 qf[KS], dof[KS];
  float dq_d = 0.0f;  // rowsum(dO * O) of query qi: this lane's 32 columns, then the 4 lanes of the query
#pragma unroll
  for (int st = 0; st < KS; ++st) {
    qf[st] = ld16_or_zero(base + static_cast<int64_t>(qi) * S3 + hh * D + 32 * st + 8 * kgrp(g), qvalid);
    dof[st] = ld16_or_zero(a.dctx + trow * HD + hh * D + 32 * st + 8 * kgrp(g), qvalid);
    float x[8], y[8];
    unpack8(dof[st], x);
    unpack8(ld16_or_zero(a.ctx + trow * HD + hh * D + 32 * st + 8 * kgrp(g), qvalid), y);
#pragma unroll
    for (int e = 0; e < 8; ++e) dq_d = fmaf(x[e], y[e], dq_d);
  }
  dq_d = sum4(dq_d);
  // The dK/dV kernel, launched next, reads it back.
  if (qvalid && g == 0 && half == 0) const_cast<float*>(a.dvec)[sidx] = dq_d;

  f32x4_t dq[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dq[db] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // Keys 0 .. key_lim are visible to query qi (none past L, none after qi
  // when causal, none for a query past L): one compare per score, no
  // branches (a short-circuit test here compiled to per-element branches).
  const int key_lim = !qvalid ? -1 : (a.causal ? min(a.L - 1, qi) : a.L - 1);
  const int kv_end = a.causal ? min(a.L, q0 + BQ) : a.L;
  const int nkb = (kv_end + 63) / 64;
  wait_compiler_loads();  // the Q, dO and O rows, lse
  wait_vm_lds();
  __syncthreads();
  for (int it = 0; it < nkb; ++it) {
    const int kv0 = it * 64, cur = it & 1;
    const int ks0 = kv0 + 16 * SUB * half;  // first key of this wave's part of the tile
    const bool more = it + 1 < nkb;
    if (more) {  // the other buffer's reads retired before the last barrier
      tk.issue(lds_k[cur ^ 1], kv0 + 64);
      tv.issue(lds_v[cur ^ 1], kv0 + 64);
    }
    if (!(a.causal && ks0 > qw0 + 15)) {
      const uint4* kt_ = lds_k[cur];
      const uint4* vt_ = lds_v[cur];
      f32x4_t ds[SUB];
#pragma unroll
      for (int j = 0; j < SUB; ++j) {
        const int kb = SUB * half + j;
        f32x4_t sv = {0.0f, 0.0f, 0.0f, 0.0f}, dp = {0.0f, 0.0f, 0.0f, 0.0f};
        uint4 kfr[KS], vfr[KS];  // all of the step's K and V fragments in flight together
#pragma unroll
        for (int st = 0; st < KS; ++st) {
          kfr[st] = row_frag(kt_, 16 * kb, st, lane);
          vfr[st] = row_frag(vt_, 16 * kb, st, lane);
        }
#pragma unroll
        for (int st = 0; st < KS; ++st) {
          sv = mfma_16x16x32(kfr[st], qf[st], sv);
          dp = mfma_16x16x32(vfr[st], dof[st], dp);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = kv0 + 16 * kb + 4 * g + r;
          const bool vis = key <= key_lim;
          // exp2(-inf) = 0: a select on the argument, not on the exponential, keeps
          // the loop free of per-element branches.
          const float p = exp2_fast(vis ? fmaf(sv[r], a.scale_log2, -lse2) : -INFINITY);
          ds[j][r] = p * (dp[r] - dq_d);
        }
      }
#pragma unroll
      for (int t2 = 0; t2 < SUB / 2; ++t2) {
        const uint4 d = pack_pair(ds[2 * t2], ds[2 * t2 + 1]);
#pragma unroll
        for (int d4 = 0; d4 < DB; d4 += 4) {  // K^T fragments four at a time, in flight together
          uint4 fk[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) fk[j] = tr_frag(kt_, 16 * (d4 + j), (SUB / 2) * half + t2, lane);
#pragma unroll
          for (int j = 0; j < 4; ++j) dq[d4 + j] = mfma_16x16x32(fk[j], d, dq[d4 + j]);
        }
      }
    }
    wait_vm_lds();  // this wave's copies of the next tile landed; its reads of this one retired
    __syncthreads();
  }
  if constexpr (NH == 2) {
    static_assert(NG * DB * 64 * 16 <= sizeof(lds_k), "merge buffer exceeds the tile buffers");
    merge_halves<DB, NG>(dq, reinterpret_cast<f32x4_t*>(&lds_k[0][0]), grp, half, lane);
    if (half != 0) return;
  }
  if (!qvalid) return;
  uint16_t* row = a.dqkv + trow * S3 + hh * D;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    uint2 v;
    v.x = pack_bf16x2(dq[db][0] * a.scale, dq[db][1] * a.scale);
    v.y = pack_bf16x2(dq[db][2] * a.scale, dq[db][3] * a.scale);
    *reinterpret_cast<uint2*>(row + 16 * db + 4 * g) = v;
  }
}

// At most 256 registers: two waves per SIMD also with 4-wave blocks, whose
// launch bound alone would let the compiler take more and run one.
template <int D, int NW, int NH>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2))) void attn_bwd_dkv_kernel(
    const AttnArgs a) {
  constexpr int NT = 64 * NW, NG = NW / NH, BK = 16 * NG, DB = D / 16, KS = D / 32, TS = D / 64 * 512;
  constexpr int SUB = 4 / NH;  // 16-query sub-blocks per wave per tile
  static_assert(NH == 1 || NH == 2, "one or two waves per row group");
  __shared__ uint4 lds_q[2][TS];
  __shared__ uint4 lds_do[2][TS];
  __shared__ __align__(16) float lds_lse[2][64];
  __shared__ __align__(16) float lds_dv[2][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, kc = lane & 15, g = lane >> 4;
  const int grp = wave % NG, half = wave / NG;
  const int nbh = a.B * a.h;
  const int bh = blockIdx.x % nbh;
  const int kb = static_cast<int>(blockIdx.x / nbh);  // early key blocks see the most queries
  const int b = bh / a.h, hh = bh % a.h;
  const int64_t S3 = 3LL * a.h * D, HD = static_cast<int64_t>(a.h) * D;
  const uint16_t* base = a.qkv + static_cast<int64_t>(b) * a.L * S3;
  const int k0 = kb * BK, kw0 = k0 + grp * 16, kj = kw0 + kc;
  const bool kvalid = kj < a.L;

  uint4 kf[KS], vf[KS];  // K^T, V^T as B operands: key kj, d = 32 st + 8 kgrp(g) .. +7
#pragma unroll
  for (int st = 0; st < KS; ++st) {
    kf[st] = ld16_or_zero(base + static_cast<int64_t>(kj) * S3 + HD + hh * D + 32 * st + 8 * kgrp(g), kvalid);
    vf[st] = ld16_or_zero(base + static_cast<int64_t>(kj) * S3 + 2 * HD + hh * D + 32 * st + 8 * kgrp(g), kvalid);
  }
  const uint16_t* dbase = a.dctx + static_cast<int64_t>(b) * a.L * HD;
  const int64_t sbase = (static_cast<int64_t>(b) * a.h + hh) * a.L;

  f32x4_t dkv[2 * DB];  // dK in [0, DB), dV in [DB, 2 DB)
#pragma unroll
  for (int v = 0; v < 2 * DB; ++v) dkv[v] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // Queries q_lo .. L-1 see key kj (as key_lim in dQ).
  const int q_lo = !kvalid ? 0x7fffffff : (a.causal ? kj : 0);
  const int q_begin = a.causal ? (k0 / 64) * 64 : 0;
  const int nqb = (a.L - q_begin + 63) / 64;
  RowTileDma<D, NT> tq, tdo;
  tq.init(base + hh * D, S3, a.L, tid);
  tdo.init(dbase + hh * D, HD, a.L, tid);
  VecDma vl, vd;  // lse and dvec of the tile's queries (zeros past L)
  vl.init(a.lse + sbase, a.L);
  vd.init(a.dvec + sbase, a.L);
  auto fetch = [&](int buf, int q0) {
    tq.issue(lds_q[buf], q0);
    tdo.issue(lds_do[buf], q0);
    if (wave == 0) {
      vl.issue(lds_lse[buf], q0, lane);
      vd.issue(lds_dv[buf], q0, lane);
    }
  };
  if (nqb > 0) fetch(0, q_begin);
  wait_compiler_loads();  // the K and V fragments
  wait_vm_lds();
  __syncthreads();
  for (int it = 0; it < nqb; ++it) {
    const int q0 = q_begin + it * 64, cur = it & 1;
    const int qs0 = q0 + 16 * SUB * half;  // first query of this wave's part of the tile
    const bool more = it + 1 < nqb;
    if (more) fetch(cur ^ 1, q0 + 64);  // the other buffer's reads retired before the last barrier
    if (!(a.causal && qs0 + 16 * SUB - 1 < kw0)) {  // else every such query precedes this wave's keys
      const uint4* qt_ = lds_q[cur];
      const uint4* dot_ = lds_do[cur];
      f32x4_t p[SUB], ds[SUB];
      // lse and dvec of this lane's queries 16 qb4 + 4 g .. +3, one 16-byte
      // read each, issued before the MFMAs that they wait for.
      f32x4_t lse4[SUB], dv4[SUB];
#pragma unroll
      for (int j = 0; j < SUB; ++j) {
        const int ql0 = 16 * (SUB * half + j) + 4 * g;
        lse4[j] = *reinterpret_cast<const f32x4_t*>(&lds_lse[cur][ql0]);
        dv4[j] = *reinterpret_cast<const f32x4_t*>(&lds_dv[cur][ql0]);
      }
#pragma unroll
      for (int j = 0; j < SUB; ++j) {
        const int qb4 = SUB * half + j;
        f32x4_t sv = {0.0f, 0.0f, 0.0f, 0.0f}, dp = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int st = 0; st < KS; ++st) {
          sv = mfma_16x16x32(row_frag(qt_, 16 * qb4, st, lane), kf[st], sv);
          dp = mfma_16x16x32(row_frag(dot_, 16 * qb4, st, lane), vf[st], dp);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int ql = 16 * qb4 + 4 * g + r, q = q0 + ql;
          const bool vis = (q >= q_lo) & (q < a.L);
          p[j][r] = exp2_fast(vis ? fmaf(sv[r], a.scale_log2, -(lse4[j][r] * kLog2eA)) : -INFINITY);  // as in dQ
          ds[j][r] = p[j][r] * (dp[r] - dv4[j][r]);
        }
      }
      // Compiled out of the one-wave-per-row form, which never stores dS^T:
      // there the store's registers took it past 128 VGPRs, one block per CU.
      if (NH == 2 && a.dst != nullptr) {
        // dS^T in 64 x 64 tiles, each 8 KiB contiguous ([B h][key tile][query
        // tile][key][query]), bf16 as the dK product takes them: this lane's 4
        // consecutive queries per 16-query block.  Keys and queries past L
        // carry zeros (p is zero there), so every tile that the dQ kernel
        // reads is fully defined.
        const int nt = (a.L + 63) / 64;
        uint16_t* tile = a.dst + ((static_cast<int64_t>(bh) * nt + kb) * nt + q0 / 64) * 4096 + (kj - k0) * 64;
#pragma unroll
        for (int j = 0; j < SUB; ++j)
          *reinterpret_cast<uint2*>(tile + 16 * (SUB * half + j) + 4 * g) =
              make_uint2(pack_bf16x2(ds[j][0], ds[j][1]), pack_bf16x2(ds[j][2], ds[j][3]));
      }
#pragma unroll
      for (int t2 = 0; t2 < SUB / 2; ++t2) {
        const int t = (SUB / 2) * half + t2;
        const uint4 pp = pack_pair(p[2 * t2], p[2 * t2 + 1]), dd = pack_pair(ds[2 * t2], ds[2 * t2 + 1]);
#pragma unroll
        for (int d4 = 0; d4 < DB; d4 += 4) {  // fragments four at a time, in flight together
          uint4 fo[4], fq[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            fo[j] = tr_frag(dot_, 16 * (d4 + j), t, lane);
            fq[j] = tr_frag(qt_, 16 * (d4 + j), t, lane);
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            dkv[DB + d4 + j] = mfma_16x16x32(fo[j], pp, dkv[DB + d4 + j]);
            dkv[d4 + j] = mfma_16x16x32(fq[j], dd, dkv[d4 + j]);
          }
        }
      }
    }
    wait_vm_lds();  // this wave's copies of the next tiles landed; its reads of these retired
    __syncthreads();
  }
  if constexpr (NH == 2) {
    // dK through the Q tile buffers, then dV through the dO tile buffers.
    static_assert(NG * DB * 64 * 16 <= sizeof(lds_q), "merge buffer exceeds the tile buffers");
    merge_halves<DB, NG>(dkv, reinterpret_cast<f32x4_t*>(&lds_q[0][0]), grp, half, lane);
    merge_halves<DB, NG>(dkv + DB, reinterpret_cast<f32x4_t*>(&lds_do[0][0]), grp, half, lane);
    if (half != 0) return;
  }
  if (!kvalid) return;
  uint16_t* row = a.dqkv + (static_cast<int64_t>(b) * a.L + kj) * S3 + hh * D;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    uint2 vk, vv;
    vk.x = pack_bf16x2(dkv[db][0] * a.scale, dkv[db][1] * a.scale);
    vk.y = pack_bf16x2(dkv[db][2] * a.scale, dkv[db][3] * a.scale);
    vv.x = pack_bf16x2(dkv[DB + db][0], dkv[DB + db][1]);
    vv.y = pack_bf16x2(dkv[DB + db][2], dkv[DB + db][3]);
    *reinterpret_cast<uint2*>(row + HD + 16 * db + 4 * g) = vk;
    *reinterpret_cast<uint2*>(row + 2 * HD + 16 * db + 4 * g) = vv;
  }
}

// Waves per block (16 rows each): 8 (128 rows, half the tile loads per row)
// when that still gives two blocks per CU, else 4 (64 rows).
static int attn_waves(int B, int L, int h) {
  const int64_t blocks8 = static_cast<int64_t>(B) * h * ceil_div(L, 128);
  return blocks8 >= 512 ? 8 : 4;
}

// Unused dynamic LDS that keeps a causal block with `lds` bytes of static LDS
// alone on its CU (static + pad > 80 KiB, half the CU's 160 KiB).  The
// heaviest causal blocks decide the kernel's time, and a block that shares
// its CU runs slower; lighter blocks then queue behind finished ones.
static unsigned causal_pad(const AttnArgs& a, unsigned lds) {
  return a.causal && lds < 96u * 1024u ? 96u * 1024u - lds : 0u;
}

// With 4-wave blocks (few (batch, head) pairs) the forward runs the split-key
// kernel instead: the same 64-query blocks on 8 waves.
template <int D, int NW>
static void launch_fwd(AttnArgs a, hipStream_t s) {
  a.nblk = static_cast<int>(ceil_div(a.L, 16 * NW));
  if constexpr (NW == 4) {
    const unsigned grid = static_cast<unsigned>(a.nblk * a.B * a.h);
    if (a.causal) attn_fwd_par_kernel<D><<<grid, 512, causal_pad(a, 1024u * D), s>>>(a);
    else attn_fwd_split_kernel<D><<<grid, 512, 0, s>>>(a);
  }
  else attn_fwd_kernel<D, NW><<<static_cast<unsigned>(a.nblk * a.B * a.h), 64 * NW, 0, s>>>(a);
}

// With 4-wave blocks (few pairs) both backward kernels run the same 64-row
// blocks on 8 waves, two per 16-row group.
template <int D, int NW>
static void launch_bwd(AttnArgs a, hipStream_t s) {
  a.nblk = static_cast<int>(ceil_div(a.L, 16 * NW));
  const unsigned grid = static_cast<unsigned>(a.nblk * a.B * a.h);
  if constexpr (NW == 4) {
    if (a.dst != nullptr) {  // stored-dS form: dvec, dK/dV writing dS^T, dQ from it
      attn_dvec_kernel<D><<<static_cast<unsigned>(ceil_div(static_cast<int64_t>(a.B) * a.L * a.h, 256 / (D / 8))),
                             256, 0, s>>>(a);
      attn_bwd_dkv_kernel<D, 8, 2><<<grid, 512, 0, s>>>(a);
      attn_bwd_dq_ds_kernel<D><<<grid, 512, 0, s>>>(a);
      return;
    }
    if (a.causal) attn_bwd_dq_kernel<D, 8, 2><<<grid, 512, causal_pad(a, 512u * D), s>>>(a);
    else attn_bwd_dq_kernel<D, 8, 2, 4><<<grid, 512, 0, s>>>(a);
    attn_bwd_dkv_kernel<D, 8, 2><<<grid, 512, 0, s>>>(a);
  } else {
    attn_bwd_dq_kernel<D, NW, 1><<<grid, 64 * NW, 0, s>>>(a);
    attn_bwd_dkv_kernel<D, NW, 1><<<grid, 64 * NW, 0, s>>>(a);
  }
}

static int validate_attn(const char* fn, mp_dtype dtype, int B, int L, int K, int h, int d) {
  MP_REQUIRE(dtype == MP_BF16, MP_ERR_DTYPE, "%s: attention runs in bf16 only", fn);
  MP_REQUIRE(B > 0 && L > 0 && K > 0 && h > 0, MP_ERR_SHAPE, "%s: bad shape", fn);
  MP_REQUIRE(d == 64 || d == 128, MP_ERR_UNSUPPORTED, "%s: head dim %d not in {64, 128}", fn, d);
  MP_REQUIRE(K % 8 == 0, MP_ERR_SHAPE, "%s: K=%d must be a multiple of 8", fn, K);
  MP_REQUIRE(static_cast<int64_t>(L) * 3 * h * d * 2 < 0x7fffffffLL, MP_ERR_UNSUPPORTED,
             "%s: one sequence's QKV exceeds 2 GiB", fn);
  return MP_OK;
}

static AttnArgs make_args(int B, int L, int h, int d, int causal) {
  AttnArgs a{};
  a.B = B;
  a.L = L;
  a.h = h;
  a.causal = causal ? 1 : 0;
  a.scale = 1.0f / sqrtf(static_cast<float>(d));
  a.scale_log2 = a.scale * kLog2eA;
  return a;
}

}  // namespace mp

using namespace mp;

extern "C" int mp_head_attention(mp_dtype dtype, int B, int L, int K, int h, int d, int causal, const void* X,
                                 const void* Wqkv_i, const void* bqkv_i, void* ctx_i, void* qkv, float* lse,
                                 hipStream_t s) {
  static const char* fn = "mp_head_attention";
  if (int rc = validate_attn(fn, dtype, B, L, K, h, d)) return rc;
  MP_REQUIRE_PTR(X);
  MP_REQUIRE_PTR(Wqkv_i);
  MP_REQUIRE_PTR(ctx_i);
  MP_REQUIRE_PTR(qkv);
  MP_REQUIRE_PTR(lse);
  MP_REQUIRE_ALIGN(X);
  MP_REQUIRE_ALIGN(Wqkv_i);
  MP_REQUIRE_OPT_ALIGN(bqkv_i);
  MP_REQUIRE_ALIGN(ctx_i);
  MP_REQUIRE_ALIGN(qkv);
  const int64_t T = static_cast<int64_t>(B) * L, N3 = 3LL * h * d;
  if (int rc = gemm(MP_BF16, NT, T, N3, K, X, K, Wqkv_i, K, qkv, N3, true, bqkv_i, MP_ACT_NONE, nullptr, false,
                    nullptr, 0, s))
    return rc;
  AttnArgs a = make_args(B, L, h, d, causal);
  a.qkv = static_cast<const uint16_t*>(qkv);
  a.ctx = static_cast<uint16_t*>(ctx_i);
  a.lse = lse;
  const int nw = attn_waves(B, L, h);
  if (d == 64) nw == 8 ? launch_fwd<64, 8>(a, s) : launch_fwd<64, 4>(a, s);
  else nw == 8 ? launch_fwd<128, 8>(a, s) : launch_fwd<128, 4>(a, s);
  return check_launch(fn);
}

// Bytes of the stored dS^T (64 x 64 bf16 tiles over [B h][L][L]) when the
// backward takes that form (4-wave blocks, at most 4096 keys), else 0.
static size_t attn_ds_bytes(int B, int L, int h) {
  if (attn_waves(B, L, h) != 4 || L > 4096) return 0;
  const size_t nt = static_cast<size_t>(ceil_div(L, 64));
  return static_cast<size_t>(B) * h * nt * nt * 8192;
}

// Workspace: dQKV, dvec, then one region that first holds dS^T (read by the
// dQ kernel) and then the split-k / column-sum scratch of the products after.
static size_t attn_bwd_parts(int B, int L, int K, int h, int d, size_t* dqkv_bytes, size_t* dvec_bytes) {
  const int64_t T = static_cast<int64_t>(B) * L, N3 = 3LL * h * d;
  *dqkv_bytes = align_up(static_cast<size_t>(T * N3) * 2, 256);
  *dvec_bytes = align_up(static_cast<size_t>(T * h) * 4, 256);
  const size_t sk = gemm_splitk_workspace(MP_BF16, N3, K, T);
  const size_t cs = colsum_workspace(T, N3);
  const size_t ds = attn_ds_bytes(B, L, h);
  return *dqkv_bytes + *dvec_bytes + std::max(ds, std::max(sk, cs));
}

extern "C" size_t mp_head_attention_bwd_workspace(mp_dtype dtype, int B, int L, int K, int h, int d) {
  if (dtype != MP_BF16 || B <= 0 || L <= 0 || K <= 0 || h <= 0 || (d != 64 && d != 128)) return 0;
  size_t a, b;
  return attn_bwd_parts(B, L, K, h, d, &a, &b);
}

extern "C" int mp_head_attention_bwd(mp_dtype dtype, int B, int L, int K, int h, int d, int causal, const void* X,
                                     const void* Wqkv_i, const void* qkv, const void* ctx_i, const float* lse,
                                     const void* dctx_i, void* dX_partial, float* dWqkv_i, float* dbqkv_i, void* ws,
                                     size_t ws_bytes, hipStream_t s) {
  static const char* fn = "mp_head_attention_bwd";
  if (int rc = validate_attn(fn, dtype, B, L, K, h, d)) return rc;
  MP_REQUIRE_PTR(X);
  MP_REQUIRE_PTR(Wqkv_i);
  MP_REQUIRE_PTR(qkv);
  MP_REQUIRE_PTR(ctx_i);
  MP_REQUIRE_PTR(lse);
  MP_REQUIRE_PTR(dctx_i);
  MP_REQUIRE_PTR(dX_partial);
  MP_REQUIRE_PTR(dWqkv_i);
  MP_REQUIRE_ALIGN(X);
  MP_REQUIRE_ALIGN(Wqkv_i);
  MP_REQUIRE_ALIGN(qkv);
  MP_REQUIRE_ALIGN(ctx_i);
  MP_REQUIRE_ALIGN(dctx_i);
  MP_REQUIRE_ALIGN(dX_partial);
  MP_REQUIRE_ALIGN(dWqkv_i);
  size_t dqkv_bytes, dvec_bytes;
  const size_t need = attn_bwd_parts(B, L, K, h, d, &dqkv_bytes, &dvec_bytes);
  MP_REQUIRE(ws != nullptr && ws_bytes >= need, MP_ERR_WORKSPACE, "%s: workspace needs %zu bytes", fn, need);
  MP_REQUIRE_ALIGN(ws);
  const int64_t T = static_cast<int64_t>(B) * L, N3 = 3LL * h * d;
  uint16_t* dqkv = static_cast<uint16_t*>(ws);
  float* dvec = reinterpret_cast<float*>(static_cast<char*>(ws) + dqkv_bytes);
  void* ws2 = static_cast<char*>(ws) + dqkv_bytes + dvec_bytes;
  AttnArgs a = make_args(B, L, h, d, causal);
  a.qkv = static_cast<const uint16_t*>(qkv);
  a.ctx = static_cast<uint16_t*>(const_cast<void*>(ctx_i));
  a.lse = const_cast<float*>(lse);
  a.dctx = static_cast<const uint16_t*>(dctx_i);
  a.dvec = dvec;
  a.dqkv = dqkv;
  if (attn_ds_bytes(B, L, h) != 0) a.dst = static_cast<uint16_t*>(ws2);
  const int nw = attn_waves(B, L, h);
  if (d == 64) nw == 8 ? launch_bwd<64, 8>(a, s) : launch_bwd<64, 4>(a, s);
  else nw == 8 ? launch_bwd<128, 8>(a, s) : launch_bwd<128, 4>(a, s);
  if (int rc = check_launch(fn)) return rc;
  // dX_partial[T,K] = dqkv[T,N3] * Wqkv_i[N3,K]
  if (int rc = gemm(MP_BF16, NN, T, K, N3, dqkv, N3, Wqkv_i, K, dX_partial, K, true, nullptr, MP_ACT_NONE, nullptr,
                    false, nullptr, 0, s))
    return rc;
  // dWqkv_i[N3,K] = dqkv^T * X
  if (int rc = gemm(MP_BF16, TN, N3, K, T, dqkv, N3, X, K, dWqkv_i, K, false, nullptr, MP_ACT_NONE, nullptr, true,
                    ws2, ws_bytes - dqkv_bytes - dvec_bytes, s))
    return rc;
  if (dbqkv_i != nullptr) return colsum(MP_BF16, T, N3, dqkv, dbqkv_i, ws2, s);
  return MP_OK;
}
