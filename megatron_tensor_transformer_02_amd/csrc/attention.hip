// Head-partitioned causal self-attention of one tensor-parallel rank: the
// fused QKV GEMM over the rank's heads, then attention per (batch, head)
// (heads are independent, so a rank's heads need no communication).
//
// Forward (flash-style, one pass over the keys): a wave owns 32 queries and
// computes S^T = K Q^T with 32x32x16 bf16 MFMAs, so each lane holds the
// scores of ONE query (16 of every 32 keys; its partner lane l^32 holds the
// other 16).  The online softmax therefore needs only a lane-pair exchange
// for the running max.  The probabilities' registers 8s..8s+7 are, as they
// stand, the B operand of O^T += V^T P^T for keys {16s+4g..+3, 16s+8+4g..+3}
// (g = lane / 32); the V^T fragments come from the plain V row tile through
// two LDS transpose reads (4 consecutive keys each) in that same key order,
// so P never leaves registers and no transposed tile is ever stored.
//
// Every kernel streams 64-row tiles through two LDS buffers: the next tile is
// loaded into registers while the current one is multiplied, then written to
// the other buffer (one barrier per tile).
//
// Backward (P recomputed from the saved log-sum-exp, no atomics):
//  * dQ kernel -- lanes own queries: S^T, dP^T = V dO^T, dS^T, dQ^T += K^T dS^T;
//  * dK/dV kernel -- lanes own keys: S = Q K^T, dV^T += dO^T P, dP = dO V^T,
//    dS, dK^T += Q^T dS.
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
  const float* dvec;     // [B, h, L] rowsum(dO * O)
  uint16_t* dqkv;        // [B*L, 3*h*D]      (backward)
  int B, L, h, causal;
  int nblk;              // query (or key) blocks per (batch, head)
  float scale;           // 1/sqrt(D)
  float scale_log2;      // log2(e)/sqrt(D)
};

// 8 consecutive bf16 of `p` (16-byte aligned) or zeros.
__device__ __forceinline__ uint4 ld16_or_zero(const uint16_t* p, bool ok) {
  return ok ? *reinterpret_cast<const uint4*>(p) : make_uint4(0, 0, 0, 0);
}

// Packs registers 8*s2 .. 8*s2+7 of a 32x32 result into a bf16 B operand.
__device__ __forceinline__ uint4 pack_half(const float* v, int s2) { return pack8(v + 8 * s2); }

// A 64-row x D-column tile of a [L, ld] bf16 matrix (a head slice), held in
// KH = D/64 LDS sub-tiles of the GEMM tile format (64 rows x 64 columns,
// rows of eight swizzled 16-byte chunks).  load() fetches rows r0..r0+63
// into registers (rows >= L read as zeros), store() writes them to LDS.
template <int D, int NT>
struct RowTile {
  TileLoader<64, true, NT> part[D / 64];
  __device__ __forceinline__ void load(const BufRes& rs, int64_t ld, int r0, int L, int tid) {
#pragma unroll
    for (int hf = 0; hf < D / 64; ++hf) part[hf].load(rs, ld, r0, L, 64 * hf, D, tid, r0);
  }
  __device__ __forceinline__ void store(uint4* lds, int tid) const {
#pragma unroll
    for (int hf = 0; hf < D / 64; ++hf) part[hf].store(lds + hf * 512, tid);
  }
};

// Row fragment (A or B operand) of a row tile: row `row`, k-step `st`
// (16 columns), lane group g.
__device__ __forceinline__ uint4 lds_row_frag(const uint4* tile, int row, int st, int g) {
  return tile[(st >> 2) * 512 + lds_slot(row, 2 * (st & 3) + g)];
}

// Byte address of element (r, d) of a row tile.
__device__ __forceinline__ const char* tile_elem(const uint4* tile, int r, int d) {
  return reinterpret_cast<const char*>(tile + (d >> 6) * 512 + lds_slot(r, (d & 63) >> 3)) + (d & 7) * 2;
}

// Transposed A-operand fragment from a row tile: operand row = tile column
// d = dt*32 + lane%32; its 8 k-slots are tile rows {kt*32 + 16*s2 + 4g .. +3}
// and {kt*32 + 16*s2 + 8 + 4g .. +3} (g = lane / 32), the register order of a
// 32x32 result used as the B operand.  Two transpose reads of 4 rows each.
__device__ __forceinline__ uint4 lds_tr_frag(const uint4* tile, int dt, int kt, int s2, int lane) {
  const int grp = lane >> 4, i = lane & 15;
  const int r = kt * 32 + 16 * s2 + 4 * (grp >> 1) + (i >> 2);
  const int d = dt * 32 + 16 * (grp & 1) + 4 * (i & 3);
  const uint2 lo = lds_read_tr16(tile_elem(tile, r, d));
  const uint2 hi = lds_read_tr16(tile_elem(tile, r + 8, d));
  return make_uint4(lo.x, lo.y, hi.x, hi.y);
}

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void attn_fwd_kernel(const AttnArgs a) {
  constexpr int NT = 64 * NW, BQ = 32 * NW, DT = D / 32, KS = D / 16, TS = D / 64 * 512;
  __shared__ uint4 lds_k[2][TS];
  __shared__ uint4 lds_v[2][TS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, frow = lane & 31, g = lane >> 5;
  const int nbh = a.B * a.h;
  const int bh = blockIdx.x % nbh;
  const int qb = a.nblk - 1 - static_cast<int>(blockIdx.x / nbh);  // heavy (late) query blocks first
  const int b = bh / a.h, hh = bh % a.h;
  const int64_t S3 = 3LL * a.h * D, HD = static_cast<int64_t>(a.h) * D;
  const uint16_t* base = a.qkv + static_cast<int64_t>(b) * a.L * S3;
  const int q0 = qb * BQ, qw0 = q0 + wave * 32, qi = qw0 + frow;
  const bool qvalid = qi < a.L;

  uint4 qf[KS];
#pragma unroll
  for (int st = 0; st < KS; ++st) qf[st] = ld16_or_zero(base + static_cast<int64_t>(qi) * S3 + hh * D + 16 * st + 8 * g, qvalid);

  const int64_t batch_bytes = static_cast<int64_t>(a.L) * S3 * 2;
  const BufRes rk = make_bufres(base + HD + hh * D, batch_bytes - (HD + hh * D) * 2);
  const BufRes rv = make_bufres(base + 2 * HD + hh * D, batch_bytes - (2 * HD + hh * D) * 2);

  float m = -INFINITY, l = 0.0f;
  f32x16_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.0f;

  const int kv_end = a.causal ? min(a.L, q0 + BQ) : a.L;
  const int nkb = (kv_end + 63) / 64;
  RowTile<D, NT> tk, tv;
  tk.load(rk, S3, 0, a.L, tid);
  tv.load(rv, S3, 0, a.L, tid);
  tk.store(lds_k[0], tid);
  tv.store(lds_v[0], tid);
  __syncthreads();
  for (int it = 0; it < nkb; ++it) {
    const int kv0 = it * 64, cur = it & 1;
    const bool more = it + 1 < nkb;
    if (more) {
      tk.load(rk, S3, kv0 + 64, a.L, tid);
      tv.load(rv, S3, kv0 + 64, a.L, tid);
    }
    if (!(a.causal && kv0 > qw0 + 31)) {  // else every key of the block is in this wave's future
      const uint4* kt_ = lds_k[cur];
      const uint4* vt_ = lds_v[cur];
      f32x16_t s[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kt][r] = 0.0f;
#pragma unroll
        for (int st = 0; st < KS; ++st) s[kt] = mfma_32x32x16(lds_row_frag(kt_, kt * 32 + frow, st, g), qf[st], s[kt]);
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kv0 + kt * 32 + mfma_row(r, lane);
          const bool vis = key < a.L && (!a.causal || key <= qi);
          if (!vis) s[kt][r] = -INFINITY;
          mx = fmaxf(mx, s[kt][r]);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mn = fmaxf(m, mx);
      const float ms = mn == -INFINITY ? 0.0f : mn;
      const float alpha = exp2f((m - ms) * a.scale_log2);
      float ps = 0.0f;
      uint4 pb[2][2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[r] = exp2f((s[kt][r] - ms) * a.scale_log2);
          ps += p[r];
        }
        pb[kt][0] = pack_half(p, 0);
        pb[kt][1] = pack_half(p, 1);
      }
      l = l * alpha + ps;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) o[dt] = mfma_32x32x16(lds_tr_frag(vt_, dt, kt, s2, lane), pb[kt][s2], o[dt]);
      }
      m = mn;
    }
    if (more) {
      tk.store(lds_k[cur ^ 1], tid);
      tv.store(lds_v[cur ^ 1], tid);
    }
    __syncthreads();
  }
  const float lt = l + __shfl_xor(l, 32, 64);
  if (!qvalid) return;
  const float inv = 1.0f / lt;
  uint16_t* crow = a.ctx + (static_cast<int64_t>(b) * a.L + qi) * HD + hh * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d = dt * 32 + 8 * q4 + 4 * g;
      uint2 v;
      v.x = pack_bf16x2(o[dt][4 * q4] * inv, o[dt][4 * q4 + 1] * inv);
      v.y = pack_bf16x2(o[dt][4 * q4 + 2] * inv, o[dt][4 * q4 + 3] * inv);
      *reinterpret_cast<uint2*>(crow + d) = v;
    }
  if (g == 0) a.lse[(static_cast<int64_t>(b) * a.h + hh) * a.L + qi] = m * a.scale + logf(lt);
}

// dvec[b, h, l] = sum_d dctx[t, h*D + d] * ctx[t, h*D + d]; one thread per (t, head).
template <int D>
__global__ __launch_bounds__(256) void attn_dvec_kernel(const AttnArgs a) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t T = static_cast<int64_t>(a.B) * a.L;
  if (idx >= T * a.h) return;
  const int64_t t = idx / a.h;
  const int hh = static_cast<int>(idx - t * a.h);
  const int64_t HD = static_cast<int64_t>(a.h) * D;
  const uint16_t* o = a.ctx + t * HD + hh * D;
  const uint16_t* dO = a.dctx + t * HD + hh * D;
  float acc = 0.0f;
#pragma unroll
  for (int c = 0; c < D / 8; ++c) {
    float x[8], y[8];
    unpack8(*reinterpret_cast<const uint4*>(o + 8 * c), x);
    unpack8(*reinterpret_cast<const uint4*>(dO + 8 * c), y);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += x[e] * y[e];
  }
  const int64_t b = t / a.L, l = t - b * a.L;
  const_cast<float*>(a.dvec)[(b * a.h + hh) * a.L + l] = acc;
}

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void attn_bwd_dq_kernel(const AttnArgs a) {
  constexpr int NT = 64 * NW, BQ = 32 * NW, DT = D / 32, KS = D / 16, TS = D / 64 * 512;
  __shared__ uint4 lds_k[2][TS];
  __shared__ uint4 lds_v[2][TS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, frow = lane & 31, g = lane >> 5;
  const int nbh = a.B * a.h;
  const int bh = blockIdx.x % nbh;
  const int qb = a.nblk - 1 - static_cast<int>(blockIdx.x / nbh);
  const int b = bh / a.h, hh = bh % a.h;
  const int64_t S3 = 3LL * a.h * D, HD = static_cast<int64_t>(a.h) * D;
  const uint16_t* base = a.qkv + static_cast<int64_t>(b) * a.L * S3;
  const int q0 = qb * BQ, qw0 = q0 + wave * 32, qi = qw0 + frow;
  const bool qvalid = qi < a.L;
  const int64_t trow = static_cast<int64_t>(b) * a.L + qi;

  uint4 qf[KS], dof[KS];
#pragma unroll
  for (int st = 0; st < KS; ++st) {
    qf[st] = ld16_or_zero(base + static_cast<int64_t>(qi) * S3 + hh * D + 16 * st + 8 * g, qvalid);
    dof[st] = ld16_or_zero(a.dctx + trow * HD + hh * D + 16 * st + 8 * g, qvalid);
  }
  const int64_t sidx = (static_cast<int64_t>(b) * a.h + hh) * a.L + qi;
  const float lse2 = qvalid ? a.lse[sidx] * kLog2eA : 0.0f;
  const float dq_d = qvalid ? a.dvec[sidx] : 0.0f;

  const int64_t batch_bytes = static_cast<int64_t>(a.L) * S3 * 2;
  const BufRes rk = make_bufres(base + HD + hh * D, batch_bytes - (HD + hh * D) * 2);
  const BufRes rv = make_bufres(base + 2 * HD + hh * D, batch_bytes - (2 * HD + hh * D) * 2);

  f32x16_t dq[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[dt][r] = 0.0f;

  const int kv_end = a.causal ? min(a.L, q0 + BQ) : a.L;
  const int nkb = (kv_end + 63) / 64;
  RowTile<D, NT> tk, tv;
  tk.load(rk, S3, 0, a.L, tid);
  tv.load(rv, S3, 0, a.L, tid);
  tk.store(lds_k[0], tid);
  tv.store(lds_v[0], tid);
  __syncthreads();
  for (int it = 0; it < nkb; ++it) {
    const int kv0 = it * 64, cur = it & 1;
    const bool more = it + 1 < nkb;
    if (more) {
      tk.load(rk, S3, kv0 + 64, a.L, tid);
      tv.load(rv, S3, kv0 + 64, a.L, tid);
    }
    if (!(a.causal && kv0 > qw0 + 31)) {
      const uint4* kt_ = lds_k[cur];
      const uint4* vt_ = lds_v[cur];
      uint4 dsb[2][2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        f32x16_t sv, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) sv[r] = dp[r] = 0.0f;
#pragma unroll
        for (int st = 0; st < KS; ++st) {
          sv = mfma_32x32x16(lds_row_frag(kt_, kt * 32 + frow, st, g), qf[st], sv);
          dp = mfma_32x32x16(lds_row_frag(vt_, kt * 32 + frow, st, g), dof[st], dp);
        }
        float ds[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kv0 + kt * 32 + mfma_row(r, lane);
          const bool vis = qvalid && key < a.L && (!a.causal || key <= qi);
          const float p = vis ? exp2f(sv[r] * a.scale_log2 - lse2) : 0.0f;
          ds[r] = p * (dp[r] - dq_d);
        }
        dsb[kt][0] = pack_half(ds, 0);
        dsb[kt][1] = pack_half(ds, 1);
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) dq[dt] = mfma_32x32x16(lds_tr_frag(kt_, dt, kt, s2, lane), dsb[kt][s2], dq[dt]);
    }
    if (more) {
      tk.store(lds_k[cur ^ 1], tid);
      tv.store(lds_v[cur ^ 1], tid);
    }
    __syncthreads();
  }
  if (!qvalid) return;
  uint16_t* row = a.dqkv + trow * S3 + hh * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d = dt * 32 + 8 * q4 + 4 * g;
      uint2 v;
      v.x = pack_bf16x2(dq[dt][4 * q4] * a.scale, dq[dt][4 * q4 + 1] * a.scale);
      v.y = pack_bf16x2(dq[dt][4 * q4 + 2] * a.scale, dq[dt][4 * q4 + 3] * a.scale);
      *reinterpret_cast<uint2*>(row + d) = v;
    }
}

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void attn_bwd_dkv_kernel(const AttnArgs a) {
  constexpr int NT = 64 * NW, BK = 32 * NW, DT = D / 32, KS = D / 16, TS = D / 64 * 512;
  __shared__ uint4 lds_q[2][TS];
  __shared__ uint4 lds_do[2][TS];
  __shared__ float lds_lse[2][64], lds_dv[2][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, frow = lane & 31, g = lane >> 5;
  const int nbh = a.B * a.h;
  const int bh = blockIdx.x % nbh;
  const int kb = static_cast<int>(blockIdx.x / nbh);  // early key blocks see the most queries
  const int b = bh / a.h, hh = bh % a.h;
  const int64_t S3 = 3LL * a.h * D, HD = static_cast<int64_t>(a.h) * D;
  const uint16_t* base = a.qkv + static_cast<int64_t>(b) * a.L * S3;
  const int k0 = kb * BK, kw0 = k0 + wave * 32, kj = kw0 + frow;
  const bool kvalid = kj < a.L;

  uint4 kf[KS], vf[KS];
#pragma unroll
  for (int st = 0; st < KS; ++st) {
    kf[st] = ld16_or_zero(base + static_cast<int64_t>(kj) * S3 + HD + hh * D + 16 * st + 8 * g, kvalid);
    vf[st] = ld16_or_zero(base + static_cast<int64_t>(kj) * S3 + 2 * HD + hh * D + 16 * st + 8 * g, kvalid);
  }
  const int64_t batch_bytes = static_cast<int64_t>(a.L) * S3 * 2;
  const BufRes rq = make_bufres(base + hh * D, batch_bytes - hh * D * 2);
  const uint16_t* dbase = a.dctx + static_cast<int64_t>(b) * a.L * HD;
  const BufRes rdo = make_bufres(dbase + hh * D, (static_cast<int64_t>(a.L) * HD - hh * D) * 2);
  const int64_t sbase = (static_cast<int64_t>(b) * a.h + hh) * a.L;

  f32x16_t dk[DT], dv[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) dk[dt][r] = dv[dt][r] = 0.0f;

  const int q_begin = a.causal ? (k0 / 64) * 64 : 0;
  const int nqb = (a.L - q_begin + 63) / 64;
  RowTile<D, NT> tq, tdo;
  float lse_r = 0.0f, dv_r = 0.0f;
  auto fetch = [&](int q0) {
    tq.load(rq, S3, q0, a.L, tid);
    tdo.load(rdo, HD, q0, a.L, tid);
    if (tid < 64) {
      const int q = q0 + tid;
      lse_r = q < a.L ? a.lse[sbase + q] * kLog2eA : 0.0f;
      dv_r = q < a.L ? a.dvec[sbase + q] : 0.0f;
    }
  };
  auto commit = [&](int buf) {
    tq.store(lds_q[buf], tid);
    tdo.store(lds_do[buf], tid);
    if (tid < 64) {
      lds_lse[buf][tid] = lse_r;
      lds_dv[buf][tid] = dv_r;
    }
  };
  if (nqb > 0) {
    fetch(q_begin);
    commit(0);
  }
  __syncthreads();
  for (int it = 0; it < nqb; ++it) {
    const int q0 = q_begin + it * 64, cur = it & 1;
    const bool more = it + 1 < nqb;
    if (more) fetch(q0 + 64);
    if (!(a.causal && q0 + 63 < kw0)) {  // else every query of the block precedes this wave's keys
      const uint4* qt_ = lds_q[cur];
      const uint4* dot_ = lds_do[cur];
      uint4 pb[2][2], dsb[2][2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        f32x16_t sv, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) sv[r] = dp[r] = 0.0f;
#pragma unroll
        for (int st = 0; st < KS; ++st) {
          sv = mfma_32x32x16(lds_row_frag(qt_, qt * 32 + frow, st, g), kf[st], sv);
          dp = mfma_32x32x16(lds_row_frag(dot_, qt * 32 + frow, st, g), vf[st], dp);
        }
        float p[16], ds[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ql = qt * 32 + mfma_row(r, lane);
          const int q = q0 + ql;
          const bool vis = kvalid && q < a.L && (!a.causal || kj <= q);
          p[r] = vis ? exp2f(sv[r] * a.scale_log2 - lds_lse[cur][ql]) : 0.0f;
          ds[r] = p[r] * (dp[r] - lds_dv[cur][ql]);
        }
        pb[qt][0] = pack_half(p, 0);
        pb[qt][1] = pack_half(p, 1);
        dsb[qt][0] = pack_half(ds, 0);
        dsb[qt][1] = pack_half(ds, 1);
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            dv[dt] = mfma_32x32x16(lds_tr_frag(dot_, dt, qt, s2, lane), pb[qt][s2], dv[dt]);
            dk[dt] = mfma_32x32x16(lds_tr_frag(qt_, dt, qt, s2, lane), dsb[qt][s2], dk[dt]);
          }
    }
    if (more) commit(cur ^ 1);
    __syncthreads();
  }
  if (!kvalid) return;
  uint16_t* row = a.dqkv + (static_cast<int64_t>(b) * a.L + kj) * S3 + hh * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d = dt * 32 + 8 * q4 + 4 * g;
      uint2 vk, vv;
      vk.x = pack_bf16x2(dk[dt][4 * q4] * a.scale, dk[dt][4 * q4 + 1] * a.scale);
      vk.y = pack_bf16x2(dk[dt][4 * q4 + 2] * a.scale, dk[dt][4 * q4 + 3] * a.scale);
      vv.x = pack_bf16x2(dv[dt][4 * q4], dv[dt][4 * q4 + 1]);
      vv.y = pack_bf16x2(dv[dt][4 * q4 + 2], dv[dt][4 * q4 + 3]);
      *reinterpret_cast<uint2*>(row + HD + d) = vk;
      *reinterpret_cast<uint2*>(row + 2 * HD + d) = vv;
    }
}

// Waves per block: 4 (128 queries) unless that leaves fewer than two blocks
// per CU, then 2 (64 queries).
static int attn_waves(int B, int L, int h) {
  const int64_t blocks4 = static_cast<int64_t>(B) * h * ceil_div(L, 128);
  return blocks4 >= 512 ? 4 : 2;
}

template <int D, int NW>
static void launch_fwd(AttnArgs a, hipStream_t s) {
  a.nblk = static_cast<int>(ceil_div(a.L, 32 * NW));
  attn_fwd_kernel<D, NW><<<static_cast<unsigned>(a.nblk * a.B * a.h), 64 * NW, 0, s>>>(a);
}

template <int D, int NW>
static void launch_bwd(AttnArgs a, hipStream_t s) {
  a.nblk = static_cast<int>(ceil_div(a.L, 32 * NW));
  const unsigned grid = static_cast<unsigned>(a.nblk * a.B * a.h);
  attn_bwd_dq_kernel<D, NW><<<grid, 64 * NW, 0, s>>>(a);
  attn_bwd_dkv_kernel<D, NW><<<grid, 64 * NW, 0, s>>>(a);
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
  if (d == 64) nw == 4 ? launch_fwd<64, 4>(a, s) : launch_fwd<64, 2>(a, s);
  else nw == 4 ? launch_fwd<128, 4>(a, s) : launch_fwd<128, 2>(a, s);
  return check_launch(fn);
}

static size_t attn_bwd_parts(int B, int L, int K, int h, int d, size_t* dqkv_bytes, size_t* dvec_bytes) {
  const int64_t T = static_cast<int64_t>(B) * L, N3 = 3LL * h * d;
  *dqkv_bytes = align_up(static_cast<size_t>(T * N3) * 2, 256);
  *dvec_bytes = align_up(static_cast<size_t>(T * h) * 4, 256);
  const size_t sk = gemm_splitk_workspace(MP_BF16, N3, K, T);
  const size_t cs = colsum_workspace(T, N3);
  return *dqkv_bytes + *dvec_bytes + (sk > cs ? sk : cs);
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
  const unsigned dgrid = static_cast<unsigned>(ceil_div(T * h, 256));
  if (d == 64) attn_dvec_kernel<64><<<dgrid, 256, 0, s>>>(a);
  else attn_dvec_kernel<128><<<dgrid, 256, 0, s>>>(a);
  const int nw = attn_waves(B, L, h);
  if (d == 64) nw == 4 ? launch_bwd<64, 4>(a, s) : launch_bwd<64, 2>(a, s);
  else nw == 4 ? launch_bwd<128, 4>(a, s) : launch_bwd<128, 2>(a, s);
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
