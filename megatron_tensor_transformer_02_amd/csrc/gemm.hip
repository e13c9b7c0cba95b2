// GEMM family of the tensor-parallel shard: C[M,N] = sum_k A(m,k) * B(n,k).
//
// Each operand is either K-contiguous (row-major [rows][K], the forward "NT"
// case) or MN-contiguous ([K][rows], as the weight in an input-gradient GEMM
// or both operands of a weight-gradient GEMM).  Both are copied into LDS as
// they lie in memory (16-byte chunks, swizzled); MN-contiguous fragments are
// then read with the LDS transpose read, so every layout runs the same MFMA
// loop and no transposed copy goes through HBM or through registers.
//
// bf16 kernel: 256-row tiles run 8 waves (two per SIMD), 128x128 tiles 4;
// block tile BM x BN x 64; each wave owns a (BM/WR) x (BN/(NW/WR)) piece of
// the output as 32x32 MFMA tiles (v_mfma_f32_32x32x16_bf16).  The k-loop is software-pipelined
// by hand (fragment double-buffering, next k-tile prefetched into registers,
// explicit MFMA/LDS/global-load interleave).  Workgroups are renumbered so
// each of the 8 XCDs takes a contiguous range of output tiles, walked in
// groups of tile-rows, for L2 reuse of the operand panels.
//
// Epilogues: bias + activation (+ pre-activation save), activation gradient,
// or fp32 split-K partials followed by a fixed-order reduce (deterministic).
#include <stdio.h>
#include <stdlib.h>

#include <mutex>

#include "gemm.h"
#include "mfma.h"

namespace mp {


struct GemmArgs {
  int64_t M, N, K;
  const void* A;
  int64_t lda;
  const void* B;
  int64_t ldb;
  void* C;            // [M, ldc], bf16 or fp32 (out_bf16)
  int64_t ldc;
  const void* bias;   // [N] in the input dtype, or NULL
  void* zsave;        // [M, ldc] pre-activation in the output dtype, or NULL
  const void* zin;    // [M, ldc] pre-activation (EPI_DACT), input dtype
  float* partial;     // [splits, M, N] fp32 (EPI_SPLITK)
  int64_t k_split;    // k-values per split, a multiple of 64
  int act;
  int out_bf16;
  int tiles_m, tiles_n, group_m;
  const int32_t* labels;  // [M] (EPI_LSE)
  int64_t v_start;        // first vocabulary row of the shard (EPI_LSE)
  float* lse_part;        // [M, lse_slots, 3] (EPI_LSE)
  int lse_slots;
  // Grouped GEMMs (one problem per group, shapes on the device).  Group e
  // owns rows [grp_off[e], grp_off[e+1]) of A and C (GRP_M; its 256-row
  // tiles start at tile grp_tiles[e] of a flat tile list) or that k-range of
  // both operands (GRP_K; group e's output at C + e * grp_stride_c).  B of
  // group e (GRP_M) starts at B + e * grp_stride_b.
  const int32_t* grp_off;    // [groups + 1]
  const int32_t* grp_tiles;  // [groups + 1] (GRP_M)
  int groups;
  int64_t grp_stride_b, grp_stride_c;
  // EPI_SWIGLU_BWD with a weighted activation (act_w = w * silu(gate) * up):
  // row_w [M] holds each row's weight w; the output d act_w is scaled by it
  // before the SwiGLU derivative, and row_part [M, N/8] receives, for every
  // 8 columns, sum d act_w * silu(gate) * up (the weight's gradient, in parts).
  const float* row_w;
  float* row_part;
};

enum GroupMode { GRP_NONE = 0, GRP_M = 1, GRP_K = 2 };
// Tiles per band of the GRP_M tile order: one round of 256-row workgroups
// (one per CU).
#ifndef MP_GRP_BAND
#define MP_GRP_BAND 256
#endif
constexpr int GRP_BAND = MP_GRP_BAND;
static_assert(GRP_BAND % 8 == 0, "bands start on the first XCD");

// Workgroup -> output tile.  Workgroups are dealt round-robin to the 8 XCDs;
// renumber so XCD x gets a contiguous range of logical tiles, then walk
// logical tiles in groups of `group_m` tile-rows (column-major inside a group).
__device__ __forceinline__ void map_tile(int wg, int nwg, int tiles_m, int tiles_n, int group_m, int& tm, int& tn) {
  const int per = nwg >> 3, rem = nwg & 7, xcd = wg & 7, idx = wg >> 3;
  const int lid = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + idx;
  const int width = group_m * tiles_n;
  const int group = lid / width;
  const int first_m = group * group_m;
  const int gsz = min(tiles_m - first_m, group_m);
  const int inner = lid - group * width;
  tm = first_m + inner % gsz;
  tn = inner / gsz;
}

// Distance, in k-tiles beyond the direct loads, of the grid-wide warm-up of
// the operands into the last-level cache (0 turns it off).
#ifndef MP_GEMM_WARM
#define MP_GEMM_WARM 2
#endif

template <int BM, int BN, int NW, int WR, bool AK, bool BKC, int EPI, int ACT, int GRP = GRP_NONE>
__global__ __launch_bounds__(64 * NW) void gemm_bf16_kernel(const GemmArgs g0) {
  // WR x (NW / WR) waves; each wave owns (BM / WR) x (BN / (NW / WR)) of the
  // tile.  Eight waves put two on each SIMD, so one wave's MFMAs run while
  // the other waits at the barrier or on its fragment reads.
  constexpr int NT = 64 * NW, WC = NW / WR, WM = BM / WR, WN = BN / WC, TM = WM / 32, TN = WN / 32;
  static_assert(TM >= 1 && TN >= 1 && WM % 32 == 0 && WN % 32 == 0, "wave tile must be whole 32x32 blocks");
  constexpr int A_SLOTS = BM * 8, B_SLOTS = BN * 8;
  __shared__ uint4 lds[2][A_SLOTS + B_SLOTS];
  __shared__ uint32_t warm_sink[64];
  // Grouped problems skip the grid-wide warm-up: their grids are sized for
  // the worst case and most of the workgroups of a group exit at once.
  constexpr int WD = GRP == GRP_NONE ? MP_GEMM_WARM : 0;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WC, wn = wave % WC;
  GemmArgs g = g0;
  int tmi, tni;
  if constexpr (GRP == GRP_M) {
    // Flat list of the groups' tiles (tile-rows of every group back to back,
    // each tile-row tiles_n wide); workgroups past its end exit.  The list is
    // taken in bands of one round of workgroups (GRP_BAND tiles), each band
    // dealt to the XCDs in contiguous runs, so every round works on
    // neighbouring tiles: mostly one group, whose B panels the XCDs then
    // share through the last-level cache.
    const int n_real = g.grp_tiles[g.groups] * g.tiles_n;
    const int wg = blockIdx.x;
    if (wg >= n_real) return;
    const int b0 = wg - wg % GRP_BAND, nb = min(GRP_BAND, n_real - b0), w = wg - b0;
    const int per = nb >> 3, rem = nb & 7, xcd = w & 7, idx = w >> 3;
    const int lid = b0 + (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + idx;
    const int mtg = lid / g.tiles_n;
    tni = lid - mtg * g.tiles_n;
    int e = 0;
    while (e + 1 < g.groups && g.grp_tiles[e + 1] <= mtg) ++e;
    tmi = mtg - g.grp_tiles[e];
    const int64_t lo = g.grp_off[e];
    g.M = g.grp_off[e + 1] - lo;
    g.A = static_cast<const uint16_t*>(g.A) + lo * g.lda;
    g.B = static_cast<const uint16_t*>(g.B) + e * g.grp_stride_b;
    if (g.out_bf16) g.C = static_cast<uint16_t*>(g.C) + lo * g.ldc;
    else g.C = static_cast<float*>(g.C) + lo * g.ldc;
    if (g.zin != nullptr) g.zin = static_cast<const uint16_t*>(g.zin) + lo * g.ldc;
    if (g.row_w != nullptr) {
      g.row_w += lo;
      g.row_part += lo * (g.N / 8);
    }
  } else {
    if constexpr (GRP == GRP_K) {
      const int e = blockIdx.y;
      const int64_t lo = g.grp_off[e];
      g.K = g.grp_off[e + 1] - lo;
      g.k_split = g.K;
      g.A = static_cast<const uint16_t*>(g.A) + lo * g.lda;
      g.B = static_cast<const uint16_t*>(g.B) + lo * g.ldb;
      if (g.out_bf16) g.C = static_cast<uint16_t*>(g.C) + e * g.grp_stride_c;
      else g.C = static_cast<float*>(g.C) + e * g.grp_stride_c;
    }
    map_tile(blockIdx.x, gridDim.x, g.tiles_m, g.tiles_n, g.group_m, tmi, tni);
  }
  const int64_t m0 = static_cast<int64_t>(tmi) * BM, n0 = static_cast<int64_t>(tni) * BN;
  const int64_t kbeg = static_cast<int64_t>(blockIdx.z) * g.k_split;
  const int64_t kend = min(g.K, kbeg + g.k_split);
  const int nk = kend > kbeg ? static_cast<int>((kend - kbeg + 63) / 64) : 0;
  const uint16_t* A = static_cast<const uint16_t*>(g.A);
  const uint16_t* B = static_cast<const uint16_t*>(g.B);

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  DmaTile<BM, AK, NT> da;
  DmaTile<BN, BKC, NT> db;
  da.init(A, g.lda, m0, g.M, g.K, tid);
  db.init(B, g.ldb, n0, g.N, g.K, tid);
  constexpr int NI = DmaTile<BM, AK, NT>::NI + DmaTile<BN, BKC, NT>::NI;
  // k-tile t of this split starts at kbeg + 64 t; only a ragged last k-tile
  // (K not a multiple of 64) needs the checked issue.
  const bool ragged = (kend - kbeg) % 64 != 0;
  auto fill = [&](uint4* buf, int t) {
    const int64_t k0 = kbeg + 64 * static_cast<int64_t>(t);
    if (ragged && t == nk - 1) {
      da.issue_checked(buf, k0, kend, tid);
      db.issue_checked(buf + A_SLOTS, k0, kend, tid);
    } else {
      da.issue(buf, k0, t < nk);
      db.issue(buf + A_SLOTS, k0, t < nk);
    }
  };
  constexpr int VPR = WN / 8;          // 8-wide vectors per epilogue strip row
  constexpr int NV = 32 * VPR / 64;    // vectors per lane per strip
  static_assert((32 * VPR) % 64 == 0, "strip vectors must cover the wave evenly");
  // Each wave warms its share of k-tile t + WD while the direct loads of
  // k-tile t are in flight.  The prologue warms k-tiles 2 .. 1+WD, ordered so
  // that exactly one warm-up load follows the last direct load, as in every
  // iteration below (whose waits leave that one in flight).
  GridWarm gw;
  if constexpr (WD > 0)
    gw.init(A, g.lda, g.M, g.K, AK, B, g.ldb, g.N, BKC,
            static_cast<int>(blockIdx.x) * NW + __builtin_amdgcn_readfirstlane(wave), static_cast<int>(gridDim.x) * NW,
            lane);
  auto warm = [&](int t) { gw.issue(warm_sink, kbeg + 64 * static_cast<int64_t>(t), t < nk); };
  constexpr int NWU = WD > 0 ? 1 : 0;
  if constexpr (WD > 1) {
#pragma unroll
    for (int t = 2; t < 1 + WD; ++t) warm(t);
  }
  fill(lds[0], 0);
  fill(lds[1], 1);
  if constexpr (WD > 0) warm(1 + WD);
  wait_vmcnt<NI + NWU>();
  __syncthreads();

  // Software pipeline.  k-tiles stream through two LDS buffers by direct
  // loads: k-tile kt+2 is issued into the buffer of k-tile kt as soon as the
  // barrier inside kt's last k-step has retired every read of it, so a load
  // has a whole k-tile of MFMAs to land.  Fragments are double-buffered in
  // registers: while the MFMAs of k-step ks run, the fragments of ks+1 are
  // read.  The barrier sits inside the last k-step, so the first fragments
  // of the next k-tile are read while that step's remaining MFMAs run.  The
  // loop body has no branches (past the end of K the loads write zeros and
  // go unused), so the interleave patterns below apply as written.
  constexpr int NRA = AK ? TM : 2 * TM, NRB = BKC ? TN : 2 * TN, NR = NRA + NRB;
  constexpr int NM = TM * TN, H = TM > 1 ? TM / 2 : 1;
  const int ar0 = wm * WM, br0 = wn * WN;
  uint4 fa[2][TM], fb[2][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) fa[0][i] = lds_frag<AK>(lds[0], ar0 + 32 * i, 0, lane);
#pragma unroll
  for (int j = 0; j < TN; ++j) fb[0][j] = lds_frag<BKC>(lds[0] + A_SLOTS, br0 + 32 * j, 0, lane);

  for (int kt = 0; kt < nk; ++kt) {
    uint4* cur = lds[kt & 1];
    const uint4* ta = cur;
    const uint4* tb = cur + A_SLOTS;
    const uint4* na = lds[(kt & 1) ^ 1];
#pragma unroll
    for (int ks = 0; ks < 3; ++ks) {
      const int c = ks & 1, n = c ^ 1;
#pragma unroll
      for (int i = 0; i < TM; ++i) fa[n][i] = lds_frag<AK>(ta, ar0 + 32 * i, ks + 1, lane);
#pragma unroll
      for (int j = 0; j < TN; ++j) fb[n][j] = lds_frag<BKC>(tb, br0 + 32 * j, ks + 1, lane);
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
    wait_vm_lds_n<NWU>();  // k-tile kt+1 has landed (this wave's share); reads of kt retired
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[0][i] = lds_frag<AK>(na, ar0 + 32 * i, 0, lane);
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[0][j] = lds_frag<BKC>(na + A_SLOTS, br0 + 32 * j, 0, lane);
    fill(cur, kt + 2);
    if constexpr (WD > 0) warm(kt + 2 + WD);
#pragma unroll
    for (int i = H; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = mfma_32x32x16(fa[1][i], fb[1][j], acc[i][j]);
  }
  wait_vm_lds();  // the trailing (all-zero) loads write LDS the epilogue reuses
  __syncthreads();

  // Row statistics of the fp32 logits instead of a store.  Each 32-row strip
  // of the wave's tile goes through the wave-private LDS strip (as in the
  // store epilogue below); there, lanes 2q and 2q+1 own strip row q and fold
  // half of its WN columns each, then combine with one exchange.
  if constexpr (EPI == EPI_LSE) {
    constexpr float kL2e = 1.4426950408889634f;
    constexpr int SP = WN + 4, HC = WN / 2;
    static_assert(HC % 4 == 0, "half a wave column must be whole float4s");
    float* strip = reinterpret_cast<float*>(&lds[0][0]) + wave * 32 * SP;
    const int rr = lane >> 1, hh = lane & 1;
    const int64_t c0 = n0 + wn * WN + hh * HC;  // first column of this lane's half
    const int slot = tni * WC + wn;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) strip[mfma_row(r, lane) * SP + j * 32 + (lane & 31)] = acc[i][j][r];
      __builtin_amdgcn_wave_barrier();
      const int64_t row = m0 + wm * WM + i * 32 + rr;
      const int64_t lab = row < g.M ? static_cast<int64_t>(g.labels[row]) - g.v_start : -1;
      float v[HC];
#pragma unroll
      for (int q = 0; q < HC / 4; ++q) {
        const float4 f = *reinterpret_cast<const float4*>(strip + rr * SP + hh * HC + 4 * q);
        v[4 * q] = f.x; v[4 * q + 1] = f.y; v[4 * q + 2] = f.z; v[4 * q + 3] = f.w;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int c = 0; c < HC; ++c)
        if (c0 + c < g.N) mx = fmaxf(mx, v[c]);
      mx = fmaxf(mx, __shfl_xor(mx, 1, 64));
      float se = 0.0f, tg = 0.0f;
      if (mx != -INFINITY) {
#pragma unroll
        for (int c = 0; c < HC; ++c)
          if (c0 + c < g.N) {
            se += exp2_fast((v[c] - mx) * kL2e);
            if (c0 + c == lab) tg = v[c];
          }
      }
      se += __shfl_xor(se, 1, 64);
      tg += __shfl_xor(tg, 1, 64);
      if (hh == 0 && row < g.M) {
        float* pp = g.lse_part + (row * g.lse_slots + slot) * 3;
        pp[0] = mx;
        pp[1] = se;
        pp[2] = tg;
      }
    }
    return;
  }

  // Bias: lane l holds column (l % 32) of every 32x32 accumulator tile, so
  // the bias is added in registers before the epilogue (one value per tile
  // column), keeping the unrolled store loop below free of it.
  if constexpr (EPI == EPI_STORE) {
    if (g.bias != nullptr) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int64_t n = n0 + wn * WN + j * 32 + (lane & 31);
        const float b =
            n < g.N ? __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(g.bias)[n]) << 16) : 0.0f;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] += b;
      }
    }
  }

  // Epilogue, staged through LDS one 32-row strip of the wave's tile at a
  // time: the accumulators (register r of lane l = row mfma_row(r, l),
  // column l % 32) are written to a wave-private LDS strip, then read back
  // row-major so each lane finishes 8 consecutive outputs of one row with
  // 16-byte loads (saved pre-activation) and 16/32-byte stores.  The
  // strip is private to the wave and a wave's LDS operations complete in
  // order, so no barrier is needed between writing and reading it (the one
  // above retires every wave's reads of the operand tiles); the loop over a
  // lane's NV vectors is unrolled so their global loads issue together.
  constexpr int SP = WN + 4;  // padded strip row (floats)
  float* strip = reinterpret_cast<float*>(&lds[0][0]) + wave * 32 * SP;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) strip[mfma_row(r, lane) * SP + j * 32 + (lane & 31)] = acc[i][j][r];
    __builtin_amdgcn_wave_barrier();
    // The saved pre-activation of the activation-gradient epilogue, likewise
    // loaded for the whole strip before any of it is used.
    // EPI_SWIGLU_BWD: the gate pre-activation sits at the output's place and
    // the up pre-activation N columns further on (rows of ldc values).
    uint4 zraw[NV], uraw[EPI == EPI_SWIGLU_BWD ? NV : 1];
    if constexpr (EPI == EPI_DACT || EPI == EPI_SWIGLU_BWD) {
#pragma unroll
      for (int it = 0; it < NV; ++it) {
        const int v = lane + 64 * it;
        const int row = v / VPR, c8 = (v - row * VPR) * 8;
        const int64_t m = m0 + wm * WM + i * 32 + row, n = n0 + wn * WN + c8;
        const int64_t o = (m < g.M && n < g.N) ? m * g.ldc + n : 0;
        zraw[it] = load_stream16(static_cast<const uint16_t*>(g.zin) + o);
        if constexpr (EPI == EPI_SWIGLU_BWD) uraw[it] = load_stream16(static_cast<const uint16_t*>(g.zin) + o + g.N);
      }
    }
#pragma unroll
    for (int it = 0; it < NV; ++it) {
      const int v = lane + 64 * it;
      const int row = v / VPR, c8 = (v - row * VPR) * 8;
      const int64_t m = m0 + wm * WM + i * 32 + row;
      const int64_t n = n0 + wn * WN + c8;
      float val[8];
      const float4 lo = *reinterpret_cast<const float4*>(strip + row * SP + c8);
      const float4 hi = *reinterpret_cast<const float4*>(strip + row * SP + c8 + 4);
      val[0] = lo.x; val[1] = lo.y; val[2] = lo.z; val[3] = lo.w;
      val[4] = hi.x; val[5] = hi.y; val[6] = hi.z; val[7] = hi.w;
      if constexpr (EPI == EPI_DACT) {
        float z[8];
        unpack8(zraw[it], z);
#pragma unroll
        for (int e = 0; e < 8; ++e) val[e] *= act_grad_fast(z[e], ACT);
      }
      if (m >= g.M || n >= g.N) continue;
      if constexpr (EPI == EPI_SWIGLU_BWD) {
        // act = silu(gate) * up with silu(x) = x s, s = 1 / (1 + e^-x):
        // d gate = d act * up * s (1 + gate (1 - s)), d up = d act * gate * s.
        // With row weights, val is d act_w: its dot with the unweighted
        // activation is the weight's gradient, and d act = w * d act_w.
        float z[8], u[8], dgv[8], duv[8];
        unpack8(zraw[it], z);
        unpack8(uraw[it], u);
        const bool wt = g.row_w != nullptr;
        const float wr = wt ? g.row_w[m] : 1.0f;
        float part = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * z[e]));
          part += val[e] * (z[e] * sg * u[e]);
          const float da = val[e] * wr;
          dgv[e] = da * u[e] * sg * (1.0f + z[e] * (1.0f - sg));
          duv[e] = da * z[e] * sg;
        }
        if (wt) g.row_part[m * (g.N / 8) + n / 8] = part;
        uint16_t* c = static_cast<uint16_t*>(g.C) + m * g.ldc + n;
        *reinterpret_cast<uint4*>(c) = pack8(dgv);
        *reinterpret_cast<uint4*>(c + g.N) = pack8(duv);
        continue;
      }
      if constexpr (EPI == EPI_SPLITK) {
        float* dst = g.partial + (static_cast<int64_t>(blockIdx.z) * g.M + m) * g.N + n;
        reinterpret_cast<float4*>(dst)[0] = lo;
        reinterpret_cast<float4*>(dst)[1] = hi;
        continue;
      }
      const int64_t o = m * g.ldc + n;
      if constexpr (EPI == EPI_STORE) {
        if (g.zsave != nullptr) {
          // The pre-activation is read back only by the backward pass.
          if (g.out_bf16) {
            store_stream16(static_cast<uint16_t*>(g.zsave) + o, pack8(val));
          } else {
            reinterpret_cast<float4*>(static_cast<float*>(g.zsave) + o)[0] = make_float4(val[0], val[1], val[2], val[3]);
            reinterpret_cast<float4*>(static_cast<float*>(g.zsave) + o)[1] = make_float4(val[4], val[5], val[6], val[7]);
          }
        }
        if constexpr (ACT != MP_ACT_NONE) {
#pragma unroll
          for (int e = 0; e < 8; ++e) val[e] = act_fwd_fast(val[e], ACT);
        }
      }
      if (g.out_bf16) {
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(g.C) + o) = pack8(val);
      } else {
        reinterpret_cast<float4*>(static_cast<float*>(g.C) + o)[0] = make_float4(val[0], val[1], val[2], val[3]);
        reinterpret_cast<float4*>(static_cast<float*>(g.C) + o)[1] = make_float4(val[4], val[5], val[6], val[7]);
      }
    }
  }
}

// out[m, n] = sum_z partial[z, m, n] in z order; fp32 or bf16 output.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ partial, int splits, int64_t M,
                                                            int64_t N, int64_t ldc, int out_bf16, void* __restrict__ C) {
  const int64_t q = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;  // index of 4 outputs
  const int64_t nq = N >> 2;
  if (q >= M * nq) return;
  const int64_t m = q / nq, n = (q - m * nq) * 4;
  float4 s = load_nt4(partial + m * N + n);
  for (int z = 1; z < splits; ++z) {
    const float4 v = load_nt4(partial + (static_cast<int64_t>(z) * M + m) * N + n);
    s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
  }
  if (out_bf16) {
    uint2 o;
    o.x = pack_bf16x2(s.x, s.y);
    o.y = pack_bf16x2(s.z, s.w);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(C) + m * ldc + n) = o;
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(C) + m * ldc + n) = s;
  }
}

// ---------------------------------------------------------- fp32 SIMT path
// 64x64 output tile, 256 threads x (4x4) outputs, 16-deep k-tiles in LDS.
template <bool AK, bool BKC, int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const GemmArgs g) {
  __shared__ float As[16][68], Bs[16][68];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * 64, n0 = static_cast<int64_t>(blockIdx.x) * 64;
  const int64_t kbeg = static_cast<int64_t>(blockIdx.z) * g.k_split;
  const int64_t kend = min(g.K, kbeg + g.k_split);
  const float* A = static_cast<const float*>(g.A);
  const float* B = static_cast<const float*>(g.B);
  float acc[4][4] = {};
  for (int64_t k0 = kbeg; k0 < kend; k0 += 16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 256 * i;
      const int r = AK ? idx >> 4 : idx & 63, c = AK ? idx & 15 : idx >> 6;
      const int64_t gm = m0 + r, gk = k0 + c;
      As[c][r] = (gm < g.M && gk < kend) ? (AK ? A[gm * g.lda + gk] : A[gk * g.lda + gm]) : 0.0f;
      const int rb = BKC ? idx >> 4 : idx & 63, cb = BKC ? idx & 15 : idx >> 6;
      const int64_t gn = n0 + rb, gkb = k0 + cb;
      Bs[cb][rb] = (gn < g.N && gkb < kend) ? (BKC ? B[gn * g.ldb + gkb] : B[gkb * g.ldb + gn]) : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = As[kk][ty * 4 + i];
        b[i] = Bs[kk][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + ty * 4 + i;
    if (m >= g.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n0 + tx * 4 + j;
      if (n >= g.N) continue;
      float v = acc[i][j];
      if constexpr (EPI == EPI_SPLITK) {
        g.partial[(static_cast<int64_t>(blockIdx.z) * g.M + m) * g.N + n] = v;
      } else {
        const int64_t o = m * g.ldc + n;
        if constexpr (EPI == EPI_DACT) {
          v *= act_grad(static_cast<const float*>(g.zin)[o], g.act);
        } else {
          if (g.bias != nullptr) v += static_cast<const float*>(g.bias)[n];
          if (g.zsave != nullptr) static_cast<float*>(g.zsave)[o] = v;
          v = act_fwd(v, g.act);
        }
        static_cast<float*>(g.C)[o] = v;
      }
    }
  }
}

// dZ = dY * act'(Z), element-wise over 16-byte vectors.
template <bool BF16>
__global__ __launch_bounds__(256) void dact_kernel(int64_t nvec, const void* __restrict__ dy, const void* __restrict__ z,
                                                   int act, void* __restrict__ dz) {
  using V = Vec16<BF16>;
  constexpr int E = V::N;
  const int64_t v = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (v >= nvec) return;
  float a[E], b[E];
  V::load(dy, v * E, a);
  V::load(z, v * E, b);
#pragma unroll
  for (int i = 0; i < E; ++i) a[i] *= BF16 ? act_grad_fast(b[i], act) : act_grad(b[i], act);
  V::store(dz, v * E, a);
}

// --------------------------------------------------------------- planning


struct Plan {
  int bm, bn, splits;
  int64_t k_split;
};

// Chooses the tile shape and the K split by estimated time (microseconds):
// rounds of workgroups x (k-steps x the time of one 64-deep k-step + the
// fixed prologue/epilogue time of a tile), plus, for a split, writing and
// re-reading the fp32 partials.  The per-tile constants were measured on
// MI355X with random bf16 operands (the layouts run within a few percent of
// each other).  128x128 tiles fit two workgroups per CU; a last round in
// which no CU holds two of them runs at ~0.6 of a full round.
// MP_GEMM_PLAN="bm,bn,splits" forces a plan (for tuning sweeps).
static Plan plan_bf16(int64_t M, int64_t N, int64_t K, bool allow_split, Layout lay) {
  (void)lay;
  struct Cand { int bm, bn, slots; double t_step_us, t_fixed_us; };
  const Cand cands[] = {{256, 256, 256, 1.57, 13.0}, {256, 192, 256, 1.41, 11.2}, {256, 128, 256, 1.14, 7.3},
                        {128, 128, 512, 0.98, 8.3}};
  const int64_t kt_total = ceil_div(K > 0 ? K : 1, 64);
  if (const char* env = getenv("MP_GEMM_PLAN")) {
    int bm = 0, bn = 0, sp = 1;
    if (sscanf(env, "%d,%d,%d", &bm, &bn, &sp) == 3 && sp >= 1 && (allow_split || sp == 1) &&
        ((bm == 256 && (bn == 256 || bn == 192 || bn == 128)) || (bm == 128 && (bn == 128 || bn == 192)))) {
      const int64_t kt = ceil_div(kt_total, sp);
      return Plan{bm, bn, static_cast<int>(ceil_div(kt_total, kt)), kt * 64};
    }
  }
  Plan best{256, 256, 1, kt_total * 64};
  double best_cost = 1e300;
  for (const Cand& c : cands) {
    const int64_t tiles = ceil_div(M, c.bm) * ceil_div(N, c.bn);
    const int max_split = allow_split ? 16 : 1;
    for (int s = 1; s <= max_split; ++s) {
      const int64_t kt = ceil_div(kt_total, s);
      if (s > 1 && kt < 4) break;
      if (ceil_div(kt_total, kt) != s) continue;  // every split non-empty
      const int64_t blocks = tiles * s;
      const int64_t full = blocks / c.slots, rem = blocks - full * c.slots;
      const double part = rem == 0 ? 0.0 : (c.slots > 256 && rem <= 256 ? 0.6 : 1.0);
      double cost = (static_cast<double>(full) + part) * (kt * c.t_step_us + c.t_fixed_us);
      if (s > 1) cost += 3.0 + (s + 1) * 4.0 * M * N / 6.5e6;
      if (cost < best_cost) {
        best_cost = cost;
        best = Plan{c.bm, c.bn, s, kt * 64};
      }
    }
  }
  return best;
}

// 256-row tiles run 8 waves (two per SIMD); 128x128 tiles 4 waves (two
// workgroups per CU).
template <int BM, int BN, bool AK, bool BKC, int EPI, int ACT>
static void launch_bf16_tile(const GemmArgs& g, int splits, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(g.tiles_m * g.tiles_n), 1, static_cast<unsigned>(splits));
  if constexpr (BM == 128) gemm_bf16_kernel<BM, BN, 4, 2, AK, BKC, EPI, ACT><<<grid, 256, 0, s>>>(g);
  else if constexpr (BN == 256) gemm_bf16_kernel<BM, BN, 8, 2, AK, BKC, EPI, ACT><<<grid, 512, 0, s>>>(g);
  else gemm_bf16_kernel<BM, BN, 8, 4, AK, BKC, EPI, ACT><<<grid, 512, 0, s>>>(g);
}

template <bool AK, bool BKC, int EPI, int ACT>
static void launch_bf16_layout(const GemmArgs& g, const Plan& p, hipStream_t s) {
  if (p.bm == 256 && p.bn == 256) launch_bf16_tile<256, 256, AK, BKC, EPI, ACT>(g, p.splits, s);
  else if (p.bm == 256 && p.bn == 192) launch_bf16_tile<256, 192, AK, BKC, EPI, ACT>(g, p.splits, s);
  else if (p.bm == 256 && p.bn == 128) launch_bf16_tile<256, 128, AK, BKC, EPI, ACT>(g, p.splits, s);
  else if (p.bn == 192) launch_bf16_tile<128, 192, AK, BKC, EPI, ACT>(g, p.splits, s);
  else launch_bf16_tile<128, 128, AK, BKC, EPI, ACT>(g, p.splits, s);
}

// Instantiated combinations: the forward (NT) with each activation, the
// input-gradient (NN) and weight-gradient (TN, plain or split-K) GEMMs.
static void launch_bf16(Layout lay, int epi, int act, const GemmArgs& g, const Plan& p, hipStream_t s) {
  if (lay == NT && epi == EPI_LSE) {
    launch_bf16_layout<true, true, EPI_LSE, MP_ACT_NONE>(g, p, s);
  } else if (lay == NT) {
    if (act == MP_ACT_GELU_ERF) launch_bf16_layout<true, true, EPI_STORE, MP_ACT_GELU_ERF>(g, p, s);
    else if (act == MP_ACT_GELU_TANH) launch_bf16_layout<true, true, EPI_STORE, MP_ACT_GELU_TANH>(g, p, s);
    else launch_bf16_layout<true, true, EPI_STORE, MP_ACT_NONE>(g, p, s);
  } else if (lay == NN) {
    if (epi == EPI_DACT && act == MP_ACT_GELU_ERF) launch_bf16_layout<true, false, EPI_DACT, MP_ACT_GELU_ERF>(g, p, s);
    else if (epi == EPI_DACT && act == MP_ACT_GELU_TANH)
      launch_bf16_layout<true, false, EPI_DACT, MP_ACT_GELU_TANH>(g, p, s);
    else launch_bf16_layout<true, false, EPI_STORE, MP_ACT_NONE>(g, p, s);
  } else if (epi == EPI_SPLITK) {
    launch_bf16_layout<false, false, EPI_SPLITK, MP_ACT_NONE>(g, p, s);
  } else {
    launch_bf16_layout<false, false, EPI_STORE, MP_ACT_NONE>(g, p, s);
  }
}

template <int EPI>
static void launch_f32_epi(Layout lay, const GemmArgs& g, int splits, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(ceil_div(g.N, 64)), static_cast<unsigned>(ceil_div(g.M, 64)),
                  static_cast<unsigned>(splits));
  if (lay == NT) gemm_f32_kernel<true, true, EPI><<<grid, 256, 0, s>>>(g);
  else if (lay == NN) gemm_f32_kernel<true, false, EPI><<<grid, 256, 0, s>>>(g);
  else gemm_f32_kernel<false, false, EPI><<<grid, 256, 0, s>>>(g);
}

// Split-K partial bytes needed for an fp32-output GEMM of this shape.
static size_t splitk_bytes(mp_dtype dt, int64_t M, int64_t N, int64_t K) {
  if (dt != MP_BF16) return 0;
  const Plan p = plan_bf16(M, N, K, true, TN);
  return p.splits > 1 ? align_up(static_cast<size_t>(p.splits) * M * N * sizeof(float), 256) : 0;
}

// C = A * B^T in the given layout.  `allow_split` (fp32-output GEMMs only)
// lets the planner split K, using `ws` for the partials.
int gemm(mp_dtype dt, Layout lay, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
         int64_t ldb, void* C, int64_t ldc, bool out_bf16, const void* bias, int act, void* zsave, bool allow_split,
         void* ws, size_t ws_bytes, hipStream_t s, int epi, const void* zin) {
  if (M == 0 || N == 0) return MP_OK;
  GemmArgs g{};
  g.M = M; g.N = N; g.K = K; g.A = A; g.lda = lda; g.B = B; g.ldb = ldb; g.C = C; g.ldc = ldc;
  g.bias = bias; g.zsave = zsave; g.zin = zin; g.act = act; g.out_bf16 = out_bf16 ? 1 : 0;
  if (dt == MP_BF16) {
    // Direct loads address an MN-contiguous operand with 32-bit offsets from
    // the tile's first column across all of K.
    const int64_t lim = 0x7fffffffLL;
    if ((lay == TN && (K + 64) * lda * 2 > lim) || (lay != NT && (K + 64) * ldb * 2 > lim))
      return fail(MP_ERR_SHAPE, "gemm: an MN-contiguous operand spans more than 2 GiB");
    const Plan p = plan_bf16(M, N, K, allow_split && epi == EPI_STORE && bias == nullptr && act == MP_ACT_NONE &&
                                          zsave == nullptr && lay == TN, lay);
    g.tiles_m = static_cast<int>(ceil_div(M, p.bm));
    g.tiles_n = static_cast<int>(ceil_div(N, p.bn));
    g.group_m = 8;
    g.k_split = p.k_split;
    if (p.splits > 1) {
      const size_t need = static_cast<size_t>(p.splits) * M * N * sizeof(float);
      if (ws == nullptr || ws_bytes < need)
        return fail(MP_ERR_WORKSPACE, "gemm: split-K needs %zu workspace bytes, got %zu", need, ws_bytes);
      if (lay != TN) return fail(MP_ERR_UNSUPPORTED, "gemm: split-K is built for the weight-gradient layout only");
      g.partial = static_cast<float*>(ws);
      launch_bf16(lay, EPI_SPLITK, MP_ACT_NONE, g, p, s);
      const int64_t nq = M * (N / 4);
      splitk_reduce_kernel<<<static_cast<unsigned>(ceil_div(nq, 256)), 256, 0, s>>>(g.partial, p.splits, M, N, ldc,
                                                                                     g.out_bf16, C);
    } else {
      const bool dact_nn = epi == EPI_DACT && lay == NN && act != MP_ACT_NONE && zin != nullptr;
      if (!dact_nn && (epi != EPI_STORE || (lay != NT && act != MP_ACT_NONE)))
        return fail(MP_ERR_UNSUPPORTED, "gemm: epilogue not built for this layout");
      launch_bf16(lay, epi, act, g, p, s);
    }
  } else {
    g.k_split = K > 0 ? K : 16;
    if (epi == EPI_DACT) launch_f32_epi<EPI_DACT>(lay, g, 1, s);
    else launch_f32_epi<EPI_STORE>(lay, g, 1, s);
  }
  return check_launch("gemm");
}

size_t gemm_splitk_workspace(mp_dtype dt, int64_t M, int64_t N, int64_t K) { return splitk_bytes(dt, M, N, K); }

// Wave columns per tile of each tile shape (see launch_bf16_tile).
static int wave_cols(const Plan& p) { return p.bm == 128 ? 2 : (p.bn == 256 ? 4 : 2); }

int gemm_lse_slots(int64_t T, int64_t V, int64_t K) {
  const Plan p = plan_bf16(T, V, K, false, NT);
  return static_cast<int>(ceil_div(V, p.bn)) * wave_cols(p);
}

int gemm_logits_lse(int64_t T, int64_t V, int64_t K, const void* H, const void* E, const int32_t* labels,
                    int64_t v_start, float* part, hipStream_t s) {
  if (T == 0) return MP_OK;
  GemmArgs g{};
  g.M = T; g.N = V; g.K = K; g.A = H; g.lda = K; g.B = E; g.ldb = K; g.ldc = V;
  g.out_bf16 = 1;
  g.labels = labels; g.v_start = v_start; g.lse_part = part;
  const Plan p = plan_bf16(T, V, K, false, NT);
  g.tiles_m = static_cast<int>(ceil_div(T, p.bm));
  g.tiles_n = static_cast<int>(ceil_div(V, p.bn));
  g.group_m = 8;
  g.k_split = p.k_split;
  g.lse_slots = g.tiles_n * wave_cols(p);
  launch_bf16(NT, EPI_LSE, MP_ACT_NONE, g, p, s);
  return check_launch("gemm_logits_lse");
}

int gemm_grouped_m(int epi, int groups, const int32_t* off, const int32_t* tiles, int64_t max_mtiles, int64_t N,
                   int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb, int64_t stride_b, void* C,
                   int64_t ldc, const void* zin, hipStream_t s, const float* row_w, float* row_part) {
  if (groups <= 0 || max_mtiles <= 0 || N == 0) return MP_OK;
  if ((K + 64) * ldb * 2 > 0x7fffffffLL)
    return fail(MP_ERR_SHAPE, "gemm_grouped_m: an MN-contiguous operand spans more than 2 GiB");
  GemmArgs g{};
  g.N = N; g.K = K; g.A = A; g.lda = lda; g.B = B; g.ldb = ldb; g.C = C; g.ldc = ldc; g.zin = zin;
  g.out_bf16 = 1;
  g.k_split = ceil_div(K > 0 ? K : 1, 64) * 64;
  g.tiles_n = static_cast<int>(ceil_div(N, 256));
  g.group_m = 1;
  g.grp_off = off;
  g.grp_tiles = tiles;
  g.groups = groups;
  g.grp_stride_b = stride_b;
  g.row_w = row_w;
  g.row_part = row_part;
  const dim3 grid(static_cast<unsigned>(max_mtiles * g.tiles_n));
  if (epi == EPI_SWIGLU_BWD)
    gemm_bf16_kernel<256, 256, 8, 2, true, false, EPI_SWIGLU_BWD, MP_ACT_NONE, GRP_M><<<grid, 512, 0, s>>>(g);
  else
    gemm_bf16_kernel<256, 256, 8, 2, true, false, EPI_STORE, MP_ACT_NONE, GRP_M><<<grid, 512, 0, s>>>(g);
  return check_launch("gemm_grouped_m");
}

int gemm_grouped_k(int groups, const int32_t* off, int64_t max_k, int64_t M, int64_t N, const void* A, int64_t lda,
                   const void* B, int64_t ldb, float* C, int64_t ldc, int64_t stride_c, hipStream_t s) {
  if (groups <= 0 || M == 0 || N == 0) return MP_OK;
  if ((max_k + 64) * (lda > ldb ? lda : ldb) * 2 > 0x7fffffffLL)
    return fail(MP_ERR_SHAPE, "gemm_grouped_k: an MN-contiguous operand spans more than 2 GiB");
  GemmArgs g{};
  g.M = M; g.N = N; g.A = A; g.lda = lda; g.B = B; g.ldb = ldb; g.C = C; g.ldc = ldc;
  g.out_bf16 = 0;
  g.tiles_m = static_cast<int>(ceil_div(M, 256));
  g.tiles_n = static_cast<int>(ceil_div(N, 256));
  g.group_m = 8;
  g.grp_off = off;
  g.groups = groups;
  g.grp_stride_c = stride_c;
  const dim3 grid(static_cast<unsigned>(g.tiles_m * g.tiles_n), static_cast<unsigned>(groups));
  gemm_bf16_kernel<256, 256, 8, 2, false, false, EPI_STORE, MP_ACT_NONE, GRP_K><<<grid, 512, 0, s>>>(g);
  return check_launch("gemm_grouped_k");
}

static int validate_mat(mp_dtype dt, int64_t contiguous, const char* fn, const char* what) {
  MP_REQUIRE(contiguous % vec_elems(dt) == 0, MP_ERR_SHAPE, "%s: %s=%lld must be a multiple of %lld", fn, what,
             (long long)contiguous, (long long)vec_elems(dt));
  return MP_OK;
}

}  // namespace mp

using namespace mp;

extern "C" int mp_column_linear_gelu(mp_dtype in_dtype, mp_dtype out_dtype, int64_t T, int64_t K, int64_t Fi,
                                     const void* X, const void* A_i, const void* a_i, int act, void* Y_i,
                                     void* Z_save, hipStream_t s) {
  static const char* fn = "mp_column_linear_gelu";
  MP_REQUIRE(dtype_ok(in_dtype) && dtype_ok(out_dtype), MP_ERR_DTYPE, "%s: bad dtype", fn);
  MP_REQUIRE(in_dtype == MP_BF16 || out_dtype == MP_F32, MP_ERR_DTYPE, "%s: fp32 input needs fp32 output", fn);
  MP_REQUIRE(act_ok(act), MP_ERR_ARG, "%s: bad activation %d", fn, act);
  MP_REQUIRE(T >= 0 && K > 0 && Fi > 0, MP_ERR_SHAPE, "%s: bad shape", fn);
  if (int rc = validate_mat(in_dtype, K, fn, "K")) return rc;
  if (int rc = validate_mat(out_dtype, Fi, fn, "Fi")) return rc;
  if (int rc = validate_mat(in_dtype, Fi, fn, "Fi")) return rc;
  MP_REQUIRE_PTR(X);
  MP_REQUIRE_PTR(A_i);
  MP_REQUIRE_PTR(Y_i);
  MP_REQUIRE_ALIGN(X);
  MP_REQUIRE_ALIGN(A_i);
  MP_REQUIRE_ALIGN(Y_i);
  MP_REQUIRE_OPT_ALIGN(a_i);
  MP_REQUIRE_OPT_ALIGN(Z_save);
  return gemm(in_dtype, NT, T, Fi, K, X, K, A_i, K, Y_i, Fi, out_dtype == MP_BF16, a_i, act, Z_save, false, nullptr, 0,
              s);
}

extern "C" size_t mp_column_linear_gelu_bwd_workspace(mp_dtype dtype, int64_t T, int64_t K, int64_t Fi) {
  if (!dtype_ok(dtype) || T < 0 || K <= 0 || Fi <= 0) return 0;
  const size_t dz = align_up(static_cast<size_t>(T * Fi) * dtype_size(dtype), 256);
  const size_t sk = gemm_splitk_workspace(dtype, Fi, K, T);
  const size_t cs = colsum_workspace(T, Fi);
  return dz + (sk > cs ? sk : cs);
}

extern "C" int mp_column_linear_gelu_bwd(mp_dtype dtype, int64_t T, int64_t K, int64_t Fi, const void* X,
                                         const void* A_i, const void* Z_save, const void* dY_i, int act,
                                         void* dX_partial, float* dA_i, float* da_i, void* ws, size_t ws_bytes,
                                         hipStream_t s) {
  static const char* fn = "mp_column_linear_gelu_bwd";
  MP_REQUIRE(dtype_ok(dtype), MP_ERR_DTYPE, "%s: bad dtype", fn);
  MP_REQUIRE(act_ok(act), MP_ERR_ARG, "%s: bad activation %d", fn, act);
  MP_REQUIRE(T >= 0 && K > 0 && Fi > 0, MP_ERR_SHAPE, "%s: bad shape", fn);
  if (int rc = validate_mat(dtype, K, fn, "K")) return rc;
  if (int rc = validate_mat(dtype, Fi, fn, "Fi")) return rc;
  MP_REQUIRE_PTR(X);
  MP_REQUIRE_PTR(A_i);
  MP_REQUIRE_PTR(dY_i);
  MP_REQUIRE_PTR(dX_partial);
  MP_REQUIRE_PTR(dA_i);
  MP_REQUIRE(act == MP_ACT_NONE || Z_save != nullptr, MP_ERR_NULL, "%s: Z_save is NULL", fn);
  MP_REQUIRE_ALIGN(X);
  MP_REQUIRE_ALIGN(A_i);
  MP_REQUIRE_ALIGN(dY_i);
  MP_REQUIRE_ALIGN(dX_partial);
  MP_REQUIRE_ALIGN(dA_i);
  MP_REQUIRE_OPT_ALIGN(Z_save);
  const size_t need = mp_column_linear_gelu_bwd_workspace(dtype, T, K, Fi);
  MP_REQUIRE(ws != nullptr && ws_bytes >= need, MP_ERR_WORKSPACE, "%s: workspace needs %zu bytes", fn, need);
  MP_REQUIRE_ALIGN(ws);
  const size_t dz_bytes = align_up(static_cast<size_t>(T * Fi) * dtype_size(dtype), 256);
  void* dz = ws;
  void* ws2 = static_cast<char*>(ws) + dz_bytes;
  const void* dZ = dY_i;
  if (act != MP_ACT_NONE && T > 0) {
    const int64_t nvec = T * Fi / vec_elems(dtype);
    if (dtype == MP_BF16)
      dact_kernel<true><<<static_cast<unsigned>(ceil_div(nvec, 256)), 256, 0, s>>>(nvec, dY_i, Z_save, act, dz);
    else
      dact_kernel<false><<<static_cast<unsigned>(ceil_div(nvec, 256)), 256, 0, s>>>(nvec, dY_i, Z_save, act, dz);
    dZ = dz;
  }
  // dX_partial[T,K] = dZ[T,Fi] * A_i[Fi,K]
  if (int rc = gemm(dtype, NN, T, K, Fi, dZ, Fi, A_i, K, dX_partial, K, dtype == MP_BF16, nullptr, MP_ACT_NONE,
                    nullptr, false, nullptr, 0, s))
    return rc;
  // dA_i[Fi,K] = dZ^T * X  (reduction over T), fp32
  if (int rc = gemm(dtype, TN, Fi, K, T, dZ, Fi, X, K, dA_i, K, false, nullptr, MP_ACT_NONE, nullptr, true, ws2,
                    ws_bytes - dz_bytes, s))
    return rc;
  if (da_i != nullptr) return colsum(dtype, T, Fi, dZ, da_i, ws2, s);
  return MP_OK;
}

extern "C" int mp_row_linear_partial(mp_dtype dtype, int64_t T, int64_t Fi, int64_t K, const void* Y_i,
                                     const void* B_i, void* P_i, hipStream_t s) {
  static const char* fn = "mp_row_linear_partial";
  MP_REQUIRE(dtype_ok(dtype), MP_ERR_DTYPE, "%s: bad dtype", fn);
  MP_REQUIRE(T >= 0 && K > 0 && Fi > 0, MP_ERR_SHAPE, "%s: bad shape", fn);
  if (int rc = validate_mat(dtype, K, fn, "K")) return rc;
  if (int rc = validate_mat(dtype, Fi, fn, "Fi")) return rc;
  MP_REQUIRE_PTR(Y_i);
  MP_REQUIRE_PTR(B_i);
  MP_REQUIRE_PTR(P_i);
  MP_REQUIRE_ALIGN(Y_i);
  MP_REQUIRE_ALIGN(B_i);
  MP_REQUIRE_ALIGN(P_i);
  return gemm(dtype, NT, T, K, Fi, Y_i, Fi, B_i, Fi, P_i, K, dtype == MP_BF16, nullptr, MP_ACT_NONE, nullptr, false,
              nullptr, 0, s);
}

extern "C" size_t mp_row_linear_partial_bwd_workspace(mp_dtype dtype, int64_t T, int64_t Fi, int64_t K) {
  if (!dtype_ok(dtype) || T < 0 || K <= 0 || Fi <= 0) return 0;
  return gemm_splitk_workspace(dtype, K, Fi, T);
}

// Backward of the row-parallel partial; with act != NONE the input gradient
// leaves the GEMM already multiplied by the activation gradient at Z_save.
static int row_linear_bwd(const char* fn, mp_dtype dtype, int64_t T, int64_t Fi, int64_t K, const void* Y_i,
                          const void* B_i, const void* dOut, const void* Z_save, int act, void* dY_i, float* dB_i,
                          void* ws, size_t ws_bytes, hipStream_t s) {
  MP_REQUIRE(dtype_ok(dtype), MP_ERR_DTYPE, "%s: bad dtype", fn);
  MP_REQUIRE(T >= 0 && K > 0 && Fi > 0, MP_ERR_SHAPE, "%s: bad shape", fn);
  if (int rc = validate_mat(dtype, K, fn, "K")) return rc;
  if (int rc = validate_mat(dtype, Fi, fn, "Fi")) return rc;
  MP_REQUIRE_PTR(Y_i);
  MP_REQUIRE_PTR(B_i);
  MP_REQUIRE_PTR(dOut);
  MP_REQUIRE_PTR(dY_i);
  MP_REQUIRE_PTR(dB_i);
  MP_REQUIRE_ALIGN(Y_i);
  MP_REQUIRE_ALIGN(B_i);
  MP_REQUIRE_ALIGN(dOut);
  MP_REQUIRE_ALIGN(dY_i);
  MP_REQUIRE_ALIGN(dB_i);
  const size_t need = mp_row_linear_partial_bwd_workspace(dtype, T, Fi, K);
  MP_REQUIRE(need == 0 || (ws != nullptr && ws_bytes >= need), MP_ERR_WORKSPACE, "%s: workspace needs %zu bytes", fn,
             need);
  MP_REQUIRE_OPT_ALIGN(ws);
  // dY_i[T,Fi] = dOut[T,K] * B_i[K,Fi]  (times act'(Z_save) in the epilogue)
  if (int rc = gemm(dtype, NN, T, Fi, K, dOut, K, B_i, Fi, dY_i, Fi, dtype == MP_BF16, nullptr, act, nullptr, false,
                    nullptr, 0, s, act != MP_ACT_NONE ? EPI_DACT : EPI_STORE, Z_save))
    return rc;
  // dB_i[K,Fi] = dOut^T * Y_i (reduction over T), fp32
  return gemm(dtype, TN, K, Fi, T, dOut, K, Y_i, Fi, dB_i, Fi, false, nullptr, MP_ACT_NONE, nullptr, true, ws, ws_bytes,
              s);
}

extern "C" int mp_row_linear_partial_bwd(mp_dtype dtype, int64_t T, int64_t Fi, int64_t K, const void* Y_i,
                                         const void* B_i, const void* dOut, void* dY_i, float* dB_i, void* ws,
                                         size_t ws_bytes, hipStream_t s) {
  return row_linear_bwd("mp_row_linear_partial_bwd", dtype, T, Fi, K, Y_i, B_i, dOut, nullptr, MP_ACT_NONE, dY_i,
                        dB_i, ws, ws_bytes, s);
}

extern "C" int mp_row_linear_partial_bwd_dact(mp_dtype dtype, int64_t T, int64_t Fi, int64_t K, const void* Y_i,
                                              const void* B_i, const void* dOut, const void* Z_save, int act,
                                              void* dZ_i, float* dB_i, void* ws, size_t ws_bytes, hipStream_t s) {
  static const char* fn = "mp_row_linear_partial_bwd_dact";
  MP_REQUIRE(act_ok(act) && act != MP_ACT_NONE, MP_ERR_ARG, "%s: bad activation %d", fn, act);
  MP_REQUIRE_PTR(Z_save);
  MP_REQUIRE_ALIGN(Z_save);
  return row_linear_bwd(fn, dtype, T, Fi, K, Y_i, B_i, dOut, Z_save, act, dZ_i, dB_i, ws, ws_bytes, s);
}

// ------------------------------------------------ no-allocation variant
// Scratch of mp_row_linear_partial_bwd_static: a file-scope device array, so
// the call needs no caller workspace and allocates nothing.  The runtime
// places one copy on every GPU that loads this code object and keeps it
// until the process ends.  In host code `scratch` names a host-side stand-in:
// its device address comes from hipGetSymbolAddress, once per device, with
// that device current, and only that address is ever passed to a kernel.
namespace mp {

constexpr size_t kStaticScratchBytes = static_cast<size_t>(64) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mutex;
static void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the device that runs stream `s`.
static int static_scratch(hipStream_t s, void** out, const char* fn) {
  int dev = 0;
  hipError_t e = s == nullptr ? hipGetDevice(&dev) : hipStreamGetDevice(s, &dev);
  if (e != hipSuccess) return fail(MP_ERR_HIP, "%s: cannot find the stream's device: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(MP_ERR_UNSUPPORTED, "%s: device %d out of range", fn, dev);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
    void* ptr = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t back = hipSetDevice(cur);
      if (e == hipSuccess) e = back;
    }
    if (e != hipSuccess || ptr == nullptr)
      return fail(MP_ERR_HIP, "%s: no device address for the static scratch on device %d: %s", fn, dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MP_OK;
}

}  // namespace mp

extern "C" size_t mp_row_linear_partial_bwd_static_max_bytes(void) { return mp::kStaticScratchBytes; }

extern "C" int mp_row_linear_partial_bwd_static(mp_dtype dtype, int64_t T, int64_t Fi, int64_t K, const void* Y_i,
                                                const void* B_i, const void* dOut, void* dY_i, float* dB_i,
                                                hipStream_t s) {
  static const char* fn = "mp_row_linear_partial_bwd_static";
  MP_REQUIRE(dtype_ok(dtype), MP_ERR_DTYPE, "%s: bad dtype", fn);
  MP_REQUIRE(T >= 0 && K > 0 && Fi > 0, MP_ERR_SHAPE, "%s: bad shape", fn);
  // Host-visible checks first, so a bad call fails before the address lookup.
  if (int rc = validate_mat(dtype, K, fn, "K")) return rc;
  if (int rc = validate_mat(dtype, Fi, fn, "Fi")) return rc;
  MP_REQUIRE_PTR(Y_i);
  MP_REQUIRE_PTR(B_i);
  MP_REQUIRE_PTR(dOut);
  MP_REQUIRE_PTR(dY_i);
  MP_REQUIRE_PTR(dB_i);
  MP_REQUIRE_ALIGN(Y_i);
  MP_REQUIRE_ALIGN(B_i);
  MP_REQUIRE_ALIGN(dOut);
  MP_REQUIRE_ALIGN(dY_i);
  MP_REQUIRE_ALIGN(dB_i);
  const size_t need = mp_row_linear_partial_bwd_workspace(dtype, T, Fi, K);
  MP_REQUIRE(need <= kStaticScratchBytes, MP_ERR_WORKSPACE,
             "%s: this shape needs %zu scratch bytes, more than the static %zu; use mp_row_linear_partial_bwd", fn,
             need, kStaticScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    if (int rc = static_scratch(s, &ws, fn)) return rc;
  }
  return row_linear_bwd(fn, dtype, T, Fi, K, Y_i, B_i, dOut, nullptr, MP_ACT_NONE, dY_i, dB_i, ws,
                        need > 0 ? kStaticScratchBytes : 0, s);
}
