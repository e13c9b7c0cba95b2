// gfx950 matrix-core helpers: the bf16 MFMA wrappers and the LDS tile format
// shared by the GEMM, grouped-GEMM and attention kernels.
//
// LDS tile format: 64-deep k-tiles of bf16, stored as rows of eight 16-byte
// chunks.  For a K-contiguous operand a row is one operand row (8 chunks of 8
// k-values); for an MN-contiguous operand the tile is split into sub-tiles of
// 64 operand columns and a row is one k-value of a sub-tile (8 chunks of 8
// consecutive columns).  Chunk c of row r lives at slot r*8 + (c ^ swz(r)),
// where swz maps (r/2) % 8 one-to-one onto 0..7 and flips bit 2 between rows
// r and r+2 when r % 4 < 2.  With 64 four-byte banks (256 bytes per LDS cycle)
// this keeps three access patterns free of bank conflicts: 16-byte fragment
// reads (one chunk of 16 consecutive rows), 16-byte row-wise stores (two
// whole rows), and transpose reads (four consecutive rows x 64 bytes).
#pragma once

#include "common.h"

namespace mp {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// D(32x32) += A(32x16) * B(16x32), bf16 inputs, fp32 accumulate.  Lane l gives
// row (l % 32) of A and column (l % 32) of B, each with 8 k-values of k-group
// (l / 32); the result holds, in register r of lane l, element
// (row 8*(r/4) + 4*(l/32) + r%4, column l%32).
__device__ __forceinline__ f32x16_t mfma_32x32x16(const uint4& a, const uint4& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// C += (A x 2^(sa-127)) (B x 2^(sb-127))^T on 32x32 with 64 k-values of FP8
// E4M3 (OCP MX), fp32 accumulators in the same layout as mfma_32x32x16.
// Operand lane l (row l%32) holds, in a0, k-values 16*(l/32) .. +15 of the
// step and, in a1, k-values 32 + 16*(l/32) .. +15 (both 16-byte chunks of a
// K-contiguous LDS row).  The scale of the step's 32-value block 0 (k 0..31)
// of row r comes from lane r, that of block 1 (k 32..63) from lane r+32, as
// byte OS of the lane's scale register (measured on gfx950 against random
// operands and scales).
template <int OS>
__device__ __forceinline__ f32x16_t mfma_mx_32x32x64(const uint4& a0, const uint4& a1, const uint4& b0,
                                                     const uint4& b1, uint32_t sa, uint32_t sb, const f32x16_t& c) {
  typedef int i32x8_t __attribute__((ext_vector_type(8)));
  const i32x8_t a = {static_cast<int>(a0.x), static_cast<int>(a0.y), static_cast<int>(a0.z), static_cast<int>(a0.w),
                     static_cast<int>(a1.x), static_cast<int>(a1.y), static_cast<int>(a1.z), static_cast<int>(a1.w)};
  const i32x8_t b = {static_cast<int>(b0.x), static_cast<int>(b0.y), static_cast<int>(b0.z), static_cast<int>(b0.w),
                     static_cast<int>(b1.x), static_cast<int>(b1.y), static_cast<int>(b1.z), static_cast<int>(b1.w)};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, OS, static_cast<int>(sa), OS,
                                                         static_cast<int>(sb));
}

// D(16x16) += A(16x32) * B(32x16), bf16 inputs, fp32 accumulate.  Lane l
// gives row (l % 16) of A and column (l % 16) of B, each with 8 k-values
// 8*(l/16) .. +7; register r of lane l receives element
// (row 4*(l/16) + r, column l%16).
__device__ __forceinline__ f32x4_t mfma_16x16x32(const uint4& a, const uint4& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

__device__ __forceinline__ int lds_swz(int row) {
  const int t = (row >> 1) & 7;
  return t ^ ((t & 1) << 2);
}
__device__ __forceinline__ int lds_slot(int row, int chunk) { return row * 8 + (chunk ^ lds_swz(row)); }

// Row m of the MFMA result held by register r of lane `lane`.
__device__ __forceinline__ int mfma_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// ------------------------------------------------- LDS transpose reads
// ds_read_b64_tr_b16 (gfx950) works on groups of 16 lanes: source lane q of a
// group supplies the address of 4 consecutive 16-bit values, and lane i of the
// group receives value (i % 4) of source lane 4*j + i/4, for j = 0..3.  If
// source lane q points at row k0 + q/4, columns m0 + 4*(q%4) .. +3 of a
// row-major [k][m] tile, lane i therefore receives column m0 + i of rows
// k0 .. k0+3: four consecutive k-values of one column, i.e. a transposed read.
typedef short i16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_read_tr16(const void* p) {
  const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4_t*)(const_cast<void*>(p)));
  return __builtin_bit_cast(uint2, v);
}

// ------------------------------------------------ direct global -> LDS
// buffer_load_dwordx4 with the LDS flag writes the 16 bytes each lane fetches
// to LDS at M0 + 16 * lane (64 consecutive 16-byte slots per wave), without
// passing through registers; a lane whose offset lies outside the resource
// writes zeros.  It is issued from inline assembly so that the compiler's
// wait-count tracking, which would otherwise wait for it before every LDS
// read, leaves it alone: completion is awaited explicitly (wait_vmcnt).
typedef int i32x4_t __attribute__((ext_vector_type(4)));

// Raw buffer descriptor: base, stride 0, num_records = bytes, default format.
__device__ __forceinline__ i32x4_t make_desc(const void* base, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const int64_t n = bytes < 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : bytes);
  i32x4_t d;
  d[0] = static_cast<int>(a & 0xffffffffu);
  d[1] = static_cast<int>((a >> 32) & 0xffffu);
  d[2] = static_cast<int>(n);
  d[3] = 0x00020000;
  return d;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)(const_cast<void*>(p))));
}

__device__ __forceinline__ void dma16(const i32x4_t& desc, uint32_t voff, uint32_t lds_base) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_base);
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(desc), "s"(base)
               : "memory", "m0");
}

// Waits until at most N vector-memory loads of this wave are outstanding.
// (Inline assembly: the compiler may relax a waitcnt builtin it believes
// unnecessary, and it does not know about the direct loads.)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Waits until this wave has no vector-memory load and no LDS operation
// outstanding.  Before a barrier that hands an LDS buffer over to direct
// loads, this retires the wave's own reads of it: a plain __syncthreads()
// only waits for LDS writes.
__device__ __forceinline__ void wait_vm_lds() { asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory"); }

// vmcnt(0) as the builtin, which the compiler's wait-count tracking sees:
// loads it issued before count as complete afterwards.  Without it, a loop
// whose first use of such a load's value lies inside it gets a vmcnt(0) at
// that use on every iteration, which also waits for the direct loads just
// issued for the next tile.
__device__ __forceinline__ void wait_compiler_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Direct loader of one operand tile (R operand rows x 64 k-values, NT
// threads) into the LDS tile format.  Wave instruction q of wave w fills
// slots (q * NT/64 + w) * 64 .. +63; lane l fetches whichever global chunk
// belongs in slot base + l (the swizzle is undone on the global side, so the
// 8 lanes of a row still read 128 contiguous bytes).  Only the per-lane part
// of the address lives in a VGPR: the copy and k-step parts go in the
// instruction's scalar offset and M0, so issuing costs no vector ALU work.
// The range check covers the sum of the vector and scalar offsets (measured
// on gfx950: a lane whose in-range vector offset plus the scalar offset ends
// past the resource receives zeros), so a copy or k-step moved past the end
// by the scalar offset alone is fetched as zeros without touching memory.
// Rows past the end of a K-contiguous operand lie outside the resource and
// arrive as zeros; columns past the end of an MN-contiguous operand read
// neighbouring values that only reach discarded outputs.  A k-tile that
// extends past the k-range must use issue_checked(), which zeroes those
// elements.  Offsets are 32-bit: the operand panel must stay below 2 GiB.
template <int R, bool KC, int NT>
struct DmaTile {
  static_assert((R * 8) % NT == 0, "tile chunks must cover the threads");
  static_assert(KC || R % 64 == 0, "MN-contiguous tiles are whole 64-column sub-tiles");
  static constexpr int NWV = NT / 64, NI = R * 8 / NT;
  static_assert(NWV == 4 || NWV == 8, "4 or 8 waves");
  static constexpr uint32_t kOOB = 0x80000000u;
  i32x4_t desc;
  uint32_t voff;   // per-lane byte offset of copy 0 at k = 0
  int wave;        // wave index (uniform)
  int64_t ld, row0, rows;

  // K-contiguous: rows [row0, rows) of a matrix with row stride ld.
  // MN-contiguous: columns [row0, rows) of a [kdim][ld] matrix.
  __device__ __forceinline__ void init(const uint16_t* base, int64_t ld_, int64_t row0_, int64_t rows_, int64_t kdim,
                                       int tid) {
    const int lane = tid & 63;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    ld = ld_;
    row0 = row0_;
    rows = rows_;
    if constexpr (KC) desc = make_desc(base + row0 * ld, (rows - row0) * ld * 2);
    else desc = make_desc(base + row0, (kdim * ld - row0) * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) desc[i] = __builtin_amdgcn_readfirstlane(desc[i]);  // uniform: scalar registers
    // Slot (q * NWV + w) * 64 + l holds row/k-row wave*8 + l/8 (+ a per-copy
    // step), chunk (l % 8) ^ swz(row): the swizzle term does not depend on q.
    const int r = wave * 8 + (lane >> 3), c = (lane & 7) ^ lds_swz(r);
    voff = static_cast<uint32_t>((r * ld + c * 8) * 2);
  }

  // Copy q covers slots (q * NWV + w) * 64 + l: K-contiguous rows
  // q * NWV * 8 + (w * 8 + l / 8); MN-contiguous sub-tile (q * NWV) / 8 and
  // k-rows ((q * NWV) % 8) * 8 + (w * 8 + l / 8) (NWV divides 8).
  static constexpr int kq(int q) { return ((q * NWV) & 7) * 8; }
  static constexpr int subq(int q) { return (q * NWV) >> 3; }

  // Scalar offset of copy q at k-tile start k0.
  __device__ __forceinline__ uint32_t soff(int q, int64_t k0) const {
    if constexpr (KC) return static_cast<uint32_t>((q * NWV * 8 * ld + k0) * 2);
    else return static_cast<uint32_t>(((kq(q) + k0) * ld + subq(q) * 64) * 2);
  }

  // Fills `tile` with the k-tile starting at k0 (all 64 k-values in range),
  // or with zeros when `live` is false.
  __device__ __forceinline__ void issue(uint4* tile, int64_t k0, bool live) const {
    const uint32_t lb = __builtin_amdgcn_readfirstlane(lds_addr(tile)) + wave * 1024;
#pragma unroll
    for (int q = 0; q < NI; ++q) {
      const uint32_t so = live ? soff(q, k0) : kOOB;
      const uint32_t m0v = lb + q * NWV * 1024;
      asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds" ::"v"(voff), "s"(desc),
                   "s"(m0v), "s"(so)
                   : "memory", "m0");
    }
  }

  // K-contiguous operand whose resource starts at row 0: fills `tile` with
  // rows row_off .. row_off + R - 1 at k-values k0 .. k0 + 63; rows past the
  // resource's end arrive as zeros.
  __device__ __forceinline__ void issue_rows(uint4* tile, int64_t row_off, int64_t k0) const {
    static_assert(KC, "row offsets are for K-contiguous operands");
    const uint32_t lb = __builtin_amdgcn_readfirstlane(lds_addr(tile)) + wave * 1024;
    const uint32_t ro = static_cast<uint32_t>(row_off * ld * 2);
#pragma unroll
    for (int q = 0; q < NI; ++q) {
      const uint32_t so = soff(q, k0) + ro;
      const uint32_t m0v = lb + q * NWV * 1024;
      asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds" ::"v"(voff), "s"(desc),
                   "s"(m0v), "s"(so)
                   : "memory", "m0");
    }
  }

  // As issue(), zeroing elements at k >= kend and, for an MN-contiguous
  // operand, columns past its end.
  __device__ __forceinline__ void issue_checked(uint4* tile, int64_t k0, int64_t kend, int tid) const {
    const int lane = tid & 63;
    const uint32_t lb = __builtin_amdgcn_readfirstlane(lds_addr(tile)) + wave * 1024;
    const int r = wave * 8 + (lane >> 3), c = (lane & 7) ^ lds_swz(r);
#pragma unroll
    for (int q = 0; q < NI; ++q) {
      bool ok;
      if constexpr (KC) ok = k0 + c * 8 < kend;
      else ok = k0 + kq(q) + r < kend && row0 + subq(q) * 64 + c * 8 < rows;
      const uint32_t v = ok ? voff + soff(q, k0) : kOOB;
      const uint32_t m0v = lb + q * NWV * 1024;
      asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(v), "s"(desc),
                   "s"(m0v)
                   : "memory", "m0");
    }
  }
};

// As wait_vm_lds(), leaving the N most recent vector-memory loads in flight.
template <int N>
__device__ __forceinline__ void wait_vm_lds_n() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(N) : "memory");
}

// Grid-wide warm-up of a future k-tile: the 128-byte lines that k-tile
// covers in both operands (all rows, not just this workgroup's) are split
// over every wave of the grid, each wave requesting its few lines with one
// 4-byte direct load into a dummy LDS word.  Each line is thus requested once
// for the whole grid, so by the time the workgroups' own loads reach it the
// line sits in the last-level cache instead of HBM.  The waves of the first
// operand's share of the grid request its lines, the others the second's.
// A K-contiguous operand has one line per row and k-tile (row r, k0..k0+63);
// an MN-contiguous one ceil(cols/64) lines per k-row.  Lanes without a line,
// and k-tiles past the end, request nothing.
struct GridWarm {
  i32x4_t desc;
  uint32_t voff;     // per-lane byte offset at k = 0, or out of range
  uint32_t kstride;  // bytes per k-value (2, or 2*ld for an MN-contiguous operand)

  // lines_a / lines_b: lines of one k-tile of each operand; slot = this wave's
  // index in the grid, nslots = waves in the grid.
  __device__ __forceinline__ void init(const uint16_t* a, int64_t lda, int64_t rows_a, int64_t kdim, bool a_kc,
                                       const uint16_t* b, int64_t ldb, int64_t rows_b, bool b_kc, int slot,
                                       int nslots, int lane) {
    const int64_t la = a_kc ? rows_a : 64 * ((rows_a + 63) / 64);
    const int64_t lb = b_kc ? rows_b : 64 * ((rows_b + 63) / 64);
    // Waves [0, sa) warm A, the rest B, in proportion to their line counts.
    int64_t sa = (nslots * la + (la + lb) / 2) / (la + lb);
    sa = sa < 1 ? 1 : (sa > nslots - 1 ? nslots - 1 : sa);
    const bool is_a = slot < sa;
    const int64_t ns = is_a ? sa : nslots - sa;
    const int64_t line = (is_a ? slot : slot - sa) + static_cast<int64_t>(lane) * ns;
    const uint16_t* base = is_a ? a : b;
    const int64_t ld = is_a ? lda : ldb, rows = is_a ? rows_a : rows_b, nl = is_a ? la : lb;
    const bool kc = is_a ? a_kc : b_kc;
    desc = make_desc(base, kc ? rows * ld * 2 : kdim * ld * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) desc[i] = __builtin_amdgcn_readfirstlane(desc[i]);  // uniform per wave
    if (line >= nl) {
      voff = 0x80000000u;
    } else if (kc) {
      voff = static_cast<uint32_t>(line * ld * 2);
    } else {
      const int64_t cpr = (rows + 63) / 64;
      voff = static_cast<uint32_t>(((line / cpr) * ld + (line % cpr) * 64) * 2);
    }
    kstride = kc ? 2u : static_cast<uint32_t>(ld * 2);
  }

  __device__ __forceinline__ void issue(const void* sink, int64_t k0, bool live) const {
    // Uniform per wave; readfirstlane keeps it in a scalar register even where
    // the compiler cannot prove that.
    const uint32_t so = __builtin_amdgcn_readfirstlane(live ? static_cast<uint32_t>(k0) * kstride : 0x80000000u);
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr(sink));
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, %3 offen lds" ::"v"(voff), "s"(desc),
                 "s"(m0v), "s"(so)
                 : "memory", "m0");
  }
};

// MFMA operand fragment of k-step ks (16 k-values) for operand rows
// r0 .. r0+31 (r0 % 32 == 0) of a tile in the LDS tile format: lane l gets row
// r0 + l%32, k-values 16*ks + 8*(l/32) .. +7.  An MN-contiguous tile is read
// with two transpose reads of four k-rows each.
template <bool KC>
__device__ __forceinline__ uint4 lds_frag(const uint4* tile, int r0, int ks, int lane) {
  if constexpr (KC) {
    return tile[lds_slot(r0 + (lane & 31), 2 * ks + (lane >> 5))];
  } else {
    const int i = lane & 15;
    const int k = 16 * ks + 8 * (lane >> 5) + (i >> 2);
    const int c = r0 + 16 * ((lane >> 4) & 1) + 4 * (i & 3);
    const char* sub = reinterpret_cast<const char*>(tile + (c >> 6) * 512) + (c & 7) * 2;
    const uint2 lo = lds_read_tr16(sub + lds_slot(k, (c & 63) >> 3) * 16);
    const uint2 hi = lds_read_tr16(sub + lds_slot(k + 4, (c & 63) >> 3) * 16);
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
  }
}

// Instruction-scheduling pattern for a software-pipelined MFMA step: NM
// MFMAs, each followed by its share of NDS LDS operations (kind DSM: 0x100
// reads, 0x200 writes) and NVM global loads.
template <int M, int NM, int DSM, int NDS, int NVM>
__device__ __forceinline__ void sched_mfma_interleave() {
  if constexpr (M < NM) {
    constexpr int dper = (NDS + NM - 1) / NM, d0 = M * dper;
    constexpr int dn = d0 >= NDS ? 0 : (NDS - d0 < dper ? NDS - d0 : dper);
    constexpr int vper = (NVM + NM - 1) / NM, v0 = M * vper;
    constexpr int vn = v0 >= NVM ? 0 : (NVM - v0 < vper ? NVM - v0 : vper);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (dn > 0) __builtin_amdgcn_sched_group_barrier(DSM, dn, 0);
    if constexpr (vn > 0) __builtin_amdgcn_sched_group_barrier(0x020, vn, 0);
    sched_mfma_interleave<M + 1, NM, DSM, NDS, NVM>();
  }
}

}  // namespace mp
