// gfx950 matrix-core helpers: the bf16 MFMA wrappers and the LDS tile format
// shared by the GEMM, grouped-GEMM and attention kernels.
//
// LDS tile format: a tile of R rows x 64 k-values (bf16) is stored as R rows
// of eight 16-byte chunks (8 k-values each).  Chunk c of row r lives at slot
// r*8 + (c ^ (r & 7)): the XOR swizzle puts the same chunk of 8 consecutive
// rows in 8 different bank groups, so both the 16-byte row-wise stores and
// the 16-byte fragment reads (32 consecutive rows, one chunk) are free of
// bank conflicts.
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

// ------------------------------------------------------------ buffer loads
// A buffer resource covers [base, base + bytes); a load at an offset outside
// it returns zeros, which the tile loaders use for every out-of-range element.
typedef __amdgpu_buffer_rsrc_t BufRes;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
constexpr uint32_t kBufOOB = 0x80000000u;  // offset past any resource (<= 2 GiB)

__device__ __forceinline__ BufRes make_bufres(const void* base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(n),
                                           0x00020000);
}

__device__ __forceinline__ uint4 buf_load16(const BufRes& r, uint32_t off) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ int lds_slot(int row, int chunk) { return row * 8 + (chunk ^ (row & 7)); }

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

// 8x8 transpose of 16-bit values: in[k] holds 8 values (columns 0..7) of row
// k; out[c] receives the 8 values of column c (rows 0..7).
__device__ __forceinline__ uint32_t u4_word(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

__device__ __forceinline__ void transpose8x8_b16(const uint4* in, uint4* out) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {      // column pair (2p, 2p+1)
    uint32_t ev[4], od[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {    // row pair (2w, 2w+1)
      const uint32_t r0 = u4_word(in[2 * w], p);
      const uint32_t r1 = u4_word(in[2 * w + 1], p);
      ev[w] = __builtin_amdgcn_perm(r1, r0, 0x05040100u);  // low halves
      od[w] = __builtin_amdgcn_perm(r1, r0, 0x07060302u);  // high halves
    }
    out[2 * p] = make_uint4(ev[0], ev[1], ev[2], ev[3]);
    out[2 * p + 1] = make_uint4(od[0], od[1], od[2], od[3]);
  }
}

// Global -> register -> LDS loader of one R x 64 operand tile, NT threads.  Loads go
// through a buffer resource whose base is the tile's first row (K-contiguous)
// or first column (MN-contiguous); an element outside the matrix or past the
// k-range gets an out-of-range offset, which the hardware returns as zeros.
template <int R, bool KC, int NT>
struct TileLoader {
  static constexpr int NBLK = KC ? 0 : (R + NT - 1) / NT;  // 8x8 blocks per thread
  static constexpr int NREG = KC ? R * 8 / NT : 8 * NBLK;
  static_assert(!KC || (R * 8) % NT == 0, "tile rows must cover the threads");
  uint4 reg[NREG];

  // Resource for rows [row0, rows) of a K-contiguous matrix with row stride
  // `ld`, or for columns [row0, ld) of an MN-contiguous matrix of `kdim` rows.
  __device__ __forceinline__ static BufRes resource(const uint16_t* base, int64_t ld, int64_t row0, int64_t rows,
                                                    int64_t kdim) {
    if constexpr (KC) return make_bufres(base + row0 * ld, (rows - row0) * ld * 2);
    else return make_bufres(base + row0, (kdim * ld - row0) * 2);
  }

  // `res_row` = rows between the resource base and row0 (K-contiguous only).
  __device__ __forceinline__ void load(const BufRes& rs, int64_t ld, int64_t row0, int64_t rows, int64_t k0,
                                       int64_t kend, int tid, int64_t res_row = 0) {
    if constexpr (KC) {
#pragma unroll
      for (int i = 0; i < NREG; ++i) {
        const int idx = tid + NT * i;
        const int64_t r = idx >> 3;
        const int64_t gk = k0 + (idx & 7) * 8;
        const bool ok = row0 + r < rows && gk < kend;
        reg[i] = buf_load16(rs, ok ? static_cast<uint32_t>(((res_row + r) * ld + gk) * 2) : kBufOOB);
      }
    } else {
#pragma unroll
      for (int b = 0; b < NBLK; ++b) {
        const int idx = tid + NT * b;
        const int64_t mm = (idx >> 3) * 8;
        const int64_t gk = k0 + (idx & 7) * 8;
        const bool ok = idx < R && row0 + mm < rows;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
          reg[8 * b + kk] =
              buf_load16(rs, (ok && gk + kk < kend) ? static_cast<uint32_t>(((gk + kk) * ld + mm) * 2) : kBufOOB);
      }
    }
  }

  __device__ __forceinline__ void store(uint4* __restrict__ tile, int tid) const {
    if constexpr (KC) {
#pragma unroll
      for (int i = 0; i < NREG; ++i) {
        const int idx = tid + NT * i;
        tile[lds_slot(idx >> 3, idx & 7)] = reg[i];
      }
    } else {
#pragma unroll
      for (int b = 0; b < NBLK; ++b) {
        const int idx = tid + NT * b;
        if (idx < R) {
          uint4 t[8];
          transpose8x8_b16(reg + 8 * b, t);
          const int mb = (idx >> 3) * 8, kb = idx & 7;
#pragma unroll
          for (int i = 0; i < 8; ++i) tile[lds_slot(mb + i, kb)] = t[i];
        }
      }
    }
  }
};

}  // namespace mp
