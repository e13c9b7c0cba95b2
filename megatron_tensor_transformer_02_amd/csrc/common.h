// Internal helpers shared by the libmp translation units: status handling,
// argument validation, bf16 conversion, vector types and the Philox4x32-10
// generator used by the shared-seed dropout.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>
#include <math.h>

#include "mp.h"

namespace mp {

// ----------------------------------------------------------------- status

// Records `msg` as this thread's last error and returns `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int ok();

// Translates the result of a kernel launch into a status.
int check_launch(const char* what);

// Debug-mode data check, active when MP_DEBUG_CHECKS is set to a value other
// than "0": copies the n int32 indices at idx (device memory) to the host
// after the work already queued on s, and returns MP_ERR_DATA naming the
// first index outside [lo, hi).  Synchronises s, so it is for debugging
// (and not for code under graph capture).  MP_OK when the variable is unset.
int debug_check_range(const char* fn, const char* what, const int32_t* idx, int64_t n, int64_t lo, int64_t hi,
                      hipStream_t s);

#define MP_REQUIRE(cond, code, ...) \
  do {                              \
    if (!(cond)) return ::mp::fail(code, __VA_ARGS__); \
  } while (0)

#define MP_REQUIRE_PTR(p) MP_REQUIRE((p) != nullptr, MP_ERR_NULL, "%s: %s is NULL", __func__, #p)
#define MP_REQUIRE_ALIGN(p) \
  MP_REQUIRE((reinterpret_cast<uintptr_t>(p) & 15u) == 0, MP_ERR_ALIGN, "%s: %s is not 16-byte aligned", __func__, #p)
#define MP_REQUIRE_OPT_ALIGN(p) \
  MP_REQUIRE((p) == nullptr || (reinterpret_cast<uintptr_t>(p) & 15u) == 0, MP_ERR_ALIGN, \
             "%s: %s is not 16-byte aligned", __func__, #p)

inline size_t dtype_size(mp_dtype t) { return t == MP_BF16 ? 2 : 4; }
inline bool dtype_ok(int t) { return t == MP_F32 || t == MP_BF16; }
// Elements per 16-byte vector.
inline int64_t vec_elems(mp_dtype t) { return t == MP_BF16 ? 8 : 4; }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t a, size_t b) { return (a + b - 1) / b * b; }

// Host-side Philox keep threshold floor(p * 2^32) from the float32 p.
inline uint32_t dropout_threshold(float p) {
  return static_cast<uint32_t>(floor(static_cast<double>(p) * 4294967296.0));
}

// --------------------------------------------------------------- bf16 math

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round-to-nearest-even float -> bf16 (NaN stays NaN; denormals are kept,
// the kernels run with f32 denormals preserved).  gfx950 converts two floats
// in one instruction (v_cvt_pk_bf16_f32), which the compiler emits for these
// conversions.
typedef float f32x2v_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f)); }

// 2^x by the hardware instruction (v_exp_f32, about 1 ulp).  Results below
// 2^-126 flush to zero instead of going through the library's denormal
// rescaling: every use is a softmax weight (the exponential of a value at or
// below the running maximum, whose own weight is 1), where a term that small
// is negligible.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v_t{lo, hi}, bf16x2v_t));
}

// 8 bf16 (one uint4) <-> 8 floats.
__device__ __forceinline__ void unpack8(const uint4& v, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ uint4 pack8(const float* f) {
  return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                    pack_bf16x2(f[6], f[7]));
}

// Loads/stores of one 16-byte vector as floats: 8 bf16 or 4 fp32.
// Streaming (non-temporal) 16-byte loads/stores for data read or written
// once, such as the shard partials of a reduce: they do not displace what the
// next kernel reads (its GEMM operands) from the last-level cache.
typedef float nt_f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int nt_u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_stream16(const void* p) {
  const nt_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ void store_stream16(void* p, const uint4& v) {
  const nt_u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<nt_u32x4*>(p));
}

template <bool BF16>
struct Vec16 {
  static constexpr int N = BF16 ? 8 : 4;
  __device__ __forceinline__ static void load(const void* base, int64_t elem, float* f) {
    unpack(*reinterpret_cast<const uint4*>(static_cast<const char*>(base) + elem * (BF16 ? 2 : 4)), f);
  }
  // As load(), for data read exactly once (streaming).
  __device__ __forceinline__ static void load_stream(const void* base, int64_t elem, float* f) {
    unpack(load_stream16(static_cast<const char*>(base) + elem * (BF16 ? 2 : 4)), f);
  }
  __device__ __forceinline__ static void unpack(const uint4& v, float* f) {
    if constexpr (BF16) {
      unpack8(v, f);
    } else {
      f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
      f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
    }
  }
  __device__ __forceinline__ static void store(void* base, int64_t elem, const float* f) {
    uint4 v;
    if constexpr (BF16) {
      v = pack8(f);
    } else {
      v = make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
    }
    *reinterpret_cast<uint4*>(static_cast<char*>(base) + elem * (BF16 ? 2 : 4)) = v;
  }
};

// ------------------------------------------------------------ Philox4x32-10
//
// Counter-based generator of Salmon, Moraes, Dror and Shaw ("Parallel Random
// Numbers: As Easy as 1, 2, 3", SC'11).  A round multiplies counter word 0 by
// 0xD2511F53 and word 2 by 0xCD9E8D57 (full 64-bit products) and forms
// (hi(w2 product) ^ w1 ^ key0, lo(w2 product), hi(w0 product) ^ w3 ^ key1,
// lo(w0 product)); the key advances by the Weyl increments 0x9E3779B9 and
// 0xBB67AE85 between the ten rounds.
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = static_cast<uint64_t>(0xD2511F53u) * c.x;
    const uint64_t p1 = static_cast<uint64_t>(0xCD9E8D57u) * c.z;
    c = make_uint4(static_cast<uint32_t>(p1 >> 32) ^ c.y ^ k0, static_cast<uint32_t>(p1),
                   static_cast<uint32_t>(p0 >> 32) ^ c.w ^ k1, static_cast<uint32_t>(p0));
  }
  return c;
}

// Dropout words for the four elements 4*blk .. 4*blk+3 of a stream.
__device__ __forceinline__ uint4 dropout_words(uint64_t blk, uint64_t seed, uint64_t offset) {
  return philox4x32_10(make_uint4(static_cast<uint32_t>(blk), static_cast<uint32_t>(blk >> 32),
                                  static_cast<uint32_t>(offset), static_cast<uint32_t>(offset >> 32)),
                       static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32));
}

struct DropoutParams {
  uint64_t seed, offset, index_base;
  uint32_t threshold;  // keep iff word >= threshold
  float scale;         // 1 / (1 - p)
  int enabled;         // p > 0
};

inline DropoutParams make_dropout(float p, uint64_t seed, uint64_t offset, uint64_t index_base) {
  DropoutParams d;
  d.seed = seed;
  d.offset = offset;
  d.index_base = index_base;
  d.threshold = dropout_threshold(p);
  d.scale = 1.0f / (1.0f - p);
  d.enabled = p > 0.0f;
  return d;
}

// Applies dropout to `n` (4 or 8) consecutive values whose first flat index
// `j0` is a multiple of 4; writes the keep flags to `keep`.
template <int N>
__device__ __forceinline__ void apply_dropout(const DropoutParams& d, uint64_t j0, float* v, uint8_t* keep) {
  if (!d.enabled) {
#pragma unroll
    for (int i = 0; i < N; ++i) keep[i] = 1;
    return;
  }
#pragma unroll
  for (int b = 0; b < N / 4; ++b) {
    const uint4 w = dropout_words((j0 >> 2) + b, d.seed, d.offset);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool k = ws[i] >= d.threshold;
      keep[4 * b + i] = k ? 1 : 0;
      v[4 * b + i] = k ? v[4 * b + i] * d.scale : 0.0f;
    }
  }
}

// Saved dropout keep flags, one bit per element: bit (e & 7) of byte e >> 3
// is the flag of flat element e (1 = kept).  A thread holds E (8 or 4)
// consecutive elements starting at e0, a multiple of E.  With E = 4 the two
// halves of a byte sit in neighbouring lanes (lane ^ 1): the lane holding
// the even half writes the byte, so every lane of the wave must make this
// call together (non-live lanes pass live = false and all-zero flags).
template <int E>
__device__ __forceinline__ void store_keep_bits(uint8_t* bits, int64_t e0, const uint8_t* keep, bool live) {
  uint32_t b = 0;
#pragma unroll
  for (int i = 0; i < E; ++i) b |= static_cast<uint32_t>(keep[i] & 1u) << i;
  if constexpr (E == 8) {
    if (live) bits[e0 >> 3] = static_cast<uint8_t>(b);
  } else {
    const uint32_t other = static_cast<uint32_t>(__shfl_xor(static_cast<int>(b), 1, 64));
    if (live && (e0 & 7) == 0) bits[e0 >> 3] = static_cast<uint8_t>(b | (other << 4));
  }
}

// The E flags of elements e0 .. e0+E-1 from saved bits.
template <int E>
__device__ __forceinline__ uint32_t load_keep_bits(const uint8_t* bits, int64_t e0) {
  const uint32_t byte = bits[e0 >> 3];
  return E == 8 ? byte : (byte >> (e0 & 7)) & 0xFu;
}

__device__ __forceinline__ float4 load_nt4(const float* p) {
  const nt_f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_f32x4*>(p));
  return make_float4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ void store_nt4(float* p, float a, float b, float c, float d) {
  nt_f32x4 v = {a, b, c, d};
  __builtin_nontemporal_store(v, reinterpret_cast<nt_f32x4*>(p));
}

// ----------------------------------------------------------- wave helpers

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace mp

namespace mp {

// ------------------------------------------------------------- activations
// GeLU is not defined on the pages; MP_ACT_GELU_ERF is the exact z*Phi(z),
// MP_ACT_GELU_TANH the usual tanh approximation.  erff/tanhf/expf are the
// device math library's.

__device__ __forceinline__ float act_fwd(float z, int act) {
  if (act == MP_ACT_GELU_ERF) return 0.5f * z * (1.0f + erff(z * 0.7071067811865476f));
  if (act == MP_ACT_GELU_TANH) {
    const float u = 0.7978845608028654f * (z + 0.044715f * z * z * z);
    return 0.5f * z * (1.0f + tanhf(u));
  }
  return z;
}

__device__ __forceinline__ float act_grad(float z, int act) {
  if (act == MP_ACT_GELU_ERF) {
    const float cdf = 0.5f * (1.0f + erff(z * 0.7071067811865476f));
    const float pdf = 0.3989422804014327f * expf(-0.5f * z * z);
    return cdf + z * pdf;
  }
  if (act == MP_ACT_GELU_TANH) {
    const float c = 0.7978845608028654f;
    const float t = tanhf(c * (z + 0.044715f * z * z * z));
    return 0.5f * (1.0f + t) + 0.5f * z * (1.0f - t * t) * c * (1.0f + 3.0f * 0.044715f * z * z);
  }
  return 1.0f;
}

// Branch-free variants for bf16 outputs, where a few 1e-7 of absolute error
// is far below the output's resolution.  erf uses Abramowitz & Stegun,
// Handbook of Mathematical Functions, formula 7.1.26 (|error| <= 1.5e-7):
// erf(a) = 1 - t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-a^2),
// t = 1 / (1 + p a), a = |x|, odd in x.  tanh(u) = 1 - 2 / (exp(2u) + 1).
// exp and the reciprocal are the hardware's exp2 and rcp instructions.
__device__ __forceinline__ float erf_fast(float x) {
  const float a = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, a, 1.0f));
  float q = fmaf(1.061405429f, t, -1.453152027f);
  q = fmaf(q, t, 1.421413741f);
  q = fmaf(q, t, -0.284496736f);
  q = fmaf(q, t, 0.254829592f);
  const float e = __builtin_amdgcn_exp2f(-a * a * 1.4426950408889634f);
  return copysignf(fmaf(-q * t, e, 1.0f), x);
}

__device__ __forceinline__ float tanh_fast(float u) {
  const float e = __builtin_amdgcn_exp2f(2.8853900817779268f * u);  // exp(2u)
  return fmaf(-2.0f, __builtin_amdgcn_rcpf(e + 1.0f), 1.0f);
}

__device__ __forceinline__ float act_fwd_fast(float z, int act) {
  if (act == MP_ACT_GELU_ERF) return 0.5f * z * (1.0f + erf_fast(z * 0.7071067811865476f));
  if (act == MP_ACT_GELU_TANH) return 0.5f * z * (1.0f + tanh_fast(0.7978845608028654f * (z + 0.044715f * z * z * z)));
  return z;
}

__device__ __forceinline__ float act_grad_fast(float z, int act) {
  if (act == MP_ACT_GELU_ERF) {
    const float cdf = 0.5f * (1.0f + erf_fast(z * 0.7071067811865476f));
    const float pdf = 0.3989422804014327f * __builtin_amdgcn_exp2f(-0.7213475204444817f * z * z);
    return cdf + z * pdf;
  }
  if (act == MP_ACT_GELU_TANH) {
    const float c = 0.7978845608028654f;
    const float t = tanh_fast(c * (z + 0.044715f * z * z * z));
    return 0.5f * (1.0f + t) + 0.5f * z * (1.0f - t * t) * c * (1.0f + 3.0f * 0.044715f * z * z);
  }
  return 1.0f;
}

inline bool act_ok(int act) { return act == MP_ACT_NONE || act == MP_ACT_GELU_ERF || act == MP_ACT_GELU_TANH; }

}  // namespace mp
