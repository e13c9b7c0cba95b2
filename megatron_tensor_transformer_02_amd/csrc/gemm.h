// Host-side entry points of the GEMM family and the column-sum helper, used
// by the attention and MoE translation units.
#pragma once

#include "common.h"

namespace mp {

enum Epilogue { EPI_STORE = 0, EPI_SPLITK = 1, EPI_DACT = 2, EPI_LSE = 3, EPI_SWIGLU_BWD = 4 };

// Operand layouts of C = A * B^T: NT = both K-contiguous; NN = A K-contiguous,
// B MN-contiguous; TN = both MN-contiguous.
enum Layout { NT = 0, NN = 1, TN = 2 };

// C[M,N] (ldc) = A * B^T (+bias[N], activation, pre-activation save).
// `allow_split` lets an fp32-output GEMM without epilogue split K, using `ws`
// (gemm_splitk_workspace bytes) for the partials.
int gemm(mp_dtype dt, Layout lay, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
         int64_t ldb, void* C, int64_t ldc, bool out_bf16, const void* bias, int act, void* zsave, bool allow_split,
         void* ws, size_t ws_bytes, hipStream_t s, int epi = EPI_STORE, const void* zin = nullptr);
size_t gemm_splitk_workspace(mp_dtype dt, int64_t M, int64_t N, int64_t K);

// Logits GEMM Z = H * E^T (bf16 in, fp32 accumulators) whose epilogue keeps
// only row statistics: for every row t and every slot of columns (one slot
// per wave-column of a tile), part[(t*P + slot)*3 + {0,1,2}] = (max, sum of
// exp(z - max), z at column labels[t] - v_start or 0) over the slot's columns.
// Nothing of Z is stored.  P = gemm_lse_slots(T, V, K).
int gemm_lse_slots(int64_t T, int64_t V, int64_t K);
int gemm_logits_lse(int64_t T, int64_t V, int64_t K, const void* H, const void* E, const int32_t* labels,
                    int64_t v_start, float* part, hipStream_t s);

// Grouped bf16 GEMMs with their shapes on the device (256x256 tiles).
// GRP_M (layout NN): group e is C[lo:hi, :N] = A[lo:hi, :K] * B_e^T with
// lo, hi = off[e], off[e+1], B_e = B + e * stride_b, and tiles[e] the first
// 256-row tile of group e in a flat tile list (tiles[groups] = its length,
// at most max_mtiles).  epi = EPI_STORE (bf16 out) or EPI_SWIGLU_BWD: C and
// zin are [rows, 2N]; zin holds the gate (columns [0, N)) and up ([N, 2N))
// pre-activations, C receives d gate and d up of d act = A * B_e^T.  With
// row_w (rows' weights, [rows] fp32), the activation was act_w = w * act:
// A * B_e^T is d act_w, d act = w * d act_w, and row_part [rows, N/8] gets
// the sums of d act_w * act over each 8 columns (the weight's gradient).
// GRP_K (layout TN, fp32 out): group e is C_e[M, N] = sum over k in
// [lo, hi) of A[k, m] * B[k, n], C_e = C + e * stride_c (zeros when lo = hi).
int gemm_grouped_m(int epi, int groups, const int32_t* off, const int32_t* tiles, int64_t max_mtiles, int64_t N,
                   int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb, int64_t stride_b, void* C,
                   int64_t ldc, const void* zin, hipStream_t s, const float* row_w = nullptr,
                   float* row_part = nullptr);
// max_k bounds every group's k-range (for the 2 GiB addressing check).
int gemm_grouped_k(int groups, const int32_t* off, int64_t max_k, int64_t M, int64_t N, const void* A, int64_t lda,
                   const void* B, int64_t ldb, float* C, int64_t ldc, int64_t stride_c, hipStream_t s);

// Deterministic column sums of a [rows, cols] matrix into out[cols] (fp32).
int colsum(mp_dtype dt, int64_t rows, int64_t cols, const void* dy, float* out, void* ws, hipStream_t s);
size_t colsum_workspace(int64_t rows, int64_t cols);

}  // namespace mp
