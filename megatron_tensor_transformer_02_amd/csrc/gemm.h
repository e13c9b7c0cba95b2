// Host-side entry points of the GEMM family and the column-sum helper, used
// by the attention and MoE translation units.
#pragma once

#include "common.h"

namespace mp {

enum Epilogue { EPI_STORE = 0, EPI_SPLITK = 1, EPI_DACT = 2, EPI_LSE = 3 };

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

// Deterministic column sums of a [rows, cols] matrix into out[cols] (fp32).
int colsum(mp_dtype dt, int64_t rows, int64_t cols, const void* dy, float* out, void* ws, hipStream_t s);
size_t colsum_workspace(int64_t rows, int64_t cols);

}  // namespace mp
