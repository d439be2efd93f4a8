/*
 * decode_gemm.h — C ABI of the decode projection with M == 1 over a
 * transposed weight, part of libpagedattn (MI355X, gfx950).
 *
 * Source: "优化" on tiny-llm (open-infra-ai.github.io/tiny-llm/performance/
 * optimization), section 4 (M==1 转置权重 GEMM 快路径): in a decode step the
 * projections multiply a single activation row by a [K, N] weight; keeping
 * the weight transposed, [N, K], lets the threads of one output read
 * consecutive k (coalesced), and the transposed copy is built once when the
 * weights are loaded. Section 1 (W8A16): int8 weights with fp16 activations
 * and symmetric scales per group of k (no zero point).
 *
 * What is computed:
 *   W[k, n] = wt[n, k]                                  (fp16 weights)
 *   W[k, n] = wt[n, k] * scales_t[n, k / group_size]    (int8 weights)
 *   y[m, n] = sum_k x[m, k] * W[k, n], accumulated in fp32, rounded to fp16
 *             (round to nearest even)
 *
 * Conventions as in paged_attn.h: device pointers owned by the caller,
 * nothing allocated, work enqueued on `stream`, PA_OK (0) or a negative
 * PA_ERR_* status, arguments checked on the host before anything is enqueued.
 */
#ifndef DECODE_GEMM_H
#define DECODE_GEMM_H

#include <stdint.h>

#include "paged_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

enum pa_weight_dtype {
  PA_W_FP16 = 0,  /* IEEE binary16 weights */
  PA_W_INT8 = 1,  /* symmetric int8 codes with fp32 scales per group of k */
};

/*
 * gemm_m1_transposed — y = x . W for 1 <= M <= 4 activation rows, W given
 * transposed.
 *   x        [M, K] fp16, 16-byte aligned
 *   wt       [N, K] fp16 or int8, 16-byte aligned (row n holds column n of W)
 *   scales_t [N, K / group_size] fp32 (int8 weights; NULL for fp16)
 *   y        [M, N] fp16
 * Requirements: N >= 1; K a multiple of 8 (fp16) or 16 (int8) with
 * M * K * 2 <= 65536 (the activation rows are staged in LDS); int8:
 * group_size a multiple of 16 dividing K. PA_ERR_SHAPE / PA_ERR_DTYPE /
 * PA_ERR_NULL otherwise.
 */
int gemm_m1_transposed(int32_t M, int32_t N, int32_t K, int32_t w_dtype,
                       int32_t group_size, const void* x, const void* wt,
                       const float* scales_t, void* y, hipStream_t stream);

/*
 * transpose_weights — the load-time [cols, rows] copy of a [rows, cols]
 * matrix, bit for bit: wt[c, r] = w[r, c] for elements of elem_bytes (1, 2
 * or 4) bytes. Builds wt (and scales_t) for gemm_m1_transposed from a [K, N]
 * weight (and its [K / group_size, N] scales). w and wt must not overlap.
 * rows <= 4194240 (65535 tiles of 64) and rows * cols < 2^40.
 */
int transpose_weights(int32_t rows, int32_t cols, int32_t elem_bytes,
                      const void* w, void* wt, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* DECODE_GEMM_H */
