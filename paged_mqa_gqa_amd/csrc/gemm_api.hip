// C ABI of the decode projection (declarations and contract in
// include/decode_gemm.h): host-side checks and dispatch only.
#include "decode_gemm.h"

#include <stdint.h>

#include "launch.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_HIP; }

}  // namespace

extern "C" {

int gemm_m1_transposed(int32_t M, int32_t N, int32_t K, int32_t w_dtype,
                       int32_t group_size, const void* x, const void* wt,
                       const float* scales_t, void* y, hipStream_t stream) {
  if (w_dtype != PA_W_FP16 && w_dtype != PA_W_INT8) return PA_ERR_DTYPE;
  const bool int8 = w_dtype == PA_W_INT8;
  if (M < 1 || M > 4 || N < 1 || K < 1) return PA_ERR_SHAPE;
  if (K % (int8 ? 16 : 8) != 0 || (int64_t)M * K * 2 > 65536) return PA_ERR_SHAPE;
  if (int8 && (group_size < 16 || group_size % 16 != 0 || K % group_size != 0))
    return PA_ERR_SHAPE;
  if (!x || !wt || !y || (int8 && !scales_t)) return PA_ERR_NULL;
  if (!aligned16(x) || !aligned16(wt)) return PA_ERR_SHAPE;
  pa::GemmArgs a{};
  a.x = static_cast<const _Float16*>(x);
  a.wt = static_cast<const uint8_t*>(wt);
  a.scales_t = scales_t;
  a.y = static_cast<_Float16*>(y);
  a.M = M;
  a.N = N;
  a.K = K;
  a.group = int8 ? group_size : K;
  return hip_status(pa::launch_gemm_m1(a, int8, stream));
}

int transpose_weights(int32_t rows, int32_t cols, int32_t elem_bytes, const void* w,
                      void* wt, hipStream_t stream) {
  if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4) return PA_ERR_DTYPE;
  // the kernel's grid has ceil(rows / 64) workgroups along y (at most 65535)
  if (rows < 1 || cols < 1 || rows > 65535 * 64 || (int64_t)rows * cols >= (1LL << 40))
    return PA_ERR_SHAPE;
  if (!w || !wt) return PA_ERR_NULL;
  return hip_status(pa::launch_transpose(w, wt, rows, cols, elem_bytes, stream));
}

}  // extern "C"
