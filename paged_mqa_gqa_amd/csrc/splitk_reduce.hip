// Log-sum-exp merge of split-K partials.
//
// tiny-llm "优化", roadmap row FlashDecoding names long-context decode
// attention; the merge of independently normalised chunks is the identity
//   out = sum_i e^{lse_i - M} o_i / sum_i e^{lse_i - M},  M = max_i lse_i,
// with empty chunks (lse = -inf) weighing zero.
//
// One wave per (sequence, q head) row; each lane owns D/64 dimensions. The
// split pass records how many partials each (sequence, kv head) received;
// a sequence with no tokens gets zeros.
#include "launch.h"
#include "device_common.h"

namespace pa {

template <int D>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(ReduceArgs a) {
  constexpr int kPer = D / 64;                // dims per lane (1 or 2)
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= a.B * a.Hq) return;
  const int b = row / a.Hq;
  const int h = (row % a.Hq) / a.G;
  int L = a.context_lens[b];
  L = L < 0 ? 0 : (L > a.cap ? a.cap : L);
  int n = 0;
  if (L > 0) {
    n = a.ws_count[(long long)b * a.Hkv + h];
    n = n < 1 ? 1 : (n > a.S ? a.S : n);
  }
  const float* lse = a.ws_lse + (long long)row * a.S;
  const float* o = a.ws_o + (long long)row * a.S * D;

  float M = -INFINITY;
  for (int i = 0; i < n; ++i) M = fmaxf(M, lse[i]);
  float acc[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) acc[k] = 0.0f;
  float den = 0.0f;
  if (M != -INFINITY) {
    for (int i = 0; i < n; ++i) {
      const float li = lse[i];
      if (li == -INFINITY) continue;           // wave-uniform
      const float w = __builtin_amdgcn_exp2f((li - M) * kLog2e);
      den += w;
      const float* oi = o + (long long)i * D + lane * kPer;
      if constexpr (kPer == 2) {
        const float2 v = *reinterpret_cast<const float2*>(oi);
        acc[0] += w * v.x;
        acc[1] += w * v.y;
      } else {
        acc[0] += w * oi[0];
      }
    }
  }
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
  _Float16* dst = a.out + (long long)row * D + lane * kPer;
#pragma unroll
  for (int k = 0; k < kPer; ++k) dst[k] = (_Float16)(acc[k] * inv);
}

hipError_t launch_reduce(const ReduceArgs& a, int D, hipStream_t stream) {
  const unsigned grid = (unsigned)(((long long)a.B * a.Hq + 3) / 4);
  if (D == 64)
    hipLaunchKernelGGL((splitk_reduce_kernel<64>), grid, 256, 0, stream, a);
  else
    hipLaunchKernelGGL((splitk_reduce_kernel<128>), grid, 256, 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
