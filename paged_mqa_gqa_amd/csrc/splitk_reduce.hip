// Log-sum-exp merge of split-K partials.
//
// tiny-llm "优化", roadmap row FlashDecoding names long-context decode
// attention; the merge of independently normalised chunks is the identity
//   out = sum_i e^{lse_i - M} o_i / sum_i e^{lse_i - M},  M = max_i lse_i,
// with empty chunks (lse = -inf) weighing zero.
//
// One wave per (sequence, q head) row; each lane owns D/64 dimensions. The
// split pass records how many partials each (sequence, kv head) received;
// a sequence with no tokens gets zeros. The lane-parallel read of the lse
// values and the output rows of up to kGroup partials in flight together
// keep a row to a few memory round trips instead of two per partial; the
// partials are still folded one after the other in index order.
#include "launch.h"
#include "device_common.h"

namespace pa {

template <int D>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(ReduceArgs a) {
  constexpr int kPer = D / 64;                // dims per lane (1 or 2)
  constexpr int kGroup = 16;                  // partial rows loaded together
  const int row = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  if (row >= a.B * a.Hq) return;
  const int b = row / a.Hq;
  const int h = (row % a.Hq) / a.G;
  const float* lse = a.ws_lse + (long long)row * a.S;
  const float* o = a.ws_o + (long long)row * a.S * D + lane * kPer;

  // The partial count and the context length first (scalar loads issued
  // together); then the lse values and the output rows of the first kGroup
  // partials, all in flight at once.
  const int cnt = load_uniform(a.ws_count + (long long)b * a.Hkv + h);
  const int L = load_uniform(a.context_lens + b);
  const int n = (L <= 0 || a.cap <= 0) ? 0 : (cnt < 1 ? 1 : (cnt > a.S ? a.S : cnt));

  // Output rows of partials first .. first + kGroup - 1; slots past the
  // count repeat the last partial's row (no extra traffic, weight zero).
  auto load_rows = [&](float (&v)[kGroup][kPer], int first) {
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      const float* oi = o + (long long)min(first + j, max(n - 1, 0)) * D;
      if constexpr (kPer == 2) {
        const float2 t = *reinterpret_cast<const float2*>(oi);
        v[j][0] = t.x;
        v[j][1] = t.y;
      } else {
        v[j][0] = oi[0];
      }
    }
  };

  const float l0 = lane < n ? lse[lane] : -INFINITY;
  float v[kGroup][kPer];
  load_rows(v, 0);

  // M = max_i lse_i, lanes over partials
  float M = l0;
  for (int c = 64; c < n; c += 64) M = fmaxf(M, c + lane < n ? lse[c + lane] : -INFINITY);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) M = fmaxf(M, xor_lanes(M, m));

  float acc[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) acc[k] = 0.0f;
  float den = 0.0f;
  if (M != -INFINITY) {
    for (int c = 0; c < n; c += 64) {
      // weight of partial c + lane; an empty partial (lse = -inf) and a slot
      // past the count weigh zero, and their output rows are never used
      const float li = c == 0 ? l0 : (c + lane < n ? lse[c + lane] : -INFINITY);
      const float wl = li == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((li - M) * kLog2e);
      const int m = min(64, n - c);
      for (int j0 = 0; j0 < m; j0 += kGroup) {
        if (c + j0 > 0) load_rows(v, c + j0);
        // Branch-free fold in index order, so that every load above stays
        // in flight: slots past the chunk's last partial read lanes whose
        // weight is zero, and a zero weight folds in an exact zero whatever
        // the row holds.
#pragma unroll
        for (int j = 0; j < kGroup; ++j) {
          const float w = __int_as_float(
              __builtin_amdgcn_readlane(__float_as_int(wl), j0 + j));
          den += w;
#pragma unroll
          for (int k = 0; k < kPer; ++k)
            acc[k] = __builtin_fmaf(w, w != 0.0f ? v[j][k] : 0.0f, acc[k]);
        }
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
