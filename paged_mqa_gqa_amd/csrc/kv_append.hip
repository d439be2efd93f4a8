// kv_append: scatter new tokens' K/V rows into their pages.
//
// tiny-llm "优化", roadmap row 分页 KV: appends write through the block
// table (scatter); section 5: the append position is a per-step device
// value. fp8 caches quantise with a per-kv-head scale ("TensorRT对Multi-Query
// Attention的专项优化支持", quantisation paragraph: K and V scaled apart).
//
// One thread handles two adjacent dimensions of one (token, kv head) row:
// it reads 4 bytes of k_new and of v_new and writes them (or their two fp8
// codes) at the positions the page layout gives them: both K values sit in
// one 16-byte chunk; the two V values are 8 elements apart.
#include "launch.h"
#include "device_common.h"

namespace pa {

template <int D, bool FP8>
__global__ __launch_bounds__(256) void kv_append_kernel(KvAppendArgs a) {
  constexpr int kPairs = D / 2;                      // threads per row
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long row = idx / kPairs;                // (token, head) index
  const int dp = (int)(idx % kPairs) * 2;            // first dimension
  if (row >= (long long)a.num_tokens * a.Hkv) return;
  const int tok = (int)(row / a.Hkv);
  const int h = (int)(row % a.Hkv);
  const int s = a.seq_ids ? a.seq_ids[tok] : tok;
  const int pos = a.positions[tok];
  if (s < 0 || s >= a.B || pos < 0 || pos >= a.max_blocks * a.bs) return;
  int page = a.block_table[(long long)s * a.max_blocks + pos / a.bs];
  page = page < 0 ? 0 : (page >= a.P ? a.P - 1 : page);
  const int slot = pos % a.bs;

  const uint32_t kin = *reinterpret_cast<const uint32_t*>(
      a.k_new + (row * D + dp) * 2);
  const uint32_t vin = *reinterpret_cast<const uint32_t*>(
      a.v_new + (row * D + dp) * 2);
  const int esz = FP8 ? 1 : 2;
  const long long tile = ((long long)page * a.Hkv + h) * a.bs * D * esz;
  store_kv_pair<D, FP8>(a.k_pages + tile, a.v_pages + tile, slot, dp, kin, vin,
                        FP8 ? a.k_scale[h] : 1.0f, FP8 ? a.v_scale[h] : 1.0f);
}

hipError_t launch_kv_append(const KvAppendArgs& a, int D, bool fp8,
                            hipStream_t stream) {
  const long long threads = (long long)a.num_tokens * a.Hkv * (D / 2);
  const unsigned grid = (unsigned)((threads + 255) / 256);
  if (D == 64) {
    if (fp8) hipLaunchKernelGGL((kv_append_kernel<64, true>), grid, 256, 0, stream, a);
    else     hipLaunchKernelGGL((kv_append_kernel<64, false>), grid, 256, 0, stream, a);
  } else {
    if (fp8) hipLaunchKernelGGL((kv_append_kernel<128, true>), grid, 256, 0, stream, a);
    else     hipLaunchKernelGGL((kv_append_kernel<128, false>), grid, 256, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace pa
