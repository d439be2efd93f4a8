// kv_append: scatter new tokens' K/V rows into their pages.
//
// tiny-llm "优化", roadmap row 分页 KV: appends write through the block
// table (scatter); section 5: the append position is a per-step device
// value. One-byte caches (fp8 e4m3fn, int8) quantise with per-kv-head scales
// ("TensorRT对Multi-Query Attention的专项优化支持", quantisation paragraph: K
// and V scaled apart).
//
// One thread handles two adjacent dimensions of one (token, kv head) row:
// it reads 4 bytes of k_new and of v_new and writes them (or their two
// one-byte codes) at the positions the page layout gives them: both K values
// sit in one 16-byte chunk; the two V values are 8 elements apart.
#include "launch.h"
#include "device_common.h"

namespace pa {

template <int D, int KV>
__global__ __launch_bounds__(256) void kv_append_kernel(KvAppendArgs a) {
  constexpr bool kByte = KV != kKvF16;
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
  const int esz = kByte ? 1 : 2;
  const long long tile = ((long long)page * a.Hkv + h) * a.bs * D * esz;
  store_kv_pair<D, KV>(a.k_pages + tile, a.v_pages + tile, slot, dp, kin, vin,
                       kByte ? a.k_scale[h] : 1.0f, kByte ? a.v_scale[h] : 1.0f);
}

// One decode step on: every live slot (position >= 0) moves its append
// position and its context length on by one token; a slot whose next
// position would leave the block table's capacity stops appending
// (position -1) and keeps its length.
__global__ __launch_bounds__(256) void advance_kernel(int32_t* lens, int32_t* positions,
                                                     int B, int cap) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= B) return;
  const int p = positions[b];
  if (p < 0) return;
  if (p + 1 >= cap) {
    positions[b] = -1;
    return;
  }
  positions[b] = p + 1;
  lens[b] = lens[b] + 1;
}

hipError_t launch_advance(int32_t* lens, int32_t* positions, int B, int cap,
                          hipStream_t stream) {
  hipLaunchKernelGGL(advance_kernel, (unsigned)((B + 255) / 256), 256, 0, stream, lens,
                     positions, B, cap);
  return hipGetLastError();
}

template <int D>
static void launch_d(const KvAppendArgs& a, int kv, unsigned grid, hipStream_t stream) {
  if (kv == kKvF8)
    hipLaunchKernelGGL((kv_append_kernel<D, kKvF8>), grid, 256, 0, stream, a);
  else if (kv == kKvI8)
    hipLaunchKernelGGL((kv_append_kernel<D, kKvI8>), grid, 256, 0, stream, a);
  else
    hipLaunchKernelGGL((kv_append_kernel<D, kKvF16>), grid, 256, 0, stream, a);
}

hipError_t launch_kv_append(const KvAppendArgs& a, int D, int kv,
                            hipStream_t stream) {
  const long long threads = (long long)a.num_tokens * a.Hkv * (D / 2);
  const unsigned grid = (unsigned)((threads + 255) / 256);
  if (D == 64) launch_d<64>(a, kv, grid, stream);
  else launch_d<128>(a, kv, grid, stream);
  return hipGetLastError();
}

}  // namespace pa
