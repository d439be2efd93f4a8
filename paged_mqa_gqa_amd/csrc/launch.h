// Internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Cache element kinds: fp16 values, or one-byte codes (fp8 e4m3fn, int8)
// with a per-kv-head fp32 scale for K and one for V.
enum KvKind : int { kKvF16 = 0, kKvF8 = 1, kKvI8 = 2 };

// The split pass runs a persistent grid of kStreamGrid workgroups with at
// most 8 waves each, so at most kMaxStreamWorkers workers.
constexpr int kStreamGrid = 256;
constexpr int kMaxStreamWorkers = kStreamGrid * 8;

struct KvAppendArgs {
  const uint8_t* k_new;      // fp16 [T, Hkv, D]
  const uint8_t* v_new;
  const int32_t* seq_ids;    // may be null: token i -> sequence i
  const int32_t* positions;
  const int32_t* block_table;
  const float* k_scale;
  const float* v_scale;
  uint8_t* k_pages;
  uint8_t* v_pages;
  int num_tokens, B, Hkv, bs, P, max_blocks;
};

struct AttnArgs {
  const _Float16* q;         // [B, Hq, D]
  const uint8_t* k_pages;    // [P, Hkv, BS, D] elements
  const uint8_t* v_pages;    // [P, Hkv, D, BS] elements
  const int32_t* block_table;
  const int32_t* context_lens;
  const float* k_scale;      // one-byte caches only
  const float* v_scale;
  _Float16* out;             // single pass: [B, Hq, D]
  float* ws_o;               // split pass: [B, Hq, S, D]
  float* ws_lse;             // split pass: [B, Hq, S]
  int32_t* ws_count;         // split pass: [B, Hkv] partials per (b, h)
  int32_t* ws_sem;           // merged split pass: [kMaxStreamWorkers] arrival
                             // counters, one per pair, at its first worker
  const _Float16* k_new;     // fused append (else null): [B, Hkv, D] fp16
  const _Float16* v_new;
  const int32_t* positions;  // [B] slot of the new token
  float scale_log2;          // scale * log2(e)
  int B, Hq, Hkv, G, P, max_blocks, S;
  int mode;                  // 0: single pass -> out; 1: one split per
                             // (b, h) -> slot 0; 2: stream-K split pass;
                             // 3: stream-K split pass merged in-kernel
};

struct ReduceArgs {
  const float* ws_o;
  const float* ws_lse;
  const int32_t* ws_count;
  const int32_t* context_lens;
  _Float16* out;
  int B, Hq, Hkv, G, S, cap;  // cap = max_blocks * block_size
};

// Decode projection, M == 1 path (gemm_m1.hip).
struct GemmArgs {
  const _Float16* x;         // [M, K]
  const uint8_t* wt;         // [N, K] fp16 or int8 codes
  const float* scales_t;     // [N, K / group] (int8 weights only)
  _Float16* y;               // [M, N]
  int M, N, K, group;
};

hipError_t launch_gemm_m1(const GemmArgs& a, bool int8, hipStream_t stream);
hipError_t launch_transpose(const void* in, void* out, int R, int C, int elem_bytes,
                            hipStream_t stream);

// kv: KvKind of the cache (device_common.h: 0 fp16, 1 fp8 e4m3fn, 2 int8).
hipError_t launch_kv_append(const KvAppendArgs& a, int D, int kv,
                            hipStream_t stream);
hipError_t launch_advance(int32_t* lens, int32_t* positions, int B, int cap,
                          hipStream_t stream);
// Attention kernels of one (cache kind, head_dim) pair; each pair is
// compiled in an object file of its own.
template <int KV, int D>
hipError_t launch_attn_inst(const AttnArgs& a, int BS, hipStream_t stream);
// Returns hipErrorInvalidValue for a shape without a kernel instance.
hipError_t launch_attn(const AttnArgs& a, int D, int BS, int kv,
                       hipStream_t stream);
hipError_t launch_reduce(const ReduceArgs& a, int D, hipStream_t stream);

}  // namespace pa
