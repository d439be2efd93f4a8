// Internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

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
  const float* k_scale;      // fp8 only
  const float* v_scale;
  _Float16* out;             // single pass: [B, Hq, D]
  float* ws_o;               // split pass: [B, Hq, S, D]
  float* ws_lse;             // split pass: [B, Hq, S]
  int32_t* ws_count;         // split pass: [B, Hkv] partials per (b, h)
  int32_t* ws_sem;           // merged split pass: [B, Hkv] arrival counters
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

hipError_t launch_kv_append(const KvAppendArgs& a, int D, bool fp8,
                            hipStream_t stream);
// Returns hipErrorInvalidValue for a shape without a kernel instance.
hipError_t launch_attn(const AttnArgs& a, int D, int BS, bool fp8,
                       hipStream_t stream);
hipError_t launch_reduce(const ReduceArgs& a, int D, hipStream_t stream);

}  // namespace pa
