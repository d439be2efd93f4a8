// Device helpers shared by the gfx950 kernels of the paged decode library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace pa {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 16x16x32 fp16 MFMA, fp32 accumulate. Operand layout on gfx950 (checked on
// the device): A row = lane % 16, B column = lane % 16, and the 8 values a
// lane holds are K-slots 8 * (lane / 16) + 0..7 for both A and B; the
// result holds column lane % 16, rows 4 * (lane / 16) + 0..3.
__device__ __forceinline__ f32x4 mfma_16x16x32(half8 a, half8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ half8 as_half8(u32x4 v) {
  return __builtin_bit_cast(half8, v);
}

// Two e4m3fn codes sitting in the low bytes of the two 16-bit halves of `t`
// become two fp16 values equal to code_value * 2^-8, exactly: the 4-bit
// exponent and 3-bit mantissa land in fp16's exponent/mantissa fields, so
// fp16's bias (15) versus e4m3's (7) scales every value, subnormals
// included, by 2^-8. Codes 0x7F/0xFF (NaN) come out as finite 1.875.
__device__ __forceinline__ uint32_t e4m3_pair_to_f16_pair(uint32_t t) {
  return ((t & 0x007F007Fu) << 7) | ((t & 0x00800080u) << 8);
}

// Four codes (one dword, byte i = code i) -> four fp16 (two dwords).
__device__ __forceinline__ u32x2 e4m3x4_to_f16x4(uint32_t w) {
  uint32_t lo = (w & 0xFFu) | ((w & 0xFF00u) << 8);
  uint32_t hi = ((w >> 16) & 0xFFu) | ((w >> 8) & 0xFF0000u);
  u32x2 r;
  r.x = e4m3_pair_to_f16_pair(lo);
  r.y = e4m3_pair_to_f16_pair(hi);
  return r;
}

// Eight codes (two dwords) -> one half8 operand (values scaled by 2^-8).
__device__ __forceinline__ half8 e4m3x8_to_half8(u32x2 w) {
  u32x2 a = e4m3x4_to_f16x4(w.x);
  u32x2 b = e4m3x4_to_f16x4(w.y);
  u32x4 r = {a.x, a.y, b.x, b.y};
  return as_half8(r);
}

// Two int8 codes in the low bytes of the two 16-bit halves of `t` become two
// fp16 values equal to the codes, exactly: with the byte's sign bit flipped
// (c + 128, 0..255) under the fp16 pattern of 1024 (0x6400) the half reads
// 1024 + c + 128, and subtracting 1152 leaves c (every integer below 2048 is
// an fp16 value, so both steps are exact).
__device__ __forceinline__ uint32_t i8_pair_to_f16_pair(uint32_t t) {
  const uint32_t biased = (t & 0x00FF00FFu) ^ 0x00800080u;
  half2v h = __builtin_bit_cast(half2v, biased | 0x64006400u);
  h = h - half2v{(_Float16)1152.0f, (_Float16)1152.0f};
  return __builtin_bit_cast(uint32_t, h);
}

// Eight int8 codes (two dwords) -> one half8 operand holding the codes.
__device__ __forceinline__ half8 i8x8_to_half8(u32x2 w) {
  auto lo = [](uint32_t x) { return i8_pair_to_f16_pair((x & 0xFFu) | ((x & 0xFF00u) << 8)); };
  auto hi = [](uint32_t x) {
    return i8_pair_to_f16_pair(((x >> 16) & 0xFFu) | ((x >> 8) & 0xFF0000u));
  };
  const u32x4 r = {lo(w.x), hi(w.x), lo(w.y), hi(w.y)};
  return as_half8(r);
}

// Eight one-byte codes -> fp16 operand: e4m3fn values times 2^-8, or int8
// values.
template <int KV>
__device__ __forceinline__ half8 codes8_to_half8(u32x2 w) {
  if constexpr (KV == kKvF8) return e4m3x8_to_half8(w);
  else return i8x8_to_half8(w);
}

// Factor that turns the fp16 operand of a code back into code units times
// the scale: 2^8 for e4m3fn (the bit placement divides by 2^8), 1 for int8.
template <int KV>
constexpr float code_unit() {
  return KV == kKvF8 ? 256.0f : 1.0f;
}

// float32 -> symmetric int8 code: round to nearest even, saturating at
// +-127 (the code -128 is never produced), NaN -> 0.
__device__ __forceinline__ uint32_t f32_to_i8(float y) {
  if (y != y) return 0u;
  float r = __builtin_rintf(y);
  r = r > 127.0f ? 127.0f : (r < -127.0f ? -127.0f : r);
  return (uint32_t)(int)r & 0xFFu;
}

// float32 -> OCP e4m3fn code, round to nearest even, saturating: written
// from the format definition (bias 7, 3 mantissa bits, max 448, min normal
// 2^-6, subnormal quantum 2^-9, NaN = S.1111.111).
__device__ __forceinline__ uint32_t f32_to_e4m3fn(float y) {
  uint32_t u = __float_as_uint(y);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return 0x7Fu;                  // NaN
  if (a >= 0x43E00000u) return sign | 0x7Eu;         // |y| >= 448 -> 448
  int e = (int)(a >> 23) - 127;
  if (e >= -6) {                                      // normal range
    uint32_t m = a & 0x7FFFFFu;
    uint32_t q = m >> 20;
    uint32_t rem = m & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) q += 1u;
    uint32_t ee = (uint32_t)(e + 7);
    if (q == 8u) { q = 0u; ee += 1u; }
    return sign | (ee << 3) | q;
  }
  // |y| < 2^-6: multiples of 2^-9; the scaling by 512 is exact
  float t = __uint_as_float(a) * 512.0f;
  uint32_t k = (uint32_t)__builtin_rintf(t);          // 0..8, 8 = 2^-6
  return sign | k;
}

// Store dims dp, dp+1 of one token's K and V rows (fp16 bits in kin / vin)
// at slot `slot` of the (page, head) tiles ktile / vtile, in the page
// layout: K rows of each 16-token block in 16-byte chunks with slots 4..7
// and 8..11 swapped (bits 2 and 3 of the slot exchanged), V as runs of 8
// tokens per dimension. One-byte tiles receive the codes of value / scale
// (IEEE fp32 division, then round to nearest even, saturating).
template <int D, int KV>
__device__ __forceinline__ void store_kv_pair(uint8_t* ktile, uint8_t* vtile,
                                              int slot, int dp, uint32_t kin,
                                              uint32_t vin, float ks, float vs) {
  constexpr bool FP8 = KV != kKvF16;                  // one-byte codes
  constexpr int X = FP8 ? 16 : 8;                     // elements per 16 B
  const int blk = slot >> 4, r = slot & 15;
  const int krow = (r & 3) | ((r & 4) << 1) | ((r & 8) >> 1);
  const int koff = ((blk * (D / X) + dp / X) * 16 + krow) * X + dp % X;
  const int voff = (((blk * (D / 16) + dp / 16) * 2 + (r >> 3)) * 16 + dp % 16) * 8 + (r & 7);
  if constexpr (!FP8) {
    *reinterpret_cast<uint32_t*>(ktile + koff * 2) = kin;
    uint16_t* vdst = reinterpret_cast<uint16_t*>(vtile) + voff;
    vdst[0] = (uint16_t)(vin & 0xFFFFu);
    vdst[8] = (uint16_t)(vin >> 16);
  } else {
    auto h2f = [](uint32_t bits) {
      return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
    };
    auto enc = [](float y) {
      if constexpr (KV == kKvF8) return f32_to_e4m3fn(y);
      else return f32_to_i8(y);
    };
    const uint32_t k0 = enc(h2f(kin & 0xFFFFu) / ks);
    const uint32_t k1 = enc(h2f(kin >> 16) / ks);
    const uint32_t v0 = enc(h2f(vin & 0xFFFFu) / vs);
    const uint32_t v1 = enc(h2f(vin >> 16) / vs);
    *reinterpret_cast<uint16_t*>(ktile + koff) = (uint16_t)(k0 | (k1 << 8));
    vtile[voff] = (uint8_t)v0;
    vtile[voff + 8] = (uint8_t)v1;
  }
}

// Cross-lane exchange inside a wave (lane ^ mask), via ds_swizzle-free
// bpermute: the address is in bytes.
__device__ __forceinline__ float xor_lanes(float v, int mask) {
  int lane = (int)__lane_id();
  return __int_as_float(
      __builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __float_as_int(v)));
}

// Max / sum over the four 16-lane rows of a wave: lanes l, l ^ 16, l ^ 32
// and l ^ 48 all end with the same value (sums in the same order, so the
// bits agree too). gfx950's row swaps work in the VALU: the 16-lane swap of
// a register with itself returns rows (0, 0, 2, 2) and (1, 1, 3, 3), the
// 32-lane swap the low and the high half twice, so each pair holds a
// lane's value and its partner's. (Measured against ds_bpermute exchanges:
// 0.1-0.7 us per launch faster.)
__device__ __forceinline__ float max_over_rows(float v) {
  const unsigned u = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m),
                                                  false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_over_rows(float v) {
  const unsigned u = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float s = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s),
                                                  false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Load of a value that every lane addresses alike (block-table entry,
// context length, scale) through the constant address space, so that it
// becomes a scalar load: it then waits on the scalar counter and never
// holds back the vector loads of K/V tiles. The memory must not change
// while the kernel runs (true for these inputs).
template <typename T>
__device__ __forceinline__ T load_uniform(const T* p) {
  return *reinterpret_cast<const __attribute__((address_space(4))) T*>(
      __builtin_bit_cast(unsigned long long, p));
}

// Device-scope relaxed atomic store / load of one float: on gfx950 a store
// written through to the device-coherent level and a load served from it
// (the per-XCD L2 caches are not coherent with each other).
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Two adjacent floats (8-byte aligned) in one device-scope atomic load.
__device__ __forceinline__ float2 load_coherent2(const float* p) {
  const unsigned long long v = __hip_atomic_load(
      reinterpret_cast<const unsigned long long*>(p), __ATOMIC_RELAXED,
      __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32)));
}

// Wait until every vector memory access this wave issued has completed
// (s_waitcnt vmcnt(0); the other counters are left alone).
__device__ __forceinline__ void wait_vector_memory() {
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Keeps the compiler from moving memory accesses across this point (it emits
// no instruction): the builtin wait above is not a barrier to the compiler.
__device__ __forceinline__ void compiler_fence() {
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ float read_lane(float v, int src) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(v)));
}

}  // namespace pa
