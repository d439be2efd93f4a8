// Decode projection with M == 1 (up to 4 activation rows) over a transposed
// weight, and the load-time transpose that builds it.
//
// tiny-llm "优化", section 4: a decode step multiplies one activation row
// by a [K, N] weight; with the weight stored [N, K] the lanes computing one
// output read consecutive k, so every load is coalesced; the transposed copy
// is built once when the weights are loaded. Section 1: int8 weights with
// fp16 activations and symmetric per-group scales along k.
//
// Design (MI355X): the work is a stream of weight bytes (1 or 2 per
// multiply-add for one activation row), so it is bound by HBM, not by the
// matrix cores. Each wave owns kRows output rows; every lane reads 16-byte
// chunks of those rows (consecutive lanes, consecutive chunks: a wave-wide
// load is 1 KB of one row) and keeps kIter chunks per row in flight before
// it computes. The activation rows are staged once per workgroup in LDS and
// read back chunk by chunk. Products are summed in fp32 with v_dot2 (fp16
// pairs); int8 codes become fp16 exactly in registers and each 16-code chunk
// (inside one scale group) is scaled once. The 64 lanes' sums of a row are
// reduced across the wave at the end, and y is rounded to fp16.
#include "launch.h"
#include "device_common.h"

namespace pa {

namespace {

constexpr int kRows = 2;        // output rows per wave
constexpr int kIter = 8;        // chunks per row in flight per lane
constexpr int kWaves = 4;       // waves per workgroup

__device__ __forceinline__ float dot8(u32x4 w, u32x4 x, float acc) {
  const half2v* wh = reinterpret_cast<const half2v*>(&w);
  const half2v* xh = reinterpret_cast<const half2v*>(&x);
#pragma unroll
  for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_fdot2(wh[i], xh[i], acc, false);
  return acc;
}

// 16 int8 codes -> two chunks of 8 fp16 values equal to the codes.
__device__ __forceinline__ void i8x16_to_f16(u32x4 w, u32x4& lo, u32x4& hi) {
  auto pair_lo = [](uint32_t x) { return i8_pair_to_f16_pair((x & 0xFFu) | ((x & 0xFF00u) << 8)); };
  auto pair_hi = [](uint32_t x) {
    return i8_pair_to_f16_pair(((x >> 16) & 0xFFu) | ((x >> 8) & 0xFF0000u));
  };
  lo = u32x4{pair_lo(w.x), pair_hi(w.x), pair_lo(w.y), pair_hi(w.y)};
  hi = u32x4{pair_lo(w.z), pair_hi(w.z), pair_lo(w.w), pair_hi(w.w)};
}

// Sum over the 64 lanes (every lane gets it): inside each 16-lane row by
// DPP (swap neighbours, then pairs, then rotate the row by 4 and by 8),
// then across the rows with the row swaps. VALU only.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf,
                                                        false));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = dpp_add<0xB1>(v);     // quad_perm [1, 0, 3, 2]
  v = dpp_add<0x4E>(v);     // quad_perm [2, 3, 0, 1]
  v = dpp_add<0x124>(v);    // row_ror:4
  v = dpp_add<0x128>(v);    // row_ror:8
  return sum_over_rows(v);
}

}  // namespace

// x [M, K] fp16, wt [N, K] (fp16, or int8 codes with scales_t [N, K/group]),
// y [M, N] fp16.
template <bool I8, int M>
__global__ __launch_bounds__(64 * kWaves) void gemm_m1_kernel(GemmArgs a) {
  extern __shared__ u32x4 xs[];                 // [M][K / 8] chunks of 8 fp16
  constexpr int E = I8 ? 16 : 8;                // weights per 16-byte chunk
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int K = a.K;
  const int xchunks = K / 8;

  // stage the activation rows in LDS (16 bytes per thread per pass)
  const u32x4* xg = reinterpret_cast<const u32x4*>(a.x);
  for (int i = threadIdx.x; i < M * xchunks; i += 64 * kWaves) xs[i] = xg[i];
  __syncthreads();

  const long long row0 = ((long long)blockIdx.x * kWaves + wave) * kRows;
  if (row0 >= a.N) return;
  const int wchunks = K / E;                    // 16-byte chunks per weight row
  const long long row_bytes = (long long)K * (I8 ? 1 : 2);
  const int groups = I8 ? K / a.group : 1;

  float acc[kRows][M];
#pragma unroll
  for (int r = 0; r < kRows; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;

  for (int c0 = 0; c0 < wchunks; c0 += 64 * kIter) {
    // 64-chunk steps of this pass that hold any of the row (the same for
    // every lane): loads past them are not issued
    const int steps = min(kIter, (wchunks - c0 + 63) / 64);
    u32x4 w[kRows][kIter];
    float sc[kRows][kIter];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const long long row = min(row0 + r, (long long)a.N - 1);
      const u32x4* wr = reinterpret_cast<const u32x4*>(a.wt + row * row_bytes);
#pragma unroll
      for (int j = 0; j < kIter; ++j) {
        if (j >= steps) break;
        // lanes past the row's end inside the last step load its last chunk
        // (in bounds) and are skipped by the compute loop
        const int ci = min(c0 + j * 64 + lane, wchunks - 1);
        w[r][j] = __builtin_nontemporal_load(wr + ci);
        if constexpr (I8) sc[r][j] = a.scales_t[row * groups + (ci * E) / a.group];
      }
    }
#pragma unroll
    for (int j = 0; j < kIter; ++j) {
      if (j >= steps) break;
      const int ci = c0 + j * 64 + lane;
      if (ci >= wchunks) continue;
      if constexpr (I8) {
        u32x4 lo[kRows], hi[kRows];
#pragma unroll
        for (int r = 0; r < kRows; ++r) i8x16_to_f16(w[r][j], lo[r], hi[r]);
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const u32x4 x0 = xs[m * xchunks + 2 * ci];
          const u32x4 x1 = xs[m * xchunks + 2 * ci + 1];
#pragma unroll
          for (int r = 0; r < kRows; ++r) {
            const float part = dot8(hi[r], x1, dot8(lo[r], x0, 0.0f));
            acc[r][m] = __builtin_fmaf(part, sc[r][j], acc[r][m]);
          }
        }
      } else {
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const u32x4 xv = xs[m * xchunks + ci];
#pragma unroll
          for (int r = 0; r < kRows; ++r) acc[r][m] = dot8(w[r][j], xv, acc[r][m]);
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kRows; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float s = wave_sum(acc[r][m]);
      if (lane == 0 && row0 + r < a.N) a.y[(long long)m * a.N + row0 + r] = (_Float16)s;
    }
}

// in [R, C] -> out [C, R], elements of T, through 64 x 64 tiles in LDS
// (reads along C and writes along R are both coalesced).
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* in, T* out, int R, int C) {
  __shared__ T tile[64][65];
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int r = r0 + i, c = c0 + tx;
    if (r < R && c < C) tile[i][tx] = in[(long long)r * C + c];
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int c = c0 + i, r = r0 + tx;
    if (r < R && c < C) out[(long long)c * R + r] = tile[tx][i];
  }
}

template <bool I8>
static hipError_t launch_m(const GemmArgs& a, hipStream_t st) {
  const unsigned grid = (unsigned)((a.N + kWaves * kRows - 1) / (kWaves * kRows));
  const size_t lds = (size_t)a.M * a.K * 2;
  switch (a.M) {
    case 1: hipLaunchKernelGGL((gemm_m1_kernel<I8, 1>), grid, 64 * kWaves, lds, st, a); break;
    case 2: hipLaunchKernelGGL((gemm_m1_kernel<I8, 2>), grid, 64 * kWaves, lds, st, a); break;
    case 3: hipLaunchKernelGGL((gemm_m1_kernel<I8, 3>), grid, 64 * kWaves, lds, st, a); break;
    case 4: hipLaunchKernelGGL((gemm_m1_kernel<I8, 4>), grid, 64 * kWaves, lds, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_m1(const GemmArgs& a, bool int8, hipStream_t st) {
  return int8 ? launch_m<true>(a, st) : launch_m<false>(a, st);
}

hipError_t launch_transpose(const void* in, void* out, int R, int C, int elem_bytes,
                            hipStream_t st) {
  const dim3 grid((unsigned)((C + 63) / 64), (unsigned)((R + 63) / 64));
  switch (elem_bytes) {
    case 1:
      hipLaunchKernelGGL(transpose_kernel<uint8_t>, grid, 256, 0, st,
                         static_cast<const uint8_t*>(in), static_cast<uint8_t*>(out), R, C);
      break;
    case 2:
      hipLaunchKernelGGL(transpose_kernel<uint16_t>, grid, 256, 0, st,
                         static_cast<const uint16_t*>(in), static_cast<uint16_t*>(out), R, C);
      break;
    case 4:
      hipLaunchKernelGGL(transpose_kernel<uint32_t>, grid, 256, 0, st,
                         static_cast<const uint32_t*>(in), static_cast<uint32_t*>(out), R, C);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
