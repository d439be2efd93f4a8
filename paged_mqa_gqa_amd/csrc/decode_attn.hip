// Paged MQA/GQA decode attention for gfx950.
//
// What it computes: for each sequence b and query head j of kv group h,
// softmax(scale * q . K_h^T) . V_h over the sequence's tokens, K_h/V_h read
// page by page through the block table ("TensorRT对Multi-Query Attention的
// 专项优化支持": MHA/MQA formulas, decode re-reads the cached K/V, K/V in
// fixed-length pages, QK^T and AV as matrix products over the shared K/V;
// tiny-llm "优化": GQA in section 3, paged gather in roadmap row 分页 KV,
// long-context decode in roadmap row FlashDecoding).
//
// Design (MI355X / gfx950):
//  * One workgroup per (sequence, kv head, split); its waves are HW groups
//    of head blocks (16 q heads per MFMA block, NH blocks per wave) times
//    TW token-parallel waves. Every wave streams its own 32-token tiles
//    straight from HBM into MFMA operand registers (16-byte loads; a K row
//    is 64 contiguous bytes per lane group, a V page column 16 bytes), with
//    the next tile's loads in flight while the current tile is computed.
//  * QK^T: K tile as the A operand (16 tokens x 32 dims), the group's q
//    heads as B (32 dims x 16 heads). The 16x16 result holds, per lane,
//    scores of one head for 4 tokens; two such blocks give the 8 tokens that
//    the P.V product needs in the same lane, so P never leaves registers.
//  * Online softmax in base 2 (scale * log2 e folded into the scores): the
//    running max per head is reduced across the four 16-lane groups, the
//    running sum stays per lane until the end.
//  * P.V: P (16 heads x 32 tokens, fp16) as A, V page columns (32 tokens x
//    16 dims) as B, accumulated in fp32.
//  * Page ids of the workgroup's range are staged once in LDS (chunks of
//    kMaxPages) and clamped into the pool; masked tail tokens re-read a valid
//    row and are zeroed by select, so NaN in unused slots never leaks.
//  * fp8 e4m3fn K/V are expanded to fp16 in registers by bit placement
//    (value * 2^-8, exact); 2^8 and the per-head scales fold into the score
//    scale and the final output scale.
//  * Token-parallel waves merge through LDS with the log-sum-exp rule; a
//    split writes (o, lse) for the separate merge kernel.
#include "launch.h"
#include "device_common.h"
#include <type_traits>

namespace pa {

constexpr int kTile = 32;       // tokens per tile
constexpr int kMaxPages = 512;  // page ids staged in LDS per chunk

template <int D, int BS, bool FP8>
struct Geo {
  static constexpr int kEsz = FP8 ? 1 : 2;
  static constexpr int kRowBytes = D * kEsz;          // one K row
  static constexpr int kPageBytes = BS * D * kEsz;    // one (page, head) tile
  static constexpr int kQkMfma = D / 32;              // per 16-token block
  static constexpr int kKLoads = kRowBytes / 64;      // 16 B loads per K row
  static constexpr int kPvMfma = D / 16;              // per 32-token tile
};

// First dimension of the 8 K-slots that lane group g (= lane / 16) holds in
// QK MFMA number jj. fp16: a 16 B K load covers one MFMA; fp8: a 16 B load
// covers 16 dims, i.e. two MFMAs.
template <bool FP8>
__device__ __forceinline__ int kslot_dim(int jj, int g) {
  return FP8 ? 64 * (jj >> 1) + 16 * g + 8 * (jj & 1) : 32 * jj + 8 * g;
}

template <int D, int BS, bool FP8>
struct TileRegs {
  using G = Geo<D, BS, FP8>;
  using VT = typename std::conditional<FP8, u32x2, u32x4>::type;
  u32x4 k[2][G::kKLoads];
  VT v[G::kPvMfma];
};

template <int D, int BS, bool FP8, int NH, int NWH, int TW>
__global__ __launch_bounds__(64 * NWH * TW) void decode_attn_kernel(AttnArgs a) {
  using Gm = Geo<D, BS, FP8>;
  using Tile = TileRegs<D, BS, FP8>;
  constexpr int kHeadsPerWg = NWH * NH * 16;

  __shared__ int sm_pages[kMaxPages];
  __shared__ float sm_m[TW][kHeadsPerWg];
  __shared__ float sm_l[TW][kHeadsPerWg];
  __shared__ float sm_acc[TW > 1 ? TW - 1 : 1][kHeadsPerWg][D];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int hw = wave % NWH;           // head-parallel index
  const int tw = wave / NWH;           // token-parallel index
  const int mrow = lane & 15;          // A row / B col / result col
  const int lg = lane >> 4;            // K-slot group, result row group

  const int bid = blockIdx.x;
  const int s = bid % a.S;
  const int h = (bid / a.S) % a.Hkv;
  const int b = bid / (a.S * a.Hkv);

  int L = a.context_lens[b];
  const int cap = a.max_blocks * BS;
  L = L < 0 ? 0 : (L > cap ? cap : L);
  int start = 0, end = L;
  if (a.split) {
    const int chunk = (L + a.S - 1) / a.S;
    const int C = BS * ((chunk + BS - 1) / BS);
    start = min(s * C, L);
    end = min(start + C, L);
  }

  // softmax scale in base 2; fp8 values carry a 2^-8 factor
  float sl = a.scale_log2;
  float oscale = 1.0f;
  if constexpr (FP8) {
    sl *= a.k_scale[h] * 256.0f;
    oscale = a.v_scale[h] * 256.0f;
  }

  // ---- q heads of this wave as B operands -------------------------------
  half8 qop[NH][Gm::kQkMfma];
#pragma unroll
  for (int hb = 0; hb < NH; ++hb) {
    const int gh = (hw * NH + hb) * 16 + mrow;     // head within the group
    const bool ok = gh < a.G;
    const _Float16* qrow = a.q + ((long long)b * a.Hq + h * a.G + (ok ? gh : 0)) * D;
#pragma unroll
    for (int jj = 0; jj < Gm::kQkMfma; ++jj) {
      u32x4 raw = *reinterpret_cast<const u32x4*>(qrow + kslot_dim<FP8>(jj, lg));
      if (!ok) raw = u32x4{0u, 0u, 0u, 0u};
      qop[hb][jj] = as_half8(raw);
    }
  }

  float mrun[NH], lrun[NH];
  f32x4 acc[NH][Gm::kPvMfma];
#pragma unroll
  for (int hb = 0; hb < NH; ++hb) {
    mrun[hb] = -INFINITY;
    lrun[hb] = 0.0f;
#pragma unroll
    for (int jd = 0; jd < Gm::kPvMfma; ++jd) acc[hb][jd] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const uint8_t* kbase = a.k_pages + (long long)h * Gm::kPageBytes;
  const uint8_t* vbase = a.v_pages + (long long)h * Gm::kPageBytes;
  const long long page_stride = (long long)a.Hkv * Gm::kPageBytes;
  const int* bt_row = a.block_table + (long long)b * a.max_blocks;

  for (int cs = start; cs < end; cs += kMaxPages * BS) {
    const int ce = min(end, cs + kMaxPages * BS);
    const int np = (ce - cs + BS - 1) / BS;
    __syncthreads();   // previous chunk's ids are no longer read
    for (int i = threadIdx.x; i < np; i += blockDim.x) {
      int p = bt_row[cs / BS + i];
      sm_pages[i] = p < 0 ? 0 : (p >= a.P ? a.P - 1 : p);
    }
    __syncthreads();
    const int ntiles = (ce - cs + kTile - 1) / kTile;

    // Issue the loads of tile k into t.
    auto load_tile = [&](Tile& t, int k) {
      const int ts = cs + k * kTile;
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int tt = 8 * (mrow >> 2) + 4 * r + (mrow & 3);
        const int tok = min(ts + tt, ce - 1);
        const int page = sm_pages[(tok - cs) / BS];
        const uint8_t* row = kbase + page * page_stride +
                             (tok % BS) * Gm::kRowBytes + 16 * lg;
#pragma unroll
        for (int jl = 0; jl < Gm::kKLoads; ++jl)
          t.k[r][jl] = *reinterpret_cast<const u32x4*>(row + 64 * jl);
      }
      int tv = ts + 8 * lg;
      if (tv >= ce) tv = (ce - 1) & ~7;
      const int vpage = sm_pages[(tv - cs) / BS];
      const uint8_t* col = vbase + vpage * page_stride +
                           (long long)mrow * BS * Gm::kEsz + (tv % BS) * Gm::kEsz;
#pragma unroll
      for (int jd = 0; jd < Gm::kPvMfma; ++jd)
        t.v[jd] = *reinterpret_cast<const typename Tile::VT*>(
            col + (long long)jd * 16 * BS * Gm::kEsz);
    };

    // Consume tile k held in t.
    auto compute_tile = [&](const Tile& t, int k) {
      const int ts = cs + k * kTile;
      const bool tail = ts + kTile > ce;
      half8 kop[2][Gm::kQkMfma];
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int jj = 0; jj < Gm::kQkMfma; ++jj) {
          if constexpr (FP8) {
            const u32x4 w = t.k[r][jj >> 1];
            const u32x2 half = (jj & 1) ? u32x2{w.z, w.w} : u32x2{w.x, w.y};
            kop[r][jj] = e4m3x8_to_half8(half);
          } else {
            kop[r][jj] = as_half8(t.k[r][jj]);
          }
        }
      half8 vop[Gm::kPvMfma];
      const int nv = ce - (ts + 8 * lg);   // valid tokens of this lane's 8
#pragma unroll
      for (int jd = 0; jd < Gm::kPvMfma; ++jd) {
        if constexpr (FP8) vop[jd] = e4m3x8_to_half8(t.v[jd]);
        else vop[jd] = as_half8(t.v[jd]);
        if (tail) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (e >= nv) vop[jd][e] = (_Float16)0.0f;
        }
      }
#pragma unroll
      for (int hb = 0; hb < NH; ++hb) {
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int jj = 0; jj < Gm::kQkMfma; ++jj) {
          s0 = mfma_16x16x32(kop[0][jj], qop[hb][jj], s0);
          s1 = mfma_16x16x32(kop[1][jj], qop[hb][jj], s1);
        }
        // element e of this lane = token 8*lg + e of the tile
        float sv[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sv[i] = s0[i] * sl;
          sv[4 + i] = s1[i] * sl;
        }
        if (tail) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (e >= nv) sv[e] = -INFINITY;
        }
        float mt = sv[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) mt = fmaxf(mt, sv[e]);
        mt = fmaxf(mt, xor_lanes(mt, 16));
        mt = fmaxf(mt, xor_lanes(mt, 32));
        const float mn = fmaxf(mrun[hb], mt);
        const float alpha = __builtin_amdgcn_exp2f(mrun[hb] - mn);
        mrun[hb] = mn;
        float ps = 0.0f;
        half8 pop;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = __builtin_amdgcn_exp2f(sv[e] - mn);
          ps += p;
          pop[e] = (_Float16)p;
        }
        lrun[hb] = lrun[hb] * alpha + ps;
        // result rows 4*lg+i belong to head 4*lg+i: fetch that head's alpha
        if (__any(alpha != 1.0f)) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float ai = read_lane(alpha, 4 * lg + i);
#pragma unroll
            for (int jd = 0; jd < Gm::kPvMfma; ++jd) acc[hb][jd][i] *= ai;
          }
        }
#pragma unroll
        for (int jd = 0; jd < Gm::kPvMfma; ++jd)
          acc[hb][jd] = mfma_16x16x32(pop, vop[jd], acc[hb][jd]);
      }
    };

    Tile ta, tb;
    int k = tw;
    if (k < ntiles) load_tile(ta, k);
    while (k < ntiles) {
      if (k + TW < ntiles) load_tile(tb, k + TW);
      compute_tile(ta, k);
      k += TW;
      if (k >= ntiles) break;
      if (k + TW < ntiles) load_tile(ta, k + TW);
      compute_tile(tb, k);
      k += TW;
    }
  }

  // ---- per-head totals: sum the per-lane partial sums over lane groups ---
#pragma unroll
  for (int hb = 0; hb < NH; ++hb) {
    lrun[hb] += xor_lanes(lrun[hb], 16);
    lrun[hb] += xor_lanes(lrun[hb], 32);
  }

  // ---- merge the token-parallel waves (log-sum-exp) ----------------------
  if (lg == 0) {
#pragma unroll
    for (int hb = 0; hb < NH; ++hb) {
      sm_m[tw][(hw * NH + hb) * 16 + mrow] = mrun[hb];
      sm_l[tw][(hw * NH + hb) * 16 + mrow] = lrun[hb];
    }
  }
  __syncthreads();
  // weight of this wave and totals for result rows (heads 4*lg + i)
  float wown[NH][4], ltot[NH][4], mtot[NH][4];
#pragma unroll
  for (int hb = 0; hb < NH; ++hb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = (hw * NH + hb) * 16 + 4 * lg + i;
      float M = -INFINITY;
#pragma unroll
      for (int t = 0; t < TW; ++t) M = fmaxf(M, sm_m[t][hh]);
      float Lsum = 0.0f;
      if (M != -INFINITY) {
#pragma unroll
        for (int t = 0; t < TW; ++t)
          Lsum += sm_l[t][hh] * __builtin_amdgcn_exp2f(sm_m[t][hh] - M);
      }
      wown[hb][i] = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(sm_m[tw][hh] - M);
      ltot[hb][i] = Lsum;
      mtot[hb][i] = M;
    }
  if constexpr (TW > 1) {
    if (tw > 0) {
#pragma unroll
      for (int hb = 0; hb < NH; ++hb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int hh = (hw * NH + hb) * 16 + 4 * lg + i;
          if (hh < a.G) {
#pragma unroll
            for (int jd = 0; jd < Gm::kPvMfma; ++jd)
              sm_acc[tw - 1][hh][16 * jd + mrow] = acc[hb][jd][i] * wown[hb][i];
          }
        }
    }
    __syncthreads();
    if (tw > 0) return;
  }

  // ---- wave tw == 0 writes the result ------------------------------------
#pragma unroll
  for (int hb = 0; hb < NH; ++hb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = (hw * NH + hb) * 16 + 4 * lg + i;
      if (hh >= a.G) continue;
      const int hq = h * a.G + hh;
      const float Lsum = ltot[hb][i];
      const float inv = Lsum > 0.0f ? oscale / Lsum : 0.0f;
      float vals[Gm::kPvMfma];
#pragma unroll
      for (int jd = 0; jd < Gm::kPvMfma; ++jd) {
        float v = acc[hb][jd][i] * wown[hb][i];
#pragma unroll
        for (int t = 1; t < TW; ++t) v += sm_acc[t - 1][hh][16 * jd + mrow];
        vals[jd] = v * inv;
      }
      if (a.split) {
        const long long row = ((long long)b * a.Hq + hq) * a.S + s;
        float* o = a.ws_o + row * D;
#pragma unroll
        for (int jd = 0; jd < Gm::kPvMfma; ++jd) o[16 * jd + mrow] = vals[jd];
        if (mrow == 0)
          a.ws_lse[row] = Lsum > 0.0f
                              ? (mtot[hb][i] + __builtin_amdgcn_logf(Lsum)) * kLn2
                              : -INFINITY;
      } else {
        _Float16* o = a.out + ((long long)b * a.Hq + hq) * D;
#pragma unroll
        for (int jd = 0; jd < Gm::kPvMfma; ++jd) o[16 * jd + mrow] = (_Float16)vals[jd];
      }
    }
}

// ---------------------------------------------------------------------------
// Instances: head_dim {64, 128} x block_size {16, 32, 64} x {fp16, fp8} x
// group-size class. Heads per workgroup: NWH * NH * 16.
template <int D, int BS, bool FP8>
static hipError_t launch_group(const AttnArgs& a, hipStream_t st) {
  const unsigned grid = (unsigned)((long long)a.B * a.Hkv * a.S);
  if (a.G <= 16) {
    hipLaunchKernelGGL((decode_attn_kernel<D, BS, FP8, 1, 1, 4>), grid, 256, 0, st, a);
  } else if (a.G <= 32) {
    hipLaunchKernelGGL((decode_attn_kernel<D, BS, FP8, 2, 1, 4>), grid, 256, 0, st, a);
  } else if (a.G <= 64) {
    hipLaunchKernelGGL((decode_attn_kernel<D, BS, FP8, 2, 2, 2>), grid, 256, 0, st, a);
  } else if (a.G <= 96) {
    hipLaunchKernelGGL((decode_attn_kernel<D, BS, FP8, 3, 2, 2>), grid, 256, 0, st, a);
  } else if (a.G <= 128) {
    hipLaunchKernelGGL((decode_attn_kernel<D, BS, FP8, 4, 2, 1>), grid, 128, 0, st, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D, bool FP8>
static hipError_t launch_bs(const AttnArgs& a, int BS, hipStream_t st) {
  switch (BS) {
    case 16: return launch_group<D, 16, FP8>(a, st);
    case 32: return launch_group<D, 32, FP8>(a, st);
    case 64: return launch_group<D, 64, FP8>(a, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attn(const AttnArgs& a, int D, int BS, bool fp8, hipStream_t st) {
  if (D == 64) return fp8 ? launch_bs<64, true>(a, BS, st) : launch_bs<64, false>(a, BS, st);
  if (D == 128) return fp8 ? launch_bs<128, true>(a, BS, st) : launch_bs<128, false>(a, BS, st);
  return hipErrorInvalidValue;
}

}  // namespace pa
