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
//  * A workgroup's waves are NWH groups of head blocks (16 q heads per MFMA
//    block, NH blocks per wave) times TW token-parallel waves. Every wave
//    streams its own 32-token tiles straight from HBM into MFMA operand
//    registers, the next tile's loads in flight while the current tile is
//    computed. The page layout stores each 16-token block in operand order,
//    so every wave-wide load reads one contiguous run (1 KB per K load,
//    512 B per fp16 V load) and the L1 sees full 64-byte requests.
//  * QK^T: a 16-token K block as the A operand (16 tokens x 32 dims), the
//    group's q heads as B (32 dims x 16 heads). The 16x16 result holds, per
//    lane, scores of one head for 4 tokens; the two blocks of a tile give
//    the 8 tokens that the P.V product needs in the same lane, so P never
//    leaves registers.
//  * Online softmax in base 2 (scale * log2 e folded into the scores): the
//    running max per head is reduced across the four 16-lane groups, the
//    running sum stays per lane until a flush.
//  * P.V: P (16 heads x 32 tokens, fp16) as A, V page columns (32 tokens x
//    16 dims) as B, accumulated in fp32.
//  * Page ids of a token range are staged in LDS (chunks of kMaxPages) and
//    clamped into the pool; masked tail tokens re-read a valid row and are
//    zeroed by select, so NaN in unused slots never leaks.
//  * fp8 e4m3fn K/V are expanded to fp16 in registers by bit placement
//    (value * 2^-8, exact); 2^8 and the per-head scales fold into the score
//    scale and the final output scale.
//  * Two schedules. Single pass: one workgroup per (sequence, kv head).
//    Split pass: a persistent grid; the tiles of all (sequence, kv head)
//    contexts, laid end to end, are cut into equal contiguous shares, one
//    per workgroup (the stream-K decomposition), so ragged batches balance
//    exactly; every (sequence, kv head) segment a workgroup covers becomes
//    one log-sum-exp partial, merged by the separate reduce kernel.
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
  // V of one 16-token block: 4 tokens of one dimension per lane
  using VT = typename std::conditional<FP8, uint32_t, u32x2>::type;
  u32x4 k[2][G::kKLoads];      // [16-token block][16 B chunk group]
  VT v[2][G::kPvMfma];         // [16-token block][16-dim group]
};

template <int NH, int NWH, int TW, int D>
struct SharedMem {
  static constexpr int kHeads = NWH * NH * 16;
  int pages[kMaxPages];
  float m[TW][kHeads];
  float l[TW][kHeads];
  float acc[TW > 1 ? TW - 1 : 1][kHeads][D];
  int scan[256];
  int loc[4];
};

template <int D, int BS, bool FP8, int NH, int NWH, int TW>
struct Decoder {
  using Gm = Geo<D, BS, FP8>;
  using Tile = TileRegs<D, BS, FP8>;
  using Smem = SharedMem<NH, NWH, TW, D>;

  const AttnArgs& a;
  Smem& sm;
  int lane, wave, hw, tw, mrow, lg;
  float sl, oscale;
  half8 qop[NH][Gm::kQkMfma];
  float mrun[NH], lrun[NH];
  f32x4 acc[NH][Gm::kPvMfma];

  __device__ __forceinline__ Decoder(const AttnArgs& args, Smem& s) : a(args), sm(s) {
    lane = threadIdx.x & 63;
    wave = threadIdx.x >> 6;
    hw = wave % NWH;
    tw = wave / NWH;
    mrow = lane & 15;
    lg = lane >> 4;
  }

  // q rows of kv group h of sequence b as B operands; softmax state reset.
  __device__ __forceinline__ void begin(int b, int h) {
    sl = a.scale_log2;
    oscale = 1.0f;
    if constexpr (FP8) {
      sl *= a.k_scale[h] * 256.0f;
      oscale = a.v_scale[h] * 256.0f;
    }
#pragma unroll
    for (int hb = 0; hb < NH; ++hb) {
      const int gh = (hw * NH + hb) * 16 + mrow;
      const bool ok = gh < a.G;
      const _Float16* qrow = a.q + ((long long)b * a.Hq + h * a.G + (ok ? gh : 0)) * D;
#pragma unroll
      for (int jj = 0; jj < Gm::kQkMfma; ++jj) {
        u32x4 raw = *reinterpret_cast<const u32x4*>(qrow + kslot_dim<FP8>(jj, lg));
        if (!ok) raw = u32x4{0u, 0u, 0u, 0u};
        qop[hb][jj] = as_half8(raw);
      }
      mrun[hb] = -INFINITY;
      lrun[hb] = 0.0f;
#pragma unroll
      for (int jd = 0; jd < Gm::kPvMfma; ++jd) acc[hb][jd] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }

  // Attend to tokens [start, end) of (b, h). Every wave of the workgroup
  // must call this with the same arguments (it synchronises the group).
  __device__ __forceinline__ void run(int b, int h, int start, int end) {
    const uint8_t* kbase = a.k_pages + (long long)h * Gm::kPageBytes;
    const uint8_t* vbase = a.v_pages + (long long)h * Gm::kPageBytes;
    const long long page_stride = (long long)a.Hkv * Gm::kPageBytes;
    const int* bt_row = a.block_table + (long long)b * a.max_blocks;

    for (int cs = start; cs < end; cs += kMaxPages * BS) {
      const int ce = min(end, cs + kMaxPages * BS);
      const int p0 = cs / BS;
      const int np = (ce - 1) / BS - p0 + 1;
      __syncthreads();   // previous chunk's ids (and flush buffers) are free
      for (int i = threadIdx.x; i < np; i += blockDim.x) {
        int p = bt_row[p0 + i];
        sm.pages[i] = p < 0 ? 0 : (p >= a.P ? a.P - 1 : p);
      }
      __syncthreads();
      const int ntiles = (ce - cs + kTile - 1) / kTile;

      // Issue the loads of tile k (two 16-token blocks). A block that lies
      // wholly past the end re-reads the last block that has tokens (in
      // bounds; its values are masked).
      auto load_tile = [&](Tile& t, int k) {
        const int ts = cs + k * kTile;
        const int last_blk = (ce - 1) & ~15;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const int tb = min(ts + 16 * r, last_blk);
          const int page = sm.pages[tb / BS - p0];
          const long long off = page * page_stride + (tb % BS) * Gm::kRowBytes;
          const uint8_t* kb = kbase + off + lane * 16;
#pragma unroll
          for (int jl = 0; jl < Gm::kKLoads; ++jl)
            t.k[r][jl] = *reinterpret_cast<const u32x4*>(kb + 1024 * jl);
          const uint8_t* vb = vbase + off + lane * 4 * Gm::kEsz;
#pragma unroll
          for (int jd = 0; jd < Gm::kPvMfma; ++jd)
            t.v[r][jd] = *reinterpret_cast<const typename Tile::VT*>(
                vb + jd * 256 * Gm::kEsz);
        }
      };

      // Two register tiles in flight. The next tile's loads are issued on
      // every iteration, unconditionally: past the last tile they re-read
      // the current tile (lines already in L2) into the idle buffer. With a
      // conditional load the compiler would have to assume the load may be
      // missing and wait for the newer tile as well, serialising latency.
      Tile ta, tb;
      int k = tw;
      if (k < ntiles) {
        load_tile(ta, k);
        while (true) {
          load_tile(tb, k + TW < ntiles ? k + TW : k);
          compute_tile(ta, cs + k * kTile, ce);
          k += TW;
          if (k >= ntiles) break;
          load_tile(ta, k + TW < ntiles ? k + TW : k);
          compute_tile(tb, cs + k * kTile, ce);
          k += TW;
          if (k >= ntiles) break;
        }
      }
    }
  }

  // Consume the tile starting at token ts (tokens >= ce are masked). Value
  // e (0..7) of this lane's scores, probabilities and V operand belongs to
  // token ts + 16 * (e / 4) + 4 * lg + e % 4.
  __device__ __forceinline__ void compute_tile(Tile& t, int ts, int ce) {
    const bool tail = ts + kTile > ce;
    half8 kop[2][Gm::kQkMfma];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int jj = 0; jj < Gm::kQkMfma; ++jj) {
        if constexpr (FP8) {
          const u32x4 w = t.k[r][jj >> 1];
          const u32x2 hlf = (jj & 1) ? u32x2{w.z, w.w} : u32x2{w.x, w.y};
          kop[r][jj] = e4m3x8_to_half8(hlf);
        } else {
          kop[r][jj] = as_half8(t.k[r][jj]);
        }
      }
    // valid tokens among this lane's 4 of each block
    const int nv0 = ce - (ts + 4 * lg);
    const int nv1 = ce - (ts + 16 + 4 * lg);
    if (tail) {
      // zero the V entries of tokens past the end, in place (a masked
      // probability of 0 times a NaN left in an unused slot is still NaN)
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int nv = r ? nv1 : nv0;
#pragma unroll
        for (int jd = 0; jd < Gm::kPvMfma; ++jd) {
          if constexpr (FP8) {
            const uint32_t keep = nv <= 0 ? 0u : (nv >= 4 ? 0xFFFFFFFFu
                                                          : (1u << (8 * nv)) - 1u);
            t.v[r][jd] &= keep;
          } else {
            const uint32_t lo0 = nv > 0 ? 0x0000FFFFu : 0u;
            const uint32_t hi0 = nv > 1 ? 0xFFFF0000u : 0u;
            const uint32_t lo1 = nv > 2 ? 0x0000FFFFu : 0u;
            const uint32_t hi1 = nv > 3 ? 0xFFFF0000u : 0u;
            t.v[r][jd].x &= (lo0 | hi0);
            t.v[r][jd].y &= (lo1 | hi1);
          }
        }
      }
    }
    half8 vop[Gm::kPvMfma];
#pragma unroll
    for (int jd = 0; jd < Gm::kPvMfma; ++jd) {
      if constexpr (FP8) {
        vop[jd] = e4m3x8_to_half8(u32x2{t.v[0][jd], t.v[1][jd]});
      } else {
        const u32x4 w = {t.v[0][jd].x, t.v[0][jd].y, t.v[1][jd].x, t.v[1][jd].y};
        vop[jd] = as_half8(w);
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
      float sv[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[i] = s0[i] * sl;
        sv[4 + i] = s1[i] * sl;
      }
      if (tail) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if ((e & 3) >= (e < 4 ? nv0 : nv1)) sv[e] = -INFINITY;
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
  }

  // Merge the token-parallel waves (log-sum-exp) and write either the fp16
  // output (slot < 0) or partial slot `slot` of (b, h). All waves call this.
  __device__ __forceinline__ void flush(int b, int h, int slot) {
#pragma unroll
    for (int hb = 0; hb < NH; ++hb) {
      lrun[hb] += xor_lanes(lrun[hb], 16);
      lrun[hb] += xor_lanes(lrun[hb], 32);
    }
    __syncthreads();   // LDS flush buffers are free (previous flush read)
    if (lg == 0) {
#pragma unroll
      for (int hb = 0; hb < NH; ++hb) {
        sm.m[tw][(hw * NH + hb) * 16 + mrow] = mrun[hb];
        sm.l[tw][(hw * NH + hb) * 16 + mrow] = lrun[hb];
      }
    }
    __syncthreads();
    float wown[NH][4], ltot[NH][4], mtot[NH][4];
#pragma unroll
    for (int hb = 0; hb < NH; ++hb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hh = (hw * NH + hb) * 16 + 4 * lg + i;
        float M = -INFINITY;
#pragma unroll
        for (int t = 0; t < TW; ++t) M = fmaxf(M, sm.m[t][hh]);
        float Lsum = 0.0f;
        if (M != -INFINITY) {
#pragma unroll
          for (int t = 0; t < TW; ++t)
            Lsum += sm.l[t][hh] * __builtin_amdgcn_exp2f(sm.m[t][hh] - M);
        }
        wown[hb][i] = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(sm.m[tw][hh] - M);
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
                sm.acc[tw - 1][hh][16 * jd + mrow] = acc[hb][jd][i] * wown[hb][i];
            }
          }
      }
      __syncthreads();
    }
    if (tw == 0) {
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
            for (int t = 1; t < TW; ++t) v += sm.acc[t - 1][hh][16 * jd + mrow];
            vals[jd] = v * inv;
          }
          if (slot >= 0) {
            const long long row = ((long long)b * a.Hq + hq) * a.S + slot;
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
            for (int jd = 0; jd < Gm::kPvMfma; ++jd)
              o[16 * jd + mrow] = (_Float16)vals[jd];
          }
        }
    }
  }
};

__device__ __forceinline__ int clamp_len(int L, int cap) {
  return L < 0 ? 0 : (L > cap ? cap : L);
}

// Single pass (or one split): one workgroup per (sequence, kv head).
template <int D, int BS, bool FP8, int NH, int NWH, int TW>
__global__ __launch_bounds__(64 * NWH * TW)
__attribute__((amdgpu_waves_per_eu(NH == 1 ? 2 : 1)))
void decode_attn_kernel(AttnArgs a) {
  using Dec = Decoder<D, BS, FP8, NH, NWH, TW>;
  __shared__ typename Dec::Smem sm;
  Dec dec(a, sm);
  const int h = blockIdx.x % a.Hkv;
  const int b = blockIdx.x / a.Hkv;
  const int L = clamp_len(a.context_lens[b], a.max_blocks * BS);
  dec.begin(b, h);
  dec.run(b, h, 0, L);
  dec.flush(b, h, a.mode == 1 ? 0 : -1);
  if (a.mode == 1 && threadIdx.x == 0) a.ws_count[(long long)b * a.Hkv + h] = 1;
}

// Split pass, stream-K: workgroup w covers global tiles [w*tpw, (w+1)*tpw)
// of the sequence-major, then kv-head-major, then token order, where each
// (sequence, kv head) has ceil(L/32) tiles. tpw = max(ceil(T / grid),
// ceil(n_max / (S - 1))) keeps every (sequence, kv head) within S partials.
template <int D, int BS, bool FP8, int NH, int NWH, int TW>
__global__ __launch_bounds__(64 * NWH * TW)
__attribute__((amdgpu_waves_per_eu(NH == 1 ? 2 : 1)))
void decode_attn_streamk_kernel(AttnArgs a) {
  using Dec = Decoder<D, BS, FP8, NH, NWH, TW>;
  __shared__ typename Dec::Smem sm;
  const int cap = a.max_blocks * BS;
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;

  // 1. per-thread share of sequences: tile counts, their sum and maximum
  const int per = (a.B + nthr - 1) / nthr;
  const int b_lo = min(a.B, tid * per), b_hi = min(a.B, b_lo + per);
  int my_sum = 0, my_max = 0;
  for (int b = b_lo; b < b_hi; ++b) {
    const int n = (clamp_len(a.context_lens[b], cap) + kTile - 1) / kTile;
    my_sum += n;
    my_max = max(my_max, n);
  }
  // block-wide inclusive scan of my_sum (Hillis-Steele in LDS) and max
  sm.scan[tid] = my_sum;
  __syncthreads();
  for (int off = 1; off < nthr; off <<= 1) {
    const int v = tid >= off ? sm.scan[tid - off] : 0;
    __syncthreads();
    sm.scan[tid] += v;
    __syncthreads();
  }
  const int seq_tiles = sm.scan[nthr - 1];
  const int excl = sm.scan[tid] - my_sum;
  __syncthreads();
  sm.scan[tid] = my_max;
  __syncthreads();
  for (int off = nthr >> 1; off > 0; off >>= 1) {
    if (tid < off) sm.scan[tid] = max(sm.scan[tid], sm.scan[tid + off]);
    __syncthreads();
  }
  const int n_max = sm.scan[0];

  const long long T = (long long)seq_tiles * a.Hkv;
  long long tpw = (T + gridDim.x - 1) / gridDim.x;
  const long long need = (n_max + (a.S - 1) - 1) / (a.S - 1);
  if (tpw < need) tpw = need;
  if (tpw < 1) tpw = 1;
  const long long r0 = (long long)blockIdx.x * tpw;
  if (r0 >= T) return;                        // whole workgroup leaves
  const long long r1 = min(T, r0 + tpw);

  // 2. locate the sequence holding global tile r0 (offsets scale by Hkv)
  if (tid == 0) sm.loc[0] = -1;
  __syncthreads();
  {
    long long off = (long long)excl * a.Hkv;
    if (r0 >= off && r0 < off + (long long)my_sum * a.Hkv) {
      for (int b = b_lo; b < b_hi; ++b) {
        const int n = (clamp_len(a.context_lens[b], cap) + kTile - 1) / kTile;
        const long long span = (long long)n * a.Hkv;
        if (r0 < off + span) {
          sm.loc[0] = b;
          sm.loc[1] = (int)((r0 - off) / n);      // kv head
          sm.loc[2] = (int)((r0 - off) % n);      // tile within (b, h)
          break;
        }
        off += span;
      }
    }
  }
  __syncthreads();
  int b = sm.loc[0], h = sm.loc[1], tile = sm.loc[2];
  long long base = r0 - tile;                 // global index of (b, h)'s tile 0

  Dec dec(a, sm);
  long long pos = r0;
  while (pos < r1) {
    const int L = clamp_len(a.context_lens[b], cap);
    const int n = (L + kTile - 1) / kTile;
    const int t_end = (int)min((long long)n, tile + (r1 - pos));
    dec.begin(b, h);
    dec.run(b, h, tile * kTile, min(t_end * kTile, L));
    const int slot = (int)(blockIdx.x - base / tpw);
    dec.flush(b, h, slot);
    if (t_end == n && tid == 0) a.ws_count[(long long)b * a.Hkv + h] = slot + 1;
    pos += t_end - tile;
    base += n;
    tile = 0;
    if (++h == a.Hkv) {
      h = 0;
      do { ++b; } while (b < a.B && pos < r1 &&
                         clamp_len(a.context_lens[b], cap) == 0);
    }
  }
}

// ---------------------------------------------------------------------------
// Instances: head_dim {64, 128} x block_size {16, 32, 64} x {fp16, fp8} x
// group-size class (heads per workgroup = NWH * NH * 16).
template <int D, int BS, bool FP8, int NH, int NWH, int TW>
static hipError_t launch_cfg(const AttnArgs& a, hipStream_t st) {
  constexpr int kThreads = 64 * NWH * TW;
  if (a.mode == 2) {
    // persistent grid: as many workgroups as fit at once on 256 CUs
    constexpr int kPerCu = NH == 1 ? 2 : 1;
    hipLaunchKernelGGL((decode_attn_streamk_kernel<D, BS, FP8, NH, NWH, TW>),
                       256u * kPerCu, kThreads, 0, st, a);
  } else {
    const unsigned grid = (unsigned)((long long)a.B * a.Hkv);
    hipLaunchKernelGGL((decode_attn_kernel<D, BS, FP8, NH, NWH, TW>), grid,
                       kThreads, 0, st, a);
  }
  return hipGetLastError();
}

template <int D, int BS, bool FP8>
static hipError_t launch_group(const AttnArgs& a, hipStream_t st) {
  if (a.G <= 16) return launch_cfg<D, BS, FP8, 1, 1, 4>(a, st);
  if (a.G <= 32) return launch_cfg<D, BS, FP8, 2, 1, 4>(a, st);
  if (a.G <= 64) return launch_cfg<D, BS, FP8, 2, 2, 2>(a, st);
  if (a.G <= 96) return launch_cfg<D, BS, FP8, 3, 2, 2>(a, st);
  if (a.G <= 128) return launch_cfg<D, BS, FP8, 4, 2, 1>(a, st);
  return hipErrorInvalidValue;
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
