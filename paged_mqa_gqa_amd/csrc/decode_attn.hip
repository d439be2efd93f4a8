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
//  * Work unit: a 32-token tile of one (sequence, kv head) for the 16-head
//    blocks of the group a wave owns (NH blocks per wave; NWH waves share a
//    tile stream when the group has more heads). Tiles stream straight from
//    HBM into MFMA operand registers, the next tile's loads in flight while
//    the current tile is computed. The page layout stores each 16-token
//    block in operand order, so every wave-wide load reads whole 128-byte
//    lines and a lane's V operand is one 16-byte (one-byte codes: 8-byte)
//    run.
//  * QK^T: 16 tokens of the tile as the A operand (16 tokens x 32 dims),
//    the group's q heads as B (32 dims x 16 heads). The 16x16 result holds,
//    per lane, scores of one head for 4 tokens; the two token halves of a
//    tile are picked so that a lane ends up with 8 consecutive tokens, the
//    8 that the P.V product needs in the same lane, so P never leaves
//    registers.
//  * Online softmax in base 2 (scale * log2 e folded into the scores): the
//    running max per head is reduced across the four 16-lane groups, the
//    running sum stays per lane until a flush.
//  * P.V: P (16 heads x 32 tokens, fp16) as A, V (32 tokens x 16 dims) as
//    B, accumulated in fp32.
//  * Page ids are clamped into the pool; tokens past the end re-read a
//    valid block and are masked by select, so NaN in unused slots never
//    leaks.
//  * One-byte K/V codes are expanded to fp16 in registers by exact bit
//    placement (fp8 e4m3fn: value * 2^-8; int8: the integer itself); the
//    code unit (2^8 or 1) and the per-head scales fold into the score scale
//    and the final output scale.
//  * Two schedules. Single pass: one workgroup per (sequence, kv head), its
//    token-parallel waves merged through LDS. Split pass (stream-K): every
//    wave (or head-parallel wave group) is a worker; the tiles of all
//    (sequence, kv head) contexts, laid end to end, are cut into equal
//    contiguous shares, one per worker, so ragged batches balance exactly.
//    A worker streams its share as one pipeline across (sequence, kv head)
//    boundaries (no barriers), and each (sequence, kv head) segment it
//    covers becomes one log-sum-exp partial, merged by the reduce kernel or,
//    in the merged call, by the last of its workers to finish.
#include "launch.h"
#include "device_common.h"

#include <type_traits>

namespace pa {

constexpr int kTile = 32;       // tokens per tile
constexpr float kLazyLog2 = 8.0f;  // headroom of the lazy softmax rescale
constexpr int kMaxPages = 512;  // page ids staged in LDS per chunk (single pass)

template <int D, int BS, int KV>
struct Geo {
  static constexpr bool kByte = KV != kKvF16;        // one-byte codes
  static constexpr int kEsz = kByte ? 1 : 2;
  static constexpr int kRowBytes = D * kEsz;          // one token row
  static constexpr int kBlockBytes = 16 * kRowBytes;  // one 16-token block
  static constexpr int kPageBytes = BS * D * kEsz;    // one (page, head) tile
  static constexpr int kQkMfma = D / 32;              // per 16-token block
  static constexpr int kKLoads = kRowBytes / 64;      // 16 B loads per block
  static constexpr int kPvMfma = D / 16;              // per 32-token tile
};

// First dimension of the 8 K-slots that lane group g (= lane / 16) holds in
// QK MFMA number jj. fp16: a 16 B K chunk covers one MFMA; one-byte codes: a
// 16 B chunk covers 16 dims, i.e. two MFMAs.
template <bool BYTE>
__device__ __forceinline__ int kslot_dim(int jj, int g) {
  return BYTE ? 64 * (jj >> 1) + 16 * g + 8 * (jj & 1) : 32 * jj + 8 * g;
}

template <bool NT, typename T>
__device__ __forceinline__ T load16(const T* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

template <int D, int BS, int KV>
struct TileRegs {
  using G = Geo<D, BS, KV>;
  // V operand of one 16-dim group: the lane's 8 tokens of one dimension,
  // one contiguous run in the page
  using VT = typename std::conditional<G::kByte, u32x2, u32x4>::type;
  u32x4 k[2][G::kKLoads];      // [QK MFMA m][chunk group]
  VT v[G::kPvMfma];            // [16-dim group]
};

// Issue the loads of one tile whose two 16-token blocks start at byte
// offsets off0 / off1 of the K and V pools (head offset included). K/V are
// read once per call, so the loads are nontemporal (NT: streamed past the
// caches' retention), except where two waves read the same tile one after
// the other and the second should find it in the cache.
//
// Token order inside the tile: QK MFMA m (0, 1) takes as its 16 A rows the
// tokens 8 * (R / 4) + 4 * m + R % 4 (R = 0..15), i.e. rows 0..7 from block
// 0 and 8..15 from block 1; its result gives lane group lg the tokens
// 8 * lg + 4 * m + 0..3, so a lane's 8 probabilities are the tokens
// 8 * lg + 0..7 of the tile, all in block lg / 2: the V operand that P.V
// needs is one run of 8 tokens. In a block's K storage rows 8 * m + 0..7
// hold exactly MFMA m's tokens of that block.
//
// A dead load (live == false) keeps the load instructions, so that the
// compiler's wait counts stay exact, but points all lanes of each
// instruction at one line of the tile given by off0 (the tile just loaded):
// 16 lines per wave instead of a whole tile re-read. (One shared address for
// every wave would pile all waves' dead loads onto one memory channel.)
template <int D, int BS, int KV, bool NT>
__device__ __forceinline__ void load_tile(TileRegs<D, BS, KV>& t,
                                          const uint8_t* kbase,
                                          const uint8_t* vbase, long long off0,
                                          long long off1, int lane, bool live) {
  using Gm = Geo<D, BS, KV>;
  const int R = lane & 15, lg = lane >> 4;
  if (!live) off1 = off0;
  const int klane = live ? (lg * 16 + (R & 7)) * 16 : 0;
  const int vlane = live ? ((lg & 1) * 16 + R) * 8 * Gm::kEsz : 0;
  const uint8_t* kb = kbase + (R < 8 ? off0 : off1) + klane;
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int jl = 0; jl < Gm::kKLoads; ++jl)
      t.k[m][jl] = load16<NT>(reinterpret_cast<const u32x4*>(kb + 128 * m + 1024 * jl));
  const uint8_t* vb = vbase + (lg < 2 ? off0 : off1) + vlane;
#pragma unroll
  for (int jd = 0; jd < Gm::kPvMfma; ++jd)
    t.v[jd] = load16<NT>(
        reinterpret_cast<const typename TileRegs<D, BS, KV>::VT*>(vb + jd * 256 * Gm::kEsz));
}

// Attention state of one wave for NH blocks of 16 q heads of one (sequence,
// kv head), and the math of one tile. The q operands live in registers, or
// with QL in this wave's LDS region `qsh` ([NH][d/32][64 lanes] of 16 bytes,
// read back conflict-free), which leaves the registers to the accumulators
// of wide groups.
template <int D, int BS, int KV, int NH, bool QL = false>
struct HeadState {
  using Gm = Geo<D, BS, KV>;
  using Tile = TileRegs<D, BS, KV>;
  half8 qop[QL ? 1 : NH][Gm::kQkMfma];
  u32x4* qsh;
  float mrun[NH], lrun[NH];
  f32x4 acc[NH][Gm::kPvMfma];
  float sl, oscale;

  // q rows of heads (hw*NH + hb)*16 + lane%16 of group h of sequence b as
  // B operands, softmax state reset. Rows past the group take the group's
  // first head (they are computed and never written out), so the loads
  // need no masking and are not waited for before the first tile's math.
  __device__ __forceinline__ void begin(const AttnArgs& a, int b, int h, int hw,
                                        int mrow, int lg) {
    load_q(a, b, h, hw, mrow, lg);
    reset(a, h);
  }

  // The q loads of begin() alone (the previous pair's rows may still be
  // written out before reset()).
  __device__ __forceinline__ void load_q(const AttnArgs& a, int b, int h, int hw,
                                         int mrow, int lg) {
#pragma unroll
    for (int hb = 0; hb < NH; ++hb) {
      const int gh = (hw * NH + hb) * 16 + mrow;
      const _Float16* qrow = a.q + ((long long)b * a.Hq + h * a.G + (gh < a.G ? gh : 0)) * D;
#pragma unroll
      for (int jj = 0; jj < Gm::kQkMfma; ++jj) {
        const u32x4 raw = *reinterpret_cast<const u32x4*>(qrow + kslot_dim<Gm::kByte>(jj, lg));
        if constexpr (QL) qsh[(hb * Gm::kQkMfma + jj) * 64 + __lane_id()] = raw;
        else qop[hb][jj] = as_half8(raw);
      }
    }
  }

  // Scales of kv head h and an empty softmax state.
  __device__ __forceinline__ void reset(const AttnArgs& a, int h) {
    sl = a.scale_log2;
    oscale = 1.0f;
    if constexpr (Gm::kByte) {
      sl *= load_uniform(a.k_scale + h) * code_unit<KV>();
      oscale = load_uniform(a.v_scale + h) * code_unit<KV>();
    }
#pragma unroll
    for (int hb = 0; hb < NH; ++hb) {
      mrun[hb] = -INFINITY;
      lrun[hb] = 0.0f;
#pragma unroll
      for (int jd = 0; jd < Gm::kPvMfma; ++jd) acc[hb][jd] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }

  // Consume the tile starting at token ts (tokens >= ce are masked). Value
  // e (0..7) of this lane's scores, probabilities and V operand belongs to
  // token ts + 8 * lg + e.
  __device__ __forceinline__ void compute(Tile& t, int ts, int ce, int lg) {
    const bool tail = ts + kTile > ce;
    half8 kop[2][Gm::kQkMfma];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int jj = 0; jj < Gm::kQkMfma; ++jj) {
        if constexpr (Gm::kByte) {
          const u32x4 w = t.k[m][jj >> 1];
          const u32x2 hlf = (jj & 1) ? u32x2{w.z, w.w} : u32x2{w.x, w.y};
          kop[m][jj] = codes8_to_half8<KV>(hlf);
        } else {
          kop[m][jj] = as_half8(t.k[m][jj]);
        }
      }
    // valid tokens among this lane's 8
    const int nv = ce - (ts + 8 * lg);
    if (tail) {
      // zero the V entries of tokens past the end, in place (a masked
      // probability of 0 times a NaN left in an unused slot is still NaN)
      auto keep8 = [](int n) {        // one-byte codes of the first n tokens
        return n <= 0 ? 0u : (n >= 4 ? 0xFFFFFFFFu : (1u << (8 * n)) - 1u);
      };
      auto keep16 = [](int n, int w) {   // fp16: halves of tokens 2w, 2w+1
        return (n > 2 * w ? 0x0000FFFFu : 0u) | (n > 2 * w + 1 ? 0xFFFF0000u : 0u);
      };
#pragma unroll
      for (int jd = 0; jd < Gm::kPvMfma; ++jd) {
        if constexpr (Gm::kByte) {
          t.v[jd].x &= keep8(nv);
          t.v[jd].y &= keep8(nv - 4);
        } else {
          t.v[jd].x &= keep16(nv, 0);
          t.v[jd].y &= keep16(nv, 1);
          t.v[jd].z &= keep16(nv, 2);
          t.v[jd].w &= keep16(nv, 3);
        }
      }
    }
    half8 vop[Gm::kPvMfma];
#pragma unroll
    for (int jd = 0; jd < Gm::kPvMfma; ++jd) {
      if constexpr (Gm::kByte) vop[jd] = codes8_to_half8<KV>(t.v[jd]);
      else vop[jd] = as_half8(t.v[jd]);
    }
#pragma unroll
    for (int hb = 0; hb < NH; ++hb) {
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jj = 0; jj < Gm::kQkMfma; ++jj) {
        half8 qv;
        if constexpr (QL) qv = as_half8(qsh[(hb * Gm::kQkMfma + jj) * 64 + __lane_id()]);
        else qv = qop[hb][jj];
        s0 = mfma_16x16x32(kop[0][jj], qv, s0);
        s1 = mfma_16x16x32(kop[1][jj], qv, s1);
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
          if (e >= nv) sv[e] = -INFINITY;
      }
      float mt = sv[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mt = fmaxf(mt, sv[e]);
      mt = max_over_rows(mt);
      // Lazy rescale: the reference max mrun moves only when the tile's max
      // exceeds it by more than kLazyLog2, so probabilities stay <= 2^8
      // (fp16 P and the fp32 sums keep their relative precision) and the
      // accumulators are rescaled a handful of times per segment instead of
      // whenever the max grows. acc / l and m + log2(l) are unchanged.
      const bool bump = mt > mrun[hb] + kLazyLog2;   // first tile: mrun = -inf
      const float mn = bump ? mt : mrun[hb];
      const float alpha = bump ? __builtin_amdgcn_exp2f(mrun[hb] - mt) : 1.0f;
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

  // Per-head totals: the running sum reduced over the four lane groups.
  __device__ __forceinline__ void reduce_sums() {
#pragma unroll
    for (int hb = 0; hb < NH; ++hb) {
      lrun[hb] = sum_over_rows(lrun[hb]);
    }
  }

  // Write this wave's result rows for (b, h) after reduce_sums(): the fp16
  // output (slot < 0) or partial slot `slot` (normalised o, natural lse).
  // COHERENT partials are stored as device-scope atomics, i.e. written
  // through to the level every compute unit reads, for a merge inside the
  // same launch.
  template <bool COHERENT = false>
  __device__ __forceinline__ void write_rows(const AttnArgs& a, int b, int h,
                                             int hw, int slot, int mrow, int lg) {
#pragma unroll
    for (int hb = 0; hb < NH; ++hb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // totals of head row 4*lg+i live in the lanes whose column is that head
        const float Lh = read_lane(lrun[hb], 4 * lg + i);
        const float Mh = read_lane(mrun[hb], 4 * lg + i);
        const int hh = (hw * NH + hb) * 16 + 4 * lg + i;
        if (hh >= a.G) continue;
        const int hq = h * a.G + hh;
        const float inv = Lh > 0.0f ? oscale / Lh : 0.0f;
        if (slot >= 0) {
          const long long row = ((long long)b * a.Hq + hq) * a.S + slot;
          float* o = a.ws_o + row * D;
          const float lse = Lh > 0.0f ? (Mh + __builtin_amdgcn_logf(Lh)) * kLn2 : -INFINITY;
#pragma unroll
          for (int jd = 0; jd < Gm::kPvMfma; ++jd) {
            if constexpr (COHERENT) store_coherent(o + 16 * jd + mrow, acc[hb][jd][i] * inv);
            else o[16 * jd + mrow] = acc[hb][jd][i] * inv;
          }
          if (mrow == 0) {
            if constexpr (COHERENT) store_coherent(a.ws_lse + row, lse);
            else a.ws_lse[row] = lse;
          }
        } else {
          _Float16* o = a.out + ((long long)b * a.Hq + hq) * D;
#pragma unroll
          for (int jd = 0; jd < Gm::kPvMfma; ++jd)
            o[16 * jd + mrow] = (_Float16)(acc[hb][jd][i] * inv);
        }
      }
  }
};

// A value every lane holds equally, moved to a scalar register.
__device__ __forceinline__ int uniform(int v) {
  return __builtin_amdgcn_readfirstlane(v);
}
__device__ __forceinline__ long long uniform(long long v) {
  const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)v);
  const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)(v >> 32));
  return (long long)(((unsigned long long)hi << 32) | lo);
}

// x / y for non-negative x, y > 0, uniform over the wave: a 32-bit
// division when both fit in 32 bits (gfx9 has no integer divide, and the
// 64-bit routine is several times longer than the 32-bit one).
__device__ __forceinline__ long long div_nn(long long x, long long y) {
  if ((((unsigned long long)x | (unsigned long long)y) >> 32) == 0)
    return (long long)((unsigned)x / (unsigned)y);
  return x / y;
}

__device__ __forceinline__ int clamp_len(int L, int cap) {
  return L < 0 ? 0 : (L > cap ? cap : L);
}

__device__ __forceinline__ int clamp_page(int p, int P) {
  return p < 0 ? 0 : (p >= P ? P - 1 : p);
}

// Fused append: write the new token of (sequence b, kv head h) at position p
// into its page (one wave, two dimensions per lane), as kv_append does.
template <int D, int BS, int KV>
__device__ __forceinline__ void append_token(const AttnArgs& a, int b, int h,
                                             int p, int lane) {
  constexpr int kEsz = KV != kKvF16 ? 1 : 2;
  const int page = clamp_page(
      load_uniform(a.block_table + (long long)b * a.max_blocks + p / BS), a.P);
  const long long tile = ((long long)page * a.Hkv + h) * BS * D * kEsz;
  uint8_t* kt = const_cast<uint8_t*>(a.k_pages) + tile;
  uint8_t* vt = const_cast<uint8_t*>(a.v_pages) + tile;
  const long long row = ((long long)b * a.Hkv + h) * D;
  for (int dp = 2 * lane; dp < D; dp += 128) {
    const uint32_t kin = *reinterpret_cast<const uint32_t*>(a.k_new + row + dp);
    const uint32_t vin = *reinterpret_cast<const uint32_t*>(a.v_new + row + dp);
    float ks = 1.0f, vs = 1.0f;
    if constexpr (KV != kKvF16) {
      ks = load_uniform(a.k_scale + h);
      vs = load_uniform(a.v_scale + h);
    }
    store_kv_pair<D, KV>(kt, vt, p % BS, dp, kin, vin, ks, vs);
  }
}

// ---------------------------------------------------------------------------
// Single pass (or one split): one workgroup per (sequence, kv head); its
// waves are NWH head-parallel groups times TW token-parallel waves whose
// results merge through LDS.
template <int NH, int NWH, int TW, int D>
struct SharedMem {
  static constexpr int kHeads = NWH * NH * 16;
  int pages[kMaxPages];
  float m[TW][kHeads];
  float l[TW][kHeads];
  float acc[TW > 1 ? TW - 1 : 1][kHeads][D];
};

template <int D, int BS, int KV, int NH, int NWH, int TW>
__global__ __launch_bounds__(64 * NWH * TW)
__attribute__((amdgpu_waves_per_eu(NH == 1 ? 2 : 1)))
void decode_attn_kernel(AttnArgs a) {
  using Gm = Geo<D, BS, KV>;
  using Tile = TileRegs<D, BS, KV>;
  using Smem = SharedMem<NH, NWH, TW, D>;
  __shared__ Smem sm;
  const int lane = threadIdx.x & 63;
  const int wave = uniform((int)(threadIdx.x >> 6));   // scalar: uniform control flow
  const int hw = wave % NWH, tw = wave / NWH;
  const int mrow = lane & 15, lg = lane >> 4;
  const int h = blockIdx.x % a.Hkv;
  const int b = blockIdx.x / a.Hkv;
  const int L = clamp_len(load_uniform(a.context_lens + b), a.max_blocks * BS);

  if (a.k_new != nullptr) {
    // fused append before any tile is read; the barrier publishes it to the
    // workgroup's other waves
    if (wave == 0) {
      const int p = load_uniform(a.positions + b);
      if (p >= 0 && p < a.max_blocks * BS) append_token<D, BS, KV>(a, b, h, p, lane);
      wait_vector_memory();
    }
    __syncthreads();
  }
  HeadState<D, BS, KV, NH> st;
  st.begin(a, b, h, hw, mrow, lg);
  const uint8_t* kbase = a.k_pages + (long long)h * Gm::kPageBytes;
  const uint8_t* vbase = a.v_pages + (long long)h * Gm::kPageBytes;
  const long long page_stride = (long long)a.Hkv * Gm::kPageBytes;
  const int* bt_row = a.block_table + (long long)b * a.max_blocks;

  for (int cs = 0; cs < L; cs += kMaxPages * BS) {
    const int ce = min(L, cs + kMaxPages * BS);
    const int p0 = cs / BS;
    const int np = (ce - 1) / BS - p0 + 1;
    __syncthreads();   // previous chunk's ids are free
    for (int i = threadIdx.x; i < np; i += blockDim.x)
      sm.pages[i] = clamp_page(bt_row[p0 + i], a.P);
    __syncthreads();
    const int ntiles = (ce - cs + kTile - 1) / kTile;
    const int last_blk = (ce - 1) & ~15;
    auto issue = [&](Tile& t, int k) {
      const bool live = k < ntiles;
      const int ts = cs + (live ? k : 0) * kTile;
      long long off[2];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int tb = min(ts + 16 * r, last_blk);
        off[r] = sm.pages[tb / BS - p0] * page_stride + (tb % BS) * Gm::kRowBytes;
      }
      load_tile<D, BS, KV, NWH == 1>(t, kbase, vbase, off[0], off[1], lane, live);
    };
    // Two register tiles in flight; the next tile's loads are issued on
    // every iteration, unconditionally (past the last tile as dead loads),
    // so the compiler waits only for the older tile's loads.
    Tile ta, tb;
    int k = tw;
    if (k < ntiles) {
      issue(ta, k);
      while (true) {
        issue(tb, k + TW);
        st.compute(ta, cs + k * kTile, ce, lg);
        k += TW;
        if (k >= ntiles) break;
        issue(ta, k + TW);
        st.compute(tb, cs + k * kTile, ce, lg);
        k += TW;
        if (k >= ntiles) break;
      }
    }
  }

  // merge the token-parallel waves (log-sum-exp) through LDS
  st.reduce_sums();
  if constexpr (TW > 1) {
    if (lg == 0) {
#pragma unroll
      for (int hb = 0; hb < NH; ++hb) {
        sm.m[tw][(hw * NH + hb) * 16 + mrow] = st.mrun[hb];
        sm.l[tw][(hw * NH + hb) * 16 + mrow] = st.lrun[hb];
      }
    }
    __syncthreads();
    // rescale this wave's rows to the common max and totals
#pragma unroll
    for (int hb = 0; hb < NH; ++hb) {
      const int hcol = (hw * NH + hb) * 16 + mrow;      // column head of lane
      float M = -INFINITY;
#pragma unroll
      for (int t = 0; t < TW; ++t) M = fmaxf(M, sm.m[t][hcol]);
      float Ls = 0.0f;
      if (M != -INFINITY) {
#pragma unroll
        for (int t = 0; t < TW; ++t)
          Ls += sm.l[t][hcol] * __builtin_amdgcn_exp2f(sm.m[t][hcol] - M);
      }
      const float w = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(st.mrun[hb] - M);
      // rows 4*lg+i of acc scale by the weight of head 4*lg+i
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float wi = read_lane(w, 4 * lg + i);
#pragma unroll
        for (int jd = 0; jd < Gm::kPvMfma; ++jd) st.acc[hb][jd][i] *= wi;
      }
      st.mrun[hb] = M;
      st.lrun[hb] = Ls;
    }
    if (tw > 0) {
#pragma unroll
      for (int hb = 0; hb < NH; ++hb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int hh = (hw * NH + hb) * 16 + 4 * lg + i;
          if (hh < a.G) {
#pragma unroll
            for (int jd = 0; jd < Gm::kPvMfma; ++jd)
              sm.acc[tw - 1][hh][16 * jd + mrow] = st.acc[hb][jd][i];
          }
        }
    }
    __syncthreads();
    if (tw > 0) return;
#pragma unroll
    for (int hb = 0; hb < NH; ++hb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hh = (hw * NH + hb) * 16 + 4 * lg + i;
        if (hh < a.G) {
#pragma unroll
          for (int jd = 0; jd < Gm::kPvMfma; ++jd)
#pragma unroll
            for (int t = 1; t < TW; ++t) st.acc[hb][jd][i] += sm.acc[t - 1][hh][16 * jd + mrow];
        }
      }
  }
  st.write_rows(a, b, h, hw, a.mode == 1 ? 0 : -1, mrow, lg);
  if (a.mode == 1 && threadIdx.x == 0) a.ws_count[(long long)b * a.Hkv + h] = 1;
}

// ---------------------------------------------------------------------------
// Split pass (stream-K).

// Tiles of sequence b (its context clamped to the block table's capacity).
__device__ __forceinline__ int seq_tiles(const AttnArgs& a, int b, int cap) {
  return (clamp_len(a.context_lens[b], cap) + kTile - 1) / kTile;
}

// Inclusive prefix sum across the 64 lanes of a wave: a scan inside each
// 16-lane row by DPP row shifts (a lane with no source lane adds 0), then
// every row adds the totals of the rows before it, read from their last
// lanes. VALU and scalar reads only: no LDS round trips.
__device__ __forceinline__ int wave_incl_sum(int v, int lane) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);   // row_shr:8
  const int t0 = __builtin_amdgcn_readlane(v, 15);
  const int t1 = __builtin_amdgcn_readlane(v, 31);
  const int t2 = __builtin_amdgcn_readlane(v, 47);
  const int row = lane >> 4;
  return v + (row >= 1 ? t0 : 0) + (row >= 2 ? t1 : 0) + (row >= 3 ? t2 : 0);
}

// Maximum over the 64 lanes (a scalar): a running maximum inside each row
// (a lane with no source lane keeps its own value), then the rows' last
// lanes.
__device__ __forceinline__ int wave_max(int v) {
  v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x111, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x112, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x114, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x118, 0xf, 0xf, false));
  return max(max(__builtin_amdgcn_readlane(v, 15), __builtin_amdgcn_readlane(v, 31)),
             max(__builtin_amdgcn_readlane(v, 47), __builtin_amdgcn_readlane(v, 63)));
}

// Value of lane src (the same for every lane) as a scalar.
__device__ __forceinline__ int lane_value(int v, int src) {
  return __builtin_amdgcn_readlane(v, src);
}
__device__ __forceinline__ long long lane_value(long long v, int src) {
  const unsigned long long u = (unsigned long long)v;
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)u, src);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(u >> 32), src);
  return (long long)(((unsigned long long)hi << 32) | lo);
}

// Position in the split pass's tile order: (sequence b, kv head h, tile t
// of n), L = tokens of b, base = global index of (b, h)'s first tile.
struct Cursor {
  int b, h, t, n, L;
  long long base;
};

// The tile after c (one must exist): next tile, next kv head, or the next
// sequence that has tokens.
__device__ __forceinline__ Cursor advance(const AttnArgs& a, Cursor c, int cap) {
  if (c.t + 1 < c.n) { ++c.t; return c; }
  c.t = 0;
  c.base += c.n;
  if (++c.h < a.Hkv) return c;
  c.h = 0;
  do {
    ++c.b;
    c.L = clamp_len(load_uniform(a.context_lens + c.b), cap);
  } while (c.L == 0);
  c.n = (c.L + kTile - 1) / kTile;
  return c;
}

// The (sequence, kv head) pair holding global tile x of the split order
// (0 <= x < total tiles): its sequence b, kv head h, tile t within it, its
// tile count n and the global index of its first tile. Scalar results.
// len0 holds the clamped lengths of sequences 0..63, one per lane, so a
// batch of up to 64 sequences is located without a memory round trip.
__device__ __forceinline__ Cursor locate(const AttnArgs& a, long long x, int cap,
                                         int lane, int len0) {
  Cursor c{0, 0, 0, 1, 1, 0};
  int L = -1;
  long long done = 0;                         // tiles (times Hkv) before chunk
  for (int c0 = 0; c0 < a.B; c0 += 64) {
    const int len = c0 == 0 ? len0
                            : (c0 + lane < a.B ? clamp_len(a.context_lens[c0 + lane], cap) : 0);
    const int n = (len + kTile - 1) / kTile;
    const int incl = wave_incl_sum(n, lane);
    const long long lo = done + (long long)(incl - n) * a.Hkv;
    const long long hi = done + (long long)incl * a.Hkv;
    const unsigned long long hit = __ballot(x >= lo && x < hi);
    if (hit) {
      const int src = __ffsll((long long)hit) - 1;
      c.b = c0 + src;
      c.n = lane_value(n, src);
      L = lane_value(len, src);
      const long long rel = x - lane_value(lo, src);
      c.h = (int)div_nn(rel, c.n);
      c.t = (int)(rel - (long long)c.h * c.n);
      break;
    }
    done += (long long)lane_value(incl, 63) * a.Hkv;
  }
  c.b = uniform(c.b);
  c.h = uniform(c.h);
  c.t = uniform(c.t);
  c.n = uniform(c.n);
  c.L = L >= 0 ? uniform(L) : clamp_len(load_uniform(a.context_lens + c.b), cap);
  c.base = x - c.t;
  return c;
}

// Byte offsets (head included) of the two 16-token blocks of c's tile. A
// block wholly past the end re-reads the first one (in bounds; masked).
template <int D, int BS, int KV>
__device__ __forceinline__ void tile_offsets(const AttnArgs& a, const Cursor& c,
                                             long long& off0, long long& off1) {
  using Gm = Geo<D, BS, KV>;
  const int* bt_row = a.block_table + (long long)c.b * a.max_blocks;
  const long long page_stride = (long long)a.Hkv * Gm::kPageBytes;
  const long long head = (long long)c.h * Gm::kPageBytes;
  const int ts = c.t * kTile;
  const int pA = clamp_page(load_uniform(bt_row + ts / BS), a.P);
  off0 = head + pA * page_stride + (ts % BS) * Gm::kRowBytes;
  if (ts + 16 >= c.L) {
    off1 = off0;
  } else if constexpr (BS == 16) {
    off1 = head + clamp_page(load_uniform(bt_row + ts / 16 + 1), a.P) * page_stride;
  } else {
    off1 = off0 + Gm::kBlockBytes;
  }
}

// Merge the nparts partials of (b, h) from the workspace into out (fp16),
// one wave: each lane owns 4 output values of one head for up to ITEMS
// heads at a time and folds the partials in by an online log-sum-exp, in
// groups of 8 (one rescale per group: the rounding depends on the grouping
// only, so every variant gives the same bits). The loads are device-scope
// atomics, so they see the partials that other compute units wrote through
// (write_rows<true>).
template <int D, int ITEMS>
__device__ __forceinline__ void merge_partials(const AttnArgs& a, int b, int h,
                                               int nparts, int lane) {
  constexpr int kCols = D / 4;
  constexpr int kParts = 8;
  const int items = a.G * kCols;
  for (int base = 0; base < items; base += 64 * ITEMS) {
    long long row[ITEMS];
    int c4[ITEMS];
    bool live[ITEMS];
#pragma unroll
    for (int u = 0; u < ITEMS; ++u) {
      const int it = base + 64 * u + lane;
      live[u] = it < items;
      const int itc = live[u] ? it : 0;
      const int g = itc / kCols;
      c4[u] = (itc % kCols) * 4;
      row[u] = ((long long)b * a.Hq + h * a.G + g) * a.S;
    }
    float M[ITEMS], den[ITEMS];
    f32x4 acc[ITEMS];
#pragma unroll
    for (int u = 0; u < ITEMS; ++u) {
      M[u] = -INFINITY;
      den[u] = 0.0f;
      acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float l[ITEMS][kParts];
    f32x4 o[ITEMS][kParts];
    // loads of group i0 (past the last partial: re-reads of it)
    auto fetch = [&](int i0) {
#pragma unroll
      for (int u = 0; u < ITEMS; ++u)
#pragma unroll
        for (int j = 0; j < kParts; ++j) {
          const long long r = row[u] + min(i0 + j, nparts - 1);
          l[u][j] = load_coherent(a.ws_lse + r);
          const float2 lo = load_coherent2(a.ws_o + r * D + c4[u]);
          const float2 hi = load_coherent2(a.ws_o + r * D + c4[u] + 2);
          o[u][j] = f32x4{lo.x, lo.y, hi.x, hi.y};
        }
    };
    auto fold = [&](int i0) {
#pragma unroll
      for (int u = 0; u < ITEMS; ++u) {
        float mc = -INFINITY;
#pragma unroll
        for (int j = 0; j < kParts; ++j) {
          if (i0 + j >= nparts) l[u][j] = -INFINITY;
          mc = fmaxf(mc, l[u][j]);
        }
        const float mn = fmaxf(M[u], mc);
        if (mn == -INFINITY) continue;             // no tokens so far
        const float sc = __builtin_amdgcn_exp2f((M[u] - mn) * kLog2e);
        den[u] *= sc;
        acc[u] *= sc;
#pragma unroll
        for (int j = 0; j < kParts; ++j) {
          const float wj = __builtin_amdgcn_exp2f((l[u][j] - mn) * kLog2e);
          den[u] += wj;
          acc[u] += wj * o[u][j];
        }
        M[u] = mn;
      }
    };
    for (int i0 = 0; i0 < nparts; i0 += kParts) {
      fetch(i0);
      fold(i0);
    }
#pragma unroll
    for (int u = 0; u < ITEMS; ++u) {
      if (!live[u]) continue;
      const float inv = den[u] > 0.0f ? 1.0f / den[u] : 0.0f;
      const long long orow = row[u] / a.S;          // b * Hq + head
      _Float16* out = a.out + orow * D + c4[u];
#pragma unroll
      for (int e = 0; e < 4; ++e) out[e] = (_Float16)(acc[u][e] * inv);
    }
  }
}

// Worker k (a wave, or NWH waves with head blocks split between them) of
// W covers global tiles [floor(k T / W), floor((k + 1) T / W)) of the
// sequence-major, then kv-head-major, then token order, where each
// (sequence, kv head) has ceil(L/32) tiles and T is their total. Every
// share thus has floor(T / W) or one more tiles; W is the grid's worker
// count unless that would cut some (sequence, kv head) into more than S
// ranges (checked exactly), in which case W is lowered until
// floor(T / W) >= ceil(n_max / (S - 1)), which bounds every pair by S
// ranges. mode 2 writes the partials and their count; mode 3 merges too: a
// (sequence, kv head) held by one worker is written out directly, otherwise
// the last of its workers to finish merges the partials (an atomic arrival
// counter per pair, kept at the index of the pair's first worker and
// returned to zero afterwards).
template <int D, int BS, int KV, int NH, int NWH, bool QL, int SLOTS>
__global__ __launch_bounds__(NH == 1 && SLOTS == 2 ? 512 : 256)
__attribute__((amdgpu_waves_per_eu(NH == 1 && SLOTS == 2 ? 2 : 1)))
void decode_attn_stream_kernel(AttnArgs a) {
  using Tile = TileRegs<D, BS, KV>;
  using Gm = Geo<D, BS, KV>;
  // one 8-wave workgroup per CU (two waves per SIMD) for the small
  // two-tile configuration, else one wave per SIMD
  constexpr int kWaves = NH == 1 && SLOTS == 2 ? 8 : 4;
  constexpr int kWorkersPerWg = kWaves / NWH;
  constexpr int kQWords = QL ? NH * Gm::kQkMfma * 64 : 1;   // 16 B each, per wave
  __shared__ u32x4 qsmem[kWaves][kQWords];
  const int lane = threadIdx.x & 63;
  // the wave index in a scalar register, so that the worker's share, the
  // loop control and the block-table reads are scalar: a vector load of a
  // page id would have to wait for the tile loads issued before it
  const int wave = uniform((int)(threadIdx.x >> 6));
  const int hw = wave % NWH;
  const int mrow = lane & 15, lg = lane >> 4;
  const int workers = gridDim.x * kWorkersPerWg;
  const int worker = blockIdx.x * kWorkersPerWg + wave / NWH;
  const int cap = a.max_blocks * BS;

  // 1. total tiles and the longest sequence (every wave, redundantly). The
  // lengths of the first 64 sequences stay in a register for every later
  // scan (one load per lane for batches of up to 64 sequences).
  const int len0 = lane < a.B ? clamp_len(a.context_lens[lane], cap) : 0;
  const int n0 = (len0 + kTile - 1) / kTile;
  int carry = 0, n_max = 0;
  for (int c0 = 0; c0 < a.B; c0 += 64) {
    const int n = c0 == 0 ? n0 : (c0 + lane < a.B ? seq_tiles(a, c0 + lane, cap) : 0);
    carry += lane_value(wave_incl_sum(n, lane), 63);
    n_max = max(n_max, wave_max(n));
  }
  carry = uniform(carry);
  n_max = uniform(n_max);
  const long long T = (long long)carry * a.Hkv;
  const long long need = (n_max + (a.S - 1) - 1) / (a.S - 1);
  // never more workers than tiles: every share holds at least one tile, so
  // the workers between a pair's first and last owner all cover part of it
  long long W = workers < T ? workers : T;     // (all of these are scalars)
  if (need > 0 && T > 0 && T / need < W) {
    // the quick bound fails at the full grid: count the ranges exactly
    int worst = 0;
    long long done = 0;
    for (int c0 = 0; c0 < a.B; c0 += 64) {
      const int n = c0 == 0 ? n0 : (c0 + lane < a.B ? seq_tiles(a, c0 + lane, cap) : 0);
      const int incl = wave_incl_sum(n, lane);
      if (n > 0) {
        const long long x0 = done + (long long)(incl - n) * a.Hkv;
        for (int h = 0; h < a.Hkv; ++h) {
          const long long f = ((x0 + (long long)h * n + 1) * W - 1) / T;
          const long long l = ((x0 + (long long)(h + 1) * n) * W - 1) / T;
          worst = max(worst, (int)(l - f + 1));
        }
      }
      done += (long long)lane_value(incl, 63) * a.Hkv;
    }
    if (uniform(wave_max(worst)) > a.S) W = T / need;
  }
  if (W < 1) W = 1;
  W = uniform(W);

  if ((a.mode == 3 || a.k_new != nullptr) && hw == 0) {
    // sequences without tokens: no worker covers them, so their zeros and
    // their fused append are done here
    for (int b = worker; b < a.B; b += workers) {
      if ((b < 64 ? lane_value(len0, b) : clamp_len(a.context_lens[b], cap)) != 0) continue;
      if (a.mode == 3)
        for (int i = lane; i < a.Hq * D; i += 64)
          a.out[(long long)b * a.Hq * D + i] = (_Float16)0.0f;
      if (a.k_new != nullptr) {
        const int p = load_uniform(a.positions + b);
        if (p >= 0 && p < cap)
          for (int h = 0; h < a.Hkv; ++h) append_token<D, BS, KV>(a, b, h, p, lane);
      }
    }
  }
  if (worker >= W) return;                    // this wave has no share
  const long long r0 = uniform(div_nn((long long)worker * T, W));
  const long long r1 = uniform(div_nn((long long)(worker + 1) * T, W));
  if (r0 >= r1) return;

  // 2. the pairs holding this share's first and last tile. Only those two
  // can extend past the share; the workers owning their far ends (tile x
  // belongs to worker floor(((x + 1) W - 1) / T)) are worked out here, so
  // the loop needs no division.
  Cursor c = locate(a, r0, cap, lane, len0);
  const Cursor e = locate(a, r1 - 1, cap, lane, len0);
  long long fw = worker, lw = worker;
  if (c.base < r0) fw = uniform(div_nn((c.base + 1) * W - 1, T));
  if (e.base + e.n > r1) lw = uniform(div_nn((e.base + e.n) * W - 1, T));

  HeadState<D, BS, KV, NH, QL> st;
  st.qsh = qsmem[wave];
  st.begin(a, c.b, c.h, hw, mrow, lg);         // q loads overlap the append

  if (a.k_new != nullptr) {
    // Fused append: the worker whose share holds the tile of a pair's new
    // token (its last tile if the position lies past the context) writes the
    // token before loading any tile and waits for the stores, so its own
    // loads of that tile see it. No other worker reads that tile; both
    // waves of a two-wave worker write the same bytes. The share's first and
    // last pairs are checked (their positions read together); pairs in
    // between lie wholly inside the share.
    auto append_if_here = [&](const Cursor& s, int p) {
      if (p < 0 || p >= cap) return;
      const long long tp = s.base + min(p / kTile, s.n - 1);
      if (tp >= r0 && tp < r1) append_token<D, BS, KV>(a, s.b, s.h, p, lane);
    };
    const int pc = load_uniform(a.positions + c.b);
    const int pe = load_uniform(a.positions + e.b);
    append_if_here(c, pc);
    if (e.base != c.base) {
      Cursor s = c;
      s.t = s.n - 1;
      s = advance(a, s, cap);                 // first tile of the next pair
      while (s.base != e.base) {
        append_if_here(s, load_uniform(a.positions + s.b));
        s.t = s.n - 1;
        s = advance(a, s, cap);
      }
      append_if_here(e, pe);
    }
    wait_vector_memory();
  }

  // Count one arrival (NWH per worker) at the counter of the pair (b, h)
  // whose first and last owners are `first` and `last`; the last to arrive
  // merges. Every partial of the pair is stored and waited for (see
  // finish) before its owner arrives. The counter of a pair is indexed by
  // its first worker: a worker is the first of at most one pair that
  // extends past its share (its last pair), so the counters sit at a fixed
  // place whatever the batch. (AT_END: the share's last pair, merged after
  // the loop two columns per lane at a time; inside the loop one column
  // keeps register pressure down. Both fold the partials in the same groups
  // of eight, so the result does not depend on which worker arrives last.)
  auto arrive = [&](int b, int h, long long first, long long last, auto at_end) __attribute__((always_inline)) {
    int old = 0;
    int* sem = a.ws_sem + first;
    if (lane == 0)
      old = __hip_atomic_fetch_add(sem, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    old = __builtin_amdgcn_readlane(old, 0);   // lane 0 holds the result
    const int arrivals = (int)(last - first + 1) * NWH;
    if (old == arrivals - 1) {
      // the other workers' partials: visible at the device-coherent level
      // (their stores completed before their increments); read past this
      // CU's caches by the device-scope loads of the merge
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      if constexpr (decltype(at_end)::value)
        merge_partials<D, 2>(a, b, h, (int)(last - first + 1), lane);
      else
        merge_partials<D, 1>(a, b, h, (int)(last - first + 1), lane);
      if (lane == 0)
        __hip_atomic_store(sem, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };

  // End of (b, h)'s segment in this share: output, or a partial and its
  // arrival.
  auto finish = [&](const Cursor& s, auto at_end) __attribute__((always_inline)) {
    st.reduce_sums();
    // workers owning the pair's first and last tile
    const long long first = s.base < r0 ? fw : worker;
    const long long last = s.base + s.n > r1 ? lw : worker;
    const int slot = (int)(worker - first);
    if (a.mode == 3 && first == last) {
      st.write_rows(a, s.b, s.h, hw, -1, mrow, lg);
      return;
    }
    if (a.mode == 2) {
      st.write_rows(a, s.b, s.h, hw, slot, mrow, lg);
      if (s.t == s.n - 1 && hw == 0 && lane == 0)
        a.ws_count[(long long)s.b * a.Hkv + s.h] = slot + 1;
      return;
    }
    // The partial is written through with device-scope atomic stores;
    // waiting for their completion before the counter update makes them
    // visible to whichever compute unit merges, which reads them with
    // device-scope atomic loads. (A release/acquire pair would instead
    // write back and invalidate the whole L2 of the XCD at every arrival.)
    st.template write_rows<true>(a, s.b, s.h, hw, slot, mrow, lg);
    compiler_fence();
    wait_vector_memory();
    compiler_fence();
    arrive(s.b, s.h, first, last, at_end);
  };

  // Leave pair s for pair nx inside the loop. Without q in LDS, nx's q loads
  // go out before s's rows are stored, so the next tile's math waits for
  // them but not for the stores.
  auto switch_pair = [&](const Cursor& s, const Cursor& nx) __attribute__((always_inline)) {
    if constexpr (QL) {
      finish(s, std::false_type{});
      st.begin(a, nx.b, nx.h, hw, mrow, lg);
    } else {
      st.load_q(a, nx.b, nx.h, hw, mrow, lg);
      finish(s, std::false_type{});
      st.reset(a, nx.h);
    }
  };

  const uint8_t* kp = a.k_pages;
  const uint8_t* vp = a.v_pages;
  long long o0, o1;
  // The loop counts tiles within the share in 32 bits: 64-bit compares have
  // no scalar form and would go through vector registers and exec masks.
  const int ntiles = (int)(r1 - r0);
  int k = 0;                                  // this share's tile being computed
  constexpr bool kNT = NWH == 1;
  // The loop runs whole passes of SLOTS steps and leaves only at the bottom
  // of a pass. A step past the share's last tile issues its dead load and
  // computes nothing, so every step of a pass sees the same loads in flight
  // and the compiler's waits stay exact (an exit after each step would merge
  // the register state of every exit into the loop's flow and drain the
  // loads once per pass).
  if constexpr (SLOTS == 2) {
    Tile ta, tb;
    tile_offsets<D, BS, KV>(a, c, o0, o1);
    load_tile<D, BS, KV, kNT>(ta, kp, vp, o0, o1, lane, true);
    // One pipeline over the whole share: the next tile's loads (even in the
    // next segment) are in flight while the current tile is computed. They
    // are issued unconditionally (past the share's end as dead loads) so
    // that the compiler waits only for the older tile.
    auto step = [&](Tile& cur, Tile& nxt) __attribute__((always_inline)) {
      const bool more = k + 1 < ntiles;
      const Cursor nx = more ? advance(a, c, cap) : c;
      tile_offsets<D, BS, KV>(a, nx, o0, o1);
      load_tile<D, BS, KV, kNT>(nxt, kp, vp, o0, o1, lane, more);
      if (k < ntiles) {
        st.compute(cur, c.t * kTile, c.L, lg);
        if (more && (nx.b != c.b || nx.h != c.h)) switch_pair(c, nx);
      }
      ++k;
      c = nx;
    };
    do {
      step(ta, tb);
      step(tb, ta);
    } while (k < ntiles);
  } else {
    // Three register tiles: the loads of the two tiles after the current one
    // are in flight while it is computed.
    Tile t0, t1, t2;
    Cursor n1 = k + 1 < ntiles ? advance(a, c, cap) : c;
    tile_offsets<D, BS, KV>(a, c, o0, o1);
    load_tile<D, BS, KV, kNT>(t0, kp, vp, o0, o1, lane, true);
    tile_offsets<D, BS, KV>(a, n1, o0, o1);
    load_tile<D, BS, KV, kNT>(t1, kp, vp, o0, o1, lane, k + 1 < ntiles);
    auto step = [&](Tile& cur, Tile& ld) __attribute__((always_inline)) {
      const bool more2 = k + 2 < ntiles;
      const Cursor n2 = more2 ? advance(a, n1, cap) : n1;
      tile_offsets<D, BS, KV>(a, n2, o0, o1);
      load_tile<D, BS, KV, kNT>(ld, kp, vp, o0, o1, lane, more2);
      if (k < ntiles) {
        st.compute(cur, c.t * kTile, c.L, lg);
        if (k + 1 < ntiles && (n1.b != c.b || n1.h != c.h)) switch_pair(c, n1);
      }
      ++k;
      c = n1;
      n1 = n2;
    };
    do {
      step(t0, t2);
      step(t1, t0);
      step(t2, t1);
    } while (k < ntiles);
  }
  finish(c, std::true_type{});
}

// ---------------------------------------------------------------------------
// Instances: head_dim {64, 128} x block_size {16, 32, 64} x {fp16, fp8, int8}
// x group-size class. Each object file of the library holds one (kind,
// head_dim) pair (PA_INST_KV, PA_INST_D), so the instances build in parallel.
template <int D, int BS, int KV, int NH, int NWH, int TW>
static hipError_t launch_single(const AttnArgs& a, hipStream_t st) {
  const unsigned grid = (unsigned)((long long)a.B * a.Hkv);
  hipLaunchKernelGGL((decode_attn_kernel<D, BS, KV, NH, NWH, TW>), grid,
                     64 * NWH * TW, 0, st, a);
  return hipGetLastError();
}

// persistent grid: as many workgroups of 4 waves as fit at once on 256 CUs
template <int D, int BS, int KV, int NH, int NWH, bool QL, int SLOTS = 2>
static hipError_t launch_stream(const AttnArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((decode_attn_stream_kernel<D, BS, KV, NH, NWH, QL, SLOTS>),
                     (unsigned)kStreamGrid, NH == 1 && SLOTS == 2 ? 512 : 256, 0, st, a);
  return hipGetLastError();
}

// Group-size classes. Split pass: one wave streams each tile for up to 64
// of the group's heads (q kept in LDS above 32), two waves (each with its
// half of the heads) beyond; single pass: head-parallel and token-parallel
// waves of one workgroup. (Workers: 1024 for fp16 groups of up to 16 heads,
// 2048 for one-byte caches, 1024 up to 64 heads, 512 beyond.)
template <int D, int BS, int KV>
static hipError_t launch_group(const AttnArgs& a, hipStream_t st) {
  if (a.mode >= 2) {
    // up to 16 heads: fp16 tiles run one wave per SIMD with three tiles in
    // flight; one-byte tiles (half the bytes) two waves per SIMD with two
    if (a.G <= 16) {
      if constexpr (KV != kKvF16) return launch_stream<D, BS, KV, 1, 1, false, 2>(a, st);
      else return launch_stream<D, BS, KV, 1, 1, false, 3>(a, st);
    }
    if (a.G <= 32) return launch_stream<D, BS, KV, 2, 1, false>(a, st);
    if (a.G <= 64) return launch_stream<D, BS, KV, 4, 1, true>(a, st);
    if (a.G <= 96) return launch_stream<D, BS, KV, 3, 2, false>(a, st);
    if (a.G <= 128) return launch_stream<D, BS, KV, 4, 2, true>(a, st);
    return hipErrorInvalidValue;
  }
  if (a.G <= 16) return launch_single<D, BS, KV, 1, 1, 4>(a, st);
  if (a.G <= 32) return launch_single<D, BS, KV, 2, 1, 4>(a, st);
  if (a.G <= 64) return launch_single<D, BS, KV, 2, 2, 2>(a, st);
  if (a.G <= 96) return launch_single<D, BS, KV, 3, 2, 2>(a, st);
  if (a.G <= 128) return launch_single<D, BS, KV, 4, 2, 2>(a, st);
  return hipErrorInvalidValue;
}

template <int KV, int D>
hipError_t launch_attn_inst(const AttnArgs& a, int BS, hipStream_t st) {
  switch (BS) {
    case 16: return launch_group<D, 16, KV>(a, st);
    case 32: return launch_group<D, 32, KV>(a, st);
    case 64: return launch_group<D, 64, KV>(a, st);
    default: return hipErrorInvalidValue;
  }
}

#if defined(PA_INST_KV) && defined(PA_INST_D)
template hipError_t launch_attn_inst<PA_INST_KV, PA_INST_D>(const AttnArgs&, int,
                                                            hipStream_t);
#endif

}  // namespace pa
