// C ABI of the paged decode library: host-side validation and dispatch.
// Declarations, argument meanings, layouts and error behaviour are in
// include/paged_attn.h. Nothing here allocates, synchronises or reads
// device memory.
#include "paged_attn.h"

#include <limits.h>

#include <mutex>

#include "launch.h"

namespace pa {

hipError_t launch_attn(const AttnArgs& a, int D, int BS, int kv, hipStream_t st) {
  if (D == 64) {
    if (kv == kKvF8) return launch_attn_inst<kKvF8, 64>(a, BS, st);
    if (kv == kKvI8) return launch_attn_inst<kKvI8, 64>(a, BS, st);
    return launch_attn_inst<kKvF16, 64>(a, BS, st);
  }
  if (D == 128) {
    if (kv == kKvF8) return launch_attn_inst<kKvF8, 128>(a, BS, st);
    if (kv == kKvI8) return launch_attn_inst<kKvI8, 128>(a, BS, st);
    return launch_attn_inst<kKvF16, 128>(a, BS, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa

namespace {

constexpr float kLog2e = 1.4426950408889634f;

int check_dims(const pa_dims* d) {
  if (!d) return PA_ERR_NULL;
  if (d->num_seqs < 0 || d->num_q_heads <= 0 || d->num_kv_heads <= 0 ||
      d->num_pages <= 0 || d->max_blocks_per_seq <= 0)
    return PA_ERR_SHAPE;
  if (d->num_q_heads % d->num_kv_heads != 0) return PA_ERR_SHAPE;
  if (d->num_q_heads / d->num_kv_heads > 128) return PA_ERR_SHAPE;
  if (d->head_dim != 64 && d->head_dim != 128) return PA_ERR_SHAPE;
  if (d->block_size != 16 && d->block_size != 32 && d->block_size != 64)
    return PA_ERR_SHAPE;
  if ((long long)d->max_blocks_per_seq * d->block_size > INT_MAX)
    return PA_ERR_SHAPE;
  if ((long long)d->num_pages * d->num_kv_heads > INT_MAX) return PA_ERR_SHAPE;
  if (d->kv_dtype != PA_KV_FP16 && d->kv_dtype != PA_KV_FP8_E4M3FN &&
      d->kv_dtype != PA_KV_INT8)
    return PA_ERR_DTYPE;
  return PA_OK;
}

// One-byte caches need their per-kv-head K and V scales.
int check_scales(const pa_dims* d, const float* ks, const float* vs) {
  if (d->kv_dtype != PA_KV_FP16 && (!ks || !vs)) return PA_ERR_DTYPE;
  return PA_OK;
}

// The kernels' cache kind (pa::KvKind) of a pa_kv_dtype.
int kv_kind(const pa_dims* d) {
  switch (d->kv_dtype) {
    case PA_KV_FP8_E4M3FN: return pa::kKvF8;
    case PA_KV_INT8: return pa::kKvI8;
    default: return pa::kKvF16;
  }
}

pa::AttnArgs make_args(const pa_dims* d, const void* q, const void* kp,
                       const void* vp, const int32_t* bt, const int32_t* lens,
                       float scale, const float* ks, const float* vs) {
  pa::AttnArgs a{};
  a.q = static_cast<const _Float16*>(q);
  a.k_pages = static_cast<const uint8_t*>(kp);
  a.v_pages = static_cast<const uint8_t*>(vp);
  a.block_table = bt;
  a.context_lens = lens;
  a.k_scale = ks;
  a.v_scale = vs;
  a.scale_log2 = scale * kLog2e;
  a.B = d->num_seqs;
  a.Hq = d->num_q_heads;
  a.Hkv = d->num_kv_heads;
  a.G = d->num_q_heads / d->num_kv_heads;
  a.P = d->num_pages;
  a.max_blocks = d->max_blocks_per_seq;
  return a;
}

// New tokens appended by the attention kernel itself (paged_decode_step).
struct Fuse {
  const void* k_new;
  const void* v_new;
  const int32_t* positions;
};

void apply_fuse(pa::AttnArgs& a, const Fuse* f) {
  if (!f) return;
  a.k_new = static_cast<const _Float16*>(f->k_new);
  a.v_new = static_cast<const _Float16*>(f->v_new);
  a.positions = f->positions;
}

// Workspace: sem i32 [PA_WORKSPACE_SEM_SLOTS] at a fixed offset (the merged
// call's arrival counters, left zero by every completed call, so a
// workspace can serve calls of any size in turn), then o f32 [B, Hq, S, D],
// lse f32 [B, Hq, S], count i32 [B, Hkv].
static_assert(PA_WORKSPACE_SEM_SLOTS >= pa::kMaxStreamWorkers,
              "one arrival counter per split-pass worker");
constexpr size_t kSemBytes = PA_WORKSPACE_SEM_SLOTS * sizeof(int32_t);

size_t ws_bytes(const pa_dims* d, int32_t S) {
  const size_t rows = (size_t)d->num_seqs * d->num_q_heads * (size_t)S;
  return kSemBytes + rows * (size_t)d->head_dim * sizeof(float) +
         rows * sizeof(float) + (size_t)d->num_seqs * d->num_kv_heads * sizeof(int32_t);
}

struct WsViews {
  float* o;
  float* lse;
  int32_t* count;
  int32_t* sem;
};

WsViews ws_views(const pa_dims* d, int32_t S, void* ws) {
  const size_t rows = (size_t)d->num_seqs * d->num_q_heads * (size_t)S;
  WsViews v;
  v.sem = static_cast<int32_t*>(ws);
  v.o = reinterpret_cast<float*>(static_cast<char*>(ws) + kSemBytes);
  v.lse = v.o + rows * d->head_dim;
  v.count = reinterpret_cast<int32_t*>(v.lse + rows);
  return v;
}

int hip_status(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_HIP; }


int single_impl(const pa_dims* dims, const void* q, const void* k_pages,
                const void* v_pages, const int32_t* block_table,
                const int32_t* context_lens, float scale, const float* k_scale,
                const float* v_scale, void* out, hipStream_t stream,
                const Fuse* fuse) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (!q || !k_pages || !v_pages || !block_table || !context_lens || !out)
    return PA_ERR_NULL;
  rc = check_scales(dims, k_scale, v_scale);
  if (rc) return rc;
  if ((long long)dims->num_seqs * dims->num_kv_heads > INT_MAX) return PA_ERR_SHAPE;
  if (dims->num_seqs == 0) return PA_OK;
  pa::AttnArgs a = make_args(dims, q, k_pages, v_pages, block_table,
                             context_lens, scale, k_scale, v_scale);
  a.out = static_cast<_Float16*>(out);
  a.S = 1;
  a.mode = 0;
  apply_fuse(a, fuse);
  return hip_status(pa::launch_attn(a, dims->head_dim, dims->block_size,
                                    kv_kind(dims), stream));
}


int split_impl(const pa_dims* dims, const void* q, const void* k_pages,
               const void* v_pages, const int32_t* block_table,
               const int32_t* context_lens, float scale, const float* k_scale,
               const float* v_scale, int32_t num_splits, void* workspace,
               size_t workspace_bytes, hipStream_t stream, const Fuse* fuse) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (!q || !k_pages || !v_pages || !block_table || !context_lens)
    return PA_ERR_NULL;
  rc = check_scales(dims, k_scale, v_scale);
  if (rc) return rc;
  if (num_splits < 1 || num_splits > PA_MAX_SPLITS) return PA_ERR_SPLITS;
  if ((long long)dims->num_seqs * dims->num_kv_heads * num_splits > INT_MAX)
    return PA_ERR_SHAPE;
  if (dims->num_seqs == 0) return PA_OK;
  if (!workspace || workspace_bytes < ws_bytes(dims, num_splits))
    return PA_ERR_WORKSPACE;
  pa::AttnArgs a = make_args(dims, q, k_pages, v_pages, block_table,
                             context_lens, scale, k_scale, v_scale);
  const WsViews v = ws_views(dims, num_splits, workspace);
  a.ws_o = v.o;
  a.ws_lse = v.lse;
  a.ws_count = v.count;
  a.ws_sem = v.sem;
  a.S = num_splits;
  a.mode = num_splits == 1 ? 1 : 2;
  apply_fuse(a, fuse);
  return hip_status(pa::launch_attn(a, dims->head_dim, dims->block_size,
                                    kv_kind(dims), stream));
}

// Largest group size (q heads per kv head) whose partials the merged call
// merges inside the attention kernel.
constexpr int kMergeInKernelMaxGroup = 16;

// Most (sequence, kv head) pairs for which paged_decode_step appends inside
// the attention kernel. Each worker owning a new token's tile writes it and
// waits for the stores before its first tile load; with a pair for nearly
// every worker that start-up wait on every worker costs more than one
// separate append launch (measured on MI355X: fused ahead by 2-14 us up to
// 1024 pairs, behind by 1-9 us at 2048).
constexpr long long kFuseAppendMaxPairs = 1536;

// Argument checks of the merged call, all done before anything is launched.
int check_merged(const pa_dims* dims, const void* q, const void* k_pages,
                 const void* v_pages, const int32_t* block_table,
                 const int32_t* context_lens, const float* k_scale,
                 const float* v_scale, int32_t num_splits, const void* workspace,
                 size_t workspace_bytes, const void* out) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (!q || !k_pages || !v_pages || !block_table || !context_lens || !out)
    return PA_ERR_NULL;
  rc = check_scales(dims, k_scale, v_scale);
  if (rc) return rc;
  if (num_splits < 1 || num_splits > PA_MAX_SPLITS) return PA_ERR_SPLITS;
  if ((long long)dims->num_seqs * dims->num_kv_heads * num_splits > INT_MAX)
    return PA_ERR_SHAPE;
  if (dims->num_seqs > 0 && num_splits > 1 &&
      (!workspace || workspace_bytes < ws_bytes(dims, num_splits)))
    return PA_ERR_WORKSPACE;
  return PA_OK;
}

int merged_impl(const pa_dims* dims, const void* q, const void* k_pages,
                const void* v_pages, const int32_t* block_table,
                const int32_t* context_lens, float scale, const float* k_scale,
                const float* v_scale, int32_t num_splits, void* workspace,
                size_t workspace_bytes, void* out, hipStream_t stream,
                const Fuse* fuse) {
  int rc = check_merged(dims, q, k_pages, v_pages, block_table, context_lens,
                        k_scale, v_scale, num_splits, workspace,
                        workspace_bytes, out);
  if (rc) return rc;
  if (dims->num_seqs == 0) return PA_OK;
  if (num_splits == 1)   // one range per (sequence, kv head): the single pass
    return single_impl(dims, q, k_pages, v_pages, block_table, context_lens,
                       scale, k_scale, v_scale, out, stream, fuse);
  if (dims->num_q_heads / dims->num_kv_heads > kMergeInKernelMaxGroup) {
    // wide groups: one wave cannot merge G heads quickly; the reduce kernel
    // spreads the merge over a wave per (sequence, q head)
    rc = split_impl(dims, q, k_pages, v_pages, block_table, context_lens, scale,
                    k_scale, v_scale, num_splits, workspace, workspace_bytes,
                    stream, fuse);
    if (rc) return rc;
    return paged_decode_attn_splitk_reduce(dims, context_lens, num_splits,
                                           workspace, workspace_bytes, out, stream);
  }
  pa::AttnArgs a = make_args(dims, q, k_pages, v_pages, block_table,
                             context_lens, scale, k_scale, v_scale);
  const WsViews v = ws_views(dims, num_splits, workspace);
  a.ws_o = v.o;
  a.ws_lse = v.lse;
  a.ws_count = v.count;
  a.ws_sem = v.sem;
  a.out = static_cast<_Float16*>(out);
  a.S = num_splits;
  a.mode = 3;
  apply_fuse(a, fuse);
  return hip_status(pa::launch_attn(a, dims->head_dim, dims->block_size,
                                    kv_kind(dims), stream));
}

}  // namespace

// ---------------------------------------------------------------------------
// Library-owned scratch for paged_decode_step_static: the split workspace
// (arrival counters, partials, counts) of callers that cannot allocate. One
// copy per GPU (a __device__ array lives in every device's copy of the code
// object). Host code never uses the array's name as an address: each
// device's copy is looked up once with hipGetSymbolAddress and that pointer
// is what the kernels receive.
static __device__ __align__(256) unsigned char scratch[PA_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];        // device address of `scratch`, per GPU

__global__ void zero_words_kernel(int32_t* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
    p[i] = 0;
}

// The current GPU's copy of `scratch`. On the first use on a GPU: look it up
// and enqueue a clear of its arrival counters on `stream` (a kernel, so that
// the clear is valid inside a graph capture too).
int scratch_for_current_device(void** out, hipStream_t stream) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return PA_ERR_HIP;
    hipLaunchKernelGGL(zero_words_kernel, 8, 256, 0, stream, static_cast<int32_t*>(p),
                       PA_WORKSPACE_SEM_SLOTS);
    if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PA_OK;
}

}  // namespace

extern "C" {

int kv_append(const pa_dims* dims, int32_t num_tokens, const void* k_new,
              const void* v_new, const int32_t* seq_ids,
              const int32_t* positions, const int32_t* block_table,
              const float* k_scale, const float* v_scale, void* k_pages,
              void* v_pages, hipStream_t stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (num_tokens < 0) return PA_ERR_SHAPE;
  if (!seq_ids && num_tokens > dims->num_seqs) return PA_ERR_SHAPE;
  if ((long long)num_tokens * dims->num_kv_heads * (dims->head_dim / 2) >
      (long long)INT_MAX * 256)
    return PA_ERR_SHAPE;
  if (!k_new || !v_new || !positions || !block_table || !k_pages || !v_pages)
    return PA_ERR_NULL;
  rc = check_scales(dims, k_scale, v_scale);
  if (rc) return rc;
  if (num_tokens == 0 || dims->num_seqs == 0) return PA_OK;
  pa::KvAppendArgs a{};
  a.k_new = static_cast<const uint8_t*>(k_new);
  a.v_new = static_cast<const uint8_t*>(v_new);
  a.seq_ids = seq_ids;
  a.positions = positions;
  a.block_table = block_table;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.k_pages = static_cast<uint8_t*>(k_pages);
  a.v_pages = static_cast<uint8_t*>(v_pages);
  a.num_tokens = num_tokens;
  a.B = dims->num_seqs;
  a.Hkv = dims->num_kv_heads;
  a.bs = dims->block_size;
  a.P = dims->num_pages;
  a.max_blocks = dims->max_blocks_per_seq;
  return hip_status(pa::launch_kv_append(a, dims->head_dim, kv_kind(dims), stream));
}


int paged_decode_attn(const pa_dims* dims, const void* q, const void* k_pages,
                      const void* v_pages, const int32_t* block_table,
                      const int32_t* context_lens, float scale,
                      const float* k_scale, const float* v_scale, void* out,
                      hipStream_t stream) {
  return single_impl(dims, q, k_pages, v_pages, block_table, context_lens,
                     scale, k_scale, v_scale, out, stream, nullptr);
}

size_t paged_decode_attn_splitk_workspace_size(const pa_dims* dims,
                                               int32_t num_splits) {
  if (check_dims(dims) != PA_OK) return 0;
  if (num_splits < 1 || num_splits > PA_MAX_SPLITS) return 0;
  return ws_bytes(dims, num_splits);
}


int paged_decode_attn_splitk(const pa_dims* dims, const void* q,
                             const void* k_pages, const void* v_pages,
                             const int32_t* block_table,
                             const int32_t* context_lens, float scale,
                             const float* k_scale, const float* v_scale,
                             int32_t num_splits, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  return split_impl(dims, q, k_pages, v_pages, block_table, context_lens, scale,
                    k_scale, v_scale, num_splits, workspace, workspace_bytes,
                    stream, nullptr);
}

// Largest group size (q heads per kv head) whose partials the merged call
// merges inside the attention kernel.

int paged_decode_attn_splitk_merged(const pa_dims* dims, const void* q,
                                    const void* k_pages, const void* v_pages,
                                    const int32_t* block_table,
                                    const int32_t* context_lens, float scale,
                                    const float* k_scale, const float* v_scale,
                                    int32_t num_splits, void* workspace,
                                    size_t workspace_bytes, void* out,
                                    hipStream_t stream) {
  return merged_impl(dims, q, k_pages, v_pages, block_table, context_lens,
                     scale, k_scale, v_scale, num_splits, workspace,
                     workspace_bytes, out, stream, nullptr);
}

int paged_decode_step(const pa_dims* dims, const void* q, const void* k_new,
                      const void* v_new, const int32_t* positions,
                      void* k_pages, void* v_pages, const int32_t* block_table,
                      const int32_t* context_lens, float scale,
                      const float* k_scale, const float* v_scale,
                      int32_t num_splits, void* workspace,
                      size_t workspace_bytes, void* out, hipStream_t stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (!k_new || !v_new || !positions) return PA_ERR_NULL;
  if (!paged_decode_step_fuses_append(dims)) {
    // many pairs: the append as its own launch, then the merged call (the
    // same bytes and the same output as the fused form)
    rc = check_merged(dims, q, k_pages, v_pages, block_table, context_lens,
                      k_scale, v_scale, num_splits, workspace, workspace_bytes,
                      out);
    if (rc) return rc;
    rc = kv_append(dims, dims->num_seqs, k_new, v_new, nullptr, positions,
                   block_table, k_scale, v_scale, k_pages, v_pages, stream);
    if (rc) return rc;
    return merged_impl(dims, q, k_pages, v_pages, block_table, context_lens,
                       scale, k_scale, v_scale, num_splits, workspace,
                       workspace_bytes, out, stream, nullptr);
  }
  const Fuse f{k_new, v_new, positions};
  return merged_impl(dims, q, k_pages, v_pages, block_table, context_lens,
                     scale, k_scale, v_scale, num_splits, workspace,
                     workspace_bytes, out, stream, &f);
}

int paged_decode_attn_splitk_reduce(const pa_dims* dims,
                                    const int32_t* context_lens,
                                    int32_t num_splits, const void* workspace,
                                    size_t workspace_bytes, void* out,
                                    hipStream_t stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (!out || !context_lens) return PA_ERR_NULL;
  if (num_splits < 1 || num_splits > PA_MAX_SPLITS) return PA_ERR_SPLITS;
  if ((long long)dims->num_seqs * dims->num_q_heads > INT_MAX) return PA_ERR_SHAPE;
  if (dims->num_seqs == 0) return PA_OK;
  if (!workspace || workspace_bytes < ws_bytes(dims, num_splits))
    return PA_ERR_WORKSPACE;
  pa::ReduceArgs a{};
  const WsViews v = ws_views(dims, num_splits, const_cast<void*>(workspace));
  a.ws_o = v.o;
  a.ws_lse = v.lse;
  a.ws_count = v.count;
  a.context_lens = context_lens;
  a.out = static_cast<_Float16*>(out);
  a.B = dims->num_seqs;
  a.Hq = dims->num_q_heads;
  a.Hkv = dims->num_kv_heads;
  a.G = dims->num_q_heads / dims->num_kv_heads;
  a.S = num_splits;
  a.cap = dims->max_blocks_per_seq * dims->block_size;
  return hip_status(pa::launch_reduce(a, dims->head_dim, stream));
}


int paged_decode_advance(const pa_dims* dims, int32_t* context_lens, int32_t* positions,
                         hipStream_t stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (!context_lens || !positions) return PA_ERR_NULL;
  if (dims->num_seqs == 0) return PA_OK;
  return hip_status(pa::launch_advance(context_lens, positions, dims->num_seqs,
                                       dims->max_blocks_per_seq * dims->block_size, stream));
}

int paged_decode_step_static(const pa_dims* dims, const void* q,
                             const void* k_new, const void* v_new,
                             const int32_t* positions, void* k_pages,
                             void* v_pages, const int32_t* block_table,
                             const int32_t* context_lens, float scale,
                             const float* k_scale, const float* v_scale,
                             int32_t num_splits, void* out, hipStream_t stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (num_splits < 1 || num_splits > PA_MAX_SPLITS) return PA_ERR_SPLITS;
  const size_t need = num_splits > 1 ? ws_bytes(dims, num_splits) : 0;
  if (need > PA_STATIC_SCRATCH_BYTES) return PA_ERR_SCRATCH;
  // every other argument is checked before the scratch is touched
  rc = check_merged(dims, q, k_pages, v_pages, block_table, context_lens, k_scale,
                    v_scale, num_splits, nullptr, 0, out);
  if (rc && rc != PA_ERR_WORKSPACE) return rc;
  if (!k_new || !v_new || !positions) return PA_ERR_NULL;
  void* ws = nullptr;
  if (dims->num_seqs > 0 && num_splits > 1) {
    rc = scratch_for_current_device(&ws, stream);
    if (rc) return rc;
  }
  return paged_decode_step(dims, q, k_new, v_new, positions, k_pages, v_pages,
                           block_table, context_lens, scale, k_scale, v_scale,
                           num_splits, ws, PA_STATIC_SCRATCH_BYTES, out, stream);
}

int32_t paged_decode_step_fuses_append(const pa_dims* dims) {
  const int rc = check_dims(dims);
  if (rc) return rc;
  return (long long)dims->num_seqs * dims->num_kv_heads <= kFuseAppendMaxPairs;
}

int32_t paged_decode_attn_suggest_splits(const pa_dims* dims,
                                         int32_t max_context_len) {
  if (check_dims(dims) != PA_OK || max_context_len <= 0) return 1;
  // The split pass spreads the batch's 32-token tiles evenly over a
  // persistent grid of W workers (<= 16 q heads per kv head: 1024 for fp16,
  // 2048 for one-byte caches; 1024 up to 64; else 512); the longest (sequence, kv head)
  // then spans about
  // n_max * W / T + 1 of them. Assuming the batch's mean context is at
  // least 1/16 of the longest (T >= pairs * n_max / 16) gives the bound.
  const int G = dims->num_q_heads / dims->num_kv_heads;
  const long long W = G <= 16 ? (dims->kv_dtype != PA_KV_FP16 ? 2048 : 1024)
                              : (G <= 64 ? 1024 : 512);
  const long long tiles = (max_context_len + 31) / 32;
  const long long pairs = (long long)dims->num_seqs * dims->num_kv_heads;
  if (tiles <= 1 || pairs <= 0) return 1;
  long long S = (16 * W + pairs - 1) / pairs + 1;
  if (S > 64) S = 64;
  if (S > tiles + 1) S = tiles + 1;
  if (S < 2) S = 2;
  return (int32_t)S;
}

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "a required pointer is NULL";
    case PA_ERR_SHAPE: return "unsupported or inconsistent sizes";
    case PA_ERR_DTYPE: return "unknown kv dtype or fp8 scales missing";
    case PA_ERR_SPLITS: return "num_splits outside [1, PA_MAX_SPLITS]";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_HIP: return "HIP kernel launch failed";
    case PA_ERR_SCRATCH: return "the call needs more than the library's static scratch";
    default: return "unknown status";
  }
}

int32_t pa_version(void) { return 100; }

}  // extern "C"
