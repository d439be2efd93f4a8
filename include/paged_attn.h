/*
 * paged_attn.h — C ABI of the MI355X (gfx950) paged MQA/GQA decode library.
 *
 * What the library computes (one new token per sequence, decode phase):
 *
 *   for every sequence b and query head j, with G = Hq / Hkv and h = j / G,
 *     out[b, j, :] = softmax_t( scale * q[b, j, :] . K_h[t, :] ) . V_h[t, :]
 *   over the tokens t = 0 .. context_lens[b]-1 of that sequence, where K_h
 *   and V_h are gathered page by page through the sequence's block table.
 *
 * Sources (page title, section):
 *   - "TensorRT对Multi-Query Attention的专项优化支持" (r-odyssey.com/news/246352):
 *     the MHA and MQA formulas (query heads keep their own projection, the
 *     K/V projection is shared); decode re-reads the whole K/V cache for
 *     every new token; the cache cut into fixed-length pages.
 *   - "优化" on tiny-llm (open-infra-ai.github.io/tiny-llm/performance/
 *     optimization): section 3, kv heads may be fewer than q heads (GQA);
 *     roadmap table, row 分页 KV (block table, scatter on append, gather on
 *     read) and row FlashDecoding (long-context decode attention).
 *   - same tiny-llm page, section 2: the per-sequence KV size
 *     2 x layers x kv_heads x head_dim x max_seq_len x bytes.
 * The pages fix no memory layout, head-to-group map, split rule or
 * one-byte code format; the choices below are this library's.
 *
 * Conventions for every entry point
 *   - Tensor arguments are DEVICE pointers owned by the caller; `dims` is a
 *     HOST pointer read during the call only. The library allocates nothing,
 *     keeps no state between calls and never synchronises: all work is
 *     enqueued on `stream` (0 = the null stream) in call order.
 *   - Return value: PA_OK (0) on success, a negative PA_ERR_* code otherwise.
 *     Arguments are validated on the host BEFORE anything is enqueued; on
 *     error nothing is enqueued and no output is touched. PA_ERR_HIP means
 *     the launch itself failed (hipGetLastError after the launch).
 *   - Device-data contracts (not checked on the host, which never reads
 *     device memory): for every sequence, block_table entries 0 ..
 *     ceil(L/bs)-1 are page ids in [0, num_pages), and 0 <= L <=
 *     max_blocks_per_seq * block_size. Kernels clamp L into that range and
 *     page ids into [0, num_pages), so a bad table can give wrong numbers
 *     but never reads or writes outside the caller's buffers.
 *   - Supported shapes: head_dim 64 or 128; block_size 16, 32 or 64;
 *     num_q_heads a multiple of num_kv_heads with G = Hq/Hkv <= 128.
 *
 * Memory layouts (densely packed):
 *   q, out          [B, Hq, d]            fp16, row-major
 *   k_pages,v_pages [P, Hkv, bs * d]      one tile of bs * d elements per
 *                                         (page, kv head), in the order below
 *   block_table     [B, max_blocks_per_seq] int32 page ids
 *   context_lens    [B]                   int32 tokens per sequence
 *   k_scale,v_scale [Hkv]                 fp32, one-byte caches only (else NULL)
 * Inside a tile, slot t (0 <= t < bs) and dimension i (0 <= i < d) sit at
 * element offset, with blk = t / 16, r = t % 16, rho(r) = r with its bits
 * 2 and 3 swapped, and X = 16 bytes / element size (8 for fp16, 16 for the
 * one-byte codes):
 *   K:  ((blk * (d / X) + i / X) * 16 + rho(r)) * X + i % X
 *   V:  (((blk * (d / 16) + i / 16) * 2 + r / 8) * 16 + i % 16) * 8 + r % 8
 * i.e. each 16-token block stores K as 16-byte chunks of one token's row,
 * chunk-major, with slots 0-3, 8-11 in the first 8 rows and 4-7, 12-15 in
 * the last 8; and V as runs of 8 tokens of one dimension. This is the order
 * in which the kernels' matrix-core operands are loaded: a lane's V operand
 * is one 16-byte (fp16) or 8-byte (one-byte codes) run and every wave-wide
 * load reads whole 128-byte lines. A page pool may be allocated as
 * [P, Hkv, bs, d] (the binding does), but its last two axes are storage, not
 * a [token, dim] matrix. Caches are written through kv_append.
 * fp8 caches hold OCP E4M3FN codes (1 byte, max 448, no infinities); int8
 * caches hold symmetric codes in [-127, 127] (two's complement bytes; -128
 * is never written); in both the value of a code is decode(code) *
 * scale[h], with one scale per kv head for K and another for V. Device
 * buffers must be 16-byte aligned (q, k_pages, v_pages, out, workspace) or
 * 4-byte aligned (k_new, v_new, index arrays, scales).
 */
#ifndef PAGED_ATTN_H
#define PAGED_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum pa_kv_dtype {
  PA_KV_FP16 = 0,        /* IEEE binary16 */
  PA_KV_FP8_E4M3FN = 1,  /* OCP E4M3FN code + per-kv-head fp32 scale */
  PA_KV_INT8 = 2,        /* symmetric int8 code + per-kv-head fp32 scale */
};

enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL = -1,       /* a required pointer is NULL */
  PA_ERR_SHAPE = -2,      /* unsupported or inconsistent sizes */
  PA_ERR_DTYPE = -3,      /* unknown kv_dtype, or scales missing for a
                             one-byte cache */
  PA_ERR_SPLITS = -4,     /* num_splits outside [1, PA_MAX_SPLITS] */
  PA_ERR_WORKSPACE = -5,  /* workspace NULL or smaller than required */
  PA_ERR_HIP = -6,        /* the kernel launch failed */
  PA_ERR_SCRATCH = -7,    /* the call needs more than the library's static
                             scratch (PA_STATIC_SCRATCH_BYTES) */
};

#define PA_MAX_SPLITS 1024
/* Arrival counters at the start of every split workspace (see below). */
#define PA_WORKSPACE_SEM_SLOTS 2048
/* Size of the library's own device scratch (paged_decode_step_static). */
#define PA_STATIC_SCRATCH_BYTES (32u << 20)

/* Sizes shared by every call on one cache. num_seqs may be 0 (no work). */
typedef struct pa_dims {
  int32_t num_seqs;            /* B   */
  int32_t num_q_heads;         /* Hq  */
  int32_t num_kv_heads;        /* Hkv */
  int32_t head_dim;            /* d   */
  int32_t block_size;          /* bs, tokens per page */
  int32_t num_pages;           /* P, pages in each of k_pages / v_pages */
  int32_t max_blocks_per_seq;  /* row length of block_table */
  int32_t kv_dtype;            /* enum pa_kv_dtype */
} pa_dims;

/*
 * kv_append — scatter new tokens' K and V into their pages.
 *
 * Source: tiny-llm "优化", roadmap row 分页 KV (scatter through the block
 * table on write) and section 5 (the append position is a per-step device
 * value); per-tensor K/V scales: "TensorRT对Multi-Query Attention的专项优化
 * 支持", quantisation paragraph.
 *
 * Token i (0 <= i < num_tokens) belongs to sequence s = seq_ids[i] (or
 * s = i when seq_ids is NULL, which requires num_tokens <= num_seqs) and
 * position p = positions[i]; its row k_new[i, h, :] is stored in the tile
 * (block_table[s, p / bs], h) of k_pages at slot p % bs (positions per the
 * layout above), v_new[i, h, :] likewise in v_pages.
 *   k_new, v_new : [num_tokens, Hkv, d] fp16, device
 *   fp16 cache   : the fp16 bits are copied unchanged
 *   fp8 cache    : code = RNE_e4m3fn(float(x) / k_scale[h]) (IEEE fp32
 *                  division; magnitudes >= 448 saturate to +-448, NaN -> 0x7F)
 *   int8 cache   : code = clamp(round_half_even(float(x) / k_scale[h]),
 *                  -127, 127) (IEEE fp32 division; NaN -> 0)
 * Only the addressed slots are written. Two tokens addressing one slot is
 * undefined. positions[i] must be < max_blocks_per_seq * bs (out-of-range
 * positions or sequence ids are skipped).
 */
int kv_append(const pa_dims* dims, int32_t num_tokens,
              const void* k_new, const void* v_new,
              const int32_t* seq_ids, const int32_t* positions,
              const int32_t* block_table,
              const float* k_scale, const float* v_scale,
              void* k_pages, void* v_pages, hipStream_t stream);

/*
 * paged_decode_attn — single-pass decode attention.
 *
 * Source: MHA/MQA formulas and the decode re-read paragraph of
 * "TensorRT对Multi-Query Attention的专项优化支持"; GQA (section 3) and the
 * paged gather (roadmap row 分页 KV) of tiny-llm "优化".
 *
 * One workgroup per (sequence, kv head) covers that sequence's whole
 * context; `out` [B, Hq, d] fp16 receives the normalised result, rounded
 * to nearest even. Sequences with L = 0 get zeros. `scale` multiplies
 * q . k (typically 1/sqrt(d)). k_scale / v_scale: one-byte caches only.
 */
int paged_decode_attn(const pa_dims* dims, const void* q,
                      const void* k_pages, const void* v_pages,
                      const int32_t* block_table, const int32_t* context_lens,
                      float scale, const float* k_scale, const float* v_scale,
                      void* out, hipStream_t stream);

/*
 * Workspace bytes needed by paged_decode_attn_splitk and
 * paged_decode_attn_splitk_merged for num_splits partial slots per
 * (sequence, q head). Layout, densely packed in this order:
 *   sem   int32   [PA_WORKSPACE_SEM_SLOTS]  arrival counters of the merged
 *                                 call, at the same place for every dims and
 *                                 num_splits: zero before the workspace's
 *                                 first use (zero-fill it once); every
 *                                 completed merged call leaves them zero, so
 *                                 one workspace serves calls of any size in
 *                                 turn (each within its own size)
 *   o     float32 [B, Hq, S, d]   normalised partial outputs
 *   lse   float32 [B, Hq, S]      natural-log sum of exp(scores) per partial
 *   count int32   [B, Hkv]        partials written for (sequence, kv head)
 * Returns 0 for invalid dims or num_splits.
 */
size_t paged_decode_attn_splitk_workspace_size(const pa_dims* dims,
                                               int32_t num_splits);

/*
 * paged_decode_attn_splitk — first pass of split decode attention.
 *
 * Source: tiny-llm "优化", roadmap row FlashDecoding (long-context decode
 * attention split over the context; the page names it only). The split
 * is this library's: the 32-token tiles of every (sequence, kv head)
 * context, laid end to end (sequence-major, then kv head, then position),
 * are cut into equal contiguous shares, one per workgroup of a persistent
 * grid, so a ragged batch spreads evenly over the chip. Each (sequence,
 * kv head) thereby falls into 1..S contiguous token ranges (the share is
 * widened when needed so that S is never exceeded); for its i-th range
 * the call writes o[b, j, i, :] (that range's softmax-weighted mean of V)
 * and lse[b, j, i] = ln(sum over the range of exp(scale * q . k_t)) for
 * every q head j of the group, and count[b, h] = number of ranges.
 * Sequences with L = 0 get no ranges (count is then not written).
 * num_splits == 1 gives one range per (sequence, kv head): the whole
 * context. num_splits >= 2 should be large enough for the longest context
 * to span several shares (see paged_decode_attn_suggest_splits); a smaller
 * value stays correct but leaves part of the grid idle.
 */
int paged_decode_attn_splitk(const pa_dims* dims, const void* q,
                             const void* k_pages, const void* v_pages,
                             const int32_t* block_table,
                             const int32_t* context_lens, float scale,
                             const float* k_scale, const float* v_scale,
                             int32_t num_splits, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

/*
 * paged_decode_attn_splitk_reduce — log-sum-exp merge of the ranges.
 *
 *   out[b, j, :] = sum_i w_i o[b, j, i, :] / sum_i w_i,
 *   w_i = exp(lse[b, j, i] - max_k lse[b, j, k]),  i < count[b, j / G];
 * sequences with context_lens[b] = 0 get zeros. Reads the workspace that
 * paged_decode_attn_splitk wrote with the same dims, context_lens and
 * num_splits (enqueue it after that call on the same stream); writes
 * out [B, Hq, d] fp16, rounded to nearest even.
 */
int paged_decode_attn_splitk_reduce(const pa_dims* dims,
                                    const int32_t* context_lens,
                                    int32_t num_splits, const void* workspace,
                                    size_t workspace_bytes, void* out,
                                    hipStream_t stream);

/*
 * paged_decode_attn_splitk_merged — split decode attention in one call.
 *
 * Same split as paged_decode_attn_splitk (ranges of the batch's tiles over
 * a persistent grid, at most num_splits per (sequence, kv head)), with the
 * log-sum-exp merge done in the same kernel when the group has at most 16
 * q heads: a (sequence, kv head) covered by one worker is normalised and
 * written straight to `out`; otherwise each of its workers writes its
 * partial to the workspace with device-scope (write-through) stores, waits
 * for them to complete, and counts its arrival on sem[b, h] with a
 * device-scope atomic; the last to arrive reads the partials with
 * device-scope loads, merges them into `out` and resets sem[b, h] to zero.
 * Larger groups run paged_decode_attn_splitk and then
 * paged_decode_attn_splitk_reduce on the same stream. out [B, Hq, d] fp16
 * is the same result as paged_decode_attn up to rounding; sequences with
 * L = 0 get zeros. Two merged calls that share one workspace must not run
 * concurrently. num_splits == 1 runs paged_decode_attn (workspace unused).
 */
int paged_decode_attn_splitk_merged(const pa_dims* dims, const void* q,
                                    const void* k_pages, const void* v_pages,
                                    const int32_t* block_table,
                                    const int32_t* context_lens, float scale,
                                    const float* k_scale, const float* v_scale,
                                    int32_t num_splits, void* workspace,
                                    size_t workspace_bytes, void* out,
                                    hipStream_t stream);

/*
 * paged_decode_step — one decode step: kv_append of every sequence's new
 * token, then paged_decode_attn_splitk_merged over the updated cache, with
 * the append done inside the attention kernel (one launch for groups of at
 * most 16 q heads; the reduce kernel follows for wider groups). Above 1536
 * (sequence, kv head) pairs the append is a launch of its own ahead of the
 * attention, where that is faster; every argument is checked before either
 * launch, so a rejected call writes nothing.
 *
 * Source: tiny-llm "优化", roadmap rows 分页 KV (the append is a scatter
 * through the block table) and FlashDecoding, and section 5 (the append
 * position of a decode step is a device value); "TensorRT对Multi-Query
 * Attention的专项优化支持", decode paragraph (each step appends one K/V row
 * per head and attends over all of them). Fusing the two is this library's.
 *
 * k_new, v_new: fp16 [B, Hkv, d] device; positions: int32 [B] device, the
 * slot of sequence b's new token (normally context_lens[b] - 1; negative or
 * beyond the table's capacity: no append). The result equals kv_append with
 * seq_ids = NULL followed by paged_decode_attn_splitk_merged on the same
 * arguments: the same cache bytes and the same output bits. The worker that
 * reads the new token's tile writes it first, so no ordering is needed
 * between sequences; a position inside the attended context other than its
 * last token is allowed. Errors as paged_decode_attn_splitk_merged, plus
 * PA_ERR_NULL for a missing k_new, v_new or positions.
 */
int paged_decode_step(const pa_dims* dims, const void* q, const void* k_new,
                      const void* v_new, const int32_t* positions,
                      void* k_pages, void* v_pages, const int32_t* block_table,
                      const int32_t* context_lens, float scale,
                      const float* k_scale, const float* v_scale,
                      int32_t num_splits, void* workspace,
                      size_t workspace_bytes, void* out, hipStream_t stream);

/*
 * paged_decode_advance — move a batch on by one decode step, on the device.
 *
 * Source: tiny-llm "优化", section 5 (the decode sequence is captured as a
 * graph; the values that change from step to step, such as the visible
 * length and the append position, are device ints in fixed buffers, so the
 * same graph replays every step).
 *
 * For every sequence b with positions[b] >= 0 (a live slot): positions[b]
 * += 1 and context_lens[b] += 1, so that paged_decode_step called again
 * with the next token's q, k_new and v_new appends it after the previous
 * one and attends over one more token. A slot whose next position would be
 * at or past max_blocks_per_seq * block_size gets positions[b] = -1 (no
 * further appends) and keeps its length. Slots with positions[b] < 0 are
 * left alone. Captured after paged_decode_step in one graph, a replay is
 * one whole decode step. The pages the next positions fall in must already
 * be in the block table (a caller reserving ahead, such as the page manager
 * below, writes them before the replays).
 *   context_lens, positions: int32 [B], device, read and written.
 */
int paged_decode_advance(const pa_dims* dims, int32_t* context_lens,
                         int32_t* positions, hipStream_t stream);

/*
 * paged_decode_step_static — paged_decode_step without a caller workspace,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Same arguments and result as paged_decode_step minus workspace and
 * workspace_bytes: the split partials and arrival counters live in a
 * library-owned device array of PA_STATIC_SCRATCH_BYTES (32 MiB), one per
 * GPU, held from the library's first use on that GPU until the process
 * ends. Nothing is allocated by the call. The first call on a GPU looks up
 * that GPU's copy of the array and enqueues a clear of its arrival counters
 * on `stream`; every completed call leaves them zero again.
 * Calls whose paged_decode_attn_splitk_workspace_size(dims, num_splits)
 * exceeds PA_STATIC_SCRATCH_BYTES return PA_ERR_SCRATCH before anything is
 * enqueued. All calls on one GPU share the array: two calls that may run at
 * the same time on one GPU (different streams, or different threads without
 * ordering) race and give wrong results; order them on one stream.
 */
int paged_decode_step_static(const pa_dims* dims, const void* q,
                             const void* k_new, const void* v_new,
                             const int32_t* positions, void* k_pages,
                             void* v_pages, const int32_t* block_table,
                             const int32_t* context_lens, float scale,
                             const float* k_scale, const float* v_scale,
                             int32_t num_splits, void* out, hipStream_t stream);

/* 1 when paged_decode_step with these dims appends inside the attention
 * kernel, 0 when it issues the append as a launch of its own first (more
 * than 1536 (sequence, kv head) pairs); a negative status for invalid dims.
 * Lets a caller time or profile the attention launch on its own. */
int32_t paged_decode_step_fuses_append(const pa_dims* dims);

/* num_splits the library suggests for a batch whose longest context is
 * max_context_len tokens, assuming the batch's mean context is at least
 * 1/16 of the longest (1 when a single tile covers every context). */
int32_t paged_decode_attn_suggest_splits(const pa_dims* dims,
                                         int32_t max_context_len);

/* Static description of a status code. Never NULL. */
const char* pa_status_string(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int32_t pa_version(void);

#ifdef __cplusplus
}
#endif
#endif /* PAGED_ATTN_H */
