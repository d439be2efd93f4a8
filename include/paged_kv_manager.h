/*
 * paged_kv_manager.h — host-side page manager for the paged KV cache of
 * libpagedattn: a fixed pool of pages handed out to batch slots through a
 * free list, and the per-step batch arrays (block table, context lengths,
 * append positions) that the decode calls of paged_attn.h take.
 *
 * Sources (page title, section):
 *   - "优化" on tiny-llm (open-infra-ai.github.io/tiny-llm/performance/
 *     optimization), section 2: the KV cache is allocated once, up front,
 *     from a configuration (layers, heads, head_dim, max_seq_len, batch), so
 *     the decode phase never allocates and the memory bound is known at
 *     start-up; per-sequence KV bytes = 2 x layers x kv_heads x head_dim x
 *     max_seq_len x bytes per element; the memory-estimate table (KV cache =
 *     that times the batch). Roadmap rows 分页 KV (block table + scatter /
 *     gather) and 连续批处理 (continuous batching).
 *   - "TensorRT对Multi-Query Attention的专项优化支持", KV-cache paragraph:
 *     the cache is cut into fixed-length pages that are handed out on demand.
 *   - zyxy.net tag page "tensorrt", in-flight batching abstract: sequences
 *     join and leave a running batch between steps.
 *
 * Model: the caller allocates the device pools once (pa_kv_pool_bytes gives
 * their size). The manager owns only host bookkeeping: which pages are free,
 * which pages each of num_slots batch slots holds, and each slot's length.
 * A batch is the fixed set of num_slots slots (the B of pa_dims); a free
 * slot takes part in a decode call as a sequence of length 0 with append
 * position -1 (the kernels skip it), so the batch shape never changes and a
 * captured decode graph stays valid while sequences come and go.
 *
 * Block-table rows: entry i of a slot's row is the page holding its tokens
 * [i * block_size, (i + 1) * block_size); entries past the pages the slot
 * holds are -1. Pages are handed out from the free list in the order they
 * were freed (last freed, first reused; initially 0, 1, 2, ...).
 *
 * Errors: the PA_ERR_* codes of paged_attn.h plus the two below. A call that
 * fails changes nothing. The manager is not thread-safe: use it from one
 * thread (or lock around it). It never touches the GPU.
 */
#ifndef PAGED_KV_MANAGER_H
#define PAGED_KV_MANAGER_H

#include <stdint.h>

#include "paged_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ERR_NO_PAGES (-8) /* not enough free pages for the request */
#define PA_ERR_NO_SLOT (-9)  /* no free batch slot, or not a live slot */

/* Bytes of one element of a cache of kv_dtype (2 for fp16, 1 for the
 * one-byte codes); 0 for an unknown dtype. */
int32_t pa_kv_elem_bytes(int32_t kv_dtype);

/* KV bytes one sequence of max_seq_len tokens needs over num_layers layers:
 * 2 (K and V) x num_layers x num_kv_heads x head_dim x max_seq_len x
 * element bytes (tiny-llm "优化", section 2). -1 for invalid arguments. */
int64_t pa_kv_bytes_per_sequence(int32_t num_layers, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_seq_len,
                                 int32_t kv_dtype);

/* Bytes of one layer's K pool plus its V pool of num_pages pages
 * ([P, Hkv, block_size, head_dim] each). -1 for invalid arguments. */
int64_t pa_kv_pool_bytes(int32_t num_pages, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, int32_t kv_dtype);

/* Most pages whose K and V pools for num_layers layers fit in budget_bytes
 * (at most INT32_MAX); -1 for invalid arguments. */
int64_t pa_kv_pages_for_budget(int64_t budget_bytes, int32_t num_layers,
                               int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, int32_t kv_dtype);

typedef struct pa_kv_manager pa_kv_manager;

/* A manager of num_pages pages of block_size tokens for num_slots batch
 * slots whose rows hold max_blocks_per_seq entries. NULL for invalid sizes
 * (any < 1, block_size not 16/32/64) or when out of host memory. */
pa_kv_manager* pa_kvm_create(int32_t num_pages, int32_t block_size,
                             int32_t num_slots, int32_t max_blocks_per_seq);
void pa_kvm_destroy(pa_kv_manager* m);

int32_t pa_kvm_free_pages(const pa_kv_manager* m);
int32_t pa_kvm_live_slots(const pa_kv_manager* m);
/* Tokens slot holds (its length), or -1 for a free slot or a bad index. */
int32_t pa_kvm_length(const pa_kv_manager* m, int32_t slot);
/* Pages slot holds (for tokens it has or has reserved), or -1. */
int32_t pa_kvm_pages_held(const pa_kv_manager* m, int32_t slot);

/* Admit a sequence whose first num_tokens tokens (its prompt, num_tokens
 * >= 0) the caller will write with kv_append at positions 0..num_tokens-1:
 * takes the lowest free slot and the pages for those tokens. Returns the
 * slot (>= 0), or PA_ERR_NO_SLOT / PA_ERR_NO_PAGES / PA_ERR_SHAPE (more
 * tokens than a row can map). */
int32_t pa_kvm_admit(pa_kv_manager* m, int32_t num_tokens);

/* Release a live slot: its pages go back to the free list (last page
 * first) and the slot becomes free. PA_ERR_NO_SLOT for a free slot. */
int pa_kvm_release(pa_kv_manager* m, int32_t slot);

/* Make every live slot hold pages for its length + steps tokens (a window
 * of `steps` decode steps that need no host work, e.g. graph replays with
 * paged_decode_advance); lengths do not change. All or nothing:
 * PA_ERR_NO_PAGES if the free list cannot cover every slot, PA_ERR_SHAPE if
 * a row would need more than max_blocks_per_seq entries. */
int pa_kvm_reserve_ahead(pa_kv_manager* m, int32_t steps);

/* Plan one decode step for the whole batch: every live slot gets the page
 * for its next token if it does not hold it yet, and the step's arrays are
 * written (host memory, num_slots entries each):
 *   context_lens[s] = length + 1, positions[s] = length  (live slot)
 *   context_lens[s] = 0,          positions[s] = -1      (free slot)
 * then every live slot's length grows by one. block_table (may be NULL)
 * receives the whole table, [num_slots, max_blocks_per_seq]. All or
 * nothing, as pa_kvm_reserve_ahead(m, 1). */
int pa_kvm_plan_step(pa_kv_manager* m, int32_t* block_table,
                     int32_t* context_lens, int32_t* positions);

/* Record `steps` decode steps taken on the device (paged_decode_advance)
 * without pa_kvm_plan_step: every live slot's length grows by steps, which
 * its reserved pages must cover (else PA_ERR_NO_PAGES and no change). */
int pa_kvm_commit_steps(pa_kv_manager* m, int32_t steps);

/* The whole block table, [num_slots, max_blocks_per_seq] int32, host. */
int pa_kvm_block_table(const pa_kv_manager* m, int32_t* block_table);

/* The batch arrays of the current state without planning a step:
 * context_lens[s] = length, positions[s] = length - 1 for live slots with
 * tokens, else 0 and -1. Either pointer may be NULL. */
int pa_kvm_batch_state(const pa_kv_manager* m, int32_t* context_lens,
                       int32_t* positions);

#ifdef __cplusplus
}
#endif
#endif /* PAGED_KV_MANAGER_H */
