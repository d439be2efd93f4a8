// Host-side page manager of the paged KV cache (declarations and contract in
// include/paged_kv_manager.h).
//
// tiny-llm "优化", section 2: the cache is allocated once from its
// configuration and the decode phase never allocates; roadmap rows 分页 KV
// and 连续批处理. "TensorRT对Multi-Query Attention的专项优化支持", KV-cache
// paragraph: fixed-length pages handed out on demand.
//
// Plain C++ bookkeeping, no device calls: a LIFO free list of page ids,
// each slot's pages in token order, each slot's length. Every mutating call
// first checks that it can complete (enough free pages, rows long enough)
// and only then changes state, so a failed call changes nothing.
#include "paged_kv_manager.h"

#include <limits.h>

#include <algorithm>
#include <new>
#include <vector>

struct pa_kv_manager {
  int32_t num_pages, block_size, num_slots, max_blocks;
  std::vector<int32_t> free_list;              // top = back = next page handed out
  std::vector<std::vector<int32_t>> pages;     // per slot, in token order
  std::vector<int32_t> length;                 // per slot; -1 = free slot
  int32_t live = 0;
};

namespace {

bool valid_block_size(int32_t bs) { return bs == 16 || bs == 32 || bs == 64; }

// Pages needed to hold n tokens.
int64_t pages_for(const pa_kv_manager* m, int64_t n) {
  return n <= 0 ? 0 : (n + m->block_size - 1) / m->block_size;
}

bool live_slot(const pa_kv_manager* m, int32_t s) {
  return m && s >= 0 && s < m->num_slots && m->length[s] >= 0;
}

// Extra pages each live slot needs to hold (length + steps) tokens; -1 if a
// row would need more than max_blocks entries.
int64_t extra_pages(const pa_kv_manager* m, int64_t steps) {
  int64_t need = 0;
  for (int32_t s = 0; s < m->num_slots; ++s) {
    if (m->length[s] < 0) continue;
    const int64_t want = pages_for(m, (int64_t)m->length[s] + steps);
    if (want > m->max_blocks) return -1;
    need += std::max<int64_t>(0, want - (int64_t)m->pages[s].size());
  }
  return need;
}

// Hand out pages until every live slot holds (length + steps) tokens; the
// caller has checked that the free list covers it.
void grow_all(pa_kv_manager* m, int64_t steps) {
  for (int32_t s = 0; s < m->num_slots; ++s) {
    if (m->length[s] < 0) continue;
    const int64_t want = pages_for(m, (int64_t)m->length[s] + steps);
    while ((int64_t)m->pages[s].size() < want) {
      m->pages[s].push_back(m->free_list.back());
      m->free_list.pop_back();
    }
  }
}

}  // namespace

extern "C" {

int32_t pa_kv_elem_bytes(int32_t kv_dtype) {
  switch (kv_dtype) {
    case PA_KV_FP16: return 2;
    case PA_KV_FP8_E4M3FN:
    case PA_KV_INT8: return 1;
    default: return 0;
  }
}

int64_t pa_kv_bytes_per_sequence(int32_t num_layers, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_seq_len,
                                 int32_t kv_dtype) {
  const int32_t e = pa_kv_elem_bytes(kv_dtype);
  if (num_layers < 1 || num_kv_heads < 1 || head_dim < 1 || max_seq_len < 0 || e == 0)
    return -1;
  return 2LL * num_layers * num_kv_heads * head_dim * (int64_t)max_seq_len * e;
}

int64_t pa_kv_pool_bytes(int32_t num_pages, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t kv_dtype) {
  const int32_t e = pa_kv_elem_bytes(kv_dtype);
  if (num_pages < 0 || num_kv_heads < 1 || head_dim < 1 || block_size < 1 || e == 0)
    return -1;
  return 2LL * num_pages * num_kv_heads * (int64_t)block_size * head_dim * e;
}

int64_t pa_kv_pages_for_budget(int64_t budget_bytes, int32_t num_layers,
                               int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, int32_t kv_dtype) {
  const int64_t per_page = pa_kv_pool_bytes(1, num_kv_heads, head_dim, block_size, kv_dtype);
  if (per_page <= 0 || num_layers < 1 || budget_bytes < 0) return -1;
  return std::min<int64_t>(budget_bytes / (per_page * num_layers), INT32_MAX);
}

pa_kv_manager* pa_kvm_create(int32_t num_pages, int32_t block_size, int32_t num_slots,
                             int32_t max_blocks_per_seq) {
  if (num_pages < 1 || num_slots < 1 || max_blocks_per_seq < 1 ||
      !valid_block_size(block_size) ||
      (int64_t)max_blocks_per_seq * block_size > INT32_MAX)
    return nullptr;
  pa_kv_manager* m = new (std::nothrow) pa_kv_manager();
  if (!m) return nullptr;
  try {
    m->num_pages = num_pages;
    m->block_size = block_size;
    m->num_slots = num_slots;
    m->max_blocks = max_blocks_per_seq;
    m->free_list.resize(num_pages);
    for (int32_t i = 0; i < num_pages; ++i) m->free_list[i] = num_pages - 1 - i;
    m->pages.resize(num_slots);
    m->length.assign(num_slots, -1);
  } catch (...) {
    delete m;
    return nullptr;
  }
  return m;
}

void pa_kvm_destroy(pa_kv_manager* m) { delete m; }

int32_t pa_kvm_free_pages(const pa_kv_manager* m) {
  return m ? (int32_t)m->free_list.size() : PA_ERR_NULL;
}

int32_t pa_kvm_live_slots(const pa_kv_manager* m) { return m ? m->live : PA_ERR_NULL; }

int32_t pa_kvm_length(const pa_kv_manager* m, int32_t slot) {
  return live_slot(m, slot) ? m->length[slot] : -1;
}

int32_t pa_kvm_pages_held(const pa_kv_manager* m, int32_t slot) {
  return live_slot(m, slot) ? (int32_t)m->pages[slot].size() : -1;
}

int32_t pa_kvm_admit(pa_kv_manager* m, int32_t num_tokens) {
  if (!m) return PA_ERR_NULL;
  if (num_tokens < 0) return PA_ERR_SHAPE;
  const int64_t need = pages_for(m, num_tokens);
  if (need > m->max_blocks) return PA_ERR_SHAPE;
  int32_t slot = -1;
  for (int32_t s = 0; s < m->num_slots; ++s)
    if (m->length[s] < 0) { slot = s; break; }
  if (slot < 0) return PA_ERR_NO_SLOT;
  if (need > (int64_t)m->free_list.size()) return PA_ERR_NO_PAGES;
  m->pages[slot].clear();
  for (int64_t i = 0; i < need; ++i) {
    m->pages[slot].push_back(m->free_list.back());
    m->free_list.pop_back();
  }
  m->length[slot] = num_tokens;
  ++m->live;
  return slot;
}

int pa_kvm_release(pa_kv_manager* m, int32_t slot) {
  if (!m) return PA_ERR_NULL;
  if (!live_slot(m, slot)) return PA_ERR_NO_SLOT;
  std::vector<int32_t>& p = m->pages[slot];
  for (auto it = p.rbegin(); it != p.rend(); ++it) m->free_list.push_back(*it);
  p.clear();
  m->length[slot] = -1;
  --m->live;
  return PA_OK;
}

int pa_kvm_reserve_ahead(pa_kv_manager* m, int32_t steps) {
  if (!m) return PA_ERR_NULL;
  if (steps < 0) return PA_ERR_SHAPE;
  const int64_t need = extra_pages(m, steps);
  if (need < 0) return PA_ERR_SHAPE;
  if (need > (int64_t)m->free_list.size()) return PA_ERR_NO_PAGES;
  grow_all(m, steps);
  return PA_OK;
}

int pa_kvm_block_table(const pa_kv_manager* m, int32_t* block_table) {
  if (!m || !block_table) return PA_ERR_NULL;
  for (int32_t s = 0; s < m->num_slots; ++s) {
    int32_t* row = block_table + (int64_t)s * m->max_blocks;
    const std::vector<int32_t>& p = m->pages[s];
    const int32_t n = m->length[s] < 0 ? 0 : (int32_t)p.size();
    for (int32_t i = 0; i < m->max_blocks; ++i) row[i] = i < n ? p[i] : -1;
  }
  return PA_OK;
}

int pa_kvm_batch_state(const pa_kv_manager* m, int32_t* context_lens, int32_t* positions) {
  if (!m) return PA_ERR_NULL;
  for (int32_t s = 0; s < m->num_slots; ++s) {
    const int32_t L = m->length[s];
    if (context_lens) context_lens[s] = L < 0 ? 0 : L;
    if (positions) positions[s] = L <= 0 ? -1 : L - 1;
  }
  return PA_OK;
}

int pa_kvm_plan_step(pa_kv_manager* m, int32_t* block_table, int32_t* context_lens,
                     int32_t* positions) {
  if (!m || !context_lens || !positions) return PA_ERR_NULL;
  const int rc = pa_kvm_reserve_ahead(m, 1);
  if (rc) return rc;
  for (int32_t s = 0; s < m->num_slots; ++s) {
    const int32_t L = m->length[s];
    context_lens[s] = L < 0 ? 0 : L + 1;
    positions[s] = L < 0 ? -1 : L;
    if (L >= 0) m->length[s] = L + 1;
  }
  return block_table ? pa_kvm_block_table(m, block_table) : PA_OK;
}

int pa_kvm_commit_steps(pa_kv_manager* m, int32_t steps) {
  if (!m) return PA_ERR_NULL;
  if (steps < 0) return PA_ERR_SHAPE;
  for (int32_t s = 0; s < m->num_slots; ++s)
    if (m->length[s] >= 0 &&
        pages_for(m, (int64_t)m->length[s] + steps) > (int64_t)m->pages[s].size())
      return PA_ERR_NO_PAGES;
  for (int32_t s = 0; s < m->num_slots; ++s)
    if (m->length[s] >= 0) m->length[s] += steps;
  return PA_OK;
}

}  // extern "C"
