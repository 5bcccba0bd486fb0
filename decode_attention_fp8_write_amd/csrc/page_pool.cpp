// page_pool.cpp — host page pool and tag tracker (host code only).
//
// Every physical page carries a 32-bit tag that changes when the page is
// handed out again; a request keeps the pages and tags it was given, and the
// batched check on the device compares them with the pool's current tags
// (manulx.blog, "Công thức của Cloudflare để phục vụ Kimi và GLM", section
// "Bảo vệ bộ nhớ đệm dùng chung"; remio.ai, "Cloudflare: Kleinere
// Modellbereitstellung senkt Speicherbedarf, doch Sicherheit wird zum
// Prüfstein", section "Sicherheit gemeinsamer KV-Caches wird zum
// Produktionsthema"). With tracking off the pool stamps nothing: the no-op
// tracker of the same sections.
//
// Free pages form a stack (the most recently freed page is handed out
// first, so pages are reused while still warm in the caches); one global
// counter stamps hand-outs, so the tags of pages in use are distinct until
// the counter wraps after 2^32 hand-outs.
#include <stdint.h>

#include <new>
#include <vector>

#include "pda.h"

struct pda_page_pool {
  std::vector<uint32_t> tags;     // current tag per page
  std::vector<int32_t> stack;     // free pages; back() is handed out next
  std::vector<uint8_t> in_use;    // 1 while handed out
  uint32_t counter = 0;
  bool track = true;
};

extern "C" int pda_pool_create(int32_t num_pages, const int32_t* initial_order,
                               uint32_t tag_start, int32_t track_tags, pda_page_pool** out) {
  if (out == nullptr || num_pages <= 0) return PDA_ERR_INVALID_ARG;
  *out = nullptr;
  pda_page_pool* p = new (std::nothrow) pda_page_pool;
  if (p == nullptr) return PDA_ERR_INVALID_ARG;
  try {
    p->tags.assign((size_t)num_pages, 0u);
    p->in_use.assign((size_t)num_pages, 0);
    p->stack.resize((size_t)num_pages);
  } catch (...) {
    delete p;
    return PDA_ERR_INVALID_ARG;
  }
  // the stack holds the hand-out order reversed: back() is the first
  for (int32_t i = 0; i < num_pages; ++i) {
    const int32_t page = initial_order ? initial_order[i] : i;
    if (page < 0 || page >= num_pages || p->in_use[(size_t)page]) {   // not a permutation
      delete p;
      return PDA_ERR_INVALID_ARG;
    }
    p->in_use[(size_t)page] = 1;   // marks "seen" while checking
    p->stack[(size_t)(num_pages - 1 - i)] = page;
  }
  p->in_use.assign((size_t)num_pages, 0);
  p->counter = tag_start;
  p->track = track_tags != 0;
  *out = p;
  return PDA_OK;
}

extern "C" void pda_pool_destroy(pda_page_pool* pool) { delete pool; }

extern "C" int pda_pool_alloc(pda_page_pool* pool, int32_t n, int32_t* pages, uint32_t* tags) {
  if (pool == nullptr || n < 0 || (n > 0 && pages == nullptr)) return PDA_ERR_INVALID_ARG;
  if ((size_t)n > pool->stack.size()) return PDA_ERR_POOL_EXHAUSTED;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t page = pool->stack.back();
    pool->stack.pop_back();
    pool->in_use[(size_t)page] = 1;
    if (pool->track) pool->tags[(size_t)page] = ++pool->counter;
    pages[i] = page;
    if (tags != nullptr) tags[i] = pool->tags[(size_t)page];
  }
  return PDA_OK;
}

extern "C" int pda_pool_free(pda_page_pool* pool, const int32_t* pages, int32_t n) {
  if (pool == nullptr || n < 0 || (n > 0 && pages == nullptr)) return PDA_ERR_INVALID_ARG;
  const int32_t num_pages = (int32_t)pool->tags.size();
  // check everything first (range, in use, no repeats), then free
  int32_t i = 0;
  for (; i < n; ++i) {
    const int32_t page = pages[i];
    if (page < 0 || page >= num_pages || pool->in_use[(size_t)page] != 1) break;
    pool->in_use[(size_t)page] = 2;   // provisionally claimed by this call
  }
  const bool ok = (i == n);
  for (int32_t j = 0; j < i; ++j) pool->in_use[(size_t)pages[j]] = ok ? 0 : 1;
  if (!ok) return PDA_ERR_INVALID_ARG;
  for (int32_t j = 0; j < n; ++j) pool->stack.push_back(pages[j]);
  return PDA_OK;
}

extern "C" const uint32_t* pda_pool_tags(const pda_page_pool* pool) {
  return pool ? pool->tags.data() : nullptr;
}

extern "C" int32_t pda_pool_num_free(const pda_page_pool* pool) {
  return pool ? (int32_t)pool->stack.size() : -1;
}
