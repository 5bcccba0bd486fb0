// validate.hip — the separate batched page-tag check run before decode
// attention reads the cache.
//
// Every physical cache page carries a tag that changes when the page is
// handed out again; the server records, per request, the pages and tags it
// expects and compares them before the supported decode operations read the
// shared cache; a mismatch aborts the request instead of returning data from
// a wrong page. The check runs as its own batched step rather than inside the
// attention kernel (aifeed.sk, "Cloudflare zrýchľuje inferenciu modelov Kimi
// a GLM kompresiou cache a váh", section "Kvalita odpovedí a integrita
// spoločnej cache"; remio.ai, "Cloudflare: Kleinere Modellbereitstellung
// senkt Speicherbedarf, doch Sicherheit wird zum Prüfstein", section
// "Sicherheit gemeinsamer KV-Caches wird zum Produktionsthema"; agentlenshq.com,
// "Cloudflare Workers AI: Kimi および GLM の推論を大規模に最適化する", section
// "KV キャッシュ整合性チェック").
//
// One wave per sequence walks its logical blocks 64 at a time (coalesced
// block-table and expected-tag reads, a gather of the current tags) and stops
// at the first window holding a failing block; the lowest failing index is a
// ballot + find-first-set, so the verdict is deterministic.
#include "pda_internal.h"

namespace pda {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void validate_kernel(
    const uint32_t* __restrict__ page_tags, int P, const int32_t* __restrict__ block_table,
    const uint32_t* __restrict__ expected, int max_blocks, const int32_t* __restrict__ lens,
    int B, int S, int32_t* __restrict__ verdict) {
  const int s = (int)((blockIdx.x * (unsigned)kThreads + threadIdx.x) >> 6);
  const int lane = threadIdx.x & 63;
  if (s >= B) return;
  const int64_t len = lens[s];
  if (len < 0 || len > (int64_t)max_blocks * S) {
    if (lane == 0) verdict[s] = -1;
    return;
  }
  const int n = (int)((len + S - 1) / S);
  const int32_t* bt = block_table + (int64_t)s * max_blocks;
  const uint32_t* ex = expected + (int64_t)s * max_blocks;
  int32_t result = 0;
  for (int j0 = 0; j0 < n; j0 += 64) {
    const int j = j0 + lane;
    bool bad = false;
    if (j < n) {
      const int32_t p = bt[j];
      const uint32_t want = ex[j];
      if (p < 0 || p >= P)
        bad = true;
      else
        bad = page_tags[p] != want;
    }
    const uint64_t mask = __ballot(bad);
    if (mask != 0) {
      result = j0 + __builtin_ctzll(mask) + 1;
      break;
    }
  }
  if (lane == 0) verdict[s] = result;
}

}  // namespace
}  // namespace pda

using namespace pda;

extern "C" int validate_page_tags(const uint32_t* page_tags, int32_t num_pages,
                                  const int32_t* block_table, const uint32_t* expected_tags,
                                  int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                  int32_t num_seqs, int32_t page_size, int32_t* verdict,
                                  void* stream) {
  if (num_seqs < 0 || num_pages <= 0 || max_blocks_per_seq <= 0 || page_size <= 0)
    return PDA_ERR_INVALID_ARG;
  if (num_seqs == 0) return PDA_OK;
  if (!page_tags || !block_table || !expected_tags || !seq_lens || !verdict)
    return PDA_ERR_INVALID_ARG;
  const int waves_per_block = kThreads / 64;
  const int blocks = (num_seqs + waves_per_block - 1) / waves_per_block;
  hipLaunchKernelGGL(validate_kernel, dim3(blocks), dim3(kThreads), 0, as_stream(stream),
                     page_tags, num_pages, block_table, expected_tags, max_blocks_per_seq,
                     seq_lens, num_seqs, page_size, verdict);
  return launch_status();
}
