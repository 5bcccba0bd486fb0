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
// The per-sequence check itself is in validate_body.h (the fused kv write +
// check launch runs the same code).
#include "validate_body.h"

namespace pda {
namespace {

__global__ __launch_bounds__(kValidateThreads) void validate_kernel(
    const uint32_t* __restrict__ page_tags, int P, const int32_t* __restrict__ block_table,
    const uint32_t* __restrict__ expected, int max_blocks, const int32_t* __restrict__ lens,
    int S, int32_t* __restrict__ verdict) {
  __shared__ int best[kValidateThreads / 64];
  validate_seq(blockIdx.x, page_tags, P, block_table, expected, max_blocks, lens, S, verdict,
               best);
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
  hipLaunchKernelGGL(validate_kernel, dim3(num_seqs), dim3(kValidateThreads), 0, as_stream(stream),
                     page_tags, num_pages, block_table, expected_tags, max_blocks_per_seq,
                     seq_lens, page_size, verdict);
  return launch_status();
}
