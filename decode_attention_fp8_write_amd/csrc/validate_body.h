// validate_body.h — the per-sequence page-tag check, shared by the
// validate_page_tags kernel and the kernel that runs the check in the same
// launch as the kv write.
//
// One workgroup (four waves) per sequence. The sequence's logical blocks are
// cut into 64-block windows; wave w takes windows w, w+4, w+8, ... two at a
// time, so each lane has two block-table entries, two expected tags and two
// tag gathers in flight (coalesced table reads, a gather of the current
// tags). A wave stops at its first window holding a failing block; the
// lowest failing index inside a window is a ballot + find-first-set, and the
// workgroup takes the minimum over its waves, so the verdict is
// deterministic.
#pragma once
#include <climits>

#include "pda_internal.h"

namespace pda {

constexpr int kValidateThreads = 256;

// The check of sequence s by one workgroup of kValidateThreads threads; best
// is kValidateThreads / 64 ints of LDS.
__device__ __forceinline__ void validate_seq(
    int s, const uint32_t* __restrict__ page_tags, int P, const int32_t* __restrict__ block_table,
    const uint32_t* __restrict__ expected, int max_blocks, const int32_t* __restrict__ lens,
    int S, int32_t* __restrict__ verdict, int* best) {
  constexpr int kThreads = kValidateThreads;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int32_t* bt = block_table + (int64_t)s * max_blocks;
  const uint32_t* ex = expected + (int64_t)s * max_blocks;
  constexpr int kStride = kThreads;           // blocks between a wave's windows
  // The first two windows' table entries and expected tags are read before
  // the length is known (every index below max_blocks lies inside the
  // sequence's row), so that the length and them arrive in one round trip;
  // the length then masks them.
  int w0 = wave * 64;
  int32_t p0 = 0, p1 = 0;
  uint32_t e0 = 0, e1 = 0;
  if (w0 + lane < max_blocks) { p0 = bt[w0 + lane]; e0 = ex[w0 + lane]; }
  if (w0 + kStride + lane < max_blocks) { p1 = bt[w0 + kStride + lane]; e1 = ex[w0 + kStride + lane]; }
  const int64_t len = lens[s];
  if (len < 0 || len > (int64_t)max_blocks * S) {
    if (threadIdx.x == 0) verdict[s] = -1;
    return;
  }
  const int n = (int)((len + S - 1) / S);
  int first = INT_MAX;
  while (w0 < n) {
    const int j0 = w0 + lane, j1 = w0 + kStride + lane;
    const bool r0 = j0 < n && (p0 < 0 || p0 >= P);
    const bool r1 = j1 < n && (p1 < 0 || p1 >= P);
    uint32_t t0 = e0, t1 = e1;
    if (j0 < n && !r0) t0 = page_tags[p0];
    if (j1 < n && !r1) t1 = page_tags[p1];
    const uint64_t m0 = __ballot(j0 < n && (r0 || t0 != e0));
    const uint64_t m1 = __ballot(j1 < n && (r1 || t1 != e1));
    if (m0 != 0) {
      first = w0 + __builtin_ctzll(m0);
      break;
    }
    if (m1 != 0) {
      first = w0 + kStride + __builtin_ctzll(m1);
      break;
    }
    // the next two windows of this wave (sequences past 2 kThreads blocks)
    w0 += 2 * kStride;
    if (w0 + lane < n) { p0 = bt[w0 + lane]; e0 = ex[w0 + lane]; }
    if (w0 + kStride + lane < n) { p1 = bt[w0 + kStride + lane]; e1 = ex[w0 + kStride + lane]; }
  }
  if (lane == 0) best[wave] = first;
  __syncthreads();
  if (threadIdx.x == 0) {
    int v = best[0];
    for (int w = 1; w < kThreads / 64; ++w) v = min(v, best[w]);
    verdict[s] = v == INT_MAX ? 0 : v + 1;
  }
}

}  // namespace pda
