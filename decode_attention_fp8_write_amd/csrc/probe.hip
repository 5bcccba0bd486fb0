// probe.hip — read-only HBM bandwidth probe (a measurement aid, not part of
// the decode path): streaming or scrambled-chunk reads of a buffer, 16 bytes
// per lane per load, sixteen loads in flight per lane.
#include "pda_internal.h"
#include "pda_probe.h"

namespace pda {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeBlocksPerCu = 32;
constexpr int kProbeU = 16;   // 16-byte loads per lane in flight: 16 KB per wave

// Each wave reads whole 16 KB blocks of the logical order (lane l, load u:
// 16-byte element 64 u + l of the block, so every load instruction of a wave
// covers 1 KB contiguous), blocks dealt round-robin over all waves.
// Logical element i is physical element i (streaming) or, in chunked mode,
// element i of scrambled chunk (i / chunk * 0x9E3779B1) mod nchunks.
// (Measured on MI355X against one element per lane with the grid as the
// stride, the form this replaces: 6.3 against 5.5 TB/s streaming.)
__global__ __launch_bounds__(kProbeThreads) void hbm_read_kernel(const uint4* __restrict__ buf,
                                                                 int64_t n16, int64_t chunk16,
                                                                 int64_t nchunks,
                                                                 uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const int lane = threadIdx.x & 63;
  const int64_t nw = (int64_t)gridDim.x * (kProbeThreads / 64);
  const int64_t w = (int64_t)blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6);
  const int64_t nblk = n16 / (64 * kProbeU);   // the host checks n16 % (64 * kProbeU) == 0
  for (int64_t b = w; b < nblk; b += nw) {
    uint4 v[kProbeU];
#pragma unroll
    for (int u = 0; u < kProbeU; ++u) {
      const int64_t i = b * (64 * kProbeU) + u * 64 + lane;
      int64_t j = i;
      if (chunk16 > 0) {
        const int64_t c = i / chunk16;
        const int64_t sc = (int64_t)(((uint64_t)c * 0x9E3779B1ull) & (uint64_t)(nchunks - 1));
        j = sc * chunk16 + (i - c * chunk16);
      }
      v[u] = buf[j];
    }
#pragma unroll
    for (int u = 0; u < kProbeU; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  // one word per workgroup
  acc = (uint32_t)__builtin_amdgcn_readfirstlane((int)acc);
  if (threadIdx.x == 0) sink[blockIdx.x] = acc;
}

}  // namespace

int device_cu_count();

}  // namespace pda

using namespace pda;

extern "C" size_t pda_hbm_read_probe_sink_words(void) {
  return (size_t)device_cu_count() * kProbeBlocksPerCu;
}

extern "C" int pda_hbm_read_probe(const void* buf, size_t bytes, int32_t chunk_bytes,
                                  uint32_t* sink, void* stream) {
  if (!buf || !sink || bytes == 0 || (reinterpret_cast<uintptr_t>(buf) & 15) != 0)
    return PDA_ERR_INVALID_ARG;
  int64_t chunk16 = 0, nchunks = 0;
  if (chunk_bytes != 0) {
    if (chunk_bytes < 256 || chunk_bytes > 65536 || (chunk_bytes & (chunk_bytes - 1)) != 0)
      return PDA_ERR_INVALID_ARG;
    if (bytes % (size_t)chunk_bytes != 0) return PDA_ERR_INVALID_ARG;
    nchunks = (int64_t)(bytes / (size_t)chunk_bytes);
    if ((nchunks & (nchunks - 1)) != 0) return PDA_ERR_INVALID_ARG;
    chunk16 = chunk_bytes / 16;
  }
  if (bytes % (16 * 64 * kProbeU) != 0) return PDA_ERR_INVALID_ARG;
  const int grid = device_cu_count() * kProbeBlocksPerCu;
  hipLaunchKernelGGL(hbm_read_kernel, dim3(grid), dim3(kProbeThreads), 0, as_stream(stream),
                     static_cast<const uint4*>(buf), (int64_t)(bytes / 16), chunk16, nchunks,
                     sink);
  return launch_status();
}
