// probe.hip — read-only HBM bandwidth probe (a measurement aid, not part of
// the decode path): streaming or scrambled-chunk reads of a buffer, 16 bytes
// per lane per load, eight loads in flight per lane.
#include "pda_internal.h"
#include "pda_probe.h"

namespace pda {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeBlocksPerCu = 8;

__global__ __launch_bounds__(kProbeThreads) void hbm_read_kernel(const uint4* __restrict__ buf,
                                                                 int64_t n16, int64_t chunk16,
                                                                 int64_t nchunks,
                                                                 uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  const int64_t t = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  constexpr int U = 8;
  for (int64_t i0 = t; i0 < n16; i0 += stride * U) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = i0 + (int64_t)u * stride;
      if (i < n16) {
        int64_t j = i;
        if (chunk16 > 0) {   // chunk c of the pass reads scrambled chunk (c * odd) mod nchunks
          const int64_t c = i / chunk16;
          const int64_t sc = (int64_t)(((uint64_t)c * 0x9E3779B1ull) & (uint64_t)(nchunks - 1));
          j = sc * chunk16 + (i - c * chunk16);
        }
        v[u] = buf[j];
      } else {
        v[u] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
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
  } else if (bytes % 16 != 0) {
    return PDA_ERR_INVALID_ARG;
  }
  const int grid = device_cu_count() * kProbeBlocksPerCu;
  hipLaunchKernelGGL(hbm_read_kernel, dim3(grid), dim3(kProbeThreads), 0, as_stream(stream),
                     static_cast<const uint4*>(buf), (int64_t)(bytes / 16), chunk16, nchunks,
                     sink);
  return launch_status();
}
