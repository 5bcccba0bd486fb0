// int4_gemv.hip — weight-only INT4 GEMV for decode: y = x · dequant(W)^T with
// bf16 activations, signed 4-bit weight codes and one bf16 scale per 128
// consecutive k of each output row.
//
// The pages report that INT4 weights speed up decode, where every generated
// token streams the weights from HBM, and slow down prefill, where unpacking
// adds work to a compute-bound phase (aifeed.sk, "Cloudflare zrýchľuje
// inferenciu modelov Kimi a GLM kompresiou cache a váh", section "Kompresia
// sa oplatí inde pri vstupe a inde pri výstupe"; the German page on the same
// changes, section "GLM-Gewichtskomprimierung verschiebt den Phasen-Trade-
// off"). The format is not on the pages; the one taken here is stated in
// include/pda_int4.h.
//
// Decode batches are small (one to a few dozen tokens), so the kernel is a
// streaming dot-product kernel on the vector ALUs, not a matrix-core tile
// loop: each weight byte is read from HBM once per launch and used by every
// token of the batch held in registers.
//
// Mapping. A workgroup of four waves owns 16 output rows, four per wave.
// Lane l of a wave takes chunks l, l+64, ... of k, 32 elements each (one
// 16-byte load per row) for up to two tokens, 16 elements (8 bytes) for more,
// where the activations take the registers; so the wave reads 1 KB or 512 B
// of each row per load instruction, and several chunks' loads are issued
// before their use. A chunk lies inside one 128-element scale group.
//
// Unpacking without integer-to-float conversions: a code u' = q + 8 in
// [0, 15] (the two's-complement code with its top bit flipped) put into the
// low mantissa bits of bf16 128.0 (0x4300) is exactly 128 + u' = q + 136.
// Two such values share a dword, so the bf16 dot-product instruction takes
// them directly against the matching pair of activations:
//   sum_k x_k q_k = sum_k x_k (q_k + 136) - 136 * sum_k x_k,
// and the dot-product chain of a chunk starts from -136 * sum x, so each
// chunk's sum comes out of the chain as x·q, then is scaled once by its
// group's scale into the fp32 accumulator.
//
// Nibble j of a word and nibble j + 4 land in the two halves of one dword
// ((word >> 4j) & 0x000F000F), so activations are paired the same way:
// (x_j, x_{j+4}) by one byte permute per pair.
//
// Tokens: a launch handles up to kMaxTok tokens per grid row (grid.y covers
// larger batches, each grid row streaming the weights again).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pda_int4.h"
#include "pda_internal.h"

namespace pda {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kGroup = 128;
constexpr int kRowsPerWave = 4;
constexpr int kWaves = 4;
constexpr int kRowsPerBlock = kRowsPerWave * kWaves;
constexpr int kMaxTok = 8;
constexpr uint32_t kMagic = 0x43004300u;   // bf16 pair (128.0, 128.0)
constexpr uint32_t kOnes = 0x3F803F80u;    // bf16 pair (1.0, 1.0)

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

// Activation pairs of one 8-element word: dwords X0 = (x0, x1), X1 = (x2,
// x3), X2 = (x4, x5), X3 = (x6, x7) become (x0, x4), (x1, x5), (x2, x6),
// (x3, x7).
__device__ __forceinline__ void pair_up(const uint4 X, uint32_t p[4]) {
  p[0] = __builtin_amdgcn_perm(X.z, X.x, 0x05040100u);
  p[1] = __builtin_amdgcn_perm(X.z, X.x, 0x07060302u);
  p[2] = __builtin_amdgcn_perm(X.w, X.y, 0x05040100u);
  p[3] = __builtin_amdgcn_perm(X.w, X.y, 0x07060302u);
}

template <int MT>
__global__ __launch_bounds__(64 * kWaves) void int4_gemv_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ w,
    const uint16_t* __restrict__ scale, int m, int n, int k, float* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row0 = blockIdx.x * kRowsPerBlock + wave * kRowsPerWave;
  const int tok0 = blockIdx.y * kMaxTok;
  // CW packed words (8*CW elements) per lane and chunk: 16-byte weight loads
  // where few tokens leave registers to spare, 8-byte loads otherwise
  constexpr int CW = MT <= 2 ? 4 : 2;
  constexpr int CH = 8 * CW;
  const int chunks = k / CH;
  const int words = k / 8;
  const int groups = k / kGroup;

  // rows past n read row n-1 and are not stored; tokens past m read token
  // m-1 and are not stored, so every load stays inside its buffer
  const uint32_t* wr[kRowsPerWave];
  const uint16_t* sr[kRowsPerWave];
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r) {
    const int row = min(row0 + r, n - 1);
    wr[r] = w + (int64_t)row * words;
    sr[r] = scale + (int64_t)row * groups;
  }
  const uint16_t* xt[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) xt[t] = x + (int64_t)min(tok0 + t, m - 1) * k;

  float acc[kRowsPerWave][MT];
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[r][t] = 0.0f;

  // U chunks per lane per step, all their loads issued before any use, so
  // enough bytes are in flight to cover HBM latency with few waves per CU
  constexpr int U = MT <= 2 ? 4 : (MT == 4 ? 2 : 1);
  for (int c0 = lane; c0 < chunks; c0 += 64 * U) {
    uint32_t wq[U][kRowsPerWave][CW];
    float sc[U][kRowsPerWave];
    uint4 xv[U][MT][CW];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + 64 * u;
      if (c < chunks) {
#pragma unroll
        for (int r = 0; r < kRowsPerWave; ++r) {
          if constexpr (CW == 4) {
            const uint4 v = *reinterpret_cast<const uint4*>(wr[r] + CW * c);
            wq[u][r][0] = v.x; wq[u][r][1] = v.y; wq[u][r][2] = v.z; wq[u][r][3] = v.w;
          } else {
            const uint2 v = *reinterpret_cast<const uint2*>(wr[r] + CW * c);
            wq[u][r][0] = v.x; wq[u][r][1] = v.y;
          }
          sc[u][r] = bf16_bits_to_f32(sr[r][c / (kGroup / CH)]);
        }
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const uint4* xs = reinterpret_cast<const uint4*>(xt[t] + CH * c);
#pragma unroll
          for (int i = 0; i < CW; ++i) xv[u][t][i] = xs[i];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (c0 + 64 * u >= chunks) break;
      // activation pairs and -136 * sum x of the chunk, per token
      uint32_t xp[MT][4 * CW];
      float base[MT];
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < CW; ++i) {
          const uint4 a = xv[u][t][i];
          pair_up(a, xp[t] + 4 * i);
          s = dot2(a.x, kOnes, s);
          s = dot2(a.y, kOnes, s);
          s = dot2(a.z, kOnes, s);
          s = dot2(a.w, kOnes, s);
        }
        base[t] = -136.0f * s;
      }
#pragma unroll
      for (int r = 0; r < kRowsPerWave; ++r) {
        uint32_t wb[4 * CW];
#pragma unroll
        for (int i = 0; i < CW; ++i) {
          const uint32_t v = wq[u][r][i] ^ 0x88888888u;
#pragma unroll
          for (int j = 0; j < 4; ++j) wb[4 * i + j] = ((v >> (4 * j)) & 0x000F000Fu) | kMagic;
        }
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          float d = base[t];
#pragma unroll
          for (int i = 0; i < 4 * CW; ++i) d = dot2(wb[i], xp[t][i], d);
          acc[r][t] = __builtin_fmaf(d, sc[u][r], acc[r][t]);
        }
      }
    }
  }

  // sum over the 64 lanes; afterwards every lane holds every total
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r)
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      float v = acc[r][t];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
      acc[r][t] = v;
    }
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r)
#pragma unroll
    for (int t = 0; t < MT; ++t)
      if (lane == r * MT + t && row0 + r < n && tok0 + t < m)
        y[(int64_t)(tok0 + t) * n + row0 + r] = acc[r][t];
}

}  // namespace
}  // namespace pda

using namespace pda;

extern "C" int int4_gemv_bf16(const void* x, const uint32_t* w, const void* scale,
                              int32_t m, int32_t n, int32_t k, int32_t group, float* y,
                              void* stream) {
  if (m < 0 || n < 0 || k < 0) return PDA_ERR_INVALID_ARG;
  if (group != kGroup || k % kGroup != 0) return PDA_ERR_UNSUPPORTED;
  if (m == 0 || n == 0) return PDA_OK;
  if (k == 0) return PDA_ERR_UNSUPPORTED;
  if (!x || !w || !scale || !y) return PDA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(x) & 15) != 0 || (reinterpret_cast<uintptr_t>(w) & 15) != 0 ||
      (reinterpret_cast<uintptr_t>(scale) & 1) != 0 || (reinterpret_cast<uintptr_t>(y) & 3) != 0)
    return PDA_ERR_INVALID_ARG;
  const int64_t blocks = ((int64_t)n + kRowsPerBlock - 1) / kRowsPerBlock;
  const int64_t tok_blocks = ((int64_t)m + kMaxTok - 1) / kMaxTok;
  if (blocks > 0x7FFFFFFF || tok_blocks > 65535) return PDA_ERR_UNSUPPORTED;
  const dim3 grid((unsigned)blocks, (unsigned)tok_blocks);
  const dim3 block(64 * kWaves);
  hipStream_t s = as_stream(stream);
  const int mt = m < kMaxTok ? m : kMaxTok;
  const auto* xb = static_cast<const uint16_t*>(x);
  const auto* sb = static_cast<const uint16_t*>(scale);
  if (mt == 1)
    hipLaunchKernelGGL(int4_gemv_kernel<1>, grid, block, 0, s, xb, w, sb, m, n, k, y);
  else if (mt == 2)
    hipLaunchKernelGGL(int4_gemv_kernel<2>, grid, block, 0, s, xb, w, sb, m, n, k, y);
  else if (mt <= 4)
    hipLaunchKernelGGL(int4_gemv_kernel<4>, grid, block, 0, s, xb, w, sb, m, n, k, y);
  else
    hipLaunchKernelGGL(int4_gemv_kernel<8>, grid, block, 0, s, xb, w, sb, m, n, k, y);
  return launch_status();
}
