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
// Decode batches are small (one to a few dozen tokens). One token takes a
// streaming dot-product kernel on the vector ALUs; two and more take a
// matrix-core kernel (below) whose products are nearly free, so both are
// limited by unpacking the codes and by moving bytes, not by arithmetic.
//
// Mapping (one token). A workgroup of four waves owns 8 output rows, two per
// wave. Lane l of a wave takes chunks l, l+64, ... of k, 32 elements each
// (one 16-byte load per row), so the wave reads 1 KB of each row per load
// instruction, and two chunks' loads are issued before their use. A chunk
// lies inside one 128-element scale group. (Two rows and two chunks ahead
// keep a wave at 89 VGPRs, so 8192 rows make four waves per SIMD: measured
// 11.1-11.4 us against 13.4 us for four rows and four chunks ahead at 213
// VGPRs, two waves per SIMD, on 8192 x 8192 weights. Pairing and summing the
// activations once per workgroup in LDS instead of per wave was slower,
// 11.8 us: the staging barrier costs more than the vector work it saves.)
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
// (x_j, x_{j+4}) by one byte permute per pair. Flipping the code's top bit
// and setting the exponent bits of 128.0 is one bitwise step on the masked
// field, (field & 0x000F000F) ^ 0x43084308 (a single v_bitop3), so a word's
// four dwords cost a shift and a bitop3 each (10.5-10.8 us against 11.0-11.6
// us with a separate xor and or, 8192 x 8192).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pda_int4.h"
#include "pda_internal.h"

namespace pda {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kGroup = 128;
constexpr int kRowsPerWave = 2;
constexpr int kWaves = 4;
constexpr int kRowsPerBlock = kRowsPerWave * kWaves;
constexpr int kChunk = 32;                 // k elements per lane and chunk
// bf16 pair (128.0, 128.0) with bit 3 of each half set: (field & 0x000F000F)
// ^ kMagicFlip flips the codes' top bits and sets the exponent bits of
// 128.0 in one bitwise step (the mask keeps the code bits, the constant
// supplies the rest)
constexpr uint32_t kMagicFlip = 0x43084308u;
constexpr uint32_t kNibbles = 0x000F000Fu;
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

__global__ __launch_bounds__(64 * kWaves) void int4_gemv_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ w,
    const uint16_t* __restrict__ scale, int n, int k, float* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row0 = blockIdx.x * kRowsPerBlock + wave * kRowsPerWave;
  const int chunks = k / kChunk;
  const int words = k / 8;
  const int groups = k / kGroup;

  // rows past n read row n-1 and are not stored, so every load stays inside
  // its buffer
  const uint32_t* wr[kRowsPerWave];
  const uint16_t* sr[kRowsPerWave];
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r) {
    const int row = min(row0 + r, n - 1);
    wr[r] = w + (int64_t)row * words;
    sr[r] = scale + (int64_t)row * groups;
  }

  float acc[kRowsPerWave];
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r) acc[r] = 0.0f;

  // U chunks per lane per step, all their loads issued before any use
  constexpr int U = 2;
  for (int c0 = lane; c0 < chunks; c0 += 64 * U) {
    uint4 wq[U][kRowsPerWave];
    float sc[U][kRowsPerWave];
    uint4 xv[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + 64 * u;
      if (c < chunks) {
#pragma unroll
        for (int r = 0; r < kRowsPerWave; ++r) {
          wq[u][r] = *reinterpret_cast<const uint4*>(wr[r] + 4 * c);
          sc[u][r] = bf16_bits_to_f32(sr[r][c / (kGroup / kChunk)]);
        }
        const uint4* xs = reinterpret_cast<const uint4*>(x + kChunk * c);
#pragma unroll
        for (int i = 0; i < 4; ++i) xv[u][i] = xs[i];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (c0 + 64 * u >= chunks) break;
      // activation pairs and -136 * sum x of the chunk
      uint32_t xp[16];
      float s = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 a = xv[u][i];
        pair_up(a, xp + 4 * i);
        s = dot2(a.x, kOnes, s);
        s = dot2(a.y, kOnes, s);
        s = dot2(a.z, kOnes, s);
        s = dot2(a.w, kOnes, s);
      }
      const float base = -136.0f * s;
#pragma unroll
      for (int r = 0; r < kRowsPerWave; ++r) {
        const uint32_t q[4] = {wq[u][r].x, wq[u][r].y, wq[u][r].z, wq[u][r].w};
        uint32_t wb[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int j = 0; j < 4; ++j) wb[4 * i + j] = ((q[i] >> (4 * j)) & kNibbles) ^ kMagicFlip;
        }
        float d = base;
#pragma unroll
        for (int i = 0; i < 16; ++i) d = dot2(wb[i], xp[i], d);
        acc[r] = __builtin_fmaf(d, sc[u][r], acc[r]);
      }
    }
  }

  // sum over the 64 lanes; afterwards every lane holds every total
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r) {
    float v = acc[r];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    acc[r] = v;
  }
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r)
    if (lane == r && row0 + r < n) y[row0 + r] = acc[r];
}

// ---- matrix-core path for two or more tokens ---------------------------
// D[token][row] = sum_k x[token][k] W[row][k] on v_mfma_f32_16x16x32_bf16:
// A = activations (16 tokens of a tile), B = unpacked codes (16 rows), both
// in the same permuted k order inside each 32-wide step (element 2j is k j,
// element 2j+1 is k j+4 of the lane's 8), which the sum does not see. Lane
// (c, g) of a wave holds, for k-step s of scale group G, words 4g + s of
// the group in row c (its 16 bytes of the group are one load) and the
// activations of the same 8 k. Products against a constant -136 operand
// give -136 * sum x of each token over the group, which seeds the group's
// accumulators, so they come out as x.q and take the group scale in one fma
// per output (0.2-0.8 us faster on 8192 x 8192 than subtracting a separate
// 136 * sum x product at the group's end).
// A workgroup owns kRT 16-row tiles and up to 32 tokens (grid rows of 32
// tokens run side by side and share the weights through the caches); its NW
// waves take every NW-th scale group and meet in LDS at the end: eight waves
// for one 16-token tile, four for two, whose registers leave room for fewer
// waves. Every row block re-reads the activations, from L2, through LDS
// (below): two row tiles serve up to 32 tokens, four beyond (8192 x 8192,
// measured over 16-, 32-, 64- and 128-row and 16- and 32-token tiles with
// four and eight waves: 64 tokens 29.2 us with four row tiles against 31.5
// with two and 50.8 with eight; 32 tokens 20.2 with two against 28.6 with
// four; up to 16 tokens the 16-token, 32-row, eight-wave form is fastest).
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMfmaTok = 32;        // tokens per grid row (two 16-token tiles)
constexpr uint32_t kNeg136 = 0xC308C308u;   // bf16 pair (-136.0, -136.0)

template <int TILES, int NW, int kRT>
__global__ __launch_bounds__(64 * NW) void int4_gemm_mfma_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ w,
    const uint16_t* __restrict__ scale, int m, int n, int k, float* __restrict__ y) {
  // U groups per wave and step, their loads issued before any use
  constexpr int U = 2;
  // Activations go through LDS: each wave copies the tiles of its U groups
  // (16 tokens x 128 inputs, 256 bytes a token) with direct global->LDS
  // copies, a copy taking four tokens' contiguous 256 bytes, and reads the
  // matrix-core operands back from there. (Loaded straight into the operand
  // layout, each load touched sixteen tokens' rows.) In the tile, token c's
  // 16-byte chunk j sits at position (j + c) mod 16 of its 256 bytes, so the
  // sixteen tokens one operand read touches hit sixteen different bank
  // quads. The final reduction reuses the same memory.
  constexpr int kTileB = 16 * 256;
  constexpr int kXsB = NW * U * TILES * kTileB;
  static_assert(kXsB <= 65536, "activation tiles fit the static LDS");
  static_assert((NW - 1) * TILES * kRT * 4 * 64 * 4 <= kXsB, "reduction fits the tiles");
  __shared__ __attribute__((aligned(16))) uint8_t xs_all[kXsB];
  float (*red)[TILES * kRT * 4][64] = reinterpret_cast<float (*)[TILES * kRT * 4][64]>(xs_all);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int row0 = blockIdx.x * 16 * kRT;
  const int tok0 = blockIdx.y * kMfmaTok;
  const int groups = k / kGroup;

  // out-of-range rows and tokens read row n-1 / token m-1 and are not stored
  const uint32_t* wr[kRT];
  const uint16_t* sr[kRT];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    const int row = min(row0 + 16 * rt + c, n - 1);
    wr[rt] = w + (int64_t)row * (k / 8) + 4 * g;
    sr[rt] = scale + (int64_t)row * groups;
  }
  uint8_t* const xs = xs_all + wave * (U * TILES * kTileB);
  const uint32_t xs_lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t*)xs));
  // copy i of tile t: lane L writes position L & 15 of token 4i + (L >> 4)
  // of the tile, i.e. chunk ((L & 15) - token) mod 16 of that token (s_nop 0:
  // one wait state between a scalar write of M0 and the copy using it)
  auto copy_tile = [&](int gi, int slot, int t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tt = 4 * i + (lane >> 4);
      const int j = ((lane & 15) - tt) & 15;
      const int tok = min(tok0 + 16 * t + tt, m - 1);
      const uint64_t ga = (uint64_t)(uintptr_t)(x + (int64_t)tok * k + kGroup * gi + 8 * j);
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                   :: "s"(xs_lds + (uint32_t)((slot * TILES + t) * kTileB + i * 1024)), "v"(ga)
                   : "memory");
    }
  };

  const uint4 cn136 = make_uint4(kNeg136, kNeg136, kNeg136, kNeg136);
  const bf16x8_t bneg136 = __builtin_bit_cast(bf16x8_t, cn136);
  f32x4_t yacc[TILES][kRT];
#pragma unroll
  for (int t = 0; t < TILES; ++t)
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) yacc[t][rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int g0 = wave; g0 < groups; g0 += NW * U) {
    uint4 wv[U][kRT];
    float sc[U][kRT];
    // the copies first: the compiler's waits for the weight loads below
    // then also cover them (loads complete in order), and the explicit wait
    // after the loads covers them in any case
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int gi = g0 + NW * u;
      if (gi < groups) {
#pragma unroll
        for (int t = 0; t < TILES; ++t) copy_tile(gi, u, t);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int gi = g0 + NW * u;
      if (gi < groups) {
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
          wv[u][rt] = *reinterpret_cast<const uint4*>(wr[rt] + 16 * gi);
          sc[u][rt] = bf16_bits_to_f32(sr[rt][gi]);
        }
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (g0 + NW * u >= groups) break;
      // activation pairs of the group's four steps, then -136 * sum x of
      // each token over the group, which seeds the group's products
      bf16x8_t av[TILES][4];
      f32x4_t nac[TILES];
#pragma unroll
      for (int t = 0; t < TILES; ++t) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          uint32_t p[4];
          const uint4 xv = *reinterpret_cast<const uint4*>(
              xs + (u * TILES + t) * kTileB + c * 256 + (((4 * g + s + c) & 15) * 16));
          pair_up(xv, p);
          av[t][s] = __builtin_bit_cast(bf16x8_t, make_uint4(p[0], p[1], p[2], p[3]));
        }
        nac[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s)
          nac[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[t][s], bneg136, nac[t], 0, 0, 0);
      }
      f32x4_t am[TILES][kRT];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8_t bw[kRT];
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
          const uint4 q = wv[u][rt];
          const uint32_t word = s == 0 ? q.x : s == 1 ? q.y : s == 2 ? q.z : q.w;
          const uint4 d = make_uint4(
              (word & kNibbles) ^ kMagicFlip, ((word >> 4) & kNibbles) ^ kMagicFlip,
              ((word >> 8) & kNibbles) ^ kMagicFlip, ((word >> 12) & kNibbles) ^ kMagicFlip);
          bw[rt] = __builtin_bit_cast(bf16x8_t, d);
        }
#pragma unroll
        for (int t = 0; t < TILES; ++t)
#pragma unroll
          for (int rt = 0; rt < kRT; ++rt)
            am[t][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[t][s], bw[rt],
                                                                s == 0 ? nac[t] : am[t][rt], 0, 0, 0);
      }
#pragma unroll
      for (int t = 0; t < TILES; ++t)
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            yacc[t][rt][r] =
                __builtin_fmaf(am[t][rt][r], sc[u][rt], yacc[t][rt][r]);
    }
  }

  // the other waves hand their partial sums to wave 0, through the memory
  // the tiles used (every wave is done with its tiles past this barrier)
  __syncthreads();
  if (wave > 0) {
#pragma unroll
    for (int t = 0; t < TILES; ++t)
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave - 1][(t * kRT + rt) * 4 + r][lane] = yacc[t][rt][r];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int t = 0; t < TILES; ++t)
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = (t * kRT + rt) * 4 + r;
        float v = yacc[t][rt][r];
#pragma unroll
        for (int o = 0; o < NW - 1; ++o) v += red[o][i][lane];
        const int tok = tok0 + 16 * t + 4 * g + r;
        const int row = row0 + 16 * rt + c;
        if (tok < m && row < n) y[(int64_t)tok * n + row] = v;
      }
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
  // one token: grid of 16-row workgroups; more: 32-row by 32-token tiles
  const int64_t blocks = ((int64_t)n + kRowsPerBlock - 1) / kRowsPerBlock;
  const int64_t tok_tiles = ((int64_t)m + kMfmaTok - 1) / kMfmaTok;
  if (blocks > 0x7FFFFFFF || tok_tiles > 65535) return PDA_ERR_UNSUPPORTED;
  hipStream_t s = as_stream(stream);
  const auto* xb = static_cast<const uint16_t*>(x);
  const auto* sb = static_cast<const uint16_t*>(scale);
  if (m >= 2) {
    // workgroups of 32 rows up to 32 tokens, of 64 rows beyond, where the
    // activations re-read by every row block dominate
    const int rows = m <= 32 ? 32 : 64;
    const dim3 g2((unsigned)(((int64_t)n + rows - 1) / rows), (unsigned)tok_tiles);
    if (m <= 16)
      hipLaunchKernelGGL((int4_gemm_mfma_kernel<1, 8, 2>), g2, dim3(64 * 8), 0, s, xb, w, sb, m, n,
                         k, y);
    else if (m <= 32)
      hipLaunchKernelGGL((int4_gemm_mfma_kernel<2, 4, 2>), g2, dim3(64 * 4), 0, s, xb, w, sb, m, n,
                         k, y);
    else
      hipLaunchKernelGGL((int4_gemm_mfma_kernel<2, 4, 4>), g2, dim3(64 * 4), 0, s, xb, w, sb, m, n,
                         k, y);
    return launch_status();
  }
  hipLaunchKernelGGL(int4_gemv_kernel, dim3((unsigned)blocks), dim3(64 * kWaves), 0, s, xb, w,
                     sb, n, k, y);
  return launch_status();
}
