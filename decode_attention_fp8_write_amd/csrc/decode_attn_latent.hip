// decode_attn_latent.hip — decode attention over a latent paged cache on
// MFMA: one kv head whose 576-dim FP8 entry is the key and whose first 512
// dims are the value, one fp32 scale per token, and 32..128 query heads
// sharing it, so every page is a dense (heads x tokens) contraction.
//
// The pages state that the cache is kept as 8-bit e4m3 and that the
// attention kernel converts what it reads (aifeed.sk, "Cloudflare zrýchľuje
// inferenciu modelov Kimi a GLM kompresiou cache a váh", section "Dve odlišné
// úzke miesta v pamäti GPU"; manulx.blog, "Công thức của Cloudflare để phục
// vụ Kimi và GLM", section "Bộ nhớ đệm KV FP8 tăng gấp đôi dung lượng ngữ
// cảnh"). The kernel design is not from the pages, which give none.
//
// Work split. The valid pages of all non-aborted sequences are laid end to
// end and cut into one equal range per workgroup (a flat split, so long and
// short sequences balance). A workgroup walks the fragments of sequences in
// its range; each fragment leaves one partial (unnormalised output rows, a
// running max and a running weight sum per head) in workspace slot
// (workgroup + sequence), which is unique. The combine kernel merges the
// fragments of each sequence with a log-sum-exp rule.
//
// Inside a fragment, one page (64 tokens) at a time, by eight waves (two per
// SIMD, so one wave's conversions and softmax overlap the other's matrix
// products; a wave's own instruction stream is in order):
//  * the workgroup copies the page's 36 KB of codes and its 64 scales into
//    LDS by direct global->LDS copies (double-buffered: the next page's copy
//    is issued after the page's QK products, at the start of its softmax,
//    and lands while the rest of the page is computed). Wave 0, which copies
//    the scales, fills the next page's per-token factors at the end of the
//    page, so a page takes one barrier before QK and one between softmax and
//    PV. Tokens past the end are written as zero codes with weight 0 (a
//    sequence's last page, behind one more barrier), so they contribute
//    nothing and poisoned bytes are never read into the arithmetic.
//  * QK is split by heads: wave w < NH owns query heads [16w, 16w+16). S^T =
//    K Q^T on v_mfma_f32_16x16x32_bf16: K codes convert exactly to bf16 (A
//    operand, lane = token row, token tile t = tokens 16t .. 16t+15), Q is
//    bf16 (B operand, lane = head; its first k-steps in registers, the rest
//    in the wave's LDS region), so Q enters exactly. The operand reads from
//    the token-major page hit every LDS bank once per half-wave (a lane reads
//    8 bytes; the 32 lanes of a half-wave cover 16 tokens' full 16-byte
//    slots).
//  * softmax in log2 units with the per-token scale folded in: for token t
//    with scale c_t, y = (q.code_t) * c_t * sm_scale * log2(e) + log2(c_t);
//    p' = 2^(y - m) = c_t * e^(score - m'), so the weights already carry the
//    value scale, and the running sum adds p' / c_t. The running max m only
//    moves when a page's max exceeds it by more than 8 (p' <= 2^8). The
//    weights go to LDS as f16, one 144-byte row per head.
//  * PV is split by value dims: wave w owns dims [64w, 64w + 64) of every
//    head, O^T = V^T P^T on v_mfma_f32_16x16x32_f16. The A operand needs
//    eight tokens of one dim per lane; the LDS transpose read
//    ds_read_b64_tr_b8 gathers them from the token-major page (in each
//    16-lane group, lane i receives byte i%8 of the eight 8-byte chunks
//    addressed by lanes 2b + i/8), and its codes convert exactly to f16 once
//    per workgroup. The B operand is the weights of a head tile from LDS.
//    The accumulators (64 dims x every head) stay in AGPRs.
#include <mutex>
#include <type_traits>

#include "pda_internal.h"

namespace pda {
namespace {

constexpr int kDk = 576;            // latent key dims
constexpr int kDv = 512;            // value dims (first 512 of the key)
constexpr int kS = 64;              // page size
constexpr int kKSteps = kDk / 32;   // 32-dim QK k-steps per token
constexpr int kDTiles = kDv / 16;   // 16-dim PV output tiles
constexpr int kPageBytes = kDk * kS;
constexpr int kMaxWavesL = 8;
constexpr int kMaxThreadsL = 64 * kMaxWavesL;
constexpr float kTauL = 8.0f;
constexpr float kLog2eL = 1.4426950408889634f;
constexpr int kHdrL = 64;           // header ints, then pref[B+1]
constexpr int kRow = kDv + 4;       // partial row: Dv sums, max, sum, 2 pad (16-byte rows)
constexpr int kMaxSeqsL = 2048;
// Q of k-steps [0, kQReg) stays in registers, the rest is read from LDS
// (registers would spill otherwise; a spill reload waits on the memory
// counter that also tracks the page copy in flight)
constexpr int kQReg = 11;
constexpr int kQLdsWave = (kKSteps - kQReg) * 64 * 16;   // bytes per wave (16 heads)
constexpr int kMaxHeadsL = 16 * kMaxWavesL;               // 128
// The page's weights p (f16) for the PV product, one row of 64 tokens per
// head, rows padded to 144 bytes so that the 16 rows one 16-byte operand read
// touches start in 16 different bank quads.
constexpr int kPRow = 144;

template <int F, int L>
struct sfor {
  template <typename Fn>
  __device__ __forceinline__ static void run(Fn&& fn) {
    if constexpr (F < L) {
      fn(std::integral_constant<int, F>{});
      sfor<F + 1, L>::run(fn);
    }
  }
};

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));

struct LatArgs {
  const uint16_t* __restrict__ q;
  const uint8_t* __restrict__ kc;
  const float* __restrict__ tscale;
  const int32_t* __restrict__ bt;
  const int32_t* __restrict__ lens;
  const int32_t* __restrict__ verdict;
  int32_t* hdr;         // [0] total pages T, [1] workgroups used, pref at kHdrL
  float* part;          // slots x Hq x (Dv + 2)
  float* out;
  int B, Hq, P, max_blocks;
  float sm_scale;
};

// Workgroup owning global page g when T pages are cut into W ranges
// [floor(wT/W), floor((w+1)T/W)).
__device__ __forceinline__ int owner_of(long long g, long long T, long long W) {
  return (int)(((g + 1) * W - 1) / T);
}

// Per-page LDS staging: codes, then three per-token arrays.
struct PageBuf {
  uint8_t codes[kPageBytes];
  float a[kS];     // scale * sm_scale * log2 e   (0 for tokens past the end)
  float b[kS];     // log2(scale)                  (-inf past the end)
  float inv[kS];   // 1 / scale                    (0 past the end)
  float sraw[kS];  // the page's scales as stored (copied with the codes)
};

// Maximum (sum) of a value over the four 16-lane rows of a wave, in every
// lane of the column: the row swaps of gfx950 (rows 2i+1 of one register
// with rows 2i of another, then the upper 32 lanes of one with the lower 32
// of the other) pair each lane with the same column of the other rows: two
// VALU swaps instead of two LDS permute round trips. Inline asm: the
// compiler folds the builtin swap of two equal values as if it changed
// nothing, and pads nothing around inline asm, so the two wait states before
// each swap (its sources were just written by VALU) are padded here.
__device__ __forceinline__ float rows_max(float x) {
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  float c = fmaxf(a, b), d = c;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(c), "+v"(d));
  return fmaxf(c, d);
}
__device__ __forceinline__ float rows_sum(float x) {
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  float c = a + b, d = c;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(c), "+v"(d));
  return c + d;
}

// The PV product is split by value dims over the workgroup's eight waves:
// wave w owns the four 16-dim column groups 4w .. 4w+3 (dims 64w .. +63).
constexpr int kPvGroups = kDTiles / kMaxWavesL;

// acc *= alpha for the (rare) running-max move, through this fragment's
// partial slot in global memory (written again at the end): the
// accumulators are stored straight from the matrix-core registers, scaled
// there, and loaded straight back, all in inline asm addressed by one
// per-lane 32-bit offset, a wave-uniform base per head tile and immediate
// offsets per column group. Nothing here takes more than a handful of
// vector registers, so the rare branch does not push the rest of the
// kernel's registers out to scratch (copying the accumulators through
// vector registers, or keeping a 64-bit address per tile, did). Every asm
// statement that loads waits for its own loads.
// acc[c][ht] register r: dim 16(cg0 + c) + 4g + r of head 16 ht + n, at
// byte 4((16 ht + n) kRow + 16(cg0 + c) + 4g + r) of the slot.
template <int C, int HT, int NH>
__device__ __forceinline__ void rescale_store(uint32_t voff, const float* b,
                                              const f32x4_t (&acc)[kPvGroups][NH]) {
  asm volatile("global_store_dwordx4 %0, %1, %2 offset:%3"
               :: "v"(voff), "a"(acc[C][HT]), "s"(b), "n"(64 * C) : "memory");
}
template <int C>
__device__ __forceinline__ void rescale_scale(uint32_t voff, const float* b, float al) {
  float t0, t1, t2, t3;
  asm volatile(
      "global_load_dword %0, %4, %5 offset:%6\n\t"
      "global_load_dword %1, %4, %5 offset:%7\n\t"
      "global_load_dword %2, %4, %5 offset:%8\n\t"
      "global_load_dword %3, %4, %5 offset:%9\n\t"
      "s_waitcnt vmcnt(0)\n\t"
      "v_mul_f32 %0, %0, %10\n\t"
      "v_mul_f32 %1, %1, %10\n\t"
      "v_mul_f32 %2, %2, %10\n\t"
      "v_mul_f32 %3, %3, %10\n\t"
      "s_nop 1\n\t"
      "global_store_dword %4, %0, %5 offset:%6\n\t"
      "global_store_dword %4, %1, %5 offset:%7\n\t"
      "global_store_dword %4, %2, %5 offset:%8\n\t"
      "global_store_dword %4, %3, %5 offset:%9"
      : "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3)
      : "v"(voff), "s"(b), "n"(64 * C), "n"(64 * C + 4), "n"(64 * C + 8), "n"(64 * C + 12),
        "v"(al)
      : "memory");
}
template <int C, int HT, int NH>
__device__ __forceinline__ void rescale_load(uint32_t voff, const float* b,
                                             f32x4_t (&acc)[kPvGroups][NH]) {
  asm volatile("global_load_dwordx4 %0, %1, %2 offset:%3\n\ts_waitcnt vmcnt(0)"
               : "=a"(acc[C][HT]) : "v"(voff), "s"(b), "n"(64 * C) : "memory");
}

template <int NH>
__device__ __forceinline__ void rescale_via(const float* slot, f32x4_t (&acc)[kPvGroups][NH],
                                            const float* alpha_lds, int cg0) {
  constexpr int CG = kPvGroups;
  const int lane = __lane_id();
  const int g = lane >> 4, n = lane & 15;
  const uint32_t voff = (uint32_t)((n * kRow + 16 * cg0 + 4 * g) * 4);
  // wave-uniform base of head tile ht (scalar registers)
  auto base = [&](int ht) -> const float* {
    const uint64_t b = (uint64_t)(uintptr_t)(slot + (int64_t)16 * ht * kRow);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    return (const float*)(uintptr_t)(((uint64_t)hi << 32) | lo);
  };
  sfor<0, NH * CG>::run([&](auto I) {
    constexpr int ht = decltype(I)::value / CG, c = decltype(I)::value % CG;
    rescale_store<c, ht, NH>(voff, base(ht), acc);
  });
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  // scale in place: one tile's four dwords per statement (the loads are
  // waited for inside it; two wait states between the multiplies and the
  // stores that read their results)
  sfor<0, NH * CG>::run([&](auto I) {
    constexpr int ht = decltype(I)::value / CG, c = decltype(I)::value % CG;
    rescale_scale<c>(voff, base(ht), alpha_lds[16 * ht + n]);
  });
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  sfor<0, NH * CG>::run([&](auto I) {
    constexpr int ht = decltype(I)::value / CG, c = decltype(I)::value % CG;
    rescale_load<c, ht, NH>(voff, base(ht), acc);
  });
}

// Eight waves for NH 16-head tiles (16 NH query heads). QK is split by
// heads: wave w < NH multiplies the page's keys with the Q of heads
// [16w, 16w+16) and takes their softmax (waves past NH have no QK work). PV
// is split by value dims: wave w owns column groups 4w .. 4w+3 of the output
// for every head, reading all heads' weights from LDS, so each V code is
// converted once per workgroup. Two waves run per SIMD, so one wave's
// conversions and softmax overlap the other's matrix products.
template <int NH>
__global__ __launch_bounds__(64 * kMaxWavesL)
__attribute__((amdgpu_waves_per_eu(2, 2)))
void latent_partial_kernel(LatArgs a) {
  constexpr int NW = kMaxWavesL;
  constexpr int CG = kPvGroups;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  PageBuf* buf = reinterpret_cast<PageBuf*>(smem);                    // [2]
  uint8_t* qlds_all = smem + 2 * sizeof(PageBuf);                     // NW x kQLdsWave
  uint8_t* pbuf = qlds_all + kMaxWavesL * kQLdsWave;                  // [Hq][kPRow]
  float* alpha_s = reinterpret_cast<float*>(pbuf + kMaxHeadsL * kPRow);  // [Hq]
  int* flag_s = reinterpret_cast<int*>(alpha_s + kMaxHeadsL);          // [NH]
  int* tmp = flag_s + kMaxWavesL;                                      // kMaxThreadsL + 1
  int* pref = tmp + kMaxThreadsL + 1;                                  // B + 1
  constexpr int NT = 64 * NW;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;        // 16-lane group: MFMA k slice / output row quad
  const int n = lane & 15;        // MFMA row (A) or column (B, output)
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int cg0 = CG * wv;        // first PV column group of this wave
  const bool qk = wv < NH;        // this wave has QK heads (wave-uniform)

  const int T = [&] {
    const int per = (a.B + NT - 1) / NT;
    const int beg = min(a.B, tid * per);
    const int end = min(a.B, beg + per);
    // each sequence's page count once (its length and verdict loaded
    // together), parked in pref[s] until the scan below overwrites it
    int local = 0;
    for (int s = beg; s < end; ++s) {
      const int len = a.lens[s];
      const int ver = a.verdict != nullptr ? a.verdict[s] : 0;
      const int np = (len <= 0 || len > a.max_blocks * kS || ver != 0) ? 0 : (len + kS - 1) / kS;
      pref[s] = np;
      local += np;
    }
    tmp[tid] = local;
    __syncthreads();
    if (tid == 0) {
      int run = 0;
      for (int i = 0; i < NT; ++i) {
        const int v = tmp[i];
        tmp[i] = run;
        run += v;
      }
      tmp[NT] = run;
    }
    __syncthreads();
    int run = tmp[tid];
    for (int s = beg; s < end; ++s) {
      const int np = pref[s];
      pref[s] = run;
      run += np;
    }
    const int total = tmp[NT];
    if (tid == 0) pref[a.B] = total;
    __syncthreads();
    return total;
  }();
  const long long W = min((long long)gridDim.x, (long long)T);
  if (blockIdx.x == 0) {
    for (int s = tid; s <= a.B; s += NT) a.hdr[kHdrL + s] = pref[s];
    if (tid == 0) {
      a.hdr[0] = T;
      a.hdr[1] = (int)W;
    }
  }
  if ((long long)blockIdx.x >= W) return;
  const int w = blockIdx.x;
  const int lo = (int)((long long)w * T / W);
  const int hi = (int)((long long)(w + 1) * T / W);
  const float c0 = a.sm_scale * kLog2eL;
  const int head0 = wave * 16;    // this wave's QK heads

  int gp = lo;
  while (gp < hi) {
    // sequence owning global page gp: last s with pref[s] <= gp
    int sl = 0, sh = a.B;
    while (sh - sl > 1) {
      const int mid = (sl + sh) >> 1;
      if (pref[mid] <= gp) sl = mid; else sh = mid;
    }
    const int s = __builtin_amdgcn_readfirstlane(sl);
    const int j0 = gp - pref[s];
    const int j1 = min(hi, pref[s + 1]) - pref[s];
    const int len = a.lens[s];
    const int32_t* btrow = a.bt + (int64_t)s * a.max_blocks;
    // this fragment's partial slot; the PV output rows this lane holds are
    // those of heads 16 ht + n
    float* const slot = a.part + (int64_t)(w + s) * a.Hq * kRow;
    float* const prow = slot + n * kRow;

    // ---- Q of this wave's heads, resident for the fragment --------------
    // B operand of k-step k: lane (head head0 + n, group g) holds dims
    // 32k + 8g .. +7. Steps below kQReg stay in registers; the others go to
    // this wave's LDS region as [k - kQReg][lane][16 bytes] (only this wave
    // reads it, after its own writes).
    bf16x8_t qreg[kQReg];
    uint8_t* qlds = qlds_all + wave * kQLdsWave + lane * 16;
    if (qk) {
      const uint16_t* qrow = a.q + ((int64_t)s * a.Hq + head0 + n) * kDk + 8 * g;
#pragma unroll
      for (int k = 0; k < kKSteps; ++k) {
        const uint4 v = *reinterpret_cast<const uint4*>(qrow + 32 * k);
        if (k < kQReg)
          qreg[k] = __builtin_bit_cast(bf16x8_t, v);
        else
          *reinterpret_cast<uint4*>(qlds + (k - kQReg) * 1024) = v;
      }
    }

    f32x4_t acc[CG][NH];
#pragma unroll
    for (int c = 0; c < CG; ++c)
#pragma unroll
      for (int ht = 0; ht < NH; ++ht) acc[c][ht] = f32x4_t{};
    // running max of y of this lane's QK head (the same in its four lanes)
    float m = -INFINITY, l = 0.0f;   // l: this lane's tokens' share of the weight sum
    bool bad = false;

    // ---- page staging ------------------------------------------------------
    // The page (36 column groups x 64 tokens x 16 bytes, contiguous) is
    // copied global -> LDS directly (global_load_lds_dwordx4: each lane's 16
    // bytes land at the wave-uniform LDS address + 16 * lane), so staging
    // takes no registers. The copy of page j+1 runs while page j computes.
    constexpr int kWaveChunks = kPageBytes / (16 * 64);    // 36 wave copies
    auto fetch = [&](int page, PageBuf& pb) {
      if (page < 0 || page >= a.P) {
        bad = true;
        page = 0;
      }
      const uint8_t* src = a.kc + (int64_t)page * kPageBytes;
      // Issued as inline asm: the compiler would make the first LDS read
      // after a copy it can see wait for all of it, which serialises the
      // copy of page j+1 with the arithmetic of page j. The wait at the top
      // of the page loop (all vector memory, then a barrier) covers it.
      const uint32_t l0 = __builtin_amdgcn_readfirstlane(
          (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t*)pb.codes));
      // The page base is wave-uniform: each copy takes an SGPR base (page +
      // i KB, scalar arithmetic) and the one per-lane offset lane * 16, so no
      // per-copy lane address is kept in (or spilled from) vector registers.
      // (readfirstlane takes and returns 32 bits: each half separately)
      const uint64_t s64 = (uint64_t)(uintptr_t)src;
      const uint32_t s_lo = __builtin_amdgcn_readfirstlane((uint32_t)s64);
      const uint32_t s_hi = __builtin_amdgcn_readfirstlane((uint32_t)(s64 >> 32));
      const uint8_t* srcu = (const uint8_t*)(uintptr_t)(((uint64_t)s_hi << 32) | s_lo);
      // recomputed here (opaque to the compiler, three VALU instructions)
      // rather than kept live across the page and spilled; s_nop 0 below:
      // one wait state between a scalar write of M0 and the copy using it
      uint32_t lane16;
      asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0\n\t"
                   "v_lshlrev_b32 %0, 4, %0" : "=v"(lane16));
#pragma unroll
      for (int ii = 0; ii < (kWaveChunks + NW - 1) / NW; ++ii) {
        const int i = ii * NW + wv;
        if (kWaveChunks % NW != 0 && i >= kWaveChunks) break;   // uniform
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                     :: "s"(l0 + (uint32_t)i * 1024u), "v"(lane16), "s"(srcu + (int64_t)i * 1024)
                     : "memory");
      }
      // the page's 64 scales, by wave 0: lane i's 4 bytes land at sraw + 4 i
      if (wv == 0) {
        const uint32_t ls = __builtin_amdgcn_readfirstlane(
            (uint32_t)(uintptr_t)((__attribute__((address_space(3))) float*)pb.sraw));
        const uint64_t t64 = (uint64_t)(uintptr_t)(a.tscale + (int64_t)page * kS);
        const uint32_t t_lo = __builtin_amdgcn_readfirstlane((uint32_t)t64);
        const uint32_t t_hi = __builtin_amdgcn_readfirstlane((uint32_t)(t64 >> 32));
        const float* tsu = (const float*)(uintptr_t)(((uint64_t)t_hi << 32) | t_lo);
        uint32_t lane4;
        asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0\n\t"
                     "v_lshlrev_b32 %0, 2, %0" : "=v"(lane4));
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
                     :: "s"(ls), "v"(lane4), "s"(tsu) : "memory");
      }
    };
    // Page j's per-token arrays, by wave 0 (the wave that copied the page's
    // scales) once its own copies of the page have landed: a = c_t sm_scale
    // log2(e), b = log2(c_t), inv = 1 / c_t, and a = 0, b = -inf, inv = 0 for
    // tokens past the end.
    auto factors = [&](int j, PageBuf& pb) {
      const int valid = min(kS, len - j * kS);   // tokens of this page in use
      // lane i: token i (v_log_f32 is log2)
      const float sc = pb.sraw[lane];
      const bool live = lane < valid;
      pb.a[lane] = live ? sc * c0 : 0.0f;
      pb.b[lane] = live ? __builtin_amdgcn_logf(sc) : -INFINITY;
      pb.inv[lane] = live ? 1.0f / sc : 0.0f;
    };

    // physical page ids are read one page ahead of their copies, through
    // scalar loads (a block-table read just before the copy stalled every
    // page by a memory round trip)
    typedef const int32_t __attribute__((address_space(4))) ci32l_t;
    ci32l_t* btc = (ci32l_t*)(uintptr_t)btrow;
    int pid_next = j0 + 1 < j1 ? btc[j0 + 1] : 0;
    fetch(btc[j0], buf[0]);
    if (wv == 0) {
      __builtin_amdgcn_s_waitcnt(0);
      factors(j0, buf[0]);
    }
    for (int j = j0; j < j1; ++j) {
      PageBuf& pb = buf[(j - j0) & 1];
      // page j's copy (and every earlier load) complete, and its per-token
      // arrays written; then publish. Past this barrier every wave has also
      // finished the PV product of page j-1, so the weights buffer and the
      // rescale factors may be rewritten.
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      // Tokens past the end (the last page of a sequence only): their codes
      // are zeroed once the copy has landed, so they add nothing whatever the
      // slot held, and a second barrier publishes the zeros.
      {
        const int valid = min(kS, len - j * kS);
        if (valid < kS) {
          for (int c = tid; c < kPageBytes / 16; c += NT)
            if ((c % kS) >= valid) *reinterpret_cast<uint4*>(pb.codes + c * 16) = make_uint4(0, 0, 0, 0);
          __syncthreads();
        }
      }
      // The next page's copy goes out after this page's QK products, at the
      // start of the softmax (the other buffer's last readers, page j - 1,
      // passed the barrier above). Nothing after the copy waits on the vector
      // memory counter until the end of the page, except the rare rescale: a
      // wait there would wait for the whole copy and serialise it with this
      // page's products.
      const int pid_copy = pid_next;   // page j + 1, copied below
      pid_next = j + 2 < j1 ? btc[j + 2] : 0;

      if (qk) {
      // ---- QK: S^T (64 tokens x 16 heads) as 4 tiles of 16 x 16 ----------
      // A operand of k-step k, token tile t: lane (row i = n, group g) holds
      // the codes of dims 32k + 8g .. +7 of token 16t + n (column group
      // 2k + g/2, bytes 8(g&1) .. +7 of its 16-byte slot; one 8-byte LDS
      // read). Unit u = 4k + t; reads run four units ahead, and the
      // scheduling barrier per unit keeps the compiler from hoisting every
      // read and conversion (a register each). A half-wave reads 16 tokens'
      // whole slots: every bank once.
      f32x4_t st[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) st[t] = f32x4_t{};
      {
        const uint8_t* rowk = pb.codes + (g >> 1) * (kS * 16) + n * 16 + 8 * (g & 1);
        auto rdk = [&](int u) -> uint2 {
          const int k = u >> 2, t = u & 3;
          return *reinterpret_cast<const uint2*>(rowk + k * (2 * kS * 16) + t * (16 * 16));
        };
        constexpr int kAhead = 4;
        constexpr int kUnits = 4 * kKSteps;
        uint2 ring[kAhead];
#pragma unroll
        for (int u = 0; u < kAhead; ++u) ring[u] = rdk(u);
        // LDS-resident Q of step k is read during step k - 1 (unit t = 1)
        auto rdq = [&](int k) -> bf16x8_t {
          return __builtin_bit_cast(bf16x8_t,
                                    *reinterpret_cast<const uint4*>(qlds + (k - kQReg) * 1024));
        };
        bf16x8_t qn[2];
        sfor<0, kUnits>::run([&](auto U) {
          constexpr int u = decltype(U)::value;
          constexpr int k = u >> 2, t = u & 3;
          const uint2 cw = ring[u % kAhead];
          const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw.x, 1.0f, false);
          const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw.x, 1.0f, true);
          const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw.y, 1.0f, false);
          const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw.y, 1.0f, true);
          if constexpr (u + kAhead < kUnits) ring[u % kAhead] = rdk(u + kAhead);
          if constexpr (t == 1 && k + 1 >= kQReg && k + 1 < kKSteps) qn[(k + 1) & 1] = rdq(k + 1);
          const bf16x8_t av = {p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
          if constexpr (k < kQReg)
            st[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, qreg[k], st[t], 0, 0, 0);
          else
            st[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, qn[k & 1], st[t], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        });
      }

      // the next page's copies, at the start of the softmax (its vector ALU
      // work leaves memory issue idle; spread over the QK products they
      // slowed QK, whose LDS reads the copies' writes then met)
      if (j + 1 < j1) fetch(pid_copy, buf[(j + 1 - j0) & 1]);
      // ---- softmax of this wave's heads (log2 units, scale folded in) -----
      // st[t] register r holds token 16t + 4g + r of head head0 + n
      float bm = -INFINITY;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int t0 = 16 * t + 4 * g;
        const float4 av = *reinterpret_cast<const float4*>(pb.a + t0);
        const float4 bv = *reinterpret_cast<const float4*>(pb.b + t0);
        const float aa[4] = {av.x, av.y, av.z, av.w};
        const float bb[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = fmaf(st[t][r], aa[r], bb[r]);
          st[t][r] = v;
          bm = fmaxf(bm, v);
        }
      }
      bm = rows_max(bm);
      // the running max moves only when the page's max exceeds it by more
      // than the threshold; alpha rescales what was summed under the old max
      const bool mv = bm > m + kTauL;
      const float m_old = m;
      if (mv) m = bm;
      const float al = mv ? __builtin_amdgcn_exp2f(m_old - m) : 1.0f;
      l *= al;
      const bool resc = __ballot(mv && m_old != -INFINITY) != 0;
      if (g == 0) alpha_s[head0 + n] = al;
      if (lane == 0) flag_s[wave] = resc ? 1 : 0;
      // p' = 2^(y - m) as f16, to this head's row of the weights buffer:
      // lane (n, g) holds tokens 16t + 4g .. +3, one 8-byte store per tile
      uint8_t* prow_p = pbuf + (head0 + n) * kPRow + 8 * g;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int t0 = 16 * t + 4 * g;
        const float4 iv = *reinterpret_cast<const float4*>(pb.inv + t0);
        const float ii[4] = {iv.x, iv.y, iv.z, iv.w};
        _Float16 ph[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = __builtin_amdgcn_exp2f(st[t][r] - m);
          l = fmaf(p, ii[r], l);
          ph[r] = (_Float16)p;
        }
        *reinterpret_cast<uint2*>(prow_p + 32 * t) = __builtin_bit_cast(uint2, ph);
      }
      }
      if (!qk && j + 1 < j1) fetch(pid_copy, buf[(j + 1 - j0) & 1]);
      __syncthreads();

      // ---- PV: O^T (this wave's dims x all heads) += V^T P^T ---------------
      // Heads whose running max moved: acc *= alpha first (rare).
      {
        int fl = 0;
#pragma unroll
        for (int i = 0; i < NH; ++i) fl |= flag_s[i];
        if (fl != 0) rescale_via<NH>(slot, acc, alpha_s, cg0);
      }
      // k-step kk covers tokens 32kk .. +31. A operand (V^T, column group
      // cg0 + c): the transpose read ds_read_b64_tr_b8, lane 2b + e of each
      // 16-lane group g addressing token 32kk + 8g + b, bytes 8e .. +7 of
      // the group's 16-byte slot, leaves in lane i the codes of dim
      // 16(cg0 + c) + i for tokens 32kk + 8g .. +7 (element b = token
      // 32kk + 8g + b). B operand (P^T, head tile ht): lane (n, g) reads
      // the weights of tokens 32kk + 8g .. +7 of head 16 ht + n, 16 bytes.
      // Four column groups' A operands are converted once and used against
      // every head tile.
      {
        const int li = lane & 15;
        const uint8_t* vbase = pb.codes + (8 * g + (li >> 1)) * 16 + 8 * (li & 1) + cg0 * (kS * 16);
        const uint8_t* pbase = pbuf + n * kPRow + 16 * g;
        auto rdp = [&](int kk, int ht) -> f16x8_t {
          return *reinterpret_cast<const f16x8_t*>(pbase + 16 * ht * kPRow + 64 * kk);
        };
        static_assert(CG == 4, "four column groups per wave");
        sfor<0, 2>::run([&](auto KK) {
          constexpr int kk = decltype(KK)::value;
          f16x8_t pw[2];
          pw[0] = rdp(kk, 0);
          f16x8_t av[CG];
#pragma unroll
          for (int c = 0; c < CG; ++c) {
            const i32x2_t cw = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (__attribute__((address_space(3))) i32x2_t*)(vbase + kk * (32 * 16) +
                                                             c * (kS * 16)));
            const f16x2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((uint32_t)cw.x, 1.0f, false);
            const f16x2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((uint32_t)cw.x, 1.0f, true);
            const f16x2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((uint32_t)cw.y, 1.0f, false);
            const f16x2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((uint32_t)cw.y, 1.0f, true);
            av[c] = f16x8_t{v0.x, v0.y, v1.x, v1.y, v2.x, v2.y, v3.x, v3.y};
          }
          __builtin_amdgcn_sched_barrier(0);
          sfor<0, NH>::run([&](auto H) {
            constexpr int ht = decltype(H)::value;
            if constexpr (ht + 1 < NH) pw[(ht + 1) & 1] = rdp(kk, ht + 1);
            const f16x8_t pv = pw[ht & 1];
            // inline asm pins the accumulators to AGPRs, leaving the VGPRs
            // to the score tiles; s_nop 1 covers a VALU write of an operand
            // just before (two wait states)
            asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_f16 %0, %1, %2, %0"
                         : "+a"(acc[0][ht]) : "v"(av[0]), "v"(pv));
            asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0"
                         : "+a"(acc[1][ht]) : "v"(av[1]), "v"(pv));
            asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0"
                         : "+a"(acc[2][ht]) : "v"(av[2]), "v"(pv));
            asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0"
                         : "+a"(acc[3][ht]) : "v"(av[3]), "v"(pv));
            __builtin_amdgcn_sched_barrier(0);
          });
        });
      }
      // The next page's per-token arrays, by wave 0 after its own copies
      // (scales included) have landed: it finishes its PV products ahead of
      // the waves that share its SIMD, so this work (and the wait) mostly
      // falls in time the barrier at the top of the next page would idle.
      // The buffer's last readers, the softmax of page j - 1, are past the
      // barrier before this page's PV.
      if (wv == 0 && j + 1 < j1) {
        __builtin_amdgcn_s_waitcnt(0);
        factors(j + 1, buf[(j + 1 - j0) & 1]);
      }
    }

    // the last PV results land before the accumulators are read (24 wait
    // states; the compiler does not see the matrix-core writes in the asm)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    // ---- partial of this fragment -------------------------------------------
    l = rows_sum(l);
    const bool any_bad = __syncthreads_or(bad ? 1 : 0) != 0;
    if (!any_bad) {
      // acc[c][ht] register r: dim 16(cg0 + c) + 4g + r of head 16 ht + n
#pragma unroll
      for (int c = 0; c < CG; ++c)
#pragma unroll
          for (int ht = 0; ht < NH; ++ht)
            *reinterpret_cast<f32x4_t*>(prow + 16 * ht * kRow + 16 * (cg0 + c) + 4 * g) = acc[c][ht];
    }
    if (qk && g == 0) {
      // the running max and weight sum of this wave's QK head head0 + n
      float* mrow = a.part + ((int64_t)(w + s) * a.Hq + head0 + n) * kRow;
      mrow[kDv] = any_bad ? __builtin_nanf("") : m;
      mrow[kDv + 1] = l;
    }
    gp = pref[s] + j1;
    __syncthreads();
  }
}

// Merge the fragments of one sequence: one workgroup per (sequence, 4 heads),
// 64 threads per head, 8 dims per thread.
__global__ __launch_bounds__(256) void latent_combine_kernel(LatArgs a) {
  const int s = blockIdx.x / (a.Hq / 4);
  const int hd = (blockIdx.x % (a.Hq / 4)) * 4 + (threadIdx.x >> 6);
  const int d0 = (threadIdx.x & 63) * 8;
  float* o = a.out + ((int64_t)s * a.Hq + hd) * kDv + d0;
  const int len = a.lens[s];
  const bool aborted = a.verdict != nullptr && a.verdict[s] != 0;
  const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
  if (aborted || len == 0) {
    reinterpret_cast<float4*>(o)[0] = z4;
    reinterpret_cast<float4*>(o)[1] = z4;
    return;
  }
  const float qnan = __builtin_nanf("");
  const float4 n4 = make_float4(qnan, qnan, qnan, qnan);
  if (len < 0 || len > a.max_blocks * kS) {
    reinterpret_cast<float4*>(o)[0] = n4;
    reinterpret_cast<float4*>(o)[1] = n4;
    return;
  }
  const long long T = a.hdr[0];
  const long long W = a.hdr[1];
  const int* pref = a.hdr + kHdrL;
  const int w0 = owner_of(pref[s], T, W);
  const int w1 = owner_of(pref[s + 1] - 1, T, W);
  // Fragments are taken kC at a time: every load of a chunk is issued before
  // any of its results is used, so a sequence costs one memory round trip
  // per chunk (two serial loops over the fragments, the maxima first, took
  // two round trips per fragment). Chunks merge by a running max; with one
  // chunk this is exactly the max-then-sum rule.
  constexpr int kC = 8;
  float M = -INFINITY, L = 0.0f;
  float4 x0 = z4, x1 = z4;
  bool nan = false;
  for (int wb = w0; wb <= w1; wb += kC) {
    float mw[kC], lw[kC];
    float4 v0[kC], v1[kC];
    // past the last fragment the index is clamped to it (no branch, so the
    // chunk's loads stay together) and the entry is given weight 0 below
#pragma unroll
    for (int i = 0; i < kC; ++i) {
      const float* pw = a.part + ((int64_t)(min(wb + i, w1) + s) * a.Hq + hd) * kRow;
      mw[i] = pw[kDv];
      lw[i] = pw[kDv + 1];
      v0[i] = reinterpret_cast<const float4*>(pw + d0)[0];
      v1[i] = reinterpret_cast<const float4*>(pw + d0)[1];
    }
    // (left to itself the compiler issues the rows' loads after the maxima
    // have arrived: two round trips a chunk)
    __builtin_amdgcn_sched_barrier(0);
    float Mc = M;
#pragma unroll
    for (int i = 0; i < kC; ++i) {
      nan |= __builtin_isnan(mw[i]);
      Mc = fmaxf(Mc, wb + i <= w1 ? mw[i] : -INFINITY);
    }
    // what earlier chunks summed under M, rescaled to Mc
    const float r = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(M - Mc);
    L *= r;
    x0.x *= r; x0.y *= r; x0.z *= r; x0.w *= r;
    x1.x *= r; x1.y *= r; x1.z *= r; x1.w *= r;
#pragma unroll
    for (int i = 0; i < kC; ++i) {
      const float f = wb + i <= w1 ? __builtin_amdgcn_exp2f(mw[i] - Mc) : 0.0f;
      L += f * lw[i];
      x0.x += f * v0[i].x; x0.y += f * v0[i].y; x0.z += f * v0[i].z; x0.w += f * v0[i].w;
      x1.x += f * v1[i].x; x1.y += f * v1[i].y; x1.z += f * v1[i].z; x1.w += f * v1[i].w;
    }
    M = Mc;
  }
  if (nan) {
    reinterpret_cast<float4*>(o)[0] = n4;
    reinterpret_cast<float4*>(o)[1] = n4;
    return;
  }
  const float inv = 1.0f / L;
  reinterpret_cast<float4*>(o)[0] = make_float4(x0.x * inv, x0.y * inv, x0.z * inv, x0.w * inv);
  reinterpret_cast<float4*>(o)[1] = make_float4(x1.x * inv, x1.y * inv, x1.z * inv, x1.w * inv);
}

size_t lat_header_bytes(int B) {
  const size_t h = (size_t)(kHdrL + B + 1) * sizeof(int32_t);
  return (size_t)((h + 255) & ~(size_t)255);
}

size_t lat_slot_bytes(const pda_attn_shape& sh) {
  return (size_t)sh.num_q_heads * kRow * sizeof(float);
}

size_t lat_lds_bytes(int B) {
  return 2 * sizeof(PageBuf) + (size_t)kMaxWavesL * kQLdsWave + (size_t)kMaxHeadsL * kPRow +
         (size_t)kMaxHeadsL * sizeof(float) +
         (size_t)(kMaxWavesL + kMaxThreadsL + 1 + B + 1) * sizeof(int);
}

typedef void (*lat_kernel_t)(LatArgs);

// head tiles of 16 query heads (Hq / 16)
lat_kernel_t pick_latent(int nh) {
  switch (nh) {
    case 2: return latent_partial_kernel<2>;
    case 4: return latent_partial_kernel<4>;
    case 6: return latent_partial_kernel<6>;
    default: return latent_partial_kernel<8>;
  }
}

}  // namespace

int device_cu_count();

bool latent_supported(const pda_attn_shape& sh) {
  return sh.v_in_k == 1 && sh.kv_dtype == PDA_KV_FP8_E4M3 &&
         sh.scale_mode == PDA_SCALE_PER_TOKEN && sh.num_kv_heads == 1 &&
         sh.head_dim_qk == kDk && sh.head_dim_v == kDv && sh.page_size == kS &&
         sh.num_q_heads % 32 == 0 && sh.num_q_heads <= 128 &&
         sh.num_seqs <= kMaxSeqsL;
}

// One workgroup per compute unit; every workgroup may leave one partial per
// sequence fragment, and slot (workgroup + sequence) is unique.
size_t latent_workspace_bytes(const pda_attn_shape& sh, int32_t max_seq_len) {
  (void)max_seq_len;
  const size_t slots = (size_t)device_cu_count() + (size_t)sh.num_seqs;
  return lat_header_bytes(sh.num_seqs) + slots * lat_slot_bytes(sh);
}

// Smallest workspace the call accepts: one partial per sequence plus one.
size_t latent_min_workspace_bytes(const pda_attn_shape& sh) {
  return lat_header_bytes(sh.num_seqs) + lat_slot_bytes(sh) * ((size_t)sh.num_seqs + 1);
}

int latent_launch(const pda_attn_shape& sh, const void* q, const void* k_cache,
                  const float* token_scale, const int32_t* block_table, const int32_t* seq_lens,
                  int32_t max_seq_len, const int32_t* verdict, void* workspace,
                  size_t workspace_bytes, float* out, hipStream_t stream) {
  (void)max_seq_len;
  const size_t hdr = lat_header_bytes(sh.num_seqs);
  const size_t slot = lat_slot_bytes(sh);
  if (workspace_bytes < latent_min_workspace_bytes(sh)) return PDA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0) return PDA_ERR_INVALID_ARG;
  long long grid = device_cu_count();
  const long long fit = (long long)((workspace_bytes - hdr) / slot) - sh.num_seqs;
  if (grid > fit) grid = fit;
  if (grid < 1) grid = 1;
  LatArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.kc = static_cast<const uint8_t*>(k_cache);
  a.tscale = token_scale;
  a.bt = block_table;
  a.lens = seq_lens;
  a.verdict = verdict;
  a.hdr = static_cast<int32_t*>(workspace);
  a.part = reinterpret_cast<float*>(static_cast<char*>(workspace) + hdr);
  a.out = out;
  a.B = sh.num_seqs;
  a.Hq = sh.num_q_heads;
  a.P = sh.num_pages;
  a.max_blocks = sh.max_blocks_per_seq;
  a.sm_scale = sh.sm_scale;
  const int nh = sh.num_q_heads / 16;
  const size_t lds = lat_lds_bytes(sh.num_seqs);
  lat_kernel_t k = pick_latent(nh);
  // the dynamic LDS limit, raised once per kernel and device
  static std::mutex mu;
  static bool raised[kMaxWavesL + 1][64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return PDA_ERR_LAUNCH;
  {
    std::lock_guard<std::mutex> lock(mu);
    if (!raised[nh][dev]) {
      if (hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                              hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)lat_lds_bytes(kMaxSeqsL)) != hipSuccess)
        return PDA_ERR_LAUNCH;
      raised[nh][dev] = true;
    }
  }
  hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(64 * kMaxWavesL), lds, stream, a);
  if (hipGetLastError() != hipSuccess) return PDA_ERR_LAUNCH;
  hipLaunchKernelGGL(latent_combine_kernel, dim3((unsigned)(sh.num_seqs * (sh.num_q_heads / 4))),
                     dim3(256), 0, stream, a);
  return launch_status();
}

}  // namespace pda
