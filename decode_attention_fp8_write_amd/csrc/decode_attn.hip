// decode_attn.hip — single-query-per-sequence attention over a paged KV
// cache, FP8 e4m3 or BF16, for GQA groups below 16 query rows per kv head.
//
// The pages describe the FP8 cache and its cost: the attention kernel has to
// convert every cached value it reads, which made it a few percent slower
// than BF16 at equal concurrency, while halving the memory per token
// (aifeed.sk, "Cloudflare zrýchľuje inferenciu modelov Kimi a GLM kompresiou
// cache a váh", section "Dve odlišné úzke miesta v pamäti GPU"; manulx.blog,
// "Công thức của Cloudflare để phục vụ Kimi và GLM", section "Bộ nhớ đệm KV
// FP8 tăng gấp đôi dung lượng ngữ cảnh"). The kernel design below is not from
// the pages, which give none.
//
// Work decomposition. A sequence's context is cut into page-aligned chunks
// (split-K). A work item is (sequence, chunk, kv head) and belongs to one
// wavefront; a workgroup of four waves takes units of four consecutive chunk
// slots of one (sequence, kv head), so the G query rows are staged in LDS once
// per unit. Each workgroup first derives the slot list from seq_lens and the
// verdicts (aborted sequences get no slots, so none of their pages is read;
// a sequence's slot count is its chunk count rounded up to a multiple of
// four, and a padding slot does nothing). Each wave leaves its partial
// (unnormalised output rows, running max, running sum) in LDS; the workgroup
// merges the unit's four with a log-sum-exp rule and writes one partial per
// unit to the workspace, and the combine kernel merges a sequence's units
// with the same rule.
//
// Inside an item a wave walks 64 tokens (a block) at a time:
//  * QK: lane = token. FP8 keys reach the wave's own LDS buffer by direct
//    global->LDS copies issued one block ahead (no registers hold them in
//    flight); BF16 keys come through registers. Code pairs convert exactly to
//    bf16 and v_dot2_f32_bf16 accumulates q.k for all G query rows. For FP8
//    the q pair is taken from another lane by a DPP row broadcast (lane
//    2r + j of each row of 16 lanes holds dwords of row r, read from the
//    unit's LDS copy of q); for BF16 it is a wave-uniform SGPR pair fetched
//    by scalar loads.
//  * softmax in log2 units with a lazy running max: it only moves when some
//    score of the block exceeds it by more than kTau (a per-row ballot), so
//    p <= 2^kTau and the wave-wide maximum is rarely needed.
//  * p goes to the wave's LDS buffer (f16, or a bf16 high part and a bf16
//    remainder for BF16 caches, relative error 2^-16).
//  * PV: lane = two dims, all 64 tokens. The V format puts the two tokens of
//    an even/odd slot pair next to each other, so one V word is (dim, 2
//    tokens) x 2 dims; its codes convert exactly to two f16 pairs and
//    v_dot2_f32_f16 takes the matching p pair. For FP8 one 8-byte LDS read
//    per lane brings the p of 8 tokens of one row, and a DPP row broadcast
//    hands each pair to every lane; for BF16 p comes as a 16-byte broadcast
//    read.
//  * V of the next block is loaded into registers once PV is done.
// Every dot product accumulates in fp32; q enters exactly (bf16), K and V
// codes convert exactly, and p is rounded once.
//
// gfx950 wait states that the compiler does not insert around inline asm,
// which the DPP dots are: a DPP operand must not have been written by a VALU
// instruction in the two instructions before, and a dot result may be read by
// a different instruction only three instructions later (a chain of the same
// dot opcode through its accumulator is forwarded). The s_nop helpers below
// pad exactly these places, and a test checks the emitted assembly.
#include <mutex>
#include <type_traits>

#include "pda_internal.h"

namespace pda {
namespace {

constexpr int kD = 128;          // head dim (qk and v) of this path
constexpr int kThreads = 256;    // 4 waves per workgroup
constexpr int kWaves = kThreads / 64;
constexpr float kTau = 8.0f;     // lazy-rescale threshold, log2 units
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kHdrInts = 64;     // workspace header, then prefix[B+1]

struct AttnArgs {
  const uint16_t* __restrict__ q;
  const uint8_t* __restrict__ kc;
  const uint8_t* __restrict__ vc;
  const float* __restrict__ k_scale;
  const float* __restrict__ v_scale;
  const int32_t* __restrict__ bt;
  const int32_t* __restrict__ lens;
  const int32_t* __restrict__ verdict;
  int32_t* ws_hdr;      // [0] chunk tokens, [1] seq-chunks, then prefix[B+1]
  float* ws_part;       // partials (one per unit and kv head) * G * (D + 2)
  float* out;
  int B, Hq, Hkv, P, max_blocks;
  int chunk0;           // requested chunk (tokens), multiple of 64 and S
  long long cap_items;  // unit partials that fit in the workspace
  float sm_scale;
};

template <int F, int L>
struct static_for {
  template <typename Fn>
  __device__ __forceinline__ static void run(Fn&& fn) {
    if constexpr (F < L) {
      fn(std::integral_constant<int, F>{});
      static_for<F + 1, L>::run(fn);
    }
  }
};

__device__ __forceinline__ int n_chunks_of(const AttnArgs& a, int s, int S, int chunk) {
  const int len = a.lens[s];
  if (len <= 0 || len > a.max_blocks * S) return 0;
  if (a.verdict != nullptr && a.verdict[s] != 0) return 0;
  return (len + chunk - 1) / chunk;
}


// Every workgroup derives the same plan: chunk size (doubled until the
// unit partials fit the workspace) and the exclusive prefix of chunk slots per
// sequence, kept in LDS (pref[0..B]). Workgroup 0 also publishes it.
__device__ int build_plan(const AttnArgs& a, int S, int* pref, int* tmp, int& chunk_out) {
  const int tid = threadIdx.x;
  const int per = (a.B + kThreads - 1) / kThreads;
  const int beg = min(a.B, tid * per);
  const int end = min(a.B, beg + per);
  const int lane = tid & 63, wave = tid >> 6;
  int chunk = a.chunk0;
  int total = 0;
  // Each sequence's length and verdict are loaded together, once, and the
  // length it contributes (0 if aborted or malformed) is parked in pref[s]
  // until the scan overwrites it (loaded on demand, every count of the plan
  // took two dependent round trips, twice over: 4.5 us of every workgroup's
  // start). A retry with a doubled chunk loads them again.
  for (int s = beg; s < end; ++s) {
    const int len = a.lens[s];
    const int ver = a.verdict != nullptr ? a.verdict[s] : 0;
    pref[s] = (len <= 0 || len > a.max_blocks * S || ver != 0) ? 0 : len;
  }
  bool parked = true;
  // chunk slots of a sequence: its chunk count rounded up to a multiple of
  // the waves of a workgroup (one work unit = kWaves consecutive chunks of
  // one (sequence, kv head), one per wave)
  auto slots = [&](int s) -> int {
    const int len = parked ? pref[s] : (n_chunks_of(a, s, S, 1) > 0 ? a.lens[s] : 0);
    return ((len + chunk - 1) / chunk + kWaves - 1) / kWaves * kWaves;
  };
  for (;;) {
    int local = 0;
    for (int s = beg; s < end; ++s) local += slots(s);
    // exclusive prefix of `local` over the workgroup: an inclusive scan
    // within each wave, then the totals of the waves before this one
    int v = local;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(v, o);
      if (lane >= o) v += t;
    }
    if (lane == 63) tmp[wave] = v;
    __syncthreads();
    int run = v - local;
    total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int t = tmp[w];
      if (w < wave) run += t;
      total += t;
    }
    for (int s = beg; s < end; ++s) {
      const int n = slots(s);
      pref[s] = run;
      run += n;
    }
    parked = false;
    __syncthreads();
    if ((long long)(total / kWaves) * a.Hkv <= a.cap_items) break;
    chunk *= 2;
  }
  if (tid == 0) pref[a.B] = total;
  __syncthreads();
  if (blockIdx.x == 0) {
    for (int s = tid; s <= a.B; s += kThreads) a.ws_hdr[kHdrInts + s] = pref[s];
    if (tid == 0) {
      a.ws_hdr[0] = chunk;
      a.ws_hdr[1] = total;
    }
  }
  chunk_out = chunk;
  return total;
}

// Query rows and block-table entries are read through the constant address
// space, so wave-uniform loads become scalar loads into SGPRs. The 512 q
// dwords of a G = 8 group cannot stay resident in SGPRs, so they are re-read
// every block in small chunks.
typedef const uint32_t __attribute__((address_space(4))) cu32_t;
typedef const int32_t __attribute__((address_space(4))) ci32_t;

// Opaque identity on the q pointer that also "uses and redefines" the score
// accumulators: loads through the returned pointer cannot move above the dot
// products that produced z, and those dot products cannot sink below it.
template <int R>
__device__ __forceinline__ cu32_t* fence_ptr_after(cu32_t* p, float (&z)[R]) {
  uint64_t v = (uint64_t)(uintptr_t)p;
  if constexpr (R == 1) {
    asm volatile("" : "+s"(v), "+v"(z[0]));
  } else if constexpr (R == 2) {
    asm volatile("" : "+s"(v), "+v"(z[0]), "+v"(z[1]));
  } else if constexpr (R == 4) {
    asm volatile("" : "+s"(v), "+v"(z[0]), "+v"(z[1]), "+v"(z[2]), "+v"(z[3]));
  } else {
    asm volatile("" : "+s"(v), "+v"(z[0]), "+v"(z[1]), "+v"(z[2]), "+v"(z[3]), "+v"(z[4]),
                 "+v"(z[5]), "+v"(z[6]), "+v"(z[7]));
  }
  return (cu32_t*)(uintptr_t)v;
}

__device__ __forceinline__ uint32_t u4_get(const uint4& v, int j) {
  return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
}

// Two wait states after the conversions of one step, tied to their results
// so that the inline-asm dots that read them cannot be scheduled closer: a
// scaled conversion's result is not forwarded to an immediately following
// instruction, and the compiler only pads consumers it can see.
template <typename T>
__device__ __forceinline__ void settle8(T (&v)[8]) {
  asm volatile("s_nop 1"
               : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]),
                 "+v"(v[6]), "+v"(v[7]));
}
template <typename T>
__device__ __forceinline__ void settle44(T (&a)[4], T (&b)[4]) {
  asm volatile("s_nop 1"
               : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(b[0]), "+v"(b[1]),
                 "+v"(b[2]), "+v"(b[3]));
}

// Wait states around runs of the inline-asm DPP dots, tied to the values
// they accumulate: a dot product's result reaches a different instruction
// only three wait states later (a following dot of the same kind reading it
// as its accumulator is forwarded), and a DPP instruction reads no VGPR a
// VALU instruction wrote in the two wait states before. The compiler pads
// neither around inline asm. N = s_nop operand (N + 1 wait states).
template <int N, int R>
__device__ __forceinline__ void settle_rows(float (&z)[R]) {
  if constexpr (R == 1) {
    asm volatile("s_nop %1" : "+v"(z[0]) : "n"(N));
  } else if constexpr (R == 2) {
    asm volatile("s_nop %2" : "+v"(z[0]), "+v"(z[1]) : "n"(N));
  } else if constexpr (R == 4) {
    asm volatile("s_nop %4" : "+v"(z[0]), "+v"(z[1]), "+v"(z[2]), "+v"(z[3]) : "n"(N));
  } else {
    asm volatile("s_nop %8"
                 : "+v"(z[0]), "+v"(z[1]), "+v"(z[2]), "+v"(z[3]), "+v"(z[4]), "+v"(z[5]),
                   "+v"(z[6]), "+v"(z[7])
                 : "n"(N));
  }
}
template <int N, int G>
__device__ __forceinline__ void settle_acc(float (&acc)[G][2]) {
  // the accumulators themselves are the operands (a copy through another
  // array made the register allocator move them on every block)
  if constexpr (G == 1) {
    asm volatile("s_nop %2" : "+v"(acc[0][0]), "+v"(acc[0][1]) : "n"(N));
  } else if constexpr (G == 2) {
    asm volatile("s_nop %4"
                 : "+v"(acc[0][0]), "+v"(acc[0][1]), "+v"(acc[1][0]), "+v"(acc[1][1])
                 : "n"(N));
  } else if constexpr (G == 4) {
    asm volatile("s_nop %8"
                 : "+v"(acc[0][0]), "+v"(acc[0][1]), "+v"(acc[1][0]), "+v"(acc[1][1]),
                   "+v"(acc[2][0]), "+v"(acc[2][1]), "+v"(acc[3][0]), "+v"(acc[3][1])
                 : "n"(N));
  } else {
    static_assert(G == 8, "G in {1, 2, 4, 8}");
    asm volatile("s_nop %16"
                 : "+v"(acc[0][0]), "+v"(acc[0][1]), "+v"(acc[1][0]), "+v"(acc[1][1]),
                   "+v"(acc[2][0]), "+v"(acc[2][1]), "+v"(acc[3][0]), "+v"(acc[3][1]),
                   "+v"(acc[4][0]), "+v"(acc[4][1]), "+v"(acc[5][0]), "+v"(acc[5][1]),
                   "+v"(acc[6][0]), "+v"(acc[6][1]), "+v"(acc[7][0]), "+v"(acc[7][1])
                 : "n"(N));
  }
}

// One step of a full-wave reduction for every row: x[r] = op(x[r], x[r] of
// the lane the DPP control names), fused as v_max_f32_dpp / v_add_f32_dpp
// (the compiler would emit a mov_dpp, for the maximum a canonicalising max,
// and the operation). Rows are interleaved, so a step's source was written
// G instructions before; for G < 3 the caller pads.
#define PDA_DPP_STEP(OP, CTRL) \
  asm volatile(OP " %0, %0, %0 " CTRL " bank_mask:0xf" : "+v"(x[r]))
template <bool ADD, int C, int G>
__device__ __forceinline__ void reduce_step(float (&x)[G]) {
#pragma unroll
  for (int r = 0; r < G; ++r) {
    if constexpr (ADD) {
      if constexpr (C == 0) PDA_DPP_STEP("v_add_f32_dpp", "quad_perm:[1,0,3,2] row_mask:0xf");
      else if constexpr (C == 1) PDA_DPP_STEP("v_add_f32_dpp", "quad_perm:[2,3,0,1] row_mask:0xf");
      else if constexpr (C == 2) PDA_DPP_STEP("v_add_f32_dpp", "row_half_mirror row_mask:0xf");
      else if constexpr (C == 3) PDA_DPP_STEP("v_add_f32_dpp", "row_mirror row_mask:0xf");
      else if constexpr (C == 4) PDA_DPP_STEP("v_add_f32_dpp", "row_bcast:15 row_mask:0xa");
      else PDA_DPP_STEP("v_add_f32_dpp", "row_bcast:31 row_mask:0xc");
    } else {
      if constexpr (C == 0) PDA_DPP_STEP("v_max_f32_dpp", "quad_perm:[1,0,3,2] row_mask:0xf");
      else if constexpr (C == 1) PDA_DPP_STEP("v_max_f32_dpp", "quad_perm:[2,3,0,1] row_mask:0xf");
      else if constexpr (C == 2) PDA_DPP_STEP("v_max_f32_dpp", "row_half_mirror row_mask:0xf");
      else if constexpr (C == 3) PDA_DPP_STEP("v_max_f32_dpp", "row_mirror row_mask:0xf");
      else if constexpr (C == 4) PDA_DPP_STEP("v_max_f32_dpp", "row_bcast:15 row_mask:0xa");
      else PDA_DPP_STEP("v_max_f32_dpp", "row_bcast:31 row_mask:0xc");
    }
  }
}
#undef PDA_DPP_STEP

// Full-wave maxima (ADD = false) or sums (ADD = true) of G rows at once, as
// wave-uniform values: after the six steps lane 63 holds each row's result
// (the row broadcasts only write the rows their masks name; the others keep
// their values), pairing lanes in the same order as the one-row reductions.
// Wait states: two before the first DPP read of values the compiler just
// wrote, two between steps when fewer than three rows separate a write from
// its DPP read, and two before the lane reads, since the compiler pads
// nothing around inline asm. A maximum ignores NaN inputs unless a whole row
// is NaN (IEEE maximum).
template <bool ADD, int G>
__device__ __forceinline__ void wave_reduce_rows(float (&x)[G], float (&out)[G]) {
  settle_rows<1>(x);
  static_for<0, 6>::run([&](auto C) {
    if constexpr (decltype(C)::value > 0 && G < 3) settle_rows<1>(x);
    reduce_step<ADD, decltype(C)::value>(x);
  });
  settle_rows<1>(x);
#pragma unroll
  for (int r = 0; r < G; ++r) out[r] = as_f32(__builtin_amdgcn_readlane((int)as_u32(x[r]), 63));
}

// acc + dot(q, k) over one bf16 pair, where q is taken from lane L of the
// lane's 16-lane row (DPP row_newbcast). Written as inline asm because the
// compiler does not fold the broadcast into v_dot2c. The q register is only
// ever written by an LDS read (never by a VALU instruction just before a
// DPP read of it), so no wait states are needed.
template <int L>
__device__ __forceinline__ float dot2_bcast(float acc, uint32_t q, bf16x2_t k) {
  asm("v_dot2c_f32_bf16_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
      : "+v"(acc)
      : "v"(q), "v"(k), "n"(L));
  return acc;
}

// Bytes of the per-wave p buffer in LDS: G rows x 64 tokens of f16 (FP8
// caches), or of a bf16 high part plus a bf16 remainder (BF16 caches).
template <int G, bool FP8>
constexpr int pbuf_bytes() {
  return G * 64 * 2 * (FP8 ? 1 : 2);
}

// Physical page ids of the (up to four) pages one 64-token block spans, as
// separate scalars (an indexed array here ends up in scratch memory).
struct Pages {
  int p0, p1, p2, p3;
  __device__ __forceinline__ int get(int k) const {
    return k == 0 ? p0 : k == 1 ? p1 : k == 2 ? p2 : p3;
  }
  __device__ __forceinline__ void set(int k, int v) {
    if (k == 0) p0 = v; else if (k == 1) p1 = v; else if (k == 2) p2 = v; else p3 = v;
  }
};

template <int G, bool FP8, int S>
struct Item {
  static constexpr int E = FP8 ? 1 : 2;        // bytes per cache element
  static constexpr int NP = 64 / S;            // pages per 64-token block
  static constexpr int KQ = 8 * E;             // 16-byte K vectors per lane per block
  static constexpr int VW = E;                 // dwords of V per lane per token pair
  using vword_t = typename std::conditional<FP8, uint32_t, uint2>::type;
};

// K of the lane's token (lane = token b0 + lane) for one 64-token block:
// the token's 128 dims as eight 16-dim column groups.
template <int G, bool FP8, int S>
__device__ __forceinline__ void load_k(const AttnArgs& a, int g, const Pages& pg,
                                       uint4 (&kk)[Item<G, FP8, S>::KQ]) {
  using I = Item<G, FP8, S>;
  const int lane = __lane_id();
  // page of the lane's token, from wave-uniform ids with arithmetic only
  int page = pg.p0;
  if constexpr (I::NP >= 2) page += (lane >= S) * (pg.p1 - pg.p0);
  if constexpr (I::NP >= 4) page += (lane >= 2 * S) * (pg.p2 - pg.p1) + (lane >= 3 * S) * (pg.p3 - pg.p2);
  const int off = lane % S;
  // element (page, g, off, 16c + i) at (((page*Hkv + g)*8 + c)*S + off)*16 + i
  const uint8_t* base = a.kc + ((((int64_t)page * a.Hkv + g) * 8) * S + off) * 16 * I::E;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    if constexpr (FP8) {
      kk[c] = *reinterpret_cast<const uint4*>(base + (int64_t)c * S * 16);
    } else {
      kk[2 * c] = *reinterpret_cast<const uint4*>(base + (int64_t)c * S * 32);
      kk[2 * c + 1] = *reinterpret_cast<const uint4*>(base + (int64_t)c * S * 32 + 16);
    }
  }
}

// FP8 keys of one 64-token block straight into the wave's LDS buffer
// (global_load_lds_dwordx4: lane i's 16 bytes land at the wave-uniform LDS
// address + 16 i), laid out [column group c][token][16 codes]: one 1 KB copy
// per column group, and a token's 16 codes at kw + c*1024 + 16*token, so the
// QK reads (lane = token) are conflict-free. No registers hold keys in flight.
// Source of the lane's token (column group 0) for a block's key copy.
template <int S>
__device__ __forceinline__ const uint8_t* k_src(const AttnArgs& a, int g, const Pages& pg) {
  const int lane = __lane_id();
  int page = pg.p0;
  if constexpr (S <= 32) page += (lane >= S) * (pg.p1 - pg.p0);
  if constexpr (S == 16) page += (lane >= 2 * S) * (pg.p2 - pg.p1) + (lane >= 3 * S) * (pg.p3 - pg.p2);
  const int off = lane % S;
  return a.kc + ((((int64_t)page * a.Hkv + g) * 8) * S + off) * 16;
}

// Copy of column group c of a block's keys into the wave's buffer. Issued
// as inline asm so that the compiler's wait-count bookkeeping does not treat
// every later LDS read as dependent on it (it would wait for all
// vector-memory operations, including the next block's V loads); the one
// reader, the QK of the next block, waits for it explicitly. (s_nop 0: one
// wait state between a scalar write of M0 and the load that uses it, which
// the compiler pads in its own code but not inside inline asm.)
template <int S>
__device__ __forceinline__ void dma_k_group(const uint8_t* src, uint8_t* kw, int c) {
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t*)kw));
  const uint8_t* gp = src + (int64_t)c * S * 16;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(lds0 + c * 1024), "v"(gp) : "memory");
}

template <int S>
__device__ __forceinline__ void dma_k(const AttnArgs& a, int g, const Pages& pg, uint8_t* kw) {
  const uint8_t* src = k_src<S>(a, g, pg);
#pragma unroll
  for (int c = 0; c < 8; ++c) dma_k_group<S>(src, kw, c);
}

// V of one 64-token block for the lane's two dims (2*lane, 2*lane+1): one
// word per token pair. In the V format the pair row (page, g, off/2) holds
// (dim d, token off) at element 2*d + off%2, so dims 2l and 2l+1 of both
// tokens are the four consecutive elements 4l..4l+3.
template <int G, bool FP8, int S>
__device__ __forceinline__ void load_v(const AttnArgs& a, int g, const Pages& pg,
                                       typename Item<G, FP8, S>::vword_t (&vv)[32]) {
  using I = Item<G, FP8, S>;
  using W = typename I::vword_t;
  const int lane = __lane_id();
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int page = pg.get((2 * i) / S);
    const int pr = ((2 * i) % S) / 2;
    const uint8_t* row = a.vc + (((int64_t)page * a.Hkv + g) * (S / 2) + pr) * (kD * 2) * I::E;
    vv[i] = *reinterpret_cast<const W*>(row + lane * 4 * I::E);
  }
}

// PV of one 64-token block for the lane's two dims: acc[r][0..1] +=
// sum over token pairs of (p pair of row r) . (V pair of dim 2l / 2l+1).
// Step k = (ic, r) takes row r's four p pairs of token pairs 4ic..4ic+3 in
// one 16-byte LDS read (a wave-uniform address, so a broadcast). Reads run
// kPD steps ahead of their use.
constexpr int kPD = 2;

__device__ __forceinline__ uint32_t word0(uint32_t w) { return w; }
__device__ __forceinline__ uint32_t word0(uint2 w) { return w.x; }

// Mask keeping the elements of tokens (2i, 2i+1) that are below `valid`, for
// a word holding one 16-bit value of each token (low half: token 2i).
__device__ __forceinline__ uint32_t pair_mask(int i, int valid) {
  return (2 * i < valid ? 0x0000FFFFu : 0u) | (2 * i + 1 < valid ? 0xFFFF0000u : 0u);
}

// The same for a word of four e4m3 codes (dim 2l: tokens 2i, 2i+1, then
// dim 2l+1: tokens 2i, 2i+1).
__device__ __forceinline__ uint32_t code_pair_mask(int i, int valid) {
  return (2 * i < valid ? 0x00FF00FFu : 0u) | (2 * i + 1 < valid ? 0xFF00FF00u : 0u);
}

// acc + dot(p, v) over one f16 pair, p taken from lane L of the lane's
// 16-lane row (DPP row_newbcast); inline asm for the same reason as
// dot2_bcast, and p registers likewise only come from LDS reads.
template <int L>
__device__ __forceinline__ float dot2_bcast_f16(float acc, uint32_t p, f16x2_t v) {
  asm("v_dot2c_f32_f16_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
      : "+v"(acc)
      : "v"(p), "v"(v), "n"(L));
  return acc;
}

// FP8 PV of one 64-token block for the lane's two dims. The softmax left p
// in the wave's LDS buffer as [8-token group ic][row r][8 tokens] (f16), so
// group ic's 4G dwords are contiguous: lane l of every 16-lane row reads
// dwords 2(l % 2G), +1 of the group (one 8-byte read per group, one group
// ahead), and the p pair (row r, token pair jj) is register jj % 2 of lane
// 2r + jj/2, handed to the dot by a DPP row broadcast.
template <int G, bool TAIL>
__device__ __forceinline__ void pv_block_fp8(const uint32_t (&vv)[32], const uint16_t* pw,
                                             float (&acc)[G][2], int valid) {
  const int lane = __lane_id();
  auto rdp = [&](int ic) -> uint2 {
    return *reinterpret_cast<const uint2*>(pw + ic * (8 * G) + (lane % (2 * G)) * 4);
  };
  uint2 pa = rdp(0), pb = pa;
  settle_acc<1, G>(acc);
  static_for<0, 8>::run([&](auto IC) {
    constexpr int ic = decltype(IC)::value;
    const uint2 pc = (ic % 2 == 0) ? pa : pb;
    if constexpr (ic + 1 < 8) {
      if constexpr (ic % 2 == 0) pb = rdp(ic + 1); else pa = rdp(ic + 1);
    }
    f16x2_t v0[4], v1[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t w = vv[4 * ic + j];
      // bytes: (dim 2l, token 2i), (2l, 2i+1), (2l+1, 2i), (2l+1, 2i+1)
      if constexpr (TAIL) w &= code_pair_mask(4 * ic + j, valid);
      v0[j] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
      v1[j] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
    }
    settle44(v0, v1);
    static_for<0, 4 * G>::run([&](auto D) {
      constexpr int d = decltype(D)::value;   // row d/4, token pair d%4 of the group
      constexpr int r = d / 4, jj = d % 4;
      const uint32_t pr = (jj % 2 == 0) ? pc.x : pc.y;
      acc[r][0] = dot2_bcast_f16<2 * r + jj / 2>(acc[r][0], pr, v0[jj]);
      acc[r][1] = dot2_bcast_f16<2 * r + jj / 2>(acc[r][1], pr, v1[jj]);
    });
    // keep the schedule in program order (see pv_block)
    __builtin_amdgcn_sched_barrier(0);
  });
  settle_acc<2, G>(acc);
}

template <int G, bool FP8, bool TAIL>
__device__ __forceinline__ void pv_block(
    const typename std::conditional<FP8, uint32_t, uint2>::type (&vv)[32], const uint16_t* pw,
    float (&acc)[G][2], int valid) {
  constexpr int NK = 8 * G;
  constexpr int D = NK < kPD ? NK : kPD;
  auto rd = [&](int k, int part) -> uint4 {
    const int ic = k / G, r = k % G;
    return *reinterpret_cast<const uint4*>(pw + part * G * 64 + r * 64 + ic * 8);
  };
  uint4 ph[D], pl[D];
#pragma unroll
  for (int k = 0; k < D; ++k) {
    ph[k] = rd(k, 0);
    if constexpr (!FP8) pl[k] = rd(k, 1);
  }
  f16x2_t v0[4], v1[4];
  static_for<0, NK>::run([&](auto K) {
    constexpr int k = decltype(K)::value;
    constexpr int ic = k / G, r = k % G;
    if constexpr (FP8 && r == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t w = word0(vv[4 * ic + j]);
        // bytes: (dim 2l, token 2i), (2l, 2i+1), (2l+1, 2i), (2l+1, 2i+1)
        if constexpr (TAIL) w &= code_pair_mask(4 * ic + j, valid);
        v0[j] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
        v1[j] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
      }
    }
    const uint4 ch = ph[k % D];
    uint4 cl = ch;
    if constexpr (!FP8) cl = pl[k % D];
    if constexpr (k + D < NK) {
      ph[k % D] = rd(k + D, 0);
      if constexpr (!FP8) pl[k % D] = rd(k + D, 1);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (FP8) {
        const f16x2_t p2 = __builtin_bit_cast(f16x2_t, u4_get(ch, j));
        acc[r][0] = __builtin_amdgcn_fdot2(p2, v0[j], acc[r][0], false);
        acc[r][1] = __builtin_amdgcn_fdot2(p2, v1[j], acc[r][1], false);
      } else {
        const bf16x2_t hi = __builtin_bit_cast(bf16x2_t, u4_get(ch, j));
        const bf16x2_t lo = __builtin_bit_cast(bf16x2_t, u4_get(cl, j));
        uint32_t wa = vv[4 * ic + j].x, wb = vv[4 * ic + j].y;
        if constexpr (TAIL) {
          const uint32_t msk = pair_mask(4 * ic + j, valid);
          wa &= msk;
          wb &= msk;
        }
        const bf16x2_t va = __builtin_bit_cast(bf16x2_t, wa);
        const bf16x2_t vb = __builtin_bit_cast(bf16x2_t, wb);
        acc[r][0] = __builtin_amdgcn_fdot2_f32_bf16(hi, va, acc[r][0], false);
        acc[r][0] = __builtin_amdgcn_fdot2_f32_bf16(lo, va, acc[r][0], false);
        acc[r][1] = __builtin_amdgcn_fdot2_f32_bf16(hi, vb, acc[r][1], false);
        acc[r][1] = __builtin_amdgcn_fdot2_f32_bf16(lo, vb, acc[r][1], false);
      }
    }
    // keep the schedule in program order: otherwise every conversion and
    // LDS read of the block is hoisted to the top, a register each
    __builtin_amdgcn_sched_barrier(0);
  });
}

template <int G, bool FP8, int S, typename QStore>
__device__ void process_item(const AttnArgs& a, int s, int c, int g, int chunk, uint16_t* pw,
                             uint8_t* kw, const uint32_t* qs, float* mg, bool active,
                             QStore&& q_store) {
  // q_store (the unit's q rows into LDS, then a workgroup barrier) runs in
  // every wave, after an active wave has issued its first block's loads, so
  // that their latency and the q loads' overlap.
  if (!active) {
    q_store();
    return;
  }
  using I = Item<G, FP8, S>;
  using W = typename I::vword_t;
  constexpr int NP = I::NP;
  const int lane = __lane_id();
  const int len = a.lens[s];
  const int tok0 = c * chunk;
  const int tok1 = min(len, tok0 + chunk);
  ci32_t* btrow = (ci32_t*)(uintptr_t)(a.bt + (int64_t)s * a.max_blocks);
  cu32_t* qbase = (cu32_t*)(uintptr_t)(a.q + ((int64_t)s * a.Hq + (int64_t)g * G) * kD);
  const float kmul = a.sm_scale * (FP8 ? a.k_scale[g] : 1.0f) * kLog2e;

  float m[G], l[G], acc[G][2];
#pragma unroll
  for (int r = 0; r < G; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.0f;
    acc[r][0] = acc[r][1] = 0.0f;
  }
  bool bad = false;

  // Physical pages of the block starting at b0 (wave-uniform), in two steps:
  // raw_pages issues the block-table loads (one scalar load of the NP
  // consecutive entries when the whole block lies inside the chunk) a block
  // ahead of their use; fix_pages checks them when the block comes up. Pages
  // past the end of the chunk are replaced by the chunk's first page, a page
  // of this sequence; their tokens are masked out below. A page id outside
  // [0, P) is never dereferenced: it marks the item bad.
  int fb = btrow[tok0 / S];
  if (fb < 0 || fb >= a.P) {
    bad = true;
    fb = 0;
  }
  auto raw_pages = [&](int b0, Pages& r) {
    r.p0 = r.p1 = r.p2 = r.p3 = fb;
    if (b0 + 64 <= tok1) {
      if constexpr (NP == 4) {
        typedef int32_t i32x4 __attribute__((ext_vector_type(4), aligned(4)));
        const i32x4 v = *(const __attribute__((address_space(4))) i32x4*)(btrow + b0 / S);
        r.p0 = v.x; r.p1 = v.y; r.p2 = v.z; r.p3 = v.w;
      } else if constexpr (NP == 2) {
        typedef int32_t i32x2 __attribute__((ext_vector_type(2), aligned(4)));
        const i32x2 v = *(const __attribute__((address_space(4))) i32x2*)(btrow + b0 / S);
        r.p0 = v.x; r.p1 = v.y;
      } else {
        r.p0 = btrow[b0 / S];
      }
    } else {
#pragma unroll
      for (int k = 0; k < NP; ++k)
        if (b0 + k * S < tok1) r.set(k, btrow[(b0 + k * S) / S]);
    }
  };
  auto fix_pages = [&](int b0, const Pages& r, Pages& pg) {
    pg.p1 = pg.p2 = pg.p3 = fb;
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      int p = fb;
      if (b0 + k * S < tok1) {
        p = r.get(k);
        if (p < 0 || p >= a.P) {
          bad = true;
          p = fb;
        }
      }
      pg.set(k, p);
    }
  };

  // FP8 keys go through the wave's LDS buffer; BF16 keys through registers
  uint4 kk[FP8 ? 1 : I::KQ];
  W vv[32];
  Pages pg, raw;
  int b0 = tok0;
  raw_pages(b0, raw);
  fix_pages(b0, raw, pg);
  if (b0 + 64 < tok1) raw_pages(b0 + 64, raw);
  if constexpr (FP8)
    dma_k<S>(a, g, pg, kw);
  else
    load_k<G, FP8, S>(a, g, pg, kk);
  load_v<G, FP8, S>(a, g, pg, vv);
  q_store();

  for (;;) {
    const int bn = b0 + 64;
    const bool has_next = bn < tok1;
    const bool tail = b0 + 64 > tok1;
    Pages npg = pg;
    if (has_next) {
      fix_pages(bn, raw, npg);
      if (bn + 64 < tok1) raw_pages(bn + 64, raw);
    }

    // ---- QK: lane = token b0 + lane ------------------------------------
    float z[G];
#pragma unroll
    for (int r = 0; r < G; ++r) z[r] = 0.0f;
    if constexpr (FP8) {
      // Keys from the wave's LDS buffer, 16 dims (one 16-byte read) at a
      // time, read one column group ahead. The key copy of this block (the
      // oldest vector-memory operations in flight; the 32 V loads of this
      // block came before it and the next block's V loads are not issued
      // yet) must have landed.
      __builtin_amdgcn_s_waitcnt(0x8F70);   // vmcnt(32): all but the 32 V loads
      // q of one column group (G rows x 8 dwords) sits in the unit's LDS
      // rows; lane l of every 16-lane row reads dwords 4(l % 2G) .. +3, so
      // dword d of the group is register d % 4 of lane d / 4 in each row,
      // and a DPP row broadcast hands it to all lanes as the dot operand.
      constexpr int QL = 2 * G;   // lanes holding one column group's q
      auto readq = [&](int c16) -> uint4 {
        return *reinterpret_cast<const uint4*>(qs + c16 * (8 * G) + (lane % QL) * 4);
      };
      auto readk = [&](int c16) -> uint4 {
        return *reinterpret_cast<const uint4*>(kw + c16 * 1024 + lane * 16);
      };
      uint4 kcur = readk(0), knext = kcur;
      uint4 qcur = readq(0), qnext = qcur;
      bf16x2_t kp[8];
      // the next block's key copy goes out group by group, each group as
      // soon as its keys here have been read and used
      const uint8_t* ksrc = has_next ? k_src<S>(a, g, npg) : nullptr;
      settle_rows<1>(z);
      static_for<0, 8>::run([&](auto C) {
        constexpr int c16 = decltype(C)::value;
        const uint4 w = (c16 % 2 == 0) ? kcur : knext;
        const uint4 qv = (c16 % 2 == 0) ? qcur : qnext;
        if constexpr (c16 + 1 < 8) {
          if constexpr (c16 % 2 == 0) {
            knext = readk(c16 + 1);
            qnext = readq(c16 + 1);
          } else {
            kcur = readk(c16 + 1);
            qcur = readq(c16 + 1);
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          kp[2 * j] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u4_get(w, j), 1.0f, false);
          kp[2 * j + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u4_get(w, j), 1.0f, true);
        }
        settle8(kp);
        static_for<0, 8 * G>::run([&](auto D) {
          constexpr int d = decltype(D)::value;   // dword of the group: row d/8, dims pair d%8
          z[d / 8] = dot2_bcast<d / 4>(z[d / 8], u4_get(qv, d % 4), kp[d % 8]);
        });
        __builtin_amdgcn_sched_barrier(0);
        // group c16's keys are in registers (converted above): its part of
        // the buffer is free
        if (has_next) dma_k_group<S>(ksrc, kw, c16);
      });
      settle_rows<2>(z);
    } else {
    // Eight dims (four q pairs per row) at a time, q in SGPRs. The loads of
    // chunk c+2 are released by a fence that consumes the scores produced by
    // chunk c, so exactly two 4-pair chunks of q are live at any time.
    {
      uint32_t qbuf[2][G][2];
      auto loadq = [&](int c4, uint32_t(&dst)[G][2]) {
        cu32_t* qp = fence_ptr_after<G>(qbase, z);
#pragma unroll
        for (int r = 0; r < G; ++r)
#pragma unroll
          for (int j = 0; j < 2; ++j) dst[r][j] = qp[r * 64 + c4 * 2 + j];
      };
      loadq(0, qbuf[0]);
      loadq(1, qbuf[1]);
      bf16x2_t kp[4];
      static_for<0, 32>::run([&](auto CC) {
        constexpr int c4 = decltype(CC)::value;   // dims 4*c4 .. 4*c4+3
        if constexpr ((c4 & 1) == 0) {
          constexpr int c8 = c4 >> 1;             // dims 8*c8 .. 8*c8+7
          if constexpr (FP8) {
            const uint32_t w0 = u4_get(kk[c8 >> 1], (c8 & 1) * 2);
            const uint32_t w1 = u4_get(kk[c8 >> 1], (c8 & 1) * 2 + 1);
            kp[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
            kp[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
            kp[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
            kp[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) kp[j] = __builtin_bit_cast(bf16x2_t, u4_get(kk[c8], j));
          }
        }
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < G; ++r)
            z[r] = __builtin_amdgcn_fdot2_f32_bf16(
                __builtin_bit_cast(bf16x2_t, qbuf[c4 & 1][r][j]), kp[(c4 & 1) * 2 + j], z[r],
                false);
        if constexpr (c4 + 2 < 32) loadq(c4 + 2, qbuf[c4 & 1]);
        if constexpr ((c4 & 1) == 1) __builtin_amdgcn_sched_barrier(0);
      });
    }
    // K registers are free: prefetch the next block's keys.
    if (has_next) load_k<G, FP8, S>(a, g, npg, kk);
    }


    // ---- online softmax (log2 units) -----------------------------------
    // zl = z*kmul - m. The running max m only moves when some score of the
    // block exceeds it by more than kTau, so p = 2^zl <= 2^kTau and the
    // exact block maximum (a wave reduction) is only taken in that case. On
    // the item's first block (m = -inf, l = acc = 0) every row's maximum is
    // taken up front, all rows in one interleaved reduction, so no row
    // takes the one-row path there.
    // The tail block (tokens at or past tok1 among its 64) takes a copy of
    // the softmax that masks them; full blocks carry no masks.
    // Per-row factor of the accumulators for this block (1 unless the
    // running max moved). It is applied to every row of every block,
    // outside the rare branch that computes it: multiplying there made the
    // compiler keep the accumulators in two sets of registers and copy them
    // on every block.
    float alpha[G];
    auto softmax = [&](auto TAILC) {
      constexpr bool TAIL = decltype(TAILC)::value;
      const bool tok_ok = !TAIL || (b0 + lane) < tok1;
      if (b0 == tok0) {
        float t[G], bm[G];
#pragma unroll
        for (int r = 0; r < G; ++r) t[r] = (TAIL && !tok_ok) ? -INFINITY : z[r] * kmul;
        wave_reduce_rows<false, G>(t, bm);
#pragma unroll
        for (int r = 0; r < G; ++r) m[r] = bm[r];
      }
      float zl[G];
      uint64_t over = 0;
#pragma unroll
      for (int r = 0; r < G; ++r) alpha[r] = 1.0f;
#pragma unroll
      for (int r = 0; r < G; ++r) {
        zl[r] = fmaf(z[r], kmul, -m[r]);
        if (TAIL && !tok_ok) zl[r] = -INFINITY;
        over |= __ballot(zl[r] > kTau);
      }
      if (over != 0) {
#pragma unroll
        for (int r = 0; r < G; ++r) {
          if (__ballot(zl[r] > kTau) != 0) {
            const float bm = wave_max((TAIL && !tok_ok) ? -INFINITY : z[r] * kmul);
            alpha[r] = as_f32(__builtin_amdgcn_readfirstlane(
                (int)as_u32(__builtin_amdgcn_exp2f(m[r] - bm))));
            m[r] = bm;
            l[r] *= alpha[r];
            zl[r] = (TAIL && !tok_ok) ? -INFINITY : fmaf(z[r], kmul, -bm);
          }
        }
      }
      // p of this lane's token for every row, to the wave's LDS buffer: FP8
      // as [t/8][r][t%8] (f16, the order pv_block_fp8 reads), BF16 as
      // pw[r*64 + t] with hi/lo bf16 parts at pw and pw + G*64.
#pragma unroll
      for (int r = 0; r < G; ++r) {
        const float p = __builtin_amdgcn_exp2f(zl[r]);
        l[r] += p;
        if constexpr (FP8) {
          pw[(lane / 8) * (8 * G) + r * 8 + (lane % 8)] = __builtin_bit_cast(uint16_t, (_Float16)p);
        } else {
          const uint32_t pu = as_u32(p);
          const float rem = p - as_f32(pu & 0xFFFF0000u);
          pw[r * 64 + lane] = (uint16_t)(pu >> 16);
          pw[G * 64 + r * 64 + lane] = (uint16_t)(as_u32(rem) >> 16);
        }
      }
    };
    // The wave's own LDS writes of p must land before its reads in PV.
    auto lds_fence = [] {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    // ---- PV: lane = dims (2*lane, 2*lane+1), all 64 tokens ---------------
    // In the tail block, tokens at or beyond tok1 have p = 0 but their V
    // codes may be stale or poisoned (NaN * 0 = NaN). FP8: their bytes of
    // the V words are zeroed first (in place), so one copy of PV serves
    // every block (a second, masking copy made the compiler keep the
    // accumulators in two sets of registers and copy them twice per block).
    // BF16: the values are zeroed inside a separate copy of the loop (the
    // register budget of two waves per SIMD holds it there).
    if constexpr (FP8) {
      if (tail) {
        softmax(std::true_type{});
        const int valid = tok1 - b0;
#pragma unroll
        for (int i = 0; i < 32; ++i)
          asm volatile("v_and_b32 %0, %0, %1" : "+v"(vv[i]) : "v"(code_pair_mask(i, valid)));
      } else {
        softmax(std::false_type{});
      }
#pragma unroll
      for (int r = 0; r < G; ++r) {
        acc[r][0] *= alpha[r];
        acc[r][1] *= alpha[r];
      }
      lds_fence();
      pv_block_fp8<G, false>(vv, pw, acc, 64);
    } else {
      if (tail)
        softmax(std::true_type{});
      else
        softmax(std::false_type{});
#pragma unroll
      for (int r = 0; r < G; ++r) {
        acc[r][0] *= alpha[r];
        acc[r][1] *= alpha[r];
      }
      lds_fence();
      if (tail) {
        asm volatile("" ::: "memory");
        pv_block<G, FP8, true>(vv, pw, acc, tok1 - b0);
      } else {
        asm volatile("" ::: "memory");
        pv_block<G, FP8, false>(vv, pw, acc, 64);
      }
    }
    if (!has_next) break;
    load_v<G, FP8, S>(a, g, npg, vv);
    pg = npg;
    b0 = bn;
    // the next block's p writes must not pass this block's p reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // ---- the partial, to the wave's merge slot in LDS ----------------------
  // [G rows x 128 dims][G maxima][G sums]; a bad item's maxima are NaN.
  // (For FP8 the slot is the key buffer, whose last copy was waited for
  // before the last QK.)
  float lt[G];
  wave_reduce_rows<true, G>(l, lt);   // l is not used after this
#pragma unroll
  for (int r = 0; r < G; ++r) {
    *reinterpret_cast<float2*>(mg + r * kD + 2 * lane) = make_float2(acc[r][0], acc[r][1]);
    if (lane == r) {
      mg[G * kD + r] = bad ? __builtin_nanf("") : m[r];
      mg[G * kD + G + r] = lt[r];
    }
  }
}

// Bytes of one partial, G rows x (128 dims + max + sum) fp32, rounded up to
// 16 so that every LDS merge slot is aligned for 16-byte reads.
template <int G>
constexpr int partial_bytes() {
  return (G * (kD + 2) * 4 + 15) / 16 * 16;
}

// Merge the partials the waves of a unit left in their LDS slots (nv of
// them, in chunk order) into one partial in the workspace: the log-sum-exp
// rule, M = max m_w, L = sum 2^(m_w - M) l_w, acc = sum 2^(m_w - M) acc_w. A
// NaN maximum (a bad item) makes the merged maximum NaN.
template <int G>
__device__ void merge_unit(const float* mg0, int slot_stride, int nv, float* part) {
  const int r = threadIdx.x >> 5;
  const int d4 = (threadIdx.x & 31) * 4;
  if (r >= G) return;
  float mw[kWaves];
  float M = -INFINITY;
  bool nan = false;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    mw[w] = w < nv ? mg0[w * slot_stride + G * kD + r] : -INFINITY;
    nan |= __builtin_isnan(mw[w]);
    M = fmaxf(M, mw[w]);
  }
  float L = 0.0f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    if (w < nv) {
      const float* pw = mg0 + w * slot_stride;
      const float e = __builtin_amdgcn_exp2f(mw[w] - M);
      const float4 v = *reinterpret_cast<const float4*>(pw + r * kD + d4);
      L += e * pw[G * kD + G + r];
      acc.x += e * v.x;
      acc.y += e * v.y;
      acc.z += e * v.z;
      acc.w += e * v.w;
    }
  }
  *reinterpret_cast<float4*>(part + r * kD + d4) = acc;
  if (d4 == 0) {
    part[G * kD + r] = nan ? __builtin_nanf("") : M;
    part[G * kD + G + r] = L;
  }
}

// Waves per SIMD the register allocator must leave room for.
template <int G, bool FP8>
constexpr int partial_waves() {
  return FP8 ? 4 : 2;
}

template <int G, bool FP8, int S>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(partial_waves<G, FP8>(), partial_waves<G, FP8>())))
void attn_partial_kernel(AttnArgs a) {
  extern __shared__ __attribute__((aligned(16))) int lds[];
  constexpr int PB = pbuf_bytes<G, FP8>();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  constexpr int KB = FP8 ? 8192 : 0;   // per-wave key buffer (FP8)
  constexpr int QB = FP8 ? G * kD * 2 : 0;   // the unit's q rows (FP8)
  uint16_t* pw = reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(lds) + wave * PB);
  uint8_t* kw = reinterpret_cast<uint8_t*>(lds) + kWaves * PB + wave * KB;
  uint32_t* qs = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(lds) + kWaves * (PB + KB));
  // merge slots: the key buffers (FP8), else a region of their own
  constexpr int MB = FP8 ? 0 : kWaves * partial_bytes<G>();
  static_assert(!FP8 || partial_bytes<G>() <= KB, "a partial must fit a key buffer");
  float* mg0 = reinterpret_cast<float*>(FP8 ? reinterpret_cast<char*>(lds) + kWaves * PB
                                            : reinterpret_cast<char*>(lds) + kWaves * PB + QB);
  constexpr int MS = (FP8 ? KB : partial_bytes<G>()) / 4;   // slot stride, floats
  int* tmp = lds + (kWaves * (PB + KB) + QB + MB) / 4;   // kWaves (the plan's wave totals)
  int* pref = tmp + kWaves;           // B + 1
  int chunk;
  const int total_slots = build_plan(a, S, pref, tmp, chunk);
  // A work unit is kWaves consecutive chunk slots of one (sequence, kv
  // head): wave w takes chunk slot w, so the workgroup shares one group of
  // query rows, staged in LDS once per unit. Units run with the kv head
  // fastest, so workgroups dispatched together read neighbouring 2 KB
  // slices of the same pages (2 % faster on a 256-sequence mixed batch,
  // unchanged on 64 x 8k). The merged partial of unit j of (s, g) is stored at
  // (pref[s] / kWaves + j) * Hkv + g.
  const long long total_units = (long long)(total_slots / kWaves) * a.Hkv;
  for (long long u = blockIdx.x; u < total_units; u += gridDim.x) {
    // sequence owning unit u: last s with (pref[s] / kWaves) * Hkv <= u
    int lo = 0, hi = a.B;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if ((long long)(pref[mid] / kWaves) * a.Hkv <= u) lo = mid; else hi = mid;
    }
    const int s = __builtin_amdgcn_readfirstlane(lo);
    const int local = (int)(u - (long long)(pref[s] / kWaves) * a.Hkv);
    const int g = __builtin_amdgcn_readfirstlane(local % a.Hkv);
    const int j = local / a.Hkv;   // unit of (s, g)
    const int c = __builtin_amdgcn_readfirstlane(j * kWaves + wave);
    __syncthreads();   // the previous unit's reads of qs and the merge slots are done
    // q rows of (s, g) (FP8) into LDS as [column group c16][row r][8
    // dwords], so the 8G dwords one QK step of 16 dims needs are contiguous.
    // The loads are issued here, before the item's first loads; the stores
    // and the barrier come after those (in process_item).
    constexpr int QPT = FP8 ? (G * kD / 2 + kThreads - 1) / kThreads : 1;   // dwords per thread
    uint32_t qreg[QPT];
    const uint32_t* qg =
        reinterpret_cast<const uint32_t*>(a.q + ((int64_t)s * a.Hq + (int64_t)g * G) * kD);
    if constexpr (FP8) {
#pragma unroll
      for (int k = 0; k < QPT; ++k) {
        const int i = threadIdx.x + k * kThreads;
        if (i < G * kD / 2) qreg[k] = qg[i];
      }
    }
    auto q_store = [&]() {
      if constexpr (FP8) {
#pragma unroll
        for (int k = 0; k < QPT; ++k) {
          const int i = threadIdx.x + k * kThreads;
          const int r = i / (kD / 2), w = i % (kD / 2);   // row, dword of the row
          if (i < G * kD / 2) qs[((w / 8) * G + r) * 8 + (w % 8)] = qreg[k];
        }
        __syncthreads();
      }
    };
    const int nch = n_chunks_of(a, s, S, chunk);
    process_item<G, FP8, S>(a, s, c, g, chunk, pw, kw, qs, mg0 + wave * MS, c < nch, q_store);
    __syncthreads();
    float* part = a.ws_part + ((int64_t)(pref[s] / kWaves + j) * a.Hkv + g) * (G * (kD + 2));
    merge_unit<G>(mg0, MS, min(kWaves, nch - j * kWaves), part);
  }
}

// Merge the unit partials of one (sequence, kv head): G rows x 128 dims,
// four dims per thread.
template <int G, bool FP8>
__global__ __launch_bounds__(kThreads) void attn_combine_kernel(AttnArgs a, int S) {
  const int s = blockIdx.x / a.Hkv;
  const int g = blockIdx.x % a.Hkv;
  const int r = threadIdx.x >> 5;
  const int d4 = (threadIdx.x & 31) * 4;
  if (r >= G) return;
  float* o = a.out + (((int64_t)s * a.Hq + (int64_t)g * G + r) * kD + d4);
  const int len = a.lens[s];
  const bool aborted = a.verdict != nullptr && a.verdict[s] != 0;
  if (aborted || len == 0) {
    *reinterpret_cast<float4*>(o) = make_float4(0.f, 0.f, 0.f, 0.f);
    return;
  }
  const float qnan = __builtin_nanf("");
  if (len < 0 || len > a.max_blocks * S) {
    *reinterpret_cast<float4*>(o) = make_float4(qnan, qnan, qnan, qnan);
    return;
  }
  const int* pref = a.ws_hdr + kHdrInts;
  const int c0 = pref[s] / kWaves, c1 = pref[s + 1] / kWaves;
  const int64_t stride = G * (kD + 2);
  // Unit partials are read sixteen at a time, all of a batch's loads (max,
  // sum, four dims) issued together; batches merge into the running result
  // with the same log-sum-exp rule (one pass, chunk order, deterministic).
  constexpr int kB = 16;
  float M = -INFINITY, L = 0.0f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  bool nan = false;
  for (int c = c0; c < c1; c += kB) {
    float mc[kB], lc[kB];
    float4 v[kB];
#pragma unroll
    for (int i = 0; i < kB; ++i) {
      if (c + i < c1) {
        const float* pc = a.ws_part + ((int64_t)(c + i) * a.Hkv + g) * stride;
        mc[i] = pc[G * kD + r];
        lc[i] = pc[G * kD + G + r];
        v[i] = *reinterpret_cast<const float4*>(pc + r * kD + d4);
      } else {
        mc[i] = -INFINITY;
        lc[i] = 0.0f;
        v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    float Mb = M;
#pragma unroll
    for (int i = 0; i < kB; ++i) {
      nan |= __builtin_isnan(mc[i]);
      Mb = fmaxf(Mb, mc[i]);
    }
    if (Mb > M) {   // every unit holds a valid token, so Mb is finite here
      const float alpha = __builtin_amdgcn_exp2f(M - Mb);   // 0 while M = -inf
      L *= alpha;
      acc.x *= alpha;
      acc.y *= alpha;
      acc.z *= alpha;
      acc.w *= alpha;
      M = Mb;
    }
#pragma unroll
    for (int i = 0; i < kB; ++i) {
      const float w = __builtin_amdgcn_exp2f(mc[i] - M);
      L += w * lc[i];
      acc.x += w * v[i].x;
      acc.y += w * v[i].y;
      acc.z += w * v[i].z;
      acc.w += w * v[i].w;
    }
  }
  if (nan) {
    *reinterpret_cast<float4*>(o) = make_float4(qnan, qnan, qnan, qnan);
    return;
  }
  const float f = (FP8 ? a.v_scale[g] : 1.0f) / L;
  *reinterpret_cast<float4*>(o) = make_float4(acc.x * f, acc.y * f, acc.z * f, acc.w * f);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

int resolve_chunk(const pda_attn_shape& sh, int32_t max_seq_len) {
  const int align = sh.page_size > 64 ? sh.page_size : 64;
  if (sh.split_tokens > 0) return sh.split_tokens;
  // automatic: 512 tokens, halved while the grid would hold fewer than
  // 4096 items, never below one 64-token block / one page
  int chunk = 512 < align ? align : 512;
  const long long ml = max_seq_len > 0 ? max_seq_len : 1;
  while (chunk > align &&
         (long long)sh.num_seqs * sh.num_kv_heads * ((ml + chunk - 1) / chunk) < 4096)
    chunk /= 2;
  return chunk;
}

size_t header_bytes(int B) {
  const size_t h = (size_t)(kHdrInts + B + 1) * sizeof(int32_t);
  return (h + 255) & ~(size_t)255;
}

size_t item_bytes(const pda_attn_shape& sh) {
  const int G = sh.num_q_heads / sh.num_kv_heads;
  return (size_t)G * (sh.head_dim_v + 2) * sizeof(float);
}

// Shape checks shared by the workspace query and the call.
int check_shape(const pda_attn_shape* sh) {
  if (!sh) return PDA_ERR_INVALID_ARG;
  if (sh->num_seqs < 0 || sh->num_q_heads <= 0 || sh->num_kv_heads <= 0 ||
      sh->head_dim_qk <= 0 || sh->head_dim_v <= 0 || sh->page_size <= 0 ||
      sh->num_pages <= 0 || sh->max_blocks_per_seq <= 0)
    return PDA_ERR_INVALID_ARG;
  if (sh->num_q_heads % sh->num_kv_heads != 0) return PDA_ERR_INVALID_ARG;
  if (!(sh->sm_scale == sh->sm_scale)) return PDA_ERR_INVALID_ARG;
  if (sh->kv_dtype != PDA_KV_BF16 && sh->kv_dtype != PDA_KV_FP8_E4M3) return PDA_ERR_INVALID_ARG;
  if (sh->split_tokens < 0) return PDA_ERR_INVALID_ARG;
  const int align = sh->page_size > 64 ? sh->page_size : 64;
  if (sh->split_tokens > 0 && (sh->split_tokens % align != 0)) return PDA_ERR_INVALID_ARG;
  if ((long long)sh->max_blocks_per_seq * sh->page_size > (1LL << 30)) return PDA_ERR_UNSUPPORTED;
  if (sh->num_seqs > 16384) return PDA_ERR_UNSUPPORTED;
  return PDA_OK;
}

bool valu_supported(const pda_attn_shape& sh) {
  const int G = sh.num_q_heads / sh.num_kv_heads;
  if (sh.v_in_k) return false;
  if (sh.head_dim_qk != kD || sh.head_dim_v != kD) return false;
  if (!(G == 1 || G == 2 || G == 4 || G == 8)) return false;
  if (!(sh.page_size == 16 || sh.page_size == 32 || sh.page_size == 64)) return false;
  if (sh.kv_dtype == PDA_KV_FP8_E4M3) return sh.scale_mode == PDA_SCALE_PER_HEAD;
  return sh.scale_mode == PDA_SCALE_NONE;
}

typedef void (*kernel_t)(AttnArgs);
typedef void (*combine_t)(AttnArgs, int);

template <int G, bool FP8>
kernel_t pick_partial_s(int S) {
  switch (S) {
    case 16: return attn_partial_kernel<G, FP8, 16>;
    case 32: return attn_partial_kernel<G, FP8, 32>;
    default: return attn_partial_kernel<G, FP8, 64>;
  }
}
template <bool FP8>
kernel_t pick_partial(int G, int S) {
  switch (G) {
    case 1: return pick_partial_s<1, FP8>(S);
    case 2: return pick_partial_s<2, FP8>(S);
    case 4: return pick_partial_s<4, FP8>(S);
    default: return pick_partial_s<8, FP8>(S);
  }
}
template <bool FP8>
combine_t pick_combine(int G) {
  switch (G) {
    case 1: return attn_combine_kernel<1, FP8>;
    case 2: return attn_combine_kernel<2, FP8>;
    case 4: return attn_combine_kernel<4, FP8>;
    default: return attn_combine_kernel<8, FP8>;
  }
}

// Resident workgroups per CU for a partial kernel (cached per kernel).
int blocks_per_cu(kernel_t k, size_t lds) {
  static std::mutex mu;
  static kernel_t keys[64];
  static int vals[64];
  static int n = 0;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < n; ++i)
    if (keys[i] == k) return vals[i];
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, reinterpret_cast<const void*>(k),
                                                   kThreads, lds) != hipSuccess ||
      nb <= 0)
    nb = 1;
  if (n < 64) {
    keys[n] = k;
    vals[n] = nb;
    ++n;
  }
  return nb;
}

// Raise a partial kernel's dynamic LDS limit to what `lds` needs, once per
// (kernel, device); false if the runtime refuses it.
bool allow_lds(kernel_t k, size_t lds) {
  if (lds <= 65536) return true;
  static std::mutex mu;
  static kernel_t keys[64];
  static int devs[64];
  static int n = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < n; ++i)
    if (keys[i] == k && devs[i] == dev) return true;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                          hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) != hipSuccess)
    return false;
  if (n < 64) {
    keys[n] = k;
    devs[n] = dev;
    ++n;
  }
  return true;
}

}  // namespace

int device_cu_count() {
  static std::mutex mu;
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (cached[dev] == 0) {
    int cu = 0;
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cu <= 0)
      cu = 256;
    cached[dev] = cu;
  }
  return cached[dev];
}

// Latent (MFMA) path, decode_attn_latent.hip.
bool latent_supported(const pda_attn_shape& sh);
size_t latent_workspace_bytes(const pda_attn_shape& sh, int32_t max_seq_len);
size_t latent_min_workspace_bytes(const pda_attn_shape& sh);
int latent_launch(const pda_attn_shape& sh, const void* q, const void* k_cache,
                  const float* token_scale, const int32_t* block_table, const int32_t* seq_lens,
                  int32_t max_seq_len, const int32_t* verdict, void* workspace,
                  size_t workspace_bytes, float* out, hipStream_t stream);

}  // namespace pda

using namespace pda;

extern "C" size_t paged_decode_attn_workspace_bytes(const pda_attn_shape* shape,
                                                    int32_t max_seq_len) {
  if (check_shape(shape) != PDA_OK) return 0;
  if (max_seq_len < 0) return 0;
  const pda_attn_shape& sh = *shape;
  if (latent_supported(sh)) return latent_workspace_bytes(sh, max_seq_len);
  if (!valu_supported(sh)) return 0;
  const int chunk = resolve_chunk(sh, max_seq_len);
  const long long ml = max_seq_len > 0 ? max_seq_len : 1;
  // units per sequence: chunks in groups of kWaves (one merged partial each)
  const long long per_seq = ((ml + chunk - 1) / chunk + kWaves - 1) / kWaves;
  const long long items = (long long)sh.num_seqs * per_seq * sh.num_kv_heads;
  return header_bytes(sh.num_seqs) + (size_t)items * item_bytes(sh);
}

namespace pda {
namespace {

// The whole call behind both entry points: shape checks, then the partial
// and combine launches with the given workspace.
int attn_call(const pda_attn_shape* shape, const void* q, const void* k_cache,
              const void* v_cache, const float* k_scale, const float* v_scale,
              const int32_t* block_table, const int32_t* seq_lens, int32_t max_seq_len,
              const int32_t* verdict, void* workspace, size_t workspace_bytes, float* out,
              void* stream) {
  int st = check_shape(shape);
  if (st != PDA_OK) return st;
  const pda_attn_shape& sh = *shape;
  if (max_seq_len < 0) return PDA_ERR_INVALID_ARG;
  if (sh.num_seqs == 0) return PDA_OK;
  if (!q || !k_cache || !block_table || !seq_lens || !out || !workspace)
    return PDA_ERR_INVALID_ARG;
  if (latent_supported(sh)) {
    if (v_cache || !k_scale || v_scale) return PDA_ERR_INVALID_ARG;
    return latent_launch(sh, q, k_cache, k_scale, block_table, seq_lens, max_seq_len, verdict,
                         workspace, workspace_bytes, out, as_stream(stream));
  }
  if (!valu_supported(sh)) return PDA_ERR_UNSUPPORTED;
  if (!v_cache) return PDA_ERR_INVALID_ARG;
  const bool fp8 = sh.kv_dtype == PDA_KV_FP8_E4M3;
  if (fp8 && (!k_scale || !v_scale)) return PDA_ERR_INVALID_ARG;
  if (!fp8 && (k_scale || v_scale)) return PDA_ERR_INVALID_ARG;
  const size_t hdr = header_bytes(sh.num_seqs);
  const size_t ib = item_bytes(sh);
  // the plan doubles the chunk until the partials fit; it cannot go below one
  // unit per (sequence, kv head)
  if (workspace_bytes < hdr + (size_t)sh.num_seqs * sh.num_kv_heads * ib)
    return PDA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0) return PDA_ERR_INVALID_ARG;
  const int G = sh.num_q_heads / sh.num_kv_heads;
  const int chunk = resolve_chunk(sh, max_seq_len);

  AttnArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.kc = static_cast<const uint8_t*>(k_cache);
  a.vc = static_cast<const uint8_t*>(v_cache);
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.bt = block_table;
  a.lens = seq_lens;
  a.verdict = verdict;
  a.ws_hdr = static_cast<int32_t*>(workspace);
  a.ws_part = reinterpret_cast<float*>(static_cast<char*>(workspace) + hdr);
  a.out = out;
  a.B = sh.num_seqs;
  a.Hq = sh.num_q_heads;
  a.Hkv = sh.num_kv_heads;
  a.P = sh.num_pages;
  a.max_blocks = sh.max_blocks_per_seq;
  a.chunk0 = chunk;
  a.cap_items = (long long)((workspace_bytes - hdr) / ib);
  a.sm_scale = sh.sm_scale;

  const kernel_t pk = fp8 ? pick_partial<true>(G, sh.page_size) : pick_partial<false>(G, sh.page_size);
  const combine_t ck = fp8 ? pick_combine<true>(G) : pick_combine<false>(G);
  const size_t pbuf = (size_t)kWaves * ((size_t)(fp8 ? 1 : 2) * (size_t)G * 64 * 2 +
                                          (fp8 ? 8192 : 0)) +
                      (fp8 ? (size_t)G * kD * 2 : (size_t)kWaves * ((ib + 15) & ~(size_t)15));
  // the plan's scan takes one int per wave; with B = 256 sequences the
  // workgroup then fits four to a CU (40 KB each), which kThreads + 1 ints
  // missed by 32 bytes
  const size_t lds = pbuf + (size_t)(kWaves + sh.num_seqs + 1) * sizeof(int);
  // the per-sequence slot prefix lives in LDS too: past 64 KB (several
  // thousand sequences) the kernel needs the larger dynamic LDS limit
  if (!allow_lds(pk, lds)) return PDA_ERR_LAUNCH;
  const long long ml = max_seq_len > 0 ? max_seq_len : 1;
  const long long units_bound =
      (long long)sh.num_seqs * sh.num_kv_heads * (((ml + chunk - 1) / chunk + kWaves - 1) / kWaves);
  // Four times the resident workgroups (each takes units round-robin): the
  // dispatcher starts workgroups as others retire, so the workgroups sharing
  // a CU reach their unit boundaries (barriers, first loads of an item) at
  // different times instead of all at once; more would mostly add workgroups
  // that find no unit when many sequences are short.
  long long grid = (long long)device_cu_count() * blocks_per_cu(pk, lds) * 4;
  if (grid > units_bound) grid = units_bound;
  if (grid < 1) grid = 1;
  hipStream_t s = as_stream(stream);
  hipLaunchKernelGGL(pk, dim3((unsigned)grid), dim3(kThreads), lds, s, a);
  if (hipGetLastError() != hipSuccess) return PDA_ERR_LAUNCH;
  hipLaunchKernelGGL(ck, dim3((unsigned)(sh.num_seqs * sh.num_kv_heads)), dim3(kThreads), 0, s, a,
                     (int)sh.page_size);
  return launch_status();
}

// Fixed device scratch of the allocation-free entry point: one copy per
// device (file scope, 256-byte aligned), never freed before the process
// ends. Host code never uses the symbol itself as an address: the device
// address of each device's copy is looked up once, with that device
// current, and kept here.
constexpr size_t kScratchBytes = (size_t)96 << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

void* scratch_address() {
  static std::mutex mu;
  static void* addr[64] = {nullptr};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    addr[dev] = p;
  }
  return addr[dev];
}

// Smallest workspace a shape can run in (see paged_decode_attn_workspace_bytes).
size_t min_workspace_bytes(const pda_attn_shape& sh) {
  if (latent_supported(sh)) return latent_min_workspace_bytes(sh);
  return header_bytes(sh.num_seqs) + (size_t)sh.num_seqs * sh.num_kv_heads * item_bytes(sh);
}

}  // namespace
}  // namespace pda

extern "C" int paged_decode_attn(const pda_attn_shape* shape, const void* q, const void* k_cache,
                                 const void* v_cache, const float* k_scale,
                                 const float* v_scale, const int32_t* block_table,
                                 const int32_t* seq_lens, int32_t max_seq_len,
                                 const int32_t* verdict, void* workspace,
                                 size_t workspace_bytes, float* out, void* stream) {
  return attn_call(shape, q, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens,
                   max_seq_len, verdict, workspace, workspace_bytes, out, stream);
}

extern "C" size_t paged_decode_attn_noalloc_scratch_bytes(void) { return kScratchBytes; }

extern "C" int paged_decode_attn_noalloc(const pda_attn_shape* shape, const void* q,
                                         const void* k_cache, const void* v_cache,
                                         const float* k_scale, const float* v_scale,
                                         const int32_t* block_table, const int32_t* seq_lens,
                                         int32_t max_seq_len, const int32_t* verdict,
                                         float* out, void* stream) {
  // host-side checks first: nothing below touches the device before they pass
  int st = check_shape(shape);
  if (st != PDA_OK) return st;
  if (max_seq_len < 0) return PDA_ERR_INVALID_ARG;
  if (shape->num_seqs == 0) return PDA_OK;
  if (!q || !k_cache || !block_table || !seq_lens || !out) return PDA_ERR_INVALID_ARG;
  if ((latent_supported(*shape) || valu_supported(*shape)) &&
      min_workspace_bytes(*shape) > kScratchBytes)
    return PDA_ERR_SCRATCH;
  void* ws = scratch_address();
  if (ws == nullptr) return PDA_ERR_LAUNCH;
  return attn_call(shape, q, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens,
                   max_seq_len, verdict, ws, kScratchBytes, out, stream);
}
