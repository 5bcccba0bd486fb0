// kv_write.hip — quantise new K/V rows to OCP FP8 e4m3 (or copy them as BF16)
// and scatter them into their physical cache slots.
//
// The pages state that the KV cache is stored as 8-bit e4m3 instead of
// 16-bit BF16, which halves its footprint (aifeed.sk, "Cloudflare zrýchľuje
// inferenciu modelov Kimi a GLM kompresiou cache a váh", section "Dve odlišné
// úzke miesta v pamäti GPU"; manulx.blog, "Công thức của Cloudflare để phục
// vụ Kimi và GLM", section "Bộ nhớ đệm KV FP8 tăng gấp đôi dung lượng ngữ
// cảnh"). Rounding, saturation and scaling are not on the pages; the reading
// taken here (fp32 division by the scale, nearest-even, saturate to ±448,
// keep the sign of zero, NaN -> 0x7F|sign) is stated in include/pda.h.
//
// One workgroup per token; each thread converts groups of 4 consecutive
// dims, which are contiguous in the K format and two bytes apart in the V
// format (the V format interleaves the two tokens of a slot pair).
#include "pda_internal.h"
#include "validate_body.h"

namespace pda {
namespace {

constexpr int kThreads = 256;

// e4m3 codes of four fp32 quotients packed little-endian into a dword, via
// the gfx950 converter (OCP e4m3, round to nearest even). Measured on every
// bf16 value: the converter's codes are exact for every finite |y| below
// 464 (values from 448 up round to 448 there) and never 0x7F/0xFF; from 464
// up and for ±inf it returns the NaN code with the input's sign, and for a
// NaN input 0xFF whatever its sign. So the bytes equal to 0x7F or 0xFF are
// exactly the ones to fix: saturation (0x7E|sign) or NaN (0x7F|sign). They
// are found four at a time with byte arithmetic; the per-element fix runs
// only when one is present (never for data scaled into ±448). The fix takes
// NaN-ness and sign from f: the quotient itself, or the dividend where the
// quotient of a positive finite scale was computed in a way that can turn
// an infinite dividend into NaN.
__device__ __forceinline__ uint32_t e4m3x4(float y0, float y1, float y2, float y3, float f0,
                                           float f1, float f2, float f3) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, w, true);
  uint32_t r = (uint32_t)w;
  // z byte == 0 exactly where the code is 0x7F or 0xFF; every z byte is at
  // most 0x7F, so z + 0x7F per byte never carries into the next byte
  const uint32_t z = (r & 0x7F7F7F7Fu) ^ 0x7F7F7F7Fu;
  const uint32_t hit = ~((z + 0x7F7F7F7Fu) | z) & 0x80808080u;
  if (hit != 0) {
    const float fs[4] = {f0, f1, f2, f3};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (hit & (0x80u << (8 * i))) {
        const uint32_t sgn = (as_u32(fs[i]) >> 31) << 7;
        const uint32_t code = (__builtin_isnan(fs[i]) ? 0x7Fu : 0x7Eu) | sgn;
        r = (r & ~(0xFFu << (8 * i))) | (code << (8 * i));
      }
    }
  }
  return r;
}

__device__ __forceinline__ uint32_t e4m3x4(float y0, float y1, float y2, float y3) {
  return e4m3x4(y0, y1, y2, y3, y0, y1, y2, y3);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return as_f32(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return as_f32(w & 0xFFFF0000u); }

// Element index of (page, head, offset, dim) in the K format.
__device__ __forceinline__ int64_t k_elem(int64_t page, int h, int off, int d, int hkv, int dk,
                                          int S) {
  return (((page * hkv + h) * (dk / 16) + d / 16) * S + off) * 16 + (d & 15);
}
// Element index of (page, head, offset, dim) in the V format.
__device__ __forceinline__ int64_t v_elem(int64_t page, int h, int off, int d, int hkv, int dv,
                                          int S) {
  return ((((page * hkv + h) * (S / 2) + off / 2) * (dv / 8) + d / 8) * 8 + (d & 7)) * 2 +
         (off & 1);
}

// Arguments of one kv write (FP8 or BF16 cache).
struct WriteArgs {
  const uint16_t* k_new;
  const uint16_t* v_new;
  const int64_t* slots;
  int hkv, dk, dv, S, P;
  const float* k_scale;
  const float* v_scale;
  float* token_scale;
  void* k_cache;
  void* v_cache;
};

// Token t of an FP8 write, by one workgroup of kThreads threads; red is
// kThreads / 64 floats of LDS.
template <bool PER_TOKEN>
__device__ __forceinline__ void write_token_fp8(const WriteArgs& w, int t, float* red) {
  const uint16_t* __restrict__ k_new = w.k_new;
  const uint16_t* __restrict__ v_new = w.v_new;
  const int hkv = w.hkv, dk = w.dk, dv = w.dv, S = w.S, P = w.P;
  const float* __restrict__ k_scale = w.k_scale;
  const float* __restrict__ v_scale = w.v_scale;
  uint8_t* __restrict__ k_cache = static_cast<uint8_t*>(w.k_cache);
  uint8_t* __restrict__ v_cache = static_cast<uint8_t*>(w.v_cache);
  const int64_t slot = w.slots[t];
  if (slot < 0 || slot >= (int64_t)P * S) return;
  const int64_t page = slot / S;
  const int off = (int)(slot % S);
  const int tid = threadIdx.x;

  float tok_sc = 1.0f;
  if (PER_TOKEN) {
    // amax over the token's K values (Hkv == 1); NaN values are ignored.
    float amax = 0.0f;
    const uint16_t* src = k_new + (int64_t)t * dk;
    for (int d = tid; d < dk; d += kThreads)
      amax = fmaxf(amax, fabsf(as_f32((uint32_t)src[d] << 16)));
    amax = wave_max(amax);
    if ((tid & 63) == 0) red[tid >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    tok_sc = (amax > 0.0f) ? amax / 448.0f : 1.0f;
    if (tid == 0) w.token_scale[slot] = tok_sc;
  }

  // K: groups of 4 dims, contiguous in the cache.
  const int kq = hkv * dk / 4;
  for (int i = tid; i < kq; i += kThreads) {
    const int h = (i * 4) / dk;
    const int d = (i * 4) % dk;
    const uint2 x = *reinterpret_cast<const uint2*>(k_new + ((int64_t)t * hkv + h) * dk + d);
    const float sc = PER_TOKEN ? tok_sc : k_scale[h];
    const uint32_t codes = e4m3x4(bf16_lo(x.x) / sc, bf16_hi(x.x) / sc, bf16_lo(x.y) / sc,
                                  bf16_hi(x.y) / sc);
    *reinterpret_cast<uint32_t*>(k_cache + k_elem(page, h, off, d, hkv, dk, S)) = codes;
  }
  if (v_new == nullptr) return;
  // V: groups of 4 dims, two bytes apart in the cache.
  const int vq = hkv * dv / 4;
  for (int i = tid; i < vq; i += kThreads) {
    const int h = (i * 4) / dv;
    const int d = (i * 4) % dv;
    const uint2 x = *reinterpret_cast<const uint2*>(v_new + ((int64_t)t * hkv + h) * dv + d);
    const float sc = v_scale[h];
    const uint32_t codes = e4m3x4(bf16_lo(x.x) / sc, bf16_hi(x.x) / sc, bf16_lo(x.y) / sc,
                                  bf16_hi(x.y) / sc);
    uint8_t* dst = v_cache + v_elem(page, h, off, d, hkv, dv, S);
    dst[0] = (uint8_t)(codes);
    dst[2] = (uint8_t)(codes >> 8);
    dst[4] = (uint8_t)(codes >> 16);
    dst[6] = (uint8_t)(codes >> 24);
  }
}

// Token t of a BF16 write (a copy into the cache formats).
__device__ __forceinline__ void write_token_bf16(const WriteArgs& w, int t) {
  const uint16_t* __restrict__ k_new = w.k_new;
  const uint16_t* __restrict__ v_new = w.v_new;
  const int hkv = w.hkv, dk = w.dk, dv = w.dv, S = w.S, P = w.P;
  uint16_t* __restrict__ k_cache = static_cast<uint16_t*>(w.k_cache);
  uint16_t* __restrict__ v_cache = static_cast<uint16_t*>(w.v_cache);
  const int64_t slot = w.slots[t];
  if (slot < 0 || slot >= (int64_t)P * S) return;
  const int64_t page = slot / S;
  const int off = (int)(slot % S);
  const int tid = threadIdx.x;
  const int kq = hkv * dk / 4;
  for (int i = tid; i < kq; i += kThreads) {
    const int h = (i * 4) / dk;
    const int d = (i * 4) % dk;
    const uint2 x = *reinterpret_cast<const uint2*>(k_new + ((int64_t)t * hkv + h) * dk + d);
    *reinterpret_cast<uint2*>(k_cache + k_elem(page, h, off, d, hkv, dk, S)) = x;
  }
  if (v_new == nullptr) return;
  const int vq = hkv * dv / 4;
  for (int i = tid; i < vq; i += kThreads) {
    const int h = (i * 4) / dv;
    const int d = (i * 4) % dv;
    const uint2 x = *reinterpret_cast<const uint2*>(v_new + ((int64_t)t * hkv + h) * dv + d);
    uint16_t* dst = v_cache + v_elem(page, h, off, d, hkv, dv, S);
    dst[0] = (uint16_t)(x.x);
    dst[2] = (uint16_t)(x.x >> 16);
    dst[4] = (uint16_t)(x.y);
    dst[6] = (uint16_t)(x.y >> 16);
  }
}

// ---- BF16 -> FP8 page transcode ---------------------------------------------
// Both formats share the element order, so a (page, head) block of either
// cache is S*Dk (K) or S*Dv (V) consecutive elements and the transcode is
// elementwise on matching indices: 8 elements (16 bytes in, 8 out) per step.

// Slot of element e of a (page, head) block. K: rows of 16 dims per slot in
// column groups of S rows. V: slot pairs interleaved element by element.
__device__ __forceinline__ int k_slot(int e, int S) { return (e >> 4) % S; }
__device__ __forceinline__ int v_slot(int e, int dv) { return 2 * (e / (2 * dv)) + (e & 1); }

__device__ __forceinline__ uint2 encode8(uint4 x, float sc) {
  return make_uint2(e4m3x4(bf16_lo(x.x) / sc, bf16_hi(x.x) / sc, bf16_lo(x.y) / sc,
                           bf16_hi(x.y) / sc),
                    e4m3x4(bf16_lo(x.z) / sc, bf16_hi(x.z) / sc, bf16_lo(x.w) / sc,
                           bf16_hi(x.w) / sc));
}

// Division by a scale through its reciprocal. With y = 1/s correctly
// rounded, q0 = x*y, the residual r = q0*s - x (exact in one fma) and
// q = q0 - r*y rounded once, q is the correctly rounded quotient x / s (the
// reciprocal-based correction step of Markstein's division) as long as the
// residual cannot underflow. For bf16 x and s in [2^-64, 2^64] that holds
// for every quotient of magnitude 2^-11 or more; smaller quotients come out
// below 2^-10 with the right sign, which encodes to the same ±0 code. The
// residual's sign is taken so that x = -0 gives -0. Compared on the host with
// the correctly rounded division over all bf16 x for 10^5 scales spread over
// that interval and beyond it: identical inside, wrong near 2^-92 and below.
__device__ __forceinline__ bool fast_divisor(float s) { return s >= 0x1p-64f && s <= 0x1p64f; }

__device__ __forceinline__ float quot(float x, float s, float y) {
  const float q0 = x * y;
  const float r = __builtin_fmaf(q0, s, -x);
  return __builtin_fmaf(-r, y, q0);
}

__device__ __forceinline__ uint32_t encode4_rcp(uint32_t a, uint32_t b, float s, float y) {
  const float x0 = bf16_lo(a), x1 = bf16_hi(a), x2 = bf16_lo(b), x3 = bf16_hi(b);
  return e4m3x4(quot(x0, s, y), quot(x1, s, y), quot(x2, s, y), quot(x3, s, y), x0, x1, x2, x3);
}

__device__ __forceinline__ uint2 encode8_rcp(uint4 x, float s, float y) {
  return make_uint2(encode4_rcp(x.x, x.y, s, y), encode4_rcp(x.z, x.w, s, y));
}

__device__ __forceinline__ bool pair_ok(int src, int dst, int n, int ps, int pd, int S) {
  return src >= 0 && src < ps && dst >= 0 && dst < pd && n >= 0 && n <= S;
}

// One workgroup per pair, per-head scales: the page's blocks of all kv heads
// are contiguous (Hkv*S*Dk K elements, then Hkv*S*Dv V elements), each
// thread takes 8 elements per step, four steps' loads issued before their
// conversions and stores.
template <bool PER_TOKEN>
__global__ __launch_bounds__(kThreads) void kv_write_fp8_kernel(WriteArgs w) {
  __shared__ float red[kThreads / 64];
  write_token_fp8<PER_TOKEN>(w, blockIdx.x, red);
}

__global__ __launch_bounds__(kThreads) void kv_write_bf16_kernel(WriteArgs w) {
  write_token_bf16(w, blockIdx.x);
}

// Arguments of one page-tag check.
struct CheckArgs {
  const uint32_t* page_tags;
  int P;
  const int32_t* block_table;
  const uint32_t* expected;
  int max_blocks;
  const int32_t* lens;
  int S;
  int32_t* verdict;
};

// The kv write and the page-tag check of one decode step in one launch:
// workgroups [0, T) write token t, workgroups [T, T + B) check sequence
// t - T. The two touch disjoint memory (the check reads tags, table and
// lengths and writes verdicts; the write reads new rows and writes cache
// bytes), so their order does not matter, and the launch boundary orders
// both before the attention that follows. MODE 0: FP8 per-head scales, 1:
// FP8 per-token scales, 2: BF16.
template <int MODE>
__global__ __launch_bounds__(kThreads) void kv_write_check_kernel(WriteArgs w, int T,
                                                                  CheckArgs c) {
  static_assert(kThreads == kValidateThreads, "one workgroup shape for both parts");
  __shared__ float red[kThreads / 64];
  __shared__ int best[kThreads / 64];
  const int b = blockIdx.x;
  if (b < T) {
    if constexpr (MODE == 2) write_token_bf16(w, b);
    else write_token_fp8<MODE == 1>(w, b, red);
  } else {
    validate_seq(b - T, c.page_tags, c.P, c.block_table, c.expected, c.max_blocks, c.lens, c.S,
                 c.verdict, best);
  }
}

template <bool V, bool FAST>
__device__ __forceinline__ void transcode_span(const uint16_t* __restrict__ src,
                                               uint8_t* __restrict__ dst, int n_elems,
                                               int head_elems, int S, int D, int valid,
                                               const float* __restrict__ scale,
                                               const float* __restrict__ rcp) {
  constexpr int U = 4;
  for (int e0 = threadIdx.x * 8; e0 < n_elems; e0 += kThreads * 8 * U) {
    uint4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = e0 + u * kThreads * 8;
      if (e < n_elems) x[u] = *reinterpret_cast<const uint4*>(src + e);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = e0 + u * kThreads * 8;
      if (e >= n_elems) break;
      const int h = e / head_elems;
      const int eh = e - h * head_elems;
      const int s0 = V ? v_slot(eh, D) : k_slot(eh, S);
      if (s0 >= valid) continue;
      const uint2 c = FAST ? encode8_rcp(x[u], scale[h], rcp[h]) : encode8(x[u], scale[h]);
      if (!V || s0 + 1 < valid) {
        *reinterpret_cast<uint2*>(dst + e) = c;
      } else {   // only the even slot of a V pair: its four bytes
        uint8_t* d = dst + e;
        d[0] = (uint8_t)c.x;
        d[2] = (uint8_t)(c.x >> 16);
        d[4] = (uint8_t)c.y;
        d[6] = (uint8_t)(c.y >> 16);
      }
    }
  }
}

// Reciprocals of the K and V scales of up to kMaxRcpHeads kv heads are
// kept in LDS; with more heads, or any scale outside the fast divisor
// interval, the workgroup divides instead.
constexpr int kMaxRcpHeads = 256;

__global__ __launch_bounds__(kThreads) void kv_transcode_head_kernel(
    const uint16_t* __restrict__ k_src, const uint16_t* __restrict__ v_src,
    const int32_t* __restrict__ src_pages, const int32_t* __restrict__ dst_pages,
    const int32_t* __restrict__ valid, int hkv, int dk, int dv, int S, int ps, int pd,
    const float* __restrict__ k_scale, const float* __restrict__ v_scale,
    uint8_t* __restrict__ k_dst, uint8_t* __restrict__ v_dst) {
  __shared__ float rcp[2 * kMaxRcpHeads];
  __shared__ int slow;
  const int pair = blockIdx.x;
  const int src = src_pages[pair], dst = dst_pages[pair], n = valid[pair];
  if (!pair_ok(src, dst, n, ps, pd, S) || n == 0) return;
  const int nsc = (v_src == nullptr) ? hkv : 2 * hkv;
  bool fast = hkv <= kMaxRcpHeads;
  if (fast) {
    if (threadIdx.x == 0) slow = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < nsc; i += kThreads) {
      const float sc = (i < hkv) ? k_scale[i] : v_scale[i - hkv];
      if (fast_divisor(sc))
        rcp[i] = 1.0f / sc;
      else
        slow = 1;
    }
    __syncthreads();
    fast = (slow == 0);
  }
  const int nk = hkv * S * dk;
  const uint16_t* ks = k_src + (int64_t)src * nk;
  uint8_t* kd = k_dst + (int64_t)dst * nk;
  if (fast)
    transcode_span<false, true>(ks, kd, nk, S * dk, S, dk, n, k_scale, rcp);
  else
    transcode_span<false, false>(ks, kd, nk, S * dk, S, dk, n, k_scale, rcp);
  if (v_src == nullptr) return;
  const int nv = hkv * S * dv;
  const uint16_t* vs = v_src + (int64_t)src * nv;
  uint8_t* vd = v_dst + (int64_t)dst * nv;
  if (fast)
    transcode_span<true, true>(vs, vd, nv, S * dv, S, dv, n, v_scale, rcp + hkv);
  else
    transcode_span<true, false>(vs, vd, nv, S * dv, S, dv, n, v_scale, rcp + hkv);
}

// One workgroup per pair, latent cache (Hkv == 1, K only), per-token scales:
// thread (slot t, quarter q) handles column groups q, q+4, ... of slot t.
__global__ __launch_bounds__(kThreads) void kv_transcode_token_kernel(
    const uint16_t* __restrict__ k_src, const int32_t* __restrict__ src_pages,
    const int32_t* __restrict__ dst_pages, const int32_t* __restrict__ valid, int dk, int S,
    int ps, int pd, float* __restrict__ token_scale, uint8_t* __restrict__ k_dst) {
  __shared__ float red[kThreads];
  const int pair = blockIdx.x;
  const int src = src_pages[pair], dst = dst_pages[pair], n = valid[pair];
  if (!pair_ok(src, dst, n, ps, pd, S) || n == 0) return;
  const int64_t sb = (int64_t)src * S * dk;
  const int64_t db = (int64_t)dst * S * dk;
  const int groups = dk / 16;
  const int per = kThreads / S;   // threads per slot (S divides kThreads)
  for (int t0 = 0; t0 < S; t0 += kThreads / per) {
    const int t = t0 + threadIdx.x % (kThreads / per);
    const int q = threadIdx.x / (kThreads / per);
    const bool live = t < S && t < n;
    float amax = 0.0f;   // NaN values are ignored (fmaxf)
    if (live)
      for (int c = q; c < groups; c += per) {
        const uint16_t* x = k_src + sb + ((int64_t)c * S + t) * 16;
        const uint4 a = *reinterpret_cast<const uint4*>(x);
        const uint4 b = *reinterpret_cast<const uint4*>(x + 8);
        const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 8; ++i)
          amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(w[i])), fabsf(bf16_hi(w[i]))));
      }
    red[threadIdx.x] = amax;
    __syncthreads();
    if (live) {
      float m = 0.0f;
      for (int i = 0; i < per; ++i) m = fmaxf(m, red[i * (kThreads / per) + threadIdx.x % (kThreads / per)]);
      const float sc = (m > 0.0f) ? m / 448.0f : 1.0f;
      if (q == 0) token_scale[(int64_t)dst * S + t] = sc;
      if (fast_divisor(sc)) {
        const float y = 1.0f / sc;
        for (int c = q; c < groups; c += per) {
          const int64_t o = ((int64_t)c * S + t) * 16;
          const uint4 a = *reinterpret_cast<const uint4*>(k_src + sb + o);
          const uint4 b = *reinterpret_cast<const uint4*>(k_src + sb + o + 8);
          const uint2 ca = encode8_rcp(a, sc, y), cb = encode8_rcp(b, sc, y);
          *reinterpret_cast<uint4*>(k_dst + db + o) = make_uint4(ca.x, ca.y, cb.x, cb.y);
        }
      } else {
        for (int c = q; c < groups; c += per) {
          const int64_t o = ((int64_t)c * S + t) * 16;
          const uint4 a = *reinterpret_cast<const uint4*>(k_src + sb + o);
          const uint4 b = *reinterpret_cast<const uint4*>(k_src + sb + o + 8);
          const uint2 ca = encode8(a, sc), cb = encode8(b, sc);
          *reinterpret_cast<uint4*>(k_dst + db + o) = make_uint4(ca.x, ca.y, cb.x, cb.y);
        }
      }
    }
    __syncthreads();   // red is reused by the next round of slots
  }
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_common(const void* k_new, const void* v_new, const int64_t* slots, int32_t T,
                 int32_t hkv, int32_t dk, int32_t dv, int32_t S, int32_t P, const void* kc,
                 const void* vc) {
  if (T < 0 || hkv <= 0 || dk <= 0 || S <= 0 || P <= 0) return PDA_ERR_INVALID_ARG;
  if (T > 0 && (!k_new || !slots)) return PDA_ERR_INVALID_ARG;
  if (!kc) return PDA_ERR_INVALID_ARG;
  const bool latent = (v_new == nullptr);
  if (latent != (vc == nullptr)) return PDA_ERR_INVALID_ARG;
  if (dk % 16 != 0 || S % 2 != 0) return PDA_ERR_UNSUPPORTED;
  if (!latent && (dv <= 0 || dv % 8 != 0)) return PDA_ERR_UNSUPPORTED;
  if (!aligned(k_new, 8) || (!latent && !aligned(v_new, 8)) || !aligned(kc, 8))
    return PDA_ERR_INVALID_ARG;
  return PDA_OK;
}

}  // namespace
}  // namespace pda

using namespace pda;

extern "C" int kv_write_fp8(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                            int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim_k,
                            int32_t head_dim_v, int32_t page_size, int32_t num_pages,
                            int32_t scale_mode, const float* k_scale, const float* v_scale,
                            float* token_scale, uint8_t* k_cache, uint8_t* v_cache,
                            void* stream) {
  int st = check_common(k_new, v_new, slot_mapping, num_tokens, num_kv_heads, head_dim_k,
                        head_dim_v, page_size, num_pages, k_cache, v_cache);
  if (st != PDA_OK) return st;
  const bool latent = (v_new == nullptr);
  if (scale_mode == PDA_SCALE_PER_HEAD) {
    if (!k_scale || (!latent && !v_scale) || token_scale) return PDA_ERR_INVALID_ARG;
  } else if (scale_mode == PDA_SCALE_PER_TOKEN) {
    if (!token_scale || k_scale || v_scale) return PDA_ERR_INVALID_ARG;
    if (!latent || num_kv_heads != 1) return PDA_ERR_UNSUPPORTED;
  } else {
    return PDA_ERR_INVALID_ARG;
  }
  if (num_tokens == 0) return PDA_OK;
  hipStream_t s = as_stream(stream);
  const auto* kn = static_cast<const uint16_t*>(k_new);
  const auto* vn = static_cast<const uint16_t*>(v_new);
  const WriteArgs w{kn, vn, slot_mapping, num_kv_heads, head_dim_k, head_dim_v, page_size,
                   num_pages, k_scale, v_scale, token_scale, k_cache, v_cache};
  if (scale_mode == PDA_SCALE_PER_TOKEN)
    hipLaunchKernelGGL(kv_write_fp8_kernel<true>, dim3(num_tokens), dim3(kThreads), 0, s, w);
  else
    hipLaunchKernelGGL(kv_write_fp8_kernel<false>, dim3(num_tokens), dim3(kThreads), 0, s, w);
  return launch_status();
}

extern "C" int kv_write_bf16(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                             int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim_k,
                             int32_t head_dim_v, int32_t page_size, int32_t num_pages,
                             void* k_cache, void* v_cache, void* stream) {
  int st = check_common(k_new, v_new, slot_mapping, num_tokens, num_kv_heads, head_dim_k,
                        head_dim_v, page_size, num_pages, k_cache, v_cache);
  if (st != PDA_OK) return st;
  if (num_tokens == 0) return PDA_OK;
  const WriteArgs w{static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                   slot_mapping, num_kv_heads, head_dim_k, head_dim_v, page_size, num_pages,
                   nullptr, nullptr, nullptr, k_cache, v_cache};
  hipLaunchKernelGGL(kv_write_bf16_kernel, dim3(num_tokens), dim3(kThreads), 0,
                     as_stream(stream), w);
  return launch_status();
}

extern "C" int kv_write_check(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                              int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim_k,
                              int32_t head_dim_v, int32_t page_size, int32_t num_pages,
                              int32_t kv_dtype, int32_t scale_mode, const float* k_scale,
                              const float* v_scale, float* token_scale, void* k_cache,
                              void* v_cache, const uint32_t* page_tags,
                              const int32_t* block_table, const uint32_t* expected_tags,
                              int32_t max_blocks_per_seq, const int32_t* seq_lens,
                              int32_t num_seqs, int32_t* verdict, void* stream) {
  // the write's arguments, as kv_write_fp8 / kv_write_bf16 check them (not
  // read at all when there are no tokens: empty tensors may come as NULL)
  int mode = 0;
  if (num_tokens < 0) return PDA_ERR_INVALID_ARG;
  if (num_tokens > 0) {
    int st = check_common(k_new, v_new, slot_mapping, num_tokens, num_kv_heads, head_dim_k,
                          head_dim_v, page_size, num_pages, k_cache, v_cache);
    if (st != PDA_OK) return st;
    const bool latent = (v_new == nullptr);
    if (kv_dtype == PDA_KV_FP8_E4M3) {
      if (scale_mode == PDA_SCALE_PER_HEAD) {
        if (!k_scale || (!latent && !v_scale) || token_scale) return PDA_ERR_INVALID_ARG;
        mode = 0;
      } else if (scale_mode == PDA_SCALE_PER_TOKEN) {
        if (!token_scale || k_scale || v_scale) return PDA_ERR_INVALID_ARG;
        if (!latent || num_kv_heads != 1) return PDA_ERR_UNSUPPORTED;
        mode = 1;
      } else {
        return PDA_ERR_INVALID_ARG;
      }
    } else if (kv_dtype == PDA_KV_BF16) {
      if (scale_mode != PDA_SCALE_NONE || k_scale || v_scale || token_scale)
        return PDA_ERR_INVALID_ARG;
      mode = 2;
    } else {
      return PDA_ERR_INVALID_ARG;
    }
  }
  // the check's arguments, as validate_page_tags checks them
  if (num_seqs < 0) return PDA_ERR_INVALID_ARG;
  if (num_seqs > 0 && (max_blocks_per_seq <= 0 || num_pages <= 0 || page_size <= 0))
    return PDA_ERR_INVALID_ARG;
  if (num_seqs > 0 && (!page_tags || !block_table || !expected_tags || !seq_lens || !verdict))
    return PDA_ERR_INVALID_ARG;
  if ((int64_t)num_tokens + num_seqs > 0x7FFFFFFF) return PDA_ERR_UNSUPPORTED;
  if (num_tokens + num_seqs == 0) return PDA_OK;
  const WriteArgs w{static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                    slot_mapping, num_kv_heads, head_dim_k, head_dim_v, page_size, num_pages,
                    k_scale, v_scale, token_scale, k_cache, v_cache};
  const CheckArgs c{page_tags, num_pages, block_table, expected_tags, max_blocks_per_seq,
                    seq_lens, page_size, verdict};
  const dim3 grid((unsigned)(num_tokens + num_seqs));
  hipStream_t s = as_stream(stream);
  if (mode == 0)
    hipLaunchKernelGGL(kv_write_check_kernel<0>, grid, dim3(kThreads), 0, s, w, num_tokens, c);
  else if (mode == 1)
    hipLaunchKernelGGL(kv_write_check_kernel<1>, grid, dim3(kThreads), 0, s, w, num_tokens, c);
  else
    hipLaunchKernelGGL(kv_write_check_kernel<2>, grid, dim3(kThreads), 0, s, w, num_tokens, c);
  return launch_status();
}

extern "C" int kv_transcode_bf16_to_fp8(const void* k_src, const void* v_src,
                                        const int32_t* src_pages, const int32_t* dst_pages,
                                        const int32_t* valid, int32_t num_pairs,
                                        int32_t num_kv_heads, int32_t head_dim_k,
                                        int32_t head_dim_v, int32_t page_size,
                                        int32_t src_num_pages, int32_t dst_num_pages,
                                        int32_t scale_mode, const float* k_scale,
                                        const float* v_scale, float* token_scale,
                                        uint8_t* k_dst, uint8_t* v_dst, void* stream) {
  if (num_pairs < 0 || num_kv_heads <= 0 || head_dim_k <= 0 || page_size <= 0 ||
      src_num_pages <= 0 || dst_num_pages <= 0)
    return PDA_ERR_INVALID_ARG;
  if (num_pairs > 0 && (!src_pages || !dst_pages || !valid)) return PDA_ERR_INVALID_ARG;
  if (!k_src || !k_dst) return PDA_ERR_INVALID_ARG;
  const bool latent = (v_src == nullptr);
  if (latent != (v_dst == nullptr)) return PDA_ERR_INVALID_ARG;
  if (head_dim_k % 16 != 0 || page_size % 2 != 0) return PDA_ERR_UNSUPPORTED;
  if (!latent && (head_dim_v <= 0 || head_dim_v % 8 != 0)) return PDA_ERR_UNSUPPORTED;
  if (!aligned(k_src, 16) || (!latent && !aligned(v_src, 16)) || !aligned(k_dst, 16) ||
      (!latent && !aligned(v_dst, 8)))
    return PDA_ERR_INVALID_ARG;
  if (scale_mode == PDA_SCALE_PER_HEAD) {
    if (!k_scale || (!latent && !v_scale) || token_scale) return PDA_ERR_INVALID_ARG;
  } else if (scale_mode == PDA_SCALE_PER_TOKEN) {
    if (!token_scale || k_scale || v_scale) return PDA_ERR_INVALID_ARG;
    if (!latent || num_kv_heads != 1) return PDA_ERR_UNSUPPORTED;
    if (kThreads % page_size != 0) return PDA_ERR_UNSUPPORTED;
  } else {
    return PDA_ERR_INVALID_ARG;
  }
  if (num_pairs == 0) return PDA_OK;
  hipStream_t s = as_stream(stream);
  if (scale_mode == PDA_SCALE_PER_TOKEN)
    hipLaunchKernelGGL(kv_transcode_token_kernel, dim3(num_pairs), dim3(kThreads), 0, s,
                       static_cast<const uint16_t*>(k_src), src_pages, dst_pages, valid,
                       head_dim_k, page_size, src_num_pages, dst_num_pages, token_scale, k_dst);
  else
    hipLaunchKernelGGL(kv_transcode_head_kernel, dim3((unsigned)num_pairs), dim3(kThreads), 0, s, static_cast<const uint16_t*>(k_src),
                       static_cast<const uint16_t*>(v_src), src_pages, dst_pages, valid,
                       num_kv_heads, head_dim_k, head_dim_v, page_size, src_num_pages,
                       dst_num_pages, k_scale, v_scale, k_dst, v_dst);
  return launch_status();
}
