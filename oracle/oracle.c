/*
 * oracle.c — plain CPU oracle (test infrastructure only; see oracle.h).
 *
 * Build: gcc -std=c11 -O2 -ffp-contract=off -fPIC -shared -pthread
 *        -o liboracle.so oracle.c -lm
 * No fast-math and no contraction: every fp32 operation below is the IEEE
 * operation it spells, and every fp64 sum is taken in loop order.
 */
#include "oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* OCP FP8 E4M3                                                              */
/* ------------------------------------------------------------------------ */

double oracle_e4m3_decode(uint8_t code) {
  int sign = code >> 7;
  int exp_field = (code >> 3) & 0xF;
  int mant = code & 0x7;
  double mag;
  if (exp_field == 0xF && mant == 0x7) return NAN;
  if (exp_field == 0)
    mag = ldexp((double)mant, -9); /* subnormal: m * 2^-6 / 8 */
  else
    mag = ldexp((double)(8 + mant), exp_field - 10); /* (1+m/8) 2^(e-7) */
  return sign ? -mag : mag;
}

/* Brute force over the 127 non-negative finite codes 0x00..0x7E. The
 * distances that decide a comparison are exact in fp64: near a tie, |x| and
 * the two neighbouring code values lie within a few binades of each other,
 * so |x| - v needs at most 24 + 5 significant bits; far candidates differ by
 * factors no rounding can flip. This is the definition the faster search
 * below is checked against. */
uint8_t oracle_e4m3_encode_brute(float x) {
  uint8_t sign = signbit(x) ? 0x80 : 0x00;
  if (isnan(x)) return (uint8_t)(0x7F | sign);
  double a = fabs((double)x);
  if (a >= 448.0) return (uint8_t)(0x7E | sign);
  int best = 0;
  double best_d = a; /* distance to code 0 (value 0) */
  for (int c = 1; c <= 0x7E; ++c) {
    double d = fabs(oracle_e4m3_decode((uint8_t)c) - a);
    if (d < best_d || (d == best_d && (c & 1) == 0)) {
      best = c;
      best_d = d;
    }
  }
  return (uint8_t)(best | sign);
}

/* The values of codes 0x00..0x7E, which increase with the code. */
static double g_e4m3_values[127];
static pthread_once_t g_e4m3_once = PTHREAD_ONCE_INIT;

static void e4m3_values_init(void) {
  for (int c = 0; c <= 0x7E; ++c) g_e4m3_values[c] = oracle_e4m3_decode((uint8_t)c);
}

/* The same nearest code, found by bisection instead of a scan: since the
 * values increase with the code, |x| lies between code lo (largest value
 * <= |x|) and lo + 1, and the nearer of the two wins, the even one on a
 * tie. The two distances are exact or far from equal, as above. */
uint8_t oracle_e4m3_encode(float x) {
  uint8_t sign = signbit(x) ? 0x80 : 0x00;
  if (isnan(x)) return (uint8_t)(0x7F | sign);
  double a = fabs((double)x);
  if (a >= 448.0) return (uint8_t)(0x7E | sign);
  pthread_once(&g_e4m3_once, e4m3_values_init);
  int lo = 0, hi = 0x7E; /* value(lo) = 0 <= a < 448 = value(hi) */
  while (hi - lo > 1) {
    int mid = (lo + hi) / 2;
    if (g_e4m3_values[mid] <= a) lo = mid; else hi = mid;
  }
  double d_lo = a - g_e4m3_values[lo], d_hi = g_e4m3_values[hi] - a;
  int c = (d_lo < d_hi) ? lo : (d_hi < d_lo) ? hi : ((lo & 1) == 0 ? lo : hi);
  return (uint8_t)(c | sign);
}

/* Closed form: codes are equally spaced inside each binade and the spacing
 * runs on across the subnormal/normal boundary, so the code index is
 * 8*(e+7) + rint((|x|/2^e - 1)*8) for |x| >= 2^-6 and rint(|x|*2^9) below,
 * with rint rounding half to even (the default rounding mode). */
uint8_t oracle_e4m3_encode_closed(float x) {
  uint8_t sign = signbit(x) ? 0x80 : 0x00;
  if (isnan(x)) return (uint8_t)(0x7F | sign);
  double a = fabs((double)x);
  if (a >= 448.0) return (uint8_t)(0x7E | sign);
  if (a < ldexp(1.0, -6)) return (uint8_t)((int)nearbyint(a * 512.0) | sign);
  int e2;
  double m = frexp(a, &e2); /* a = m * 2^e2, m in [0.5, 1) */
  int e = e2 - 1;           /* a = (2m) * 2^e, 2m in [1, 2) */
  double frac = (2.0 * m - 1.0) * 8.0;
  int code = 8 * (e + 7) + (int)nearbyint(frac);
  return (uint8_t)(code | sign);
}

float oracle_bf16_to_f32(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* ------------------------------------------------------------------------ */
/* Cache format (include/pda.h): element indices of one (page, head, o, d).  */
/* ------------------------------------------------------------------------ */

static size_t k_index(int64_t page, int32_t head, int32_t off, int32_t d,
                      int32_t hkv, int32_t dk, int32_t s) {
  int64_t group = ((page * hkv + head) * (dk / 16) + d / 16);
  return (size_t)((group * s + off) * 16 + d % 16);
}

static size_t v_index(int64_t page, int32_t head, int32_t off, int32_t d,
                      int32_t hkv, int32_t dv, int32_t s) {
  int64_t pair_row = ((page * hkv + head) * (s / 2) + off / 2);
  return (size_t)(((pair_row * (dv / 8) + d / 8) * 8 + d % 8) * 2 + off % 2);
}

/* ------------------------------------------------------------------------ */
/* KV write                                                                  */
/* ------------------------------------------------------------------------ */

static int kv_args_ok(int32_t num_tokens, int32_t hkv, int32_t dk, int32_t dv,
                      int32_t s, int32_t p, int latent) {
  if (num_tokens < 0 || hkv <= 0 || dk <= 0 || s <= 0 || p <= 0) return 0;
  if (dk % 16 != 0 || s % 2 != 0) return 0;
  if (!latent && (dv <= 0 || dv % 8 != 0)) return 0;
  return 1;
}

/* Quantise-and-scatter as the header of kv_write_fp8 defines it. Reading of
 * the pages, which only say the cache is stored as e4m3 ([VN] § "Bộ nhớ đệm
 * KV FP8 tăng gấp đôi dung lượng ngữ cảnh"): code = e4m3(x / scale), the
 * division an IEEE fp32 division. */
int oracle_kv_write_fp8(const uint16_t* k_new, const uint16_t* v_new,
                        const int64_t* slot_mapping, int32_t num_tokens,
                        int32_t hkv, int32_t dk, int32_t dv, int32_t s,
                        int32_t p, int32_t scale_mode, const float* k_scale,
                        const float* v_scale, float* token_scale,
                        uint8_t* k_cache, uint8_t* v_cache) {
  int latent = (v_new == NULL);
  if (!kv_args_ok(num_tokens, hkv, dk, dv, s, p, latent)) return -1;
  if (scale_mode == 1) {
    if (!k_scale || (!latent && !v_scale) || token_scale) return -1;
  } else if (scale_mode == 2) {
    if (!latent || hkv != 1 || !token_scale || k_scale || v_scale) return -1;
  } else {
    return -1;
  }
  if (latent != (v_cache == NULL)) return -1;
  int64_t nslots = (int64_t)p * s;
  for (int32_t t = 0; t < num_tokens; ++t) {
    int64_t slot = slot_mapping[t];
    if (slot < 0 || slot >= nslots) continue;
    int64_t page = slot / s;
    int32_t off = (int32_t)(slot % s);
    float tok_sc = 0.0f;
    if (scale_mode == 2) {
      float amax = 0.0f;
      for (int32_t d = 0; d < dk; ++d) {
        float a = fabsf(oracle_bf16_to_f32(k_new[(size_t)t * dk + d]));
        /* NaN inputs, quiet or signaling, are ignored (C's fmaxf would let a
         * signaling NaN reset the running maximum) */
        if (!isnan(a) && a > amax) amax = a;
      }
      tok_sc = (amax > 0.0f) ? amax / 448.0f : 1.0f;
      token_scale[slot] = tok_sc;
    }
    for (int32_t h = 0; h < hkv; ++h) {
      float ks = (scale_mode == 2) ? tok_sc : k_scale[h];
      for (int32_t d = 0; d < dk; ++d) {
        float x = oracle_bf16_to_f32(k_new[((size_t)t * hkv + h) * dk + d]);
        float y = x / ks;
        k_cache[k_index(page, h, off, d, hkv, dk, s)] = oracle_e4m3_encode(y);
      }
      if (!latent) {
        float vs = v_scale[h];
        for (int32_t d = 0; d < dv; ++d) {
          float x = oracle_bf16_to_f32(v_new[((size_t)t * hkv + h) * dv + d]);
          float y = x / vs;
          v_cache[v_index(page, h, off, d, hkv, dv, s)] =
              oracle_e4m3_encode(y);
        }
      }
    }
  }
  return 0;
}

int oracle_kv_write_bf16(const uint16_t* k_new, const uint16_t* v_new,
                         const int64_t* slot_mapping, int32_t num_tokens,
                         int32_t hkv, int32_t dk, int32_t dv, int32_t s,
                         int32_t p, uint16_t* k_cache, uint16_t* v_cache) {
  int latent = (v_new == NULL);
  if (!kv_args_ok(num_tokens, hkv, dk, dv, s, p, latent)) return -1;
  if (latent != (v_cache == NULL)) return -1;
  int64_t nslots = (int64_t)p * s;
  for (int32_t t = 0; t < num_tokens; ++t) {
    int64_t slot = slot_mapping[t];
    if (slot < 0 || slot >= nslots) continue;
    int64_t page = slot / s;
    int32_t off = (int32_t)(slot % s);
    for (int32_t h = 0; h < hkv; ++h) {
      for (int32_t d = 0; d < dk; ++d)
        k_cache[k_index(page, h, off, d, hkv, dk, s)] =
            k_new[((size_t)t * hkv + h) * dk + d];
      if (!latent)
        for (int32_t d = 0; d < dv; ++d)
          v_cache[v_index(page, h, off, d, hkv, dv, s)] =
              v_new[((size_t)t * hkv + h) * dv + d];
    }
  }
  return 0;
}

/* Page transcode BF16 -> FP8 between the prefill pool's BF16 cache and the
 * decode pool's FP8 cache ([SK] § "Kompresia sa oplatí inde pri vstupe a
 * inde pri výstupe"; [VN] § "Bộ nhớ đệm KV FP8 tăng gấp đôi dung lượng ngữ
 * cảnh"). Definition (the reading of include/pda.h): read each re-encoded
 * slot's BF16 rows back out of the source cache and write them with
 * oracle_kv_write_fp8 to the same slot of the destination page. */
int oracle_kv_transcode_bf16_to_fp8(
    const uint16_t* k_src, const uint16_t* v_src, const int32_t* src_pages,
    const int32_t* dst_pages, const int32_t* valid, int32_t num_pairs,
    int32_t hkv, int32_t dk, int32_t dv, int32_t s, int32_t src_num_pages,
    int32_t dst_num_pages, int32_t scale_mode, const float* k_scale,
    const float* v_scale, float* token_scale, uint8_t* k_dst,
    uint8_t* v_dst) {
  int latent = (v_src == NULL);
  if (num_pairs < 0 || src_num_pages <= 0) return -1;
  if (!kv_args_ok(num_pairs, hkv, dk, dv, s, dst_num_pages, latent)) return -1;
  if (latent != (v_dst == NULL)) return -1;
  uint16_t* krow = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)hkv * dk);
  uint16_t* vrow = latent ? NULL : (uint16_t*)malloc(sizeof(uint16_t) * (size_t)hkv * dv);
  int rc = 0;
  for (int32_t i = 0; i < num_pairs && rc == 0; ++i) {
    int32_t src = src_pages[i], dst = dst_pages[i], n = valid[i];
    if (src < 0 || src >= src_num_pages || dst < 0 || dst >= dst_num_pages ||
        n < 0 || n > s)
      continue;
    for (int32_t off = 0; off < n && rc == 0; ++off) {
      for (int32_t h = 0; h < hkv; ++h) {
        for (int32_t d = 0; d < dk; ++d)
          krow[(size_t)h * dk + d] = k_src[k_index(src, h, off, d, hkv, dk, s)];
        if (!latent)
          for (int32_t d = 0; d < dv; ++d)
            vrow[(size_t)h * dv + d] = v_src[v_index(src, h, off, d, hkv, dv, s)];
      }
      int64_t slot = (int64_t)dst * s + off;
      rc = oracle_kv_write_fp8(krow, vrow, &slot, 1, hkv, dk, dv, s,
                               dst_num_pages, scale_mode, k_scale, v_scale,
                               token_scale, k_dst, v_dst);
    }
  }
  free(krow);
  free(vrow);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Page-tag validation                                                       */
/* ------------------------------------------------------------------------ */

/* Each physical page carries a tag that changes when the page is handed out
 * again; a request records the pages and tags it expects and is aborted when
 * they no longer match ([VN] § "Bảo vệ bộ nhớ đệm dùng chung"; [DE]
 * § "Sicherheit gemeinsamer KV-Caches wird zum Produktionsthema"). */
void oracle_validate_page_tags(const uint32_t* page_tags, int32_t num_pages,
                               const int32_t* block_table,
                               const uint32_t* expected_tags,
                               int32_t max_blocks, const int32_t* seq_lens,
                               int32_t num_seqs, int32_t page_size,
                               int32_t* verdict) {
  for (int32_t s = 0; s < num_seqs; ++s) {
    int64_t len = seq_lens[s];
    if (len < 0 || len > (int64_t)max_blocks * page_size) {
      verdict[s] = -1;
      continue;
    }
    int64_t nblocks = (len + page_size - 1) / page_size;
    int32_t v = 0;
    for (int64_t j = 0; j < nblocks; ++j) {
      int32_t pg = block_table[(size_t)s * max_blocks + j];
      if (pg < 0 || pg >= num_pages ||
          page_tags[pg] != expected_tags[(size_t)s * max_blocks + j]) {
        v = (int32_t)(j + 1);
        break;
      }
    }
    verdict[s] = v;
  }
}

/* ------------------------------------------------------------------------ */
/* Attention                                                                 */
/* ------------------------------------------------------------------------ */

typedef struct {
  int32_t num_seqs, hq, hkv, dk, dv, s, p, max_blocks, kv_dtype, scale_mode,
      v_in_k;
  double sm_scale;
  const uint16_t* q;
  const void* k_cache;
  const void* v_cache;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* verdict;
  float* out;
  const int32_t* rows;
  int32_t n_rows;
  int32_t n_threads;
  int32_t tid;
} attn_job;

static double cache_value(const attn_job* J, int is_v, int64_t page,
                          int32_t head, int32_t off, int32_t d) {
  /* Latent caches: V is the first Dv dims of the K entry. */
  int from_k = !is_v || J->v_in_k;
  size_t idx = from_k ? k_index(page, head, off, d, J->hkv, J->dk, J->s)
                      : v_index(page, head, off, d, J->hkv, J->dv, J->s);
  const void* base = from_k ? J->k_cache : J->v_cache;
  if (J->kv_dtype == 0) return oracle_bf16_to_f32(((const uint16_t*)base)[idx]);
  double code_val = oracle_e4m3_decode(((const uint8_t*)base)[idx]);
  double scale;
  if (J->scale_mode == 2)
    scale = J->k_scale[page * J->s + off]; /* one scale per slot, K and V */
  else
    scale = from_k ? J->k_scale[head] : J->v_scale[head];
  return code_val * scale;
}

static void attn_row(const attn_job* J, int32_t sq, int32_t h) {
  float* o = J->out + ((size_t)sq * J->hq + h) * J->dv;
  int64_t len = J->seq_lens[sq];
  if (J->verdict && J->verdict[sq] != 0) {
    for (int32_t d = 0; d < J->dv; ++d) o[d] = 0.0f;
    return;
  }
  if (len < 0 || len > (int64_t)J->max_blocks * J->s) {
    for (int32_t d = 0; d < J->dv; ++d) o[d] = NAN;
    return;
  }
  if (len == 0) {
    for (int32_t d = 0; d < J->dv; ++d) o[d] = 0.0f;
    return;
  }
  int64_t nblocks = (len + J->s - 1) / J->s;
  const int32_t* bt = J->block_table + (size_t)sq * J->max_blocks;
  for (int64_t j = 0; j < nblocks; ++j) {
    if (bt[j] < 0 || bt[j] >= J->p) {
      for (int32_t d = 0; d < J->dv; ++d) o[d] = NAN;
      return;
    }
  }
  int32_t g = h / (J->hq / J->hkv);
  const uint16_t* qrow = J->q + ((size_t)sq * J->hq + h) * J->dk;
  double* z = (double*)malloc(sizeof(double) * (size_t)len);
  double* acc = (double*)calloc((size_t)J->dv, sizeof(double));
  /* pass 1: scores and their maximum */
  double zmax = -INFINITY;
  for (int64_t t = 0; t < len; ++t) {
    int64_t page = bt[t / J->s];
    int32_t off = (int32_t)(t % J->s);
    double dot = 0.0;
    for (int32_t d = 0; d < J->dk; ++d)
      dot += (double)oracle_bf16_to_f32(qrow[d]) *
             cache_value(J, 0, page, g, off, d);
    z[t] = J->sm_scale * dot;
    if (z[t] > zmax) zmax = z[t];
  }
  /* pass 2: weights, weighted sum of values, normalisation */
  double wsum = 0.0;
  for (int64_t t = 0; t < len; ++t) {
    int64_t page = bt[t / J->s];
    int32_t off = (int32_t)(t % J->s);
    double w = exp(z[t] - zmax);
    wsum += w;
    for (int32_t d = 0; d < J->dv; ++d)
      acc[d] += w * cache_value(J, 1, page, g, off, d);
  }
  for (int32_t d = 0; d < J->dv; ++d) o[d] = (float)(acc[d] / wsum);
  free(z);
  free(acc);
}

static void* attn_worker(void* arg) {
  const attn_job* J = (const attn_job*)arg;
  int64_t total = J->rows ? J->n_rows : (int64_t)J->num_seqs * J->hq;
  for (int64_t i = J->tid; i < total; i += J->n_threads) {
    int32_t sq, h;
    if (J->rows) {
      sq = J->rows[2 * i];
      h = J->rows[2 * i + 1];
    } else {
      sq = (int32_t)(i / J->hq);
      h = (int32_t)(i % J->hq);
    }
    attn_row(J, sq, h);
  }
  return NULL;
}

void oracle_paged_decode_attn(
    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim_qk, int32_t head_dim_v, int32_t page_size,
    int32_t num_pages, int32_t max_blocks_per_seq, int32_t kv_dtype,
    int32_t scale_mode, int32_t v_in_k, double sm_scale, const uint16_t* q,
    const void* k_cache, const void* v_cache, const float* k_scale,
    const float* v_scale, const int32_t* block_table, const int32_t* seq_lens,
    const int32_t* verdict, float* out, const int32_t* rows, int32_t n_rows,
    int32_t num_threads) {
  attn_job base = {num_seqs, num_q_heads, num_kv_heads, head_dim_qk,
                   head_dim_v, page_size, num_pages, max_blocks_per_seq,
                   kv_dtype, scale_mode, v_in_k, sm_scale, q, k_cache,
                   v_cache, k_scale, v_scale, block_table, seq_lens, verdict,
                   out, rows, n_rows, 1, 0};
  int32_t nt = num_threads > 0 ? num_threads : 1;
  if (nt == 1) {
    attn_worker(&base);
    return;
  }
  attn_job* jobs = (attn_job*)malloc(sizeof(attn_job) * (size_t)nt);
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nt);
  for (int32_t i = 0; i < nt; ++i) {
    jobs[i] = base;
    jobs[i].n_threads = nt;
    jobs[i].tid = i;
    pthread_create(&th[i], NULL, attn_worker, &jobs[i]);
  }
  for (int32_t i = 0; i < nt; ++i) pthread_join(th[i], NULL);
  free(jobs);
  free(th);
}

/* ---- INT4 weight-only GEMV: the definition, one output at a time ---- */

/* value of code j (0..7) of a packed word: bits 4j..4j+3 as two's complement */
static int int4_code(uint32_t word, int j) {
  int u = (int)((word >> (4 * j)) & 0xFu);
  return u >= 8 ? u - 16 : u;
}

int oracle_int4_gemv(const uint16_t* x, const uint32_t* w, const uint16_t* scale,
                     int32_t m, int32_t n, int32_t k, int32_t group,
                     const int32_t* cols, int32_t n_cols, double* y, double* yabs) {
  if (m < 0 || n < 0 || k < 0 || group <= 0 || k % group != 0 || k % 8 != 0) return -1;
  int32_t count = cols ? n_cols : n;
  for (int32_t ci = 0; ci < count; ++ci) {
    int32_t c = cols ? cols[ci] : ci;
    if (c < 0 || c >= n) return -1;
    for (int32_t i = 0; i < m; ++i) {
      double acc = 0.0, aabs = 0.0;
      for (int32_t kk = 0; kk < k; ++kk) {
        uint32_t word = w[(size_t)c * (k / 8) + kk / 8];
        double wv = (double)int4_code(word, kk % 8) *
                    (double)oracle_bf16_to_f32(scale[(size_t)c * (k / group) + kk / group]);
        double t = (double)oracle_bf16_to_f32(x[(size_t)i * k + kk]) * wv;
        acc += t;
        aabs += fabs(t);
      }
      y[(size_t)i * n + c] = acc;
      yabs[(size_t)i * n + c] = aabs;
    }
  }
  return 0;
}
