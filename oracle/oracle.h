/*
 * oracle.h — plain CPU oracle for the FP8 paged decode-attention path.
 *
 * TEST INFRASTRUCTURE ONLY. Only tests/, the smoke check and the CPU-baseline
 * leg of the benchmark may load this library. It shares no code with the GPU
 * path: its own e4m3 codec, its own BF16 decode, its own reading of the cache
 * format, and the plain definitions of every step (dense two-pass softmax in
 * fp64, no paging order, no online softmax, no split).
 *
 * Page citations (four web pages on Cloudflare's serving of Kimi K2.6 and
 * GLM 5.2; same keys as include/pda.h):
 *   [SK] aifeed.sk, "Cloudflare zrýchľuje inferenciu modelov Kimi a GLM
 *        kompresiou cache a váh"
 *   [VN] manulx.blog, "Công thức của Cloudflare để phục vụ Kimi và GLM: ..."
 *   [DE] remio.ai, "Cloudflare: Kleinere Modellbereitstellung senkt
 *        Speicherbedarf, doch Sicherheit wird zum Prüfstein"
 *   [JA] agentlenshq.com, "Cloudflare Workers AI: Kimi および GLM の推論を
 *        大規模に最適化する"
 * The pages name the format ("e4m3") but not its rounding, saturation or
 * scaling; the readings taken here are listed with each function.
 *
 * Parity pins: every function below is pinned by CPU tests against closed
 * forms, brute force or invariants (tests/test_oracle_*.py); none is
 * "parity unpinned".
 */
#ifndef PDA_ORACLE_H
#define PDA_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* --- OCP FP8 E4M3 codec --------------------------------------------------
 * Reading of [SK] § "Dve odlišné úzke miesta v pamäti GPU" / [JA] § "並行性を
 * 高めるための KV キャッシュ量子化" ("FP8, e4m3"): the OCP 8-bit floating point
 * E4M3 format — sign, 4 exponent bits with bias 7, 3 mantissa bits, no
 * infinities, NaN = S.1111.111, largest finite 448. */
double oracle_e4m3_decode(uint8_t code);          /* NaN for 0x7F / 0xFF   */
/* Definition: NaN -> 0x7F|sign; |x| >= 448 (incl. inf) -> 0x7E|sign; else the
 * non-negative finite code nearest to |x| by exact comparison, ties to the
 * even code, then the sign bit of x is ORed in (so -0 and negative underflow
 * give 0x80). */
uint8_t oracle_e4m3_encode(float x);
/* The same definition computed by a scan over all 127 candidates (the form
 * the definition states); oracle_e4m3_encode finds the same code by bisection
 * over the increasing code values and is checked against this one. */
uint8_t oracle_e4m3_encode_brute(float x);
/* Closed-form bit-level encoder; a cross-check of oracle_e4m3_encode only. */
uint8_t oracle_e4m3_encode_closed(float x);
float oracle_bf16_to_f32(uint16_t bits);

/* --- KV write (quantise + scatter) ----------------------------------------
 * Same argument meaning as kv_write_fp8 / kv_write_bf16 in include/pda.h,
 * with host arrays. Returns 0, or -1 for arguments the GPU call rejects. */
int oracle_kv_write_fp8(const uint16_t* k_new, const uint16_t* v_new,
                        const int64_t* slot_mapping, int32_t num_tokens,
                        int32_t num_kv_heads, int32_t head_dim_k,
                        int32_t head_dim_v, int32_t page_size,
                        int32_t num_pages, int32_t scale_mode,
                        const float* k_scale, const float* v_scale,
                        float* token_scale, uint8_t* k_cache,
                        uint8_t* v_cache);
int oracle_kv_write_bf16(const uint16_t* k_new, const uint16_t* v_new,
                         const int64_t* slot_mapping, int32_t num_tokens,
                         int32_t num_kv_heads, int32_t head_dim_k,
                         int32_t head_dim_v, int32_t page_size,
                         int32_t num_pages, uint16_t* k_cache,
                         uint16_t* v_cache);

/* Page transcode: same argument meaning as kv_transcode_bf16_to_fp8 in
 * include/pda.h, with host arrays. Returns 0, or -1 for arguments the GPU
 * call rejects. */
int oracle_kv_transcode_bf16_to_fp8(
    const uint16_t* k_src, const uint16_t* v_src, const int32_t* src_pages,
    const int32_t* dst_pages, const int32_t* valid, int32_t num_pairs,
    int32_t num_kv_heads, int32_t head_dim_k, int32_t head_dim_v,
    int32_t page_size, int32_t src_num_pages, int32_t dst_num_pages,
    int32_t scale_mode, const float* k_scale, const float* v_scale,
    float* token_scale, uint8_t* k_dst, uint8_t* v_dst);

/* --- page-tag validation --------------------------------------------------
 * Verdict per sequence exactly as validate_page_tags documents it. */
void oracle_validate_page_tags(const uint32_t* page_tags, int32_t num_pages,
                               const int32_t* block_table,
                               const uint32_t* expected_tags,
                               int32_t max_blocks_per_seq,
                               const int32_t* seq_lens, int32_t num_seqs,
                               int32_t page_size, int32_t* verdict);

/* --- attention ------------------------------------------------------------
 * Dense two-pass softmax attention in fp64 over the dequantised cache
 * contents of each sequence, rounded once to fp32.
 *   kv_dtype 0 = BF16 caches (uint16 elements), 1 = FP8 (uint8 elements).
 *   scale_mode 0 none, 1 per head (k_scale, v_scale [Hkv]),
 *              2 per token (k_scale = token_scale[P*S], V uses it too).
 *   verdict may be NULL (no tracker).
 *   rows: optional list of n_rows (s, h) pairs (2*n_rows int32) to compute;
 *   NULL computes every row. Rows not listed are left untouched.
 *   num_threads: worker threads (<= 0: 1).
 * Aborted sequences (verdict != 0) and len == 0 give zero rows; a malformed
 * length or an out-of-range page id gives NaN rows. */
void oracle_paged_decode_attn(
    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim_qk, int32_t head_dim_v, int32_t page_size,
    int32_t num_pages, int32_t max_blocks_per_seq, int32_t kv_dtype,
    int32_t scale_mode, int32_t v_in_k, double sm_scale, const uint16_t* q,
    const void* k_cache, const void* v_cache, const float* k_scale,
    const float* v_scale, const int32_t* block_table, const int32_t* seq_lens,
    const int32_t* verdict, float* out, const int32_t* rows, int32_t n_rows,
    int32_t num_threads);

/* --- INT4 weight-only decode GEMV ------------------------------------------
 * The pages report INT4 weights for the decode phase, where the weights are
 * streamed from memory for every generated token (aifeed.sk, "Cloudflare
 * zrýchľuje inferenciu modelov Kimi a GLM kompresiou cache a váh", section
 * "Kompresia sa oplatí inde pri vstupe a inde pri výstupe"; the German page
 * "Cloudflare: Kleinere Modellbereitstellung senkt Speicherbedarf, doch
 * Sicherheit wird zum Prüfstein" (remio.ai), section "GLM-
 * Gewichtskomprimierung verschiebt den Phasen-Trade-off"). They fix no
 * format; the reading taken here: weight W[n][kk] = q[n][kk] * scale[n][kk/G]
 * with q a signed two's-complement 4-bit code, eight codes per uint32 word
 * along kk (code j of word w is element kk = 8w + j, in bits 4j..4j+3),
 * w[n][k/8]; scale bf16 [n][k/G]; x bf16 [m][k].
 *   y[i][c]    = sum_kk x[i][kk] * W[c][kk]         (fp64, plain loop)
 *   yabs[i][c] = sum_kk |x[i][kk] * W[c][kk]|       (for error bounds)
 * cols: optional list of n_cols output columns to compute (NULL: all n);
 * y and yabs are [m][n] and only the listed columns are written.
 * Returns 0, or -1 for k not a multiple of G or of 8, G <= 0, m, n < 0. */
int oracle_int4_gemv(const uint16_t* x, const uint32_t* w, const uint16_t* scale,
                     int32_t m, int32_t n, int32_t k, int32_t group,
                     const int32_t* cols, int32_t n_cols, double* y, double* yabs);

#ifdef __cplusplus
}
#endif

#endif /* PDA_ORACLE_H */
