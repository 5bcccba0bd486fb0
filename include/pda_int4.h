/*
 * pda_int4.h — weight-only INT4 GEMV for the decode phase, part of libpda.so.
 *
 * The pages report that INT4 weights (from FP8) make decode faster, since
 * each generated token streams the weights from HBM and fewer bytes move,
 * while prefill, compute-bound, gets slower from the unpacking; hence INT4
 * weights for decode next to the FP8 KV cache (aifeed.sk, "Cloudflare
 * zrýchľuje inferenciu modelov Kimi a GLM kompresiou cache a váh", section
 * "Kompresia sa oplatí inde pri vstupe a inde pri výstupe"; the German page
 * "Cloudflare: Kleinere Modellbereitstellung senkt Speicherbedarf, doch
 * Sicherheit wird zum Prüfstein" (remio.ai), section "GLM-
 * Gewichtskomprimierung verschiebt den Phasen-Trade-off"). The pages fix no
 * format. The one taken here: signed two's-complement 4-bit codes with one
 * scale per 128 consecutive inputs of each output row.
 */
#ifndef PDA_INT4_H
#define PDA_INT4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * int4_gemv_bf16 — y[i][c] = sum_kk x[i][kk] * q[c][kk] * scale[c][kk / 128]
 *  x      device bf16 [m][k], 16-byte aligned (activations of m tokens).
 *  w      device uint32 [n][k / 8], 16-byte aligned: code j (bits 4j..4j+3,
 *         two's complement, -8..7) of word kk / 8 of row c is q[c][kk] for
 *         kk = 8 * word + j.
 *  scale  device bf16 [n][k / 128], 2-byte aligned.
 *  m, n, k  tokens, output rows, inputs; k a multiple of 128.
 *  group  must be 128 (the scale group length).
 *  y      device fp32 [m][n], 4-byte aligned; written, never read.
 * Arithmetic: the codes enter as bf16 values q + 136 (exact) and the 136
 * offset is subtracted per 128-input group in fp32; one token runs on bf16
 * dot-product pairs, two and more on 16x16x32 bf16 matrix-core products,
 * both with fp32 accumulation. The result differs from the exact sum by at
 * most 8192 * 2^-24 * sum_kk |x[i][kk]| * |scale[c][kk / 128]|.
 * Asynchronous on `stream`; nothing is allocated. Returns 0,
 * PDA_ERR_INVALID_ARG (1) for negative sizes, NULL or misaligned pointers,
 * PDA_ERR_UNSUPPORTED (2) for group != 128, k not a positive multiple of 128
 * (k == 0 with m, n > 0 included) or more than 2097120 tokens (65535
 * grid rows of 32 tokens), PDA_ERR_LAUNCH
 * (3) on a launch failure. m == 0 or n == 0 does nothing.
 */
int int4_gemv_bf16(const void* x, const uint32_t* w, const void* scale, int32_t m, int32_t n,
                   int32_t k, int32_t group, float* y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PDA_INT4_H */
