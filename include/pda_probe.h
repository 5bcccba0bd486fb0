/*
 * pda_probe.h — a measurement aid of libpda.so, not part of the decode path:
 * a read-only HBM bandwidth probe that gives the measured ceiling the
 * kernels' bandwidth is reported against, next to the 8 TB/s figure.
 */
#ifndef PDA_PROBE_H
#define PDA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * pda_hbm_read_probe — read every byte of a device buffer once.
 *  buf          device buffer of `bytes` bytes, 16-byte aligned; bytes a
 *               multiple of 16 KiB (the block one wave reads per step) and
 *               of chunk_bytes.
 *  chunk_bytes  0: one streaming pass in address order. Else a power of two
 *               in [256, 65536]: the buffer is read as chunks of that size
 *               in a scrambled order (chunk i -> (i * 0x9E3779B1) mod the
 *               chunk count, which must then be a power of two), the access
 *               pattern of paged caches.
 *  sink         device uint32 [gridDim] receiving an XOR of the data read
 *               (keeps the loads alive); its size is returned by
 *               pda_hbm_read_probe_sink_words.
 * Asynchronous on `stream`; returns PDA_ERR_INVALID_ARG (1) for bad
 * arguments, PDA_ERR_LAUNCH (3) on a launch failure, else 0.
 */
size_t pda_hbm_read_probe_sink_words(void);
int pda_hbm_read_probe(const void* buf, size_t bytes, int32_t chunk_bytes, uint32_t* sink,
                       void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PDA_PROBE_H */
