/*
 * kvrope_probes.h -- measurement helpers of libkvrope_probes.so.  NOT part of the
 * attention path and not in libkvrope.so: a benchmark uses them to report the ceilings
 * the box actually reaches beside the spec peaks, and the host tests use the kernels'
 * f16 rounding compiled for the host.
 *
 * All pointers are DEVICE pointers except where stated; every launch is asynchronous on
 * `stream` (a hipStream_t; NULL = the null stream).  Return values are the status codes
 * of kvrope.h: ATTN_OK, ATTN_ERR_NULL, ATTN_ERR_SHAPE, ATTN_ERR_CAPACITY, ATTN_ERR_HIP.
 * None of the kernels writes anything in practice: each folds what it read or computed
 * into one word and stores it to `sink` only when it equals a value no input produces.
 */
#ifndef KVROPE_PROBES_H
#define KVROPE_PROBES_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* kvprobe_read -- the plain HBM read ceiling: `blocks` workgroups of 256 threads read
 * `bytes` (a multiple of 16) of `buf` once, front to back, with 16-byte lane loads, each
 * workgroup 32 KB at a time (eight loads per lane in flight) in a grid-stride loop.
 * sink: >= 4 bytes. */
int kvprobe_read(const void *buf, size_t bytes, int blocks, void *sink, void *stream);

/* kvprobe_stream -- reads, and only reads, the cache rows a decode step reads: rows
 * [0, lens[u]] of K and V of every (unit, KV head) (caches [n, hkv, s_cap, d], lens
 * device int32 [n]), one workgroup per chunk, a unit's rows cut as attn_decode cuts them
 * for chunk = attn_decode_chunk_keys(...) (the fewest chunks of at most `chunk` rows, of
 * equal size rounded up to 32), 16-byte lane loads.  Its time is the streaming ceiling of that access pattern.
 * Requires max_len + 1 <= s_cap (every lens[u] <= max_len); a row past s_cap is never
 * read.  sink: >= 4 bytes. */
int kvprobe_stream(const void *cache_k, const void *cache_v, const int32_t *lens, int n, int hkv,
                   int s_cap, int d, int max_len, int chunk, void *sink, void *stream);

/* kvprobe_mfma -- `blocks` workgroups of 4 waves; each wave runs `iters` rounds of four
 * independent v_mfma_f32_32x32x16_f16 chains (32 x 32 x 16 x 2 FLOPs each).  sink
 * (>= 32 * (blocks + 1) bytes): for workgroup b, sink[4 + 4b .. 4b + 7] as uint64 = the
 * 100 MHz real-time counter at start and end, the shader-clock counter at start and end;
 * their ratio gives the clock the matrix cores ran at. */
int kvprobe_mfma(int blocks, int iters, void *sink, void *stream);

/* The fp64 -> f16 (nearest, ties to even) conversion the kernels apply to every rotated
 * K value, compiled for the host (no GPU needed). */
uint16_t kvprobe_f64_to_f16(double x);

#ifdef __cplusplus
}
#endif

#endif /* KVROPE_PROBES_H */
