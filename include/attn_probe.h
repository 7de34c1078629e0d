/*
 * attn_probe.h -- measurement aids shipped with the decode-attention library.
 *
 * They are not part of the attention path; the benchmark uses them to report
 * the achievable HBM read rate next to the datasheet peak, and to calibrate
 * the hardware byte counters against a copy of known size.  Pointers are
 * device pointers owned by the caller; calls only enqueue on `stream`.
 * Return 0 on success, -1 for a NULL pointer, -7 for a size or pointer not a
 * multiple of 16 bytes, -8 when the launch fails.
 */
#ifndef ATTN_PROBE_H
#define ATTN_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` from `src` once with 16-byte streaming loads and discard the
 * data (`sink`, 4 bytes, is written only in a practically impossible case).
 * `blocks` <= 0 picks 8 work groups of 256 lanes per compute unit. */
int attn_probe_read(const void* src, size_t bytes, uint32_t* sink, int blocks,
                    void* stream);

/* dst[0:bytes] = src[0:bytes] with 16-byte loads and stores. */
int attn_probe_copy(void* dst, const void* src, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_PROBE_H */
