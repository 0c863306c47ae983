/*
 * stream_ceiling.h - C ABI of the streaming-ceiling kernels (libstream_ceiling.so).
 *
 * Measurement only, not part of the all-reduce path. One call reads n_in
 * buffers and writes n_out buffers of the same size once each, with plain
 * streaming code: a workgroup of `lanes` lanes covering lanes x packs 16-byte
 * packs of every buffer per step, consecutive steps on consecutive
 * workgroups. Loads are 16-byte non-temporal global loads, or (the *_BL
 * shapes) 16-byte non-temporal buffer loads from the step's start address.
 * Stores are 16-byte non-temporal global stores, or (the *_SC1 shapes)
 * 16-byte buffer stores at device scope (cache-policy field sc1, temporal).
 * Timing it in each shape on the very buffers an all-reduce call uses (same
 * sizes, same addresses, same numbers of read and write streams) and keeping
 * the fastest gives the practical HBM ceiling of that call, next to the
 * 8 TB/s peak. No one shape, load form or store form is fastest for every mix
 * of streams.
 *
 * What it computes, per 16-byte pack i:
 *     x = in[0][i] ^ in[1][i] ^ ... ^ in[n_in-1][i]      (bitwise, as 4 x u32)
 *     out[k][i] = x for every k < n_out
 * With n_out = 0 nothing is written; the loads are kept by an empty asm
 * statement that consumes x.
 *
 * Arguments: `in` and `out` are host arrays of device pointers (the caller
 * owns every buffer); `bytes` is the size of each buffer; `shape` is an
 * SC_SHAPE_* value. Outputs may not overlap inputs or each other (not
 * checked). The call is asynchronous on `hip_stream` (NULL = default stream)
 * of the current device.
 *
 * Returns SC_OK, or a negative SC_ERR_* code without launching anything.
 */
#ifndef STREAM_CEILING_H
#define STREAM_CEILING_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SC_MAX_IN 12
#define SC_MAX_OUT 2

/* Workgroup shapes: lanes x packs per lane per step (0-3), plus SC_SHAPE_SC1
 * for device-scope buffer stores and SC_SHAPE_BL for buffer loads. */
enum {
    SC_SHAPE_512x2 = 0,
    SC_SHAPE_256x4 = 1,
    SC_SHAPE_256x8 = 2,
    SC_SHAPE_128x8 = 3,
    SC_SHAPE_SC1 = 4,
    SC_SHAPE_BL = 8,
    SC_SHAPE_512x2_SC1 = 4,
    SC_SHAPE_256x4_SC1 = 5,
    SC_SHAPE_256x8_SC1 = 6,
    SC_SHAPE_128x8_SC1 = 7,
    SC_NUM_SHAPES = 16
};

enum {
    SC_OK = 0,
    SC_ERR_COUNT = -1, /* n_in outside 1..SC_MAX_IN or n_out outside 0..SC_MAX_OUT    */
    SC_ERR_NULL = -2,  /* in or out array, or one of its first n pointers, is NULL     */
    SC_ERR_ALIGN = -3, /* a pointer not 16-byte aligned, or bytes not a multiple of 16 */
    SC_ERR_SHAPE = -4, /* shape outside 0..SC_NUM_SHAPES-1                             */
    SC_ERR_HIP = -100  /* the launch failed                                             */
};

int32_t sc_stream(const void *const *in, int32_t n_in, void *const *out, int32_t n_out, size_t bytes,
                  int32_t shape, void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* STREAM_CEILING_H */
