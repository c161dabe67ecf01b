/* hq_diag.h -- measurement helpers of libhyquant (not steps of the method).
 *
 * They exist so that a kernel's achieved HBM rate can be compared with the
 * rate this GPU reaches for the same access pattern, not only with the
 * specification peak. Conventions as in hq.h: device pointers, asynchronous
 * on `stream`, host-side validation with nothing enqueued on error. */
#ifndef HQ_DIAG_H_
#define HQ_DIAG_H_

#include <stddef.h>
#include <stdint.h>

#include "hq.h"

#ifdef __cplusplus
extern "C" {
#endif

/* hq_diag_read_int4 -- read the INT4 store of `cache` (K and V codes, K and V
 * scale/zero of the n_q quantized tokens of every (b, g)) exactly as
 * hq_decode_attn's INT4 workgroups read it: the same splits (those of a
 * decode with up to four query heads per KV head), 64-token tiles, 128-bit
 * loads with the non-temporal hint and two tiles in flight per wave; nothing is
 * computed but an
 * XOR of the loaded words, written to `sink` (one word per thread, so the
 * loads cannot be dropped). The bytes read are 160 per quantized
 * token-head; the call's time gives the achievable streaming-read rate of
 * that pattern.
 *   sink  device buffer of hq_diag_read_int4_sink_bytes(cache) bytes; its
 *         contents are meaningless. Errors as for hq_decode_attn's cache
 *         argument; HQ_ERR_CAPACITY if sink_bytes is too small. */
hq_status hq_diag_read_int4(const hq_cache* cache, void* sink, size_t sink_bytes, void* stream);
size_t hq_diag_read_int4_sink_bytes(const hq_cache* cache);

/* hq_diag_exp2_error -- accuracy of the hardware base-2 exponential
 * (v_exp_f32) that the probe's first pass takes 2^f with, |f| <= 1/2 (the
 * probe's score bound in hq_probe_select's kernel source counts its largest
 * relative error there). Evaluates it on every fp32 value x in [lo, hi] and
 * compares with the fp64 exponential 2^x: out[i], i < out_count, receives the
 * largest |v_exp_f32(x) - 2^x| / 2^x seen by workgroup i (the grid has
 * out_count workgroups, which split the inputs between them); the answer is
 * the largest of the out_count values.
 *   lo, hi     finite, -64 <= lo <= hi <= 64 (results stay normal fp32);
 *   out        device buffer of out_count doubles, out_count in [1, 65536].
 * Errors: HQ_ERR_INVALID_ARG for a range or count outside these limits or a
 * null out, with nothing enqueued. */
hq_status hq_diag_exp2_error(float lo, float hi, double* out, size_t out_count, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HQ_DIAG_H_ */
