/*
 * kvq_measure.h -- measurement aids of libkvq, beside the decode path.
 *
 * None of these calls is part of quantise-append or decode attention.  They
 * exist so that a caller can time the decode split kernel and set its rate
 * against the device's own read ceilings: decode moves the whole cache
 * through HBM for every generated token, so its bytes per second against
 * what the memory system delivers is the figure of merit (encorp.ai, "KV
 * cache compression is an infrastructure decision, not a model debate",
 * section on the HBM ceiling).
 *
 * Conventions (status codes, device pointers, streams) are those of kvq.h.
 */
#ifndef KVQ_MEASURE_H
#define KVQ_MEASURE_H

#include "kvq.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Timing hook.  While start_event / stop_event (hipEvent_t handles created
 * by the caller; either may be NULL) are set, every decode split kernel that
 * a kvq call on this thread launches records them at its own start and end
 * (hipExtLaunchKernel's kernel events: no extra packets on the stream, so the
 * elapsed time is the kernel's execution time).  kvq_set_split_kernel_events
 * (NULL, NULL) clears the hook.  Always returns KVQ_OK. */
kvq_status kvq_set_split_kernel_events(void *start_event, void *stop_event);

/* Measurement aid, not part of the decode path: one launch that reads
 * `bytes` of device memory from `buffer` front to back (16-byte loads, two
 * work-groups of 256 lanes per compute unit, grid-stride), so that a caller
 * can time the plain streaming-read rate of the device the decode runs on
 * and set the decode's bytes per second against it (decode moves the whole
 * cache through HBM per token (encorp.ai, section on the HBM ceiling)).
 *   buffer  (device) 16-byte aligned; bytes a positive multiple of 16
 *           (at most 2^40; else KVQ_ERR_SHAPE).
 *   sink    (device) one uint32, written only in the rare case that the
 *           XOR of everything read equals a fixed constant (it keeps the
 *           loads from being optimised away); may hold anything.
 * Nothing is allocated; the call is enqueued on `stream`. */
kvq_status kvq_stream_read_probe(const void *buffer, size_t bytes, uint32_t *sink, void *stream);

/* Measurement aid, not part of the decode path: one launch that reads the
 * bytes a decode split kernel reads for these arguments, in the same work
 * decomposition, and does nothing else.  Work-group (split, KV head,
 * sequence); 4 waves; wave w walks page pairs w, w + 4, ... of its split,
 * with the page ids that block_tables gives; each 16-token region of the
 * KV head is read whole (16-byte loads).  Timing it beside the decode sets
 * the decode against the cost of its own access pattern: random page
 * regions of a few KB rather than a sequential stream (encorp.ai, section on the HBM ceiling).
 *   fmt      (host) a quantised format with 16-token pages
 *            (else KVQ_ERR_UNSUPPORTED).
 *   cache, block_tables, seq_lens, num_pages, max_pages_per_seq, num_seqs,
 *   num_kv_heads, max_seq_len: as for kvq_decode_attention (the same
 *            preconditions on the device-resident arguments).
 *   pages_per_split  even, 2..512: the decode's split size
 *            (kvq_decode_pages_per_split gives the heuristic's).
 *   sink     (device) one uint32, written only in the rare case that the
 *            XOR of everything read equals a fixed constant; may hold
 *            anything.
 * Errors: KVQ_ERR_NULL, KVQ_ERR_SHAPE (sizes as above, or more than 65535
 * splits), KVQ_ERR_ALIGN (cache 16 bytes; block_tables, seq_lens and sink
 * 4 bytes), KVQ_ERR_HIP.  Nothing is allocated; the call is enqueued on
 * `stream`. */
kvq_status kvq_page_walk_probe(const kvq_format *fmt, const uint8_t *cache, int64_t num_pages,
                               const int32_t *block_tables, int32_t max_pages_per_seq, const int32_t *seq_lens,
                               int32_t num_seqs, int32_t num_kv_heads, int32_t max_seq_len,
                               int32_t pages_per_split, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_MEASURE_H */
