/*
 * wf_stream_copy.h - reference copy for bandwidth measurement.
 *
 * Not part of the attention path (wf_chunk_attn.h): a plain device copy in the
 * shape that moves a few tens of MB fastest, whose rate over the bytes of one
 * KV append is what a single kernel moving that many bytes reaches, launch and
 * ramp included.  The append's bandwidth is reported against it.  Same status
 * codes and wf_last_error() as the attention library, which exports it.
 */
#ifndef WF_STREAM_COPY_H
#define WF_STREAM_COPY_H

#include "wf_chunk_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Measurement aid, not part of the attention path: copy `bytes` bytes from
 * src to dst (device pointers) on `stream` with a plain streaming copy kernel
 * (persistent grid, nontemporal 16-byte loads and stores).  Its rate over the
 * bytes of one append is the reference the append's bandwidth is compared
 * with: what a single kernel moving that many bytes reaches.  Requires bytes a
 * multiple of 16, src and dst 16-byte aligned and not overlapping
 * (WF_ERR_INVALID_ARG otherwise, nothing enqueued); bytes == 0 is a no-op.
 */
wf_status wf_stream_copy(const void *src, void *dst, uint64_t bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* WF_STREAM_COPY_H */
