/*
 * awq_probe.h -- measurement aid exported by the same library as awq.h, not
 * part of the layer's interface.
 *
 * The pages tie decode speed to memory bandwidth ("Applied LLM Quantisation
 * Sagemaker", section "How does it help?": fewer bits per weight, less memory
 * to move; the TensorRT-LLM news page quotes the H200's HBM bandwidth beside
 * its Falcon-180B result). A weight-streaming launch is therefore compared
 * with the rate a plain read of the same number of bytes reaches on the same
 * GPU, which includes the launch and first-data latency a kernel of that size
 * cannot avoid.
 */
#ifndef AWQ_MI355X_AWQ_PROBE_H
#define AWQ_MI355X_AWQ_PROBE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * A plain streaming read of `bytes` bytes (a multiple of 16) at device
 * address `buf` (16-byte aligned) with 16-byte loads. The 16 bytes at device
 * address `sink` (16-byte aligned) may receive a value derived from the data
 * (it keeps the loads live). `start_event` and `stop_event` are hipEvent_t
 * handles (either may be NULL) recorded at the start and end of the kernel.
 * Returns AWQ_OK, AWQ_ERR_NULL, AWQ_ERR_SHAPE (bytes % 16), AWQ_ERR_ALIGN or
 * AWQ_ERR_HIP (awq.h); bytes == 0 launches nothing.
 */
int awq_stream_read(const void* buf, size_t bytes, void* sink, void* stream,
                    void* start_event, void* stop_event);

#ifdef __cplusplus
}
#endif

#endif /* AWQ_MI355X_AWQ_PROBE_H */
