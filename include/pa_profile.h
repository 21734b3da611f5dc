/*
 * pa_profile.h -- optional per-kernel timing of libpa.so with HIP events.
 *
 * For benchmarks and tracing only; not part of the attention ABI in pa.h.
 * While profiling is on, the library records a pair of HIP events on the
 * launch stream around each of its kernel launches. Off by default; when off,
 * no event is created or recorded.
 *
 * Kernel ids: 0 KV write, 1 decode (split-K partitions), 2 partition reduce,
 * 3 prefill plan, 4 chunked prefill (which also combines the decode's
 * partitions when it runs after the decode on the launch stream), 5 KV write
 * and plan in one launch (steps whose prefill runs after the decode), 6 the
 * decode's work order (ahead of decode launches of more than one round of
 * workgroups).
 */
#ifndef PA_PROFILE_H_
#define PA_PROFILE_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_PROFILE_KERNELS 7

/* Drop earlier records and start recording. Returns 0 (PA_OK). */
int pa_profile_start(void);

/* Stop recording (records are kept until the next start). Returns 0. */
int pa_profile_stop(void);

/* Wait for the recorded events of kernel `id` and report the summed
 * launch-to-completion time in milliseconds and the number of launches.
 * Returns 0, or PA_ERR_SHAPE (3) for an unknown id, PA_ERR_HIP (7) if a HIP
 * event call fails. Outputs may be NULL. */
int pa_profile_kernel(int id, double* total_ms, int64_t* launches);

/* Name of kernel `id` ("" for an unknown id). */
const char* pa_profile_kernel_name(int id);

/* Launch, on `stream` (a hipStream_t), one read of every byte of the device
 * buffer `buf` with non-temporal 16-byte loads, as the decode reads K/V;
 * nothing is written. Time it with events around the call to measure the
 * GPU's sustained read bandwidth. `buf` 16-byte aligned, `bytes` a multiple
 * of 16. Returns 0, PA_ERR_SHAPE (3) for a bad buffer, PA_ERR_HIP (7) if the
 * launch fails. */
int pa_profile_read_probe(const void* buf, uint64_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_PROFILE_H_ */
