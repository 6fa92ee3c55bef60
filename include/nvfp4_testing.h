/*
 * nvfp4_testing.h — testing hooks of the NVFP4 library (not for production
 * use; declared apart from the interface in nvfp4.h).
 */
#ifndef NVFP4_TESTING_H
#define NVFP4_TESTING_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Process-wide: the single-launch quantiser's bounded wait for the other
 * workgroups' maxima, in ticks of the GPU's 100 MHz real-time counter (default
 * 100000 = 1 ms).  Returns the previous value.  With 0, each workgroup waits
 * for at most one poll of the other workgroups' slots and reads the shares of
 * those it has not heard from itself; the bytes written are the same either
 * way.  Affects launches made after the call.  This exercises, from the host,
 * the path a workgroup takes when the grid is not resident all at once.
 */
uint64_t nvfp4_testing_set_quantize_wait(uint64_t ticks);

/*
 * Process-wide, not thread-safe: per-launch timing for benchmarks.  The next
 * `count` launch steps of the library's calls each record one event of
 * `events` (hipEvent_t values passed as void*, in order) on the call's stream
 * right after the step's launch.  A launch step is one kernel launch, except
 * that a quantisation too large for the single-launch kernel may take two
 * (both before its event).  nvfp4_linear_q, for example, has three steps: the
 * activation quantiser, the GEMM and the encoder of the output.  The list
 * must stay valid until `count` events are recorded; count 0 clears it.
 * Returns 0, or 1 (NVFP4_EINVAL) for count < 0 or a NULL list with count > 0.
 */
int nvfp4_testing_set_launch_events(void *const *events, int count);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_TESTING_H */
