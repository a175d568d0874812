/*
 * cce_profile.h -- opt-in per-kernel timing of libcce (diagnostics only).
 *
 * For callers that measure the library's kernels against a roofline: while
 * profiling is on, every kernel that cce_forward / cce_backward launch is
 * bracketed by two hipEvents recorded on the caller's stream.  Profiling is
 * off by default and then costs nothing; turning it on makes the calls create
 * events (host-side objects) and is not meant for production loops.
 */
#ifndef LIBCCE_CCE_PROFILE_H
#define LIBCCE_CCE_PROFILE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct cce_kernel_time {
  char name[32];     /* kernel family, e.g. "tile_bwd", "dh_gemm" */
  int64_t launches;  /* launches recorded since the last read */
  double total_ms;   /* summed event-to-event time of those launches */
} cce_kernel_time;

/* Turn profiling on (1) or off (0); returns the previous state.  Process-wide. */
int cce_profile_enable(int on);

/*
 * Wait for every recorded launch, fill up to `max` entries (one per kernel
 * family seen), release the events and clear the record.  Returns the number
 * of entries written, or -1 on a HIP error.
 */
int cce_profile_read(cce_kernel_time *out, int max);

#ifdef __cplusplus
}
#endif

#endif /* LIBCCE_CCE_PROFILE_H */
