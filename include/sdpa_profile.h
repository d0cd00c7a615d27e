/*
 * sdpa_profile.h - optional per-kernel launch timing of libsdpa (tracing aid).
 *
 * When enabled, the library records a pair of hipEvents on the launching stream around
 * every kernel it launches (forward, backward pre-pass, dK/dV, dQ, merge, THD scheduler)
 * and can report the summed GPU time per kernel.  Disabled by default; when disabled the
 * launch path does nothing extra.  Events come from a pool the library keeps for the life
 * of the process; no device memory is allocated.  Meant for one host thread at a time.
 */
#ifndef SDPA_MI355X_PROFILE_H
#define SDPA_MI355X_PROFILE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* on = 1: clear the record table and start recording; on = 0: stop recording (the table
 * is kept for sdpa_profile_read).  Returns SDPA_OK. */
int sdpa_profile_enable(int on);

/* Wait for every recorded launch to finish and write one line per kernel,
 * "<kernel> <launches> <total_ms>\n", into buf (NUL-terminated, truncated to len).
 * Returns SDPA_OK, or SDPA_ERR_HIP if an event query fails. */
int sdpa_profile_read(char* buf, size_t len);

#ifdef __cplusplus
}
#endif

#endif /* SDPA_MI355X_PROFILE_H */
