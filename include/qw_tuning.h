/*
 * qw_tuning.h -- test and benchmark hooks of libqw (not needed by callers).
 *
 * Every entry point picks its kernel path, launch shape and work split by
 * itself from the shape of the call. These hooks force a choice the
 * automatic rule would not make, so that tests can run every kernel path
 * on the same inputs and compare them. A forced choice that does not apply
 * to a call (a path the shape does not fit, a part count that does not
 * divide it) is ignored for that call, which then takes the automatic
 * choice. Results under any setting stay within the same error bounds
 * (the exact bits may differ between paths, as the summation order does).
 *
 * The settings are process-wide and read at each call; change them only
 * while no other host thread is calling the library. Host only.
 */
#ifndef QW_TUNING_H_
#define QW_TUNING_H_

#include "qw.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  /* 2-bit GEMV kernel: -1 automatic, 0 the matrix-core kernel wherever it
   * takes the shape, 1 the vector-ALU kernel. */
  QW_TUNE_GEMV2_PATH = 1,
  /* 2-bit GEMV K parts (qgemv_2bit_ws with a workspace): -1 automatic,
   * n >= 2 forces n parts where n divides the 512-channel runs and every
   * part fits. */
  QW_TUNE_GEMV2_SPLIT = 2,
  /* 2-bit matrix-core GEMV register ring: -1 / 0 three slots, 1 the deep
   * ring (6 slots up to batch 2, 4 beyond). */
  QW_TUNE_GEMV2_DEEP_RING = 3,
  /* NF4 GEMV row ring: -1 / 0 three slots, 1 six slots. */
  QW_TUNE_NF4_DEEP_RING = 4,
  /* Prefill without anchors: -1 automatic, n >= 0 the number of 256-wide
   * column tiles (the rest runs as 128-wide tiles). */
  QW_TUNE_PREFILL_WIDE_TILES = 5,
  /* INT4 GEMV kernel: -1 / 0 the matrix-core kernel wherever it takes the
   * shape, 1 the vector-ALU kernel. */
  QW_TUNE_INT4_PATH = 6
} qw_tune_key;

#define QW_TUNE_AUTO (-1)

/* Sets a hook (QW_TUNE_AUTO restores the automatic choice). Errors:
 * INVALID_ARG for an unknown key or a value below -1. */
qw_status qw_tune_set(qw_tune_key key, int value);

/* Current value of a hook (QW_TUNE_AUTO when unset or unknown). */
int qw_tune_get(qw_tune_key key);

#ifdef __cplusplus
}
#endif

#endif /* QW_TUNING_H_ */
