/* Minimal pthread work loop for the oracle.  TEST INFRASTRUCTURE ONLY. */
#ifndef PAN_ORACLE_THREADS_H
#define PAN_ORACLE_THREADS_H
#include <stdint.h>

/* Runs fn(arg, item, scratch) for item in [0, n_items) on nthreads threads
 * (<= 0: one per online core).  Items are claimed from a shared counter, so
 * rows of different length balance.  scratch is a per-thread buffer of
 * scratch_doubles doubles.  Returns 0, or -3 when memory is short. */
typedef void (*orc_item_fn)(void* arg, int64_t item, double* scratch);
int orc_parallel_for(orc_item_fn fn, void* arg, int64_t n_items, int64_t scratch_doubles, int nthreads);

#endif
