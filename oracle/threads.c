/* Minimal pthread work loop for the oracle.  TEST INFRASTRUCTURE ONLY. */
#include <pthread.h>
#include <stdlib.h>
#include <unistd.h>
#include "threads.h"

typedef struct {
  orc_item_fn fn;
  void* arg;
  int64_t n;
  int64_t next;
  int64_t scratch_doubles;
  pthread_mutex_t mu;
} pool_t;

static void* worker(void* p) {
  pool_t* pool = (pool_t*)p;
  double* scratch = (double*)malloc(sizeof(double) * (size_t)(pool->scratch_doubles > 0 ? pool->scratch_doubles : 1));
  if (!scratch) return (void*)1;
  for (;;) {
    pthread_mutex_lock(&pool->mu);
    int64_t item = pool->next++;
    pthread_mutex_unlock(&pool->mu);
    if (item >= pool->n) break;
    pool->fn(pool->arg, item, scratch);
  }
  free(scratch);
  return NULL;
}

int orc_parallel_for(orc_item_fn fn, void* arg, int64_t n_items, int64_t scratch_doubles, int nthreads) {
  if (nthreads <= 0) {
    long c = sysconf(_SC_NPROCESSORS_ONLN);
    nthreads = c > 0 ? (int)c : 1;
  }
  if (nthreads > 256) nthreads = 256;
  if ((int64_t)nthreads > n_items) nthreads = (int)(n_items > 0 ? n_items : 1);
  pool_t pool = {fn, arg, n_items, 0, scratch_doubles, PTHREAD_MUTEX_INITIALIZER};
  pthread_t th[256];
  int started = 0, rc = 0;
  for (int t = 0; t < nthreads; ++t) {
    if (pthread_create(&th[t], NULL, worker, &pool) != 0) break;
    ++started;
  }
  if (started == 0) { /* run inline */
    void* r = worker(&pool);
    return r ? -3 : 0;
  }
  for (int t = 0; t < started; ++t) {
    void* r = NULL;
    pthread_join(th[t], &r);
    if (r) rc = -3;
  }
  return rc;
}
