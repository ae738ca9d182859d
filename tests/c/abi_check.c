/*
 * abi_check.c -- the C ABI of libra.so used from plain C: device buffers from
 * hipMalloc, a host array of pointers, no Python and no torch.
 *
 * Rank r, element i holds the int32 value (r + 1) * (i % 1000) - 7 * r.  An int32
 * sum is exact whatever the order, so every algorithm must leave every rank
 * with sum_r of that value, i.e. (i % 1000) * p(p+1)/2 - 7 * p(p-1)/2.  After a
 * reduce-scatter alone, rank r's owned chunk (r + 1) mod p (chunk c starting at
 * c * floor(n/p) + min(c, n mod p)) holds that sum.
 *
 * Prints one line per check and exits 0 when all pass, 1 otherwise.
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <hip/hip_runtime_api.h>

#include "ra.h"

static int failures = 0;

static void check(int ok, const char* what) {
  printf("%s %s\n", ok ? "ok  " : "FAIL", what);
  if (!ok) failures++;
}

static int32_t input(int r, int64_t i) { return (int32_t)((r + 1) * (int32_t)(i % 1000) - 7 * r); }

static int32_t total(int p, int64_t i) {
  return (int32_t)((i % 1000) * (p * (p + 1) / 2) - 7 * (p * (p - 1) / 2));
}

static int fill(void** bufs, int p, int64_t n, int32_t* host) {
  for (int r = 0; r < p; ++r) {
    for (int64_t i = 0; i < n; ++i) host[i] = input(r, i);
    if (hipMemcpy(bufs[r], host, (size_t)n * 4, hipMemcpyHostToDevice) != hipSuccess) return 0;
  }
  return 1;
}

/* every rank equals the full sum on [lo, hi) */
static int all_equal_sum(void** bufs, int p, int64_t n, int32_t* host, int64_t lo, int64_t hi, int rank) {
  if (hipMemcpy(host, bufs[rank], (size_t)n * 4, hipMemcpyDeviceToHost) != hipSuccess) return 0;
  for (int64_t i = lo; i < hi; ++i)
    if (host[i] != total(p, i)) return 0;
  return 1;
}

int main(void) {
  const int p = 9;
  const int64_t n = 1000003;
  void* bufs[9];
  int32_t* host = (int32_t*)malloc((size_t)n * 4);
  for (int r = 0; r < p; ++r)
    if (hipMalloc(&bufs[r], (size_t)n * 4) != hipSuccess) { printf("FAIL hipMalloc\n"); return 1; }
  hipStream_t s;
  if (hipStreamCreate(&s) != hipSuccess) { printf("FAIL hipStreamCreate\n"); return 1; }

  const int algos[] = {RA_ALGO_DEFAULT, RA_ALGO_RING_STEP, RA_ALGO_RING_PIPELINED, RA_ALGO_RING_BIDIR,
                       RA_ALGO_FUSED, RA_ALGO_TREE, RA_ALGO_RING_CHANNELS, RA_ALGO_AUTO,
                       RA_ALGO_HIER, RA_ALGO_HIER_FUSED, RA_ALGO_RING_PIPELINED_FLAGS};
  for (unsigned a = 0; a < sizeof algos / sizeof algos[0]; ++a) {
    char what[96];
    snprintf(what, sizeof what, "ra_allreduce_ex algo %d, p=9 n=1000003 int32", algos[a]);
    int ok = fill(bufs, p, n, host);
    ra_options opt;
    memset(&opt, 0, sizeof opt);
    opt.group = 3;
    ok = ok && ra_allreduce_ex(bufs, p, n, RA_INT32, RA_SUM, algos[a], &opt, s) == RA_OK;
    ok = ok && ra_stream_status(s) == RA_OK;
    for (int r = 0; r < p && ok; ++r) ok = all_equal_sum(bufs, p, n, host, 0, n, r);
    check(ok, what);
  }

  /* reduce-scatter alone: the owned chunk of every rank */
  int64_t starts[10];
  check(ra_chunk_bounds(n, p, starts) == RA_OK && starts[0] == 0 && starts[p] == n &&
            starts[1] == 111112 && starts[5] == 555559,
        "ra_chunk_bounds: first n mod p chunks one longer");
  {
    int ok = fill(bufs, p, n, host);
    ok = ok && ra_reduce_scatter(bufs, p, n, RA_INT32, RA_SUM, s) == RA_OK;
    ok = ok && ra_stream_status(s) == RA_OK;
    for (int r = 0; r < p && ok; ++r) {
      const int c = (r + 1) % p;
      ok = all_equal_sum(bufs, p, n, host, starts[c], starts[c + 1], r);
    }
    check(ok, "ra_reduce_scatter: rank r owns chunk (r+1) mod p");
    ok = ok && ra_all_gather(bufs, p, n, RA_INT32, s) == RA_OK && ra_stream_status(s) == RA_OK;
    for (int r = 0; r < p && ok; ++r) ok = all_equal_sum(bufs, p, n, host, 0, n, r);
    check(ok, "ra_all_gather after ra_reduce_scatter: the all-reduce");
  }

  /* argument errors come back before anything is enqueued */
  check(ra_allreduce(NULL, p, n, RA_INT32, RA_SUM, s) == RA_ERR_INVALID_ARG, "NULL bufs");
  check(ra_allreduce(bufs, p, n, 17, RA_SUM, s) == RA_ERR_INVALID_ARG, "unknown dtype");
  check(ra_allreduce(bufs, p, n, RA_INT32, RA_AVG, s) == RA_ERR_UNSUPPORTED, "avg on int32");
  {
    void* alias[2] = {bufs[0], bufs[0]};
    check(ra_allreduce(alias, 2, n, RA_INT32, RA_SUM, s) == RA_ERR_ALIAS, "overlapping buffers");
    check(strstr(ra_last_error(), "overlap") != NULL, "ra_last_error names the overlap");
  }
  check(strcmp(ra_status_string(RA_ERR_TIMEOUT), "RA_ERR_TIMEOUT") == 0, "ra_status_string");
  int algo = -1;
  check(ra_select_algo(64, 512, RA_BFLOAT16, NULL, &algo) == RA_OK && algo == RA_ALGO_FUSED,
        "ra_select_algo without a link: fused");

  for (int r = 0; r < p; ++r) hipFree(bufs[r]);
  hipStreamDestroy(s);
  free(host);
  printf("%s: %d failure(s)\n", failures ? "FAILED" : "PASSED", failures);
  return failures ? 1 : 0;
}
