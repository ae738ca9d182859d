// host_check.cpp -- the host side of the C ABI (argument checks, chunk bounds,
// algorithm selection, status strings) exercised without a GPU, built with
// AddressSanitizer on the library's host code.  No call here reaches a kernel:
// every call either fails validation or needs no device.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "ra.h"

static int failures = 0;
static void expect(bool ok, const char* what) {
  if (!ok) {
    std::printf("FAIL %s (last error: %s)\n", what, ra_last_error());
    ++failures;
  }
}

int main() {
  // chunk bounds: p + 1 starts, first n mod p chunks one longer, for many (n, p)
  for (int p = 1; p <= RA_MAX_RANKS; ++p) {
    for (int64_t n : {int64_t(0), int64_t(1), int64_t(63), int64_t(1000003), int64_t(8000000000),
                      (int64_t(1) << 40) + 7}) {
      std::vector<int64_t> s(p + 1, -1);
      expect(ra_chunk_bounds(n, p, s.data()) == RA_OK, "ra_chunk_bounds");
      const int64_t b = n / p, e = n % p;
      for (int i = 0; i < p; ++i)
        expect(s[i + 1] - s[i] == b + (i < e ? 1 : 0), "chunk size rule");
      expect(s[0] == 0 && s[p] == n, "chunk bounds cover the buffer");
    }
  }
  int64_t dummy[4];
  expect(ra_chunk_bounds(4, 0, dummy) == RA_ERR_INVALID_ARG, "p = 0");
  expect(ra_chunk_bounds(4, RA_MAX_RANKS + 1, dummy) == RA_ERR_UNSUPPORTED, "p too large");
  expect(ra_chunk_bounds(-1, 2, dummy) == RA_ERR_INVALID_ARG, "n < 0");

  // overlap detection on random pointer sets (never dereferenced: n would be
  // accessed only after validation, and every set here overlaps somewhere)
  std::mt19937_64 rng(7);
  const uintptr_t base = uintptr_t(0x7f0000000000ull);
  for (int trial = 0; trial < 2000; ++trial) {
    const int p = 2 + int(rng() % 63);
    const int64_t n = 1 + int64_t(rng() % 4096);
    std::vector<void*> bufs(p);
    for (int r = 0; r < p; ++r) bufs[r] = reinterpret_cast<void*>(base + uintptr_t(r) * 16 * 8192);
    const int a = int(rng() % p), b = (a + 1 + int(rng() % (p - 1))) % p;
    bufs[b] = reinterpret_cast<void*>(reinterpret_cast<uintptr_t>(bufs[a]) + 16 * (rng() % 4));
    const int64_t nn = n + 8192 * 4;     // every neighbour pair overlaps at this length too
    expect(ra_allreduce(bufs.data(), p, nn, RA_FLOAT32, RA_SUM, nullptr) == RA_ERR_ALIAS, "alias");
    expect(std::strstr(ra_last_error(), "overlap") != nullptr, "alias message");
  }

  // every other argument error, on every entry point
  std::vector<void*> ok(8);
  for (int r = 0; r < 8; ++r) ok[r] = reinterpret_cast<void*>(base + uintptr_t(r) * (1 << 20));
  void** P = ok.data();
  expect(ra_allreduce(nullptr, 8, 16, RA_FLOAT32, RA_SUM, nullptr) == RA_ERR_INVALID_ARG, "null bufs");
  expect(ra_allreduce(P, 0, 16, RA_FLOAT32, RA_SUM, nullptr) == RA_ERR_INVALID_ARG, "p = 0");
  expect(ra_allreduce(P, 8, -1, RA_FLOAT32, RA_SUM, nullptr) == RA_ERR_INVALID_ARG, "n < 0");
  expect(ra_allreduce(P, 8, 16, 9, RA_SUM, nullptr) == RA_ERR_INVALID_ARG, "dtype");
  expect(ra_allreduce(P, 8, 16, RA_FLOAT32, 9, nullptr) == RA_ERR_UNSUPPORTED, "op");
  expect(ra_allreduce(P, 8, 16, RA_INT64, RA_AVG, nullptr) == RA_ERR_UNSUPPORTED, "avg on int64");
  expect(ra_reduce_scatter(P, 8, 16, RA_FLOAT32, 9, nullptr) == RA_ERR_UNSUPPORTED, "rs op");
  expect(ra_all_gather(nullptr, 8, 16, RA_FLOAT32, nullptr) == RA_ERR_INVALID_ARG, "ag null");
  expect(ra_allreduce_ex(P, 8, 16, RA_FLOAT32, RA_SUM, 99, nullptr, nullptr) == RA_ERR_INVALID_ARG, "algo");
  expect(ra_reduce_scatter_ex(P, 8, 16, RA_FLOAT32, RA_SUM, RA_ALGO_TREE, nullptr, nullptr) ==
             RA_ERR_UNSUPPORTED, "rs tree");
  expect(ra_all_gather_ex(P, 8, 16, RA_FLOAT32, RA_ALGO_AUTO, nullptr, nullptr) == RA_ERR_UNSUPPORTED,
         "ag auto");
  {
    void* mis[2] = {reinterpret_cast<void*>(base + 8), reinterpret_cast<void*>(base + 4096)};
    expect(ra_allreduce(mis, 2, 16, RA_FLOAT32, RA_SUM, nullptr) == RA_ERR_MISALIGNED, "misaligned");
  }
  ra_options o;
  std::memset(&o, 0, sizeof o);
  o.channels = 65;
  expect(ra_allreduce_ex(P, 8, 16, RA_FLOAT32, RA_SUM, RA_ALGO_RING_CHANNELS, &o, nullptr) ==
             RA_ERR_INVALID_ARG, "channels");
  o.channels = 0;
  o.group = 3;
  expect(ra_allreduce_ex(P, 8, 16, RA_FLOAT32, RA_SUM, RA_ALGO_HIER, &o, nullptr) == RA_ERR_INVALID_ARG,
         "group");
  o.group = 0;
  o.flags = RA_FLAG_WIDE_ACCUM;
  expect(ra_allreduce_ex(P, 8, 16, RA_INT32, RA_SUM, RA_ALGO_FUSED, &o, nullptr) == RA_ERR_UNSUPPORTED,
         "wide int32");
  o.flags = 0;
  o.link_alpha_us = -1.0;
  int algo = -1;
  expect(ra_select_algo(8, 16, RA_FLOAT32, &o, &algo) == RA_ERR_INVALID_ARG, "negative alpha");

  // algorithm selection over a grid of (p, n, alpha, B); no-ops need no device
  for (int p = 1; p <= RA_MAX_RANKS; p *= 2)
    for (int64_t n : {int64_t(1), int64_t(1) << 12, int64_t(1) << 20, int64_t(1) << 33})
      for (double a : {1.0, 10.0})
        for (double g : {25.0, 450.0}) {
          o.link_alpha_us = a;
          o.link_GBps = g;
          expect(ra_select_algo(p, n, RA_BFLOAT16, &o, &algo) == RA_OK &&
                     (algo == RA_ALGO_RING_STEP || algo == RA_ALGO_TREE), "select with a link");
        }
  expect(ra_select_algo(8, 16, RA_BFLOAT16, nullptr, &algo) == RA_OK && algo == RA_ALGO_FUSED,
         "select without a link");
  expect(ra_allreduce(P, 1, 1 << 20, RA_FLOAT32, RA_SUM, nullptr) == RA_OK, "p = 1 is a no-op");
  expect(ra_allreduce(P, 8, 0, RA_FLOAT32, RA_SUM, nullptr) == RA_OK, "n = 0 is a no-op");
  for (int c = 0; c <= 7; ++c) expect(ra_status_string(c) != nullptr, "status string");
  expect(std::strcmp(ra_status_string(1234), "RA_ERR_UNKNOWN") == 0, "unknown status");

  std::printf("%s: %d failure(s)\n", failures ? "FAILED" : "PASSED", failures);
  return failures ? 1 : 0;
}
