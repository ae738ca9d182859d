// ra_api.cpp -- host side of libra.so: argument checks, per-stream workspace,
// algorithm dispatch and error reporting for the C ABI declared in include/ra.h.
#include "ra.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <vector>
#include <mutex>
#include <string>
#include <utility>

#include "ra_elem.h"
#include "ra_sync.h"
#include "ra_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int fail_hip(hipError_t e, const char* what) {
  return fail(RA_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

bool debug_on() {
  static int on = [] {
    const char* v = std::getenv("RA_DEBUG");
    return v && *v && std::strcmp(v, "0") != 0 ? 1 : 0;
  }();
  return on != 0;
}

constexpr int kLastAlgo = RA_ALGO_RING_PIPELINED_FLAGS;

const char* algo_name(int a) {
  switch (a) {
    case RA_ALGO_RING_STEP: return "ring_step";
    case RA_ALGO_RING_PIPELINED: return "ring_pipelined";
    case RA_ALGO_RING_BIDIR: return "ring_bidir";
    case RA_ALGO_FUSED: return "fused";
    case RA_ALGO_TREE: return "tree";
    case RA_ALGO_RING_CHANNELS: return "ring_channels";
    case RA_ALGO_AUTO: return "auto";
    case RA_ALGO_HIER: return "hier";
    case RA_ALGO_HIER_FUSED: return "hier_fused";
    case RA_ALGO_RING_PIPELINED_FLAGS: return "ring_pipelined_flags";
    default: return "?";
  }
}

// RA_ALGO overrides the default algorithm (diagnosis only), by name or number.
int env_algo(int fallback) {
  const char* v = std::getenv("RA_ALGO");
  if (!v || !*v) return fallback;
  for (int a = RA_ALGO_RING_STEP; a <= kLastAlgo; ++a)
    if (std::strcmp(v, algo_name(a)) == 0) return a;
  char* end = nullptr;
  long x = std::strtol(v, &end, 10);
  if (end && *end == 0 && x >= RA_ALGO_RING_STEP && x <= kLastAlgo) return (int)x;
  return fallback;
}

// ---------------------------------------------------------------- validation

int check_args(void* const* bufs, int p, int64_t n, int dtype) {
  if (!bufs) return fail(RA_ERR_INVALID_ARG, "bufs is NULL");
  if (p < 1) return fail(RA_ERR_INVALID_ARG, "p = %d, need p >= 1", p);
  if (p > RA_MAX_RANKS) return fail(RA_ERR_UNSUPPORTED, "p = %d exceeds RA_MAX_RANKS = %d", p, RA_MAX_RANKS);
  if (n < 0) return fail(RA_ERR_INVALID_ARG, "n = %lld, need n >= 0", (long long)n);
  if (dtype < RA_INT32 || dtype > RA_INT64) return fail(RA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (n == 0) return RA_OK;   // nothing is accessed: empty buffers may be NULL
  for (int r = 0; r < p; ++r) {
    if (!bufs[r]) return fail(RA_ERR_INVALID_ARG, "bufs[%d] is NULL", r);
    if (reinterpret_cast<uintptr_t>(bufs[r]) % 16 != 0)
      return fail(RA_ERR_MISALIGNED, "bufs[%d] = %p is not 16-byte aligned", r, bufs[r]);
  }
  {
    const uint64_t bytes = (uint64_t)n * (uint64_t)ra::elem_bytes(dtype);
    if (bytes / (uint64_t)ra::elem_bytes(dtype) != (uint64_t)n)
      return fail(RA_ERR_INVALID_ARG, "n = %lld overflows the address space", (long long)n);
    std::pair<uintptr_t, int> starts[RA_MAX_RANKS];   // no heap: the no-alloc entry uses this too
    for (int r = 0; r < p; ++r) starts[r] = {reinterpret_cast<uintptr_t>(bufs[r]), r};
    std::sort(starts, starts + p);
    for (int i = 0; i + 1 < p; ++i)
      if (starts[i].first + bytes > starts[i + 1].first)
        return fail(RA_ERR_ALIAS, "buffers of ranks %d and %d overlap", starts[i].second,
                    starts[i + 1].second);
  }
  return RA_OK;
}

int check_channels(const ra_options* opt) {
  if (opt && (opt->channels < 0 || opt->channels > ra::kMaxChannels))
    return fail(RA_ERR_INVALID_ARG, "channels = %d, need 0..%d", opt->channels, ra::kMaxChannels);
  return RA_OK;
}

// Ranks per node of the hierarchical algorithms: the caller's, or the largest
// divisor of p that is at most 8 (eight GPUs to a node).
int hier_group(const ra_options* opt, int p) {
  if (opt && opt->group > 0) return opt->group;
  for (int g = std::min(p, 8); g > 1; --g)
    if (p % g == 0) return g;
  return 1;
}

int check_group(const ra_options* opt, int p) {
  if (!opt || opt->group == 0) return RA_OK;
  if (opt->group < 0 || opt->group > p || p % opt->group != 0)
    return fail(RA_ERR_INVALID_ARG, "group = %d must divide p = %d", opt->group, p);
  return RA_OK;
}

int check_link(const ra_options* opt) {
  if (!opt) return RA_OK;
  const double a = opt->link_alpha_us, b = opt->link_GBps;
  if (!(a >= 0.0) || !(b >= 0.0) || a > 1e300 || b > 1e300)
    return fail(RA_ERR_INVALID_ARG, "link_alpha_us / link_GBps must be finite and >= 0");
  return RA_OK;
}

// The pages' latency-bandwidth model: a ring of 2(p-1) steps, each sending a
// chunk of S/p bytes, against a binomial tree of 2 ceil(log2 p) steps, each
// sending the whole buffer.  The ring wins ties.
int model_choice(int p, double size_bytes, double alpha_s, double bytes_per_s) {
  int levels = 0;
  while ((1 << levels) < p) ++levels;
  const double t_ring = 2.0 * (p - 1) * alpha_s + 2.0 * (p - 1) / p * size_bytes / bytes_per_s;
  const double t_tree = 2.0 * levels * (alpha_s + size_bytes / bytes_per_s);
  return t_tree < t_ring ? RA_ALGO_TREE : RA_ALGO_RING_STEP;
}

bool phase_algo(int algo) {
  return algo == RA_ALGO_RING_STEP || algo == RA_ALGO_RING_PIPELINED ||
         algo == RA_ALGO_RING_PIPELINED_FLAGS || algo == RA_ALGO_RING_CHANNELS ||
         algo == RA_ALGO_FUSED;
}

bool is_float(int dtype) {
  return dtype == RA_FLOAT32 || dtype == RA_BFLOAT16 || dtype == RA_FLOAT16 || dtype == RA_FLOAT64;
}

int check_op(int op, int dtype) {
  if (op < RA_SUM || op > RA_AVG) return fail(RA_ERR_UNSUPPORTED, "op %d not supported", op);
  if (op == RA_AVG && !is_float(dtype))
    return fail(RA_ERR_UNSUPPORTED, "RA_AVG needs a floating-point dtype, not %d", dtype);
  return RA_OK;
}

bool wide_requested(const ra_options* opt) { return opt && (opt->flags & RA_FLAG_WIDE_ACCUM); }

// The one-pass all-reduce's read/write phases as the options ask (no flag: the
// library decides; RA_FLAG_NO_PHASES wins over RA_FLAG_PHASES).  Averages keep
// the one-shot pass unless forced: dividing every term by p lengthens the fold
// between a wave's loads and its stores, and at 8 x 16 GB bfloat16 the phased
// average took 41.0 ms where the phased sum and maximum took 39.9.
int phase_mode(const ra_options* opt, int op) {
  if (opt && (opt->flags & RA_FLAG_NO_PHASES)) return ra::kPhasesOff;
  if (opt && (opt->flags & RA_FLAG_PHASES)) return ra::kPhasesForce;
  return op == RA_AVG ? ra::kPhasesOff : ra::kPhasesAuto;
}

// Wider accumulation exists for the one-pass algorithm, for bfloat16, float16
// and float32 (a maximum is exact, so there it changes nothing).
int check_wide(const ra_options* opt, int dtype, int algo) {
  if (!wide_requested(opt)) return RA_OK;
  if (algo != RA_ALGO_FUSED)
    return fail(RA_ERR_UNSUPPORTED, "RA_FLAG_WIDE_ACCUM needs RA_ALGO_FUSED");
  if (dtype != RA_FLOAT32 && dtype != RA_BFLOAT16 && dtype != RA_FLOAT16)
    return fail(RA_ERR_UNSUPPORTED, "RA_FLAG_WIDE_ACCUM needs bfloat16, float16 or float32");
  return RA_OK;
}

// ---------------------------------------------------------------- workspace

struct Workspace {
  ra::WsHeader* hdr = nullptr;     // device
  uint32_t* flags = nullptr;       // device, pipelined ready counters
  int64_t flag_cap = 0;            // entries
  uint32_t epoch = 0;              // pipelined calls so far (flag base = epoch * kFlagStride)
  bool fixed = false;              // the device's no-alloc scratch: never reallocated, reset
                                   // by fill kernels on the calling stream
  bool captured = false;           // a HIP graph holds `flags`: never freed from then on
  std::vector<void*> retired;      // counter buffers replaced after a capture (kept alive)
};

// Whether work enqueued on s is being captured into a HIP graph.
bool stream_capturing(hipStream_t s) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  return hipStreamIsCapturing(s, &cs) == hipSuccess && cs == hipStreamCaptureStatusActive;
}

constexpr uint32_t kFlagStride = 128;   // > 2(p-1) hops for p <= 64

std::mutex g_ws_mu;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;

int get_workspace(hipStream_t s, Workspace** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(g_ws_mu);
  Workspace& w = g_ws[{dev, s}];
  if (!w.hdr && stream_capturing(s))
    return fail(RA_ERR_UNSUPPORTED,
                "this call needs the stream's workspace, which the first such call on a stream "
                "allocates: make one outside graph capture first");
  if (!w.hdr) {
    void* p = nullptr;
    e = hipMalloc(&p, sizeof(ra::WsHeader));
    if (e != hipSuccess) return fail_hip(e, "hipMalloc(workspace)");
    e = hipMemset(p, 0, sizeof(ra::WsHeader));
    if (e != hipSuccess) { (void)hipFree(p); return fail_hip(e, "hipMemset(workspace)"); }
    w.hdr = static_cast<ra::WsHeader*>(p);
  }
  *out = &w;
  return RA_OK;
}

// Make room for `entries` ready counters and return the flag base of this call.
// renew (test hook): reallocate the counters (fresh zeros) and number this call
// from 2^31, as a stream would after about 16.7 million calls and a larger one.
int reserve_flags(Workspace* w, int64_t entries, hipStream_t s, bool renew, uint32_t* base) {
  std::lock_guard<std::mutex> lock(g_ws_mu);
  if (w->fixed) {
    // the no-alloc scratch: a fixed number of counters, zeroed by a kernel on s
    if (entries > w->flag_cap)
      return fail(RA_ERR_UNSUPPORTED,
                  "the call needs %lld ready counters; the no-alloc workspace holds %lld "
                  "(use larger slices)", (long long)entries, (long long)w->flag_cap);
    if (renew) w->epoch = (1u << 31) / kFlagStride - 1;
    w->epoch += 1;
    const bool wrap = (uint64_t)w->epoch * kFlagStride + kFlagStride >= 0xFFFFFFFFull;
    if (wrap) w->epoch = 1;
    if (renew || wrap) {
      hipError_t e = ra::launch_fill_u32(w->flags, 0u, w->flag_cap, s);
      if (e != hipSuccess) return fail_hip(e, "resetting flags");
    }
    *base = w->epoch * kFlagStride;
    return RA_OK;
  }
  if (renew) w->epoch = (1u << 31) / kFlagStride - 1;
  if (entries > w->flag_cap || (renew && w->flags)) {
    if (w->flags) {
      // the old counters may still be read by queued work on this stream, or by
      // a captured graph (those are kept until the process ends)
      hipError_t e = hipStreamSynchronize(s);
      if (e != hipSuccess) return fail_hip(e, "hipStreamSynchronize");
      if (w->captured)
        w->retired.push_back(w->flags);
      else
        (void)hipFree(w->flags);
      w->flags = nullptr;
      w->flag_cap = 0;
      w->captured = false;
    }
    const int64_t cap = std::max<int64_t>(entries, 4096);
    void* p = nullptr;
    hipError_t e = hipMalloc(&p, (size_t)cap * sizeof(uint32_t));
    if (e != hipSuccess) return fail_hip(e, "hipMalloc(flags)");
    e = hipMemset(p, 0, (size_t)cap * sizeof(uint32_t));
    if (e != hipSuccess) { (void)hipFree(p); return fail_hip(e, "hipMemset(flags)"); }
    w->flags = static_cast<uint32_t*>(p);
    w->flag_cap = cap;
  }
  // counters only grow: every call starts above anything an earlier call left
  w->epoch += 1;
  if ((uint64_t)w->epoch * kFlagStride + kFlagStride >= 0xFFFFFFFFull) {
    hipError_t e = hipStreamSynchronize(s);
    if (e == hipSuccess) e = hipMemset(w->flags, 0, (size_t)w->flag_cap * sizeof(uint32_t));
    if (e != hipSuccess) return fail_hip(e, "resetting flags");
    w->epoch = 1;
  }
  *base = w->epoch * kFlagStride;
  return RA_OK;
}

// The ready counters of a call being captured into a HIP graph: the buffer must
// already hold `entries` (it cannot be allocated, nor an old one freed, during
// capture), is kept alive from now on, and is zeroed by a captured fill kernel.
int capture_flags(Workspace* w, int64_t entries, hipStream_t s) {
  std::lock_guard<std::mutex> lock(g_ws_mu);
  if (entries > w->flag_cap)
    return fail(RA_ERR_UNSUPPORTED,
                "under graph capture the stream's ready counters cannot grow: the call needs "
                "%lld, the stream holds %lld (make the same call once outside capture first)",
                (long long)entries, (long long)w->flag_cap);
  if (!w->fixed) w->captured = true;
  hipError_t e = ra::launch_fill_u32(w->flags, 0u, entries, s);
  if (e != hipSuccess) return fail_hip(e, "zeroing ready counters");
  return RA_OK;
}

// ---------------------------------------------------------------- no-alloc workspace

// The workspace of ra_allreduce_noalloc: one array per GPU, in the library's
// device data, so that calls which must not allocate (HIP graph capture, tight
// serving loops) still have barrier words, a status word and ready counters.
// Layout: the WsHeader at offset 0, the ready counters from kScratchFlagsAt on.
// Every call on a GPU shares its array, and the array keeps what the last call
// left; calls that overlap on one GPU race.  The array's host-side name is only
// a stand-in for the device symbol: host code uses the address that
// hipGetSymbolAddress returns for the current device, never the name itself.
constexpr size_t kScratchBytes = 1u << 20;
constexpr size_t kScratchFlagsAt = 32u << 10;
static_assert(sizeof(ra::WsHeader) <= kScratchFlagsAt, "scratch header does not fit");
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
Workspace g_scratch_ws[kMaxDevices];   // guarded by g_ws_mu; hdr == nullptr until set up
bool g_scratch_used[kMaxDevices];

// This device's scratch workspace, its address looked up once per device with
// that device current.
int get_scratch(Workspace** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(RA_ERR_UNSUPPORTED, "device %d: the no-alloc workspace serves devices 0..%d",
                dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_ws_mu);
  Workspace& w = g_scratch_ws[dev];
  if (!w.hdr) {
    unsigned char* ptr = nullptr;
    e = hipGetSymbolAddress(reinterpret_cast<void**>(&ptr), HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) return fail_hip(e, "hipGetSymbolAddress(scratch)");
    w.hdr = reinterpret_cast<ra::WsHeader*>(ptr);
    w.flags = reinterpret_cast<uint32_t*>(ptr + kScratchFlagsAt);
    w.flag_cap = (int64_t)((kScratchBytes - kScratchFlagsAt) / sizeof(uint32_t));
    w.epoch = 0;
    w.fixed = true;
  }
  g_scratch_used[dev] = true;
  *out = &w;
  return RA_OK;
}

// Whether a step call may run the persistent grid, and so needs the stream's
// workspace (status word, barrier words, ready counters): the pipelined and
// channel algorithms always; the other step algorithms only for a caller's
// grid, step timestamps or a test hook.  Otherwise their steps run as ordinary
// launches with no device-side waits, and the call allocates nothing -- it can
// be captured in a HIP graph, even as the stream's first call.
bool needs_workspace(int algo, const ra_options* opt) {
  if (algo == RA_ALGO_RING_PIPELINED_FLAGS || algo == RA_ALGO_RING_CHANNELS) return true;
  if (algo == RA_ALGO_RING_PIPELINED) return false;   // no device-side waits at all
  return opt && (opt->grid > 0 || opt->step_ts != nullptr ||
                 (opt->flags & (RA_FLAG_FORCE_TIMEOUT | RA_FLAG_STRESS)) != 0);
}

int sync_cfg(const ra_options* opt, Workspace* w, hipStream_t s, ra::SyncCfg* sc) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
  int khz = 0;
  e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
  if (e != hipSuccess || khz <= 0) khz = 100000;   // 100 MHz, the gfx9 constant clock
  const int64_t us = opt && opt->timeout_us > 0 ? opt->timeout_us : 10 * 1000 * 1000;
  sc->ws = w ? w->hdr : nullptr;
  sc->limit_ticks = (uint64_t)us * (uint64_t)khz / 1000u;
  sc->expect_extra = opt && (opt->flags & RA_FLAG_FORCE_TIMEOUT) ? 1u : 0u;
  // a different delay pattern on every call
  static std::atomic<uint32_t> calls{0};
  sc->stress = opt && (opt->flags & RA_FLAG_STRESS) ? 1u + calls.fetch_add(1u) : 0u;
  sc->step_ts = opt ? opt->step_ts : nullptr;
  sc->grid = opt && opt->grid > 0 ? opt->grid : 0;
  sc->channels = 1;
  sc->group = 1;
  // the placement probe allocates and copies: not in a call that must not
  // allocate, nor under graph capture
  sc->may_probe = !(w && w->fixed) && !stream_capturing(s);
  return RA_OK;
}

void fill_ptrs(void* const* bufs, int p, ra::RankPtrs* P) {
  std::memset(P, 0, sizeof(*P));
  for (int r = 0; r < p; ++r) P->b[r] = bufs[r];
}

// launches: kernels the call enqueued (the step algorithms run one per step on
// larger buffers)
void debug_line(const char* call, int algo, int p, int64_t n, int dtype, int grid,
                int launches = 1) {
  if (!debug_on()) return;
  std::fprintf(stderr, "[ra] %s algo=%s p=%d n=%lld dtype=%d grid=%d launches=%d ring=", call,
               algo_name(algo), p, (long long)n, dtype, grid, launches);
  for (int r = 0; r < p; ++r) std::fprintf(stderr, "%d%s", r, r + 1 < p ? "->" : "->0\n");
}

// Run phases [hop_begin, hop_end) (0..p-2 reduce-scatter, p-1..2p-3 all-gather)
// with a ring algorithm.
// noalloc: the persistent grids' workspace is this device's scratch array.
int run_ring(const char* call, void* const* bufs, int p, int64_t n, int dtype, int op, int algo,
             int hop_begin, int hop_end, const ra_options* opt, hipStream_t s,
             bool noalloc = false) {
  if (algo == RA_ALGO_FUSED) {
    // the fused pass covers whole phases only
    const int mode = hop_begin == 0 && hop_end == 2 * (p - 1) ? 0 : hop_begin == 0 ? 1 : 2;
    ra::RankPtrs P;
    fill_ptrs(bufs, p, &P);
    int grid = 0;
    hipError_t e = ra::launch_fused(P, p, n, dtype, op, wide_requested(opt), mode,
                                    phase_mode(opt, op), s, &grid);
    if (e != hipSuccess) return fail_hip(e, "kernel launch");
    debug_line(call, algo, p, n, dtype, grid);
    return RA_OK;
  }
  if (algo == RA_ALGO_RING_PIPELINED) {
    // slices carried through every hop by one workgroup: one ordinary launch
    const int mode = hop_begin == 0 && hop_end == 2 * (p - 1) ? 0 : hop_begin == 0 ? 1 : 2;
    ra::RankPtrs P;
    fill_ptrs(bufs, p, &P);
    ra::SyncCfg sc;
    int rc = sync_cfg(opt, nullptr, s, &sc);
    if (rc != RA_OK) return rc;
    int grid = 0;
    hipError_t e = ra::launch_rider(P, p, n, dtype, op, mode, opt ? opt->slice_elems : 0, sc.stress,
                                    s, &grid);
    if (e != hipSuccess) return fail_hip(e, "kernel launch");
    debug_line(call, algo, p, n, dtype, grid);
    return RA_OK;
  }
  Workspace* w = nullptr;
  int rc = RA_OK;
  if (needs_workspace(algo, opt)) {
    rc = noalloc ? get_scratch(&w) : get_workspace(s, &w);
    if (rc != RA_OK) return rc;
  }
  ra::SyncCfg sc;
  rc = sync_cfg(opt, w, s, &sc);
  if (rc != RA_OK) return rc;
  ra::RankPtrs P;
  fill_ptrs(bufs, p, &P);
  int grid = 0, launches = 1;
  hipError_t e;
  if (algo == RA_ALGO_RING_PIPELINED_FLAGS) {
    int64_t slice = opt && opt->slice_elems > 0
                        ? opt->slice_elems
                        : ra::pipelined_default_slice(p, n, dtype, sc.grid);
    const int64_t L = 16 / ra::elem_bytes(dtype) * ra::kLineVecs;   // whole 128-byte lines
    slice = (slice + L - 1) / L * L;
    const int64_t kmax = ra::pipelined_slices_per_chunk(p, n, dtype, slice);
    uint32_t base = 0;
    if (stream_capturing(s)) {
      // Under HIP graph capture the call cannot take a number from the host:
      // every replay would reuse it, and the counters its last replay left would
      // read as already reached.  It zeroes the counters with a fill kernel (a
      // node of the graph) and numbers itself from 0.  Eager calls number from
      // 128 up, above anything a replay leaves (at most 2(p-1)), so the two mix.
      rc = capture_flags(w, kmax * p, s);
      if (rc != RA_OK) return rc;
    } else {
      rc = reserve_flags(w, kmax * p, s, opt && (opt->flags & RA_FLAG_RENEW_COUNTERS), &base);
      if (rc != RA_OK) return rc;
    }
    e = ra::launch_pipelined(P, p, n, dtype, op, hop_begin, hop_end, slice, kmax, w->flags, base,
                             sc, s, &grid);
  } else {
    if (algo == RA_ALGO_RING_CHANNELS) sc.channels = opt ? opt->channels : 0;   // 0: automatic
    e = ra::launch_steps(P, p, n, dtype, op, ra::kModeRing, hop_begin, hop_end, sc, s, &grid,
                         &launches);
  }
  if (e != hipSuccess) return fail_hip(e, "kernel launch");
  debug_line(call, algo, p, n, dtype, grid, launches);
  return RA_OK;
}

// ra_allreduce_ex and ra_allreduce_noalloc: noalloc takes the persistent grids'
// workspace from this device's scratch array instead of the stream's.
int allreduce_impl(void* const* bufs, int p, int64_t n, int dtype, int op, int algo,
                   const ra_options* opt, hipStream_t stream, bool noalloc) {
  int rc = check_args(bufs, p, n, dtype);
  if (rc == RA_OK) rc = check_op(op, dtype);
  if (rc == RA_OK) rc = check_channels(opt);
  if (rc != RA_OK) return rc;
  if (algo == RA_ALGO_DEFAULT) algo = env_algo(RA_ALGO_FUSED);
  if (algo < RA_ALGO_RING_STEP || algo > kLastAlgo)
    return fail(RA_ERR_INVALID_ARG, "unknown algo %d", algo);
  if (algo == RA_ALGO_AUTO) {
    rc = ra_select_algo(p, n, dtype, opt, &algo);
    if (rc != RA_OK) return rc;
  }
  rc = check_wide(opt, dtype, algo);
  if (rc == RA_OK) rc = check_group(opt, p);
  if (rc != RA_OK) return rc;
  if (p == 1 || n == 0) return RA_OK;
  if (phase_algo(algo))
    return run_ring("allreduce", bufs, p, n, dtype, op, algo, 0, 2 * (p - 1), opt, stream,
                    noalloc);
  if (algo == RA_ALGO_HIER_FUSED) {
    ra::RankPtrs P;
    fill_ptrs(bufs, p, &P);
    int grid = 0;
    hipError_t e = ra::launch_fused_hier(P, p, n, dtype, op, hier_group(opt, p), stream, &grid);
    if (e != hipSuccess) return fail_hip(e, "kernel launch");
    debug_line("allreduce", algo, p, n, dtype, grid);
    return RA_OK;
  }
  // bidirectional rings, tree or hierarchy: the step kernels
  Workspace* w = nullptr;
  if (needs_workspace(algo, opt)) {
    rc = noalloc ? get_scratch(&w) : get_workspace(stream, &w);
    if (rc != RA_OK) return rc;
  }
  ra::SyncCfg sc;
  rc = sync_cfg(opt, w, stream, &sc);
  if (rc != RA_OK) return rc;
  ra::RankPtrs P;
  fill_ptrs(bufs, p, &P);
  int grid = 0, launches = 1;
  hipError_t e;
  if (algo == RA_ALGO_RING_BIDIR) {
    e = ra::launch_steps(P, p, n, dtype, op, ra::kModeBidir, 0, 2 * (p - 1), sc, stream, &grid,
                         &launches);
  } else if (algo == RA_ALGO_HIER) {
    sc.group = hier_group(opt, p);
    const int m = p / sc.group;
    e = ra::launch_steps(P, p, n, dtype, op, ra::kModeHier, 0, 2 * (sc.group - 1) + 2 * (m - 1), sc,
                         stream, &grid, &launches);
  } else {
    int levels = 0;
    while ((1 << levels) < p) ++levels;
    e = ra::launch_steps(P, p, n, dtype, op, ra::kModeTree, 0, 2 * levels, sc, stream, &grid,
                         &launches);
  }
  if (e != hipSuccess) return fail_hip(e, "kernel launch");
  debug_line("allreduce", algo, p, n, dtype, grid, launches);
  return RA_OK;
}

}  // namespace

extern "C" {

int ra_chunk_bounds(int64_t n, int p, int64_t* starts) {
  if (!starts) return fail(RA_ERR_INVALID_ARG, "starts is NULL");
  if (p < 1) return fail(RA_ERR_INVALID_ARG, "p = %d, need p >= 1", p);
  if (p > RA_MAX_RANKS) return fail(RA_ERR_UNSUPPORTED, "p = %d exceeds RA_MAX_RANKS", p);
  if (n < 0) return fail(RA_ERR_INVALID_ARG, "n = %lld, need n >= 0", (long long)n);
  const int64_t base = n / p, extra = n % p;
  for (int i = 0; i <= p; ++i) starts[i] = (int64_t)i * base + std::min<int64_t>(i, extra);
  return RA_OK;
}

int ra_reduce_scatter_ex(void* const* bufs, int p, int64_t n, int dtype, int op, int algo,
                         const ra_options* opt, hipStream_t stream) {
  int rc = check_args(bufs, p, n, dtype);
  if (rc == RA_OK) rc = check_op(op, dtype);
  if (rc == RA_OK) rc = check_channels(opt);
  if (rc != RA_OK) return rc;
  if (algo == RA_ALGO_DEFAULT) algo = RA_ALGO_FUSED;
  if (!phase_algo(algo))
    return fail(RA_ERR_UNSUPPORTED,
                "reduce-scatter runs RING_STEP, RING_PIPELINED(_FLAGS), RING_CHANNELS or FUSED, not %d",
                algo);
  rc = check_wide(opt, dtype, algo);
  if (rc != RA_OK) return rc;
  if (p == 1 || n == 0) return RA_OK;
  return run_ring("reduce_scatter", bufs, p, n, dtype, op, algo, 0, p - 1, opt, stream);
}

int ra_all_gather_ex(void* const* bufs, int p, int64_t n, int dtype, int algo,
                     const ra_options* opt, hipStream_t stream) {
  int rc = check_args(bufs, p, n, dtype);
  if (rc == RA_OK) rc = check_channels(opt);
  if (rc != RA_OK) return rc;
  if (algo == RA_ALGO_DEFAULT) algo = RA_ALGO_FUSED;
  if (!phase_algo(algo))
    return fail(RA_ERR_UNSUPPORTED,
                "all-gather runs RING_STEP, RING_PIPELINED(_FLAGS), RING_CHANNELS or FUSED, not %d",
                algo);
  if (p == 1 || n == 0) return RA_OK;
  return run_ring("all_gather", bufs, p, n, dtype, RA_SUM, algo, p - 1, 2 * (p - 1), opt, stream);
}

int ra_reduce_scatter(void* const* bufs, int p, int64_t n, int dtype, int op, hipStream_t stream) {
  return ra_reduce_scatter_ex(bufs, p, n, dtype, op, RA_ALGO_DEFAULT, nullptr, stream);
}

int ra_all_gather(void* const* bufs, int p, int64_t n, int dtype, hipStream_t stream) {
  return ra_all_gather_ex(bufs, p, n, dtype, RA_ALGO_DEFAULT, nullptr, stream);
}

int ra_allreduce_ex(void* const* bufs, int p, int64_t n, int dtype, int op, int algo,
                    const ra_options* opt, hipStream_t stream) {
  return allreduce_impl(bufs, p, n, dtype, op, algo, opt, stream, false);
}

int ra_allreduce_noalloc(void* const* bufs, int p, int64_t n, int dtype, int op, int algo,
                         const ra_options* opt, hipStream_t stream) {
  return allreduce_impl(bufs, p, n, dtype, op, algo, opt, stream, true);
}

int ra_allreduce(void* const* bufs, int p, int64_t n, int dtype, int op, hipStream_t stream) {
  return ra_allreduce_ex(bufs, p, n, dtype, op, RA_ALGO_DEFAULT, nullptr, stream);
}

int ra_stream_status(hipStream_t stream) {
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail_hip(e, "hipStreamSynchronize");
  int dev = 0;
  e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
  // the stream's own workspace, and the device's no-alloc scratch if a call used it
  ra::WsHeader* hdrs[2] = {nullptr, nullptr};
  {
    std::lock_guard<std::mutex> lock(g_ws_mu);
    auto it = g_ws.find({dev, stream});
    if (it != g_ws.end()) hdrs[0] = it->second.hdr;
    if (dev >= 0 && dev < kMaxDevices && g_scratch_used[dev]) hdrs[1] = g_scratch_ws[dev].hdr;
  }
  for (ra::WsHeader* hdr : hdrs) {
    if (!hdr) continue;
    uint32_t status = 0;
    e = hipMemcpy(&status, &hdr->status, sizeof status, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return fail_hip(e, "reading device status");
    if (status == 0) continue;
    // clear the sticky error and the barrier words the aborted kernel left behind
    e = hipMemset(hdr, 0, sizeof(ra::WsHeader));
    if (e != hipSuccess) return fail_hip(e, "clearing device status");
    return fail((int)status, "a device-side wait timed out (status %u)", status);
  }
  return RA_OK;
}

int ra_select_algo(int p, int64_t n, int dtype, const ra_options* opt, int* algo_out) {
  if (!algo_out) return fail(RA_ERR_INVALID_ARG, "algo_out is NULL");
  if (p < 1) return fail(RA_ERR_INVALID_ARG, "p = %d, need p >= 1", p);
  if (p > RA_MAX_RANKS) return fail(RA_ERR_UNSUPPORTED, "p = %d exceeds RA_MAX_RANKS = %d", p, RA_MAX_RANKS);
  if (n < 0) return fail(RA_ERR_INVALID_ARG, "n = %lld, need n >= 0", (long long)n);
  if (dtype < RA_INT32 || dtype > RA_INT64) return fail(RA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  int rc = check_link(opt);
  if (rc != RA_OK) return rc;
  if (opt && opt->link_alpha_us > 0.0 && opt->link_GBps > 0.0) {
    const double size = (double)n * (double)ra::elem_bytes(dtype);
    *algo_out = model_choice(p, size, opt->link_alpha_us * 1e-6, opt->link_GBps * 1e9);
  } else {
    *algo_out = RA_ALGO_FUSED;
  }
  return RA_OK;
}

const char* ra_status_string(int code) {
  switch (code) {
    case RA_OK: return "RA_OK";
    case RA_ERR_INVALID_ARG: return "RA_ERR_INVALID_ARG";
    case RA_ERR_UNSUPPORTED: return "RA_ERR_UNSUPPORTED";
    case RA_ERR_ALIAS: return "RA_ERR_ALIAS";
    case RA_ERR_MISALIGNED: return "RA_ERR_MISALIGNED";
    case RA_ERR_HIP: return "RA_ERR_HIP";
    case RA_ERR_TIMEOUT: return "RA_ERR_TIMEOUT";
    default: return "RA_ERR_UNKNOWN";
  }
}

const char* ra_last_error(void) { return g_last_error.c_str(); }

int ra_wallclock_hz(int64_t* hz) {
  if (!hz) return fail(RA_ERR_INVALID_ARG, "hz is NULL");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
  int khz = 0;
  e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
  if (e != hipSuccess) return fail_hip(e, "hipDeviceGetAttribute(WallClockRate)");
  *hz = (int64_t)khz * 1000;
  return RA_OK;
}

int ra_stream_copy_resident(void* dst, const void* src, int64_t bytes, int grid,
                            hipStream_t stream) {
  if (!dst || !src) return fail(RA_ERR_INVALID_ARG, "NULL pointer");
  if (bytes < 0 || bytes % 16 != 0) return fail(RA_ERR_INVALID_ARG, "bytes must be a multiple of 16");
  if (grid < 0) return fail(RA_ERR_INVALID_ARG, "grid = %d, need grid >= 0", grid);
  if (reinterpret_cast<uintptr_t>(dst) % 16 || reinterpret_cast<uintptr_t>(src) % 16)
    return fail(RA_ERR_MISALIGNED, "pointers must be 16-byte aligned");
  if (grid == 0) grid = ra::default_persistent_workgroups();
  if (grid <= 0) return fail(RA_ERR_HIP, "cannot query the device's compute units");
  Workspace* w = nullptr;
  int rc = get_workspace(stream, &w);
  if (rc != RA_OK) return rc;
  hipError_t e = ra::launch_copy_resident(dst, src, bytes, grid, &w->hdr->tiles[0][0], stream);
  if (e != hipSuccess) return fail_hip(e, "kernel launch");
  return RA_OK;
}

int ra_stream_copy(void* dst, const void* src, int64_t bytes, hipStream_t stream) {
  if (!dst || !src) return fail(RA_ERR_INVALID_ARG, "NULL pointer");
  if (bytes < 0 || bytes % 16 != 0) return fail(RA_ERR_INVALID_ARG, "bytes must be a multiple of 16");
  if (reinterpret_cast<uintptr_t>(dst) % 16 || reinterpret_cast<uintptr_t>(src) % 16)
    return fail(RA_ERR_MISALIGNED, "pointers must be 16-byte aligned");
  hipError_t e = ra::launch_copy(dst, src, bytes, stream);
  if (e != hipSuccess) return fail_hip(e, "kernel launch");
  return RA_OK;
}

}  // extern "C"
