// Host side of the C ABI declared in include/mscl.h: argument validation,
// the channel registry (semaphore state per device and rank count), the
// algorithm selector and launch geometry, and the launches of the kernels in
// kernels.hpp; the port channel's proxy thread is in port_proxy.hpp.  Every
// entry point returns a status code; nothing here aborts.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <string>
#include <utility>

#include "../../include/mscl.h"
#include "kernels.hpp"
#include "port_proxy.hpp"

// Channel state of mscl_allreduce_noalloc (see there): 128 KiB of device
// memory in the library's code object, one copy per device the library runs
// on, held until the process ends.  Host code never passes this name to a
// kernel (on the host it is only a stand-in for the symbol): it uses the
// address hipGetSymbolAddress returns for the current device.
constexpr size_t kScratchWords = (size_t(128) << 10) / sizeof(uint32_t);
static __device__ __align__(256) uint32_t scratch[kScratchWords];

// ----------------------------------------------------------------------------
// Host side
// ----------------------------------------------------------------------------

namespace {

using namespace mscl;

thread_local std::string g_last_error;

int log_level();

// MSCL_LOG (environment, read once): 0 (default) silent; 1 every failure a
// call returns; 2 also each call's plan and each channel set's geometry;
// 3 also every kernel launch.  Lines go to stderr, prefixed "[mscl]".
void log_line(int level, const std::string& msg) {
  if (log_level() >= level) fprintf(stderr, "[mscl] %s\n", msg.c_str());
}

mscl_status_t fail(mscl_status_t s, const std::string& msg) {
  g_last_error = msg;
  log_line(1, "error " + std::to_string(s) + ": " + msg);
  return s;
}

mscl_status_t fail_hip(hipError_t e, const char* what) {
  return fail(MSCL_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

size_t elem_bytes(int dtype) { return dtype == MSCL_FLOAT32 ? 4 : 2; }

bool valid_algo(int algo) {
  return algo == MSCL_ALGO_AUTO || algo == MSCL_ALGO_ONE_SHOT || algo == MSCL_ALGO_TWO_SHOT ||
         algo == MSCL_ALGO_TWO_SHOT_FUSED || algo == MSCL_ALGO_TWO_SHOT_PORT ||
         algo == MSCL_ALGO_TWO_SHOT_FUSED_NOBARRIER || algo == MSCL_ALGO_TWO_SHOT_PERTILE;
}

bool is_fused(int algo) { return algo == MSCL_ALGO_TWO_SHOT_FUSED || algo == MSCL_ALGO_TWO_SHOT_FUSED_NOBARRIER;
}

size_t env_size(const char* name, size_t dflt) {
  const char* v = getenv(name);
  if (!v || !*v) return dflt;
  char* end = nullptr;
  unsigned long long x = strtoull(v, &end, 10);
  return (end && *end == 0) ? static_cast<size_t>(x) : dflt;
}

struct Config {
  size_t oneshot_max_bytes;  // selector threshold on bytes per rank buffer (SIZE_MAX = built-in table)
  size_t wg_target_total;    // workgroups per launch, all ranks (0 = one per compute unit)
  size_t wg_per_rank;        // fixed workgroups per rank (0 = automatic)
  uint64_t wait_timeout_us;  // default bound of one device-side wait
  size_t cached_puts_max_footprint;  // bound on 2*R*S for device-scope puts (SIZE_MAX = built-in)
  bool two_shot_hold;                // the two-shot may keep reduced tiles in LDS (mscl_twoshot_held)
  bool tile_interleave;              // whole-R-tile held slices deal tiles to the ranks in turn
  int log_level;                     // MSCL_LOG: 0..3
  bool check_protocol;               // MSCL_CHECK_PROTOCOL: channel sets start with their waits checking counts
};

const Config& config() {
  static Config c;
  static std::once_flag once;
  std::call_once(once, [] {
    c.oneshot_max_bytes = env_size("MSCL_ONESHOT_MAX_BYTES", SIZE_MAX);  // SIZE_MAX: per-R table
    c.wg_target_total = env_size("MSCL_WG_TOTAL", 0);
    c.wg_per_rank = env_size("MSCL_WG_PER_RANK", 0);
    c.cached_puts_max_footprint = env_size("MSCL_CACHED_PUTS_MAX_BYTES", SIZE_MAX);
    c.two_shot_hold = env_size("MSCL_TWO_SHOT_HOLD", 1) != 0;
    c.tile_interleave = env_size("MSCL_TILE_INTERLEAVE", 1) != 0;
    c.log_level = static_cast<int>(std::min<size_t>(env_size("MSCL_LOG", 0), 3));
    c.check_protocol = env_size("MSCL_CHECK_PROTOCOL", 0) != 0;
    // clamped to a day, so the microsecond count (and its tick count) cannot wrap
    c.wait_timeout_us = std::min<size_t>(env_size("MSCL_WAIT_TIMEOUT_MS", 2000), size_t(86400000)) * 1000;
  });
  return c;
}

int log_level() { return config().log_level; }

const char* algo_name(int algo) {
  switch (algo) {
    case MSCL_ALGO_AUTO: return "auto";
    case MSCL_ALGO_ONE_SHOT: return "one_shot";
    case MSCL_ALGO_TWO_SHOT: return "two_shot";
    case MSCL_ALGO_TWO_SHOT_FUSED: return "two_shot_fused";
    case MSCL_ALGO_TWO_SHOT_PORT: return "two_shot_port";
    case MSCL_ALGO_TWO_SHOT_FUSED_NOBARRIER: return "two_shot_fused_nobarrier";
    case MSCL_ALGO_TWO_SHOT_PERTILE: return "two_shot_pertile";
  }
  return "?";
}

}  // namespace

struct mscl_channel_s {
  int device = 0;
  int nranks = 0;
  int refcount = 0;
  int cus = 0;
  uint32_t slots = 0;            // barrier slots allocated per rank (= max co-resident workgroups per rank)
  uint32_t held_slots = 0;       // the same bound for the two-shot that keeps tiles in LDS (one per CU)
  uint64_t wall_clock_khz = 100000;
  uint32_t* inbound = nullptr;   // device [R][R][slots] barrier counters, then [R][R][slots] per-tile `seen`
  uint32_t* consumed = nullptr;  // device [R][slots] consumed signals, then [R][slots] per-tile `progress`
  int* status_host = nullptr;    // host-mapped status word
  int* status_dev = nullptr;
  uint64_t wait_timeout_us = 0;  // 0 = config default
  int drop_rank = -1;
  int double_rank = -1;          // test control: this rank signals twice each time
  int check_protocol = 0;        // waits check the counts they read (MSCL_ERR_PROTOCOL)
  mscl::proxy::PortState* port = nullptr;  // started by the first port-channel call
};

namespace {

std::mutex g_mutex;
std::map<std::pair<int, int>, mscl_channel_s*> g_registry;

bool registered(mscl_channel_s* ch) {
  for (auto& kv : g_registry)
    if (kv.second == ch) return true;
  return false;
}

// The port channel of a channel set (port_proxy.hpp); callers hold g_mutex.
mscl_status_t port_start(mscl_channel_s* ch) {
  if (ch->port) return MSCL_SUCCESS;
  std::string why;
  const mscl_status_t st = proxy::open_port(ch->device, ch->nranks, ch->status_host, &ch->port, &why);
  return st == MSCL_SUCCESS ? st : fail(st, why);
}

void port_stop(mscl_channel_s* ch) {
  proxy::close_port(ch->port, ch->device);
  ch->port = nullptr;
}

hipError_t port_reset(mscl_channel_s* ch) { return proxy::restart_port(ch->port, ch->status_host); }

mscl_status_t validate_call(const void* const inputs[], void* const outputs[], size_t count, int dtype,
                            int nranks, int algo, bool* in_place) {
  if (nranks < 1 || nranks > MSCL_MAX_RANKS)
    return fail(MSCL_ERR_INVALID_ARGUMENT, "nranks must be in 1..16");
  if (dtype != MSCL_FLOAT32 && dtype != MSCL_FLOAT16 && dtype != MSCL_BFLOAT16)
    return fail(MSCL_ERR_INVALID_ARGUMENT, "unknown dtype");
  if (!valid_algo(algo)) return fail(MSCL_ERR_INVALID_ARGUMENT, "unknown algo");
  if (!inputs || !outputs) return fail(MSCL_ERR_INVALID_ARGUMENT, "inputs/outputs array is null");
  const size_t e = elem_bytes(dtype);
  if (count > SIZE_MAX / e) return fail(MSCL_ERR_INVALID_ARGUMENT, "count * element size overflows");
  const uintptr_t bytes = count * e;
  *in_place = false;
  for (int r = 0; r < nranks; ++r) {
    if (!inputs[r] || !outputs[r]) return fail(MSCL_ERR_INVALID_ARGUMENT, "null buffer pointer");
    if ((reinterpret_cast<uintptr_t>(inputs[r]) & 15u) || (reinterpret_cast<uintptr_t>(outputs[r]) & 15u))
      return fail(MSCL_ERR_MISALIGNED, "buffers must be 16-byte aligned");
    const uintptr_t a = reinterpret_cast<uintptr_t>(inputs[r]);
    const uintptr_t b = reinterpret_cast<uintptr_t>(outputs[r]);
    if (UINTPTR_MAX - a < bytes || UINTPTR_MAX - b < bytes)
      return fail(MSCL_ERR_INVALID_ARGUMENT, "buffer range wraps the address space");
  }
  if (count == 0) return MSCL_SUCCESS;
  auto overlap = [bytes](const void* x, const void* y) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(x), b = reinterpret_cast<uintptr_t>(y);
    return a < b + bytes && b < a + bytes;
  };
  for (int r = 0; r < nranks; ++r) {
    for (int q = r + 1; q < nranks; ++q)
      if (overlap(outputs[r], outputs[q])) return fail(MSCL_ERR_INVALID_ARGUMENT, "outputs overlap");
    for (int p = 0; p < nranks; ++p) {
      if (p == r && outputs[r] == inputs[r]) {
        *in_place = true;
        continue;
      }
      if (overlap(outputs[r], inputs[p]))
        return fail(MSCL_ERR_INVALID_ARGUMENT,
                    "an output overlaps an input (only outputs[r] == inputs[r] is allowed)");
    }
  }
  return MSCL_SUCCESS;
}

// AUTO's size bands (bytes per rank buffer), from device time per call on
// MI355X, bf16, calls replayed from a graph, over the same buffers ("hot")
// and over buffer sets rotated past the 256 MB Infinity Cache ("cold"); a
// band goes to the algorithm with the smaller hot + cold sum.  Every
// algorithm AUTO picks carries the method's synchronisation: the one-shot
// needs none, the two-shot runs its barrier between reduce-scatter and
// all-gather, the fused two-shot its completion barrier.
//   one-shot        up to oneshot_max_bytes(R): it reads R*S per rank, from
//                   cache while the buffers fit, and has no barrier (R = 8,
//                   256 KiB: 2.8 / 3.8 us against 3.6 / 4.4 fused; 512 KiB:
//                   4.2 / 6.5 against 3.9 / 5.0);
//   fused two-shot  up to fused_max_bytes(R): no re-read, one barrier at the
//                   end (R = 8, 2 MiB: 5.7 / 8.9 against 6.2 / 8.7 two-shot);
//                   with few ranks at every size (R = 3, 128 MiB: 145 against
//                   149);
//   two-shot        above: its separate read and write phases stream HBM best
//                   with many ranks (R = 8, 4 MiB 11.3 / 15.4 against
//                   12.4 / 15.0; 128 MiB 356 against 405 fused).
// In place the one-shot needs a barrier between each batch of tiles' loads
// and stores (a rank overwrites an input its peers still read), so in-place
// calls skip the first band; the fused band is then wider at R = 5 and 8
// (R = 8 in place, 8 MiB: 21.1 / 20.9 against 22.5 / 25.6).
size_t oneshot_max_bytes(int nranks) {
  const size_t env = config().oneshot_max_bytes;
  if (env != SIZE_MAX) return env;
  if (nranks <= 2) return size_t(8) << 20;  // R = 2, 8 MiB: 5.5 / 10.0 against 5.8 / 9.6 fused
  if (nranks == 3) return size_t(2) << 20;
  if (nranks <= 5) return size_t(1) << 20;  // R = 4, 2 MiB: 4.7 / 8.3 against 4.4 / 5.8 fused
  if (nranks <= 7) return size_t(512) << 10;
  if (nranks <= 11) return size_t(256) << 10;
  return size_t(128) << 10;  // R = 16, 256 KiB: 5.8 / 8.8 against 5.4 / 6.2 fused
}

// Up to this many bytes per rank buffer the fused two-shot also gets two
// workgroups per compute unit (make_plan).
constexpr size_t kFusedMaxBytes = size_t(4) << 20;

// The fused two-shot's upper bound in AUTO (see above).
size_t fused_max_bytes(int nranks, bool in_place) {
  switch (nranks) {
    case 1:
    case 2:
    case 3: return SIZE_MAX;
    case 4: return size_t(16) << 20;  // 32 MiB: 49.5 / 51.4 against 48.5 / 48.3 two-shot
    case 5: return in_place ? SIZE_MAX : size_t(8) << 20;
    case 8: return size_t(in_place ? 8 : 2) << 20;
    case 16: return size_t(256) << 10;  // 512 KiB: 7.1 / 8.2 against 6.3 / 7.7 two-shot
  }
  return size_t(1) << 20;  // R = 6, 7, 9..15; R = 12, 2 MiB: 14.0 / 15.0 against 10.0 / 13.0 two-shot
}

mscl_algo_t resolve_algo(size_t count, int dtype, int nranks, int algo, bool in_place) {
  if (algo != MSCL_ALGO_AUTO) return static_cast<mscl_algo_t>(algo);
  const size_t bytes = count * elem_bytes(dtype);
  if (!in_place && bytes <= oneshot_max_bytes(nranks)) return MSCL_ALGO_ONE_SHOT;
  if (nranks == 1) return MSCL_ALGO_ONE_SHOT;  // a copy (or nothing, in place)
  return bytes <= fused_max_bytes(nranks, in_place) ? MSCL_ALGO_TWO_SHOT_FUSED : MSCL_ALGO_TWO_SHOT;
}

// Put policy of the two-shot kernels.  Their puts stream past the caches
// unless the call's footprint (R inputs and R outputs, 2*R*S bytes) fits in
// half of the 256 MiB Infinity Cache; then device-scope temporal stores
// leave the outputs there for the kernel that reads them next.  Measured on
// MI355X, bf16, with a producer kernel writing the inputs before each call
// and a consumer kernel reading the outputs after it, replayed from a graph
// (the call's share of the time, streaming -> device-scope puts): fused
// two-shot R = 8 4 MiB 14.7 -> 11.1 us, 8 MiB 18.1 -> 13.8, R = 4 8 MiB
// 15.2 -> 11.4, R = 16 2 MiB 13.3 -> 11.7; two-shot R = 8 8 MiB 20.2 -> 15.2.
// With a 256 MiB footprint the gain is gone or reversed (fused R = 8 16 MiB
// 39.1 -> 41.5, R = 16 8 MiB 34.6 -> 35.1) and calls whose buffers are not
// cached pay 10-20% (two-shot R = 8 16 MiB 42.7 -> 51.1).
constexpr size_t kCachedPutsMaxFootprint = size_t(128) << 20;

// The held two-shot writes its outputs in a pure write phase, and there
// device-scope puts pay up to a 256 MiB footprint: R = 8, 16 MiB, streaming ->
// device-scope puts, 42.3 -> 38.7 us on the same buffers, 40.4 -> 32.6 us
// between a producer and a consumer kernel, 43.1 -> 43.0 us over four rotated
// buffer sets; at 512 MiB they lose between a producer and a consumer (R = 8,
// 32 MiB: 81.1 -> 92.7 us; R = 16, 16 MiB: 91.7 -> 97.0 us).
constexpr size_t kHeldCachedPutsMaxFootprint = size_t(256) << 20;
bool held_cached_puts(int nranks, size_t bytes) {
  if (bytes > (size_t(1) << 31)) return false;
  const size_t env = config().cached_puts_max_footprint;
  const size_t limit = env != SIZE_MAX ? env : kHeldCachedPutsMaxFootprint;
  return 2 * static_cast<size_t>(nranks) * bytes <= limit;
}

// Fewest full tiles per workgroup for which the held two-shot pays.  With
// device-scope puts (the put policy of calls up to 128-256 MiB of footprint)
// it pays from 4 tiles (us, unheld -> held, same buffers / four rotated
// buffer sets / between a producer and a consumer kernel: R = 6, 4 MiB
// 11.4 / 13.0 / 12.4 -> 10.7 / 12.1 / 11.6; R = 8, 8 MiB 21.5 / 24.0 / 22.4
// -> 21.2 / 22.6 / 21.7; R = 12, 8 MiB 34.5 / 36.4 / 32.5 -> 31.7 / 36.2 /
// 20.3); below 4 tiles per workgroup nothing is held.
constexpr uint64_t kHeldMinTiles = 4;

// Tiles per workgroup a slice of a large held two-shot aims at up to R = 8
// (R = 8, 128 MiB: slices of 16 tiles 352 us, of 32 tiles 360-364 us, of 8
// tiles 371 us, as one call 378 us).
constexpr uint64_t kSliceTiles = 16;
bool cached_puts(mscl_algo_t algo, int nranks, size_t bytes) {
  if (algo != MSCL_ALGO_TWO_SHOT && algo != MSCL_ALGO_TWO_SHOT_PERTILE && !is_fused(algo)) return false;
  if (bytes > (size_t(1) << 31)) return false;  // the two-shot's buffer store takes a 32-bit byte range
  const size_t env = config().cached_puts_max_footprint;
  const size_t limit = env != SIZE_MAX ? env : kCachedPutsMaxFootprint;
  return 2 * static_cast<size_t>(nranks) * bytes <= limit;
}

void make_plan(const mscl_channel_s* ch, size_t count, int dtype, mscl_algo_t algo, bool in_place,
               mscl_plan_t* plan, bool allow_slices = true) {
  const int R = ch->nranks;
  const uint64_t V = 16 / elem_bytes(dtype);
  uint64_t tile = static_cast<uint64_t>(kThreads) * unroll_for_runtime(R);
  const Config& cfg = config();
  memset(plan, 0, sizeof(*plan));
  plan->algo = algo;
  plan->nranks = R;
  plan->threads_per_workgroup = kThreads;
  plan->vectors_per_thread = unroll_for_runtime(R);
  plan->cached_puts = cached_puts(algo, R, count * elem_bytes(dtype)) ? 1 : 0;
  uint64_t vectors;  // full vectors one rank covers
  if (algo == MSCL_ALGO_TWO_SHOT || is_fused(algo) || algo == MSCL_ALGO_TWO_SHOT_PORT ||
      algo == MSCL_ALGO_TWO_SHOT_PERTILE) {
    const uint64_t per = (count + R - 1) / R;
    // Chunks are whole 16-byte vectors; from 32 pages of 4 KiB per rank up,
    // whole 4 KiB pages, so that every rank's chunk starts where its tiles
    // line up with the buffer's pages (a chunk starting 16 bytes off a page
    // measured 20-30% slower: R = 8 bf16, 12582912 -> 12582976 elements, held
    // two-shot 67.6 -> 81.4 us; fused 2097152 -> 2097216, 9.5 -> 12.3 us;
    // R = 16, 16777216 -> 16777280, 180.7 -> 221.1 us).  The last ranks' chunks
    // absorb the rounding (at most a page each); the sum does not depend on it.
    const uint64_t page = 4096 / elem_bytes(dtype);
    const uint64_t align = per >= 32 * page ? page : V;
    const uint64_t c = (per + align - 1) / align * align;
    plan->chunk_elems = c;
    vectors = c / V;
    plan->uses_barrier =
        (algo == MSCL_ALGO_TWO_SHOT || algo == MSCL_ALGO_TWO_SHOT_FUSED || algo == MSCL_ALGO_TWO_SHOT_PERTILE) ? 1 : 0;
  } else {
    vectors = count / V;
    plan->uses_barrier = in_place ? 1 : 0;
  }
  uint64_t want = std::max<uint64_t>(1, (vectors + tile - 1) / tile);
  // One workgroup per compute unit in total measured best for the streaming
  // phases (fewer concurrent streams keep HBM pages open longer).  The fused
  // two-shot takes two in AUTO's middle band, up to kFusedMaxBytes per rank,
  // where a rank's chunk is only a few tiles per workgroup (R = 8 bf16, 4 MiB:
  // 12.2 -> 10.3 us); above it two are slower (128 MiB: 390 -> 401 us).
  const bool fused_band = is_fused(algo) && count * elem_bytes(dtype) <= kFusedMaxBytes;
  const uint64_t per_cu = fused_band ? 2 : 1;
  const uint64_t total = cfg.wg_target_total ? cfg.wg_target_total : static_cast<uint64_t>(ch->cus) * per_cu;
  uint64_t cap = cfg.wg_per_rank ? cfg.wg_per_rank : std::max<uint64_t>(1, total / R);
  cap = std::min<uint64_t>(cap, ch->slots);  // every workgroup of a barrier must be resident
  if (fused_band && want < cap && want * R < static_cast<uint64_t>(ch->cus)) {
    // Too few 256-lane tiles to give every compute unit one: halve the
    // workgroup (and so the tile) to spread the loads over twice as many
    // workgroups (R = 8 bf16, 512 KiB: 16 -> 32 per rank, 2.79 -> 2.72 us;
    // R = 16 fp16, 256 KiB: 3.50 -> 3.13 us).  Where 256-lane tiles already
    // reach every compute unit, halving measured slower (R = 4 fp32, 2 MiB:
    // 3.19 -> 3.85 us).
    plan->threads_per_workgroup = kThreads / 2;
    tile /= 2;
    want = std::max<uint64_t>(1, (vectors + tile - 1) / tile);
  }
  uint64_t b = std::min(want, cap);
  if (algo == MSCL_ALGO_ONE_SHOT && cap >= kXcds)
    b = std::min((b + kXcds - 1) / kXcds * kXcds, cap / kXcds * kXcds);  // whole XCD groups
  plan->workgroups_per_rank = static_cast<int>(b);
  // The two-shot keeps every workgroup's reduced tiles in LDS across the
  // barrier (mscl_twoshot_held) when its whole share fits there and is large
  // enough to pay for the all-gather's extra store: kHeldMinTiles to kHeldTiles full
  // tiles per workgroup, one vector per lane, one workgroup per compute unit,
  // from R = 6 up (R = 5, where AUTO never takes the two-shot, measured
  // 3-4% slower held at 24-40 MiB and 2% faster sliced at 64-128 MiB; R = 6
  // and 7 gain 8-13% sliced at 64-128 MiB: R = 7, 128 MiB, 404 -> 350 us).
  plan->slices = 1;
  plan->slice_elems = count;
  if (algo == MSCL_ALGO_TWO_SHOT && cfg.two_shot_hold && plan->vectors_per_thread == 1 && R >= 6 &&
      b <= ch->held_slots) {
    const uint64_t per_slot = (vectors / tile + b - 1) / b;  // full tiles of the busiest workgroup
    if (per_slot >= kHeldMinTiles && per_slot <= static_cast<uint64_t>(kHeldTiles)) {
      plan->held_tiles = static_cast<int>(per_slot);
      plan->cached_puts = held_cached_puts(R, count * elem_bytes(dtype)) ? 1 : 0;
    } else if (per_slot > static_cast<uint64_t>(kHeldTiles) && allow_slices) {
      // Too large to hold: run the call as consecutive slices, each a
      // complete two-shot whose shares fit in LDS.  Slice boundaries keep
      // every rank's chunk a whole number of tiles (chunks that start off a
      // 4 KiB tile boundary measured far slower: R = 8, 128 MiB in 25.6 MiB
      // slices 417 us against 364 in 32 MiB ones).  Shares of 16 tiles
      // measured best with up to 8 ranks (R = 8, 128 MiB: 8 slices 352 us,
      // 4 slices 360-364, one call 378), the fewest slices that fit with
      // more (R = 16, 128 MiB: 4 slices 712-725 us, 8 slices 729-748, one
      // call 770-815).
      const uint64_t tile_elems = tile * V;
      const uint64_t unit = static_cast<uint64_t>(R) * tile_elems;
      uint64_t k = R <= 8 ? per_slot / kSliceTiles : (per_slot + kHeldTiles - 1) / kHeldTiles;
      for (; k >= 2 && k <= 1024; ++k) {
        const uint64_t m = ((count + k - 1) / k + unit - 1) / unit * unit;
        mscl_plan_t first;
        make_plan(ch, m, dtype, algo, in_place, &first, /*allow_slices=*/false);
        if (first.held_tiles == 0) {
          if ((m / unit + first.workgroups_per_rank - 1) / first.workgroups_per_rank < kHeldMinTiles) break;
          continue;  // a share still too large: one slice more
        }
        *plan = first;
        plan->slice_elems = m;
        plan->slices = static_cast<int>((count + m - 1) / m);
        plan->cached_puts = held_cached_puts(R, count * elem_bytes(dtype)) ? 1 : 0;  // the whole call's footprint
        // Slices that are a whole number of R tiles (all but a ragged last one:
        // m is a multiple of R tiles) deal their tiles to the ranks in turn, so
        // that at any moment every workgroup reads and writes one neighbourhood
        // of each buffer: R = 8, 128 MiB in 8 slices 347.8 -> 340.9 us, 64 MiB
        // 173.5 -> 168.8 us.  With more ranks it measured slower (R = 16,
        // 128 MiB in 4 slices: 678.8 -> 708.5 us), as it did for single held
        // launches (R = 8, 16 MiB: 42.6 -> 47.3 us on uncached buffers).
        plan->tile_interleave = (cfg.tile_interleave && R <= 8) ? 1 : 0;
        break;
      }
    }
  }
}

// The channel set for (current device, R) and its per-call controls.
struct Bound {
  mscl_channel_s* ch = nullptr;
  uint64_t timeout_us = 0;
  int drop_rank = -1;
  int double_rank = -1;
  int check_protocol = 0;
};

// SUCCESS, or the failure an earlier call recorded in the set's status word
// (a wait that timed out, or a port-channel request the proxy refused or
// could not issue), which stands until mscl_channel_reset.
mscl_status_t recorded_failure(const mscl_channel_s* ch) {
  const int s = __atomic_load_n(ch->status_host, __ATOMIC_ACQUIRE);
  if (s == MSCL_SUCCESS) return MSCL_SUCCESS;
  return fail(static_cast<mscl_status_t>(s), std::string("an earlier call on this channel set failed (") +
                                                 mscl_status_string(s) + "); call mscl_channel_reset");
}

mscl_status_t bind_channel(int nranks, Bound* b) {
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
  {
    std::lock_guard<std::mutex> lock(g_mutex);
    auto it = g_registry.find(std::make_pair(device, nranks));
    if (it == g_registry.end())
      return fail(MSCL_ERR_NOT_INITIALIZED, "call mscl_channel_create for this device and rank count first");
    b->ch = it->second;
    b->timeout_us = b->ch->wait_timeout_us ? b->ch->wait_timeout_us : config().wait_timeout_us;
    b->drop_rank = b->ch->drop_rank;
    b->double_rank = b->ch->double_rank;
    b->check_protocol = b->ch->check_protocol;
  }
  return recorded_failure(b->ch);
}

void fill_args(KernelArgs* a, const Bound& b, const void* const inputs[], void* const outputs[], int nranks,
               size_t count) {
  memset(a, 0, sizeof(*a));
  for (int r = 0; r < nranks; ++r) {
    a->in[r] = inputs[r];
    a->out[r] = outputs[r];
  }
  a->count = count;
  a->ch.inbound = b.ch->inbound;
  a->ch.consumed = b.ch->consumed;
  a->ch.seen = b.ch->inbound + static_cast<size_t>(nranks) * nranks * b.ch->slots;
  a->ch.progress = b.ch->consumed + static_cast<size_t>(nranks) * b.ch->slots;
  a->ch.status = b.ch->status_dev;
  a->ch.slots = b.ch->slots;
  a->ch.drop_rank = b.drop_rank;
  a->ch.double_rank = b.double_rank;
  a->ch.check_protocol = b.check_protocol;
  a->ch.timeout_ticks = b.timeout_us * b.ch->wall_clock_khz / 1000;
}

mscl_status_t launch(int kind, int dtype, int nranks, KernelArgs& a, void* stream) {
  KernelFn fn = kernel_lookup(kind, dtype, nranks);
  if (!fn) return fail(MSCL_ERR_INVALID_ARGUMENT, "no kernel for this dtype and rank count");
  const dim3 grid(static_cast<unsigned>(nranks) * a.nblk);
  if (log_level() >= 3)
    log_line(3, "launch kind " + std::to_string(kind) + " grid " + std::to_string(grid.x) + " x " +
                    std::to_string(threads_for_kind(kind)) + " count " + std::to_string(a.count));
  void* kargs[] = {&a};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(fn), grid, dim3(threads_for_kind(kind)), kargs, 0,
                                 static_cast<hipStream_t>(stream));
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) return fail_hip(e, "kernel launch");
  return MSCL_SUCCESS;
}

// Validation of ReduceScatter (gather = false: inputs hold R blocks, outputs
// one) and AllGather (gather = true: inputs hold one block, outputs R).
// Pointers need only element alignment; *vec tells whether every block
// boundary is 16-byte aligned.  In place: ReduceScatter's outputs[r] may be
// block r of inputs[r]; AllGather's inputs[r] may be block r of outputs[r]
// (bit r of *in_place_mask).  Any other overlap of an output with an input,
// or of two outputs, is rejected.
mscl_status_t validate_blocks(const void* const inputs[], void* const outputs[], size_t count, int dtype, int nranks,
                              bool gather, bool* vec, uint32_t* in_place_mask) {
  if (nranks < 1 || nranks > MSCL_MAX_RANKS) return fail(MSCL_ERR_INVALID_ARGUMENT, "nranks must be in 1..16");
  if (dtype != MSCL_FLOAT32 && dtype != MSCL_FLOAT16 && dtype != MSCL_BFLOAT16)
    return fail(MSCL_ERR_INVALID_ARGUMENT, "unknown dtype");
  if (!inputs || !outputs) return fail(MSCL_ERR_INVALID_ARGUMENT, "inputs/outputs array is null");
  const size_t e = elem_bytes(dtype);
  if (count > SIZE_MAX / e / static_cast<size_t>(nranks))
    return fail(MSCL_ERR_INVALID_ARGUMENT, "count * nranks * element size overflows");
  const uintptr_t blk = count * e;
  const uintptr_t in_len = gather ? blk : blk * nranks;
  const uintptr_t out_len = gather ? blk * nranks : blk;
  bool aligned16 = (blk % 16) == 0;
  for (int r = 0; r < nranks; ++r) {
    if (!inputs[r] || !outputs[r]) return fail(MSCL_ERR_INVALID_ARGUMENT, "null buffer pointer");
    const uintptr_t a = reinterpret_cast<uintptr_t>(inputs[r]);
    const uintptr_t o = reinterpret_cast<uintptr_t>(outputs[r]);
    if ((a % e) || (o % e)) return fail(MSCL_ERR_MISALIGNED, "buffers must be aligned to the element size");
    if (UINTPTR_MAX - a < in_len || UINTPTR_MAX - o < out_len)
      return fail(MSCL_ERR_INVALID_ARGUMENT, "buffer range wraps the address space");
    aligned16 = aligned16 && (a % 16) == 0 && (o % 16) == 0;
  }
  *vec = aligned16;
  *in_place_mask = 0;
  if (count == 0) return MSCL_SUCCESS;
  auto overlap = [](const void* x, uintptr_t xl, const void* y, uintptr_t yl) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(x), b = reinterpret_cast<uintptr_t>(y);
    return a < b + yl && b < a + xl;
  };
  for (int r = 0; r < nranks; ++r) {
    for (int q = r + 1; q < nranks; ++q)
      if (overlap(outputs[r], out_len, outputs[q], out_len)) return fail(MSCL_ERR_INVALID_ARGUMENT, "outputs overlap");
    for (int p = 0; p < nranks; ++p) {
      if (!overlap(outputs[r], out_len, inputs[p], in_len)) continue;
      const uintptr_t o = reinterpret_cast<uintptr_t>(outputs[r]);
      const uintptr_t i = reinterpret_cast<uintptr_t>(inputs[p]);
      const bool own_block = p == r && (gather ? i == o + r * blk : o == i + r * blk);
      if (!own_block)
        return fail(MSCL_ERR_INVALID_ARGUMENT,
                    gather ? "an input overlaps an output (only inputs[r] == outputs[r] + r * block is allowed)"
                           : "an output overlaps an input (only outputs[r] == inputs[r] + r * block is allowed)");
      if (gather) *in_place_mask |= 1u << r;
    }
  }
  return MSCL_SUCCESS;
}

// Workgroups per rank for ReduceScatter / AllGather: enough to cover a
// rank's block, at most one workgroup per compute unit in total.
uint32_t blocks_for(const mscl_channel_s* ch, size_t count, int dtype, int nranks, bool vec, bool gather) {
  const uint64_t per_lane = vec ? (gather ? kAllGatherU : unroll_for_runtime(nranks)) * (16 / elem_bytes(dtype)) : 1;
  const uint64_t per_wg = static_cast<uint64_t>(kThreads) * per_lane;
  const uint64_t want = std::max<uint64_t>(1, (count + per_wg - 1) / per_wg);
  const uint64_t cap = std::max<uint64_t>(1, static_cast<uint64_t>(ch->cus) / nranks);
  return static_cast<uint32_t>(std::min(want, cap));
}

// Barrier slots for `nranks` ranks on the current device: the fewest
// workgroups per rank that can be resident at once over every kernel that runs
// a barrier (so a barrier never waits on a workgroup that has not been
// scheduled), and the same bound for the held two-shot, whose 160 KiB of LDS
// leaves room for one workgroup per compute unit (kept apart so that the other
// kernels keep theirs).
hipError_t barrier_slots(int nranks, int cus, uint32_t* slots, uint32_t* held_slots) {
  int min_resident = 1 << 30;
  for (int dt = 0; dt < 3; ++dt) {
    for (int kind : {kAlgoOneShotInPlace, kAlgoTwoShot, kAlgoTwoShotCachedPuts, kAlgoTwoShotFusedSync,
                     kAlgoTwoShotFusedCachedPutsSync, kAlgoTwoShotFusedHalfSync, kAlgoTwoShotFusedHalfCachedPutsSync,
                     kAlgoTwoShotPerTile, kAlgoTwoShotPerTileCachedPuts}) {
      int per_cu = 0;
      const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu, reinterpret_cast<const void*>(kernel_lookup(kind, dt, nranks)), threads_for_kind(kind), 0);
      if (e != hipSuccess) return e;
      min_resident = std::min(min_resident, per_cu * cus);
    }
  }
  *slots = static_cast<uint32_t>(std::max(1, std::min(min_resident / nranks, 4096)));
  int held_resident = 1 << 30;
  for (int dt = 0; dt < 3; ++dt) {
    int per_cu = 0;
    for (int kind : {kAlgoTwoShotHeld, kAlgoTwoShotHeldInterleaved, kAlgoTwoShotHeldCachedPuts}) {
      const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu, reinterpret_cast<const void*>(kernel_lookup(kind, dt, nranks)), kThreads, 0);
      if (e != hipSuccess) return e;
      held_resident = std::min(held_resident, per_cu * cus);
    }
  }
  *held_slots = static_cast<uint32_t>(std::min<int>(held_resident / nranks, static_cast<int>(*slots)));
  return hipSuccess;
}

// The kernel kind a planned call (or slice) launches.
int kind_for(const mscl_plan_t& plan, bool in_place) {
  const bool cached = plan.cached_puts != 0;
  const bool wide = plan.threads_per_workgroup == kThreads;
  switch (plan.algo) {
    case MSCL_ALGO_TWO_SHOT:
      if (plan.held_tiles) return cached ? kAlgoTwoShotHeldCachedPuts : kAlgoTwoShotHeld;
      return cached ? kAlgoTwoShotCachedPuts : kAlgoTwoShot;
    case MSCL_ALGO_TWO_SHOT_FUSED:
      return wide ? (cached ? kAlgoTwoShotFusedCachedPutsSync : kAlgoTwoShotFusedSync)
                  : (cached ? kAlgoTwoShotFusedHalfCachedPutsSync : kAlgoTwoShotFusedHalfSync);
    case MSCL_ALGO_TWO_SHOT_FUSED_NOBARRIER:
      return wide ? (cached ? kAlgoTwoShotFusedCachedPuts : kAlgoTwoShotFused)
                  : (cached ? kAlgoTwoShotFusedHalfCachedPuts : kAlgoTwoShotFusedHalf);
    case MSCL_ALGO_TWO_SHOT_PORT:
      return kAlgoTwoShotPort;
    case MSCL_ALGO_TWO_SHOT_PERTILE:
      return cached ? kAlgoTwoShotPerTileCachedPuts : kAlgoTwoShotPerTile;
    default:
      return in_place ? kAlgoOneShotInPlace : kAlgoOneShot;
  }
}

// Launch a validated AllReduce as planned on `ch`'s geometry: one kernel, or
// one per slice for a sliced two-shot (each slice a complete two-shot on its
// own element range, planned on its own; an AllReduce is elementwise, so the
// result is the same), in stream order.  `proto` carries the channel state
// (and port arguments) every launch uses.
mscl_status_t launch_allreduce(const mscl_channel_s* ch, const KernelArgs& proto, const void* const inputs[],
                               void* const outputs[], size_t count, int dtype, int nranks, mscl_algo_t resolved,
                               bool in_place, void* stream) {
  mscl_plan_t plan;
  make_plan(ch, count, dtype, resolved, in_place, &plan);
  if (log_level() >= 2)
    log_line(2, "allreduce R=" + std::to_string(nranks) + " count=" + std::to_string(count) + " dtype=" +
                    std::to_string(dtype) + (in_place ? " in place" : "") + ": " + algo_name(plan.algo) + ", " +
                    std::to_string(plan.workgroups_per_rank) + " workgroups/rank x " +
                    std::to_string(plan.threads_per_workgroup) + " threads, barrier " +
                    std::to_string(plan.uses_barrier) + ", chunk " + std::to_string(plan.chunk_elems) +
                    ", cached_puts " + std::to_string(plan.cached_puts) + ", held_tiles " +
                    std::to_string(plan.held_tiles) + ", slices " + std::to_string(plan.slices) +
                    (plan.tile_interleave ? " (tiles interleaved)" : ""));
  const size_t e = elem_bytes(dtype);
  const size_t step = plan.slices > 1 ? plan.slice_elems : count;
  for (size_t lo = 0; lo < count; lo += step) {
    const size_t c = std::min(step, count - lo);
    KernelArgs a = proto;
    for (int r = 0; r < nranks; ++r) {
      a.in[r] = static_cast<const char*>(inputs[r]) + lo * e;
      a.out[r] = static_cast<char*>(outputs[r]) + lo * e;
    }
    a.count = c;
    mscl_plan_t sp = plan;
    if (plan.slices > 1) {
      make_plan(ch, c, dtype, resolved, in_place, &sp, /*allow_slices=*/false);
      sp.cached_puts = plan.cached_puts;  // a slice keeps the whole call's put policy
    }
    a.chunk = sp.chunk_elems;
    a.nblk = static_cast<uint32_t>(sp.workgroups_per_rank);
    a.xcd_grouped = (resolved == MSCL_ALGO_ONE_SHOT && a.nblk % kXcds == 0) ? 1u : 0u;
    int kind = kind_for(sp, in_place);
    if (plan.tile_interleave && c == plan.slice_elems && kind == kAlgoTwoShotHeld) kind = kAlgoTwoShotHeldInterleaved;
    if (const mscl_status_t st = launch(kind, dtype, nranks, a, stream); st != MSCL_SUCCESS) return st;
  }
  return MSCL_SUCCESS;
}

// ----------------------------------------------------------------------------
// Allocation-free AllReduce (mscl_allreduce_noalloc): the channel state lives
// in `scratch`, a device array of the library's own code object, so the call
// allocates nothing.  Layout for R ranks and a slot stride S (per device and
// R): inbound [R][R][S] counters, the per-tile semaphores' seen [R][R][S],
// consumed [R][S] counters, the per-tile semaphores' progress [R][S], then the
// status word.  Each call clears the words it uses (a fill kernel on the stream: no
// memset node in a captured graph) before its barrier kernels run, so a call
// never inherits the counters of an earlier one.
// ----------------------------------------------------------------------------

__global__ __launch_bounds__(kThreads) void mscl_scratch_clear(uint32_t* p, uint32_t nwords) {
  for (uint32_t i = threadIdx.x; i < nwords; i += kThreads) p[i] = 0u;
}

constexpr int kMaxDevices = 64;

struct NoAllocDevice {
  bool ready = false;
  uint32_t* scratch = nullptr;  // this device's copy of `scratch` (from hipGetSymbolAddress)
  int cus = 0;
  uint64_t wall_clock_khz = 100000;
  uint32_t slots[kMaxRanks + 1] = {};       // per R: slot stride (0 = not yet computed)
  uint32_t held_slots[kMaxRanks + 1] = {};
};

std::mutex g_noalloc_mutex;
NoAllocDevice g_noalloc[kMaxDevices];

// Set-up of the current device (once) and of R on it (once): the device
// address of `scratch`, the compute-unit count and the slot bounds.  Host
// queries only; nothing is allocated.
mscl_status_t noalloc_geometry(int device, int nranks, NoAllocDevice* out) {
  if (device < 0 || device >= kMaxDevices) return fail(MSCL_ERR_INVALID_ARGUMENT, "device ordinal out of range");
  std::lock_guard<std::mutex> lock(g_noalloc_mutex);
  NoAllocDevice& d = g_noalloc[device];
  if (!d.ready) {
    hipDeviceProp_t prop;
    hipError_t e = hipGetDeviceProperties(&prop, device);
    if (e != hipSuccess) return fail_hip(e, "hipGetDeviceProperties");
    if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
      return fail(MSCL_ERR_UNSUPPORTED, std::string("this library is built for gfx950, device is ") + prop.gcnArchName);
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return fail_hip(e, "hipGetSymbolAddress(scratch)");
    d.scratch = static_cast<uint32_t*>(ptr);
    d.cus = prop.multiProcessorCount;
    int khz = 0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, device) == hipSuccess && khz > 0)
      d.wall_clock_khz = static_cast<uint64_t>(khz);
    d.ready = true;
  }
  if (d.slots[nranks] == 0) {
    uint32_t slots = 0, held = 0;
    const hipError_t e = barrier_slots(nranks, d.cus, &slots, &held);
    if (e != hipSuccess) return fail_hip(e, "hipOccupancyMaxActiveBlocksPerMultiprocessor");
    // No launch has more than two workgroups per compute unit in total, so
    // that bounds the stride too; then it must fit the array.
    const uint32_t widest = static_cast<uint32_t>(std::max(1, 2 * d.cus / nranks));
    const uint32_t fits =
        static_cast<uint32_t>((kScratchWords - 1) / (2 * (static_cast<size_t>(nranks) * nranks + nranks)));
    slots = std::min({slots, widest, fits});
    if (slots == 0) return fail(MSCL_ERR_INVALID_ARGUMENT, "the scratch array cannot hold one barrier slot per rank");
    d.held_slots[nranks] = std::min(held, slots);
    d.slots[nranks] = slots;
  }
  *out = d;
  return MSCL_SUCCESS;
}

}  // namespace

extern "C" {

int mscl_version(void) { return MSCL_VERSION_MAJOR * 10000 + MSCL_VERSION_MINOR * 100 + MSCL_VERSION_PATCH; }

const char* mscl_status_string(mscl_status_t s) {
  switch (s) {
    case MSCL_SUCCESS: return "success";
    case MSCL_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MSCL_ERR_UNSUPPORTED: return "unsupported device";
    case MSCL_ERR_MISALIGNED: return "buffer misaligned (allreduce: 16 bytes; reduce-scatter, allgather: element size)";
    case MSCL_ERR_NOT_INITIALIZED: return "no channel set for this device and rank count";
    case MSCL_ERR_OUT_OF_MEMORY: return "out of memory";
    case MSCL_ERR_HIP: return "HIP runtime error";
    case MSCL_ERR_TIMEOUT: return "device-side wait timed out";
    case MSCL_ERR_PROTOCOL: return "a semaphore count that ordered calls cannot produce (overlapping calls on one channel set?)";
  }
  return "unknown status";
}

const char* mscl_last_error_string(void) { return g_last_error.c_str(); }

mscl_status_t mscl_select_algo(size_t count, mscl_dtype_t dtype, int nranks, mscl_algo_t* out) {
  if (!out) return fail(MSCL_ERR_INVALID_ARGUMENT, "out is null");
  if (nranks < 1 || nranks > MSCL_MAX_RANKS) return fail(MSCL_ERR_INVALID_ARGUMENT, "nranks must be in 1..16");
  if (dtype != MSCL_FLOAT32 && dtype != MSCL_FLOAT16 && dtype != MSCL_BFLOAT16)
    return fail(MSCL_ERR_INVALID_ARGUMENT, "unknown dtype");
  if (count > SIZE_MAX / elem_bytes(dtype)) return fail(MSCL_ERR_INVALID_ARGUMENT, "size overflows");
  *out = resolve_algo(count, dtype, nranks, MSCL_ALGO_AUTO, /*in_place=*/false);
  if (log_level() >= 2)
    log_line(2, "select R=" + std::to_string(nranks) + " count=" + std::to_string(count) + " dtype=" +
                    std::to_string(dtype) + ": " + algo_name(*out));
  return MSCL_SUCCESS;
}

mscl_status_t mscl_channel_create(int nranks, int device, mscl_channel_t* out) {
  if (!out) return fail(MSCL_ERR_INVALID_ARGUMENT, "out is null");
  *out = nullptr;
  if (nranks < 1 || nranks > MSCL_MAX_RANKS) return fail(MSCL_ERR_INVALID_ARGUMENT, "nranks must be in 1..16");
  if (device < 0) return fail(MSCL_ERR_INVALID_ARGUMENT, "device must be >= 0");
  std::lock_guard<std::mutex> lock(g_mutex);
  auto key = std::make_pair(device, nranks);
  auto it = g_registry.find(key);
  if (it != g_registry.end()) {
    it->second->refcount += 1;
    *out = it->second;
    return MSCL_SUCCESS;
  }
  int ndev = 0;
  hipError_t e = hipGetDeviceCount(&ndev);
  if (e != hipSuccess) return fail_hip(e, "hipGetDeviceCount");
  if (device >= ndev) return fail(MSCL_ERR_INVALID_ARGUMENT, "no such device");
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, device);
  if (e != hipSuccess) return fail_hip(e, "hipGetDeviceProperties");
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(MSCL_ERR_UNSUPPORTED, std::string("this library is built for gfx950, device is ") + prop.gcnArchName);
  int prev = 0;
  e = hipGetDevice(&prev);
  if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
  e = hipSetDevice(device);
  if (e != hipSuccess) return fail_hip(e, "hipSetDevice");

  auto* ch = new mscl_channel_s();
  ch->device = device;
  ch->nranks = nranks;
  ch->refcount = 1;
  ch->check_protocol = config().check_protocol ? 1 : 0;
  ch->cus = prop.multiProcessorCount;
  int khz = 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, device) == hipSuccess && khz > 0)
    ch->wall_clock_khz = static_cast<uint64_t>(khz);
  e = barrier_slots(nranks, ch->cus, &ch->slots, &ch->held_slots);
  if (e != hipSuccess) {
    delete ch;
    (void)hipSetDevice(prev);
    return fail_hip(e, "hipOccupancyMaxActiveBlocksPerMultiprocessor");
  }
  // Each array holds the barrier's counters followed by the per-tile
  // semaphores' (seen after inbound, progress after consumed).
  const size_t inbound_bytes = 2 * sizeof(uint32_t) * nranks * nranks * ch->slots;
  const size_t consumed_bytes = 2 * sizeof(uint32_t) * nranks * ch->slots;
  mscl_status_t st = MSCL_SUCCESS;
  if ((e = hipMalloc(&ch->inbound, inbound_bytes)) != hipSuccess ||
      (e = hipMalloc(&ch->consumed, consumed_bytes)) != hipSuccess) {
    st = fail(MSCL_ERR_OUT_OF_MEMORY, std::string("hipMalloc: ") + hipGetErrorString(e));
  } else if ((e = hipHostMalloc(&ch->status_host, sizeof(int), hipHostMallocMapped | hipHostMallocCoherent)) != hipSuccess) {
    st = fail(MSCL_ERR_OUT_OF_MEMORY, std::string("hipHostMalloc: ") + hipGetErrorString(e));
  } else if ((e = hipHostGetDevicePointer(reinterpret_cast<void**>(&ch->status_dev), ch->status_host, 0)) != hipSuccess) {
    st = fail_hip(e, "hipHostGetDevicePointer");
  } else {
    *ch->status_host = MSCL_SUCCESS;
    if ((e = hipMemset(ch->inbound, 0, inbound_bytes)) != hipSuccess ||
        (e = hipMemset(ch->consumed, 0, consumed_bytes)) != hipSuccess || (e = hipDeviceSynchronize()) != hipSuccess)
      st = fail_hip(e, "zeroing channel state");
  }
  if (st != MSCL_SUCCESS) {
    if (ch->inbound) (void)hipFree(ch->inbound);
    if (ch->consumed) (void)hipFree(ch->consumed);
    if (ch->status_host) (void)hipHostFree(ch->status_host);
    delete ch;
    (void)hipSetDevice(prev);
    return st;
  }
  (void)hipSetDevice(prev);
  g_registry[key] = ch;
  *out = ch;
  log_line(2, "channel set R=" + std::to_string(nranks) + " device " + std::to_string(device) + ": " +
                  std::to_string(ch->cus) + " compute units, " + std::to_string(ch->slots) + " slots, " +
                  std::to_string(ch->held_slots) + " held slots");
  return MSCL_SUCCESS;
}

mscl_status_t mscl_channel_destroy(mscl_channel_t ch) {
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!ch || !registered(ch)) return fail(MSCL_ERR_INVALID_ARGUMENT, "unknown channel handle");
  if (--ch->refcount > 0) return MSCL_SUCCESS;
  g_registry.erase(std::make_pair(ch->device, ch->nranks));
  port_stop(ch);
  int prev = 0;
  (void)hipGetDevice(&prev);
  (void)hipSetDevice(ch->device);
  hipError_t e1 = hipFree(ch->inbound);
  hipError_t e2 = hipFree(ch->consumed);
  hipError_t e3 = hipHostFree(ch->status_host);
  (void)hipSetDevice(prev);
  delete ch;
  if (e1 != hipSuccess) return fail_hip(e1, "hipFree");
  if (e2 != hipSuccess) return fail_hip(e2, "hipFree");
  if (e3 != hipSuccess) return fail_hip(e3, "hipHostFree");
  return MSCL_SUCCESS;
}

mscl_status_t mscl_channel_check(mscl_channel_t ch) {
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!ch || !registered(ch)) return fail(MSCL_ERR_INVALID_ARGUMENT, "unknown channel handle");
  return recorded_failure(ch);
}

mscl_status_t mscl_channel_reset(mscl_channel_t ch) {
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!ch || !registered(ch)) return fail(MSCL_ERR_INVALID_ARGUMENT, "unknown channel handle");
  int prev = 0;
  (void)hipGetDevice(&prev);
  (void)hipSetDevice(ch->device);
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = port_reset(ch);
  if (e == hipSuccess) e = hipMemset(ch->inbound, 0, 2 * sizeof(uint32_t) * ch->nranks * ch->nranks * ch->slots);
  if (e == hipSuccess) e = hipMemset(ch->consumed, 0, 2 * sizeof(uint32_t) * ch->nranks * ch->slots);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  (void)hipSetDevice(prev);
  if (e != hipSuccess) return fail_hip(e, "resetting channel state");
  __atomic_store_n(ch->status_host, MSCL_SUCCESS, __ATOMIC_RELEASE);
  return MSCL_SUCCESS;
}

mscl_status_t mscl_channel_set_fault_controls(mscl_channel_t ch, uint64_t wait_timeout_us, int drop_signal_rank) {
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!ch || !registered(ch)) return fail(MSCL_ERR_INVALID_ARGUMENT, "unknown channel handle");
  if (drop_signal_rank < -1 || drop_signal_rank >= ch->nranks)
    return fail(MSCL_ERR_INVALID_ARGUMENT, "drop_signal_rank must be -1 or a rank");
  ch->wait_timeout_us = std::min<uint64_t>(wait_timeout_us, 86400000000ull);  // at most a day
  ch->drop_rank = drop_signal_rank;
  return MSCL_SUCCESS;
}

mscl_status_t mscl_channel_set_checks(mscl_channel_t ch, int check_protocol, int double_signal_rank) {
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!ch || !registered(ch)) return fail(MSCL_ERR_INVALID_ARGUMENT, "unknown channel handle");
  if (double_signal_rank < -1 || double_signal_rank >= ch->nranks)
    return fail(MSCL_ERR_INVALID_ARGUMENT, "double_signal_rank must be -1 or a rank");
  ch->check_protocol = check_protocol ? 1 : 0;
  ch->double_rank = double_signal_rank;
  return MSCL_SUCCESS;
}

mscl_status_t mscl_channel_plan(mscl_channel_t ch, size_t count, mscl_dtype_t dtype, mscl_algo_t algo,
                                int in_place, mscl_plan_t* plan) {
  if (!plan) return fail(MSCL_ERR_INVALID_ARGUMENT, "plan is null");
  if (dtype != MSCL_FLOAT32 && dtype != MSCL_FLOAT16 && dtype != MSCL_BFLOAT16)
    return fail(MSCL_ERR_INVALID_ARGUMENT, "unknown dtype");
  if (!valid_algo(algo)) return fail(MSCL_ERR_INVALID_ARGUMENT, "unknown algo");
  if (count > SIZE_MAX / elem_bytes(dtype)) return fail(MSCL_ERR_INVALID_ARGUMENT, "size overflows");
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!ch || !registered(ch)) return fail(MSCL_ERR_INVALID_ARGUMENT, "unknown channel handle");
  make_plan(ch, count, dtype, resolve_algo(count, dtype, ch->nranks, algo, in_place != 0), in_place != 0, plan);
  return MSCL_SUCCESS;
}

mscl_status_t mscl_allreduce(const void* const inputs[], void* const outputs[], size_t count, mscl_dtype_t dtype,
                             int nranks, mscl_algo_t algo, void* stream) {
  bool in_place = false;
  mscl_status_t st = validate_call(inputs, outputs, count, dtype, nranks, algo, &in_place);
  if (st != MSCL_SUCCESS || count == 0) return st;
  if (nranks == 1 && in_place) return MSCL_SUCCESS;  // the sum of one buffer is already in place
  Bound b;
  if ((st = bind_channel(nranks, &b)) != MSCL_SUCCESS) return st;

  const mscl_algo_t resolved = resolve_algo(count, dtype, nranks, algo, in_place);
  KernelArgs a;
  fill_args(&a, b, inputs, outputs, nranks, count);
  if (resolved == MSCL_ALGO_TWO_SHOT_PORT) {
    std::lock_guard<std::mutex> lock(g_mutex);
    if ((st = port_start(b.ch)) != MSCL_SUCCESS) return st;
    const proxy::PortState* ps = b.ch->port;
    a.port.fifo = ps->fifo_dev;
    a.port.head = ps->head;
    a.port.done = ps->done_dev;
    a.port.issued = ps->issued;
    a.port.arrived = ps->arrived;
    a.port.fifo_mask = proxy::PortState::kEntries - 1;
  }
  return launch_allreduce(b.ch, a, inputs, outputs, count, dtype, nranks, resolved, in_place, stream);
}

mscl_status_t mscl_allreduce_noalloc(const void* const inputs[], void* const outputs[], size_t count,
                                     mscl_dtype_t dtype, int nranks, mscl_algo_t algo, void* stream) {
  bool in_place = false;
  mscl_status_t st = validate_call(inputs, outputs, count, dtype, nranks, algo, &in_place);
  if (st != MSCL_SUCCESS || count == 0) return st;
  if (algo == MSCL_ALGO_TWO_SHOT_PORT)
    return fail(MSCL_ERR_INVALID_ARGUMENT, "the port channel allocates its request ring: use mscl_allreduce");
  if (nranks == 1 && in_place) return MSCL_SUCCESS;
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
  NoAllocDevice d;
  if ((st = noalloc_geometry(device, nranks, &d)) != MSCL_SUCCESS) return st;
  mscl_channel_s geom;  // geometry only: no channel state is allocated or registered
  geom.device = device;
  geom.nranks = nranks;
  geom.cus = d.cus;
  geom.slots = d.slots[nranks];
  geom.held_slots = d.held_slots[nranks];

  const mscl_algo_t resolved = resolve_algo(count, dtype, nranks, algo, in_place);
  mscl_plan_t plan;
  make_plan(&geom, count, dtype, resolved, in_place, &plan);
  const uint32_t stride = geom.slots;
  const size_t pair = static_cast<size_t>(nranks) * nranks * stride, own = static_cast<size_t>(nranks) * stride;
  uint32_t words = static_cast<uint32_t>(2 * pair + 2 * own + 1);
  if (words > kScratchWords) return fail(MSCL_ERR_INVALID_ARGUMENT, "channel state exceeds the 128 KiB scratch array");
  KernelArgs a;
  memset(&a, 0, sizeof(a));
  a.ch.inbound = d.scratch;
  a.ch.seen = d.scratch + pair;
  a.ch.consumed = d.scratch + 2 * pair;
  a.ch.progress = d.scratch + 2 * pair + own;
  a.ch.status = reinterpret_cast<int*>(d.scratch + words - 1);
  a.ch.slots = stride;
  a.ch.drop_rank = -1;
  a.ch.double_rank = -1;
  a.ch.check_protocol = config().check_protocol ? 1 : 0;
  a.ch.timeout_ticks = config().wait_timeout_us * d.wall_clock_khz / 1000;
  if (plan.uses_barrier) {
    void* kargs[] = {&d.scratch, &words};
    e = hipLaunchKernel(reinterpret_cast<const void*>(&mscl_scratch_clear), dim3(1), dim3(kThreads), kargs, 0,
                        static_cast<hipStream_t>(stream));
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess) return fail_hip(e, "scratch clear launch");
  }
  return launch_allreduce(&geom, a, inputs, outputs, count, dtype, nranks, resolved, in_place, stream);
}

mscl_status_t mscl_reduce_scatter(const void* const inputs[], void* const outputs[], size_t recvcount,
                                  mscl_dtype_t dtype, int nranks, void* stream) {
  bool vec = false;
  uint32_t mask = 0;
  mscl_status_t st = validate_blocks(inputs, outputs, recvcount, dtype, nranks, /*gather=*/false, &vec, &mask);
  if (st != MSCL_SUCCESS || recvcount == 0) return st;
  Bound b;
  if ((st = bind_channel(nranks, &b)) != MSCL_SUCCESS) return st;
  KernelArgs a;
  fill_args(&a, b, inputs, outputs, nranks, recvcount);
  a.nblk = blocks_for(b.ch, recvcount, dtype, nranks, vec, /*gather=*/false);
  return launch(vec ? kReduceScatterVec : kReduceScatterElem, dtype, nranks, a, stream);
}

mscl_status_t mscl_allgather(const void* const inputs[], void* const outputs[], size_t sendcount, mscl_dtype_t dtype,
                             int nranks, void* stream) {
  bool vec = false;
  uint32_t mask = 0;
  mscl_status_t st = validate_blocks(inputs, outputs, sendcount, dtype, nranks, /*gather=*/true, &vec, &mask);
  if (st != MSCL_SUCCESS || sendcount == 0) return st;
  Bound b;
  if ((st = bind_channel(nranks, &b)) != MSCL_SUCCESS) return st;
  KernelArgs a;
  fill_args(&a, b, inputs, outputs, nranks, sendcount);
  a.nblk = blocks_for(b.ch, sendcount, dtype, nranks, vec, /*gather=*/true);
  a.in_place_mask = mask;
  return launch(vec ? kAllGatherVec : kAllGatherElem, dtype, nranks, a, stream);
}

mscl_status_t mscl_channel_selftest(mscl_channel_t ch, uint32_t rounds, uint64_t* mismatches) {
  if (!mismatches) return fail(MSCL_ERR_INVALID_ARGUMENT, "mismatches is null");
  *mismatches = 0;
  Bound b;
  {
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!ch || !registered(ch)) return fail(MSCL_ERR_INVALID_ARGUMENT, "unknown channel handle");
    b.ch = ch;
    b.timeout_us = ch->wait_timeout_us ? ch->wait_timeout_us : config().wait_timeout_us;
    b.drop_rank = ch->drop_rank;
    b.double_rank = ch->double_rank;
    b.check_protocol = ch->check_protocol;
  }
  if (const mscl_status_t st = recorded_failure(ch); st != MSCL_SUCCESS) return st;
  if (rounds == 0) return MSCL_SUCCESS;
  const int R = ch->nranks;
  KernelArgs a;
  const void* none_in[kMaxRanks] = {};
  void* none_out[kMaxRanks] = {};
  fill_args(&a, b, none_in, none_out, R, 0);
  a.nblk = std::max<uint32_t>(1, std::min<uint32_t>(ch->slots, static_cast<uint32_t>(ch->cus / R)));
  int prev = 0;
  (void)hipGetDevice(&prev);
  hipError_t e = hipSetDevice(ch->device);
  uint32_t* mailbox = nullptr;
  uint32_t* counter = nullptr;
  const size_t mb_bytes = sizeof(uint32_t) * kSelftestWords * R * a.nblk;
  if (e == hipSuccess) e = hipMalloc(&mailbox, mb_bytes);
  if (e == hipSuccess) e = hipMalloc(&counter, sizeof(uint32_t));
  if (e == hipSuccess) e = hipMemset(counter, 0, sizeof(uint32_t));
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e == hipSuccess) {
    using SelftestFn = void (*)(KernelArgs, uint32_t*, uint32_t, uint32_t*);
    SelftestFn table[kMaxRanks] = {
        &mscl_channel_selftest_kernel<1>,  &mscl_channel_selftest_kernel<2>,  &mscl_channel_selftest_kernel<3>,
        &mscl_channel_selftest_kernel<4>,  &mscl_channel_selftest_kernel<5>,  &mscl_channel_selftest_kernel<6>,
        &mscl_channel_selftest_kernel<7>,  &mscl_channel_selftest_kernel<8>,  &mscl_channel_selftest_kernel<9>,
        &mscl_channel_selftest_kernel<10>, &mscl_channel_selftest_kernel<11>, &mscl_channel_selftest_kernel<12>,
        &mscl_channel_selftest_kernel<13>, &mscl_channel_selftest_kernel<14>, &mscl_channel_selftest_kernel<15>,
        &mscl_channel_selftest_kernel<16>};
    void* kargs[] = {&a, &mailbox, &rounds, &counter};
    e = hipLaunchKernel(reinterpret_cast<const void*>(table[R - 1]), dim3(static_cast<unsigned>(R) * a.nblk),
                        dim3(kThreads), kargs, 0, nullptr);
  }
  uint32_t host_count = 0;
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(&host_count, counter, sizeof(uint32_t), hipMemcpyDeviceToHost);
  if (mailbox) (void)hipFree(mailbox);
  if (counter) (void)hipFree(counter);
  (void)hipSetDevice(prev);
  if (e != hipSuccess) return fail_hip(e, "channel self-test");
  *mismatches = host_count;
  if (__atomic_load_n(ch->status_host, __ATOMIC_ACQUIRE) != MSCL_SUCCESS)
    return fail(MSCL_ERR_TIMEOUT, "a wait timed out during the self-test");
  return MSCL_SUCCESS;
}

}  // extern "C"
