// MemoryChannel-style collectives over R emulated peer ranks on one gfx950 GPU.
//
// The MSCCL++ pages present AllReduce as the collective their library speeds
// up for tensor-parallel LLM serving (project summary, "Highlighted
// Details"), built from GPU-side channel methods (README, Key Concepts,
// "On-GPU Communication Interfaces: Channels") of which the MemoryChannel
// moves data with many GPU threads loading and storing peer memory directly
// ("PortChannel and MemoryChannel").  This header holds the device side: the
// kernels and the table the host code launches them from (mscl.hip holds
// the host side of the C ABI declared in include/mscl.h):
//
//   mscl_oneshot        every rank reads all R inputs and writes its own
//                       output; in place, a barrier that waits for every
//                       rank's loads of a tile separates them from the
//                       tile's stores (a rank overwrites an input its peers
//                       are still reading).
//   mscl_twoshot        reduce-scatter (rank r reduces chunk r of all
//                       inputs into its own output), an arrival-only
//                       barrier, all-gather (rank r puts its chunk into every
//                       peer's output).
//   mscl_twoshot_held   the two-shot with each workgroup's reduced tiles kept
//                       in LDS across the barrier (no store and re-read of
//                       the rank's chunk); the host runs large calls as
//                       consecutive slices of it.
//   mscl_twoshot_fused  reduce-scatter whose result goes from registers
//                       straight into every output as device-scope puts,
//                       then a completion barrier (or, as an explicitly
//                       requested variant, no barrier).
//   mscl_twoshot_pertile
//                       reduce-scatter that signals every finished tile on a
//                       per-tile semaphore, and an all-gather that gets each
//                       peer's tile as soon as its semaphore shows it.
//   mscl_twoshot_port   reduce-scatter, then all-gather puts posted to a host
//                       proxy that copies them with the DMA engines.
//   mscl_reduce_scatter_kernel / mscl_allgather_kernel
//                       the two halves as standard collectives.
//   mscl_channel_selftest_kernel
//                       the barriers' publish/acquire and write-after-read
//                       contracts.
//
// Rank layout.  Workgroup w of a launch is emulated rank (w % R), channel
// slot (w / R); with the hardware's round-robin dispatch of workgroups over
// the 8 XCDs, a rank's workgroups stay on a fixed XCD subset.  The one-shot
// instead groups the R ranks of a slot on one XCD, because there every rank
// re-reads the same input lines.  Each workgroup has 256 threads (4
// wavefronts of 64; the fused two-shot also comes in a 128-thread form for
// small messages); a tile is U 16-byte vectors per lane.
//
// Two-shot chunks: rank r owns elements [r*c, min((r+1)*c, n)) with
// c = roundup(ceil(n/R), V), V = 16 / element size (rounded up to whole
// 4 KiB pages for large chunks; the slices of large held calls instead deal
// whole tiles to the ranks in turn).  Each lane handles the same vectors in
// both phases, which keeps in-place calls safe: the only reader of
// in[p][chunk r] is rank r itself, earlier, in the same lane.
//
// Every reduction adds in rank order 0..R-1 starting from rank 0's value and
// rounds once, so all algorithms give bit-identical results.


#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <utility>

#include "../../include/mscl.h"
#include "channel.hpp"
#include "codec.hpp"
#include "port.hpp"

namespace mscl {

constexpr int kThreads = 256;

// gfx950 parts (MI350 series) have 8 accelerator complex dies (XCDs), each
// with its own L2; the dispatcher deals workgroups to them round-robin, so
// workgroup w runs on XCD w % 8.
constexpr int kXcds = 8;

// 16-byte vectors per thread per rank buffer per tile.  With the software
// pipelining of the two-shot, one vector per rank buffer (R loads in flight
// per lane, 2R while the next tile is prefetched) measured fastest for R >= 5
// on MI355X; small R keeps 8+ loads in flight with two or four.
template <int R>
constexpr int unroll_for() {
  return R <= 2 ? 4 : (R <= 4 ? 2 : 1);
}

struct KernelArgs {
  const void* in[kMaxRanks];
  void* out[kMaxRanks];
  uint64_t count;  // elements per rank buffer
  uint64_t chunk;  // two-shot: elements per rank chunk, a multiple of V
  uint32_t nblk;   // workgroups (slots) per rank in this launch
  uint32_t xcd_grouped;  // one-shot: all ranks of a slot on one XCD (needs nblk % 8 == 0)
  uint32_t in_place_mask;  // allgather: bit r set when rank r's input already is its own output block
  ChannelArgs ch;
  PortArgs port;  // two-shot over a port channel only
};

// binary32 sum of one 16-byte vector position over the R ranks, in rank
// order starting from rank 0's value, rounded once to the element type.
template <class C, int R>
__device__ inline u32x4 reduce_vec(const u32x4 (&x)[R]) {
  float acc[C::V];
  C::unpack(x[0], acc);
#pragma unroll
  for (int p = 1; p < R; ++p) {
    float t[C::V];
    C::unpack(x[p], t);
#pragma unroll
    for (int i = 0; i < C::V; ++i) acc[i] = acc[i] + t[i];
  }
  return C::pack(acc);
}

// The partial vector at the end of the buffer (n % V elements), reduced by
// a single thread.
template <class C, int R>
__device__ inline u32x4 reduce_partial(const KernelArgs& a, uint64_t vi, int ntail) {
  u32x4 x[R];
#pragma unroll
  for (int p = 0; p < R; ++p) x[p] = load_partial<C>(a.in[p], vi, ntail);
  return reduce_vec<C, R>(x);
}

// A tile is U*256 consecutive 16-byte vectors: lane l of the workgroup takes
// vectors base+l, base+256+l, ... so each wavefront instruction covers 1 KiB
// contiguous.  Full tiles (kFull) need no bounds checks, which keeps every
// load of the tile issued back to back; the last, partial tile re-reads the
// range's last vector in lanes past the end and skips their stores.
template <int R, int U, bool kFull, bool kStream, int T = kThreads>
__device__ inline void load_tile(u32x4 (&x)[U][R], const void* const* src, uint64_t base, uint64_t vend) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    uint64_t vi = base + static_cast<uint64_t>(u) * T;
    if (!kFull) vi = std::min<uint64_t>(vi, vend - 1);
#pragma unroll
    for (int p = 0; p < R; ++p) x[u][p] = kStream ? load_vec_nt(src[p], vi) : load_vec(src[p], vi);
  }
}

// Store policy of a tile: cacheable (data re-read inside the call),
// streaming (written once, not read soon), or device-scope temporal (a put
// whose destination the next kernel reads while the call's buffers fit the
// Infinity Cache; stores stay below vend, so vend * 16 bytes bound the range).
// The host uses the device-scope form only for buffers below 2 GiB; should a
// larger range ever reach it, the range is zero and its stores are dropped
// rather than written at a wrapped 32-bit offset.
enum class Put { kCached, kStream, kDevice };

template <int U, bool kFull, Put kP, int T = kThreads>
__device__ inline void store_tile(void* dst, const u32x4 (&y)[U], uint64_t base, uint64_t vend) {
  const uint32_t range = vend * 16 <= 0xFFFFFFFFull ? static_cast<uint32_t>(vend * 16) : 0u;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint64_t vi = base + static_cast<uint64_t>(u) * T;
    if (kFull || vi < vend) {
      if constexpr (kP == Put::kStream)
        store_vec_nt(dst, vi, y[u]);
      else if constexpr (kP == Put::kDevice)
        store_vec_device(dst, range, vi, y[u]);
      else
        store_vec(dst, vi, y[u]);
    }
  }
}

template <class C, int R, int U>
__device__ inline void reduce_tile(u32x4 (&y)[U], const u32x4 (&x)[U][R]) {
#pragma unroll
  for (int u = 0; u < U; ++u) y[u] = reduce_vec<C, R>(x[u]);
}

// One tile of the one-shot: all R inputs reduced into this lane's vectors.
template <class C, int R, int U, bool kFull>
__device__ inline void oneshot_reduce(u32x4 (&y)[U], const KernelArgs& a, uint64_t base, uint64_t vend) {
  u32x4 x[U][R];
  load_tile<R, U, kFull, false>(x, a.in, base, vend);  // every rank re-reads these: keep them cached
  reduce_tile<C, R, U>(y, x);
}

// In place, tiles reduced per barrier: up to 8 vectors per lane are held in
// registers between a batch's loads and its stores.
template <int U>
constexpr int inplace_batch() {
  return 8 / U > 0 ? 8 / U : 1;
}

template <class C, int R, bool kInPlace>
__global__ __launch_bounds__(kThreads) void mscl_oneshot(KernelArgs a) {
  constexpr int V = C::V;
  constexpr int U = unroll_for<R>();
  constexpr uint64_t kTile = static_cast<uint64_t>(kThreads) * U;
  // Every rank reads the same tile of all R inputs.  Putting the R ranks'
  // workgroups of one slot on the same XCD lets that XCD's L2 serve the R-fold
  // re-reads of each line (measured: R = 8 at 1 MiB per rank, 12.2 -> 6.6 us).
  const int w = blockIdx.x;
  const int rank = a.xcd_grouped ? (w / kXcds) % R : w % R;
  const int slot = a.xcd_grouped ? (w / kXcds / R) * kXcds + w % kXcds : w / R;
  const uint64_t B = a.nblk;
  const uint64_t n = a.count;
  const uint64_t nfull = n / V;
  const int ntail = static_cast<int>(n % V);
  const uint64_t ntiles = (nfull + kTile - 1) / kTile;
  const RankChannels chans{a.ch, R, rank, slot};
  void* const dst = a.out[rank];

  if constexpr (!kInPlace) {
    for (uint64_t t = slot; t < ntiles; t += B) {
      const uint64_t base = t * kTile + threadIdx.x;
      u32x4 y[U];
      if ((t + 1) * kTile <= nfull) {
        oneshot_reduce<C, R, U, true>(y, a, base, nfull);
        store_tile<U, true, Put::kCached>(dst, y, base, nfull);
      } else {
        oneshot_reduce<C, R, U, false>(y, a, base, nfull);
        store_tile<U, false, Put::kCached>(dst, y, base, nfull);
      }
    }
  } else {
    // Peers read this rank's input until they signal; their loads of a batch
    // of tiles must be complete before this rank overwrites those tiles
    // (write after read across ranks, no data handed over), so one barrier
    // separates each batch's loads from its stores.  Every rank's slot runs
    // the same number of batches.
    constexpr int H = inplace_batch<U>();
    for (uint64_t t0 = slot; t0 < ntiles; t0 += H * B) {
      u32x4 y[H][U];
#pragma unroll
      for (int h = 0; h < H; ++h) {
        const uint64_t t = t0 + h * B;
        const uint64_t base = t * kTile + threadIdx.x;
        if ((t + 1) * kTile <= nfull)
          oneshot_reduce<C, R, U, true>(y[h], a, base, nfull);
        else if (t < ntiles)
          oneshot_reduce<C, R, U, false>(y[h], a, base, nfull);
      }
      chans.template barrier_all<Sync::kAfterReads>();
#pragma unroll
      for (int h = 0; h < H; ++h) {
        const uint64_t t = t0 + h * B;
        const uint64_t base = t * kTile + threadIdx.x;
        if ((t + 1) * kTile <= nfull)
          store_tile<U, true, Put::kCached>(dst, y[h], base, nfull);
        else if (t < ntiles)
          store_tile<U, false, Put::kCached>(dst, y[h], base, nfull);
      }
    }
  }

  if (ntail != 0 && slot == 0) {
    u32x4 y = {0u, 0u, 0u, 0u};
    if (threadIdx.x == 0) y = reduce_partial<C, R>(a, nfull, ntail);
    if constexpr (kInPlace) chans.template barrier_all<Sync::kAfterReads>();
    if (threadIdx.x == 0) store_partial<C>(dst, nfull, y, ntail);
  }
}

// Cache policy of the two-shot: inputs are read exactly once, so they
// stream past the caches; the rank's own reduced chunk is written and read
// back, so it stays cacheable.  The peers' outputs are written once inside
// the call; the put policy (streaming, or device-scope temporal when the
// call's buffers fit the Infinity Cache and the next kernel will find the
// outputs there) is a template parameter the host picks by size.
constexpr bool kStreamRsLoads = true;

template <bool kCachedPuts>
constexpr Put put_policy() {
  return kCachedPuts ? Put::kDevice : Put::kStream;
}

template <int R, int U, bool kFull, Put kP>
__device__ inline void ag_store(const KernelArgs& a, int rank, const u32x4 (&y)[U], uint64_t base, uint64_t vend) {
#pragma unroll
  for (int p = 0; p < R; ++p)  // put() to every peer, written once
    if (p != rank) store_tile<U, kFull, kP>(a.out[p], y, base, vend);
}

template <int U, bool kFull>
__device__ inline void ag_load(u32x4 (&y)[U], const void* mine, uint64_t base, uint64_t vend) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    uint64_t vi = base + static_cast<uint64_t>(u) * kThreads;
    if (!kFull) vi = std::min<uint64_t>(vi, vend - 1);
    y[u] = load_vec(mine, vi);
  }
}

// Rank `rank`'s two-shot chunk, seen from one slot: elements [lo, hi), its
// full 16-byte vectors [v_lo, v_full), the partial vector's element count,
// and the slot's tiles t = slot, slot + B, ...: tiles below `nfull_tiles` lie
// wholly inside the chunk; at most one partial tile (index nfull_tiles)
// follows.
struct Chunk {
  uint64_t lo, hi, v_lo, v_full, nfull_tiles;
  int ntail;  // nonzero only for the non-empty chunk that holds the buffer's end
  bool owns_partial_tile;
};

template <class C, int U>
__device__ inline Chunk chunk_of(const KernelArgs& a, int rank, int slot) {
  constexpr int V = C::V;
  constexpr uint64_t kTile = static_cast<uint64_t>(kThreads) * U;
  Chunk g;
  g.lo = std::min<uint64_t>(static_cast<uint64_t>(rank) * a.chunk, a.count);
  g.hi = std::min<uint64_t>(g.lo + a.chunk, a.count);
  g.v_lo = g.lo / V;  // chunk starts are multiples of V
  g.v_full = g.hi / V;
  g.ntail = g.hi > g.lo ? static_cast<int>(g.hi % V) : 0;
  const uint64_t nv = g.v_full - g.v_lo;
  g.nfull_tiles = nv / kTile;
  g.owns_partial_tile = (nv % kTile) != 0 && slot == static_cast<int>(g.nfull_tiles % a.nblk);
  return g;
}

// Reduced tiles one workgroup of the held two-shot keeps in LDS: 40 tiles of
// 256 lanes x 16 bytes = 160 KiB, all of a gfx950 compute unit's LDS.
constexpr int kHeldTiles = 40;
constexpr int kStatusInvalid = 1;  // MSCL_ERR_INVALID_ARGUMENT in the channel's status word

// A slot's full tiles t = slot, slot + B, ... (all below nfull_tiles), of
// which the newest `held` ones (j >= first_held, j counting the slot's tiles
// from 0) stay in LDS instead of going to the rank's own output.
struct Held {
  u32x4 (*lds)[kThreads];  // [kHeldTiles][kThreads], or null: nothing held
  uint64_t first_held;
};

__device__ inline Held held_range(u32x4 (*lds)[kThreads], uint64_t nfull_tiles, int slot, uint64_t B) {
  if (!lds || static_cast<uint64_t>(slot) >= nfull_tiles) return Held{lds, ~0ull};
  const uint64_t nts = (nfull_tiles - 1 - slot) / B + 1;
  return Held{lds, nts > kHeldTiles ? nts - kHeldTiles : 0};
}

// Reduce-scatter: chunk `rank` of every input -> own output `mine` (or, for
// the tiles `h` names, this lane's LDS slots).  The lane's vector of the
// rank's tile t is vector lane_base + t * tstride of every buffer (tstride is
// one tile for a contiguous chunk, R tiles for interleaved shares).
// Software pipelined: the loads of the slot's next tile are issued before
// the current tile is reduced and stored, so each wave keeps R*U 16-byte
// loads in flight while it computes.
template <class C, int R, bool kHold = false>
__device__ inline void twoshot_reduce_scatter(const KernelArgs& a, const Chunk& g, int slot, void* mine,
                                              uint64_t lane_base, uint64_t tstride,
                                              const Held h = Held{nullptr, ~0ull}) {
  constexpr int U = unroll_for<R>();
  const uint64_t B = a.nblk;
  if (static_cast<uint64_t>(slot) < g.nfull_tiles) {
    uint64_t t = slot;
    uint64_t j = 0;  // index of t among this slot's tiles
    u32x4 cur[U][R];
    load_tile<R, U, true, kStreamRsLoads>(cur, a.in, lane_base + t * tstride, g.v_full);
    while (true) {
      const uint64_t tn = t + B;
      const bool more = tn < g.nfull_tiles;
      u32x4 nxt[U][R];
      if (more) load_tile<R, U, true, kStreamRsLoads>(nxt, a.in, lane_base + tn * tstride, g.v_full);
      u32x4 y[U];
      reduce_tile<C, R, U>(y, cur);
      if constexpr (kHold && U == 1) {
        if (j >= h.first_held) {
          h.lds[j - h.first_held][threadIdx.x] = y[0];  // kept for the all-gather, read back by this lane only
        } else {
          store_tile<U, true, Put::kCached>(mine, y, lane_base + t * tstride, g.v_full);  // re-read by the all-gather
        }
      } else {
        store_tile<U, true, Put::kCached>(mine, y, lane_base + t * tstride, g.v_full);  // re-read by the all-gather
      }
      ++j;
      if (!more) break;
      for (int u = 0; u < U; ++u)
        for (int p = 0; p < R; ++p) cur[u][p] = nxt[u][p];
      t = tn;
    }
  }
  if (g.owns_partial_tile) {
    u32x4 x[U][R];
    u32x4 y[U];
    const uint64_t base = lane_base + g.nfull_tiles * tstride;
    load_tile<R, U, false, kStreamRsLoads>(x, a.in, base, g.v_full);
    reduce_tile<C, R, U>(y, x);
    store_tile<U, false, Put::kCached>(mine, y, base, g.v_full);
  }
  if (g.ntail != 0 && slot == 0 && threadIdx.x == 0)
    store_partial<C>(mine, g.v_full, reduce_partial<C, R>(a, g.v_full, g.ntail), g.ntail);
}

// A rank's share when whole tiles are dealt to the ranks in turn (tile T to
// rank T mod R), for calls whose length is a whole number of R tiles: every
// rank then has count / (R * tile) full tiles and nothing else.  Tile t of
// the rank is the call's tile t * R + rank.
template <class C, int R, int U>
__device__ inline Chunk interleaved_share(const KernelArgs& a) {
  constexpr uint64_t kTile = static_cast<uint64_t>(kThreads) * U;
  Chunk g;
  g.lo = 0;
  g.hi = a.count;
  g.v_lo = 0;
  g.v_full = a.count / C::V;
  g.ntail = 0;
  g.nfull_tiles = g.v_full / kTile / R;
  g.owns_partial_tile = false;
  return g;
}

// kIlv: tiles dealt to the ranks in turn (interleaved_share) instead of one
// contiguous chunk per rank; the host uses it only for whole-R-tile slices.
template <class C, int R, bool kCachedPuts, bool kHold, bool kIlv = false>
__device__ inline void twoshot_body(const KernelArgs& a, u32x4 (*lds)[kThreads]) {
  constexpr int U = unroll_for<R>();
  constexpr Put kP = put_policy<kCachedPuts>();
  constexpr uint64_t kTile = static_cast<uint64_t>(kThreads) * U;
  const int rank = blockIdx.x % R;
  const int slot = blockIdx.x / R;
  const uint64_t B = a.nblk;
  const Chunk g = kIlv ? interleaved_share<C, R, U>(a) : chunk_of<C, U>(a, rank, slot);
  // vector index of this lane's vector in the rank's tile t: lane_base + t * tstride
  const uint64_t tstride = kIlv ? kTile * R : kTile;
  const uint64_t v_full = g.v_full, nfull_tiles = g.nfull_tiles;
  const int ntail = g.ntail;
  const bool owns_partial_tile = g.owns_partial_tile;
  const RankChannels chans{a.ch, R, rank, slot};
  void* const mine = a.out[rank];
  const uint64_t lane_base = (kIlv ? static_cast<uint64_t>(rank) * kTile : g.v_lo) + threadIdx.x;

  const Held h = held_range(lds, nfull_tiles, slot, B);
  twoshot_reduce_scatter<C, R, kHold>(a, g, slot, mine, lane_base, tstride, h);
  const bool tail_owner = ntail != 0 && slot == 0 && threadIdx.x == 0;

  // signal / wait with the same slot of every peer rank.  Arrival only: no
  // data crosses ranks here.  The all-gather below reads only vectors this
  // lane itself wrote above (program order), and writes peer locations that
  // no peer reads during this call (rank p reads only its own chunk of every
  // input, and in place rank r alone reads in[p][chunk r], earlier, in this
  // lane).  Publishing or acquiring memory here would only cost an L2
  // write-back and invalidate per workgroup.
  chans.template barrier_all<Sync::kArrival>();

  // All-gather: put the reduced chunk into every peer's output, newest tiles
  // first (they are the likeliest to still be in cache), again pipelined one
  // tile ahead.  The same workgroup handles the same vectors as in the
  // reduce-scatter, so in-place calls stay safe.
  if (tail_owner) {
    const u32x4 y = load_partial<C>(mine, v_full, ntail);
    put_to_peers<C, R>(a.out, rank, v_full, y, v_full, ntail);
  }
  if (owns_partial_tile) {
    u32x4 y[U];
    const uint64_t base = lane_base + nfull_tiles * tstride;
    ag_load<U, false>(y, mine, base, v_full);
    ag_store<R, U, false, kP>(a, rank, y, base, v_full);
  }
  if (static_cast<uint64_t>(slot) < nfull_tiles) {
  if constexpr (kHold && U == 1) {
    // Every full tile of this slot is in LDS: the all-gather writes each to
    // the rank's own output and to every peer's.  The host launches this
    // kernel only when a workgroup's whole share fits (at most kHeldTiles
    // tiles); a share that does not is recorded as a failed call, not served
    // in part.  (The partial form, with the remaining tiles re-read and put
    // by the pipelined loop below, gained nothing where measured, and the
    // ROCm 7.2 compiler built that loop wrongly in this kernel: its select
    // of the next tile read a carry flag left by an unrelated add.)
    if (h.first_held != 0) {
      if (threadIdx.x == 0) __hip_atomic_store(a.ch.status, kStatusInvalid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      return;
    }
    // The held tiles go out one output at a time, two tiles per step: each
    // workgroup streams into one buffer, which measured faster on MI355X than
    // writing each tile to all R outputs in turn (R = 8, 32 MiB: 85.9 -> 84.2
    // us; R = 16, 32 MiB: 175.8 -> 165.4 us).  With more than 16 tiles per
    // workgroup rank r starts at output r, so the ranks' streams go to
    // different buffers; with 16 or fewer (the slices of large calls) every
    // rank starting at output 0 measured faster (R = 8, 128 MiB in 8 slices:
    // 347.4 us against 354.3 rotated and 350.1 tile by tile).
    const uint64_t nts = (nfull_tiles - 1 - slot) / B + 1;
    const int rot = nts > 16 ? rank : 0;
    for (int pp = 0; pp < R; ++pp) {
      void* const dst = a.out[(pp + rot) % R];
      uint64_t j = nts;
      for (; j >= 2; j -= 2) {
        u32x4 y0[U], y1[U];
        y0[0] = h.lds[j - 1][threadIdx.x];
        y1[0] = h.lds[j - 2][threadIdx.x];
        store_tile<U, true, kP>(dst, y0, lane_base + (slot + (j - 1) * B) * tstride, v_full);
        store_tile<U, true, kP>(dst, y1, lane_base + (slot + (j - 2) * B) * tstride, v_full);
      }
      if (j == 1) {
        u32x4 y[U];
        y[0] = h.lds[0][threadIdx.x];
        store_tile<U, true, kP>(dst, y, lane_base + slot * tstride, v_full);
      }
    }
  } else {
    uint64_t t = slot + (nfull_tiles - 1 - slot) / B * B;  // this slot's last full tile
    u32x4 cur[U];
    ag_load<U, true>(cur, mine, lane_base + t * tstride, v_full);
    while (true) {
      const bool more = t >= static_cast<uint64_t>(slot) + B;
      const uint64_t tn = more ? t - B : t;
      u32x4 nxt[U];
      if (more) ag_load<U, true>(nxt, mine, lane_base + tn * tstride, v_full);
      ag_store<R, U, true, kP>(a, rank, cur, lane_base + t * tstride, v_full);
      if (!more) break;
#pragma unroll
      for (int u = 0; u < U; ++u) cur[u] = nxt[u];
      t = tn;
    }
  }
  }
}

template <class C, int R, bool kCachedPuts>
__global__ __launch_bounds__(kThreads) void mscl_twoshot(KernelArgs a) {
  twoshot_body<C, R, kCachedPuts, false>(a, nullptr);
}

// The two-shot with each workgroup's newest reduced tiles (up to kHeldTiles
// per lane, 160 KiB) kept in LDS across the barrier: those tiles skip the
// store to the rank's own output during the reduce-scatter and its re-read
// during the all-gather, which writes them to every output, the rank's own
// included, so the call moves 2*R*S bytes when a workgroup's whole share is
// held.  Its LDS leaves room for one workgroup per compute unit.  Measured on
// MI355X, R = 8 bf16, where the host uses it (4 to 40 tiles per workgroup):
// 16 MiB 44.3 -> 43.3 us, 32 MiB 92.0 -> 87.2 us; R = 16: 16 MiB 93.1 -> 89.2
// us, 32 MiB 191.2 -> 178.1 us.  Holding part of a larger share gains
// nothing (R = 8, 128 MiB, 40 of 128 tiles: 375 -> 377 us).  With streaming
// puts, few tiles lost (R = 16, 8 MiB, 8 tiles: 47.7 -> 49.0 us); with
// device-scope puts they gain (R = 16, 8 MiB: 50-54 -> 44-47 us; R = 6,
// 4 MiB, 4 tiles: 11.4 -> 10.7 us).
//
// kIlv: the tiles of the call are dealt to the ranks in turn instead of one
// contiguous chunk per rank, so at any moment all workgroups read and write
// one neighbourhood of each buffer; the host uses it for the whole-R-tile
// slices of large calls at R <= 8 (R = 8, 128 MiB in 8 slices: 347.8 ->
// 340.9 us; 64 MiB in 4 slices: 173.5 -> 168.8 us; it loses on single held
// launches and at R = 16).
//
// kCachedPuts: device-scope temporal puts (the host's choice while the call's
// 2*R*S bytes fit the Infinity Cache), else streaming puts.
template <class C, int R, bool kIlv, bool kCachedPuts = false>
__global__ __launch_bounds__(kThreads) void mscl_twoshot_held(KernelArgs a) {
  if constexpr (unroll_for<R>() == 1) {
    __shared__ u32x4 held[kHeldTiles][kThreads];
    twoshot_body<C, R, kCachedPuts, true, kIlv>(a, held);
  } else {
    twoshot_body<C, R, false, false>(a, nullptr);  // several vectors per lane: the host never picks this
  }
}

// Two-shot over a port channel: the reduce-scatter runs here, as in the
// two-shot; the all-gather puts go to the host proxy, which copies each rank's
// reduced chunk into the R-1 peer outputs with DMA engines.  Every workgroup
// publishes its part of the chunk to memory at system scope (the copy engines
// read memory, not this XCD's L2) and counts itself in; the rank's last
// workgroup posts the R-1 puts, one lane per peer, and its first lane waits
// until the proxy reports them done, so the call ends on the stream only once
// every output is complete.  In place, rank r's puts overwrite in[p][chunk r],
// which only rank r read, before its workgroups counted in.
template <class C, int R>
__global__ __launch_bounds__(kThreads) void mscl_twoshot_port(KernelArgs a) {
  constexpr int U = unroll_for<R>();
  const int rank = blockIdx.x % R;
  const int slot = blockIdx.x / R;
  const Chunk g = chunk_of<C, U>(a, rank, slot);
  char* const mine = static_cast<char*>(a.out[rank]);
  twoshot_reduce_scatter<C, R>(a, g, slot, mine, g.v_lo + threadIdx.x, static_cast<uint64_t>(kThreads) * U);

  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "");  // this thread's stores, published at system scope
  __syncthreads();
  __shared__ bool last;
  if (threadIdx.x == 0) {
    const uint32_t prior =
        __hip_atomic_fetch_add(a.port.arrived + rank, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    last = prior + 1 == a.nblk;
    if (last) __hip_atomic_store(a.port.arrived + rank, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!last || threadIdx.x >= 64) return;

  const PortChannel port{a.port, a.ch};
  const uint64_t off = g.lo * C::kElemBytes;
  const uint64_t bytes = (g.hi - g.lo) * C::kElemBytes;
  if (bytes == 0) return;
  const int peer = threadIdx.x;
  if (peer < R && peer != rank && rank != a.ch.drop_rank)
    port.put(rank, static_cast<char*>(a.out[peer]) + off, mine + off, bytes);
  if (threadIdx.x == 0) {
    const uint32_t target = __hip_atomic_load(a.port.issued + rank, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) +
                            static_cast<uint32_t>(R - 1);
    __hip_atomic_store(a.port.issued + rank, target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    port.flush(rank, target);
  }
}

// Two-shot with the all-gather put issued from registers: rank r reduces each
// tile of chunk r and writes the rounded vector straight into every rank's
// output (its own included), so the reduced chunk is never re-read and the
// call moves exactly R*S bytes in and R*S out.  Inputs are read once and
// stream past the caches.  Rank r writes only chunk r of every output, which
// no other rank reads or writes during the call, and in place the only
// reader of in[p][chunk r] is rank r itself, each lane loading a vector from
// every input before it stores that vector; so no barrier is needed between
// the reduction and the puts.
//
// kComplete: the call ends with the method's completion barrier.  The puts
// are device-scope stores (store_vec_scoped), and each workgroup, once its
// puts are acknowledged, signals the same slot of every peer ("my puts into
// your output are done") and waits for theirs (Sync::kAfterWrites); a
// workgroup leaves the kernel only when every rank has finished putting its
// slot's tiles into this rank's output.  Measured on MI355X (R = 8 bf16,
// graph replay, us, with -> without the barrier): 512 KiB 3.8 -> 2.5, 2 MiB
// 5.6 -> 4.3, 8 MiB 21.0 -> 19.6.  Without kComplete (an explicitly requested
// variant) completion is the end of the kernel on the stream, which on one
// GPU covers every rank at once.
template <class C, int R, int U, bool kFull, int T, Put kP>
__device__ inline void put_all_tile(const KernelArgs& a, const u32x4 (&y)[U], uint64_t base, uint64_t vend) {
#pragma unroll
  for (int p = 0; p < R; ++p) store_tile<U, kFull, kP, T>(a.out[p], y, base, vend);
}

// The same puts as device-scope stores: tile base `v0` (wave-uniform), `nvec`
// vectors in the tile's range, lane `lane` writing vectors lane, lane + T, ...
template <int R, int U, int T, int kCpol>
__device__ inline void put_all_tile_scoped(const KernelArgs& a, const u32x4 (&y)[U], uint64_t v0, uint64_t nvec,
                                           uint32_t lane) {
#pragma unroll
  for (int p = 0; p < R; ++p) {
    const __amdgpu_buffer_rsrc_t rsrc = tile_rsrc(a.out[p], v0, nvec);
#pragma unroll
    for (int u = 0; u < U; ++u) store_vec_scoped<kCpol>(rsrc, lane + static_cast<uint32_t>(u * T), y[u]);
  }
}

// T threads per workgroup: 256, or 128 for messages too small to give every
// CU one 256-lane tile (more, smaller workgroups spread the loads).
template <class C, int R, int T, bool kCachedPuts, bool kComplete>
__global__ __launch_bounds__(T) void mscl_twoshot_fused(KernelArgs a) {
  constexpr int V = C::V;
  constexpr Put kP = put_policy<kCachedPuts>();
  constexpr int kCpol = kCachedPuts ? kBufferSc1 : (kBufferSc1 | kBufferNt);
  constexpr int U = unroll_for<R>();
  constexpr uint64_t kTile = static_cast<uint64_t>(T) * U;
  const int rank = blockIdx.x % R;
  const int slot = blockIdx.x / R;
  const uint64_t B = a.nblk;
  const uint64_t n = a.count;
  const uint64_t lo = std::min<uint64_t>(static_cast<uint64_t>(rank) * a.chunk, n);
  const uint64_t hi = std::min<uint64_t>(lo + a.chunk, n);
  const uint64_t v_lo = lo / V;
  const uint64_t v_full = hi / V;
  const int ntail = hi > lo ? static_cast<int>(hi % V) : 0;
  const uint64_t nv = v_full - v_lo;
  const uint64_t nfull_tiles = nv / kTile;
  const bool owns_partial_tile = (nv % kTile) != 0 && slot == static_cast<int>(nfull_tiles % B);
  const uint64_t lane_base = v_lo + threadIdx.x;

  if (static_cast<uint64_t>(slot) < nfull_tiles) {
    uint64_t t = slot;
    u32x4 cur[U][R];
    load_tile<R, U, true, true, T>(cur, a.in, lane_base + t * kTile, v_full);
    while (true) {
      const uint64_t tn = t + B;
      const bool more = tn < nfull_tiles;
      u32x4 nxt[U][R];
      if (more) load_tile<R, U, true, true, T>(nxt, a.in, lane_base + tn * kTile, v_full);
      u32x4 y[U];
      reduce_tile<C, R, U>(y, cur);
      if constexpr (kComplete)
        put_all_tile_scoped<R, U, T, kCpol>(a, y, v_lo + t * kTile, kTile, threadIdx.x);
      else
        put_all_tile<C, R, U, true, T, kP>(a, y, lane_base + t * kTile, v_full);
      if (!more) break;
      for (int u = 0; u < U; ++u)
        for (int p = 0; p < R; ++p) cur[u][p] = nxt[u][p];
      t = tn;
    }
  }
  if (owns_partial_tile) {
    u32x4 x[U][R];
    u32x4 y[U];
    const uint64_t base = lane_base + nfull_tiles * kTile;
    load_tile<R, U, false, true, T>(x, a.in, base, v_full);
    reduce_tile<C, R, U>(y, x);
    if constexpr (kComplete) {
      const uint64_t v0 = v_lo + nfull_tiles * kTile;
      put_all_tile_scoped<R, U, T, kCpol>(a, y, v0, v_full - v0, threadIdx.x);  // lanes past v_full dropped
    } else {
      put_all_tile<C, R, U, false, T, kP>(a, y, base, v_full);
    }
  }
  if (ntail != 0 && slot == 0 && threadIdx.x == 0) {
    const u32x4 y = reduce_partial<C, R>(a, v_full, ntail);
#pragma unroll
    for (int p = 0; p < R; ++p) {
      if constexpr (kComplete)
        store_partial_scoped<C, kBufferSc1>(a.out[p], v_full, y, ntail);
      else
        store_partial<C>(a.out[p], v_full, y, ntail);
    }
  }

  if constexpr (kComplete) {
    const RankChannels chans{a.ch, R, rank, slot};
    chans.template barrier_all<Sync::kAfterWrites>();
  }
}

// ----------------------------------------------------------------------------
// Two-shot with per-tile semaphores and a pull (get) all-gather.
//
// Reduce-scatter: slot b of rank r reduces its tiles of chunk r, stores each
// into rank r's own output with device-scope stores and, once they are
// acknowledged, signals one more finished tile on its per-tile semaphore.
// All-gather: slot b of rank r then gets, from every peer p's output, the
// tiles of chunk p that slot b of rank p reduced, each one as soon as that
// tile's semaphore shows it finished (no barrier between the phases: a tile
// waits only for its own reduce-scatter), and stores it into its own output.
// A get is a device-scope load, which reads what the peer's device-scope
// stores left rather than a stale line of this XCD's L2.  In place, rank r's
// store into out[r][chunk p] overwrites in[r][chunk p], which only slot b of
// rank p reads, before it signals that tile.
// ----------------------------------------------------------------------------

// Slot `slot`'s tiles of a chunk, in the order both phases visit them: its
// full tiles t = slot, slot + B, ..., then the partial tile if it owns it, then
// (slot 0) the buffer's partial vector.
template <class C, int U>
__device__ inline uint32_t slot_tiles(const Chunk& g, int slot, uint64_t B) {
  const uint64_t full = static_cast<uint64_t>(slot) < g.nfull_tiles ? (g.nfull_tiles - 1 - slot) / B + 1 : 0;
  return static_cast<uint32_t>(full + (g.owns_partial_tile ? 1 : 0) + (g.ntail != 0 && slot == 0 ? 1 : 0));
}

// Wait for the tile's stores, then signal it (whole workgroup).
__device__ inline void tile_finished(const TileSemaphores& sem) {
  __builtin_amdgcn_s_waitcnt(0);  // this thread's stores (and loads) of the tile, completed
  __syncthreads();
  if (threadIdx.x == 0) sem.signal_tile();
}

template <class C, int R, bool kCachedPuts>
__global__ __launch_bounds__(kThreads) void mscl_twoshot_pertile(KernelArgs a) {
  constexpr int U = unroll_for<R>();
  constexpr uint64_t kTile = static_cast<uint64_t>(kThreads) * U;
  constexpr int kPutPol = kCachedPuts ? kBufferSc1 : (kBufferSc1 | kBufferNt);
  const int rank = blockIdx.x % R;
  const int slot = blockIdx.x / R;
  const uint64_t B = a.nblk;
  const uint32_t lane = threadIdx.x;
  const TileSemaphores sem{a.ch, R, rank, slot};
  const Chunk g = chunk_of<C, U>(a, rank, slot);
  void* const mine = a.out[rank];

  // Reduce-scatter into the own output, one signal per tile.  The next tile's
  // loads are issued before the current tile's stores, so they overlap the
  // wait for the stores' acknowledgements.
  if (static_cast<uint64_t>(slot) < g.nfull_tiles) {
    uint64_t t = slot;
    u32x4 cur[U][R];
    load_tile<R, U, true, true>(cur, a.in, g.v_lo + lane + t * kTile, g.v_full);
    while (true) {
      const uint64_t tn = t + B;
      const bool more = tn < g.nfull_tiles;
      u32x4 nxt[U][R];
      if (more) load_tile<R, U, true, true>(nxt, a.in, g.v_lo + lane + tn * kTile, g.v_full);
      u32x4 y[U];
      reduce_tile<C, R, U>(y, cur);
      const __amdgpu_buffer_rsrc_t rs = tile_rsrc(mine, g.v_lo + t * kTile, kTile);
#pragma unroll
      for (int u = 0; u < U; ++u) store_vec_scoped<kBufferSc1>(rs, lane + static_cast<uint32_t>(u * kThreads), y[u]);
      tile_finished(sem);
      if (!more) break;
      for (int u = 0; u < U; ++u)
        for (int p = 0; p < R; ++p) cur[u][p] = nxt[u][p];
      t = tn;
    }
  }
  if (g.owns_partial_tile) {
    u32x4 x[U][R];
    u32x4 y[U];
    const uint64_t v0 = g.v_lo + g.nfull_tiles * kTile;
    load_tile<R, U, false, true>(x, a.in, v0 + lane, g.v_full);
    reduce_tile<C, R, U>(y, x);
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(mine, v0, g.v_full - v0);  // lanes past the chunk are dropped
#pragma unroll
    for (int u = 0; u < U; ++u) store_vec_scoped<kBufferSc1>(rs, lane + static_cast<uint32_t>(u * kThreads), y[u]);
    tile_finished(sem);
  }
  if (g.ntail != 0 && slot == 0) {
    if (lane == 0) store_partial_scoped<C, kBufferSc1>(mine, g.v_full, reduce_partial<C, R>(a, g.v_full, g.ntail), g.ntail);
    tile_finished(sem);
  }

  // All-gather by get: the same slot's tiles of every peer's chunk, each as
  // soon as its semaphore shows it finished.  The tiles go in columns: step j
  // gets tile j of every peer's chunk, all loads issued before any store, so
  // up to R - 1 loads per lane are in flight.  ready_sh[p] caches how many
  // of peer p's tiles are known finished (first from one read of every
  // peer's semaphore, lane p of wave 0 reading peer p's), so a semaphore is
  // polled again only when the tile needed next is not yet known finished.
  __shared__ uint32_t base_sh[kMaxRanks], ready_sh[kMaxRanks], nvec_sh[kMaxRanks], total_sh[kMaxRanks];
  if (lane < static_cast<uint32_t>(R)) {
    const int p = static_cast<int>(lane);
    const Chunk gp = chunk_of<C, U>(a, p, slot);
    const uint64_t nfull_mine = static_cast<uint64_t>(slot) < gp.nfull_tiles ? (gp.nfull_tiles - 1 - slot) / B + 1 : 0;
    nvec_sh[p] = p == rank ? 0u : static_cast<uint32_t>(nfull_mine + (gp.owns_partial_tile ? 1 : 0));
    total_sh[p] = p == rank ? 0u : slot_tiles<C, U>(gp, slot, B);
    const uint32_t b0 = __hip_atomic_load(sem.seen_of(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    base_sh[p] = b0;
    const uint32_t have =
        p == rank ? 0u : __hip_atomic_load(sem.progress_of(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) - b0;
    sem.check_tiles(have, total_sh[p]);
    ready_sh[p] = static_cast<int32_t>(have) > 0 ? have : 0u;
  }
  __syncthreads();
  uint32_t columns = 0;
#pragma unroll
  for (int p = 0; p < R; ++p) columns = std::max(columns, nvec_sh[p]);
  for (uint32_t j = 0; j < columns; ++j) {
    if (lane == 0) {
      for (int k = 1; k < R; ++k) {
        const int p = (rank + k) % R;
        if (j < nvec_sh[p] && j >= ready_sh[p]) ready_sh[p] = sem.wait_tiles(p, base_sh[p], j + 1, total_sh[p]);
      }
    }
    __syncthreads();
    u32x4 y[R][U];
#pragma unroll
    for (int p = 0; p < R; ++p) {
      if (p != rank && j < nvec_sh[p]) {
        const Chunk gp = chunk_of<C, U>(a, p, slot);
        const uint64_t nfull_mine = (gp.nfull_tiles - 1 - slot) / B + 1;  // j < nvec implies slot has a tile
        const uint64_t t = static_cast<uint64_t>(slot) < gp.nfull_tiles && j < nfull_mine ? slot + j * B
                                                                                         : gp.nfull_tiles;
        const uint64_t v0 = gp.v_lo + t * kTile;
        const uint64_t nv = std::min<uint64_t>(kTile, gp.v_full - v0);  // lanes past it read zero
        const __amdgpu_buffer_rsrc_t src = tile_rsrc(a.out[p], v0, nv);
#pragma unroll
        for (int u = 0; u < U; ++u) y[p][u] = load_vec_scoped<kBufferSc1>(src, lane + static_cast<uint32_t>(u * kThreads));
      }
    }
#pragma unroll
    for (int p = 0; p < R; ++p) {
      if (p != rank && j < nvec_sh[p]) {
        const Chunk gp = chunk_of<C, U>(a, p, slot);
        const uint64_t nfull_mine = (gp.nfull_tiles - 1 - slot) / B + 1;
        const uint64_t t = static_cast<uint64_t>(slot) < gp.nfull_tiles && j < nfull_mine ? slot + j * B
                                                                                         : gp.nfull_tiles;
        const uint64_t v0 = gp.v_lo + t * kTile;
        const uint64_t nv = std::min<uint64_t>(kTile, gp.v_full - v0);  // lanes past it store nothing
        const __amdgpu_buffer_rsrc_t dst = tile_rsrc(mine, v0, nv);
#pragma unroll
        for (int u = 0; u < U; ++u) store_vec_scoped<kPutPol>(dst, lane + static_cast<uint32_t>(u * kThreads), y[p][u]);
      }
    }
  }
  // The buffer's partial vector, the last item of slot 0 of the chunk that
  // holds the buffer's end.
  if (slot == 0 && lane == 0) {
#pragma unroll
    for (int p = 0; p < R; ++p) {
      if (p == rank) continue;
      const Chunk gp = chunk_of<C, U>(a, p, slot);
      if (gp.ntail == 0) continue;
      if (ready_sh[p] < nvec_sh[p] + 1) sem.wait_tiles(p, base_sh[p], nvec_sh[p] + 1, total_sh[p]);
      store_partial<C>(mine, gp.v_full, load_partial_scoped<C, kBufferSc1>(a.out[p], gp.v_full, gp.ntail), gp.ntail);
    }
  }
  if (lane < static_cast<uint32_t>(R) && static_cast<int>(lane) != rank) {
    const Chunk gp = chunk_of<C, U>(a, static_cast<int>(lane), slot);
    __hip_atomic_store(sem.seen_of(static_cast<int>(lane)), base_sh[lane] + slot_tiles<C, U>(gp, slot, B),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
}

// ----------------------------------------------------------------------------
// ReduceScatter and AllGather: the two halves of the two-shot as standard
// collectives of their own (the pages' library implements the standard
// collective API; MSCCL++ ASPLOS'26 abstract).
//
// ReduceScatter: rank r gets block r (recvcount elements) of every input and
// writes the reduced block to its own output.  Rank r writes nothing a peer
// reads and reads nothing a peer writes, so no barrier is needed inside the
// call; stream order stands in for the start and end synchronisation.
// AllGather: rank r puts its input into block r of every rank's output
// (skipping its own when that block already is its input, in place).  Each
// rank's puts go to a block no other rank writes, and the call's end on the
// stream is the completion point.
//
// kVec: every block boundary is 16-byte aligned, so blocks move as 16-byte
// vectors; otherwise one element per lane per step (coalesced 2- or 4-byte
// accesses).
// ----------------------------------------------------------------------------

template <class C, int R, bool kVec>
__global__ __launch_bounds__(kThreads) void mscl_reduce_scatter_kernel(KernelArgs a) {
  constexpr int U = unroll_for<R>();
  constexpr uint64_t kTile = static_cast<uint64_t>(kThreads) * U;
  const int rank = blockIdx.x % R;
  const int slot = blockIdx.x / R;
  const uint64_t rc = a.count;  // elements per block
  void* const dst = a.out[rank];
  if constexpr (kVec) {
    const uint64_t nv = rc / C::V;  // rc is a multiple of V here
    const uint64_t src0 = static_cast<uint64_t>(rank) * nv;  // block start, in vectors
    const uint64_t ntiles = (nv + kTile - 1) / kTile;
    const void* src[R];
#pragma unroll
    for (int p = 0; p < R; ++p) src[p] = static_cast<const u32x4*>(a.in[p]) + src0;
    // Full tiles, software pipelined as in the two-shot's reduce-scatter:
    // the next tile's loads are issued before the current one is reduced
    // and stored (R = 4 fp32, 128 MiB inputs: 125 -> 117 us).  Inputs are
    // read once and stream past the caches; the block is stored cacheable
    // (streaming stores measured slower: R = 8 bf16, 220 vs 215 us).  In
    // place (outputs[r] is block r of inputs[r]) a lane stores only vectors
    // it has already loaded.
    const uint64_t B = a.nblk;
    const uint64_t nfull_tiles = nv / kTile;
    const uint64_t lane = threadIdx.x;
    if (static_cast<uint64_t>(slot) < nfull_tiles) {
      uint64_t t = slot;
      u32x4 cur[U][R];
      load_tile<R, U, true, true>(cur, src, t * kTile + lane, nv);
      while (true) {
        const uint64_t tn = t + B;
        const bool more = tn < nfull_tiles;
        u32x4 nxt[U][R];
        if (more) load_tile<R, U, true, true>(nxt, src, tn * kTile + lane, nv);
        u32x4 y[U];
        reduce_tile<C, R, U>(y, cur);
        store_tile<U, true, Put::kCached>(dst, y, t * kTile + lane, nv);
        if (!more) break;
        for (int u = 0; u < U; ++u)
          for (int p = 0; p < R; ++p) cur[u][p] = nxt[u][p];
        t = tn;
      }
    }
    if (nfull_tiles < ntiles && static_cast<uint64_t>(slot) == nfull_tiles % B) {  // the partial tile
      u32x4 x[U][R];
      u32x4 y[U];
      const uint64_t base = nfull_tiles * kTile + lane;
      load_tile<R, U, false, true>(x, src, base, nv);
      reduce_tile<C, R, U>(y, x);
      store_tile<U, false, Put::kCached>(dst, y, base, nv);
    }
  } else {
    using Bits = typename C::Bits;
    const uint64_t off = static_cast<uint64_t>(rank) * rc;
    for (uint64_t j = static_cast<uint64_t>(slot) * kThreads + threadIdx.x; j < rc;
         j += static_cast<uint64_t>(a.nblk) * kThreads) {
      float acc = C::widen(static_cast<const Bits*>(a.in[0])[off + j]);
#pragma unroll
      for (int p = 1; p < R; ++p) acc = acc + C::widen(static_cast<const Bits*>(a.in[p])[off + j]);
      static_cast<Bits*>(dst)[j] = C::narrow(acc);
    }
  }
}

// AllGather keeps two vectors per lane in flight (it holds no R-fold
// operands; one measured 337 us, four 267 us, two 243 us at R = 8 with 16 MiB
// blocks) and loads the next tile while it stores the current one.
constexpr int kAllGatherU = 2;

template <int R>
__device__ inline void allgather_store(const KernelArgs& a, int rank, bool skip_own, uint64_t dst0,
                                       const u32x4 (&y)[kAllGatherU], uint64_t base, uint64_t nv, bool full) {
#pragma unroll
  for (int p = 0; p < R; ++p) {
    if (p == rank && skip_own) continue;
    u32x4* out = static_cast<u32x4*>(a.out[p]) + dst0;  // put() into block `rank`
#pragma unroll
    for (int u = 0; u < kAllGatherU; ++u) {
      const uint64_t vi = base + static_cast<uint64_t>(u) * kThreads;
      if (full || vi < nv) store_vec_nt(out, vi, y[u]);
    }
  }
}

__device__ inline void allgather_load(u32x4 (&y)[kAllGatherU], const void* src, uint64_t base, uint64_t nv,
                                      bool full) {
#pragma unroll
  for (int u = 0; u < kAllGatherU; ++u) {
    uint64_t vi = base + static_cast<uint64_t>(u) * kThreads;
    if (!full) vi = std::min<uint64_t>(vi, nv - 1);
    y[u] = load_vec(src, vi);  // cacheable: measured 185 us vs 243 us with streaming loads (R=8, 16 MiB blocks)
  }
}

template <class C, int R, bool kVec>
__global__ __launch_bounds__(kThreads) void mscl_allgather_kernel(KernelArgs a) {
  const int rank = blockIdx.x % R;
  const int slot = blockIdx.x / R;
  const uint64_t sc = a.count;  // elements per input block
  const void* const src = a.in[rank];
  const bool skip_own = (a.in_place_mask >> rank) & 1u;
  if constexpr (kVec) {
    constexpr uint64_t kTile = static_cast<uint64_t>(kThreads) * kAllGatherU;
    const uint64_t nv = sc / C::V;
    const uint64_t dst0 = static_cast<uint64_t>(rank) * nv;
    const uint64_t ntiles = (nv + kTile - 1) / kTile;
    if (static_cast<uint64_t>(slot) >= ntiles) return;
    uint64_t t = slot;
    u32x4 cur[kAllGatherU];
    allgather_load(cur, src, t * kTile + threadIdx.x, nv, (t + 1) * kTile <= nv);
    while (true) {
      const uint64_t tn = t + a.nblk;
      const bool more = tn < ntiles;
      u32x4 nxt[kAllGatherU];
      if (more) allgather_load(nxt, src, tn * kTile + threadIdx.x, nv, (tn + 1) * kTile <= nv);
      allgather_store<R>(a, rank, skip_own, dst0, cur, t * kTile + threadIdx.x, nv, (t + 1) * kTile <= nv);
      if (!more) break;
      for (int u = 0; u < kAllGatherU; ++u) cur[u] = nxt[u];
      t = tn;
    }
  } else {
    using Bits = typename C::Bits;
    const uint64_t off = static_cast<uint64_t>(rank) * sc;
    for (uint64_t j = static_cast<uint64_t>(slot) * kThreads + threadIdx.x; j < sc;
         j += static_cast<uint64_t>(a.nblk) * kThreads) {
      const Bits v = static_cast<const Bits*>(src)[j];
#pragma unroll
      for (int p = 0; p < R; ++p)
        if (!(p == rank && skip_own)) static_cast<Bits*>(a.out[p])[off + j] = v;
    }
  }
}

// ----------------------------------------------------------------------------
// Channel self-test: the barriers' contracts checked directly.  Every round,
// each (rank, slot) workgroup writes a 4 KiB mailbox, runs the publishing
// barrier (the pages' signal/wait), reads the mailbox of the next rank's same
// slot (a workgroup on a different XCD) and counts words that differ from
// what that peer wrote before it signalled; then a write-after-read barrier
// (Sync::kAfterReads) must keep the peer from overwriting its mailbox with
// the next round's words before those reads are done.
// ----------------------------------------------------------------------------

constexpr int kSelftestWords = 1024;  // u32 words per mailbox (4 per lane)

__device__ inline uint32_t selftest_word(uint32_t round, int rank, int slot, int i) {
  uint32_t h = round * 0x9E3779B1u ^ (static_cast<uint32_t>(rank) << 24) ^ (static_cast<uint32_t>(slot) << 12) ^
               static_cast<uint32_t>(i);
  h ^= h >> 16;
  h *= 0x85EBCA6Bu;
  h ^= h >> 13;
  return h;
}

template <int R>
__global__ __launch_bounds__(kThreads) void mscl_channel_selftest_kernel(KernelArgs a, uint32_t* mailbox,
                                                                          uint32_t rounds, uint32_t* mismatches) {
  const int rank = blockIdx.x % R;
  const int slot = blockIdx.x / R;
  const RankChannels chans{a.ch, R, rank, slot};
  const int peer = (rank + 1) % R;
  uint32_t* mine = mailbox + (static_cast<uint64_t>(rank) * a.nblk + slot) * kSelftestWords;
  const uint32_t* theirs = mailbox + (static_cast<uint64_t>(peer) * a.nblk + slot) * kSelftestWords;
  uint32_t bad = 0;
  for (uint32_t k = 0; k < rounds; ++k) {
#pragma unroll
    for (int j = 0; j < kSelftestWords / kThreads; ++j) {
      const int i = j * kThreads + threadIdx.x;
      mine[i] = selftest_word(k, rank, slot, i);
    }
    chans.template barrier_all<Sync::kPublish>();
#pragma unroll
    for (int j = 0; j < kSelftestWords / kThreads; ++j) {
      const int i = j * kThreads + threadIdx.x;
      bad += theirs[i] != selftest_word(k, peer, slot, i);
    }
    chans.template barrier_all<Sync::kAfterReads>();
  }
  if (bad) __hip_atomic_fetch_add(mismatches, bad, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ----------------------------------------------------------------------------
// Kernel tables
// ----------------------------------------------------------------------------

using KernelFn = void (*)(KernelArgs);
enum {
  kAlgoOneShot = 0,
  kAlgoOneShotInPlace = 1,
  kAlgoTwoShot = 2,
  kAlgoTwoShotFused = 3,
  kReduceScatterVec = 4,
  kReduceScatterElem = 5,
  kAllGatherVec = 6,
  kAllGatherElem = 7,
  kAlgoTwoShotPort = 8,
  kAlgoTwoShotFusedHalf = 9,  // the fused two-shot on kThreads / 2 threads per workgroup
  // the same three with device-scope temporal puts (Put::kDevice)
  kAlgoTwoShotCachedPuts = 10,
  kAlgoTwoShotFusedCachedPuts = 11,
  kAlgoTwoShotFusedHalfCachedPuts = 12,
  kAlgoTwoShotHeld = 13,  // the two-shot keeping reduced tiles in LDS (mscl_twoshot_held)
  // the fused two-shot with its completion barrier (the kinds above run it
  // without): 256 / 128 threads, streaming / device-scope temporal puts
  kAlgoTwoShotFusedSync = 14,
  kAlgoTwoShotFusedHalfSync = 15,
  kAlgoTwoShotFusedCachedPutsSync = 16,
  kAlgoTwoShotFusedHalfCachedPutsSync = 17,
  kAlgoTwoShotHeldInterleaved = 18,  // the held two-shot with tiles dealt to the ranks in turn
  kAlgoTwoShotPerTile = 19,          // per-tile semaphores, pull all-gather (streaming / device-scope puts)
  kAlgoTwoShotPerTileCachedPuts = 20,
  kAlgoTwoShotHeldCachedPuts = 21  // the held two-shot with device-scope temporal puts
};

template <class C, int R>
constexpr KernelFn kernel_for(int kind) {
  switch (kind) {
    case kAlgoOneShot: return &mscl_oneshot<C, R, false>;
    case kAlgoOneShotInPlace: return &mscl_oneshot<C, R, true>;
    case kAlgoTwoShot: return &mscl_twoshot<C, R, false>;
    case kAlgoTwoShotFused: return &mscl_twoshot_fused<C, R, kThreads, false, false>;
    case kAlgoTwoShotFusedHalf: return &mscl_twoshot_fused<C, R, kThreads / 2, false, false>;
    case kAlgoTwoShotCachedPuts: return &mscl_twoshot<C, R, true>;
    case kAlgoTwoShotFusedCachedPuts: return &mscl_twoshot_fused<C, R, kThreads, true, false>;
    case kAlgoTwoShotFusedHalfCachedPuts: return &mscl_twoshot_fused<C, R, kThreads / 2, true, false>;
    case kAlgoTwoShotFusedSync: return &mscl_twoshot_fused<C, R, kThreads, false, true>;
    case kAlgoTwoShotFusedHalfSync: return &mscl_twoshot_fused<C, R, kThreads / 2, false, true>;
    case kAlgoTwoShotFusedCachedPutsSync: return &mscl_twoshot_fused<C, R, kThreads, true, true>;
    case kAlgoTwoShotFusedHalfCachedPutsSync: return &mscl_twoshot_fused<C, R, kThreads / 2, true, true>;
    case kAlgoTwoShotHeld: return &mscl_twoshot_held<C, R, false>;
    case kAlgoTwoShotHeldInterleaved: return &mscl_twoshot_held<C, R, true>;
    case kAlgoTwoShotHeldCachedPuts: return &mscl_twoshot_held<C, R, false, true>;
    case kAlgoTwoShotPerTile: return &mscl_twoshot_pertile<C, R, false>;
    case kAlgoTwoShotPerTileCachedPuts: return &mscl_twoshot_pertile<C, R, true>;
    case kReduceScatterVec: return &mscl_reduce_scatter_kernel<C, R, true>;
    case kReduceScatterElem: return &mscl_reduce_scatter_kernel<C, R, false>;
    case kAllGatherVec: return &mscl_allgather_kernel<C, R, true>;
    case kAllGatherElem: return &mscl_allgather_kernel<C, R, false>;
    case kAlgoTwoShotPort: return &mscl_twoshot_port<C, R>;
  }
  return nullptr;
}

template <class C, int... Rs>
KernelFn pick(int kind, int R, std::integer_sequence<int, Rs...>) {
  KernelFn fn = nullptr;
  ((R == Rs + 1 ? (fn = kernel_for<C, Rs + 1>(kind), 0) : 0), ...);
  return fn;
}

inline KernelFn kernel_lookup(int kind, int dtype, int R) {
  auto seq = std::make_integer_sequence<int, kMaxRanks>{};
  switch (dtype) {
    case MSCL_FLOAT32: return pick<F32>(kind, R, seq);
    case MSCL_FLOAT16: return pick<F16>(kind, R, seq);
    case MSCL_BFLOAT16: return pick<BF16>(kind, R, seq);
  }
  return nullptr;
}

inline int unroll_for_runtime(int R) { return R <= 2 ? 4 : (R <= 4 ? 2 : 1); }

inline int threads_for_kind(int kind) {
  return (kind == kAlgoTwoShotFusedHalf || kind == kAlgoTwoShotFusedHalfCachedPuts || kind == kAlgoTwoShotFusedHalfSync ||
          kind == kAlgoTwoShotFusedHalfCachedPutsSync)
             ? kThreads / 2
             : kThreads;
}

}  // namespace mscl
