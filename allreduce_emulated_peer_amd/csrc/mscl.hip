// MemoryChannel-style collectives over R emulated peer ranks on one gfx950 GPU.
//
// The MSCCL++ pages present AllReduce as the collective their library speeds
// up for tensor-parallel LLM serving (project summary, "Highlighted
// Details"), built from GPU-side channel methods (README, Key Concepts,
// "On-GPU Communication Interfaces: Channels") of which the MemoryChannel
// moves data with many GPU threads loading and storing peer memory directly
// ("PortChannel and MemoryChannel").  This file holds the kernels and the
// host side of the C ABI declared in include/mscl.h:
//
//   mscl_oneshot        every rank reads all R inputs and writes its own
//                       output; in place, an ordered barrier separates each
//                       tile's loads from its stores (a rank overwrites an
//                       input its peers are still reading).
//   mscl_twoshot        reduce-scatter (rank r reduces chunk r of all
//                       inputs into its own output), an arrival-only
//                       barrier, all-gather (rank r puts its chunk into every
//                       peer's output).
//   mscl_twoshot_fused  reduce-scatter whose result goes from registers
//                       straight into every output; no barrier.
//   mscl_reduce_scatter_kernel / mscl_allgather_kernel
//                       the two halves as standard collectives.
//   mscl_channel_selftest_kernel
//                       the ordered barrier's publish/acquire contract.
//
// Rank layout.  Workgroup w of a launch is emulated rank (w % R), channel
// slot (w / R); with the hardware's round-robin dispatch of workgroups over
// the 8 XCDs, a rank's workgroups stay on a fixed XCD subset.  The one-shot
// instead groups the R ranks of a slot on one XCD, because there every rank
// re-reads the same input lines.  Each workgroup has 256 threads (4
// wavefronts of 64); a tile is U 16-byte vectors per lane.
//
// Two-shot chunks: rank r owns elements [r*c, min((r+1)*c, n)) with
// c = roundup(ceil(n/R), V), V = 16 / element size.  Each lane handles the
// same vectors in both phases, which keeps in-place calls safe: the only
// reader of in[p][chunk r] is rank r itself, earlier, in the same lane.
//
// Every reduction adds in rank order 0..R-1 starting from rank 0's value and
// rounds once, so all algorithms give bit-identical results.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <string>
#include <utility>

#include "../../include/mscl.h"
#include "channel.hpp"
#include "codec.hpp"

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
template <int R, int U, bool kFull, bool kStream>
__device__ inline void load_tile(u32x4 (&x)[U][R], const void* const* src, uint64_t base, uint64_t vend) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    uint64_t vi = base + static_cast<uint64_t>(u) * kThreads;
    if (!kFull) vi = std::min<uint64_t>(vi, vend - 1);
#pragma unroll
    for (int p = 0; p < R; ++p) x[u][p] = kStream ? load_vec_nt(src[p], vi) : load_vec(src[p], vi);
  }
}

template <int U, bool kFull, bool kStream>
__device__ inline void store_tile(void* dst, const u32x4 (&y)[U], uint64_t base, uint64_t vend) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint64_t vi = base + static_cast<uint64_t>(u) * kThreads;
    if (kFull || vi < vend) {
      if (kStream)
        store_vec_nt(dst, vi, y[u]);
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

// One tile of the one-shot: all R inputs -> own output, with the channel
// barrier between loads and stores when running in place.
template <class C, int R, int U, bool kInPlace, bool kFull>
__device__ inline void oneshot_tile(const KernelArgs& a, const RankChannels& chans, void* dst, uint64_t base,
                                    uint64_t vend) {
  u32x4 x[U][R];
  u32x4 y[U];
  load_tile<R, U, kFull, false>(x, a.in, base, vend);  // every rank re-reads these: keep them cached
  reduce_tile<C, R, U>(y, x);
  // Peers read this rank's input until they signal; their loads must be
  // complete before this rank overwrites it (write after read across ranks).
  if constexpr (kInPlace) chans.template barrier_all<true>();
  store_tile<U, kFull, false>(dst, y, base, vend);
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
  const uint64_t n = a.count;
  const uint64_t nfull = n / V;
  const int ntail = static_cast<int>(n % V);
  const uint64_t ntiles = (nfull + kTile - 1) / kTile;
  const RankChannels chans{a.ch, R, rank, slot};
  void* const dst = a.out[rank];

  for (uint64_t t = slot; t < ntiles; t += a.nblk) {
    const uint64_t base = t * kTile + threadIdx.x;
    if ((t + 1) * kTile <= nfull)
      oneshot_tile<C, R, U, kInPlace, true>(a, chans, dst, base, nfull);
    else
      oneshot_tile<C, R, U, kInPlace, false>(a, chans, dst, base, nfull);
  }

  if (ntail != 0 && slot == 0) {
    u32x4 y = {0u, 0u, 0u, 0u};
    if (threadIdx.x == 0) y = reduce_partial<C, R>(a, nfull, ntail);
    if constexpr (kInPlace) chans.template barrier_all<true>();
    if (threadIdx.x == 0) store_partial<C>(dst, nfull, y, ntail);
  }
}

// Cache policy of the two-shot: inputs are read exactly once and the peers'
// outputs written exactly once, so both stream past the caches; the rank's
// own reduced chunk is written and read back, so it stays cacheable.
constexpr bool kStreamRsLoads = true;
constexpr bool kStreamAgStores = true;

template <int R, int U, bool kFull>
__device__ inline void ag_store(const KernelArgs& a, int rank, const u32x4 (&y)[U], uint64_t base, uint64_t vend) {
#pragma unroll
  for (int p = 0; p < R; ++p)  // put() to every peer, written once
    if (p != rank) store_tile<U, kFull, kStreamAgStores>(a.out[p], y, base, vend);
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

template <class C, int R>
__global__ __launch_bounds__(kThreads) void mscl_twoshot(KernelArgs a) {
  constexpr int V = C::V;
  constexpr int U = unroll_for<R>();
  constexpr uint64_t kTile = static_cast<uint64_t>(kThreads) * U;
  const int rank = blockIdx.x % R;
  const int slot = blockIdx.x / R;
  const uint64_t B = a.nblk;
  const uint64_t n = a.count;
  const uint64_t lo = std::min<uint64_t>(static_cast<uint64_t>(rank) * a.chunk, n);
  const uint64_t hi = std::min<uint64_t>(lo + a.chunk, n);
  const uint64_t v_lo = lo / V;    // chunk starts are multiples of V
  const uint64_t v_full = hi / V;  // end of the chunk's full vectors
  // nonzero only for the non-empty chunk that holds the buffer's end
  const int ntail = hi > lo ? static_cast<int>(hi % V) : 0;
  const uint64_t nv = v_full - v_lo;
  // Tiles t = slot, slot + B, ... belong to this slot.  Tiles below
  // `nfull_tiles` lie wholly inside the chunk; at most one partial tile
  // (index nfull_tiles) follows.
  const uint64_t nfull_tiles = nv / kTile;
  const bool owns_partial_tile = (nv % kTile) != 0 && slot == static_cast<int>(nfull_tiles % B);
  const RankChannels chans{a.ch, R, rank, slot};
  void* const mine = a.out[rank];
  const uint64_t lane_base = v_lo + threadIdx.x;

  // Reduce-scatter: chunk `rank` of every input -> own output.  Software
  // pipelined: the loads of the slot's next tile are issued before the
  // current tile is reduced and stored, so each wave keeps R*U 16-byte
  // loads in flight while it computes.
  if (static_cast<uint64_t>(slot) < nfull_tiles) {
    uint64_t t = slot;
    u32x4 cur[U][R];
    load_tile<R, U, true, kStreamRsLoads>(cur, a.in, lane_base + t * kTile, v_full);
    while (true) {
      const uint64_t tn = t + B;
      const bool more = tn < nfull_tiles;
      u32x4 nxt[U][R];
      if (more) load_tile<R, U, true, kStreamRsLoads>(nxt, a.in, lane_base + tn * kTile, v_full);
      u32x4 y[U];
      reduce_tile<C, R, U>(y, cur);
      store_tile<U, true, false>(mine, y, lane_base + t * kTile, v_full);  // re-read by the all-gather: cached
      if (!more) break;
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int p = 0; p < R; ++p) cur[u][p] = nxt[u][p];
      t = tn;
    }
  }
  if (owns_partial_tile) {
    u32x4 x[U][R];
    u32x4 y[U];
    const uint64_t base = lane_base + nfull_tiles * kTile;
    load_tile<R, U, false, kStreamRsLoads>(x, a.in, base, v_full);
    reduce_tile<C, R, U>(y, x);
    store_tile<U, false, false>(mine, y, base, v_full);
  }
  const bool tail_owner = ntail != 0 && slot == 0 && threadIdx.x == 0;
  if (tail_owner) store_partial<C>(mine, v_full, reduce_partial<C, R>(a, v_full, ntail), ntail);

  // signal / wait with the same slot of every peer rank.  Arrival only: no
  // data crosses ranks here.  The all-gather below reads only vectors this
  // lane itself wrote above (program order), and writes peer locations that
  // no peer reads during this call (rank p reads only its own chunk of every
  // input, and in place rank r alone reads in[p][chunk r], earlier, in this
  // lane).  Publishing or acquiring memory here would only cost an L2
  // write-back and invalidate per workgroup.
  chans.template barrier_all<false>();

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
    const uint64_t base = lane_base + nfull_tiles * kTile;
    ag_load<U, false>(y, mine, base, v_full);
    ag_store<R, U, false>(a, rank, y, base, v_full);
  }
  if (static_cast<uint64_t>(slot) < nfull_tiles) {
    uint64_t t = slot + (nfull_tiles - 1 - slot) / B * B;  // this slot's last full tile
    u32x4 cur[U];
    ag_load<U, true>(cur, mine, lane_base + t * kTile, v_full);
    while (true) {
      const bool more = t >= static_cast<uint64_t>(slot) + B;
      const uint64_t tn = more ? t - B : t;
      u32x4 nxt[U];
      if (more) ag_load<U, true>(nxt, mine, lane_base + tn * kTile, v_full);
      ag_store<R, U, true>(a, rank, cur, lane_base + t * kTile, v_full);
      if (!more) break;
#pragma unroll
      for (int u = 0; u < U; ++u) cur[u] = nxt[u];
      t = tn;
    }
  }
}

// Two-shot with the all-gather put issued from registers: rank r reduces each
// tile of chunk r and writes the rounded vector straight into every rank's
// output (its own included), so the reduced chunk is never re-read and the
// call moves exactly R*S bytes in and R*S out.  Inputs are read once and
// outputs written once, so both stream past the caches.  No barrier runs
// inside the call: rank r writes only chunk r of every output, which no
// other rank reads or writes during the call, and in place the only reader
// of in[p][chunk r] is rank r itself, each lane loading a vector from every
// input before it stores that vector.
template <class C, int R, int U, bool kFull>
__device__ inline void put_all_tile(const KernelArgs& a, const u32x4 (&y)[U], uint64_t base, uint64_t vend) {
#pragma unroll
  for (int p = 0; p < R; ++p) store_tile<U, kFull, true>(a.out[p], y, base, vend);
}

template <class C, int R>
__global__ __launch_bounds__(kThreads) void mscl_twoshot_fused(KernelArgs a) {
  constexpr int V = C::V;
  constexpr int U = unroll_for<R>();
  constexpr uint64_t kTile = static_cast<uint64_t>(kThreads) * U;
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
  const RankChannels chans{a.ch, R, rank, slot};
  const uint64_t lane_base = v_lo + threadIdx.x;

  if (static_cast<uint64_t>(slot) < nfull_tiles) {
    uint64_t t = slot;
    u32x4 cur[U][R];
    load_tile<R, U, true, true>(cur, a.in, lane_base + t * kTile, v_full);
    while (true) {
      const uint64_t tn = t + B;
      const bool more = tn < nfull_tiles;
      u32x4 nxt[U][R];
      if (more) load_tile<R, U, true, true>(nxt, a.in, lane_base + tn * kTile, v_full);
      u32x4 y[U];
      reduce_tile<C, R, U>(y, cur);
      put_all_tile<C, R, U, true>(a, y, lane_base + t * kTile, v_full);
      if (!more) break;
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int p = 0; p < R; ++p) cur[u][p] = nxt[u][p];
      t = tn;
    }
  }
  if (owns_partial_tile) {
    u32x4 x[U][R];
    u32x4 y[U];
    const uint64_t base = lane_base + nfull_tiles * kTile;
    load_tile<R, U, false, true>(x, a.in, base, v_full);
    reduce_tile<C, R, U>(y, x);
    put_all_tile<C, R, U, false>(a, y, base, v_full);
  }
  if (ntail != 0 && slot == 0 && threadIdx.x == 0) {
    const u32x4 y = reduce_partial<C, R>(a, v_full, ntail);
#pragma unroll
    for (int p = 0; p < R; ++p) store_partial<C>(a.out[p], v_full, y, ntail);
  }

  // Completion is the end of the kernel on the stream: nothing inside the
  // call reads the outputs.  (Across GPUs this is where each rank would
  // signal "my puts into your output are done" and wait for its peers'; on
  // one GPU an in-kernel ordered handshake measured 20-30 us per call for no
  // observer.)
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
    for (uint64_t t = slot; t < ntiles; t += a.nblk) {
      const uint64_t base = t * kTile + threadIdx.x;
      u32x4 x[U][R];
      u32x4 y[U];
      if ((t + 1) * kTile <= nv) {
        load_tile<R, U, true, true>(x, src, base, nv);  // read once: streaming
        reduce_tile<C, R, U>(y, x);
        store_tile<U, true, false>(dst, y, base, nv);
      } else {
        load_tile<R, U, false, true>(x, src, base, nv);
        reduce_tile<C, R, U>(y, x);
        store_tile<U, false, false>(dst, y, base, nv);
      }
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
#pragma unroll
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
// Channel self-test: the pages' signal/wait contract checked directly.  Every
// round, each (rank, slot) workgroup writes a 4 KiB mailbox, runs the ordered
// barrier, reads the mailbox of the next rank's same slot (a workgroup on a
// different XCD) and counts words that differ from what that peer wrote
// before it signalled; a second ordered barrier keeps the peer from
// overwriting its mailbox before the reads are done.
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
    chans.template barrier_all<true>();
#pragma unroll
    for (int j = 0; j < kSelftestWords / kThreads; ++j) {
      const int i = j * kThreads + threadIdx.x;
      bad += theirs[i] != selftest_word(k, peer, slot, i);
    }
    chans.template barrier_all<true>();
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
  kAllGatherElem = 7
};

template <class C, int R>
constexpr KernelFn kernel_for(int kind) {
  switch (kind) {
    case kAlgoOneShot: return &mscl_oneshot<C, R, false>;
    case kAlgoOneShotInPlace: return &mscl_oneshot<C, R, true>;
    case kAlgoTwoShot: return &mscl_twoshot<C, R>;
    case kAlgoTwoShotFused: return &mscl_twoshot_fused<C, R>;
    case kReduceScatterVec: return &mscl_reduce_scatter_kernel<C, R, true>;
    case kReduceScatterElem: return &mscl_reduce_scatter_kernel<C, R, false>;
    case kAllGatherVec: return &mscl_allgather_kernel<C, R, true>;
    case kAllGatherElem: return &mscl_allgather_kernel<C, R, false>;
  }
  return nullptr;
}

template <class C, int... Rs>
KernelFn pick(int kind, int R, std::integer_sequence<int, Rs...>) {
  KernelFn fn = nullptr;
  ((R == Rs + 1 ? (fn = kernel_for<C, Rs + 1>(kind), 0) : 0), ...);
  return fn;
}

KernelFn kernel_lookup(int kind, int dtype, int R) {
  auto seq = std::make_integer_sequence<int, kMaxRanks>{};
  switch (dtype) {
    case MSCL_FLOAT32: return pick<F32>(kind, R, seq);
    case MSCL_FLOAT16: return pick<F16>(kind, R, seq);
    case MSCL_BFLOAT16: return pick<BF16>(kind, R, seq);
  }
  return nullptr;
}

int unroll_for_runtime(int R) { return R <= 2 ? 4 : (R <= 4 ? 2 : 1); }

}  // namespace mscl

// ----------------------------------------------------------------------------
// Host side
// ----------------------------------------------------------------------------

namespace {

using namespace mscl;

thread_local std::string g_last_error;

mscl_status_t fail(mscl_status_t s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

mscl_status_t fail_hip(hipError_t e, const char* what) {
  return fail(MSCL_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

size_t elem_bytes(int dtype) { return dtype == MSCL_FLOAT32 ? 4 : 2; }

bool valid_algo(int algo) {
  return algo == MSCL_ALGO_AUTO || algo == MSCL_ALGO_ONE_SHOT || algo == MSCL_ALGO_TWO_SHOT ||
         algo == MSCL_ALGO_TWO_SHOT_FUSED;
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
};

const Config& config() {
  static Config c;
  static std::once_flag once;
  std::call_once(once, [] {
    c.oneshot_max_bytes = env_size("MSCL_ONESHOT_MAX_BYTES", SIZE_MAX);  // SIZE_MAX: per-R table
    c.wg_target_total = env_size("MSCL_WG_TOTAL", 0);
    c.wg_per_rank = env_size("MSCL_WG_PER_RANK", 0);
    c.wait_timeout_us = env_size("MSCL_WAIT_TIMEOUT_MS", 2000) * 1000;
  });
  return c;
}

}  // namespace

struct mscl_channel_s {
  int device = 0;
  int nranks = 0;
  int refcount = 0;
  int cus = 0;
  uint32_t slots = 0;            // barrier slots allocated per rank (= max co-resident workgroups per rank)
  uint64_t wall_clock_khz = 100000;
  uint32_t* inbound = nullptr;   // device [R][R][slots]
  uint32_t* consumed = nullptr;  // device [R][slots]
  int* status_host = nullptr;    // host-mapped status word
  int* status_dev = nullptr;
  uint64_t wait_timeout_us = 0;  // 0 = config default
  int drop_rank = -1;
};

namespace {

std::mutex g_mutex;
std::map<std::pair<int, int>, mscl_channel_s*> g_registry;

bool registered(mscl_channel_s* ch) {
  for (auto& kv : g_registry)
    if (kv.second == ch) return true;
  return false;
}

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

// AUTO's size bands, from device time per call (calls replayed from a graph)
// on MI355X with bf16 buffers, for R = 2, 4, 8, 16:
//   one-shot        up to oneshot_max_bytes(R): every size at R <= 2, 512 KiB
//                   at R <= 4, 128 KiB at R <= 8, 64 KiB above (it reads R*S
//                   per rank, from cache while the buffers fit);
//   fused two-shot  up to 4 MiB: no barrier and no re-read, best in the middle
//                   (R = 8, 1 MiB: 3.7 us against 5.2 two-shot, 6.4 one-shot);
//   two-shot        above: its separate read and write phases stream HBM best
//                   (R = 8, 128 MiB: 376 us against 381 fused).
// In place, the one-shot would need an ordered barrier on every tile (a rank
// overwrites an input its peers still read: R = 8, 512 KiB, 109 us), so
// in-place calls skip the first band.
size_t oneshot_max_bytes(int nranks) {
  const size_t env = config().oneshot_max_bytes;
  if (env != SIZE_MAX) return env;
  if (nranks <= 2) return SIZE_MAX;
  if (nranks <= 4) return size_t(512) << 10;
  if (nranks <= 8) return size_t(128) << 10;
  return size_t(64) << 10;
}

constexpr size_t kFusedMaxBytes = size_t(4) << 20;

mscl_algo_t resolve_algo(size_t count, int dtype, int nranks, int algo, bool in_place) {
  if (algo != MSCL_ALGO_AUTO) return static_cast<mscl_algo_t>(algo);
  const size_t bytes = count * elem_bytes(dtype);
  if (!in_place && bytes <= oneshot_max_bytes(nranks)) return MSCL_ALGO_ONE_SHOT;
  if (nranks == 1) return MSCL_ALGO_ONE_SHOT;  // a copy (or nothing, in place)
  return bytes <= kFusedMaxBytes ? MSCL_ALGO_TWO_SHOT_FUSED : MSCL_ALGO_TWO_SHOT;
}

void make_plan(const mscl_channel_s* ch, size_t count, int dtype, mscl_algo_t algo, bool in_place,
               mscl_plan_t* plan) {
  const int R = ch->nranks;
  const uint64_t V = 16 / elem_bytes(dtype);
  const uint64_t tile = static_cast<uint64_t>(kThreads) * unroll_for_runtime(R);
  const Config& cfg = config();
  memset(plan, 0, sizeof(*plan));
  plan->algo = algo;
  plan->nranks = R;
  plan->threads_per_workgroup = kThreads;
  plan->vectors_per_thread = unroll_for_runtime(R);
  uint64_t vectors;  // full vectors one rank covers
  if (algo == MSCL_ALGO_TWO_SHOT || algo == MSCL_ALGO_TWO_SHOT_FUSED) {
    const uint64_t per = (count + R - 1) / R;
    const uint64_t c = (per + V - 1) / V * V;
    plan->chunk_elems = c;
    vectors = c / V;
    plan->uses_barrier = algo == MSCL_ALGO_TWO_SHOT ? 1 : 0;
  } else {
    vectors = count / V;
    plan->uses_barrier = in_place ? 1 : 0;
  }
  uint64_t want = std::max<uint64_t>(1, (vectors + tile - 1) / tile);
  // One workgroup per compute unit in total measured best for the streaming
  // phases (fewer concurrent streams keep HBM pages open longer).
  const uint64_t total = cfg.wg_target_total ? cfg.wg_target_total : static_cast<uint64_t>(ch->cus);
  uint64_t cap = cfg.wg_per_rank ? cfg.wg_per_rank : std::max<uint64_t>(1, total / R);
  cap = std::min<uint64_t>(cap, ch->slots);  // every workgroup of a barrier must be resident
  uint64_t b = std::min(want, cap);
  if (algo == MSCL_ALGO_ONE_SHOT && cap >= kXcds)
    b = std::min((b + kXcds - 1) / kXcds * kXcds, cap / kXcds * kXcds);  // whole XCD groups
  plan->workgroups_per_rank = static_cast<int>(b);
}

// The channel set for (current device, R) and its per-call controls.
struct Bound {
  mscl_channel_s* ch = nullptr;
  uint64_t timeout_us = 0;
  int drop_rank = -1;
};

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
  }
  if (__atomic_load_n(b->ch->status_host, __ATOMIC_ACQUIRE) != MSCL_SUCCESS)
    return fail(MSCL_ERR_TIMEOUT, "an earlier call timed out; call mscl_channel_reset");
  return MSCL_SUCCESS;
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
  a->ch.status = b.ch->status_dev;
  a->ch.slots = b.ch->slots;
  a->ch.drop_rank = b.drop_rank;
  a->ch.timeout_ticks = b.timeout_us * b.ch->wall_clock_khz / 1000;
}

mscl_status_t launch(int kind, int dtype, int nranks, KernelArgs& a, void* stream) {
  KernelFn fn = kernel_lookup(kind, dtype, nranks);
  if (!fn) return fail(MSCL_ERR_INVALID_ARGUMENT, "no kernel for this dtype and rank count");
  const dim3 grid(static_cast<unsigned>(nranks) * a.nblk);
  void* kargs[] = {&a};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(fn), grid, dim3(kThreads), kargs, 0,
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

}  // namespace

extern "C" {

int mscl_version(void) { return MSCL_VERSION_MAJOR * 10000 + MSCL_VERSION_MINOR * 100 + MSCL_VERSION_PATCH; }

const char* mscl_status_string(mscl_status_t s) {
  switch (s) {
    case MSCL_SUCCESS: return "success";
    case MSCL_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MSCL_ERR_UNSUPPORTED: return "unsupported device";
    case MSCL_ERR_MISALIGNED: return "buffer not 16-byte aligned";
    case MSCL_ERR_NOT_INITIALIZED: return "no channel set for this device and rank count";
    case MSCL_ERR_OUT_OF_MEMORY: return "out of memory";
    case MSCL_ERR_HIP: return "HIP runtime error";
    case MSCL_ERR_TIMEOUT: return "device-side wait timed out";
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
  ch->cus = prop.multiProcessorCount;
  int khz = 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, device) == hipSuccess && khz > 0)
    ch->wall_clock_khz = static_cast<uint64_t>(khz);
  // Slots: the fewest workgroups per rank that can be resident at once over
  // every kernel that runs the barrier, so a barrier can never wait on a
  // workgroup that has not been scheduled.
  int min_resident = 1 << 30;
  for (int dt = 0; dt < 3; ++dt) {
    for (int kind : {kAlgoOneShotInPlace, kAlgoTwoShot, kAlgoTwoShotFused}) {
      int per_cu = 0;
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kernel_lookup(kind, dt, nranks)),
                                                       kThreads, 0);
      if (e != hipSuccess) {
        delete ch;
        (void)hipSetDevice(prev);
        return fail_hip(e, "hipOccupancyMaxActiveBlocksPerMultiprocessor");
      }
      min_resident = std::min(min_resident, per_cu * ch->cus);
    }
  }
  ch->slots = static_cast<uint32_t>(std::max(1, std::min(min_resident / nranks, 4096)));
  const size_t inbound_bytes = sizeof(uint32_t) * nranks * nranks * ch->slots;
  const size_t consumed_bytes = sizeof(uint32_t) * nranks * ch->slots;
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
  return MSCL_SUCCESS;
}

mscl_status_t mscl_channel_destroy(mscl_channel_t ch) {
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!ch || !registered(ch)) return fail(MSCL_ERR_INVALID_ARGUMENT, "unknown channel handle");
  if (--ch->refcount > 0) return MSCL_SUCCESS;
  g_registry.erase(std::make_pair(ch->device, ch->nranks));
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
  const int s = __atomic_load_n(ch->status_host, __ATOMIC_ACQUIRE);
  if (s != MSCL_SUCCESS) return fail(s, "a device-side wait timed out in an earlier call");
  return MSCL_SUCCESS;
}

mscl_status_t mscl_channel_reset(mscl_channel_t ch) {
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!ch || !registered(ch)) return fail(MSCL_ERR_INVALID_ARGUMENT, "unknown channel handle");
  int prev = 0;
  (void)hipGetDevice(&prev);
  (void)hipSetDevice(ch->device);
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemset(ch->inbound, 0, sizeof(uint32_t) * ch->nranks * ch->nranks * ch->slots);
  if (e == hipSuccess) e = hipMemset(ch->consumed, 0, sizeof(uint32_t) * ch->nranks * ch->slots);
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
  ch->wait_timeout_us = wait_timeout_us;
  ch->drop_rank = drop_signal_rank;
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
  mscl_plan_t plan;
  make_plan(b.ch, count, dtype, resolved, in_place, &plan);

  KernelArgs a;
  fill_args(&a, b, inputs, outputs, nranks, count);
  a.chunk = plan.chunk_elems;
  a.nblk = static_cast<uint32_t>(plan.workgroups_per_rank);
  a.xcd_grouped = (resolved == MSCL_ALGO_ONE_SHOT && a.nblk % kXcds == 0) ? 1u : 0u;
  const int kind = resolved == MSCL_ALGO_TWO_SHOT         ? kAlgoTwoShot
                   : resolved == MSCL_ALGO_TWO_SHOT_FUSED ? kAlgoTwoShotFused
                   : in_place                             ? kAlgoOneShotInPlace
                                                          : kAlgoOneShot;
  return launch(kind, dtype, nranks, a, stream);
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
  }
  if (__atomic_load_n(ch->status_host, __ATOMIC_ACQUIRE) != MSCL_SUCCESS)
    return fail(MSCL_ERR_TIMEOUT, "an earlier call timed out; call mscl_channel_reset");
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
