// MemoryChannel-style device layer for R emulated ranks on one GPU.
//
// Semantics follow the channel methods described for MSCCL++ (README, Key
// Concepts, "On-GPU Communication Interfaces: Channels" and "PortChannel and
// MemoryChannel"):
//   put(dstOffset, srcOffset, size)  copy `size` bytes from local memory at
//                                    srcOffset to the peer's memory at
//                                    dstOffset (offsets and size in bytes);
//                                    a MemoryChannel does it with many GPU
//                                    threads loading and storing directly.
//   get                              the reverse direction: read the peer's
//                                    memory directly.
//   signal()                         tell the peer this side has arrived and
//                                    its earlier writes have completed.
//   flush()                          wait until this side's earlier channel
//                                    operations are finished as the local
//                                    GPU sees them.
//   wait()                           block until the peer has signalled.
//   barrier                          signal, (flush,) wait, then a local
//                                    workgroup barrier so the other local
//                                    threads are synchronised too.
//   per-tile semaphores              a signal per finished tile, so a peer
//                                    waits only for the tile it needs
//                                    (TileSemaphores).
//
// On one GPU a "peer's memory" is another buffer in the same HBM, reached by
// ordinary global loads and stores; the rank boundary that matters is the
// workgroup boundary (and, across the 8 XCDs, separate L2 caches).  A
// channel therefore connects (rank r, slot b) with (rank p, slot b): slot b is
// the b-th workgroup of each rank.  Its semaphore is a 32-bit counter in
// global memory, inbound[r][p][b], counting signals rank p's slot b has sent
// to rank r's slot b.  Counters only grow; the number of signals a slot has
// already consumed is kept per (rank, slot) in device memory (not in kernel
// arguments), so repeated launches and replays of a captured graph wait for
// the right epoch.  Comparisons are wrap-safe.
//
// Memory ordering across XCDs: signal is an agent-scope release atomic add
// (the compiler emits an L2 write-back before it), wait spins on agent-scope
// relaxed loads (which bypass the non-coherent caches) and ends with an
// agent-scope acquire fence (L1/L2 invalidate).  Waits are bounded by a
// wall-clock budget; on expiry the kernel records MSCL_ERR_TIMEOUT in the
// host-mapped status word and carries on, so no wave is ever left spinning.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "codec.hpp"

namespace mscl {

constexpr int kMaxRanks = 16;
constexpr int kStatusTimeout = 7;   // MSCL_ERR_TIMEOUT
constexpr int kStatusProtocol = 8;  // MSCL_ERR_PROTOCOL

// Channel state of one launch, passed by value in the kernel arguments.
struct ChannelArgs {
  uint32_t* inbound;       // [R][R][slots] signal counters
  uint32_t* consumed;      // [R][slots] signals consumed per peer so far
  int* status;             // host-mapped status word
  uint32_t slots;          // slot stride of inbound / consumed
  int32_t drop_rank;       // test control: this rank skips signal(); -1 = none
  int32_t double_rank;     // test control: this rank signals twice each time; -1 = none
  int32_t check_protocol;  // nonzero: every wait checks the count it reads (kStatusProtocol)
  uint64_t timeout_ticks;  // bound of one wait(), in wall-clock ticks (100 MHz)
  uint32_t* progress;      // [R][slots] per-tile semaphores: tiles each (rank, slot) has finished, all calls
  uint32_t* seen;          // [R][R][slots] the peer's progress a (rank, slot) had consumed before this call
};

// A semaphore held a count that calls ordered on one stream cannot produce.
__device__ inline void record_protocol_fault(const ChannelArgs& ch) {
  __hip_atomic_store(ch.status, kStatusProtocol, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// What a barrier orders across ranks (see RankChannels::barrier_all).
enum class Sync { kPublish, kAfterReads, kAfterWrites, kArrival };

// The channels of rank `rank`'s slot `slot` to all of its peers.
struct RankChannels {
  const ChannelArgs& ch;
  int nranks;
  int rank;
  int slot;

  __device__ uint32_t* inbound_from(int peer) const {
    return ch.inbound + (static_cast<uint64_t>(rank) * nranks + peer) * ch.slots + slot;
  }
  __device__ uint32_t* inbound_of(int peer) const {  // the peer's counter for signals from us
    return ch.inbound + (static_cast<uint64_t>(peer) * nranks + rank) * ch.slots + slot;
  }

  // signal(): release-ordered increment of the peer's inbound counter.
  __device__ void signal(int peer) const {
    if (rank == ch.drop_rank) return;
    __hip_atomic_fetch_add(inbound_of(peer), rank == ch.double_rank ? 2u : 1u, __ATOMIC_RELEASE,
                           __HIP_MEMORY_SCOPE_AGENT);
  }

  // Arrival-only signal: the same increment with no ordering of earlier
  // memory operations (no L2 write-back).  For rendezvous points where the
  // peer will not read anything this rank wrote.
  __device__ void signal_arrival(int peer) const {
    if (rank == ch.drop_rank) return;
    __hip_atomic_fetch_add(inbound_of(peer), rank == ch.double_rank ? 2u : 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
  }

  // flush(): earlier stores complete from this device's point of view.
  __device__ static void flush() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }

  // wait(): until the peer's signal count reaches `epoch`; false on timeout.
  // The caller adds the acquire fence when it will read the peer's data.
  // With ch.check_protocol every count read must lie within one signal of
  // the epoch: this slot passed its previous barrier only once the peer had
  // signalled epoch - 1, and the peer cannot signal epoch + 1 before this
  // slot has signalled it.  A count outside that window means another call,
  // or a reset, touched the same counters; it is recorded as kStatusProtocol
  // and the wait goes on as usual.
  __device__ bool wait(int peer, uint32_t epoch) const {
    if (ch.check_protocol) return wait_checked(peer, epoch);
    const uint32_t* c = inbound_from(peer);
    const uint64_t start = wall_clock64();
    while (static_cast<int32_t>(__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) - epoch) < 0) {
      if (wall_clock64() - start > ch.timeout_ticks) {
        __hip_atomic_store(ch.status, kStatusTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        return false;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    return true;
  }

  // wait() with the protocol checks, a loop of its own so that the unchecked
  // wait keeps its short exit path (measured 0.08 us per call at 512 KiB).
  __device__ bool wait_checked(int peer, uint32_t epoch) const {
    const uint32_t* c = inbound_from(peer);
    int32_t d = static_cast<int32_t>(__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) - epoch);
    if (d < 0) {
      const uint64_t start = wall_clock64();
      while (true) {
        if (d < -1) record_protocol_fault(ch);
        if (wall_clock64() - start > ch.timeout_ticks) {
          __hip_atomic_store(ch.status, kStatusTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
          return false;
        }
        __builtin_amdgcn_s_sleep(1);
        d = static_cast<int32_t>(__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) - epoch);
        if (d >= 0) break;
      }
    }
    if (d > 1) record_protocol_fault(ch);
    return true;
  }

  // Barrier of this slot with the same slot of every peer.  Executed by the
  // whole workgroup.  Lane p of wave 0 drives the channel to peer p, so the
  // R-1 signals and waits of a slot go out as one vector instruction each.
  //
  // Sync::kPublish is the pages' barrier: signal() publishes everything this
  // workgroup wrote before it, and an acquire after the waits makes what the
  // peers wrote before their signals visible here.  It fences every thread,
  // not only the signalling wave: on gfx950 a workgroup barrier does not wait
  // for the other waves' global loads and stores to complete, and the
  // signalling wave's release covers only its own, so a peer on another XCD
  // could otherwise see the signal before a sibling wave's stores reached
  // memory (found by mscl_channel_selftest: a few stale words per 10^5).
  //
  // Sync::kAfterReads orders this workgroup's earlier loads before the
  // peers' later stores (write after read across ranks, no data handed
  // over): every thread waits until its own loads and stores have completed,
  // then the signal goes out arrival-only and nothing is acquired.  A load
  // that has returned its value cannot observe a store issued later, and a
  // peer issues its stores only after its wait has seen this signal.  It
  // skips kPublish's L2 write-back and invalidate, which on MI355X also
  // discard the L2 lines every rank is re-reading.
  //
  // Sync::kAfterWrites is the completion barrier of puts made with
  // device-scope stores (store_vec_scoped): every thread waits until its own
  // stores have been acknowledged, which for device-scope stores means every
  // XCD can see them, so the arrival-only signal that follows already carries
  // the pages' promise that earlier writes are complete, without the L2
  // write-back of a release fence.  Nothing is acquired after the waits: the
  // kernels that end with this barrier read nothing afterwards, and the next
  // kernel on the stream starts with invalidated caches.  (A consumer fused
  // behind it in the same kernel would add an agent-scope acquire, an L2
  // invalidate that measured 1.3-3 us per call on MI355X.)
  //
  // Sync::kArrival is a pure rendezvous (arrival-only signal, no waiting for
  // earlier accesses, no acquire) for protocols in which no memory is shared
  // across ranks at this point; on MI355X it saves the per-workgroup L2
  // write-back and invalidate, 6-10 us per launch.
  template <Sync kSync>
  __device__ void barrier_all() const {
    constexpr bool kPublishing = kSync == Sync::kPublish;
    constexpr bool kCompleting = kSync == Sync::kAfterReads || kSync == Sync::kAfterWrites;
    if (kPublishing) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");  // this thread's accesses, published
    if (kCompleting) __builtin_amdgcn_s_waitcnt(0);  // this thread's accesses, completed
    __syncthreads();  // every local thread has reached the barrier
    if (threadIdx.x < 64) {
      const int peer = threadIdx.x;
      uint32_t* consumed = ch.consumed + static_cast<uint64_t>(rank) * ch.slots + slot;
      // vector (atomic) accesses: the counter is rewritten inside the kernel
      const uint32_t epoch = __hip_atomic_load(consumed, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) + 1u;
      const bool active = peer < nranks && peer != rank;
      if (active) {
        if (kPublishing)
          signal(peer);
        else
          signal_arrival(peer);
      }
      if (active) wait(peer, epoch);
      if (kPublishing) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      if (peer == 0) __hip_atomic_store(consumed, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    __syncthreads();  // the rest of the workgroup is now synchronised with the peers
    if (kPublishing) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // and sees what they published
  }
};

// Per-tile semaphores of slot `slot` of rank `rank`.  Slot b of rank p counts
// the tiles it has finished in progress[p][b]; the counter only grows.  Slot b
// of rank r keeps, in seen[r][p][b], how much of peer p's count it had
// consumed before the current call, so "tile j of this call is ready" is
// progress - seen >= j + 1 (wrap-safe).  Producer and consumer of a tile are
// always the same slot of two ranks, so slots whose workgroup count changes
// between calls stay consistent pairwise, as with the barrier's epochs.
struct TileSemaphores {
  const ChannelArgs& ch;
  int nranks;
  int rank;
  int slot;

  __device__ uint32_t* progress_of(int p) const {
    return ch.progress + static_cast<uint64_t>(p) * ch.slots + slot;
  }
  __device__ uint32_t* seen_of(int p) const {
    return ch.seen + (static_cast<uint64_t>(rank) * nranks + p) * ch.slots + slot;
  }

  // One more tile of this slot is finished.  The caller has waited for the
  // tile's device-scope stores to be acknowledged, so the arrival-only
  // increment already promises the peers that the tile's data is complete.
  __device__ void signal_tile() const {
    if (rank == ch.drop_rank) return;
    __hip_atomic_fetch_add(progress_of(rank), rank == ch.double_rank ? 2u : 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
  }

  // With ch.check_protocol: a peer's count of finished tiles in this call
  // lies between 0 and the `total` tiles its slot signals in the call;
  // anything else is recorded as kStatusProtocol.
  __device__ void check_tiles(uint32_t have, uint32_t total) const {
    if (ch.check_protocol && (static_cast<int32_t>(have) < 0 || have > total)) record_protocol_fault(ch);
  }

  // Tiles of this call peer p's slot has finished (progress - base), polled
  // until at least `need` (of `total`).  On running out of time the status
  // records TIMEOUT and every tile of the peer is reported finished, so the
  // caller waits for that peer at most once per call (its outputs are then
  // wrong).
  __device__ uint32_t wait_tiles(int p, uint32_t base, uint32_t need, uint32_t total) const {
    const uint32_t* c = progress_of(p);
    uint32_t have = __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) - base;
    if (static_cast<int32_t>(have - need) >= 0) {
      check_tiles(have, total);
      return have;
    }
    const uint64_t start = wall_clock64();
    while (true) {
      check_tiles(have, total);
      __builtin_amdgcn_s_sleep(1);
      have = __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) - base;
      if (static_cast<int32_t>(have - need) >= 0) {
        check_tiles(have, total);
        return have;
      }
      if (wall_clock64() - start > ch.timeout_ticks) {
        __hip_atomic_store(ch.status, kStatusTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        return 0x7FFFFFFFu;
      }
    }
  }
};

// put() at lane granularity: vector `vi` of this rank's buffer `src` is
// written to the same vector offset of every peer's buffer.  A workgroup
// whose lanes cover consecutive vectors performs the pages' cooperative
// put(dstOffset, srcOffset, size) to all R-1 peers at once, reading the
// source once instead of once per peer.
template <class C, int R>
__device__ inline void put_to_peers(void* const* dst, int rank, uint64_t vi, const u32x4& v,
                                    uint64_t nfull, int ntail) {
#pragma unroll
  for (int p = 0; p < R; ++p)
    if (p != rank) store_any<C>(dst[p], vi, v, nfull, ntail);
}

}  // namespace mscl
