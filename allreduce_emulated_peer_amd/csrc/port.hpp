// PortChannel-style device side: put requests handed to a host proxy.
//
// The pages' second channel kind (MSCCL++ README, Key Concepts, "PortChannel
// and MemoryChannel" and "Host-Side Communication Proxy"): instead of GPU
// threads copying the data themselves, one GPU thread posts a request into a
// FIFO that a CPU proxy thread drains, and the proxy moves the bytes with a
// DMA engine, so the GPU spends no compute units on the transfer.
//
// Here the FIFO is a ring of PortRequest entries in host-mapped memory.  A
// request is one put (`bytes` bytes from device address `src` to device
// address `dst`) tagged with the rank whose completion counter the proxy
// bumps once that copy has finished.  The proxy issues the copies on the
// SDMA engines through HSA (a copy forced onto a given engine, completion
// polled on an HSA signal) and checks each request's ranges against the
// device allocations before it copies anything.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "channel.hpp"

namespace mscl {

struct PortRequest {
  uint64_t dst;
  uint64_t src;
  uint64_t bytes;
  uint32_t rank;  // whose completion counter the proxy bumps
  uint32_t seq;   // ring index + 1, written last: the entry is complete once it matches
};
static_assert(sizeof(PortRequest) == 32, "ring entries are 32 bytes");

// Port channel state of one launch, passed by value in the kernel arguments.
struct PortArgs {
  PortRequest* fifo;   // host-mapped ring
  uint64_t* head;      // device memory: next ring index to reserve
  uint32_t* done;      // host-mapped, written by the proxy: puts completed per rank
  uint32_t* issued;    // device memory: puts posted per rank so far
  uint32_t* arrived;   // device memory: workgroups of a rank done with this call's reduce-scatter
  uint32_t fifo_mask;  // ring capacity - 1
};

struct PortChannel {
  const PortArgs& pa;
  const ChannelArgs& ch;

  // put(): post one request.  Executed by one thread per request.
  __device__ void put(int rank, const void* dst, const void* src, uint64_t bytes) const {
    const uint64_t idx = __hip_atomic_fetch_add(pa.head, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    PortRequest* e = pa.fifo + (idx & pa.fifo_mask);
    __hip_atomic_store(&e->dst, reinterpret_cast<uint64_t>(dst), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    __hip_atomic_store(&e->src, reinterpret_cast<uint64_t>(src), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    __hip_atomic_store(&e->bytes, bytes, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    __hip_atomic_store(&e->rank, static_cast<uint32_t>(rank), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    __hip_atomic_store(&e->seq, static_cast<uint32_t>(idx + 1), __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
  }

  // flush(): until the proxy has completed `target` puts of `rank` in total
  // (wrap-safe compare), bounded like every wait; false on timeout.
  __device__ bool flush(int rank, uint32_t target) const {
    const uint32_t* c = pa.done + rank;
    const uint64_t start = wall_clock64();
    while (static_cast<int32_t>(__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) - target) < 0) {
      if (wall_clock64() - start > ch.timeout_ticks) {
        __hip_atomic_store(ch.status, kStatusTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        return false;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    return true;
  }
};

}  // namespace mscl
