// Host side of the port channel: the proxy thread that turns the requests
// GPU threads post (port.hpp) into copies on the SDMA engines, driven
// through HSA directly.  One PortState per channel set, created by its first
// port-channel call.  Included once, by mscl.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <hsa/hsa.h>
#include <hsa/hsa_ext_amd.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cstdlib>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "../../include/mscl.h"
#include "port.hpp"

namespace mscl {
namespace proxy {

// Host side of the port channel of one channel set: the request ring and
// completion counters the kernels see, and the proxy thread that drains the
// ring into copies on the SDMA engines.  The proxy talks to the engines
// through HSA directly (an async copy with a completion signal), not through
// HIP streams: a stream's packets can share a hardware queue with the very
// kernel that is waiting for the copy, and would then wait behind it.
struct PortState {
  static constexpr uint32_t kEntries = 256;  // > R*(R-1), the most requests one call can post
  PortRequest* fifo_host = nullptr;    // host-mapped ring
  PortRequest* fifo_dev = nullptr;
  uint32_t* done_host = nullptr;             // host-mapped completion counters [R]
  uint32_t* done_dev = nullptr;
  uint64_t* head = nullptr;                  // device memory
  uint32_t* issued = nullptr;                // device memory [R]
  uint32_t* arrived = nullptr;               // device memory [R]
  hsa_agent_t agent{};                       // the GPU, as an HSA agent
  std::vector<hsa_amd_sdma_engine_id_t> engines;  // SDMA engines the copies rotate over
  bool hsa_up = false;
  std::thread proxy;
  std::atomic<bool> stop{false};
  int device = 0;
  int nranks = 0;
};


// True when [p, p + bytes) lies inside one device allocation.
inline bool in_one_allocation(uint64_t p, uint64_t bytes) {
  void* base = nullptr;
  size_t size = 0;
  if (hipMemGetAddressRange(&base, &size, reinterpret_cast<void*>(p)) != hipSuccess || !base) return false;
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  return p >= b && bytes <= size && p - b <= size - bytes;
}

// The proxy: take requests off the ring in order, check their ranges, issue
// each as an SDMA copy (the engines taken in turn) with a completion signal,
// and bump the rank's completion counter once the signal has dropped to
// zero.  A request that fails the check or whose copy cannot be issued is
// not counted, so the posting kernel's bounded wait reports
// MSCL_ERR_TIMEOUT.
inline void proxy_loop(PortState* ps, int* status_host) {
  struct Inflight {
    hsa_signal_t sig;
    uint32_t rank;
  };
  std::vector<Inflight> inflight;
  std::vector<hsa_signal_t> pool;
  uint64_t tail = 0;
  uint64_t next_engine = 0;
  // Poll without sleeping for 2 ms after the last request or completion (a
  // sleep, with the kernel's timer slack, costs tens of microseconds per
  // call); after that, back off to short sleeps so an idle set costs no core.
  using Clock = std::chrono::steady_clock;
  Clock::time_point last_activity = Clock::now();
  auto fail_status = [&](mscl_status_t s) { __atomic_store_n(status_host, static_cast<int>(s), __ATOMIC_RELEASE); };
  while (!ps->stop.load(std::memory_order_acquire)) {
    bool progress = false;
    for (;;) {
      PortRequest* e = ps->fifo_host + (tail & (PortState::kEntries - 1));
      if (__atomic_load_n(&e->seq, __ATOMIC_ACQUIRE) != static_cast<uint32_t>(tail + 1)) break;
      const uint64_t dst = e->dst, src = e->src, bytes = e->bytes;
      const uint32_t rank = e->rank;
      ++tail;
      progress = true;
      if (rank >= static_cast<uint32_t>(ps->nranks) || !in_one_allocation(dst, bytes) ||
          !in_one_allocation(src, bytes)) {
        fail_status(MSCL_ERR_INVALID_ARGUMENT);
        continue;
      }
      hsa_signal_t sig{};
      if (!pool.empty()) {
        sig = pool.back();
        pool.pop_back();
        hsa_signal_store_relaxed(sig, 1);
      } else if (hsa_signal_create(1, 0, nullptr, &sig) != HSA_STATUS_SUCCESS) {
        fail_status(MSCL_ERR_HIP);
        continue;
      }
      const hsa_amd_sdma_engine_id_t engine = ps->engines[next_engine++ % ps->engines.size()];
      if (hsa_amd_memory_async_copy_on_engine(reinterpret_cast<void*>(dst), ps->agent,
                                              reinterpret_cast<const void*>(src), ps->agent, bytes, 0, nullptr, sig,
                                              engine, true) != HSA_STATUS_SUCCESS) {
        fail_status(MSCL_ERR_HIP);
        pool.push_back(sig);
        continue;
      }
      inflight.push_back({sig, rank});
    }
    for (size_t i = 0; i < inflight.size();) {
      if (hsa_signal_load_scacquire(inflight[i].sig) != 0) {
        ++i;
        continue;
      }
      __atomic_fetch_add(ps->done_host + inflight[i].rank, 1u, __ATOMIC_RELEASE);
      pool.push_back(inflight[i].sig);
      inflight[i] = inflight.back();
      inflight.pop_back();
      progress = true;
    }
    if (progress)
      last_activity = Clock::now();
    else if (Clock::now() - last_activity > std::chrono::milliseconds(2))
      std::this_thread::sleep_for(std::chrono::microseconds(20));
  }
  for (auto& f : inflight) {
    hsa_signal_wait_scacquire(f.sig, HSA_SIGNAL_CONDITION_EQ, 0, UINT64_MAX, HSA_WAIT_STATE_BLOCKED);
    pool.push_back(f.sig);
  }
  for (hsa_signal_t sig : pool) hsa_signal_destroy(sig);
}

// The HSA agent of HIP device `device` (matched by PCI domain, bus and
// device), and a CPU agent.
inline bool find_hsa_agents(int device, hsa_agent_t* out, hsa_agent_t* cpu) {
  int bus = -1, dev = -1, dom = 0;
  if (hipDeviceGetAttribute(&bus, hipDeviceAttributePciBusId, device) != hipSuccess ||
      hipDeviceGetAttribute(&dev, hipDeviceAttributePciDeviceId, device) != hipSuccess)
    return false;
  (void)hipDeviceGetAttribute(&dom, hipDeviceAttributePciDomainID, device);
  struct Want {
    uint32_t dom, bus, dev;
    hsa_agent_t found, cpu;
    bool ok, cpu_ok;
  } want{static_cast<uint32_t>(dom), static_cast<uint32_t>(bus), static_cast<uint32_t>(dev), {}, {}, false, false};
  auto visit = [](hsa_agent_t a, void* data) -> hsa_status_t {
    auto* w = static_cast<Want*>(data);
    hsa_device_type_t type;
    if (hsa_agent_get_info(a, HSA_AGENT_INFO_DEVICE, &type) != HSA_STATUS_SUCCESS) return HSA_STATUS_SUCCESS;
    if (type == HSA_DEVICE_TYPE_CPU && !w->cpu_ok) {
      w->cpu = a;
      w->cpu_ok = true;
    }
    if (type != HSA_DEVICE_TYPE_GPU) return HSA_STATUS_SUCCESS;
    uint32_t bdf = 0, adom = 0;
    if (hsa_agent_get_info(a, static_cast<hsa_agent_info_t>(HSA_AMD_AGENT_INFO_BDFID), &bdf) != HSA_STATUS_SUCCESS)
      return HSA_STATUS_SUCCESS;
    (void)hsa_agent_get_info(a, static_cast<hsa_agent_info_t>(HSA_AMD_AGENT_INFO_DOMAIN), &adom);
    if (((bdf >> 8) & 0xff) == w->bus && ((bdf >> 3) & 0x1f) == w->dev && adom == w->dom) {
      w->found = a;
      w->ok = true;
    }
    return HSA_STATUS_SUCCESS;
  };
  (void)hsa_iterate_agents(visit, &want);
  if (want.ok) *out = want.found;
  if (want.cpu_ok) *cpu = want.cpu;
  return want.ok && want.cpu_ok;
}

inline void port_free(PortState* ps) {
  if (ps->fifo_host) (void)hipHostFree(ps->fifo_host);
  if (ps->done_host) (void)hipHostFree(ps->done_host);
  if (ps->head) (void)hipFree(ps->head);
  if (ps->issued) (void)hipFree(ps->issued);
  if (ps->arrived) (void)hipFree(ps->arrived);
  if (ps->hsa_up) (void)hsa_shut_down();  // drops this reference; the HIP runtime holds its own
  delete ps;
}

inline void proxy_join(PortState* ps) {
  ps->stop.store(true, std::memory_order_release);
  if (ps->proxy.joinable()) ps->proxy.join();
}

// Proxies started in this process, for the exit hook.
inline std::mutex& live_mutex() {
  static std::mutex m;
  return m;
}
inline std::vector<PortState*>& live_proxies() {
  static std::vector<PortState*> v;
  return v;
}

// At process exit, before the HIP runtime tears itself down (this handler
// is registered after the runtime has started, so it runs first): stop every
// proxy thread, so none is left calling into HIP.
inline void join_all_proxies() {
  std::lock_guard<std::mutex> lock(live_mutex());
  for (PortState* ps : live_proxies()) proxy_join(ps);
}

// Stop the proxy and release the port state (the caller has synchronised
// every stream that used it).
inline void close_port(PortState* ps, int device) {
  if (!ps) return;
  {
    std::lock_guard<std::mutex> lock(live_mutex());
    auto& v = live_proxies();
    v.erase(std::remove(v.begin(), v.end(), ps), v.end());
  }
  proxy_join(ps);
  int prev = 0;
  (void)hipGetDevice(&prev);
  (void)hipSetDevice(device);
  port_free(ps);
  (void)hipSetDevice(prev);
}

// Back to the state of a fresh port channel, keeping its allocations (so a
// graph captured earlier still points at live memory): stop the proxy, zero
// the ring and every counter, start the proxy again.  The caller has
// synchronised the device.
inline hipError_t restart_port(PortState* ps, int* status_host) {
  if (!ps) return hipSuccess;
  proxy_join(ps);
  memset(ps->fifo_host, 0, sizeof(PortRequest) * PortState::kEntries);
  memset(ps->done_host, 0, sizeof(uint32_t) * ps->nranks);
  hipError_t e = hipMemset(ps->head, 0, sizeof(uint64_t));
  if (e == hipSuccess) e = hipMemset(ps->issued, 0, sizeof(uint32_t) * ps->nranks);
  if (e == hipSuccess) e = hipMemset(ps->arrived, 0, sizeof(uint32_t) * ps->nranks);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  ps->stop.store(false, std::memory_order_release);
  ps->proxy = std::thread(proxy_loop, ps, status_host);
  return e;
}

// Allocate the ring and counters, find the copy engines and start the proxy
// for `nranks` ranks on `device`.  On failure returns the status and sets
// `why`; nothing is left allocated.
inline mscl_status_t open_port(int device, int nranks, int* status_host, PortState** out, std::string* why_out) {
  auto* ps = new PortState();
  ps->device = device;
  ps->nranks = nranks;
  int prev = 0;
  (void)hipGetDevice(&prev);
  hipError_t e = hipSetDevice(device);
  const size_t fifo_bytes = sizeof(PortRequest) * PortState::kEntries;
  const size_t ctr_bytes = sizeof(uint32_t) * nranks;
  if (e == hipSuccess)
    e = hipHostMalloc(reinterpret_cast<void**>(&ps->fifo_host), fifo_bytes, hipHostMallocMapped | hipHostMallocCoherent);
  if (e == hipSuccess)
    e = hipHostMalloc(reinterpret_cast<void**>(&ps->done_host), ctr_bytes, hipHostMallocMapped | hipHostMallocCoherent);
  if (e == hipSuccess) e = hipHostGetDevicePointer(reinterpret_cast<void**>(&ps->fifo_dev), ps->fifo_host, 0);
  if (e == hipSuccess) e = hipHostGetDevicePointer(reinterpret_cast<void**>(&ps->done_dev), ps->done_host, 0);
  if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void**>(&ps->head), sizeof(uint64_t));
  if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void**>(&ps->issued), ctr_bytes);
  if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void**>(&ps->arrived), ctr_bytes);
  if (e == hipSuccess) {
    memset(ps->fifo_host, 0, fifo_bytes);
    memset(ps->done_host, 0, ctr_bytes);
  }
  if (e == hipSuccess) e = hipMemset(ps->head, 0, sizeof(uint64_t));
  if (e == hipSuccess) e = hipMemset(ps->issued, 0, ctr_bytes);
  if (e == hipSuccess) e = hipMemset(ps->arrived, 0, ctr_bytes);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    port_free(ps);
    (void)hipSetDevice(prev);
    *why_out = std::string("port channel set-up: ") + hipGetErrorString(e);
    return MSCL_ERR_HIP;
  }
  // The copy engines: HSA (already started by the HIP runtime; this takes a
  // reference), the device's agent, and the SDMA engines free for
  // device-to-device copies on it.
  // The device-to-device status lists only the engines free at this moment;
  // when it lists none, the engines the device has for host transfers are
  // used (a copy forced onto SDMA may run on any of them).
  uint32_t mask = 0;
  const char* why = nullptr;
  hsa_agent_t cpu{};
  if (hsa_init() != HSA_STATUS_SUCCESS) why = "hsa_init failed";
  else ps->hsa_up = true;
  if (!why && !find_hsa_agents(device, &ps->agent, &cpu)) why = "no HSA agent matches the device";
  if (!why && (hsa_amd_memory_copy_engine_status(ps->agent, ps->agent, &mask) != HSA_STATUS_SUCCESS || mask == 0)) {
    uint32_t in = 0, out = 0;
    if (hsa_amd_memory_copy_engine_status(ps->agent, cpu, &in) != HSA_STATUS_SUCCESS) in = 0;
    if (hsa_amd_memory_copy_engine_status(cpu, ps->agent, &out) != HSA_STATUS_SUCCESS) out = 0;
    mask = in | out;
  }
  if (!why && mask == 0) why = "the device has no SDMA engine";
  for (uint32_t bit = 0; bit < 16 && !why; ++bit)
    if (mask & (1u << bit)) ps->engines.push_back(static_cast<hsa_amd_sdma_engine_id_t>(1u << bit));
  if (why) {
    port_free(ps);
    (void)hipSetDevice(prev);
    *why_out = std::string("port channel: ") + why;
    return MSCL_ERR_UNSUPPORTED;
  }
  (void)hipSetDevice(prev);
  // The live list and its mutex are built before the hook is registered, so
  // that at exit they are destroyed only after the hook has run.
  static std::once_flag exit_hook;
  std::call_once(exit_hook, [] {
    (void)live_mutex();
    (void)live_proxies();
    std::atexit(join_all_proxies);
  });
  ps->proxy = std::thread(proxy_loop, ps, status_host);
  {
    std::lock_guard<std::mutex> lock(live_mutex());
    live_proxies().push_back(ps);
  }
  *out = ps;
  return MSCL_SUCCESS;
}

}  // namespace proxy
}  // namespace mscl
