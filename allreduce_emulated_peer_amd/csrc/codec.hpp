// 16-byte vector I/O and element codecs for gfx950.
//
// Every rank buffer is moved in 16-byte vectors (one global_load_dwordx4 /
// global_store_dwordx4 per lane, 1 KiB per wavefront instruction, fully
// coalesced).  A vector holds V = 16 / sizeof(element) elements.  Elements are
// widened to binary32 exactly and the binary32 totals are rounded back with
// the hardware's round-to-nearest-even conversions:
//   bf16 -> f32 : 16-bit shift (exact)
//   f16  -> f32 : v_cvt_f32_f16 (exact, subnormals kept)
//   f32  -> bf16: v_cvt_pk_bf16_f32 (gfx950; RNE, NaN stays NaN)
//   f32  -> f16 : v_cvt_f16_f32 (RNE, subnormals kept, overflow to Inf)
// The partial vector at the end of a rank's range is handled element by
// element so that no access goes past the buffer.
//
// Vector lanes are always copied into a scalar before __builtin_bit_cast:
// bit-casting a subscripted ext_vector element directly reads lane 0.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mscl {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

struct F32 {
  static constexpr int kElemBytes = 4;
  static constexpr int V = 4;
  using Bits = uint32_t;
  __device__ static inline float widen(Bits b) { return __builtin_bit_cast(float, b); }
  __device__ static inline Bits narrow(float f) { return __builtin_bit_cast(uint32_t, f); }
  __device__ static inline void unpack(const u32x4& v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = v[i];
      f[i] = __builtin_bit_cast(float, w);
    }
  }
  __device__ static inline u32x4 pack(const float* f) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x = f[i];
      v[i] = __builtin_bit_cast(uint32_t, x);
    }
    return v;
  }
};

struct BF16 {
  static constexpr int kElemBytes = 2;
  static constexpr int V = 8;
  using Bits = uint16_t;
  __device__ static inline float widen(Bits b) { return __builtin_bit_cast(float, static_cast<uint32_t>(b) << 16); }
  __device__ static inline Bits narrow(float f) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f)); }
  __device__ static inline void unpack(const u32x4& v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __builtin_bit_cast(float, v[i] << 16);
      f[2 * i + 1] = __builtin_bit_cast(float, v[i] & 0xFFFF0000u);
    }
  }
  __device__ static inline u32x4 pack(const float* f) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x2 pair = {f[2 * i], f[2 * i + 1]};
      const bf16x2 h = __builtin_convertvector(pair, bf16x2);
      v[i] = __builtin_bit_cast(uint32_t, h);
    }
    return v;
  }
};

struct F16 {
  static constexpr int kElemBytes = 2;
  static constexpr int V = 8;
  using Bits = uint16_t;
  __device__ static inline float widen(Bits b) { return static_cast<float>(__builtin_bit_cast(_Float16, b)); }
  __device__ static inline Bits narrow(float f) { return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f)); }
  __device__ static inline void unpack(const u32x4& v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = v[i];
      const f16x2 h = __builtin_bit_cast(f16x2, w);
      f[2 * i] = (float)h[0];
      f[2 * i + 1] = (float)h[1];
    }
  }
  __device__ static inline u32x4 pack(const float* f) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x2 pair = {f[2 * i], f[2 * i + 1]};
      const f16x2 h = __builtin_convertvector(pair, f16x2);
      v[i] = __builtin_bit_cast(uint32_t, h);
    }
    return v;
  }
};

// Full 16-byte vector `vi` of a buffer.
__device__ inline u32x4 load_vec(const void* base, uint64_t vi) {
  return reinterpret_cast<const u32x4*>(base)[vi];
}
__device__ inline void store_vec(void* base, uint64_t vi, const u32x4& v) {
  reinterpret_cast<u32x4*>(base)[vi] = v;
}

// Streaming (non-temporal) forms, for data touched once: on gfx950 they set
// the instruction's nt bit so the lines do not displace reusable data in the
// caches.  Measured on MI355X: streaming loads lift an 8-input reduction from
// about 5.2 to 6.0 TB/s, and streaming stores lift a one-to-seven fan-out
// copy from about 5.5 to 6.4 TB/s.
__device__ inline u32x4 load_vec_nt(const void* base, uint64_t vi) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base) + vi);
}
__device__ inline void store_vec_nt(void* base, uint64_t vi, const u32x4& v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(base) + vi);
}

// Device-scope temporal form, for puts whose destination is read soon by the
// next kernel: the sc1 bit writes the line through this XCD's L2 to the
// memory side at once (no dirty lines left for the end-of-kernel L2
// write-back), and without the nt bit the Infinity Cache keeps it for the
// reader.  Issued as a raw buffer store whose range is [base, base + nbytes):
// the 32-bit byte offset limits it to buffers below 4 GiB, and a store past
// nbytes is dropped by the hardware's range check instead of landing outside
// the buffer.
constexpr int kBufferSc1 = 1 << 4;                  // cache-policy operand: sc1
constexpr int kRawBufferWord3 = 0x00020000;         // raw (untyped) buffer, 32-bit data format
__device__ inline void store_vec_device(void* base, uint32_t nbytes, uint64_t vi, const u32x4& v) {
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(base, 0, nbytes, kRawBufferWord3);
  __builtin_amdgcn_raw_buffer_store_b128(v, rsrc, static_cast<uint32_t>(vi * 16), 0, kBufferSc1);
}

// Device-scope puts addressed from a wave-uniform base: a buffer resource
// starts at vector `v0` of `base` and covers `nvec` vectors, so every offset
// fits 32 bits whatever the buffer's size, and a lane whose vector lies past
// the range has its store dropped by the hardware's range check.  kCpol is
// the cache-policy operand: kBufferSc1 (device scope, temporal) or
// kBufferSc1 | kBufferNt (device scope, streaming).  A store with device
// scope is acknowledged only once every XCD can see it, so waiting for the
// acknowledgement (s_waitcnt) is all a later signal needs to publish it: the
// whole-L2 write-back of a release fence is not needed for these stores.
constexpr int kBufferNt = 1 << 1;  // cache-policy operand: nt
__device__ inline __amdgpu_buffer_rsrc_t tile_rsrc(void* base, uint64_t v0, uint64_t nvec) {
  return __builtin_amdgcn_make_buffer_rsrc(static_cast<char*>(base) + v0 * 16, 0, static_cast<int>(nvec * 16),
                                           kRawBufferWord3);
}
template <int kCpol>
__device__ inline void store_vec_scoped(__amdgpu_buffer_rsrc_t rsrc, uint32_t vi, const u32x4& v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, rsrc, vi * 16, 0, kCpol);
}

// The first `nvalid` (< V) elements of vector `vi` of `base`, stored element
// by element with device scope (the partial vector at a buffer's end).
template <class C, int kCpol>
__device__ inline void store_partial_scoped(void* base, uint64_t vi, const u32x4& v, int nvalid) {
  const __amdgpu_buffer_rsrc_t rsrc = tile_rsrc(base, vi, 1);
  if constexpr (C::kElemBytes == 4) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (k < nvalid) __builtin_amdgcn_raw_buffer_store_b32(v[k], rsrc, 4 * k, 0, kCpol);
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (k < nvalid)
        __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(v[k >> 1] >> (16 * (k & 1))), rsrc, 2 * k, 0,
                                              kCpol);
  }
}

// Device-scope loads: what another XCD stored with device scope, read past
// this XCD's (possibly stale) L2 lines.  Lanes past the resource's range read
// zero.
template <int kCpol>
__device__ inline u32x4 load_vec_scoped(__amdgpu_buffer_rsrc_t rsrc, uint32_t vi) {
  return __builtin_amdgcn_raw_buffer_load_b128(rsrc, vi * 16, 0, kCpol);
}

// The first `nvalid` (< V) elements of vector `vi` of `base`, loaded element
// by element with device scope; the rest read as zero bits.
template <class C, int kCpol>
__device__ inline u32x4 load_partial_scoped(const void* base, uint64_t vi, int nvalid) {
  const __amdgpu_buffer_rsrc_t rsrc = tile_rsrc(const_cast<void*>(base), vi, 1);
  u32x4 v = {0u, 0u, 0u, 0u};
  if constexpr (C::kElemBytes == 4) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (k < nvalid) v[k] = __builtin_amdgcn_raw_buffer_load_b32(rsrc, 4 * k, 0, kCpol);
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (k < nvalid)
        v[k >> 1] |= static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(rsrc, 2 * k, 0, kCpol)) << (16 * (k & 1));
  }
  return v;
}

// First `nvalid` (< V) elements of vector `vi`; the rest read as zero bits.
template <class C>
__device__ inline u32x4 load_partial(const void* base, uint64_t vi, int nvalid) {
  u32x4 v = {0u, 0u, 0u, 0u};
  if constexpr (C::kElemBytes == 4) {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(base) + vi * 4;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (k < nvalid) v[k] = p[k];
  } else {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(base) + vi * 8;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (k < nvalid) v[k >> 1] |= static_cast<uint32_t>(p[k]) << (16 * (k & 1));
  }
  return v;
}

// Store only the first `nvalid` (< V) elements of vector `vi`.
template <class C>
__device__ inline void store_partial(void* base, uint64_t vi, const u32x4& v, int nvalid) {
  if constexpr (C::kElemBytes == 4) {
    uint32_t* p = reinterpret_cast<uint32_t*>(base) + vi * 4;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (k < nvalid) p[k] = v[k];
  } else {
    uint16_t* p = reinterpret_cast<uint16_t*>(base) + vi * 8;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (k < nvalid) p[k] = static_cast<uint16_t>(v[k >> 1] >> (16 * (k & 1)));
  }
}

// Vector `vi` of a range holding `nfull` full vectors followed by a partial
// vector of `ntail` elements.
template <class C>
__device__ inline u32x4 load_any(const void* base, uint64_t vi, uint64_t nfull, int ntail) {
  if (vi < nfull) return load_vec(base, vi);
  return load_partial<C>(base, vi, ntail);
}
template <class C>
__device__ inline void store_any(void* base, uint64_t vi, const u32x4& v, uint64_t nfull, int ntail) {
  if (vi < nfull)
    store_vec(base, vi, v);
  else
    store_partial<C>(base, vi, v, ntail);
}

}  // namespace mscl
