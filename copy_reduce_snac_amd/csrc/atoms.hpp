// atoms.hpp -- gfx950 datapath primitives: the copy and N-to-1 reduce Atoms
// work on 16-byte units (one global_load/store_dwordx4 per lane), accumulate
// in binary32 in source order, and round bf16 outputs to nearest-even with
// the hardware converter (v_cvt_pk_bf16_f32).
//
// The two primitives are the ones Purlin 0.6.4 ("# Purlin") puts under every
// collective: copy, and an N-to-1 reduce that combines several input buffers
// into one output.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace snac {

constexpr int kThreads = 256;  // 4 wave64 per workgroup

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// same vector with 4-byte alignment: still one global_load_dwordx4 (the
// hardware needs only dword alignment for multi-dword accesses)
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Cache policies for collective inputs and outputs: streaming accesses carry
// the non-temporal hint (global_load/store ... nt), so single-use data does
// not displace other lines.
enum : int { kCached = 0, kCacheStream = 1, kCacheStreamStores = 2, kCacheStreamLoads = 3 };

template <int CP>
__device__ __forceinline__ u32x4 ld16(const char* p) {
  if constexpr (CP == kCacheStream || CP == kCacheStreamLoads)
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  else
    return *reinterpret_cast<const u32x4*>(p);
}

template <int CP>
__device__ __forceinline__ void st16(char* p, u32x4 v) {
  if constexpr (CP == kCacheStream || CP == kCacheStreamStores)
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
  else
    *reinterpret_cast<u32x4*>(p) = v;
}

// Buffer-resource accesses.  A raw buffer resource covers [base, base +
// bytes); the hardware returns zero for a load whose offset is at or past
// `bytes` and drops such a store.  Sizing the resource to the bytes left in
// a tile lets full and partial tiles run the same branch-free code, with a
// scalar base and 32-bit lane offsets.  Word 3 selects the 32-bit data
// format that untyped (raw) loads and stores on gfx9-family parts need.
constexpr uint32_t kRawBufferWord3 = 0x00020000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, (int)kRawBufferWord3);
}

// cache-policy bits of a buffer access: 2 = nt (streaming)
template <int CP>
constexpr int load_aux() {
  return (CP == kCacheStream || CP == kCacheStreamLoads) ? 2 : 0;
}
template <int CP>
constexpr int store_aux() {
  return (CP == kCacheStream || CP == kCacheStreamStores) ? 2 : 0;
}

template <int CP>
__device__ __forceinline__ u32x4 bld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, load_aux<CP>());
}

template <int CP>
__device__ __forceinline__ void bst16(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, store_aux<CP>());
}

// 16 bytes from any address.  m = p & 3 must be uniform across the wave.
// m == 0: one dword-aligned dwordx4.  Otherwise the 20 bytes starting at the
// dword below p are loaded (every dword touched holds at least one wanted
// byte, so nothing outside the source range's dwords is read) and shifted
// into place with v_alignbyte_b32.
template <int CP>
__device__ __forceinline__ u32x4 ld16_a4(const char* p) {
  if constexpr (CP == kCacheStream || CP == kCacheStreamLoads)
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4_a4*>(p));
  else
    return *reinterpret_cast<const u32x4_a4*>(p);
}

template <int CP>
__device__ __forceinline__ u32x4 ld16_any(const char* p, uint32_t m) {
  if (m == 0) return ld16_a4<CP>(p);
  const char* b = p - m;
  const u32x4 a = ld16_a4<CP>(b);
  const uint32_t e = *reinterpret_cast<const uint32_t*>(b + 16);
  u32x4 r;
  r.x = __builtin_amdgcn_alignbyte(a.y, a.x, m);
  r.y = __builtin_amdgcn_alignbyte(a.z, a.y, m);
  r.z = __builtin_amdgcn_alignbyte(a.w, a.z, m);
  r.w = __builtin_amdgcn_alignbyte(e, a.w, m);
  return r;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two binary32 values -> two bf16 (round to nearest even), lo in bits 0..15.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

__device__ __forceinline__ uint16_t to_bf16(float x) { return (uint16_t)(pack_bf16(x, 0.0f) & 0xffffu); }

struct F32 {
  static constexpr int kSize = 4;
};
struct BF16 {
  static constexpr int kSize = 2;
};

// One 16-byte unit of the N-to-1 reduce: out = R(v[0] + v[1] + ... + v[N-1])
// per element, added in index order starting from v[0].
template <typename T, int N>
__device__ __forceinline__ u32x4 reduce_unit(const u32x4 (&v)[N]) {
  u32x4 out;
  if constexpr (T::kSize == 4) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float acc = __uint_as_float(v[0][c]);
#pragma unroll
      for (int k = 1; k < N; ++k) acc = acc + __uint_as_float(v[k][c]);
      out[c] = __float_as_uint(acc);
    }
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float lo = bf16_lo(v[0][c]);
      float hi = bf16_hi(v[0][c]);
#pragma unroll
      for (int k = 1; k < N; ++k) {
        lo = lo + bf16_lo(v[k][c]);
        hi = hi + bf16_hi(v[k][c]);
      }
      out[c] = pack_bf16(lo, hi);
    }
  }
  return out;
}

// Binary32 accumulator of one 16-byte unit: 4 lanes for F32, 8 for BF16
// (lane 2c is the low half of word c, lane 2c + 1 its high half).  Sources
// are added one at a time, so a reduce holds one accumulator per unit
// instead of all N source values.
template <typename T>
struct UnitAcc {
  static constexpr int kLanes = 16 / T::kSize;
  float a[kLanes];

  __device__ __forceinline__ void set(const u32x4& w) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if constexpr (T::kSize == 4) {
        a[c] = __uint_as_float(w[c]);
      } else {
        a[2 * c] = bf16_lo(w[c]);
        a[2 * c + 1] = bf16_hi(w[c]);
      }
    }
  }
  __device__ __forceinline__ void add(const u32x4& w) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if constexpr (T::kSize == 4) {
        a[c] = a[c] + __uint_as_float(w[c]);
      } else {
        a[2 * c] = a[2 * c] + bf16_lo(w[c]);
        a[2 * c + 1] = a[2 * c + 1] + bf16_hi(w[c]);
      }
    }
  }
  __device__ __forceinline__ u32x4 out() const {
    u32x4 r;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if constexpr (T::kSize == 4)
        r[c] = __float_as_uint(a[c]);
      else
        r[c] = pack_bf16(a[2 * c], a[2 * c + 1]);
    }
    return r;
  }
};

template <typename T>
__device__ __forceinline__ float load_elem(const char* p) {
  if constexpr (T::kSize == 4)
    return *reinterpret_cast<const float*>(p);
  else
    return __uint_as_float((uint32_t)(*reinterpret_cast<const uint16_t*>(p)) << 16);
}

template <typename T>
__device__ __forceinline__ void store_elem(char* p, float v) {
  if constexpr (T::kSize == 4)
    *reinterpret_cast<float*>(p) = v;
  else
    *reinterpret_cast<uint16_t*>(p) = to_bf16(v);
}

// Force a wave-uniform value into a scalar register.
__device__ __forceinline__ uint32_t uniform(uint32_t x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ uint64_t uniform64(uint64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  return ((uint64_t)hi << 32) | lo;
}

}  // namespace snac
