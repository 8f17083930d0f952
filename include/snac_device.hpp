// snac_device.hpp -- the device-side API: the copy and N-to-1 reduce Atoms,
// the Stage / Notify / And Consume flag primitives and the single-kernel
// collectives, callable from inside any HIP kernel for gfx950 (MI355X).
//
// Purlin 0.6.5 ("Device-side", "Samples") lets a kernel call an Atom or a
// whole collective between pieces of its own work, with the collective's
// arguments and a context passed in by value.  This header is that layer
// for one MI355X whose N logical ranks all live in its HBM:
//
//   snac::copy(dst, src, bytes)                workgroup-cooperative copy of
//                                              one slice, any alignment
//   snac::reduce<T, N>(dst, ndst, src, count)  workgroup-cooperative N-to-1
//                                              reduce of one slice
//   snac::wait_geq / snac::notify              SNAC flag primitives (bounded
//                                              acquire polls, release stores)
//   snac::stage(staging, src, bytes)           copy a slice into a staging
//                                              buffer with write-through
//                                              stores (then notify())
//   snac::group_barrier(ctx, blocks)           all `blocks` workgroups meet;
//                                              stores before it are visible
//                                              to every one of them after it
//   snac::collective<T, N, TH>(args, ctx)      any of the seven collectives
//                                              of a snac_coll_desc, run by
//                                              the calling workgroups
//                                              (snac_args: descriptor, LDS
//                                              workspace, blocks,
//                                              coll_blocks, block)
//   snac::Atom<950>                            the launch contract: THREADS
//                                              and the LDS bytes each call
//                                              needs (PIPELINE_LDS_BYTES)
//
// The library's own collective kernels are thin wrappers over the same
// tile engine (run_reduce / run_copy), so host and device calls move data
// with identical code and give identical bits.
//
// Arithmetic: binary32 accumulation in source order 0..N-1 starting from the
// source-0 value, one rounding to the output type (bf16: round to nearest
// even with v_cvt_pk_bf16_f32).  Translation units including this header
// should be built with -ffp-contract=off so that no add is fused.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "snac.h"
#include "snac_layout.hpp"

namespace snac {

// ======================================================== gfx950 primitives

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// same vector with 4-byte alignment: still one global_load_dwordx4 (the
// hardware needs only dword alignment for multi-dword accesses)
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Cache policies for collective inputs and outputs: streaming accesses carry
// the non-temporal hint, so single-use data does not displace other lines.
// kWriteThrough (buffer accesses only): stores carry sc0 sc1, so the L2
// writes them through and a later release fence finds nothing of them left
// to write back; loads stream.  SNAC staging uses it: on MI355X it made the
// 4096x8192 pipeline 10 % faster than write-back staging stores.
enum : int { kCached = 0, kCacheStream = 1, kCacheStreamStores = 2, kCacheStreamLoads = 3, kWriteThrough = 5 };

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

// cache-policy bits of a buffer access: 1 = sc0, 2 = nt (streaming),
// 16 = sc1
template <int CP>
constexpr int load_aux() {
  return (CP == kCacheStream || CP == kCacheStreamLoads || CP == kWriteThrough) ? 2 : 0;
}
template <int CP>
constexpr int store_aux() {
  return CP == kWriteThrough ? (1 | 16) : ((CP == kCacheStream || CP == kCacheStreamStores) ? 2 : 0);
}

template <int CP>
__device__ __forceinline__ u32x4 bld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, load_aux<CP>());
}

template <int CP>
__device__ __forceinline__ void bst16(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, store_aux<CP>());
}

template <int CP>
__device__ __forceinline__ u32x4 ld16_a4(const char* p) {
  if constexpr (CP == kCacheStream || CP == kCacheStreamLoads)
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4_a4*>(p));
  else
    return *reinterpret_cast<const u32x4_a4*>(p);
}

template <int CP>
__device__ __forceinline__ uint32_t ld4(const char* p) {
  if constexpr (CP == kCacheStream || CP == kCacheStreamLoads)
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
  else
    return *reinterpret_cast<const uint32_t*>(p);
}

// 16 bytes from any address p, in two steps, for m = p & 3 (uniform across
// the wave) not 0: ld20 loads the 20 bytes starting at the dword below p
// (every dword touched holds at least one wanted byte, so nothing outside
// the source range's dwords is read), shift16 moves them into place with
// v_alignbyte_b32.  Callers test m once per tile (m == 0: one dword-aligned
// dwordx4 per unit, ld16_a4) and issue every unit's loads before the first
// shift: with the test and the shift inside each unit's load, each unit
// became its own block and the compiler waited for its loads before issuing
// the next unit's, which made a 1 GiB copy from a source one byte off its
// destination's alignment 2.3x slower on MI355X.  The extra dword takes the
// same cache policy as the dwordx4: it is the next lane's first dword, and
// a plain load behind a streaming one fetched those lines again.
// (m == 0 is allowed: the extra dword is then the unit's own last one, so
// nothing past the unit is read, and shift16 by 0 returns the dwordx4.)
template <int CP>
__device__ __forceinline__ void ld20(const char* p, uint32_t m, u32x4& a, uint32_t& e) {
  const char* b = p - m;
  a = ld16_a4<CP>(b);
  e = ld4<CP>(b + (m ? 16u : 12u));
}

// Lane i gets lane i + 1's v (DPP whole-wave shift left, wave_shl:1); lane
// 63, which has no next lane, keeps `old`.
__device__ __forceinline__ uint32_t from_next_lane(uint32_t v, uint32_t old) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, 0x130, 0xf, 0xf, false);
}

// Byte-misaligned units whose lanes cover consecutive 16 bytes of a full
// tile (every lane active): v[u] holds the aligned 16 bytes at c = p - m16
// (m16 = 4 Q + s, s != 0), e[u] in lane 63 of each wave the 16 bytes at
// c + 4 (Q + 1), which end at the last dword of the next 16 it needs (the
// other lanes get those dwords from their next lane).  On return v[u] holds
// the 16 bytes at p.
template <int Q, int U>
__device__ __forceinline__ void funnel_next(u32x4 (&v)[U], const u32x4 (&e)[U], uint32_t s) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    uint32_t n[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) n[i] = from_next_lane(v[u][i], i <= Q ? e[u][(i + 3 - Q) & 3] : 0u);
    const uint32_t w[8] = {v[u].x, v[u].y, v[u].z, v[u].w, n[0], n[1], n[2], n[3]};
    u32x4 r;
#pragma unroll
    for (int k = 0; k < 4; ++k) r[k] = __builtin_amdgcn_alignbyte(w[Q + k + 1], w[Q + k], s);
    v[u] = r;
  }
}

__device__ __forceinline__ u32x4 shift16(u32x4 a, uint32_t e, uint32_t m) {
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

// Element types of the reduce: tags carrying the storage size.
struct F32 {
  static constexpr int kSize = 4;
};
struct BF16 {
  static constexpr int kSize = 2;
};

// One 16-byte unit of the N-to-1 reduce from all N source values at once:
// out = R(v[0] + v[1] + ... + v[N-1]) per element, added in index order.
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

// ================================================= workgroup-level Atoms
//
// Every thread of the calling workgroup calls these with the same arguments
// (blockDim.x threads, a multiple of 64).  They move one slice; splitting a
// buffer into slices across workgroups is the caller's business, as in the
// copy sample of Purlin 0.6.5.

// dst[0..bytes) = src[0..bytes), bytewise, any alignment; the ranges must
// not overlap.  The destination is stored in aligned 16-byte units after a
// head of at most 15 bytes; the source is read with ld16_a4, or ld20 and
// shift16 when it is not dword-aligned there.
template <int CP = kCacheStream>
__device__ void copy(void* dst, const void* src, uint64_t bytes) {
  char* d = static_cast<char*>(dst);
  const char* s = static_cast<const char*>(src);
  const uint32_t nt = blockDim.x;
  uint64_t head = (16u - ((uintptr_t)d & 15u)) & 15u;
  if (head > bytes) head = bytes;
  const uint64_t body = (bytes - head) & ~(uint64_t)15;
  const char* sb = s + head;
  char* db = d + head;
  const uint32_t m = (uint32_t)((uintptr_t)sb & 3u);
  constexpr int U = 4;
  const uint64_t step = (uint64_t)nt * 16u * U;
  for (uint64_t base = 0; base < body; base += step) {
    u32x4 v[U];
    uint32_t e[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      v[u] = u32x4{0u, 0u, 0u, 0u};
      e[u] = 0u;
    }
    if (m == 0) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint64_t o = base + ((uint64_t)threadIdx.x + (uint64_t)u * nt) * 16u;
        if (o < body) v[u] = ld16_a4<CP>(sb + o);
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint64_t o = base + ((uint64_t)threadIdx.x + (uint64_t)u * nt) * 16u;
        if (o < body) ld20<CP>(sb + o, m, v[u], e[u]);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = shift16(v[u], e[u], m);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint64_t o = base + ((uint64_t)threadIdx.x + (uint64_t)u * nt) * 16u;
      if (o < body) st16<CP>(db + o, v[u]);
    }
  }
  const uint64_t tail = bytes - head - body;
  for (uint64_t i = threadIdx.x; i < head + tail; i += nt) {
    const uint64_t o = i < head ? i : head + body + (i - head);
    d[o] = s[o];
  }
}

// for d < ndst, i < count: dst[d][i] = R(src[0][i] + ... + src[N-1][i]),
// binary32 in source order, R the rounding to T.  Every pointer must be
// aligned to the element size; a destination may equal a source (in place),
// no other overlap.  Destinations must share their address residue modulo
// 16 (they are stored in aligned 16-byte units after a common head).
template <typename T, int N, int CP = kCacheStream>
__device__ void reduce(void* const* dst, int ndst, const void* const* src, uint64_t count) {
  constexpr uint32_t E = T::kSize;
  const uint32_t nt = blockDim.x;
  const uint64_t bytes = count * E;
  uint64_t head = (16u - ((uintptr_t)dst[0] & 15u)) & 15u;
  if (head > bytes) head = bytes;
  const uint64_t body = (bytes - head) & ~(uint64_t)15;
  uint32_t m[N];
  uint32_t any = 0;
#pragma unroll
  for (int k = 0; k < N; ++k) {
    m[k] = (uint32_t)(((uintptr_t)src[k] + head) & 3u);
    any |= m[k];
  }
  // one test per call, not per source and unit (see ld20): dword-aligned
  // sources take one dwordx4 each; otherwise every source takes ld20, whose
  // shift by m[k] = 0 leaves the dwordx4 as it is
  for (uint64_t o = (uint64_t)threadIdx.x * 16u; o < body; o += (uint64_t)nt * 16u) {
    u32x4 v[N];
    if (any == 0) {
#pragma unroll
      for (int k = 0; k < N; ++k) v[k] = ld16_a4<CP>(static_cast<const char*>(src[k]) + head + o);
    } else {
      uint32_t e[N];
#pragma unroll
      for (int k = 0; k < N; ++k) ld20<CP>(static_cast<const char*>(src[k]) + head + o, m[k], v[k], e[k]);
#pragma unroll
      for (int k = 0; k < N; ++k) v[k] = shift16(v[k], e[k], m[k]);
    }
    UnitAcc<T> acc;
    acc.set(v[0]);
#pragma unroll
    for (int k = 1; k < N; ++k) acc.add(v[k]);
    const u32x4 r = acc.out();
    for (int d = 0; d < ndst; ++d) st16<CP>(static_cast<char*>(dst[d]) + head + o, r);
  }
  const uint64_t ne = (head + (bytes - head - body)) / E;
  for (uint64_t i = threadIdx.x; i < ne; i += nt) {
    const uint64_t o = i * E < head ? i * E : body + i * E;
    float acc = load_elem<T>(static_cast<const char*>(src[0]) + o);
#pragma unroll
    for (int k = 1; k < N; ++k) acc = acc + load_elem<T>(static_cast<const char*>(src[k]) + o);
    for (int d = 0; d < ndst; ++d) store_elem<T>(static_cast<char*>(dst[d]) + o, acc);
  }
}

// ============================================= SNAC signal primitives
//
// Flags are uint64 words, one per 128-byte line (SNAC_FLAG_STRIDE words
// apart), carrying monotonic sequence numbers: a producer stores seq, a
// consumer waits for flag >= seq.  Ordering follows the HIP agent-scope
// memory model: release = write the L2 back (buffer_wbl2) then store,
// acquire = relaxed polls then invalidate (buffer_inv).  Each is issued by
// one lane for the whole workgroup, because on MI355X these fences
// serialise across the GPU.

enum : uint64_t { kStatusTimeout = SNAC_E_TIMEOUT, kStatusAborted = SNAC_E_ABORTED };

__device__ __forceinline__ uint64_t ld_relaxed(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void st_relaxed(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Latch the first device error in a status word (later codes are dropped).
__device__ __forceinline__ void latch_status(uint64_t* status, uint64_t code) {
  uint64_t expected = 0;
  __hip_atomic_compare_exchange_strong(status, &expected, code, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until every vector memory operation this wave has issued is done
// (s_waitcnt vmcnt(0); the gfx9 encoding leaves expcnt and lgkmcnt free).
// A store is done once the L2 has accepted it.
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// What a bounded wait needs to know: where errors latch, the host-mapped
// abort word, and the poll budget.
struct WaitCtl {
  uint64_t* status;
  const uint32_t* abort_word;
  uint32_t spin_limit_log2;
};

__device__ __forceinline__ WaitCtl wait_ctl(const snac_dev_ctx& c) {
  return WaitCtl{c.status, c.abort_word, c.spin_limit_log2};
}

// One lane waits until *flag >= target with relaxed agent-scope loads: 16
// polls 64 clocks apart (each poll is a memory round trip, so this covers
// the first several microseconds, where small messages finish), then
// exponential s_sleep back-off to 512 clocks between polls (with hundreds of
// workgroups waiting, tight polling took enough of the memory system to
// slow the producers they waited for -- up to 3x on MI355X).
// Returns false, with the status word set, after 2^spin_limit_log2 polls
// (SNAC_E_TIMEOUT), when the abort word is set (SNAC_E_ABORTED), or at once
// when an error is already latched -- so every wait ends.  The caller adds
// the acquire fence where it needs one.
__device__ inline bool wait_geq(const uint64_t* flag, uint64_t target, const WaitCtl& w) {
  const uint64_t limit = 1ull << w.spin_limit_log2;
  uint64_t spins = 0;
  uint32_t naps = 1;  // s_sleep(1) rounds between polls
  while (ld_relaxed(flag) < target) {
    if ((spins & 15u) == 15u) {
      if (ld_relaxed(w.status) != 0) return false;
      uint32_t* ab = const_cast<uint32_t*>(w.abort_word);
      if (ab && __hip_atomic_load(ab, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) != 0) {
        latch_status(w.status, kStatusAborted);
        return false;
      }
    }
    if (++spins >= limit) {
      latch_status(w.status, kStatusTimeout);
      return false;
    }
    for (uint32_t i = 0; i < naps; ++i) __builtin_amdgcn_s_sleep(1);
    if (spins >= 16 && naps < 8) naps <<= 1;
  }
  return true;
}

// Wave-level wait: the calling wave (all 64 lanes active, and no other wave
// of the workgroup in it) waits until flags[i * stride] >= target for every
// i < n, lane i polling flag i (flags 64 and up in further groups of 64), so
// a poll costs one memory round trip however many flags there are.  One
// lane polling n flags in turn paid n round trips (about 1 us each on
// MI355X) even when every flag was already set.  Back-off, bounds and
// errors as in wait_geq; the result is the same in every lane.
__device__ inline bool wait_group_geq(const uint64_t* flags, int n, uint64_t stride, uint64_t target,
                                      const WaitCtl& w);

__device__ inline bool wait_all_geq(const uint64_t* flags, int n, uint64_t stride, uint64_t target, const WaitCtl& w) {
  for (int base = 0; base < n; base += 64)
    if (!wait_group_geq(flags + (uint64_t)base * stride, n - base < 64 ? n - base : 64, stride, target, w)) return false;
  return true;
}

// One group of at most 64 flags (wait_all_geq).
__device__ inline bool wait_group_geq(const uint64_t* flags, int n, uint64_t stride, uint64_t target,
                                      const WaitCtl& w) {
  const uint32_t lane = threadIdx.x & 63u;
  const bool mine = (int)lane < n;
  const uint64_t* f = flags + (uint64_t)(mine ? lane : 0u) * stride;
  const uint64_t limit = 1ull << w.spin_limit_log2;
  uint64_t spins = 0;
  uint32_t naps = 1;
  for (;;) {
    const bool ok = !mine || ld_relaxed(f) >= target;
    if (__builtin_amdgcn_ballot_w64(!ok) == 0) return true;
    if ((spins & 15u) == 15u) {
      if (uniform64(ld_relaxed(w.status)) != 0) return false;
      uint32_t* ab = const_cast<uint32_t*>(w.abort_word);
      if (ab && uniform(__hip_atomic_load(ab, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM)) != 0) {
        if (lane == 0) latch_status(w.status, kStatusAborted);
        return false;
      }
    }
    if (++spins >= limit) {
      if (lane == 0) latch_status(w.status, kStatusTimeout);
      return false;
    }
    for (uint32_t i = 0; i < naps; ++i) __builtin_amdgcn_s_sleep(1);
    if (spins >= 16 && naps < 8) naps <<= 1;
  }
}

// Notify (workgroup-level; every thread calls it): once every wave's stores
// are accepted by the L2, one lane writes the L2 back at agent scope and
// stores *flag = value.  After a consumer's acquire sees the value, every
// store this workgroup made before notify() is visible to it.
__device__ inline void notify(uint64_t* flag, uint64_t value) {
  wait_vm();
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    wait_vm();
    st_relaxed(flag, value);
  }
}

// Stage (workgroup-level; every thread calls it): copy `bytes` from src (any
// alignment) into a staging buffer for a consumer, as the producers of
// snac_pipeline_scale_reduce do.  The 16-byte units of the staging side are
// stored with sc0 sc1, writing through the L2, so that the release fence of
// the notify() that follows finds little left to write back (on MI355X
// write-through staging made the library's pipeline 10 % faster than
// write-back stores); the source is read with streaming loads.  `staging`
// should be 16-byte aligned: otherwise the slice is moved by copy(), which
// is correct but leaves the write-back to the fence.  The last bytes % 16
// bytes go one per lane.  Nothing is visible to other workgroups until
// notify().
template <int LCP = kCacheStreamLoads>
__device__ void stage(void* staging, const void* src, uint64_t bytes) {
  char* d = static_cast<char*>(staging);
  const char* s = static_cast<const char*>(src);
  if ((uintptr_t)d & 15u) {
    copy<kCacheStream>(staging, src, bytes);
    return;
  }
  const uint32_t nt = blockDim.x;
  const uint64_t body = bytes & ~(uint64_t)15;
  const uint32_t m = uniform((uint32_t)((uintptr_t)s & 3u));
  constexpr int U = 4;
  const uint64_t step = (uint64_t)nt * 16u * U;
  for (uint64_t base = 0; base < body; base += step) {
    const uint64_t left = body - base;
    const uint32_t rem = left < step ? (uint32_t)left : (uint32_t)step;
    u32x4 v[U];
    uint32_t e[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      v[u] = u32x4{0u, 0u, 0u, 0u};
      e[u] = 0u;
    }
    // one test per call (see ld20): the whole body under one load form
    if (m == 0) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t o = (threadIdx.x + (uint32_t)u * nt) * 16u;
        if (o < rem) v[u] = ld16_a4<LCP>(s + base + o);
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t o = (threadIdx.x + (uint32_t)u * nt) * 16u;
        if (o < rem) ld20<LCP>(s + base + o, m, v[u], e[u]);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = shift16(v[u], e[u], m);
    }
    // units at or past rem fall outside the resource: the hardware drops them
    const __amdgpu_buffer_rsrc_t r = buffer_rsrc(d + base, rem);
#pragma unroll
    for (int u = 0; u < U; ++u) bst16<kWriteThrough>(r, (threadIdx.x + (uint32_t)u * nt) * 16u, v[u]);
  }
  for (uint64_t i = threadIdx.x; i < bytes - body; i += nt) d[body + i] = s[body + i];
}

// Consume (workgroup-level): the first wave waits for flags[i * stride] >=
// target for i < n (one lane per flag, in groups of 64), then issues one
// acquire fence; the workgroup meets at a barrier.  Returns false on
// timeout or abort (the same in every thread).
__device__ inline bool consume(const uint64_t* flags, int n, uint64_t stride, uint64_t target, const WaitCtl& w) {
  __shared__ uint32_t s_ok;
  if (threadIdx.x < 64) {
    const bool ok = wait_all_geq(flags, n, stride, target, w);
    if (ok) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      wait_vm();
    }
    if (threadIdx.x == 0) s_ok = ok ? 1u : 0u;
  }
  __syncthreads();
  const uint32_t ok = uniform(s_ok);
  __syncthreads();
  return ok != 0;
}

// All `blocks` calling workgroups meet (a grid barrier over a subset of the
// grid).  Stores made before it by any of them are visible to all of them
// after it.  The workgroups must be co-resident (at most what the device
// runs at once for this kernel), and only one group may use a context's
// barrier at a time.  Returns false on timeout or abort.
//
// Words: barrier[0] counts arrivals, barrier[SNAC_FLAG_STRIDE] is the
// generation.  A workgroup reads the generation, releases its stores (one
// fence) and counts itself in with a relaxed add.  The last arrival acquires
// every other arrival's stores (their fences head the release sequence of
// the count), resets the count and advances the generation with a release
// store; the others wait for it and acquire.  So a workgroup pays two
// agent-scope fences, which serialise GPU-wide, and the last one four; an
// acquire-release add cost every workgroup two more.
// `s_ok` is one LDS word of the workgroup that carries the verdict to
// every wave; the overloads without it keep that word in static LDS.
__device__ inline bool group_barrier(uint64_t* barrier, uint32_t blocks, const WaitCtl& w, uint32_t* s_ok_word) {
  uint32_t& s_ok = *s_ok_word;
  wait_vm();
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t* count = barrier;
    uint64_t* gen = barrier + SNAC_FLAG_STRIDE;
    const uint64_t g = ld_relaxed(gen);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const uint64_t old = __hip_atomic_fetch_add(count, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bool ok = true;
    if (old + 1 == blocks) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      st_relaxed(count, 0);
      __hip_atomic_store(gen, g + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      ok = wait_geq(gen, g + 1, w);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    s_ok = ok ? 1u : 0u;
  }
  __syncthreads();
  const uint32_t ok = uniform(s_ok);
  __syncthreads();
  return ok != 0;
}

__device__ inline bool group_barrier(uint64_t* barrier, uint32_t blocks, const WaitCtl& w) {
  __shared__ uint32_t s_ok;
  return group_barrier(barrier, blocks, w, &s_ok);
}

__device__ inline bool group_barrier(const snac_dev_ctx& c, uint32_t blocks) {
  return group_barrier(c.barrier, blocks, wait_ctl(c));
}

__device__ inline bool group_barrier(const snac_dev_ctx& c, uint32_t blocks, uint32_t* s_ok_word) {
  return group_barrier(c.barrier, blocks, wait_ctl(c), s_ok_word);
}

// ======================================================== the tile engine
//
// A collective's jobs (snac_layout.hpp) are cut into tiles of kTileBytes of
// each source.  Every workgroup rebuilds the job table in LDS from the
// descriptor, numbers the tiles of all jobs with an exclusive scan, and
// walks tiles block, block + blocks, ...  A lane moves U = kTileBytes /
// (TH * 16) 16-byte units per tile.  A job whose destination does not start
// on the 16 KiB grid first gets a short tile up to it (job_lead), so that
// every later tile fills one aligned block of the destination.
//
//  * copy: the U loads of a tile, then its stores to one destination or to
//    all of them (a multicast: one read, N writes).
//  * reduce: the sources are taken one at a time -- source k + 1's loads are
//    in flight while source k is added into binary32 accumulators -- and
//    the finished tile goes to each destination as one contiguous run.
//    Accumulators rather than all N sources keep the register footprint
//    independent of N, and a workgroup writes one destination at a time; on
//    MI355X this beat loading all N sources at once and storing every
//    destination per unit by 3-6 %.
//
// Two variants of each:
//  * aligned (SNAC_DESC_ALIGNED): every job address 16-byte aligned and every
//    job length a multiple of 16 -- raw buffer loads and stores whose
//    resource is sized to the tile, so partial tiles need no guards.
//  * generic: any element-aligned address.  Each job is split into a head
//    (bytes until the destination reaches a 128-byte line), a body of
//    aligned 16-byte stores (buffer stores, as above) whose sources are read
//    with ld16_a4, or ld20 and shift16 when not dword-aligned, and a tail;
//    head and tail move one element per lane in tile 0 of the job.

constexpr uint32_t kTileBytes = 16384;

template <int TH, uint32_t TILE = kTileBytes>
constexpr int tile_units() {
  static_assert(TH % 64 == 0 && TH >= 64 && TH <= 1024, "workgroup size must be a multiple of 64, at most 1024");
  static_assert(TILE % (TH * 16u) == 0 && TILE >= TH * 16u, "a tile is a whole number of units per lane");
  return (int)(TILE / (TH * 16u));
}

struct JobL {
  uint64_t src_off;
  uint64_t dst_off;
  uint64_t bytes;
  int32_t src_rank;
  int32_t dst_rank;
  uint32_t head;
  uint32_t tile0;
  uint32_t lead;  // body bytes before the destination's tile grid (job_lead)
};

// LDS the tile engine needs in a workgroup of TH threads: the job table
// (MAXJ entries), the tile-count scan (one word per thread) and one word for
// the verdict of collective()'s closing barrier, rounded up to 128 bytes.
// The engine keeps nothing else in LDS.
template <int TH, int MAXJ = kMaxJobs>
constexpr uint32_t engine_lds_bytes() {
  return ((uint32_t)(MAXJ * sizeof(JobL) + (uint32_t)TH * 4u + 16u) + 127u) & ~127u;
}

// Where the engine's words sit in its workspace.
template <int TH, int MAXJ>
struct EngineLds {
  JobL* jobs;
  uint32_t* scan;
  uint32_t* verdict;
  __device__ __forceinline__ explicit EngineLds(void* lds)
      : jobs(static_cast<JobL*>(lds)),
        scan(reinterpret_cast<uint32_t*>(static_cast<char*>(lds) + MAXJ * sizeof(JobL))),
        verdict(reinterpret_cast<uint32_t*>(static_cast<char*>(lds) + MAXJ * sizeof(JobL) + (uint32_t)TH * 4u)) {}
};

// Build the job table and its tile numbering in LDS.  Returns the total
// number of tiles; every thread of the workgroup must call it.  Thread t
// owns jobs t*K .. t*K + K - 1 (K = ceil(MAXJ / TH)).
template <int TH, int MAXJ, bool ALIGNED>
__device__ uint32_t build_table(const CollDesc& d, uint32_t tile_bytes, JobL* jobs, uint32_t* scan, int& nj) {
  constexpr int K = (MAXJ + TH - 1) / TH;
  nj = num_jobs(d);
  const int t = threadIdx.x;
  if (nj <= 64) {
    // one wave: lane j owns job j; an inclusive scan over the wave with
    // shuffles, then a single barrier (no LDS scan rounds)
    if (t < 64) {
      uint32_t mine = 0;
      if (t < nj) {
        const Job jb = make_job(d, t);
        const uint32_t head = ALIGNED ? 0u : job_head_bytes(d, jb);
        const uint64_t body = (jb.bytes - head) & ~(uint64_t)15;
        const uint32_t lead = (uint32_t)job_lead(d, jb, head, body, tile_bytes);
        mine = (uint32_t)job_tiles(jb, head, lead, tile_bytes);
        jobs[t] = JobL{jb.src_off, jb.dst_off, jb.bytes, jb.src_rank, jb.dst_rank, head, 0u, lead};
      }
      uint32_t incl = mine;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t v = __shfl_up(incl, off, 64);
        if (t >= off) incl += v;
      }
      if (t < nj) jobs[t].tile0 = incl - mine;
      if (t == 63) scan[0] = incl;
    }
    __syncthreads();
    const uint32_t total = scan[0];
    __syncthreads();  // scan[0] may be reused by the next table build
    return total;
  }
  uint32_t mine[K];
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < K; ++i) {
    const int j = t * K + i;
    mine[i] = 0;
    if (j < nj) {
      const Job jb = make_job(d, j);
      const uint32_t head = ALIGNED ? 0u : job_head_bytes(d, jb);
      const uint64_t body = (jb.bytes - head) & ~(uint64_t)15;
      const uint32_t lead = (uint32_t)job_lead(d, jb, head, body, tile_bytes);
      mine[i] = (uint32_t)job_tiles(jb, head, lead, tile_bytes);
      jobs[j] = JobL{jb.src_off, jb.dst_off, jb.bytes, jb.src_rank, jb.dst_rank, head, 0u, lead};
    }
    sum += mine[i];
  }
  scan[t] = sum;
  __syncthreads();
#pragma unroll
  for (int off = 1; off < TH; off <<= 1) {
    const uint32_t v = t >= off ? scan[t - off] : 0u;
    __syncthreads();
    scan[t] += v;
    __syncthreads();
  }
  uint32_t run = scan[t] - sum;
#pragma unroll
  for (int i = 0; i < K; ++i) {
    const int j = t * K + i;
    if (j < nj) jobs[j].tile0 = run;
    run += mine[i];
  }
  const uint32_t total = scan[TH - 1];
  __syncthreads();
  return total;
}

// Store U units (unit u at lane + u * TH * 16 bytes past base, if below
// rem) to one destination or, for a multicast, to every destination in
// turn.  NU > 0 unrolls the multicast for the common case ndst == NU.
template <int TH, int U, int CP, bool ALIGNED>
__device__ __forceinline__ void store_one(char* p, uint32_t lane, uint32_t rem, const u32x4 (&v)[U]) {
  // Buffer stores whenever the destination is 16-byte aligned: always on
  // the aligned path, and on the generic path for body tiles, whose
  // destination the job head has brought to a 128-byte line (the other
  // destinations of a multicast reduce may sit elsewhere).  Units at or
  // past rem fall outside the resource.  On MI355X the buffer form made
  // single-wave multicast copies about 8 % faster than 64-bit global stores.
  if (ALIGNED || ((uint32_t)(uintptr_t)p & 15u) == 0) {
    const __amdgpu_buffer_rsrc_t r = buffer_rsrc(p, rem);
#pragma unroll
    for (int u = 0; u < U; ++u) bst16<CP>(r, lane + (uint32_t)u * TH * 16u, v[u]);
    return;
  }
  if (rem == (uint32_t)TH * 16u * U) {  // full tile: no per-unit guards
#pragma unroll
    for (int u = 0; u < U; ++u) st16<CP>(p + lane + (uint32_t)u * TH * 16u, v[u]);
    return;
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t o = lane + (uint32_t)u * TH * 16u;
    if (o < rem) st16<CP>(p + o, v[u]);
  }
}

template <int TH, int U, int CP, int NU, bool ALIGNED>
__device__ __forceinline__ void store_units(const CollDesc& d, int32_t dst_rank, uint64_t base, uint32_t lane,
                                            uint32_t rem, const u32x4 (&v)[U]) {
  if (dst_rank >= 0) {
    store_one<TH, U, CP, ALIGNED>(static_cast<char*>(d.dst[dst_rank]) + base, lane, rem, v);
    return;
  }
  if constexpr (NU > 0) {
    if (d.ndst == NU) {
#pragma unroll
      for (int k = 0; k < NU; ++k) store_one<TH, U, CP, ALIGNED>(static_cast<char*>(d.dst[k]) + base, lane, rem, v);
      return;
    }
  }
  const int nd = d.ndst;
  for (int k = 0; k < nd; ++k) store_one<TH, U, CP, ALIGNED>(static_cast<char*>(d.dst[k]) + base, lane, rem, v);
}

// A tile resolved against its job: everything the loads and stores need.
struct TileRef {
  JobL J;
  uint32_t lt;     // tile index within the job
  uint64_t toff;   // byte offset of the tile's first 16-byte unit in the job
  uint32_t rem;    // body bytes of this tile (multiple of 16; 0 for an edge-only tile)
  uint32_t head;   // job head bytes (generic path)
  uint64_t body;   // job body bytes
};

// Walks the job table in tile order.  The current job lives in scalar
// registers; LDS is read only when a tile crosses into a later job, so a
// tile of a long job costs a compare and a few scalar ops.
template <uint32_t TILE, bool ALIGNED>
struct JobCursor {
  const JobL* jobs;
  int nj;
  int j;
  uint32_t next_tile0;  // first tile of job j + 1 (or ~0)
  JobL J;

  __device__ __forceinline__ void load_job() {
    J.src_off = uniform64(jobs[j].src_off);
    J.dst_off = uniform64(jobs[j].dst_off);
    J.bytes = uniform64(jobs[j].bytes);
    J.src_rank = (int32_t)uniform((uint32_t)jobs[j].src_rank);
    J.dst_rank = (int32_t)uniform((uint32_t)jobs[j].dst_rank);
    J.head = ALIGNED ? 0u : uniform(jobs[j].head);
    J.tile0 = uniform(jobs[j].tile0);
    J.lead = TILE >= kLeadMinTile ? uniform(jobs[j].lead) : 0u;
    next_tile0 = j + 1 < nj ? uniform(jobs[j + 1].tile0) : 0xffffffffu;
  }

  // first job: binary search for the last job whose first tile is <= tile
  // (tile0 ascends; a linear walk cost up to 63 dependent LDS reads)
  __device__ __forceinline__ void init(const JobL* t, int n, uint32_t tile) {
    jobs = t;
    nj = n;
    int lo = 0, hi = nj - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (jobs[mid].tile0 <= tile)
        lo = mid;
      else
        hi = mid - 1;
    }
    j = lo;
    // zero-tile jobs share their tile0 with the next job: step past them
    while (j + 1 < nj && jobs[j + 1].tile0 <= tile) ++j;
    load_job();
  }

  __device__ __forceinline__ TileRef at(uint32_t tile) {
    if (tile >= next_tile0) {
      while (j + 1 < nj && jobs[j + 1].tile0 <= tile) ++j;
      load_job();
    }
    TileRef r;
    r.J = J;
    r.lt = tile - J.tile0;
    r.head = J.head;
    r.body = ALIGNED ? J.bytes : ((J.bytes - r.head) & ~(uint64_t)15);
    if constexpr (TILE >= kLeadMinTile) {  // job_lead is always 0 for smaller tiles
      const TileSpan sp = tile_span(r.head, J.lead, r.body, r.lt, TILE);
      r.toff = sp.off;
      r.rem = sp.bytes;
    } else {
      r.toff = (uint64_t)r.head + (uint64_t)r.lt * TILE;
      const uint64_t end = (uint64_t)r.head + r.body;
      const uint64_t left = end > r.toff ? end - r.toff : 0;
      r.rem = left > TILE ? TILE : (uint32_t)left;
    }
    return r;
  }
};

// ------------------------------------------------------------ reduce tiles

// Head and tail elements of a job (< 128 + 16 bytes), one element per lane.
template <typename T, int N>
__device__ void reduce_edges(const CollDesc& d, const JobL& J, uint32_t head, uint64_t body) {
  constexpr uint32_t E = T::kSize;
  const uint32_t nh = head / E;
  const uint32_t ne = nh + (uint32_t)(J.bytes - head - body) / E;
  for (uint32_t t = threadIdx.x; t < ne; t += blockDim.x) {
    const uint64_t off = t < nh ? (uint64_t)t * E : (uint64_t)head + body + (uint64_t)(t - nh) * E;
    float acc = load_elem<T>(static_cast<const char*>(d.src[0]) + J.src_off + off);
#pragma unroll
    for (int k = 1; k < N; ++k) acc = acc + load_elem<T>(static_cast<const char*>(d.src[k]) + J.src_off + off);
    if (J.dst_rank >= 0) {
      store_elem<T>(static_cast<char*>(d.dst[J.dst_rank]) + J.dst_off + off, acc);
    } else {
      for (int k = 0; k < d.ndst; ++k) store_elem<T>(static_cast<char*>(d.dst[k]) + J.dst_off + off, acc);
    }
  }
}

// Issue the U loads of source k of one tile.  FULL: the tile holds U whole
// units per lane; otherwise units past the tile's body are left zero (and
// are never stored).  SHIFT (generic jobs only): some source of the tile is
// not dword-aligned, so every source is read with ld20 and shift16 (a
// shift by 0 leaves a dword-aligned source as it is); without SHIFT each
// unit is one dword-aligned dwordx4.  The caller picks SHIFT once per tile
// and runs load, add and store under that one test (see ld20).
template <int TH, int U, int CP, bool ALIGNED, bool FULL, bool SHIFT = false>
__device__ __forceinline__ void reduce_load(const CollDesc& d, const TileRef& t, int k, u32x4 (&v)[U]) {
  const uint32_t lane = threadIdx.x * 16u;
  const char* sp = static_cast<const char*>(d.src[k]) + t.J.src_off + t.toff;
  if constexpr (ALIGNED) {  // units at or past rem read as zero
    const __amdgpu_buffer_rsrc_t r = buffer_rsrc(sp, t.rem);
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = bld16<CP>(r, lane + (uint32_t)u * TH * 16u);
  } else if constexpr (!SHIFT) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t o = lane + (uint32_t)u * TH * 16u;
      if constexpr (FULL) {
        v[u] = ld16_a4<CP>(sp + o);
      } else {
        v[u] = u32x4{0u, 0u, 0u, 0u};
        if (o < t.rem) v[u] = ld16_a4<CP>(sp + o);
      }
    }
  } else {
    const uint32_t m = uniform((uint32_t)(uintptr_t)sp & 3u);
    uint32_t e[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t o = lane + (uint32_t)u * TH * 16u;
      if constexpr (FULL) {
        ld20<CP>(sp + o, m, v[u], e[u]);
      } else {
        v[u] = u32x4{0u, 0u, 0u, 0u};
        e[u] = 0u;
        if (o < t.rem) ld20<CP>(sp + o, m, v[u], e[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = shift16(v[u], e[u], m);
  }
}

// Whether any source of a generic tile is not dword-aligned (uniform).
template <int N>
__device__ __forceinline__ bool tile_needs_shift(const CollDesc& d, const TileRef& t) {
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < N; ++k) m |= (uint32_t)(uintptr_t)(static_cast<const char*>(d.src[k]) + t.J.src_off + t.toff);
  return uniform(m & 3u) != 0;
}

// The reduced units of one tile as a rolling pipeline over its N * U
// loads, taken source by source (rank order) and unit by unit: U loads are
// in flight, and each unit's load is issued right after the add that frees
// its register, so the memory sees a steady stream rather than bursts.  On
// MI355X (AllReduce bf16 N=8, 256 MiB per rank, tiles handed out in order)
// U in flight took 0.694-0.698 ms, against 0.697 with U + 1, 0.710 with
// U + 2, 0.715-0.716 with 2U or 3U, 0.720 with U - 1, and 0.712-0.714 for
// two sources loaded as blocks in turn (reduce_tile below).  In the library
// (one machine, two alternations) it ran that AllReduce 1% faster in calls back
// to back and 2.3-4.3% faster in graph replays from 128 MiB per rank up;
// bf16 N=6 and f32 N=8 even, but bf16 N=4 up to 1.3% and ReduceScatter of
// 8 ranks (one destination: more reads in flight pay) 14% slower; at 16
// sources its unrolled schedule spills scalar registers.
// Hence only the bf16 AllReduce of 8 ranks takes it.  Left to itself the
// compiler issues every load of the tile first, so each load's offset
// takes a zero it cannot see, made from the sum just added (an empty
// register move): the load then cannot move above that add.
template <int N, typename T, int TH, int U, int CP, bool ALIGNED, bool FULL>
__device__ __forceinline__ void reduce_tile_rolling(const CollDesc& d, const TileRef& t, u32x4 (&r)[U]) {
  constexpr int K = N * U;
  const uint32_t lane = threadIdx.x * 16u;
  auto load = [&](int i, uint32_t z) -> u32x4 {
    const int k = i / U, u = i % U;
    const char* sp = static_cast<const char*>(d.src[k]) + t.J.src_off + t.toff;
    const uint32_t o = lane + (uint32_t)u * TH * 16u;
    if constexpr (ALIGNED) {  // units at or past rem read as zero
      return bld16<CP>(buffer_rsrc(sp, t.rem), o + z);
    } else if constexpr (FULL) {
      return ld16_a4<CP>(sp + o + z);
    } else {
      u32x4 v{0u, 0u, 0u, 0u};
      if (o < t.rem) v = ld16_a4<CP>(sp + o + z);
      return v;
    }
  };
  u32x4 ring[U];
#pragma unroll
  for (int i = 0; i < U; ++i) ring[i] = load(i, 0u);
  UnitAcc<T> acc[U];
#pragma unroll
  for (int i = 0; i < K; ++i) {
    const u32x4 v = ring[i % U];
    if (i < U)
      acc[i % U].set(v);
    else
      acc[i % U].add(v);
    if (i + U < K) {
      uint32_t z;
      asm volatile("v_mov_b32 %0, 0" : "=v"(z) : "v"(acc[i % U].a[0]));
      ring[i % U] = load(i + U, z);
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) r[u] = acc[u].out();
}

// The reduced units of one tile, sources added in rank order, for every
// tile not given the rolling pipeline.  Two register buffers alternate:
// while source k is added from one, source k + 1 loads into the other.
// The source loop is deliberately not unrolled: unrolled, the compiler
// issues every source's loads before the first add.
template <int N, typename T, int TH, int U, int CP, bool ALIGNED, bool FULL, bool SHIFT = false>
__device__ __forceinline__ void reduce_tile(const CollDesc& d, const TileRef& t, u32x4 (&r)[U]) {
  u32x4 a[U], b[U];
  UnitAcc<T> acc[U];
  reduce_load<TH, U, CP, ALIGNED, FULL, SHIFT>(d, t, 0, a);
  if constexpr (N > 1) reduce_load<TH, U, CP, ALIGNED, FULL, SHIFT>(d, t, 1, b);
#pragma unroll
  for (int u = 0; u < U; ++u) acc[u].set(a[u]);
  int k = 1;  // next source to add; it is in b
#pragma unroll 1
  for (; k + 1 < N; k += 2) {
    reduce_load<TH, U, CP, ALIGNED, FULL, SHIFT>(d, t, k + 1, a);
    __builtin_amdgcn_sched_barrier(0);  // issue these loads before waiting on b
#pragma unroll
    for (int u = 0; u < U; ++u) acc[u].add(b[u]);
    if (k + 2 < N) reduce_load<TH, U, CP, ALIGNED, FULL, SHIFT>(d, t, k + 2, b);
    __builtin_amdgcn_sched_barrier(0);  // ... and these before waiting on a
#pragma unroll
    for (int u = 0; u < U; ++u) acc[u].add(a[u]);
  }
  if (k < N) {
#pragma unroll
    for (int u = 0; u < U; ++u) acc[u].add(b[u]);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) r[u] = acc[u].out();
}

// Small tiles (one unit per lane): every source's load is issued before
// the first add, so a tile costs one memory round trip -- what matters when
// a message has fewer tiles than the GPU has CUs.
template <int N, typename T, int TH, int CP, bool ALIGNED, bool FULL, bool SHIFT = false>
__device__ __forceinline__ void reduce_tile_allin(const CollDesc& d, const TileRef& t, u32x4 (&r)[1]) {
  u32x4 v[N][1];
#pragma unroll
  for (int k = 0; k < N; ++k) reduce_load<TH, 1, CP, ALIGNED, FULL, SHIFT>(d, t, k, v[k]);
  UnitAcc<T> acc;
  acc.set(v[0][0]);
#pragma unroll
  for (int k = 1; k < N; ++k) acc.add(v[k][0]);
  r[0] = acc.out();
}

// -------------------------------------------------------------- copy tiles

__device__ inline void copy_edges(const CollDesc& d, const JobL& J, uint32_t head, uint64_t body) {
  const uint32_t ne = head + (uint32_t)(J.bytes - head - body);
  for (uint32_t t = threadIdx.x; t < ne; t += blockDim.x) {
    const uint64_t off = t < head ? (uint64_t)t : (uint64_t)head + body + (t - head);
    const uint8_t b = *(static_cast<const uint8_t*>(d.src[J.src_rank]) + J.src_off + off);
    if (J.dst_rank >= 0) {
      *(static_cast<uint8_t*>(d.dst[J.dst_rank]) + J.dst_off + off) = b;
    } else {
      for (int k = 0; k < d.ndst; ++k) *(static_cast<uint8_t*>(d.dst[k]) + J.dst_off + off) = b;
    }
  }
}

// The U loads of one copy tile; FULL and SHIFT as for reduce_load.
template <int TH, int U, int CP, bool ALIGNED, bool FULL = false, bool SHIFT = false>
__device__ __forceinline__ void copy_load(const CollDesc& d, const TileRef& t, u32x4 (&v)[U]) {
  const char* sp = static_cast<const char*>(d.src[t.J.src_rank]) + t.J.src_off + t.toff;
  const uint32_t lane = threadIdx.x * 16u;
  if constexpr (ALIGNED) {  // units at or past rem read as zero (never stored)
    const __amdgpu_buffer_rsrc_t r = buffer_rsrc(sp, t.rem);
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = bld16<CP>(r, lane + (uint32_t)u * TH * 16u);
  } else if constexpr (!SHIFT) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t o = lane + (uint32_t)u * TH * 16u;
      if constexpr (FULL) {
        v[u] = ld16_a4<CP>(sp + o);
      } else {
        v[u] = u32x4{0u, 0u, 0u, 0u};
        if (o < t.rem) v[u] = ld16_a4<CP>(sp + o);
      }
    }
  } else if constexpr (FULL && TH >= 256) {
    // aligned loads; each lane takes the next lane's first words through a
    // DPP shift, and lane 63 of each wave loads its own (see funnel_next)
    const uint32_t m16 = uniform((uint32_t)(uintptr_t)sp & 15u);
    const uint32_t q = m16 >> 2, s = m16 & 3u;
    const char* c = sp - m16;
    const bool last = (threadIdx.x & 63u) == 63u;
    u32x4 e[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = ld16<CP>(c + lane + (uint32_t)u * TH * 16u);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      e[u] = u32x4{0u, 0u, 0u, 0u};
      if (last) e[u] = ld16_a4<CP>(c + lane + (uint32_t)u * TH * 16u + 4u * (q + 1u));
    }
    switch (q) {
      case 0: funnel_next<0, U>(v, e, s); break;
      case 1: funnel_next<1, U>(v, e, s); break;
      case 2: funnel_next<2, U>(v, e, s); break;
      default: funnel_next<3, U>(v, e, s); break;
    }
  } else {
    const uint32_t m = uniform((uint32_t)(uintptr_t)sp & 3u);
    uint32_t e[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t o = lane + (uint32_t)u * TH * 16u;
      if constexpr (FULL) {
        ld20<CP>(sp + o, m, v[u], e[u]);
      } else {
        v[u] = u32x4{0u, 0u, 0u, 0u};
        e[u] = 0u;
        if (o < t.rem) ld20<CP>(sp + o, m, v[u], e[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = shift16(v[u], e[u], m);
  }
}

// One whole copy tile: loads (FULL, SHIFT as above) and stores under one
// compile-time path, so that no loaded value crosses a branch.
template <int TH, int U, int CP, bool ALIGNED, bool FULL, bool SHIFT>
__device__ __forceinline__ void copy_tile(const CollDesc& d, const TileRef& t, uint32_t lane) {
  u32x4 v[U];
  copy_load<TH, U, CP, ALIGNED, FULL, SHIFT>(d, t, v);
  store_units<TH, U, CP, 0, ALIGNED>(d, t.J.dst_rank, t.J.dst_off + t.toff, lane, t.rem, v);
}

// One whole reduce tile, likewise.  ROLL: the rolling pipeline for tiles
// on the dword grid (the host launcher asks for it for the bf16 AllReduce
// of 8 ranks, every destination written; see reduce_tile_rolling).
template <int N, typename T, int TH, int U, int CP, bool ALIGNED, bool FULL, bool SHIFT, bool ROLL = false>
__device__ __forceinline__ void reduce_tile_store(const CollDesc& d, const TileRef& t, uint32_t lane) {
  u32x4 r[U];
  if constexpr (U == 1)
    reduce_tile_allin<N, T, TH, CP, ALIGNED, FULL, SHIFT>(d, t, r);
  else if constexpr (ROLL && !SHIFT)
    reduce_tile_rolling<N, T, TH, U, CP, ALIGNED, FULL>(d, t, r);
  else
    reduce_tile<N, T, TH, U, CP, ALIGNED, FULL, SHIFT>(d, t, r);
  store_units<TH, U, CP, N, ALIGNED>(d, t.J.dst_rank, t.J.dst_off + t.toff, lane, t.rem, r);
}

// ----------------------------------------------------------- tile loops
//
// run_reduce / run_copy: this workgroup's share of a reduce or copy
// collective.  blockDim.x must equal TH; TILE (bytes of each source per
// tile) defaults to kTileBytes, and TILE = TH * 16 gives the small-tile form
// for messages too small to fill the GPU.
// Every thread of the workgroup calls them; they return once the share is
// stored (not yet visible to other workgroups: see group_barrier).  `lds`
// is the workgroup's workspace for the job table and scan: at least
// engine_lds_bytes<TH, kMaxRanks>() bytes for run_reduce and
// engine_lds_bytes<TH>() for run_copy, 16-byte aligned; the engine declares
// no LDS of its own.
//
// The share: without a pool, tiles block, block + blocks, ... (grid-stride).
// With a pool (the host collectives' long launches), the workgroup takes
// its first `rounds` tiles that way and the rest one at a time, in order,
// from a counter all workgroups share.  On MI355X the grid-stride split
// leaves the workgroups of one or two XCDs up to five 16 KiB tiles behind
// the others by the end of a 256 MiB-per-rank AllReduce, and the tiles in
// flight then spread over a wider window of each buffer; handing out the
// tiles in order keeps every workgroup at the same place, and the
// AllReduce bf16 N=8 twin ran 0.717 ms against 0.751 (8 grid-stride rounds,
// then the counter).
// Counters in global memory, named as such so that their atomics are global
// ones (a flat atomic would also count against the LDS wait counter).
typedef __attribute__((address_space(1))) unsigned long long global_u64;

struct TilePool {
  global_u64* next;          // the first of `counters` agent-scope tile counters, SNAC_FLAG_STRIDE words
                             // apart, zero between launches; nullptr: grid-stride only
  global_u64* done;          // workgroups finished; zero between launches
  unsigned long long* xchg;  // two LDS words that pass thread 0's fetch to the workgroup
  uint32_t rounds;           // grid-stride rounds first (0 counts as 1)
  uint32_t counters;         // counter c serves the pooled tiles first + c + counters * k to the workgroups with
                             // (block / 8) % counters == c; every c must have one (0 counts as 1)
};

// Calls step(tile) for every tile of this workgroup's share, in ascending
// order.  With a pool, every workgroup of the grid must call it (the last
// one to finish clears the counters for the next launch), and thread 0
// fetches the next tile while the current one moves: the fetch is an
// atomic add whose value is first needed after the tile (the translation
// unit is built with the compiler's atomic optimizer off, which would
// otherwise wait for it at once).
template <typename Step>
__device__ __forceinline__ void for_each_tile(uint32_t block, uint32_t blocks, uint32_t total, const TilePool& pool,
                                              Step&& step) {
  // one call site of step, so that the tile code is emitted once
  const bool pooled = pool.next != nullptr;
  const uint32_t rounds = pooled ? (pool.rounds ? pool.rounds : 1u) : 0u;
  const uint32_t ncount = pooled && pool.counters ? pool.counters : 1u;
  // workgroups are dealt to the XCDs in turn (block % 8), so each counter's
  // group of workgroups holds every XCD alike
  const uint32_t c = (block / 8u) % ncount;
  global_u64* const mine = pooled ? pool.next + (uint64_t)c * SNAC_FLAG_STRIDE : nullptr;
  const uint64_t first = (uint64_t)rounds * blocks + c;  // this group's first pooled tile
  uint32_t left = rounds;                                // grid-stride rounds still to run
  uint64_t t = block;
  int p = 0;
  while (t < total) {
    // from the last grid-stride round on, each tile's successor comes from
    // the group's counter, fetched while the tile moves
    const bool fetch = pooled && left <= 1;
    unsigned long long nxt = 0;
    if (fetch && threadIdx.x == 0) nxt = __hip_atomic_fetch_add(mine, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    step((uint32_t)t);
    if (!fetch) {
      t += blocks;
      --left;
      continue;
    }
    // xchg[p] was last read before the previous barrier, so it is free
    if (threadIdx.x == 0) pool.xchg[p] = nxt;
    __syncthreads();
    t = first + (uint64_t)ncount * uniform64(pool.xchg[p]);
    p ^= 1;
  }
  if (pooled && threadIdx.x == 0) {
    // every workgroup took its last tile index before counting itself done,
    // so the last one to count may clear every counter
    const unsigned long long d = __hip_atomic_fetch_add(pool.done, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (d == (unsigned long long)blocks - 1) {
      for (uint32_t i = 0; i < ncount; ++i)
        __hip_atomic_exchange(pool.next + (uint64_t)i * SNAC_FLAG_STRIDE, 0ull, __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_exchange(pool.done, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <int N, typename T, int TH, int CP, bool ALIGNED, uint32_t TILE = kTileBytes, bool ROLL = false>
__device__ void run_reduce(const CollDesc& d, uint32_t block, uint32_t blocks, void* lds,
                           const TilePool& pool = TilePool{}) {
  constexpr int U = tile_units<TH, TILE>();
  // edge elements (head < 128 bytes, tail < 16) and jobs are looped over
  const EngineLds<TH, kMaxRanks> w(lds);
  JobL* const jobs = w.jobs;
  int nj;
  const uint32_t total = build_table<TH, kMaxRanks, ALIGNED>(d, TILE, jobs, w.scan, nj);
  if (block >= total) return;
  const uint32_t lane = threadIdx.x * 16u;
  JobCursor<TILE, ALIGNED> jc;
  jc.init(jobs, nj, block);
  for_each_tile(block, blocks, total, pool, [&](uint32_t tile) {
    const TileRef t = jc.at(tile);
    if constexpr (ALIGNED) {
      reduce_tile_store<N, T, TH, U, CP, true, true, false, ROLL>(d, t, lane);
    } else {
      if (t.lt == 0) reduce_edges<T, N>(d, t.J, t.head, t.body);
      const bool full = t.rem == TILE;
      // one test per tile, around load, add and store (see ld20)
      if (tile_needs_shift<N>(d, t)) {
        if (full)
          reduce_tile_store<N, T, TH, U, CP, false, true, true, ROLL>(d, t, lane);
        else
          reduce_tile_store<N, T, TH, U, CP, false, false, true, ROLL>(d, t, lane);
      } else {
        if (full)
          reduce_tile_store<N, T, TH, U, CP, false, true, false, ROLL>(d, t, lane);
        else
          reduce_tile_store<N, T, TH, U, CP, false, false, false, ROLL>(d, t, lane);
      }
    }
  });
}

template <int TH, int CP, bool ALIGNED, uint32_t TILE = kTileBytes>
__device__ void run_copy(const CollDesc& d, uint32_t block, uint32_t blocks, void* lds,
                         const TilePool& pool = TilePool{}) {
  constexpr int U = tile_units<TH, TILE>();
  const EngineLds<TH, kMaxJobs> w(lds);
  JobL* const jobs = w.jobs;
  int nj;
  const uint32_t total = build_table<TH, kMaxJobs, ALIGNED>(d, TILE, jobs, w.scan, nj);
  if (block >= total) return;
  const uint32_t lane = threadIdx.x * 16u;
  JobCursor<TILE, ALIGNED> jc;
  jc.init(jobs, nj, block);
  for_each_tile(block, blocks, total, pool, [&](uint32_t tile) {
    const TileRef cur = jc.at(tile);
    if constexpr (ALIGNED) {
      copy_tile<TH, U, CP, true, true, false>(d, cur, lane);
    } else {
      if (cur.lt == 0) copy_edges(d, cur.J, cur.head, cur.body);
      // one test per tile, around loads and stores (see ld20)
      const char* sp = static_cast<const char*>(d.src[cur.J.src_rank]) + cur.J.src_off + cur.toff;
      const bool shift = uniform((uint32_t)(uintptr_t)sp & 3u) != 0;
      const bool full = cur.rem == (uint32_t)TH * 16u * U;
      if (shift) {
        if (full)
          copy_tile<TH, U, CP, false, true, true>(d, cur, lane);
        else
          copy_tile<TH, U, CP, false, false, true>(d, cur, lane);
      } else {
        if (full)
          copy_tile<TH, U, CP, false, true, false>(d, cur, lane);
        else
          copy_tile<TH, U, CP, false, false, false>(d, cur, lane);
      }
    }
  });
}

// ================================================ device-side collectives

}  // namespace snac

// Arguments of a device-side collective call, one per workgroup (Purlin
// 0.6.5 "Samples": the kernel fills them in and passes them with the
// host-created context).  The pages' per-rank dst, src and bytes describe
// the calling rank's buffers in symmetric memory; with N logical ranks in
// one GPU every rank's buffers, byte count and V counts travel together in
// the descriptor that snac_describe() validated on the host, so `desc`
// stands for them here.
struct snac_args {
  const snac_coll_desc* desc;  // the collective (snac_describe); usually the address of a kernel argument
  void* workspace;             // this workgroup's LDS: at least snac::Atom<950>::PIPELINE_LDS_BYTES bytes
                               // (for TH = THREADS; Atom<950>::collective_lds_bytes<TH>() otherwise),
                               // 16-byte aligned -- the dynamic shared memory of the launch
  uint32_t blocks;             // workgroups that enter the call: exactly this many must
  uint32_t coll_blocks;        // the first coll_blocks of them (0 < coll_blocks <= blocks) move data
  uint32_t block;              // this workgroup's index in [0, blocks)
};

namespace snac {

// Run the collective of a.desc inside the caller's kernel.  Exactly
// a.blocks workgroups of TH threads call it, each with its own a.block;
// workgroups a.block < a.coll_blocks move the data (tiles shared
// round-robin), the others only wait for it.  All LDS it uses is
// a.workspace.  When it returns true in a workgroup, the whole collective's
// output is stored and visible to that workgroup.  It returns false (in
// every participant) on timeout or abort, with the status word latched for
// snac_check().
//
// T and N must match desc->esize and desc->nsrc for reduce collectives
// (AllReduce, ReduceScatter, ReduceScatterV); copy collectives ignore them.
// On a mismatch, a NULL desc or workspace, or a misaligned workspace,
// nothing is moved and SNAC_E_ARG latches.  The a.blocks workgroups must be
// co-resident; the context's barrier serves one group at a time.
//
// SYNC = false leaves out that closing grid barrier: the call returns as
// soon as this workgroup's share is stored, and the output is complete and
// visible once the kernel has ended (to the next kernel on the stream), not
// inside it.  It suits a kernel whose collective is its last step; the
// workgroups need not be co-resident, and it returns false only on an
// argument mismatch.  On MI355X the barrier costs about 24 us at the end of
// a 256 MiB-per-rank bf16 N=8 AllReduce (0.779 against 0.755 ms), most of it
// the release fence of every workgroup (see group_barrier).
template <typename T = F32, int N = 1, int TH = 256, int CP = kCacheStream, bool SYNC = true>
__device__ bool collective(const snac_args& a, const snac_dev_ctx& ctx) {
  bool good = a.desc != nullptr && a.workspace != nullptr && ((uintptr_t)a.workspace & 15u) == 0;
  if (a.coll_blocks == 0 || a.coll_blocks > a.blocks) good = false;
  bool reduce = false;
  if (good) {
    const CollDesc& desc = *a.desc;
    reduce = coll_is_reduce(desc.coll);
    if (reduce && (desc.nsrc != N || desc.esize != T::kSize)) good = false;
  }
  if (!good) {
    if (a.block == 0 && threadIdx.x == 0) latch_status(ctx.status, SNAC_E_ARG);
  } else if (a.block < a.coll_blocks) {
    const CollDesc& desc = *a.desc;
    const bool aligned = desc_aligned(desc);
    if (reduce) {
      if (aligned)
        run_reduce<N, T, TH, CP, true>(desc, a.block, a.coll_blocks, a.workspace);
      else
        run_reduce<N, T, TH, CP, false>(desc, a.block, a.coll_blocks, a.workspace);
    } else {
      if (aligned)
        run_copy<TH, CP, true>(desc, a.block, a.coll_blocks, a.workspace);
      else
        run_copy<TH, CP, false>(desc, a.block, a.coll_blocks, a.workspace);
    }
  }
  if constexpr (!SYNC) {
    return good;
  } else {
    // without a workspace there is no LDS word to meet in: return at once
    // (the error is latched; a group that all passes the same arguments
    // returns together)
    if (a.blocks == 0 || a.workspace == nullptr || ((uintptr_t)a.workspace & 15u)) return false;
    // the verdict word lies past the job table and scan
    const bool met = group_barrier(ctx.barrier, a.blocks, wait_ctl(ctx), EngineLds<TH, kMaxJobs>(a.workspace).verdict);
    return good && met;
  }
}

// The Atoms of one target and their launch contract (Purlin 0.6.5
// "Samples": a kernel using an Atom launches with its THREADS threads per
// block and the dynamic shared memory it names; Purlin 0.6.4 "Atom
// implementations": one Atom set per architecture).  This library has one
// target, gfx950 (MI355X), so Atom<950> is the only one.
template <int ARCH>
struct Atom;

template <>
struct Atom<950> {
  // workgroup size the collectives are tuned for (a wave on each of a CU's
  // four SIMDs); copy() and reduce() take any multiple of 64 up to 1024
  static constexpr int THREADS = 256;
  // copy() and reduce() keep their pipeline in registers (four 16-byte
  // units per lane in flight): they need no LDS, and ignore `workspace`
  static constexpr uint32_t COPY_LDS_BYTES = 0;
  static constexpr uint32_t REDUCE_LDS_BYTES = 0;
  // LDS a collective() call needs in a workgroup of TH threads
  template <int TH = THREADS>
  static constexpr uint32_t collective_lds_bytes() {
    return engine_lds_bytes<TH>();
  }
  static constexpr uint32_t COLLECTIVE_LDS_BYTES = engine_lds_bytes<THREADS>();
  // the dynamic LDS a kernel of THREADS threads that calls any of them
  // must be launched with (the largest of the three)
  static constexpr uint32_t PIPELINE_LDS_BYTES = COLLECTIVE_LDS_BYTES;

  template <int CP = kCacheStream>
  __device__ static void copy(void* dst, const void* src, uint64_t bytes, void* workspace = nullptr) {
    (void)workspace;
    snac::copy<CP>(dst, src, bytes);
  }
  template <typename T, int N, int CP = kCacheStream>
  __device__ static void reduce(void* const* dst, int ndst, const void* const* src, uint64_t count,
                                void* workspace = nullptr) {
    (void)workspace;
    snac::reduce<T, N, CP>(dst, ndst, src, count);
  }
};

static_assert(Atom<950>::PIPELINE_LDS_BYTES >= kMaxJobs * sizeof(JobL) + 256 * 4 + 4,
              "the collective workspace holds the job table, the scan and the barrier word");
static_assert(Atom<950>::PIPELINE_LDS_BYTES <= 64 * 1024, "fits the LDS one workgroup may allocate");

}  // namespace snac
