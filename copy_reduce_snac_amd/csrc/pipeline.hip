// pipeline.hip -- a collective fused with compute in one kernel, coordinated
// by Stage / Notify / And Consume (Purlin 0.6.4 "Key Idea"; Purlin 0.6.5
// "Samples" calls a collective from inside a kernel between other work).
//
// Work items.  The message (count elements per rank) is cut into tiles of
// tile_bytes per rank.  Tile t of rank r has a producer item P(t, r) and
// tile t has one consumer item C(t).  Items are handed out in a fixed order
// by an atomic ticket counter: group g holds P(g, 0..N-1) followed by
// C(g - L), so a consumer trails its producers by L tiles (the lookahead).
//
//   P(t, r)  Stage:   wait until slot t mod S of rank r is free, compute
//                     y = 0.5 * x_r + r in binary32, round to the data type,
//                     store into staging[r][slot].
//            Notify:  every wave fences (release, agent scope), the
//                     workgroup meets at a barrier, one lane stores
//                     ready[r][slot] = seq with release semantics.
//   C(t)     Consume: one lane polls ready[r][slot] >= seq for every r
//                     (relaxed loads, s_sleep back-off, then an acquire
//                     fence); the workgroup meets at a barrier and every
//                     wave fences (acquire, agent scope); N-to-1 reduce of
//                     the staged tiles into out; barrier; one lane releases
//                     free[slot] = seq.
//
// Forward progress: a workgroup only ever waits for items with smaller
// tickets (P(t) waits for C(t - S), ticketed in group t - S + L < t because
// L <= S - 1; C(t) waits for P(t, *), ticketed in group t).  Tickets are
// taken only by running workgroups, so the smallest unfinished ticket can
// always advance -- no co-residency assumption about the grid is needed.
//
// Sequence numbers are monotonic across calls: seq = epoch + round + 1 with
// round = t / S.  The last workgroup to finish (an acq_rel counter) adds the
// number of rounds to the epoch and clears the ticket and done counters, all
// in device memory, so consecutive launches (also inside a replayed graph)
// need no host bookkeeping and no reset pass.
//
// Waits are bounded: after 2^spin_limit_log2 polls a wait latches
// SNAC_E_TIMEOUT in the status word and gives up; a host-mapped abort word
// does the same with SNAC_E_ABORTED.  Once the status word is set every
// later wait gives up at once, so the grid always drains.
#include <hip/hip_runtime.h>

#include "atoms.hpp"
#include "internal.hpp"

namespace snac {

enum : uint64_t { kStatusTimeout = 5, kStatusAborted = 7 };

__device__ __forceinline__ uint64_t ld_relaxed(uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void latch_status(uint64_t* ctrl, uint64_t code) {
  uint64_t expected = 0;
  __hip_atomic_compare_exchange_strong(&ctrl[kCtrlStatus], &expected, code, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
}

// One lane waits until *flag >= target.  Returns false (and the status word
// is set) on timeout, abort, or an error latched elsewhere.
__device__ bool wait_geq(uint64_t* flag, uint64_t target, const PipeArgs& a) {
  const uint64_t limit = 1ull << a.spin_limit_log2;
  uint64_t spins = 0;
  while (ld_relaxed(flag) < target) {
    if ((spins & 15u) == 15u) {
      if (ld_relaxed(&a.ctrl[kCtrlStatus]) != 0) return false;
      uint32_t* ab = const_cast<uint32_t*>(a.abort_word);
      if (__hip_atomic_load(ab, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) != 0) {
        latch_status(a.ctrl, kStatusAborted);
        return false;
      }
    }
    if (++spins >= limit) {
      latch_status(a.ctrl, kStatusTimeout);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return true;
}

// y = 0.5 * x + r on one 16-byte unit, rounded to T.
template <typename T>
__device__ __forceinline__ u32x4 scale_unit(u32x4 x, float r) {
  u32x4 y;
  if constexpr (T::kSize == 4) {
#pragma unroll
    for (int c = 0; c < 4; ++c) y[c] = __float_as_uint(__uint_as_float(x[c]) * 0.5f + r);
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) y[c] = pack_bf16(bf16_lo(x[c]) * 0.5f + r, bf16_hi(x[c]) * 0.5f + r);
  }
  return y;
}

// Every value that decides a branch or a loop around a barrier is made
// wave-uniform explicitly (kernel arguments, or readfirstlane): if the
// compiler cannot prove a loop exit uniform it may restructure the loop so
// that lanes of one wave reach a barrier on different iterations.

template <typename T>
__device__ void produce(const PipeArgs& a, uint32_t t, uint32_t r, uint64_t epoch, uint32_t* s_ok) {
  constexpr uint32_t E = T::kSize;
  const uint32_t S = a.slots;
  const uint32_t slot = uniform(t % S);
  const uint32_t round = uniform(t / S);
  if (round > 0) {
    if (threadIdx.x == 0) *s_ok = wait_geq(&a.freed[(uint64_t)slot * kFlagStride], epoch + round, a) ? 1u : 0u;
    __syncthreads();
    const uint32_t ok = uniform(*s_ok);
    __syncthreads();
    if (ok == 0) return;
  }
  const uint64_t e0 = (uint64_t)t * a.tile_elems;
  const uint32_t ne = uniform(t + 1 < a.tiles ? a.tile_elems : (uint32_t)(a.count - e0));
  const uint32_t nbytes = ne * E;
  const char* src = static_cast<const char*>(a.x[r]) + e0 * E;
  char* stg = a.staging + ((uint64_t)r * S + slot) * a.tile_bytes;
  const float rf = (float)r;
  const uint32_t nvec = nbytes & ~15u;
  constexpr int U = 4;
  for (uint32_t base = 0; base < nvec; base += kThreads * 16u * U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t o = base + (threadIdx.x + (uint32_t)u * kThreads) * 16u;
      if (o < nvec) v[u] = ld16<kCacheStreamLoads>(src + o);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t o = base + (threadIdx.x + (uint32_t)u * kThreads) * 16u;
      if (o < nvec) st16<kCacheDefault>(stg + o, scale_unit<T>(v[u], rf));
    }
  }
  const uint32_t tail = (nbytes - nvec) / E;
  if (threadIdx.x < tail) {
    const uint32_t o = nvec + threadIdx.x * E;
    store_elem<T>(stg + o, load_elem<T>(src + o) * 0.5f + rf);
  }
  // Notify: every wave's staging stores are written back at agent scope
  // before any lane can observe the flag
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (threadIdx.x == 0 && a.drop_notify != (int32_t)r + 1)
    __hip_atomic_store(&a.ready[((uint64_t)r * S + slot) * kFlagStride], epoch + round + 1, __ATOMIC_RELEASE,
                       __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T, int N>
__device__ void consume(const PipeArgs& a, uint32_t t, uint64_t epoch, uint32_t* s_ok) {
  constexpr uint32_t E = T::kSize;
  const uint32_t S = a.slots;
  const uint32_t slot = uniform(t % S);
  const uint64_t seq = epoch + uniform(t / S) + 1;
  if (threadIdx.x == 0) {
    bool ok = true;
    for (int r = 0; r < N && ok; ++r) ok = wait_geq(&a.ready[((uint64_t)r * S + slot) * kFlagStride], seq, a);
    *s_ok = ok ? 1u : 0u;
  }
  __syncthreads();
  const uint32_t ok = uniform(*s_ok);
  __syncthreads();
  if (ok == 0) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  const uint64_t e0 = (uint64_t)t * a.tile_elems;
  const uint32_t ne = uniform(t + 1 < a.tiles ? a.tile_elems : (uint32_t)(a.count - e0));
  const uint32_t nbytes = ne * E;
  const uint64_t rank_stride = (uint64_t)S * a.tile_bytes;
  const char* stg = a.staging + (uint64_t)slot * a.tile_bytes;
  char* out = static_cast<char*>(a.out) + e0 * E;
  const uint32_t nvec = nbytes & ~15u;
  constexpr int U = N <= 4 ? 2 : 1;
  for (uint32_t base = 0; base < nvec; base += kThreads * 16u * U) {
    u32x4 v[U][N];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t o = base + (threadIdx.x + (uint32_t)u * kThreads) * 16u;
      if (o < nvec) {
#pragma unroll
        for (int k = 0; k < N; ++k) v[u][k] = ld16<kCacheDefault>(stg + k * rank_stride + o);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t o = base + (threadIdx.x + (uint32_t)u * kThreads) * 16u;
      if (o < nvec) st16<kCacheDefault>(out + o, reduce_unit<T, N>(v[u]));
    }
  }
  const uint32_t tail = (nbytes - nvec) / E;
  if (threadIdx.x < tail) {
    const uint32_t o = nvec + threadIdx.x * E;
    float acc = load_elem<T>(stg + o);
#pragma unroll
    for (int k = 1; k < N; ++k) acc = acc + load_elem<T>(stg + k * rank_stride + o);
    store_elem<T>(out + o, acc);
  }
  // every wave has its staged values in registers (they were used above);
  // the slot may be overwritten once the flag is seen
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_store(&a.freed[(uint64_t)slot * kFlagStride], seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T, int N>
__global__ __launch_bounds__(kThreads) void pipeline_kernel(const PipeArgs a) {
  __shared__ uint32_t s_item;
  __shared__ uint32_t s_ok;
  const uint64_t epoch = uniform64(ld_relaxed(&a.ctrl[kCtrlEpoch]));
  const uint32_t items = a.items;
  const uint32_t L = a.lookahead;
  const uint32_t tiles = a.tiles;
  for (;;) {
    // The barrier at the top closes the previous item's single-lane flag
    // store before the next single-lane ticket fetch; without it the
    // compiler may thread the two lane-0 regions into one back edge that
    // the other lanes skip, so that the lanes of a wave meet the barriers
    // below on different iterations.  It also keeps s_item from being
    // overwritten before every wave has read it.
    __syncthreads();
    if (threadIdx.x == 0)
      s_item = (uint32_t)__hip_atomic_fetch_add(&a.ctrl[kCtrlTicket], (uint64_t)1, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const uint32_t item = uniform(s_item);
    if (item >= items) break;
    const uint32_t g = item / (uint32_t)(N + 1);
    const uint32_t w = item - g * (uint32_t)(N + 1);
    if (w < (uint32_t)N) {
      if (g < tiles) produce<T>(a, g, w, epoch, &s_ok);
    } else if (g >= L) {
      consume<T, N>(a, g - L, epoch, &s_ok);
    }
  }
  if (threadIdx.x == 0) {
    const uint64_t old =
        __hip_atomic_fetch_add(&a.ctrl[kCtrlDone], (uint64_t)1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (old == (uint64_t)gridDim.x - 1) {
      __hip_atomic_store(&a.ctrl[kCtrlTicket], (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&a.ctrl[kCtrlDone], (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&a.ctrl[kCtrlEpoch], epoch + a.rounds, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

using PipeFn = void (*)(const PipeArgs);

template <typename T>
static PipeFn pipe_kernel(int n) {
  switch (n) {
    case 1: return &pipeline_kernel<T, 1>;
    case 2: return &pipeline_kernel<T, 2>;
    case 3: return &pipeline_kernel<T, 3>;
    case 4: return &pipeline_kernel<T, 4>;
    case 5: return &pipeline_kernel<T, 5>;
    case 6: return &pipeline_kernel<T, 6>;
    case 7: return &pipeline_kernel<T, 7>;
    case 8: return &pipeline_kernel<T, 8>;
    case 9: return &pipeline_kernel<T, 9>;
    case 10: return &pipeline_kernel<T, 10>;
    case 11: return &pipeline_kernel<T, 11>;
    case 12: return &pipeline_kernel<T, 12>;
    case 13: return &pipeline_kernel<T, 13>;
    case 14: return &pipeline_kernel<T, 14>;
    case 15: return &pipeline_kernel<T, 15>;
    case 16: return &pipeline_kernel<T, 16>;
    default: return nullptr;
  }
}

hipError_t launch_pipeline(const PipeArgs& in, int dtype_bf16, const LaunchCfg& cfg, hipStream_t stream,
                           uint32_t* grid_out) {
  PipeArgs a = in;
  PipeFn fn = dtype_bf16 ? pipe_kernel<BF16>(a.nranks) : pipe_kernel<F32>(a.nranks);
  if (!fn) return hipErrorInvalidValue;
  const uint64_t e = (uint64_t)a.esize;
  const uint64_t te = a.tile_bytes / e;
  const uint64_t tiles = (a.count + te - 1) / te;
  if (tiles == 0) return hipSuccess;
  if (tiles > 0x3fffffffull || te > 0xffffffffull) return hipErrorInvalidValue;
  int per_cu = 0;
  hipError_t err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(fn), kThreads, 0);
  if (err != hipSuccess) return err;
  if (per_cu < 1) per_cu = 1;
  if (cfg.wgs_per_cu > 0 && cfg.wgs_per_cu < per_cu) per_cu = cfg.wgs_per_cu;
  const int cus = device_cu_count();
  uint64_t grid = (uint64_t)(cus > 0 ? cus : 1) * (uint64_t)per_cu;
  // lookahead: enough tiles staged ahead that a consumer's producers have
  // usually finished when it is ticketed; at most S - 1 (forward progress)
  uint64_t L = a.lookahead ? a.lookahead : (grid + a.nranks) / (uint64_t)(a.nranks + 1);
  if (L > a.slots - 1) L = a.slots - 1;
  if (L > tiles) L = tiles;
  a.lookahead = (uint32_t)L;
  const uint64_t items = (tiles + L) * (uint64_t)(a.nranks + 1);
  if (items > 0xffffffffull - 0x100000ull) return hipErrorInvalidValue;
  if (grid > items) grid = items;
  a.grid = (uint32_t)grid;
  a.tiles = (uint32_t)tiles;
  a.items = (uint32_t)items;
  a.rounds = (uint32_t)((tiles + a.slots - 1) / a.slots);
  a.tile_elems = (uint32_t)te;
  if (grid_out) *grid_out = (uint32_t)grid;
  hipLaunchKernelGGL(fn, dim3((uint32_t)grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace snac
