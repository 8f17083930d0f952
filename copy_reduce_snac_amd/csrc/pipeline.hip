// pipeline.hip -- a collective fused with compute in one kernel, coordinated
// by Stage / Notify / And Consume (Purlin 0.6.4 "Key Idea"; Purlin 0.6.5
// "Samples" calls a collective from inside a kernel between other work).
//
// Work items.  The message (count elements per rank) is cut into tiles of
// tile_bytes per rank.  Tile t of rank r has a producer item P(t, r); the
// reduction of tile t is split into N consumer parts C(t, p), each reducing
// 1/N of the tile's elements across all N ranks, so every item moves about
// the same number of bytes.  Tiles are dealt round-robin to Q independent
// queues (tile t -> queue t % Q), each with its own ring of staging slots
// and its own ticket counter; workgroup b draws tickets from queue b % Q.
// Within a queue, local tile g has group g of the ticket order holding
// P(g, 0..N-1) followed by C(g - L, 0..N-1), so consumers trail their
// producers by L tiles (the lookahead).
//
//   P(t, r)  Stage:   wait until the tile's slot is free (all N consumer
//                     parts of the slot's previous tile are done), compute
//                     y = 0.5 * x_r + r in binary32, round to the data type,
//                     store into staging[r][slot].
//            Notify:  every wave waits until its stores are accepted by
//                     the L2, the workgroup meets at a barrier, and one lane
//                     issues the agent-scope release fence (L2 write-back),
//                     waits for it, and stores ready[r][slot] = seq.
//   C(t, p)  Consume: one lane polls ready[r][slot] >= seq for every r
//                     (relaxed loads with s_sleep back-off) and issues one
//                     agent-scope acquire fence; barrier; N-to-1 reduce of
//                     part p of the staged tile into out; barrier; one lane
//                     stores freed[slot][p] = seq.
//
// One fence per item, not one per wave: agent-scope fences write back or
// invalidate a whole L2 and serialise across the GPU (measured on MI355X at
// about 28 ns per workgroup-fence with every CU fencing), so they set the
// cost of small tiles.
//
// Forward progress: within a queue a workgroup only ever waits for items
// with smaller tickets of the same queue (P(g) waits for C(g - S), ticketed
// in group g - S + L < g because L <= S - 1; C(g) waits for P(g, *),
// ticketed in group g).  Tickets are taken only by running workgroups, so
// the smallest unfinished ticket of each queue can always advance; no
// co-residency assumption about the grid is needed.
//
// Sequence numbers are monotonic across calls: seq = epoch + round + 1 with
// round = g / S.  The last workgroup to finish (acq_rel counters, per queue
// then global) adds the largest round count to the epoch and clears the
// ticket and done counters, all in device memory, so consecutive launches (also inside a replayed
// graph) need no host bookkeeping and no reset pass.
//
// Waits are bounded: after 2^spin_limit_log2 polls a wait latches
// SNAC_E_TIMEOUT in the status word and gives up; a host-mapped abort word
// does the same with SNAC_E_ABORTED.  Once the status word is set every
// later wait gives up at once, so the grid always drains.
#include <hip/hip_runtime.h>

#include "internal.hpp"
#include "snac_device.hpp"

namespace snac {

// The bounded waits of this kernel: status word and abort word of the
// context, its poll budget (the flag primitives are snac_device.hpp's).
__device__ __forceinline__ WaitCtl pipe_wait(const PipeArgs& a) {
  return WaitCtl{&a.ctrl[kCtrlStatus], a.abort_word, a.spin_limit_log2};
}

// The constant-rate wall clock (s_memrealtime), 100 MHz on MI300-family
// parts; only the test-hook delay below uses it.
constexpr uint64_t kWallTicksPerUs = 100;

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

// Elements of tile t (the last tile may be short).
__device__ __forceinline__ uint32_t tile_count(const PipeArgs& a, uint32_t t) {
  const uint64_t e0 = (uint64_t)t * a.tile_elems;
  return uniform(t + 1 < a.tiles ? a.tile_elems : (uint32_t)(a.count - e0));
}

template <typename T, int N>
__device__ void stage_item(const PipeArgs& a, uint32_t t, uint32_t gslot, uint32_t round, uint32_t r, uint64_t epoch,
                        uint32_t* s_ok) {
  constexpr uint32_t E = T::kSize;
  if (round > 0) {
    if (threadIdx.x == 0) {
      bool ok = true;
      for (int p = 0; p < N && ok; ++p)
        ok = wait_geq(&a.freed[((uint64_t)gslot * N + p) * kFlagStride], epoch + round, pipe_wait(a));
      *s_ok = ok ? 1u : 0u;
    }
    __syncthreads();
    const uint32_t ok = uniform(*s_ok);
    __syncthreads();
    if (ok == 0) return;
  }
  if (a.producer_delay_us) {  // test hook: skew a quarter of the producers
    const uint32_t h = (t * 0x9E3779B1u) ^ (r * 0x85EBCA6Bu);
    if ((h >> 29) < 2) {
      const uint64_t until = wall_clock64() + (uint64_t)a.producer_delay_us * kWallTicksPerUs;
      while (wall_clock64() < until) __builtin_amdgcn_s_sleep(8);
    }
  }
  const uint64_t e0 = (uint64_t)t * a.tile_elems;
  const uint32_t nbytes = tile_count(a, t) * E;
  const char* src = static_cast<const char*>(a.x[r]) + e0 * E;
  char* stg = a.staging + ((uint64_t)r * a.slots + gslot) * a.tile_bytes;
  const float rf = (float)r;
  const uint32_t nvec = nbytes & ~15u;
  constexpr int U = 4;
  // staging stores write through the L2 (see kWriteThrough), so the release
  // fence below has little left to write back
  const __amdgpu_buffer_rsrc_t stg_r = buffer_rsrc(stg, nvec);
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
      if (o < nvec) bst16<kWriteThrough>(stg_r, o, scale_unit<T>(v[u], rf));
    }
  }
  const uint32_t tail = (nbytes - nvec) / E;
  if (threadIdx.x < tail) {
    const uint32_t o = nvec + threadIdx.x * E;
    store_elem<T>(stg + o, load_elem<T>(src + o) * 0.5f + rf);
  }
  // Notify.  Every wave waits until the L2 has accepted its staging stores;
  // after the barrier one lane writes the L2 back at agent scope (a single
  // release fence per tile: these fences serialise across the GPU, so one per
  // wave would cost four times as much), waits for the write-back, and only
  // then stores the flag.
  wait_vm();
  __syncthreads();
  if (threadIdx.x == 0 && a.drop_notify != (int32_t)r + 1) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    wait_vm();
    __hip_atomic_store(&a.ready[((uint64_t)r * a.slots + gslot) * kFlagStride], epoch + round + 1, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <typename T, int N>
__device__ void consume_item(const PipeArgs& a, uint32_t t, uint32_t gslot, uint32_t round, uint32_t part, uint64_t epoch,
                        uint32_t* s_ok) {
  constexpr uint32_t E = T::kSize;
  const uint64_t seq = epoch + round + 1;
  // Consume: one lane sees every rank's flag, then one acquire fence (an L2
  // and L1 invalidate shared by the whole workgroup's CU) before the barrier
  // releases the other waves to read the staged data.
  if (threadIdx.x == 0) {
    bool ok = true;
    for (int r = 0; r < N && ok; ++r)
      ok = wait_geq(&a.ready[((uint64_t)r * a.slots + gslot) * kFlagStride], seq, pipe_wait(a));
    if (ok) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      wait_vm();
    }
    *s_ok = ok ? 1u : 0u;
  }
  __syncthreads();
  const uint32_t ok = uniform(*s_ok);
  __syncthreads();
  if (ok == 0) return;
  const uint32_t ne = tile_count(a, t);
  const uint32_t p0 = part * a.part_elems;
  const uint32_t pn = p0 >= ne ? 0u : (ne - p0 < a.part_elems ? ne - p0 : a.part_elems);
  const uint32_t nbytes = pn * E;
  const uint64_t rank_stride = (uint64_t)a.slots * a.tile_bytes;
  const char* stg = a.staging + (uint64_t)gslot * a.tile_bytes + (uint64_t)p0 * E;
  char* out = static_cast<char*>(a.out) + ((uint64_t)t * a.tile_elems + p0) * E;
  const uint32_t nvec = nbytes & ~15u;
  // the output is written through the L2 as the staging is: the producers'
  // release fences write back every dirty line of their XCD's L2, and
  // write-back output lines would add to that (f32 4096x8192 N=8: 0.629 ms
  // against 0.638 with streaming write-back stores; bf16 0.2-0.6 % faster)
  const __amdgpu_buffer_rsrc_t out_r = buffer_rsrc(out, nvec);
  constexpr int U = N <= 4 ? 2 : 1;
  for (uint32_t base = 0; base < nvec; base += kThreads * 16u * U) {
    u32x4 v[U][N];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t o = base + (threadIdx.x + (uint32_t)u * kThreads) * 16u;
      if (o < nvec) {
#pragma unroll
        for (int k = 0; k < N; ++k) v[u][k] = bld16<kWriteThrough>(buffer_rsrc(stg + k * rank_stride, nvec), o);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t o = base + (threadIdx.x + (uint32_t)u * kThreads) * 16u;
      if (o < nvec) bst16<kWriteThrough>(out_r, o, reduce_unit<T, N>(v[u]));
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
  // Free the slot.  This edge only has to order this workgroup's staging
  // loads before the producer's next stores to the slot: every load has
  // returned its data (the values were used above) before the barrier, and
  // the producer issues its stores only after it has seen the flag, so a
  // relaxed store and a relaxed wait suffice and no cache maintenance is
  // spent on it.
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_store(&a.freed[((uint64_t)gslot * N + part) * kFlagStride], seq, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T, int N>
__global__ __launch_bounds__(kThreads) void pipeline_kernel(const PipeArgs a) {
  __shared__ uint32_t s_item;
  __shared__ uint32_t s_ok;
  const uint64_t epoch = uniform64(ld_relaxed(&a.ctrl[kCtrlEpoch]));
  const uint32_t Q = a.queues;
  const uint32_t S = a.qslots;
  const uint32_t q = uniform(blockIdx.x % Q);
  // local tiles of this queue: t = g * Q + q
  const uint32_t qtiles = uniform(a.tiles > q ? (a.tiles - q + Q - 1) / Q : 0u);
  const uint32_t L = uniform(a.lookahead < qtiles ? a.lookahead : qtiles);
  const uint32_t items = uniform((qtiles + L) * (uint32_t)(2 * N));
  uint64_t* ticket = &a.ctrl[kCtrlTicket + q * kFlagStride];
  for (;;) {
    // The barrier at the top closes the previous item's single-lane flag
    // store before the next single-lane ticket fetch; without it the
    // compiler may thread the two lane-0 regions into one back edge that
    // the other lanes skip, so that the lanes of a wave meet the barriers
    // below on different iterations.  It also keeps s_item from being
    // overwritten before every wave has read it.
    __syncthreads();
    if (threadIdx.x == 0)
      s_item = (uint32_t)__hip_atomic_fetch_add(ticket, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const uint32_t item = uniform(s_item);
    if (item >= items) break;
    const uint32_t g = uniform(item / (uint32_t)(2 * N));
    const uint32_t w = uniform(item - g * (uint32_t)(2 * N));
    if (w < (uint32_t)N) {
      if (g < qtiles) stage_item<T, N>(a, g * Q + q, uniform(q * S + g % S), uniform(g / S), w, epoch, &s_ok);
    } else if (g >= L) {
      const uint32_t gc = g - L;
      consume_item<T, N>(a, gc * Q + q, uniform(q * S + gc % S), uniform(gc / S), w - (uint32_t)N, epoch, &s_ok);
    }
  }
  // Completion, counted per queue first (each queue's workgroups hit their
  // own counter; a same-address atomic costs ~12 ns, so one global counter
  // would serialise the whole grid), then once per queue globally.  The last
  // workgroup of a queue resets that queue's counters; the last queue to
  // finish advances the epoch.
  if (threadIdx.x == 0) {
    const uint64_t per_queue = gridDim.x / Q;  // the grid is a multiple of Q
    uint64_t* qdone = &a.ctrl[kCtrlQDone + q * kFlagStride];
    const uint64_t oq = __hip_atomic_fetch_add(qdone, (uint64_t)1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (oq == per_queue - 1) {
      __hip_atomic_store(ticket, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(qdone, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint64_t old =
          __hip_atomic_fetch_add(&a.ctrl[kCtrlDone], (uint64_t)1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      if (old == (uint64_t)Q - 1) {
        __hip_atomic_store(&a.ctrl[kCtrlDone], (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&a.ctrl[kCtrlEpoch], epoch + a.rounds, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      }
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
  // queues: as many as there are tiles and 2-slot rings allow
  uint64_t Q = kMaxQueues;
  if (Q > tiles) Q = tiles;
  if (Q > a.slots / 2) Q = a.slots / 2;
  if (Q < 1) return hipErrorInvalidValue;
  const uint64_t S = a.slots / Q;
  const uint64_t qtiles = (tiles + Q - 1) / Q;
  int per_cu = 0;
  hipError_t err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(fn), kThreads, 0);
  if (err != hipSuccess) return err;
  if (per_cu < 1) per_cu = 1;
  // Measured on MI355X: when the ring holds the whole message no producer
  // waits for a slot and 4 workgroups per CU keep HBM busiest; when slots
  // are reused, more workgroups only add waiting ones, and 2 did best.
  const int want = cfg.wgs_per_cu > 0 ? cfg.wgs_per_cu : (qtiles <= S ? 4 : 2);
  if (want < per_cu) per_cu = want;
  const int cus = device_cu_count();
  uint64_t grid = (uint64_t)(cus > 0 ? cus : 1) * (uint64_t)per_cu;
  // lookahead: tiles staged ahead of the consumers, at most S - 1 (forward
  // progress); the whole ring by default
  uint64_t L = a.lookahead ? a.lookahead : S - 1;
  if (L > S - 1) L = S - 1;
  if (L > qtiles) L = qtiles;  // as the kernel does: sizes the grid to the real work
  // enough workgroups to keep every queue's lookahead window busy, and a
  // multiple of Q so that the queues get equal shares
  const uint64_t items_per_q = (qtiles + L) * (uint64_t)(2 * a.nranks);
  if (grid > items_per_q * Q) grid = items_per_q * Q;
  grid = (grid + Q - 1) / Q * Q;
  a.queues = (uint32_t)Q;
  a.qslots = (uint32_t)S;
  a.lookahead = (uint32_t)L;
  a.grid = (uint32_t)grid;
  a.tiles = (uint32_t)tiles;
  a.rounds = (uint32_t)((qtiles + S - 1) / S);
  a.tile_elems = (uint32_t)te;
  const uint64_t vec = 16 / e;  // elements per 16-byte unit
  uint64_t pe = (te + (uint64_t)a.nranks - 1) / (uint64_t)a.nranks;
  pe = (pe + vec - 1) / vec * vec;
  a.part_elems = (uint32_t)pe;
  if (grid_out) *grid_out = (uint32_t)grid;
  hipLaunchKernelGGL(fn, dim3((uint32_t)grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace snac
