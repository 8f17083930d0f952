// pipeline.hip -- a collective fused with compute in one kernel, coordinated
// by Stage / Notify / And Consume (Purlin 0.6.4 "Key Idea"; Purlin 0.6.5
// "Samples" calls a collective from inside a kernel between other work).
//
// Work items.  The message (count elements per rank) is cut into tiles of
// tile_bytes per rank.  Tile t of rank r has a producer item P(t, r); the
// reduction of tile t is split into N consumer parts C(t, p), so every item
// moves about the same number of bytes.  Tiles are dealt round-robin to Q
// independent queues (tile t -> queue t % Q), each with its own ring of
// staging slots and its own ticket counter; workgroup b draws tickets from
// queue b % Q.  Within a queue, local tile g has group g of the ticket order
// holding P(g, 0..N-1) followed by C(g - L, 0..N-1), so consumers trail
// their producers by L tiles (the lookahead).
//
// Layout.  Each rank's message is a row of layout units of 1, 2 or 4
// pieces, a piece being 4 KiB (one 16-byte access per lane of a 256-lane
// workgroup).  Of nt tiles, tile t owns units t, t + nt, t + 2 nt, ..., and
// in the rank's staging ring unit j of slot s sits at unit j * slots + s.
// All the items in flight therefore sweep one compact window of x, staging
// and out together instead of streaming through separate contiguous tiles:
// on MI355X (bf16 4096x8192, N=8, 16 KiB units) the producer phase alone
// took 182 us this way against 201 us with contiguous 1 MiB tiles, and the
// consumer phase 95 against 107 us.  Producers take a tile's pieces in
// order; consumer part p takes pieces p, p + N, p + 2 N, ...  Only the
// message's last unit can be short (whole pieces, then at most one short
// piece); it belongs to tile (whole units) % nt.
//
//   P(t, r)  Stage:   wait until the tile's slot is free (all N consumer
//                     parts of the slot's previous tile are done), compute
//                     y = 0.5 * x_r + r in binary32, round to the data type,
//                     store into the slot's units of staging[r].
//            Notify:  every wave waits until its stores are accepted by
//                     the L2, the workgroup meets at a barrier, and one lane
//                     issues the agent-scope release fence (L2 write-back),
//                     waits for it, and stores ready[r][slot] = seq.
//   C(t, p)  Consume: the first wave polls ready[r][slot] >= seq, lane r
//                     for rank r (relaxed loads with s_sleep back-off), and
//                     issues one agent-scope acquire fence; barrier; N-to-1
//                     reduce of the staged units of part p into out;
//                     barrier; one lane stores freed[slot][p] = seq.
//
// One fence per item, not one per wave: agent-scope fences write back or
// invalidate a whole L2 and serialise across the GPU (measured on MI355X at
// about 28 ns per workgroup-fence with every CU fencing), so they set the
// cost of small tiles; the host cuts the ring into about one producer item
// per workgroup.
//
// Forward progress: within a queue a workgroup only ever waits for items
// with smaller tickets of the same queue (P(g) waits for C(g - S), ticketed
// in group g - S + L < g because L <= S - 1; C(g) waits for P(g, *),
// ticketed in group g).  Tickets are taken only by running workgroups, so
// the smallest unfinished ticket of each queue can always advance; no
// co-residency assumption about the grid is needed.
//
// Sequence numbers are monotonic across calls: seq = epoch + round + 1 with
// round = g / S.  The last workgroup to finish (release adds on per-queue
// counters, then one global counter) adds the largest round count to the
// epoch and clears the ticket and done counters, all in device memory, so
// consecutive launches (also inside a replayed graph) need no host
// bookkeeping and no reset pass.
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

// A piece is one 16-byte access for each of the kThreads lanes; a layout
// unit is 1 << unit_shift pieces (a.unit_bytes).
constexpr uint32_t kPiece = kThreads * 16u;

// Where piece s of tile t lives, as byte offsets from the tile's first unit
// in x / out (units nt apart) and from the slot's first unit in staging
// (units `slots` apart).
struct PieceAt {
  uint64_t x, stg;
};
__device__ __forceinline__ PieceAt piece_at(const PipeArgs& a, uint32_t s) {
  const uint64_t j = s >> a.unit_shift;
  const uint64_t w = (uint64_t)(s & ((1u << a.unit_shift) - 1u)) * kPiece;
  return PieceAt{j * a.tiles * a.unit_bytes + w, j * a.slots * a.unit_bytes + w};
}

// Whole pieces of tile t: its units below the message's whole units, and on
// the tile holding the short last unit, that unit's whole pieces.  The one
// short piece (if any) follows them.
__device__ __forceinline__ uint32_t tile_pieces(const PipeArgs& a, uint32_t t) {
  const uint32_t jf = a.full_units > t ? (a.full_units - t + a.tiles - 1) / a.tiles : 0u;
  return uniform((jf << a.unit_shift) + (t == a.tail_tile ? a.tail_pieces : 0u));
}

template <typename T, int N>
__device__ void stage_item(const PipeArgs& a, uint32_t t, uint32_t gslot, uint32_t round, uint32_t r, uint64_t epoch,
                        uint32_t* s_ok) {
  constexpr uint32_t E = T::kSize;
  if (round > 0) {
    if (threadIdx.x < 64) {  // the first wave, lane p polling part p's flag
      const bool ok = wait_all_geq(&a.freed[(uint64_t)gslot * N * kFlagStride], N, kFlagStride, epoch + round,
                                   pipe_wait(a));
      if (threadIdx.x == 0) *s_ok = ok ? 1u : 0u;
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
  const uint32_t np = tile_pieces(a, t);
  const char* src = static_cast<const char*>(a.x[r]) + (uint64_t)t * a.unit_bytes;
  char* stg = a.staging + (uint64_t)r * a.slots * a.tile_bytes + (uint64_t)gslot * a.unit_bytes;
  const float rf = (float)r;
  const uint32_t lane = threadIdx.x * 16u;
  constexpr uint32_t U = 4;
  // staging stores write through the L2 (see kWriteThrough), so the release
  // fence below has little left to write back
  uint32_t s = 0;
  for (; s + U <= np; s += U) {
    u32x4 v[U];
#pragma unroll
    for (uint32_t u = 0; u < U; ++u) v[u] = ld16<kCacheStreamLoads>(src + piece_at(a, s + u).x + lane);
#pragma unroll
    for (uint32_t u = 0; u < U; ++u)
      bst16<kWriteThrough>(buffer_rsrc(stg + piece_at(a, s + u).stg, kPiece), lane, scale_unit<T>(v[u], rf));
  }
  for (; s < np; ++s) {
    const PieceAt p = piece_at(a, s);
    bst16<kWriteThrough>(buffer_rsrc(stg + p.stg, kPiece), lane, scale_unit<T>(ld16<kCacheStreamLoads>(src + p.x + lane), rf));
  }
  if (a.last_bytes && t == a.tail_tile) {  // the message's short last piece, piece np of this tile
    const PieceAt p = piece_at(a, np);
    const char* xs = src + p.x;
    char* d = stg + p.stg;
    const uint32_t nvec = a.last_bytes & ~15u;
    if (lane < nvec)
      bst16<kWriteThrough>(buffer_rsrc(d, nvec), lane, scale_unit<T>(ld16<kCacheStreamLoads>(xs + lane), rf));
    const uint32_t tail = (a.last_bytes - nvec) / E;
    if (threadIdx.x < tail) {
      const uint32_t o = nvec + threadIdx.x * E;
      store_elem<T>(d + o, load_elem<T>(xs + o) * 0.5f + rf);
    }
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
  if (threadIdx.x < 64) {  // the first wave, lane r polling rank r's flag
    const bool ok = wait_all_geq(&a.ready[(uint64_t)gslot * kFlagStride], N, (uint64_t)a.slots * kFlagStride, seq,
                                 pipe_wait(a));
    if (ok) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      wait_vm();
    }
    if (threadIdx.x == 0) *s_ok = ok ? 1u : 0u;
  }
  __syncthreads();
  const uint32_t ok = uniform(*s_ok);
  __syncthreads();
  if (ok == 0) return;
  // this part's pieces of the tile: part + N i
  const uint32_t np = tile_pieces(a, t);
  const uint32_t ni = uniform(np > part ? (np - part + (uint32_t)N - 1) / (uint32_t)N : 0u);
  const uint64_t rank_stride = (uint64_t)a.slots * a.tile_bytes;
  const char* stg = a.staging + (uint64_t)gslot * a.unit_bytes;
  char* out = static_cast<char*>(a.out) + (uint64_t)t * a.unit_bytes;
  const uint32_t lane = threadIdx.x * 16u;
  // the output is written through the L2 as the staging is: the producers'
  // release fences write back every dirty line of their XCD's L2, and
  // write-back output lines would add to that (f32 4096x8192 N=8: 0.629 ms
  // against 0.638 with streaming write-back stores; bf16 0.2-0.6 % faster)
  constexpr uint32_t U = N <= 4 ? 2 : 1;
  uint32_t i = 0;
  for (; i + U <= ni; i += U) {
    u32x4 v[U][N];
#pragma unroll
    for (uint32_t u = 0; u < U; ++u) {
      const uint64_t so = piece_at(a, part + (uint32_t)N * (i + u)).stg;
#pragma unroll
      for (int k = 0; k < N; ++k) v[u][k] = bld16<kWriteThrough>(buffer_rsrc(stg + k * rank_stride + so, kPiece), lane);
    }
#pragma unroll
    for (uint32_t u = 0; u < U; ++u) {
      const uint64_t oo = piece_at(a, part + (uint32_t)N * (i + u)).x;
      bst16<kWriteThrough>(buffer_rsrc(out + oo, kPiece), lane, reduce_unit<T, N>(v[u]));
    }
  }
  for (; i < ni; ++i) {
    u32x4 v[N];
    const PieceAt p = piece_at(a, part + (uint32_t)N * i);
#pragma unroll
    for (int k = 0; k < N; ++k) v[k] = bld16<kWriteThrough>(buffer_rsrc(stg + k * rank_stride + p.stg, kPiece), lane);
    bst16<kWriteThrough>(buffer_rsrc(out + p.x, kPiece), lane, reduce_unit<T, N>(v));
  }
  if (a.last_bytes && t == a.tail_tile && np % (uint32_t)N == part) {  // the short last piece, piece np
    const PieceAt p = piece_at(a, np);
    const char* s = stg + p.stg;
    char* d = out + p.x;
    const uint32_t nvec = a.last_bytes & ~15u;
    if (lane < nvec) {
      u32x4 v[N];
#pragma unroll
      for (int k = 0; k < N; ++k) v[k] = bld16<kWriteThrough>(buffer_rsrc(s + k * rank_stride, nvec), lane);
      bst16<kWriteThrough>(buffer_rsrc(d, nvec), lane, reduce_unit<T, N>(v));
    }
    const uint32_t tail = (a.last_bytes - nvec) / E;
    if (threadIdx.x < tail) {
      const uint32_t o = nvec + threadIdx.x * E;
      float acc = load_elem<T>(s + o);
#pragma unroll
      for (int k = 1; k < N; ++k) acc = acc + load_elem<T>(s + k * rank_stride + o);
      store_elem<T>(d + o, acc);
    }
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
  // The epoch load is issued here and read only after the first ticket has
  // come back, so the two round trips to memory overlap: at small messages
  // every workgroup's start is on the call's critical path.
  const uint64_t epoch_word = ld_relaxed(&a.ctrl[kCtrlEpoch]);
  const uint32_t Q = a.queues;
  const uint32_t S = a.qslots;
  const uint32_t q = uniform(blockIdx.x % Q);
  // local tiles of this queue: t = g * Q + q
  const uint32_t qtiles = uniform(a.tiles > q ? (a.tiles - q + Q - 1) / Q : 0u);
  const uint32_t L = uniform(a.lookahead < qtiles ? a.lookahead : qtiles);
  const uint32_t items = uniform((qtiles + L) * (uint32_t)(2 * N));
  uint64_t* ticket = &a.ctrl[kCtrlTicket + q * kFlagStride];
  if (threadIdx.x == 0)
    s_item = (uint32_t)__hip_atomic_fetch_add(ticket, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const uint64_t epoch = uniform64(epoch_word);
  uint32_t item = uniform(s_item);
  for (;;) {
    if (item >= items) break;
    const uint32_t g = uniform(item / (uint32_t)(2 * N));
    const uint32_t w = uniform(item - g * (uint32_t)(2 * N));
    if (w < (uint32_t)N) {
      if (g < qtiles) stage_item<T, N>(a, g * Q + q, uniform(q * S + g % S), uniform(g / S), w, epoch, &s_ok);
    } else if (g >= L) {
      const uint32_t gc = g - L;
      consume_item<T, N>(a, gc * Q + q, uniform(q * S + gc % S), uniform(gc / S), w - (uint32_t)N, epoch, &s_ok);
    }
    // The barrier before the next ticket closes the item's single-lane flag
    // store before the next single-lane ticket fetch; without it the
    // compiler may thread the two lane-0 regions into one back edge that
    // the other lanes skip, so that the lanes of a wave meet the barriers
    // on different iterations.  It also keeps s_item from being overwritten
    // before every wave has read it.
    __syncthreads();
    if (threadIdx.x == 0)
      s_item = (uint32_t)__hip_atomic_fetch_add(ticket, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    item = uniform(s_item);
  }
  // Completion, counted per queue first (each queue's workgroups hit their
  // own counter; a same-address atomic costs ~12 ns, so one global counter
  // would serialise the whole grid), then once per queue globally.  The last
  // workgroup of a queue resets that queue's counters; the last queue to
  // finish advances the epoch.
  if (threadIdx.x == 0) {
    const uint64_t per_queue = gridDim.x / Q;  // the grid is a multiple of Q
    uint64_t* qdone = &a.ctrl[kCtrlQDone + q * kFlagStride];
    // a release add (one write-back per workgroup; acquire-release added an
    // invalidate to every one of them, serialising GPU-wide), and one
    // acquire in the last workgroup before it resets the queue's counters
    const uint64_t oq = __hip_atomic_fetch_add(qdone, (uint64_t)1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    if (oq == per_queue - 1) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      __hip_atomic_store(ticket, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(qdone, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (Q == 1) {
        // the only queue: its last workgroup is the grid's last, and the
        // global count (one more round trip at the end of a small call)
        // is not needed
        __hip_atomic_store(&a.ctrl[kCtrlEpoch], epoch + a.rounds, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        const uint64_t old =
            __hip_atomic_fetch_add(&a.ctrl[kCtrlDone], (uint64_t)1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        if (old == (uint64_t)Q - 1) {
          __hip_atomic_store(&a.ctrl[kCtrlDone], (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(&a.ctrl[kCtrlEpoch], epoch + a.rounds, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  }
}

using PipeFn = void (*)(const PipeArgs);

// One workgroup per CU unless a rule or the tuning says otherwise: with
// about one producer item per workgroup, more workgroups only wait.
int pipe_wgs_per_cu(const LaunchCfg& cfg) { return cfg.wgs_per_cu > 0 ? cfg.wgs_per_cu : 1; }

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
  // The layout needs whole pieces per tile.  A unit is 4 pieces (16 KiB),
  // or fewer where they do not divide the tile; at 16 ranks one piece.
  // Measured on MI355X, bf16 64 MiB per rank: N = 6 and 8 ran fastest with
  // 16 KiB units (N=8: 283 us against 289 with 8 KiB and 297 with 4 KiB),
  // N = 12 alike within 2 %, N = 16 with 4 KiB units (554 us against 600
  // with 16 KiB and 625 with 8 KiB).
  if (a.tile_bytes == 0 || a.tile_bytes % kPiece) return hipErrorInvalidValue;
  uint32_t shift = a.nranks >= 16 ? 0u : 2u;
  while (shift > 0 && (a.tile_bytes / kPiece) % (1u << shift)) --shift;
  const uint64_t ub = (uint64_t)kPiece << shift;
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
  const int want = pipe_wgs_per_cu(cfg);
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
  const uint64_t nbytes = a.count * e;
  const uint64_t full = nbytes / ub;
  if ((full << shift) >= 0xffffffffull) return hipErrorInvalidValue;
  a.unit_shift = shift;
  a.unit_bytes = (uint32_t)ub;
  a.full_units = (uint32_t)full;
  a.tail_tile = (uint32_t)(full % tiles);
  a.tail_pieces = (uint32_t)(nbytes % ub / kPiece);
  a.last_bytes = (uint32_t)(nbytes % kPiece);
  if (grid_out) *grid_out = (uint32_t)grid;
  hipLaunchKernelGGL(fn, dim3((uint32_t)grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace snac
