// collectives.hip -- the single-kernel collectives launched from the host:
// one persistent grid per call runs the copy or N-to-1 reduce tile engine of
// snac_device.hpp over the job table of the collective's layout
// (snac_layout.hpp).  Reduces and one-to-one copies use 256-thread
// workgroups (4 units of 16 bytes per lane per 16 KiB tile); the small-tile
// reduce uses 128 threads, multicast copies single waves, and one-to-one
// copies that move at least 1 GiB single waves on 4 KiB tiles.
#include <hip/hip_runtime.h>

#include <atomic>

#include "internal.hpp"
#include "snac_device.hpp"

namespace snac {

constexpr int kCopyThreads = 256;

// Reduce workgroup sizes.  The 16 KiB-tile reduce runs a whole wave per
// SIMD (256 threads, one workgroup per CU): on MI355X that moved AllReduce
// 2-8 % faster than 128-thread workgroups at one or two per CU (N = 3..16,
// bf16 and f32; ReduceScatter even).  The small-tile form keeps 128 threads
// so that a small message still splits into 2 KiB tiles over many CUs.
constexpr int kReduceThreads = 256;
constexpr int kSmallReduceThreads = 128;

// N-to-1 reduce of element type T over N sources, the whole grid.  SMALL:
// the small-tile form (one 16-byte unit per lane, all sources in flight)
// for messages with fewer 16 KiB tiles than the GPU has CUs.  ROLL: tiles
// on the dword grid take the rolling load pipeline (the bf16 AllReduce of
// 8 ranks only).
template <int N, typename T, int CP, bool ALIGNED, bool SMALL = false, bool ROLL = false>
__global__ __launch_bounds__(SMALL ? kSmallReduceThreads : kReduceThreads) void reduce_kernel(const CollDesc d,
                                                                                            const PoolArg pa) {
  constexpr int TH = SMALL ? kSmallReduceThreads : kReduceThreads;
  constexpr uint32_t TILE = SMALL ? TH * 16u : kTileBytes;
  __shared__ __align__(16) char lds[engine_lds_bytes<TH, kMaxRanks>()];
  __shared__ unsigned long long xchg[2];
  const TilePool pool{(global_u64*)pa.next, (global_u64*)(pa.next + (uint64_t)pa.counters * kFlagStride), xchg,
                      pa.rounds, pa.counters};
  run_reduce<N, T, TH, CP, ALIGNED, TILE, ROLL>(d, blockIdx.x, gridDim.x, lds, pool);
}

// Byte copy of the collective's jobs, the whole grid.  TH = 256 for
// one-to-one copies; multicast copies (AllGather, AllGatherV: one read, N
// writes per unit) use single-wave workgroups, which on MI355X sustain
// about 6 % more write bandwidth than 256-thread ones.
constexpr int kMulticastThreads = 64;

template <int CP, bool ALIGNED, int TH, uint32_t TILE = kTileBytes>
__global__ __launch_bounds__(TH) void copy_kernel(const CollDesc d, const PoolArg pa) {
  __shared__ __align__(16) char lds[engine_lds_bytes<TH>()];
  __shared__ unsigned long long xchg[2];
  const TilePool pool{(global_u64*)pa.next, (global_u64*)(pa.next + (uint64_t)pa.counters * kFlagStride), xchg,
                      pa.rounds, pa.counters};
  run_copy<TH, CP, ALIGNED, TILE>(d, blockIdx.x, gridDim.x, lds, pool);
}

// One-to-one copies that move at least kStreamCopyBytes (read plus
// written): single-wave workgroups on 4 KiB tiles, five per CU.  Measured
// on three MI355X machines against 256-thread workgroups on 16 KiB tiles at
// two per CU: copy 1 GiB
// 6.29-6.34 against 5.95-6.02 TB/s, AllToAll u32 N=8 128 MiB per rank
// 5.96-5.97 against 5.58-5.69, AllToAllV with misaligned Dirichlet counts
// 5.74 against 5.61-5.63.  Below about 512 MiB moved the 16 KiB tiles are
// faster (copy 64 MiB: 6.05 against 5.75; AllToAll 16 MiB per rank: 5.85
// against 5.64).  Five per CU also beat four for jobs off the 16-byte grid
// (two machines, three alternations each: AllToAllV u32 N=8 with Dirichlet
// counts 0.362 against 0.373 ms, a 1 GiB copy from a source 4 bytes off
// 0.354 against 0.362).  Copies whose source sits at a byte offset from the
// destination's dword grid keep the 16 KiB tiles at every size: their full
// tiles funnel through DPP lane shifts (funnel_next), which single-wave
// 4 KiB tiles did not profit from.
constexpr int kStreamThreads = 64;
constexpr uint32_t kStreamTile = 4096;
constexpr uint64_t kStreamCopyBytes = 1ull << 30;

SNAC_HD bool is_multicast_copy(const CollDesc& d) {
  return (d.coll == kAllGather || d.coll == kAllGatherV) && !d.split_multicast;
}

// ------------------------------------------------------------- launchers

using KernelFn = void (*)(const CollDesc, const PoolArg);

template <int N, typename T, int CP, bool A, bool SMALL>
KernelFn kernel_ptr() {
  return &reduce_kernel<N, T, CP, A, SMALL>;
}

template <typename T, int CP, bool A, bool SMALL = false>
KernelFn reduce_kernel_n(int n) {
  switch (n) {
    case 1: return kernel_ptr<1, T, CP, A, SMALL>();
    case 2: return kernel_ptr<2, T, CP, A, SMALL>();
    case 3: return kernel_ptr<3, T, CP, A, SMALL>();
    case 4: return kernel_ptr<4, T, CP, A, SMALL>();
    case 5: return kernel_ptr<5, T, CP, A, SMALL>();
    case 6: return kernel_ptr<6, T, CP, A, SMALL>();
    case 7: return kernel_ptr<7, T, CP, A, SMALL>();
    case 8: return kernel_ptr<8, T, CP, A, SMALL>();
    case 9: return kernel_ptr<9, T, CP, A, SMALL>();
    case 10: return kernel_ptr<10, T, CP, A, SMALL>();
    case 11: return kernel_ptr<11, T, CP, A, SMALL>();
    case 12: return kernel_ptr<12, T, CP, A, SMALL>();
    case 13: return kernel_ptr<13, T, CP, A, SMALL>();
    case 14: return kernel_ptr<14, T, CP, A, SMALL>();
    case 15: return kernel_ptr<15, T, CP, A, SMALL>();
    case 16: return kernel_ptr<16, T, CP, A, SMALL>();
    default: return nullptr;
  }
}

// The bf16 AllReduce of 8 ranks, every destination written by each tile.
static KernelFn rolling_reduce_kernel_cp(int cp, bool aligned) {
  if (!aligned)
    return cp == kCached ? &reduce_kernel<8, BF16, kCached, false, false, true>
                         : &reduce_kernel<8, BF16, kCacheStream, false, false, true>;
  switch (cp) {
    case kCacheStream: return &reduce_kernel<8, BF16, kCacheStream, true, false, true>;
    case kCacheStreamStores: return &reduce_kernel<8, BF16, kCacheStreamStores, true, false, true>;
    case kCacheStreamLoads: return &reduce_kernel<8, BF16, kCacheStreamLoads, true, false, true>;
    default: return &reduce_kernel<8, BF16, kCached, true, false, true>;
  }
}

template <typename T>
KernelFn reduce_kernel_cp(int n, int cp, bool aligned) {
  if (!aligned) return cp == kCached ? reduce_kernel_n<T, kCached, false>(n) : reduce_kernel_n<T, kCacheStream, false>(n);
  switch (cp) {
    case kCacheStream: return reduce_kernel_n<T, kCacheStream, true>(n);
    case kCacheStreamStores: return reduce_kernel_n<T, kCacheStreamStores, true>(n);
    case kCacheStreamLoads: return reduce_kernel_n<T, kCacheStreamLoads, true>(n);
    default: return reduce_kernel_n<T, kCached, true>(n);
  }
}

template <int TH, uint32_t TILE = kTileBytes>
static KernelFn copy_kernel_cp(int cp, bool aligned) {
  if (!aligned) {
    if (cp == kCached) return &copy_kernel<kCached, false, TH, TILE>;
    if (cp == kCacheStreamStores) return &copy_kernel<kCacheStreamStores, false, TH, TILE>;
    return &copy_kernel<kCacheStream, false, TH, TILE>;
  }
  switch (cp) {
    case kCacheStream: return &copy_kernel<kCacheStream, true, TH, TILE>;
    case kCacheStreamStores: return &copy_kernel<kCacheStreamStores, true, TH, TILE>;
    case kCacheStreamLoads: return &copy_kernel<kCacheStreamLoads, true, TH, TILE>;
    default: return &copy_kernel<kCached, true, TH, TILE>;
  }
}

static int coll_threads(const CollDesc& d, int shape) {
  if (coll_is_reduce(d.coll)) return shape == kShapeSmall ? kSmallReduceThreads : kReduceThreads;
  if (shape == kShapeStream) return kStreamThreads;
  return is_multicast_copy(d) ? kMulticastThreads : kCopyThreads;
}

uint32_t coll_tile_bytes(const CollDesc& d, int shape) {
  if (shape == kShapeSmall) return (uint32_t)coll_threads(d, shape) * 16u;
  return shape == kShapeStream ? kStreamTile : kTileBytes;
}

int large_shape(const CollDesc& d, uint64_t job_bytes, bool byte_shift) {
  if (coll_is_reduce(d.coll) || is_multicast_copy(d) || byte_shift) return kShapeTile;
  return 2 * job_bytes >= kStreamCopyBytes ? kShapeStream : kShapeTile;
}

// CU count of the current device, cached per device.  Several host threads
// may launch at once (different contexts), so the cache is a table of
// atomics: a thread that finds no entry queries the device and stores it;
// two threads doing so at once store the same value.
constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < kMaxDevices) {
    const int c = g_cu_count[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < kMaxDevices) g_cu_count[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// Small-tile kernels: streaming accesses (the cache policy does not matter
// for a message this small), aligned or generic.
static KernelFn small_kernel(const CollDesc& d, bool aligned) {
  if (coll_is_reduce(d.coll)) {
    if (d.esize == 4)
      return aligned ? reduce_kernel_n<F32, kCacheStream, true, true>(d.nsrc)
                     : reduce_kernel_n<F32, kCacheStream, false, true>(d.nsrc);
    return aligned ? reduce_kernel_n<BF16, kCacheStream, true, true>(d.nsrc)
                   : reduce_kernel_n<BF16, kCacheStream, false, true>(d.nsrc);
  }
  if (is_multicast_copy(d))
    return aligned ? &copy_kernel<kCacheStream, true, kMulticastThreads, kMulticastThreads * 16u>
                   : &copy_kernel<kCacheStream, false, kMulticastThreads, kMulticastThreads * 16u>;
  return aligned ? &copy_kernel<kCacheStream, true, kCopyThreads, kCopyThreads * 16u>
                 : &copy_kernel<kCacheStream, false, kCopyThreads, kCopyThreads * 16u>;
}

// Workgroups per CU when neither a rule nor the process-wide tuning names
// one.  Measured on MI355X: the 1:1 read/write streams of 16 KiB tiles run
// fastest with few workgroups per CU (more concurrent write streams lower
// HBM efficiency): one for reduces of three or more sources, two otherwise.
// A small message instead wants its tiles spread wide, about one per
// workgroup: four per CU for reduces and multicast copies (AllReduce
// bf16 N=8 at 2 MiB per rank 10 % faster than at one per CU, AllGather at
// 256 KiB per rank in 28 % faster than at two), two for other copies,
// whose workgroups each rebuild a larger job table.  One-to-one copies
// with at most 8 tiles per CU (up to 32 MiB moved at 256 CUs) are latency
// bound rather than stream bound, and four per CU finish them sooner:
// AllToAll u32 N=8 at 1.5, 2 and 4 MiB per rank took 9.8, 11.8 and 18.0 us
// against 13.0, 13.9 and 19.6 at two (single calls, inputs evicted), and
// 7.1, 8.8 and 14.8 against 9.2, 11.2 and 16.2 us in graph replays; a
// 16 MiB copy 4-6 % less.  From 6 MiB per rank up two per CU is faster.
// Reduces of at most 2 tiles per CU (AllReduce and ReduceScatter of 4-8 MiB
// per rank) likewise run two per CU, one tile each: bf16 N=8 AllReduce at
// 6 and 8 MiB per rank 18.7 and 21.9 us against 20.1 and 23.3 in graph
// replays, ReduceScatter at 5-8 MiB per rank 4-7 % less.
static int default_wgs_per_cu(const CollDesc& d, int shape, uint64_t tiles, int cus) {
  const bool reduce = coll_is_reduce(d.coll);
  if (shape == kShapeSmall) return reduce || is_multicast_copy(d) ? 4 : 2;
  if (shape == kShapeStream) return 5;
  if (reduce) return d.nsrc >= 3 && tiles > 2u * (uint64_t)(cus > 0 ? cus : 1) ? 1 : 2;
  return !is_multicast_copy(d) && tiles <= 8u * (uint64_t)(cus > 0 ? cus : 1) ? 4 : 2;
}

// Tile counters serve launches in the 16 KiB-tile shape with at least
// kPoolMinRounds tiles per workgroup.  The first kPoolGridRounds rounds are
// grid-stride, since every workgroup starting on the counters at once only
// queues on them; the rest of the tiles are handed out in order.  One
// address takes about 84 M atomic adds per second on MI355X, and a counter
// serves fastest at about a quarter of that, so a launch takes one counter
// per 16 streams of 16 KiB its tiles move (sources read plus destinations
// written), at most kPoolMaxUse.  Measured, one machine, two alternations, ms:
//   AllReduce bf16 N=8 256 MiB (16 streams): 1 counter 0.718, 2 0.719,
//     4 0.721, grid-stride 0.758-0.763;
//   ReduceScatter bf16 N=8 (9 streams): 1 0.181, 2 0.180, 4 0.181, 8 0.183,
//     grid-stride 0.194-0.195;  AllGather bf16 N=8 (9): 1 0.169, 2 0.167,
//     4 0.167-0.168, grid-stride 0.174;
//   AllToAll u32 N=8 128 MiB (2 streams, on 16 KiB tiles): 1 0.786, 2 0.426,
//     4 0.332, 8 0.335, against 0.360 for grid-stride 4 KiB tiles.
constexpr uint64_t kPoolMinRounds = 16;
constexpr uint32_t kPoolGridRounds = 8;
constexpr uint32_t kPoolMaxUse = 4;
static_assert(kPoolMaxUse <= kPoolMaxCounters, "a slot holds the counters a launch uses");

// 16 KiB streams one tile of this descriptor's kernel moves.
static int tile_streams(const CollDesc& d) {
  if (coll_is_reduce(d.coll)) return d.nsrc + (d.coll == kAllReduce && !d.split_multicast ? d.ndst : 1);
  return is_multicast_copy(d) ? 1 + d.ndst : 2;
}

hipError_t launch_collective(const CollDesc& d, bool aligned, int shape, uint64_t tiles, const LaunchCfg& cfg,
                             hipStream_t stream, unsigned long long* pool) {
  if (tiles == 0) return hipSuccess;
  KernelFn fn = nullptr;
  // tuning value 0 = library default (streaming loads and stores), 4 = cached
  const int cp = cfg.cache_policy == 0 ? kCacheStream : (cfg.cache_policy == 4 ? kCached : cfg.cache_policy);
  const bool reduce = coll_is_reduce(d.coll);
  if (reduce && num_jobs(d) > kMaxRanks) return hipErrorInvalidValue;
  if (shape == kShapeSmall) {
    fn = small_kernel(d, aligned);
  } else if (reduce) {
    if (shape != kShapeTile) return hipErrorInvalidValue;
    if (d.esize == 2 && d.nsrc == 8 && d.coll == kAllReduce && !d.split_multicast && d.ndst == 8)
      fn = rolling_reduce_kernel_cp(cp, aligned);
    else
      fn = d.esize == 4 ? reduce_kernel_cp<F32>(d.nsrc, cp, aligned) : reduce_kernel_cp<BF16>(d.nsrc, cp, aligned);
  } else if (shape == kShapeStream) {
    if (is_multicast_copy(d)) return hipErrorInvalidValue;
    fn = copy_kernel_cp<kStreamThreads, kStreamTile>(cp, aligned);
  } else {
    fn = is_multicast_copy(d) ? copy_kernel_cp<kMulticastThreads>(cp, aligned) : copy_kernel_cp<kCopyThreads>(cp, aligned);
  }
  if (!fn) return hipErrorInvalidValue;
  const int threads = coll_threads(d, shape);
  int per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(fn), threads, 0);
  if (e != hipSuccess) return e;
  if (per_cu < 1) per_cu = 1;
  const int cus = device_cu_count();
  const int want = cfg.wgs_per_cu > 0 ? cfg.wgs_per_cu : default_wgs_per_cu(d, shape, tiles, cus);
  if (want < per_cu) per_cu = want;
  uint64_t grid = (uint64_t)(cus > 0 ? cus : 1) * (uint64_t)per_cu;
  if (grid > tiles) grid = tiles;
  PoolArg pa{nullptr, 0, 1};
  const uint64_t rounds = tiles / grid;
  if (pool && shape == kShapeTile && (cfg.tile_schedule == 2 || (cfg.tile_schedule == 0 && rounds >= kPoolMinRounds))) {
    pa.next = pool;
    pa.rounds = rounds >= 2 * kPoolGridRounds ? kPoolGridRounds : (uint32_t)(rounds > 2 ? rounds / 2 : 1);
    const int streams = tile_streams(d);
    uint32_t cnt = (uint32_t)((16 + streams - 1) / streams);
    if (cnt > kPoolMaxUse) cnt = kPoolMaxUse;
    const uint64_t groups = (grid + 7) / 8;  // every counter needs a workgroup: (block / 8) % counters
    if (cnt > groups) cnt = (uint32_t)groups;
    pa.counters = cnt;
  }
  hipLaunchKernelGGL(fn, dim3((uint32_t)grid), dim3(threads), 0, stream, d, pa);
  return hipGetLastError();
}

// -------------------------------------------- non-deterministic AllReduce
//
// Each (tile, source rank) item adds its 16 KiB of the source into a
// binary32 accumulator with hardware float atomics (global_atomic_add_f32),
// as Iris's all_reduce_atomic adds every rank's tile into the destination;
// the N items of a tile run on different workgroups, so the order of the
// adds -- and the last bits of the sum -- depend on timing.  A second
// kernel rounds the accumulator once into every destination.

constexpr int kAtomicThreads = 256;
constexpr int kAtomicUnits = 4;  // 16-byte units per lane per item

// The accumulator is kept lane-major within each group of 64 units: element
// j of unit l of a group (L elements per unit) sits at word j * 64 + l, so
// the j-th atomic of a wave covers 64 consecutive words -- two 128-byte
// lines -- instead of 64 words 32 or 16 bytes apart.  Only the two kernels
// below see this layout.
template <uint32_t L>
__device__ __forceinline__ uint64_t acc_index(uint64_t e) {
  const uint64_t g = e / (64u * L);
  const uint32_t r = (uint32_t)(e - g * 64u * L);
  return g * 64u * L + (uint64_t)(r % L) * 64u + r / L;
}

template <typename T, bool VEC>
__global__ __launch_bounds__(kAtomicThreads) void atomic_accumulate_kernel(const CollDesc d, float* acc,
                                                                           uint64_t first, uint64_t elems,
                                                                           uint64_t items) {
  constexpr uint32_t E = T::kSize;
  constexpr uint32_t L = 16 / E;  // elements per 16-byte unit
  constexpr uint64_t TILE_E = (uint64_t)kAtomicThreads * kAtomicUnits * L;
  const uint64_t n = (uint64_t)d.nsrc;
  for (uint64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const uint64_t t = it / n;
    const int k = (int)(it - t * n);
    const char* src = static_cast<const char*>(d.src[k]) + first * E;
#pragma unroll
    for (int u = 0; u < kAtomicUnits; ++u) {
      const uint64_t e0 = t * TILE_E + ((uint64_t)u * kAtomicThreads + threadIdx.x) * L;
      if (VEC && e0 + L <= elems) {
        UnitAcc<T> v;
        v.set(ld16<kCacheStream>(src + e0 * E));
        float* a = acc + acc_index<L>(e0);
#pragma unroll
        for (uint32_t j = 0; j < L; ++j)
          __hip_atomic_fetch_add(a + j * 64u, v.a[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        for (uint32_t j = 0; j < L && e0 + j < elems; ++j)
          __hip_atomic_fetch_add(acc + acc_index<L>(e0 + j), load_elem<T>(src + (e0 + j) * E), __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

// dst[d][first + e] = R(acc[e]) for every destination.
template <typename T, bool VEC>
__global__ __launch_bounds__(kAtomicThreads) void atomic_finish_kernel(const CollDesc d, const float* acc,
                                                                       uint64_t first, uint64_t elems) {
  constexpr uint32_t E = T::kSize;
  constexpr uint32_t L = 16 / E;
  const uint64_t stride = (uint64_t)gridDim.x * kAtomicThreads * L;
  for (uint64_t e0 = ((uint64_t)blockIdx.x * kAtomicThreads + threadIdx.x) * L; e0 < elems; e0 += stride) {
    if (VEC && e0 + L <= elems) {
      UnitAcc<T> v;
      const float* a = acc + acc_index<L>(e0);
#pragma unroll
      for (uint32_t j = 0; j < L; ++j) v.a[j] = a[j * 64u];
      const u32x4 w = v.out();
      for (int k = 0; k < d.ndst; ++k) st16<kCacheStream>(static_cast<char*>(d.dst[k]) + (first + e0) * E, w);
    } else {
      for (uint32_t j = 0; j < L && e0 + j < elems; ++j) {
        const float x = acc[acc_index<L>(e0 + j)];
        for (int k = 0; k < d.ndst; ++k) store_elem<T>(static_cast<char*>(d.dst[k]) + (first + e0 + j) * E, x);
      }
    }
  }
}

uint64_t atomic_chunk_elems(int esize) {
  const uint64_t tile_e = (uint64_t)kAtomicThreads * kAtomicUnits * (16u / (uint32_t)esize);
  return tile_e;  // chunks are whole tiles
}

hipError_t launch_atomic_allreduce(const CollDesc& d, float* acc, uint64_t first, uint64_t elems, bool vec,
                                   hipStream_t stream) {
  if (elems == 0) return hipSuccess;
  const uint64_t tile_e = atomic_chunk_elems(d.esize);
  const uint64_t items = (elems + tile_e - 1) / tile_e * (uint64_t)d.nsrc;
  const int cus = device_cu_count();
  uint64_t grid = (uint64_t)(cus > 0 ? cus : 1) * 4;
  if (grid > items) grid = items;
  // the accumulator's words of a partial last group lie past elems: clear
  // whole groups (the chunk capacity is whole tiles, so they fit)
  const uint64_t group_e = 64u * (16u / (uint64_t)d.esize);
  const uint64_t acc_words = (elems + group_e - 1) / group_e * group_e;
  hipError_t e = fill_u64(reinterpret_cast<uint64_t*>(acc), acc_words / 2, 0, stream);
  if (e != hipSuccess) return e;
  const bool bf = d.esize == 2;
  if (bf) {
    if (vec)
      hipLaunchKernelGGL((atomic_accumulate_kernel<BF16, true>), dim3((uint32_t)grid), dim3(kAtomicThreads), 0, stream, d,
                         acc, first, elems, items);
    else
      hipLaunchKernelGGL((atomic_accumulate_kernel<BF16, false>), dim3((uint32_t)grid), dim3(kAtomicThreads), 0, stream, d,
                         acc, first, elems, items);
  } else {
    if (vec)
      hipLaunchKernelGGL((atomic_accumulate_kernel<F32, true>), dim3((uint32_t)grid), dim3(kAtomicThreads), 0, stream, d,
                         acc, first, elems, items);
    else
      hipLaunchKernelGGL((atomic_accumulate_kernel<F32, false>), dim3((uint32_t)grid), dim3(kAtomicThreads), 0, stream, d,
                         acc, first, elems, items);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const uint64_t units = (elems + (16u / d.esize) - 1) / (16u / d.esize);
  uint64_t fgrid = (units + kAtomicThreads - 1) / kAtomicThreads;
  if (fgrid > (uint64_t)(cus > 0 ? cus : 1) * 4) fgrid = (uint64_t)(cus > 0 ? cus : 1) * 4;
  if (bf) {
    if (vec)
      hipLaunchKernelGGL((atomic_finish_kernel<BF16, true>), dim3((uint32_t)fgrid), dim3(kAtomicThreads), 0, stream, d, acc,
                         first, elems);
    else
      hipLaunchKernelGGL((atomic_finish_kernel<BF16, false>), dim3((uint32_t)fgrid), dim3(kAtomicThreads), 0, stream, d, acc,
                         first, elems);
  } else {
    if (vec)
      hipLaunchKernelGGL((atomic_finish_kernel<F32, true>), dim3((uint32_t)fgrid), dim3(kAtomicThreads), 0, stream, d, acc,
                         first, elems);
    else
      hipLaunchKernelGGL((atomic_finish_kernel<F32, false>), dim3((uint32_t)fgrid), dim3(kAtomicThreads), 0, stream, d, acc,
                         first, elems);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------ fill

__global__ void fill_u64_kernel(uint64_t* p, uint64_t n, uint64_t v) {
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (uint64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

hipError_t fill_u64(uint64_t* p, uint64_t n, uint64_t v, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  uint64_t blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(fill_u64_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream, p, n, v);
  return hipGetLastError();
}

}  // namespace snac
