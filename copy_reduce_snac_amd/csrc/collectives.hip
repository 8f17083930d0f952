// collectives.hip -- the single-kernel collectives: one persistent grid per
// call runs the copy or N-to-1 reduce Atom over the job table of the
// collective's layout.
//
// Every workgroup rebuilds the job table in LDS from the kernel argument
// (layout.hpp), numbers the tiles of all jobs with an exclusive scan, and
// walks tiles blockIdx.x, blockIdx.x + gridDim.x, ...  A tile is
// TH * 16 * U bytes of each source; each lane moves U 16-byte units.
//
//  * copy (256 threads, U = 4): the U loads of a tile, then its stores to one
//    destination or to all of them (a multicast: one read, N writes).
//  * reduce (128 threads, U = 8, 16 KiB per source): the sources are taken
//    one at a time -- source k + 1's U loads are in flight while source k is
//    added into binary32 accumulators -- and the finished tile is stored to
//    each destination as one contiguous 16 KiB run.  Holding accumulators
//    rather than all N sources keeps the register footprint independent of
//    N, and a workgroup writes one destination at a time; on MI355X this
//    beat loading all N sources at once and storing every destination per
//    unit by 3-6 %.
//
// Two variants per Atom:
//  * aligned: every job address is 16-byte aligned and every job length a
//    multiple of 16 (the normal case for tensor buffers): plain dwordx4.
//  * generic: any element-aligned address.  Each job is split into a head
//    (bytes until the destination reaches a 128-byte line), a body of aligned
//    16-byte stores whose sources are read with ld16_any, and a tail; head
//    and tail are moved one element per lane by tile 0 of the job.  The
//    generic variant exists with streaming (default) and cached accesses.
#include <hip/hip_runtime.h>

#include "atoms.hpp"
#include "internal.hpp"
#include "layout.hpp"

namespace snac {

struct JobL {
  uint64_t src_off;
  uint64_t dst_off;
  uint64_t bytes;
  int32_t src_rank;
  int32_t dst_rank;
  uint32_t head;
  uint32_t tile0;
};

constexpr int kCopyThreads = kThreads;
constexpr int kCopyUnroll = 4;
constexpr int kReduceThreads = 128;
constexpr int kReduceUnroll = 8;
// reduce collectives have at most kMaxRanks jobs (one per destination)
static_assert(kMaxRanks <= kReduceThreads, "job scan needs a thread per job");
// head (< 128 bytes) plus tail (< 16 bytes) edge elements, one per lane
static_assert(kHeadAlign / 2 + 16 / 2 <= kReduceThreads, "edge elements need a lane each");

template <int TH, int U>
constexpr uint32_t tile_of() {
  return (uint32_t)TH * 16u * (uint32_t)U;
}

// Build the job table and its tile numbering in LDS.  Returns the total
// number of tiles; every thread of the workgroup must call it.
template <int TH, bool ALIGNED>
__device__ uint32_t build_table(const CollDesc& d, uint32_t tile_bytes, JobL* jobs, uint32_t* scan, int& nj) {
  nj = num_jobs(d);
  const int t = threadIdx.x;
  uint32_t tiles = 0;
  if (t < nj) {
    const Job j = make_job(d, t);
    const uint32_t head = ALIGNED ? 0u : job_head_bytes(d, j);
    tiles = (uint32_t)job_tiles(j, head, tile_bytes);
    jobs[t] = JobL{j.src_off, j.dst_off, j.bytes, j.src_rank, j.dst_rank, head, 0u};
  }
  if (nj == 1) {
    if (t == 0) scan[0] = tiles;
    __syncthreads();
    return scan[0];
  }
  scan[t] = tiles;
  __syncthreads();
#pragma unroll
  for (int off = 1; off < TH; off <<= 1) {
    const uint32_t v = t >= off ? scan[t - off] : 0u;
    __syncthreads();
    scan[t] += v;
    __syncthreads();
  }
  if (t < nj) jobs[t].tile0 = scan[t] - tiles;
  const uint32_t total = scan[TH - 1];
  __syncthreads();
  return total;
}

// Store U units (unit u at lane + u * TH * 16 bytes past base, if below
// rem) to one destination or, for a multicast, to every destination in
// turn.  NU > 0 unrolls the multicast for the common case ndst == NU.
template <int TH, int U, int CP, bool ALIGNED>
__device__ __forceinline__ void store_one(char* p, uint32_t lane, uint32_t rem, const u32x4 (&v)[U]) {
  if constexpr (ALIGNED) {  // units at or past rem fall outside the resource
    const __amdgpu_buffer_rsrc_t r = buffer_rsrc(p, rem);
#pragma unroll
    for (int u = 0; u < U; ++u) bst16<CP>(r, lane + (uint32_t)u * TH * 16u, v[u]);
    return;
  }
  if (rem == tile_of<TH, U>()) {  // full tile: no per-unit guards
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
    next_tile0 = j + 1 < nj ? uniform(jobs[j + 1].tile0) : 0xffffffffu;
  }

  __device__ __forceinline__ void init(const JobL* t, int n, uint32_t tile) {
    jobs = t;
    nj = n;
    j = 0;
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
    r.toff = (uint64_t)r.head + (uint64_t)r.lt * TILE;
    const uint64_t end = (uint64_t)r.head + r.body;
    const uint64_t left = end > r.toff ? end - r.toff : 0;
    r.rem = left > TILE ? TILE : (uint32_t)left;
    return r;
  }
};

// ---------------------------------------------------------------- reduce

template <typename T, int N>
__device__ void reduce_edges(const CollDesc& d, const JobL& J, uint32_t head, uint64_t body) {
  constexpr uint32_t E = T::kSize;
  const uint32_t nh = head / E;
  const uint32_t nt = (uint32_t)(J.bytes - head - body) / E;
  const uint32_t t = threadIdx.x;
  if (t >= nh + nt) return;
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

// Issue the U loads of source k of one tile.  FULL: the tile holds U whole
// units per lane; otherwise units past the tile's body are left zero (and
// are never stored).
template <int TH, int U, int CP, bool ALIGNED, bool FULL>
__device__ __forceinline__ void reduce_load(const CollDesc& d, const TileRef& t, int k, u32x4 (&v)[U]) {
  const uint32_t lane = threadIdx.x * 16u;
  const char* sp = static_cast<const char*>(d.src[k]) + t.J.src_off + t.toff;
  if constexpr (ALIGNED) {  // units at or past rem read as zero
    const __amdgpu_buffer_rsrc_t r = buffer_rsrc(sp, t.rem);
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = bld16<CP>(r, lane + (uint32_t)u * TH * 16u);
    return;
  }
  const uint32_t m = ALIGNED ? 0u : uniform((uint32_t)(uintptr_t)sp & 3u);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t o = lane + (uint32_t)u * TH * 16u;
    if constexpr (FULL) {
      v[u] = ALIGNED ? ld16<CP>(sp + o) : ld16_any<CP>(sp + o, m);
    } else {
      v[u] = u32x4{0u, 0u, 0u, 0u};
      if (o < t.rem) v[u] = ALIGNED ? ld16<CP>(sp + o) : ld16_any<CP>(sp + o, m);
    }
  }
}

// The reduced units of one tile, sources added in rank order.  Two register
// buffers alternate: while source k is added from one, source k + 1 loads
// into the other.  The source loop is deliberately not unrolled: unrolled,
// the compiler issues every source's loads before the first add, which
// measured about 5 % slower on MI355X than keeping two sources in flight.
template <int N, typename T, int TH, int U, int CP, bool ALIGNED, bool FULL>
__device__ __forceinline__ void reduce_tile(const CollDesc& d, const TileRef& t, u32x4 (&r)[U]) {
  u32x4 a[U], b[U];
  UnitAcc<T> acc[U];
  reduce_load<TH, U, CP, ALIGNED, FULL>(d, t, 0, a);
  if constexpr (N > 1) reduce_load<TH, U, CP, ALIGNED, FULL>(d, t, 1, b);
#pragma unroll
  for (int u = 0; u < U; ++u) acc[u].set(a[u]);
  int k = 1;  // next source to add; it is in b
#pragma unroll 1
  for (; k + 1 < N; k += 2) {
    reduce_load<TH, U, CP, ALIGNED, FULL>(d, t, k + 1, a);
    __builtin_amdgcn_sched_barrier(0);  // issue these loads before waiting on b
#pragma unroll
    for (int u = 0; u < U; ++u) acc[u].add(b[u]);
    if (k + 2 < N) reduce_load<TH, U, CP, ALIGNED, FULL>(d, t, k + 2, b);
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

// ------------------------------------------------------------------ copy

__device__ void copy_edges(const CollDesc& d, const JobL& J, uint32_t head, uint64_t body) {
  const uint32_t nt = (uint32_t)(J.bytes - head - body);
  const uint32_t t = threadIdx.x;
  if (t >= head + nt) return;
  const uint64_t off = t < head ? (uint64_t)t : (uint64_t)head + body + (t - head);
  const uint8_t b = *(static_cast<const uint8_t*>(d.src[J.src_rank]) + J.src_off + off);
  if (J.dst_rank >= 0) {
    *(static_cast<uint8_t*>(d.dst[J.dst_rank]) + J.dst_off + off) = b;
  } else {
    for (int k = 0; k < d.ndst; ++k) *(static_cast<uint8_t*>(d.dst[k]) + J.dst_off + off) = b;
  }
}

template <int TH, int U, int CP, bool ALIGNED>
__device__ __forceinline__ void copy_load(const CollDesc& d, const TileRef& t, u32x4 (&v)[U]) {
  const char* sp = static_cast<const char*>(d.src[t.J.src_rank]) + t.J.src_off + t.toff;
  const uint32_t lane = threadIdx.x * 16u;
  if constexpr (ALIGNED) {  // units at or past rem read as zero (never stored)
    const __amdgpu_buffer_rsrc_t r = buffer_rsrc(sp, t.rem);
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = bld16<CP>(r, lane + (uint32_t)u * TH * 16u);
    return;
  }
  const uint32_t m = ALIGNED ? 0u : uniform((uint32_t)(uintptr_t)sp & 3u);
  if (t.rem == tile_of<TH, U>()) {  // full tile: no per-unit guards
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const char* q = sp + lane + (uint32_t)u * TH * 16u;
      v[u] = ALIGNED ? ld16<CP>(q) : ld16_any<CP>(q, m);
    }
    return;
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t o = lane + (uint32_t)u * TH * 16u;
    if (o < t.rem) v[u] = ALIGNED ? ld16<CP>(sp + o) : ld16_any<CP>(sp + o, m);
  }
}

// ---------------------------------------------------------------- kernels

// N-to-1 reduce of element type T over N sources.
template <int N, typename T, int CP, bool ALIGNED>
__global__ __launch_bounds__(kReduceThreads) void reduce_kernel(const CollDesc d) {
  constexpr int TH = kReduceThreads;
  constexpr int U = kReduceUnroll;
  constexpr uint32_t TILE = tile_of<TH, U>();
  __shared__ JobL jobs[kMaxRanks];
  __shared__ uint32_t scan[TH];
  int nj;
  const uint32_t total = build_table<TH, ALIGNED>(d, TILE, jobs, scan, nj);
  uint32_t tile = blockIdx.x;
  if (tile >= total) return;
  const uint32_t lane = threadIdx.x * 16u;
  JobCursor<TILE, ALIGNED> jc;
  jc.init(jobs, nj, tile);
  for (; tile < total; tile += gridDim.x) {
    const TileRef t = jc.at(tile);
    u32x4 r[U];
    if (ALIGNED || t.rem == TILE)
      reduce_tile<N, T, TH, U, CP, ALIGNED, true>(d, t, r);
    else
      reduce_tile<N, T, TH, U, CP, ALIGNED, false>(d, t, r);
    if constexpr (!ALIGNED) {
      if (t.lt == 0) reduce_edges<T, N>(d, t.J, t.head, t.body);
    }
    store_units<TH, U, CP, N, ALIGNED>(d, t.J.dst_rank, t.J.dst_off + t.toff, lane, t.rem, r);
  }
}

// Byte copy of the collective's jobs.
template <int CP, bool ALIGNED>
__global__ __launch_bounds__(kCopyThreads) void copy_kernel(const CollDesc d) {
  constexpr int TH = kCopyThreads;
  constexpr int U = kCopyUnroll;
  constexpr uint32_t TILE = tile_of<TH, U>();
  __shared__ JobL jobs[kMaxJobs];
  __shared__ uint32_t scan[TH];
  static_assert(kMaxJobs <= TH, "job scan needs a thread per job");
  int nj;
  const uint32_t total = build_table<TH, ALIGNED>(d, TILE, jobs, scan, nj);
  uint32_t tile = blockIdx.x;
  if (tile >= total) return;
  const uint32_t lane = threadIdx.x * 16u;
  JobCursor<TILE, ALIGNED> jc;
  jc.init(jobs, nj, tile);
  for (; tile < total; tile += gridDim.x) {
    const TileRef cur = jc.at(tile);
    u32x4 v[U];
    copy_load<TH, U, CP, ALIGNED>(d, cur, v);
    if constexpr (!ALIGNED) {
      if (cur.lt == 0) copy_edges(d, cur.J, cur.head, cur.body);
    }
    store_units<TH, U, CP, 0, ALIGNED>(d, cur.J.dst_rank, cur.J.dst_off + cur.toff, lane, cur.rem, v);
  }
}

// ------------------------------------------------------------- launchers

using KernelFn = void (*)(const CollDesc);

template <int N, typename T, int CP, bool A>
KernelFn kernel_ptr() {
  return &reduce_kernel<N, T, CP, A>;
}

template <typename T, int CP, bool A>
KernelFn reduce_kernel_n(int n) {
  switch (n) {
    case 1: return kernel_ptr<1, T, CP, A>();
    case 2: return kernel_ptr<2, T, CP, A>();
    case 3: return kernel_ptr<3, T, CP, A>();
    case 4: return kernel_ptr<4, T, CP, A>();
    case 5: return kernel_ptr<5, T, CP, A>();
    case 6: return kernel_ptr<6, T, CP, A>();
    case 7: return kernel_ptr<7, T, CP, A>();
    case 8: return kernel_ptr<8, T, CP, A>();
    case 9: return kernel_ptr<9, T, CP, A>();
    case 10: return kernel_ptr<10, T, CP, A>();
    case 11: return kernel_ptr<11, T, CP, A>();
    case 12: return kernel_ptr<12, T, CP, A>();
    case 13: return kernel_ptr<13, T, CP, A>();
    case 14: return kernel_ptr<14, T, CP, A>();
    case 15: return kernel_ptr<15, T, CP, A>();
    case 16: return kernel_ptr<16, T, CP, A>();
    default: return nullptr;
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

static KernelFn copy_kernel_cp(int cp, bool aligned) {
  if (!aligned) return cp == kCached ? &copy_kernel<kCached, false> : &copy_kernel<kCacheStream, false>;
  switch (cp) {
    case kCacheStream: return &copy_kernel<kCacheStream, true>;
    case kCacheStreamStores: return &copy_kernel<kCacheStreamStores, true>;
    case kCacheStreamLoads: return &copy_kernel<kCacheStreamLoads, true>;
    default: return &copy_kernel<kCached, true>;
  }
}

uint32_t coll_tile_bytes(const CollDesc& d, bool aligned) {
  (void)aligned;
  return coll_is_reduce(d.coll) ? tile_of<kReduceThreads, kReduceUnroll>() : tile_of<kCopyThreads, kCopyUnroll>();
}

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  static int cached_dev = -1;
  static int cached_cus = 0;
  if (dev != cached_dev) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cached_dev = dev;
    cached_cus = cus;
  }
  return cached_cus;
}

hipError_t launch_collective(const CollDesc& d, bool aligned, uint64_t tiles, const LaunchCfg& cfg,
                             hipStream_t stream) {
  if (tiles == 0) return hipSuccess;
  KernelFn fn = nullptr;
  // tuning value 0 = library default (streaming loads and stores), 4 = cached
  const int cp = cfg.cache_policy == 0 ? kCacheStream : (cfg.cache_policy == 4 ? kCached : cfg.cache_policy);
  const bool reduce = coll_is_reduce(d.coll);
  if (reduce) {
    if (num_jobs(d) > kMaxRanks) return hipErrorInvalidValue;
    fn = d.esize == 4 ? reduce_kernel_cp<F32>(d.nsrc, cp, aligned) : reduce_kernel_cp<BF16>(d.nsrc, cp, aligned);
  } else {
    fn = copy_kernel_cp(cp, aligned);
  }
  if (!fn) return hipErrorInvalidValue;
  const int threads = reduce ? kReduceThreads : kCopyThreads;
  int per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(fn), threads, 0);
  if (e != hipSuccess) return e;
  if (per_cu < 1) per_cu = 1;
  // Measured on MI355X: the 1:1 read/write streams run fastest with few
  // workgroups per CU (more concurrent write streams lower HBM efficiency).
  const int want = cfg.wgs_per_cu > 0 ? cfg.wgs_per_cu : (reduce && d.nsrc >= 4 ? 1 : 2);
  if (want < per_cu) per_cu = want;
  const int cus = device_cu_count();
  uint64_t grid = (uint64_t)(cus > 0 ? cus : 1) * (uint64_t)per_cu;
  if (grid > tiles) grid = tiles;
  hipLaunchKernelGGL(fn, dim3((uint32_t)grid), dim3(threads), 0, stream, d);
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
