// collectives.hip -- the single-kernel collectives: one persistent grid per
// call runs the copy or N-to-1 reduce Atom over the job table of the
// collective's layout.
//
// Every workgroup rebuilds the job table in LDS from the kernel argument
// (layout.hpp), numbers the tiles of all jobs with an exclusive scan, and
// walks tiles blockIdx.x, blockIdx.x + gridDim.x, ...  A tile is
// kThreads * 16 * U bytes of each source; each lane moves U 16-byte units,
// issuing all U*N loads before the first add, then stores the result to one
// destination or to all of them (a multicast: one read, N writes).
//
// Two variants per Atom:
//  * aligned: every job address is 16-byte aligned and every job length a
//    multiple of 16 (the normal case for tensor buffers): plain dwordx4.
//  * generic: any element-aligned address.  Each job is split into a head
//    (bytes until the destination is 16-byte aligned), a body of aligned
//    16-byte stores whose sources are read with ld16_any, and a tail; head
//    and tail are moved one element per lane by tile 0 of the job.
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

// Units per lane per tile: enough independent 16-byte loads in flight
// (about 16 per lane) without exceeding the register budget.
template <int N>
constexpr int reduce_unroll() {
  return N <= 4 ? 4 : (N <= 5 ? 3 : (N <= 8 ? 2 : 1));
}
constexpr int kCopyUnroll = 4;

template <int U>
constexpr uint32_t tile_of() {
  return (uint32_t)kThreads * 16u * (uint32_t)U;
}

// Build the job table and its tile numbering in LDS.  Returns the total
// number of tiles; every thread of the workgroup must call it.
template <bool ALIGNED>
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
  for (int off = 1; off < kThreads; off <<= 1) {
    const uint32_t v = t >= off ? scan[t - off] : 0u;
    __syncthreads();
    scan[t] += v;
    __syncthreads();
  }
  if (t < nj) jobs[t].tile0 = scan[t] - tiles;
  const uint32_t total = scan[kThreads - 1];
  __syncthreads();
  return total;
}

// Store U units (unit u at lane + u * kThreads * 16 bytes past base, if
// below rem) to one destination or, for a multicast, to every destination.
// NU > 0 unrolls the multicast for the common case ndst == NU.
template <int U, int CP>
__device__ __forceinline__ void store_one(char* p, uint32_t lane, uint32_t rem, const u32x4 (&v)[U]) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t o = lane + (uint32_t)u * kThreads * 16u;
    if (o < rem) st16<CP>(p + o, v[u]);
  }
}

template <int U, int CP, int NU>
__device__ __forceinline__ void store_units(const CollDesc& d, int32_t dst_rank, uint64_t base, uint32_t lane,
                                            uint32_t rem, const u32x4 (&v)[U]) {
  if (dst_rank >= 0) {
    store_one<U, CP>(static_cast<char*>(d.dst[dst_rank]) + base, lane, rem, v);
    return;
  }
  if constexpr (NU > 0) {
    if (d.ndst == NU) {
#pragma unroll
      for (int k = 0; k < NU; ++k) store_one<U, CP>(static_cast<char*>(d.dst[k]) + base, lane, rem, v);
      return;
    }
  }
  const int nd = d.ndst;
  for (int k = 0; k < nd; ++k) store_one<U, CP>(static_cast<char*>(d.dst[k]) + base, lane, rem, v);
}

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

template <typename T, int N, int U, int CP, bool ALIGNED>
__device__ __forceinline__ void reduce_tile(const CollDesc& d, const JobL& J, uint32_t lt) {
  constexpr uint32_t TILE = tile_of<U>();
  const uint32_t head = ALIGNED ? 0u : J.head;
  const uint64_t body = ALIGNED ? J.bytes : ((J.bytes - head) & ~(uint64_t)15);
  if constexpr (!ALIGNED) {
    if (lt == 0) reduce_edges<T, N>(d, J, head, body);
    if (body == 0) return;
  }
  const uint64_t toff = (uint64_t)head + (uint64_t)lt * TILE;
  const uint64_t left = (uint64_t)head + body - toff;
  const uint32_t rem = left > TILE ? TILE : (uint32_t)left;
  const char* sp[N];
  uint32_t m[N];
#pragma unroll
  for (int k = 0; k < N; ++k) {
    sp[k] = static_cast<const char*>(d.src[k]) + J.src_off + toff;
    m[k] = uniform((uint32_t)(uintptr_t)sp[k] & 3u);
  }
  const uint32_t lane = threadIdx.x * 16u;
  u32x4 v[U][N];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t o = lane + (uint32_t)u * kThreads * 16u;
    if (o < rem) {
#pragma unroll
      for (int k = 0; k < N; ++k) v[u][k] = ALIGNED ? ld16<CP>(sp[k] + o) : ld16_any(sp[k] + o, m[k]);
    }
  }
  u32x4 r[U];
#pragma unroll
  for (int u = 0; u < U; ++u) r[u] = reduce_unit<T, N>(v[u]);
  store_units<U, CP, N>(d, J.dst_rank, J.dst_off + toff, lane, rem, r);
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

template <int U, int CP, bool ALIGNED>
__device__ __forceinline__ void copy_tile(const CollDesc& d, const JobL& J, uint32_t lt) {
  constexpr uint32_t TILE = tile_of<U>();
  const uint32_t head = ALIGNED ? 0u : J.head;
  const uint64_t body = ALIGNED ? J.bytes : ((J.bytes - head) & ~(uint64_t)15);
  if constexpr (!ALIGNED) {
    if (lt == 0) copy_edges(d, J, head, body);
    if (body == 0) return;
  }
  const uint64_t toff = (uint64_t)head + (uint64_t)lt * TILE;
  const uint64_t left = (uint64_t)head + body - toff;
  const uint32_t rem = left > TILE ? TILE : (uint32_t)left;
  const char* sp = static_cast<const char*>(d.src[J.src_rank]) + J.src_off + toff;
  const uint32_t m = uniform((uint32_t)(uintptr_t)sp & 3u);
  const uint32_t lane = threadIdx.x * 16u;
  u32x4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t o = lane + (uint32_t)u * kThreads * 16u;
    if (o < rem) v[u] = ALIGNED ? ld16<CP>(sp + o) : ld16_any(sp + o, m);
  }
  store_units<U, CP, 0>(d, J.dst_rank, J.dst_off + toff, lane, rem, v);
}

// ---------------------------------------------------------------- kernel

// N > 0: N-to-1 reduce of element type T.  N == 0: byte copy.
template <int N, typename T, int CP, bool ALIGNED>
__global__ __launch_bounds__(kThreads) void coll_kernel(const CollDesc d) {
  constexpr int U = N > 0 ? reduce_unroll<N>() : kCopyUnroll;
  __shared__ JobL jobs[kMaxJobs];
  __shared__ uint32_t scan[kThreads];
  int nj;
  const uint32_t total = build_table<ALIGNED>(d, tile_of<U>(), jobs, scan, nj);
  int j = 0;
  for (uint32_t tile = blockIdx.x; tile < total; tile += gridDim.x) {
    while (j + 1 < nj && jobs[j + 1].tile0 <= tile) ++j;
    JobL J;
    J.src_off = uniform64(jobs[j].src_off);
    J.dst_off = uniform64(jobs[j].dst_off);
    J.bytes = uniform64(jobs[j].bytes);
    J.src_rank = (int32_t)uniform((uint32_t)jobs[j].src_rank);
    J.dst_rank = (int32_t)uniform((uint32_t)jobs[j].dst_rank);
    J.head = uniform(jobs[j].head);
    J.tile0 = uniform(jobs[j].tile0);
    const uint32_t lt = tile - J.tile0;
    if constexpr (N > 0)
      reduce_tile<T, N, U, CP, ALIGNED>(d, J, lt);
    else
      copy_tile<U, CP, ALIGNED>(d, J, lt);
  }
}

// ------------------------------------------------------------- launchers

using KernelFn = void (*)(const CollDesc);

template <int N, typename T, int CP, bool A>
KernelFn kernel_ptr() {
  return &coll_kernel<N, T, CP, A>;
}

template <typename T, int CP, bool A>
KernelFn reduce_kernel(int n) {
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
  if (!aligned) return reduce_kernel<T, kCacheDefault, false>(n);
  switch (cp) {
    case kCacheStream: return reduce_kernel<T, kCacheStream, true>(n);
    case kCacheStreamStores: return reduce_kernel<T, kCacheStreamStores, true>(n);
    case kCacheStreamLoads: return reduce_kernel<T, kCacheStreamLoads, true>(n);
    default: return reduce_kernel<T, kCacheDefault, true>(n);
  }
}

static KernelFn copy_kernel(int cp, bool aligned) {
  if (!aligned) return kernel_ptr<0, F32, kCacheDefault, false>();
  switch (cp) {
    case kCacheStream: return kernel_ptr<0, F32, kCacheStream, true>();
    case kCacheStreamStores: return kernel_ptr<0, F32, kCacheStreamStores, true>();
    case kCacheStreamLoads: return kernel_ptr<0, F32, kCacheStreamLoads, true>();
    default: return kernel_ptr<0, F32, kCacheDefault, true>();
  }
}

static int unroll_for(const CollDesc& d) {
  if (!coll_is_reduce(d.coll)) return kCopyUnroll;
  switch (d.nsrc) {
    case 1: return reduce_unroll<1>();
    case 2: return reduce_unroll<2>();
    case 3: return reduce_unroll<3>();
    case 4: return reduce_unroll<4>();
    case 5: return reduce_unroll<5>();
    case 6: return reduce_unroll<6>();
    case 7: return reduce_unroll<7>();
    case 8: return reduce_unroll<8>();
    default: return reduce_unroll<16>();
  }
}

uint32_t coll_tile_bytes(const CollDesc& d, bool aligned) {
  (void)aligned;
  return (uint32_t)kThreads * 16u * (uint32_t)unroll_for(d);
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
  if (coll_is_reduce(d.coll)) {
    fn = d.esize == 4 ? reduce_kernel_cp<F32>(d.nsrc, cfg.cache_policy, aligned)
                      : reduce_kernel_cp<BF16>(d.nsrc, cfg.cache_policy, aligned);
  } else {
    fn = copy_kernel(cfg.cache_policy, aligned);
  }
  if (!fn) return hipErrorInvalidValue;
  int per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(fn), kThreads, 0);
  if (e != hipSuccess) return e;
  if (per_cu < 1) per_cu = 1;
  if (cfg.wgs_per_cu > 0 && cfg.wgs_per_cu < per_cu) per_cu = cfg.wgs_per_cu;
  const int cus = device_cu_count();
  uint64_t grid = (uint64_t)(cus > 0 ? cus : 1) * (uint64_t)per_cu;
  if (grid > tiles) grid = tiles;
  hipLaunchKernelGGL(fn, dim3((uint32_t)grid), dim3(kThreads), 0, stream, d);
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
