// probes.hip -- HBM ceiling probes (snac_hbm_probe in include/snac.h).
//
// A measurement helper, not part of the collectives: the plainest stream of
// each kind -- read only, write only, or one read and one write per byte --
// with the access primitives the collective kernels use (16-byte buffer
// loads and stores with the streaming hint, grid-stride tiles).  What these
// reach on a given MI355X is the ceiling a collective with the same mix of
// reads and writes is judged against on that machine.  An ordered probe
// takes its tiles as the collectives' long launches do: 8 grid-stride
// rounds, then in order from 4 counters (TilePool in snac_device.hpp).
#include <hip/hip_runtime.h>

#include <atomic>

#include "internal.hpp"
#include "snac_device.hpp"

namespace snac {
namespace {

enum : int { kProbeRead = 0, kProbeWrite = 1, kProbeCopy = 2, kProbeOrdered = 8 };

constexpr uint32_t kProbeCounters = 4;
constexpr uint32_t kProbeGridRounds = 8;

// The ordered probes' counters and done count, a 128-byte line each; zero
// at load, and every ordered launch leaves them zero.
__device__ __align__(256) unsigned long long probe_pool[(kProbeCounters + 1) * kFlagStride];

struct ProbePool {
  unsigned long long* next;  // nullptr: grid-stride only
  uint32_t rounds;
};

// Tile t of [0, bytes) is bytes [t TILE, (t + 1) TILE); the last may be
// short (the buffer resource drops the units past it).  READ folds every
// loaded word into an XOR so the loads are live; the fold reaches memory
// only in the (data-dependent, practically never taken) case that it
// equals `magic`.
template <int KIND, int TH, uint32_t TILE>
__global__ __launch_bounds__(TH) void probe_kernel(char* dst, const char* src, uint64_t bytes, uint32_t magic,
                                                   const ProbePool pp) {
  constexpr int U = tile_units<TH, TILE>();
  __shared__ unsigned long long xchg[2];
  const uint64_t tiles = (bytes + TILE - 1) / TILE;
  const uint32_t lane = threadIdx.x * 16u;
  uint32_t fold = 0;
  const TilePool pool{(global_u64*)pp.next, (global_u64*)(pp.next + (uint64_t)kProbeCounters * kFlagStride), xchg,
                      pp.rounds, kProbeCounters};
  for_each_tile(blockIdx.x, gridDim.x, (uint32_t)tiles, pool, [&](uint32_t t) {
    const uint64_t base = (uint64_t)t * TILE;
    const uint64_t left = bytes - base;
    const uint32_t rem = left < TILE ? (uint32_t)left : TILE;
    u32x4 v[U];
    if constexpr (KIND == kProbeWrite) {
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = u32x4{magic, magic, magic, magic};
    } else {
      const __amdgpu_buffer_rsrc_t r = buffer_rsrc(src + base, rem);
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = bld16<kCacheStream>(r, lane + (uint32_t)u * TH * 16u);
    }
    if constexpr (KIND == kProbeRead) {
#pragma unroll
      for (int u = 0; u < U; ++u) fold ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    } else {
      const __amdgpu_buffer_rsrc_t r = buffer_rsrc(dst + base, rem);
#pragma unroll
      for (int u = 0; u < U; ++u) bst16<kCacheStream>(r, lane + (uint32_t)u * TH * 16u, v[u]);
    }
  });
  if constexpr (KIND == kProbeRead) {
    if (fold == magic) *reinterpret_cast<uint32_t*>(dst) = fold;
  }
}

using ProbeFn = void (*)(char*, const char*, uint64_t, uint32_t, const ProbePool);

// probe_pool's address on the current device, looked up once per device.
constexpr int kMaxProbeDevices = 64;
std::atomic<unsigned long long*> g_probe_pool[kMaxProbeDevices];

hipError_t probe_pool_ptr(unsigned long long** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxProbeDevices) return hipErrorInvalidDevice;
  unsigned long long* p = g_probe_pool[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(reinterpret_cast<void**>(&p), HIP_SYMBOL(probe_pool));
    if (e != hipSuccess) return e;
    g_probe_pool[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

template <int TH, uint32_t TILE>
ProbeFn probe_fn(int kind) {
  switch (kind) {
    case kProbeRead: return &probe_kernel<kProbeRead, TH, TILE>;
    case kProbeWrite: return &probe_kernel<kProbeWrite, TH, TILE>;
    case kProbeCopy: return &probe_kernel<kProbeCopy, TH, TILE>;
    default: return nullptr;
  }
}

}  // namespace

hipError_t launch_probe(int kind, void* dst, const void* src, uint64_t bytes, int threads, int tile_bytes,
                        int wgs_per_cu, uint32_t magic, hipStream_t stream) {
  const bool ordered = (kind & kProbeOrdered) != 0;
  kind &= ~kProbeOrdered;
  ProbeFn fn = nullptr;
  if (threads == 64 && tile_bytes == 4096) fn = probe_fn<64, 4096>(kind);
  else if (threads == 64 && tile_bytes == 16384) fn = probe_fn<64, 16384>(kind);
  else if (threads == 256 && tile_bytes == 4096) fn = probe_fn<256, 4096>(kind);
  else if (threads == 256 && tile_bytes == 16384) fn = probe_fn<256, 16384>(kind);
  if (!fn) return hipErrorInvalidValue;
  if (bytes == 0) return hipSuccess;
  const uint64_t tiles = (bytes + (uint64_t)tile_bytes - 1) / (uint64_t)tile_bytes;
  if (tiles > 0xffffffffull) return hipErrorInvalidValue;
  const int cus = device_cu_count();
  uint64_t grid = (uint64_t)(cus > 0 ? cus : 1) * (uint64_t)wgs_per_cu;
  if (grid > tiles) grid = tiles;
  ProbePool pp{nullptr, 0};
  // the counters' groups need a workgroup each: (block / 8) % counters
  if (ordered && grid >= 8ull * kProbeCounters) {
    hipError_t e = probe_pool_ptr(&pp.next);
    if (e != hipSuccess) return e;
    const uint64_t rounds = tiles / grid;
    pp.rounds = rounds >= 2 * kProbeGridRounds ? kProbeGridRounds : (uint32_t)(rounds > 2 ? rounds / 2 : 1);
  }
  hipLaunchKernelGGL(fn, dim3((uint32_t)grid), dim3(threads), 0, stream, static_cast<char*>(dst),
                     static_cast<const char*>(src), bytes, magic, pp);
  return hipGetLastError();
}

}  // namespace snac
