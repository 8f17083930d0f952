// probes.hip -- HBM ceiling probes (snac_hbm_probe in include/snac.h).
//
// A measurement helper, not part of the collectives: the plainest stream of
// each kind -- read only, write only, or one read and one write per byte --
// with the access primitives the collective kernels use (16-byte buffer
// loads and stores with the streaming hint, grid-stride tiles).  What these
// reach on a given MI355X is the ceiling a collective with the same mix of
// reads and writes is judged against on that machine.
#include <hip/hip_runtime.h>

#include "internal.hpp"
#include "snac_device.hpp"

namespace snac {
namespace {

enum : int { kProbeRead = 0, kProbeWrite = 1, kProbeCopy = 2 };

// Tile t of [0, bytes) is bytes [t TILE, (t + 1) TILE); the last may be
// short (the buffer resource drops the units past it).  READ folds every
// loaded word into an XOR so the loads are live; the fold reaches memory
// only in the (data-dependent, practically never taken) case that it
// equals `magic`.
template <int KIND, int TH, uint32_t TILE>
__global__ __launch_bounds__(TH) void probe_kernel(char* dst, const char* src, uint64_t bytes, uint32_t magic) {
  constexpr int U = tile_units<TH, TILE>();
  const uint64_t tiles = (bytes + TILE - 1) / TILE;
  const uint32_t lane = threadIdx.x * 16u;
  uint32_t fold = 0;
  for (uint64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
    const uint64_t base = t * TILE;
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
  }
  if constexpr (KIND == kProbeRead) {
    if (fold == magic) *reinterpret_cast<uint32_t*>(dst) = fold;
  }
}

using ProbeFn = void (*)(char*, const char*, uint64_t, uint32_t);

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
  ProbeFn fn = nullptr;
  if (threads == 64 && tile_bytes == 4096) fn = probe_fn<64, 4096>(kind);
  else if (threads == 64 && tile_bytes == 16384) fn = probe_fn<64, 16384>(kind);
  else if (threads == 256 && tile_bytes == 4096) fn = probe_fn<256, 4096>(kind);
  else if (threads == 256 && tile_bytes == 16384) fn = probe_fn<256, 16384>(kind);
  if (!fn) return hipErrorInvalidValue;
  if (bytes == 0) return hipSuccess;
  const uint64_t tiles = (bytes + (uint64_t)tile_bytes - 1) / (uint64_t)tile_bytes;
  const int cus = device_cu_count();
  uint64_t grid = (uint64_t)(cus > 0 ? cus : 1) * (uint64_t)wgs_per_cu;
  if (grid > tiles) grid = tiles;
  hipLaunchKernelGGL(fn, dim3((uint32_t)grid), dim3(threads), 0, stream, static_cast<char*>(dst),
                     static_cast<const char*>(src), bytes, magic);
  return hipGetLastError();
}

}  // namespace snac
