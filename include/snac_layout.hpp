// snac_layout.hpp -- the layout engine: a collective -> a list of copy or
// reduce jobs over byte ranges.
//
// In Purlin 0.6.4 (project description, "Key Idea") a layout is what defines
// a collective: where its inputs and outputs sit across the ranks and which
// of the two Atoms, copy or reduce, moves each part.  The same functions run
// on the host (snac_plan, argument checks) and in every workgroup of a
// collective kernel, which rebuilds the job table in LDS from the compact
// descriptor (snac_coll_desc, include/snac.h) passed as a kernel argument --
// so no per-call host-to-device copy is needed.
//
// Per-collective layouts (N ranks, B per-rank input bytes, e element size,
// D(c) exclusive prefix sum of counts, every offset in bytes):
//   AllReduce       1 reduce job: all sources [0,B) -> all destinations [0,B)
//   ReduceScatter   job r: all sources [r*B/N, (r+1)*B/N) -> dst r [0, B/N)
//   AllGather       job k: src k [0,B) -> all destinations [k*B, (k+1)*B)
//   AllToAll        job (s,d): src s [d*B/N, ..) -> dst d [s*B/N, ..)
//   AllGatherV      job k: src k [0, c_k e) -> all destinations at D(c)_k e
//   ReduceScatterV  job r: all sources [D(c)_r e, ..) -> dst r [0, c_r e)
//   AllToAllV       job (s,d): src s at sum_{j<d} C[s][j] e -> dst d at
//                   sum_{j<s} C[j][d] e, C[s][d] e bytes
// "All destinations" jobs are multicasts: one read, N writes.  When the
// destination buffers do not share an address residue modulo 16 the host
// sets split_multicast and each multicast becomes N single-destination jobs
// so that every job can store with aligned 16-byte vectors.
#pragma once

#include <stdint.h>

#include "snac.h"

#if defined(__HIPCC__)
#define SNAC_HD __host__ __device__ inline
#else
#define SNAC_HD inline
#endif

namespace snac {

constexpr int kMaxRanks = SNAC_MAX_RANKS;
constexpr int kMaxJobs = kMaxRanks * kMaxRanks;

// Collective kinds: the public snac_coll values, plus the two raw Atoms.
enum Coll : int32_t {
  kAllReduce = 0,
  kReduceScatter = 1,
  kAllGather = 2,
  kAllToAll = 3,
  kAllGatherV = 4,
  kReduceScatterV = 5,
  kAllToAllV = 6,
  kAtomCopy = 100,    // src[0] -> dst[0], `bytes`
  kAtomReduce = 101,  // src[0..nsrc) -> dst[0..ndst), `bytes` per buffer
};

SNAC_HD bool coll_is_reduce(int32_t c) {
  return c == kAllReduce || c == kReduceScatter || c == kReduceScatterV || c == kAtomReduce;
}

// Compact description of one collective call; passed by value to kernels.
using CollDesc = snac_coll_desc;

SNAC_HD bool desc_aligned(const CollDesc& d) { return (d.flags & SNAC_DESC_ALIGNED) != 0; }

struct Job {
  uint64_t src_off;
  uint64_t dst_off;
  uint64_t bytes;
  int32_t src_rank;  // -1: every source (reduce)
  int32_t dst_rank;  // -1: every destination (multicast)
};

SNAC_HD int num_jobs(const CollDesc& d) {
  const int n = d.nsrc;
  switch (d.coll) {
    case kAllReduce:
    case kAtomReduce: return d.split_multicast ? d.ndst : 1;
    case kReduceScatter:
    case kReduceScatterV: return n;
    case kAllGather:
    case kAllGatherV: return d.split_multicast ? n * n : n;
    case kAllToAll:
    case kAllToAllV: return n * n;
    case kAtomCopy: return 1;
    default: return 0;
  }
}

// Job j of a collective.  A job may have zero bytes (V counts of zero).
SNAC_HD Job make_job(const CollDesc& d, int j) {
  const int n = d.nsrc;
  const uint64_t e = (uint64_t)d.esize;
  Job r{0, 0, 0, -1, -1};
  switch (d.coll) {
    case kAllReduce:
    case kAtomReduce:
      r.bytes = d.bytes;
      r.dst_rank = d.split_multicast ? j : -1;
      break;
    case kReduceScatter: {
      const uint64_t chunk = d.bytes / (uint64_t)n;
      r.src_off = (uint64_t)j * chunk;
      r.bytes = chunk;
      r.dst_rank = j;
      break;
    }
    case kAllGather: {
      const int k = d.split_multicast ? j / n : j;
      r.src_rank = k;
      r.dst_off = (uint64_t)k * d.bytes;
      r.bytes = d.bytes;
      r.dst_rank = d.split_multicast ? j % n : -1;
      break;
    }
    case kAllToAll: {
      const int s = j / n, dd = j % n;
      const uint64_t chunk = d.bytes / (uint64_t)n;
      r.src_rank = s;
      r.dst_rank = dd;
      r.src_off = (uint64_t)dd * chunk;
      r.dst_off = (uint64_t)s * chunk;
      r.bytes = chunk;
      break;
    }
    case kAllGatherV: {
      const int k = d.split_multicast ? j / n : j;
      uint64_t disp = 0;
      for (int i = 0; i < k; ++i) disp += d.counts[i];
      r.src_rank = k;
      r.dst_off = disp * e;
      r.bytes = d.counts[k] * e;
      r.dst_rank = d.split_multicast ? j % n : -1;
      break;
    }
    case kReduceScatterV: {
      uint64_t disp = 0;
      for (int i = 0; i < j; ++i) disp += d.counts[i];
      r.src_off = disp * e;
      r.bytes = d.counts[j] * e;
      r.dst_rank = j;
      break;
    }
    case kAllToAllV: {
      const int s = j / n, dd = j % n;
      uint64_t sd = 0, rd = 0;
      for (int i = 0; i < dd; ++i) sd += d.counts[s * n + i];
      for (int i = 0; i < s; ++i) rd += d.counts[i * n + dd];
      r.src_rank = s;
      r.dst_rank = dd;
      r.src_off = sd * e;
      r.dst_off = rd * e;
      r.bytes = d.counts[s * n + dd] * e;
      break;
    }
    case kAtomCopy:
      r.src_rank = 0;
      r.dst_rank = 0;
      r.bytes = d.bytes;
      break;
    default: break;
  }
  return r;
}

// Bytes of a job before its destination reaches a 128-byte (cache line)
// boundary, always a multiple of the element size.  The body that follows
// is stored in whole 16-byte units starting on a line, so a wave's 1 KiB
// store covers whole lines instead of straddling nine.  Head (< 128 bytes)
// plus tail (< 16 bytes) fit in one workgroup's lanes, one element each.
constexpr uint32_t kHeadAlign = 128;

SNAC_HD uint32_t job_head_bytes(const CollDesc& d, const Job& j) {
  const int dr = j.dst_rank < 0 ? 0 : j.dst_rank;
  const uint64_t a = (uint64_t)(uintptr_t)d.dst[dr] + j.dst_off;
  uint64_t h = (kHeadAlign - (uint32_t)(a & (kHeadAlign - 1))) & (kHeadAlign - 1);
  if (h > j.bytes) h = j.bytes;
  return (uint32_t)h;
}

// Body bytes of a job before its destination reaches a tile_bytes
// boundary.  When a job's destination does not start on that grid, its
// first tile is cut short there and every later tile covers one whole
// aligned block of the destination.  Tiles offset from the grid straddle an
// extra block each, which two workgroups then write at different times: on
// MI355X that made write-heavy copies with uneven offsets up to 30 % slower
// (AllGatherV, 8 ranks, 128 MiB).  Bodies shorter than two tiles keep the
// plain split.  The body starts 16-byte aligned in the destination, so the
// lead is a multiple of 16.
SNAC_HD uint64_t job_lead_grid(const CollDesc& d, const Job& j, uint32_t head, uint64_t body, uint64_t tile_bytes) {
  if (body < 2 * tile_bytes) return 0;
  const int dr = j.dst_rank < 0 ? 0 : j.dst_rank;
  const uint64_t a = (uint64_t)(uintptr_t)d.dst[dr] + j.dst_off + head;
  return (tile_bytes - a % tile_bytes) % tile_bytes;
}

// The lead the kernels use: tiles of 16 KiB and more follow the destination
// grid; smaller ones (the 4 KiB tiles of big one-to-one copies, the small-
// tile kernels) keep the plain split, since aligning the 4 KiB tiles made
// AllToAllV with Dirichlet counts 1.5 % slower (0.378 against 0.373 ms).
constexpr uint64_t kLeadMinTile = 16384;

SNAC_HD uint64_t job_lead(const CollDesc& d, const Job& j, uint32_t head, uint64_t body, uint64_t tile_bytes) {
  return tile_bytes >= kLeadMinTile ? job_lead_grid(d, j, head, body, tile_bytes) : 0;
}

// Tiles of a job: a first piece of `lead` body bytes when lead > 0, then
// tile_bytes-sized pieces of the rest of its 16-byte body; the head and
// tail bytes ride on tile 0.  A job with bytes but no body still gets one.
SNAC_HD uint64_t job_tiles(const Job& j, uint32_t head, uint64_t lead, uint64_t tile_bytes) {
  if (j.bytes == 0) return 0;
  const uint64_t body = (j.bytes - head) & ~(uint64_t)15;
  const uint64_t t = (lead ? 1 : 0) + (body - lead + tile_bytes - 1) / tile_bytes;
  return t ? t : 1;
}

// Tile lt of a job (numbered as job_tiles does): its offset in the job and
// its body bytes (a multiple of 16; 0 for an edge-only tile).
struct TileSpan {
  uint64_t off;
  uint32_t bytes;
};

SNAC_HD TileSpan tile_span(uint32_t head, uint64_t lead, uint64_t body, uint32_t lt, uint64_t tile_bytes) {
  if (lead && lt == 0) return TileSpan{head, (uint32_t)lead};
  const uint64_t off = (uint64_t)head + lead + (uint64_t)(lead ? lt - 1 : lt) * tile_bytes;
  const uint64_t end = (uint64_t)head + body;
  const uint64_t left = end > off ? end - off : 0;
  return TileSpan{off, (uint32_t)(left > tile_bytes ? tile_bytes : left)};
}

}  // namespace snac
