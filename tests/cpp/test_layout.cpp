// test_layout.cpp -- the layout engine (include/snac_layout.hpp) on the
// host, built with g++ under AddressSanitizer and UndefinedBehaviorSanitizer
// by tests/test_layout_sanitized.py.  For random collectives, rank counts,
// element sizes, sizes, V counts with zeros and misaligned destinations it
// checks that the jobs write every destination byte exactly once, read only
// inside the sources, keep heads and bodies consistent, and that tile
// counts add up -- the properties the kernels rely on.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "snac_layout.hpp"

using namespace snac;

static int failures = 0;
#define CHECK(cond, ...)                                   \
  do {                                                     \
    if (!(cond)) {                                         \
      if (failures < 20) {                                 \
        std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
        std::fprintf(stderr, __VA_ARGS__);                 \
        std::fprintf(stderr, "\n");                        \
      }                                                    \
      ++failures;                                          \
    }                                                      \
  } while (0)

static uint64_t prefix(const uint64_t* c, int k) {
  uint64_t s = 0;
  for (int i = 0; i < k; ++i) s += c[i];
  return s;
}

int main() {
  std::mt19937_64 rng(12345);
  const int colls[] = {kAllReduce, kReduceScatter, kAllGather, kAllToAll, kAllGatherV, kReduceScatterV, kAllToAllV};
  const int esizes[] = {1, 2, 4};
  int cases = 0;
  long leads = 0;  // jobs whose tiles were cut to the destination grid
  for (int iter = 0; iter < 4000; ++iter) {
    const int coll = colls[rng() % 7];
    const bool reduce = coll_is_reduce(coll);
    const int e = reduce ? (rng() % 2 ? 2 : 4) : esizes[rng() % 3];
    const int n = 1 + (int)(rng() % SNAC_MAX_RANKS);
    CollDesc d;
    std::memset(&d, 0, sizeof d);
    d.coll = coll;
    d.nsrc = d.ndst = n;
    d.esize = e;
    d.split_multicast = (int)(rng() % 2);
    // fake, distinct base addresses with random element-aligned residues
    for (int k = 0; k < n; ++k) {
      d.src[k] = reinterpret_cast<const void*>((uintptr_t)(k + 1) << 32 | (uintptr_t)(e * (rng() % 8)));
      d.dst[k] = reinterpret_cast<void*>((uintptr_t)(k + 101) << 32 | (uintptr_t)(e * (rng() % 8)));
    }
    std::vector<uint64_t> in_b(n), out_b(n);
    const uint64_t elems = rng() % 700;  // small enough for byte maps
    if (coll == kAllGatherV || coll == kReduceScatterV || coll == kAllToAllV) {
      const int nc = coll == kAllToAllV ? n * n : n;
      for (int i = 0; i < nc; ++i) d.counts[i] = rng() % 5 == 0 ? 0 : rng() % 97;
    } else {
      uint64_t m = elems;
      if (coll == kReduceScatter || coll == kAllToAll) m -= m % (uint64_t)n;
      d.bytes = m * (uint64_t)e;
    }
    for (int k = 0; k < n; ++k) {
      switch (coll) {
        case kAllReduce: in_b[k] = out_b[k] = d.bytes; break;
        case kReduceScatter: in_b[k] = d.bytes; out_b[k] = d.bytes / n; break;
        case kAllGather: in_b[k] = d.bytes; out_b[k] = d.bytes * n; break;
        case kAllToAll: in_b[k] = out_b[k] = d.bytes; break;
        case kAllGatherV: in_b[k] = d.counts[k] * e; out_b[k] = prefix(d.counts, n) * e; break;
        case kReduceScatterV: in_b[k] = prefix(d.counts, n) * e; out_b[k] = d.counts[k] * e; break;
        default: {
          uint64_t row = 0, col = 0;
          for (int j = 0; j < n; ++j) {
            row += d.counts[k * n + j];
            col += d.counts[j * n + k];
          }
          in_b[k] = row * e;
          out_b[k] = col * e;
        }
      }
    }
    // destination byte maps
    std::vector<std::vector<uint8_t>> cover(n);
    for (int k = 0; k < n; ++k) cover[k].assign(out_b[k], 0);
    const int nj = num_jobs(d);
    CHECK(nj >= 0 && nj <= kMaxJobs, "coll %d: %d jobs", coll, nj);
    if (reduce) CHECK(nj <= kMaxRanks, "reduce coll %d: %d jobs", coll, nj);
    // the kernels' tile sizes, and small ones so that these small jobs also
    // get tiles cut to the destination grid (bodies of two tiles or more)
    const uint64_t tile_bytes[] = {16384, 2048, 1024, 4096, 512, 256};
    constexpr int kTileSizes = 6;
    uint64_t tiles[kTileSizes] = {};
    for (int j = 0; j < nj; ++j) {
      const Job jb = make_job(d, j);
      CHECK(jb.bytes % (uint64_t)e == 0, "coll %d job %d: %llu bytes not whole elements", coll, j,
            (unsigned long long)jb.bytes);
      CHECK(reduce == (jb.src_rank < 0), "coll %d job %d: src_rank %d", coll, j, jb.src_rank);
      const int s0 = jb.src_rank < 0 ? 0 : jb.src_rank, s1 = jb.src_rank < 0 ? n : jb.src_rank + 1;
      for (int s = s0; s < s1; ++s)
        CHECK(jb.src_off + jb.bytes <= in_b[s], "coll %d job %d: reads past src %d", coll, j, s);
      const int d0 = jb.dst_rank < 0 ? 0 : jb.dst_rank, d1 = jb.dst_rank < 0 ? n : jb.dst_rank + 1;
      for (int t = d0; t < d1; ++t) {
        CHECK(jb.dst_off + jb.bytes <= out_b[t], "coll %d job %d: writes past dst %d", coll, j, t);
        if (jb.dst_off + jb.bytes <= out_b[t])
          for (uint64_t b = 0; b < jb.bytes; ++b) cover[t][jb.dst_off + b]++;
      }
      const uint32_t head_g = job_head_bytes(d, jb);
      CHECK(head_g <= jb.bytes && head_g < kHeadAlign && head_g % (uint32_t)e == 0, "coll %d job %d: head %u", coll,
            j, head_g);
      // the generic path's head, and the aligned path's (none) where the job
      // qualifies for it: 16-byte aligned destination and length
      const int dr0 = jb.dst_rank < 0 ? 0 : jb.dst_rank;
      const bool al = ((uint64_t)(uintptr_t)d.dst[dr0] + jb.dst_off) % 16 == 0 && jb.bytes % 16 == 0;
      for (int path = 0; path < (al ? 2 : 1); ++path)
      for (int q = 0; q < kTileSizes; ++q) {
        const uint32_t head = path == 0 ? head_g : 0u;
        const uint64_t T = tile_bytes[q];
        const uint64_t body = jb.bytes ? (jb.bytes - head) & ~(uint64_t)15 : 0;
        // the kernels align only 16 KiB tiles (job_lead); the grid rule
        // itself is checked at every size here
        CHECK(job_lead(d, jb, head, body, T) == (T >= kLeadMinTile ? job_lead_grid(d, jb, head, body, T) : 0),
              "coll %d job %d: job_lead", coll, j);
        const uint64_t lead = job_lead_grid(d, jb, head, body, T);
        const uint64_t t = job_tiles(jb, head, lead, T);
        CHECK(jb.bytes == 0 ? t == 0 : t >= 1, "coll %d job %d: %llu tiles", coll, j, (unsigned long long)t);
        CHECK(jb.bytes - head - body < 16, "coll %d job %d: tail of %llu bytes", coll, j,
              (unsigned long long)(jb.bytes - head - body));
        CHECK(lead < T && lead % 16 == 0 && lead <= body, "coll %d job %d: lead %llu", coll, j,
              (unsigned long long)lead);
        if (lead) ++leads;
        // the tiles, as the kernels number them, cover the body once and in
        // order; every tile after the lead starts on the destination's grid
        const int dr = jb.dst_rank < 0 ? 0 : jb.dst_rank;
        const uint64_t dst0 = (uint64_t)(uintptr_t)d.dst[dr] + jb.dst_off;
        uint64_t next = head;
        for (uint64_t lt = 0; lt < t; ++lt) {
          const TileSpan sp = tile_span(head, lead, body, (uint32_t)lt, T);
          CHECK(sp.off == next, "coll %d job %d tile %llu: starts at %llu, not %llu", coll, j,
                (unsigned long long)lt, (unsigned long long)sp.off, (unsigned long long)next);
          CHECK(sp.bytes <= T && sp.bytes % 16 == 0, "coll %d job %d tile %llu: %u bytes", coll, j,
                (unsigned long long)lt, sp.bytes);
          CHECK(sp.bytes > 0 || body == 0, "coll %d job %d tile %llu: empty", coll, j, (unsigned long long)lt);
          if (lead && lt > 0)
            CHECK((dst0 + sp.off) % T == 0, "coll %d job %d tile %llu: off the destination grid", coll, j,
                  (unsigned long long)lt);
          next = sp.off + sp.bytes;
        }
        CHECK(next == head + body, "coll %d job %d: tiles end at %llu, body at %llu", coll, j,
              (unsigned long long)next, (unsigned long long)(head + body));
        if (path == 0) tiles[q] += t;
      }
    }
    for (int t = 0; t < n; ++t)
      for (uint64_t b = 0; b < out_b[t]; ++b)
        if (cover[t][b] != 1) {
          CHECK(false, "coll %d n %d: dst %d byte %llu written %d times", coll, n, t, (unsigned long long)b,
                cover[t][b]);
          break;
        }
    ++cases;
  }
  std::printf("%d layouts checked, %ld jobs with a lead tile, %d failures\n", cases, leads, failures);
  return failures ? 1 : 0;
}
