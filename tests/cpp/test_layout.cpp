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
    const uint64_t tile_bytes[] = {16384, 2048, 1024, 4096};
    uint64_t tiles[4] = {0, 0, 0, 0};
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
      const uint32_t head = job_head_bytes(d, jb);
      CHECK(head <= jb.bytes && head < kHeadAlign && head % (uint32_t)e == 0, "coll %d job %d: head %u", coll, j, head);
      for (int q = 0; q < 4; ++q) {
        const uint64_t t = job_tiles(jb, head, tile_bytes[q]);
        const uint64_t body = jb.bytes ? (jb.bytes - head) & ~(uint64_t)15 : 0;
        CHECK(jb.bytes == 0 ? t == 0 : t >= 1, "coll %d job %d: %llu tiles", coll, j, (unsigned long long)t);
        CHECK(t * tile_bytes[q] >= body && (t == 0 || (t - 1) * tile_bytes[q] < body || body == 0),
              "coll %d job %d: tiles do not fit the body", coll, j);
        CHECK(jb.bytes - head - body < 16, "coll %d job %d: tail of %llu bytes", coll, j,
              (unsigned long long)(jb.bytes - head - body));
        tiles[q] += t;
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
  std::printf("%d layouts checked, %d failures\n", cases, failures);
  return failures ? 1 : 0;
}
