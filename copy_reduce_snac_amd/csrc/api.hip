// api.hip -- the C ABI declared in include/snac.h: argument validation,
// layout planning on the host, context and workspace management, launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstdarg>
#include <cstdlib>
#include <iterator>
#include <vector>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <shared_mutex>
#include <string>

#include "internal.hpp"
#include "snac.h"
#include "snac_layout.hpp"

using namespace snac;

struct snac_ctx {
  int nranks;
  int device;
  size_t staging_bytes;  // per rank
  uint32_t slots;       // staging slots at the context's tile size
  uint32_t tile_bytes;  // the context's (largest) pipeline tile
  uint32_t flag_slots;  // slots the flag arrays cover (>= slots)
  char* workspace;  // device: staging then signal area
  char* staging;
  uint64_t* ready;
  uint64_t* freed;
  uint64_t* ctrl;
  uint64_t* user_flags;  // kUserFlags flags for device-side users
  uint64_t* pool;        // kPoolSlots tile-counter slots (kPoolSlotWords each)
  uint32_t pool_seq;     // the next call's slot
  uint64_t signal_words;
  uint32_t* abort_host;  // host-mapped word (hipHostMalloc)
  uint32_t* abort_dev;   // its device-visible address
};

namespace {

thread_local std::string g_err;

snac_status fail(snac_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

snac_status ok() {
  g_err.clear();
  return SNAC_OK;
}

snac_status hip_fail(hipError_t e, const char* what) {
  return fail(SNAC_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Process-wide tuning, initialised from the environment when the library
// loads: SNAC_WGS_PER_CU, SNAC_CACHE_POLICY, SNAC_PIPELINE_TILE_BYTES,
// SNAC_PIPELINE_LOOKAHEAD, SNAC_SPIN_LIMIT_LOG2, SNAC_COPY_MULTICAST,
// SNAC_TILE_SCHEDULE (decimal integers; a value snac_set_tuning would
// reject, or that does not parse, is ignored).
bool tuning_valid(const snac_tuning& t) {
  return t.wgs_per_cu >= 0 && t.wgs_per_cu <= 32 && t.cache_policy >= 0 && t.cache_policy <= 4 &&
         t.pipeline_tile_bytes >= 0 && t.pipeline_tile_bytes % 4096 == 0 && t.pipeline_lookahead >= 0 &&
         t.spin_limit_log2 >= 0 && t.spin_limit_log2 <= 40 && t.debug_drop_notify >= 0 &&
         t.debug_drop_notify <= SNAC_MAX_RANKS && t.copy_multicast >= 0 && t.copy_multicast <= 2 &&
         t.debug_producer_delay >= 0 && t.debug_producer_delay <= 100000 && t.tile_schedule >= 0 &&
         t.tile_schedule <= 2;
}

int env_int(const char* name, bool* ok) {
  const char* v = std::getenv(name);
  *ok = false;
  if (!v || !*v) return 0;
  char* end = nullptr;
  const long x = std::strtol(v, &end, 10);
  if (*end != '\0' || x < INT32_MIN || x > INT32_MAX) return 0;
  *ok = true;
  return (int)x;
}

snac_tuning tuning_from_env() {
  snac_tuning t{0, 0, 0, 0, 0, 0, 0, 0, 0};
  struct {
    const char* name;
    int32_t* field;
  } vars[] = {{"SNAC_WGS_PER_CU", &t.wgs_per_cu},
              {"SNAC_CACHE_POLICY", &t.cache_policy},
              {"SNAC_PIPELINE_TILE_BYTES", &t.pipeline_tile_bytes},
              {"SNAC_PIPELINE_LOOKAHEAD", &t.pipeline_lookahead},
              {"SNAC_SPIN_LIMIT_LOG2", &t.spin_limit_log2},
              {"SNAC_COPY_MULTICAST", &t.copy_multicast},
              {"SNAC_TILE_SCHEDULE", &t.tile_schedule}};
  for (auto& v : vars) {
    bool ok = false;
    const int x = env_int(v.name, &ok);
    if (!ok) continue;
    const int32_t before = *v.field;
    *v.field = x;
    if (!tuning_valid(t)) *v.field = before;
  }
  return t;
}

snac_tuning g_tuning = tuning_from_env();

// Guards g_tuning and g_rules.  The set calls write; every call reads one
// consistent copy, since collectives may run on other host threads with
// their own contexts while the tuning changes.
std::shared_mutex g_tuning_mu;

snac_tuning tuning_now() {
  std::shared_lock<std::shared_mutex> lk(g_tuning_mu);
  return g_tuning;
}

constexpr uint32_t kMaxPipeTile = 2048u * 1024u;
constexpr uint32_t kMinPipeTile = 4096u;
constexpr uint32_t kMinAutoSlots = 64u;
constexpr uint32_t kMaxFlagSlots = 4096u;
constexpr uint32_t kMinSplitTile = 65536u;  // smallest tile a call cuts the ring into
constexpr uint32_t kMaxCallTile = 16u << 20;  // largest tile a call merges slots into
constexpr size_t kDefaultStaging = 64u * 1024u * 1024u;
// the streaming cut of big pipeline messages (snac_pipeline_scale_reduce)
constexpr uint64_t kStreamPipeMinBytes = 128ull << 20;  // per rank
constexpr uint32_t kStreamPipeTile = 1u << 20;
constexpr uint32_t kStreamPipeLookahead = 3;
constexpr int kDefaultSpinLog2 = 22;

// ---- tuning rules

// Built-in rules, measured on MI355X: reduces of 4 or more sources run one
// workgroup per CU (more concurrent write streams lower HBM efficiency),
// smaller reduces and copies two; streaming (non-temporal) accesses,
// except that AllGather(V) reads its inputs with cached loads -- N
// destinations are written per input byte, so inputs small enough for the
// Infinity Cache stay there across calls (6.3-6.7 TB/s against 4.9 with
// streaming loads when they are reused; no difference when they are not).
// The pipeline runs one workgroup per CU at every size: bf16 4096x8192
// N=8, 2 MiB tiles, 295 us against 391 at two per CU; f32 with 4 MiB tiles
// 604 against 771 (at 1 MiB per rank: 24.6 us against 31.3).
const snac_tuning_rule kBuiltinRules[] = {
    {SNAC_RULE_PIPELINE, 1, SNAC_MAX_RANKS, 0, 0, UINT64_MAX, 1, 0},
    // multicast copies: cached loads, streaming stores.  AllGather bf16 N=8,
    // 16 MiB per rank in: 180 us against 210 with streaming loads when a
    // producer kernel had just written the inputs, 228 against 235 right
    // after the ReduceScatter that wrote them
    {SNAC_COLL_ALL_GATHER, 1, SNAC_MAX_RANKS, 0, 0, UINT64_MAX, 0, 2},
    {SNAC_COLL_ALL_GATHER_V, 1, SNAC_MAX_RANKS, 0, 0, UINT64_MAX, 0, 2},
    // everything else (ReduceScatterV included: 205 us at the kernel's one
    // workgroup per CU against 215 at two, f32 N=8, 128 MiB per rank with
    // Dirichlet counts): the kernel's workgroups per CU, which depend on the
    // message's tile size and source count, and streaming accesses.  Cached
    // loads measured up to 30 % faster at 4-32 MiB per rank, but only when
    // the same inputs were read again call after call; with inputs freshly
    // written by a producer kernel they gained nothing, and at 64 MiB they
    // lost 17-30 %
    {SNAC_RULE_ANY_REDUCE, 1, SNAC_MAX_RANKS, 0, 0, UINT64_MAX, 0, 1},
    {SNAC_RULE_ANY_COPY, 1, SNAC_MAX_RANKS, 0, 0, UINT64_MAX, 0, 1},
};

std::vector<snac_tuning_rule> g_rules(std::begin(kBuiltinRules), std::end(kBuiltinRules));

bool rule_matches(const snac_tuning_rule& r, int32_t coll, int nsrc, int esize, uint64_t bytes) {
  bool c = false;
  if (r.coll == SNAC_RULE_ANY) c = true;
  else if (r.coll == SNAC_RULE_ANY_REDUCE) c = coll != SNAC_RULE_PIPELINE && coll_is_reduce(coll);
  else if (r.coll == SNAC_RULE_ANY_COPY) c = coll != SNAC_RULE_PIPELINE && !coll_is_reduce(coll);
  else c = r.coll == coll;
  return c && nsrc >= r.min_ranks && nsrc <= r.max_ranks && (r.esize == 0 || r.esize == esize) &&
         bytes >= r.min_bytes && bytes <= r.max_bytes;
}

// Launch parameters of a call: the first matching rule, then the explicit
// process-wide values on top.  The caller holds g_tuning_mu.
LaunchCfg launch_cfg_locked(int32_t coll, int nsrc, int esize, uint64_t bytes) {
  LaunchCfg c{0, 0, g_tuning.tile_schedule};
  for (const snac_tuning_rule& r : g_rules) {
    if (rule_matches(r, coll, nsrc, esize, bytes)) {
      c = LaunchCfg{r.wgs_per_cu, r.cache_policy, g_tuning.tile_schedule};
      break;
    }
  }
  if (g_tuning.wgs_per_cu) c.wgs_per_cu = g_tuning.wgs_per_cu;
  if (g_tuning.cache_policy) c.cache_policy = g_tuning.cache_policy;
  return c;
}

LaunchCfg launch_cfg(int32_t coll, int nsrc, int esize, uint64_t bytes) {
  std::shared_lock<std::shared_mutex> lk(g_tuning_mu);
  return launch_cfg_locked(coll, nsrc, esize, bytes);
}

bool rule_ok(const snac_tuning_rule& r) {
  const bool coll_ok = r.coll == SNAC_RULE_ANY || r.coll == SNAC_RULE_ANY_REDUCE || r.coll == SNAC_RULE_ANY_COPY ||
                       (r.coll >= 0 && r.coll <= 6) || r.coll == SNAC_RULE_ATOM_COPY ||
                       r.coll == SNAC_RULE_ATOM_REDUCE || r.coll == SNAC_RULE_PIPELINE;
  return coll_ok && r.min_ranks >= 1 && r.min_ranks <= r.max_ranks && r.max_ranks <= SNAC_MAX_RANKS &&
         (r.esize == 0 || r.esize == 1 || r.esize == 2 || r.esize == 4) && r.min_bytes <= r.max_bytes &&
         r.wgs_per_cu >= 0 && r.wgs_per_cu <= 32 && r.cache_policy >= 0 && r.cache_policy <= 4;
}

int esize_of(snac_dtype t) {
  switch (t) {
    case SNAC_BYTE: return 1;
    case SNAC_U32: return 4;
    case SNAC_F32: return 4;
    case SNAC_BF16: return 2;
    default: return 0;
  }
}

bool is_float(snac_dtype t) { return t == SNAC_F32 || t == SNAC_BF16; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

// Shared argument checks and planning for every collective.
struct Plan {
  CollDesc d;
  snac_ctx* ctx;  // the call's context (its tile counters), or nullptr
  bool aligned;
  int shape;   // kShape*: 16 KiB tiles, small tiles (message too small to fill the GPU
               // at 16 KiB tiles), or the 4 KiB streaming shape of big one-to-one copies
  uint64_t tiles;
  uint64_t rule_bytes;  // per-rank input bytes the tuning rules match on
};

// Host copy of the layout: total tiles and the aligned flag.
void finish_plan(Plan& p) {
  const int nj = num_jobs(p.d);
  bool aligned = true;
  for (int j = 0; j < nj && aligned; ++j) {
    const Job jb = make_job(p.d, j);
    if (jb.bytes == 0) continue;
    if (jb.bytes & 15u) aligned = false;
    const int s0 = jb.src_rank < 0 ? 0 : jb.src_rank, s1 = jb.src_rank < 0 ? p.d.nsrc : jb.src_rank + 1;
    for (int s = s0; s < s1; ++s)
      if (((uintptr_t)p.d.src[s] + jb.src_off) & 15u) aligned = false;
    const int t0 = jb.dst_rank < 0 ? 0 : jb.dst_rank, t1 = jb.dst_rank < 0 ? p.d.ndst : jb.dst_rank + 1;
    for (int t = t0; t < t1; ++t)
      if (((uintptr_t)p.d.dst[t] + jb.dst_off) & 15u) aligned = false;
  }
  p.aligned = aligned;
  auto count_tiles = [&](int shape) {
    const uint64_t tile = coll_tile_bytes(p.d, shape);
    uint64_t tiles = 0;
    for (int j = 0; j < nj; ++j) {
      const Job jb = make_job(p.d, j);
      const uint32_t head = aligned ? 0u : job_head_bytes(p.d, jb);
      const uint64_t body = (jb.bytes - head) & ~(uint64_t)15;
      tiles += job_tiles(jb, head, job_lead(p.d, jb, head, body, tile), tile);
    }
    return tiles;
  };
  p.shape = kShapeTile;
  p.tiles = count_tiles(kShapeTile);
  const int cus = device_cu_count();
  if (p.tiles > 0 && cus > 0 && p.tiles < (uint64_t)cus) {
    p.shape = kShapeSmall;
    p.tiles = count_tiles(kShapeSmall);
  } else if (p.tiles > 0) {
    uint64_t job_bytes = 0;
    bool byte_shift = false;  // a one-to-one copy reading across the dword grid
    for (int j = 0; j < nj; ++j) {
      const Job jb = make_job(p.d, j);
      job_bytes += jb.bytes;
      if (!aligned && jb.bytes && !coll_is_reduce(p.d.coll) && jb.src_rank >= 0 && jb.dst_rank >= 0 &&
          (((uintptr_t)p.d.src[jb.src_rank] + jb.src_off) - ((uintptr_t)p.d.dst[jb.dst_rank] + jb.dst_off)) & 3u)
        byte_shift = true;
    }
    p.shape = large_shape(p.d, job_bytes, byte_shift);
    // A call with a context hands big one-to-one copies out from its tile
    // counters, on 16 KiB tiles: AllToAll u32 N=8 at 128 MiB per rank took
    // 0.332 ms so, against 0.360 on grid-stride 4 KiB tiles
    if (p.shape == kShapeStream && p.ctx && tuning_now().tile_schedule != 1) p.shape = kShapeTile;
    if (p.shape != kShapeTile) p.tiles = count_tiles(p.shape);
  }
}

// Copy multicasts split into one job per destination when asked to.
int split_copy(void* const* dst, int ndst);

// Multicast jobs need one destination residue modulo 16.
int needs_split(void* const* dst, int ndst) {
  for (int i = 1; i < ndst; ++i)
    if ((((uintptr_t)dst[i]) & 15u) != (((uintptr_t)dst[0]) & 15u)) return 1;
  return 0;
}

// A buffer may be NULL only when its extent (in_bytes/out_bytes) is zero.
int split_copy(void* const* dst, int ndst) {
  if (tuning_now().copy_multicast == 2) return 1;
  return needs_split(dst, ndst);
}

snac_status check_ptrs(const void* const* src, const uint64_t* in_bytes, int nsrc, void* const* dst,
                       const uint64_t* out_bytes, int ndst, int esize) {
  if (!src || !dst) return fail(SNAC_E_ARG, "src and dst pointer arrays must not be NULL");
  for (int i = 0; i < nsrc; ++i) {
    if (!src[i] && in_bytes[i]) return fail(SNAC_E_ARG, "src[%d] is NULL", i);
    if ((uintptr_t)src[i] % (uintptr_t)esize) return fail(SNAC_E_ARG, "src[%d] not aligned to %d bytes", i, esize);
  }
  for (int i = 0; i < ndst; ++i) {
    if (!dst[i] && out_bytes[i]) return fail(SNAC_E_ARG, "dst[%d] is NULL", i);
    if ((uintptr_t)dst[i] % (uintptr_t)esize) return fail(SNAC_E_ARG, "dst[%d] not aligned to %d bytes", i, esize);
  }
  return SNAC_OK;
}

// in_bytes[i]/out_bytes[i]: extents of each src/dst buffer.  `inplace_ok`
// says whether dst d may start exactly at src s (position-aligned reuse).
template <typename InplaceFn>
snac_status check_overlap(const void* const* src, const uint64_t* in_bytes, int nsrc, void* const* dst,
                          const uint64_t* out_bytes, int ndst, InplaceFn inplace_ok) {
  for (int a = 0; a < ndst; ++a) {
    const Range ra{(uintptr_t)dst[a], (uintptr_t)dst[a] + out_bytes[a]};
    if (ra.lo == ra.hi) continue;
    for (int b = a + 1; b < ndst; ++b) {
      const Range rb{(uintptr_t)dst[b], (uintptr_t)dst[b] + out_bytes[b]};
      if (rb.lo != rb.hi && overlaps(ra, rb)) return fail(SNAC_E_ARG, "dst[%d] and dst[%d] overlap", a, b);
    }
    for (int s = 0; s < nsrc; ++s) {
      const Range rs{(uintptr_t)src[s], (uintptr_t)src[s] + in_bytes[s]};
      if (rs.lo == rs.hi || !overlaps(ra, rs)) continue;
      if (!inplace_ok(a, s)) return fail(SNAC_E_ARG, "dst[%d] overlaps src[%d] (not a supported in-place form)", a, s);
    }
  }
  return SNAC_OK;
}

snac_status check_ctx(const snac_ctx* ctx) {
  if (!ctx) return fail(SNAC_E_ARG, "ctx is NULL");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(SNAC_E_HIP, "hipGetDevice failed");
  if (dev != ctx->device) return fail(SNAC_E_STATE, "context belongs to device %d, current device is %d", ctx->device, dev);
  return SNAC_OK;
}

// Set by snac_describe around a call of fixed_collective / v_collective:
// the validated plan is copied out instead of launched.
thread_local snac_coll_desc* g_describe = nullptr;

snac_status run(Plan& p, hipStream_t stream) {
  finish_plan(p);
  p.d.flags = p.aligned ? SNAC_DESC_ALIGNED : 0;
  if (g_describe) {
    *g_describe = p.d;
    return ok();
  }
  if (p.tiles == 0) return ok();
  unsigned long long* pool = nullptr;
  if (p.ctx) {
    pool = reinterpret_cast<unsigned long long*>(p.ctx->pool + (uint64_t)(p.ctx->pool_seq % kPoolSlots) * kPoolSlotWords);
    ++p.ctx->pool_seq;
  }
  hipError_t e = launch_collective(p.d, p.aligned, p.shape, p.tiles,
                                   launch_cfg(p.d.coll, p.d.nsrc, p.d.esize, p.rule_bytes), stream, pool);
  if (e != hipSuccess) return hip_fail(e, "collective launch");
  return ok();
}

Plan base_plan(int32_t coll, int nsrc, int ndst, int esize) {
  Plan p;
  std::memset(&p, 0, sizeof p);
  p.d.coll = coll;
  p.d.nsrc = nsrc;
  p.d.ndst = ndst;
  p.d.esize = esize;
  return p;
}

// A request with nothing to move: no launch, or an empty descriptor.
snac_status describe_empty(int32_t coll, int n, int e) {
  if (g_describe) {
    Plan p = base_plan(coll, n, n, e);
    p.d.flags = SNAC_DESC_ALIGNED;
    *g_describe = p.d;
  }
  return ok();
}

// fixed-size collectives share their checks (n ranks; the context's rank
// count, or the caller's for the context-free entry point)
snac_status fixed_collective_n(int32_t coll, snac_ctx* ctx, int n, const void* const* src, void* const* dst,
                               size_t bytes, snac_dtype dtype, snac_stream stream) {
  snac_status st = SNAC_OK;
  const int e = esize_of(dtype);
  if (!e) return fail(SNAC_E_ARG, "unknown dtype %d", (int)dtype);
  const bool reduce = coll == kAllReduce || coll == kReduceScatter;
  if (reduce && !is_float(dtype)) return fail(SNAC_E_ARG, "reductions need SNAC_F32 or SNAC_BF16");
  if (bytes > SNAC_MAX_BYTES) return fail(SNAC_E_ARG, "bytes (%zu) above SNAC_MAX_BYTES", bytes);
  if (bytes % (size_t)e) return fail(SNAC_E_ARG, "bytes (%zu) is not a multiple of the element size %d", bytes, e);
  if ((coll == kReduceScatter || coll == kAllToAll) && bytes % ((size_t)n * e))
    return fail(SNAC_E_ARG, "bytes (%zu) is not a multiple of N * element size (%d)", bytes, n * e);
  if (bytes == 0) return describe_empty(coll, n, e);
  uint64_t in_b[kMaxRanks], out_b[kMaxRanks];
  for (int i = 0; i < n; ++i) {
    in_b[i] = bytes;
    out_b[i] = coll == kAllGather ? bytes * n : (coll == kReduceScatter ? bytes / n : bytes);
  }
  if ((st = check_ptrs(src, in_b, n, dst, out_b, n, e)) != SNAC_OK) return st;
  const size_t chunk = bytes / (size_t)n;
  st = check_overlap(src, in_b, n, dst, out_b, n, [&](int d, int s) {
    if (d != s) return false;
    if (coll == kAllReduce) return (uintptr_t)dst[d] == (uintptr_t)src[s];
    if (coll == kReduceScatter) return (uintptr_t)dst[d] == (uintptr_t)src[s] + (uintptr_t)d * chunk;
    if (coll == kAllGather) return (uintptr_t)src[s] == (uintptr_t)dst[d] + (uintptr_t)d * bytes;
    return false;
  });
  if (st != SNAC_OK) return st;
  Plan p = base_plan(coll, n, n, e);
  p.ctx = ctx;
  p.d.bytes = bytes;
  p.rule_bytes = bytes;
  for (int i = 0; i < n; ++i) {
    p.d.src[i] = src[i];
    p.d.dst[i] = dst[i];
  }
  if (coll == kAllReduce) p.d.split_multicast = needs_split(dst, n);
  if (coll == kAllGather) p.d.split_multicast = split_copy(dst, n);
  return run(p, (hipStream_t)stream);
}

snac_status fixed_collective(int32_t coll, snac_ctx* ctx, const void* const* src, void* const* dst, size_t bytes,
                             snac_dtype dtype, snac_stream stream) {
  const snac_status st = check_ctx(ctx);
  if (st != SNAC_OK) return st;
  return fixed_collective_n(coll, ctx, ctx->nranks, src, dst, bytes, dtype, stream);
}

snac_status v_collective(int32_t coll, snac_ctx* ctx, const void* const* src, void* const* dst, const size_t* counts,
                         snac_dtype dtype, snac_stream stream) {
  snac_status st = check_ctx(ctx);
  if (st != SNAC_OK) return st;
  const int n = ctx->nranks;
  const int e = esize_of(dtype);
  if (!e) return fail(SNAC_E_ARG, "unknown dtype %d", (int)dtype);
  if (coll == kReduceScatterV && !is_float(dtype)) return fail(SNAC_E_ARG, "reductions need SNAC_F32 or SNAC_BF16");
  if (!counts) return fail(SNAC_E_ARG, "counts is NULL");
  const int nc = coll == kAllToAllV ? n * n : n;
  uint64_t total = 0;
  for (int i = 0; i < nc; ++i) {
    if (counts[i] > SNAC_MAX_BYTES) return fail(SNAC_E_ARG, "counts[%d] above SNAC_MAX_BYTES", i);
    total += counts[i];
  }
  if (total == 0) return describe_empty(coll, n, e);
  uint64_t in_b[kMaxRanks], out_b[kMaxRanks];
  for (int i = 0; i < n; ++i) {
    if (coll == kAllGatherV) {
      in_b[i] = counts[i] * e;
      out_b[i] = total * e;
    } else if (coll == kReduceScatterV) {
      in_b[i] = total * e;
      out_b[i] = counts[i] * e;
    } else {
      uint64_t row = 0, col = 0;
      for (int j = 0; j < n; ++j) {
        row += counts[i * n + j];
        col += counts[j * n + i];
      }
      in_b[i] = row * e;
      out_b[i] = col * e;
    }
  }
  if ((st = check_ptrs(src, in_b, n, dst, out_b, n, e)) != SNAC_OK) return st;
  st = check_overlap(src, in_b, n, dst, out_b, n, [](int, int) { return false; });
  if (st != SNAC_OK) return st;
  Plan p = base_plan(coll, n, n, e);
  p.ctx = ctx;
  for (int i = 0; i < n; ++i) {
    p.d.src[i] = src[i];
    p.d.dst[i] = dst[i];
    p.rule_bytes = std::max<uint64_t>(p.rule_bytes, in_b[i]);
  }
  for (int i = 0; i < nc; ++i) p.d.counts[i] = counts[i];
  if (coll == kAllGatherV) p.d.split_multicast = split_copy(dst, n);
  return run(p, (hipStream_t)stream);
}

}  // namespace

extern "C" {

int snac_abi_version(void) { return SNAC_ABI_VERSION; }

const char* snac_status_str(snac_status s) {
  switch (s) {
    case SNAC_OK: return "SNAC_OK";
    case SNAC_E_ARG: return "SNAC_E_ARG: invalid argument";
    case SNAC_E_UNSUPPORTED: return "SNAC_E_UNSUPPORTED: not implemented";
    case SNAC_E_NOMEM: return "SNAC_E_NOMEM: device allocation failed";
    case SNAC_E_HIP: return "SNAC_E_HIP: HIP runtime error";
    case SNAC_E_TIMEOUT: return "SNAC_E_TIMEOUT: device-side wait timed out";
    case SNAC_E_STATE: return "SNAC_E_STATE: context unusable";
    case SNAC_E_ABORTED: return "SNAC_E_ABORTED: device-side waits aborted";
    default: return "SNAC_E_?: unknown status";
  }
}

const char* snac_last_error(void) { return g_err.c_str(); }

int snac_ctx_nranks(const snac_ctx* ctx) { return ctx ? ctx->nranks : 0; }

snac_status snac_get_tuning(snac_tuning* out) {
  if (!out) return fail(SNAC_E_ARG, "out is NULL");
  *out = tuning_now();
  return ok();
}

snac_status snac_set_tuning(const snac_tuning* in) {
  if (!in) return fail(SNAC_E_ARG, "in is NULL");
  if (in->wgs_per_cu < 0 || in->wgs_per_cu > 32) return fail(SNAC_E_ARG, "wgs_per_cu out of range [0, 32]");
  if (in->cache_policy < 0 || in->cache_policy > 4) return fail(SNAC_E_ARG, "cache_policy out of range [0, 4]");
  if (in->pipeline_tile_bytes < 0 || in->pipeline_tile_bytes % 4096)
    return fail(SNAC_E_ARG, "pipeline_tile_bytes must be a non-negative multiple of 4096");
  if (in->pipeline_lookahead < 0) return fail(SNAC_E_ARG, "pipeline_lookahead must be >= 0");
  if (in->spin_limit_log2 < 0 || in->spin_limit_log2 > 40) return fail(SNAC_E_ARG, "spin_limit_log2 out of range");
  if (in->debug_drop_notify < 0 || in->debug_drop_notify > SNAC_MAX_RANKS)
    return fail(SNAC_E_ARG, "debug_drop_notify out of range");
  if (in->copy_multicast < 0 || in->copy_multicast > 2) return fail(SNAC_E_ARG, "copy_multicast out of range [0, 2]");
  if (in->debug_producer_delay < 0 || in->debug_producer_delay > 100000)
    return fail(SNAC_E_ARG, "debug_producer_delay out of range [0, 100000]");
  if (in->tile_schedule < 0 || in->tile_schedule > 2) return fail(SNAC_E_ARG, "tile_schedule out of range [0, 2]");
  {
    std::unique_lock<std::shared_mutex> lk(g_tuning_mu);
    g_tuning = *in;
  }
  return ok();
}

snac_status snac_init(int nranks, size_t staging_bytes_per_rank, snac_stream stream, snac_ctx** out) {
  if (!out) return fail(SNAC_E_ARG, "out is NULL");
  *out = nullptr;
  if (nranks < 1 || nranks > SNAC_MAX_RANKS) return fail(SNAC_E_ARG, "nranks %d outside 1..%d", nranks, SNAC_MAX_RANKS);
  const size_t staging = staging_bytes_per_rank ? staging_bytes_per_rank : kDefaultStaging;
  // pipeline tile: the tuning value, else the largest power of two up to
  // 2 MiB that still leaves at least 64 slots in the ring
  uint32_t tile = (uint32_t)tuning_now().pipeline_tile_bytes;
  if (!tile) {
    tile = kMaxPipeTile;
    while (tile > kMinPipeTile && staging / tile < kMinAutoSlots) tile >>= 1;
  }
  if (staging % tile) return fail(SNAC_E_ARG, "staging_bytes_per_rank must be a multiple of the pipeline tile (%u)", tile);
  const uint64_t slots = staging / tile;
  if (slots < 2 || slots > (1u << 20)) return fail(SNAC_E_ARG, "staging ring needs 2 .. 2^20 slots (got %llu)", (unsigned long long)slots);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  snac_ctx* c = new (std::nothrow) snac_ctx();
  if (!c) return fail(SNAC_E_NOMEM, "host allocation failed");
  c->nranks = nranks;
  c->device = dev;
  c->staging_bytes = staging;
  c->slots = (uint32_t)slots;
  c->tile_bytes = tile;
  // flags for the smaller tiles a call may cut the same ring into
  uint64_t fslots = staging / kMinPipeTile;
  if (fslots > kMaxFlagSlots) fslots = kMaxFlagSlots;
  if (fslots < slots) fslots = slots;
  c->flag_slots = (uint32_t)fslots;
  const uint64_t ready_words = (uint64_t)nranks * fslots * kFlagStride;
  const uint64_t free_words = (uint64_t)nranks * fslots * kFlagStride;
  c->signal_words = ready_words + free_words + kCtrlWords + (uint64_t)kUserFlags * kFlagStride +
                    (uint64_t)kPoolSlots * kPoolSlotWords;
  const size_t staging_total = (size_t)nranks * staging;
  const size_t bytes = staging_total + c->signal_words * sizeof(uint64_t);
  e = hipMalloc(reinterpret_cast<void**>(&c->workspace), bytes);
  if (e != hipSuccess) {
    delete c;
    return fail(SNAC_E_NOMEM, "hipMalloc(%zu) failed: %s", bytes, hipGetErrorString(e));
  }
  c->staging = c->workspace;
  c->ready = reinterpret_cast<uint64_t*>(c->workspace + staging_total);
  c->freed = c->ready + ready_words;
  c->ctrl = c->freed + free_words;
  c->user_flags = c->ctrl + kCtrlWords;
  c->pool = c->user_flags + (uint64_t)kUserFlags * kFlagStride;
  c->pool_seq = 0;
  e = hipHostMalloc(reinterpret_cast<void**>(&c->abort_host), sizeof(uint32_t), hipHostMallocMapped | hipHostMallocCoherent);
  if (e != hipSuccess) {
    (void)hipFree(c->workspace);
    delete c;
    return fail(SNAC_E_NOMEM, "hipHostMalloc failed: %s", hipGetErrorString(e));
  }
  *c->abort_host = 0;
  e = hipHostGetDevicePointer(reinterpret_cast<void**>(&c->abort_dev), c->abort_host, 0);
  if (e == hipSuccess) e = fill_u64(c->ready, c->signal_words, 0, (hipStream_t)stream);
  if (e != hipSuccess) {
    (void)hipHostFree(c->abort_host);
    (void)hipFree(c->workspace);
    delete c;
    return hip_fail(e, "workspace set-up");
  }
  *out = c;
  return ok();
}

snac_status snac_check(snac_ctx* ctx, snac_stream stream) {
  if (!ctx) return fail(SNAC_E_ARG, "ctx is NULL");
  hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  uint64_t status = 0;
  e = hipMemcpy(&status, ctx->ctrl + kCtrlStatus, sizeof status, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "reading the status word");
  const bool aborted = __atomic_load_n(ctx->abort_host, __ATOMIC_SEQ_CST) != 0;
  if (status == 0 && !aborted) return ok();
  // re-arm: clear the abort word, every flag and the control words
  __atomic_store_n(ctx->abort_host, 0u, __ATOMIC_SEQ_CST);
  e = fill_u64(ctx->ready, ctx->signal_words, 0, (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "re-arming the signal area");
  if (status == SNAC_E_TIMEOUT) return fail(SNAC_E_TIMEOUT, "a device-side SNAC wait exceeded its spin limit");
  if (status == SNAC_E_ARG)
    return fail(SNAC_E_ARG, "a device-side collective's template arguments did not match its descriptor");
  return fail(SNAC_E_ABORTED, "device-side SNAC waits were aborted");
}

snac_status snac_abort(snac_ctx* ctx) {
  if (!ctx) return fail(SNAC_E_ARG, "ctx is NULL");
  __atomic_store_n(ctx->abort_host, 1u, __ATOMIC_SEQ_CST);
  return ok();
}

snac_status snac_finalize(snac_ctx* ctx, snac_stream stream) {
  if (!ctx) return ok();
  snac_status st = snac_check(ctx, stream);
  std::string err = g_err;
  (void)hipStreamSynchronize((hipStream_t)stream);
  (void)hipHostFree(ctx->abort_host);
  hipError_t e = hipFree(ctx->workspace);
  delete ctx;
  if (st != SNAC_OK) return fail(st, "%s", err.c_str());
  if (e != hipSuccess) return hip_fail(e, "hipFree");
  return ok();
}

snac_status snac_copy(void* dst, const void* src, size_t bytes, snac_stream stream) {
  if (bytes == 0) return ok();
  if (bytes > SNAC_MAX_BYTES) return fail(SNAC_E_ARG, "bytes (%zu) above SNAC_MAX_BYTES", bytes);
  if (!dst || !src) return fail(SNAC_E_ARG, "NULL pointer");
  const Range a{(uintptr_t)dst, (uintptr_t)dst + bytes}, b{(uintptr_t)src, (uintptr_t)src + bytes};
  if (overlaps(a, b)) return fail(SNAC_E_ARG, "src and dst overlap");
  Plan p = base_plan(kAtomCopy, 1, 1, 1);
  p.d.bytes = bytes;
  p.rule_bytes = bytes;
  p.d.src[0] = src;
  p.d.dst[0] = dst;
  return run(p, (hipStream_t)stream);
}

snac_status snac_hbm_probe(int kind, void* dst, const void* src, size_t bytes, int threads, int tile_bytes,
                           int wgs_per_cu, uint32_t magic, snac_stream stream) {
  const int base = kind & ~(int)SNAC_PROBE_ORDERED;
  if (base < SNAC_PROBE_READ || base > SNAC_PROBE_COPY) return fail(SNAC_E_ARG, "unknown probe kind %d", kind);
  if (threads != 64 && threads != 256) return fail(SNAC_E_ARG, "threads must be 64 or 256");
  if (tile_bytes != 4096 && tile_bytes != 16384) return fail(SNAC_E_ARG, "tile_bytes must be 4096 or 16384");
  if (wgs_per_cu < 1 || wgs_per_cu > 32) return fail(SNAC_E_ARG, "wgs_per_cu outside 1..32");
  if (bytes % 16) return fail(SNAC_E_ARG, "bytes must be a multiple of 16");
  if (bytes > SNAC_MAX_BYTES) return fail(SNAC_E_ARG, "bytes (%zu) above SNAC_MAX_BYTES", bytes);
  if (bytes == 0) return ok();
  if (!dst) return fail(SNAC_E_ARG, "dst is NULL");
  if (base != SNAC_PROBE_WRITE && !src) return fail(SNAC_E_ARG, "src is NULL");
  if (((uintptr_t)dst | (base != SNAC_PROBE_WRITE ? (uintptr_t)src : 0)) & 15u)
    return fail(SNAC_E_ARG, "dst and src must be 16-byte aligned");
  if (base == SNAC_PROBE_COPY &&
      overlaps(Range{(uintptr_t)dst, (uintptr_t)dst + bytes}, Range{(uintptr_t)src, (uintptr_t)src + bytes}))
    return fail(SNAC_E_ARG, "src and dst overlap");
  const hipError_t e = launch_probe(kind, dst, src, bytes, threads, tile_bytes, wgs_per_cu, magic, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "probe launch");
  return ok();
}

snac_status snac_reduce_n(void* const* dst, int ndst, const void* const* src, int nsrc, size_t count,
                          snac_dtype dtype, snac_stream stream) {
  if (nsrc < 1 || nsrc > SNAC_MAX_RANKS) return fail(SNAC_E_ARG, "nsrc %d outside 1..%d", nsrc, SNAC_MAX_RANKS);
  if (ndst < 1 || ndst > SNAC_MAX_RANKS) return fail(SNAC_E_ARG, "ndst %d outside 1..%d", ndst, SNAC_MAX_RANKS);
  if (!is_float(dtype)) return fail(SNAC_E_ARG, "reduce needs SNAC_F32 or SNAC_BF16");
  if (count == 0) return ok();
  const int e = esize_of(dtype);
  if (count > SNAC_MAX_BYTES / (uint64_t)e) return fail(SNAC_E_ARG, "count (%zu) above SNAC_MAX_BYTES bytes", count);
  const uint64_t bytes = (uint64_t)count * e;
  uint64_t in_b[kMaxRanks], out_b[kMaxRanks];
  for (int i = 0; i < kMaxRanks; ++i) in_b[i] = out_b[i] = bytes;
  snac_status st = check_ptrs(src, in_b, nsrc, dst, out_b, ndst, e);
  if (st != SNAC_OK) return st;
  st = check_overlap(src, in_b, nsrc, dst, out_b, ndst,
                     [&](int d, int s) { return (uintptr_t)dst[d] == (uintptr_t)src[s]; });
  if (st != SNAC_OK) return st;
  Plan p = base_plan(kAtomReduce, nsrc, ndst, e);
  p.d.bytes = bytes;
  p.rule_bytes = bytes;
  for (int i = 0; i < nsrc; ++i) p.d.src[i] = src[i];
  for (int i = 0; i < ndst; ++i) p.d.dst[i] = dst[i];
  p.d.split_multicast = needs_split(dst, ndst);
  return run(p, (hipStream_t)stream);
}

snac_status snac_all_reduce(snac_ctx* ctx, const void* const* src, void* const* dst, size_t bytes, snac_dtype dtype,
                            snac_stream stream) {
  return fixed_collective(kAllReduce, ctx, src, dst, bytes, dtype, stream);
}

snac_status snac_all_reduce_ex(snac_ctx* ctx, const void* const* src, void* const* dst, size_t bytes,
                               snac_dtype dtype, snac_reduce_mode mode, snac_stream stream) {
  if (mode == SNAC_REDUCE_DETERMINISTIC) return fixed_collective(kAllReduce, ctx, src, dst, bytes, dtype, stream);
  if (mode != SNAC_REDUCE_ATOMIC) return fail(SNAC_E_ARG, "unknown reduction mode %d", (int)mode);
  // validate exactly as the deterministic call, without launching
  snac_coll_desc d;
  g_describe = &d;
  snac_status st = fixed_collective(kAllReduce, ctx, src, dst, bytes, dtype, stream);
  g_describe = nullptr;
  if (st != SNAC_OK) return st;
  if (bytes == 0) return ok();
  const uint64_t e = (uint64_t)d.esize;
  const uint64_t elems = bytes / e;
  bool vec = true;
  for (int i = 0; i < d.nsrc; ++i)
    if (((uintptr_t)d.src[i] | (uintptr_t)d.dst[i]) & 15u) vec = false;
  // accumulator: the staging rings, whole tiles at a time
  const uint64_t tile_e = atomic_chunk_elems(d.esize);
  const uint64_t cap = (uint64_t)ctx->nranks * ctx->staging_bytes / sizeof(float) / tile_e * tile_e;
  if (cap == 0) return fail(SNAC_E_STATE, "staging too small for the atomic accumulator");
  float* acc = reinterpret_cast<float*>(ctx->staging);
  for (uint64_t first = 0; first < elems; first += cap) {
    const uint64_t n = std::min(cap, elems - first);
    hipError_t he = launch_atomic_allreduce(d, acc, first, n, vec && (first * e) % 16 == 0, (hipStream_t)stream);
    if (he != hipSuccess) return hip_fail(he, "atomic all-reduce launch");
  }
  return ok();
}

snac_status snac_all_reduce_atomic_static(int nranks, const void* const* src, void* const* dst, size_t bytes,
                                          snac_dtype dtype, snac_stream stream) {
  if (nranks < 1 || nranks > SNAC_MAX_RANKS) return fail(SNAC_E_ARG, "nranks %d outside 1..%d", nranks, SNAC_MAX_RANKS);
  if (!is_float(dtype)) return fail(SNAC_E_ARG, "reductions need SNAC_F32 or SNAC_BF16");
  const uint64_t e = (uint64_t)esize_of(dtype);
  const uint64_t max_elems = kStaticScratchBytes / sizeof(float);
  if (bytes / e > max_elems)
    return fail(SNAC_E_ARG,
                "%zu bytes per rank need a %llu-element accumulator; the static scratch holds %llu elements "
                "(%llu MiB)",
                bytes, (unsigned long long)(bytes / e), (unsigned long long)max_elems,
                (unsigned long long)(kStaticScratchBytes >> 20));
  // validate exactly as the AllReduce does, without launching
  snac_coll_desc d;
  g_describe = &d;
  snac_status st = fixed_collective_n(kAllReduce, nullptr, nranks, src, dst, bytes, dtype, stream);
  g_describe = nullptr;
  if (st != SNAC_OK) return st;
  if (bytes == 0) return ok();
  float* acc = nullptr;
  hipError_t he = static_scratch(&acc);
  if (he != hipSuccess) return hip_fail(he, "static scratch address");
  bool vec = true;
  for (int i = 0; i < d.nsrc; ++i)
    if (((uintptr_t)d.src[i] | (uintptr_t)d.dst[i]) & 15u) vec = false;
  he = launch_atomic_allreduce(d, acc, 0, bytes / e, vec, (hipStream_t)stream);
  if (he != hipSuccess) return hip_fail(he, "atomic all-reduce launch");
  return ok();
}

snac_status snac_reduce_scatter(snac_ctx* ctx, const void* const* src, void* const* dst, size_t bytes,
                                snac_dtype dtype, snac_stream stream) {
  return fixed_collective(kReduceScatter, ctx, src, dst, bytes, dtype, stream);
}

snac_status snac_all_gather(snac_ctx* ctx, const void* const* src, void* const* dst, size_t bytes, snac_dtype dtype,
                            snac_stream stream) {
  return fixed_collective(kAllGather, ctx, src, dst, bytes, dtype, stream);
}

snac_status snac_all_to_all(snac_ctx* ctx, const void* const* src, void* const* dst, size_t bytes, snac_dtype dtype,
                            snac_stream stream) {
  return fixed_collective(kAllToAll, ctx, src, dst, bytes, dtype, stream);
}

snac_status snac_all_gather_v(snac_ctx* ctx, const void* const* src, void* const* dst, const size_t* counts,
                              snac_dtype dtype, snac_stream stream) {
  return v_collective(kAllGatherV, ctx, src, dst, counts, dtype, stream);
}

snac_status snac_reduce_scatter_v(snac_ctx* ctx, const void* const* src, void* const* dst, const size_t* counts,
                                  snac_dtype dtype, snac_stream stream) {
  return v_collective(kReduceScatterV, ctx, src, dst, counts, dtype, stream);
}

snac_status snac_all_to_all_v(snac_ctx* ctx, const void* const* src, void* const* dst, const size_t* counts,
                              snac_dtype dtype, snac_stream stream) {
  return v_collective(kAllToAllV, ctx, src, dst, counts, dtype, stream);
}

snac_status snac_pipeline_scale_reduce(snac_ctx* ctx, const void* const* x, void* out, size_t count,
                                       snac_dtype dtype, snac_stream stream) {
  snac_status st = check_ctx(ctx);
  if (st != SNAC_OK) return st;
  if (!is_float(dtype)) return fail(SNAC_E_ARG, "the pipeline needs SNAC_F32 or SNAC_BF16");
  if (count == 0) return ok();
  const int n = ctx->nranks;
  const int e = esize_of(dtype);
  if (count > SNAC_MAX_BYTES / (uint64_t)e) return fail(SNAC_E_ARG, "count (%zu) above SNAC_MAX_BYTES bytes", count);
  if (!x || !out) return fail(SNAC_E_ARG, "NULL pointer");
  for (int i = 0; i < n; ++i) {
    if (!x[i]) return fail(SNAC_E_ARG, "x[%d] is NULL", i);
    if ((uintptr_t)x[i] & 15u) return fail(SNAC_E_ARG, "x[%d] must be 16-byte aligned", i);
  }
  if ((uintptr_t)out & 15u) return fail(SNAC_E_ARG, "out must be 16-byte aligned");
  const Range ro{(uintptr_t)out, (uintptr_t)out + count * (uint64_t)e};
  for (int i = 0; i < n; ++i)
    if (overlaps(ro, Range{(uintptr_t)x[i], (uintptr_t)x[i] + count * (uint64_t)e}))
      return fail(SNAC_E_ARG, "out overlaps x[%d]", i);
  if (ctx->tile_bytes % (uint32_t)e) return fail(SNAC_E_STATE, "pipeline tile not a multiple of the element size");
  PipeArgs a;
  std::memset(&a, 0, sizeof a);
  for (int i = 0; i < n; ++i) a.x[i] = x[i];
  a.out = out;
  a.count = count;
  a.nranks = n;
  a.esize = e;
  a.staging = ctx->staging;
  a.ready = ctx->ready;
  a.freed = ctx->freed;
  a.ctrl = ctx->ctrl;
  a.abort_word = ctx->abort_dev;
  // Tile of this call, cut from the context's ring (slots * tile bytes per
  // rank): about one producer item per workgroup per pass over the ring,
  // N * min(tiles, slots) ~ the grid.  Bigger items mean fewer release and
  // acquire fences, which serialise GPU-wide; fewer items than workgroups
  // leave some idle.  On MI355X, one workgroup per CU, bf16 4096x8192 N=8:
  // 295 us with 32 tiles of 2 MiB, 309 with 64 of 1 MiB, 408 with 16 of
  // 4 MiB (f32: 604 us with 32 tiles of 4 MiB, 631 with 64 of 2 MiB); in a
  // 16 MiB ring, 336 us with 32 slots of 512 KiB, 399 with 64 of 256 KiB,
  // 417 with 16 of 1 MiB.  Tiles are split no finer than 64 KiB.
  const uint64_t msg = count * (uint64_t)e;
  const LaunchCfg cfg = launch_cfg(SNAC_RULE_PIPELINE, n, e, msg);
  const snac_tuning tn = tuning_now();
  uint32_t tile = ctx->tile_bytes, slots = ctx->slots;
  uint32_t lookahead = (uint32_t)tn.pipeline_lookahead;
  // Streaming cut for big messages: 1 MiB tiles with the consumers three
  // tiles behind the producers, so that the two phases overlap over the
  // whole call instead of all producers running before all consumers.  On
  // MI355X (N=8, one workgroup per CU), against the cut below:
  //   128 MiB per rank: f32 4096x8192 0.567 against 0.604-0.619 ms, bf16
  //   4096x16384 0.568 against 0.602;  256 MiB per rank: f32 1.09 against
  //   1.25-1.28, bf16 1.13 against 1.23-1.30.
  // At 64 MiB per rank (bf16 4096x8192, f32 4096x4096) the cut below is
  // faster (0.283-0.290 against 0.307-0.309 ms with 1 MiB tiles).
  const uint64_t ring_bytes = (uint64_t)slots * tile;
  const bool streaming = !tn.pipeline_tile_bytes && msg >= kStreamPipeMinBytes && ring_bytes % kStreamPipeTile == 0 &&
                         ring_bytes / kStreamPipeTile >= 16 && ring_bytes / kStreamPipeTile <= ctx->flag_slots;
  if (streaming) {
    tile = kStreamPipeTile;
    slots = (uint32_t)(ring_bytes / kStreamPipeTile);
    if (!lookahead) lookahead = kStreamPipeLookahead;
  } else if (!tn.pipeline_tile_bytes) {
    const uint64_t ring = (uint64_t)slots * tile;
    const uint64_t grid = (uint64_t)(device_cu_count() > 0 ? device_cu_count() : 1) * (uint64_t)pipe_wgs_per_cu(cfg);
    const uint64_t target = (grid + (uint64_t)n - 1) / (uint64_t)n;
    auto tiles_of = [&](uint64_t t) { return (msg + t - 1) / t; };
    // merge: a message that fits the ring keeps at least `target` tiles, one
    // that does not keeps at least `target` slots (the tiles of one pass)
    while (slots % 2 == 0 && slots / 2 >= 2 && (uint64_t)tile * 2 <= kMaxCallTile &&
           (msg <= ring ? tiles_of((uint64_t)tile * 2) >= target : slots / 2 >= target)) {
      tile <<= 1;
      slots >>= 1;
    }
    while (tile / 2 >= kMinSplitTile && (uint64_t)slots * 2 <= ctx->flag_slots && tiles_of(tile) < target) {
      tile >>= 1;
      slots <<= 1;
    }
  }
  // A message that fits the ring takes only the slots it needs (rounded up
  // to 16: 8 queues of at least 2 slots), so that the staging units, which
  // interleave the slots, sweep as compact a window as x and out.  bf16
  // 4096x8192 N=8 in a 128 MiB ring with 2 MiB tiles: 284 us on 32 slots,
  // 295 on all 64.
  {
    const uint64_t need = ((msg + tile - 1) / tile + 15) / 16 * 16;
    if (msg <= (uint64_t)slots * tile && need < slots) slots = (uint32_t)need;
  }
  a.slots = slots;
  a.tile_bytes = tile;
  a.lookahead = lookahead;
  a.spin_limit_log2 = (uint32_t)(tn.spin_limit_log2 ? tn.spin_limit_log2 : kDefaultSpinLog2);
  a.drop_notify = tn.debug_drop_notify;
  a.producer_delay_us = (uint32_t)tn.debug_producer_delay;
  hipError_t err = launch_pipeline(a, dtype == SNAC_BF16, cfg, (hipStream_t)stream, nullptr);
  if (err != hipSuccess) return hip_fail(err, "pipeline launch");
  return ok();
}

snac_status snac_set_tuning_rules(const snac_tuning_rule* rules, int n) {
  if (n < 0 || n > SNAC_MAX_TUNING_RULES) return fail(SNAC_E_ARG, "rule count %d outside 0..%d", n, SNAC_MAX_TUNING_RULES);
  if (n > 0 && !rules) return fail(SNAC_E_ARG, "rules is NULL");
  for (int i = 0; i < n; ++i)
    if (!rule_ok(rules[i])) return fail(SNAC_E_ARG, "rule %d is invalid", i);
  std::unique_lock<std::shared_mutex> lk(g_tuning_mu);
  if (n == 0)
    g_rules.assign(std::begin(kBuiltinRules), std::end(kBuiltinRules));
  else
    g_rules.assign(rules, rules + n);
  return ok();
}

snac_status snac_get_tuning_rules(snac_tuning_rule* out, int max, int* n) {
  if (!n) return fail(SNAC_E_ARG, "n is NULL");
  std::shared_lock<std::shared_mutex> lk(g_tuning_mu);
  *n = (int)g_rules.size();
  if (!out) return ok();
  if (max < (int)g_rules.size()) return fail(SNAC_E_ARG, "max (%d) is smaller than the table (%d rules)", max, *n);
  std::copy(g_rules.begin(), g_rules.end(), out);
  return ok();
}

snac_status snac_tuning_lookup(int32_t coll, int nranks, int esize, size_t bytes, snac_tuning* out) {
  if (!out) return fail(SNAC_E_ARG, "out is NULL");
  if (nranks < 1 || nranks > SNAC_MAX_RANKS) return fail(SNAC_E_ARG, "nranks %d outside 1..%d", nranks, SNAC_MAX_RANKS);
  std::shared_lock<std::shared_mutex> lk(g_tuning_mu);
  const LaunchCfg c = launch_cfg_locked(coll, nranks, esize, bytes);
  *out = g_tuning;
  out->wgs_per_cu = c.wgs_per_cu;
  out->cache_policy = c.cache_policy;
  return ok();
}

snac_status snac_get_device_context(const snac_ctx* ctx, snac_dev_ctx* out) {
  if (!ctx || !out) return fail(SNAC_E_ARG, "NULL argument");
  std::memset(out, 0, sizeof *out);
  out->nranks = ctx->nranks;
  const uint32_t spin = (uint32_t)tuning_now().spin_limit_log2;
  out->spin_limit_log2 = spin ? spin : kDefaultSpinLog2;
  out->status = ctx->ctrl + kCtrlStatus;
  out->abort_word = ctx->abort_dev;
  out->barrier = ctx->ctrl + kCtrlBarrier;
  out->flags = ctx->user_flags;
  out->nflags = kUserFlags;
  out->staging = ctx->staging;
  out->staging_bytes = ctx->staging_bytes;
  return ok();
}

snac_status snac_describe(const snac_ctx* ctx, snac_coll coll, const void* const* src, void* const* dst, size_t bytes,
                          const size_t* counts, snac_dtype dtype, snac_coll_desc* out) {
  if (!out) return fail(SNAC_E_ARG, "out is NULL");
  std::memset(out, 0, sizeof *out);
  snac_ctx* c = const_cast<snac_ctx*>(ctx);
  g_describe = out;
  snac_status st;
  switch (coll) {
    case SNAC_COLL_ALL_REDUCE:
    case SNAC_COLL_REDUCE_SCATTER:
    case SNAC_COLL_ALL_GATHER:
    case SNAC_COLL_ALL_TO_ALL: st = fixed_collective((int32_t)coll, c, src, dst, bytes, dtype, nullptr); break;
    case SNAC_COLL_ALL_GATHER_V:
    case SNAC_COLL_REDUCE_SCATTER_V:
    case SNAC_COLL_ALL_TO_ALL_V: st = v_collective((int32_t)coll, c, src, dst, counts, dtype, nullptr); break;
    default: st = fail(SNAC_E_ARG, "unknown collective %d", (int)coll);
  }
  g_describe = nullptr;
  if (st != SNAC_OK) std::memset(out, 0, sizeof *out);
  return st;
}

snac_status snac_plan(snac_coll coll, int nranks, snac_dtype dtype, size_t bytes, const size_t* counts,
                      snac_job* jobs, int max_jobs, int* njobs) {
  if (!njobs) return fail(SNAC_E_ARG, "njobs is NULL");
  *njobs = 0;
  if (nranks < 1 || nranks > SNAC_MAX_RANKS) return fail(SNAC_E_ARG, "nranks %d outside 1..%d", nranks, SNAC_MAX_RANKS);
  const int e = esize_of(dtype);
  if (!e) return fail(SNAC_E_ARG, "unknown dtype %d", (int)dtype);
  if ((int)coll < 0 || (int)coll > 6) return fail(SNAC_E_ARG, "unknown collective %d", (int)coll);
  const bool v = coll == SNAC_COLL_ALL_GATHER_V || coll == SNAC_COLL_REDUCE_SCATTER_V || coll == SNAC_COLL_ALL_TO_ALL_V;
  const bool red = coll == SNAC_COLL_ALL_REDUCE || coll == SNAC_COLL_REDUCE_SCATTER || coll == SNAC_COLL_REDUCE_SCATTER_V;
  if (red && !is_float(dtype)) return fail(SNAC_E_ARG, "reductions need SNAC_F32 or SNAC_BF16");
  Plan p = base_plan((int32_t)coll, nranks, nranks, e);
  if (v) {
    if (!counts) return fail(SNAC_E_ARG, "counts is NULL");
    const int nc = coll == SNAC_COLL_ALL_TO_ALL_V ? nranks * nranks : nranks;
    for (int i = 0; i < nc; ++i) {
      if (counts[i] > SNAC_MAX_BYTES) return fail(SNAC_E_ARG, "counts[%d] above SNAC_MAX_BYTES", i);
      p.d.counts[i] = counts[i];
    }
  } else {
    if (bytes > SNAC_MAX_BYTES) return fail(SNAC_E_ARG, "bytes (%zu) above SNAC_MAX_BYTES", bytes);
    if (bytes % (size_t)e) return fail(SNAC_E_ARG, "bytes not a multiple of the element size");
    if ((coll == SNAC_COLL_REDUCE_SCATTER || coll == SNAC_COLL_ALL_TO_ALL) && bytes % ((size_t)nranks * e))
      return fail(SNAC_E_ARG, "bytes not a multiple of N * element size");
    p.d.bytes = bytes;
  }
  const int nj = num_jobs(p.d);
  int w = 0;
  for (int j = 0; j < nj; ++j) {
    const Job jb = make_job(p.d, j);
    if (jb.bytes == 0) continue;
    if (w >= max_jobs || !jobs) return fail(SNAC_E_ARG, "more than max_jobs (%d) jobs", max_jobs);
    jobs[w].src_off = jb.src_off;
    jobs[w].dst_off = jb.dst_off;
    jobs[w].bytes = jb.bytes;
    jobs[w].src_rank = jb.src_rank;
    jobs[w].dst_rank = jb.dst_rank;
    ++w;
  }
  *njobs = w;
  return ok();
}

}  // extern "C"
