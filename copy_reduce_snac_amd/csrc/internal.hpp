// internal.hpp -- host-side interface between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "snac_layout.hpp"

namespace snac {

constexpr int kThreads = 256;  // workgroup size of the pipeline and copy kernels

struct LaunchCfg {
  int wgs_per_cu;     // 0: as many as fit
  int cache_policy;   // kCache*
  int tile_schedule;  // snac_tuning.tile_schedule: 0 default, 1 grid-stride only, 2 shared counter
};

// Shared tile counters of one launch (TilePool in snac_device.hpp): `next`,
// and the done count kFlagStride words after it; nullptr: grid-stride.
struct PoolArg {
  unsigned long long* next;  // counter 0; counter c kFlagStride * c words on, then the done count
  uint32_t rounds;           // grid-stride rounds before the counters
  uint32_t counters;         // counters of the launch
};

// Tile shapes of the host-launched collective kernels:
//   kShapeTile    16 KiB tiles (the default)
//   kShapeSmall   one 16-byte unit per lane, for a message with fewer
//                 16 KiB tiles than the GPU has CUs
//   kShapeStream  one-to-one copies that move at least 1 GiB: single-wave
//                 workgroups on 4 KiB tiles
enum Shape : int { kShapeTile = 0, kShapeSmall = 1, kShapeStream = 2 };

// Tile size (bytes of each source per workgroup iteration) of the kernel
// that serves this descriptor in this shape; the host needs it to count
// tiles.
uint32_t coll_tile_bytes(const CollDesc& d, int shape);

// The shape of a message that fills the GPU with 16 KiB tiles, given the
// bytes its jobs copy or reduce (each job's bytes once) and whether some
// one-to-one copy job reads its source at a byte offset from its
// destination's dword grid.
int large_shape(const CollDesc& d, uint64_t job_bytes, bool byte_shift);

// Launch the copy or reduce kernel for a collective descriptor.  `tiles` is
// the total tile count of the layout at coll_tile_bytes(d, shape) (computed
// on the host with the same layout functions the kernel uses).  `pool`: a
// pair of zeroed counters (two words kFlagStride apart) this launch may
// hand its tiles out from, or nullptr; a launch leaves them zeroed again.
hipError_t launch_collective(const CollDesc& d, bool aligned, int shape, uint64_t tiles, const LaunchCfg& cfg,
                             hipStream_t stream, unsigned long long* pool = nullptr);

// Non-deterministic AllReduce of elements [first, first + elems) of every
// source: zero acc[0..elems), add every source into it with float atomics,
// round it into every destination.  vec: every source and destination
// address of the range 16-byte aligned.  Chunks are whole tiles of
// atomic_chunk_elems(esize) elements (except the last).
hipError_t launch_atomic_allreduce(const CollDesc& d, float* acc, uint64_t first, uint64_t elems, bool vec,
                                   hipStream_t stream);
uint64_t atomic_chunk_elems(int esize);

// Device-side SNAC pipeline (y = 0.5 x + r staged, then N-to-1 reduce).
constexpr int kMaxQueues = 8;

struct PipeArgs {
  const void* x[kMaxRanks];
  void* out;
  uint64_t count;      // elements
  int32_t nranks;
  int32_t esize;
  char* staging;       // [nranks][slots * tile_bytes], units of slots interleaved
  uint64_t* ready;     // [nranks][slots], kFlagStride words apart
  uint64_t* freed;     // [slots][nranks] (one flag per consumer part)
  uint64_t* ctrl;      // control words, kFlagStride apart (kCtrl*)
  const uint32_t* abort_word;  // host-mapped
  uint32_t slots;      // total slots = queues * slots_per_queue (+ unused)
  uint32_t tile_bytes;
  uint32_t lookahead;
  uint32_t grid;
  uint32_t spin_limit_log2;
  int32_t drop_notify;  // r+1: rank r never notifies (test hook)
  uint32_t producer_delay_us;  // > 0: some producer items sleep first (test hook)
  // Derived on the host so that every loop and branch condition in the
  // kernel is a scalar (kernel-argument) value: a condition the compiler
  // cannot prove uniform lets it restructure a loop that holds barriers.
  uint32_t tiles;       // ceil(count / tile elements)
  uint32_t queues;      // independent ticket queues (tile t -> queue t % queues)
  uint32_t qslots;      // slots per queue
  uint32_t rounds;      // max over queues of ceil(tiles_q / qslots)
  uint32_t unit_shift;   // a layout unit is 1 << unit_shift pieces (4 KiB each)
  uint32_t unit_bytes;   // bytes per unit
  uint32_t full_units;   // whole units in a rank's message
  uint32_t tail_tile;    // the tile that owns the short last unit: full_units % tiles
  uint32_t tail_pieces;  // whole pieces of that unit
  uint32_t last_bytes;   // bytes of the message's short last piece (0: none)
};

// control words (uint64 indices into ctrl)
enum : uint32_t {
  kCtrlTicket = 0,                   // kMaxQueues tickets, kFlagStride apart
  kCtrlQDone = kMaxQueues * 16,      // kMaxQueues per-queue done counters
  kCtrlDone = kCtrlQDone + kMaxQueues * 16,  // queues finished
  kCtrlEpoch = kCtrlDone + 16,
  kCtrlStatus = kCtrlEpoch + 16,
  kCtrlBarrier = kCtrlStatus + 16,   // group barrier: count, then generation
  kCtrlWords = kCtrlBarrier + 32
};
constexpr uint32_t kFlagStride = SNAC_FLAG_STRIDE;  // uint64 words between flags (128 B)
constexpr uint32_t kUserFlags = 1024;               // flags handed to device-side users
// Tile-counter slots per context: consecutive collective calls take
// consecutive slots, so that calls in flight at once rarely share one.
constexpr uint32_t kPoolSlots = 64;
constexpr uint32_t kPoolMaxCounters = 8;
constexpr uint32_t kPoolSlotWords = (kPoolMaxCounters + 1) * kFlagStride;  // counters, then done, a line each

// workgroups per CU of a pipeline launch under cfg
int pipe_wgs_per_cu(const LaunchCfg& cfg);
hipError_t launch_pipeline(const PipeArgs& a, int dtype_bf16, const LaunchCfg& cfg, hipStream_t stream,
                           uint32_t* grid_out);

// Fill `n` uint64 words with `v` (a kernel, so it may sit inside a captured
// graph, unlike a memset node).
hipError_t fill_u64(uint64_t* p, uint64_t n, uint64_t v, hipStream_t stream);

int device_cu_count();

// The static device array of snac_all_reduce_atomic_static (noalloc.hip):
// its size, and its address on the current device (looked up once per
// device with hipGetSymbolAddress, then kept).
constexpr uint64_t kStaticScratchBytes = 32ull << 20;
hipError_t static_scratch(float** out);

// HBM ceiling probes (probes.hip): kind 0 read, 1 write, 2 copy.
hipError_t launch_probe(int kind, void* dst, const void* src, uint64_t bytes, int threads, int tile_bytes,
                        int wgs_per_cu, uint32_t magic, hipStream_t stream);

}  // namespace snac
