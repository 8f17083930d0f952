/*
 * snac.h -- C ABI of the copy / N-to-1 reduce collective datapath for AMD
 * Instinct MI355X (gfx950).
 *
 * The library runs single-kernel collectives over N "logical ranks" whose
 * source, destination, staging and signal buffers all live in one GPU's HBM.
 * Underneath every collective are two data-movement primitives (Atoms):
 * copy, and N-to-1 reduce, which combines several input buffers into one
 * output (Purlin 0.6.4 project description, "# Purlin").  A per-collective
 * layout says which Atom runs on which byte ranges ("Key Idea": layouts
 * describe the collective, SNAC coordinates execution, Atoms move the data).
 *
 * Conventions for every entry point:
 *   - Pointers named src/dst/x/out are device pointers the caller owns; the
 *     library never allocates per call.  A buffer whose extent is zero (a
 *     rank with a zero count in a V collective) may be NULL.  Pointer arrays (src[], dst[],
 *     counts[]) are host arrays read during the call, before it returns.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL is the null
 *     stream).  Buffers must stay alive until the stream has passed the call.
 *   - Argument errors are reported synchronously (SNAC_E_ARG) and nothing is
 *     enqueued.  A buffer extent or V count above SNAC_MAX_BYTES bytes (or
 *     elements), far beyond any GPU's memory, is an argument error, so that
 *     no extent or offset the checks compute can wrap.  Errors detected on the device (a consumer that waited too
 *     long, an abort) latch in the context's status word; snac_check() and
 *     snac_finalize() report them.
 *   - A context is used from one host thread and one stream at a time.
 *     Different contexts may be used from different threads at once.
 *     (Long collective calls hand out their tiles from counters in the
 *     context; consecutive calls take different counters, 64 in turn, so
 *     calls of one context must not run 64 or more at a time, nor two
 *     replays of one captured graph at once.)  The process-wide tuning
 *     (snac_set_tuning, the rule table) may be changed from any thread;
 *     every call uses one consistent copy of it.
 *   - Reductions accumulate in binary32 in rank order 0..N-1 starting from
 *     the rank-0 value and round once to the output type (bf16:
 *     round-to-nearest-even).  Results are therefore bitwise repeatable, the
 *     deterministic mode of Purlin 0.6.5 ("Reduction determinism");
 *     snac_all_reduce_ex also offers a non-deterministic (float-atomic) mode.
 *   - No C++ exception crosses this interface.
 */
#ifndef SNAC_H
#define SNAC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SNAC_ABI_VERSION 3
#define SNAC_MAX_RANKS 16
/* largest buffer extent (bytes) or V count (elements) a call accepts: 1 TiB */
#define SNAC_MAX_BYTES (1ull << 40)

typedef enum snac_status {
  SNAC_OK = 0,
  SNAC_E_ARG = 1,         /* invalid argument; nothing was enqueued */
  SNAC_E_UNSUPPORTED = 2, /* valid request the library does not implement */
  SNAC_E_NOMEM = 3,       /* device allocation failed (snac_init only) */
  SNAC_E_HIP = 4,         /* a HIP runtime call failed */
  SNAC_E_TIMEOUT = 5,     /* a device-side wait exceeded its spin limit */
  SNAC_E_STATE = 6,       /* context unusable (aborted, or wrong device) */
  SNAC_E_ABORTED = 7      /* device-side waits were abandoned by snac_abort */
} snac_status;

typedef enum snac_dtype {
  SNAC_BYTE = 0, /* 1-byte opaque element: copy-only collectives */
  SNAC_U32 = 1,  /* 4-byte opaque element: copy-only collectives */
  SNAC_F32 = 2,  /* IEEE binary32 */
  SNAC_BF16 = 3  /* bfloat16 (upper half of a binary32) */
} snac_dtype;

typedef enum snac_coll {
  SNAC_COLL_ALL_REDUCE = 0,
  SNAC_COLL_REDUCE_SCATTER = 1,
  SNAC_COLL_ALL_GATHER = 2,
  SNAC_COLL_ALL_TO_ALL = 3,
  SNAC_COLL_ALL_GATHER_V = 4,
  SNAC_COLL_REDUCE_SCATTER_V = 5,
  SNAC_COLL_ALL_TO_ALL_V = 6
} snac_coll;

typedef void* snac_stream; /* hipStream_t */
typedef struct snac_ctx snac_ctx;

/*
 * snac_coll_desc -- one collective call, validated and laid out: what the
 * collective kernels take as their argument, and what a user kernel points
 * to from the snac_args it passes to snac::collective()
 * (include/snac_device.hpp) to run the same collective inside its own grid.
 * Filled by snac_describe(); plain data, so it can be copied into a kernel
 * argument by value (2336 bytes).
 */
#define SNAC_MAX_COUNTS (SNAC_MAX_RANKS * SNAC_MAX_RANKS)
#define SNAC_DESC_ALIGNED 1 /* flags: every job's addresses and length are 16-byte aligned */
typedef struct snac_coll_desc {
  int32_t coll;            /* snac_coll value (internal Atom kinds use 100, 101) */
  int32_t nsrc;            /* source buffers (= N for collectives) */
  int32_t ndst;            /* destination buffers (= N for collectives) */
  int32_t esize;           /* element size in bytes */
  int32_t split_multicast; /* multicast jobs split into one job per destination */
  int32_t flags;           /* SNAC_DESC_* bits */
  uint64_t bytes;          /* per-rank input bytes (fixed-size collectives) */
  const void* src[SNAC_MAX_RANKS];
  void* dst[SNAC_MAX_RANKS];
  uint64_t counts[SNAC_MAX_COUNTS]; /* V collectives: element counts */
} snac_coll_desc;

/*
 * snac_dev_ctx -- what device code needs of a context: the signal words and
 * the staging rings, for kernels that use the device-side API of
 * include/snac_device.hpp.  Filled by snac_get_device_context(); plain data,
 * passed to a kernel by value.  The pointers stay valid until
 * snac_finalize().  (Purlin 0.6.5 "Samples": the host-created context is
 * passed to the kernel, which hands it to the collective.)
 */
#define SNAC_FLAG_STRIDE 16 /* uint64 words between flags: one 128-byte line each */
typedef struct snac_dev_ctx {
  int32_t nranks;
  uint32_t spin_limit_log2;   /* device waits give up after 2^k polls */
  uint64_t* status;           /* first device error latched here; snac_check() reports and clears it */
  const uint32_t* abort_word; /* host-mapped; nonzero after snac_abort() */
  uint64_t* barrier;          /* two words (count, generation) for snac::group_barrier */
  uint64_t* flags;            /* user SNAC flags: flag i at flags + i * SNAC_FLAG_STRIDE; zero after
                                 snac_init and after a re-arming snac_check; the library never writes them */
  uint32_t nflags;            /* number of user flags */
  uint32_t reserved;
  char* staging;              /* rank r's staging ring at staging + r * staging_bytes */
  uint64_t staging_bytes;     /* per rank; shared with snac_pipeline_scale_reduce (not concurrently) */
} snac_dev_ctx;

/* ------------------------------------------------------------------ info */

/* ABI version of the loaded library (SNAC_ABI_VERSION at build time). */
int snac_abi_version(void);

/* Static string naming a status code; never NULL. */
const char* snac_status_str(snac_status s);

/* Human-readable detail of the last error returned to this host thread
 * (empty string when none).  The pointer stays valid until the next call
 * on this thread. */
const char* snac_last_error(void);

/* ------------------------------------------------------------- context */

/*
 * snac_init -- create a context for `nranks` logical ranks on the current
 * HIP device (Purlin 0.6.5 "Host-side": create a context once with symmetric
 * staging and signal buffers and reuse it for every collective).
 *
 *   nranks                  1 .. SNAC_MAX_RANKS
 *   staging_bytes_per_rank  size of each rank's staging ring, used by the
 *                           device-side SNAC pipeline and as the accumulator
 *                           of the atomic AllReduce mode.  0 selects the
 *                           default (64 MiB).  It is split into slots of the
 *                           pipeline tile size: the tuning value if set,
 *                           else the largest power of two up to 2 MiB that
 *                           leaves at least 64 slots (minimum 4 KiB).  Without
 *                           a tuning value a call re-cuts the same ring for
 *                           about one producer item per workgroup (N * tiles
 *                           ~ workgroups): it merges slots into tiles of up to
 *                           16 MiB while the message fits the ring, and
 *                           splits them down to 64 KiB while there are fewer
 *                           tiles than that.  The size must be
 *                           a multiple of the tile and give at least 2
 *                           slots.  A ring that holds a whole message runs
 *                           fastest.
 *   stream                  signals are cleared on this stream.
 *   out                     receives the context; on error *out is NULL.
 *
 * The context owns its workspace: staging[nranks][slots][tile] and the
 * signal area (one 128-byte line per ready flag, per free flag, per control
 * word and per tile counter of the collectives' shared tile schedule).  Errors: SNAC_E_ARG (bad nranks/size/out), SNAC_E_NOMEM,
 * SNAC_E_HIP.
 */
snac_status snac_init(int nranks, size_t staging_bytes_per_rank, snac_stream stream, snac_ctx** out);

/*
 * snac_finalize -- wait for `stream`, report any latched device error, and
 * free the workspace (Purlin 0.6.5 "Host-side": finalize frees the internal
 * buffers after the last collective).  NULL ctx is a no-op returning
 * SNAC_OK.  The context is freed even when an error is returned.
 */
snac_status snac_finalize(snac_ctx* ctx, snac_stream stream);

/*
 * snac_check -- synchronise `stream`, read the context's device status word
 * and clear it.  Returns SNAC_OK, or the latched code: SNAC_E_TIMEOUT,
 * SNAC_E_ABORTED, or SNAC_E_ARG (a device-side collective whose template
 * arguments did not match its descriptor).  A latched error also re-arms
 * the context: every signal word (flags, barrier, tickets) is cleared.
 */
snac_status snac_check(snac_ctx* ctx, snac_stream stream);

/* Number of logical ranks of a context (0 for NULL). */
int snac_ctx_nranks(const snac_ctx* ctx);

/*
 * snac_abort -- ask every device-side wait of this context to give up.  Sets
 * a word in host-mapped memory that waiting workgroups poll; they exit
 * without finishing their tile and latch SNAC_E_ABORTED.  Safe to call while
 * a kernel runs.  snac_check() then reports SNAC_E_ABORTED and re-arms the
 * context (clears the word and the signal state on its stream).
 */
snac_status snac_abort(snac_ctx* ctx);

/* ---------------------------------------------------------------- Atoms */

/*
 * snac_copy -- the copy Atom: dst[0..bytes) = src[0..bytes), byte for byte
 * (Purlin 0.6.5 "Samples": an Atom copies a slice from src to dst).  Any
 * alignment and length; bytes == 0 is a no-op.  The ranges must not
 * overlap (SNAC_E_ARG).  No context is needed.
 */
snac_status snac_copy(void* dst, const void* src, size_t bytes, snac_stream stream);

/*
 * snac_reduce_n -- the N-to-1 reduce Atom (Purlin 0.6.4 "# Purlin": it
 * combines several input buffers into one output), writing the result to
 * one or more outputs:
 *     for d < ndst, i < count:  dst[d][i] = R(src[0][i] + ... + src[nsrc-1][i])
 * summed in binary32 in index order, R = output rounding (identity for F32,
 * round-to-nearest-even for BF16).
 *   dst, ndst   1 <= ndst <= SNAC_MAX_RANKS output pointers
 *   src, nsrc   1 <= nsrc <= SNAC_MAX_RANKS input pointers
 *   count       elements per buffer (0 is a no-op)
 *   dtype       SNAC_F32 or SNAC_BF16
 * Every pointer must be aligned to the element size.  An output may equal
 * an input (in place); any other overlap is SNAC_E_ARG.
 */
snac_status snac_reduce_n(void* const* dst, int ndst, const void* const* src, int nsrc, size_t count,
                          snac_dtype dtype, snac_stream stream);

/* ---------------------------------------------------- measurement probes */

typedef enum snac_probe_kind {
  SNAC_PROBE_READ = 0,    /* read src[0, bytes) */
  SNAC_PROBE_WRITE = 1,   /* write dst[0, bytes) */
  SNAC_PROBE_COPY = 2,    /* dst[0, bytes) = src[0, bytes): one read and one write per byte */
  SNAC_PROBE_ORDERED = 8  /* or'ed into a kind: after 8 grid-stride rounds the tiles are handed out in
                             order from 4 counters, as the collectives' long launches take them */
} snac_probe_kind;

/*
 * snac_hbm_probe -- a measurement helper, not one of the collectives and
 * not from the pages: the plainest HBM stream of one kind, to measure on
 * the machine at hand the ceilings the collective kernels are judged
 * against (read-only, write-only and 1:1 read/write rates).  It uses the
 * collectives' access primitives: 16-byte buffer loads and stores with the
 * streaming hint over grid-stride tiles of `tile_bytes` per workgroup
 * iteration, `wgs_per_cu` workgroups per CU of `threads` threads.
 *   kind        SNAC_PROBE_READ, _WRITE or _COPY, optionally | SNAC_PROBE_ORDERED
 *               (its counters are a static device array of the library:
 *               ordered probes must not run at the same time on one GPU)
 *   dst         WRITE/COPY: output of `bytes`; READ: a 4-byte sink written
 *               only if the XOR of every word read equals `magic`
 *   src         READ/COPY: input of `bytes`; WRITE: unused (may be NULL)
 *   bytes       multiple of 16; dst and src 16-byte aligned; 0 is a no-op
 *   threads     64 or 256;  tile_bytes  4096 or 16384;  wgs_per_cu  1..32
 *   magic       WRITE: the 32-bit word written; READ: see dst
 * Asynchronous on `stream`; SNAC_E_ARG for anything else.  No context.
 */
snac_status snac_hbm_probe(int kind, void* dst, const void* src, size_t bytes, int threads, int tile_bytes,
                           int wgs_per_cu, uint32_t magic, snac_stream stream);

/* ----------------------------------------------------------- collectives
 *
 * Every collective takes ctx (which fixes N = snac_ctx_nranks(ctx)), an array
 * of N source pointers and an array of N destination pointers, one per
 * logical rank, and runs as one kernel on `stream`.  Byte sizes must be
 * multiples of the element size and pointers aligned to it.  A size of zero
 * is a no-op.  Destination ranges may not overlap each other; a destination
 * may overlap a source only in the in-place forms noted per call.
 */

/*
 * snac_all_reduce -- AllReduce(sum): every dst[r] receives the reduction of
 * all src[0..N-1] (NKI Collective Communication Kernels API,
 * all_reduce_hbm_kernel and its worked example; Purlin 0.6.5 "Host-side").
 *   bytes   per-rank input size = per-rank output size ("Understanding
 *           totalBytes": the input size per rank)
 *   dtype   SNAC_F32 or SNAC_BF16
 * In place: dst[r] == src[r] is allowed.
 */
snac_status snac_all_reduce(snac_ctx* ctx, const void* const* src, void* const* dst, size_t bytes,
                            snac_dtype dtype, snac_stream stream);

/*
 * Reduction modes (Purlin 0.6.5 and 0.6.4 "Reduction determinism": a
 * deterministic mode gives bitwise repeatable results; the default there is
 * non-deterministic, which lets the hardware reduce in any order).
 *
 *   SNAC_REDUCE_DETERMINISTIC  binary32 in rank order 0..N-1, one rounding:
 *                              what snac_all_reduce does.
 *   SNAC_REDUCE_ATOMIC         every rank's tile is added into a binary32
 *                              accumulator with hardware float atomics
 *                              (Iris all_reduce_atomic), in whatever order the
 *                              workgroups reach it, from +0.0; one rounding
 *                              into every destination.  The result may differ
 *                              between runs in the last bits: |result - exact
 *                              sum| <= N * 2^-24 * sum|x_k| before the final
 *                              rounding.  On one GPU it is slower than the
 *                              deterministic mode (N float atomics per
 *                              element); it exists for comparison.
 */
typedef enum snac_reduce_mode { SNAC_REDUCE_DETERMINISTIC = 0, SNAC_REDUCE_ATOMIC = 1 } snac_reduce_mode;

/*
 * snac_all_reduce_ex -- snac_all_reduce with a reduction mode.  Arguments,
 * errors and in-place rules as for snac_all_reduce.  SNAC_REDUCE_ATOMIC uses
 * the context's staging rings (N * staging_bytes_per_rank bytes) as its
 * accumulator, in chunks of up to that size / 4 elements; it must not run
 * concurrently with snac_pipeline_scale_reduce on the same context.
 */
snac_status snac_all_reduce_ex(snac_ctx* ctx, const void* const* src, void* const* dst, size_t bytes,
                               snac_dtype dtype, snac_reduce_mode mode, snac_stream stream);

/*
 * snac_all_reduce_atomic_static -- for callers that cannot allocate (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): snac_all_reduce_ex(..., SNAC_REDUCE_ATOMIC, ...) without a
 * context, allocating nothing.  Its binary32 accumulator is a static device
 * array of 32 MiB inside the library, so a message may have at most 2^23
 * elements per rank (16 MiB of bf16, 32 MiB of f32); a larger one is
 * SNAC_E_ARG and nothing is enqueued.
 *   nranks  1..SNAC_MAX_RANKS: the length of src[] and dst[]
 *   src, dst, bytes, dtype, stream, in-place rule, result bounds:
 *           as snac_all_reduce_ex in SNAC_REDUCE_ATOMIC mode
 * Every call on one GPU uses that GPU's one array (each call clears the
 * accumulator with a kernel before using it), so calls that overlap on the
 * same GPU -- on different streams, or from different host threads -- race
 * and their results are undefined; calls in stream order do not.  The first
 * call on a device looks up the array's address there (hipGetSymbolAddress)
 * and keeps it; no call allocates memory.
 */
snac_status snac_all_reduce_atomic_static(int nranks, const void* const* src, void* const* dst, size_t bytes,
                                          snac_dtype dtype, snac_stream stream);

/*
 * snac_reduce_scatter -- dst[r] (bytes/N) receives the reduction of chunk r
 * of every src, dim 0 split into N equal contiguous chunks (NKI
 * reduce_scatter_hbm_kernel).  `bytes` is the per-rank input size and must
 * be a multiple of N * element size (else SNAC_E_ARG; uneven splits use
 * snac_reduce_scatter_v).  dtype: SNAC_F32 or SNAC_BF16.
 * In place: dst[r] == src[r] + r * bytes/N is allowed.
 */
snac_status snac_reduce_scatter(snac_ctx* ctx, const void* const* src, void* const* dst, size_t bytes,
                                snac_dtype dtype, snac_stream stream);

/*
 * snac_all_gather -- dst[r] (N * bytes) receives src[0..N-1] concatenated in
 * rank order (NKI all_gather_hbm_kernel, dim 0).  `bytes` is the per-rank
 * input size.  Any dtype.  In place: src[r] == dst[r] + r * bytes.
 */
snac_status snac_all_gather(snac_ctx* ctx, const void* const* src, void* const* dst, size_t bytes,
                            snac_dtype dtype, snac_stream stream);

/*
 * snac_all_to_all -- chunk d of src[s] goes to chunk s of dst[d], chunks being
 * bytes/N contiguous bytes (NKI all_to_all_hbm_kernel: rank s sends
 * input[d, :] to rank d).  `bytes` is the per-rank input (= output) size and
 * must be a multiple of N * element size.  Any dtype.  No in-place form.
 */
snac_status snac_all_to_all(snac_ctx* ctx, const void* const* src, void* const* dst, size_t bytes,
                            snac_dtype dtype, snac_stream stream);

/*
 * snac_all_gather_v -- variable-length AllGather (Purlin 0.6.4 "# Purlin"
 * lists variable-length variants).  counts[k] (elements) is rank k's input
 * length; every dst[r] receives src[k][0..counts[k]) at element offset
 * sum_{j<k} counts[j], packed.  Zero counts are allowed.  Any dtype.
 */
snac_status snac_all_gather_v(snac_ctx* ctx, const void* const* src, void* const* dst, const size_t* counts,
                              snac_dtype dtype, snac_stream stream);

/*
 * snac_reduce_scatter_v -- variable-length ReduceScatter.  Every src holds
 * sum(counts) elements; dst[r] receives counts[r] elements, the reduction of
 * elements [D_r, D_r + counts[r]) of every src with D_r = sum_{j<r} counts[j].
 * dtype: SNAC_F32 or SNAC_BF16.
 */
snac_status snac_reduce_scatter_v(snac_ctx* ctx, const void* const* src, void* const* dst, const size_t* counts,
                                  snac_dtype dtype, snac_stream stream);

/*
 * snac_all_to_all_v -- variable-length AllToAll.  counts is an N x N
 * row-major matrix, counts[s*N + d] = elements rank s sends to rank d.  Rank
 * s's chunk for d starts at element sum_{j<d} counts[s*N+j] of src[s]; it
 * lands in dst[d] at element sum_{j<s} counts[j*N+d].  dst[d] holds
 * sum_s counts[s*N+d] elements.  Any dtype.
 */
snac_status snac_all_to_all_v(snac_ctx* ctx, const void* const* src, void* const* dst, const size_t* counts,
                              snac_dtype dtype, snac_stream stream);

/* ----------------------------------------------------- SNAC pipeline */

/*
 * snac_pipeline_scale_reduce -- a collective fused with compute inside one
 * kernel, coordinated by the Stage / Notify / And Consume protocol (Purlin
 * 0.6.4 "Key Idea"; Purlin 0.6.5 "Samples": a collective called from inside
 * a kernel between other work).  Producer workgroups compute
 * y_r = 0.5 * x[r] + r in binary32, round y_r to `dtype`, stage the tile in
 * rank r's staging slot and raise that slot's ready flag with a release
 * store.  Consumer workgroups acquire all N ready flags of a slot, N-to-1
 * reduce the staged tiles in rank order into `out`, and release the slot.
 *   x       N device pointers, each `count` elements
 *   out     one output of `count` elements
 *   dtype   SNAC_F32 or SNAC_BF16
 * The context's staging ring bounds the work in flight; any count works.
 */
snac_status snac_pipeline_scale_reduce(snac_ctx* ctx, const void* const* x, void* out, size_t count,
                                       snac_dtype dtype, snac_stream stream);

/* ----------------------------------------------------- device-side API */

/*
 * snac_get_device_context -- the device view of a context (snac_dev_ctx) for
 * kernels that call the device-side API.  Errors: SNAC_E_ARG.
 */
snac_status snac_get_device_context(const snac_ctx* ctx, snac_dev_ctx* out);

/*
 * snac_describe -- validate a collective exactly as the matching host entry
 * point would and lay it out into *out instead of launching it, for a
 * kernel that runs the collective itself with snac::collective()
 * (Purlin 0.6.5 "Samples": a collective called from inside a kernel).
 *   coll    which collective
 *   src, dst, dtype
 *           as for the host entry point
 *   bytes   per-rank input bytes (fixed-size collectives; ignored for V)
 *   counts  element counts (V collectives: N, or N*N for ALL_TO_ALL_V;
 *           ignored otherwise)
 * A request that the host call would treat as a no-op (zero bytes) gives a
 * descriptor with no jobs.  Errors: SNAC_E_ARG, SNAC_E_STATE.
 */
snac_status snac_describe(const snac_ctx* ctx, snac_coll coll, const void* const* src, void* const* dst, size_t bytes,
                          const size_t* counts, snac_dtype dtype, snac_coll_desc* out);

/* -------------------------------------------------------- layout engine */

/*
 * One unit of work of a collective: move `bytes` bytes from the source
 * buffer(s) at byte offset src_off to the destination buffer(s) at dst_off.
 * src_rank == -1 means "every rank's source buffer" (an N-to-1 reduce job);
 * dst_rank == -1 means "every rank's destination buffer" (a multicast).
 */
typedef struct snac_job {
  uint64_t src_off;
  uint64_t dst_off;
  uint64_t bytes;
  int32_t src_rank;
  int32_t dst_rank;
} snac_job;

/*
 * snac_plan -- host-only: the layout of a collective as the kernels see it
 * ("Key Idea": layouts describe how inputs and outputs are distributed and
 * whether to copy or reduce).  Runs no GPU code.
 *   coll, nranks, dtype   the collective
 *   bytes                 per-rank input size (fixed-size collectives)
 *   counts                element counts (V collectives: N for ALL_GATHER_V
 *                         and REDUCE_SCATTER_V, N*N for ALL_TO_ALL_V)
 *   jobs, max_jobs        output array; *njobs receives the job count.
 * Zero-length jobs are omitted.  Returns SNAC_E_ARG if the request is
 * invalid or more than max_jobs jobs result.
 */
snac_status snac_plan(snac_coll coll, int nranks, snac_dtype dtype, size_t bytes, const size_t* counts,
                      snac_job* jobs, int max_jobs, int* njobs);

/* --------------------------------------------------------------- tuning */

/*
 * Process-wide launch parameters (Purlin 0.6.4 "Key Idea" mentions tuning
 * for peak performance).  Zero fields select the defaults.  When the library
 * loads, the fields start from the environment variables SNAC_WGS_PER_CU,
 * SNAC_CACHE_POLICY, SNAC_PIPELINE_TILE_BYTES, SNAC_PIPELINE_LOOKAHEAD,
 * SNAC_SPIN_LIMIT_LOG2, SNAC_COPY_MULTICAST and SNAC_TILE_SCHEDULE (decimal integers; values
 * snac_set_tuning would reject are ignored).
 */
typedef struct snac_tuning {
  int32_t wgs_per_cu;      /* workgroups per compute unit in the persistent grid
                              (0: the kernel default.  Messages of at least
                              one 16 KiB tile per CU: 1 for reduces of >= 3
                              sources and more than 2 tiles per CU, 4 for
                              one-to-one copies of at most 8 tiles per CU,
                              5 single-wave workgroups for one-to-one copies
                              moving >= 1 GiB, else 2.  Smaller messages: 4
                              for reduces and AllGather(V), else 2.  The
                              pipeline: 1) */
  int32_t cache_policy;    /* 0 library default (= 1), 1 streaming (non-temporal)
                              loads and stores, 2 streaming stores only,
                              3 streaming loads only, 4 cached loads and stores */
  int32_t pipeline_tile_bytes; /* per-rank bytes per pipeline tile (multiple of
                                  4096), fixed when a context is created */
  int32_t pipeline_lookahead;  /* tiles staged ahead of the consumers (0: as
                                  many as the ring allows) */
  int32_t spin_limit_log2;     /* device waits give up after 2^k polls */
  int32_t debug_drop_notify;   /* test hook: when r+1, rank r's producers never
                                  raise their ready flags, so consumers time out */
  int32_t copy_multicast;      /* copy collectives that send one source to
                                  every destination (AllGather, AllGatherV):
                                  0 library default, 1 one job per source
                                  writing all N destinations (one read),
                                  2 one job per (source, destination) */
  int32_t debug_producer_delay; /* test hook: when > 0, a quarter of the pipeline's
                                    producer items (chosen by a hash of tile and
                                    rank) first sleep about this many microseconds,
                                    to skew producers against consumers */
  int32_t tile_schedule;       /* how a collective call's workgroups share its
                                  16 KiB tiles: 0 library default (for calls of
                                  at least 16 tiles per workgroup, grid-stride
                                  rounds and then the rest in order from 1-4
                                  counters in the context; one-to-one copies
                                  moving >= 1 GiB then also take 16 KiB tiles),
                                  1 grid-stride only, 2 the counters for every
                                  call in the 16 KiB-tile shape */
} snac_tuning;

snac_status snac_get_tuning(snac_tuning* out);
snac_status snac_set_tuning(const snac_tuning* in);

/*
 * Tuning rules: launch parameters keyed by collective, source count,
 * element size and per-rank size, so that each regime runs with the launch
 * shape measured best for it (Purlin 0.6.4 "Key Idea": extensive tuning for
 * peak performance; Purlin 0.6.5 "Device-side": tuning policies).
 *
 * A call takes the first rule that matches it; a non-zero wgs_per_cu or
 * cache_policy in the process-wide snac_tuning overrides the rule.  Rule
 * fields that are 0 keep the kernel's own default.  The built-in table
 * (restored by snac_set_tuning_rules(NULL, 0)) encodes the defaults measured
 * on MI355X; copy_reduce_snac_amd/autotune.py measures and installs a table
 * for the GPU at hand.
 *
 * Matching:
 *   coll                a snac_coll value, SNAC_RULE_ATOM_COPY (snac_copy),
 *                       SNAC_RULE_ATOM_REDUCE (snac_reduce_n),
 *                       SNAC_RULE_PIPELINE (snac_pipeline_scale_reduce),
 *                       SNAC_RULE_ANY_REDUCE (every reduce: AllReduce,
 *                       ReduceScatter(V), reduce_n), SNAC_RULE_ANY_COPY
 *                       (every copy collective and snac_copy), SNAC_RULE_ANY
 *   min_ranks..max_ranks  source buffers of the call (N; nsrc for reduce_n;
 *                       1 for snac_copy), inclusive
 *   esize               element size in bytes, 0 = any
 *   min_bytes..max_bytes  per-rank input bytes, inclusive (V collectives:
 *                       the largest per-rank input; the pipeline: count *
 *                       element size)
 */
#define SNAC_RULE_ANY (-1)
#define SNAC_RULE_ANY_REDUCE (-2)
#define SNAC_RULE_ANY_COPY (-3)
#define SNAC_RULE_ATOM_COPY 100
#define SNAC_RULE_ATOM_REDUCE 101
#define SNAC_RULE_PIPELINE 200
#define SNAC_MAX_TUNING_RULES 256

typedef struct snac_tuning_rule {
  int32_t coll;
  int32_t min_ranks;
  int32_t max_ranks;
  int32_t esize;
  uint64_t min_bytes;
  uint64_t max_bytes;
  int32_t wgs_per_cu;   /* 1..32, or 0 for the kernel's default */
  int32_t cache_policy; /* as in snac_tuning (1..4), or 0 for the default */
} snac_tuning_rule;

/* Replace the rule table (rules copied; at most SNAC_MAX_TUNING_RULES).
 * n == 0 restores the built-in table.  Errors: SNAC_E_ARG (bad field,
 * min > max, too many rules); the table is unchanged on error. */
snac_status snac_set_tuning_rules(const snac_tuning_rule* rules, int n);

/* Copy the current table to out[0..max); *n receives its length.  With
 * out == NULL only *n is set. */
snac_status snac_get_tuning_rules(snac_tuning_rule* out, int max, int* n);

/* The launch parameters a call would use (host-only, runs no GPU code):
 * the process-wide tuning with wgs_per_cu and cache_policy resolved
 * through the rules as described above. */
snac_status snac_tuning_lookup(int32_t coll, int nranks, int esize, size_t bytes, snac_tuning* out);

#ifdef __cplusplus
}
#endif

#endif /* SNAC_H */
