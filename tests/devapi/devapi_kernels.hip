// devapi_kernels.hip -- kernels that use the device-side API of
// include/snac_device.hpp the way a user's kernel would, with plain C
// launchers for the GPU tests (tests/test_gpu_device_api.py).  Test
// infrastructure: built into tests/devapi/libsnac_devtest.so.
//
// Every launcher checks its grid against what the device can run at once
// (the device-side collective and group barrier need co-resident
// workgroups) and returns a hipError_t (or -1 for that check).
#include <hip/hip_runtime.h>

#include "snac_device.hpp"

namespace {

using Atom = snac::Atom<950>;
constexpr int TH = Atom::THREADS;
// dynamic LDS of every kernel here that calls a collective: the workspace
// the launch contract names
constexpr uint32_t LDS = Atom::PIPELINE_LDS_BYTES;

int fits(const void* fn, int grid, uint32_t lds = LDS) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, TH, lds) != hipSuccess) return 0;
  return grid <= per_cu * cus;
}

// ---- workgroup Atoms: block b handles slice b (the copy sample's shape)

__global__ __launch_bounds__(TH) void copy_slices_kernel(char* dst, const char* src, uint64_t bytes_per_block) {
  const uint64_t off = (uint64_t)blockIdx.x * bytes_per_block;
  snac::copy(dst + off, src + off, bytes_per_block);
}

template <typename T, int N>
__global__ __launch_bounds__(TH) void reduce_slices_kernel(snac_coll_desc bufs, uint64_t count_per_block) {
  // bufs.src / bufs.dst carry the pointers; nothing else of it is used
  const uint64_t off = (uint64_t)blockIdx.x * count_per_block * T::kSize;
  const void* src[N];
  void* dst[SNAC_MAX_RANKS];
#pragma unroll
  for (int k = 0; k < N; ++k) src[k] = static_cast<const char*>(bufs.src[k]) + off;
  for (int k = 0; k < bufs.ndst; ++k) dst[k] = static_cast<char*>(bufs.dst[k]) + off;
  snac::reduce<T, N>(dst, bufs.ndst, src, count_per_block);
}

// ---- a described collective run by workgroups [0, blocks) of a larger grid

// The workspace is the launch's dynamic LDS, as in the pages' sample; with
// no_workspace the call gets a NULL workspace and must latch SNAC_E_ARG.
template <typename T, int N, bool SYNC = true>
__global__ __launch_bounds__(TH) void collective_kernel(const snac_coll_desc desc, const snac_dev_ctx ctx,
                                                        uint32_t blocks, uint32_t coll_blocks, int no_workspace,
                                                        uint32_t* ok_out) {
  extern __shared__ __align__(128) char workspace[];
  if (blockIdx.x >= blocks) return;  // workgroups doing "other work"
  const snac_args args{&desc, no_workspace ? nullptr : workspace, blocks, coll_blocks, blockIdx.x};
  const bool ok = snac::collective<T, N, TH, snac::kCacheStream, SYNC>(args, ctx);
  if (threadIdx.x == 0) ok_out[blockIdx.x] = ok ? 1u : 0u;
}

// ---- compute, in-kernel AllReduce, compute on the result
//
// Phase 1: every workgroup computes y_r = 0.5 * x_r + r (binary32, rounded
// to T) for its slice of every rank into tmp[r]; all workgroups meet.
// Phase 2: AllReduce tmp -> out inside the kernel (desc describes it).
// Phase 3: every workgroup copies a slice of out[0] -- written by other
// workgroups in phase 2 -- into check.

template <typename T>
__device__ void scale_slice(const char* x, char* y, uint64_t first, uint64_t n, float r) {
  for (uint64_t i = first + threadIdx.x; i < first + n; i += TH)
    snac::store_elem<T>(y + i * T::kSize, snac::load_elem<T>(x + i * T::kSize) * 0.5f + r);
}

template <typename T, int N>
__global__ __launch_bounds__(TH) void fused_kernel(const snac_coll_desc desc, const snac_dev_ctx ctx,
                                                   snac_coll_desc xs, uint64_t count, char* check,
                                                   uint32_t* ok_out) {
  extern __shared__ __align__(128) char workspace[];
  const uint32_t blocks = gridDim.x;
  const uint64_t per = (count + blocks - 1) / blocks;
  const uint64_t first = (uint64_t)blockIdx.x * per;
  const uint64_t n = first >= count ? 0 : (count - first < per ? count - first : per);
  for (int r = 0; r < N; ++r)
    scale_slice<T>(static_cast<const char*>(xs.src[r]), static_cast<char*>(const_cast<void*>(desc.src[r])), first, n,
                   (float)r);
  // the workspace is free until the collective: its first word carries the
  // barrier's verdict, so the kernel declares no LDS of its own
  bool ok = snac::group_barrier(ctx, blocks, reinterpret_cast<uint32_t*>(workspace));
  const snac_args args{&desc, workspace, blocks, blocks, blockIdx.x};
  if (ok) ok = snac::collective<T, N, TH>(args, ctx);
  if (ok) {
    // read another workgroup's part of the result: slice (b + 1) mod blocks
    const uint32_t other = (blockIdx.x + 1) % blocks;
    const uint64_t f2 = (uint64_t)other * per;
    const uint64_t n2 = f2 >= count ? 0 : (count - f2 < per ? count - f2 : per);
    snac::copy(check + f2 * T::kSize, static_cast<const char*>(desc.dst[0]) + f2 * T::kSize, n2 * T::kSize);
  }
  if (threadIdx.x == 0) ok_out[blockIdx.x] = ok ? 1u : 0u;
}

// ---- the public SNAC primitives, stage / notify / consume by hand
//
// Workgroups p < n are producers: round r copies block r of x_p into rank
// p's staging slot r % S (after waiting for the consumer to free it) and
// notifies ready[p][slot] = base + r + 1.  The last workgroup is the
// consumer: it consumes all n ready flags of the slot, reduces the n staged
// blocks in rank order into out[r], and notifies free[slot].  User flags:
// ready[p][slot] at p * S + slot, free[slot] at n * S + slot.

__global__ __launch_bounds__(TH) void flags_kernel(const snac_dev_ctx ctx, snac_coll_desc xs, float* stage, float* out,
                                                   int n, uint32_t S, uint32_t R, uint32_t B, uint64_t base,
                                                   uint32_t* ok_out) {
  const snac::WaitCtl w = snac::wait_ctl(ctx);
  constexpr uint64_t F = SNAC_FLAG_STRIDE;
  bool ok = true;
  if ((int)blockIdx.x < n) {
    const int p = blockIdx.x;
    for (uint32_t r = 0; r < R && ok; ++r) {
      const uint32_t slot = r % S;
      if (r >= S) ok = snac::consume(ctx.flags + ((uint64_t)n * S + slot) * F, 1, F, base + r - S + 1, w);
      if (!ok) break;
      float* dst = stage + ((uint64_t)p * S + slot) * B;
      const float* src = static_cast<const float*>(xs.src[p]) + (uint64_t)r * B;
      snac::stage(dst, src, (uint64_t)B * sizeof(float));
      snac::notify(ctx.flags + ((uint64_t)p * S + slot) * F, base + r + 1);
    }
  } else {
    for (uint32_t r = 0; r < R && ok; ++r) {
      const uint32_t slot = r % S;
      ok = snac::consume(ctx.flags + (uint64_t)slot * F, n, (uint64_t)S * F, base + r + 1, w);
      if (!ok) break;
      for (uint32_t i = threadIdx.x; i < B; i += TH) {
        float acc = stage[(uint64_t)slot * B + i];
        for (int p = 1; p < n; ++p) acc = acc + stage[((uint64_t)p * S + slot) * B + i];
        out[(uint64_t)r * B + i] = acc;
      }
      snac::notify(ctx.flags + ((uint64_t)n * S + slot) * F, base + r + 1);
    }
  }
  if (threadIdx.x == 0) ok_out[blockIdx.x] = ok ? 1u : 0u;
}

// ---- one consumer of many flags
//
// Workgroups k < K each store vals[k] = k + 1 and notify user flag k =
// target; the last workgroup consumes all K flags at once (more than one
// wave's worth when K > 64), then sums vals[] -- every value must be the
// producer's, made visible by its release and the consumer's acquire.

__global__ __launch_bounds__(TH) void many_flags_kernel(const snac_dev_ctx ctx, uint32_t* vals, int K, uint64_t target,
                                                        uint64_t* sum_out, uint32_t* ok_out) {
  const snac::WaitCtl w = snac::wait_ctl(ctx);
  constexpr uint64_t F = SNAC_FLAG_STRIDE;
  if ((int)blockIdx.x < K) {
    if (threadIdx.x == 0) vals[blockIdx.x] = blockIdx.x + 1u;
    snac::notify(ctx.flags + (uint64_t)blockIdx.x * F, target);
    if (threadIdx.x == 0) ok_out[blockIdx.x] = 1u;
    return;
  }
  const bool ok = snac::consume(ctx.flags, K, F, target, w);
  if (threadIdx.x == 0) {
    uint64_t sum = 0;
    for (int k = 0; k < K; ++k) sum += vals[k];
    *sum_out = sum;
    ok_out[K] = ok ? 1u : 0u;
  }
}

// N dispatch tables (N in {1, 2, 3, 4, 8, 16})
#define SNAC_DISPATCH_N(MACRO) MACRO(1) MACRO(2) MACRO(3) MACRO(4) MACRO(8) MACRO(16)

}  // namespace

extern "C" {

int devtest_copy_slices(void* dst, const void* src, uint64_t bytes_per_block, int blocks, hipStream_t s) {
  if (blocks <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(copy_slices_kernel, dim3(blocks), dim3(TH), 0, s, static_cast<char*>(dst),
                     static_cast<const char*>(src), bytes_per_block);
  return hipGetLastError();
}

// bufs: ndst and src[0..nsrc) / dst[0..ndst) set by the caller
int devtest_reduce_slices(const snac_coll_desc* bufs, int nsrc, uint64_t count_per_block, int blocks, int bf16,
                          hipStream_t s) {
  if (blocks <= 0 || !bufs || bufs->ndst < 1 || bufs->ndst > SNAC_MAX_RANKS) return hipErrorInvalidValue;
#define SNAC_CASE(NN)                                                                                         \
  case NN:                                                                                                    \
    if (bf16)                                                                                                 \
      hipLaunchKernelGGL((reduce_slices_kernel<snac::BF16, NN>), dim3(blocks), dim3(TH), 0, s, *bufs,         \
                         count_per_block);                                                                    \
    else                                                                                                      \
      hipLaunchKernelGGL((reduce_slices_kernel<snac::F32, NN>), dim3(blocks), dim3(TH), 0, s, *bufs,          \
                         count_per_block);                                                                    \
    break;
  switch (nsrc) {
    SNAC_DISPATCH_N(SNAC_CASE)
    default: return hipErrorInvalidValue;
  }
#undef SNAC_CASE
  return hipGetLastError();
}

// Runs `desc` with workgroups [0, blocks) of a grid of blocks + extra;
// template arguments from (bf16, nsrc) -- deliberately taken from the
// caller, so a test can pass a mismatch.  ok_out[b] = 1 where it returned
// true.
int devtest_collective(const snac_coll_desc* desc, const snac_dev_ctx* ctx, int bf16, int nsrc, int blocks,
                       int coll_blocks, int extra, int no_workspace, uint32_t* ok_out, hipStream_t s) {
  if (!desc || !ctx || blocks <= 0 || coll_blocks < 0 || extra < 0) return hipErrorInvalidValue;
  const int grid = blocks + extra;
  const void* fn = nullptr;
#define SNAC_CASE(NN)                                                                                           \
  case NN:                                                                                                      \
    fn = bf16 ? (const void*)&collective_kernel<snac::BF16, NN> : (const void*)&collective_kernel<snac::F32, NN>; \
    break;
  switch (nsrc) {
    SNAC_DISPATCH_N(SNAC_CASE)
    default: return hipErrorInvalidValue;
  }
#undef SNAC_CASE
  if (!fits(fn, grid)) return -1;
#define SNAC_CASE(NN)                                                                                      \
  case NN:                                                                                                 \
    if (bf16)                                                                                              \
      hipLaunchKernelGGL((collective_kernel<snac::BF16, NN>), dim3(grid), dim3(TH), LDS, s, *desc, *ctx,   \
                         (uint32_t)blocks, (uint32_t)coll_blocks, no_workspace, ok_out);                   \
    else                                                                                                   \
      hipLaunchKernelGGL((collective_kernel<snac::F32, NN>), dim3(grid), dim3(TH), LDS, s, *desc, *ctx,    \
                         (uint32_t)blocks, (uint32_t)coll_blocks, no_workspace, ok_out);                   \
    break;
  switch (nsrc) {
    SNAC_DISPATCH_N(SNAC_CASE)
    default: return hipErrorInvalidValue;
  }
#undef SNAC_CASE
  return hipGetLastError();
}

// The same without the closing grid barrier (SYNC = false): all `blocks`
// workgroups move data, need not be co-resident, and the output is checked
// after the kernel.
int devtest_collective_nosync(const snac_coll_desc* desc, const snac_dev_ctx* ctx, int bf16, int nsrc, int blocks,
                              uint32_t* ok_out, hipStream_t s) {
  if (!desc || !ctx || blocks <= 0) return hipErrorInvalidValue;
#define SNAC_CASE(NN)                                                                                       \
  case NN:                                                                                                  \
    if (bf16)                                                                                               \
      hipLaunchKernelGGL((collective_kernel<snac::BF16, NN, false>), dim3(blocks), dim3(TH), LDS, s, *desc, \
                         *ctx, (uint32_t)blocks, (uint32_t)blocks, 0, ok_out);                              \
    else                                                                                                    \
      hipLaunchKernelGGL((collective_kernel<snac::F32, NN, false>), dim3(blocks), dim3(TH), LDS, s, *desc,  \
                         *ctx, (uint32_t)blocks, (uint32_t)blocks, 0, ok_out);                              \
    break;
  switch (nsrc) {
    SNAC_DISPATCH_N(SNAC_CASE)
    default: return hipErrorInvalidValue;
  }
#undef SNAC_CASE
  return hipGetLastError();
}

// desc: AllReduce tmp -> out (snac_describe); xs.src[r]: the inputs x_r.
int devtest_fused_scale_allreduce(const snac_coll_desc* desc, const snac_dev_ctx* ctx, const snac_coll_desc* xs,
                                  uint64_t count, void* check, int blocks, uint32_t* ok_out, hipStream_t s) {
  if (!desc || !ctx || !xs || blocks <= 0) return hipErrorInvalidValue;
  const int n = desc->nsrc;
  const bool bf16 = desc->esize == 2;
  const void* fn = nullptr;
#define SNAC_CASE(NN)                                                                                  \
  case NN:                                                                                             \
    fn = bf16 ? (const void*)&fused_kernel<snac::BF16, NN> : (const void*)&fused_kernel<snac::F32, NN>; \
    break;
  switch (n) {
    SNAC_DISPATCH_N(SNAC_CASE)
    default: return hipErrorInvalidValue;
  }
#undef SNAC_CASE
  if (!fits(fn, blocks)) return -1;
#define SNAC_CASE(NN)                                                                                          \
  case NN:                                                                                                     \
    if (bf16)                                                                                                  \
      hipLaunchKernelGGL((fused_kernel<snac::BF16, NN>), dim3(blocks), dim3(TH), LDS, s, *desc, *ctx, *xs,      \
                         count, static_cast<char*>(check), ok_out);                                            \
    else                                                                                                       \
      hipLaunchKernelGGL((fused_kernel<snac::F32, NN>), dim3(blocks), dim3(TH), LDS, s, *desc, *ctx, *xs,      \
                         count, static_cast<char*>(check), ok_out);                                            \
    break;
  switch (n) {
    SNAC_DISPATCH_N(SNAC_CASE)
    default: return hipErrorInvalidValue;
  }
#undef SNAC_CASE
  return hipGetLastError();
}

// n producers + 1 consumer over S slots for R rounds of B floats; stage
// holds n * S * B floats, out R * B, ok_out n + 1 words; flags from
// base + 1 upward (base must exceed every value the flags already hold).
int devtest_flags(const snac_dev_ctx* ctx, const snac_coll_desc* xs, float* stage, float* out, int n, uint32_t S,
                  uint32_t R, uint32_t B, uint64_t base, uint32_t* ok_out, hipStream_t s) {
  if (!ctx || !xs || n < 1 || n > SNAC_MAX_RANKS || S < 1 || ((uint64_t)n + 1) * S > ctx->nflags)
    return hipErrorInvalidValue;
  if (!fits((const void*)&flags_kernel, n + 1, 0)) return -1;
  hipLaunchKernelGGL(flags_kernel, dim3(n + 1), dim3(TH), 0, s, *ctx, *xs, stage, out, n, S, R, B, base, ok_out);
  return hipGetLastError();
}

int devtest_many_flags(const snac_dev_ctx* ctx, uint32_t* vals, int K, uint64_t target, uint64_t* sum_out,
                       uint32_t* ok_out, hipStream_t s) {
  if (!ctx || K < 1 || (uint64_t)K > ctx->nflags) return hipErrorInvalidValue;
  if (!fits((const void*)&many_flags_kernel, K + 1, 0)) return -1;
  hipLaunchKernelGGL(many_flags_kernel, dim3(K + 1), dim3(TH), 0, s, *ctx, vals, K, target, sum_out, ok_out);
  return hipGetLastError();
}

// The launch contract as the header publishes it: out[0] = THREADS,
// out[1] = PIPELINE_LDS_BYTES, out[2] = COPY_LDS_BYTES, out[3] =
// REDUCE_LDS_BYTES, out[4] = COLLECTIVE_LDS_BYTES.
int devtest_atom_contract(uint32_t* out) {
  if (!out) return hipErrorInvalidValue;
  out[0] = (uint32_t)Atom::THREADS;
  out[1] = Atom::PIPELINE_LDS_BYTES;
  out[2] = Atom::COPY_LDS_BYTES;
  out[3] = Atom::REDUCE_LDS_BYTES;
  out[4] = Atom::COLLECTIVE_LDS_BYTES;
  return hipSuccess;
}

// Static LDS (bytes the kernel declares itself, beyond the dynamic
// workspace) of the collective test kernels: which 0 = collective_kernel
// <BF16, 8>, 1 = collective_kernel<F32, 1>, 2 = fused_kernel<BF16, 8>,
// 3 = copy_slices_kernel.
int devtest_static_lds(int which, uint32_t* out) {
  const void* fn = nullptr;
  switch (which) {
    case 0: fn = (const void*)&collective_kernel<snac::BF16, 8>; break;
    case 1: fn = (const void*)&collective_kernel<snac::F32, 1>; break;
    case 2: fn = (const void*)&fused_kernel<snac::BF16, 8>; break;
    case 3: fn = (const void*)&copy_slices_kernel; break;
    default: return hipErrorInvalidValue;
  }
  hipFuncAttributes attr;
  const hipError_t e = hipFuncGetAttributes(&attr, fn);
  if (e != hipSuccess) return e;
  *out = (uint32_t)attr.sharedSizeBytes;
  return hipSuccess;
}

}  // extern "C"
