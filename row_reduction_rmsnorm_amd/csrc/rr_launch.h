// Internal interface between the C ABI (rr_api.cpp) and the kernels
// (rr_kernels.hip).  Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rowreduce.h"

namespace rr {

// Largest number of wavefronts one workgroup may hold (1024 threads); also
// the width of the DPP row that combines the per-wavefront LDS slots.
constexpr int kMaxWavesPerGroup = 16;

// Row strides in elements: row i of x starts at x + i * x (likewise y and
// the fused op's residual r).  A contiguous [M, N] matrix has stride N.
struct RowStrides {
  int64_t x;
  int64_t y;
  int64_t r;
};

// Arguments of the norm kernels (residual only for the fused op, beta only
// for LayerNorm and possibly null).
struct NormArgs {
  void* y;
  void* residual;
  const void* x;
  const void* gamma;
  const void* beta;
  int64_t M;
  int32_t N;
  float eps;
  RowStrides ld;
};

// Operation codes for launch_norm.
constexpr int kLaunchRms = 0;
constexpr int kLaunchFused = 1;
constexpr int kLaunchLayer = 2;

// Enqueue the norm kernel (kind: kLaunchRms, kLaunchFused or kLaunchLayer)
// that `plan` names, with `grid` workgroups, on `stream`.
hipError_t launch_norm(const rr_plan& plan, rr_dtype dtype, int kind, const NormArgs& args,
                       int64_t grid, hipStream_t stream);

// Arguments of the softmax kernels.  causal_period == 0 keeps every key;
// otherwise row r keeps keys j <= (r mod causal_period) + causal_offset.
struct SoftmaxArgs {
  void* y;
  const void* x;
  void* workspace;
  int64_t M;
  int32_t N;
  int64_t causal_period;
  int64_t causal_offset;
  int log_output;
  RowStrides ld;   // r unused
  // causal rule only: > 0 runs two rows of a period per workgroup (rows q
  // and P - 1 - q) with this many vectors per lane; 0 one row per workgroup
  int pair_nv;
  // the one-kernel split's bounded wait for another chunk's summary, in
  // ticks of the 100 MHz real-time clock (kSplitWaitTicks)
  uint64_t split_wait_ticks;
};

// LDS a cut LayerNorm row held by a workgroup takes for gamma and beta, for
// elements of `elem_bytes` bytes: fp32, one 8-byte entry per element (both
// values) plus a pad of a 64-byte frame's lead before the row and a vector
// after it; bf16, each parameter's aligned 16-byte blocks, 2 x (N + 14) / 8
// of them.  The host cuts such rows only while this is at most
// kNormLdsParamMax (bf16: up to 15353 elements, fp32: up to 7661).
constexpr size_t norm_lds_param_bytes_for(int64_t N, int elem_bytes) {
  return elem_bytes == 4 ? (size_t)(N + 64 / 4 - 1 + 4) * 8u : 2u * (size_t)((N + 14) / 8) * 16u;
}
constexpr size_t kNormLdsParamMax = 61440;

// The one-kernel split's wait: 40 us.  Its workgroups all run at once (the
// host launches it only when the device holds the whole grid), so a
// summary normally arrives within a few microseconds.
constexpr uint64_t kSplitWaitTicks = 4000;

// Enqueue the softmax kernel(s) that `plan` names (two for SPLIT).
hipError_t launch_softmax(const rr_plan& plan, rr_dtype in_dtype, rr_dtype out_dtype,
                          const SoftmaxArgs& args, int64_t grid, hipStream_t stream);

// Scratch memory of the no-allocation softmax entry point: a static device
// array of this many bytes (each device the library runs on holds its own
// copy until the process ends).  It holds the split row's (m, d) slots, 16
// bytes per chunk, i.e. up to 262144 chunks per call.
constexpr size_t kNoAllocScratchBytes = (size_t)4 << 20;

// Device address of the current device's scratch array (looked up once per
// device with hipGetSymbolAddress, then cached), or null with *err set.
void* noalloc_scratch(hipError_t* err);

// Device address of the current device's count of one-kernel split chunks
// summarised again after their wait expired (looked up as above).
unsigned int* split_fallback_counter(hipError_t* err);

// Diagnostics build only (rr_diag.hip): the wave all-reduce self-test kernel.
hipError_t launch_selftest_wave(const float* in, float* out, int64_t count, int kind,
                                hipStream_t stream);

// Diagnostics build only (rr_diag.hip): the streaming copy of `bytes` bytes
// (a positive multiple of 16, both pointers 16-byte aligned).
hipError_t launch_stream_copy(void* dst, const void* src, int64_t bytes, hipStream_t stream);

}  // namespace rr
