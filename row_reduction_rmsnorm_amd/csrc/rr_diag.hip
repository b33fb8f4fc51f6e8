// Diagnostic kernels of librowreduce_diag.so (not linked into the product
// library librowreduce.so): the wave64 all-reduce self-test and a plain
// streaming copy used as a measurement reference.  The diagnostics build
// links the product's kernel object unchanged and adds these.
#include "rr_device.h"
#include "rr_launch.h"

namespace rr {

namespace {

inline dim3 grid1(int64_t g) { return dim3((unsigned)g, 1, 1); }

// ===========================================================================
// self-test of the wave all-reduce: one wavefront per 64-value group
// ===========================================================================
__global__ __launch_bounds__(64) void selftest_wave_kernel(const float* in, float* out, int kind) {
  const int64_t gidx = blockIdx.x;
  const int lane = threadIdx.x;
  if (kind == 0) {
    out[gidx * 64 + lane] = wave_sum(in[gidx * 64 + lane]);
  } else if (kind == 1) {
    out[gidx * 64 + lane] = wave_max(in[gidx * 64 + lane]);
  } else {
    MD p;
    p.m = in[gidx * 128 + lane];
    p.d = in[gidx * 128 + 64 + lane];
    p = wave_md(p);
    out[gidx * 128 + lane] = p.m;
    out[gidx * 128 + 64 + lane] = p.d;
  }
}

// ===========================================================================
// streaming copy (a measurement reference, not an operation of the pages):
// one 16-byte vector per lane per step, non-temporal loads and stores, no
// dependency between lanes.  The grid covers the copy in one step unless it
// was capped (then workgroups stride by the grid).
// ===========================================================================
template <int BS>
__global__ __launch_bounds__(BS) void stream_copy_kernel(const u32x4_t* __restrict__ src,
                                                         u32x4_t* __restrict__ dst, int64_t nvec) {
  const int64_t stride = (int64_t)gridDim.x * BS;
  for (int64_t i = (int64_t)blockIdx.x * BS + threadIdx.x; i < nvec; i += stride)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

}  // namespace

hipError_t launch_selftest_wave(const float* in, float* out, int64_t count, int kind,
                                hipStream_t stream) {
  selftest_wave_kernel<<<grid1(count), dim3(64), 0, stream>>>(in, out, kind);
  return hipGetLastError();
}

hipError_t launch_stream_copy(void* dst, const void* src, int64_t bytes, hipStream_t stream) {
  const int64_t nvec = bytes / 16;
  const u32x4_t* s = static_cast<const u32x4_t*>(src);
  u32x4_t* d = static_cast<u32x4_t*>(dst);
  // 1024-lane groups measured fastest below 1 GiB, 256-lane groups above;
  // the grid is capped so that a dispatch's work-items fit in 32 bits
  if (bytes < ((int64_t)1 << 30)) {
    const int64_t grid = (nvec + 1023) / 1024;
    stream_copy_kernel<1024><<<grid1(grid < (1 << 22) ? grid : (1 << 22)), dim3(1024), 0, stream>>>(s, d, nvec);
  } else {
    const int64_t grid = (nvec + 255) / 256;
    stream_copy_kernel<256><<<grid1(grid < (1 << 24) ? grid : (1 << 24)), dim3(256), 0, stream>>>(s, d, nvec);
  }
  return hipGetLastError();
}

}  // namespace rr
