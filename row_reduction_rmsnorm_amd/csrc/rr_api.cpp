// C ABI of librowreduce.so: argument checks, kernel-variant choice and
// launch sizing.  The arithmetic is all in rr_kernels.hip.
//
// Variant choice by row length follows [P2] "GPU Kernel 工程（04）" section 六
// (a wavefront per row when the row fits a wavefront's registers, a workgroup
// per row for thousands of elements) and [P4] "Softmax 与归一化" section
// "按行长度选择并行方式" (several workgroups per row for very long rows with
// few rows).  The thresholds are this library's: a wavefront holds up to 32
// fp32 values per lane, a workgroup up to 16 wavefronts.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>

#include "rowreduce.h"
#include "rr_launch.h"

// RR_DIAG: the diagnostics build (librowreduce_diag.so), which adds the
// entry points of rowreduce_diag.h -- a forced kernel variant for tests and
// measurement, the all-reduce self-test and the streaming copy.  The product
// library carries none of them and keeps no process state beyond the
// calling thread's last error message.
#ifndef RR_DIAG
#define RR_DIAG 0
#endif
#if RR_DIAG
#include "rowreduce_diag.h"
#endif

namespace {

thread_local char g_err[512] = "";
#if RR_DIAG
std::atomic<int> g_override{RR_VARIANT_AUTO};
std::atomic<uint64_t> g_split_wait{rr::kSplitWaitTicks};
#endif

// The variant a call is forced to (diagnostics build), else RR_VARIANT_AUTO.
int forced_variant() {
#if RR_DIAG
  return g_override.load(std::memory_order_relaxed);
#else
  return RR_VARIANT_AUTO;
#endif
}

// The one-kernel split's bounded wait (the diagnostics build can shorten it).
uint64_t split_wait_ticks() {
#if RR_DIAG
  return g_split_wait.load(std::memory_order_relaxed);
#else
  return rr::kSplitWaitTicks;
#endif
}

rr_status fail(rr_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
rr_status fail(rr_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

bool valid_dtype(int d) { return d == RR_F32 || d == RR_BF16; }
size_t dtype_size(int d) { return d == RR_F32 ? 4 : 2; }
int vec_width(int d) { return d == RR_F32 ? 4 : 8; }  // elements per 16 bytes

// Elements per vector load of an op: 16 bytes of input, except a softmax
// reading bf16 and writing fp32, which loads 8 bytes (4 elements) so that
// each lane's output is one 16-byte store (the kernels' softmax_vec).
int op_vec_width(rr_op op, int din, int dout) {
  return (op == RR_OP_SOFTMAX && din == RR_BF16 && dout == RR_F32) ? 4 : vec_width(din);
}

// Vectors of `vec` elements of dtype din in 16 bytes: 1, or 2 for the 8-byte
// vectors (a scalar path counts as 1).  Per-lane vector counts sized for
// 16-byte vectors scale by it, which keeps the registers a lane holds.
int vecs_per_16_bytes(int din, int vec) { return vec > 1 ? (int)(16 / (dtype_size(din) * vec)) : 1; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// [a, a + na) and [b, b + nb) share a byte.
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a);
  const uintptr_t pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + nb && pb < pa + na;
}

// A row-major matrix of M rows of w bytes, row i starting at p + i * ld
// bytes (ld >= w).
struct Mat {
  const void* p;
  size_t ld;
  size_t w;
};

// Bytes from the first to one past the last byte of the matrix.
size_t span(const Mat& a, int64_t M) { return (size_t)(M - 1) * a.ld + a.w; }

// The two matrices share a byte.  Disjoint spans never do; with equal
// strides, each matrix covers a fixed window of byte positions modulo the
// stride, and the matrices are disjoint when those windows are (two column
// slices of one wider matrix, say).  Anything else with overlapping spans
// counts as overlapping.
bool mats_overlap(const Mat& a, const Mat& b, int64_t M) {
  if (!overlaps(a.p, span(a, M), b.p, span(b, M))) return false;
  if (a.ld != b.ld || a.ld == 0) return true;
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a.p);
  const uintptr_t pb = reinterpret_cast<uintptr_t>(b.p);
  const size_t ld = a.ld;
  // position of b's window relative to a's, in [0, ld)
  const size_t d = pb >= pa ? (size_t)(pb - pa) % ld : (ld - (size_t)(pa - pb) % ld) % ld;
  return !(d >= a.w && d + b.w <= ld);
}

// Rows of the matrix start 16-byte aligned.
bool rows_aligned(const Mat& a, size_t bytes) {
  return (reinterpret_cast<uintptr_t>(a.p) % bytes) == 0 && a.ld % bytes == 0;
}
bool rows_aligned16(const Mat& a) { return rows_aligned(a, 16); }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int pow2_at_least(int64_t v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}

constexpr int64_t kMaxN = (int64_t)1 << 30;  // keeps every in-row index in int32
constexpr int64_t kMaxStride = (int64_t)1 << 40;  // row strides, in elements
constexpr int kMaxWaves = rr::kMaxWavesPerGroup;
constexpr int kWaveRowsPerGroup = 4;         // rows per 256-thread workgroup (WAVE)
constexpr int64_t kSplitMaxRows = 1024;      // SPLIT only below this many rows
// 16-byte loads each lane keeps in flight per row in the workgroup-per-row
// kernels (summed over the input tensors); more wavefronts per row rather
// than more registers per lane measured faster on MI355X.
constexpr int kLoadsPerLane = 2;
// Split row: 16-byte vectors per lane in pass A's 256-lane chunks (a chunk
// is 256 * kSplitVecsPerLane vectors; twice as many of 8 bytes).
constexpr int kSplitVecsPerLane = 4;

// Register budget per lane, in fp32 values held for the row: softmax keeps
// one array (x, then e_i); the norms keep x (and the residual) plus gamma,
// so they stop at 16 values per lane and longer rows stream (LOOP).
int max_floats(rr_op op) { return op == RR_OP_SOFTMAX ? 32 : 16; }
int inputs_of(rr_op op) { return op == RR_OP_FUSED_ADD_RMSNORM ? 2 : 1; }

// Short rows: L lanes per row (the smallest power of two covering the row's
// vectors, at most 32), 256/L rows per 256-thread workgroup.
constexpr int64_t kSubMaxVectors = 32;
bool plan_sub(rr_plan* p, int vec, int64_t nvec) {
  if (nvec > kSubMaxVectors) return false;
  p->variant = RR_VARIANT_SUBWAVE;
  p->vec_elems = vec;
  p->waves_per_row = pow2_at_least(nvec);   // lanes per row
  p->rows_per_group = 256 / p->waves_per_row;
  p->vecs_per_lane = 1;
  p->block_threads = 256;
  return true;
}

void plan_wave(rr_plan* p, int vec, int64_t nvec) {
  p->variant = RR_VARIANT_WAVE;
  p->vec_elems = vec;
  p->waves_per_row = 1;
  p->rows_per_group = kWaveRowsPerGroup;
  p->vecs_per_lane = pow2_at_least(ceil_div(nvec, 64));
  p->block_threads = 64 * kWaveRowsPerGroup;
}

bool wave_fits(rr_op op, int vec, int64_t nvec) { return nvec <= 64 * (max_floats(op) / vec); }

// Workgroup-per-row: NV vectors per lane such that each lane has
// kLoadsPerLane loads in flight, then as many wavefronts as the row needs
// (at most 16); NV doubles while the row needs more than 16 wavefronts and
// the lane's register budget allows.
bool plan_block(rr_op op, rr_plan* p, int vec, int64_t nvec) {
  int nv = kLoadsPerLane / inputs_of(op);
  if (nv < 1) nv = 1;
  for (; nv * vec <= max_floats(op); nv *= 2) {
    const int64_t wpr = ceil_div(nvec, 64 * (int64_t)nv);
    if (wpr <= kMaxWaves) {
      p->variant = RR_VARIANT_BLOCK;
      p->vec_elems = vec;
      p->waves_per_row = (int32_t)wpr;
      p->rows_per_group = 1;
      p->vecs_per_lane = nv;
      p->block_threads = (int32_t)(64 * wpr);
      return true;
    }
  }
  return false;
}

// Softmax rows beyond that, up to 20 16-byte vectors (40 of 8 bytes) per lane
// of a 1024-lane workgroup, held in their storage format (one workgroup per
// CU).  From packed_min_rows() rows up this beats both the two-kernel split
// and the streaming path (cold, e.g. 256 x 152064 bf16 -> fp32: 46.0 us
// packed, 65.4 split, 78.6 streaming; 256 x 65536 fp32: 28.1, 41.5, 39.8);
// below it the split spreads a few rows over more CUs.  A causal call cannot
// split, and packed beats streaming at any row count, so it takes this path
// whenever the row fits.
constexpr int kPackedNV[] = {12, 16, 19, 20};
// Where the packed workgroup overtakes the split, by dtype pair: a packed
// workgroup's time is about one row's, so the cheaper a row is for one CU
// (bf16 in and out) the more rows the split needs to lose.  Measured cold on
// rows 50256 to 152064 wide (fp32 in: 36-48 rows; bf16 -> fp32: 56-68;
// bf16 -> bf16: 72-85).
// The split now runs as one kernel where the device holds its grid (one
// workgroup per chunk), which moved the crossovers up (cold, forced plans,
// one launch after a 512 MiB write, median of 21; split / packed, us): fp32
// x 65536 at 40 rows 10.8 / 13.8, at 48 11.4 / 13.8, at 56 12.2 / 14.2;
// fp32 -> bf16 x 65536 at 56 11.8 / 15.8, at 64 12.3 / 16.0; bf16 -> fp32 x
// 152064 at 56 15.6 / 23.0, at 64 17.0 / 23.1.  Captured in a HIP graph the
// split runs as two kernels; these thresholds keep that form within a few
// percent of the packed workgroup (at 40 / 56 / 56 rows respectively: 9.35 /
// 9.24, 10.95 / 11.04, 20.08 / 20.09 us per launch).
int64_t packed_min_rows(int din, int dout) {
  if (din == RR_F32) return dout == RR_F32 ? 48 : 64;
  return dout == RR_F32 ? 64 : 80;
}
// Rows cut at aligned addresses cost the packed kernel more than the split
// (its row's partial vectors, one row per CU): the crossovers move up by
// about 16 rows (measured cold on 50257-152065-wide rows: fp32 54-60,
// bf16 -> fp32 68-88, bf16 -> bf16 92-100; with the split in one kernel,
// bf16 -> fp32 x 50257 at 80 rows 16.2 / 16.9 us split / packed, at 88
// 17.7 / 16.8).
constexpr int64_t kCutPackedExtraRows = 24;
bool plan_packed(rr_op op, rr_plan* p, int vec, int per16, int64_t nvec) {
  if (op != RR_OP_SOFTMAX) return false;
  for (int nv16 : kPackedNV) {
    const int nv = nv16 * per16;
    if (nvec <= (int64_t)kMaxWaves * 64 * nv) {
      p->variant = RR_VARIANT_BLOCK;
      p->vec_elems = vec;
      p->waves_per_row = kMaxWaves;
      p->rows_per_group = 1;
      p->vecs_per_lane = nv;
      p->block_threads = 64 * kMaxWaves;
      return true;
    }
  }
  return false;
}

// Norm rows beyond the block budget (16 widened values per lane), up to 64K
// elements: 1024 lanes hold the row in its storage format, NV vectors each
// (bf16 4 or 8; fp32 8, 12 or 16; the fused op in fp32 holds x and the
// residual while loading, so only 8).  Any number of rows: the alternative,
// streaming the row twice, is slower at every row count.
bool plan_norm_packed(rr_op op, rr_plan* p, int vec, int64_t nvec) {
  if (op == RR_OP_SOFTMAX) return false;
  static const int kBf16[] = {4, 8};
  static const int kF32[] = {8, 12, 16};
  const int* list = vec == 8 ? kBf16 : kF32;
  const int count = vec == 8 ? 2 : (op == RR_OP_FUSED_ADD_RMSNORM ? 1 : 3);
  if (vec == 1) return false;
  for (int i = 0; i < count; ++i) {
    if (nvec <= (int64_t)kMaxWaves * 64 * list[i]) {
      p->variant = RR_VARIANT_BLOCK;
      p->vec_elems = vec;
      p->waves_per_row = kMaxWaves;
      p->rows_per_group = 1;
      p->vecs_per_lane = list[i];
      p->block_threads = 64 * kMaxWaves;
      return true;
    }
  }
  return false;
}

void plan_split(rr_plan* p, int vec, int per16, int64_t nvec) {
  p->variant = RR_VARIANT_SPLIT;
  p->vec_elems = vec;
  p->waves_per_row = 4;
  p->rows_per_group = 1;
  p->vecs_per_lane = kSplitVecsPerLane * per16;
  p->block_threads = 256;
  p->chunks_per_row = ceil_div(nvec, 256 * (int64_t)p->vecs_per_lane);
}

void plan_loop(rr_plan* p, int vec, int64_t nvec) {
  p->variant = RR_VARIANT_LOOP;
  p->vec_elems = vec;
  p->waves_per_row = nvec > 4096 ? 16 : 4;
  p->rows_per_group = 1;
  p->vecs_per_lane = 1;
  p->block_threads = 64 * p->waves_per_row;
}

// A cut RMSNorm row (fused or not) that takes a workgroup: 2 or 3 vectors
// per lane, whichever needs fewer wavefronts (2 on a tie), 4 for fp32 rows
// that 3 cannot hold in 16 wavefronts.  Each wavefront of a cut row costs a
// fixed share of address and frame work, so fewer wavefronts per row win
// where rounding the row up to whole wavefronts leaves them as full.
// Measured back to back on 64 MiB inputs (us): bf16 8190 x 4097 (516
// vectors at most) 28.1 as 5 wavefronts of 2 vectors, 26.1 as 3 of 3
// (aligned 8192 x 4096: 22.6); 32736 x 1025 42.9 as 2 of 2, 31.6 as 1 of 3;
// fused 8190 x 4097 71 as 9 of 1 (the aligned rule), 48.8 as 5 of 2 or 3 of
// 3 (aligned: 43.9); fp32 4095 x 4097 26.8 as 9 of 2, 25.8 as 6 of 3, 26.9
// as 5 of 4.  A cut LayerNorm row takes the same choice: its workgroup
// stages gamma's and beta's elements in LDS once (up to kNormLdsParamMax
// bytes), so its lanes hold no more than an RMSNorm row's.
bool plan_block_cut(rr_plan* p, int vw, int64_t nvec) {
  int best_nv = 0;
  int64_t best_w = 0;
  for (int nv = 2; nv <= 3; ++nv) {
    const int64_t w = ceil_div(nvec, 64 * (int64_t)nv);
    if (w <= kMaxWaves && (best_nv == 0 || w < best_w)) {
      best_nv = nv;
      best_w = w;
    }
  }
  if (best_nv == 0 && vw == 4 && ceil_div(nvec, 64 * 4) <= kMaxWaves) {
    best_nv = 4;
    best_w = ceil_div(nvec, 64 * 4);
  }
  if (best_nv == 0) return false;
  p->variant = RR_VARIANT_BLOCK;
  p->vec_elems = vw;
  p->waves_per_row = (int32_t)best_w;
  p->rows_per_group = 1;
  p->vecs_per_lane = best_nv;
  p->block_threads = (int32_t)(64 * best_w);
  return true;
}

// Rows cut into vectors at aligned addresses (row_shift): the row
// starts at element `lead` of its first vector, so it spans up to nvec_s
// vectors (see make_plan).  The same choice as for aligned rows: a
// wavefront, a workgroup, the packed workgroup from packed_min_rows() rows (or
// for a causal call), else the split below kSplitMaxRows rows, else the
// streaming kernel, all cut the same way.  The split sizes its chunks for a
// row at any offset (nvec_any) so that the workspace query, which sees no
// addresses, covers every call.
bool plan_shifted(rr_op op, bool causal, int64_t M, int64_t N, int64_t packed_rows, rr_plan* p, int vw,
                  int per16, int64_t nvec_s, int64_t nvec_any) {
  bool ok = true;
  if (op != RR_OP_SOFTMAX) {
    // a wavefront's cut row holds gamma's (and beta's) two aligned blocks
    // per vector while the row loads: an fp32 LayerNorm wavefront keeps to 2
    // vectors per lane (4 would spill); longer norm rows stream element by
    // element
    const int max_nv = (op == RR_OP_LAYERNORM && vw == 4) ? 2 : 16;
    if (wave_fits(op, vw, nvec_s) && ceil_div(nvec_s, 64) <= max_nv) {
      plan_wave(p, vw, nvec_s);
    } else {
      // a workgroup's cut LayerNorm row stages gamma and beta in LDS, sized
      // for a row at any offset; its kernel exists for 1 to 3 vectors per lane
      const bool lds_ok = op != RR_OP_LAYERNORM || rr::norm_lds_param_bytes_for(N, 16 / vw) <= rr::kNormLdsParamMax;
      ok = lds_ok && plan_block_cut(p, vw, nvec_s) &&
           (op != RR_OP_LAYERNORM || p->vecs_per_lane <= 3);
    }
  } else if (wave_fits(op, vw, nvec_s)) {
    plan_wave(p, vw, nvec_s);
  } else if (plan_block(op, p, vw, nvec_s)) {
  } else if ((M >= packed_rows || causal) && plan_packed(op, p, vw, per16, nvec_s)) {
  } else if (op == RR_OP_SOFTMAX && !causal && M < kSplitMaxRows) {
    plan_split(p, vw, per16, nvec_any);
  } else {
    plan_loop(p, vw, nvec_s);
  }
  if (ok) p->row_shift = 1;
  return ok;
}

// Host-only plan.  `align`: 1 every row start of the call is vector-aligned;
// 2 row starts anywhere, but input and output rows sit at the same element
// offset within a vector (rows are then cut at aligned addresses);
// 0 neither (scalar access).
rr_status make_plan(rr_op op, int64_t M, int64_t N, int din, int dout, int align,
                    rr_plan* p) {
  memset(p, 0, sizeof(*p));
  if (op != RR_OP_RMSNORM && op != RR_OP_FUSED_ADD_RMSNORM && op != RR_OP_SOFTMAX &&
      op != RR_OP_LAYERNORM && op != RR_OP_SOFTMAX_CAUSAL)
    return fail(RR_ERR_INVALID_ARG, "unknown op %d", (int)op);
  // a causal softmax runs the softmax kernels but never splits a row (the
  // split kernels keep every key)
  const bool causal = op == RR_OP_SOFTMAX_CAUSAL;
  if (causal) op = RR_OP_SOFTMAX;
  if (!valid_dtype(din) || !valid_dtype(dout))
    return fail(RR_ERR_INVALID_ARG, "unknown dtype (%d, %d)", din, dout);
  if (op != RR_OP_SOFTMAX && din != dout)
    return fail(RR_ERR_INVALID_ARG, "norm input and output dtypes must match");
  if (M < 0) return fail(RR_ERR_INVALID_ARG, "M = %lld < 0", (long long)M);
  if (N < 1) return fail(RR_ERR_INVALID_ARG, "row width %lld < 1 (empty rows have no statistic)", (long long)N);
  if (N > kMaxN) return fail(RR_ERR_UNSUPPORTED, "row width %lld > 2^30", (long long)N);

  const int vw = op_vec_width(op, din, dout);
  const bool plain = align == 1 && N % vw == 0;
  // rows that are not whole aligned vectors but can be cut at aligned
  // addresses: aligned starts with a ragged width, or starts at a common
  // offset (the norms read gamma in each row's frame, only in the register
  // kernels, and from three vectors up: gamma's windows are cut from pairs of
  // aligned blocks inside it)
  const bool shiftable = !plain && align != 0 && (op == RR_OP_SOFTMAX || N >= 3 * (int64_t)vw);
  const int vec = plain ? vw : 1;
  const int per16 = vecs_per_16_bytes(din, vec);
  const int64_t nvec = N / vec;
  // vectors a cut row spans: with aligned starts (lead 0) ceil(N / vw), with
  // starts at any offset up to ceil((N + vw - 1) / vw)
  const int64_t nvec_any = (N + 2 * (int64_t)vw - 2) / vw;
  const int64_t nvec_s = align == 1 ? ceil_div(N, vw) : nvec_any;
  const int per16_s = vecs_per_16_bytes(din, vw);
  const int forced = forced_variant();
  const int64_t packed_rows = packed_min_rows(din, dout);

  bool ok = false;
  switch (forced) {
    case RR_VARIANT_AUTO:
      if (plan_sub(p, vec, nvec)) {
      } else if (shiftable && plan_shifted(op, causal, M, N, packed_rows + kCutPackedExtraRows, p, vw, per16_s,
                                           nvec_s, nvec_any)) {
      } else if (vec == 1) {
        plan_loop(p, vec, nvec);
      } else if (wave_fits(op, vec, nvec)) {
        plan_wave(p, vec, nvec);
        // a softmax written as fp32 with many rows: workgroups of lanes that
        // hold 2 vectors beat a wavefront holding 8 from 16384 rows up, and
        // one holding 4 from 65536 rows up (cold; bf16 -> fp32 65536 x 2048:
        // 134.9 -> 127.9 us, 131072 x 1024: 140.3 -> 128.4; fp32 65536 x
        // 2048: 179.7 -> 171.9)
        if (op == RR_OP_SOFTMAX && dout == RR_F32 &&
            ((p->vecs_per_lane == 8 && M >= 16384) || (p->vecs_per_lane == 4 && M >= 65536)))
          plan_block(op, p, vec, nvec);
      } else if (plan_block(op, p, vec, nvec)) {
      } else if (plan_norm_packed(op, p, vec, nvec)) {
      } else if ((M >= packed_rows || causal) && plan_packed(op, p, vec, per16, nvec)) {
      } else if (op == RR_OP_SOFTMAX && !causal && M < kSplitMaxRows) {
        plan_split(p, vec, per16, nvec);
      } else {
        plan_loop(p, vec, nvec);
      }
      ok = true;
      break;
    case RR_VARIANT_WAVE:
      ok = vec > 1 && wave_fits(op, vec, nvec);
      if (ok) {
        plan_wave(p, vec, nvec);
      } else if (shiftable && wave_fits(op, vw, nvec_s)) {
        plan_wave(p, vw, nvec_s);
        p->row_shift = 1;
        ok = true;
      }
      break;
    case RR_VARIANT_BLOCK:
      ok = vec > 1 && (plan_block(op, p, vec, nvec) || plan_packed(op, p, vec, per16, nvec) ||
                       plan_norm_packed(op, p, vec, nvec));
      if (!ok && shiftable) {
        ok = plan_block(op, p, vw, nvec_s) || plan_packed(op, p, vw, per16_s, nvec_s);
        if (ok) p->row_shift = 1;
      }
      break;
    case RR_VARIANT_SPLIT:
    case RR_VARIANT_SPLIT_ONE_KERNEL:
    case RR_VARIANT_SPLIT_TWO_KERNELS:
      ok = vec > 1 && op == RR_OP_SOFTMAX && !causal;
      if (ok) {
        plan_split(p, vec, per16, nvec);
        p->variant = forced;
      } else if (forced != RR_VARIANT_SPLIT_ONE_KERNEL && shiftable && op == RR_OP_SOFTMAX && !causal) {
        plan_split(p, vw, per16_s, nvec_any);   // the one-kernel form takes aligned rows only
        p->variant = forced;
        p->row_shift = 1;
        ok = true;
      }
      break;
    case RR_VARIANT_LOOP:
      if (shiftable && op == RR_OP_SOFTMAX) {
        plan_loop(p, vw, nvec_s);
        p->row_shift = 1;
      } else {
        plan_loop(p, vec, nvec);
      }
      ok = true;
      break;
    case RR_VARIANT_SUBWAVE:
      ok = plan_sub(p, vec, nvec);
      break;
    default:
      break;
  }
  if (!ok) {
    return fail(RR_ERR_UNSUPPORTED, "forced variant %d cannot run op %d with N = %lld (vector width %d)",
                forced, (int)op, (long long)N, vec);
  }
  // cut LayerNorm rows, also when a variant is forced (plan_shifted): an
  // fp32 wavefront keeps to 2 vectors per lane; a workgroup to 3, with
  // gamma's and beta's blocks staged in LDS
  if (ok && p->row_shift && op == RR_OP_LAYERNORM) {
    if (p->variant == RR_VARIANT_WAVE)
      ok = !(vw == 4 && p->vecs_per_lane > 2);
    else
      ok = p->variant == RR_VARIANT_BLOCK && p->vecs_per_lane <= 3 &&
           rr::norm_lds_param_bytes_for(N, 16 / vw) <= rr::kNormLdsParamMax;
  }
  if (!ok) {
    return fail(RR_ERR_UNSUPPORTED, "forced variant %d cannot run op %d with N = %lld (vector width %d)",
                forced, (int)op, (long long)N, vec);
  }
  if (p->chunks_per_row == 0) p->chunks_per_row = 1;
  if (p->variant == RR_VARIANT_SPLIT || p->variant == RR_VARIANT_SPLIT_ONE_KERNEL ||
      p->variant == RR_VARIANT_SPLIT_TWO_KERNELS) {
    if (p->chunks_per_row > (int64_t)1 << 30) return fail(RR_ERR_UNSUPPORTED, "too many chunks");
    p->work_items = M * p->chunks_per_row;
    // M * S slots of 16 bytes, then one 32-bit epoch per row (the
    // one-kernel form's tags), padded to 16 bytes
    p->workspace_bytes = (size_t)M * (size_t)p->chunks_per_row * 16u + ((size_t)M * 4u + 15u) / 16u * 16u;
  } else {
    p->work_items = ceil_div(M, p->rows_per_group);
  }
  return RR_OK;
}

// Grid size: one workgroup per work item (grid-stride persistent grids
// measured slower on MI355X for every kernel here), capped so that a
// dispatch's work-items fit in 32 bits (grid x threads below 2^32; every
// kernel walks its rows grid-stride, so a capped grid still covers them all).
#ifndef RR_STRESS
#define RR_STRESS 0
#endif

int64_t grid_for(const rr_plan& p) {
  const int64_t g = p.work_items;
  const int64_t kMaxGrid = 0xffffffffLL / (p.block_threads > 0 ? p.block_threads : 1);
#if RR_STRESS
  // the race-stress build (see rr_kernels.hip): few workgroups, each walking
  // many rows, so that the LDS slot sets are reused many times (the
  // one-kernel split sizes its own grid, one workgroup per chunk)
  if (g > 37) return 37;
#endif
  return g > kMaxGrid ? kMaxGrid : g;
}

rr_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return RR_OK;
  return fail(RR_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool valid_eps(float eps) { return eps >= 0.0f && eps <= 3.0e38f; }

// kind: rr::kLaunchRms, kLaunchFused or kLaunchLayer.
// Row strides of a call, in elements, checked: each at least the row width
// (rows of one matrix never overlap) and small enough that the last row's
// end fits in memory.
rr_status check_strides(const char* name, int64_t M, int64_t H, const int64_t* lds, const char* const* what,
                        int n) {
  for (int i = 0; i < n; ++i) {
    if (lds[i] < H)
      return fail(RR_ERR_INVALID_ARG, "%s: %s = %lld < row width %lld", name, what[i], (long long)lds[i],
                  (long long)H);
    if (lds[i] > kMaxStride || (uint64_t)(M - 1) > (uint64_t)(SIZE_MAX / 8) / (uint64_t)lds[i])
      return fail(RR_ERR_INVALID_ARG, "%s: %s = %lld too large for M = %lld", name, what[i],
                  (long long)lds[i], (long long)M);
  }
  return RR_OK;
}

rr_status norm_entry(int kind, void* y, int64_t ldy, void* residual, int64_t ldr, const void* x,
                     int64_t ldx, const void* gamma, const void* beta, int64_t M, int64_t H, float eps,
                     rr_dtype dtype, void* stream, const char* name) {
  g_err[0] = '\0';
  const bool fused = kind == rr::kLaunchFused;
  const bool layer = kind == rr::kLaunchLayer;
  if (!valid_dtype(dtype)) return fail(RR_ERR_INVALID_ARG, "%s: unknown dtype %d", name, (int)dtype);
  if (M < 0) return fail(RR_ERR_INVALID_ARG, "%s: M = %lld < 0", name, (long long)M);
  if (H < 1) return fail(RR_ERR_INVALID_ARG, "%s: H = %lld < 1", name, (long long)H);
  if (!valid_eps(eps)) return fail(RR_ERR_INVALID_ARG, "%s: eps must be finite and >= 0", name);
  if (M == 0) return RR_OK;
  if (!y || !x || !gamma || (fused && !residual))
    return fail(RR_ERR_INVALID_ARG, "%s: null pointer", name);
  if (H > kMaxN) return fail(RR_ERR_UNSUPPORTED, "%s: H = %lld > 2^30", name, (long long)H);
  const int64_t lds[3] = {ldy, ldx, fused ? ldr : H};
  const char* const what[3] = {"ldy", "ldx", "ldr"};
  const rr_status sst = check_strides(name, M, H, lds, what, 3);
  if (sst != RR_OK) return sst;
  const size_t es = dtype_size(dtype);
  const size_t w = (size_t)H * es;
  const Mat my{y, (size_t)ldy * es, w}, mx{x, (size_t)ldx * es, w}, mr{residual, (size_t)ldr * es, w};
  const size_t gbytes = w;
  // y may be x itself (same stride): each lane reads its elements before it
  // writes them
  if (!(y == x && ldy == ldx) && mats_overlap(my, mx, M))
    return fail(RR_ERR_INVALID_ARG, "%s: y partly overlaps x", name);
  if (overlaps(gamma, gbytes, y, span(my, M))) return fail(RR_ERR_INVALID_ARG, "%s: gamma overlaps y", name);
  if (layer && beta && overlaps(beta, gbytes, y, span(my, M)))
    return fail(RR_ERR_INVALID_ARG, "%s: beta overlaps y", name);
  if (fused) {
    if (mats_overlap(mr, mx, M) || mats_overlap(mr, my, M) || overlaps(residual, span(mr, M), gamma, gbytes))
      return fail(RR_ERR_INVALID_ARG, "%s: residual overlaps x, y or gamma", name);
  }
  const bool al = rows_aligned16(my) && rows_aligned16(mx) && aligned16(gamma) &&
                  (!fused || rows_aligned16(mr)) && (!layer || !beta || aligned16(beta));
  // otherwise: x, y (and the residual) rows at one element offset within a
  // vector, and gamma (beta) element-aligned, lets the register kernels cut
  // the rows at aligned addresses
  int align = al ? 1 : 0;
  if (!al) {
    const int64_t vw = op_vec_width(RR_OP_RMSNORM, dtype, dtype);
    auto elem = [&](const void* q) { return reinterpret_cast<uintptr_t>(q) % es == 0; };
    auto lead = [&](const void* q) { return (int64_t)((reinterpret_cast<uintptr_t>(q) / es) % (uintptr_t)vw); };
    bool same = elem(x) && elem(y) && elem(gamma) && (!layer || !beta || elem(beta)) &&
                lead(x) == lead(y) && ldx % vw == ldy % vw;
    if (fused) same = same && elem(residual) && lead(residual) == lead(x) && ldr % vw == ldx % vw;
    if (same) align = 2;
  }
  const rr_op op = fused ? RR_OP_FUSED_ADD_RMSNORM : layer ? RR_OP_LAYERNORM : RR_OP_RMSNORM;
  rr_plan p;
  const rr_status st = make_plan(op, M, H, dtype, dtype, align, &p);
  if (st != RR_OK) return st;
  rr::NormArgs a;
  a.y = y;
  a.residual = residual;
  a.x = x;
  a.gamma = gamma;
  a.beta = layer ? beta : nullptr;
  a.M = M;
  a.N = (int32_t)H;
  a.eps = eps;
  a.ld = rr::RowStrides{ldx, ldy, fused ? ldr : H};
  const hipError_t e = rr::launch_norm(p, dtype, kind, a, grid_for(p), static_cast<hipStream_t>(stream));
  return hip_status(e, name);
}

}  // namespace

extern "C" {

rr_status rr_rmsnorm(void* y, const void* x, const void* gamma, int64_t M, int64_t H, float eps,
                     rr_dtype dtype, void* stream) {
  return norm_entry(rr::kLaunchRms, y, H, nullptr, H, x, H, gamma, nullptr, M, H, eps, dtype, stream,
                    "rr_rmsnorm");
}

rr_status rr_fused_add_rmsnorm(void* y, void* residual, const void* x, const void* gamma,
                               int64_t M, int64_t H, float eps, rr_dtype dtype, void* stream) {
  return norm_entry(rr::kLaunchFused, y, H, residual, H, x, H, gamma, nullptr, M, H, eps, dtype, stream,
                    "rr_fused_add_rmsnorm");
}

rr_status rr_layernorm(void* y, const void* x, const void* gamma, const void* beta, int64_t M,
                       int64_t H, float eps, rr_dtype dtype, void* stream) {
  return norm_entry(rr::kLaunchLayer, y, H, nullptr, H, x, H, gamma, beta, M, H, eps, dtype, stream,
                    "rr_layernorm");
}

rr_status rr_rmsnorm_strided(void* y, int64_t ldy, const void* x, int64_t ldx, const void* gamma,
                             int64_t M, int64_t H, float eps, rr_dtype dtype, void* stream) {
  return norm_entry(rr::kLaunchRms, y, ldy, nullptr, H, x, ldx, gamma, nullptr, M, H, eps, dtype, stream,
                    "rr_rmsnorm_strided");
}

rr_status rr_fused_add_rmsnorm_strided(void* y, int64_t ldy, void* residual, int64_t ldr,
                                       const void* x, int64_t ldx, const void* gamma, int64_t M,
                                       int64_t H, float eps, rr_dtype dtype, void* stream) {
  return norm_entry(rr::kLaunchFused, y, ldy, residual, ldr, x, ldx, gamma, nullptr, M, H, eps, dtype,
                    stream, "rr_fused_add_rmsnorm_strided");
}

rr_status rr_layernorm_strided(void* y, int64_t ldy, const void* x, int64_t ldx, const void* gamma,
                               const void* beta, int64_t M, int64_t H, float eps, rr_dtype dtype,
                               void* stream) {
  return norm_entry(rr::kLaunchLayer, y, ldy, nullptr, H, x, ldx, gamma, beta, M, H, eps, dtype, stream,
                    "rr_layernorm_strided");
}

}  // extern "C"

namespace {

// Options of a softmax call, checked; NULL means all zero.
rr_status softmax_options(const rr_softmax_opts* o, const char* who, rr_softmax_opts* out) {
  memset(out, 0, sizeof(*out));
  if (!o) return RR_OK;
  if (o->log_output != 0 && o->log_output != 1)
    return fail(RR_ERR_INVALID_ARG, "%s: log_output = %d (0 or 1)", who, (int)o->log_output);
  if (o->causal != 0 && o->causal != 1)
    return fail(RR_ERR_INVALID_ARG, "%s: causal = %d (0 or 1)", who, (int)o->causal);
  *out = *o;
  if (o->causal) {
    if (o->causal_period < 1)
      return fail(RR_ERR_INVALID_ARG, "%s: causal_period = %lld < 1", who, (long long)o->causal_period);
    if (o->causal_offset < 0)
      return fail(RR_ERR_INVALID_ARG, "%s: causal_offset = %lld < 0", who, (long long)o->causal_offset);
  } else {
    out->causal_period = 0;
    out->causal_offset = 0;
  }
  return RR_OK;
}

// Causal calls of the workgroup plan on aligned rows may hold two rows of a
// period per workgroup, rows q and P - 1 - q, so that every workgroup reads
// about one row of kept keys ([P1] section "二、它们在 Qwen2.5-7B 里的真实位置"
// sizes the per-layer score softmax this serves).  Worth it where the kept
// counts vary along the period (P + 2O at most 1.25 N) over whole periods;
// each row is held as the plan holds it, so the two rows together stay
// within 32 values per lane (the plan's at most 16 each).  Returns the
// plan's vectors per lane when pairing, 0 for one row per workgroup.
int causal_pair_nv(const rr_plan& p, int64_t M, int64_t N, int64_t P, int64_t O) {
  if (p.variant != RR_VARIANT_BLOCK || p.row_shift || p.vec_elems <= 1 || N % p.vec_elems != 0) return 0;
  if (p.vecs_per_lane * p.vec_elems > 16) return 0;
  if (P < 2 || M < P || 4 * (P + 2 * O) > 5 * N) return 0;
  return p.vecs_per_lane;
}

// noalloc: the workspace comes from the library's static scratch array
// (rr_softmax_rows_strided_noalloc); workspace and workspace_bytes are unused.
rr_status softmax_entry(const char* who, void* y, int64_t ldy, const void* x, int64_t ldx, int64_t M,
                        int64_t N, rr_dtype in_dtype, rr_dtype out_dtype, const rr_softmax_opts* opts,
                        void* workspace, size_t workspace_bytes, void* stream, bool noalloc = false) {
  g_err[0] = '\0';
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype))
    return fail(RR_ERR_INVALID_ARG, "%s: unknown dtype (%d, %d)", who, (int)in_dtype, (int)out_dtype);
  rr_softmax_opts o;
  const rr_status so = softmax_options(opts, who, &o);
  if (so != RR_OK) return so;
  if (M < 0) return fail(RR_ERR_INVALID_ARG, "%s: M = %lld < 0", who, (long long)M);
  if (N < 1) return fail(RR_ERR_INVALID_ARG, "%s: N = %lld < 1", who, (long long)N);
  if (M == 0) return RR_OK;
  if (!y || !x) return fail(RR_ERR_INVALID_ARG, "%s: null pointer", who);
  if (N > kMaxN) return fail(RR_ERR_UNSUPPORTED, "%s: N = %lld > 2^30", who, (long long)N);
  const int64_t lds[2] = {ldy, ldx};
  const char* const what[2] = {"ldy", "ldx"};
  const rr_status sst = check_strides(who, M, N, lds, what, 2);
  if (sst != RR_OK) return sst;
  const Mat mx{x, (size_t)ldx * dtype_size(in_dtype), (size_t)N * dtype_size(in_dtype)};
  const Mat my{y, (size_t)ldy * dtype_size(out_dtype), (size_t)N * dtype_size(out_dtype)};
  const size_t xb = span(mx, M), yb = span(my, M);
  if (mats_overlap(mx, my, M) && !(x == y && ldx == ldy && in_dtype == out_dtype))
    return fail(RR_ERR_INVALID_ARG,
                "%s: x and y overlap (in place needs equal pointers, strides and dtypes)", who);
  // a bf16 input written as fp32 is read 8 bytes per vector (op_vec_width)
  const size_t in_align = (in_dtype == RR_BF16 && out_dtype == RR_F32) ? 8 : 16;
  int align = 0;
  if (rows_aligned(mx, in_align) && rows_aligned16(my)) {
    align = 1;
  } else {
    // every row of x and of y at the same element offset within a vector:
    // element-aligned bases at the same offset, strides equal modulo the
    // vector width (contiguous rows of any width, in place, column slices)
    const int64_t vw = op_vec_width(RR_OP_SOFTMAX, in_dtype, out_dtype);
    const uintptr_t ux = reinterpret_cast<uintptr_t>(x), uy = reinterpret_cast<uintptr_t>(y);
    const size_t sx = dtype_size(in_dtype), sy = dtype_size(out_dtype);
    if (ux % sx == 0 && uy % sy == 0 && (int64_t)((ux / sx) % vw) == (int64_t)((uy / sy) % vw) &&
        ldx % vw == ldy % vw)
      align = 2;
  }
  rr_plan p;
  const rr_status st = make_plan(o.causal ? RR_OP_SOFTMAX_CAUSAL : RR_OP_SOFTMAX, M, N, in_dtype,
                                 out_dtype, align, &p);
  if (st != RR_OK) return st;
  if (noalloc && p.workspace_bytes > 0) {
    // the scratch array holds one call's slots; larger splits are refused
    // before anything touches the device
    if (p.workspace_bytes > rr::kNoAllocScratchBytes)
      return fail(RR_ERR_WORKSPACE, "%s: this shape needs %zu bytes of split-row scratch; the static scratch holds %zu",
                  who, p.workspace_bytes, rr::kNoAllocScratchBytes);
    hipError_t se = hipSuccess;
    workspace = rr::noalloc_scratch(&se);
    if (!workspace) return hip_status(se != hipSuccess ? se : hipErrorInvalidSymbol, who);
    workspace_bytes = rr::kNoAllocScratchBytes;
  } else if (p.workspace_bytes > 0) {
    if (!workspace || workspace_bytes < p.workspace_bytes)
      return fail(RR_ERR_WORKSPACE, "%s: needs a workspace of %zu bytes, got %zu", who,
                  p.workspace_bytes, workspace ? workspace_bytes : (size_t)0);
    if ((reinterpret_cast<uintptr_t>(workspace) & 15u) != 0)
      return fail(RR_ERR_INVALID_ARG, "%s: workspace must be 16-byte aligned", who);
    if (overlaps(workspace, p.workspace_bytes, x, xb) || overlaps(workspace, p.workspace_bytes, y, yb))
      return fail(RR_ERR_INVALID_ARG, "%s: workspace overlaps x or y", who);
  }
  rr::SoftmaxArgs a;
  a.y = y;
  a.x = x;
  a.workspace = workspace;
  a.M = M;
  a.N = (int32_t)N;
  a.causal_period = o.causal ? o.causal_period : 0;
  // keys kept by row i: min(N, (i mod P) + O + 1); an offset of N or more
  // keeps every key, so clamp it to keep the kernels' sums in range
  a.causal_offset = o.causal_offset < N ? o.causal_offset : N;
  a.log_output = o.log_output;
  a.ld = rr::RowStrides{ldx, ldy, 0};
  a.pair_nv = o.causal ? causal_pair_nv(p, M, N, o.causal_period, a.causal_offset) : 0;
  a.split_wait_ticks = split_wait_ticks();
  const hipError_t e = rr::launch_softmax(p, in_dtype, out_dtype, a, grid_for(p),
                                          static_cast<hipStream_t>(stream));
  return hip_status(e, who);
}

}  // namespace

extern "C" {

size_t rr_softmax_rows_workspace_bytes(int64_t M, int64_t N, rr_dtype in_dtype,
                                       rr_dtype out_dtype) {
  return rr_softmax_rows_ex_workspace_bytes(M, N, in_dtype, out_dtype, nullptr);
}

size_t rr_softmax_rows_ex_workspace_bytes(int64_t M, int64_t N, rr_dtype in_dtype,
                                          rr_dtype out_dtype, const rr_softmax_opts* opts) {
  rr_softmax_opts o;
  if (softmax_options(opts, "rr_softmax_rows_ex_workspace_bytes", &o) != RR_OK) return 0;
  // the most any call that can run needs: aligned rows, or rows cut at
  // aligned addresses (their split may take one more chunk per row; a forced
  // variant may refuse them)
  const rr_op op = o.causal ? RR_OP_SOFTMAX_CAUSAL : RR_OP_SOFTMAX;
  size_t most = 0;
  for (int align = 1; align <= 2; ++align) {
    rr_plan p;
    if (make_plan(op, M, N, in_dtype, out_dtype, align, &p) == RR_OK && p.workspace_bytes > most)
      most = p.workspace_bytes;
  }
  return most;
}

rr_status rr_softmax_rows(void* y, const void* x, int64_t M, int64_t N, rr_dtype in_dtype,
                          rr_dtype out_dtype, void* workspace, size_t workspace_bytes,
                          void* stream) {
  return softmax_entry("rr_softmax_rows", y, N, x, N, M, N, in_dtype, out_dtype, nullptr, workspace,
                       workspace_bytes, stream);
}

rr_status rr_softmax_rows_ex(void* y, const void* x, int64_t M, int64_t N, rr_dtype in_dtype,
                             rr_dtype out_dtype, const rr_softmax_opts* opts, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return softmax_entry("rr_softmax_rows_ex", y, N, x, N, M, N, in_dtype, out_dtype, opts, workspace,
                       workspace_bytes, stream);
}

rr_status rr_softmax_rows_strided(void* y, int64_t ldy, const void* x, int64_t ldx, int64_t M,
                                  int64_t N, rr_dtype in_dtype, rr_dtype out_dtype,
                                  const rr_softmax_opts* opts, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  return softmax_entry("rr_softmax_rows_strided", y, ldy, x, ldx, M, N, in_dtype, out_dtype, opts,
                       workspace, workspace_bytes, stream);
}

rr_status rr_softmax_rows_strided_noalloc(void* y, int64_t ldy, const void* x, int64_t ldx, int64_t M,
                                          int64_t N, rr_dtype in_dtype, rr_dtype out_dtype,
                                          const rr_softmax_opts* opts, void* stream) {
  return softmax_entry("rr_softmax_rows_strided_noalloc", y, ldy, x, ldx, M, N, in_dtype, out_dtype, opts,
                       nullptr, 0, stream, true);
}

const char* rr_status_string(rr_status s) {
  switch (s) {
    case RR_OK: return "RR_OK";
    case RR_ERR_INVALID_ARG: return "RR_ERR_INVALID_ARG";
    case RR_ERR_UNSUPPORTED: return "RR_ERR_UNSUPPORTED";
    case RR_ERR_WORKSPACE: return "RR_ERR_WORKSPACE";
    case RR_ERR_HIP: return "RR_ERR_HIP";
  }
  return "RR_UNKNOWN_STATUS";
}

const char* rr_last_error_message(void) { return g_err; }

rr_status rr_query_plan(rr_op op, int64_t M, int64_t N, rr_dtype in_dtype, rr_dtype out_dtype,
                        int is_aligned16, rr_plan* plan) {
  g_err[0] = '\0';
  if (!plan) return fail(RR_ERR_INVALID_ARG, "rr_query_plan: null plan");
  return make_plan(op, M, N, in_dtype, out_dtype, is_aligned16 == 2 ? 2 : (is_aligned16 != 0 ? 1 : 0), plan);
}

#if RR_DIAG
rr_status rr_set_variant_override(rr_variant v) {
  g_err[0] = '\0';
  if (v < RR_VARIANT_AUTO || v > RR_VARIANT_SPLIT_TWO_KERNELS)
    return fail(RR_ERR_INVALID_ARG, "rr_set_variant_override: unknown variant %d", (int)v);
  g_override.store(v, std::memory_order_relaxed);
  return RR_OK;
}

rr_status rr_selftest_wave_allreduce(const float* in, float* out, int64_t count, int kind,
                                     void* stream) {
  g_err[0] = '\0';
  if (!in || !out || count < 1 || count > 0xffffffffLL / 64 || kind < 0 || kind > 2)
    return fail(RR_ERR_INVALID_ARG, "rr_selftest_wave_allreduce: bad arguments");
  return hip_status(rr::launch_selftest_wave(in, out, count, kind, static_cast<hipStream_t>(stream)),
                    "rr_selftest_wave_allreduce");
}

rr_status rr_stream_copy(void* dst, const void* src, int64_t bytes, void* stream) {
  g_err[0] = '\0';
  if (bytes < 0 || bytes % 16 != 0)
    return fail(RR_ERR_INVALID_ARG, "rr_stream_copy: bytes must be a non-negative multiple of 16");
  if (bytes == 0) return RR_OK;
  if (!dst || !src) return fail(RR_ERR_INVALID_ARG, "rr_stream_copy: null pointer");
  if (!aligned16(dst) || !aligned16(src))
    return fail(RR_ERR_INVALID_ARG, "rr_stream_copy: pointers must be 16-byte aligned");
  if (overlaps(dst, (size_t)bytes, src, (size_t)bytes))
    return fail(RR_ERR_INVALID_ARG, "rr_stream_copy: source and destination overlap");
  return hip_status(rr::launch_stream_copy(dst, src, bytes, static_cast<hipStream_t>(stream)),
                    "rr_stream_copy");
}

rr_status rr_set_split_wait_ticks(uint64_t ticks) {
  g_err[0] = '\0';
  if (ticks > (uint64_t)100000000)
    return fail(RR_ERR_INVALID_ARG, "rr_set_split_wait_ticks: at most 10^8 ticks (1 s)");
  g_split_wait.store(ticks, std::memory_order_relaxed);
  return RR_OK;
}

rr_status rr_split_fallbacks(uint32_t* count, int reset) {
  g_err[0] = '\0';
  if (!count) return fail(RR_ERR_INVALID_ARG, "rr_split_fallbacks: null count");
  hipError_t e = hipSuccess;
  unsigned int* c = rr::split_fallback_counter(&e);
  if (!c) return hip_status(e, "rr_split_fallbacks");
  e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(count, c, sizeof(unsigned int), hipMemcpyDeviceToHost);
  if (e == hipSuccess && reset) e = hipMemset(c, 0, sizeof(unsigned int));
  if (e == hipSuccess && reset) e = hipDeviceSynchronize();
  return hip_status(e, "rr_split_fallbacks");
}
#endif  // RR_DIAG

}  // extern "C"
