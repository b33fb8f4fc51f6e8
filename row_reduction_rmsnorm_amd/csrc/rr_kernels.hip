// Row-reduce kernels for MI355X (gfx950): RMSNorm, fused residual add +
// RMSNorm, LayerNorm, and row softmax (and log-softmax, optionally under a
// causal rule) on the online normaliser.
//
// Every kernel follows the same shape: each lane reduces the elements it
// holds to a partial statistic (the sum of squares, or the online pair
// (m, d)); a wave64 all-reduce gives every lane the wavefront's statistic;
// when several wavefronts share a row, one LDS slot per wavefront and one
// barrier combine them, every lane folding the slots in the same order; then
// each lane rescales its own elements and stores them.
//
// Sources (web pages, cited by title and section):
//  [P1] "两个融合算子：RMSNorm 与 online softmax" (daleiyang.github.io)
//  [P2] "GPU Kernel 工程（04）：共享内存与 reduction——softmax、LayerNorm 与
//       online softmax" (arganzheng.life)
//  [P4] "Softmax 与归一化" (anrans.github.io ai-infra-handbooks)
//  [P5] "RMSNorm、Softmax 与在线归约" (notes.kuangjux.top)
//
// Launch shapes (chosen on the host, see rr_api.cpp):
//  * register kernels: blockDim = 64 * waves_per_row * rows_per_group with
//    either waves_per_row == 1 (a wavefront per row, no LDS, no barrier) or
//    rows_per_group == 1 (a workgroup per row).  Lane t of a row owns vectors
//    t, t + T, t + 2T, ... (T = 64 * waves_per_row) so every 16-byte access
//    of a wavefront is one contiguous 1 KiB segment.
//  * packed kernels (norm_packed_kernel, softmax_packed_kernel): 1024 lanes
//    per row holding up to 20 vectors each in the storage format.
//  * split softmax: 256-lane workgroups per chunk of a row, (m, d) pairs in a
//    caller workspace.
//  * the grid may be smaller than the number of rows (it is capped so that a
//    dispatch's work-items fit in 32 bits): workgroups then walk rows with a
//    stride of gridDim.x; gamma stays in registers across rows.
#include <atomic>
#include <map>
#include <mutex>
#include <tuple>
#include <utility>

#include "rr_device.h"
#include "rr_launch.h"

namespace rr {

// The norm kernels' three operations.
constexpr int kNormRms = 0;     // RMSNorm
constexpr int kNormFused = 1;   // residual add, then RMSNorm of the stored sum
constexpr int kNormLayer = 2;   // LayerNorm
static_assert(kNormRms == kLaunchRms && kNormFused == kLaunchFused && kNormLayer == kLaunchLayer,
              "operation codes");

namespace {

// ---------------------------------------------------------------------------
// Race stress.  A build with RR_STRESS defined to 1 (a separate library that
// only the tests load) adds two hooks to every LDS slot stage below, and its
// host side caps grids at a few dozen workgroups so that each workgroup walks
// many rows and reuses its slot sets over and over:
//  * stress_delay: a pause of 0-7 x 512 cycles, drawn per wavefront from its
//    clock, before every slot write and before every slot read, so that the
//    wavefronts of a workgroup reach them in shuffled order;
//  * stress_poison: right after a stage's barrier every wavefront has
//    finished reading the other slot set (its next write comes after this
//    barrier), so each wavefront overwrites its own slot there with NaN: a
//    read the barriers failed to order would see NaN, not a plausible value.
// Neither hook changes any arithmetic, so a correct stage gives the stress
// build the same bits as the normal one; the tests require exactly that.
// Normal builds contain no code for either.
// ---------------------------------------------------------------------------
#ifndef RR_STRESS
#define RR_STRESS 0
#endif

__device__ __forceinline__ void stress_delay() {
#if RR_STRESS
  const int n = (int)((__builtin_amdgcn_s_memtime() >> 4) & 7);
  for (int i = 0; i < n; ++i) __builtin_amdgcn_s_sleep(8);
#endif
}

template <typename S>
__device__ __forceinline__ void stress_poison(S (*slots)[kMaxWavesPerGroup], int parity, int w, int lane) {
#if RR_STRESS
  if (lane == 0) {
    S bad;
    float* f = reinterpret_cast<float*>(&bad);
    for (int i = 0; i < (int)(sizeof(S) / sizeof(float)); ++i) f[i] = __builtin_nanf("");
    slots[parity ^ 1][w] = bad;
  }
#else
  (void)slots;
  (void)parity;
  (void)w;
  (void)lane;
#endif
}

// LDS stage for one value per wavefront ([P2] section 四 and [P5] section
// "原 RMSNorm 草稿的两个关键错误": one slot per wavefront, a barrier, then a
// single combine).  Lane l of every wavefront reads slot (l mod 16) (the
// identity beyond the nw slots) and a four-step DPP butterfly inside each
// 16-lane row combines the 16 values, so every lane of the workgroup ends
// with the same bits and no broadcast step is needed.  `parity` selects one
// of two slot sets: a loop that reduces once per row alternates them, which
// makes the single barrier per row enough (a wavefront can only write a slot
// set again after the next barrier, which every wavefront reaches after
// finishing its reads of that set) -- the reuse hazard [P2] section 十 and
// [P4] section "实现" close with a trailing barrier.
__device__ __forceinline__ float group_sum(float v, int nw, int w, int lane,
                                           float (*slots)[kMaxWavesPerGroup], int parity) {
  stress_delay();
  if (lane == 0) slots[parity][w] = v;
  __syncthreads();
  stress_poison(slots, parity, w, lane);
  stress_delay();
  const int j = lane & (kMaxWavesPerGroup - 1);
  float t = (j < nw) ? slots[parity][j] : 0.0f;
  t = t + dpp_f32<kDppQuadXor1>(t);
  t = t + dpp_f32<kDppQuadXor2>(t);
  t = t + dpp_f32<kDppRowHalfMirror>(t);
  return t + dpp_f32<kDppRowMirror>(t);
}

__device__ __forceinline__ MD group_md(MD v, int nw, int w, int lane,
                                       MD (*slots)[kMaxWavesPerGroup], int parity) {
  stress_delay();
  if (lane == 0) slots[parity][w] = v;
  __syncthreads();
  stress_poison(slots, parity, w, lane);
  stress_delay();
  const int j = lane & (kMaxWavesPerGroup - 1);
  MD t;
  if (j < nw) {
    t = slots[parity][j];
  } else {
    t.m = kNegInf;
    t.d = 0.0f;
  }
  t = md_merge(t, dpp_md<kDppQuadXor1>(t));
  t = md_merge(t, dpp_md<kDppQuadXor2>(t));
  t = md_merge(t, dpp_md<kDppRowHalfMirror>(t));
  return md_merge(t, dpp_md<kDppRowMirror>(t));
}

// Two sums across the workgroup with one barrier: the slot scheme of
// group_sum, each slot holding a pair.
__device__ __forceinline__ void group_sum2(float& a, float& b, int nw, int w, int lane,
                                           float2 (*slots)[kMaxWavesPerGroup], int parity) {
  stress_delay();
  if (lane == 0) slots[parity][w] = make_float2(a, b);
  __syncthreads();
  stress_poison(slots, parity, w, lane);
  stress_delay();
  const int j = lane & (kMaxWavesPerGroup - 1);
  const float2 t = (j < nw) ? slots[parity][j] : make_float2(0.0f, 0.0f);
  float u = t.x, v = t.y;
  u = u + dpp_f32<kDppQuadXor1>(u);
  v = v + dpp_f32<kDppQuadXor1>(v);
  u = u + dpp_f32<kDppQuadXor2>(u);
  v = v + dpp_f32<kDppQuadXor2>(v);
  u = u + dpp_f32<kDppRowHalfMirror>(u);
  v = v + dpp_f32<kDppRowHalfMirror>(v);
  a = u + dpp_f32<kDppRowMirror>(u);
  b = v + dpp_f32<kDppRowMirror>(v);
}

// LayerNorm moments from the sums s1 = sum(d), s2 = sum(d^2) of d = x - K over
// a row of N values: c = s1 / N is the mean's offset from K and
// var = s2 / N - c^2.  That difference cancels when K lies far from the
// mean, and then every d also carries a rounding error at the scale of
// |K - mean| rather than of the spread; so it is accepted only when
// c^2 <= 4 var (K within two standard deviations of the mean).  Otherwise
// the caller re-centres on K + c (the mean, rounded to fp32) and sums again:
// the new offset is tiny, the difference no longer cancels, and x - (K + c)
// is exact wherever the mean is large next to the spread.
__device__ __forceinline__ bool ln_moments(float s1, float s2, int N, float& c, float& var) {
  c = s1 / (float)N;
  var = s2 / (float)N - c * c;
  return c * c <= 4.0f * var;
}

// The causal rule along a thread's rows: with period cp >= 1, row r keeps
// the keys j <= (r mod cp) + co, i.e. min(N, (r mod cp) + co + 1); cp == 0
// keeps every key.  A thread visits rows row0, row0 + stride, ...; the
// residue r mod cp is carried from row to row by one add and one compare,
// so the only division happens once, before the row loop.
struct CausalRows {
  int64_t cp, co, q, step;
  __device__ __forceinline__ CausalRows(int64_t row0, int64_t stride, int64_t cp_, int64_t co_)
      : cp(cp_), co(co_), q(0), step(0) {
    if (cp > 0) {
      q = row0 % cp;
      step = stride % cp;
    }
  }
  __device__ __forceinline__ int keys(int N) const {
    if (cp <= 0) return N;
    const int64_t k = q + co + 1;
    return k < (int64_t)N ? (int)k : N;
  }
  __device__ __forceinline__ void next() {
    if (cp > 0) {
      q += step;
      if (q >= cp) q -= cp;
    }
  }
};

// Entries of the vector starting at element e0 that lie at or past `keys`
// become -inf (they are masked keys; only the vector holding the last kept
// key can contain any).
template <int VEC>
__device__ __forceinline__ void mask_keys(float (&v)[VEC], int e0, int keys) {
  if (e0 + VEC <= keys) return;   // the whole vector is kept (always, without the rule)
#pragma unroll
  for (int i = 0; i < VEC; ++i)
    if (e0 + i >= keys) v[i] = kNegInf;
}

// Rows whose starts are not vector-aligned (SHIFT kernels; the host checks
// that input and output rows share their offset within a vector): row r is
// cut into vectors at aligned addresses, so vector j covers the row's
// elements [j * VEC - lead, (j + 1) * VEC - lead), lead = the row start's
// element offset within its vector (row_lead), or within the output's 64-byte
// block (frame_lead, below).  Vectors inside the row are accessed whole; the
// partial ones at its ends may reach outside it, and only their elements
// inside the row are accessed, one at a time (nothing outside the row is
// ever read or written).
template <typename T>
__device__ __forceinline__ int row_lead(const T* row_start, int vec) {
  return (int)((reinterpret_cast<uintptr_t>(row_start) / sizeof(T)) % (uintptr_t)vec);
}

// The frame of a cut row that is written: lead = the output row start's
// element offset within its 64-byte block, so that every wavefront's stores
// fill whole 64-byte sectors (stores that cover part of a sector, from two
// wavefronts, measured ~15% slower over a launch: 256 x 50256 bf16 -> fp32
// rows 32 bytes past a block 23.1 us, on block starts 20.1 us).  Vectors that
// lie wholly before the row start are empty.  The input row starts at the
// same element offset within a vector (checked by the host), so its vectors
// stay aligned.  The host sizes plans for the vector frame (a lead below one
// vector); a kernel that holds the row in `cap` vectors takes the 64-byte
// frame only where the row still fits, else the vector frame of the input.
template <typename Tout>
__device__ __forceinline__ int frame_lead(const Tout* out_row) {
  return (int)((reinterpret_cast<uintptr_t>(out_row) % 64u) / sizeof(Tout));
}
template <typename Tin, typename Tout>
__device__ __forceinline__ int frame_lead_within(const Tin* in_row, const Tout* out_row, int vec, int n,
                                                 int cap) {
  const int lead = frame_lead(out_row);
  return (lead + n + vec - 1) / vec <= cap ? lead : row_lead(in_row, vec);
}

// The elements e0 + i of a vector that lie in [0, keys), the rest `fill`
// (-inf for a softmax, 0 for the norms); keys >= 1.  Every element's load is
// issued before any is used: an index outside [0, keys) reads the nearest
// element inside (never anything outside the row) and is replaced by `fill`
// afterwards.  A load in a branch of its own, widened there, would wait for
// that one load before the next is issued.
//
// EdgeLoad splits that in two: issue() starts the element loads, values()
// widens them.  A kernel issues a row's partial vectors right after its whole
// vectors and widens them only once every load of the row is in flight (a
// wait for one edge vector would otherwise hold back the loads issued after
// it: a second memory round trip per row).  touch() marks the point from
// which the words may be used.
template <typename T, int VEC>
struct EdgeLoad {
  uint32_t raw[VEC];
  __device__ __forceinline__ void issue(const T* row, int e0, int keys) {
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      const int e = e0 + i;
      const int ec = e < 0 ? 0 : (e >= keys ? keys - 1 : e);
      if constexpr (std::is_same_v<T, float>) raw[i] = __float_as_uint(row[ec]);
      else raw[i] = static_cast<uint32_t>(row[ec]);
    }
  }
  __device__ __forceinline__ void touch() {
#pragma unroll
    for (int i = 0; i < VEC; ++i) asm volatile("" : "+v"(raw[i]));
  }
  __device__ __forceinline__ void values(int e0, int keys, float (&v)[VEC], float fill) const {
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      const int e = e0 + i;
      const float f = std::is_same_v<T, float> ? __uint_as_float(raw[i]) : __uint_as_float(raw[i] << 16);
      v[i] = (e >= 0 && e < keys) ? f : fill;
    }
  }
};
template <typename T, int VEC>
__device__ __forceinline__ void load_edge(const T* row, int e0, int keys, float (&v)[VEC],
                                          float fill = kNegInf) {
  EdgeLoad<T, VEC> el;
  el.issue(row, e0, keys);
  el.touch();
  el.values(e0, keys, v, fill);
}

// A cut row's partial vectors: its first (vector lead / VEC, held by lane
// lead / VEC at k = 0) and its last (vector nvec_row - 1, at k = k1), where
// either holds kept keys but is not whole inside the row.  issue() reads
// their elements in [0, keys) with load_cut into registers of their own, to
// be called right after the row's whole vectors are issued; finish(), once
// every load of the row is issued, completes them (-inf elsewhere) and puts
// them in place.  One memory round trip per row: an edge vector read or
// used in between would wait for every load before it.
template <typename Tin, int VEC>
struct CutEdges {
  Packed<Tin, VEC> c0, c1;
  bool has0, has1;
  int k1, lo0, hi0, hi1;
  __device__ __forceinline__ void issue(const Tin* xr, int t, int T, int lead, int nvec_row, int N, int keys) {
    const int nvec_keys = (lead + keys + VEC - 1) / VEC;
    auto partial = [&](int vi) {
      const int e0 = vi * VEC - lead;
      return vi < nvec_keys && !(e0 >= 0 && e0 + VEC <= N);
    };
    const int first = lead / VEC, last = nvec_row - 1;
    const int ef = first * VEC - lead, el = last * VEC - lead;   // ef <= 0 <= el
    has0 = t == first && partial(first);
    has1 = last > first && t == last % T && partial(last);
    k1 = last / T;
    lo0 = -ef;
    hi0 = keys - ef < VEC ? keys - ef : VEC;
    hi1 = keys - el < VEC ? keys - el : VEC;
    if (has0) c0.load_cut(xr + ef, lo0, hi0);
    if (has1) c1.load_cut(xr + el, 0, hi1);
  }
  template <int NV>
  __device__ __forceinline__ void finish(Packed<Tin, VEC> (&v)[NV]) {
    if (has0) {
      c0.finish_cut(lo0, hi0, kNegInf);
      v[0] = c0;
    }
    if (has1) {
      c1.finish_cut(0, hi1, kNegInf);
#pragma unroll
      for (int k = 0; k < NV; ++k)
        if (k == k1) v[k] = c1;
    }
  }
};

// Store the elements e0 + i that lie in [0, n).
template <typename T, int VEC>
__device__ __forceinline__ void store_edge(T* row, int e0, int n, const float (&o)[VEC]) {
#pragma unroll
  for (int i = 0; i < VEC; ++i) {
    const int e = e0 + i;
    if (e >= 0 && e < n) {
      const float one[1] = {o[i]};
      store_vec<T, 1>(row + e, one);
    }
  }
}

// Thread coordinates.  WAVE: each wavefront owns a row, the workgroup holds
// blockDim/64 rows.  Otherwise the whole workgroup (blockDim/64 wavefronts)
// owns one row.
struct RowLane {
  int lane;   // 0..63
  int w;      // wavefront within the row
  int nw;     // wavefronts per row
  int g;      // row slot within the workgroup
  int t;      // lane within the row (0 .. T-1)
  int T;      // lanes per row
  int rpg;    // rows per workgroup step
};

template <bool WAVE>
__device__ __forceinline__ RowLane row_lane() {
  RowLane r;
  const int wave = threadIdx.x >> 6;
  r.lane = threadIdx.x & 63;
  if constexpr (WAVE) {
    r.w = 0;
    r.nw = 1;
    r.g = wave;
    r.t = r.lane;
    r.T = kWave;
    r.rpg = blockDim.x >> 6;
  } else {
    r.w = wave;
    r.nw = blockDim.x >> 6;
    r.g = 0;
    r.t = threadIdx.x;
    r.T = blockDim.x;
    r.rpg = 1;
  }
  return r;
}

}  // namespace

// A row's vectors k * T + t (k < NV) are loaded in two steps: issue_row
// starts every load (packed words, 0 past the row's nvec vectors), and
// widen_row waits for them and widens to fp32.  Work that needs other loads
// (gamma's) goes between the two, and nothing is widened inside a load's
// bounds branch, where it would wait for that one load: every wait comes
// after all of the row's loads are in flight (one HBM round trip per row).
template <typename T, int VEC, int NV>
__device__ __forceinline__ void issue_row(const T* row, int nvec, int T_, int t, Packed<T, VEC> (&p)[NV]) {
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int vi = k * T_ + t;
    if (vi < nvec) p[k].template load<true>(row + (int64_t)vi * VEC);
    else p[k].zero();
  }
}
template <typename T, int VEC, int NV>
__device__ __forceinline__ void widen_row(Packed<T, VEC> (&p)[NV], float (&h)[NV][VEC]) {
#pragma unroll
  for (int k = 0; k < NV; ++k) p[k].touch();
#pragma unroll
  for (int k = 0; k < NV; ++k)
#pragma unroll
    for (int i = 0; i < VEC; ++i) h[k][i] = p[k].get(i);
}

// VEC elements p[e .. e + VEC) of a vector (gamma or beta), for windows
// that need not be aligned: window k is cut out of A[k], the aligned block
// holding its first element, and B[k], the block after it, d = that
// element's offset inside A[k] (a shift by whole dwords, then v_alignbyte for
// the 2-byte remainder of a bf16 offset).  Every window of a cut row has the
// same d (its vectors lie whole multiples of VEC apart), so callers pass a
// workgroup-uniform d and one uniform branch picks the dword shift for all
// the windows.  (Measured on 8192 x 4097 bf16 RMSNorm rows: 26.6 us; the
// shift chosen per dword, 28.8; the words indexed by the shift, which the
// compiler stages through LDS, 58.7.)
template <int Q, typename T, int VEC, int NV>
__device__ __forceinline__ void windows_cut_q(int r, const Packed<T, VEC> (&A)[NV], const Packed<T, VEC> (&B)[NV],
                                              Packed<T, VEC> (&out)[NV]) {
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const uint32_t C[8] = {A[k].w[0], A[k].w[1], A[k].w[2], A[k].w[3], B[k].w[0], B[k].w[1], B[k].w[2], B[k].w[3]};
#pragma unroll
    for (int j = 0; j < 4; ++j) out[k].w[j] = __builtin_amdgcn_alignbyte(C[j + Q + 1], C[j + Q], r);
  }
}
template <typename T, int VEC, int NV>
__device__ __forceinline__ void windows_cut(int d, const Packed<T, VEC> (&A)[NV], const Packed<T, VEC> (&B)[NV],
                                            Packed<T, VEC> (&out)[NV]) {
  static_assert(Packed<T, VEC>::kWords == 4, "16-byte vectors");
  const int bo = d * (int)sizeof(T);      // byte offset 0 .. 15
  const int r = bo & 3;
  switch (bo >> 2) {
    case 0: windows_cut_q<0>(r, A, B, out); break;
    case 1: windows_cut_q<1>(r, A, B, out); break;
    case 2: windows_cut_q<2>(r, A, B, out); break;
    default: windows_cut_q<3>(r, A, B, out); break;
  }
}

// ===========================================================================
// RMSNorm / fused add + RMSNorm, row held in registers (WAVE and BLOCK)
//
// [P1] section "三、N3：把 x 留在寄存器": keeping the row in registers with
// fully unrolled constant indices is what makes the kernel read x once.
// Fused: [P4] section "算子融合：fused_add_rms_norm", [P2] section 八.3.
// The fp32 sum x + r is rounded once to the I/O dtype; that rounded value is
// stored as the new residual and is the h whose squares are summed and which
// is rescaled.  Widening bf16 is exact and fp32 carries more than twice bf16's
// precision plus two bits, so rounding the fp32 sum to bf16 gives the
// correctly rounded sum.
//
// SHIFT: rows cut at aligned addresses.  x, y (and the residual) rows start
// at the same element offset within a vector (the host checks it); vector j
// covers the row's elements [j * VEC - lead, (j + 1) * VEC - lead), the frame
// starting at y's 64-byte block where the row still fits (frame_lead_within).
// Whole vectors inside the row are accessed whole, the row's partial vectors
// element by element (0 outside the row), and gamma (beta), which lie in a
// frame of their own, are read for each row in the row's frame: each lane's
// window is cut out of the two aligned blocks of gamma that hold it
// (window_cut; they stay in the cache across rows).
// ===========================================================================
// Cut LayerNorm rows held by a workgroup read gamma and beta through LDS:
// the workgroup stages both in LDS once, before its first row (layouts
// below), and each row reads its vectors' values there after its reduction.
// Held in registers (two blocks of each per vector while the row loads) they
// cost a cut LayerNorm row so many registers that a CU held half as many
// rows as for RMSNorm.
template <int KIND, bool WAVE, bool SHIFT>
constexpr bool norm_lds_params() {
  return SHIFT && !WAVE && KIND == kNormLayer;
}
// Two layouts of the staged parameters:
//  * fp32: one 8-byte entry per element, gamma's and beta's bits side by
//    side, element e at entry e + kParamPad: a row's vectors start at most a
//    64-byte frame's lead before the row (vectors wholly before it are
//    empty, and read the pad) and the last reaches VEC - 1 past its end.  A
//    vector's 4 entries are read as they lie, at any element offset.
//  * bf16: gamma's (beta's) aligned 16-byte blocks 0 .. amax, gamma at
//    [0, nbmax) and beta at [nbmax, 2 nbmax), and each vector's window cut
//    from two blocks.  (Per-element entries measured slower for bf16: in
//    element order a lane's 8 entries lie 32 bytes from the next lane's and
//    those 4-byte reads collide in the LDS banks; transposed so that the
//    lanes read consecutive words, every vector takes 8 reads and 8 address
//    additions.)
template <typename T>
constexpr bool kParamEntries = std::is_same_v<T, float>;
template <typename T>
constexpr int kParamPad = 64 / (int)sizeof(T) - 1;
// Bytes of LDS such a kernel takes for rows of N elements (the host's plan
// uses the same count).
template <typename T>
constexpr size_t norm_lds_param_bytes(int N) {
  static_assert(norm_lds_param_bytes_for(1, sizeof(T)) ==
                    (kParamEntries<T> ? (1 + kParamPad<T> + Elem<T>::kVec) * 8
                                      : 2 * ((1 + 2 * Elem<T>::kVec - 2) / Elem<T>::kVec) * 16),
                "staged parameter layout");
  return norm_lds_param_bytes_for(N, sizeof(T));
}

template <typename T, int NV, int KIND, bool WAVE, bool SHIFT>
__global__ __launch_bounds__(1024) void norm_regs_kernel(T* y, T* residual, const T* x,
                                                         const T* __restrict__ gamma,
                                                         const T* __restrict__ beta, int64_t M,
                                                         int N, float eps, RowStrides ld) {
  constexpr int VEC = Elem<T>::kVec;
  __shared__ float slots[2][kMaxWavesPerGroup];
  const RowLane rl = row_lane<WAVE>();
  const int nvec = N / VEC;
  // A cut LayerNorm row held by a workgroup stages gamma and beta in LDS
  // (norm_lds_params); the other forms keep them in registers.
  constexpr bool kLdsParams = norm_lds_params<KIND, WAVE, SHIFT>();
  extern __shared__ uint4 params_lds[];   // kLdsParams only (layouts above)
  uint2* const param_entries = reinterpret_cast<uint2*>(params_lds);
  const int nbmax = (N + 2 * VEC - 2) / VEC;

  if constexpr (kLdsParams) {
    // the parameters staged once; kBatch loads per lane in flight at once
    // (one round trip per batch).  The barrier orders these writes before
    // every read; nothing rewrites them.
    constexpr int kBatch = 8;
    if constexpr (kParamEntries<T>) {
      // element e at entry e + kParamPad (the pads are never written: only
      // elements outside the row, whose outputs are not stored, read them)
      for (int e0 = threadIdx.x; e0 < N; e0 += kBatch * blockDim.x) {
        float g[kBatch], b[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const int e = e0 + j * blockDim.x;
          if (e < N) {
            g[j] = gamma[e];
            b[j] = beta ? beta[e] : 0.0f;
          }
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const int e = e0 + j * blockDim.x;
          if (e < N) param_entries[e + kParamPad<T>] = make_uint2(__float_as_uint(g[j]), __float_as_uint(b[j]));
        }
      }
    } else {
      // gamma's blocks then beta's
      const int lg = row_lead(gamma, VEC);
      const int lb = beta ? row_lead(beta, VEC) : lg;
      const int ng = (N - 1 + lg) / VEC + 1, nb = (N - 1 + lb) / VEC + 1;
      const T* g0 = gamma - lg;
      const T* b0 = beta ? beta - lb : nullptr;
      const int total = ng + (beta ? nb : 0);
      for (int c0 = threadIdx.x; c0 < total; c0 += kBatch * blockDim.x) {
        Packed<T, VEC> q[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const int c = c0 + j * blockDim.x;
          if (c < ng) q[j].load(g0 + c * VEC);
          else if (c < total) q[j].load(b0 + (c - ng) * VEC);
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const int c = c0 + j * blockDim.x;
          if (c < total)
            params_lds[c < ng ? c : nbmax + (c - ng)] = make_uint4(q[j].w[0], q[j].w[1], q[j].w[2], q[j].w[3]);
        }
      }
    }
    __syncthreads();
  }

  Packed<T, VEC> gv[NV];
  Packed<T, VEC> bv[KIND == kNormLayer ? NV : 1];
  if constexpr (!SHIFT) {
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int vi = k * rl.T + rl.t;
      if (vi < nvec) gv[k].load(gamma + (int64_t)vi * VEC);
      else gv[k].fill(0.0f);
      if constexpr (KIND == kNormLayer) {
        if (vi < nvec && beta) bv[k].load(beta + (int64_t)vi * VEC);
        else bv[k].fill(0.0f);
      }
    }
  }

  const int64_t stride = (int64_t)gridDim.x * rl.rpg;
  int parity = 0;
  // a reduction over the row: wave butterfly, then (BLOCK) the LDS stage
  auto row_sum = [&](float v) {
    v = wave_sum(v);
    if constexpr (!WAVE) {
      v = group_sum(v, rl.nw, rl.w, rl.lane, slots, parity);
      parity ^= 1;
    }
    return v;
  };
  for (int64_t row = (int64_t)blockIdx.x * rl.rpg + rl.g; row < M; row += stride) {
    const int64_t ox = row * ld.x, oy = row * ld.y, orr = row * ld.r;
    // LayerNorm's shift (below), the row's first element: loaded ahead of
    // the row so that it arrives with the row rather than a round trip later
    float k_first = 0.0f;
    if constexpr (KIND == kNormLayer) k_first = load_one<T>(x + ox);
    float h[NV][VEC];
    // SHIFT: the row's frame (without SHIFT lead is 0 and nvec_row nvec)
    const int lead = SHIFT ? frame_lead_within(x + ox, y + oy, VEC, N, NV * rl.T) : 0;
    const int nvec_row = SHIFT ? (lead + N + VEC - 1) / VEC : nvec;
    // y's vector k of this lane (and, SHIFT, the row's partial vectors)
    auto store_row = [&](T* base, int k, const float (&o)[VEC]) {
      const int vi = k * rl.T + rl.t;
      if constexpr (SHIFT) {
        const int e0 = vi * VEC - lead;
        if (vi < nvec_row) {
          if (e0 >= 0 && e0 + VEC <= N) store_vec<T, VEC>(base + e0, o);
          else store_edge<T, VEC>(base, e0, N, o);
        }
      } else {
        if (vi < nvec) store_vec<T, VEC>(base + (int64_t)vi * VEC, o);
      }
    };
    // gamma (and beta) were loaded before the loop; marking their words here,
    // after this row's loads are issued, keeps their wait (and widening)
    // behind those loads instead of before the first row's
    auto params_after_loads = [&]() {
      if constexpr (kLdsParams) return;
#pragma unroll
      for (int k = 0; k < NV; ++k) gv[k].touch();
      if constexpr (KIND == kNormLayer) {
#pragma unroll
        for (int k = 0; k < NV; ++k) bv[k].touch();
      }
    };
    if constexpr (SHIFT) {
      // gamma (beta) in the row's frame: each lane's window [e0, e0 + VEC)
      // is cut out of the two aligned blocks of gamma that hold it.  Block a
      // holds gamma's elements [a * VEC - lg, (a + 1) * VEC - lg); blocks 0 ..
      // amax hold all of gamma, and each is read whole (the bytes around
      // gamma's two ends that share its first and last blocks are read and
      // ignored).  A window block outside that range is replaced by the
      // nearest one inside: the elements it supplies then lie outside
      // [0, N), where x counts zero and nothing is stored, so no window needs
      // mending.  The blocks are loaded first (from the cache), then the
      // row's whole vectors and its partial ones, then the windows are cut.
      const int lg = row_lead(gamma, VEC);
      const int lb = (KIND == kNormLayer && beta) ? row_lead(beta, VEC) : lg;
      constexpr int NB = KIND == kNormLayer ? NV : 1;
      constexpr int NW = kLdsParams ? 1 : NV;   // (no window blocks held in registers with LDS staging)
      Packed<T, VEC> ga[NW], gb[NW], ba[kLdsParams ? 1 : NB], bb[kLdsParams ? 1 : NB];
      auto inside = [&](int vi) {
        const int e0 = vi * VEC - lead;
        return vi < nvec_row && e0 >= 0 && e0 + VEC <= N;
      };
      // the aligned block holding element e of a parameter led by l
      // elements (floor division: e + l may be negative), clamped to 0 .. amax
      auto block = [&](int e, int l) {
        const int a = (e + l) >= 0 ? (e + l) / VEC : -((VEC - 1 - (e + l)) / VEC);
        const int amax = (N - 1 + l) / VEC;
        return a < 0 ? 0 : (a > amax ? amax : a);
      };
      auto block_base = [&](const T* p, int l) { return p - l; };   // block 0's first element
      if constexpr (!kLdsParams) {
#pragma unroll
        for (int k = 0; k < NW; ++k) {
          const int e0 = (k * rl.T + rl.t) * VEC - lead;
          const T* g0 = block_base(gamma, lg);
          ga[k].load(g0 + block(e0, lg) * VEC);
          gb[k].load(g0 + block(e0 + VEC, lg) * VEC);
          if constexpr (KIND == kNormLayer) {
            if (beta) {
              const T* b0 = block_base(beta, lb);
              ba[k].load(b0 + block(e0, lb) * VEC);
              bb[k].load(b0 + block(e0 + VEC, lb) * VEC);
            } else {
              ba[k].zero();
              bb[k].zero();
            }
          }
        }
      }
      Packed<T, VEC> px[NV], pr[KIND == kNormFused ? NV : 1];
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        const int vi = k * rl.T + rl.t;
        const int e0 = vi * VEC - lead;
        if (inside(vi)) {
          px[k].template load<true>(x + ox + e0);
          if constexpr (KIND == kNormFused) pr[k].template load<true>(residual + orr + e0);
        } else {
          px[k].zero();
          if constexpr (KIND == kNormFused) pr[k].zero();
        }
      }
      // the row's first vector (vector lead / VEC, k = 0; those before it are
      // empty) and its last, where partial: only their elements inside the
      // row are read (load_cut), into words of their own (loads into the
      // whole vectors' registers would have to wait for those), issued here
      // with the whole vectors and completed at the end
      auto partial = [&](int vi) {
        const int e0 = vi * VEC - lead;
        return vi < nvec_row && !(e0 >= 0 && e0 + VEC <= N);
      };
      const int last = nvec_row - 1;
      const int first = lead / VEC;
      const bool edge0 = rl.t == first && partial(first);
      const bool edge1 = last > first && rl.t == last % rl.T && partial(last);
      const int e_first = first * VEC - lead, e_last = last * VEC - lead;
      const int lo0 = e_first < 0 ? -e_first : 0, hi0 = N - e_first < VEC ? N - e_first : VEC;
      const int hi1 = N - e_last < VEC ? N - e_last : VEC;   // (its start lies inside the row)
      Packed<T, VEC> cx[2], cr[KIND == kNormFused ? 2 : 1];
      if (edge0) {
        cx[0].load_cut(x + ox + e_first, lo0, hi0);
        if constexpr (KIND == kNormFused) cr[0].load_cut(residual + orr + e_first, lo0, hi0);
      }
      if (edge1) {
        cx[1].load_cut(x + ox + e_last, 0, hi1);
        if constexpr (KIND == kNormFused) cr[1].load_cut(residual + orr + e_last, 0, hi1);
      }
      if constexpr (!kLdsParams) {
        // gamma's blocks are read only below, after every load above is
        // issued (an empty asm that may touch memory and "changes" the
        // blocks): else the compiler cuts each window as soon as its blocks
        // arrive, to free their registers, which holds back the loads after
        // them
#pragma unroll
        for (int k = 0; k < NW; ++k) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            asm volatile("" : "+v"(ga[k].w[j]), "+v"(gb[k].w[j]) : : "memory");
            if constexpr (KIND == kNormLayer) asm volatile("" : "+v"(ba[k].w[j]), "+v"(bb[k].w[j]) : : "memory");
          }
        }
        // the windows' offset inside their first block: (e0 + l) mod VEC
        // with e0 = vi * VEC - lead, the same for every vector of the row
        const int dg = (lg - lead) & (VEC - 1), db = (lb - lead) & (VEC - 1);
        windows_cut<T, VEC, NW>(dg, ga, gb, gv);
        if constexpr (KIND == kNormLayer) windows_cut<T, VEC, NW>(db, ba, bb, bv);
      }
      // the partial vectors completed, now that every load is in flight;
      // a LayerNorm row's elements outside it take the value K (below)
      // (every vector not read whole, before the partial ones are set)
      const float fill = KIND == kNormLayer ? uniform_f32(k_first) : 0.0f;
      if constexpr (KIND == kNormLayer) {
#pragma unroll
        for (int k = 0; k < NV; ++k)
          if (!inside(k * rl.T + rl.t)) px[k].fill(fill);
      }
      if (edge0) {
        cx[0].finish_cut(lo0, hi0, fill);
        px[0] = cx[0];
        if constexpr (KIND == kNormFused) {
          cr[0].finish_cut(lo0, hi0, 0.0f);
          pr[0] = cr[0];
        }
      }
      if (edge1) {
        const int kl = last / rl.T;
        cx[1].finish_cut(0, hi1, fill);
        if constexpr (KIND == kNormFused) cr[1].finish_cut(0, hi1, 0.0f);
#pragma unroll
        for (int k = 0; k < NV; ++k) {
          if (k == kl) {
            px[k] = cx[1];
            if constexpr (KIND == kNormFused) pr[k] = cr[1];
          }
        }
      }
      params_after_loads();
      widen_row<T, VEC, NV>(px, h);
      if constexpr (KIND == kNormFused) {
        float r[NV][VEC];
        widen_row<T, VEC, NV>(pr, r);
#pragma unroll
        for (int k = 0; k < NV; ++k) {
#pragma unroll
          for (int i = 0; i < VEC; ++i) h[k][i] = round_to<T>(h[k][i] + r[k][i]);
          store_row(residual + orr, k, h[k]);
        }
      }
    } else if constexpr (KIND == kNormFused) {
      float r[NV][VEC];
      Packed<T, VEC> px[NV], pr[NV];
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        const int vi = k * rl.T + rl.t;
        if (vi < nvec) {
          px[k].template load<true>(x + ox + (int64_t)vi * VEC);
          pr[k].template load<true>(residual + orr + (int64_t)vi * VEC);
        } else {
          px[k].zero();
          pr[k].zero();
        }
      }
      params_after_loads();
      widen_row<T, VEC, NV>(px, h);
      widen_row<T, VEC, NV>(pr, r);
#pragma unroll
      for (int k = 0; k < NV; ++k) {
#pragma unroll
        for (int i = 0; i < VEC; ++i) h[k][i] = round_to<T>(h[k][i] + r[k][i]);
        const int vi = k * rl.T + rl.t;
        if (vi < nvec) store_vec<T, VEC>(residual + orr + (int64_t)vi * VEC, h[k]);
      }
    } else {
      Packed<T, VEC> px[NV];
      issue_row<T, VEC, NV>(x + ox, nvec, rl.T, rl.t, px);
      params_after_loads();
      if constexpr (KIND == kNormLayer) {
        // lanes past the row's end hold the value K (below); a row that
        // fills every lane's vectors (a uniform test) has none
        if (nvec < NV * rl.T) {
          const float fill = uniform_f32(k_first);
#pragma unroll
          for (int k = 0; k < NV; ++k)
            if (k * rl.T + rl.t >= nvec) px[k].fill(fill);
        }
      }
      widen_row<T, VEC, NV>(px, h);
    }

    if constexpr (KIND == kNormLayer) {
      // [P4] section "练习" (LayerNorm): mean and variance from the values held
      // in registers, about a shift K: the row's first element, so that
      // x - K is exact for values near it and the sums carry no rounding at
      // the scale of the mean ([P2] section 八.2 warns about rows whose mean
      // is far larger than their spread).  One reduction carries sum(x - K)
      // and sum((x - K)^2), and x - mean = (x - K) - c.  A row whose first
      // element lies far from its mean (ln_moments) is shifted by K + c, its
      // mean rounded to fp32, and summed again: x - mean = (x - (K + c)) - c'.
      // The row is shifted in place, so one copy of it stays live.
      // K and the reduced sums are the same in every lane of the row (the
      // butterflies give every lane the same bits), so lane 0's copies are
      // moved to scalar registers, which frees vector registers
      const float K = uniform_f32(k_first);
      // sum(h - S) and sum((h - S)^2) over the lane's values, one
      // reduction.  A value outside the row holds S (K in the first pass,
      // 0 in the second), so it adds exactly zero and needs no test.
      auto pair_sums = [&](float S, float& s1, float& s2) {
        s1 = 0.0f;
        s2 = 0.0f;
#pragma unroll
        for (int k = 0; k < NV; ++k) {
#pragma unroll
          for (int i = 0; i < VEC; ++i) {
            const float d = h[k][i] - S;
            s1 += d;
            s2 += d * d;
          }
        }
        s1 = wave_sum(s1);
        s2 = wave_sum(s2);
        if constexpr (!WAVE) {
          __shared__ float2 pslots[2][kMaxWavesPerGroup];
          group_sum2(s1, s2, rl.nw, rl.w, rl.lane, pslots, parity);
          parity ^= 1;
        }
        s1 = uniform_f32(s1);
        s2 = uniform_f32(s2);
      };
      // pass 0 sums about K; a row whose K lies far from its mean (every lane
      // holds the same bits, so the whole row decides alike) is shifted by
      // K + c and summed once more (pass 1), about 0.  One copy of the
      // reduction code: the loop is not unrolled.
      float S = K, c = 0.0f, var = 0.0f;
#pragma nounroll
      for (int pass = 0; pass < 2; ++pass) {
        float s1, s2;
        pair_sums(S, s1, s2);
        const bool near = ln_moments(s1, s2, N, c, var) || pass == 1;
        const float shift = near ? S : S + c;
#pragma unroll
        for (int k = 0; k < NV; ++k)
#pragma unroll
          for (int i = 0; i < VEC; ++i) h[k][i] = h[k][i] - shift;
        if (near) break;
        // the values outside the row, K before the shift, are set to the
        // second pass's S.  (The vector's first element index is made
        // opaque here: else the compiler computes these tests before the
        // loop, for every row, and holds their masks through it.)
#pragma unroll
        for (int k = 0; k < NV; ++k) {
          int vi = k * rl.T + rl.t;
          asm volatile("" : "+v"(vi));
#pragma unroll
          for (int i = 0; i < VEC; ++i) {
            const int e = vi * VEC - lead + i;
            const bool in = SHIFT ? (vi < nvec_row && (unsigned)e < (unsigned)N) : vi < nvec;
            if (!in) h[k][i] = 0.0f;
          }
        }
        S = 0.0f;
      }
#pragma unroll
      for (int k = 0; k < NV; ++k)
#pragma unroll
        for (int i = 0; i < VEC; ++i) h[k][i] = h[k][i] - c;
      const float rstd = 1.0f / __builtin_sqrtf(__builtin_fmaxf(var, 0.0f) + eps);
      if constexpr (kLdsParams && kParamEntries<T>) {
        // each vector's gamma and beta from the entries of its elements (a
        // vector past the row reads the last ones)
#pragma unroll
        for (int k = 0; k < NV; ++k) {
          const int e0 = (k * rl.T + rl.t) * VEC - lead;
          const uint2* q = param_entries + ((e0 < N ? e0 : N - 1) + kParamPad<T>);
          float o[VEC];
#pragma unroll
          for (int i = 0; i < VEC; ++i) o[i] = (h[k][i] * rstd) * __uint_as_float(q[i].x) + __uint_as_float(q[i].y);
          store_row(y + oy, k, o);
        }
      } else if constexpr (kLdsParams) {
        // each vector's gamma and beta windows cut from the blocks in LDS
        const int lg = row_lead(gamma, VEC);
        const int lb = beta ? row_lead(beta, VEC) : lg;
        const int amg = (N - 1 + lg) / VEC, amb = (N - 1 + lb) / VEC;
        // vector vi's window starts in block vi + q, q = floor((l - lead) /
        // VEC) (the same for the whole row); blocks clamped to 0 .. amax
        auto floor_div = [](int v) { return v >= 0 ? v / VEC : -((VEC - 1 - v) / VEC); };
        const int qg = floor_div(lg - lead), qb = floor_div(lb - lead);
        auto clamp_block = [](int a, int amax) { return a < 0 ? 0 : (a > amax ? amax : a); };
        auto lds_block = [&](int a, Packed<T, VEC>& out) {
          const uint4 q = params_lds[a];
          out.w[0] = q.x; out.w[1] = q.y; out.w[2] = q.z; out.w[3] = q.w;
        };
        const int dg = (lg - lead) & (VEC - 1), db = (lb - lead) & (VEC - 1);
#pragma unroll
        for (int k = 0; k < NV; ++k) {
          const int vi = k * rl.T + rl.t;
          Packed<T, VEC> A[1], Bk[1], G[1], Bt[1];
          lds_block(clamp_block(vi + qg, amg), A[0]);
          lds_block(clamp_block(vi + qg + 1, amg), Bk[0]);
          windows_cut<T, VEC, 1>(dg, A, Bk, G);
          if (beta) {
            lds_block(nbmax + clamp_block(vi + qb, amb), A[0]);
            lds_block(nbmax + clamp_block(vi + qb + 1, amb), Bk[0]);
            windows_cut<T, VEC, 1>(db, A, Bk, Bt);
          } else {
            Bt[0].zero();
          }
          float o[VEC];
#pragma unroll
          for (int i = 0; i < VEC; ++i) o[i] = (h[k][i] * rstd) * G[0].get(i) + Bt[0].get(i);
          store_row(y + oy, k, o);
        }
      } else {
#pragma unroll
        for (int k = 0; k < NV; ++k) {
          float o[VEC];
#pragma unroll
          for (int i = 0; i < VEC; ++i) o[i] = (h[k][i] * rstd) * gv[k].get(i) + bv[k].get(i);
          store_row(y + oy, k, o);
        }
      }
    } else {
      float ss = 0.0f;
#pragma unroll
      for (int k = 0; k < NV; ++k)
#pragma unroll
        for (int i = 0; i < VEC; ++i) ss += h[k][i] * h[k][i];
      // eps inside the root, mean over N ([P5] section "RMSNorm 归约什么").
      const float rstd = 1.0f / __builtin_sqrtf(row_sum(ss) / (float)N + eps);
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        float o[VEC];
#pragma unroll
        for (int i = 0; i < VEC; ++i) o[i] = (h[k][i] * rstd) * gv[k].get(i);
        store_row(y + oy, k, o);
      }
    }
  }
}

// ===========================================================================
// RMSNorm / fused, streaming (LOOP): any N, any alignment (VEC may be 1).
// Pass 1 reads the row (and for the fused op writes the new residual) and
// sums squares; pass 2 reads it again -- x, or the stored residual -- and
// writes y.  Each lane revisits exactly the elements it handled in pass 1.
// ===========================================================================
template <typename T, int VEC, int KIND>
__global__ __launch_bounds__(1024) void norm_loop_kernel(T* y, T* residual, const T* x,
                                                         const T* __restrict__ gamma,
                                                         const T* __restrict__ beta, int64_t M,
                                                         int N, float eps, RowStrides ld) {
  __shared__ float slots[2][kMaxWavesPerGroup];
  const RowLane rl = row_lane<false>();
  const int nvec = N / VEC;
  int parity = 0;
  auto row_sum = [&](float v) {
    v = wave_sum(v);
    v = group_sum(v, rl.nw, rl.w, rl.lane, slots, parity);
    parity ^= 1;
    return v;
  };
  for (int64_t row = blockIdx.x; row < M; row += gridDim.x) {
    const int64_t ox = row * ld.x, oy = row * ld.y, orr = row * ld.r;
    if constexpr (KIND == kNormLayer) {
      // one pass for sum(x - K) and sum((x - K)^2) about the row's first
      // element (a second about the mean when the first element lies far
      // from it, see ln_moments), then the output pass, centred as
      // (x - K) - c as in the register kernel
      float K = load_one<T>(x + ox);
      float c, var;
      auto moments = [&]() {
        float s1 = 0.0f, s2 = 0.0f;
        for (int vi = rl.t; vi < nvec; vi += rl.T) {
          float h[VEC];
          load_vec<T, VEC, false>(x + ox + (int64_t)vi * VEC, h);
#pragma unroll
          for (int i = 0; i < VEC; ++i) {
            const float d = h[i] - K;
            s1 += d;
            s2 += d * d;
          }
        }
        s1 = wave_sum(s1);
        s2 = wave_sum(s2);
        __shared__ float2 pslots[2][kMaxWavesPerGroup];
        group_sum2(s1, s2, rl.nw, rl.w, rl.lane, pslots, parity);
        parity ^= 1;
        return ln_moments(s1, s2, N, c, var);
      };
      if (!moments()) {
        K = K + c;
        moments();
      }
      const float rstd = 1.0f / __builtin_sqrtf(__builtin_fmaxf(var, 0.0f) + eps);
      for (int vi = rl.t; vi < nvec; vi += rl.T) {
        float h[VEC], g[VEC], bb[VEC];
        load_vec<T, VEC>(x + ox + (int64_t)vi * VEC, h);
        load_vec<T, VEC, false>(gamma + (int64_t)vi * VEC, g);
        if (beta) {
          load_vec<T, VEC, false>(beta + (int64_t)vi * VEC, bb);
        } else {
#pragma unroll
          for (int i = 0; i < VEC; ++i) bb[i] = 0.0f;
        }
#pragma unroll
        for (int i = 0; i < VEC; ++i) h[i] = (((h[i] - K) - c) * rstd) * g[i] + bb[i];
        store_vec<T, VEC>(y + oy + (int64_t)vi * VEC, h);
      }
    } else {
      float ss = 0.0f;
      for (int vi = rl.t; vi < nvec; vi += rl.T) {
        float h[VEC];
        load_vec<T, VEC>(x + ox + (int64_t)vi * VEC, h);
        if constexpr (KIND == kNormFused) {
          float r[VEC];
          load_vec<T, VEC>(residual + orr + (int64_t)vi * VEC, r);
#pragma unroll
          for (int i = 0; i < VEC; ++i) h[i] = round_to<T>(h[i] + r[i]);
          store_vec<T, VEC>(residual + orr + (int64_t)vi * VEC, h);
        }
#pragma unroll
        for (int i = 0; i < VEC; ++i) ss += h[i] * h[i];
      }
      const float rstd = 1.0f / __builtin_sqrtf(row_sum(ss) / (float)N + eps);
      const T* src = KIND == kNormFused ? residual + orr : x + ox;
      for (int vi = rl.t; vi < nvec; vi += rl.T) {
        float h[VEC], g[VEC];
        load_vec<T, VEC>(src + (int64_t)vi * VEC, h);
        load_vec<T, VEC, false>(gamma + (int64_t)vi * VEC, g);
#pragma unroll
        for (int i = 0; i < VEC; ++i) h[i] = (h[i] * rstd) * g[i];
        store_vec<T, VEC>(y + oy + (int64_t)vi * VEC, h);
      }
    }
  }
}

// ===========================================================================
// RMSNorm / fused / LayerNorm, long rows held packed in registers (BLOCK,
// large NV): rows beyond the register budget of norm_regs_kernel (16 widened
// values per lane) and up to 64K elements.  1024 lanes hold the row in its
// storage format (bf16 stays two to a register; the fused op keeps the
// rounded sum h, exact in the storage format), so x is still read once; gamma
// and beta are not kept but read again at store time, from L2 (one vector
// per row and launch).  Same reductions and arithmetic as norm_regs_kernel.
// ===========================================================================
template <typename T, int NV, int KIND>
__global__ __launch_bounds__(1024) void norm_packed_kernel(T* y, T* residual, const T* x,
                                                           const T* __restrict__ gamma,
                                                           const T* __restrict__ beta, int64_t M,
                                                           int N, float eps, RowStrides ld) {
  constexpr int VEC = Elem<T>::kVec;
  constexpr int kThreads = 1024;
  __shared__ float slots[2][kMaxWavesPerGroup];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int nvec = N / VEC;
  int parity = 0;
  auto row_sum = [&](float v) {
    v = wave_sum(v);
    v = group_sum(v, kThreads / kWave, w, lane, slots, parity);
    parity ^= 1;
    return v;
  };
  for (int64_t row = blockIdx.x; row < M; row += gridDim.x) {
    const T* xr = x + row * ld.x;   // uniform row bases
    T* yr = y + row * ld.y;
    // lane offsets recomputed at each use from an opaque copy of the lane
    // index, which frees the registers the packed row needs
    int t_ld = t;
    asm volatile("" : "+v"(t_ld));
    Packed<T, VEC> v[NV];
    if constexpr (KIND == kNormFused) {
      T* rr = residual + row * ld.r;
      Packed<T, VEC> r[NV];
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        const int vi = k * kThreads + t_ld;
        if (vi < nvec) {
          v[k].template load<true>(xr + vi * VEC);
          r[k].template load<true>(rr + vi * VEC);
        } else {
          v[k].zero();
          r[k].zero();
        }
      }
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        const int vi = k * kThreads + t_ld;
        float h[VEC];
#pragma unroll
        for (int i = 0; i < VEC; ++i) h[i] = round_to<T>(v[k].get(i) + r[k].get(i));
        if (vi < nvec) store_vec<T, VEC>(rr + vi * VEC, h);
        v[k].set(h);
      }
    } else {
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        const int vi = k * kThreads + t_ld;
        if (vi < nvec) v[k].template load<true>(xr + vi * VEC);
        else v[k].zero();
      }
    }
#pragma unroll
    for (int k = 0; k < NV; ++k) v[k].touch();
    int t_st = t;
    asm volatile("" : "+v"(t_st));
    if constexpr (KIND == kNormLayer) {
      // about a shift K (the row's first element, or the mean after a second
      // sum), as in norm_regs_kernel
      float K = load_one<T>(xr);
      float c, var;
      auto moments = [&]() {
        float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
        for (int k = 0; k < NV; ++k) {
          const bool valid = k * kThreads + t < nvec;
#pragma unroll
          for (int i = 0; i < VEC; ++i) {
            const float d = valid ? v[k].get(i) - K : 0.0f;
            s1 += d;
            s2 += d * d;
          }
        }
#pragma unroll
        for (int k = 0; k < NV; ++k) v[k].touch();
        s1 = wave_sum(s1);
        s2 = wave_sum(s2);
        __shared__ float2 pslots[2][kMaxWavesPerGroup];
        group_sum2(s1, s2, kThreads / kWave, w, lane, pslots, parity);
        parity ^= 1;
        return ln_moments(s1, s2, N, c, var);
      };
      if (!moments()) {
        K = K + c;
        moments();
      }
      const float rstd = 1.0f / __builtin_sqrtf(__builtin_fmaxf(var, 0.0f) + eps);
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        const int vi = k * kThreads + t_st;
        if (vi < nvec) {
          float g[VEC], b[VEC], o[VEC];
          load_vec<T, VEC, false>(gamma + vi * VEC, g);
          if (beta) {
            load_vec<T, VEC, false>(beta + vi * VEC, b);
          } else {
#pragma unroll
            for (int i = 0; i < VEC; ++i) b[i] = 0.0f;
          }
#pragma unroll
          for (int i = 0; i < VEC; ++i) o[i] = (((v[k].get(i) - K) - c) * rstd) * g[i] + b[i];
          store_vec<T, VEC>(yr + vi * VEC, o);
        }
      }
    } else {
      float ss = 0.0f;
#pragma unroll
      for (int k = 0; k < NV; ++k)
#pragma unroll
        for (int i = 0; i < VEC; ++i) ss += v[k].get(i) * v[k].get(i);
#pragma unroll
      for (int k = 0; k < NV; ++k) v[k].touch();
      const float rstd = 1.0f / __builtin_sqrtf(row_sum(ss) / (float)N + eps);
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        const int vi = k * kThreads + t_st;
        if (vi < nvec) {
          float g[VEC], o[VEC];
          load_vec<T, VEC, false>(gamma + vi * VEC, g);
#pragma unroll
          for (int i = 0; i < VEC; ++i) o[i] = (v[k].get(i) * rstd) * g[i];
          store_vec<T, VEC>(yr + vi * VEC, o);
        }
      }
    }
  }
}

// ===========================================================================
// Short rows, several per wavefront (SUBWAVE).
//
// [P4] section "按行长度选择并行方式": rows of a few dozen elements should not
// occupy a whole wavefront.  A wavefront holds 64/L rows of L lanes each;
// lane j of a row owns vector j (one vector, VEC elements, or one element when
// VEC = 1, so unaligned short rows take this path too).  The reductions run
// only the butterfly steps inside an L-lane group, so no LDS and no barrier.
// ===========================================================================
template <typename T, int VEC, int L, int KIND>
__global__ __launch_bounds__(256) void norm_sub_kernel(T* y, T* residual, const T* x,
                                                       const T* __restrict__ gamma,
                                                       const T* __restrict__ beta, int64_t M,
                                                       int N, float eps, RowStrides ld) {
  constexpr int kRowsPerGroup = 256 / L;
  const int j = threadIdx.x & (L - 1);              // lane within the row
  const int nvec = N / VEC;
  const bool active = j < nvec;
  Packed<T, VEC> g, bb;
  if (active) g.load(gamma + (int64_t)j * VEC);
  else g.fill(0.0f);
  if (active && KIND == kNormLayer && beta) bb.load(beta + (int64_t)j * VEC);
  else bb.fill(0.0f);
  for (int64_t row = (int64_t)blockIdx.x * kRowsPerGroup + (threadIdx.x / L); row < M;
       row += (int64_t)gridDim.x * kRowsPerGroup) {
    const int64_t cj = (int64_t)j * VEC;
    const int64_t ox = row * ld.x + cj, oy = row * ld.y + cj, orr = row * ld.r + cj;
    // the row's loads first, then gamma's words (loaded before the loop), then
    // the widening: every wait comes after the row's loads are in flight
    Packed<T, VEC> px, pr;
    if (active) {
      px.template load<true>(x + ox);
      if constexpr (KIND == kNormFused) pr.template load<true>(residual + orr);
    } else {
      px.zero();
      pr.zero();
    }
    g.touch();
    if constexpr (KIND == kNormLayer) bb.touch();
    px.touch();
    float h[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) h[i] = px.get(i);
    if constexpr (KIND == kNormFused) {
      pr.touch();
#pragma unroll
      for (int i = 0; i < VEC; ++i) h[i] = round_to<T>(h[i] + pr.get(i));
      if (active) store_vec<T, VEC>(residual + orr, h);
    }
    float o[VEC];
    if constexpr (KIND == kNormLayer) {
      // about a shift K (the row's first element, or the mean after a second
      // sum), as in norm_regs_kernel; the group's lanes hold the same bits
      float K = load_one<T>(x + row * ld.x);
      float c, var;
      auto moments = [&]() {
        float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          const float d = active ? h[i] - K : 0.0f;
          s1 += d;
          s2 += d * d;
        }
        return ln_moments(group_lanes_sum<L>(s1), group_lanes_sum<L>(s2), N, c, var);
      };
      if (!moments()) {
        K = K + c;
        moments();
      }
      const float rstd = 1.0f / __builtin_sqrtf(__builtin_fmaxf(var, 0.0f) + eps);
#pragma unroll
      for (int i = 0; i < VEC; ++i) o[i] = (((h[i] - K) - c) * rstd) * g.get(i) + bb.get(i);
    } else {
      float ss = 0.0f;
#pragma unroll
      for (int i = 0; i < VEC; ++i) ss += h[i] * h[i];
      ss = group_lanes_sum<L>(ss);
      const float rstd = 1.0f / __builtin_sqrtf(ss / (float)N + eps);
#pragma unroll
      for (int i = 0; i < VEC; ++i) o[i] = (h[i] * rstd) * g.get(i);
    }
    if (active) store_vec<T, VEC>(y + oy, o);
  }
}

// Elements per vector of a softmax kernel.  A bf16 row written as fp32 is
// read four elements (8 bytes) at a time, so that each lane writes one 16-byte
// fp32 vector and a wavefront's store covers 1 KiB without gaps; eight per
// load (16 bytes) would give each lane two stores 16 bytes apart and every
// store instruction only half of each line it touches (measured on a
// 4096 x 32000 softmax: 3.6 TB/s that way, 4.35 TB/s this way).  Every other
// pairing reads 16 bytes per load.
template <typename Tin, typename Tout>
constexpr int softmax_vec() {
  return (std::is_same_v<Tin, bf16_t> && std::is_same_v<Tout, float>) ? 4 : Elem<Tin>::kVec;
}

template <typename Tin, typename Tout, int VEC, int L, bool LOG, bool CAUSAL>
__global__ __launch_bounds__(256) void softmax_sub_kernel(const Tin* x, Tout* y, int64_t M, int N,
                                                          int64_t cp, int64_t co, RowStrides ld) {
  constexpr int kRowsPerGroup = 256 / L;
  const int j = threadIdx.x & (L - 1);
  const int nvec = N / VEC;
  const int64_t row0 = (int64_t)blockIdx.x * kRowsPerGroup + (threadIdx.x / L);
  const int64_t stride = (int64_t)gridDim.x * kRowsPerGroup;
  CausalRows cr(row0, stride, CAUSAL ? cp : 0, co);
  for (int64_t row = row0; row < M; row += stride, cr.next()) {
    const int keys = cr.keys(N);
    const int64_t ox = row * ld.x + (int64_t)j * VEC, oy = row * ld.y + (int64_t)j * VEC;
    float v[VEC];
    if (j * VEC < keys) {
      load_vec<Tin, VEC>(x + ox, v);
      mask_keys<VEC>(v, j * VEC, keys);
    } else {
#pragma unroll
      for (int i = 0; i < VEC; ++i) v[i] = kNegInf;
    }
    float ml = v[0];
#pragma unroll
    for (int i = 1; i < VEC; ++i) ml = __builtin_fmaxf(ml, v[i]);
    const float shift = (ml == kNegInf) ? 0.0f : ml;
    float dl = 0.0f;
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      const float e = exp_out<Tout>(v[i] - shift);
      dl += e;
      if constexpr (!LOG) v[i] = e;
    }
    MD p;
    p.m = ml;
    p.d = dl;
    p = group_lanes_md<L>(p);
    float o[VEC];
    if constexpr (LOG) {
      const float ld = __builtin_logf(p.d);
#pragma unroll
      for (int i = 0; i < VEC; ++i) o[i] = (v[i] - p.m) - ld;
    } else {
      float c = (ml == kNegInf) ? 0.0f : exp_out<Tout>(ml - p.m) / p.d;
      if (p.m == kNegInf) c = __builtin_nanf("");
#pragma unroll
      for (int i = 0; i < VEC; ++i) o[i] = v[i] * c;
    }
    if (j < nvec) store_vec<Tout, VEC>(y + oy, o);
  }
}

// ===========================================================================
// Softmax, row held in registers (WAVE and BLOCK).
//
// Each lane summarises the NV*VEC values it holds as a pair (m_l, d_l): its
// maximum, then the sum of e_i = exp(x_i - m_l), keeping the e_i in the
// registers that held x ([P1] section "四、S4：float4，顺便演示了分块合并": a
// chunk summary merged into the running pair).  The pairs are combined with
// the merge across the wavefront and, for BLOCK, across wavefronts, which
// gives the row's (m, d) in every lane.  The outputs are then
//   y_i = e_i * c_l,  c_l = exp(m_l - m) / d,
// one exponential per element plus one per lane: e_i * exp(m_l - m) =
// exp(x_i - m) is the rescale of [P1] section "二、递推式怎么来的".
// Entries equal to -inf give e_i = 0 and so y_i = 0 exactly.  A lane whose
// entries are all -inf has m_l = -inf and c_l = 0; a row whose entries are
// all -inf has m = -inf and every output is NaN, as exp(x - m)/d is.
// ===========================================================================
template <typename Tin, typename Tout, int NV, bool WAVE, bool LOG, bool CAUSAL, bool SHIFT>
__global__ __launch_bounds__(1024) void softmax_regs_kernel(const Tin* x, Tout* y, int64_t M,
                                                            int N, int64_t cp, int64_t co, RowStrides ld) {
  constexpr int VEC = softmax_vec<Tin, Tout>();
  __shared__ MD slots[2][kMaxWavesPerGroup];
  const RowLane rl = row_lane<WAVE>();
  const int nvec = N / VEC;
  const int64_t stride = (int64_t)gridDim.x * rl.rpg;
  const int64_t row0 = (int64_t)blockIdx.x * rl.rpg + rl.g;
  CausalRows cr(row0, stride, CAUSAL ? cp : 0, co);
  int parity = 0;
  for (int64_t row = row0; row < M; row += stride, cr.next()) {
    const int keys = cr.keys(N);
    const Tin* xr = x + row * ld.x;
    Tout* yr = y + row * ld.y;
    // SHIFT: vector j covers the row's elements [j * VEC - lead, ...)
    const int lead = SHIFT ? frame_lead_within(xr, yr, VEC, N, NV * rl.T) : 0;
    const int nvec_row = SHIFT ? (lead + N + VEC - 1) / VEC : nvec;
    const int nvec_keys = (lead + keys + VEC - 1) / VEC;   // vectors holding kept keys
    float v[NV][VEC];
    if constexpr (SHIFT && WAVE) {
      // a wavefront's row holds both of its partial vectors: their element
      // loads are issued after the whole vectors and completed once all are
      // in flight, so that the wavefront waits once (the packed words, fp32:
      // the values themselves, are widened only after that)
      Packed<Tin, VEC> raw[NV];
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        const int vi = k * rl.T + rl.t;
        const int e0 = vi * VEC - lead;
        if (vi < nvec_keys && e0 >= 0 && e0 + VEC <= N) raw[k].template load<true>(xr + e0);
        else raw[k].fill(kNegInf);
      }
      CutEdges<Tin, VEC> edges;
      edges.issue(xr, rl.t, rl.T, lead, nvec_row, N, keys);
      edges.finish(raw);
#pragma unroll
      for (int k = 0; k < NV; ++k) raw[k].touch();
#pragma unroll
      for (int k = 0; k < NV; ++k)
#pragma unroll
        for (int i = 0; i < VEC; ++i) v[k][i] = raw[k].get(i);
    } else if constexpr (std::is_same_v<Tin, float>) {
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        const int vi = k * rl.T + rl.t;
        const int e0 = vi * VEC - lead;
        if (vi < nvec_keys && (!SHIFT || (e0 >= 0 && e0 + VEC <= N))) {
          load_vec<Tin, VEC>(xr + e0, v[k]);
        } else {
#pragma unroll
          for (int i = 0; i < VEC; ++i) v[k][i] = kNegInf;
        }
      }
      if constexpr (SHIFT) {
        // the row's first and last vector, element by element, once every
        // whole vector's load is issued (their loads reuse those registers,
        // so an edge vector read in between would wait for the loads before it)
#pragma unroll
        for (int k = 0; k < NV; ++k) {
          const int vi = k * rl.T + rl.t;
          const int e0 = vi * VEC - lead;
          if (vi < nvec_keys && !(e0 >= 0 && e0 + VEC <= N)) load_edge<Tin, VEC>(xr, e0, keys, v[k]);
        }
      }
    } else {
      // bf16: load the packed words and widen them only once every load is
      // issued.  Widened inside each load's branch, every branch would wait
      // for its own load: one HBM round trip per vector instead of one in all.
      Packed<Tin, VEC> raw[NV];
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        const int vi = k * rl.T + rl.t;
        const int e0 = vi * VEC - lead;
        if (vi < nvec_keys && (!SHIFT || (e0 >= 0 && e0 + VEC <= N))) raw[k].template load<true>(xr + e0);
        else raw[k].fill(kNegInf);
      }
#pragma unroll
      for (int k = 0; k < NV; ++k) raw[k].touch();
#pragma unroll
      for (int k = 0; k < NV; ++k)
#pragma unroll
        for (int i = 0; i < VEC; ++i) v[k][i] = raw[k].get(i);
      if constexpr (SHIFT) {
        // the row's first and last vector, element by element, after the rest
#pragma unroll
        for (int k = 0; k < NV; ++k) {
          const int vi = k * rl.T + rl.t;
          const int e0 = vi * VEC - lead;
          if (vi < nvec_keys && !(e0 >= 0 && e0 + VEC <= N)) load_edge<Tin, VEC>(xr, e0, keys, v[k]);
        }
      }
    }
    // a row the causal rule cuts: keys past the count inside the vector
    // holding the last kept key become -inf (after all loads are issued)
    if (keys < N) {
#pragma unroll
      for (int k = 0; k < NV; ++k) mask_keys<VEC>(v[k], (k * rl.T + rl.t) * VEC - lead, keys);
    }
    float ml = kNegInf;
#pragma unroll
    for (int k = 0; k < NV; ++k)
#pragma unroll
      for (int i = 0; i < VEC; ++i) ml = __builtin_fmaxf(ml, v[k][i]);
    // shift by 0 when the lane holds only -inf so that exp(-inf - 0) = 0
    const float shift = (ml == kNegInf) ? 0.0f : ml;
    float dl = 0.0f;
#pragma unroll
    for (int k = 0; k < NV; ++k)
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        const float e = exp_out<Tout>(v[k][i] - shift);
        dl += e;
        if constexpr (!LOG) v[k][i] = e;   // plain softmax keeps e_i, log-softmax keeps x_i
      }
    MD p;
    p.m = ml;
    p.d = dl;
    p = wave_md(p);
    if constexpr (!WAVE) {
      p = group_md(p, rl.nw, rl.w, rl.lane, slots, parity);
      parity ^= 1;
    }
    float c = 0.0f, ld = 0.0f;
    if constexpr (LOG) {
      ld = __builtin_logf(p.d);
    } else {
      c = (ml == kNegInf) ? 0.0f : exp_out<Tout>(ml - p.m) / p.d;
      if (p.m == kNegInf) c = __builtin_nanf("");
    }
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int vi = k * rl.T + rl.t;
      const int e0 = vi * VEC - lead;
      float o[VEC];
#pragma unroll
      for (int i = 0; i < VEC; ++i) o[i] = LOG ? (v[k][i] - p.m) - ld : v[k][i] * c;
      if (vi < nvec_row) {
        if (!SHIFT || (e0 >= 0 && e0 + VEC <= N)) store_vec<Tout, VEC>(yr + e0, o);
        else store_edge<Tout, VEC>(yr, e0, N, o);
      }
    }
  }
}

// ===========================================================================
// Causal rule, two rows per workgroup (aligned rows of the workgroup plan).
//
// Under the causal rule row q of a period keeps q + O + 1 keys ([P1] section
// "二、它们在 Qwen2.5-7B 里的真实位置": the attention scores of a layer), so a
// workgroup per row reads anywhere from one key to a whole row while always
// writing a whole row: a workgroup with a short row is bound by the latency
// of its few loads, not by bytes, and the short rows of each period come
// together in launch order.  Pairing row q with row P - 1 - q of the same
// period gives every workgroup P + 2O + 1 kept keys between its two rows
// (about one row) and two rows to write.  Each row is held exactly as
// softmax_regs_kernel holds it (lane t owns vectors t, t + T, ...), with the
// same per-lane pair, butterfly and slot stage, so both rows come out with
// the bits that kernel gives them; the two rows share one barrier.  Rows past
// the last whole period, and the middle row of an odd period, go alone.
// ===========================================================================
template <typename Tin, typename Tout, int NV, bool LOG>
__global__ __launch_bounds__(1024) void softmax_causal_pair_kernel(const Tin* x, Tout* y, int64_t M, int N,
                                                                   int64_t P, int64_t O, RowStrides ld) {
  constexpr int VEC = softmax_vec<Tin, Tout>();
  __shared__ MD slots_a[2][kMaxWavesPerGroup];   // [parity][wavefront], one set per row of the pair
  __shared__ MD slots_b[2][kMaxWavesPerGroup];
  MD (*const sl[2])[kMaxWavesPerGroup] = {slots_a, slots_b};
  const RowLane rl = row_lane<false>();
  const int nvec = N / VEC;
  const int64_t per = (P + 1) / 2;          // work items per whole period
  const int64_t whole = M / P;              // whole periods
  const int64_t items = whole * per + (M - whole * P);
  int parity = 0;
  for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
    int64_t row[2], q[2];                   // row[1] < 0: row[0] alone
    if (item < whole * per) {
      const int64_t blk = item / per;
      q[0] = item - blk * per;
      q[1] = P - 1 - q[0];
      row[0] = blk * P + q[0];
      row[1] = q[1] != q[0] ? blk * P + q[1] : -1;
    } else {
      row[0] = whole * P + (item - whole * per);
      q[0] = row[0] - whole * P;
      row[1] = -1;
      q[1] = 0;
    }
    const int npair = row[1] < 0 ? 1 : 2;
    int keys[2], nkv[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      keys[r] = r < npair ? (int)(q[r] + O + 1 < (int64_t)N ? q[r] + O + 1 : (int64_t)N) : 0;
      nkv[r] = (keys[r] + VEC - 1) / VEC;   // vectors holding kept keys
    }
    float v[2][NV][VEC];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const Tin* xr = x + (r < npair ? row[r] : row[0]) * ld.x;
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        const int vi = k * rl.T + rl.t;
        if (vi < nkv[r]) {
          load_vec<Tin, VEC>(xr + (int64_t)vi * VEC, v[r][k]);
        } else {
#pragma unroll
          for (int i = 0; i < VEC; ++i) v[r][k][i] = kNegInf;
        }
      }
    }
    MD p[2];
    float ml[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      if (keys[r] < N) {
#pragma unroll
        for (int k = 0; k < NV; ++k) mask_keys<VEC>(v[r][k], (k * rl.T + rl.t) * VEC, keys[r]);
      }
      float m = kNegInf;
#pragma unroll
      for (int k = 0; k < NV; ++k)
#pragma unroll
        for (int i = 0; i < VEC; ++i) m = __builtin_fmaxf(m, v[r][k][i]);
      const float shift = (m == kNegInf) ? 0.0f : m;
      float dl = 0.0f;
#pragma unroll
      for (int k = 0; k < NV; ++k)
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          const float e = exp_out<Tout>(v[r][k][i] - shift);
          dl += e;
          if constexpr (!LOG) v[r][k][i] = e;   // plain softmax keeps e_i, log-softmax keeps x_i
        }
      ml[r] = m;
      p[r].m = m;
      p[r].d = dl;
      p[r] = wave_md(p[r]);
    }
    {
      // both rows through the slot stage of group_md, with one barrier
      stress_delay();
      if (rl.lane == 0) {
        sl[0][parity][rl.w] = p[0];
        sl[1][parity][rl.w] = p[1];
      }
      __syncthreads();
      stress_poison(sl[0], parity, rl.w, rl.lane);
      stress_poison(sl[1], parity, rl.w, rl.lane);
      stress_delay();
      const int j = rl.lane & (kMaxWavesPerGroup - 1);
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        MD t;
        if (j < rl.nw) {
          t = sl[r][parity][j];
        } else {
          t.m = kNegInf;
          t.d = 0.0f;
        }
        t = md_merge(t, dpp_md<kDppQuadXor1>(t));
        t = md_merge(t, dpp_md<kDppQuadXor2>(t));
        t = md_merge(t, dpp_md<kDppRowHalfMirror>(t));
        p[r] = md_merge(t, dpp_md<kDppRowMirror>(t));
      }
      parity ^= 1;
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      if (r >= npair) break;
      float c = 0.0f, lg = 0.0f;
      if constexpr (LOG) {
        lg = __builtin_logf(p[r].d);
      } else {
        c = (ml[r] == kNegInf) ? 0.0f : exp_out<Tout>(ml[r] - p[r].m) / p[r].d;
        if (p[r].m == kNegInf) c = __builtin_nanf("");
      }
      Tout* yr = y + row[r] * ld.y;
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        const int vi = k * rl.T + rl.t;
        float o[VEC];
#pragma unroll
        for (int i = 0; i < VEC; ++i) o[i] = LOG ? (v[r][k][i] - p[r].m) - lg : v[r][k][i] * c;
        if (vi < nvec) store_vec<Tout, VEC>(yr + (int64_t)vi * VEC, o);
      }
    }
  }
}

// ===========================================================================
// Softmax, a long row held packed in registers (BLOCK, large NV).
//
// For rows too long for 32 widened values per lane, a workgroup of up to 16
// wavefronts keeps the row in its storage format (bf16 stays two per dword)
// and recomputes exp(x - m) when it writes, instead of keeping e_i: two
// exponentials per element, still one HBM read and one write.  A 152064-wide
// bf16 row needs 19 vectors (76 VGPRs) per lane of a 1024-lane workgroup, one
// workgroup per CU.
// ===========================================================================
template <typename Tin, typename Tout, int NV, bool LOG, bool CAUSAL, bool SHIFT>
__global__ __launch_bounds__(1024) void softmax_packed_kernel(const Tin* x, Tout* y, int64_t M,
                                                              int N, int64_t cp, int64_t co, RowStrides ld) {
  constexpr int VEC = softmax_vec<Tin, Tout>();
  constexpr int kThreads = 1024;
  __shared__ MD slots[2][kMaxWavesPerGroup];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int nvec = N / VEC;
  int parity = 0;
  CausalRows cr(blockIdx.x, gridDim.x, CAUSAL ? cp : 0, co);
  for (int64_t row = blockIdx.x; row < M; row += gridDim.x, cr.next()) {
    const int keys = cr.keys(N);
    const Tin* xr = x + row * ld.x;   // uniform row bases
    Tout* yr = y + row * ld.y;
    // SHIFT: vector j covers the row's elements [j * VEC - lead, ...)
    const int lead = SHIFT ? frame_lead_within(xr, yr, VEC, N, NV * kThreads) : 0;
    const int nvec_row = SHIFT ? (lead + N + VEC - 1) / VEC : nvec;
    const int nvec_keys = (lead + keys + VEC - 1) / VEC;
    // the lane's vector offsets are recomputed at each use rather than kept
    // live across the row (an opaque copy of the lane index), which frees
    // the registers the packed row needs
    int t_ld = t;
    asm volatile("" : "+v"(t_ld));
    Packed<Tin, VEC> v[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int vi = k * kThreads + t_ld;
      const int e0 = vi * VEC - lead;
      if (vi < nvec_keys && (!SHIFT || (e0 >= 0 && e0 + VEC <= N))) v[k].template load<true>(xr + e0);
      else v[k].fill(kNegInf);
    }
    if constexpr (SHIFT) {
      // A cut row's only partial vectors are its first (lane lead / VEC,
      // k = 0) and its last; they are read element by element once every
      // whole vector's load is issued (read in between, their element loads
      // would wait for the loads issued before them).  The two lie in
      // different wavefronts unless the row's last vector falls in the first
      // 64 of a 1024-lane pass, so each wavefront still waits once.  (Held in
      // registers of their own until the end, as the narrower kernels do,
      // they would cost this kernel's packed rows occupancy.)
      auto partial = [&](int vi) {
        const int e0 = vi * VEC - lead;
        return vi < nvec_keys && !(e0 >= 0 && e0 + VEC <= N);
      };
      const int first = lead / VEC;     // vectors before it are empty
      if (t_ld == first && partial(first)) {
        float f[VEC];
        load_edge<Tin, VEC>(xr, first * VEC - lead, keys, f);
        v[0].set(f);
      }
      const int last = nvec_row - 1;
      if (last > first && t_ld == last % kThreads && partial(last)) {
        float f[VEC];
        load_edge<Tin, VEC>(xr, last * VEC - lead, keys, f);
        const int kl = last / kThreads;
#pragma unroll
        for (int k = 0; k < NV; ++k)
          if (k == kl) v[k].set(f);
      }
    }
    // a row the causal rule cuts: keys past the count inside the vector
    // holding the last kept key become -inf
    if (keys < N) {
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        const int first = keys - ((k * kThreads + t) * VEC - lead);
        if (first > 0 && first < VEC) v[k].mask_from(first);
      }
    }
    auto key = [&](int k, int i) { return v[k].get(i); };
    float ml = kNegInf;
#pragma unroll
    for (int k = 0; k < NV; ++k)
#pragma unroll
      for (int i = 0; i < VEC; ++i) ml = __builtin_fmaxf(ml, key(k, i));
#pragma unroll
    for (int k = 0; k < NV; ++k) v[k].touch();
    const float shift = (ml == kNegInf) ? 0.0f : ml;
    float dl = 0.0f;
#pragma unroll
    for (int k = 0; k < NV; ++k)
#pragma unroll
      for (int i = 0; i < VEC; ++i) dl += exp_shifted(key(k, i) - shift);
    MD p;
    p.m = ml;
    p.d = dl;
#pragma unroll
    for (int k = 0; k < NV; ++k) v[k].touch();
    p = wave_md(p);
    p = group_md(p, kThreads / kWave, w, lane, slots, parity);
    parity ^= 1;
    const float inv_d = (p.m == kNegInf) ? __builtin_nanf("") : 1.0f / p.d;
    const float ld = LOG ? __builtin_logf(p.d) : 0.0f;
    int t_st = t;
    asm volatile("" : "+v"(t_st));
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int vi = k * kThreads + t_st;
      const int e0 = vi * VEC - lead;
      float o[VEC];
#pragma unroll
      for (int i = 0; i < VEC; ++i)
        o[i] = LOG ? (key(k, i) - p.m) - ld : exp_out<Tout>(key(k, i) - p.m) * inv_d;
      if (vi < nvec_row) {
        if (!SHIFT || (e0 >= 0 && e0 + VEC <= N)) store_vec<Tout, VEC>(yr + e0, o);
        else store_edge<Tout, VEC>(yr, e0, N, o);
      }
    }
  }
}

// ===========================================================================
// Softmax, streaming (LOOP): any N, any alignment.  Pass 1 runs the online
// recurrence per lane, one vector (chunk) at a time: the chunk's own summary
// merged into the lane's running pair ([P1] section "四、S4"; [P2] section
// 七.3; [P4] section "Online softmax：一次遍历求出最大值和指数和").  The
// lanes' pairs are merged into the row's (m, d); pass 2 reads the row again
// and writes exp(x - m) / d.  HBM traffic: two reads and one write per
// element ([P2] section 七.3: "read twice, write once").
// ===========================================================================
template <typename Tin, typename Tout, int VEC, bool LOG, bool CAUSAL, bool SHIFT>
__global__ __launch_bounds__(1024) void softmax_loop_kernel(const Tin* x, Tout* y, int64_t M,
                                                            int N, int64_t cp, int64_t co, RowStrides ld) {
  __shared__ MD slots[2][kMaxWavesPerGroup];
  const RowLane rl = row_lane<false>();
  int parity = 0;
  CausalRows cr(blockIdx.x, gridDim.x, CAUSAL ? cp : 0, co);
  for (int64_t row = blockIdx.x; row < M; row += gridDim.x, cr.next()) {
    const int keys = cr.keys(N);
    const Tin* xr = x + row * ld.x;
    Tout* yr = y + row * ld.y;
    // SHIFT: vector j covers the row's elements [j * VEC - lead, ...); the
    // first and last vector are accessed element by element
    const int lead = SHIFT ? frame_lead(yr) : 0;
    const int nvec_row = (lead + N + VEC - 1) / VEC;
    const int nvec_keys = (lead + keys + VEC - 1) / VEC;
    auto whole = [&](int e0) { return !SHIFT || (e0 >= 0 && e0 + VEC <= N); };
    MD p;
    p.m = kNegInf;
    p.d = 0.0f;
    for (int vi = rl.t; vi < nvec_keys; vi += rl.T) {
      const int e0 = vi * VEC - lead;
      float v[VEC];
      if (whole(e0)) {
        load_vec<Tin, VEC>(xr + e0, v);
        mask_keys<VEC>(v, e0, keys);
      } else {
        load_edge<Tin, VEC>(xr, e0, keys, v);
      }
      p = md_merge(p, chunk_summary<VEC>(v));
    }
    p = wave_md(p);
    p = group_md(p, rl.nw, rl.w, rl.lane, slots, parity);
    parity ^= 1;
    const float inv_d = (p.m == kNegInf) ? __builtin_nanf("") : 1.0f / p.d;
    const float ld = LOG ? __builtin_logf(p.d) : 0.0f;
    for (int vi = rl.t; vi < nvec_row; vi += rl.T) {
      const int e0 = vi * VEC - lead;
      float v[VEC];
      if (vi >= nvec_keys) {
#pragma unroll
        for (int i = 0; i < VEC; ++i) v[i] = kNegInf;
      } else if (whole(e0)) {
        load_vec<Tin, VEC>(xr + e0, v);
        mask_keys<VEC>(v, e0, keys);
      } else {
        load_edge<Tin, VEC>(xr, e0, keys, v);
      }
#pragma unroll
      for (int i = 0; i < VEC; ++i) v[i] = LOG ? (v[i] - p.m) - ld : exp_out<Tout>(v[i] - p.m) * inv_d;
      if (whole(e0)) store_vec<Tout, VEC>(yr + e0, v);
      else store_edge<Tout, VEC>(yr, e0, N, v);
    }
  }
}

// ===========================================================================
// Softmax, split row (SPLIT): a row is cut into S chunks of CV vectors, one
// workgroup per (row, chunk).  [P4] section "练习" (the vocabulary-split
// exercise): each workgroup writes its chunk's (m, d) to a buffer, a second
// kernel merges them; the merge is associative and commutative ([P1] section
// "三、结合律"), so the chunks may be combined in any grouping.
//
// Pass A writes workspace[row * S + c] = (m_c, d_c).
// Pass B: every wavefront merges the row's S pairs itself (lane j folds pairs
// j, j + 64, ... in order, then the wave all-reduce), so every workgroup of
// a row obtains the same bits without another barrier; it then rescales its
// chunk.  The chunk's vectors are loaded before the pairs are merged so the
// HBM reads are in flight during the merge.
// ===========================================================================
// One (m, d) slot per chunk, 16 bytes: the two-kernel form uses m and d; the
// one-kernel form reads the 16 bytes as two tagged words (SplitWords).  After
// the M * S slots the workspace holds one 32-bit epoch per row, which only
// the one-kernel form uses.
struct SplitSlot {
  float m;
  float d;
  uint64_t tag;
};
static_assert(sizeof(SplitSlot) == 16, "slot layout");

// Pass A's summary of a chunk held in v (NV packed vectors per lane): the
// maximum, then the sum of exp(x - max), per lane; the wave all-reduce; the
// LDS stage.  Every lane of the workgroup ends with the same bits.  The
// one-kernel split calls the same code, so both forms agree bit for bit.
template <int NV, typename Tin, int VEC>
__device__ __forceinline__ MD split_chunk_stat(const Packed<Tin, VEC> (&v)[NV], const RowLane& rl,
                                               MD (*slots)[kMaxWavesPerGroup], int& parity) {
  float ml = kNegInf;
#pragma unroll
  for (int k = 0; k < NV; ++k)
#pragma unroll
    for (int i = 0; i < VEC; ++i) ml = __builtin_fmaxf(ml, v[k].get(i));
  const float shift = (ml == kNegInf) ? 0.0f : ml;
  float dl = 0.0f;
#pragma unroll
  for (int k = 0; k < NV; ++k)
#pragma unroll
    for (int i = 0; i < VEC; ++i) dl += exp_shifted(v[k].get(i) - shift);
  MD p;
  p.m = ml;
  p.d = dl;
  p = wave_md(p);
  p = group_md(p, rl.nw, rl.w, rl.lane, slots, parity);
  parity ^= 1;
  return p;
}

// Pass A's loads of chunk c of an aligned row: lane t's vectors
// c * 256 * NV + k * 256 + t, streaming; -inf past the row's nvec vectors.
template <int NV, typename Tin, int VEC>
__device__ __forceinline__ void split_chunk_load(const Tin* xr, int nvec, int c, int t,
                                                 Packed<Tin, VEC> (&v)[NV]) {
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int vi = c * 256 * NV + k * 256 + t;
    if (vi < nvec) v[k].template load<true>(xr + (int64_t)vi * VEC);
    else v[k].fill(kNegInf);
  }
}

template <typename Tin, typename Tout, int NV, bool SHIFT>
__global__ __launch_bounds__(256) void softmax_split_stats_kernel(const Tin* x, SplitSlot* ws,
                                                                  int64_t M, int N, int S, RowStrides ld) {
  constexpr int VEC = softmax_vec<Tin, Tout>();
  constexpr int kThreads = 256;
  constexpr int CV = kThreads * NV;
  __shared__ MD slots[2][kMaxWavesPerGroup];
  const RowLane rl = row_lane<false>();
  const int nvec = N / VEC;
  const int64_t items = M * (int64_t)S;
  int parity = 0;
  for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
    const int64_t row = item / S;
    const int c = (int)(item - row * S);
    const Tin* xr = x + row * ld.x;
    // SHIFT: vector j covers the row's elements [j * VEC - lead, ...)
    const int lead = SHIFT ? row_lead(xr, VEC) : 0;   // (its own frame: it writes no row)
    const int nvec_row = SHIFT ? (lead + N + VEC - 1) / VEC : nvec;
    Packed<Tin, VEC> v[NV];
    // streaming loads (measured faster than temporal ones that would leave
    // the chunk in the last-level cache for pass B, with inputs cold in HBM)
    if constexpr (!SHIFT) {
      split_chunk_load<NV>(xr, nvec, c, rl.t, v);
    } else {
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        const int vi = c * CV + k * kThreads + rl.t;
        const int e0 = vi * VEC - lead;
        if (vi < nvec_row && e0 >= 0 && e0 + VEC <= N) v[k].template load<true>(xr + e0);
        else v[k].fill(kNegInf);
      }
    }
    if constexpr (SHIFT) {
      // the row's first and last vector after every whole vector is in flight
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        const int vi = c * CV + k * kThreads + rl.t;
        const int e0 = vi * VEC - lead;
        if (vi < nvec_row && !(e0 >= 0 && e0 + VEC <= N)) {
          float f[VEC];
          load_edge<Tin, VEC>(xr, e0, N, f);
          v[k].set(f);
        }
      }
    }
    const MD p = split_chunk_stat<NV>(v, rl, slots, parity);
    if (threadIdx.x == 0) {
      ws[item].m = p.m;
      ws[item].d = p.d;
    }
  }
}

// Rows with many chunks: fold each row's S summaries into one pair, stored
// in the row's first slot, so that pass B reads one pair per row instead of
// S per wavefront (whose cost would grow with the square of the row length).
// One workgroup per row; thread t merges slots t, t + 256, ... in order,
// then the wave and cross-wave merges combine the threads.
__global__ __launch_bounds__(256) void softmax_split_merge_kernel(SplitSlot* ws, int64_t M, int S) {
  __shared__ MD slots[2][kMaxWavesPerGroup];
  const RowLane rl = row_lane<false>();
  int parity = 0;
  for (int64_t row = blockIdx.x; row < M; row += gridDim.x) {
    SplitSlot* r = ws + row * S;
    MD p;
    p.m = kNegInf;
    p.d = 0.0f;
    for (int s = threadIdx.x; s < S; s += 256) {
      MD b;
      b.m = r[s].m;
      b.d = r[s].d;
      p = md_merge(p, b);
    }
    p = wave_md(p);
    // every thread's slot reads have returned before this barrier
    p = group_md(p, rl.nw, rl.w, rl.lane, slots, parity);
    parity ^= 1;
    if (threadIdx.x == 0) {
      r[0].m = p.m;
      r[0].d = p.d;
    }
  }
}

// Rows with at most this many chunks skip the merge kernel: each lane of a
// pass-B wavefront then reads at most one summary.
constexpr int kSplitDirectMerge = kWave;

// Pass B's chunks need not be pass A's: a row's summaries start at slot
// row * SA, and SC of them are read (SA, or 1 after the merge kernel); the
// row is cut into SB chunks of 256 * NV vectors here.
template <typename Tin, typename Tout, int NV, bool LOG, bool SHIFT>
__global__ __launch_bounds__(256) void softmax_split_apply_kernel(const Tin* x, Tout* y,
                                                                  const SplitSlot* __restrict__ ws,
                                                                  int64_t M, int N, int SA, int SC,
                                                                  int SB, RowStrides ld) {
  constexpr int VEC = softmax_vec<Tin, Tout>();
  constexpr int kThreads = 256;
  constexpr int CV = kThreads * NV;
  const RowLane rl = row_lane<false>();
  const int nvec = N / VEC;
  const int64_t items = M * (int64_t)SB;
  for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
    const int64_t row = item / SB;
    const int c = (int)(item - row * SB);
    const Tin* xr = x + row * ld.x;
    Tout* yr = y + row * ld.y;
    const int lead = SHIFT ? frame_lead(yr) : 0;
    const int nvec_row = SHIFT ? (lead + N + VEC - 1) / VEC : nvec;
    Packed<Tin, VEC> v[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int vi = c * CV + k * kThreads + rl.t;
      const int e0 = vi * VEC - lead;
      if (vi < nvec_row && (!SHIFT || (e0 >= 0 && e0 + VEC <= N))) v[k].template load<true>(xr + e0);
      else v[k].fill(kNegInf);
    }
    if constexpr (SHIFT) {
      // the row's first and last vector after every whole vector is in flight
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        const int vi = c * CV + k * kThreads + rl.t;
        const int e0 = vi * VEC - lead;
        if (vi < nvec_row && !(e0 >= 0 && e0 + VEC <= N)) {
          float f[VEC];
          load_edge<Tin, VEC>(xr, e0, N, f);
          v[k].set(f);
        }
      }
    }
    MD p;
    p.m = kNegInf;
    p.d = 0.0f;
    for (int s = rl.lane; s < SC; s += kWave) {
      MD b;
      b.m = ws[row * SA + s].m;
      b.d = ws[row * SA + s].d;
      p = md_merge(p, b);
    }
    p = wave_md(p);
    const float inv_d = (p.m == kNegInf) ? __builtin_nanf("") : 1.0f / p.d;
    const float ld = LOG ? __builtin_logf(p.d) : 0.0f;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int vi = c * CV + k * kThreads + rl.t;
      const int e0 = vi * VEC - lead;
      float o[VEC];
#pragma unroll
      for (int i = 0; i < VEC; ++i)
        o[i] = LOG ? (v[k].get(i) - p.m) - ld : exp_out<Tout>(v[k].get(i) - p.m) * inv_d;
      // plain (write-back) stores: measured faster than non-temporal ones here
      if (vi < nvec_row) {
        if (!SHIFT || (e0 >= 0 && e0 + VEC <= N)) store_vec<Tout, VEC, false>(yr + e0, o);
        else store_edge<Tout, VEC>(yr, e0, N, o);
      }
    }
  }
}

// ===========================================================================
// Softmax, split row in ONE kernel (SPLIT_ONE_KERNEL).
//
// The same chunks and the same arithmetic as the two kernels above, but a
// workgroup keeps its chunk in registers while the row's other chunks are
// summarised, so x is read from HBM once ([P4] section "练习": the last block
// to finish instead of a second kernel; [P2] section 九 reads the same
// last-arrival idea in PyTorch's reductions).
//
//  * Launch: an ordinary launch, one workgroup per chunk, taken only when
//    the device holds the whole grid at once (its occupancy) and rows have
//    at most 64 chunks.
//  * Tag: the workspace holds, after the M * S slots, one 32-bit epoch per
//    row.  Every workgroup of the row reads it first; the call's tag for the
//    row is a fixed bijection of it (split_tag).  A workgroup that has all
//    of its row's summaries in hand advances the epoch by one with a
//    compare-and-swap from the value it read (the first such workgroup wins;
//    the others find it advanced and leave it): every workgroup of the row
//    has published, so has read the epoch, before any can do so.  The next
//    call on the workspace therefore tags the row differently, and the tag
//    is read on the device, not fixed at launch, so a replayed graph tags
//    each replay afresh.  (A workgroup kept from starting until its
//    row-mates gave up on it reads the advanced epoch, finds no partner
//    carrying its tag, summarises the row's other chunks itself and advances
//    the epoch once more: slow, still exact, still a fresh tag next call.)
//  * Publish: thread 0 writes the chunk's (m, d) as two 64-bit words with
//    relaxed agent-scope atomic stores: the low half of each word holds m's
//    (d's) bits, the high half the row's tag for this call.  No fence is
//    needed: each word is read whole, so a reader that finds the tag in both
//    words holds this call's m and d.  (Both words carry the same tag: were
//    they to carry two halves of a longer one, a reader could pair this
//    call's m with another call's d.)  Slots left by the previous call on
//    the row carry the previous tag; memory never written by this kernel
//    (a fresh workspace, or one the two-kernel form used) matches in both
//    words with probability 2^-64.
//  * Wait: lane s of wavefront 0 polls slot s with relaxed agent-scope
//    loads until both words carry the tag, for at most wait_ticks of the
//    100 MHz real-time clock (the library passes kSplitWaitTicks, 40 us).  A
//    chunk still missing then (its workgroup kept from running by other work
//    on the device, say) is summarised by this workgroup from x itself with
//    pass A's code, so the result has the same bits whichever way a summary
//    arrived, and the number of chunks so summarised is added to a
//    per-device counter (split_fallbacks, below), which the diagnostics
//    build reads: a wait that expires is recorded, not silent.
//  * The row's summaries go through LDS to every wavefront, lane s holding
//    chunk s's pair, which is exactly what pass B's lanes hold after
//    folding the workspace into the identity; the wave all-reduce and the
//    outputs, written from the registers, follow as in pass B.
// ===========================================================================
constexpr int kSplitFusedMaxChunks = kWave;         // one slot per lane of a wavefront

// A row's tag for the call that finds its epoch at e: an odd multiplier and
// an offset make it a bijection of the 32-bit epochs, and a zeroed
// workspace (epoch 0, slot words 0) does not match.
__device__ __forceinline__ uint32_t split_tag(uint32_t e) { return e * 0x9E3779B1u + 0x7F4A7C15u; }

// The one-kernel form's view of a workspace slot: two tagged 64-bit words.
struct SplitWords {
  uint64_t w0;   // tag << 32 | m's bits
  uint64_t w1;   // tag << 32 | d's bits
};
static_assert(sizeof(SplitWords) == sizeof(SplitSlot), "slot layout");

template <typename Tin, typename Tout, int NV, bool LOG>
__global__ __launch_bounds__(256) void softmax_split_fused_kernel(const Tin* x, Tout* y, SplitSlot* ws,
                                                                  int64_t M, int N, int S, uint64_t wait_ticks,
                                                                  unsigned int* fallbacks, RowStrides ld) {
  constexpr int VEC = softmax_vec<Tin, Tout>();
  constexpr int CV = 256 * NV;
  __shared__ MD slots[2][kMaxWavesPerGroup];
  __shared__ MD got[kSplitFusedMaxChunks];
  __shared__ uint64_t missing_mask;
  const RowLane rl = row_lane<false>();
  const int nvec = N / VEC;
  const int64_t item = blockIdx.x;            // the host launches one workgroup per chunk
  if (item >= M * (int64_t)S) return;         // (uniform)
  const int64_t row = item / S;
  const int c = (int)(item - row * S);
  const Tin* xr = x + row * ld.x;
  // the row's epoch (after the M * S slots) and this call's tag for the row
  uint32_t* epoch = reinterpret_cast<uint32_t*>(ws + M * (int64_t)S) + row;
  const uint32_t e0 = __hip_atomic_load(epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint32_t tag = split_tag(e0);
  int parity = 0;
  Packed<Tin, VEC> v[NV];
  split_chunk_load<NV>(xr, nvec, c, rl.t, v);
  const MD p = split_chunk_stat<NV>(v, rl, slots, parity);
  SplitWords* words = reinterpret_cast<SplitWords*>(ws + row * S);
  if (threadIdx.x == 0) {
    __hip_atomic_store(&words[c].w0, ((uint64_t)tag << 32) | __float_as_uint(p.m), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&words[c].w1, ((uint64_t)tag << 32) | __float_as_uint(p.d), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
  if (rl.w == 0) {
    // lane s waits for chunk s (its own chunk it already has)
    MD b;
    b.m = kNegInf;
    b.d = 0.0f;
    bool have = rl.lane >= S;
    if (rl.lane == c) {
      b = p;
      have = true;
    }
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while (!have) {
      const uint64_t a = __hip_atomic_load(&words[rl.lane].w0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint64_t e = __hip_atomic_load(&words[rl.lane].w1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if ((uint32_t)(a >> 32) == tag && (uint32_t)(e >> 32) == tag) {
        b.m = __uint_as_float((uint32_t)a);
        b.d = __uint_as_float((uint32_t)e);
        have = true;
        break;
      }
      if (__builtin_amdgcn_s_memrealtime() - t0 > wait_ticks) break;
      __builtin_amdgcn_s_sleep(2);
    }
    if (rl.lane < S) got[rl.lane] = b;
    const uint64_t miss = __ballot(!have);
    if (rl.lane == 0) missing_mask = miss;
  }
  __syncthreads();
  // chunks whose summaries did not arrive in time: counted, and summarised
  // here, from x
  uint64_t miss = missing_mask;                 // (uniform)
  if (miss != 0 && threadIdx.x == 0) atomicAdd(fallbacks, (unsigned int)__builtin_popcountll(miss));
  while (miss) {
    const int s = __builtin_ctzll(miss);
    miss &= miss - 1;
    Packed<Tin, VEC> u[NV];
    split_chunk_load<NV>(xr, nvec, s, rl.t, u);
    const MD r = split_chunk_stat<NV>(u, rl, slots, parity);
    if (threadIdx.x == 0) got[s] = r;
  }
  __syncthreads();
  // every summary of the row is in hand: the next call tags the row afresh
  if (threadIdx.x == 0) {
    uint32_t expected = e0;
    __hip_atomic_compare_exchange_strong(epoch, &expected, e0 + 1u, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
  }
  MD q;
  if (rl.lane < S) {
    q = got[rl.lane];
  } else {
    q.m = kNegInf;
    q.d = 0.0f;
  }
  q = wave_md(q);
  const float inv_d = (q.m == kNegInf) ? __builtin_nanf("") : 1.0f / q.d;
  const float lg = LOG ? __builtin_logf(q.d) : 0.0f;
  Tout* yr = y + row * ld.y;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int vi = c * CV + k * 256 + rl.t;
    float o[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i)
      o[i] = LOG ? (v[k].get(i) - q.m) - lg : exp_out<Tout>(v[k].get(i) - q.m) * inv_d;
    // plain (write-back) stores, as pass B
    if (vi < nvec) store_vec<Tout, VEC, false>(yr + (int64_t)vi * VEC, o);
  }
}

// ===========================================================================
// launchers
// ===========================================================================
namespace {

inline dim3 grid1(int64_t g) { return dim3((unsigned)g, 1, 1); }

int resident_groups(const void* kernel, int threads, size_t lds);

template <typename T, int KIND, bool WAVE, bool SHIFT>
hipError_t norm_regs(const rr_plan& p, const NormArgs& a, int64_t grid, hipStream_t s) {
  T* yy = static_cast<T*>(a.y);
  T* rr_ = static_cast<T*>(a.residual);
  const T* xx = static_cast<const T*>(a.x);
  const T* gg = static_cast<const T*>(a.gamma);
  const T* bb = static_cast<const T*>(a.beta);
  const dim3 b(p.block_threads);
  // LDS for a cut LayerNorm row's gamma and beta blocks (the host plans such
  // rows only while it fits kNormLdsParamMax)
  const size_t lds = norm_lds_params<KIND, WAVE, SHIFT>() ? norm_lds_param_bytes<T>(a.N) : 0;
  if (lds > kNormLdsParamMax) return hipErrorInvalidValue;
  if constexpr (norm_lds_params<KIND, WAVE, SHIFT>()) {
    // each workgroup stages the parameters once and walks rows grid-stride:
    // no more workgroups than the device holds at once
    const void* k = nullptr;
    switch (p.vecs_per_lane) {
      case 1: k = reinterpret_cast<const void*>(&norm_regs_kernel<T, 1, KIND, WAVE, SHIFT>); break;
      case 2: k = reinterpret_cast<const void*>(&norm_regs_kernel<T, 2, KIND, WAVE, SHIFT>); break;
      case 3: k = reinterpret_cast<const void*>(&norm_regs_kernel<T, 3, KIND, WAVE, SHIFT>); break;
      default: return hipErrorInvalidValue;
    }
    const int cap = resident_groups(k, p.block_threads, lds);
    if (cap > 0 && grid > cap) grid = cap;
  }
  // The host plans at most 16 values per lane for the norms (NV * VEC <=
  // 16), 24 for cut rows (3 bf16 vectors), so only those instantiations exist.
  switch (p.vecs_per_lane) {
    case 1: norm_regs_kernel<T, 1, KIND, WAVE, SHIFT><<<grid1(grid), b, lds, s>>>(yy, rr_, xx, gg, bb, a.M, a.N, a.eps, a.ld); break;
    case 2: norm_regs_kernel<T, 2, KIND, WAVE, SHIFT><<<grid1(grid), b, lds, s>>>(yy, rr_, xx, gg, bb, a.M, a.N, a.eps, a.ld); break;
    case 3:
      // (cut rows only: fewer wavefronts per row where that saves some)
      if constexpr (SHIFT && !WAVE) {
        norm_regs_kernel<T, 3, KIND, WAVE, SHIFT><<<grid1(grid), b, lds, s>>>(yy, rr_, xx, gg, bb, a.M, a.N, a.eps, a.ld);
        break;
      }
      return hipErrorInvalidValue;
    case 4:
      // (cut fp32 LayerNorm rows keep to 2 vectors per lane: 4 would spill)
      if constexpr (Elem<T>::kVec * 4 <= 16 && !(SHIFT && KIND == kNormLayer)) {
        norm_regs_kernel<T, 4, KIND, WAVE, SHIFT><<<grid1(grid), b, lds, s>>>(yy, rr_, xx, gg, bb, a.M, a.N, a.eps, a.ld);
        break;
      }
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, int KIND>
hipError_t norm_loop(const rr_plan& p, const NormArgs& a, int64_t grid, hipStream_t s) {
  T* yy = static_cast<T*>(a.y);
  T* rr_ = static_cast<T*>(a.residual);
  const T* xx = static_cast<const T*>(a.x);
  const T* gg = static_cast<const T*>(a.gamma);
  const T* bb = static_cast<const T*>(a.beta);
  const dim3 b(p.block_threads);
  if (p.vec_elems == 1)
    norm_loop_kernel<T, 1, KIND><<<grid1(grid), b, 0, s>>>(yy, rr_, xx, gg, bb, a.M, a.N, a.eps, a.ld);
  else
    norm_loop_kernel<T, Elem<T>::kVec, KIND><<<grid1(grid), b, 0, s>>>(yy, rr_, xx, gg, bb, a.M, a.N, a.eps, a.ld);
  return hipGetLastError();
}

template <typename T, int VEC, int KIND>
hipError_t norm_sub(const rr_plan& p, const NormArgs& a, int64_t grid, hipStream_t s) {
  T* yy = static_cast<T*>(a.y);
  T* rr_ = static_cast<T*>(a.residual);
  const T* xx = static_cast<const T*>(a.x);
  const T* gg = static_cast<const T*>(a.gamma);
  const T* bb = static_cast<const T*>(a.beta);
  const dim3 b(256);
  switch (p.waves_per_row) {  // for SUBWAVE: lanes per row
    case 1: norm_sub_kernel<T, VEC, 1, KIND><<<grid1(grid), b, 0, s>>>(yy, rr_, xx, gg, bb, a.M, a.N, a.eps, a.ld); break;
    case 2: norm_sub_kernel<T, VEC, 2, KIND><<<grid1(grid), b, 0, s>>>(yy, rr_, xx, gg, bb, a.M, a.N, a.eps, a.ld); break;
    case 4: norm_sub_kernel<T, VEC, 4, KIND><<<grid1(grid), b, 0, s>>>(yy, rr_, xx, gg, bb, a.M, a.N, a.eps, a.ld); break;
    case 8: norm_sub_kernel<T, VEC, 8, KIND><<<grid1(grid), b, 0, s>>>(yy, rr_, xx, gg, bb, a.M, a.N, a.eps, a.ld); break;
    case 16: norm_sub_kernel<T, VEC, 16, KIND><<<grid1(grid), b, 0, s>>>(yy, rr_, xx, gg, bb, a.M, a.N, a.eps, a.ld); break;
    case 32: norm_sub_kernel<T, VEC, 32, KIND><<<grid1(grid), b, 0, s>>>(yy, rr_, xx, gg, bb, a.M, a.N, a.eps, a.ld); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Rows held packed: bf16 NV 4 or 8 (32K / 64K elements), fp32 NV 8, 12 or 16
// (32K / 48K / 64K; the fused op, which holds x and the residual while
// loading, only NV 8).
template <typename T, int KIND>
hipError_t norm_packed(const rr_plan& p, const NormArgs& a, int64_t grid, hipStream_t s) {
  T* yy = static_cast<T*>(a.y);
  T* rr_ = static_cast<T*>(a.residual);
  const T* xx = static_cast<const T*>(a.x);
  const T* gg = static_cast<const T*>(a.gamma);
  const T* bb = static_cast<const T*>(a.beta);
  const dim3 b(1024);
  const dim3 g = grid1(grid);
  if constexpr (std::is_same_v<T, bf16_t>) {
    switch (p.vecs_per_lane) {
      case 4: norm_packed_kernel<T, 4, KIND><<<g, b, 0, s>>>(yy, rr_, xx, gg, bb, a.M, a.N, a.eps, a.ld); break;
      case 8: norm_packed_kernel<T, 8, KIND><<<g, b, 0, s>>>(yy, rr_, xx, gg, bb, a.M, a.N, a.eps, a.ld); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (p.vecs_per_lane) {
      case 8: norm_packed_kernel<T, 8, KIND><<<g, b, 0, s>>>(yy, rr_, xx, gg, bb, a.M, a.N, a.eps, a.ld); break;
      case 12:
      case 16:
        if constexpr (KIND != kNormFused) {
          if (p.vecs_per_lane == 12)
            norm_packed_kernel<T, 12, KIND><<<g, b, 0, s>>>(yy, rr_, xx, gg, bb, a.M, a.N, a.eps, a.ld);
          else
            norm_packed_kernel<T, 16, KIND><<<g, b, 0, s>>>(yy, rr_, xx, gg, bb, a.M, a.N, a.eps, a.ld);
          break;
        }
        return hipErrorInvalidValue;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

template <typename T, int KIND>
hipError_t norm_any(const rr_plan& p, const NormArgs& a, int64_t grid, hipStream_t s) {
  if (p.variant == RR_VARIANT_LOOP) return norm_loop<T, KIND>(p, a, grid, s);
  if (p.variant == RR_VARIANT_BLOCK && !p.row_shift && p.vecs_per_lane * p.vec_elems > 16)
    return norm_packed<T, KIND>(p, a, grid, s);
  if (p.variant == RR_VARIANT_SUBWAVE) {
    if (p.vec_elems == 1) return norm_sub<T, 1, KIND>(p, a, grid, s);
    return norm_sub<T, Elem<T>::kVec, KIND>(p, a, grid, s);
  }
  if (p.row_shift) {
    if (p.variant == RR_VARIANT_WAVE) return norm_regs<T, KIND, true, true>(p, a, grid, s);
    if (p.variant == RR_VARIANT_BLOCK) return norm_regs<T, KIND, false, true>(p, a, grid, s);
    return hipErrorInvalidValue;   // the planner cuts norm rows for these two only
  }
  if (p.variant == RR_VARIANT_WAVE) return norm_regs<T, KIND, true, false>(p, a, grid, s);
  return norm_regs<T, KIND, false, false>(p, a, grid, s);
}

template <typename T>
hipError_t norm_typed(const rr_plan& p, int kind, const NormArgs& a, int64_t grid, hipStream_t s) {
  switch (kind) {
    case kNormRms: return norm_any<T, kNormRms>(p, a, grid, s);
    case kNormFused: return norm_any<T, kNormFused>(p, a, grid, s);
    case kNormLayer: return norm_any<T, kNormLayer>(p, a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

// Vectors per lane in the split path's pass B: its chunks are 256 lanes x
// this many vectors, independent of pass A's.  Two measured fastest with cold
// inputs: the 256 x 152064 bf16 -> fp32 softmax (8-byte vectors) takes
// 64.6 us at two, 82.5 at one and 65.6 at four; a 16 x 2^20 fp32 one 43.5 us
// at two and 47.0 at one.
constexpr int kSplitApplyNV = 2;

// One softmax launch: typed pointers plus the row rule (causal period cp,
// offset co; cp == 0 keeps every key).
template <typename Tin, typename Tout>
struct SmCall {
  const Tin* x;
  Tout* y;
  int64_t M;
  int N;
  int64_t cp;
  int64_t co;
  RowStrides ld;
  uint64_t wait_ticks;   // the one-kernel split's bounded wait
};

template <typename Tin, typename Tout, bool WAVE, bool LOG, bool CAUSAL, bool SHIFT>
hipError_t softmax_regs(const rr_plan& p, const SmCall<Tin, Tout>& c, int64_t grid, hipStream_t s) {
  const dim3 b(p.block_threads);
  const dim3 g = grid1(grid);
  // At most 32 values per lane (NV * VEC <= 32).
  switch (p.vecs_per_lane) {
    case 1: softmax_regs_kernel<Tin, Tout, 1, WAVE, LOG, CAUSAL, SHIFT><<<g, b, 0, s>>>(c.x, c.y, c.M, c.N, c.cp, c.co, c.ld); break;
    case 2: softmax_regs_kernel<Tin, Tout, 2, WAVE, LOG, CAUSAL, SHIFT><<<g, b, 0, s>>>(c.x, c.y, c.M, c.N, c.cp, c.co, c.ld); break;
    case 4: softmax_regs_kernel<Tin, Tout, 4, WAVE, LOG, CAUSAL, SHIFT><<<g, b, 0, s>>>(c.x, c.y, c.M, c.N, c.cp, c.co, c.ld); break;
    case 8:
      if constexpr (softmax_vec<Tin, Tout>() * 8 <= 32) {
        softmax_regs_kernel<Tin, Tout, 8, WAVE, LOG, CAUSAL, SHIFT><<<g, b, 0, s>>>(c.x, c.y, c.M, c.N, c.cp, c.co, c.ld);
        break;
      }
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// The workgroup-per-row kernels: the register form, or (more than 32 values
// per lane) the packed form, either for vector-aligned rows or for rows cut
// at aligned addresses (SHIFT).
template <typename Tin, typename Tout, bool LOG, bool CAUSAL, bool SHIFT>
hipError_t softmax_rows_held(const rr_plan& p, const SmCall<Tin, Tout>& c, int64_t grid, hipStream_t s) {
  const dim3 b(p.block_threads);
  const dim3 g = grid1(grid);
  if (p.variant == RR_VARIANT_WAVE) return softmax_regs<Tin, Tout, true, LOG, CAUSAL, SHIFT>(p, c, grid, s);
  if (p.vecs_per_lane * p.vec_elems > 32) {
    // long rows held in their storage format (see softmax_packed_kernel); 8-byte
    // vectors (bf16 written as fp32) come twice as many per lane
    constexpr int X = softmax_vec<Tin, Tout>() * (int)sizeof(Tin) == 8 ? 2 : 1;
    switch (p.vecs_per_lane) {
      case 12 * X: softmax_packed_kernel<Tin, Tout, 12 * X, LOG, CAUSAL, SHIFT><<<g, b, 0, s>>>(c.x, c.y, c.M, c.N, c.cp, c.co, c.ld); break;
      case 16 * X: softmax_packed_kernel<Tin, Tout, 16 * X, LOG, CAUSAL, SHIFT><<<g, b, 0, s>>>(c.x, c.y, c.M, c.N, c.cp, c.co, c.ld); break;
      case 19 * X: softmax_packed_kernel<Tin, Tout, 19 * X, LOG, CAUSAL, SHIFT><<<g, b, 0, s>>>(c.x, c.y, c.M, c.N, c.cp, c.co, c.ld); break;
      case 20 * X: softmax_packed_kernel<Tin, Tout, 20 * X, LOG, CAUSAL, SHIFT><<<g, b, 0, s>>>(c.x, c.y, c.M, c.N, c.cp, c.co, c.ld); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  return softmax_regs<Tin, Tout, false, LOG, CAUSAL, SHIFT>(p, c, grid, s);
}

// Workgroups of `kernel` (`threads` threads, `lds` bytes of dynamic LDS)
// the current device holds at once (its occupancy times the compute units),
// or 0 if unknown.  Cached per device, kernel, size and LDS.
int resident_groups(const void* kernel, int threads, size_t lds) {
  static std::mutex mu;
  static std::map<std::tuple<int, const void*, int, size_t>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  auto key = std::make_tuple(dev, kernel, threads, lds);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int cus = 0, per_cu = 0;
  int cap = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, lds) == hipSuccess)
    cap = cus * per_cu;
  cache[key] = cap;
  return cap;
}

int resident_capacity(const void* kernel) { return resident_groups(kernel, 256, 0); }

// SPLIT (and SPLIT_ONE_KERNEL, which only forces the plan): the one-kernel
// form when the rows are aligned, a row has at most 64 chunks and the device
// holds the whole grid at once (also on a capturing stream: its tags come
// from the workspace's epochs, read on the device); else the two kernels.  SPLIT_TWO_KERNELS: always the two kernels.  Both forms use
// the same chunks and the same merge order, so they give the same bits.  The
// split forms keep every key (the planner never splits a causal call).
template <typename Tin, typename Tout, int NV, bool LOG, bool SHIFT>
hipError_t softmax_split(const rr_plan& p, const SmCall<Tin, Tout>& c, SplitSlot* w, int S,
                         int64_t grid, hipStream_t s) {
  const dim3 b(p.block_threads);
  if (c.cp > 0) return hipErrorInvalidValue;
  if constexpr (!SHIFT) {
    if (p.variant != RR_VARIANT_SPLIT_TWO_KERNELS && S <= kSplitFusedMaxChunks) {
      const void* k = reinterpret_cast<const void*>(&softmax_split_fused_kernel<Tin, Tout, NV, LOG>);
      const int64_t items = c.M * (int64_t)S;
      if (items <= resident_capacity(k)) {
        hipError_t e = hipSuccess;
        unsigned int* counter = split_fallback_counter(&e);
        if (!counter) return e;
        softmax_split_fused_kernel<Tin, Tout, NV, LOG><<<grid1(items), b, 0, s>>>(
            c.x, c.y, w, c.M, c.N, S, c.wait_ticks, counter, c.ld);
        return hipGetLastError();
      }
    }
  }
  softmax_split_stats_kernel<Tin, Tout, NV, SHIFT><<<grid1(grid), b, 0, s>>>(c.x, w, c.M, c.N, S, c.ld);
  int SC = S;
  if (S > kSplitDirectMerge) {
    int64_t gm = c.M < 65536 ? c.M : 65536;
#if RR_STRESS
    gm = gm < 37 ? gm : 37;   // the race-stress build's grid cap
#endif
    softmax_split_merge_kernel<<<grid1(gm), dim3(256), 0, s>>>(w, c.M, S);
    SC = 1;
  }
  // pass B in chunks of its own size
  constexpr int VEC = softmax_vec<Tin, Tout>();
  // vectors a row spans (SHIFT: with a lead of up to a 64-byte block of y)
  constexpr int kLeadMax = 64 / (int)sizeof(Tout) - 1;
  const int nvec = SHIFT ? (c.N + kLeadMax + VEC - 1) / VEC : c.N / VEC;
  const int SB = (nvec + 256 * kSplitApplyNV - 1) / (256 * kSplitApplyNV);
  const int64_t items_b = c.M * (int64_t)SB;
  const int64_t grid_b = grid < c.M * (int64_t)S ? (grid < items_b ? grid : items_b) : items_b;
  softmax_split_apply_kernel<Tin, Tout, kSplitApplyNV, LOG, SHIFT><<<grid1(grid_b), b, 0, s>>>(c.x, c.y, w, c.M, c.N, S,
                                                                                       SC, SB, c.ld);
  return hipGetLastError();
}

template <typename Tin, typename Tout, int VEC, bool LOG, bool CAUSAL>
hipError_t softmax_sub(const rr_plan& p, const SmCall<Tin, Tout>& c, int64_t grid, hipStream_t s) {
  const dim3 b(256);
  const dim3 g = grid1(grid);
  switch (p.waves_per_row) {  // for SUBWAVE: lanes per row
    case 1: softmax_sub_kernel<Tin, Tout, VEC, 1, LOG, CAUSAL><<<g, b, 0, s>>>(c.x, c.y, c.M, c.N, c.cp, c.co, c.ld); break;
    case 2: softmax_sub_kernel<Tin, Tout, VEC, 2, LOG, CAUSAL><<<g, b, 0, s>>>(c.x, c.y, c.M, c.N, c.cp, c.co, c.ld); break;
    case 4: softmax_sub_kernel<Tin, Tout, VEC, 4, LOG, CAUSAL><<<g, b, 0, s>>>(c.x, c.y, c.M, c.N, c.cp, c.co, c.ld); break;
    case 8: softmax_sub_kernel<Tin, Tout, VEC, 8, LOG, CAUSAL><<<g, b, 0, s>>>(c.x, c.y, c.M, c.N, c.cp, c.co, c.ld); break;
    case 16: softmax_sub_kernel<Tin, Tout, VEC, 16, LOG, CAUSAL><<<g, b, 0, s>>>(c.x, c.y, c.M, c.N, c.cp, c.co, c.ld); break;
    case 32: softmax_sub_kernel<Tin, Tout, VEC, 32, LOG, CAUSAL><<<g, b, 0, s>>>(c.x, c.y, c.M, c.N, c.cp, c.co, c.ld); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// The causal rule with two rows of a period per workgroup (the host chose
// it for aligned rows of the workgroup plan; pair_nv is the plan's vectors
// per lane, held for each of the two rows).
template <typename Tin, typename Tout, bool LOG>
hipError_t softmax_causal_pairs(const rr_plan& p, const SmCall<Tin, Tout>& c, int pair_nv, hipStream_t s) {
  const int64_t per = (c.cp + 1) / 2;
  const int64_t whole = c.M / c.cp;
  const int64_t items = whole * per + (c.M - whole * c.cp);
  int64_t grid = items;
  const int64_t cap = 0xffffffffLL / p.block_threads;
  if (grid > cap) grid = cap;
#if RR_STRESS
  grid = grid < 37 ? grid : 37;   // the race-stress build's grid cap
#endif
  const dim3 b(p.block_threads);
  // the plan's vectors per lane for each of the two rows (16 values at most)
  if (pair_nv != p.vecs_per_lane) return hipErrorInvalidValue;
  switch (pair_nv) {
    case 1: softmax_causal_pair_kernel<Tin, Tout, 1, LOG><<<grid1(grid), b, 0, s>>>(c.x, c.y, c.M, c.N, c.cp, c.co, c.ld); break;
    case 2: softmax_causal_pair_kernel<Tin, Tout, 2, LOG><<<grid1(grid), b, 0, s>>>(c.x, c.y, c.M, c.N, c.cp, c.co, c.ld); break;
    case 4:
      if constexpr (softmax_vec<Tin, Tout>() * 4 <= 16) {
        softmax_causal_pair_kernel<Tin, Tout, 4, LOG><<<grid1(grid), b, 0, s>>>(c.x, c.y, c.M, c.N, c.cp, c.co, c.ld);
        break;
      }
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename Tin, typename Tout, bool LOG, bool CAUSAL>
hipError_t softmax_typed(const rr_plan& p, const SmCall<Tin, Tout>& c, void* ws, int64_t grid,
                         hipStream_t s, int pair_nv = 0) {
  const dim3 b(p.block_threads);
  const dim3 g = grid1(grid);
  if constexpr (CAUSAL) {
    if (pair_nv > 0) return softmax_causal_pairs<Tin, Tout, LOG>(p, c, pair_nv, s);
  }
  if (p.variant == RR_VARIANT_SUBWAVE) {
    if (p.vec_elems == 1) return softmax_sub<Tin, Tout, 1, LOG, CAUSAL>(p, c, grid, s);
    return softmax_sub<Tin, Tout, softmax_vec<Tin, Tout>(), LOG, CAUSAL>(p, c, grid, s);
  }
  if (p.variant == RR_VARIANT_LOOP) {
    constexpr int V = softmax_vec<Tin, Tout>();
    if (p.vec_elems == 1)
      softmax_loop_kernel<Tin, Tout, 1, LOG, CAUSAL, false><<<g, b, 0, s>>>(c.x, c.y, c.M, c.N, c.cp, c.co, c.ld);
    else if (p.row_shift)
      softmax_loop_kernel<Tin, Tout, V, LOG, CAUSAL, true><<<g, b, 0, s>>>(c.x, c.y, c.M, c.N, c.cp, c.co, c.ld);
    else
      softmax_loop_kernel<Tin, Tout, V, LOG, CAUSAL, false><<<g, b, 0, s>>>(c.x, c.y, c.M, c.N, c.cp, c.co, c.ld);
    return hipGetLastError();
  }
  if (p.variant == RR_VARIANT_SPLIT || p.variant == RR_VARIANT_SPLIT_ONE_KERNEL ||
      p.variant == RR_VARIANT_SPLIT_TWO_KERNELS) {
    if constexpr (CAUSAL) return hipErrorInvalidValue;   // the planner never splits a causal call
    SplitSlot* w = static_cast<SplitSlot*>(ws);
    const int S = (int)p.chunks_per_row;
    if (p.row_shift) {
      if (p.variant == RR_VARIANT_SPLIT_ONE_KERNEL) return hipErrorInvalidValue;   // the planner never asks
      switch (p.vecs_per_lane) {
        case 4: return softmax_split<Tin, Tout, 4, LOG, true>(p, c, w, S, grid, s);
        case 8: return softmax_split<Tin, Tout, 8, LOG, true>(p, c, w, S, grid, s);
        default: return hipErrorInvalidValue;
      }
    }
    switch (p.vecs_per_lane) {
      case 2: return softmax_split<Tin, Tout, 2, LOG, false>(p, c, w, S, grid, s);
      case 4: return softmax_split<Tin, Tout, 4, LOG, false>(p, c, w, S, grid, s);
      case 8: return softmax_split<Tin, Tout, 8, LOG, false>(p, c, w, S, grid, s);
      default: return hipErrorInvalidValue;
    }
  }
  if (p.row_shift) return softmax_rows_held<Tin, Tout, LOG, CAUSAL, true>(p, c, grid, s);
  return softmax_rows_held<Tin, Tout, LOG, CAUSAL, false>(p, c, grid, s);
}

template <typename Tin, typename Tout>
hipError_t softmax_io(const rr_plan& p, const SoftmaxArgs& a, int64_t grid, hipStream_t s) {
  SmCall<Tin, Tout> c;
  c.x = static_cast<const Tin*>(a.x);
  c.y = static_cast<Tout*>(a.y);
  c.M = a.M;
  c.N = a.N;
  c.cp = a.causal_period;
  c.co = a.causal_offset;
  c.ld = a.ld;
  c.wait_ticks = a.split_wait_ticks;
  // the causal rule and log output are compile-time switches, so the plain
  // softmax kernels carry none of their code
  if (c.cp > 0) {
    if (a.log_output) return softmax_typed<Tin, Tout, true, true>(p, c, a.workspace, grid, s, a.pair_nv);
    return softmax_typed<Tin, Tout, false, true>(p, c, a.workspace, grid, s, a.pair_nv);
  }
  if (a.log_output) return softmax_typed<Tin, Tout, true, false>(p, c, a.workspace, grid, s);
  return softmax_typed<Tin, Tout, false, false>(p, c, a.workspace, grid, s);
}

}  // namespace

hipError_t launch_norm(const rr_plan& plan, rr_dtype dtype, int kind, const NormArgs& args,
                       int64_t grid, hipStream_t stream) {
  if (dtype == RR_F32) return norm_typed<float>(plan, kind, args, grid, stream);
  return norm_typed<bf16_t>(plan, kind, args, grid, stream);
}

hipError_t launch_softmax(const rr_plan& plan, rr_dtype in_dtype, rr_dtype out_dtype,
                          const SoftmaxArgs& args, int64_t grid, hipStream_t stream) {
  if (in_dtype == RR_F32) {
    if (out_dtype == RR_F32) return softmax_io<float, float>(plan, args, grid, stream);
    return softmax_io<float, bf16_t>(plan, args, grid, stream);
  }
  if (out_dtype == RR_F32) return softmax_io<bf16_t, float>(plan, args, grid, stream);
  return softmax_io<bf16_t, bf16_t>(plan, args, grid, stream);
}

}  // namespace rr

// ===========================================================================
// Scratch of the no-allocation softmax entry point.  Callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops)
// get the split row's (m, d) slots from this array instead of a workspace
// argument.  Its name is a host-side stand-in in host code: kernels are
// given the device address that hipGetSymbolAddress returns for the device
// that is current, looked up once per device and cached.  Every call on a
// device shares that device's copy, so calls that overlap in time on one
// device race; nothing in it needs to start at zero (the split's first
// kernel writes every slot its second kernel reads).
// ===========================================================================
static __device__ __align__(256) unsigned char scratch[rr::kNoAllocScratchBytes];

// ===========================================================================
// Hand-offs the one-kernel split gave up on (chunks a workgroup summarised
// again from x because their summaries did not arrive within its bounded
// wait): one counter per device, added to with a device-scope atomic; only
// the diagnostics build reads or clears it.
// ===========================================================================
static __device__ unsigned int split_fallbacks;

namespace rr {
namespace {

// The current device's address of a file-scope device variable, looked up
// once per device by `lookup` (a hipGetSymbolAddress call) and cached; null
// with *err set.
constexpr int kMaxDevices = 64;
template <typename Lookup>
void* device_symbol(std::atomic<void*> (&cache)[kMaxDevices], std::mutex& mu, hipError_t* err,
                    Lookup lookup) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *err = e;
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  void* p = cache[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(mu);
  p = cache[dev].load(std::memory_order_relaxed);
  if (p) return p;
  e = lookup(&p);
  if (e != hipSuccess || !p) {
    *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
    return nullptr;
  }
  cache[dev].store(p, std::memory_order_release);
  return p;
}

}  // namespace

void* noalloc_scratch(hipError_t* err) {
  static std::mutex mu;
  static std::atomic<void*> addr[kMaxDevices];
  return device_symbol(addr, mu, err, [](void** p) { return hipGetSymbolAddress(p, HIP_SYMBOL(scratch)); });
}

unsigned int* split_fallback_counter(hipError_t* err) {
  static std::mutex mu;
  static std::atomic<void*> addr[kMaxDevices];
  return static_cast<unsigned int*>(
      device_symbol(addr, mu, err, [](void** p) { return hipGetSymbolAddress(p, HIP_SYMBOL(split_fallbacks)); }));
}

}  // namespace rr
