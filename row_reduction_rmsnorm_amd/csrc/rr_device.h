// Device primitives for the row-reduce kernels on CDNA4 (gfx950, wave64).
//
//  * element codec: bf16 <-> fp32 (widening is a shift, narrowing is the
//    hardware round-to-nearest-even pack), 16-byte vector loads and stores;
//  * the wave64 all-reduce: six symmetric butterfly steps (two DPP quad
//    permutes, DPP half-row and row mirrors, then the gfx950 permlane16 and
//    permlane32 swaps) after which every lane holds the same statistic,
//    bit for bit;
//  * the online-softmax pair (m, d) and its merge, with -inf as the identity
//    of the maximum.
//
// Sources (web pages, cited by title and section):
//  [P1] "两个融合算子：RMSNorm 与 online softmax" (daleiyang.github.io)
//  [P2] "GPU Kernel 工程（04）：共享内存与 reduction" (arganzheng.life)
//  [P4] "Softmax 与归一化" (anrans.github.io ai-infra-handbooks)
//  [P5] "RMSNorm、Softmax 与在线归约" (notes.kuangjux.top)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace rr {

typedef uint16_t bf16_t;  // storage of one bfloat16 element

constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWave = 64;

// exp(t) for the arguments used here (t = x - m <= 0, or -inf): the hardware
// base-2 exponential of t * log2(e).  t is formed by one subtraction first,
// so the rounding of the product is relative to |x - m|, never to |x|.
__device__ __forceinline__ float exp_shifted(float t) {
  return __builtin_amdgcn_exp2f(t * kLog2e);
}

// The same where the result may be a subnormal that matters: v_exp_f32
// flushes results below 2^-126 to zero, so an argument whose result would
// be that small is raised by 64 first and the result multiplied by 2^-64
// (one rounding, into the subnormal range).  Results below 2^-190 stay 0,
// which is their correct rounding in fp32 as well.
__device__ __forceinline__ float exp_shifted_full(float t) {
  const float u = t * kLog2e;
  const bool tiny = u < -126.0f;
  const float r = __builtin_amdgcn_exp2f(tiny ? u + 64.0f : u);
  return tiny ? r * 0x1p-64f : r;
}

// The exponential that becomes a softmax output of type Tout.  A bf16
// output keeps its subnormals (down to 2^-133, which the full form reaches);
// an fp32 output below 2^-126 comes out as 0, an absolute error below
// 1.2e-38, and spares the extra instructions per element.
template <typename Tout>
__device__ __forceinline__ float exp_out(float t) {
  if constexpr (std::is_same_v<Tout, bf16_t>) return exp_shifted_full(t);
  else return exp_shifted(t);
}

// ---------------------------------------------------------------------------
// element codec
// ---------------------------------------------------------------------------
template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int kVec = 4;  // elements per 16-byte access
};
template <>
struct Elem<bf16_t> {
  static constexpr int kVec = 8;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 hw_bf16x2 __attribute__((ext_vector_type(2)));
typedef float hw_f32x2 __attribute__((ext_vector_type(2)));

// Two floats -> two bf16 in one dword (lo in bits 0..15), round to nearest
// even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  hw_f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, hw_bf16x2));
}

// Round a float to the nearest bf16 and widen it back (the value a bf16
// store would hold).
__device__ __forceinline__ float round_to_bf16(float v) {
  return bf16_lo(pack_bf16x2(v, 0.0f));
}

template <typename T>
__device__ __forceinline__ float round_to(float v) {
  if constexpr (std::is_same_v<T, bf16_t>) return round_to_bf16(v);
  else return v;
}

// Streaming accesses carry the non-temporal hint (the `nt` bit of the
// global load/store): row data is touched once, so it should not displace
// reusable lines (gamma, the split-row workspace) from the caches.  A load
// whose data is read again soon (the split-row first pass, whose chunk the
// second pass re-reads) uses NT = false.
template <bool NT, typename V>
__device__ __forceinline__ V ld(const V* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}
template <bool NT, typename V>
__device__ __forceinline__ void st(V* p, V v) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

// Load VEC consecutive elements at p into fp32.  VEC * sizeof(T) == 16 is
// one 16-byte load (p must be 16-byte aligned); VEC == 1 is a scalar load.
template <typename T, int VEC, bool NT = true>
__device__ __forceinline__ void load_vec(const T* __restrict__ p, float (&v)[VEC]) {
  if constexpr (std::is_same_v<T, float>) {
    if constexpr (VEC == 4) {
      const f32x4_t q = ld<NT>(reinterpret_cast<const f32x4_t*>(p));
      v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    } else {
      static_assert(VEC == 1, "fp32 loads are 1 or 4 wide");
      v[0] = ld<NT>(p);
    }
  } else {
    if constexpr (VEC == 8) {
      const u32x4_t q = ld<NT>(reinterpret_cast<const u32x4_t*>(p));
      v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x);
      v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
      v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z);
      v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
    } else if constexpr (VEC == 4) {
      const u32x2_t q = ld<NT>(reinterpret_cast<const u32x2_t*>(p));
      v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x);
      v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
    } else {
      static_assert(VEC == 1, "bf16 loads are 1, 4 or 8 wide");
      v[0] = __uint_as_float(static_cast<uint32_t>(ld<NT>(p)) << 16);
    }
  }
}

// One element at p, widened to fp32 (a plain cached load: used where every
// lane of a row reads the same element).
template <typename T>
__device__ __forceinline__ float load_one(const T* p) {
  if constexpr (std::is_same_v<T, float>) return *p;
  else return __uint_as_float(static_cast<uint32_t>(*p) << 16);
}

// A vector of VEC elements kept in registers in its storage format (bf16
// stays packed two per dword: half the registers of widened fp32).  Used for
// gamma, which a workgroup keeps across all the rows it visits, and for the
// split-row chunks, which are widened element by element when used.
template <typename T, int VEC>
struct Packed {
  // whole dwords; a single bf16 element still takes one
  static constexpr int kWords = (VEC * (int)sizeof(T) + 3) / 4;
  static_assert(kWords >= 1, "at least one register");
  uint32_t w[kWords];
  template <bool NT = false>
  __device__ __forceinline__ void load(const T* __restrict__ p) {
    if constexpr (kWords == 4) {
      const u32x4_t q = ld<NT>(reinterpret_cast<const u32x4_t*>(p));
      w[0] = q.x; w[1] = q.y; w[2] = q.z; w[3] = q.w;
    } else if constexpr (kWords == 2) {
      const u32x2_t q = ld<NT>(reinterpret_cast<const u32x2_t*>(p));
      w[0] = q.x; w[1] = q.y;
    } else if constexpr (std::is_same_v<T, float>) {
      w[0] = __float_as_uint(ld<NT>(p));
    } else {
      w[0] = static_cast<uint32_t>(ld<NT>(p));
    }
  }
  __device__ __forceinline__ void fill(float v) {
    const uint32_t b = std::is_same_v<T, float> ? __float_as_uint(v)
                                                : ((__float_as_uint(v) >> 16) * 0x10001u);
#pragma unroll
    for (int i = 0; i < kWords; ++i) w[i] = b;
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < kWords; ++i) w[i] = 0u;
  }
  // A cut row's partial vector: the aligned vector at `base` of which only
  // the elements [lo, hi) lie inside the row (0 <= lo < hi <= VEC).  Only
  // those elements are read (bf16: a whole word where both its halves lie
  // inside), straight into this vector's words, so a partial vector takes no
  // registers beyond a whole one's and no wait of its own.  finish_cut(),
  // called once every load of the row is issued, moves a lone bf16 element
  // of an odd index into its word's high half and sets the elements outside
  // [lo, hi) to `fill`.
  __device__ __forceinline__ void load_cut(const T* base, int lo, int hi) {
    if constexpr (std::is_same_v<T, float>) {
#pragma unroll
      for (int i = 0; i < kWords; ++i) w[i] = (i >= lo && i < hi) ? __float_as_uint(base[i]) : 0u;
    } else {
      static_assert(VEC % 2 == 0, "bf16 partial vectors are whole words");
#pragma unroll
      for (int j = 0; j < kWords; ++j) {
        const bool a = 2 * j >= lo && 2 * j < hi, b = 2 * j + 1 >= lo && 2 * j + 1 < hi;
        if (a && b) w[j] = *reinterpret_cast<const uint32_t*>(base + 2 * j);
        else if (a) w[j] = static_cast<uint32_t>(base[2 * j]);
        else if (b) w[j] = static_cast<uint32_t>(base[2 * j + 1]);
        else w[j] = 0u;
      }
    }
  }
  __device__ __forceinline__ void finish_cut(int lo, int hi, float fill) {
    touch();
    const uint32_t fb = std::is_same_v<T, float> ? __float_as_uint(fill) : (__float_as_uint(fill) >> 16);
    if constexpr (std::is_same_v<T, float>) {
#pragma unroll
      for (int i = 0; i < kWords; ++i) w[i] = (i >= lo && i < hi) ? w[i] : fb;
    } else {
#pragma unroll
      for (int j = 0; j < kWords; ++j) {
        const bool a = 2 * j >= lo && 2 * j < hi, b = 2 * j + 1 >= lo && 2 * j + 1 < hi;
        const uint32_t lo16 = a ? (w[j] & 0xffffu) : fb;
        const uint32_t hi16 = b ? (a ? (w[j] >> 16) : (w[j] & 0xffffu)) : fb;
        w[j] = lo16 | (hi16 << 16);
      }
    }
  }
  // Hold VEC values that are exactly representable in T (packing rounds to
  // nearest even, which leaves such values unchanged).
  __device__ __forceinline__ void set(const float (&f)[VEC]) {
    if constexpr (std::is_same_v<T, float>) {
#pragma unroll
      for (int i = 0; i < VEC; ++i) w[i] = __float_as_uint(f[i]);
    } else if constexpr (VEC == 1) {
      w[0] = __float_as_uint(f[0]) >> 16;
    } else {
#pragma unroll
      for (int i = 0; i < kWords; ++i) w[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
    }
  }
  // Elements `first` and above become -inf (first in [0, VEC)).
  __device__ __forceinline__ void mask_from(int first) {
    if constexpr (std::is_same_v<T, float>) {
#pragma unroll
      for (int i = 0; i < kWords; ++i)
        if (i >= first) w[i] = 0xff800000u;
    } else if constexpr (VEC == 1) {
      if (first <= 0) w[0] = 0xff80u;
    } else {
#pragma unroll
      for (int i = 0; i < kWords; ++i) {
        if (2 * i >= first) w[i] = (w[i] & 0xffff0000u) | 0xff80u;
        if (2 * i + 1 >= first) w[i] = (w[i] & 0x0000ffffu) | 0xff800000u;
      }
    }
  }
  // Tell the compiler the words may have changed (an empty asm that "reads
  // and writes" them), so values widened earlier are not kept live across
  // this point: the next get() widens again from the packed words.
  __device__ __forceinline__ void touch() {
#pragma unroll
    for (int i = 0; i < kWords; ++i) asm volatile("" : "+v"(w[i]));
  }
  __device__ __forceinline__ float get(int i) const {
    if constexpr (std::is_same_v<T, float>) return __uint_as_float(w[i]);
    else if constexpr (VEC == 1) return __uint_as_float(w[0] << 16);
    else return (i & 1) ? bf16_hi(w[i >> 1]) : bf16_lo(w[i >> 1]);
  }
};

// Store VEC fp32 values at p as T (bf16: round to nearest even), with the
// non-temporal hint unless NT is false.  Widths: fp32 4 or 8 (one or two
// 16-byte stores), bf16 8 (16 bytes) or 4 (8 bytes), or 1 (scalar).
template <typename T, int VEC, bool NT = true>
__device__ __forceinline__ void store_vec(T* __restrict__ p, const float (&v)[VEC]) {
  if constexpr (std::is_same_v<T, float>) {
    if constexpr (VEC % 4 == 0) {
#pragma unroll
      for (int i = 0; i < VEC / 4; ++i)
        st<NT>(reinterpret_cast<f32x4_t*>(p) + i, f32x4_t{v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]});
    } else {
      static_assert(VEC == 1, "fp32 stores are 1, 4 or 8 wide");
      st<NT>(p, v[0]);
    }
  } else {
    if constexpr (VEC == 8) {
      st<NT>(reinterpret_cast<u32x4_t*>(p), u32x4_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                                 pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])});
    } else if constexpr (VEC == 4) {
      st<NT>(reinterpret_cast<u32x2_t*>(p), u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])});
    } else {
      static_assert(VEC == 1, "bf16 stores are 1, 4 or 8 wide");
      st<NT>(p, static_cast<bf16_t>(pack_bf16x2(v[0], 0.0f) & 0xffffu));
    }
  }
}

// Lane 0's value, as a wave-uniform (scalar-register) value.  Only for values
// that every active lane holds with the same bits.
__device__ __forceinline__ float uniform_f32(float v) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}

// ---------------------------------------------------------------------------
// wave64 all-reduce
//
// [P1] section "一、down 还是 xor": an xor butterfly is an involution, so each
// step is a two-way exchange and after log2(width) steps every lane holds the
// total, which is what a kernel needs when every lane rescales its own
// elements.  On a 64-lane CDNA wave the six exchanges are
//   1. DPP quad_perm [1,0,3,2]   (lane ^ 1)
//   2. DPP quad_perm [2,3,0,1]   (lane ^ 2)
//   3. DPP row_half_mirror       (i <-> 7 - i inside 8 lanes: pairs the two quads)
//   4. DPP row_mirror            (i <-> 15 - i inside 16 lanes: pairs the two halves)
//   5. v_permlane16_swap          (16-lane rows 0<->1 and 2<->3)
//   6. v_permlane32_swap          (lanes 0..31 <-> 32..63)
// Steps 3 and 4 are mirrors rather than xors, which is still a pairing of
// lanes whose partial totals cover disjoint halves once steps 1-2 (resp. 3)
// are done.  Every pairing is symmetric and the combine operator is applied
// as op(own, partner) on one side and op(partner, own) on the other, so a
// commutative op gives both partners the same bits; the swap steps hand every
// lane the (even-row, odd-row) pair in the same order.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

constexpr int kDppQuadXor1 = 0xB1;     // quad_perm:[1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm:[2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

// Exchange v with its step-5 partner: returns {value held by the even row,
// value held by the odd row} of the lane's 32-lane pair of rows.
__device__ __forceinline__ void swap16(float v, float& even, float& odd) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  even = __uint_as_float(r[0]);
  odd = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap32(float v, float& lo, float& hi) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}

__device__ __forceinline__ float wave_sum(float v) {
  v = v + dpp_f32<kDppQuadXor1>(v);
  v = v + dpp_f32<kDppQuadXor2>(v);
  v = v + dpp_f32<kDppRowHalfMirror>(v);
  v = v + dpp_f32<kDppRowMirror>(v);
  float a, b;
  swap16(v, a, b);
  v = a + b;
  swap32(v, a, b);
  return a + b;
}

__device__ __forceinline__ float wave_max(float v) {
  v = __builtin_fmaxf(v, dpp_f32<kDppQuadXor1>(v));
  v = __builtin_fmaxf(v, dpp_f32<kDppQuadXor2>(v));
  v = __builtin_fmaxf(v, dpp_f32<kDppRowHalfMirror>(v));
  v = __builtin_fmaxf(v, dpp_f32<kDppRowMirror>(v));
  float a, b;
  swap16(v, a, b);
  v = __builtin_fmaxf(a, b);
  swap32(v, a, b);
  return __builtin_fmaxf(a, b);
}

// The same butterfly restricted to groups of L consecutive lanes (L a power of
// two, at most 32): the first log2(L) steps of the six above.  Every lane of a
// group ends with the group's total, bit for bit; groups do not mix.
template <int L>
__device__ __forceinline__ float group_lanes_sum(float v) {
  static_assert(L >= 1 && L <= 32 && (L & (L - 1)) == 0, "L must be a power of two <= 32");
  if constexpr (L >= 2) v = v + dpp_f32<kDppQuadXor1>(v);
  if constexpr (L >= 4) v = v + dpp_f32<kDppQuadXor2>(v);
  if constexpr (L >= 8) v = v + dpp_f32<kDppRowHalfMirror>(v);
  if constexpr (L >= 16) v = v + dpp_f32<kDppRowMirror>(v);
  if constexpr (L >= 32) {
    float a, b;
    swap16(v, a, b);
    v = a + b;
  }
  return v;
}

// ---------------------------------------------------------------------------
// the online-softmax pair
//
// (m, d): m the maximum of a set of entries, d = sum exp(x - m) over it.
// Merge, [P1] section "三、结合律：为什么能做树形归约" and [P5] section
// "从逐元素更新到合并两个 tile":
//   (m1, d1) (+) (m2, d2) = (m, d1*exp(m1 - m) + d2*exp(m2 - m)),  m = max(m1, m2)
// with identity (-inf, 0), the summary of an empty or fully masked set.  The
// -inf guard ([P2] section 十, the online kernel's update and merge; [P4]
// section "实现", md_combine) stops (-inf) - (-inf) = NaN: a side whose m is
// -inf contributes 0.  Each side's product is rounded on its own and then the
// two are added, so merge(a, b) and merge(b, a) give the same bits (a fused
// multiply-add would round the two sides differently).
// ---------------------------------------------------------------------------
struct MD {
  float m;
  float d;
};

__device__ __forceinline__ MD md_merge(MD a, MD b) {
#pragma clang fp contract(off)
  const float m = __builtin_fmaxf(a.m, b.m);
  const float pa = (a.m == kNegInf) ? 0.0f : a.d * exp_shifted(a.m - m);
  const float pb = (b.m == kNegInf) ? 0.0f : b.d * exp_shifted(b.m - m);
  MD r;
  r.m = m;
  r.d = pa + pb;
  return r;
}

template <int CTRL>
__device__ __forceinline__ MD dpp_md(MD v) {
  MD r;
  r.m = dpp_f32<CTRL>(v.m);
  r.d = dpp_f32<CTRL>(v.d);
  return r;
}

__device__ __forceinline__ MD wave_md(MD v) {
  v = md_merge(v, dpp_md<kDppQuadXor1>(v));
  v = md_merge(v, dpp_md<kDppQuadXor2>(v));
  v = md_merge(v, dpp_md<kDppRowHalfMirror>(v));
  v = md_merge(v, dpp_md<kDppRowMirror>(v));
  MD e, o;
  swap16(v.m, e.m, o.m);
  swap16(v.d, e.d, o.d);
  v = md_merge(e, o);
  swap32(v.m, e.m, o.m);
  swap32(v.d, e.d, o.d);
  return md_merge(e, o);
}

// The pair all-reduce restricted to groups of L consecutive lanes.
template <int L>
__device__ __forceinline__ MD group_lanes_md(MD v) {
  static_assert(L >= 1 && L <= 32 && (L & (L - 1)) == 0, "L must be a power of two <= 32");
  if constexpr (L >= 2) v = md_merge(v, dpp_md<kDppQuadXor1>(v));
  if constexpr (L >= 4) v = md_merge(v, dpp_md<kDppQuadXor2>(v));
  if constexpr (L >= 8) v = md_merge(v, dpp_md<kDppRowHalfMirror>(v));
  if constexpr (L >= 16) v = md_merge(v, dpp_md<kDppRowMirror>(v));
  if constexpr (L >= 32) {
    MD e, o;
    swap16(v.m, e.m, o.m);
    swap16(v.d, e.d, o.d);
    v = md_merge(e, o);
  }
  return v;
}

// Summary pair of VEC register values (the chunk summary of [P1] section
// "四、S4：float4，顺便演示了分块合并"): maximum first, then the sum of
// exp(x - max).  A chunk whose entries are all -inf is the identity.
template <int VEC>
__device__ __forceinline__ MD chunk_summary(const float (&v)[VEC]) {
  float m = v[0];
#pragma unroll
  for (int i = 1; i < VEC; ++i) m = __builtin_fmaxf(m, v[i]);
  MD r;
  r.m = m;
  if (m == kNegInf) {
    r.d = 0.0f;
    return r;
  }
  float d = 0.0f;
#pragma unroll
  for (int i = 0; i < VEC; ++i) d += exp_shifted(v[i] - m);
  r.d = d;
  return r;
}

}  // namespace rr
