// Device-side building blocks shared by the gfx950 kernels of this library:
// MFMA fragment types and wrappers, bf16 conversion, 16-lane DPP reductions.
//
// MFMA conventions (CDNA3/CDNA4, wave64), used by every contraction here:
//   * A 16 x 32 "slab" operand: lane l holds 8 values of row (l % 16) at
//     reduction positions 8 * (l / 16) + e, e = 0..7.  The B operand (32 x 16)
//     is the mirror image: lane l holds column (l % 16) at the same reduction
//     positions.  A and B pair their slots identically, so any placement of
//     the reduction index that both operands share gives the full sum.
//   * A 16 x 16 fp32 accumulator: lane l holds rows 4 * (l / 16) + i,
//     i = 0..3, of column (l % 16).
// bf16 slabs run as one v_mfma_f32_16x16x32_bf16; fp32 slabs as eight
// v_mfma_f32_16x16x4_f32 (slot e of every lane in step e), which keeps the
// exact fp32 products for fp32 inputs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16_t;   // compute type of the bf16-io contractions
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint16_t bf16_t;  // raw bf16 bits in memory

// ---------------------------------------------------------------- bf16 bits
// A 16-byte store marked nontemporal (streaming): for results that this
// kernel writes once and does not read back.  On gfx950 such stores were
// seen to complete much sooner under heavy write traffic, and every
// vmcnt wait of the storing wave covers its stores as well as its loads.
template <typename V>
__device__ __forceinline__ void store_nt16(void* p, const V& v) {
  static_assert(sizeof(V) == 16, "16-byte stores");
  typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4_nt, v), reinterpret_cast<u32x4_nt*>(p));
}

// ... of 8 bytes
__device__ __forceinline__ void store_nt8(void* p, uint2 v) {
  typedef uint32_t u32x2_nt __attribute__((ext_vector_type(2)));
  __builtin_nontemporal_store(u32x2_nt{v.x, v.y}, reinterpret_cast<u32x2_nt*>(p));
}

__device__ __forceinline__ float bf2f(bf16_t h) {
  return __builtin_bit_cast(float, (uint32_t)h << 16);
}
// Round-to-nearest-even float -> bf16 (the hardware v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16_t f2bf(float x) {
  return __builtin_bit_cast(bf16_t, (__bf16)x);
}
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// Two floats -> two round-to-nearest-even bf16 in one word (lo first): one
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// Four consecutive fp32 state values at element `off` of a stored-state array
// (streaming store): fp32, or rounded to nearest-even bf16 when `bf16`.
__device__ __forceinline__ void store_state4(void* base, size_t off, const float (&x)[4], bool bf16) {
  if (bf16) {
    store_nt8(reinterpret_cast<bf16_t*>(base) + off, uint2{pack_bf2(x[0], x[1]), pack_bf2(x[2], x[3])});
  } else {
    typedef float f4 __attribute__((ext_vector_type(4)));
    store_nt16(reinterpret_cast<float*>(base) + off, f4{x[0], x[1], x[2], x[3]});
  }
}
// Eight consecutive fp32 state values at element `off`: one 16-byte store in
// bf16 (a full 16-byte unit per lane, so that four lanes on one row fill a
// 64-byte segment), two in fp32.
__device__ __forceinline__ void store_state8(void* base, size_t off, const float (&x)[8], bool bf16) {
  if (bf16) {
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    store_nt16(reinterpret_cast<bf16_t*>(base) + off,
               u4{pack_bf2(x[0], x[1]), pack_bf2(x[2], x[3]), pack_bf2(x[4], x[5]), pack_bf2(x[6], x[7])});
  } else {
    typedef float f4 __attribute__((ext_vector_type(4)));
    store_nt16(reinterpret_cast<float*>(base) + off, f4{x[0], x[1], x[2], x[3]});
    store_nt16(reinterpret_cast<float*>(base) + off + 4, f4{x[4], x[5], x[6], x[7]});
  }
}

// ------------------------------------------------------- 16-lane reductions
// Sum over the 16 lanes of a DPP row; every lane of the row gets the total.
// quad_perm [1,0,3,2] and [2,3,0,1] sum each quad, row_half_mirror adds the
// neighbouring quad, row_mirror the other half row.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f<0xB1>(x);
  x += dpp_f<0x4E>(x);
  x += dpp_f<0x141>(x);
  x += dpp_f<0x140>(x);
  return x;
}

// ---------------------------------------------------------- MFMA fragments
// Fragment of one 16 x 32 slab for element type T (bf16 or fp32).
template <typename T> struct Frag;
template <> struct Frag<bf16_t> {
  bf16x8 v;
  __device__ __forceinline__ void zero() {
    for (int e = 0; e < 8; ++e) v[e] = (__bf16)0.0f;
  }
  __device__ __forceinline__ void set(int e, float x) { v[e] = (__bf16)x; }
  __device__ __forceinline__ float get(int e) const { return (float)v[e]; }
};
template <> struct Frag<f16_t> {
  f16x8 v;
  __device__ __forceinline__ void zero() {
    for (int e = 0; e < 8; ++e) v[e] = (_Float16)0.0f;
  }
  __device__ __forceinline__ void set(int e, float x) {
    v[e] = (_Float16)__builtin_amdgcn_fmed3f(x, -65504.0f, 65504.0f);
  }
  __device__ __forceinline__ float get(int e) const { return (float)v[e]; }
};
template <> struct Frag<float> {
  f32x8 v;
  __device__ __forceinline__ void zero() {
    for (int e = 0; e < 8; ++e) v[e] = 0.0f;
  }
  __device__ __forceinline__ void set(int e, float x) { v[e] = x; }
  __device__ __forceinline__ float get(int e) const { return v[e]; }
};

__device__ __forceinline__ f32x4 mma(const Frag<bf16_t>& a, const Frag<bf16_t>& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const Frag<f16_t>& a, const Frag<f16_t>& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const Frag<float>& a, const Frag<float>& b, f32x4 c) {
#pragma unroll
  for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], c, 0, 0, 0);
  return c;
}

// Load 8 consecutive elements (one slab row segment) from memory of type T
// into a fragment; the pointer must be 16-byte (bf16) / 32-byte (fp32)
// aligned.
__device__ __forceinline__ void load8(Frag<bf16_t>& f, const bf16_t* p) {
  f.v = *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ void load8(Frag<f16_t>& f, const f16_t* p) {
  f.v = *reinterpret_cast<const f16x8*>(p);
}
__device__ __forceinline__ void load8(Frag<float>& f, const float* p) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
  f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}

// Element conversions between the io / compute types and fp32.  Conversions
// to fp16 saturate at +-65504, so no finite input becomes inf.
__device__ __forceinline__ float to_f(bf16_t x) { return bf2f(x); }
__device__ __forceinline__ float to_f(f16_t x) { return (float)x; }
__device__ __forceinline__ float to_f(float x) { return x; }
template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ bf16_t from_f<bf16_t>(float x) { return f2bf(x); }
template <> __device__ __forceinline__ f16_t from_f<f16_t>(float x) {
  return (_Float16)__builtin_amdgcn_fmed3f(x, -65504.0f, 65504.0f);
}
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }

// Convert a fragment of raw inputs between element types (identity when
// equal).  bf16 -> fp16 is exact for |x| in fp16's normal range; inputs are
// not clamped here (q and k are expected far below 65504 in magnitude).
template <typename C, typename T>
__device__ __forceinline__ Frag<C> conv(const Frag<T>& a);
template <>
__device__ __forceinline__ Frag<float> conv<float, float>(const Frag<float>& a) { return a; }
template <>
__device__ __forceinline__ Frag<f16_t> conv<f16_t, bf16_t>(const Frag<bf16_t>& a) {
  Frag<f16_t> r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r.v[e] = (_Float16)(float)a.v[e];
  return r;
}

// Compute type of the MFMA operands for an io type: fp16 for bf16 io (one
// rounding of 2^-11 instead of 2^-8 on every intermediate operand; the
// bf16 inputs themselves convert exactly in fp16's normal range), fp32 for
// fp32 io.
template <typename T> struct ComputeOf;
template <> struct ComputeOf<bf16_t> { typedef f16_t type; };
template <> struct ComputeOf<float> { typedef float type; };

// Two floats -> two 16-bit values of type T packed in a word (lo first),
// one packed conversion (fp16 saturating as from_f).
template <typename T>
__device__ __forceinline__ uint32_t pack2(float lo, float hi);
template <>
__device__ __forceinline__ uint32_t pack2<bf16_t>(float lo, float hi) { return pack_bf2(lo, hi); }
template <>
__device__ __forceinline__ uint32_t pack2<f16_t>(float lo, float hi) {
  return __builtin_bit_cast(
      uint32_t, __builtin_convertvector(f32x2_t{__builtin_amdgcn_fmed3f(lo, -65504.0f, 65504.0f),
                                                __builtin_amdgcn_fmed3f(hi, -65504.0f, 65504.0f)},
                                        f16x2_t));
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

}  // namespace gdn
