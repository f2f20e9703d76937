// Shared device helpers for the gfx950 attention kernels: MFMA wrappers,
// LDS access (including the gfx950 transposing LDS read), element conversion
// and cross-lane exchange. Everything here is specific to CDNA4 / wave64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) char lds_t;

// 16-bit element types. Values travel as raw bits (short vectors) and are
// reinterpreted only at the MFMA and conversion instructions.
struct BF16 {};
struct F16 {};

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D(32x32) += A(32x16) * B(16x32), fp32 accumulate. Lane l supplies row (A) /
// column (B) l % 32 and k = 8 * (l / 32) + 0..7; the result gives lane l
// column l % 32 and rows 8 * (i / 4) + 4 * (l / 32) + i % 4, i = 0..15.
template <class T>
__device__ __forceinline__ f32x16 mfma32(s16x8 a, s16x8 b, f32x16 c);

template <>
__device__ __forceinline__ f32x16 mfma32<BF16>(s16x8 a, s16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x16 mfma32<F16>(s16x8 a, s16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Two floats -> two 16-bit values (round to nearest even), low half first.
template <class T>
__device__ __forceinline__ unsigned int pack2(float lo, float hi);

template <>
__device__ __forceinline__ unsigned int pack2<BF16>(float lo, float hi) {
  bf16x2 p;
  p[0] = (__bf16)lo;
  p[1] = (__bf16)hi;
  return __builtin_bit_cast(unsigned int, p);
}
template <>
__device__ __forceinline__ unsigned int pack2<F16>(float lo, float hi) {
  f16x2 p;
  p[0] = (_Float16)lo;
  p[1] = (_Float16)hi;
  return __builtin_bit_cast(unsigned int, p);
}

template <class T>
__device__ __forceinline__ float to_f32(unsigned short bits);
template <>
__device__ __forceinline__ float to_f32<BF16>(unsigned short bits) {
  return __builtin_bit_cast(float, (unsigned int)bits << 16);
}
template <>
__device__ __forceinline__ float to_f32<F16>(unsigned short bits) {
  return (float)__builtin_bit_cast(_Float16, bits);
}

// Eight packed 16-bit values as an MFMA operand, built from four dwords.
__device__ __forceinline__ s16x8 as_operand(unsigned int a, unsigned int b, unsigned int c,
                                            unsigned int d) {
  u32x4 v = {a, b, c, d};
  return __builtin_bit_cast(s16x8, v);
}

__device__ __forceinline__ s16x8 lds_read16(const lds_t* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) s16x8*>(p);
}
__device__ __forceinline__ void lds_write16(lds_t* p, s16x8 v) {
  *reinterpret_cast<__attribute__((address_space(3))) s16x8*>(p) = v;
}
__device__ __forceinline__ void lds_write8(lds_t* p, u32x2 v) {
  *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(p) = v;
}

// gfx950 transposing LDS read of 4 x 16-bit values. Within each group of 16
// lanes, lane 4e + c supplies the address of 4 consecutive elements of some
// row r_e; afterwards lane i of the group holds column (4 * (i / 4) + i % 4)
// of that 4 x 16 block, i.e. element i % 4 of lane 4e + i / 4, for e = 0..3.
// Used with lane (g, e, c) pointing at row base + e, column col0 + 4c, lane i
// receives column col0 + i of rows base .. base + 3.
__device__ __forceinline__ s16x4 lds_read_tr(const lds_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
}

__device__ __forceinline__ s16x8 concat(s16x4 lo, s16x4 hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Value of the lane 32 positions away (lanes l and l ^ 32 exchange).
__device__ __forceinline__ float swap_halves(float x) {
  int xi = __builtin_bit_cast(int, x);
  auto r = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  // lanes 0..31 get (own, partner); lanes 32..63 get (partner, own)
  int lane = __lane_id();
  return __builtin_bit_cast(float, lane < 32 ? r[1] : r[0]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ s16x8 gload16(const unsigned short* p) {
  return *reinterpret_cast<const s16x8*>(p);
}

// Buffer resources: a base address and a size in bytes. Loads past the size
// return zeros and stores / atomics past it are dropped by the hardware, so
// ragged tails need no branches (and the compiler can track every load).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;  // gfx9 raw buffer: 32-bit data format, no swizzle

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, unsigned int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}
__device__ __forceinline__ s16x8 bload16(rsrc_t r, unsigned int off) {
  return __builtin_bit_cast(s16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ float bload_f32(rsrc_t r, unsigned int off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ void bstore8(rsrc_t r, unsigned int off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) int, v), r,
                                        off, 0, 0);
}
__device__ __forceinline__ void bstore_f32(rsrc_t r, unsigned int off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, v), r, off, 0, 0);
}
__device__ __forceinline__ void batomic_add(rsrc_t r, unsigned int off, float v) {
  __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(v, r, off, 0, 0);
}

}  // namespace fa
