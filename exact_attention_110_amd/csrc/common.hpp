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
__device__ __forceinline__ unsigned int bload_u32(rsrc_t r, unsigned int off) {
  return (unsigned int)__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ u32x2 bload_u32x2(rsrc_t r, unsigned int off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
// Element-mask bit tiles of partial blocks: tile t holds 128 rows of four
// 32-bit words; bit k of word c of row r is key 32 c + k of the block for
// query r of the block. Byte offset of word c of row r of tile t:
__device__ __forceinline__ unsigned int bits_off(int t, int r, int c) {
  return (unsigned)t * 2048u + (unsigned)(r * 16 + c * 4);
}
__device__ __forceinline__ void batomic_add(rsrc_t r, unsigned int off, float v) {
  __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(v, r, off, 0, 0);
}

// ---------------------------------------------------------------------------
// Dropout keep decisions: Philox4x32-10 (Salmon, Moraes, Dror and Shaw,
// "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11), a counter-based
// generator, so that the forward and backward passes draw the same bits for an
// element without storing a mask. Element (query i, key j) of query head
// bh = b * H + h uses counter (i >> 2, j >> 2, bh, 0) under the call's 64-bit
// key, word i & 3 and byte j & 3 of the output: one call decides a 4 x 4 block,
// so four consecutive keys of a row, or four consecutive queries of a column,
// come from one call.
struct Philox4 {
  unsigned int v[4];
};
__device__ __forceinline__ Philox4 philox4x32_10(unsigned int c0, unsigned int c1, unsigned int c2,
                                                 unsigned int c3, unsigned int k0, unsigned int k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const unsigned int lo0 = 0xD2511F53u * c0, hi0 = __umulhi(0xD2511F53u, c0);
    const unsigned int lo1 = 0xCD9E8D57u * c2, hi1 = __umulhi(0xCD9E8D57u, c2);
    c0 = hi1 ^ c1 ^ k0;
    c1 = lo1;
    c2 = hi0 ^ c3 ^ k1;
    c3 = lo0;
    k0 += 0x9E3779B9u;  // key schedule between rounds
    k1 += 0xBB67AE85u;
  }
  return {{c0, c1, c2, c3}};
}
// The generator shared across a quad. In every kernel layout the four lanes
// of a quad (lanes 4a .. 4a + 3) cover four consecutive query rows (or keys)
// of one generator block and need the same four Philox calls; each lane
// computes one of them and a 4 x 4 transpose across the quad hands every lane
// its words, a quarter of the generator work.

// x[c] of lane r becomes x[r] of lane c (r = lane & 3): two stages that swap
// across lane distance 1 and 2 with quad-permute DPP moves.
template <int CTRL>
__device__ __forceinline__ unsigned int dpp_quad(unsigned int v) {
  return (unsigned int)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ void quad_transpose(unsigned int (&x)[4], int r) {
  const bool h1 = (r & 1) != 0, h2 = (r & 2) != 0;
#pragma unroll
  for (int c0 = 0; c0 < 4; c0 += 2) {  // lanes r, r ^ 1 swap elements c0 + 1 and c0
    const unsigned int t = dpp_quad<0xB1>(h1 ? x[c0] : x[c0 + 1]);
    x[c0] = h1 ? t : x[c0];
    x[c0 + 1] = h1 ? x[c0 + 1] : t;
  }
#pragma unroll
  for (int c0 = 0; c0 < 2; ++c0) {     // lanes r, r ^ 2 swap elements c0 + 2 and c0
    const unsigned int t = dpp_quad<0x4E>(h2 ? x[c0] : x[c0 + 2]);
    x[c0] = h2 ? t : x[c0];
    x[c0 + 2] = h2 ? x[c0 + 2] : t;
  }
}

// Lane holds query row qi (qi & 3 == lane & 3) and needs, for the four key
// groups kg0 + gs g (g = 0..3, kg0 and gs multiples of 4, equal across the
// quad), the word of its row: w[g] afterwards.
__device__ __forceinline__ void drop_words_row4(unsigned int k0, unsigned int k1, int bh, int qi, int kg0, int gs,
                                                unsigned int (&w)[4]) {
  const int r = qi & 3;
  const Philox4 p = philox4x32_10((unsigned)qi >> 2, (unsigned)(kg0 + gs * r) >> 2, (unsigned)bh, 0u, k0, k1);
#pragma unroll
  for (int c = 0; c < 4; ++c) w[c] = p.v[c];
  quad_transpose(w, r);
}

// Lane holds key kj (kj & 3 == lane & 3) and needs, for the four query groups
// qg0 + qs j (j = 0..3, multiples of 4, equal across the quad), the decisions
// of rows qg0 + qs j + 0..3 for its key: byte r of w[j] afterwards is the byte
// of row qg0 + qs j + r (a byte transpose inside the lane, then the quad's).
__device__ __forceinline__ void drop_words_col4(unsigned int k0, unsigned int k1, int bh, int kj, int qg0, int qs,
                                                unsigned int (&w)[4]) {
  const int r = kj & 3;
  const Philox4 p = philox4x32_10((unsigned)(qg0 + qs * r) >> 2, (unsigned)kj >> 2, (unsigned)bh, 0u, k0, k1);
  // byte b of p.v[k] -> byte k of w[b]; perm(a, b, sel) picks bytes 0-3 from b, 4-7 from a
  const unsigned int lo01 = __builtin_amdgcn_perm(p.v[1], p.v[0], 0x05010400u);  // v0.0 v1.0 v0.1 v1.1
  const unsigned int hi01 = __builtin_amdgcn_perm(p.v[1], p.v[0], 0x07030602u);  // v0.2 v1.2 v0.3 v1.3
  const unsigned int lo23 = __builtin_amdgcn_perm(p.v[3], p.v[2], 0x05010400u);
  const unsigned int hi23 = __builtin_amdgcn_perm(p.v[3], p.v[2], 0x07030602u);
  w[0] = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u);
  w[1] = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u);
  w[2] = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
  w[3] = __builtin_amdgcn_perm(hi23, hi01, 0x07060302u);
  quad_transpose(w, r);
}

// keep decision of byte t (0..3) of a word
__device__ __forceinline__ bool drop_keep(unsigned int word, int t, int thr) {
  return ((word >> (8 * t)) & 0xffu) >= (unsigned)thr;
}

// ---------------------------------------------------------------------------
// Tiles staged by LDS DMA (buffer_load ... lds): one wave instruction copies
// 64 x 16 bytes from per-lane global offsets into 1024 contiguous LDS bytes
// (lane L at M0 + 16 L); out-of-range lanes deposit zeros. Rows therefore have
// no padding; instead the 16-byte chunk c of row r is stored at chunk position
// c ^ swz<D>(r) of that row. The swizzle keeps both access patterns of the
// MFMA operands free of bank conflicts (64 banks of 4 bytes = 16 chunk slots
// per 256-byte line):
//  * 16-byte row reads: 16 lanes read chunk c of 16 consecutive rows, and the
//    16 (line row, c ^ swz) slots they hit are all distinct;
//  * transposing reads: 8 consecutive rows x 4 consecutive chunks (64 bytes of
//    a row); each half of the wave covers 4 rows, whose chunks land in 16
//    distinct slots.
// Rows of D 16-bit values; D = 32, 64 or 128. swz has period 16 in r.
template <int D>
__device__ __forceinline__ int swz(int r) {
  constexpr int RP = 128 / D;  // rows per 256-byte line
  constexpr int CPR = D / 8;   // 16-byte chunks per row
  return (4 * ((r / RP) & 3) + ((r >> 2) & 3)) & (CPR - 1);
}
// byte offset of chunk c (16-byte units, logical) of row r in a swizzled tile
template <int D>
__device__ __forceinline__ int swz_off(int r, int c) {
  return r * 2 * D + 16 * (c ^ swz<D>(r));
}

// The DMA loads are written as inline assembly on purpose: the compiler
// cannot tell which LDS bytes an in-flight LDS DMA will write, so for the
// builtin it waits for the load to finish before the next LDS read of any
// buffer, which would expose the full memory latency on every pipeline step.
// Issued from assembly the loads are invisible to its wait counting; the
// caller waits for them explicitly (dma_wait) before the barrier that
// publishes the buffer. M0 (the LDS address) is saved and restored around
// each load. The LDS address is a wave-uniform value computed by scalar
// instructions (the callers pass the wave index as a scalar), so M0 is
// written from an SGPR that no vector instruction produced, and the
// descriptor likewise comes from scalar arithmetic; one wait state separates
// the M0 write from the load.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 rsrc_words(const void* base, unsigned int bytes) {
  const unsigned long long p = (unsigned long long)base;
  return (i32x4){(int)(unsigned)p, (int)((p >> 32) & 0xffffu), (int)bytes, kRsrcWord3};
}
// 16 bytes per lane at a per-lane byte offset into LDS address m0 + 16 lane
__device__ __forceinline__ void dma16(i32x4 r, unsigned int voff, int m0) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(m0), "v"(voff), "s"(r)
      : "memory");
}
// 4 bytes per lane at a per-lane byte offset into LDS address m0 + 4 lane
__device__ __forceinline__ void dma4(i32x4 r, unsigned int voff, int m0) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
      "buffer_load_dword %2, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(m0), "v"(voff), "s"(r)
      : "memory");
}
// LDS byte address of an LDS pointer, for M0
__device__ __forceinline__ int lds_addr(const lds_t* p) { return (int)(size_t)p; }
// wait until every DMA load of this wave has landed in LDS
__device__ __forceinline__ void dma_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Copy rows [row0, row0 + ROWS) of a [*, D] 16-bit tensor (buffer words r,
// row-major) into the swizzled LDS tile at dst. NW waves share the 1 KB
// segments; wave ws (wave-uniform, from readfirstlane) takes segments
// ws, ws + NW, ...
template <int D, int ROWS, int NW>
__device__ __forceinline__ void dma_tile(i32x4 r, int row0, lds_t* dst, int ws, int lane) {
  constexpr int SEG = ROWS * 2 * D / 1024;
  constexpr int RPS = 1024 / (2 * D);  // rows per segment
  constexpr int CPR = D / 8;
  static_assert(SEG >= 1 && (ROWS * 2 * D) % 1024 == 0, "tile must be whole 1 KB segments");
#pragma unroll
  for (int sg = 0; sg < (SEG + NW - 1) / NW; ++sg) {
    const int seg = ws + sg * NW;
    if (SEG % NW == 0 || seg < SEG) {
      const int row = seg * RPS + lane / CPR;
      const int c = (lane % CPR) ^ swz<D>(row);
      dma16(r, (unsigned)((row0 + row) * 2 * D + 16 * c), lds_addr(dst) + seg * 1024);
    }
  }
}

}  // namespace fa
