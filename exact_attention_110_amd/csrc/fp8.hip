// FP8 forward pass of IO-aware exact attention on gfx950.
//
// The same online-softmax recurrence as the 16-bit forward kernels
// (pranaymahendrakar.com lesson "FlashAttention", Researcher tier, "Online
// softmax"), with both contractions on the FP8 matrix cores: the lesson's
// version lineage names an FP8 forward pass as FlashAttention-3's addition,
// without a format; this one takes OCP E4M3 codes and one float descale per
// tensor (real value = code value * descale).
//
// gfx950 mapping:
//  * v_mfma_f32_32x32x64_f8f6f4 (E4M3 on both sides): lane l supplies row or
//    column l % 32 and 32 bytes of the contraction; byte s of lane half h of
//    A meets byte s of lane half h of B (checked on the device with an
//    in-bounds probe), so any order of the contraction index works as long as
//    both operands use it.
//  * S^T = K Q^T per 32-key half tile: Q^T (the B operand, d = 64c + 32h + s)
//    stays in registers; lane l reads K row pi(l % 32) of the half tile, where
//    pi(8j + 4h + m) = 16 (j / 2) + 8h + 4 (j % 2) + m. With that order, the
//    result element i of lane half h is key 16 (i / 8) + 8h + i % 8 of the
//    half tile, so the four consecutive elements 4j .. 4j + 3 of either half
//    tile pack into one dword of the P^T operand in byte order.
//  * O^T += V^T P^T per 64-key tile: the V^T operand comes from LDS with the
//    8-bit transposing read ds_read_b64_tr_b8 (within a group of 16 lanes,
//    byte t of lane i is byte i % 8 of lane 2t + i / 8's 8-byte read): lanes
//    2t and 2t + 1 of a group point at key row 16u + 8h + t, columns c0 and
//    c0 + 8, and lane i receives column c0 + i of those 8 keys, in the byte
//    order the packed probabilities have.
//  * The probabilities are converted to E4M3 (round to nearest even) after
//    the exponential; the lazy reference keeps them at most 2^8, inside the
//    format's range (largest finite 448). The running sum uses the
//    unconverted values.
//  * LDS pitches D + 16 (K rows) and D + 32 (V rows) make the 16-byte K reads
//    and the transposing V reads free of bank conflicts.
#include "common.hpp"
#include "params.hpp"

namespace fa {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr int F8_NW = 4;            // waves per workgroup
constexpr int F8_BM = 32 * F8_NW;   // query rows per workgroup
constexpr int F8_BN = 64;           // keys per tile

__device__ __forceinline__ f32x16 mfma_f8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ i32x8 cat32(s16x8 lo, s16x8 hi) {
  const i32x4 a = __builtin_bit_cast(i32x4, lo), b = __builtin_bit_cast(i32x4, hi);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ i32x2 lds_read_tr8(const lds_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)(p));
}

// four probabilities -> one dword of E4M3 codes, p0 in the low byte
__device__ __forceinline__ int pack4_e4m3(float p0, float p1, float p2, float p3) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, w, true);
}

template <class TO, int D, int BAND>
__global__ __launch_bounds__(F8_NW * 64, 2) void fwd_fp8_kernel(Fp8FwdArgs a) {
  constexpr int KP = D + 16;  // K row pitch in LDS, bytes
  constexpr int VP = D + 32;  // V row pitch in LDS, bytes
  constexpr int KBUF = F8_BN * KP;
  constexpr int VBUF = F8_BN * VP;
  constexpr int CH = D / 16;                           // 16-byte chunks per row
  constexpr int PER = F8_BN * CH / (F8_NW * 64);      // chunks per thread per tensor per tile
  static_assert(PER >= 1 && (F8_BN * CH) % (F8_NW * 64) == 0, "tile loader shape");
  constexpr int NC = D / 64;  // contraction steps of Q K^T
  constexpr int ND = D / 32;  // 32-wide d blocks of the output
  static_assert(BAND == 0 || BAND == 1, "the FP8 kernel takes no lower band edge");

  __shared__ __attribute__((aligned(16))) char smem_raw[2 * KBUF + 2 * VBUF];
  lds_t* kbuf = (lds_t*)smem_raw;
  lds_t* vbuf = kbuf + 2 * KBUF;

  const AttnShape& s = a.s;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  // grid (tile_grid); under causal masking the longest blocks first
  const GridPos gp = grid_pos(s);
  const int qb = BAND ? gp.nblk - 1 - gp.blk : gp.blk;
  const int h = query_head(s, blockIdx.x), b = gp.b;
  const int hk = h / s.G;
  const SeqView sv = seq_view(s, b, h, hk);
  const int nq = sv.nq, nk = sv.nk;
  const int q0 = qb * F8_BM;
  if (q0 >= nq) return;
  const size_t qrow0 = sv.qrow0, krow0 = sv.krow0;
  const unsigned int qbytes = (unsigned int)nq * D, kbytes = (unsigned int)nk * D;
  const rsrc_t rq = make_rsrc((const unsigned char*)a.q + qrow0 * D, qbytes);
  const rsrc_t rk = make_rsrc((const unsigned char*)a.k + krow0 * D, kbytes);
  const rsrc_t rv = make_rsrc((const unsigned char*)a.v + krow0 * D, kbytes);
  const int qw = q0 + 32 * w;
  const int qi = qw + l32;
  // S * c is the score in log2 units: softmax scale and both descales folded in
  const float c = fmaxf(s.scale * a.q_descale * a.k_descale * kLog2e, 1e-30f);
  const int offu = sv.off + s.wr;  // causal: row i sees keys up to i + offu

  const int kend = BAND ? min(nk, max(0, q0 + F8_BM + offu)) : nk;
  const int ntiles = (kend + F8_BN - 1) / F8_BN;

  // Q^T operand: lane holds query qi, d = 64 c + 32 hh + 0..31
  i32x8 qf[NC];
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) {
    const unsigned int o = (unsigned)(qi * D + 64 * cc + 32 * hh);
    qf[cc] = cat32(bload16(rq, o), bload16(rq, o + 16u));
  }

  f32x16 acc[ND];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;
  constexpr float kSlack = 8.f;  // probabilities stay <= 2^8 < 448
  float m = -INFINITY;
  float l = 0.f;

  // K row this lane supplies to the S^T contraction (see pi above)
  const int kr = 16 * (l32 >> 4) + 8 * ((l32 >> 2) & 1) + 4 * ((l32 >> 3) & 1) + (l32 & 3);
  // transposing-read source of this lane: key row 16 u + 8 hh + (i / 2), column c0 + 8 (i % 2)
  const int i16 = lane & 15;
  const int vr = 8 * hh + (i16 >> 1);
  const int vc = 16 * ((lane >> 4) & 1) + 8 * (i16 & 1);

  s16x8 kreg[PER], vreg[PER];
  auto gload = [&](int t) {
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const int ci = tid + r * (F8_NW * 64);
      const int row = ci / CH, col = (ci % CH) * 16;
      const unsigned int o = (unsigned)((t * F8_BN + row) * D + col);
      kreg[r] = bload16(rk, o);
      vreg[r] = bload16(rv, o);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const int ci = tid + r * (F8_NW * 64);
      const int row = ci / CH, col = (ci % CH) * 16;
      lds_write16(kbuf + buf * KBUF + row * KP + col, kreg[r]);
      lds_write16(vbuf + buf * VBUF + row * VP + col, vreg[r]);
    }
  };

  gload(0);
  lstore(0);
  __syncthreads();

  for (int e = 0; e < ntiles; ++e) {
    const int buf = e & 1;
    const int ks = e * F8_BN;
    gload(e + 1 < ntiles ? e + 1 : e);

    const bool active = !(BAND && ks > qw + 31 + offu);  // wave-uniform
    if (active) {
      const lds_t* kb = kbuf + buf * KBUF;
      const lds_t* vb = vbuf + buf * VBUF;
      f32x16 sc[2];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sc[0][i] = 0.f;
        sc[1][i] = 0.f;
      }
#pragma unroll
      for (int cc = 0; cc < NC; ++cc)
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          const lds_t* kp = kb + (32 * t2 + kr) * KP + 64 * cc + 32 * hh;
          sc[t2] = mfma_f8(cat32(lds_read16(kp), lds_read16(kp + 16)), qf[cc], sc[t2]);
        }
      // sc[t2][i] is S (times c / scale) for query qi and key ks + 32 t2 + 16 (i / 8) + 8 hh + i % 8
      const bool need_mask = (BAND && ks + F8_BN - 1 > qw + offu) || (ks + F8_BN > nk);
      if (need_mask) {
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = ks + 32 * t2 + 16 * (i >> 3) + 8 * hh + (i & 7);
            if ((BAND && key > qi + offu) || key >= nk) sc[t2][i] = -INFINITY;
          }
      }
      float mx = sc[0][0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sc[0][i]);
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[1][i]);
      mx = fmaxf(mx, swap_halves(mx)) * c;
      if (__any(mx > m + kSlack)) {  // wave-uniform: raise the reference, rescale
        const float m_new = fmaxf(m, mx);
        const float corr = fast_exp2(m - ((m_new == -INFINITY) ? 0.f : m_new));
        m = m_new;
        l *= corr;
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[dt][i] *= corr;
      }
      const float m_use = (m == -INFINITY) ? 0.f : m;
      // P^T operand: byte 16 t2 + 4 j + r is element 4 j + r of half tile t2
      i32x8 pb;
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float p[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) p[r] = fast_exp2(fmaf(sc[t2][4 * j + r], c, -m_use));
          l += (p[0] + p[1]) + (p[2] + p[3]);
          pb[4 * t2 + j] = pack4_e4m3(p[0], p[1], p[2], p[3]);
        }
      // O^T(d x q) += V^T(d x key) P^T(key x q); byte 8u + t of lane half hh is key 16u + 8hh + t
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) {
        const lds_t* vp = vb + vr * VP + 32 * dt + vc;
        const i32x2 r0 = lds_read_tr8(vp), r1 = lds_read_tr8(vp + 16 * VP), r2 = lds_read_tr8(vp + 32 * VP),
                    r3 = lds_read_tr8(vp + 48 * VP);
        const i32x8 va = {r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
        acc[dt] = mfma_f8(va, pb, acc[dt]);
      }
    }
    lstore(buf ^ 1);
    __syncthreads();
  }

  const float lt = l + swap_halves(l);
  const float inv = lt > 0.f ? a.v_descale / lt : 0.f;
  const float lse = lt > 0.f ? (m + fast_log2(lt)) * kLn2 : -INFINITY;
  const rsrc_t ro = make_rsrc((unsigned short*)a.o + qrow0 * D, (unsigned int)nq * D * 2);
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x2 v2 = {pack2<TO>(acc[dt][4 * j] * inv, acc[dt][4 * j + 1] * inv),
                  pack2<TO>(acc[dt][4 * j + 2] * inv, acc[dt][4 * j + 3] * inv)};
      bstore8(ro, (unsigned)(qi * D + 32 * dt + 8 * j + 4 * hh) * 2u, v2);
    }
  if (hh == 0) bstore_f32(make_rsrc(a.lse + qrow0, (unsigned)nq * 4u), (unsigned)qi * 4u, lse);
}

template <class TO, int D>
static hipError_t launch_fp8_t(const Fp8FwdArgs& a, hipStream_t st) {
  Fp8FwdArgs la = a;
  const dim3 grid = tile_grid(la.s, a.s.H, (a.s.Nq + F8_BM - 1) / F8_BM);
  if (a.s.band) hipLaunchKernelGGL((fwd_fp8_kernel<TO, D, 1>), grid, dim3(F8_NW * 64), 0, st, la);
  else hipLaunchKernelGGL((fwd_fp8_kernel<TO, D, 0>), grid, dim3(F8_NW * 64), 0, st, la);
  return hipGetLastError();
}

hipError_t launch_forward_fp8(const Fp8FwdArgs& a, int out_dtype, hipStream_t st) {
  if (out_dtype == 2) return a.s.d == 64 ? launch_fp8_t<BF16, 64>(a, st) : launch_fp8_t<BF16, 128>(a, st);
  return a.s.d == 64 ? launch_fp8_t<F16, 64>(a, st) : launch_fp8_t<F16, 128>(a, st);
}

}  // namespace fa
