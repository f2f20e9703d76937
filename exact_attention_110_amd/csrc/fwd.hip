// Forward pass of IO-aware exact attention on gfx950.
//
// A workgroup owns a block of query rows of one (batch, head) and streams the
// visible key/value tiles of its kv head through LDS, keeping a reference row
// maximum m, the running sum l of exponentials and the unnormalised output in
// registers; whenever m is raised the earlier partial sums are rescaled by
// exp(m_old - m_new). This is the online-softmax recurrence of the
// pranaymahendrakar.com lesson "FlashAttention" (Researcher tier, "Online
// softmax"); the output is O / l and the saved statistic is m + ln(l).
//
// gfx950 mapping (16-bit inputs):
//  * Each wave computes S^T = K Q^T with v_mfma_f32_32x32x16 (Q^T is the B
//    operand and stays in registers). In the 32x32 result layout a lane owns
//    one query column, so a row maximum needs one cross-half exchange
//    (permlane32 swap) and the row sum none until the end.
//  * The probabilities, converted to 16 bits, are already laid out as the B
//    operand of O^T = V^T P^T. The matching V^T operand comes from LDS with the
//    gfx950 transposing read ds_read_b64_tr_b16, so V needs no transpose pass.
//  * LDS row pitches are padded so that the 16-byte row reads of K and the
//    transposing reads of V are free of bank conflicts.
//  * fwd64_kernel (64 query rows per wave pair, 256 rows per workgroup; at
//    d = 128 as a producer wave forming the probabilities and a consumer wave
//    holding O on each SIMD, otherwise as one wave per SIMD) runs at head size
//    128 when its grid holds at least 256 workgroups and the rows have 4096
//    keys or more (1024 without a causal or window band), or when the grid
//    holds at least 2048; the others, and all block-sparse inputs, run
//    fwd_kernel (32 rows per wave, two waves per SIMD, 128 rows per workgroup
//    = one mask block row).
//  * Causal: a workgroup stops at its diagonal tile, waves skip tiles that lie
//    wholly after their rows, and only diagonal and tail tiles are masked
//    element by element. Heaviest query blocks are launched first.
//  * Block-sparse: the nonzero 128-key blocks of the workgroup's mask row are
//    compacted into an LDS list first; zero blocks are never loaded.
//  * Grouped-query: query head h reads kv head h / (H / Hkv).
//
// float32 inputs take a separate VALU kernel (fp32 FMA throughout) that runs
// the same recurrence one query row per lane.
#include "common.hpp"
#include "params.hpp"

namespace fa {

constexpr int FWD_NW = 4;             // waves per workgroup
constexpr int FWD_BM = 32 * FWD_NW;   // query rows per workgroup (= mask block)
constexpr int FWD_BN = 64;            // keys per tile
constexpr int FWD_LIST = 2048;        // capacity of the compacted mask-block list
static_assert(FWD_BM == 128, "a forward workgroup must cover exactly one mask block row");

template <class T, int D, int BAND, bool MASK, bool DROP, bool ALIBI>
__global__ __launch_bounds__(FWD_NW * 64, 2) void fwd_kernel(FwdArgs a) {
  constexpr int KP = D * 2 + 16;  // K row pitch in LDS, bytes (16 mod 128: conflict-free 16-byte reads)
  constexpr int VP = D * 2 + 32;  // V row pitch in LDS, bytes (32 mod 128: conflict-free transposing reads)
  constexpr int KBUF = FWD_BN * KP;
  constexpr int VBUF = FWD_BN * VP;
  constexpr int CH = D / 8;                            // 16-byte chunks per row
  constexpr int PER = FWD_BN * CH / (FWD_NW * 64);     // chunks per thread per tensor per tile
  static_assert(PER >= 1 && (FWD_BN * CH) % (FWD_NW * 64) == 0, "tile loader shape");
  constexpr int NS = D / 16;  // k-steps of Q K^T
  constexpr int ND = D / 32;  // 32-wide d tiles of the output

  __shared__ __attribute__((aligned(16))) char smem_raw[2 * KBUF + 2 * VBUF + (MASK ? 2 * FWD_LIST + 16 : 16)];
  lds_t* smem = (lds_t*)smem_raw;
  lds_t* kbuf = smem;
  lds_t* vbuf = smem + 2 * KBUF;
  __attribute__((address_space(3))) short* blist =
      (__attribute__((address_space(3))) short*)(smem + 2 * KBUF + 2 * VBUF);
  __attribute__((address_space(3))) int* bcount =
      (__attribute__((address_space(3))) int*)(smem + 2 * KBUF + 2 * VBUF + (MASK ? 2 * FWD_LIST : 0));

  const AttnShape& s = a.s;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  // grid (tile_grid): heads fastest; under a band mask the later (under causal
  // masking, longer) query blocks are dispatched first
  const GridPos gp = grid_pos(s);
  const int qb = BAND ? gp.nblk - 1 - gp.blk : gp.blk;
  const int h = query_head(s, blockIdx.x), b = gp.b;
  const int hk = h / s.G;
  const SeqView sv = seq_view(s, b, h, hk);
  const int nq = sv.nq, nk = sv.nk, off = sv.off;
  const int q0 = qb * FWD_BM;
  if (q0 >= nq) return;  // a sequence shorter than the grid (packed batches)
  const size_t qrow0 = sv.qrow0, krow0 = sv.krow0;
  // per-sequence buffer resources: rows past the sequence read as zeros, stores
  // past it are dropped
  const unsigned int qbytes = (unsigned int)nq * D * 2, kbytes = (unsigned int)nk * D * 2;
  const rsrc_t rq = make_rsrc((const unsigned short*)a.q + qrow0 * D, qbytes);
  const rsrc_t rk = make_rsrc((const unsigned short*)a.k + krow0 * D, kbytes);
  const rsrc_t rv = make_rsrc((const unsigned short*)a.v + krow0 * D, kbytes);
  const int qw = q0 + 32 * w;   // first query row of this wave
  const int qi = qw + l32;      // query row of this lane's column
  // exponent scale: S * c is the score in log2 units; a zero scale is kept just
  // above zero so that masked entries stay -inf (-inf * 0 would be NaN)
  const float c = fmaxf(s.scale * kLog2e, 1e-30f);
  const float nsl2 = ALIBI ? -s.alibi[h] * kLog2e : 0.f;  // ALiBi slope of this head, log2 units
  // Distance from the row to its nearest key, max(0, -(qi + off)): the bias is
  // taken relative to it, which the softmax does not see, so that fp32 scores
  // stay small where every key lies far from the diagonal (more queries than
  // keys); the LSE gets the shift back at the end
  const float dmin = ALIBI ? (float)max(0, -(qi + off)) : 0.f;

  // keys [kbeg, kend) are seen by some row of the workgroup: row q0 has the
  // lowest band start, the last row the highest band end
  // (band: row i sees keys i + offl .. i + offu; offl binds only with a lower edge)
  constexpr bool LOWER = BAND == 2;
  const int offu = off + s.wr, offl = off - s.wl;
  const int kbeg = LOWER ? max(0, q0 + offl) : 0;
  const int kend = BAND ? min(nk, max(0, q0 + FWD_BM + offu)) : nk;
  const int tbeg = kbeg / FWD_BN;
  const int ntile_all = (kend + FWD_BN - 1) / FWD_BN;
  int ntiles = max(0, ntile_all - tbeg);
  if constexpr (MASK) {
    const int nbk = (kend + 127) / 128;
    if (w == 0) {
      int cnt = 0;
      for (int j0 = kbeg / 128; j0 < nbk; j0 += 64) {
        const int j = j0 + lane;
        const bool keep = j < nbk && s.mask[(size_t)qb * s.nbk + j] != 0;
        const unsigned long long bal = __ballot(keep);
        if (keep) blist[cnt + __popcll(bal & ((1ull << lane) - 1ull))] = (short)j;
        cnt += __popcll(bal);
      }
      if (lane == 0) *bcount = cnt;
    }
    __syncthreads();
    const int cnt = *bcount;
    ntiles = 2 * cnt;
    if (cnt > 0 && 2 * blist[cnt - 1] + 1 >= ntile_all) ntiles -= 1;  // half block past kend
  }
  auto tile_at = [&](int e) -> int {
    if constexpr (MASK) return 2 * blist[e >> 1] + (e & 1);
    else return tbeg + e;
  };

  // Q^T operand: lane holds query qi, d = 16 * ss + 8 * hh + 0..7
  s16x8 qf[NS];
#pragma unroll
  for (int ss = 0; ss < NS; ++ss) qf[ss] = bload16(rq, (unsigned)(qi * D + 16 * ss + 8 * hh) * 2u);

  f32x16 acc[ND];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;
  // Running reference m (in log2 units) and this lane's share l of the running
  // sum (its half of the keys). m is raised only when a row of the wave
  // exceeds it by more than kSlack, so most tiles skip the rescale; any common
  // reference gives the same O / l and m + log2(l), and P stays <= 2^kSlack
  // (2^7 for float16 with dropout, whose keep scale reaches 256: the scaled
  // probability must stay below float16's largest value, 65504).
  constexpr float kSlack = (std::is_same<T, F16>::value && DROP) ? 7.f : 8.f;
  float m = -INFINITY;
  float l = 0.f;

  // lane offsets for the transposing V reads (row = key, column = d)
  const int g16 = lane >> 4;
  const int roff = 4 * (g16 >> 1) + ((lane & 15) >> 2);
  const int coff = 16 * (g16 & 1) + 4 * (lane & 3);

  s16x8 kreg[PER], vreg[PER];
  auto gload_tile = [&](int t) {
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const int ci = tid + r * (FWD_NW * 64);
      const int row = ci / CH, col = (ci % CH) * 8;
      const unsigned int off = (unsigned)((t * FWD_BN + row) * D + col) * 2u;
      kreg[r] = bload16(rk, off);
      vreg[r] = bload16(rv, off);
    }
  };
  auto lstore_tile = [&](int buf) {
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const int ci = tid + r * (FWD_NW * 64);
      const int row = ci / CH, col = (ci % CH) * 8;
      lds_write16(kbuf + buf * KBUF + row * KP + col * 2, kreg[r]);
      lds_write16(vbuf + buf * VBUF + row * VP + col * 2, vreg[r]);
    }
  };

  // Loads are issued on every path (indices clamped; buffer loads make a
  // redundant or out-of-range tile harmless) so that the compiler can count
  // outstanding loads exactly and never waits on a prefetch before computing.
  gload_tile(ntiles > 0 ? tile_at(0) : 0);
  lstore_tile(0);
  __syncthreads();

  // element masks of partial blocks: bit tiles through a buffer resource
  const rsrc_t rbits = make_rsrc(s.bits, (unsigned)s.ntiles * 2048u);
  for (int e = 0; e < ntiles; ++e) {
    const int buf = e & 1;
    const int ks = tile_at(e) * FWD_BN;
    gload_tile(tile_at(e + 1 < ntiles ? e + 1 : e));

    // wave-uniform: does any row of the wave see a key of the tile
    const bool active = !(BAND && ks > qw + 31 + offu) && !(LOWER && ks + FWD_BN - 1 < qw + offl);
    if (active) {
      // a partial block: this row's bits for the tile's two 32-key halves
      int tidx = -1;
      if constexpr (MASK) {
        if (s.btile) tidx = s.btile[(size_t)qb * s.nbk + (ks >> 7)];
      }
      u32x2 bw = {~0u, ~0u};
      if (tidx >= 0) bw = bload_u32x2(rbits, bits_off(tidx, qi & 127, (ks & 127) >> 5));
      const lds_t* kb = kbuf + buf * KBUF;
      const lds_t* vb = vbuf + buf * VBUF;
      f32x16 sc[2];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sc[0][i] = 0.f;
        sc[1][i] = 0.f;
      }
#pragma unroll
      for (int ss = 0; ss < NS; ++ss) {
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          const s16x8 ka = lds_read16(kb + (32 * t2 + l32) * KP + (16 * ss + 8 * hh) * 2);
          sc[t2] = mfma32<T>(ka, qf[ss], sc[t2]);
        }
      }
      // sc[t2][i] is S for query qi and key ks + 32 t2 + 8 (i / 4) + 4 hh + i % 4
      const bool need_mask = (BAND && ks + FWD_BN - 1 > qw + offu) || (LOWER && ks < qw + 31 + offl) ||
                             (ks + FWD_BN > nk) || tidx >= 0;
      if (need_mask) {
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int kofs = 8 * (i >> 2) + 4 * hh + (i & 3);  // key within the 32-key half
            const int key = ks + 32 * t2 + kofs;
            if ((BAND && key > qi + offu) || (LOWER && key < qi + offl) || key >= nk || !((bw[t2] >> kofs) & 1u))
              sc[t2][i] = -INFINITY;
          }
      }
      // ALiBi: the scores move to log2 units with the bias added, -slope log2(e)
      // (|qi + off - key| - dmin); key - ks - 4 hh is a constant of the element
      float cs = c;
      if constexpr (ALIBI) {
        const float dqf = (float)(qi + off - ks - 4 * hh);
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            sc[t2][i] = fmaf(sc[t2][i], c,
                             nsl2 * (fabsf(dqf - (float)(32 * t2 + 8 * (i >> 2) + (i & 3))) - dmin));
        cs = 1.f;
      }
      float mx = sc[0][0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sc[0][i]);
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[1][i]);
      mx = fmaxf(mx, swap_halves(mx)) * cs;
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
      const float m_use = (m == -INFINITY) ? 0.f : m;  // a row with no visible key yet

      unsigned int pk[2][8];
      // dropout words of this row for key groups ks + 32 t2 + 8 g + 4 hh (g = 0..3)
      unsigned int dw[2][4];
      if constexpr (DROP) {
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) drop_words_row4(s.seed0, s.seed1, b * s.H + h, qi, ks + 32 * t2 + 4 * hh, 8, dw[t2]);
      }
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float p0 = fast_exp2(fmaf(sc[t2][2 * j], cs, -m_use));
          const float p1 = fast_exp2(fmaf(sc[t2][2 * j + 1], cs, -m_use));
          l += p0 + p1;  // the normaliser sums the probabilities before dropout
          if constexpr (DROP) {
            // elements 2j, 2j + 1 are keys kg + (2j & 3) + 0, 1 of group kg
            const unsigned int wd = dw[t2][j >> 1];
            const int t0 = (2 * j) & 3;
            pk[t2][j] = pack2<T>(drop_keep(wd, t0, s.drop_t) ? p0 * s.drop_scale : 0.f,
                                 drop_keep(wd, t0 + 1, s.drop_t) ? p1 * s.drop_scale : 0.f);
          } else {
            pk[t2][j] = pack2<T>(p0, p1);
          }
        }
      // O^T(d x q) += V^T(d x key) P^T(key x q); B operand k-slot j of step (t2, u)
      // is key 32 t2 + 16 u + 8 (j / 4) + 4 hh + j % 4, matched by the V^T reads.
      // The two waves of a SIMD run this block at raised priority, so that one
      // wave's P V products issue back to back while the other computes its
      // exponentials (measured: 5% faster at 32 heads x 8192, same-box)
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const lds_t* vp = vb + (32 * t2 + 16 * u + roff) * VP + (32 * dt + coff) * 2;
            const s16x8 va = concat(lds_read_tr(vp), lds_read_tr(vp + 8 * VP));
            const s16x8 pb = as_operand(pk[t2][4 * u], pk[t2][4 * u + 1], pk[t2][4 * u + 2],
                                        pk[t2][4 * u + 3]);
            acc[dt] = mfma32<T>(va, pb, acc[dt]);
          }
      __builtin_amdgcn_s_setprio(0);
    }
    lstore_tile(buf ^ 1);
    __syncthreads();
  }

  const float lt = l + swap_halves(l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  float lse = lt > 0.f ? (m + fast_log2(lt)) * kLn2 : -INFINITY;
  if constexpr (ALIBI) lse = fmaf(-s.alibi[h], dmin, lse);
  const rsrc_t ro = make_rsrc((unsigned short*)a.o + qrow0 * D, qbytes);
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x2 v2 = {pack2<T>(acc[dt][4 * j] * inv, acc[dt][4 * j + 1] * inv),
                  pack2<T>(acc[dt][4 * j + 2] * inv, acc[dt][4 * j + 3] * inv)};
      bstore8(ro, (unsigned)(qi * D + 32 * dt + 8 * j + 4 * hh) * 2u, v2);
    }
  if (hh == 0) bstore_f32(make_rsrc(a.lse + qrow0, (unsigned)nq * 4u), (unsigned)qi * 4u, lse);
}

// acc *= s for an accumulator held in AGPRs, one element at a time through a
// single temporary VGPR. Written out because the compiler otherwise moves all
// accumulators of a wave into VGPRs at once, which the 64-row kernel cannot
// afford. The leading s_nops cover the wait an AGPR read needs after the MFMA
// that wrote it, the trailing ones the wait before an MFMA reads it again.
__device__ __forceinline__ void scale_acc(f32x16& x, float s) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float e = x[i];
    float t;
    asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                 : "+a"(e), "=&v"(t)
                 : "v"(s));
    x[i] = e;
  }
  asm volatile("s_nop 7" ::: "memory");
}

// Dense and causal inputs: 64 query rows per wave, one wave per SIMD.
//
// Each K fragment read from LDS feeds the two 32-row column blocks of the wave
// and each V^T fragment the two matching output blocks, which halves LDS reads
// per MFMA against 32 rows per wave (at 32 rows the reads of K and V^T cost as
// much LDS time as the MFMAs take). The register file then holds one wave per
// SIMD, so latency is hidden inside the wave: the tile loop is pipelined three
// deep. Iteration j issues S of tile j + 1, the probabilities of tile j and
// P V of tile j - 1, which are independent of each other, then stages tile
// j + 2 in the LDS slot tile j - 2 used (a ring of four K/V slots) and ends
// with one barrier. In this loop the reference maximum is fixed at the first
// tile's row maximum (any reference gives the same O / l and m + log2 l), so
// the loop body has no rescale and no branch and the compiler can interleave
// the exponentials with the MFMAs. Only tiles that every row of the workgroup
// sees in full run here; the diagonal tiles of causal attention and a ragged
// last tile follow in a plain loop with element masks and lazy rescaling,
// which also takes over the whole workgroup in the rare case that a later
// score outgrows the fixed reference.
constexpr int F64_NW = 4;                 // waves per workgroup (wave pairs in the split-role form)
constexpr int F64_RW = 64;                // query rows per wave
constexpr int F64_BM = F64_NW * F64_RW;   // query rows per workgroup
constexpr int F64_BN = 32;                // keys per tile
constexpr int F64_NB = 4;                 // LDS ring slots

// The same rows and tiles with split roles (d = 128; every band kind and
// dropout): eight waves, two per SIMD. Producer wave j
// (0..3) holds Q^T of rows q0 + 64 j .. + 63 and forms S^T and the
// probabilities; it hands P^T, as the consumer's MFMA B operands, through one
// of two LDS buffers to consumer wave j + 4 on the same SIMD, which holds the
// O^T accumulators and adds V^T P^T one tile behind. Each role fits in half
// the register file, so the producer's softmax arithmetic runs while the
// consumer's products occupy the matrix unit. Main loop (the tiles every row
// sees in full, fixed reference): iteration j forms S of tile j + 1 and P of
// tile j on the producer side, in slots of one MFMA and two probability
// elements each (fenced order: the compiler's own order put the products of
// a tile ahead of all its exponentials, which left the producer waiting on
// the matrix unit the consumer shares), and P V of tile j - 1 on the consumer
// side. The producers also start the LDS DMA of tile j + 3 (swizzled rows; K
// in a ring of four slots, V, which the consumers read four iterations after
// it is started, in a ring of eight) and wait only for the loads they started
// an iteration earlier; all eight waves meet at one barrier. The general
// loop (diagonal and ragged tiles, or a restart) raises the reference lazily:
// the producer then also hands over, per tile, whether its rows see the tile
// and whether the reference rose, with the per-row factors exp(m_old - m_new)
// by which the consumer scales O first. Finally the producer writes the
// log-sum-exp and hands 1 / l to the consumer, which writes O.
template <int D, int BAND, bool DROP>
constexpr bool f64_split() {
  return D == 128;
}

template <class T, int D, int BAND, bool DROP>
__device__ __forceinline__ void fwd64_split_body(const FwdArgs& a) {
  constexpr int KBUF = F64_BN * 2 * D;  // K tile: swizzled rows (16-byte row reads)
  constexpr int VBUF = F64_BN * 2 * D;  // V tile: swizzled rows (transposing reads)
  constexpr int NS = D / 16;
  constexpr int ND = D / 32;
  constexpr float kSlack = (std::is_same<T, F16>::value && DROP) ? 7.f : 8.f;  // as in fwd_kernel
  // one pair's hand-over buffer: P^T (four 16-byte chunks per lane, chunk
  // 2 rb + u holding the B operand of MFMA step u of row block rb), then the
  // 64 rows' rescale factors, then the flags (bit 0: the pair's rows see the
  // tile, bit 1: the reference rose)
  constexpr int HB = 4096 + 256 + 16;
  constexpr int VNB = 2 * F64_NB;  // V ring slots
  __shared__ __attribute__((aligned(16))) char smem_raw[F64_NB * KBUF + VNB * VBUF + 2 * F64_NW * HB + F64_NW * 256];
  lds_t* kbuf = (lds_t*)smem_raw;
  lds_t* vbuf = kbuf + F64_NB * KBUF;
  lds_t* hbuf = vbuf + VNB * VBUF;    // [2][pairs][HB]
  lds_t* ibuf = hbuf + 2 * F64_NW * HB;  // [pairs][64 rows] final 1 / l

  const AttnShape& s = a.s;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wu = __builtin_amdgcn_readfirstlane(tid >> 6);  // the wave index as a scalar
  const bool producer = wu < F64_NW;
  const int pw = wu & (F64_NW - 1);  // the pair: rows q0 + 64 pw .. + 63
  const int l32 = lane & 31, hh = lane >> 5;
  const int g16 = lane >> 4;
  const int roff = 4 * (g16 >> 1) + ((lane & 15) >> 2);
  const int coff = 16 * (g16 & 1) + 4 * (lane & 3);
  const GridPos gp = grid_pos(s);
  const int qb = BAND ? gp.nblk - 1 - gp.blk : gp.blk;
  const int h = query_head(s, blockIdx.x), b = gp.b;
  const int hk = h / s.G;
  const SeqView sv = seq_view(s, b, h, hk);
  const int nq = sv.nq, nk = sv.nk, off = sv.off;
  const int q0 = qb * F64_BM;
  if (q0 >= nq) return;  // a sequence shorter than the grid (packed batches)
  const size_t qrow0 = sv.qrow0, krow0 = sv.krow0;
  const unsigned int qbytes = (unsigned int)nq * D * 2, kbytes = (unsigned int)nk * D * 2;
  const int qw = q0 + F64_RW * pw;  // block rb of the pair holds rows qw + 32 rb + 0..31
  const float c = fmaxf(s.scale * kLog2e, 1e-30f);
  // tiles [tbeg, tbeg + ntiles) hold every key some row of the workgroup sees,
  // tiles [fbeg, fend) only keys that every row sees (row i sees keys i + off -
  // wl .. i + off + wr; offl binds only with a lower edge); processing order:
  // the full tiles, the partial ones above them, then those below (tile_of)
  constexpr bool LOWER = BAND == 2;
  const int offu = off + s.wr, offl = off - s.wl;
  const int kbeg = LOWER ? max(0, q0 + offl) : 0;
  const int kend = BAND ? min(nk, max(0, q0 + F64_BM + offu)) : nk;
  const int tbeg = kbeg / F64_BN;
  const int ntiles = max(0, (kend + F64_BN - 1) / F64_BN - tbeg);
  const int fbeg =
      LOWER ? min(tbeg + ntiles, max(tbeg, (max(0, q0 + F64_BM - 1 + offl) + F64_BN - 1) / F64_BN)) : 0;
  const int fend = BAND ? max(fbeg, min(max(0, q0 + offu + 1) / F64_BN, nk / F64_BN)) : nk / F64_BN;
  const int nfull = fend - fbeg;
  const int nhead = tbeg + ntiles - fbeg;
  auto tile_of = [&](int e) -> int {
    if constexpr (LOWER) return e < nhead ? fbeg + e : tbeg + (e - nhead);
    else return e;
  };

  const i32x4 rkw = rsrc_words((const unsigned short*)a.k + krow0 * D, kbytes);
  const i32x4 rvw = rsrc_words((const unsigned short*)a.v + krow0 * D, kbytes);
  // the producer waves stage key tile t, the e-th of the processing order, by
  // LDS DMA into K slot e % 4 and V slot e % 8 (keys past the sequence read as
  // zeros); a stager's wait for all but its last stage's four loads lets each
  // load run for a whole iteration
  auto stage = [&](int t, int e) {
    dma_tile<D, F64_BN, F64_NW>(rkw, t * F64_BN, kbuf + (e & (F64_NB - 1)) * KBUF, wu, lane);
    dma_tile<D, F64_BN, F64_NW>(rvw, t * F64_BN, vbuf + (e & (VNB - 1)) * VBUF, wu, lane);
  };
  auto dma_wait_prev = [&]() { asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); };
  auto hand = [&](int buf) -> lds_t* { return hbuf + (buf * F64_NW + pw) * HB; };

  // Every wave takes the same sequence of barriers: the prologue's, one per
  // main-loop tile, the restart vote, one per general-loop tile, the final one.
  if (producer) {
    stage(tile_of(0), 0);
    stage(tile_of(max(0, min(1, ntiles - 1))), 1);
    stage(tile_of(max(0, min(2, ntiles - 1))), 2);
    dma_wait();
  }
  __syncthreads();

  // restart bound of the fixed-reference loop, as in the one-role form below
  const float lmax = std::is_same<T, F16>::value ? 65504.f / (DROP ? s.drop_scale : 1.f) : 0x1p60f;
  int j = 0;
  if (producer) {
    const rsrc_t rq = make_rsrc((const unsigned short*)a.q + qrow0 * D, qbytes);
    s16x8 qf[2][NS];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int ss = 0; ss < NS; ++ss)
        qf[rb][ss] = bload16(rq, (unsigned)((qw + 32 * rb + l32) * D + 16 * ss + 8 * hh) * 2u);
    // running reference m (log2 units) and this lane's half of the running sum, per row block
    float m[2] = {-INFINITY, -INFINITY};
    float l[2] = {0.f, 0.f};
    // S^T = K Q^T of the tile in a slot: st[rb][i] is S of query qw + 32 rb + l32
    // and key 8 (i / 4) + 4 hh + i % 4 of the tile
    auto s_tile = [&](int slot, f32x16 (&st)[2]) {
      const lds_t* kb = kbuf + slot * KBUF;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        st[0][i] = 0.f;
        st[1][i] = 0.f;
      }
#pragma unroll
      for (int ss = 0; ss < NS; ++ss) {
        const s16x8 ka = lds_read16(kb + swz_off<D>(l32, 2 * ss + hh));
        st[0] = mfma32<T>(ka, qf[0][ss], st[0]);
        st[1] = mfma32<T>(ka, qf[1][ss], st[1]);
      }
    };
    // 16-bit probabilities of a pair of elements, with dropout when built for
    // it (dw: the row's dropout words for key groups ks + 8 g + 4 hh, g = 0..3,
    // from drop_words_row4; jj: the pair, keys ks + 8 (jj / 2) + 4 hh + (2 jj & 3) + 0, 1)
    auto pack_p = [&](float p0, float p1, int jj, const unsigned int (&dw)[4]) -> unsigned int {
      if constexpr (DROP) {
        const unsigned int wd = dw[jj >> 1];
        const int t0 = (2 * jj) & 3;
        return pack2<T>(drop_keep(wd, t0, s.drop_t) ? p0 * s.drop_scale : 0.f,
                        drop_keep(wd, t0 + 1, s.drop_t) ? p1 * s.drop_scale : 0.f);
      } else {
        return pack2<T>(p0, p1);
      }
    };
    auto write_p = [&](lds_t* hb, const unsigned int (&pk)[2][8]) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int u = 0; u < 2; ++u)
          lds_write16(hb + (2 * rb + u) * 1024 + lane * 16,
                      __builtin_bit_cast(s16x8, (u32x4){pk[rb][4 * u], pk[rb][4 * u + 1], pk[rb][4 * u + 2],
                                                        pk[rb][4 * u + 3]}));
    };
    if (nfull > 0) {
      // one iteration in slots: S product t of the next tile, then elements
      // 2 t and 2 t + 1 of the current tile's probabilities (fenced order)
      auto iter = [&](int jj, const f32x16 (&scur)[2], f32x16 (&snext)[2]) {
        stage(tile_of(min(jj + 3, ntiles - 1)), jj + 3);
        const lds_t* kb = kbuf + ((jj + 1) & (F64_NB - 1)) * KBUF;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          snext[0][i] = 0.f;
          snext[1][i] = 0.f;
        }
        s16x8 ka[NS];
#pragma unroll
        for (int ss = 0; ss < NS; ++ss) ka[ss] = lds_read16(kb + swz_off<D>(l32, 2 * ss + hh));
        unsigned int dw[2][4];
        if constexpr (DROP) {
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
            drop_words_row4(s.seed0, s.seed1, b * s.H + h, qw + 32 * rb + l32, tile_of(jj) * F64_BN + 4 * hh, 8,
                            dw[rb]);
        }
        unsigned int pk[2][8];
        float sum[2] = {0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 2 * NS; ++t) {
          __builtin_amdgcn_sched_barrier(0);
          const int rb = t & 1, ss = t >> 1;
          snext[rb] = mfma32<T>(ka[ss], qf[rb][ss], snext[rb]);
          const int e = 2 * t, rbe = e >> 4, i = e & 15;
          const float p0 = fast_exp2(fmaf(scur[rbe][i], c, -m[rbe]));
          const float p1 = fast_exp2(fmaf(scur[rbe][i + 1], c, -m[rbe]));
          sum[rbe] += p0 + p1;
          pk[rbe][i >> 1] = pack_p(p0, p1, i >> 1, dw[rbe]);
        }
        __builtin_amdgcn_sched_barrier(0);
        l[0] += sum[0];
        l[1] += sum[1];
        write_p(hand(jj & 1), pk);
        dma_wait_prev();
        __syncthreads();
      };
      // the reference: the first tile's row maximum
      f32x16 sa[2], sb[2];
      s_tile(0, sa);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        float x = sa[rb][0];
#pragma unroll
        for (int i = 1; i < 16; ++i) x = fmaxf(x, sa[rb][i]);
        m[rb] = fmaxf(x, swap_halves(x)) * c;
      }
      for (; j + 1 < nfull; j += 2) {
        iter(j, sa, sb);
        iter(j + 1, sb, sa);
      }
      if (j < nfull) {
        iter(j, sa, sb);
        ++j;
      }
      // workgroup-wide vote (the consumers vote no): start over in the general loop
      dma_wait();
      if (__syncthreads_or(l[0] > lmax || l[1] > lmax)) {
        j = 0;
        m[0] = m[1] = -INFINITY;
        l[0] = l[1] = 0.f;
        stage(tile_of(0), 0);
        stage(tile_of(max(0, min(1, ntiles - 1))), 1);
        stage(tile_of(max(0, min(2, ntiles - 1))), 2);
        dma_wait();
        __syncthreads();
      }
    }
    // general loop: element masks, lazy rescaling; a pair whose rows see no key of the tile skips it
    for (; j < ntiles; ++j) {
      stage(tile_of(min(j + 3, ntiles - 1)), j + 3);
      const int ks = tile_of(j) * F64_BN;
      lds_t* hb = hand(j & 1);
      const bool act = (!BAND || ks <= qw + F64_RW - 1 + offu) && (!LOWER || ks + F64_BN - 1 >= qw + offl);
      bool resc = false;
      if (act) {
        f32x16 st[2];
        s_tile(j & (F64_NB - 1), st);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const int qi = qw + 32 * rb + l32;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = ks + 8 * (i >> 2) + 4 * hh + (i & 3);
            if ((BAND && key > qi + offu) || (LOWER && key < qi + offl) || key >= nk) st[rb][i] = -INFINITY;
          }
        }
        float mx[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          float x = st[rb][0];
#pragma unroll
          for (int i = 1; i < 16; ++i) x = fmaxf(x, st[rb][i]);
          mx[rb] = fmaxf(x, swap_halves(x)) * c;
        }
        resc = __any(mx[0] > m[0] + kSlack || mx[1] > m[1] + kSlack);
        unsigned int pk[2][8];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const float mn = resc ? fmaxf(m[rb], mx[rb]) : m[rb];
          const float mu = mn == -INFINITY ? 0.f : mn;
          float sum = 0.f;
          unsigned int dw[4];
          if constexpr (DROP) drop_words_row4(s.seed0, s.seed1, b * s.H + h, qw + 32 * rb + l32, ks + 4 * hh, 8, dw);
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) {
            const float p0 = fast_exp2(fmaf(st[rb][2 * jj], c, -mu));
            const float p1 = fast_exp2(fmaf(st[rb][2 * jj + 1], c, -mu));
            sum += p0 + p1;
            pk[rb][jj] = pack_p(p0, p1, jj, dw);
          }
          if (resc) {
            const float corr = fast_exp2(m[rb] - mu);
            l[rb] *= corr;
            if (hh == 0) *(__attribute__((address_space(3))) float*)(hb + 4096 + (32 * rb + l32) * 4) = corr;
          }
          l[rb] += sum;
          m[rb] = mn;
        }
        write_p(hb, pk);
      }
      if (lane == 0) *(__attribute__((address_space(3))) int*)(hb + 4096 + 256) = (act ? 1 : 0) | (resc ? 2 : 0);
      dma_wait_prev();
      __syncthreads();
    }
    dma_wait();
    // 1 / l per row for the consumer; the log-sum-exp from here
    const rsrc_t rl = make_rsrc(a.lse + qrow0, (unsigned)nq * 4u);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int qi = qw + 32 * rb + l32;
      const float lt = l[rb] + swap_halves(l[rb]);
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      const float lse = lt > 0.f ? (m[rb] + fast_log2(lt)) * kLn2 : -INFINITY;
      if (hh == 0) {
        *(__attribute__((address_space(3))) float*)(ibuf + pw * 256 + (32 * rb + l32) * 4) = inv;
        bstore_f32(rl, (unsigned)qi * 4u, lse);
      }
    }
    __syncthreads();
  } else {
    f32x16 acc[2][ND];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[rb][dt][i] = 0.f;
    // O^T += V^T P^T of the tile in a slot with P from a hand-over buffer
    auto pv = [&](int slot, const lds_t* hb) {
      s16x8 pop[2][2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int u = 0; u < 2; ++u) pop[rb][u] = lds_read16(hb + (2 * rb + u) * 1024 + lane * 16);
      const lds_t* vb = vbuf + slot * VBUF;  // slot: tile index modulo 8
#pragma unroll
      for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int cc = 4 * dt + (coff >> 3), within = 2 * (coff & 7);
          const s16x8 va = concat(lds_read_tr(vb + swz_off<D>(16 * u + roff, cc) + within),
                                  lds_read_tr(vb + swz_off<D>(16 * u + roff + 8, cc) + within));
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) acc[rb][dt] = mfma32<T>(va, pop[rb][u], acc[rb][dt]);
        }
    };
    // a general-loop tile: its flags, the rescale when the reference rose, then P V
    auto consume = [&](int t) {
      const lds_t* hb = hand(t & 1);
      const int fl = __builtin_amdgcn_readfirstlane(*(const __attribute__((address_space(3))) int*)(hb + 4096 + 256));
      if (fl & 1) {
        if (fl & 2) {
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            const float corr = *(const __attribute__((address_space(3))) float*)(hb + 4096 + (32 * rb + l32) * 4);
#pragma unroll
            for (int dt = 0; dt < ND; ++dt)
#pragma unroll
              for (int i = 0; i < 16; ++i) acc[rb][dt][i] *= corr;
          }
        }
        pv(t & (VNB - 1), hb);
      }
    };
    if (nfull > 0) {
      // main loop: iteration j takes P V of tile j - 1 (fixed reference: no rescale)
      for (; j < nfull; ++j) {
        if (j > 0) pv((j - 1) & (VNB - 1), hand((j - 1) & 1));
        __syncthreads();
      }
      pv((nfull - 1) & (VNB - 1), hand((nfull - 1) & 1));
      if (__syncthreads_or(0)) {
        j = 0;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int dt = 0; dt < ND; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[rb][dt][i] = 0.f;
        __syncthreads();
      }
    }
    // general loop: iteration j takes tile j - 1, the last tile follows the last barrier
    const int j0 = j;
    for (; j < ntiles; ++j) {
      if (j > j0) consume(j - 1);
      __syncthreads();
    }
    if (ntiles > j0) consume(ntiles - 1);
    __syncthreads();
    const rsrc_t ro = make_rsrc((unsigned short*)a.o + qrow0 * D, qbytes);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int qi = qw + 32 * rb + l32;
      const float inv = *(const __attribute__((address_space(3))) float*)(ibuf + pw * 256 + (32 * rb + l32) * 4);
#pragma unroll
      for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          u32x2 v2 = {pack2<T>(acc[rb][dt][4 * jj] * inv, acc[rb][dt][4 * jj + 1] * inv),
                      pack2<T>(acc[rb][dt][4 * jj + 2] * inv, acc[rb][dt][4 * jj + 3] * inv)};
          bstore8(ro, (unsigned)(qi * D + 32 * dt + 8 * jj + 4 * hh) * 2u, v2);
        }
    }
  }
}

template <class T, int D, int BAND, bool DROP>
__global__ __launch_bounds__((f64_split<D, BAND, DROP>() ? 2 * F64_NW * 64 : F64_NW * 64), 1)
    void fwd64_kernel(FwdArgs a) {
  if constexpr (f64_split<D, BAND, DROP>()) {
    fwd64_split_body<T, D, BAND, DROP>(a);
    return;
  } else {
    constexpr int KP = D * 2 + 16;  // K row pitch (bytes): conflict-free 16-byte row reads
    constexpr int VP = D * 2 + 32;  // V row pitch (bytes): conflict-free transposing reads
    constexpr int KBUF = F64_BN * KP;
    constexpr int VBUF = F64_BN * VP;
    constexpr int NT = F64_NW * 64;
    constexpr int CH = D / 8;
    constexpr int TCH = F64_BN * CH;            // 16-byte chunks per tile per tensor
    constexpr int PER = (TCH + NT - 1) / NT;
    static_assert(TCH % NT == 0 || TCH < NT, "tile loader shape");
    constexpr int NS = D / 16;
    constexpr int ND = D / 32;
    constexpr float kSlack = (std::is_same<T, F16>::value && DROP) ? 7.f : 8.f;  // as in fwd_kernel

    __shared__ __attribute__((aligned(16))) char smem_raw[F64_NB * (KBUF + VBUF)];
    lds_t* kbuf = (lds_t*)smem_raw;
    lds_t* vbuf = kbuf + F64_NB * KBUF;

    const AttnShape& s = a.s;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    const int g16 = lane >> 4;
    const int roff = 4 * (g16 >> 1) + ((lane & 15) >> 2);
    const int coff = 16 * (g16 & 1) + 4 * (lane & 3);
    // grid (tile_grid): heads fastest; under a band mask the later (under causal
    // masking, longer) query blocks are dispatched first
    const GridPos gp = grid_pos(s);
    const int qb = BAND ? gp.nblk - 1 - gp.blk : gp.blk;
    const int h = query_head(s, blockIdx.x), b = gp.b;
    const int hk = h / s.G;
    const SeqView sv = seq_view(s, b, h, hk);
    const int nq = sv.nq, nk = sv.nk, off = sv.off;
    const int q0 = qb * F64_BM;
    if (q0 >= nq) return;  // a sequence shorter than the grid (packed batches)
    const size_t qrow0 = sv.qrow0, krow0 = sv.krow0;
    const unsigned int qbytes = (unsigned int)nq * D * 2, kbytes = (unsigned int)nk * D * 2;
    const rsrc_t rq = make_rsrc((const unsigned short*)a.q + qrow0 * D, qbytes);
    const rsrc_t rk = make_rsrc((const unsigned short*)a.k + krow0 * D, kbytes);
    const rsrc_t rv = make_rsrc((const unsigned short*)a.v + krow0 * D, kbytes);
    const int qw = q0 + F64_RW * w;  // first query row of this wave; block rb holds rows qw + 32 rb + 0..31
    const float c = fmaxf(s.scale * kLog2e, 1e-30f);

    // tiles [tbeg, tbeg + ntiles) hold every key some row of the workgroup sees
    // (row q0's band starts lowest, the last row's ends highest); tiles
    // [fbeg, fend) hold only keys that every row sees (the last row's band starts
    // highest, row q0's ends lowest)
    // (band: row i sees keys i + offl .. i + offu; offl binds only with a lower edge)
    constexpr bool LOWER = BAND == 2;
    const int offu = off + s.wr, offl = off - s.wl;
    const int kbeg = LOWER ? max(0, q0 + offl) : 0;
    const int kend = BAND ? min(nk, max(0, q0 + F64_BM + offu)) : nk;
    const int tbeg = kbeg / F64_BN;
    const int ntiles = max(0, (kend + F64_BN - 1) / F64_BN - tbeg);
    // (clamped to the tile range: padding rows past the sequence can put the
    // last row's band start beyond the last key)
    const int fbeg =
        LOWER ? min(tbeg + ntiles, max(tbeg, (max(0, q0 + F64_BM - 1 + offl) + F64_BN - 1) / F64_BN)) : 0;
    const int fend = BAND ? max(fbeg, min(max(0, q0 + offu + 1) / F64_BN, nk / F64_BN)) : nk / F64_BN;
    const int nfull = fend - fbeg;
    // processing order e = 0, 1, ...: the full tiles, then the partial tiles
    // above them (together the run fbeg, fbeg + 1, ...), then those below (the
    // result does not depend on the order); without a lower edge the order is
    // simply the tile index
    const int nhead = tbeg + ntiles - fbeg;
    auto tile_of = [&](int e) -> int {
      if constexpr (LOWER) return e < nhead ? fbeg + e : tbeg + (e - nhead);
      else return e;
    };

    // Q^T operands of both row blocks: lane holds query qw + 32 rb + l32, d = 16 ss + 8 hh + 0..7
    s16x8 qf[2][NS];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int ss = 0; ss < NS; ++ss)
        qf[rb][ss] = bload16(rq, (unsigned)((qw + 32 * rb + l32) * D + 16 * ss + 8 * hh) * 2u);

    f32x16 acc[2][ND];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[rb][dt][i] = 0.f;
    // running reference m (log2 units) and this lane's half of the running sum,
    // per row block, raised lazily as in the 32-row kernel
    float m[2] = {-INFINITY, -INFINITY};
    float l[2] = {0.f, 0.f};

    s16x8 kreg[PER], vreg[PER];
    auto gload = [&](int t) {
#pragma unroll
      for (int r = 0; r < PER; ++r) {
        const int ci = min(tid + r * NT, TCH - 1);  // spare threads repeat the last chunk
        const int row = ci / CH, col = (ci % CH) * 8;
        const unsigned int off = (unsigned)((t * F64_BN + row) * D + col) * 2u;
        kreg[r] = bload16(rk, off);
        vreg[r] = bload16(rv, off);
      }
    };
    auto lstore = [&](int slot) {
#pragma unroll
      for (int r = 0; r < PER; ++r) {
        const int ci = min(tid + r * NT, TCH - 1);
        const int row = ci / CH, col = (ci % CH) * 8;
        lds_write16(kbuf + slot * KBUF + row * KP + col * 2, kreg[r]);
        lds_write16(vbuf + slot * VBUF + row * VP + col * 2, vreg[r]);
      }
    };
    // S^T = K Q^T of the tile in a slot; st[rb][i] is S of query qw + 32 rb + l32
    // and key 8 (i / 4) + 4 hh + i % 4 of the tile
    auto s_tile = [&](int slot, f32x16 (&st)[2]) {
      const lds_t* kb = kbuf + slot * KBUF + l32 * KP + 16 * hh;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        st[0][i] = 0.f;
        st[1][i] = 0.f;
      }
#pragma unroll
      for (int ss = 0; ss < NS; ++ss) {
        const s16x8 ka = lds_read16(kb + 32 * ss);
        st[0] = mfma32<T>(ka, qf[0][ss], st[0]);
        st[1] = mfma32<T>(ka, qf[1][ss], st[1]);
      }
    };
    // O^T += V^T P^T for the tile in a slot; B operand k-slot j of step u is key
    // 16 u + 8 (j / 4) + 4 hh + j % 4, matched by the transposing reads of V
    auto pv_tile = [&](int slot, const unsigned int (&pk)[2][8]) {
      const lds_t* vb = vbuf + slot * VBUF;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const lds_t* vp = vb + (16 * u + roff) * VP + (32 * dt + coff) * 2;
          const s16x8 va = concat(lds_read_tr(vp), lds_read_tr(vp + 8 * VP));
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
            acc[rb][dt] = mfma32<T>(va, as_operand(pk[rb][4 * u], pk[rb][4 * u + 1], pk[rb][4 * u + 2],
                                                   pk[rb][4 * u + 3]),
                                    acc[rb][dt]);
        }
    };
    // Softmax of one tile against the running reference: returns whether the
    // reference rises (wave-uniform), with the new reference in mn, the 16-bit
    // probabilities in pk and this lane's share of their row sums in ls.
    // 16-bit probabilities of elements 2 jj, 2 jj + 1 of row block rb, with dropout
    // when built for it (keys ks + 8 (jj / 2) + 4 hh + (2 jj & 3) + 0, 1)
    // (dw: this row's dropout words for key groups ks + 8 g + 4 hh, g = 0..3,
    // from drop_words_row4)
    auto pack_p = [&](float p0, float p1, int jj, const unsigned int (&dw)[4]) -> unsigned int {
      if constexpr (DROP) {
        const unsigned int wd = dw[jj >> 1];
        const int t0 = (2 * jj) & 3;
        return pack2<T>(drop_keep(wd, t0, s.drop_t) ? p0 * s.drop_scale : 0.f,
                        drop_keep(wd, t0 + 1, s.drop_t) ? p1 * s.drop_scale : 0.f);
      } else {
        return pack2<T>(p0, p1);
      }
    };
    auto softmax = [&](const f32x16 (&st)[2], float (&mn)[2], unsigned int (&pk)[2][8], float (&ls)[2], int ks) {
      float mx[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        float x = st[rb][0];
#pragma unroll
        for (int i = 1; i < 16; ++i) x = fmaxf(x, st[rb][i]);
        mx[rb] = fmaxf(x, swap_halves(x)) * c;
      }
      const bool resc = __any(mx[0] > m[0] + kSlack || mx[1] > m[1] + kSlack);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        mn[rb] = resc ? fmaxf(m[rb], mx[rb]) : m[rb];
        const float mu = mn[rb] == -INFINITY ? 0.f : mn[rb];  // a row with no visible key yet
        float sum = 0.f;
        unsigned int dw[4];
        if constexpr (DROP) drop_words_row4(s.seed0, s.seed1, b * s.H + h, qw + 32 * rb + l32, ks + 4 * hh, 8, dw);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float p0 = fast_exp2(fmaf(st[rb][2 * j], c, -mu));
          const float p1 = fast_exp2(fmaf(st[rb][2 * j + 1], c, -mu));
          sum += p0 + p1;
          pk[rb][j] = pack_p(p0, p1, j, dw);
        }
        ls[rb] = sum;
      }
      return resc;
    };
    // fold a tile's statistics into the running ones; when the reference rose,
    // scale the output and the sum by exp(m_old - m_new) first
    auto update = [&](bool resc, const float (&mn)[2], const float (&ls)[2]) {
      if (resc) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const float corr = fast_exp2(m[rb] - (mn[rb] == -INFINITY ? 0.f : mn[rb]));
          l[rb] *= corr;
#pragma unroll
          for (int dt = 0; dt < ND; ++dt) scale_acc(acc[rb][dt], corr);
        }
      }
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        l[rb] += ls[rb];
        m[rb] = mn[rb];
      }
    };

    // Prologue: tiles 0 and 1 in slots 0 and 1; the V half of slot 3 is zeroed
    // because the first iteration multiplies it with zero probabilities.
    for (int i = tid; i < VBUF / 16; i += NT)
      lds_write16(vbuf + (F64_NB - 1) * VBUF + i * 16, (s16x8){0, 0, 0, 0, 0, 0, 0, 0});
    gload(tile_of(0));
    lstore(0);
    gload(tile_of(max(0, min(1, ntiles - 1))));
    lstore(1);
    __syncthreads();

    // Main loop over the tiles that every row sees in full. The reference m is
    // fixed at the first tile's row maximum, so the loop never rescales and has
    // no branch: probabilities relative to that reference stay finite while no
    // later score exceeds it by more than about 120 in log2 units, and the result
    // O / l, m + log2(l) does not depend on the reference chosen. Should a row's
    // sum end above 2^60 (some later score at least 60 above the first tile's
    // maximum), the whole workgroup starts over in the general loop below, which
    // raises the reference as it goes. With float16 the 16-bit probabilities
    // have the tighter bound: the restart comes once a row sum exceeds 65504
    // divided by the dropout keep scale, which every probability (so scaled)
    // beyond float16's range implies, since the sum holds each probability.
    int j = 0;
    if (nfull > 0) {
      auto probs = [&](const f32x16 (&st)[2], unsigned int (&pk)[2][8], int ks) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          float sum = 0.f;
          unsigned int dw[4];
          if constexpr (DROP) drop_words_row4(s.seed0, s.seed1, b * s.H + h, qw + 32 * rb + l32, ks + 4 * hh, 8, dw);
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) {
            const float p0 = fast_exp2(fmaf(st[rb][2 * jj], c, -m[rb]));
            const float p1 = fast_exp2(fmaf(st[rb][2 * jj + 1], c, -m[rb]));
            sum += p0 + p1;
            pk[rb][jj] = pack_p(p0, p1, jj, dw);
          }
          l[rb] += sum;
        }
      };
      // one iteration: S of tile jj + 1, probabilities of tile jj, P V of tile
      // jj - 1 (mutually independent), then tile jj + 2 into the slot of tile
      // jj - 2. Loads are issued on every path (tile index clamped; a redundant
      // copy lands in a slot nobody reads). Without dropout the iteration is laid
      // out in slots of one MFMA each, products of S and of P V alternating, with
      // the probabilities of the current tile spread over the slots (one element,
      // or a few at small head sizes, per slot) and the K and V^T fragments read
      // two fragment groups ahead; scheduling fences keep that order, which the
      // compiler's own schedule (MFMAs in runs, the exponentials and sums bunched
      // between them) ran 4% slower at N = 16384, d = 128.
      auto iter = [&](int jj, const f32x16 (&scur)[2], f32x16 (&snext)[2], const unsigned int (&pprev)[2][8],
                      unsigned int (&pcur)[2][8]) {
        gload(tile_of(min(jj + 2, ntiles - 1)));
        if constexpr (DROP) {
          s_tile((jj + 1) & (F64_NB - 1), snext);
          probs(scur, pcur, (fbeg + jj) * F64_BN);
          pv_tile((jj + F64_NB - 1) & (F64_NB - 1), pprev);
        } else {
          const lds_t* kb = kbuf + ((jj + 1) & (F64_NB - 1)) * KBUF + l32 * KP + 16 * hh;
          const lds_t* vb = vbuf + ((jj + F64_NB - 1) & (F64_NB - 1)) * VBUF;
          auto vread = [&](int g) {
            const lds_t* vp = vb + (16 * (g & 1) + roff) * VP + (32 * (g >> 1) + coff) * 2;
            return concat(lds_read_tr(vp), lds_read_tr(vp + 8 * VP));
          };
          constexpr int NG = NS;          // fragment groups: K fragment g and V^T fragment g
          constexpr int NSLOT = 4 * NG;   // MFMAs: 2 NS products of S, 4 ND = 2 NS of P V
          constexpr int EPS = 32 / NSLOT; // softmax elements per slot
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            snext[0][i] = 0.f;
            snext[1][i] = 0.f;
          }
          s16x8 ka[NG], va[NG];
          ka[0] = lds_read16(kb);
          va[0] = vread(0);
          if constexpr (NG > 1) {
            ka[1] = lds_read16(kb + 32);
            va[1] = vread(1);
          }
          float sum[2] = {0.f, 0.f};
          float pe = 0.f;
#pragma unroll
          for (int t = 0; t < NSLOT; ++t) {
            __builtin_amdgcn_sched_barrier(0);
            const int g = t >> 2;
            if ((t & 3) == 0 && g + 2 < NG) {
              ka[g + 2] = lds_read16(kb + 32 * (g + 2));
              va[g + 2] = vread(g + 2);
            }
            if ((t & 1) == 0) {
              const int n = t >> 1, rb = n & 1;
              snext[rb] = mfma32<T>(ka[n >> 1], qf[rb][n >> 1], snext[rb]);
            } else {
              const int n = t >> 1, rb = n & 1, pg = n >> 1, u = pg & 1;
              acc[rb][pg >> 1] = mfma32<T>(va[pg], as_operand(pprev[rb][4 * u], pprev[rb][4 * u + 1],
                                                              pprev[rb][4 * u + 2], pprev[rb][4 * u + 3]),
                                           acc[rb][pg >> 1]);
            }
#pragma unroll
            for (int x = 0; x < EPS; ++x) {
              const int e = t * EPS + x, rb = e >> 4, i = e & 15;
              const float p = fast_exp2(fmaf(scur[rb][i], c, -m[rb]));
              if (i & 1) {
                sum[rb] += pe + p;
                pcur[rb][i >> 1] = pack2<T>(pe, p);
              } else {
                pe = p;
              }
            }
          }
          __builtin_amdgcn_sched_barrier(0);
          l[0] += sum[0];
          l[1] += sum[1];
        }
        lstore((jj + 2) & (F64_NB - 1));
        __syncthreads();
      };
      f32x16 sa[2], sb[2];
      unsigned int pa[2][8], pb[2][8];
      s_tile(0, sa);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        float x = sa[rb][0];
#pragma unroll
        for (int i = 1; i < 16; ++i) x = fmaxf(x, sa[rb][i]);
        m[rb] = fmaxf(x, swap_halves(x)) * c;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) pb[rb][jj] = 0u;
      }
      for (; j + 1 < nfull; j += 2) {
        iter(j, sa, sb, pb, pa);
        iter(j + 1, sb, sa, pa, pb);
      }
      if (j < nfull) {
        iter(j, sa, sb, pb, pa);
        pv_tile(j & (F64_NB - 1), pa);
        ++j;
      } else {
        pv_tile((nfull - 1) & (F64_NB - 1), pb);
      }
      // workgroup-uniform decision (it also orders the reads above before any
      // slot is refilled)
      const float lmax = std::is_same<T, F16>::value ? 65504.f / (DROP ? s.drop_scale : 1.f) : 0x1p60f;
      if (__syncthreads_or(l[0] > lmax || l[1] > lmax)) {
        j = 0;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          m[rb] = -INFINITY;
          l[rb] = 0.f;
#pragma unroll
          for (int dt = 0; dt < ND; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[rb][dt][i] = 0.f;
        }
        gload(tile_of(0));
        lstore(0);
        gload(tile_of(max(0, min(1, ntiles - 1))));
        lstore(1);
        __syncthreads();
      }
    }

    // general loop (diagonal and ragged tiles, or a restart): element masks,
    // lazy rescaling, waves without a visible key skip the tile
    for (; j < ntiles; ++j) {
      gload(tile_of(min(j + 2, ntiles - 1)));
      const int ks = tile_of(j) * F64_BN;
      if ((!BAND || ks <= qw + F64_RW - 1 + offu) && (!LOWER || ks + F64_BN - 1 >= qw + offl)) {
        f32x16 st[2];
        s_tile(j & (F64_NB - 1), st);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const int qi = qw + 32 * rb + l32;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = ks + 8 * (i >> 2) + 4 * hh + (i & 3);
            if ((BAND && key > qi + offu) || (LOWER && key < qi + offl) || key >= nk) st[rb][i] = -INFINITY;
          }
        }
        float mn[2], ls[2];
        unsigned int pt[2][8];
        const bool resc = softmax(st, mn, pt, ls, ks);
        update(resc, mn, ls);
        pv_tile(j & (F64_NB - 1), pt);
      }
      lstore((j + 2) & (F64_NB - 1));
      __syncthreads();
    }

    const rsrc_t ro = make_rsrc((unsigned short*)a.o + qrow0 * D, qbytes);
    const rsrc_t rl = make_rsrc(a.lse + qrow0, (unsigned)nq * 4u);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int qi = qw + 32 * rb + l32;
      const float lt = l[rb] + swap_halves(l[rb]);
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      const float lse = lt > 0.f ? (m[rb] + fast_log2(lt)) * kLn2 : -INFINITY;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          u32x2 v2 = {pack2<T>(acc[rb][dt][4 * j] * inv, acc[rb][dt][4 * j + 1] * inv),
                      pack2<T>(acc[rb][dt][4 * j + 2] * inv, acc[rb][dt][4 * j + 3] * inv)};
          bstore8(ro, (unsigned)(qi * D + 32 * dt + 8 * j + 4 * hh) * 2u, v2);
        }
      if (hh == 0) bstore_f32(rl, (unsigned)qi * 4u, lse);
    }
  }
}

// float32: fp32 FMA for every product. The float32 inputs are small (the
// worked example is one 512 x 32 head), so the kernel is built for latency:
// each query row is split over F32_S threads that run the online recurrence
// over interleaved 4-key chunks of the row's keys, each keeping its own
// (m, l, o); the partial states of a row are then merged through LDS with the
// same correction factors, m = max m_s, l = sum l_s exp(m_s - m),
// o = sum o_s exp(m_s - m), each thread of the row finishing D / F32_S
// output columns.
constexpr int F32_R = 8;    // query rows per workgroup (divides the 128-row mask block)
constexpr int F32_S = 16;   // threads (key splits) per row
constexpr int F32_C = 4;    // keys per chunk

template <int D>
__global__ __launch_bounds__(F32_R * F32_S) void fwd_f32_kernel(FwdArgs a) {
  __shared__ float part[F32_R][F32_S][D + 2];  // o[0..D), m, l of each split
  const AttnShape& s = a.s;
  const int tid = threadIdx.x;
  const int r = tid % F32_R, sp = tid / F32_R;  // a wave holds 8 splits of the 8 rows
  const int qb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int hk = h / s.G;
  const SeqView sv = seq_view(s, b, h, hk);
  const int nq = sv.nq, nk = sv.nk, off = sv.off;
  const int q0 = qb * F32_R;
  if (q0 >= nq) return;  // a sequence shorter than the grid (packed batches)
  const size_t qrow0 = sv.qrow0, krow0 = sv.krow0;
  const float* Q = (const float*)a.q + qrow0 * D;
  const float* K = (const float*)a.k + krow0 * D;
  const float* V = (const float*)a.v + krow0 * D;
  const int qi = q0 + r;
  const float c = fmaxf(s.scale * kLog2e, 1e-30f);
  const float nsl2 = s.alibi ? -s.alibi[h] * kLog2e : 0.f;  // ALiBi slope, log2 units
  // the bias is taken relative to the row's nearest key, max(0, -(qi + off))
  // away, and the LSE gets that shift back (fp32 scores stay small)
  const int dmin = s.alibi ? max(0, -(qi + off)) : 0;
  const int mrow = q0 / 128;  // every row of the workgroup is in this mask block row

  float q[D], o[D];
#pragma unroll
  for (int dd = 0; dd < D; ++dd) {
    q[dd] = qi < nq ? Q[(size_t)qi * D + dd] : 0.f;
    o[dd] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  // this row's band [kbeg_row, kend_row) and the workgroup's [kbeg, kend)
  const int kbeg_row = s.band ? max(0, qi + off - s.wl) : 0;
  const int kend_row = s.band ? min(nk, max(0, qi + 1 + off + s.wr)) : nk;
  const int kbeg = s.band ? max(0, q0 + off - s.wl) : 0;
  const int kend = s.band ? min(nk, max(0, q0 + F32_R + off + s.wr)) : nk;
  constexpr int STRIDE = F32_S * F32_C;
  for (int j0 = kbeg / STRIDE * STRIDE + sp * F32_C; j0 < kend; j0 += STRIDE) {
    float x[F32_C];
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < F32_C; ++t) {
      const int j = j0 + t;
      bool vis = j >= kbeg_row && j < kend_row && (!s.mask || s.mask[(size_t)mrow * s.nbk + j / 128] != 0);
      if (vis && s.mask && s.btile) {  // a partial block: the element's bit (tiles past the last read as 0)
        const int t = s.btile[(size_t)mrow * s.nbk + j / 128];
        if (t >= 0) vis = t < s.ntiles && ((s.bits[(size_t)t * 512 + (qi & 127) * 4 + ((j & 127) >> 5)] >> (j & 31)) & 1u);
      }
      float dot = 0.f;
      if (vis) {
        const float4* kr = (const float4*)(K + (size_t)j * D);
#pragma unroll
        for (int d4 = 0; d4 < D / 4; ++d4) {
          const float4 kv = kr[d4];
          dot = fmaf(q[4 * d4], kv.x, dot);
          dot = fmaf(q[4 * d4 + 1], kv.y, dot);
          dot = fmaf(q[4 * d4 + 2], kv.z, dot);
          dot = fmaf(q[4 * d4 + 3], kv.w, dot);
        }
      }
      x[t] = vis ? (s.alibi ? fmaf(dot, c, nsl2 * (float)(abs(qi + off - j) - dmin)) : dot * c) : -INFINITY;
      mx = fmaxf(mx, x[t]);
    }
    if (mx == -INFINITY) continue;  // nothing visible in this chunk for this row
    if (mx > m) {
      const float corr = fast_exp2(m - mx);  // 0 while m is still -inf
      l *= corr;
#pragma unroll
      for (int dd = 0; dd < D; ++dd) o[dd] *= corr;
      m = mx;
    }
#pragma unroll
    for (int t = 0; t < F32_C; ++t) {
      const float p = fast_exp2(x[t] - m);  // 0 for hidden keys
      if (p == 0.f) continue;
      l += p;
      const float4* vr = (const float4*)(V + (size_t)(j0 + t) * D);
#pragma unroll
      for (int d4 = 0; d4 < D / 4; ++d4) {
        const float4 vv = vr[d4];
        o[4 * d4] = fmaf(p, vv.x, o[4 * d4]);
        o[4 * d4 + 1] = fmaf(p, vv.y, o[4 * d4 + 1]);
        o[4 * d4 + 2] = fmaf(p, vv.z, o[4 * d4 + 2]);
        o[4 * d4 + 3] = fmaf(p, vv.w, o[4 * d4 + 3]);
      }
    }
  }

  // merge the F32_S partial states of each row
#pragma unroll
  for (int dd = 0; dd < D; ++dd) part[r][sp][dd] = o[dd];
  part[r][sp][D] = m;
  part[r][sp][D + 1] = l;
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int t = 0; t < F32_S; ++t) M = fmaxf(M, part[r][t][D]);
  const float Mu = M == -INFINITY ? 0.f : M;
  float wgt[F32_S];
  float L = 0.f;
#pragma unroll
  for (int t = 0; t < F32_S; ++t) {
    wgt[t] = fast_exp2(part[r][t][D] - Mu);  // 0 for a split that saw no key
    L = fmaf(part[r][t][D + 1], wgt[t], L);
  }
  if (qi < nq) {
    const float inv = L > 0.f ? 1.f / L : 0.f;
    constexpr int DS = D / F32_S;  // output columns finished by each split
    float* Op = (float*)a.o + (qrow0 + qi) * D + sp * DS;
#pragma unroll
    for (int dd = 0; dd < DS; ++dd) {
      float acc = 0.f;
#pragma unroll
      for (int t = 0; t < F32_S; ++t) acc = fmaf(part[r][t][sp * DS + dd], wgt[t], acc);
      Op[dd] = acc * inv;
    }
    if (sp == 0) {
      const float lse = L > 0.f ? (M + fast_log2(L)) * kLn2 : -INFINITY;
      a.lse[qrow0 + qi] = s.alibi ? fmaf(-s.alibi[h], (float)dmin, lse) : lse;
    }
  }
}

template <class T, int D, int BAND, bool DROP>
static hipError_t launch_fwd_t3(const FwdArgs& a, hipStream_t st, bool mask, bool use64) {
  const bool alibi = a.s.alibi != nullptr;
  if (use64) {  // the caller has checked: no block mask, no score bias
    FwdArgs la = a;
    const dim3 grid = tile_grid(la.s, a.s.H, (a.s.Nq + F64_BM - 1) / F64_BM);
    const dim3 block(f64_split<D, BAND, DROP>() ? 2 * F64_NW * 64 : F64_NW * 64);  // split roles: eight waves
    hipLaunchKernelGGL((fwd64_kernel<T, D, BAND, DROP>), grid, block, 0, st, la);
    return hipGetLastError();
  }
  FwdArgs la = a;
  const dim3 grid = tile_grid(la.s, a.s.H, (a.s.Nq + FWD_BM - 1) / FWD_BM);
  const dim3 block(FWD_NW * 64);
  if (alibi) {
    if (mask) hipLaunchKernelGGL((fwd_kernel<T, D, BAND, true, DROP, true>), grid, block, 0, st, la);
    else hipLaunchKernelGGL((fwd_kernel<T, D, BAND, false, DROP, true>), grid, block, 0, st, la);
  } else {
    if (mask) hipLaunchKernelGGL((fwd_kernel<T, D, BAND, true, DROP, false>), grid, block, 0, st, la);
    else hipLaunchKernelGGL((fwd_kernel<T, D, BAND, false, DROP, false>), grid, block, 0, st, la);
  }
  return hipGetLastError();
}

template <class T, int D, bool DROP>
static hipError_t launch_fwd_t2(const FwdArgs& a, hipStream_t st, int band, bool mask, bool use64) {
  if (band == 2) return launch_fwd_t3<T, D, 2, DROP>(a, st, mask, use64);
  if (band == 1) return launch_fwd_t3<T, D, 1, DROP>(a, st, mask, use64);
  return launch_fwd_t3<T, D, 0, DROP>(a, st, mask, use64);
}

template <class T, int D>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t st, int rows) {
  const int band = a.s.band;
  const bool mask = a.s.mask != nullptr;
  const bool use64 = rows == 64;
  if (use64 && (mask || a.s.alibi)) return hipErrorInvalidValue;  // the 64-row kernel has neither
  if (a.s.drop_t > 0) return launch_fwd_t2<T, D, true>(a, st, band, mask, use64);
  return launch_fwd_t2<T, D, false>(a, st, band, mask, use64);
}

template <int D>
static hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t st) {
  const dim3 grid((a.s.Nq + F32_R - 1) / F32_R, a.s.H, a.s.B);
  hipLaunchKernelGGL((fwd_f32_kernel<D>), grid, dim3(F32_R * F32_S), 0, st, a);
  return hipGetLastError();
}

// Which 16-bit kernel a forward call takes by default. At head size 128 the
// 64-row kernel (in its split-role form) needs a grid of at least one
// 256-row workgroup per CU to pay off: with fewer, the 32-row kernel's twice
// as many workgroups fill more of the chip (measured, bf16, one box, forward
// time 64-row / 32-row: causal N = 16384 with 2 heads 1.08, 4 heads 0.97, 16
// heads 0.87; N = 8192 with 4 heads 1.08, 8 heads 1.00, 16 heads 0.85;
// without a band N = 2048 with 16 heads 1.17, N = 4096 with 8 heads 1.16, 16
// heads 0.97). Given that grid, it pays off from 4096 keys per row with a
// band (causal or windowed) and from 1024 without, and at shorter rows only
// once the grid holds about eight workgroups per CU (without a band N = 768
// with 1024 heads 0.82, N = 512 with 1024 heads 0.95 but with 256 heads 1.07;
// causal N = 2048 with 1024 heads 0.84, N = 3072 with 256 heads 0.90 but with
// 64 heads 1.04). At head size 64 the exponentials dominate and the 32-row
// kernel's two waves per SIMD do better (N = 16384: 6% faster). Block masks
// and score biases always take the 32-row kernel. Float32 inputs take the
// float32 kernel (0).
int forward_rows(const AttnShape& s, int dtype) {
  if (dtype == 0) return 0;
  if (s.mask || s.alibi || s.d != 128) return 32;
  const long long grid = (long long)s.B * s.H * ((s.Nq + F64_BM - 1) / F64_BM);  // 64-row workgroups
  const int len = min(s.Nq, s.Nk);
  return (grid >= 256 && (len >= (s.band ? 4096 : 1024) || grid >= 2048)) ? 64 : 32;
}

hipError_t launch_forward(const FwdArgs& a, int dtype, hipStream_t st, int rows) {
  const int d = a.s.d;
  if (dtype == 0) {
    if (d == 32) return launch_fwd_f32<32>(a, st);
    if (d == 64) return launch_fwd_f32<64>(a, st);
    return launch_fwd_f32<128>(a, st);
  }
  if (rows == 0) rows = forward_rows(a.s, dtype);
  if (dtype == 2) {
    if (d == 32) return launch_fwd_t<BF16, 32>(a, st, rows);
    if (d == 64) return launch_fwd_t<BF16, 64>(a, st, rows);
    return launch_fwd_t<BF16, 128>(a, st, rows);
  }
  if (d == 32) return launch_fwd_t<F16, 32>(a, st, rows);
  if (d == 64) return launch_fwd_t<F16, 64>(a, st, rows);
  return launch_fwd_t<F16, 128>(a, st, rows);
}

}  // namespace fa
