// Backward pass of IO-aware exact attention on gfx950.
//
// The probabilities are never read back from memory: they are recomputed tile
// by tile as P = exp(S - LSE) from Q, K and the saved per-row log-sum-exp
// (nadeemcite.github.io summary "FlashAttention: Fast and Memory-Efficient
// Exact Attention with IO-Awareness", Core Idea item 3; the pranaymahendrakar.com
// lesson "FlashAttention", Researcher tier, "IO complexity"). The gradient
// formulas are the chain rule through the row softmax (not on the pages):
//   dV_j = sum_i P_ij dO_i          dP_ij = dO_i . V_j
//   D_i  = sum_d dO_id O_id         dS_ij = P_ij (dP_ij - D_i)
//   dK_j = scale sum_i dS_ij Q_i    dQ_i  = scale sum_j dS_ij K_j
// (dS is kept unscaled; dK and dQ take the scale once, at their final rounding)
//
// Three stages on the caller's stream, none with atomics (dq, dk and dv are
// each written once, so the backward pass is bitwise reproducible):
//  0. D per query row, in fp32;
//  1. key-block kernel (dK, dV): one workgroup per 128 keys of one (batch, kv
//     head), four waves of 32 keys. K^T and V^T stay in registers as MFMA
//     operands and dK^T, dV^T accumulate in registers across every 32-row
//     query block (and every query head of a grouped-query group). The
//     32x32 result layout of S = Q K^T is already the B operand of dV^T =
//     dO^T P and dK^T = Q^T dS; dO^T and Q^T come from LDS through the gfx950
//     transposing read. The step loop is software-pipelined three deep: one
//     iteration issues S and dP of the next query block, P and dS of this
//     block and dV, dK of the previous block, which do not depend on each
//     other, so the MFMAs overlap the softmax arithmetic within one wave.
//     At d = 128 without block mask the same grid runs eight waves per
//     workgroup in two roles instead:
//     producers form S, dP, P and dS; consumers accumulate dV and dK
//     (bwd_kv_split_body).
//  2. query-block kernel (dQ): one workgroup per 128 query rows, four waves of
//     32 rows, laid out like the forward pass: S^T = K Q^T and dP^T = V dO^T
//     with Q^T and dO^T in registers, so a lane owns one query row and its LSE
//     and D are two scalars; dQ^T += K^T dS^T with K^T read transposed from LDS.
// Recomputing S and dP in stage 2 costs two more contractions than scattering
// dQ from stage 1, but a scatter needs floating-point atomics, which on this
// chip are executed past the L2 and cost more than the contractions they save.
// Causal masking trims both kernels to their diagonal; block sparsity
// compacts the nonzero blocks of the mask column (stage 1) or row (stage 2).
#include <type_traits>

#include "common.hpp"
#include "params.hpp"

namespace fa {


// ---------------------------------------------------------------------------
// stage 0: per query row, D = rowsum(dO * O) in fp32 and the log2-scaled LSE,
// into the workspace's two planes (padding rows past the sequence up to npad
// included). The plane holds -D: the key-block kernel starts its dP
// accumulators at it, so that dP - D comes straight out of the MFMA.
// ---------------------------------------------------------------------------
template <class T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdArgs a) {
  constexpr int CH = D / 8;  // lanes per row, 8 elements each
  constexpr int RPB = 256 / CH;
  const int tid = threadIdx.x;
  const int nblk = (a.npad + RPB - 1) / RPB;  // blocks per (b, h) head
  const int bh = blockIdx.x / nblk;
  const int r = (blockIdx.x % nblk) * RPB + tid / CH;  // row within the sequence
  const int part = tid % CH;
  const int h = bh % a.s.H;
  const SeqView sv = seq_view(a.s, bh / a.s.H, h, h / a.s.G);
  const int nq = sv.nq;
  float sum = 0.f;
  if (r < nq) {
    const size_t off = (sv.qrow0 + r) * D + part * 8;
    const s16x8 o = gload16((const unsigned short*)a.o + off);
    const s16x8 g = gload16((const unsigned short*)a.dO + off);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      sum = fmaf(to_f32<T>((unsigned short)o[j]), to_f32<T>((unsigned short)g[j]), sum);
  }
#pragma unroll
  for (int msk = CH / 2; msk >= 1; msk >>= 1) sum += __shfl_xor(sum, msk, 64);
  if (r < a.npad && part == 0) {
    // a row past the sequence, or one that saw no key, gets +inf so that its P is 0
    const float lv = r < nq ? a.lse[sv.qrow0 + r] : -INFINITY;
    float* st = a.stats + (size_t)bh * 2 * a.npad;
    st[r] = lv != -INFINITY ? lv * kLog2e : INFINITY;
    st[a.npad + r] = -sum;
  }
}

// ---------------------------------------------------------------------------
// stage 1: per key block, recompute P and dS; accumulate dV and dK
// ---------------------------------------------------------------------------
constexpr int KV_NW = 4;              // waves per workgroup
constexpr int KV_BKV = 32 * KV_NW;    // keys per workgroup (= mask block)
constexpr int KV_BQ = 32;             // query rows per step
constexpr int KV_R = 128 / KV_BQ;     // steps per 128-row mask block
constexpr int MASK_LIST = 2048;       // capacity of a compacted mask row / column
static_assert(KV_BKV == 128, "a key-block workgroup must cover exactly one mask block column");

// position of a step in the key-block kernel's ring of LDS buffers, when known
// at compile time (-1: known only at run time)
template <int P>
using RingAt = std::integral_constant<int, P>;

// position of a step: index qi into the key block's query-block list, and the
// query head's element offset in Q / dO and float offset in the statistics
struct StepPos {
  int qi;
  int hb;  // query head b * H + h
  int soff;
  unsigned long long qoff;
};

// (d <= 64 halves the register operands and accumulators: two workgroups per CU)
template <class T, int D, int BAND, bool MASK, bool DROP, bool ALIBI>
__device__ __forceinline__ void bwd_kv_body(const BwdArgs& a, const int hk, const int b, const int kblk) {
  constexpr int BQ = KV_BQ;
  constexpr int QBUF = BQ * 2 * D;       // one Q or dO block, swizzled rows without padding
  constexpr int STB = 2 * BQ * 4;        // one statistics block: BQ log2-scaled LSE, then BQ D
  constexpr int NS = D / 16;
  constexpr int ND = D / 32;

  // LDS: row statistics, Q and dO in a ring of four buffers (step e uses e % 4:
  // during step e's iteration, step e + 1's buffer feeds S and dP, step e's
  // statistics feed P and dS, step e - 1's buffer feeds dV and dK, and step
  // e + 2 is loaded into the buffer step e - 2 used) and the compacted mask
  // list. The buffers are filled by LDS DMA, straight from memory. The
  // statistics come first, so that every read of them addresses its ring
  // buffer with the instruction's immediate offset (offsets reach 64 KB).
  constexpr int NB = 4;  // the unrolled step loop below covers the ring once per pass
  __shared__ __attribute__((aligned(16))) char smem_raw[2 * NB * QBUF + NB * STB + (MASK ? 2 * MASK_LIST + 16 : 16)];
  lds_t* smem = (lds_t*)smem_raw;
  lds_t* stat = smem;                   // [NB][2 BQ] float
  lds_t* qbuf = stat + NB * STB;        // [NB][BQ rows, swizzled]
  lds_t* obuf = qbuf + NB * QBUF;       // dO, [NB][BQ rows, swizzled]
  __attribute__((address_space(3))) short* blist = (__attribute__((address_space(3))) short*)(obuf + NB * QBUF);
  __attribute__((address_space(3))) int* bcount =
      (__attribute__((address_space(3))) int*)(obuf + NB * QBUF + (MASK ? 2 * MASK_LIST : 0));

  const AttnShape& s = a.s;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(w);  // the wave index as a scalar
  const int l32 = lane & 31, hh = lane >> 5;
  const int g16 = lane >> 4;
  const int roff = 4 * (g16 >> 1) + ((lane & 15) >> 2);   // transposing-read row offset
  const int coff = 16 * (g16 & 1) + 4 * (lane & 3);       // transposing-read column offset
  // workgroup: kv head hk, batch b, key block kblk (under causal masking block 0
  // has the most work and is dispatched first)
  // the sequence as seen from the group's first query head
  const SeqView sv = seq_view(s, b, hk * s.G, hk);
  const int len_q = sv.nq, len_k = sv.nk, off = sv.off;
  const int k0 = kblk * KV_BKV;
  if (k0 >= len_k) return;  // a sequence shorter than the grid (packed batches)
  const int kj = k0 + 32 * w + l32;  // this lane's key (its column of S)
  const float c = s.scale * kLog2e;

  // per-sequence buffer resources: rows past the sequence read as zeros, writes
  // past it are dropped
  const unsigned int qbytes = (unsigned int)len_q * D * 2, kbytes = (unsigned int)len_k * D * 2;
  const size_t krow0 = sv.krow0;
  const rsrc_t rk = make_rsrc((const unsigned short*)a.k + krow0 * D, kbytes);
  const rsrc_t rv = make_rsrc((const unsigned short*)a.v + krow0 * D, kbytes);

  // K^T and V^T operands: lane holds key kj, d = 16 ss + 8 hh + 0..7. Keys past
  // the sequence read as zeros; their dK, dV are never stored.
  s16x8 kf[NS], vf[NS];
#pragma unroll
  for (int ss = 0; ss < NS; ++ss) {
    kf[ss] = bload16(rk, (unsigned)(kj * D + 16 * ss + 8 * hh) * 2u);
    vf[ss] = bload16(rv, (unsigned)(kj * D + 16 * ss + 8 * hh) * 2u);
  }

  // query blocks this key block meets: a band keeps key j for rows
  // j - off - wr <= i <= j - off + wl, so rows from k0 - off - wr up to
  // k0 + 127 - off + wl (offu = off + wr, offl = off - wl; offl binds only with a
  // lower edge)
  constexpr bool LOWER = BAND == 2;
  const int offu = off + s.wr, offl = off - s.wl;
  const int nqb_all = (len_q + BQ - 1) / BQ;
  const int qb_first = BAND ? max(0, k0 - offu) / BQ : 0;
  const int qb_end = LOWER ? min(nqb_all, (max(0, k0 + KV_BKV - offl) + BQ - 1) / BQ) : nqb_all;
  int nq = max(0, qb_end - qb_first);
  if constexpr (MASK) {
    // mask rows I with mask[I][kblk] != 0, from the first one needed to the last
    const int i_first = qb_first / KV_R;
    const int i_end = min(s.nbq, (qb_end + KV_R - 1) / KV_R);
    if (w == 0) {
      int cnt = 0;
      for (int j0 = i_first; j0 < i_end; j0 += 64) {
        const int j = j0 + lane;
        const bool keep = j < i_end && s.mask[(size_t)j * s.nbk + kblk] != 0;
        const unsigned long long bal = __ballot(keep);
        if (keep) blist[cnt + __popcll(bal & ((1ull << lane) - 1ull))] = (short)j;
        cnt += __popcll(bal);
      }
      if (lane == 0) *bcount = cnt;
    }
    __syncthreads();
    const int cnt = *bcount;
    nq = KV_R * cnt;
    if (cnt > 0) nq -= max(0, KV_R * (blist[cnt - 1] + 1) - qb_end);  // steps past the band or the sequence
  }
  auto qblock_at = [&](int qi) -> int {
    if constexpr (MASK) return KV_R * blist[qi / KV_R] + qi % KV_R;
    else return qb_first + qi;
  };
  // steps run over every query block of the list for each query head of the group
  const int nsteps = nq * s.G;
  auto advance = [&](StepPos p) -> StepPos {
    const bool next_head = p.qi + 1 >= nq;
    return StepPos{next_head ? 0 : p.qi + 1, next_head ? p.hb + 1 : p.hb, next_head ? p.soff + 2 * a.npad : p.soff,
                   next_head ? p.qoff + (unsigned long long)sv.qstride * D : p.qoff};
  };

  f32x16 dka[ND], dva[ND];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dka[dt][i] = 0.f;
      dva[dt][i] = 0.f;
    }

  // A step's Q and dO rows and its row statistics, by LDS DMA into ring buffer
  // buf: every wave moves its share of the 1 KB segments; the last wave also
  // moves the statistics (lanes 0..31 the LSE plane, 32..63 the D plane; rows
  // up to the padded length are in range).
  auto dma_q = [&](StepPos p, int buf) {
    const int q0 = qblock_at(p.qi) * BQ;
    const i32x4 rq = rsrc_words((const unsigned short*)a.q + p.qoff, qbytes);
    const i32x4 rg = rsrc_words((const unsigned short*)a.dO + p.qoff, qbytes);
    dma_tile<D, BQ, KV_NW>(rq, q0, qbuf + buf * QBUF, wu, lane);
    dma_tile<D, BQ, KV_NW>(rg, q0, obuf + buf * QBUF, wu, lane);
    if (wu == KV_NW - 1) {
      const i32x4 rs = rsrc_words(a.stats + p.soff, (unsigned)a.npad * 8u);
      dma4(rs, (unsigned)(((lane >> 5) * a.npad + q0 + (lane & 31)) * 4), lds_addr(stat + buf * STB));
    }
  };

  // S = Q K^T and dP = dO V^T of this wave's 32 keys, from Q / dO buffer qbi.
  // Without dropout dP starts at -D (the statistics plane holds -D; element i
  // is row 8 (i / 4) + 4 hh + i % 4), so the MFMAs leave dP - D behind.
  auto sdp = [&](int qbi, f32x16& sc, f32x16& dp) {
    const lds_t* qb = qbuf + qbi * QBUF;
    const lds_t* ob = obuf + qbi * QBUF;
    const __attribute__((address_space(3))) float* ndl =
        (const __attribute__((address_space(3))) float*)(stat + qbi * STB) + BQ;
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      f32x4 n4 = {0.f, 0.f, 0.f, 0.f};
      if constexpr (!DROP) n4 = *(const __attribute__((address_space(3))) f32x4*)(ndl + 8 * j4 + 4 * hh);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sc[4 * j4 + r] = 0.f;
        dp[4 * j4 + r] = n4[r];
      }
    }
#pragma unroll
    for (int ss = 0; ss < NS; ++ss) {
      const int off = swz_off<D>(l32, 2 * ss + hh);
      const s16x8 qa = lds_read16(qb + off);
      const s16x8 ga = lds_read16(ob + off);
      sc = mfma32<T>(qa, kf[ss], sc);
      dp = mfma32<T>(ga, vf[ss], dp);
    }
  };

  // P and dS (unscaled) of a step from its S, dP - D (dP alone with dropout)
  // and statistics buffer. Element
  // i is query q0 + 8 (i / 4) + 4 hh + i % 4 of key kj; under a band mask it is
  // kept only if kj - off - wr <= q0 + 4 hh + 8 (i / 4) + i % 4 <= kj - off + wl.
  // Keys past the sequence need no mask: their K and V rows read as zeros and
  // nothing of theirs is stored.
  // With dropout (z the keep decision, c its scale): P V uses z c P, and
  // dS = P (z c dP - D), the gradient flowing to P through the dropped values.
  // ALiBi adds -slope log2(e) |query + off - kj| of the step's query head to
  // the log2-unit score (a constant bias: dS is unchanged in form).
  // Element masks of partial blocks (block masks with bit tiles): such steps
  // run the masked variant, whose bitrow bit i says whether element i is
  // visible; the lane's key is bit kj % 32 = l32 of word (kj % 128) / 32 = w
  // of each of its 16 rows.
  const rsrc_t rbits = make_rsrc(s.bits, (unsigned)s.ntiles * 2048u);
  auto probs = [&](auto masked, const f32x16& sc, const f32x16& dp, int q0, int stb, int bh, unsigned int (&pk)[8],
                   unsigned int (&sk)[8]) {
    constexpr bool MASKED = decltype(masked)::value;
    unsigned int bitrow = 0xffffu;
    // (masked variant) whether this step needs element masks at all: a
    // partial block, or rows that cross a band edge (the upper while
    // q0 + off + wr < k0 + 127, the lower while q0 + 31 + off - wl > k0);
    // with element masks every step takes this variant, and full blocks inside
    // the band skip the per-element selects
    bool domask = true;
    if constexpr (MASKED && MASK) {
      if (s.btile) {
        const int t = s.btile[(size_t)(q0 >> 7) * s.nbk + kblk];
        domask = t >= 0 || (BAND && q0 + offu < k0 + KV_BKV - 1) || (LOWER && q0 + BQ - 1 + offl > k0);
        if (t >= 0) {
          bitrow = 0u;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const unsigned int word = bload_u32(rbits, bits_off(t, (q0 & 127) + 8 * (i >> 2) + 4 * hh + (i & 3), w));
            bitrow |= ((word >> l32) & 1u) << i;
          }
        }
      }
    }
    const __attribute__((address_space(3))) float* lsel =
        (const __attribute__((address_space(3))) float*)(stat + stb * STB);
    const __attribute__((address_space(3))) float* ndl = lsel + BQ;  // -D
    const int thr = kj - offu - q0 - 4 * hh;   // first kept 8 (i / 4) + i % 4
    const int thr2 = kj - offl - q0 - 4 * hh;  // last kept (with a lower edge)
    // dropout: byte r of dwc[j4] decides query q0 + 8 j4 + 4 hh + r of key kj
    unsigned int dwc[4];
    if constexpr (DROP) drop_words_col4(s.seed0, s.seed1, bh, kj, q0 + 4 * hh, 8, dwc);
    const float nsl2 = ALIBI ? -s.alibi[bh - b * s.H] * kLog2e : 0.f;
    const int dbase = q0 + 4 * hh + off - kj;  // query + off - kj less 8 (i / 4) + i % 4
    float pvv[16];
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const f32x4 L4 = *(const __attribute__((address_space(3))) f32x4*)(lsel + 8 * j4 + 4 * hh);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float sh = ALIBI ? fmaf(nsl2, fabsf((float)(dbase + 8 * j4 + r)), -L4[r]) : -L4[r];
        pvv[4 * j4 + r] = fast_exp2(fmaf(sc[4 * j4 + r], c, sh));
      }
    }
    if constexpr (MASKED) {
      if (domask) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int o = 8 * (i >> 2) + (i & 3);
          pvv[i] = (o < thr || (LOWER && o > thr2) || !((bitrow >> i) & 1u)) ? 0.f : pvv[i];
        }
      }
    }
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      f32x4 nd4 = {0.f, 0.f, 0.f, 0.f};
      if constexpr (DROP) nd4 = *(const __attribute__((address_space(3))) f32x4*)(ndl + 8 * j4 + 4 * hh);
      float p[4], d2[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * j4 + r;
        const float pv = pvv[i];
        if constexpr (DROP) {
          const bool z = drop_keep(dwc[j4], r, s.drop_t);
          p[r] = z ? pv * s.drop_scale : 0.f;
          d2[r] = pv * ((z ? dp[i] * s.drop_scale : 0.f) + nd4[r]);
        } else {
          p[r] = pv;
          d2[r] = pv * dp[i];
        }
      }
      pk[2 * j4] = pack2<T>(p[0], p[1]);
      pk[2 * j4 + 1] = pack2<T>(p[2], p[3]);
      sk[2 * j4] = pack2<T>(d2[0], d2[1]);
      sk[2 * j4 + 1] = pack2<T>(d2[2], d2[3]);
    }
  };

  // dV^T(d x key) += dO^T(d x q) P(q x key); dK^T += Q^T dS. B operand k-slot j
  // of step u is query 16 u + 8 (j / 4) + 4 hh + j % 4, matched by the reads.
  auto dvdk = [&](int qbi, const unsigned int (&pk)[8], const unsigned int (&sk)[8]) {
    const lds_t* qb = qbuf + qbi * QBUF;
    const lds_t* ob = obuf + qbi * QBUF;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        // rows 16 u + roff and 8 below it, columns 32 dt + coff .. + 3
        const int c = 4 * dt + (coff >> 3), within = 2 * (coff & 7);
        const int off0 = swz_off<D>(16 * u + roff, c) + within;
        const int off1 = swz_off<D>(16 * u + roff + 8, c) + within;
        const s16x8 ga = concat(lds_read_tr(ob + off0), lds_read_tr(ob + off1));
        const s16x8 qa = concat(lds_read_tr(qb + off0), lds_read_tr(qb + off1));
        dva[dt] = mfma32<T>(ga, as_operand(pk[4 * u], pk[4 * u + 1], pk[4 * u + 2], pk[4 * u + 3]), dva[dt]);
        dka[dt] = mfma32<T>(qa, as_operand(sk[4 * u], sk[4 * u + 1], sk[4 * u + 2], sk[4 * u + 3]), dka[dt]);
      }
  };

  // Software pipeline. Iteration e issues three mutually independent pieces of
  // work: S and dP of step e + 1, P and dS of step e, dV and dK of step e - 1;
  // step e + 2 is loaded into the buffer step e - 2 used, and one barrier ends
  // the step. Loads are issued on every path (indices clamped; a redundant
  // block lands in a buffer nobody reads). The first iteration's "step -1"
  // multiplies zero P and dS with a zeroed buffer. Only a few steps at the start
  // of each query head's list (the band's upper edge, the causal diagonal) and
  // at its end (the band's lower edge) cross a band edge; they run a masked
  // variant, the others none, and the unmasked steps alternate between two
  // register sets so that nothing is copied from one step to the next.
  for (int i = tid; i < 2 * QBUF / 16; i += KV_NW * 64) {
    const int t = i / (QBUF / 16), off = (i % (QBUF / 16)) * 16;
    lds_write16((t ? obuf : qbuf) + (NB - 1) * QBUF + off, (s16x8){0, 0, 0, 0, 0, 0, 0, 0});
  }
  const int hb0 = b * s.H + hk * s.G;  // first query head of the group, batch included
  StepPos cur{0, hb0, hb0 * 2 * a.npad, (unsigned long long)sv.qrow0 * D};
  StepPos nxt = nsteps > 1 ? advance(cur) : cur;
  dma_q(cur, 0);
  dma_q(nxt, 1);
  dma_wait();
  __syncthreads();
  // iteration e: (sc, dp) = S, dP of step e; (pk, sk) = P, dS of step e - 1;
  // fills (scn, dpn) with step e + 1 and (pkn, skn) with step e. phase is
  // RingAt<e % NB> where the caller knows it at compile time (the buffers are
  // then fixed LDS offsets, folded into the reads' immediate offsets instead
  // of an address add per read), RingAt<-1> otherwise.
  auto iter = [&](int e, auto masked, auto phase, const f32x16& sc, const f32x16& dp, const unsigned int (&pk)[8],
                  const unsigned int (&sk)[8], f32x16& scn, f32x16& dpn, unsigned int (&pkn)[8],
                  unsigned int (&skn)[8]) {
    constexpr int P = decltype(phase)::value;
    const int er = P >= 0 ? P : e;  // congruent to e modulo NB
    const StepPos nn = e + 2 < nsteps ? advance(nxt) : nxt;
    dma_q(nn, (er + 2) & (NB - 1));
    sdp((er + 1) & (NB - 1), scn, dpn);
    probs(masked, sc, dp, qblock_at(cur.qi) * BQ, er & (NB - 1), cur.hb, pkn, skn);
    dvdk((er + NB - 1) & (NB - 1), pk, sk);
    dma_wait();
    __syncthreads();
    cur = nxt;
    nxt = nn;
  };
  f32x16 scA, dpA, scB, dpB;
  unsigned int pkA[8], skA[8], pkB[8], skB[8];
  sdp(0, scA, dpA);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    pkA[j] = 0u;
    skA[j] = 0u;
  }
  auto b_to_a = [&]() {
    scA = scB;
    dpA = dpB;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      pkA[j] = pkB[j];
      skA[j] = skB[j];
    }
  };
  // Masked steps: a query block from q0 crosses the band's upper edge while
  // q0 + off + wr < k0 + 127 (the block's last key) and its lower edge while
  // q0 + 31 + off - wl > k0 (its first key). The list rises, so the former
  // form a prefix and the latter a suffix (each at most five steps without a
  // block mask, two mask rows with one).
  int ndiag = 0, nsuf = 0;
  if constexpr (BAND) {
    const int lim = k0 + KV_BKV - 1 - offu;
    while (ndiag < nq && qblock_at(ndiag) * BQ < lim) ++ndiag;
  }
  if constexpr (LOWER) {
    const int lim2 = k0 - (BQ - 1) - offl;
    while (nsuf < nq - ndiag && qblock_at(nq - 1 - nsuf) * BQ > lim2) ++nsuf;
  }
  const int nmid_end = nq - nsuf;
  const std::true_type masked;
  const std::false_type plain;
  const RingAt<-1> rt;
  int e = 0;
  // with element masks of partial blocks any step may need masking: every step
  // runs the masked variant (the plain schedule below serves all other calls)
  const bool all_masked = MASK && s.btile != nullptr;
  for (int hg = 0; all_masked && hg < s.G; ++hg) {
    for (int t = 0; t < nq; ++t, ++e) {
      iter(e, masked, rt, scA, dpA, pkA, skA, scB, dpB, pkB, skB);
      b_to_a();
    }
  }
  for (int hg = 0; !all_masked && hg < s.G; ++hg) {
    for (int t = 0; t < ndiag; ++t, ++e) {
      iter(e, masked, rt, scA, dpA, pkA, skA, scB, dpB, pkB, skB);
      b_to_a();
    }
    int t = ndiag;
    // unmasked steps: first up to three to bring e to a multiple of NB, then
    // four at a time with the ring position fixed at compile time, then the
    // rest; pairs alternate the register sets, a single step copies them back
    if ((e & 1) && t < nmid_end) {
      iter(e, plain, rt, scA, dpA, pkA, skA, scB, dpB, pkB, skB);
      b_to_a();
      ++e;
      ++t;
    }
    if ((e & 2) && t + 1 < nmid_end) {
      iter(e, plain, rt, scA, dpA, pkA, skA, scB, dpB, pkB, skB);
      iter(e + 1, plain, rt, scB, dpB, pkB, skB, scA, dpA, pkA, skA);
      e += 2;
      t += 2;
    }
    if ((e & (NB - 1)) == 0) {
      for (; t + 3 < nmid_end; t += 4, e += 4) {
        iter(e, plain, RingAt<0>{}, scA, dpA, pkA, skA, scB, dpB, pkB, skB);
        iter(e + 1, plain, RingAt<1>{}, scB, dpB, pkB, skB, scA, dpA, pkA, skA);
        iter(e + 2, plain, RingAt<2>{}, scA, dpA, pkA, skA, scB, dpB, pkB, skB);
        iter(e + 3, plain, RingAt<3>{}, scB, dpB, pkB, skB, scA, dpA, pkA, skA);
      }
    }
    for (; t + 1 < nmid_end; t += 2, e += 2) {
      iter(e, plain, rt, scA, dpA, pkA, skA, scB, dpB, pkB, skB);
      iter(e + 1, plain, rt, scB, dpB, pkB, skB, scA, dpA, pkA, skA);
    }
    if (t < nmid_end) {
      iter(e, plain, rt, scA, dpA, pkA, skA, scB, dpB, pkB, skB);
      b_to_a();
      ++e;
      ++t;
    }
    if constexpr (LOWER) {
      for (; t < nq; ++t, ++e) {
        iter(e, masked, rt, scA, dpA, pkA, skA, scB, dpB, pkB, skB);
        b_to_a();
      }
    }
  }
  if (nsteps > 0) dvdk((nsteps - 1) & (NB - 1), pkA, skA);

  // dK^T / dV^T: lane holds key kj, d = 32 dt + 8 j + 4 hh + 0..3; dK takes the scale
  const float scale = s.scale;
  const rsrc_t rdk = make_rsrc((unsigned short*)a.dk + krow0 * D, kbytes);
  const rsrc_t rdv = make_rsrc((unsigned short*)a.dv + krow0 * D, kbytes);
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x2 kv = {pack2<T>(dka[dt][4 * j] * scale, dka[dt][4 * j + 1] * scale),
                  pack2<T>(dka[dt][4 * j + 2] * scale, dka[dt][4 * j + 3] * scale)};
      u32x2 vv = {pack2<T>(dva[dt][4 * j], dva[dt][4 * j + 1]),
                  pack2<T>(dva[dt][4 * j + 2], dva[dt][4 * j + 3])};
      const unsigned int off = (unsigned)(kj * D + 32 * dt + 8 * j + 4 * hh) * 2u;
      bstore8(rdk, off, kv);
      bstore8(rdv, off, vv);
    }
}

// ---------------------------------------------------------------------------
// stage 1 with split roles (d = 128 without block mask; band edges, dropout
// and ALiBi included): eight waves per key block, two per SIMD. Producer wave j
// (0..3) holds K^T and V^T of keys k0 + 32 j .. + 31, forms S and dP of each
// step and from them P and dS, and hands P and dS through LDS to consumer wave
// j + 4, which holds dK^T and dV^T of the same keys and accumulates dV^T +=
// dO^T P and dK^T += Q^T dS one step behind. Each role fits in half the
// register file, so the two waves of a SIMD overlap one's softmax arithmetic
// with the other's MFMAs, which the one-role kernel (all 512 registers, one
// wave per SIMD) can only do within a single in-order instruction stream.
//
// Iteration e (one barrier at its end): producers load step e + 2 into the
// ring buffer step e - 2 used, form S and dP of step e + 1 and P and dS of
// step e (into hand-over buffer e % 2); consumers take dV, dK of step e - 1
// with P and dS from hand-over buffer (e - 1) % 2 and the transposed Q, dO of
// step e - 1 read in iteration e - 1, then read those of step e. Step e's ring
// buffer is read by producers in iterations e - 1 and e and by consumers in e,
// and rewritten in e + 2; a hand-over buffer is written in e, read in e + 1
// and rewritten in e + 2.
// ---------------------------------------------------------------------------
constexpr int KS_NW = 8;  // waves per split-role workgroup: 4 producers, 4 consumers

template <int D, int BAND, bool MASK, bool DROP, bool ALIBI>
constexpr bool kv_split() {
  return D == 128 && !MASK;
}

template <class T, int D, int BAND, bool DROP, bool ALIBI>
__device__ __forceinline__ void bwd_kv_split_body(const BwdArgs& a, const int hk, const int b, const int kblk) {
  constexpr int BQ = KV_BQ;
  constexpr int QBUF = BQ * 2 * D;  // one Q or dO block, swizzled rows
  constexpr int STB = 2 * BQ * 4;   // one statistics block: BQ log2-scaled LSE, then BQ -D
  constexpr int PSB = 64 * 64;      // one producer's P and dS of a step: 64 bytes per lane
  constexpr int NS = D / 16;
  constexpr int ND = D / 32;
  constexpr int NB = 4;             // the unrolled step loops cover the ring once per pass
  __shared__ __attribute__((aligned(16))) char smem_raw[NB * STB + 2 * NB * QBUF + 2 * 4 * PSB];
  lds_t* stat = (lds_t*)smem_raw;   // [NB][2 BQ] float
  lds_t* qbuf = stat + NB * STB;    // [NB][BQ rows, swizzled]
  lds_t* obuf = qbuf + NB * QBUF;   // dO, [NB][BQ rows, swizzled]
  lds_t* psbuf = obuf + NB * QBUF;  // [2][4 producers][4 chunks of 16 bytes][64 lanes]

  const AttnShape& s = a.s;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wu = __builtin_amdgcn_readfirstlane(tid >> 6);  // the wave index as a scalar
  const bool producer = wu < 4;
  const int jw = wu & 3;  // the wave's 32 keys within the block
  const int l32 = lane & 31, hh = lane >> 5;
  const int g16 = lane >> 4;
  const int roff = 4 * (g16 >> 1) + ((lane & 15) >> 2);  // transposing-read row offset
  const int coff = 16 * (g16 & 1) + 4 * (lane & 3);      // transposing-read column offset
  // the sequence as seen from the group's first query head
  const SeqView sv = seq_view(s, b, hk * s.G, hk);
  const int len_q = sv.nq, len_k = sv.nk, off = sv.off;
  const int k0 = kblk * KV_BKV;
  if (k0 >= len_k) return;  // a sequence shorter than the grid (packed batches)
  const int kj = k0 + 32 * jw + l32;  // this lane's key (its column of S)
  const unsigned int qbytes = (unsigned int)len_q * D * 2, kbytes = (unsigned int)len_k * D * 2;
  const size_t krow0 = sv.krow0;
  // query blocks that see a key of the block: rows from k0 - off - wr to
  // k0 + 127 - off + wl (offu = off + wr, offl = off - wl; offl binds only
  // with a lower edge), for each query head of the group
  constexpr bool LOWER = BAND == 2;
  const int offu = off + s.wr, offl = off - s.wl;
  const int nqb_all = (len_q + BQ - 1) / BQ;
  const int qb_first = BAND ? max(0, k0 - offu) / BQ : 0;
  const int qb_end = LOWER ? min(nqb_all, (max(0, k0 + KV_BKV - offl) + BQ - 1) / BQ) : nqb_all;
  const int nq = max(0, qb_end - qb_first);
  const int nsteps = nq * s.G;

  if (producer) {
    const float c = s.scale * kLog2e;
    // K^T and V^T operands: lane holds key kj, d = 16 ss + 8 hh + 0..7 (keys
    // past the sequence read as zeros)
    const rsrc_t rk = make_rsrc((const unsigned short*)a.k + krow0 * D, kbytes);
    const rsrc_t rv = make_rsrc((const unsigned short*)a.v + krow0 * D, kbytes);
    s16x8 kf[NS], vf[NS];
#pragma unroll
    for (int ss = 0; ss < NS; ++ss) {
      kf[ss] = bload16(rk, (unsigned)(kj * D + 16 * ss + 8 * hh) * 2u);
      vf[ss] = bload16(rv, (unsigned)(kj * D + 16 * ss + 8 * hh) * 2u);
    }
    auto advance = [&](StepPos p) -> StepPos {
      const bool next_head = p.qi + 1 >= nq;
      return StepPos{next_head ? 0 : p.qi + 1, next_head ? p.hb + 1 : p.hb, next_head ? p.soff + 2 * a.npad : p.soff,
                     next_head ? p.qoff + (unsigned long long)sv.qstride * D : p.qoff};
    };
    // a step's Q and dO rows and statistics into ring buffer buf by LDS DMA,
    // shared by the four producers (the last also moves the statistics)
    auto dma_q = [&](StepPos p, int buf) {
      const int q0 = (qb_first + p.qi) * BQ;
      const i32x4 rq = rsrc_words((const unsigned short*)a.q + p.qoff, qbytes);
      const i32x4 rg = rsrc_words((const unsigned short*)a.dO + p.qoff, qbytes);
      dma_tile<D, BQ, 4>(rq, q0, qbuf + buf * QBUF, wu, lane);
      dma_tile<D, BQ, 4>(rg, q0, obuf + buf * QBUF, wu, lane);
      if (wu == 3) {
        const i32x4 rs = rsrc_words(a.stats + p.soff, (unsigned)a.npad * 8u);
        dma4(rs, (unsigned)(((lane >> 5) * a.npad + q0 + (lane & 31)) * 4), lds_addr(stat + buf * STB));
      }
    };
    // one plane of a ring buffer's statistics (0: LSE, 1: -D) for this lane's
    // rows 8 j4 + 4 hh + 0..3
    auto stats4 = [&](int sb, int plane, f32x4 (&v)[4]) {
      const __attribute__((address_space(3))) float* pl =
          (const __attribute__((address_space(3))) float*)(stat + sb * STB) + plane * BQ;
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) v[j4] = *(const __attribute__((address_space(3))) f32x4*)(pl + 8 * j4 + 4 * hh);
    };
    // S = Q K^T and dP - D = dO V^T - D of this wave's 32 keys from ring buffer
    // sb (dP starts at -D; with dropout at 0, the -D term added after the keep
    // factor)
    auto sdp = [&](int sb, f32x16& sc, f32x16& dp, const f32x4 (&nd)[4]) {
      const lds_t* qb = qbuf + sb * QBUF;
      const lds_t* ob = obuf + sb * QBUF;
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          sc[4 * j4 + r] = 0.f;
          dp[4 * j4 + r] = DROP ? 0.f : nd[j4][r];
        }
#pragma unroll
      for (int ss = 0; ss < NS; ++ss) {
        const int o = swz_off<D>(l32, 2 * ss + hh);
        const s16x8 qa = lds_read16(qb + o);
        const s16x8 ga = lds_read16(ob + o);
        sc = mfma32<T>(qa, kf[ss], sc);
        dp = mfma32<T>(ga, vf[ss], dp);
      }
    };
    // P and dS (unscaled) of a step into hand-over buffer pb, as the consumer's
    // B operands: chunk 2 m + u holds slots of MFMA step u (m = 0 P, 1 dS), lane
    // by lane. Element i is query q0 + 8 (i / 4) + 4 hh + i % 4 of key kj;
    // under causal masking or a right window it is kept only while
    // kj - off - wr <= query, and with a lower edge while query <= kj - off + wl
    // (the masked variant, for blocks crossing an edge).
    // With dropout (z the keep decision, cz its scale) P V uses z cz P and
    // dS = P (z cz dP - D); ALiBi adds the query head's distance bias to the
    // log2-unit score (bh: the step's query head, batch included; nd: -D of the
    // step's rows, read only with dropout).
    auto probs = [&](auto masked, const f32x16& sc, const f32x16& dp, int q0, const f32x4 (&lv)[4], int pb, int bh,
                     const f32x4 (&nd)[4]) {
      constexpr bool MASKED = decltype(masked)::value;
      unsigned int dwc[4];
      if constexpr (DROP) drop_words_col4(s.seed0, s.seed1, bh, kj, q0 + 4 * hh, 8, dwc);
      const float nsl2 = ALIBI ? -s.alibi[bh - b * s.H] * kLog2e : 0.f;
      const int dbase = q0 + 4 * hh + off - kj;  // query + off - kj less 8 (i / 4) + i % 4
      float pvv[16];
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float sh = ALIBI ? fmaf(nsl2, fabsf((float)(dbase + 8 * j4 + r)), -lv[j4][r]) : -lv[j4][r];
          pvv[4 * j4 + r] = fast_exp2(fmaf(sc[4 * j4 + r], c, sh));
        }
      if constexpr (MASKED) {
        const int thr = kj - offu - q0 - 4 * hh;   // first kept 8 (i / 4) + i % 4
        const int thr2 = kj - offl - q0 - 4 * hh;  // last kept (with a lower edge)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int o = 8 * (i >> 2) + (i & 3);
          pvv[i] = (o < thr || (LOWER && o > thr2)) ? 0.f : pvv[i];
        }
      }
      unsigned int pk[8], sk[8];
#pragma unroll
      for (int j2 = 0; j2 < 8; ++j2) {
        float p2[2], d2[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const int i = 2 * j2 + r;
          if constexpr (DROP) {
            const bool z = drop_keep(dwc[i >> 2], i & 3, s.drop_t);
            p2[r] = z ? pvv[i] * s.drop_scale : 0.f;
            d2[r] = pvv[i] * ((z ? dp[i] * s.drop_scale : 0.f) + nd[i >> 2][i & 3]);
          } else {
            p2[r] = pvv[i];
            d2[r] = pvv[i] * dp[i];
          }
        }
        pk[j2] = pack2<T>(p2[0], p2[1]);
        sk[j2] = pack2<T>(d2[0], d2[1]);
      }
      lds_t* pw = psbuf + (pb * 4 + jw) * PSB + lane * 16;
      lds_write16(pw, __builtin_bit_cast(s16x8, (u32x4){pk[0], pk[1], pk[2], pk[3]}));
      lds_write16(pw + 1024, __builtin_bit_cast(s16x8, (u32x4){pk[4], pk[5], pk[6], pk[7]}));
      lds_write16(pw + 2048, __builtin_bit_cast(s16x8, (u32x4){sk[0], sk[1], sk[2], sk[3]}));
      lds_write16(pw + 3072, __builtin_bit_cast(s16x8, (u32x4){sk[4], sk[5], sk[6], sk[7]}));
    };
    const int hb0 = b * s.H + hk * s.G;  // first query head of the group, batch included
    StepPos cur{0, hb0, hb0 * 2 * a.npad, (unsigned long long)sv.qrow0 * D};
    StepPos nxt = nsteps > 1 ? advance(cur) : cur;
    dma_q(cur, 0);
    dma_q(nxt, 1);
    dma_wait();
    __syncthreads();
    // iteration e: P and dS of step e from (sc, dp), S and dP of step e + 1
    // into (scn, dpn). phase is RingAt<e % NB> where the caller knows it at
    // compile time, RingAt<-1> otherwise. Loads are issued on every path
    // (indices clamped; a redundant block lands in a buffer nobody reads), and
    // the last iteration's S and dP of a step past the list go unused.
    auto iter = [&](int e, auto masked, auto phase, const f32x16& sc, const f32x16& dp, f32x16& scn, f32x16& dpn) {
      constexpr int P = decltype(phase)::value;
      const int er = P >= 0 ? P : e;  // congruent to e modulo NB
      const StepPos nn = e + 2 < nsteps ? advance(nxt) : nxt;
      f32x4 lv[4], nd[4], ndp[4];
      stats4(er & (NB - 1), 0, lv);
      if constexpr (DROP) stats4(er & (NB - 1), 1, ndp);
      else stats4((er + 1) & (NB - 1), 1, nd);
      dma_q(nn, (er + 2) & (NB - 1));
      sdp((er + 1) & (NB - 1), scn, dpn, nd);
      probs(masked, sc, dp, (qb_first + cur.qi) * BQ, lv, er & 1, cur.hb, ndp);
      dma_wait();
      __syncthreads();
      cur = nxt;
      nxt = nn;
    };
    f32x16 scA, dpA, scB, dpB;
    {
      f32x4 nd0[4];
      stats4(0, 1, nd0);
      sdp(0, scA, dpA, nd0);  // (the first step's -D, unused with dropout)
    }
    auto b_to_a = [&]() {
      scA = scB;
      dpA = dpB;
    };
    // the first ndiag steps of each query head's list cross the band's upper
    // edge (q0 + off + wr < k0 + 127), the last nsuf its lower edge
    // (q0 + 31 + off - wl > k0); they take the masked variant
    int ndiag = 0, nsuf = 0;
    if constexpr (BAND) {
      const int lim = k0 + KV_BKV - 1 - offu;
      while (ndiag < nq && (qb_first + ndiag) * BQ < lim) ++ndiag;
    }
    if constexpr (LOWER) {
      const int lim2 = k0 - (BQ - 1) - offl;
      while (nsuf < nq - ndiag && (qb_first + nq - 1 - nsuf) * BQ > lim2) ++nsuf;
    }
    const int nmid_end = nq - nsuf;
    const std::true_type masked;
    const std::false_type plain;
    const RingAt<-1> rt;
    int e = 0;
    for (int hg = 0; hg < s.G; ++hg) {
      for (int t = 0; t < ndiag; ++t, ++e) {
        iter(e, masked, rt, scA, dpA, scB, dpB);
        b_to_a();
      }
      // unmasked steps: up to three to bring e to a multiple of NB, then four
      // at a time with the ring position fixed at compile time, then the rest;
      // pairs alternate the register sets, a single step copies them back
      int t = ndiag;
      if ((e & 1) && t < nmid_end) {
        iter(e, plain, rt, scA, dpA, scB, dpB);
        b_to_a();
        ++e;
        ++t;
      }
      if ((e & 2) && t + 1 < nmid_end) {
        iter(e, plain, rt, scA, dpA, scB, dpB);
        iter(e + 1, plain, rt, scB, dpB, scA, dpA);
        e += 2;
        t += 2;
      }
      if ((e & (NB - 1)) == 0) {
        for (; t + 3 < nmid_end; t += 4, e += 4) {
          iter(e, plain, RingAt<0>{}, scA, dpA, scB, dpB);
          iter(e + 1, plain, RingAt<1>{}, scB, dpB, scA, dpA);
          iter(e + 2, plain, RingAt<2>{}, scA, dpA, scB, dpB);
          iter(e + 3, plain, RingAt<3>{}, scB, dpB, scA, dpA);
        }
      }
      for (; t + 1 < nmid_end; t += 2, e += 2) {
        iter(e, plain, rt, scA, dpA, scB, dpB);
        iter(e + 1, plain, rt, scB, dpB, scA, dpA);
      }
      if (t < nmid_end) {
        iter(e, plain, rt, scA, dpA, scB, dpB);
        b_to_a();
        ++e;
        ++t;
      }
      if constexpr (LOWER) {
        for (; t < nq; ++t, ++e) {
          iter(e, masked, rt, scA, dpA, scB, dpB);
          b_to_a();
        }
      }
    }
  } else {
    f32x16 dka[ND], dva[ND];
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        dka[dt][i] = 0.f;
        dva[dt][i] = 0.f;
      }
    // transposing reads of a step's dO^T and Q^T (its ring buffer is complete
    // two barriers before the step's dV, dK), issued an iteration ahead
    auto tr_read = [&](int sb, s16x8 (&ga)[ND][2], s16x8 (&qa)[ND][2]) {
      const lds_t* qb = qbuf + sb * QBUF;
      const lds_t* ob = obuf + sb * QBUF;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int cc = 4 * dt + (coff >> 3), within = 2 * (coff & 7);
          const int off0 = swz_off<D>(16 * u + roff, cc) + within;
          const int off1 = swz_off<D>(16 * u + roff + 8, cc) + within;
          ga[dt][u] = concat(lds_read_tr(ob + off0), lds_read_tr(ob + off1));
          qa[dt][u] = concat(lds_read_tr(qb + off0), lds_read_tr(qb + off1));
        }
    };
    // dV^T += dO^T P, dK^T += Q^T dS of a step with P, dS from hand-over buffer pb
    auto dvdk = [&](int pb, const s16x8 (&ga)[ND][2], const s16x8 (&qa)[ND][2]) {
      const lds_t* pr = psbuf + (pb * 4 + jw) * PSB + lane * 16;
      const s16x8 pop[2] = {lds_read16(pr), lds_read16(pr + 1024)};
      const s16x8 sop[2] = {lds_read16(pr + 2048), lds_read16(pr + 3072)};
#pragma unroll
      for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          dva[dt] = mfma32<T>(ga[dt][u], pop[u], dva[dt]);
          dka[dt] = mfma32<T>(qa[dt][u], sop[u], dka[dt]);
        }
    };
    s16x8 ga[ND][2], qa[ND][2];
    // as many barriers as the producers: the prologue's, then one per step
    __syncthreads();
    if (nsteps > 0) {
      tr_read(0, ga, qa);
      __syncthreads();  // iteration 0: step 0's P and dS
    }
    // iteration e (1 <= e < nsteps) takes step e - 1 while the producers form
    // step e, then reads step e's transposed operands, so that after the barrier
    // only the four hand-over reads stand between it and its products (1.6%
    // faster than reading everything after the barrier); four at a time with
    // the ring position fixed at compile time
    int e = 1;
    for (; e + 3 < nsteps; e += 4) {
      dvdk(0, ga, qa);
      tr_read(1, ga, qa);
      __syncthreads();
      dvdk(1, ga, qa);
      tr_read(2, ga, qa);
      __syncthreads();
      dvdk(0, ga, qa);
      tr_read(3, ga, qa);
      __syncthreads();
      dvdk(1, ga, qa);
      tr_read(0, ga, qa);
      __syncthreads();
    }
    for (; e < nsteps; ++e) {
      dvdk((e - 1) & 1, ga, qa);
      tr_read(e & (NB - 1), ga, qa);
      __syncthreads();
    }
    if (nsteps > 0) dvdk((nsteps - 1) & 1, ga, qa);  // after the producers' last barrier

    // dK^T / dV^T: lane holds key kj, d = 32 dt + 8 j + 4 hh + 0..3; dK takes the scale
    const float scale = s.scale;
    const rsrc_t rdk = make_rsrc((unsigned short*)a.dk + krow0 * D, kbytes);
    const rsrc_t rdv = make_rsrc((unsigned short*)a.dv + krow0 * D, kbytes);
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x2 kv = {pack2<T>(dka[dt][4 * j] * scale, dka[dt][4 * j + 1] * scale),
                    pack2<T>(dka[dt][4 * j + 2] * scale, dka[dt][4 * j + 3] * scale)};
        u32x2 vv = {pack2<T>(dva[dt][4 * j], dva[dt][4 * j + 1]), pack2<T>(dva[dt][4 * j + 2], dva[dt][4 * j + 3])};
        const unsigned int o = (unsigned)(kj * D + 32 * dt + 8 * j + 4 * hh) * 2u;
        bstore8(rdk, o, kv);
        bstore8(rdv, o, vv);
      }
  }
}

template <class T, int D, int BAND, bool MASK, bool DROP, bool ALIBI>
__global__ __launch_bounds__((kv_split<D, BAND, MASK, DROP, ALIBI>() ? KS_NW * 64 : KV_NW * 64), D <= 64 ? 2 : 1)
    void bwd_kv_kernel(BwdArgs a) {
  const GridPos gp = grid_pos(a.s);  // grid: tile_grid over kv heads and key blocks
  if constexpr (kv_split<D, BAND, MASK, DROP, ALIBI>())
    bwd_kv_split_body<T, D, BAND, DROP, ALIBI>(a, blockIdx.x, gp.b, gp.blk);
  else
    bwd_kv_body<T, D, BAND, MASK, DROP, ALIBI>(a, blockIdx.x, gp.b, gp.blk);
}

// ---------------------------------------------------------------------------
// stage 2: per query block, recompute P and dS; accumulate dQ
// ---------------------------------------------------------------------------
constexpr int Q_NW = 4;              // waves per workgroup
constexpr int Q_BM = 32 * Q_NW;      // query rows per workgroup (= mask block)
#ifndef FA_Q_BN
#define FA_Q_BN 32
#endif
#ifndef FA_Q_OCC
#define FA_Q_OCC 2
#endif
constexpr int Q_BN = FA_Q_BN;        // keys per tile
constexpr int Q_T2 = Q_BN / 32;      // 32-key halves per tile
constexpr int Q_R = 128 / Q_BN;      // tiles per 128-key mask block
static_assert(Q_BM == 128, "a query-block workgroup must cover exactly one mask block row");

template <class T, int D, int BAND, bool MASK, bool DROP, bool ALIBI>
__device__ __forceinline__ void bwd_q_body(const BwdArgs& a, const int h, const int b, const int blk,
                                           const int nblk) {
  constexpr int KBUF = Q_BN * 2 * D;     // K tile: swizzled rows, row reads and transposing reads
  constexpr int VBUF = Q_BN * 2 * D;     // V tile: swizzled rows, row reads
  constexpr int NS = D / 16;
  constexpr int ND = D / 32;

  __shared__ __attribute__((aligned(16))) char smem_raw[2 * KBUF + 2 * VBUF + (MASK ? 2 * MASK_LIST + 16 : 16)];
  lds_t* kbuf = (lds_t*)smem_raw;
  lds_t* vbuf = kbuf + 2 * KBUF;
  __attribute__((address_space(3))) short* blist = (__attribute__((address_space(3))) short*)(vbuf + 2 * VBUF);
  __attribute__((address_space(3))) int* bcount =
      (__attribute__((address_space(3))) int*)(vbuf + 2 * VBUF + (MASK ? 2 * MASK_LIST : 0));

  const AttnShape& s = a.s;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(w);  // the wave index as a scalar
  const int l32 = lane & 31, hh = lane >> 5;
  const int g16 = lane >> 4;
  const int roff = 4 * (g16 >> 1) + ((lane & 15) >> 2);
  const int coff = 16 * (g16 & 1) + 4 * (lane & 3);
  // grid (tile_grid), as in the forward pass
  // workgroup: query head h, batch b, block blk of nblk in launch order; under
  // a band mask the later (under causal masking, longer) query blocks first
  const int qb = BAND ? nblk - 1 - blk : blk;
  const int hk = h / s.G;
  const SeqView sv = seq_view(s, b, h, hk);
  const int len_q = sv.nq, len_k = sv.nk, off = sv.off;
  const int q0 = qb * Q_BM;
  if (q0 >= len_q) return;  // a sequence shorter than the grid (packed batches)
  const size_t qrow0 = sv.qrow0, krow0 = sv.krow0;
  const unsigned int qbytes = (unsigned int)len_q * D * 2, kbytes = (unsigned int)len_k * D * 2;
  const rsrc_t rq = make_rsrc((const unsigned short*)a.q + qrow0 * D, qbytes);
  const rsrc_t rg = make_rsrc((const unsigned short*)a.dO + qrow0 * D, qbytes);
  const i32x4 rk = rsrc_words((const unsigned short*)a.k + krow0 * D, kbytes);
  const i32x4 rv = rsrc_words((const unsigned short*)a.v + krow0 * D, kbytes);
  const int qw = q0 + 32 * w;
  const int qi = qw + l32;   // this lane's query row
  const float c = s.scale * kLog2e;
  const float nsl2 = ALIBI ? -s.alibi[h] * kLog2e : 0.f;  // ALiBi slope, log2 units

  // Q^T and dO^T operands: lane holds query qi, d = 16 ss + 8 hh + 0..7
  s16x8 qf[NS], gf[NS];
#pragma unroll
  for (int ss = 0; ss < NS; ++ss) {
    qf[ss] = bload16(rq, (unsigned)(qi * D + 16 * ss + 8 * hh) * 2u);
    gf[ss] = bload16(rg, (unsigned)(qi * D + 16 * ss + 8 * hh) * 2u);
  }
  // this lane's row statistics from stage 0 (qi < npad); a row past the
  // sequence, or one that saw no key, has LSE +inf and so P = 0
  const float* st = a.stats + ((size_t)b * s.H + h) * 2 * a.npad;
  const float lse2 = st[qi];
  const float ndd = st[a.npad + qi];  // -D

  // keys [kbeg, kend) are seen by some row of the block (band as in the forward pass)
  constexpr bool LOWER = BAND == 2;
  const int offu = off + s.wr, offl = off - s.wl;
  const int kbeg = LOWER ? max(0, q0 + offl) : 0;
  const int kend = BAND ? min(len_k, max(0, q0 + Q_BM + offu)) : len_k;
  const int tbeg = kbeg / Q_BN;
  const int ntile_all = (kend + Q_BN - 1) / Q_BN;
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
    ntiles = Q_R * cnt;
    if (cnt > 0) ntiles -= max(0, Q_R * (blist[cnt - 1] + 1) - ntile_all);  // tiles past kend
  }
  auto tile_at = [&](int e) -> int {
    if constexpr (MASK) return Q_R * blist[e / Q_R] + e % Q_R;
    else return tbeg + e;
  };

  f32x16 acc[ND];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;
  // element masks of partial blocks: bit tiles through a buffer resource
  const rsrc_t rbits = make_rsrc(s.bits, (unsigned)s.ntiles * 2048u);

  // K and V tiles by LDS DMA into the buffer the previous step read (the
  // barrier that ended it has passed); rows past the sequence arrive as zeros
  auto dma_kv = [&](int t, int buf) {
    dma_tile<D, Q_BN, Q_NW>(rk, t * Q_BN, kbuf + buf * KBUF, wu, lane);
    dma_tile<D, Q_BN, Q_NW>(rv, t * Q_BN, vbuf + buf * VBUF, wu, lane);
  };

  dma_kv(ntiles > 0 ? tile_at(0) : 0, 0);
  dma_wait();
  __syncthreads();

  // tile e reads buffer e % 2 and loads tile e + 1 into the other; tiles go in
  // pairs so that each knows its buffer at compile time (fixed LDS offsets in
  // the reads' immediate fields rather than an address add per read)
  auto tile = [&](int e, auto phase) {
    constexpr int buf = decltype(phase)::value;
    const int ks = tile_at(e) * Q_BN;
    dma_kv(tile_at(e + 1 < ntiles ? e + 1 : e), buf ^ 1);

    // wave-uniform: does any row of the wave see a key of the tile
    const bool active = !(BAND && ks > qw + 31 + offu) && !(LOWER && ks + Q_BN - 1 < qw + offl);
    if (active) {
      // a partial block: this row's bits for the tile's 32-key halves
      int tidx = -1;
      if constexpr (MASK) {
        if (s.btile) tidx = s.btile[(size_t)qb * s.nbk + (ks >> 7)];
      }
      unsigned int bwq[Q_T2];
#pragma unroll
      for (int t2 = 0; t2 < Q_T2; ++t2)
        bwq[t2] = tidx >= 0 ? bload_u32(rbits, bits_off(tidx, qi & 127, ((ks & 127) >> 5) + t2)) : ~0u;
      const lds_t* kb = kbuf + buf * KBUF;
      const lds_t* vb = vbuf + buf * VBUF;
      // S^T = K Q^T and dP^T = V dO^T for the tile's keys (32-key halves)
      f32x16 sc[Q_T2], dp[Q_T2];
#pragma unroll
      for (int t2 = 0; t2 < Q_T2; ++t2)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          sc[t2][i] = 0.f;
          dp[t2][i] = 0.f;
        }
#pragma unroll
      for (int ss = 0; ss < NS; ++ss)
#pragma unroll
        for (int t2 = 0; t2 < Q_T2; ++t2) {
          const int off = swz_off<D>(32 * t2 + l32, 2 * ss + hh);
          const s16x8 ka = lds_read16(kb + off);
          const s16x8 va = lds_read16(vb + off);
          sc[t2] = mfma32<T>(ka, qf[ss], sc[t2]);
          dp[t2] = mfma32<T>(va, gf[ss], dp[t2]);
        }
      // dS for query qi and key ks + 32 t2 + 8 (i / 4) + 4 hh + i % 4. Band: kept
      // only if qi + off - wl <= key <= qi + off + wr. Keys past the sequence read
      // as zeros, so their dS multiplies a zero row of K and needs no mask.
      const bool diag = (BAND && ks + Q_BN - 1 > qw + offu) || (LOWER && ks < qw + 31 + offl) || tidx >= 0;
      const int thr = qi + offu - ks - 4 * hh;   // last kept 32 t2 + 8 (i / 4) + i % 4
      const int thr2 = qi + offl - ks - 4 * hh;  // first kept (with a lower edge)
      unsigned int sk[Q_T2][8];
      // dropout words of row qi for key groups ks + 32 t2 + 8 g + 4 hh (g = 0..3)
      unsigned int dwq[Q_T2][4];
      if constexpr (DROP) {
#pragma unroll
        for (int t2 = 0; t2 < Q_T2; ++t2)
          drop_words_row4(s.seed0, s.seed1, b * s.H + h, qi, ks + 32 * t2 + 4 * hh, 8, dwq[t2]);
      }
      const float dqf = (float)(qi + off - ks - 4 * hh);  // ALiBi distance less the element's key offset
      auto ds_tile = [&](auto masked) {
        constexpr bool MASKED = decltype(masked)::value;
#pragma unroll
        for (int t2 = 0; t2 < Q_T2; ++t2)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            float v2[2];
            unsigned int wd = 0;
            if constexpr (DROP) wd = dwq[t2][j >> 1];  // keys ks + 32 t2 + 8 (j / 2) + 4 hh + 0..3 of row qi
#pragma unroll
            for (int r = 0; r < 2; ++r) {
              const int i = 2 * j + r;
              const float kofs = (float)(32 * t2 + 8 * (i >> 2) + (i & 3));
              const float sh = ALIBI ? fmaf(nsl2, fabsf(dqf - kofs), -lse2) : -lse2;
              float pv = fast_exp2(fmaf(sc[t2][i], c, sh));
              if constexpr (MASKED) {
                const int kidx = 32 * t2 + 8 * (i >> 2) + (i & 3);
                pv = (kidx > thr || (LOWER && kidx < thr2) || !((bwq[t2] >> (kidx - 32 * t2 + 4 * hh)) & 1u)) ? 0.f
                                                                                                      : pv;
              }
              if constexpr (DROP)
                v2[r] = pv * ((drop_keep(wd, i & 3, s.drop_t) ? dp[t2][i] * s.drop_scale : 0.f) + ndd);
              else
                v2[r] = pv * (dp[t2][i] + ndd);
            }
            sk[t2][j] = pack2<T>(v2[0], v2[1]);
          }
      };
      if (diag) ds_tile(std::true_type{});
      else ds_tile(std::false_type{});
      // dQ^T(d x q) += K^T(d x key) dS^T(key x q); B operand k-slot j of step
      // (t2, u) is key 32 t2 + 16 u + 8 (j / 4) + 4 hh + j % 4, matched by the
      // transposing reads of K
#pragma unroll
      for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int t2 = 0; t2 < Q_T2; ++t2)
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            // rows 32 t2 + 16 u + roff and 8 below it, columns 32 dt + coff .. + 3
            const int c = 4 * dt + (coff >> 3), within = 2 * (coff & 7);
            const int r0 = 32 * t2 + 16 * u + roff;
            const s16x8 ka = concat(lds_read_tr(kb + swz_off<D>(r0, c) + within),
                                    lds_read_tr(kb + swz_off<D>(r0 + 8, c) + within));
            acc[dt] = mfma32<T>(ka, as_operand(sk[t2][4 * u], sk[t2][4 * u + 1], sk[t2][4 * u + 2],
                                               sk[t2][4 * u + 3]), acc[dt]);
          }
    }
    dma_wait();
    __syncthreads();
  };
  int e = 0;
  for (; e + 1 < ntiles; e += 2) {
    tile(e, RingAt<0>{});
    tile(e + 1, RingAt<1>{});
  }
  if (e < ntiles) tile(e, RingAt<0>{});

  // dQ = scale * acc; lane holds query qi, d = 32 dt + 8 j + 4 hh + 0..3
  const float scale = s.scale;
  const rsrc_t rdq = make_rsrc((unsigned short*)a.dq + qrow0 * D, qbytes);
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x2 v2 = {pack2<T>(acc[dt][4 * j] * scale, acc[dt][4 * j + 1] * scale),
                  pack2<T>(acc[dt][4 * j + 2] * scale, acc[dt][4 * j + 3] * scale)};
      bstore8(rdq, (unsigned)(qi * D + 32 * dt + 8 * j + 4 * hh) * 2u, v2);
    }
}

template <class T, int D, int BAND, bool MASK, bool DROP, bool ALIBI>
__global__ __launch_bounds__(Q_NW * 64, FA_Q_OCC) void bwd_q_kernel(BwdArgs a) {
  const GridPos gp = grid_pos(a.s);  // grid: tile_grid over query heads and query blocks
  bwd_q_body<T, D, BAND, MASK, DROP, ALIBI>(a, query_head(a.s, blockIdx.x), gp.b, gp.blk, gp.nblk);
}

// ---------------------------------------------------------------------------
// stages 1 + 2 in one launch (d <= 64; no dropout, score bias or block mask): at these
// head sizes both kernels run two workgroups per CU, so one grid of the
// key-block workgroups followed by the query-block workgroups (each set
// costliest first) lets the query blocks fill the CUs the key blocks' causal
// tail leaves idle. Workgroup ids: [0, nkv) key blocks, then query blocks, each
// set heads fastest, then batch and block in the order tile_grid would choose
// (bo = batch slowest).
// ---------------------------------------------------------------------------
static_assert(KV_NW == Q_NW && FA_Q_OCC == 2, "the fused launch assumes both kernels' workgroup shape");
template <class T, int D, int BAND>
__global__ __launch_bounds__(KV_NW * 64, 2) void bwd_fused_kernel(BwdArgs a, int nkv, int kv_bo, int q_bo) {
  static_assert(D <= 64, "two workgroups per CU only for d <= 64");
  const int id = blockIdx.x;
  if (id < nkv) {
    const int nkb = (a.s.Nk + KV_BKV - 1) / KV_BKV;
    const int hk = id % a.s.Hkv, r = id / a.s.Hkv;
    bwd_kv_body<T, D, BAND, false, false, false>(a, hk, kv_bo ? r / nkb : r % a.s.B, kv_bo ? r % nkb : r / a.s.B);
  } else {
    const int nqb = (a.s.Nq + Q_BM - 1) / Q_BM;
    const int i = id - nkv;
    const int h = query_head(a.s, i % a.s.H), r = i / a.s.H;
    bwd_q_body<T, D, BAND, false, false, false>(a, h, q_bo ? r / nqb : r % a.s.B, q_bo ? r % nqb : r / a.s.B, nqb);
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <class T, int D>
static hipError_t launch_pre_t(const BwdArgs& a, hipStream_t st) {
  const int rpb = 256 / (D / 8);
  const unsigned int blocks = (unsigned)((a.npad + rpb - 1) / rpb) * (unsigned)(a.s.B * a.s.H);
  hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3(blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <class T, int D, int BAND, bool DROP>
static hipError_t launch_kv_t3(const BwdArgs& a, hipStream_t st) {
  BwdArgs la = a;
  const dim3 grid = tile_grid(la.s, a.s.Hkv, (a.s.Nk + KV_BKV - 1) / KV_BKV);
  // workgroup size: eight waves for the split-role instantiations, else four
  auto block = [](bool split) { return dim3(split ? KS_NW * 64 : KV_NW * 64); };
  if (a.s.alibi) {
    if (a.s.mask)
      hipLaunchKernelGGL((bwd_kv_kernel<T, D, BAND, true, DROP, true>), grid,
                         block(kv_split<D, BAND, true, DROP, true>()), 0, st, la);
    else
      hipLaunchKernelGGL((bwd_kv_kernel<T, D, BAND, false, DROP, true>), grid,
                         block(kv_split<D, BAND, false, DROP, true>()), 0, st, la);
  } else {
    if (a.s.mask)
      hipLaunchKernelGGL((bwd_kv_kernel<T, D, BAND, true, DROP, false>), grid,
                         block(kv_split<D, BAND, true, DROP, false>()), 0, st, la);
    else
      hipLaunchKernelGGL((bwd_kv_kernel<T, D, BAND, false, DROP, false>), grid,
                         block(kv_split<D, BAND, false, DROP, false>()), 0, st, la);
  }
  return hipGetLastError();
}

template <class T, int D, bool DROP>
static hipError_t launch_kv_t2(const BwdArgs& a, hipStream_t st) {
  if (a.s.band == 2) return launch_kv_t3<T, D, 2, DROP>(a, st);
  if (a.s.band == 1) return launch_kv_t3<T, D, 1, DROP>(a, st);
  return launch_kv_t3<T, D, 0, DROP>(a, st);
}

template <class T, int D>
static hipError_t launch_kv_t(const BwdArgs& a, hipStream_t st) {
  return a.s.drop_t > 0 ? launch_kv_t2<T, D, true>(a, st) : launch_kv_t2<T, D, false>(a, st);
}

template <class T, int D, int BAND, bool DROP>
static hipError_t launch_q_t3(const BwdArgs& a, hipStream_t st) {
  BwdArgs la = a;
  const dim3 grid = tile_grid(la.s, a.s.H, (a.s.Nq + Q_BM - 1) / Q_BM);
  const dim3 block(Q_NW * 64);
  if (a.s.alibi) {
    if (a.s.mask) hipLaunchKernelGGL((bwd_q_kernel<T, D, BAND, true, DROP, true>), grid, block, 0, st, la);
    else hipLaunchKernelGGL((bwd_q_kernel<T, D, BAND, false, DROP, true>), grid, block, 0, st, la);
  } else {
    if (a.s.mask) hipLaunchKernelGGL((bwd_q_kernel<T, D, BAND, true, DROP, false>), grid, block, 0, st, la);
    else hipLaunchKernelGGL((bwd_q_kernel<T, D, BAND, false, DROP, false>), grid, block, 0, st, la);
  }
  return hipGetLastError();
}

template <class T, int D, bool DROP>
static hipError_t launch_q_t2(const BwdArgs& a, hipStream_t st) {
  if (a.s.band == 2) return launch_q_t3<T, D, 2, DROP>(a, st);
  if (a.s.band == 1) return launch_q_t3<T, D, 1, DROP>(a, st);
  return launch_q_t3<T, D, 0, DROP>(a, st);
}

template <class T, int D>
static hipError_t launch_q_t(const BwdArgs& a, hipStream_t st) {
  return a.s.drop_t > 0 ? launch_q_t2<T, D, true>(a, st) : launch_q_t2<T, D, false>(a, st);
}

template <class T, int D, int BAND>
static hipError_t launch_fused_t3(const BwdArgs& a, hipStream_t st) {
  const int nkb = (a.s.Nk + KV_BKV - 1) / KV_BKV, nqb = (a.s.Nq + Q_BM - 1) / Q_BM;
  const int kv_bo = (long long)a.s.Hkv * nkb >= FA_BATCH_OUTER_MIN ? 1 : 0;
  const int q_bo = (long long)a.s.H * nqb >= FA_BATCH_OUTER_MIN ? 1 : 0;
  const long long nkv = (long long)a.s.Hkv * a.s.B * nkb, nq = (long long)a.s.H * a.s.B * nqb;
  if (nkv + nq > 0x7fffffffLL) return hipErrorInvalidValue;  // the caller checks this first
  const dim3 grid((unsigned)(nkv + nq)), block(KV_NW * 64);
  hipLaunchKernelGGL((bwd_fused_kernel<T, D, BAND>), grid, block, 0, st, a, (int)nkv, kv_bo, q_bo);
  return hipGetLastError();
}

template <class T, int D>
static hipError_t launch_fused_t(const BwdArgs& a, hipStream_t st) {
  if constexpr (D <= 64) {
    if (a.s.drop_t > 0 || a.s.alibi || a.s.mask) return hipErrorInvalidValue;
    if (a.s.band == 2) return launch_fused_t3<T, D, 2>(a, st);
    if (a.s.band == 1) return launch_fused_t3<T, D, 1>(a, st);
    return launch_fused_t3<T, D, 0>(a, st);
  } else {
    return hipErrorInvalidValue;
  }
}

template <class T, int D>
static hipError_t stage_d(int stage, const BwdArgs& a, hipStream_t st) {
  if (stage == 0) return launch_pre_t<T, D>(a, st);
  if (stage == 1) return launch_kv_t<T, D>(a, st);
  if (stage == 3) return launch_fused_t<T, D>(a, st);
  return launch_q_t<T, D>(a, st);
}

template <class T>
static hipError_t stage_t(int stage, const BwdArgs& a, hipStream_t st) {
  if (a.s.d == 32) return stage_d<T, 32>(stage, a, st);
  if (a.s.d == 64) return stage_d<T, 64>(stage, a, st);
  return stage_d<T, 128>(stage, a, st);
}

hipError_t launch_backward_stage(int stage, const BwdArgs& a, int dtype, hipStream_t st) {
  if (dtype == 2) return stage_t<BF16>(stage, a, st);
  return stage_t<F16>(stage, a, st);
}

}  // namespace fa
