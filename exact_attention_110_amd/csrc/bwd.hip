// Backward pass of IO-aware exact attention on gfx950.
//
// The probabilities are never read back from memory: each key block
// recomputes P = exp(S - LSE) tile by tile from Q, K and the saved per-row
// log-sum-exp (nadeemcite.github.io summary "FlashAttention: Fast and
// Memory-Efficient Exact Attention with IO-Awareness", Core Idea item 3; the
// pranaymahendrakar.com lesson "FlashAttention", Researcher tier, "IO
// complexity"). The gradient formulas are the chain rule through the row
// softmax (not on the pages):
//   dV_j = sum_i P_ij dO_i          dP_ij = dO_i . V_j
//   D_i  = sum_d dO_id O_id         dS_ij = P_ij (dP_ij - D_i)
//   dK_j = scale sum_i dS_ij Q_i    dQ_i  = scale sum_j dS_ij K_j
//
// Three stages, all on the caller's stream:
//  0. preprocess: D per query row (fp32) and a cleared fp32 dQ accumulator;
//  1. key-block kernel: one workgroup per 128 keys of one (batch, kv head),
//     four waves of 32 keys. K and V stay in registers as MFMA operands and dK,
//     dV accumulate in registers across every query block (and every query head
//     of a grouped-query group). For each 64-row query block it recomputes
//     S = Q K^T and dP = dO V^T on v_mfma_f32_32x32x16, forms P and dS, adds
//     dO^T P and Q^T dS into dV^T and dK^T (the 32x32 result layout of S is
//     already the B operand of those products; dO^T and Q^T come from LDS with
//     the gfx950 transposing read), stages dS in LDS and adds dS K into the
//     fp32 dQ accumulator with global float atomics;
//  2. convert: dQ = accumulator rounded to the element type.
// Causal masking starts each key block at its diagonal query block; block
// sparsity compacts the nonzero query blocks of the key block's mask column.
#include "common.hpp"
#include "params.hpp"

namespace fa {

constexpr int BWD_NW = 4;              // waves per workgroup
constexpr int BWD_BKV = 32 * BWD_NW;   // keys per workgroup (= mask block)
constexpr int BWD_BQ = 64;             // query rows per step
constexpr int BWD_LIST = 2048;         // capacity of the compacted mask-row list
static_assert(BWD_BKV == 128, "a key-block workgroup must cover exactly one mask block column");

// ---------------------------------------------------------------------------
// stage 0: D = rowsum(dO * O) in fp32, and dq accumulator := 0
// ---------------------------------------------------------------------------
template <class T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdArgs a, int rows) {
  constexpr int CH = D / 8;  // lanes per row, 8 elements each
  constexpr int RPB = 256 / CH;
  const int tid = threadIdx.x;
  const int row = blockIdx.x * RPB + tid / CH;
  const int part = tid % CH;
  float sum = 0.f;
  if (row < rows) {
    const size_t off = (size_t)row * D + part * 8;
    const s16x8 o = gload16((const unsigned short*)a.o + off);
    const s16x8 g = gload16((const unsigned short*)a.dO + off);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      sum = fmaf(to_f32<T>((unsigned short)o[j]), to_f32<T>((unsigned short)g[j]), sum);
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f32x4*>(a.dqacc + off) = z;
    *reinterpret_cast<f32x4*>(a.dqacc + off + 4) = z;
  }
#pragma unroll
  for (int msk = CH / 2; msk >= 1; msk >>= 1) sum += __shfl_xor(sum, msk, 64);
  if (row < rows && part == 0) a.dvec[row] = sum;
}

// ---------------------------------------------------------------------------
// stage 1: per key block, recompute P; accumulate dV, dK; scatter dQ
// ---------------------------------------------------------------------------
template <class T, int D, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(BWD_NW * 64, 1) void bwd_kv_kernel(BwdArgs a) {
  constexpr int QP = D * 2 + 32;        // Q / dO row pitch in LDS (bytes)
  constexpr int KP = D * 2 + 32;        // K row pitch (bytes)
  constexpr int SP = BWD_BQ * 2 + 32;   // dS row pitch: rows are keys, columns queries
  constexpr int QBUF = BWD_BQ * QP;
  constexpr int SBUF = BWD_BKV * SP;
  constexpr int CH = D / 8;
  constexpr int PERQ = BWD_BQ * CH / (BWD_NW * 64);
  constexpr int PERK = BWD_BKV * CH / (BWD_NW * 64);
  static_assert(PERQ >= 1 && (BWD_BQ * CH) % (BWD_NW * 64) == 0, "query loader shape");
  static_assert(PERK >= 1 && (BWD_BKV * CH) % (BWD_NW * 64) == 0, "key loader shape");
  static_assert(2 * BWD_BQ <= BWD_NW * 64, "row statistics loader shape");
  constexpr int NS = D / 16;
  constexpr int ND = D / 32;
  constexpr int NQT = BWD_BQ / 32;     // 32-row query tiles per step
  constexpr int NDQ = NQT * ND;        // 32x32 dQ tiles per step

  // LDS: Q and dO blocks (double-buffered), per-row statistics (double-buffered),
  // the K block, dS (double-buffered) and the compacted mask list
  __shared__ __attribute__((aligned(16))) char smem_raw[4 * QBUF + 2 * 2 * BWD_BQ * 4 + BWD_BKV * KP +
                                                        2 * SBUF + (MASK ? 2 * BWD_LIST + 16 : 16)];
  lds_t* smem = (lds_t*)smem_raw;
  lds_t* qbuf = smem;                      // [2][BQ][QP]
  lds_t* obuf = qbuf + 2 * QBUF;           // dO, [2][BQ][QP]
  lds_t* stat = obuf + 2 * QBUF;           // [2][2][BQ] float: log2-scaled LSE, D
  lds_t* kl = stat + 2 * 2 * BWD_BQ * 4;   // K block, [BKV][KP]
  lds_t* dsl = kl + BWD_BKV * KP;          // dS, [2][BKV][SP]
  __attribute__((address_space(3))) short* blist =
      (__attribute__((address_space(3))) short*)(dsl + 2 * SBUF);
  __attribute__((address_space(3))) int* bcount =
      (__attribute__((address_space(3))) int*)(dsl + 2 * SBUF + (MASK ? 2 * BWD_LIST : 0));

  const AttnShape& s = a.s;
  const int N = s.N;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int g16 = lane >> 4;
  const int roff = 4 * (g16 >> 1) + ((lane & 15) >> 2);   // transposing-read row offset
  const int coff = 16 * (g16 & 1) + 4 * (lane & 3);       // transposing-read column offset
  // grid = (Hkv, key blocks, B); under causal masking block 0 has the most work
  const int hk = blockIdx.x, kblk = blockIdx.y, b = blockIdx.z;
  const int k0 = kblk * BWD_BKV;
  const int kj = k0 + 32 * w + l32;  // this lane's key (its column of S)
  const float c = s.scale * kLog2e;
  const float scale = s.scale;

  // per-head buffer resources: rows past N read as zeros, writes past N are dropped
  const unsigned int head_bytes = (unsigned int)N * D * 2;
  const size_t krow0 = (size_t)(b * s.Hkv + hk) * N;
  const rsrc_t rk = make_rsrc((const unsigned short*)a.k + krow0 * D, head_bytes);
  const rsrc_t rv = make_rsrc((const unsigned short*)a.v + krow0 * D, head_bytes);

  // K^T and V^T operands: lane holds key kj, d = 16 ss + 8 hh + 0..7
  s16x8 kf[NS], vf[NS];
#pragma unroll
  for (int ss = 0; ss < NS; ++ss) {
    kf[ss] = bload16(rk, (unsigned)(kj * D + 16 * ss + 8 * hh) * 2u);
    vf[ss] = bload16(rv, (unsigned)(kj * D + 16 * ss + 8 * hh) * 2u);
  }
  // the whole K block in LDS for the dQ product
#pragma unroll
  for (int r = 0; r < PERK; ++r) {
    const int ci = tid + r * (BWD_NW * 64);
    const int row = ci / CH, col = (ci % CH) * 8;
    lds_write16(kl + row * KP + col * 2, bload16(rk, (unsigned)((k0 + row) * D + col) * 2u));
  }

  // query blocks this key block meets
  const int nqb_all = (N + BWD_BQ - 1) / BWD_BQ;
  const int qb_first = CAUSAL ? k0 / BWD_BQ : 0;
  int nq = nqb_all - qb_first;
  if constexpr (MASK) {
    // mask rows I (128 queries = 2 steps) with mask[I][kblk] != 0, from the first one needed
    const int i_first = qb_first / 2;
    if (w == 0) {
      int cnt = 0;
      for (int j0 = i_first; j0 < s.nb; j0 += 64) {
        const int j = j0 + lane;
        const bool keep = j < s.nb && s.mask[(size_t)j * s.nb + kblk] != 0;
        const unsigned long long bal = __ballot(keep);
        if (keep) blist[cnt + __popcll(bal & ((1ull << lane) - 1ull))] = (short)j;
        cnt += __popcll(bal);
      }
      if (lane == 0) *bcount = cnt;
    }
    __syncthreads();
    const int cnt = *bcount;
    nq = 2 * cnt;
    if (cnt > 0 && 2 * blist[cnt - 1] + 1 >= nqb_all) nq -= 1;  // half block past N
  }
  auto qblock_at = [&](int e) -> int {
    if constexpr (MASK) return 2 * blist[e >> 1] + (e & 1);
    else return qb_first + e;
  };
  const int nsteps = nq * s.G;  // every query head of the group, every query block
  // divisor for step -> (head, query block); a key block with no visible query
  // block (nq = 0, block-sparse only) still issues its first, unused prefetch
  const int nqd = nq > 0 ? nq : 1;

  f32x16 dka[ND], dva[ND];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dka[dt][i] = 0.f;
      dva[dt][i] = 0.f;
    }

  // prefetch of step e's Q and dO rows (registers) and its row statistics:
  // threads 0..BQ-1 take log2-scaled LSE, threads BQ..2BQ-1 take D
  s16x8 qreg[PERQ], oreg[PERQ];
  float sreg = 0.f;
  auto gload_q = [&](int e) {
    const int h = hk * s.G + e / nqd;
    const int q0 = qblock_at(e % nqd) * BWD_BQ;
    const size_t qrow0 = (size_t)(b * s.H + h) * N;
    const rsrc_t rq = make_rsrc((const unsigned short*)a.q + qrow0 * D, head_bytes);
    const rsrc_t rg = make_rsrc((const unsigned short*)a.dO + qrow0 * D, head_bytes);
#pragma unroll
    for (int r = 0; r < PERQ; ++r) {
      const int ci = tid + r * (BWD_NW * 64);
      const int row = ci / CH, col = (ci % CH) * 8;
      const unsigned int off = (unsigned)((q0 + row) * D + col) * 2u;
      qreg[r] = bload16(rq, off);
      oreg[r] = bload16(rg, off);
    }
    {
      // threads 0..BQ-1: LSE in log2 units; BQ..2BQ-1: D. Rows past N, and rows
      // that saw no key, get LSE = +inf so that their P is 0.
      // (two wave-uniform resources; a per-lane choice of base would not be uniform)
      const int q = q0 + (tid % BWD_BQ);
      const float lv = bload_f32(make_rsrc(a.lse + qrow0, (unsigned)N * 4u), (unsigned)q * 4u);
      const float dv = bload_f32(make_rsrc(a.dvec + qrow0, (unsigned)N * 4u), (unsigned)q * 4u);
      const float L = (q < N && lv != -INFINITY) ? lv * kLog2e : INFINITY;
      sreg = tid < BWD_BQ ? L : dv;
    }
  };
  auto lstore_q = [&](int buf) {
#pragma unroll
    for (int r = 0; r < PERQ; ++r) {
      const int ci = tid + r * (BWD_NW * 64);
      const int row = ci / CH, col = (ci % CH) * 8;
      lds_write16(qbuf + buf * QBUF + row * QP + col * 2, qreg[r]);
      lds_write16(obuf + buf * QBUF + row * QP + col * 2, oreg[r]);
    }
    if (tid < 2 * BWD_BQ)
      *((__attribute__((address_space(3))) float*)(stat + buf * 2 * BWD_BQ * 4) + tid) = sreg;
  };

  // dQ(q x d) += dS(q x key) K(key x d) over the block's 128 keys for the step
  // whose dS sits in buffer sb; each wave takes whole 32x32 tiles of the 64 x D result
  auto dq_phase = [&](int e, int sb) {
    const int h = hk * s.G + e / nqd;
    const int q0 = qblock_at(e % nqd) * BWD_BQ;
    const size_t qrow0 = (size_t)(b * s.H + h) * N;
    const rsrc_t racc = make_rsrc(a.dqacc + qrow0 * D, (unsigned)N * D * 4u);
    const lds_t* ds = dsl + sb * SBUF;
    for (int ti = w; ti < NDQ; ti += BWD_NW) {
      const int qt = ti % NQT, dt = ti / NQT;
      f32x16 acc;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
      for (int u = 0; u < BWD_BKV / 16; ++u) {
        const lds_t* sp = ds + (16 * u + roff) * SP + (32 * qt + coff) * 2;
        const lds_t* kp = kl + (16 * u + roff) * KP + (32 * dt + coff) * 2;
        const s16x8 sa = concat(lds_read_tr(sp), lds_read_tr(sp + 8 * SP));
        const s16x8 kb = concat(lds_read_tr(kp), lds_read_tr(kp + 8 * KP));
        acc = mfma32<T>(sa, kb, acc);
      }
      // acc: column d = 32 dt + l32, rows q0 + 32 qt + 8 (i / 4) + 4 hh + i % 4
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int q = q0 + 32 * qt + 8 * (i >> 2) + 4 * hh + (i & 3);
        batomic_add(racc, (unsigned)(q * D + 32 * dt + l32) * 4u, acc[i]);
      }
    }
  };

  // loads are issued on every path (indices clamped; buffer loads make a
  // redundant block harmless) so that outstanding loads are counted exactly
  gload_q(0);
  lstore_q(0);
  __syncthreads();

  for (int e = 0; e < nsteps; ++e) {
    const int buf = e & 1;
    const int q0 = qblock_at(e % nqd) * BWD_BQ;
    gload_q(e + 1 < nsteps ? e + 1 : e);

    const lds_t* qb = qbuf + buf * QBUF;
    const lds_t* ob = obuf + buf * QBUF;
    const __attribute__((address_space(3))) float* lsel =
        (const __attribute__((address_space(3))) float*)(stat + buf * 2 * BWD_BQ * 4);
    const __attribute__((address_space(3))) float* ddl = lsel + BWD_BQ;

    // S = Q K^T and dP = dO V^T for this wave's 32 keys
    f32x16 sc[NQT], dp[NQT];
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sc[qt][i] = 0.f;
        dp[qt][i] = 0.f;
      }
#pragma unroll
    for (int ss = 0; ss < NS; ++ss)
#pragma unroll
      for (int qt = 0; qt < NQT; ++qt) {
        const s16x8 qa = lds_read16(qb + (32 * qt + l32) * QP + (16 * ss + 8 * hh) * 2);
        sc[qt] = mfma32<T>(qa, kf[ss], sc[qt]);
        const s16x8 ga = lds_read16(ob + (32 * qt + l32) * QP + (16 * ss + 8 * hh) * 2);
        dp[qt] = mfma32<T>(ga, vf[ss], dp[qt]);
      }

    // P and dS; element i of tile qt is query q0 + 32 qt + 8 (i / 4) + 4 hh + i % 4, key kj
    const bool need_mask = (CAUSAL && q0 < k0 + BWD_BKV) || (k0 + BWD_BKV > N);
    unsigned int pk[NQT][8], sk[NQT][8];
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        const f32x4 L4 = *(const __attribute__((address_space(3))) f32x4*)(lsel + 32 * qt + 8 * j4 + 4 * hh);
        const f32x4 D4 = *(const __attribute__((address_space(3))) f32x4*)(ddl + 32 * qt + 8 * j4 + 4 * hh);
        float p[4], d2[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 4 * j4 + r;
          float pv = fast_exp2(fmaf(sc[qt][i], c, -L4[r]));
          if (need_mask) {
            const int q = q0 + 32 * qt + 8 * j4 + 4 * hh + r;
            if ((CAUSAL && kj > q) || kj >= N) pv = 0.f;
          }
          p[r] = pv;
          d2[r] = pv * (dp[qt][i] - D4[r]) * scale;
        }
        pk[qt][2 * j4] = pack2<T>(p[0], p[1]);
        pk[qt][2 * j4 + 1] = pack2<T>(p[2], p[3]);
        sk[qt][2 * j4] = pack2<T>(d2[0], d2[1]);
        sk[qt][2 * j4 + 1] = pack2<T>(d2[2], d2[3]);
      }
    // dS into LDS as [key][query]: 4 consecutive queries per 8-byte write
    lds_t* dsw = dsl + buf * SBUF;
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x2 v2 = {sk[qt][2 * j], sk[qt][2 * j + 1]};
        lds_write8(dsw + (32 * w + l32) * SP + (32 * qt + 8 * j + 4 * hh) * 2, v2);
      }

    // dV^T(d x key) += dO^T(d x q) P(q x key); dK^T += Q^T dS. B operand k-slot j of
    // step (qt, u) is query 32 qt + 16 u + 8 (j / 4) + 4 hh + j % 4.
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
      for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int off = (32 * qt + 16 * u + roff) * QP + (32 * dt + coff) * 2;
          const s16x8 ga = concat(lds_read_tr(ob + off), lds_read_tr(ob + off + 8 * QP));
          const s16x8 qa = concat(lds_read_tr(qb + off), lds_read_tr(qb + off + 8 * QP));
          dva[dt] = mfma32<T>(ga, as_operand(pk[qt][4 * u], pk[qt][4 * u + 1], pk[qt][4 * u + 2],
                                             pk[qt][4 * u + 3]), dva[dt]);
          dka[dt] = mfma32<T>(qa, as_operand(sk[qt][4 * u], sk[qt][4 * u + 1], sk[qt][4 * u + 2],
                                             sk[qt][4 * u + 3]), dka[dt]);
        }

    // dQ of the previous step: its dS was completed by every wave before the
    // barrier that ended that step
    if (e > 0) dq_phase(e - 1, buf ^ 1);

    lstore_q(buf ^ 1);
    __syncthreads();
  }
  if (nsteps > 0) dq_phase(nsteps - 1, (nsteps - 1) & 1);

  // dK^T / dV^T: lane holds key kj, d = 32 dt + 8 j + 4 hh + 0..3
  const rsrc_t rdk = make_rsrc((unsigned short*)a.dk + krow0 * D, head_bytes);
  const rsrc_t rdv = make_rsrc((unsigned short*)a.dv + krow0 * D, head_bytes);
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x2 kv = {pack2<T>(dka[dt][4 * j], dka[dt][4 * j + 1]),
                  pack2<T>(dka[dt][4 * j + 2], dka[dt][4 * j + 3])};
      u32x2 vv = {pack2<T>(dva[dt][4 * j], dva[dt][4 * j + 1]),
                  pack2<T>(dva[dt][4 * j + 2], dva[dt][4 * j + 3])};
      const unsigned int off = (unsigned)(kj * D + 32 * dt + 8 * j + 4 * hh) * 2u;
      bstore8(rdk, off, kv);
      bstore8(rdv, off, vv);
    }
}

// ---------------------------------------------------------------------------
// stage 2: dq = accumulator, rounded to the element type
// ---------------------------------------------------------------------------
template <class T>
__global__ __launch_bounds__(256) void bwd_dq_kernel(BwdArgs a, size_t n8) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (size_t)gridDim.x * 256) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(a.dqacc + 8 * i);
    const f32x4 y = *reinterpret_cast<const f32x4*>(a.dqacc + 8 * i + 4);
    u32x4 r = {pack2<T>(x[0], x[1]), pack2<T>(x[2], x[3]), pack2<T>(y[0], y[1]),
               pack2<T>(y[2], y[3])};
    *reinterpret_cast<u32x4*>((unsigned short*)a.dq + 8 * i) = r;
  }
}

template <class T, int D>
static hipError_t launch_kv_t(const BwdArgs& a, hipStream_t st) {
  const dim3 grid(a.s.Hkv, (a.s.N + BWD_BKV - 1) / BWD_BKV, a.s.B);
  const dim3 block(BWD_NW * 64);
  const bool causal = a.s.causal != 0, mask = a.s.mask != nullptr;
  if (causal && mask) hipLaunchKernelGGL((bwd_kv_kernel<T, D, true, true>), grid, block, 0, st, a);
  else if (causal) hipLaunchKernelGGL((bwd_kv_kernel<T, D, true, false>), grid, block, 0, st, a);
  else if (mask) hipLaunchKernelGGL((bwd_kv_kernel<T, D, false, true>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((bwd_kv_kernel<T, D, false, false>), grid, block, 0, st, a);
  return hipGetLastError();
}

template <class T, int D>
static hipError_t launch_pre_t(const BwdArgs& a, hipStream_t st) {
  const int rows = a.s.B * a.s.H * a.s.N;
  const int rpb = 256 / (D / 8);
  hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3((rows + rpb - 1) / rpb), dim3(256), 0, st, a, rows);
  return hipGetLastError();
}

template <class T>
static hipError_t launch_dq_t(const BwdArgs& a, hipStream_t st) {
  const size_t n8 = (size_t)a.s.B * a.s.H * a.s.N * a.s.d / 8;
  size_t blocks = (n8 + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL((bwd_dq_kernel<T>), dim3((unsigned)blocks), dim3(256), 0, st, a, n8);
  return hipGetLastError();
}

template <class T>
static hipError_t stage_t(int stage, const BwdArgs& a, hipStream_t st) {
  const int d = a.s.d;
  if (stage == 0) {
    if (d == 32) return launch_pre_t<T, 32>(a, st);
    if (d == 64) return launch_pre_t<T, 64>(a, st);
    return launch_pre_t<T, 128>(a, st);
  }
  if (stage == 1) {
    if (d == 32) return launch_kv_t<T, 32>(a, st);
    if (d == 64) return launch_kv_t<T, 64>(a, st);
    return launch_kv_t<T, 128>(a, st);
  }
  return launch_dq_t<T>(a, st);
}

hipError_t launch_backward_stage(int stage, const BwdArgs& a, int dtype, hipStream_t st) {
  if (dtype == 2) return stage_t<BF16>(stage, a, st);
  return stage_t<F16>(stage, a, st);
}

}  // namespace fa
