// Kernel argument blocks and the internal launch interface shared by the
// forward, backward and C-ABI translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

// A band side that never binds: larger than any sequence, small enough that
// row + offset +- kUnbounded stays inside int32.
constexpr int kUnbounded = 1 << 30;

struct AttnShape {
  int B, H, Hkv;
  int Nq, Nk;     // query rows and keys per sequence (packed batches: the longest)
  int d;
  int G;          // H / Hkv, query heads per kv head
  float scale;    // multiplies Q K^T
  // band mask around the query's position p = i + (nk - nq) of its sequence:
  // key j visible only if p - wl <= j <= p + wr; an unbounded side holds
  // kUnbounded. band: 0 none (every key visible), 1 upper edge only (wl
  // unbounded; causal masking is wr = 0), 2 both edges. The kernels are
  // instantiated per band kind, so causal attention pays nothing for the
  // lower edge.
  int band;
  int wl, wr;
  const uint8_t* mask;  // NULL or uint8 [nbq][nbk] (fixed lengths only)
  // element masks of partial blocks (only with mask): btile NULL, or int32
  // [nbq][nbk] with -1 for a kept block whose every element is visible and
  // t >= 0 for one whose elements are tile t of bits: uint32 [ntiles][128][4],
  // bit j % 32 of word j / 32 of row i set = key j of the block visible to
  // query i of the block. Tiles are read through a buffer resource of ntiles
  // tiles, so an index past the last tile reads zeros (no element visible).
  const int* btile;
  const unsigned int* bits;
  int ntiles;
  // NULL or float [H]: ALiBi slopes, s_ij += -alibi[h] * |i + (nk - nq) - j|
  const float* alibi;
  int nbq, nbk;   // ceil(Nq / 128), ceil(Nk / 128)
  // packed variable-length batches (NULL for fixed lengths): sequence b holds
  // rows cu_q[b] .. cu_q[b + 1] - 1 of every query head's [tq][d] plane and
  // keys cu_k[b] .. cu_k[b + 1] - 1 of every kv head's [tk][d] plane
  const int* cu_q;
  const int* cu_k;
  int tq, tk;
  // dropout on the probabilities (used only by the kernels built for it): an
  // element is kept iff its generator byte >= drop_t, and kept values are
  // multiplied by drop_scale = 256 / (256 - drop_t); the generator key is
  // (seed0, seed1)
  int drop_t;
  float drop_scale;
  unsigned int seed0, seed1;
  // launch-grid layout, set by the launcher (tile_grid): 0 = (heads, B, blocks),
  // 1 = (heads, blocks, B)
  int batch_outer;
};

struct FwdArgs {
  AttnShape s;
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
};

struct BwdArgs {
  AttnShape s;
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dO;
  void* dq;
  void* dk;
  void* dv;
  // workspace, [B][H][2][npad] float: plane 0 the log2-scaled LSE (+inf for a
  // row that saw no key and for the padding rows past the sequence), plane 1
  // -D = -rowsum(dO * O) (0 for padding rows); npad = Nq rounded up to 128
  float* stats;
  int npad;
};

// One sequence of a batch as seen by a workgroup: its lengths, the causal
// offset and where its rows start. Fixed lengths: Q is [B][H][Nq][d], K and V
// [B][Hkv][Nk][d]. Packed batches: Q is [H][tq][d], K and V [Hkv][tk][d], with
// the sequence's rows at cu_q[b] and cu_k[b]. The offsets read from cu_q and
// cu_k are clamped to the planes and the lengths to Nq, Nk, so that offsets
// that break their contract cannot move an access outside the buffers.
struct SeqView {
  int nq, nk;       // query rows and keys of this sequence
  int off;          // nk - nq: a causal query i sees keys j <= i + off
  size_t qrow0;     // first row of query head h (rows of d elements)
  size_t krow0;     // first row of kv head hk
  size_t qstride;   // rows from one query head to the next
};

__device__ __forceinline__ SeqView seq_view(const AttnShape& s, int b, int h, int hk) {
  SeqView v;
  if (s.cu_q) {
    const int q0 = min(max(s.cu_q[b], 0), s.tq), q1 = min(max(s.cu_q[b + 1], q0), s.tq);
    const int k0 = min(max(s.cu_k[b], 0), s.tk), k1 = min(max(s.cu_k[b + 1], k0), s.tk);
    v.nq = min(q1 - q0, s.Nq);
    v.nk = min(k1 - k0, s.Nk);
    v.qrow0 = (size_t)h * s.tq + q0;
    v.krow0 = (size_t)hk * s.tk + k0;
    v.qstride = (size_t)s.tq;
  } else {
    v.nq = s.Nq;
    v.nk = s.Nk;
    v.qrow0 = (size_t)(b * s.H + h) * s.Nq;
    v.krow0 = (size_t)(b * s.Hkv + hk) * s.Nk;
    v.qstride = (size_t)s.Nq;
  }
  v.off = v.nk - v.nq;
  return v;
}

// Launch grid of the tiled kernels, one workgroup per (head, batch, 128- or
// 256-row block). Consecutive workgroups take different heads, so the
// round-robin over the 8 XCDs keeps each head on one XCD's L2. The block index
// varies slowest, (heads, B, blocks), so that under causal masking every head
// and batch starts its costliest block before any cheaper one; when one batch
// alone holds FA_BATCH_OUTER_MIN workgroups or more (several times what the chip
// runs at once, so the order within a batch already balances the load) the
// batch varies slowest instead, (heads, blocks, B), which keeps the running
// workgroups on fewer batches and so fewer K/V heads per XCD's L2.
#ifndef FA_BATCH_OUTER_MIN
#define FA_BATCH_OUTER_MIN 1024
#endif
inline dim3 tile_grid(AttnShape& s, int heads, int nblk) {
  s.batch_outer = (long long)heads * nblk >= FA_BATCH_OUTER_MIN ? 1 : 0;
  return s.batch_outer ? dim3(heads, nblk, s.B) : dim3(heads, s.B, nblk);
}

// Query head of grid column x (columns run fastest): the G query heads of kv
// head g take columns g, g + Hkv, g + 2 Hkv, ..., so with the round-robin over
// the 8 XCDs a group's heads share one XCD's L2 and its K/V tiles instead of
// each XCD fetching them; the identity when G = 1.
#ifndef FA_GROUP_HEADS_BY_XCD
#define FA_GROUP_HEADS_BY_XCD 1
#endif
__device__ __forceinline__ int query_head(const AttnShape& s, int x) {
  return FA_GROUP_HEADS_BY_XCD ? (x % s.Hkv) * s.G + x / s.Hkv : x;
}

struct GridPos {
  int b;     // batch (sequence)
  int blk;   // block index in launch order
  int nblk;  // blocks per head
};
__device__ __forceinline__ GridPos grid_pos(const AttnShape& s) {
  return s.batch_outer ? GridPos{(int)blockIdx.z, (int)blockIdx.y, (int)gridDim.y}
                       : GridPos{(int)blockIdx.y, (int)blockIdx.z, (int)gridDim.z};
}

// FP8 forward: q, k, v hold OCP E4M3 codes; the real inputs are code value
// times the tensor's descale. o is 16-bit (out dtype), lse float.
struct Fp8FwdArgs {
  AttnShape s;
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  float q_descale, k_descale, v_descale;
};

// Internal launchers (return a hipError_t from the launch).
// forward_rows: query rows per wave of the 16-bit forward kernel a call takes
// by default (64 or 32; 0 for float32 inputs). launch_forward: rows 0 takes
// that choice, 32 or 64 forces a kernel (64 with a block mask or score bias is
// hipErrorInvalidValue; the caller rejects it first).
int forward_rows(const AttnShape& s, int dtype);
hipError_t launch_forward(const FwdArgs& a, int dtype, hipStream_t stream, int rows);
hipError_t launch_forward_fp8(const Fp8FwdArgs& a, int out_dtype, hipStream_t stream);
// stage 0: D and the log2-scaled LSE; 1: dK, dV; 2: dQ; 3: stages 1 and 2 in one
// launch (d <= 64; no dropout, score bias or block mask)
hipError_t launch_backward_stage(int stage, const BwdArgs& a, int dtype, hipStream_t stream);

}  // namespace fa
