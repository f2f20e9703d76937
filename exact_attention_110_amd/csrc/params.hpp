// Kernel argument blocks and the internal launch interface shared by the
// forward, backward and C-ABI translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

struct AttnShape {
  int B, H, Hkv, N, d;
  int G;          // H / Hkv, query heads per kv head
  float scale;    // multiplies Q K^T
  int causal;     // key j visible to query i only if j <= i
  const uint8_t* mask;  // NULL or uint8 [nb][nb], nb = ceil(N / 128)
  int nb;         // ceil(N / 128)
  // dropout on the probabilities (used only by the kernels built for it): an
  // element is kept iff its generator byte >= drop_t, and kept values are
  // multiplied by drop_scale = 256 / (256 - drop_t); the generator key is
  // (seed0, seed1)
  int drop_t;
  float drop_scale;
  unsigned int seed0, seed1;
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
  // row that saw no key and for the padding rows N..npad-1), plane 1 D =
  // rowsum(dO * O) (0 for padding rows); npad = N rounded up to 128
  float* stats;
  int npad;
};

// Internal launchers (return a hipError_t from the launch).
hipError_t launch_forward(const FwdArgs& a, int dtype, hipStream_t stream);
hipError_t launch_backward_stage(int stage, const BwdArgs& a, int dtype, hipStream_t stream);

}  // namespace fa
