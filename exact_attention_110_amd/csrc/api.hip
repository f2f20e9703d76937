// C-ABI entry points of the attention library (declared in include/fa.h).
// Every argument is validated before the HIP runtime is touched; on success
// the kernels are enqueued on the caller's stream and the call returns.
#include <math.h>
#include <stdint.h>

#include "../../include/fa.h"
#include "params.hpp"

namespace {

constexpr size_t kAlign = 256;

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Shape checks shared by every entry point. Sizes must keep per-head offsets
// and row counts inside 32-bit signed range and fit the launch grid.
int check_shape(int B, int H, int Hkv, int N, int d, float scale, int dtype) {
  if (B < 1 || H < 1 || Hkv < 1 || N < 1) return FA_ERR_INVALID_ARG;
  if (H % Hkv != 0) return FA_ERR_INVALID_ARG;
  if (d != 32 && d != 64 && d != 128) return FA_ERR_INVALID_ARG;
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_INVALID_ARG;
  if (!isfinite(scale) || scale < 0.f) return FA_ERR_INVALID_ARG;
  const long long rows = (long long)B * H * N;
  // one head of a tensor must be addressable with 32-bit byte offsets (with room
  // to spare: N * d * 4 < 2^32)
  if (rows > INT32_MAX || (long long)N * d >= (1LL << 30)) return FA_ERR_INVALID_ARG;
  if (B > 65535 || (N + 127) / 128 > 65535) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

fa::AttnShape make_shape(int B, int H, int Hkv, int N, int d, float scale, int causal,
                         const uint8_t* mask) {
  fa::AttnShape s;
  s.B = B;
  s.H = H;
  s.Hkv = Hkv;
  s.N = N;
  s.d = d;
  s.G = H / Hkv;
  s.scale = scale;
  s.causal = causal != 0;
  s.mask = mask;
  s.nb = (N + 127) / 128;
  s.drop_t = 0;
  s.drop_scale = 1.f;
  s.seed0 = s.seed1 = 0;
  return s;
}

// Dropout rate -> byte threshold t = round(256 rate), at most 255 (keep
// probability (256 - t) / 256, kept values scaled by 256 / (256 - t)).
// Returns false for a rate outside [0, 1) or not finite.
bool set_dropout(fa::AttnShape& s, float rate, unsigned long long seed) {
  if (!(rate >= 0.f && rate < 1.f)) return false;  // also rejects NaN
  int t = (int)floorf(rate * 256.f + 0.5f);
  if (t > 255) t = 255;
  s.drop_t = t;
  s.drop_scale = 256.f / (float)(256 - t);
  s.seed0 = (unsigned int)(seed & 0xffffffffull);
  s.seed1 = (unsigned int)(seed >> 32);
  return true;
}

// Block masks are compacted per row / column in LDS lists of 2048 entries.
constexpr int kMaxMaskBlocks = 2048;

// Backward workspace: per (b, h) two float planes (log2-scaled LSE and D) of
// npad = N rounded up to 128 rows, so that whole 128-row blocks load in bounds.
int stats_rows(int N) { return (N + 127) / 128 * 128; }
size_t stats_bytes(int B, int H, int N) {
  return round_up((size_t)B * H * 2 * stats_rows(N) * sizeof(float));
}

int check_backward(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dO, void* dq, void* dk, void* dv, int B, int H, int Hkv, int N,
                   int d, float scale, const uint8_t* block_mask, int dtype, void* workspace,
                   size_t workspace_bytes) {
  if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dO) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || ((uintptr_t)lse & 3u))
    return FA_ERR_INVALID_ARG;
  int st = check_shape(B, H, Hkv, N, d, scale, dtype);
  if (st != FA_OK) return st;
  if (dtype == FA_F32) return FA_ERR_UNSUPPORTED;
  if (block_mask && (N + 127) / 128 > kMaxMaskBlocks) return FA_ERR_UNSUPPORTED;
  if (!workspace || ((uintptr_t)workspace % kAlign) != 0) return FA_ERR_WORKSPACE;
  if ((long long)B * H * 2 * stats_rows(N) > INT32_MAX) return FA_ERR_INVALID_ARG;
  if (workspace_bytes < stats_bytes(B, H, N)) return FA_ERR_WORKSPACE;
  return FA_OK;
}

int forward_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                 int Hkv, int N, int d, float scale, int causal, const uint8_t* block_mask, int dtype,
                 float rate, unsigned long long seed, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || ((uintptr_t)lse & 3u))
    return FA_ERR_INVALID_ARG;
  int st = check_shape(B, H, Hkv, N, d, scale, dtype);
  if (st != FA_OK) return st;
  if (block_mask && (N + 127) / 128 > kMaxMaskBlocks) return FA_ERR_UNSUPPORTED;
  fa::FwdArgs a;
  a.s = make_shape(B, H, Hkv, N, d, scale, causal, block_mask);
  if (!set_dropout(a.s, rate, seed)) return FA_ERR_INVALID_ARG;
  if (a.s.drop_t > 0 && dtype == FA_F32) return FA_ERR_UNSUPPORTED;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  (void)hipGetLastError();  // clear a stale error so the check below sees only this launch
  return fa::launch_forward(a, dtype, (hipStream_t)stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int stage_impl(int stage, const void* q, const void* k, const void* v, const void* o, const float* lse,
               const void* dO, void* dq, void* dk, void* dv, int B, int H, int Hkv, int N, int d,
               float scale, int causal, const uint8_t* block_mask, int dtype, float rate,
               unsigned long long seed, void* workspace, size_t workspace_bytes, void* stream) {
  if (stage < 0 || stage > 2) return FA_ERR_INVALID_ARG;
  int st = check_backward(q, k, v, o, lse, dO, dq, dk, dv, B, H, Hkv, N, d, scale, block_mask,
                          dtype, workspace, workspace_bytes);
  if (st != FA_OK) return st;
  fa::BwdArgs a;
  a.s = make_shape(B, H, Hkv, N, d, scale, causal, block_mask);
  if (!set_dropout(a.s, rate, seed)) return FA_ERR_INVALID_ARG;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.dO = dO;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.stats = (float*)workspace;
  a.npad = stats_rows(N);
  (void)hipGetLastError();
  return fa::launch_backward_stage(stage, a, dtype, (hipStream_t)stream) == hipSuccess ? FA_OK
                                                                                        : FA_ERR_HIP;
}

int backward_impl(const void* q, const void* k, const void* v, const void* o, const float* lse,
                  const void* dO, void* dq, void* dk, void* dv, int B, int H, int Hkv, int N, int d,
                  float scale, int causal, const uint8_t* block_mask, int dtype, float rate,
                  unsigned long long seed, void* workspace, size_t workspace_bytes, void* stream) {
  for (int stage = 0; stage < 3; ++stage) {
    int st = stage_impl(stage, q, k, v, o, lse, dO, dq, dk, dv, B, H, Hkv, N, d, scale, causal,
                        block_mask, dtype, rate, seed, workspace, workspace_bytes, stream);
    if (st != FA_OK) return st;
  }
  return FA_OK;
}

}  // namespace

extern "C" {

size_t fa_backward_workspace_size(int B, int H, int Hkv, int N, int d, int dtype) {
  if (check_shape(B, H, Hkv, N, d, 1.0f, dtype) != FA_OK || dtype == FA_F32) return 0;
  (void)d;
  if ((long long)B * H * 2 * stats_rows(N) > INT32_MAX) return 0;
  return stats_bytes(B, H, N);
}

int fa_forward(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
               int Hkv, int N, int d, float scale, int causal, const uint8_t* block_mask,
               int dtype, void* stream) {
  return forward_impl(q, k, v, o, lse, B, H, Hkv, N, d, scale, causal, block_mask, dtype, 0.f, 0ull,
                      stream);
}

int fa_forward_dropout(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                       int H, int Hkv, int N, int d, float scale, int causal,
                       const uint8_t* block_mask, int dtype, float dropout_rate,
                       unsigned long long seed, void* stream) {
  return forward_impl(q, k, v, o, lse, B, H, Hkv, N, d, scale, causal, block_mask, dtype,
                      dropout_rate, seed, stream);
}

int fa_backward_stage(int stage, const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dO, void* dq, void* dk, void* dv, int B, int H,
                      int Hkv, int N, int d, float scale, int causal, const uint8_t* block_mask,
                      int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return stage_impl(stage, q, k, v, o, lse, dO, dq, dk, dv, B, H, Hkv, N, d, scale, causal,
                    block_mask, dtype, 0.f, 0ull, workspace, workspace_bytes, stream);
}

int fa_backward_stage_dropout(int stage, const void* q, const void* k, const void* v,
                              const void* o, const float* lse, const void* dO, void* dq, void* dk,
                              void* dv, int B, int H, int Hkv, int N, int d, float scale,
                              int causal, const uint8_t* block_mask, int dtype,
                              float dropout_rate, unsigned long long seed, void* workspace,
                              size_t workspace_bytes, void* stream) {
  return stage_impl(stage, q, k, v, o, lse, dO, dq, dk, dv, B, H, Hkv, N, d, scale, causal,
                    block_mask, dtype, dropout_rate, seed, workspace, workspace_bytes, stream);
}

int fa_backward(const void* q, const void* k, const void* v, const void* o, const float* lse,
                const void* dO, void* dq, void* dk, void* dv, int B, int H, int Hkv, int N, int d,
                float scale, int causal, const uint8_t* block_mask, int dtype, void* workspace,
                size_t workspace_bytes, void* stream) {
  return backward_impl(q, k, v, o, lse, dO, dq, dk, dv, B, H, Hkv, N, d, scale, causal, block_mask,
                       dtype, 0.f, 0ull, workspace, workspace_bytes, stream);
}

int fa_backward_dropout(const void* q, const void* k, const void* v, const void* o,
                        const float* lse, const void* dO, void* dq, void* dk, void* dv, int B,
                        int H, int Hkv, int N, int d, float scale, int causal,
                        const uint8_t* block_mask, int dtype, float dropout_rate,
                        unsigned long long seed, void* workspace, size_t workspace_bytes,
                        void* stream) {
  return backward_impl(q, k, v, o, lse, dO, dq, dk, dv, B, H, Hkv, N, d, scale, causal, block_mask,
                       dtype, dropout_rate, seed, workspace, workspace_bytes, stream);
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID_ARG: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported configuration";
    case FA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case FA_ERR_HIP: return "HIP runtime error at launch";
    default: return "unknown status";
  }
}

int fa_version(void) { return 101; }

}  // extern "C"
