// C-ABI entry points of the attention library (declared in include/fa.h).
// Every argument is validated before the HIP runtime is touched; on success
// the kernels are enqueued on the caller's stream and the call returns.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/fa.h"
#include "params.hpp"

namespace {

constexpr size_t kAlign = 256;

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Sequence geometry of a call: fixed lengths (cu_q == NULL; Q [B][H][Nq][d],
// K and V [B][Hkv][Nk][d]) or a packed batch (Q [H][tq][d], K and V
// [Hkv][tk][d], sequence b at rows cu_q[b], cu_k[b], Nq and Nk its longest).
struct Geo {
  int B, H, Hkv, Nq, Nk, d;
  const int* cu_q;
  const int* cu_k;
  int tq, tk;
};

Geo fixed_geo(int B, int H, int Hkv, int Nq, int Nk, int d) {
  return Geo{B, H, Hkv, Nq, Nk, d, nullptr, nullptr, 0, 0};
}

// Shape checks shared by every entry point. Sizes must keep per-sequence byte
// offsets inside 32 bits, row counts inside 32-bit signed range and the
// launch grid inside its limits.
int check_shape(const Geo& g, float scale, int dtype) {
  if (g.B < 1 || g.H < 1 || g.Hkv < 1 || g.Nq < 1 || g.Nk < 1) return FA_ERR_INVALID_ARG;
  if (g.H % g.Hkv != 0) return FA_ERR_INVALID_ARG;
  if (g.d != 32 && g.d != 64 && g.d != 128) return FA_ERR_INVALID_ARG;
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_INVALID_ARG;
  if (!isfinite(scale) || scale < 0.f) return FA_ERR_INVALID_ARG;
  long long rq, rk;
  if (g.cu_q || g.cu_k) {
    if (!g.cu_q || !g.cu_k || ((uintptr_t)g.cu_q & 3u) || ((uintptr_t)g.cu_k & 3u)) return FA_ERR_INVALID_ARG;
    if (g.tq < 0 || g.tk < 0) return FA_ERR_INVALID_ARG;
    rq = (long long)g.H * g.tq;
    rk = (long long)g.Hkv * g.tk;
  } else {
    rq = (long long)g.B * g.H * g.Nq;
    rk = (long long)g.B * g.Hkv * g.Nk;
  }
  // one sequence of a head must be addressable with 32-bit byte offsets (with
  // room to spare: n * d * 4 < 2^32)
  if (rq > INT32_MAX || rk > INT32_MAX) return FA_ERR_INVALID_ARG;
  if ((long long)g.Nq * g.d >= (1LL << 30) || (long long)g.Nk * g.d >= (1LL << 30)) return FA_ERR_INVALID_ARG;
  if (g.B > 65535 || (g.Nq + 127) / 128 > 65535 || (g.Nk + 127) / 128 > 65535) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

// Band limits from the causal flag and a (left, right) window, -1 unbounded:
// causal masking is the right limit 0. on: 0 no band, 1 upper edge only, 2 a
// lower edge too. Returns false for a limit below -1.
struct Band {
  int on, wl, wr;
};

bool make_band(int causal, int window_left, int window_right, Band* b) {
  if (window_left < -1 || window_right < -1) return false;
  const int wl = window_left < 0 ? fa::kUnbounded : (window_left < fa::kUnbounded ? window_left : fa::kUnbounded);
  int wr = window_right < 0 ? fa::kUnbounded : (window_right < fa::kUnbounded ? window_right : fa::kUnbounded);
  if (causal) wr = 0;
  b->on = window_left >= 0 ? 2 : (causal || window_right >= 0 ? 1 : 0);
  b->wl = wl;
  b->wr = wr;
  return true;
}

// Element masks of partial blocks (fa_forward_bitmask / fa_backward_bitmask).
struct ElemMask {
  const int32_t* btile;
  const uint32_t* bits;
  int ntiles;
};
constexpr int kMaxTiles = 1 << 21;  // tile offsets (2 KB per tile) stay inside 32 bits

// NULL (no element mask) or a well-formed one: a block mask beside it, block_tile
// 4-byte aligned, tile_bits 16-byte aligned and present when there are tiles.
int check_elem(const ElemMask* em, const uint8_t* block_mask) {
  if (!em) return FA_OK;
  if (!block_mask || !em->btile || ((uintptr_t)em->btile & 3u)) return FA_ERR_INVALID_ARG;
  if (em->ntiles < 0 || em->ntiles > kMaxTiles) return FA_ERR_INVALID_ARG;
  if (em->ntiles > 0 && (!em->bits || !aligned16(em->bits))) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

void set_elem(fa::AttnShape& s, const ElemMask* em) {
  s.btile = em ? em->btile : nullptr;
  s.bits = em && em->ntiles > 0 ? em->bits : nullptr;
  s.ntiles = em ? em->ntiles : 0;
}

fa::AttnShape make_shape(const Geo& g, float scale, const Band& band, const uint8_t* mask) {
  fa::AttnShape s;
  s.B = g.B;
  s.H = g.H;
  s.Hkv = g.Hkv;
  s.Nq = g.Nq;
  s.Nk = g.Nk;
  s.d = g.d;
  s.G = g.H / g.Hkv;
  s.scale = scale;
  s.band = band.on;
  s.wl = band.wl;
  s.wr = band.wr;
  s.mask = mask;
  s.nbq = (g.Nq + 127) / 128;
  s.nbk = (g.Nk + 127) / 128;
  s.cu_q = g.cu_q;
  s.cu_k = g.cu_k;
  s.tq = g.tq;
  s.tk = g.tk;
  s.drop_t = 0;
  s.drop_scale = 1.f;
  s.seed0 = s.seed1 = 0;
  s.alibi = nullptr;
  s.btile = nullptr;
  s.bits = nullptr;
  s.ntiles = 0;
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

bool mask_too_long(const Geo& g, const uint8_t* mask) {
  return mask && ((g.Nq + 127) / 128 > kMaxMaskBlocks || (g.Nk + 127) / 128 > kMaxMaskBlocks);
}

// Backward workspace: per (b, h) two float planes (log2-scaled LSE and D) of
// npad = Nq rounded up to 128 rows, so that whole 128-row blocks load in bounds.
int stats_rows(int N) { return (N + 127) / 128 * 128; }
size_t stats_bytes(int B, int H, int N) {
  return round_up((size_t)B * H * 2 * stats_rows(N) * sizeof(float));
}

int check_backward(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dO, void* dq, void* dk, void* dv, const Geo& g, float scale,
                   const uint8_t* block_mask, int dtype, void* workspace, size_t workspace_bytes) {
  if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dO) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || ((uintptr_t)lse & 3u))
    return FA_ERR_INVALID_ARG;
  int st = check_shape(g, scale, dtype);
  if (st != FA_OK) return st;
  if (dtype == FA_F32) return FA_ERR_UNSUPPORTED;
  if (mask_too_long(g, block_mask)) return FA_ERR_UNSUPPORTED;
  if (!workspace || ((uintptr_t)workspace % kAlign) != 0) return FA_ERR_WORKSPACE;
  if ((long long)g.B * g.H * 2 * stats_rows(g.Nq) > INT32_MAX) return FA_ERR_INVALID_ARG;
  if (workspace_bytes < stats_bytes(g.B, g.H, g.Nq)) return FA_ERR_WORKSPACE;
  return FA_OK;
}

int forward_impl(const void* q, const void* k, const void* v, void* o, float* lse, const Geo& g,
                 float scale, int causal, int window_left, int window_right, const float* alibi,
                 const uint8_t* block_mask, int dtype, float rate, unsigned long long seed, void* stream,
                 int rows = 0, const ElemMask* em = nullptr) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || ((uintptr_t)lse & 3u) ||
      ((uintptr_t)alibi & 3u))
    return FA_ERR_INVALID_ARG;
  int st = check_shape(g, scale, dtype);
  if (st != FA_OK) return st;
  if (mask_too_long(g, block_mask)) return FA_ERR_UNSUPPORTED;
  if (check_elem(em, block_mask) != FA_OK) return FA_ERR_INVALID_ARG;
  Band band;
  if (!make_band(causal, window_left, window_right, &band)) return FA_ERR_INVALID_ARG;
  fa::FwdArgs a;
  a.s = make_shape(g, scale, band, block_mask);
  a.s.alibi = alibi;
  set_elem(a.s, em);
  if (!set_dropout(a.s, rate, seed)) return FA_ERR_INVALID_ARG;
  if (a.s.drop_t > 0 && dtype == FA_F32) return FA_ERR_UNSUPPORTED;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  if (rows != 0 && rows != 32 && rows != 64) return FA_ERR_INVALID_ARG;
  if (dtype == FA_F32 && rows != 0) return FA_ERR_UNSUPPORTED;
  if (rows == 64 && (block_mask || alibi)) return FA_ERR_UNSUPPORTED;
  (void)hipGetLastError();  // clear a stale error so the check below sees only this launch
  return fa::launch_forward(a, dtype, (hipStream_t)stream, rows) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

// The one-launch backward (stage 3) covers d <= 64 without dropout, score bias
// or block mask, with all its workgroups in one grid dimension.
bool fused_ok(const Geo& g, float rate, const float* alibi, const uint8_t* block_mask) {
  const long long nkb = (g.Nk + 127) / 128, nqb = (g.Nq + 127) / 128;
  const long long wgs = (long long)g.B * ((long long)g.Hkv * nkb + (long long)g.H * nqb);
  return g.d <= 64 && rate == 0.f && alibi == nullptr && block_mask == nullptr && wgs <= 0x7fffffffLL;
}

int stage_impl(int stage, const void* q, const void* k, const void* v, const void* o, const float* lse,
               const void* dO, void* dq, void* dk, void* dv, const Geo& g, float scale, int causal,
               int window_left, int window_right, const float* alibi, const uint8_t* block_mask, int dtype,
               float rate, unsigned long long seed, void* workspace, size_t workspace_bytes, void* stream,
               const ElemMask* em = nullptr) {
  if (stage < 0 || stage > 3) return FA_ERR_INVALID_ARG;
  if ((uintptr_t)alibi & 3u) return FA_ERR_INVALID_ARG;
  if (check_elem(em, block_mask) != FA_OK) return FA_ERR_INVALID_ARG;
  int st = check_backward(q, k, v, o, lse, dO, dq, dk, dv, g, scale, block_mask, dtype, workspace,
                          workspace_bytes);
  if (st != FA_OK) return st;
  Band band;
  if (!make_band(causal, window_left, window_right, &band)) return FA_ERR_INVALID_ARG;
  fa::BwdArgs a;
  a.s = make_shape(g, scale, band, block_mask);
  a.s.alibi = alibi;
  set_elem(a.s, em);
  if (!set_dropout(a.s, rate, seed)) return FA_ERR_INVALID_ARG;
  if (stage == 3 && (!fused_ok(g, 0.f, alibi, block_mask) || a.s.drop_t > 0)) return FA_ERR_UNSUPPORTED;
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
  a.npad = stats_rows(g.Nq);
  (void)hipGetLastError();
  return fa::launch_backward_stage(stage, a, dtype, (hipStream_t)stream) == hipSuccess ? FA_OK
                                                                                        : FA_ERR_HIP;
}

int backward_impl(const void* q, const void* k, const void* v, const void* o, const float* lse,
                  const void* dO, void* dq, void* dk, void* dv, const Geo& g, float scale, int causal,
                  int window_left, int window_right, const float* alibi, const uint8_t* block_mask,
                  int dtype, float rate, unsigned long long seed, void* workspace, size_t workspace_bytes,
                  void* stream, const ElemMask* em = nullptr) {
  // For d <= 64 without dropout, score bias or block mask, the dK/dV and dQ
  // kernels run two workgroups per CU each and go out as one launch (stage 3),
  // so the dQ workgroups fill the CUs the dK/dV kernel's causal tail leaves
  // idle (a block-sparse grid is balanced already and gains nothing).
  fa::AttnShape probe = make_shape(g, scale, Band{0, 0, 0}, nullptr);
  if (!set_dropout(probe, rate, seed)) return FA_ERR_INVALID_ARG;
  const bool fused = fused_ok(g, probe.drop_t > 0 ? rate : 0.f, alibi, block_mask);
  const int stages[3] = {0, fused ? 3 : 1, 2};
  for (int i = 0; i < (fused ? 2 : 3); ++i) {
    const int stage = stages[i];
    int st = stage_impl(stage, q, k, v, o, lse, dO, dq, dk, dv, g, scale, causal, window_left, window_right,
                        alibi, block_mask, dtype, rate, seed, workspace, workspace_bytes, stream, em);
    if (st != FA_OK) return st;
  }
  return FA_OK;
}

// Device scratch of the allocation-free backward entry point: the two
// statistics planes of the backward workspace, in a file-scope device array
// that every GPU the library runs on holds until the process ends. Host code
// never passes `scratch` itself (on the host it only names the symbol): the
// first call on a device looks up the array's device address with
// hipGetSymbolAddress (with that device current) and keeps it per device.
constexpr size_t kScratchBytes = (size_t)FA_NOALLOC_SCRATCH_BYTES;
static __device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch[kMaxDevices] = {};

// The scratch array's device address on the current device, or NULL.
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" {

size_t fa_backward_workspace_size(int B, int H, int Hkv, int N, int d, int dtype) {
  if (check_shape(fixed_geo(B, H, Hkv, N, N, d), 1.0f, dtype) != FA_OK || dtype == FA_F32) return 0;
  if ((long long)B * H * 2 * stats_rows(N) > INT32_MAX) return 0;
  return stats_bytes(B, H, N);
}

int fa_forward(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
               int Hkv, int N, int d, float scale, int causal, const uint8_t* block_mask,
               int dtype, void* stream) {
  return forward_impl(q, k, v, o, lse, fixed_geo(B, H, Hkv, N, N, d), scale, causal, -1, -1, nullptr, block_mask, dtype,
                      0.f, 0ull, stream);
}

int fa_forward_dropout(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                       int H, int Hkv, int N, int d, float scale, int causal,
                       const uint8_t* block_mask, int dtype, float dropout_rate,
                       unsigned long long seed, void* stream) {
  return forward_impl(q, k, v, o, lse, fixed_geo(B, H, Hkv, N, N, d), scale, causal, -1, -1, nullptr, block_mask, dtype,
                      dropout_rate, seed, stream);
}

int fa_forward_qk(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                  int Hkv, int Nq, int Nk, int d, float scale, int causal, int window_left,
                  int window_right, const float* alibi_slopes, const uint8_t* block_mask, int dtype,
                  float dropout_rate, unsigned long long seed, void* stream) {
  return forward_impl(q, k, v, o, lse, fixed_geo(B, H, Hkv, Nq, Nk, d), scale, causal, window_left, window_right,
                      alibi_slopes, block_mask, dtype, dropout_rate, seed, stream);
}

int fa_forward_select(int rows_per_wave, const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int H, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                      int window_left, int window_right, const float* alibi_slopes,
                      const uint8_t* block_mask, int dtype, float dropout_rate,
                      unsigned long long seed, void* stream) {
  if (rows_per_wave != 0 && rows_per_wave != 32 && rows_per_wave != 64) return FA_ERR_INVALID_ARG;
  return forward_impl(q, k, v, o, lse, fixed_geo(B, H, Hkv, Nq, Nk, d), scale, causal, window_left, window_right,
                      alibi_slopes, block_mask, dtype, dropout_rate, seed, stream, rows_per_wave);
}

int fa_forward_bitmask(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv,
                       int Nq, int Nk, int d, float scale, int causal, const uint8_t* block_mask,
                       const int32_t* block_tile, const uint32_t* tile_bits, int n_tiles, int dtype,
                       float dropout_rate, unsigned long long seed, void* stream) {
  if (!block_mask || !block_tile) return FA_ERR_INVALID_ARG;
  const ElemMask em{block_tile, tile_bits, n_tiles};
  return forward_impl(q, k, v, o, lse, fixed_geo(B, H, Hkv, Nq, Nk, d), scale, causal, -1, -1, nullptr, block_mask,
                      dtype, dropout_rate, seed, stream, 0, &em);
}

int fa_backward_bitmask(const void* q, const void* k, const void* v, const void* o, const float* lse,
                        const void* dO, void* dq, void* dk, void* dv, int B, int H, int Hkv, int Nq, int Nk, int d,
                        float scale, int causal, const uint8_t* block_mask, const int32_t* block_tile,
                        const uint32_t* tile_bits, int n_tiles, int dtype, float dropout_rate,
                        unsigned long long seed, void* workspace, size_t workspace_bytes, void* stream) {
  if (!block_mask || !block_tile) return FA_ERR_INVALID_ARG;
  const ElemMask em{block_tile, tile_bits, n_tiles};
  return backward_impl(q, k, v, o, lse, dO, dq, dk, dv, fixed_geo(B, H, Hkv, Nq, Nk, d), scale, causal, -1, -1,
                       nullptr, block_mask, dtype, dropout_rate, seed, workspace, workspace_bytes, stream, &em);
}

int fa_forward_kernel_rows(int B, int H, int Hkv, int Nq, int Nk, int d, int causal, int window_left,
                           int window_right, int has_alibi, int has_block_mask, int dtype) {
  const Geo g = fixed_geo(B, H, Hkv, Nq, Nk, d);
  int st = check_shape(g, 1.0f, dtype);
  if (st != FA_OK) return st;
  Band band;
  if (!make_band(causal, window_left, window_right, &band)) return FA_ERR_INVALID_ARG;
  fa::AttnShape s = make_shape(g, 1.0f, band, has_block_mask ? (const uint8_t*)1 : nullptr);
  s.alibi = has_alibi ? (const float*)1 : nullptr;  // only tested for NULL
  return fa::forward_rows(s, dtype);
}

int fa_backward_launches(int B, int H, int Hkv, int Nq, int Nk, int d, float dropout_rate, int has_alibi,
                         int has_block_mask, int dtype) {
  const Geo g = fixed_geo(B, H, Hkv, Nq, Nk, d);
  int st = check_shape(g, 1.0f, dtype);
  if (st != FA_OK) return st;
  if (dtype == FA_F32) return FA_ERR_UNSUPPORTED;
  if (!(dropout_rate >= 0.f && dropout_rate < 1.f)) return FA_ERR_INVALID_ARG;
  fa::AttnShape s = make_shape(g, 1.0f, Band{0, 0, 0}, nullptr);
  set_dropout(s, dropout_rate, 0ull);
  const bool fused = fused_ok(g, s.drop_t > 0 ? dropout_rate : 0.f, has_alibi ? (const float*)1 : nullptr,
                              has_block_mask ? (const uint8_t*)1 : nullptr);
  return fused ? 2 : 3;
}

int fa_forward_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                      const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int H, int Hkv,
                      int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int d,
                      float scale, int causal, int window_left, int window_right,
                      const float* alibi_slopes, int dtype, float dropout_rate, unsigned long long seed,
                      void* stream) {
  if (!cu_seqlens_q || !cu_seqlens_k) return FA_ERR_INVALID_ARG;
  const Geo g{B, H, Hkv, max_seqlen_q, max_seqlen_k, d, cu_seqlens_q, cu_seqlens_k, total_q, total_k};
  return forward_impl(q, k, v, o, lse, g, scale, causal, window_left, window_right, alibi_slopes, nullptr, dtype,
                      dropout_rate, seed, stream);
}

int fa_backward_stage(int stage, const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dO, void* dq, void* dk, void* dv, int B, int H,
                      int Hkv, int N, int d, float scale, int causal, const uint8_t* block_mask,
                      int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (stage < 0 || stage > 3) return FA_ERR_INVALID_ARG;
  return stage_impl(stage, q, k, v, o, lse, dO, dq, dk, dv, fixed_geo(B, H, Hkv, N, N, d), scale, causal,
                    -1, -1, nullptr, block_mask, dtype, 0.f, 0ull, workspace, workspace_bytes, stream);
}

int fa_backward_stage_dropout(int stage, const void* q, const void* k, const void* v,
                              const void* o, const float* lse, const void* dO, void* dq, void* dk,
                              void* dv, int B, int H, int Hkv, int N, int d, float scale,
                              int causal, const uint8_t* block_mask, int dtype,
                              float dropout_rate, unsigned long long seed, void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (stage < 0 || stage > 3) return FA_ERR_INVALID_ARG;
  return stage_impl(stage, q, k, v, o, lse, dO, dq, dk, dv, fixed_geo(B, H, Hkv, N, N, d), scale, causal,
                    -1, -1, nullptr, block_mask, dtype, dropout_rate, seed, workspace, workspace_bytes, stream);
}

int fa_backward(const void* q, const void* k, const void* v, const void* o, const float* lse,
                const void* dO, void* dq, void* dk, void* dv, int B, int H, int Hkv, int N, int d,
                float scale, int causal, const uint8_t* block_mask, int dtype, void* workspace,
                size_t workspace_bytes, void* stream) {
  return backward_impl(q, k, v, o, lse, dO, dq, dk, dv, fixed_geo(B, H, Hkv, N, N, d), scale, causal,
                       -1, -1, nullptr, block_mask, dtype, 0.f, 0ull, workspace, workspace_bytes, stream);
}

int fa_backward_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                        const void* dO, void* dq, void* dk, void* dv, int B, int H, int Hkv, int N, int d,
                        float scale, int causal, const uint8_t* block_mask, int dtype, void* stream) {
  const Geo g = fixed_geo(B, H, Hkv, N, N, d);
  // the full argument check first, with a stand-in workspace of the scratch
  // array's size (aligned, never dereferenced): nothing touches the runtime
  // before the arguments are known to be good
  int st = check_backward(q, k, v, o, lse, dO, dq, dk, dv, g, scale, block_mask, dtype, (void*)kAlign,
                          kScratchBytes);
  if (st == FA_ERR_WORKSPACE) return FA_ERR_UNSUPPORTED;  // needs more than the scratch array holds
  if (st != FA_OK) return st;
  Band band;
  if (!make_band(causal, -1, -1, &band)) return FA_ERR_INVALID_ARG;
  void* ws = scratch_ptr();
  if (!ws) return FA_ERR_HIP;
  return backward_impl(q, k, v, o, lse, dO, dq, dk, dv, g, scale, causal, -1, -1, nullptr, block_mask, dtype,
                       0.f, 0ull, ws, kScratchBytes, stream);
}

int fa_backward_dropout(const void* q, const void* k, const void* v, const void* o,
                        const float* lse, const void* dO, void* dq, void* dk, void* dv, int B,
                        int H, int Hkv, int N, int d, float scale, int causal,
                        const uint8_t* block_mask, int dtype, float dropout_rate,
                        unsigned long long seed, void* workspace, size_t workspace_bytes,
                        void* stream) {
  return backward_impl(q, k, v, o, lse, dO, dq, dk, dv, fixed_geo(B, H, Hkv, N, N, d), scale, causal,
                       -1, -1, nullptr, block_mask, dtype, dropout_rate, seed, workspace, workspace_bytes, stream);
}

int fa_backward_qk(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dO, void* dq, void* dk, void* dv, int B, int H, int Hkv, int Nq,
                   int Nk, int d, float scale, int causal, int window_left, int window_right,
                   const float* alibi_slopes, const uint8_t* block_mask, int dtype, float dropout_rate,
                   unsigned long long seed, void* workspace, size_t workspace_bytes,
                   void* stream) {
  return backward_impl(q, k, v, o, lse, dO, dq, dk, dv, fixed_geo(B, H, Hkv, Nq, Nk, d), scale, causal,
                       window_left, window_right, alibi_slopes, block_mask, dtype, dropout_rate, seed, workspace,
                       workspace_bytes, stream);
}

int fa_backward_varlen(const void* q, const void* k, const void* v, const void* o,
                       const float* lse, const void* dO, void* dq, void* dk, void* dv,
                       const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int H, int Hkv,
                       int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int d,
                       float scale, int causal, int window_left, int window_right,
                       const float* alibi_slopes, int dtype, float dropout_rate, unsigned long long seed,
                       void* workspace, size_t workspace_bytes, void* stream) {
  if (!cu_seqlens_q || !cu_seqlens_k) return FA_ERR_INVALID_ARG;
  const Geo g{B, H, Hkv, max_seqlen_q, max_seqlen_k, d, cu_seqlens_q, cu_seqlens_k, total_q, total_k};
  return backward_impl(q, k, v, o, lse, dO, dq, dk, dv, g, scale, causal, window_left, window_right,
                       alibi_slopes, nullptr, dtype, dropout_rate, seed, workspace, workspace_bytes, stream);
}

int fa_forward_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                   int Hkv, int N, int d, float scale, float q_descale, float k_descale,
                   float v_descale, int causal, int out_dtype, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || ((uintptr_t)lse & 3u))
    return FA_ERR_INVALID_ARG;
  if (out_dtype != FA_BF16 && out_dtype != FA_F16) return FA_ERR_INVALID_ARG;
  const Geo g = fixed_geo(B, H, Hkv, N, N, d);
  int st = check_shape(g, scale, out_dtype);
  if (st != FA_OK) return st;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;  // the FP8 contraction takes 64 values at a time
  for (float x : {q_descale, k_descale, v_descale})
    if (!isfinite(x) || !(x > 0.f)) return FA_ERR_INVALID_ARG;
  Band band;
  make_band(causal, -1, -1, &band);
  fa::Fp8FwdArgs a;
  a.s = make_shape(g, scale, band, nullptr);
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.q_descale = q_descale;
  a.k_descale = k_descale;
  a.v_descale = v_descale;
  (void)hipGetLastError();
  return fa::launch_forward_fp8(a, out_dtype, (hipStream_t)stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
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

int fa_version(void) { return 105; }

}  // extern "C"
