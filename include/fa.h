/*
 * fa.h - IO-aware exact attention for AMD MI355X (gfx950): forward and backward.
 *
 * What is computed. For every batch b and query head h, with kv head
 * g = h / (H / Hkv) (grouped-query attention: contiguous groups of query heads
 * share one key/value head, as on the "Grouped-query attention" card of the
 * pranaymahendrakar.com lesson "FlashAttention"):
 *
 *     S = scale * Q K^T,  P = softmax(S) row by row,  O = P V
 *
 * (that lesson, Researcher tier, "The problem being solved"), computed tile by
 * tile with a running row maximum m and running sum l of exponentials, the
 * partial output rescaled by exp(m_old - m_new) whenever the maximum grows
 * (same lesson, "Online softmax"), so that S and P are never written to memory
 * (nadeemcite.github.io summary "FlashAttention: Fast and Memory-Efficient
 * Exact Attention with IO-Awareness", Core Idea items 1, 2 and 4). The forward
 * pass saves one statistic per row, LSE = m + ln(l), the natural-log
 * log-sum-exp of the row's scaled scores; the backward pass recomputes P tile
 * by tile as exp(S - LSE) instead of reading it back (Core Idea item 3).
 *
 * Masks. causal != 0 keeps key j visible to query i only when j <= i (the
 * lesson's Beginner tier: a word looks at earlier words). block_mask, when not
 * NULL, is a device array of uint8 [ceil(N/128)][ceil(N/128)], row-major; block
 * (I, J) nonzero keeps keys 128J..128J+127 visible to queries 128I..128I+127
 * (the summary's "Block-sparse extension", Key Method Details). The same mask
 * serves every batch and head; with causal it is intersected. Zero blocks are
 * skipped without being read. A query that sees no key at all gets O = 0,
 * LSE = -inf and zero gradients.
 *
 * Layouts. All tensors are dense, row-major, device-resident:
 *   q, o, dO, dq : [B][H][N][d]        k, v, dk, dv : [B][Hkv][N][d]
 *   lse          : [B][H][N] float32
 * q, k, v, o, dO, dq, dk, dv share one element type, FA_BF16, FA_F16 or FA_F32
 * (FA_F32: forward only). q, k, v, o, dO, dq, dk, dv must be 16-byte aligned,
 * lse 4-byte aligned. d is 32, 64 or 128; N >= 1 is any length (no
 * multiple-of-tile restriction) with N * d < 2^30 and B * H * N < 2^31; with a
 * block mask, ceil(N / 128) <= 2048 (else FA_ERR_UNSUPPORTED); H must be a
 * multiple of Hkv; B <= 65535; scale must be finite and >= 0 (1/sqrt(d) is the
 * usual one).
 *
 * Ownership. The caller owns every buffer. The library allocates no device or
 * host memory and keeps no state between calls; outputs are overwritten, never
 * accumulated into, and must not alias inputs. Calls are thread-safe.
 *
 * Streams and errors. `stream` is a hipStream_t (NULL = the default stream).
 * Every entry point checks all of its arguments before it touches the HIP
 * runtime; on a bad argument it returns a negative status and enqueues
 * nothing. Otherwise it enqueues its kernels on `stream` and returns at once
 * (no host synchronisation); a launch failure reported by the runtime returns
 * FA_ERR_HIP. Non-finite inputs propagate into the outputs; they are not
 * checked.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define FA_OK 0
#define FA_ERR_INVALID_ARG (-1) /* NULL pointer, bad size, bad dtype, bad scale, misaligned */
#define FA_ERR_UNSUPPORTED (-2) /* well-formed but not implemented (e.g. FA_F32 backward)  */
#define FA_ERR_WORKSPACE (-3)   /* workspace NULL or smaller than fa_backward_workspace_size */
#define FA_ERR_HIP (-4)         /* the HIP runtime reported an error at launch              */

/* Element types of q, k, v, o, dO, dq, dk, dv. */
#define FA_F32 0
#define FA_F16 1
#define FA_BF16 2

/* Block-mask granularity, in rows and in columns. */
#define FA_MASK_BLOCK 128

/*
 * fa_forward: O and LSE from Q, K, V.
 *   q [B][H][N][d], k, v [B][Hkv][N][d]    inputs (device)
 *   o [B][H][N][d]                          output (device), same dtype as q
 *   lse [B][H][N] float32                   output (device): m + ln(l) per row,
 *                                           -inf for a row that sees no key
 *   block_mask                              NULL (dense) or device uint8 mask
 *   dtype                                   FA_BF16, FA_F16 or FA_F32
 * Returns FA_OK or a negative status.
 */
int fa_forward(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int Hkv, int N, int d, float scale, int causal,
               const uint8_t* block_mask, int dtype, void* stream);

/*
 * fa_backward_workspace_size: bytes of device scratch fa_backward needs for
 * these sizes: two float32 per query row (D = rowsum(dO * O) and the log-sum-
 * exp in base 2) for N rounded up to a multiple of 128 rows, per (batch, head),
 * rounded up to 256 bytes: 8 * B * H * roundup(N, 128). Linear in N. Returns
 * 0 for arguments fa_backward would reject.
 */
size_t fa_backward_workspace_size(int B, int H, int Hkv, int N, int d, int dtype);

/*
 * fa_backward: dq, dk, dv of sum(O * dO) from the forward pass's inputs and
 * its saved o and lse. The probabilities are recomputed tile by tile from q,
 * k and lse. For grouped-query attention dk and dv of a kv head are summed
 * over its group of query heads. dtype is FA_BF16 or FA_F16 (FA_F32 returns
 * FA_ERR_UNSUPPORTED). causal, block_mask and scale must be those of the
 * forward call that produced o and lse. No atomics are used: every output
 * element is written once, so results are bitwise reproducible.
 *   workspace        device buffer of at least fa_backward_workspace_size()
 *                    bytes, 256-byte aligned; its contents on entry do not
 *                    matter and on return are unspecified. Owned by the caller;
 *                    two calls in flight at once need two workspaces.
 * Returns FA_OK or a negative status.
 */
int fa_backward(const void* q, const void* k, const void* v, const void* o, const float* lse,
                const void* dO, void* dq, void* dk, void* dv,
                int B, int H, int Hkv, int N, int d, float scale, int causal,
                const uint8_t* block_mask, int dtype,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_backward_noalloc: fa_backward for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. Same arguments, results and errors as fa_backward, minus
 * the workspace: the per-row statistics go to a device array of
 * FA_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends. Arguments whose fa_backward_workspace_size exceeds
 * it return FA_ERR_UNSUPPORTED (16 MiB: B * H * roundup(N, 128) up to 2^21
 * query rows). The call allocates nothing; its first call on a device looks
 * up the array's address there (with that device current). Every call on one
 * GPU uses the same array: two calls that overlap on one GPU (on different
 * streams, or from threads without ordering between them) race and give
 * wrong results; calls in order on one stream are safe. The array needs no
 * clearing: each call writes every statistic it reads.
 */
#define FA_NOALLOC_SCRATCH_BYTES (16u << 20)
int fa_backward_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                        const void* dO, void* dq, void* dk, void* dv,
                        int B, int H, int Hkv, int N, int d, float scale, int causal,
                        const uint8_t* block_mask, int dtype, void* stream);

/*
 * fa_backward_stage: one of the stages fa_backward runs, with the same
 * arguments and the same workspace:
 *   stage 0  D = rowsum(dO * O) and the base-2 LSE per query row, into the
 *            workspace
 *   stage 1  per key block: recompute P and dS, write dk and dv
 *   stage 2  per query block: recompute P and dS, write dq
 *   stage 3  stages 1 and 2 in one launch (key-block workgroups first, then
 *            query-block ones); only for d <= 64 without a block mask, the
 *            case where fa_backward runs stages 0, 3 instead of 0, 1, 2
 *            (FA_ERR_UNSUPPORTED otherwise)
 * Stages 1 and 2 both need stage 0's result and nothing from each other.
 * Running stages 0, 1, 2 (or 0, 3) in order equals one fa_backward call. It
 * exists so that each stage can be timed on its own. Returns FA_OK or a
 * negative status (FA_ERR_INVALID_ARG for a stage outside 0..3).
 */
int fa_backward_stage(int stage, const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dO, void* dq, void* dk, void* dv,
                      int B, int H, int Hkv, int N, int d, float scale, int causal,
                      const uint8_t* block_mask, int dtype,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_backward_launches: how many kernels fa_backward (and fa_backward_qk,
 * fa_backward_dropout) enqueues for these arguments: 3 for stages 0, 1, 2, or
 * 2 for stages 0, 3 (d <= 64 without dropout, ALiBi slopes or a block mask),
 * or a negative status for arguments the backward calls reject. A rate that
 * rounds to no dropout counts as none. has_alibi and has_block_mask say
 * whether slopes or a mask would be passed. Touches no device.
 */
int fa_backward_launches(int B, int H, int Hkv, int Nq, int Nk, int d, float dropout_rate, int has_alibi,
                         int has_block_mask, int dtype);

/*
 * Dropout on the attention probabilities, fused into the same kernels
 * (chipfoundryservices.com glossary "flash attention algorithm", "Kernel
 * Fusion", lists dropout among the operations fused into one kernel; the
 * pages do not define it, so the usual reading is taken): after the row
 * softmax each probability is kept with probability (256 - t) / 256 and then
 * multiplied by 256 / (256 - t), or set to 0, where t = round(256 *
 * dropout_rate), at most 255 (the rate is quantised to multiples of 1/256).
 * lse is still the log-sum-exp of the scaled scores before dropout. The keep
 * decision of element (query i, key j) of query head h of batch b is byte
 * j & 3 of word i & 3 of Philox4x32-10 (Salmon et al., SC'11) at counter
 * (i >> 2, j >> 2, b * H + h, 0) under key (seed & 0xffffffff, seed >> 32),
 * kept iff that byte >= t: the forward and backward calls with the same seed
 * and rate draw the same decisions, and nothing is stored.
 *   dropout_rate    in [0, 1); a rate that rounds to t = 0 is no dropout
 *   seed            64-bit generator key
 * Other arguments, layouts, ownership and errors as for fa_forward /
 * fa_backward / fa_backward_stage, plus FA_ERR_INVALID_ARG for a rate outside
 * [0, 1) and FA_ERR_UNSUPPORTED for FA_F32 with dropout (t > 0).
 */
int fa_forward_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                       int B, int H, int Hkv, int N, int d, float scale, int causal,
                       const uint8_t* block_mask, int dtype,
                       float dropout_rate, unsigned long long seed, void* stream);
int fa_backward_dropout(const void* q, const void* k, const void* v, const void* o,
                        const float* lse, const void* dO, void* dq, void* dk, void* dv,
                        int B, int H, int Hkv, int N, int d, float scale, int causal,
                        const uint8_t* block_mask, int dtype,
                        float dropout_rate, unsigned long long seed,
                        void* workspace, size_t workspace_bytes, void* stream);
int fa_backward_stage_dropout(int stage, const void* q, const void* k, const void* v,
                              const void* o, const float* lse, const void* dO,
                              void* dq, void* dk, void* dv,
                              int B, int H, int Hkv, int N, int d, float scale, int causal,
                              const uint8_t* block_mask, int dtype,
                              float dropout_rate, unsigned long long seed,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Unequal query and key lengths (chipfoundryservices.com glossary "flash
 * attention algorithm", "Inference Optimization": attention beside a KV cache,
 * where a few new queries meet many cached keys). The Nq queries are read as
 * the last Nq positions of a sequence of Nk keys, so under causal masking key
 * j is visible to query i iff j <= i + (Nk - Nq) ("bottom-right" alignment;
 * the pages do not fix it, this is the reading that fits a KV cache). With
 * Nq > Nk the first Nq - Nk queries see no key (O = 0, LSE = -inf, zero
 * gradients). Nq == Nk is exactly fa_forward / fa_backward.
 *   q, o, dO, dq : [B][H][Nq][d]       k, v, dk, dv : [B][Hkv][Nk][d]
 *   lse          : [B][H][Nq] float32
 *   block_mask   NULL or uint8 [ceil(Nq/128)][ceil(Nk/128)] (both <= 2048)
 *   workspace    fa_backward_workspace_size(B, H, Hkv, Nq, d, dtype) bytes
 * Sliding-window (local) masks, one family of the many masks a single tiled
 * kernel can serve (pranaymahendrakar.com lesson "FlashAttention", Researcher
 * tier, "Beyond hand-written kernels"; the pages fix no convention, this is
 * the reading taken): with the query at position p = i + (Nk - Nq), key j is
 * visible only if p - window_left <= j <= p + window_right; -1 leaves that
 * side unbounded, and causal != 0 sets the right limit to 0 (so causal with
 * window_left = W - 1 keeps the query and the W - 1 keys before it). Band,
 * causal and block masks intersect. The kernels skip the tiles outside the
 * band and mask elements only in tiles that straddle its edges.
 *   window_left, window_right   >= -1 (FA_ERR_INVALID_ARG below -1)
 * Score modification, the other half of that lesson section (functions that
 * change scores inside the tiled kernel; it names none, and the one taken is
 * ALiBi's linear distance bias, Press, Smith and Lewis 2022): with
 * alibi_slopes not NULL, the scaled score of query i and key j becomes
 * scale * q_i . k_j - alibi_slopes[h] * |i + (Nk - Nq) - j| for query head h
 * before the softmax, masks applied as before; LSE is that of the biased
 * scores and the bias has no gradient of its own. The backward call must get
 * the slopes the forward call got.
 *   alibi_slopes   NULL, or device float32 [H], 4-byte aligned (else
 *                  FA_ERR_INVALID_ARG); finite values, not checked (they
 *                  live in device memory). The forward pass uses its 32-row
 *                  kernel for these calls (see fa_forward_kernel_rows).
 * dropout_rate 0 is no dropout; dropout otherwise as described above. Other
 * arguments, limits (each of Nq and Nk as N), ownership and errors as for
 * fa_forward / fa_backward.
 */
int fa_forward_qk(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int H, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                  int window_left, int window_right, const float* alibi_slopes,
                  const uint8_t* block_mask, int dtype, float dropout_rate,
                  unsigned long long seed, void* stream);
int fa_backward_qk(const void* q, const void* k, const void* v, const void* o,
                   const float* lse, const void* dO, void* dq, void* dk, void* dv,
                   int B, int H, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                   int window_left, int window_right, const float* alibi_slopes,
                   const uint8_t* block_mask, int dtype, float dropout_rate,
                   unsigned long long seed, void* workspace, size_t workspace_bytes,
                   void* stream);

/*
 * Element masks for partial blocks (pranaymahendrakar.com lesson
 * "FlashAttention", Researcher tier, "Beyond hand-written kernels": one tiled
 * kernel serving user mask functions evaluated per query-key pair; the pages
 * fix no encoding, this is the reading taken). A C ABI takes no device code,
 * so the predicate arrives evaluated, in block form: the block mask says
 * which 128 x 128 blocks hold any visible element (zero blocks are skipped
 * without being read), and for each kept block block_tile says whether all of
 * its elements are visible (-1) or only those set in one 128 x 128 bit tile
 * (t >= 0). Key j is then visible to query i iff block_mask[I][J] != 0 and,
 * for t = block_tile[I][J] >= 0, bit j % 32 of word (j % 128) / 32 of row
 * i % 128 of tile t is set (I = i / 128, J = j / 128), intersected with causal
 * masking as for fa_forward_qk (queries aligned to the last key). Full blocks
 * run the unmasked tile code; only partial blocks read their bits.
 *   block_mask   device uint8 [ceil(Nq/128)][ceil(Nk/128)] (both <= 2048)
 *   block_tile   device int32 [ceil(Nq/128)][ceil(Nk/128)], 4-byte aligned
 *   tile_bits    device uint32 [n_tiles][128][4], 16-byte aligned (may be
 *                NULL when n_tiles is 0)
 *   n_tiles      0 <= n_tiles <= 2^21; an index in block_tile at or past
 *                n_tiles reads as an all-zero tile (no element visible) - the
 *                kernels never read past the tiles
 * The same mask serves every batch and head. block_tile and tile_bits live in
 * device memory and are not checked by the host beyond alignment. Dropout as
 * for fa_forward_dropout. Other arguments, layouts, limits and errors as for
 * fa_forward_qk / fa_backward_qk (no window, no ALiBi); FA_ERR_INVALID_ARG for
 * a NULL block_mask or block_tile, misalignment or n_tiles out of range. The
 * backward call must get the mask arrays the forward call got.
 */
int fa_forward_bitmask(const void* q, const void* k, const void* v, void* o, float* lse,
                       int B, int H, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                       const uint8_t* block_mask, const int32_t* block_tile, const uint32_t* tile_bits,
                       int n_tiles, int dtype, float dropout_rate, unsigned long long seed, void* stream);
int fa_backward_bitmask(const void* q, const void* k, const void* v, const void* o, const float* lse,
                        const void* dO, void* dq, void* dk, void* dv,
                        int B, int H, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                        const uint8_t* block_mask, const int32_t* block_tile, const uint32_t* tile_bits,
                        int n_tiles, int dtype, float dropout_rate, unsigned long long seed,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Forward kernel choice. The 16-bit forward pass has two kernels: one with 64
 * query rows per wave (head size 128 when its grid, B * H * ceil(Nq / 256)
 * workgroups, holds at least 256 of them and either the shorter of Nq, Nk is
 * at least 4096 under a causal or window band, 1024 without, or the grid
 * holds at least 2048; at that
 * head size a producer wave forming the probabilities and a consumer wave
 * holding the output share each SIMD, at smaller head sizes, when forced, it
 * runs one wave per SIMD) and one with 32 rows per wave (two waves per SIMD;
 * everything else, and every call with a block mask or score bias). Both
 * compute the same attention (results agree within the tolerances, not bit
 * for bit).
 *
 * fa_forward_kernel_rows: the rows per wave of the kernel that fa_forward /
 * fa_forward_qk / fa_forward_dropout take for these arguments: 64 or 32, 0
 * for FA_F32 (the float32 kernel), or a negative status for arguments they
 * would reject. has_alibi and has_block_mask say whether slopes or a mask
 * would be passed (any nonzero value = yes). Touches no device.
 *
 * fa_forward_select: fa_forward_qk with the kernel forced: rows_per_wave 0
 * takes the library's choice, 32 or 64 force that kernel (64 with a block
 * mask or ALiBi slopes is FA_ERR_UNSUPPORTED, as is a nonzero value with
 * FA_F32; other values are FA_ERR_INVALID_ARG). For tests and benchmarks
 * that compare the two kernels. Other arguments as for fa_forward_qk.
 */
int fa_forward_kernel_rows(int B, int H, int Hkv, int Nq, int Nk, int d, int causal, int window_left,
                           int window_right, int has_alibi, int has_block_mask, int dtype);
int fa_forward_select(int rows_per_wave, const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int H, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                      int window_left, int window_right, const float* alibi_slopes,
                      const uint8_t* block_mask, int dtype, float dropout_rate,
                      unsigned long long seed, void* stream);

/*
 * Packed variable-length batches (the same glossary, "Sequence Length
 * Flexibility": any lengths, no padding). B sequences are stored one after
 * another per head, with no padding between them:
 *   q, o, dO, dq : [H][total_q][d]     k, v, dk, dv : [Hkv][total_k][d]
 *   lse          : [H][total_q] float32
 * Sequence b holds query rows cu_seqlens_q[b] .. cu_seqlens_q[b + 1] - 1 and
 * keys cu_seqlens_k[b] .. cu_seqlens_k[b + 1] - 1 of every head; each is an
 * independent attention problem (causal alignment and windows as for
 * fa_forward_qk, with the sequence's own lengths; a sequence may have no
 * queries or no keys). alibi_slopes as for fa_forward_qk, the distance
 * taken within the sequence.
 *   cu_seqlens_q, cu_seqlens_k   device int32 [B + 1], 4-byte aligned, rising
 *                                from 0 to total_q / total_k
 *   max_seqlen_q, max_seqlen_k   >= 1 and >= every sequence's length; the
 *                                launch grid and the limits (as N) use these
 *   total_q, total_k             >= 0, rows of each head's plane
 *   workspace                    fa_backward_workspace_size(B, H, Hkv,
 *                                max_seqlen_q, d, dtype) bytes
 * Dropout draws stream b * H + h for query head h of sequence b, indexed by
 * positions within the sequence. No block mask. The offsets live in device
 * memory and are not checked by the host; the kernels clamp them to the
 * planes and the lengths to max_seqlen_*, so offsets that break the contract
 * give wrong results but no access outside the buffers. Other arguments,
 * ownership and errors as for fa_forward / fa_backward; FA_ERR_INVALID_ARG
 * also for a NULL or misaligned offset array, H * total_q or Hkv * total_k of
 * 2^31 or more.
 */
int fa_forward_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                      const int* cu_seqlens_q, const int* cu_seqlens_k,
                      int B, int H, int Hkv, int total_q, int total_k,
                      int max_seqlen_q, int max_seqlen_k, int d, float scale, int causal,
                      int window_left, int window_right, const float* alibi_slopes,
                      int dtype, float dropout_rate, unsigned long long seed, void* stream);
int fa_backward_varlen(const void* q, const void* k, const void* v, const void* o,
                       const float* lse, const void* dO, void* dq, void* dk, void* dv,
                       const int* cu_seqlens_q, const int* cu_seqlens_k,
                       int B, int H, int Hkv, int total_q, int total_k,
                       int max_seqlen_q, int max_seqlen_k, int d, float scale, int causal,
                       int window_left, int window_right, const float* alibi_slopes,
                       int dtype, float dropout_rate, unsigned long long seed,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * FP8 forward (pranaymahendrakar.com lesson "FlashAttention", version lineage:
 * FlashAttention-3 adds an FP8 forward pass; the pages fix no format, so this
 * is the reading taken). q, k, v hold OCP E4M3 codes (one byte each: sign,
 * exponent bias 7, 3 mantissa bits, subnormals, 0x7F / 0xFF NaN, largest
 * finite 448) with one float descale per tensor: the attention computed is
 * that of the real inputs code * q_descale, code * k_descale and
 * code * v_descale, with S = scale * Q K^T as for fa_forward. Both
 * contractions run on the FP8 matrix cores; the probabilities are rounded to
 * E4M3 (nearest even) before they weight V, the running sum and LSE use them
 * unrounded, so O carries that rounding (relative 2^-4 per probability at
 * most) and LSE does not.
 *   q : [B][H][N][d] bytes     k, v : [B][Hkv][N][d] bytes (16-byte aligned)
 *   o : [B][H][N][d] of out_dtype (FA_BF16 or FA_F16)   lse : [B][H][N] float
 *   d : 64 or 128 (others FA_ERR_UNSUPPORTED)
 *   q_descale, k_descale, v_descale : finite and > 0
 *   causal : as for fa_forward
 * Other limits, ownership and errors as for fa_forward; no block mask,
 * window or dropout, and no backward pass.
 */
int fa_forward_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int Hkv, int N, int d, float scale,
                   float q_descale, float k_descale, float v_descale,
                   int causal, int out_dtype, void* stream);

/* fa_status_string: a static, human-readable description of a status code. */
const char* fa_status_string(int status);

/* fa_version: the library version as 10000*major + 100*minor + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
