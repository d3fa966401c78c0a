/*
 * attn.h -- C ABI of the MI355X (gfx950) tiled exact attention library.
 *
 * Operations, each computing exactly softmax(scale * Q K^T) V, or its
 * gradients, without the score matrix ever reaching device memory:
 *
 *   attn_fwd           prefill: every query row of a sequence against its keys,
 *                      optionally causal, with grouped-query heads, writing O
 *                      and the per-row log-sum-exp.
 *   attn_fwd_window    the same, causal, limited to a sliding window of keys.
 *   attn_bwd           the gradients dQ, dK, dV of attn_fwd's output for a
 *                      given output gradient dO, rebuilding the probabilities
 *                      tile by tile from the saved log-sum-exp.
 *   attn_prefill_paged chunked prefill: the new query tokens of each sequence
 *                      against its paged key/value cache, causal.
 *   attn_decode_paged  decode: one query token per sequence against a key/value
 *                      cache stored in fixed-size pages reached through a
 *                      block table.
 *   attn_decode_paged_fp8  the same over fp8 (E4M3) pages with scales.
 *   attn_decode_paged_int8 the same over int8 pages with scales.
 *
 * Definitions (page titles and sections of the sources):
 *   - "Advanced Attention Mechanisms - II" (A. Das), section Tiling, steps 1-3:
 *     Q, K, V are cut into tiles; per Q/K tile pair the scaled dot product
 *     gives a tile of scores that is softmax-weighted against the V tile, and
 *     the per-tile results accumulate into the full attention result.
 *   - same page, sections "Softmax stabiliser" and "Incremental / online
 *     softmax": the max-subtracted softmax, computed block by block with the
 *     normaliser incomplete until the last block.
 *   - same page, section "Flash Attention": the attention matrix is neither
 *     read from nor written to device memory; only row statistics are kept.
 *   - "Fast attention kernels and operator fusion accelerate AI models",
 *     section on FlashAttention-style and paged attention: blocks of scores,
 *     softmax statistics updated and outputs accumulated on chip; the paged KV
 *     cache with its block table of logical-to-physical blocks; 16-token
 *     blocks in the serving example.
 *   - "Accelerating Mamba-2 with high-performance forward-pass kernels in
 *     NVIDIA CUDA Tile": causal masking removes terms with i < j; exp2 with
 *     log2(e) folded into the scale.
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     never allocates, frees, or synchronises, and keeps no state between calls
 *     (except attn_decode_paged_noalloc, whose scratch is a device-resident
 *     array of the library, and the timing events of attn_time_next_call, which
 *     last for one call: see there).
 *   - Tensors are dense row-major (C order) with the shapes given below.
 *   - `stream` is a hipStream_t passed as void*; NULL means the default stream.
 *     Work is enqueued asynchronously on it; results are valid once the stream
 *     has reached the point after the call.
 *   - Every argument check happens on the host before any HIP call.  A call
 *     that returns anything other than ATTN_OK has enqueued nothing.
 *   - There is no fallback path: an unsupported input returns
 *     ATTN_EUNSUPPORTED rather than being computed some other way.
 *   - attn_last_error() returns a human-readable detail for the calling
 *     thread's most recent non-OK return.
 */
#ifndef ATTN_H_
#define ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_EINVAL = 1,        /* bad pointer, size, alignment or combination      */
  ATTN_EUNSUPPORTED = 2,  /* well-formed but outside what the kernels handle  */
  ATTN_EHIP = 3           /* the HIP runtime reported an error at launch      */
} attn_status;

typedef enum {
  ATTN_F32 = 0,           /* float32 q/k/v/o                                   */
  ATTN_BF16 = 1           /* bfloat16 q/k/v/o, float32 accumulation            */
} attn_dtype;

/*
 * attn_fwd -- prefill attention with log-sum-exp.
 *
 *   q   [B, Hq,  T, d]  dtype        queries
 *   k   [B, Hkv, S, d]  dtype        keys
 *   v   [B, Hkv, S, d]  dtype        values
 *   o   [B, Hq,  T, d]  dtype        output (written)
 *   lse [B, Hq,  T]     float32      natural-log log-sum-exp of the scaled
 *                                    logits of each row (written); may be NULL
 *
 * "Advanced Attention Mechanisms - II" (A. Das), section Tiling, step 2 and
 * section "Softmax stabiliser"; the tile-by-tile computation follows its
 * section "Incremental / online softmax", and the log-sum-exp is the row
 * statistic its section "Flash Attention" keeps instead of the matrix:
 * O[b,h,i,:] = sum_j P[i,j] V[b,hk,j,:] with P = softmax_j(scale * q_i . k_j)
 * over the visible keys j, where hk = h / (Hq / Hkv) (consecutive query heads
 * share a KV head; Hq == Hkv is ordinary multi-head, Hkv == 1 multi-query).
 * causal != 0 hides key j from query i when j > i + (S - T) (bottom-right
 * alignment; the usual j > i when T == S).  bf16 outputs are rounded to
 * nearest even from float32.
 *
 * Requirements: B, Hq, Hkv, T, S >= 1; Hq % Hkv == 0; causal implies T <= S;
 * T * d and S * d below 2^31; scale finite and > 0; q, k, v, o 16-byte
 * aligned, lse 4-byte aligned; o and lse must not overlap q, k, v or each
 * other.  d must be 64 or 128 (else ATTN_EUNSUPPORTED); dtype ATTN_F32 or
 * ATTN_BF16.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int Hq, int Hkv, int T, int S, int d, float scale, int causal,
             int dtype, void* stream);

/*
 * attn_fwd_window -- causal prefill with a sliding window.
 *
 * As attn_fwd with causal = 1, except that query i also loses every key
 * j <= i + (S - T) - window: it sees its own position and the window - 1
 * before it.  "Advanced Attention Mechanisms - II" (A. Das), section "Flash
 * Attention", names sliding-window attention among the methods that cut
 * memory and compute; this window rule is our reading of that name.  Key
 * tiles wholly outside a query tile's window are skipped, not masked.
 *
 * Requirements: as for attn_fwd (causal); window >= 1 (else ATTN_EINVAL).
 * window >= S gives exactly attn_fwd's causal result.
 */
int attn_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int Hq, int Hkv, int T, int S, int d, float scale, int window,
                    int dtype, void* stream);

/*
 * attn_bwd -- gradients of attn_fwd.
 *
 *   q, k, v, o, lse   as for attn_fwd; o and lse are what attn_fwd wrote for
 *                     these q, k, v, scale and causal (lse may not be NULL)
 *   dout [B, Hq,  T, d]  bf16     gradient of the loss with respect to o
 *   dq   [B, Hq,  T, d]  bf16     gradient with respect to q (written)
 *   dk   [B, Hkv, S, d]  bf16     gradient with respect to k (written)
 *   dv   [B, Hkv, S, d]  bf16     gradient with respect to v (written)
 *   workspace  >= attn_bwd_workspace_size(B, Hq, Hkv, T, S, d) bytes of
 *              device memory, 16-byte aligned: per-row statistics and
 *              partial dK/dV, contents on entry ignored.
 *              Calls that share a workspace must not overlap in time.
 *
 * "Advanced Attention Mechanisms - II" (A. Das), section "Flash Attention":
 * the attention matrix is not kept for the backward pass, only the row
 * statistics, so the probabilities are recomputed per tile:
 *   P = exp(scale q_i . k_j - lse_i) on visible (i, j), else 0;
 *   D_i = sum_c dout[i,c] o[i,c];  dS = P * (dout V^T - D);
 *   dv = P^T dout,  dq = scale dS k,  dk = scale dS^T q,
 * the derivative of attn_fwd's definition (same mask and head mapping).  A KV
 * head's dk and dv sum the contributions of all Hq / Hkv query heads that
 * read it, in a fixed order; no atomics are used, so equal inputs give
 * bitwise equal results.  Accumulation is float32; outputs are rounded to
 * nearest even bf16.
 *
 * Requirements: as for attn_fwd, plus: dtype must be ATTN_BF16 (else
 * ATTN_EUNSUPPORTED); every pointer non-NULL; dout, dq, dk, dv and workspace
 * 16-byte aligned; dq, dk, dv and workspace must not overlap each other or
 * any input.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dout, void* dq, void* dk, void* dv,
             int B, int Hq, int Hkv, int T, int S, int d, float scale, int causal,
             int dtype, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace attn_bwd needs (0 if invalid): r(2 * B * Hq * T floats)
 * (per query row, its log-sum-exp in base 2 and D above), r() rounding up to
 * a multiple of 256, plus 2 * n * B * Hkv * S * d floats when n > 1, where n,
 * the number of workgroups that share the query heads of one KV head in the
 * dK/dV pass, is the smallest divisor of Hq / Hkv with
 * ceil(S / 128) * B * Hkv * n >= 512 (Hq / Hkv if there is none): their fp32
 * partial dK and dV, summed in a fixed order at the end.  About 67 MB at
 * B=4, Hq=12, Hkv=2, T=S=4096, d=128 (n = 2); 0.4 MB with n = 1 at B=8,
 * Hq=Hkv=12, T=S=1024, d=64. */
size_t attn_bwd_workspace_size(int B, int Hq, int Hkv, int T, int S, int d);

/*
 * attn_prefill_paged -- chunked prefill: new query tokens of each sequence
 * against its paged KV cache, causal.
 *
 *   q           [N, Hq, T, d]                    bf16   queries; sequence n uses
 *                                                       rows 0 .. q_lens[n]-1
 *   k_pool      [num_pages, Hkv, page, d]        bf16   key pages
 *   v_pool      [num_pages, Hkv, page, d]        bf16   value pages
 *   block_table [N, max_blocks]                  int32  physical page of each
 *                                                       logical block
 *   seq_lens    [N]                              int32  cached tokens per sequence,
 *                                                       the new ones included
 *   q_lens      [N]                              int32  new tokens per sequence
 *   o           [N, Hq, T, d]                    bf16   output rows 0 .. q_lens[n]-1
 *                                                       (written; other rows untouched)
 *   lse         [N, Hq, T]                       float32 log-sum-exp of the same
 *                                                       rows (written); may be NULL
 *
 * The new tokens are the last q_lens[n] of the seq_lens[n] cached ones: row
 * i of sequence n is the query at position p = seq_lens[n] - q_lens[n] + i
 * and attends the cached keys j <= p (j > p - window too if window > 0), the
 * bottom-right causal rule of attn_fwd with T = q_lens[n], S = seq_lens[n].
 * Keys and values are read through the block table as in attn_decode_paged
 * ("Fast attention kernels and operator fusion accelerate AI models",
 * section on paged attention: a block table maps logical blocks to physical
 * ones); the pages must therefore already hold the new tokens' keys and
 * values.  Key tiles are loaded page by page straight into on-chip memory.
 *
 * Requirements checked on the host: N, Hq, Hkv, T, num_pages, max_blocks
 * >= 1; Hq % Hkv == 0; window >= 0; scale finite and > 0; pointers aligned
 * as for attn_decode_paged; o and lse overlap no input or each other.
 * page must be 16, d 64 or 128 and dtype ATTN_BF16, else ATTN_EUNSUPPORTED.
 * Device contents are a caller contract: 1 <= q_lens[n] <= min(T, seq_lens[n]),
 * seq_lens[n] <= max_blocks * page, block_table[n, b] in [0, num_pages) for
 * b < ceil(seq_lens[n] / page).  The kernels never read outside the pool
 * (an out-of-range page id is clamped; that sequence's output is then
 * unspecified) and write nothing for a sequence with q_lens[n] <= 0.
 */
int attn_prefill_paged(const void* q, const void* k_pool, const void* v_pool,
                       const int32_t* block_table, const int32_t* seq_lens,
                       const int32_t* q_lens, void* o, float* lse,
                       int N, int Hq, int Hkv, int T, int d, int page, int num_pages,
                       int max_blocks, float scale, int window, int dtype, void* stream);

/*
 * attn_decode_paged -- one query token per sequence against a paged KV cache.
 *
 *   q           [N, Hq, d]                       bf16   queries (one per sequence)
 *   k_pool      [num_pages, Hkv, page, d]        bf16   key pages
 *   v_pool      [num_pages, Hkv, page, d]        bf16   value pages
 *   block_table [N, max_blocks]                  int32  physical page of each
 *                                                       logical block
 *   seq_lens    [N]                              int32  cached tokens per sequence
 *   o           [N, Hq, d]                       bf16   output (written)
 *   lse         [N, Hq]                          float32 log-sum-exp (written);
 *                                                       may be NULL
 *   workspace   >= attn_decode_workspace_size(N, Hq, d, max_blocks, page) bytes,
 *               16-byte aligned, device memory; scratch for the partial
 *               results of sequences divided between workers, contents on
 *               entry are ignored.  Two calls that share a workspace must not overlap
 *               in time (same stream, or ordered).
 *
 * "Fast attention kernels and operator fusion accelerate AI models", section
 * on paged attention: keys and values live in fixed-size pages, and a block
 * table maps each logical block of a sequence to its physical page, which the
 * kernel translates for every position (16-token blocks in its serving
 * example); the attention over the gathered keys is attn_fwd's definition with
 * one query row.
 * Token t of sequence n sits in page block_table[n, t / page] at slot
 * t % page.  The query attends every cached token t < seq_lens[n] (no mask
 * beyond the length).  The page pairs (32 tokens) of all (sequence, KV head)
 * segments are divided evenly over a fixed set of workers on the device; a
 * segment divided between workers is merged by its log-sum-exp.  The
 * division depends on seq_lens only, so equal inputs give bitwise equal
 * results, and it only changes rounding.
 *
 * Requirements checked on the host: N, Hq, Hkv, num_pages, max_blocks >= 1;
 * Hq % Hkv == 0; N * Hkv * ceil(max_blocks / 2) < 2^31; scale finite and
 * > 0; pointers aligned as for attn_fwd (block_table, seq_lens 4-byte).
 * page must be 16, d 64 or 128, dtype ATTN_BF16 and Hq / Hkv <= 16, else
 * ATTN_EUNSUPPORTED.
 *
 * Device contents are a caller contract: 0 <= seq_lens[n] <= max_blocks*page
 * and block_table[n, b] in [0, num_pages) for b < ceil(seq_lens[n] / page);
 * the values of entries past the end are never used.  The kernels never
 * dereference a page outside [0, num_pages) (such a block is skipped, and
 * that sequence's output is then unspecified), clamp lengths above max_blocks*page, and give a
 * sequence of length 0 the output 0 and log-sum-exp -inf.  Slots of a page at
 * or past the sequence length are never used, whatever they hold.
 */
int attn_decode_paged(const void* q, const void* k_pool, const void* v_pool,
                      const int32_t* block_table, const int32_t* seq_lens,
                      void* o, float* lse,
                      int N, int Hq, int Hkv, int d, int page, int num_pages,
                      int max_blocks, float scale, int dtype,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_decode_paged_fp8 -- attn_decode_paged over fp8 key/value pages.
 *
 *   k_pool, v_pool  [num_pages, Hkv, page, d]  uint8  E4M3 codes (OCP 8-bit
 *                   floating point, "fn" variant: sign, 4 exponent bits with
 *                   bias 7, 3 mantissa bits, no infinities, S.1111.111 NaN)
 *   k_scale, v_scale  float  per-tensor scales: K = k_scale * e4m3(code),
 *                            V = v_scale * e4m3(code)
 *   every other argument as for attn_decode_paged (q and o bf16; the same
 *   workspace size, attn_decode_workspace_size).
 *
 * "Fast attention kernels and operator fusion accelerate AI models",
 * section on kernel fusion: dequantisation is fused into the matrix product
 * that consumes it.  Here the codes are widened to bf16 (exactly: every
 * E4M3 value is a bf16 value) in registers right before the MFMAs; k_scale
 * folds into the logit scale and v_scale into the output normalisation, so
 * the result is attn_decode_paged's definition on the dequantised cache,
 * with half the bytes per token read from HBM.  A NaN code in a used slot
 * gives NaN results; slots past a sequence's length are never used.
 *
 * Requirements: as for attn_decode_paged, plus k_scale and v_scale finite
 * and > 0 (else ATTN_EINVAL), and k_pool, v_pool 16-byte aligned.
 */
int attn_decode_paged_fp8(const void* q, const void* k_pool, const void* v_pool,
                          float k_scale, float v_scale, const int32_t* block_table,
                          const int32_t* seq_lens, void* o, float* lse,
                          int N, int Hq, int Hkv, int d, int page, int num_pages,
                          int max_blocks, float scale, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * attn_decode_paged_int8 -- attn_decode_paged over int8 key/value pages.
 *
 *   k_pool, v_pool  [num_pages, Hkv, page, d]  8-bit two's-complement integer
 *                   codes (-128 .. 127, passed as bytes)
 *   k_scale, v_scale  float  per-tensor scales: K = k_scale * code,
 *                            V = v_scale * code (symmetric quantisation)
 *   every other argument as for attn_decode_paged_fp8.
 *
 * "Fast attention kernels and operator fusion accelerate AI models",
 * section on kernel fusion: dequantisation is fused into the matrix product
 * that consumes it; the integer format and per-tensor scales are our reading.
 * The codes are widened to bf16 in registers (exactly: every integer in
 * -128 .. 127 is a bf16 value) right before the MFMAs, k_scale folds into the
 * logit scale and v_scale into the output normalisation, so the result is
 * attn_decode_paged's definition on the dequantised cache with half the bytes
 * per token read from HBM.  Slots past a sequence's length are never used.
 *
 * Requirements: as for attn_decode_paged_fp8.
 */
int attn_decode_paged_int8(const void* q, const void* k_pool, const void* v_pool,
                           float k_scale, float v_scale, const int32_t* block_table,
                           const int32_t* seq_lens, void* o, float* lse,
                           int N, int Hq, int Hkv, int d, int page, int num_pages,
                           int max_blocks, float scale, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * attn_decode_paged_noalloc -- attn_decode_paged without a workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * Every argument, requirement and result is as for attn_decode_paged (bf16
 * pages); the same kernels run, with their scratch in a device-resident array
 * of the library instead of caller memory: 17,432,576 bytes on each device
 * the library runs on, held until the process ends, enough for
 * N * Hq <= 65536 (a larger N * Hq returns ATTN_EINVAL).  The call allocates
 * nothing.  Its first call on a device looks up that device's copy of the
 * array (an error there returns ATTN_EHIP).  The kernels run on the device
 * of `stream` (NULL: the calling thread's current device).  Every call on a
 * device shares that device's array: two calls that overlap in time on one
 * device race and their results are undefined; calls ordered on one stream
 * (or otherwise ordered) are safe.  Nothing in the array needs clearing
 * between calls.
 */
int attn_decode_paged_noalloc(const void* q, const void* k_pool, const void* v_pool,
                              const int32_t* block_table, const int32_t* seq_lens,
                              void* o, float* lse,
                              int N, int Hq, int Hkv, int d, int page, int num_pages,
                              int max_blocks, float scale, int dtype, void* stream);

/* Bytes of workspace attn_decode_paged needs for these sizes (0 if invalid):
 * r(N * Hq * 8) (which workers hold each sequence's pieces)
 * + r(2 * 768 * 16 * d * 4) (partial outputs) + r(2 * 768 * 16 * 4) (their
 * log-sum-exps), r() rounding up to a multiple of 256; about 13 MB at
 * d = 128.  It does not depend on max_blocks. */
size_t attn_decode_workspace_size(int N, int Hq, int d, int max_blocks, int page);

/* Static English name of a status code. */
const char* attn_status_string(int status);

/* Detail of the calling thread's last non-OK return ("" if none yet). */
const char* attn_last_error(void);

/*
 * attn_time_next_call -- kernel timing for profiling and benchmarks.
 *
 * start_event and stop_event are hipEvent_t handles (created by the caller
 * with timing enabled), passed as void*.  The calling thread's next call of a
 * computing entry point (attn_fwd, attn_fwd_window, attn_bwd,
 * attn_prefill_paged and the attn_decode_paged family) launches its first
 * kernel so that it records start_event when the kernel begins, and each of
 * its kernels so that it records stop_event when the kernel ends; after the
 * call's work has finished, hipEventElapsedTime(start, stop) is the time from
 * the start of its first kernel to the end of its last, without the time the
 * stream spends reaching the first kernel.  The events apply to that one call
 * only, whether it succeeds or fails, and are then forgotten.  Both NULL:
 * cancels a pending pair.  Exactly one NULL: ATTN_EINVAL.  The events are not
 * owned by the library.
 */
int attn_time_next_call(void* start_event, void* stop_event);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H_ */
