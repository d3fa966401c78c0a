// kernels.hpp -- host-side launchers of the HIP kernels (internal to libattn).
// Arguments are already validated by the C ABI layer; the launchers only pick
// the template instance and the grid, launch on `stream`, and report the HIP
// launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// Prefill, bf16 in/out, fp32 accumulation on MFMA.  scale_log2 = scale*log2(e).
hipError_t launch_prefill_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                               int B, int Hq, int Hkv, int T, int S, int d,
                               float scale_log2, bool causal, hipStream_t stream);

// Prefill, fp32 in/out, fp32 arithmetic on the vector ALUs.
hipError_t launch_prefill_f32(const void* q, const void* k, const void* v, void* o, float* lse,
                              int B, int Hq, int Hkv, int T, int S, int d,
                              float scale_log2, bool causal, hipStream_t stream);

// Paged decode: split kernel + log-sum-exp combine, back to back on `stream`.
// o_part/lse_part live in the caller's workspace with `max_splits` splits per
// (sequence, head); split_pages pages per split (even, >= 16).
hipError_t launch_decode_paged(const void* q, const void* k_pool, const void* v_pool,
                               const int32_t* block_table, const int32_t* seq_lens,
                               void* o, float* lse, float* o_part, float* lse_part,
                               int N, int Hq, int Hkv, int d, int num_pages, int max_blocks,
                               int split_pages, int max_splits, float scale_log2,
                               hipStream_t stream);

}  // namespace attn
