// kernels.hpp -- host-side launchers of the HIP kernels (internal to libattn).
// Arguments are already validated by the C ABI layer; the launchers only pick
// the template instance and the grid, launch on `stream`, and report the HIP
// launch status.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// Timing events for the calling thread's next library call (attn_time_next_call):
// its first kernel records `start` as it begins, and each of its kernels records
// `stop` as it ends, so once the call's work is done `stop` holds the end of its
// last kernel.  Both null: plain launches.
struct CallEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
CallEvents& call_events();

// Every kernel of the library is launched through here.
template <typename K, typename... A>
inline void launch_kernel(K kernel, dim3 grid, dim3 block, uint32_t lds_bytes, hipStream_t stream,
                          A... args) {
  CallEvents& ev = call_events();
  if (ev.start == nullptr && ev.stop == nullptr) {
    hipLaunchKernelGGL(kernel, grid, block, lds_bytes, stream, args...);
  } else {
    hipExtLaunchKernelGGL(kernel, grid, block, lds_bytes, stream, ev.start, ev.stop, 0u, args...);
    ev.start = nullptr;
  }
}

// Prefill, bf16 in/out, fp32 accumulation on MFMA.  scale_log2 = scale*log2(e).
// window > 0 (causal only): sliding window of that many keys; 0: none.
hipError_t launch_prefill_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                               int B, int Hq, int Hkv, int T, int S, int d,
                               float scale_log2, bool causal, int window, hipStream_t stream);

// Chunked prefill on a paged cache (causal, bf16): sequence n's T_n =
// q_lens[n] queries (rows of q [N][Hq][T][d]) are the last T_n of its
// seq_lens[n] cached tokens, whose keys and values sit in 16-token pages
// [num_pages][Hkv][16][d] found through block_table [N][max_blocks].
struct PagedKv {
  const int32_t* block_table = nullptr;
  const int32_t* seq_lens = nullptr;
  const int32_t* q_lens = nullptr;
  int max_blocks = 0;
  int num_pages = 0;
};

hipError_t launch_prefill_paged_bf16(const void* q, const void* k_pool, const void* v_pool,
                                     void* o, float* lse, const PagedKv& pkv, int N, int Hq,
                                     int Hkv, int T, int d, float scale_log2, int window,
                                     hipStream_t stream);

// Prefill, fp32 in/out, fp32 arithmetic on the vector ALUs.
hipError_t launch_prefill_f32(const void* q, const void* k, const void* v, void* o, float* lse,
                              int B, int Hq, int Hkv, int T, int S, int d,
                              float scale_log2, bool causal, int window, hipStream_t stream);

// Paged decode: a persistent grid of kDecodeWaves single-wave workgroups that
// split all page pairs evenly, then a combine kernel for the sequences they
// cut.  Workspace pieces, all 16-byte aligned, laid out by the C ABI layer:
// Three waves per CU: enough 16 KiB page pairs in flight to keep HBM busy
// with fewer pieces per sequence (partials to merge) than four or more; a
// whole number per CU so that no CU holds more waves than the others.
#ifndef DECODE_WAVES
#define DECODE_WAVES 768
#endif
constexpr int kDecodeWaves = DECODE_WAVES;   // 3 per CU on 256 CUs
constexpr int kDecodeMaxG = 16;      // query heads per KV head, slot stride

struct DecodeWorkspace {
  int2* seg_waves;                   // [N * Hkv] first and last wave of each segment
  float* o_part;                     // [2 * kDecodeWaves][kDecodeMaxG][d] cut-segment partials
  float* lse_part;                   // [2 * kDecodeWaves][kDecodeMaxG]
};

// Device-resident decode scratch for attn_decode_paged_noalloc: a
// file-scope array in decode_paged.hip, one copy per device, large enough
// for the workspace layout of N * Hq <= kDecodeScratchMaxRows at d <= 128.
constexpr long long kDecodeScratchMaxRows = 65536;
constexpr size_t kDecodeScratchBytes =
    (size_t)kDecodeScratchMaxRows * 8 + (size_t)2 * kDecodeWaves * kDecodeMaxG * 128 * 4 +
    (size_t)2 * kDecodeWaves * kDecodeMaxG * 4;
static_assert(kDecodeScratchBytes % 256 == 0, "each region of the layout is a multiple of 256");

// Device address of that scratch on the device `stream` runs on (null: the
// calling thread's current device), looked up once per device with that
// device current.
hipError_t decode_scratch(hipStream_t stream, void** ptr);

// fmt: 0 bf16 pools; 1 E4M3 codes; 2 int8 codes.  With codes scale_log2
// includes the key scale and v_scale multiplies the output (ignored for bf16).
hipError_t launch_decode_paged(const void* q, const void* k_pool, const void* v_pool,
                               const int32_t* block_table, const int32_t* seq_lens,
                               void* o, float* lse, const DecodeWorkspace& ws,
                               int N, int Hq, int Hkv, int d, int num_pages, int max_blocks,
                               float scale_log2, int fmt, float v_scale, hipStream_t stream);

// Backward, bf16 in/out, fp32 accumulation on MFMA: dQ, whose kernel also
// writes the row statistics (LSE * log2 e, D = rowsum(dO * O)) into ws.stats
// [B*Hq*T][2] floats, then dK and dV; when the query heads of a group are divided between
// workgroups (bwd_kv_splits > 1), their fp32 partials go to ws.kv_part
// [splits][2][B*Hkv*S*d] and a last kernel sums them.  No atomics.
constexpr int kBwdTargetBlocks = 512;   // dK/dV workgroups wanted: two rounds of 256 CUs

struct BwdWorkspace {
  float* stats;
  float* kv_part;                      // null when bwd_kv_splits(...) == 1
};

// Head splits of the dK/dV kernel for these sizes: the smallest divisor n of
// Hq / Hkv with ceil(S / 128) * B * Hkv * n >= kBwdTargetBlocks (else Hq / Hkv).
int bwd_kv_splits(int B, int Hq, int Hkv, int S);
size_t bwd_kv_part_bytes(int B, int Hq, int Hkv, int S, int d);

hipError_t launch_backward_bf16(const void* q, const void* k, const void* v, const void* o,
                                const float* lse, const void* dout, void* dq, void* dk, void* dv,
                                const BwdWorkspace& ws, int B, int Hq, int Hkv, int T, int S,
                                int d, float scale, bool causal, hipStream_t stream);

}  // namespace attn
