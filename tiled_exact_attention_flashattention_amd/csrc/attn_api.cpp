// attn_api.cpp -- the C ABI declared in include/attn.h.
//
// Every check runs on the host before any HIP call, so a rejected call has no
// side effect on the device and can be exercised without a GPU.  An
// unsupported input is reported, never computed some other way: forcing a
// backend that cannot take the inputs is an error ("Fast attention kernels and
// operator fusion accelerate AI models", section on FlashAttention-style
// attention; the serving example checks backend compatibility up front).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../include/attn.h"
#include "kernels.hpp"

namespace {

thread_local char g_last_error[256] = "";
thread_local attn::CallEvents g_call_events;

// Held by every computing entry point: whatever becomes of the call, timing
// events set by attn_time_next_call apply to it and to no later call.
struct CallEventsScope {
  ~CallEventsScope() { g_call_events = attn::CallEvents{}; }
};

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Byte ranges [p, p+n) and [q, q+m) intersect.
bool overlap(const void* p, size_t n, const void* q, size_t m) {
  if (p == nullptr || q == nullptr || n == 0 || m == 0) return false;
  const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
  return a < b + m && b < a + n;
}

constexpr int kPage = 16;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int64_t kMaxElems = (int64_t)1 << 40;
// One head's rows are addressed with 32-bit element offsets inside the kernels.
constexpr int64_t kMaxHeadElems = (int64_t)1 << 31;

size_t round256(int64_t x) { return (size_t)((x + 255) / 256 * 256); }

// Decode workspace: [segment -> (first, last) wave, N*Hq int2][partials of
// cut segments: 2 slots per wave x 16 heads x d floats][their log-sum-exps].
// Independent of the sequence lengths, which only the device sees.
struct WsLayout {
  size_t o_part, lse_part, total;
};

WsLayout decode_workspace_layout(int64_t N, int64_t Hq, int64_t d) {
  WsLayout l;
  l.o_part = round256(N * Hq * 8);
  l.lse_part = l.o_part + round256((int64_t)2 * attn::kDecodeWaves * attn::kDecodeMaxG * d * 4);
  l.total = l.lse_part + round256((int64_t)2 * attn::kDecodeWaves * attn::kDecodeMaxG * 4);
  return l;
}

}  // namespace

attn::CallEvents& attn::call_events() { return g_call_events; }

extern "C" {

int attn_time_next_call(void* start_event, void* stop_event) {
  if ((start_event == nullptr) != (stop_event == nullptr))
    return fail(ATTN_EINVAL, "attn_time_next_call: give both events or neither");
  g_call_events.start = static_cast<hipEvent_t>(start_event);
  g_call_events.stop = static_cast<hipEvent_t>(stop_event);
  return ATTN_OK;
}

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_EINVAL: return "ATTN_EINVAL: invalid argument";
    case ATTN_EUNSUPPORTED: return "ATTN_EUNSUPPORTED: input outside what the kernels support";
    case ATTN_EHIP: return "ATTN_EHIP: HIP runtime error";
    default: return "unknown attn status";
  }
}

const char* attn_last_error(void) { return g_last_error; }

size_t attn_bwd_workspace_size(int B, int Hq, int Hkv, int T, int S, int d) {
  if (B < 1 || Hq < 1 || Hkv < 1 || T < 1 || S < 1 || d < 1 || Hq % Hkv != 0) return 0;
  return round256((int64_t)B * Hq * T * 8) + attn::bwd_kv_part_bytes(B, Hq, Hkv, S, d);
}

size_t attn_decode_workspace_size(int N, int Hq, int d, int max_blocks, int page) {
  if (N < 1 || Hq < 1 || d < 1 || max_blocks < 1 || page != kPage) return 0;
  return decode_workspace_layout(N, Hq, d).total;
}

}  // extern "C"

namespace {

// attn_fwd and attn_fwd_window: `fn` names the entry point in messages.
int fwd_common(const char* fn, const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int Hq, int Hkv, int T, int S, int d, float scale, int causal, int window,
               int dtype, void* stream) {
  CallEventsScope events_scope;
  if (!q || !k || !v || !o) return fail(ATTN_EINVAL, "%s: q, k, v and o must be non-NULL", fn);
  if (B < 1 || Hq < 1 || Hkv < 1 || T < 1 || S < 1 || d < 1)
    return fail(ATTN_EINVAL, "%s: sizes must be >= 1 (B=%d Hq=%d Hkv=%d T=%d S=%d d=%d)", fn, B,
                Hq, Hkv, T, S, d);
  if (Hq % Hkv != 0) return fail(ATTN_EINVAL, "%s: Hq=%d is not a multiple of Hkv=%d", fn, Hq, Hkv);
  if (causal && T > S)
    return fail(ATTN_EINVAL, "%s: causal attention needs T <= S (T=%d S=%d)", fn, T, S);
  if (window < 0) return fail(ATTN_EINVAL, "%s: window must be >= 1", fn);
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(ATTN_EINVAL, "%s: scale must be finite and > 0", fn);
  if (dtype != ATTN_F32 && dtype != ATTN_BF16)
    return fail(ATTN_EUNSUPPORTED, "%s: unknown dtype %d", fn, dtype);
  if (d != 64 && d != 128) return fail(ATTN_EUNSUPPORTED, "%s: head dim %d (need 64 or 128)", fn, d);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      (lse && !aligned(lse, 4)))
    return fail(ATTN_EINVAL, "%s: q/k/v/o need 16-byte alignment, lse 4-byte", fn);
  const int64_t qn = (int64_t)B * Hq * T * d, kn = (int64_t)B * Hkv * S * d;
  if (qn > kMaxElems || kn > kMaxElems) return fail(ATTN_EINVAL, "%s: tensor too large", fn);
  if ((int64_t)T * d >= kMaxHeadElems || (int64_t)S * d >= kMaxHeadElems)
    return fail(ATTN_EINVAL, "%s: T*d and S*d must be below 2^31", fn);
  const int64_t grid = ((int64_t)T + 127) / 128 * B * Hq;
  if (grid > 0x7fffffff) return fail(ATTN_EINVAL, "%s: too many query tiles", fn);
  const size_t es = dtype == ATTN_BF16 ? 2 : 4;
  const size_t qb = qn * es, kb = kn * es, lb = lse ? (size_t)B * Hq * T * 4 : 0;
  if (overlap(o, qb, q, qb) || overlap(o, qb, k, kb) || overlap(o, qb, v, kb) ||
      overlap(lse, lb, q, qb) || overlap(lse, lb, k, kb) || overlap(lse, lb, v, kb) ||
      overlap(lse, lb, o, qb))
    return fail(ATTN_EINVAL, "%s: o/lse overlap an input or each other", fn);

  const float scale_log2 = scale * kLog2e;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = dtype == ATTN_BF16
                     ? attn::launch_prefill_bf16(q, k, v, o, lse, B, Hq, Hkv, T, S, d, scale_log2,
                                                 causal != 0, window, st)
                     : attn::launch_prefill_f32(q, k, v, o, lse, B, Hq, Hkv, T, S, d, scale_log2,
                                                causal != 0, window, st);
  if (e != hipSuccess) return fail(ATTN_EHIP, "%s: %s", fn, hipGetErrorString(e));
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
             int Hkv, int T, int S, int d, float scale, int causal, int dtype, void* stream) {
  return fwd_common("attn_fwd", q, k, v, o, lse, B, Hq, Hkv, T, S, d, scale, causal, 0, dtype,
                    stream);
}

int attn_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                    int Hq, int Hkv, int T, int S, int d, float scale, int window, int dtype,
                    void* stream) {
  if (window < 1) {
    g_call_events = attn::CallEvents{};
    return fail(ATTN_EINVAL, "attn_fwd_window: window must be >= 1 (got %d)", window);
  }
  return fwd_common("attn_fwd_window", q, k, v, o, lse, B, Hq, Hkv, T, S, d, scale, 1, window,
                    dtype, stream);
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int T, int S,
             int d, float scale, int causal, int dtype, void* workspace, size_t workspace_bytes,
             void* stream) {
  CallEventsScope events_scope;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !workspace)
    return fail(ATTN_EINVAL, "attn_bwd: every pointer must be non-NULL");
  if (B < 1 || Hq < 1 || Hkv < 1 || T < 1 || S < 1 || d < 1)
    return fail(ATTN_EINVAL, "attn_bwd: sizes must be >= 1 (B=%d Hq=%d Hkv=%d T=%d S=%d d=%d)", B,
                Hq, Hkv, T, S, d);
  if (Hq % Hkv != 0) return fail(ATTN_EINVAL, "attn_bwd: Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (causal && T > S)
    return fail(ATTN_EINVAL, "attn_bwd: causal attention needs T <= S (T=%d S=%d)", T, S);
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(ATTN_EINVAL, "attn_bwd: scale must be finite and > 0");
  if (dtype != ATTN_BF16) return fail(ATTN_EUNSUPPORTED, "attn_bwd: only bf16 is supported");
  if (d != 64 && d != 128) return fail(ATTN_EUNSUPPORTED, "attn_bwd: head dim %d (need 64 or 128)", d);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
      !aligned(lse, 4) || !aligned(workspace, 16))
    return fail(ATTN_EINVAL, "attn_bwd: tensors need 16-byte alignment, lse 4-byte");
  const int64_t qn = (int64_t)B * Hq * T * d, kn = (int64_t)B * Hkv * S * d;
  if (qn > kMaxElems || kn > kMaxElems) return fail(ATTN_EINVAL, "attn_bwd: tensor too large");
  if ((int64_t)T * d >= kMaxHeadElems || (int64_t)S * d >= kMaxHeadElems)
    return fail(ATTN_EINVAL, "attn_bwd: T*d and S*d must be below 2^31");
  if (((int64_t)T + 127) / 128 * B * Hq > 0x7fffffff || ((int64_t)S + 127) / 128 * B * Hq > 0x7fffffff ||
      ((int64_t)B * Hq * T + 15) / 16 > 0x7fffffff)
    return fail(ATTN_EINVAL, "attn_bwd: too many tiles");
  const size_t need = attn_bwd_workspace_size(B, Hq, Hkv, T, S, d);
  if (workspace_bytes < need)
    return fail(ATTN_EINVAL, "attn_bwd: workspace of %zu bytes needed, %zu given", need,
                workspace_bytes);
  const size_t qb = (size_t)qn * 2, kb = (size_t)kn * 2, lb = (size_t)B * Hq * T * 4;
  const void* ins[] = {q, k, v, o, lse, dout};
  const size_t in_bytes[] = {qb, kb, kb, qb, lb, qb};
  void* outs[] = {dq, dk, dv, workspace};
  const size_t out_bytes[] = {qb, kb, kb, need};
  for (int a = 0; a < 4; ++a) {
    for (int i = 0; i < 6; ++i)
      if (overlap(outs[a], out_bytes[a], ins[i], in_bytes[i]))
        return fail(ATTN_EINVAL, "attn_bwd: dq/dk/dv/workspace overlap an input");
    for (int c = a + 1; c < 4; ++c)
      if (overlap(outs[a], out_bytes[a], outs[c], out_bytes[c]))
        return fail(ATTN_EINVAL, "attn_bwd: dq, dk, dv and workspace must not overlap");
  }

  attn::BwdWorkspace bw;
  bw.stats = static_cast<float*>(workspace);
  bw.kv_part = attn::bwd_kv_part_bytes(B, Hq, Hkv, S, d) == 0
                   ? nullptr
                   : reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                              round256((int64_t)B * Hq * T * 8));
  hipError_t e = attn::launch_backward_bf16(q, k, v, o, lse, dout, dq, dk, dv, bw, B, Hq, Hkv, T,
                                            S, d, scale, causal != 0,
                                            static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(ATTN_EHIP, "attn_bwd: %s", hipGetErrorString(e));
  return ATTN_OK;
}

int attn_prefill_paged(const void* q, const void* k_pool, const void* v_pool,
                       const int32_t* block_table, const int32_t* seq_lens, const int32_t* q_lens,
                       void* o, float* lse, int N, int Hq, int Hkv, int T, int d, int page,
                       int num_pages, int max_blocks, float scale, int window, int dtype,
                       void* stream) {
  CallEventsScope events_scope;
  const char* fn = "attn_prefill_paged";
  if (!q || !k_pool || !v_pool || !block_table || !seq_lens || !q_lens || !o)
    return fail(ATTN_EINVAL, "%s: tensor pointers must be non-NULL", fn);
  if (N < 1 || Hq < 1 || Hkv < 1 || T < 1 || d < 1 || num_pages < 1 || max_blocks < 1 || page < 1)
    return fail(ATTN_EINVAL, "%s: sizes must be >= 1", fn);
  if (Hq % Hkv != 0) return fail(ATTN_EINVAL, "%s: Hq=%d is not a multiple of Hkv=%d", fn, Hq, Hkv);
  if (window < 0) return fail(ATTN_EINVAL, "%s: window must be >= 0", fn);
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(ATTN_EINVAL, "%s: scale must be finite and > 0", fn);
  if (dtype != ATTN_BF16) return fail(ATTN_EUNSUPPORTED, "%s: only bf16 is supported", fn);
  if (page != kPage) return fail(ATTN_EUNSUPPORTED, "%s: page size %d (need 16)", fn, page);
  if (d != 64 && d != 128) return fail(ATTN_EUNSUPPORTED, "%s: head dim %d (need 64 or 128)", fn, d);
  if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(o, 16) ||
      !aligned(block_table, 4) || !aligned(seq_lens, 4) || !aligned(q_lens, 4) ||
      (lse && !aligned(lse, 4)))
    return fail(ATTN_EINVAL, "%s: misaligned pointer", fn);
  const int64_t qn = (int64_t)N * Hq * T * d, pn = (int64_t)num_pages * Hkv * kPage * d;
  if (qn > kMaxElems || pn > kMaxElems || (int64_t)T * d >= kMaxHeadElems ||
      (int64_t)max_blocks * kPage > 0x7fffffff)
    return fail(ATTN_EINVAL, "%s: tensor too large", fn);
  if (((int64_t)T + 127) / 128 * N * Hq > 0x7fffffff)
    return fail(ATTN_EINVAL, "%s: too many query tiles", fn);
  const size_t qb = (size_t)qn * 2, pb = (size_t)pn * 2, lb = lse ? (size_t)N * Hq * T * 4 : 0;
  const size_t btb = (size_t)N * max_blocks * 4, nb = (size_t)N * 4;
  if (overlap(o, qb, q, qb) || overlap(o, qb, k_pool, pb) || overlap(o, qb, v_pool, pb) ||
      overlap(o, qb, block_table, btb) || overlap(o, qb, seq_lens, nb) ||
      overlap(o, qb, q_lens, nb) || overlap(lse, lb, q, qb) || overlap(lse, lb, k_pool, pb) ||
      overlap(lse, lb, v_pool, pb) || overlap(lse, lb, block_table, btb) ||
      overlap(lse, lb, seq_lens, nb) || overlap(lse, lb, q_lens, nb) || overlap(lse, lb, o, qb))
    return fail(ATTN_EINVAL, "%s: o/lse overlap an input or each other", fn);

  attn::PagedKv pkv;
  pkv.block_table = block_table;
  pkv.seq_lens = seq_lens;
  pkv.q_lens = q_lens;
  pkv.max_blocks = max_blocks;
  pkv.num_pages = num_pages;
  hipError_t e = attn::launch_prefill_paged_bf16(q, k_pool, v_pool, o, lse, pkv, N, Hq, Hkv, T, d,
                                                 scale * kLog2e, window,
                                                 static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(ATTN_EHIP, "%s: %s", fn, hipGetErrorString(e));
  return ATTN_OK;
}

}  // extern "C"

namespace {

// Page formats of the decode entry points (launch_decode_paged's fmt).
constexpr int kFmtBf16 = 0, kFmtE4m3 = 1, kFmtInt8 = 2;

// attn_decode_paged(_noalloc), attn_decode_paged_fp8 and attn_decode_paged_int8
// (8-bit code pools with per-tensor scales).
int decode_common(const char* fn, int fmt, const void* q, const void* k_pool, const void* v_pool,
                  float k_scale, float v_scale, const int32_t* block_table,
                  const int32_t* seq_lens, void* o, float* lse, int N, int Hq, int Hkv, int d,
                  int page, int num_pages, int max_blocks, float scale, int dtype,
                  void* workspace, size_t workspace_bytes, void* stream, bool noalloc = false) {
  CallEventsScope events_scope;
  if (!q || !k_pool || !v_pool || !block_table || !seq_lens || !o)
    return fail(ATTN_EINVAL, "%s: tensor pointers must be non-NULL", fn);
  if (N < 1 || Hq < 1 || Hkv < 1 || d < 1 || num_pages < 1 || max_blocks < 1 || page < 1)
    return fail(ATTN_EINVAL, "%s: sizes must be >= 1", fn);
  if (Hq % Hkv != 0)
    return fail(ATTN_EINVAL, "%s: Hq=%d is not a multiple of Hkv=%d", fn, Hq, Hkv);
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(ATTN_EINVAL, "%s: scale must be finite and > 0", fn);
  const bool codes8 = fmt != kFmtBf16;
  if (codes8 && (!std::isfinite(k_scale) || !(k_scale > 0.f) || !std::isfinite(v_scale) ||
              !(v_scale > 0.f) || !std::isfinite(scale * k_scale * kLog2e)))
    return fail(ATTN_EINVAL, "%s: k_scale and v_scale must be finite and > 0", fn);
  if (dtype != ATTN_BF16) return fail(ATTN_EUNSUPPORTED, "%s: only bf16 queries are supported", fn);
  if (page != kPage) return fail(ATTN_EUNSUPPORTED, "%s: page size %d (need 16)", fn, page);
  if (d != 64 && d != 128)
    return fail(ATTN_EUNSUPPORTED, "%s: head dim %d (need 64 or 128)", fn, d);
  if (Hq / Hkv > 16)
    return fail(ATTN_EUNSUPPORTED, "%s: %d query heads per KV head (max 16)", fn, Hq / Hkv);
  if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(o, 16) ||
      !aligned(block_table, 4) || !aligned(seq_lens, 4) || (lse && !aligned(lse, 4)))
    return fail(ATTN_EINVAL, "%s: misaligned pointer", fn);
  if ((int64_t)max_blocks * kPage > 0x7fffffff || (int64_t)num_pages * Hkv * kPage * d > kMaxElems)
    return fail(ATTN_EINVAL, "%s: cache too large", fn);
  if ((int64_t)N * Hq > 0x7fffffff / 1024 || N > 65535 || Hkv > 65535)
    return fail(ATTN_EINVAL, "%s: N, Hkv or N*Hq too large", fn);
  if ((int64_t)N * Hkv * ((max_blocks + 1) / 2) > 0x7fffffff)
    return fail(ATTN_EINVAL, "%s: too many page pairs (N*Hkv*max_blocks/2 >= 2^31)", fn);
  const WsLayout lay = decode_workspace_layout(N, Hq, d);
  if (noalloc) {
    if (workspace != nullptr || workspace_bytes != 0)
      return fail(ATTN_EINVAL, "%s: takes no workspace", fn);
    if ((int64_t)N * Hq > attn::kDecodeScratchMaxRows || lay.total > attn::kDecodeScratchBytes)
      return fail(ATTN_EINVAL,
                  "%s: N*Hq=%lld exceeds the %lld rows the static scratch (%zu bytes) holds", fn,
                  (long long)N * Hq, attn::kDecodeScratchMaxRows, attn::kDecodeScratchBytes);
  } else {
    if (!workspace || workspace_bytes < lay.total)
      return fail(ATTN_EINVAL, "%s: workspace of %zu bytes needed, %zu given", fn, lay.total,
                  workspace_bytes);
    if (!aligned(workspace, 16)) return fail(ATTN_EINVAL, "%s: misaligned workspace", fn);
  }
  {
    const size_t es = codes8 ? 1 : 2;
    const size_t qb = (size_t)N * Hq * d * 2, pb = (size_t)num_pages * Hkv * kPage * d * es;
    const size_t btb = (size_t)N * max_blocks * 4, nb = (size_t)N * 4;
    const size_t lb = lse ? (size_t)N * Hq * 4 : 0;
    const void* ins[] = {q, k_pool, v_pool, block_table, seq_lens};
    const size_t in_bytes[] = {qb, pb, pb, btb, nb};
    void* outs[] = {o, lse, workspace};
    const size_t out_bytes[] = {qb, lb, noalloc ? 0 : lay.total};
    for (int a = 0; a < 3; ++a) {
      for (int i = 0; i < 5; ++i)
        if (overlap(outs[a], out_bytes[a], ins[i], in_bytes[i]))
          return fail(ATTN_EINVAL, "%s: o, lse or the workspace overlaps an input", fn);
      for (int c = a + 1; c < 3; ++c)
        if (overlap(outs[a], out_bytes[a], outs[c], out_bytes[c]))
          return fail(ATTN_EINVAL, "%s: o, lse and the workspace must not overlap", fn);
    }
  }

  if (noalloc) {
    hipError_t e = attn::decode_scratch(static_cast<hipStream_t>(stream), &workspace);
    if (e != hipSuccess)
      return fail(ATTN_EHIP, "%s: static scratch: %s", fn, hipGetErrorString(e));
  }
  char* ws = static_cast<char*>(workspace);
  attn::DecodeWorkspace dw;
  dw.seg_waves = reinterpret_cast<int2*>(ws);
  dw.o_part = reinterpret_cast<float*>(ws + lay.o_part);
  dw.lse_part = reinterpret_cast<float*>(ws + lay.lse_part);
  const float scale_log2 = scale * kLog2e * (codes8 ? k_scale : 1.f);
  hipError_t e = attn::launch_decode_paged(q, k_pool, v_pool, block_table, seq_lens, o, lse, dw,
                                           N, Hq, Hkv, d, num_pages, max_blocks, scale_log2, fmt,
                                           v_scale, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(ATTN_EHIP, "%s: %s", fn, hipGetErrorString(e));
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_decode_paged(const void* q, const void* k_pool, const void* v_pool,
                      const int32_t* block_table, const int32_t* seq_lens, void* o, float* lse,
                      int N, int Hq, int Hkv, int d, int page, int num_pages, int max_blocks,
                      float scale, int dtype, void* workspace, size_t workspace_bytes,
                      void* stream) {
  return decode_common("attn_decode_paged", kFmtBf16, q, k_pool, v_pool, 1.f, 1.f, block_table,
                       seq_lens, o, lse, N, Hq, Hkv, d, page, num_pages, max_blocks, scale, dtype,
                       workspace, workspace_bytes, stream);
}

int attn_decode_paged_noalloc(const void* q, const void* k_pool, const void* v_pool,
                              const int32_t* block_table, const int32_t* seq_lens, void* o,
                              float* lse, int N, int Hq, int Hkv, int d, int page, int num_pages,
                              int max_blocks, float scale, int dtype, void* stream) {
  return decode_common("attn_decode_paged_noalloc", kFmtBf16, q, k_pool, v_pool, 1.f, 1.f,
                       block_table, seq_lens, o, lse, N, Hq, Hkv, d, page, num_pages, max_blocks,
                       scale, dtype, nullptr, 0, stream, true);
}

int attn_decode_paged_fp8(const void* q, const void* k_pool, const void* v_pool, float k_scale,
                          float v_scale, const int32_t* block_table, const int32_t* seq_lens,
                          void* o, float* lse, int N, int Hq, int Hkv, int d, int page,
                          int num_pages, int max_blocks, float scale, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return decode_common("attn_decode_paged_fp8", kFmtE4m3, q, k_pool, v_pool, k_scale, v_scale,
                       block_table, seq_lens, o, lse, N, Hq, Hkv, d, page, num_pages, max_blocks,
                       scale, ATTN_BF16, workspace, workspace_bytes, stream);
}

int attn_decode_paged_int8(const void* q, const void* k_pool, const void* v_pool, float k_scale,
                           float v_scale, const int32_t* block_table, const int32_t* seq_lens,
                           void* o, float* lse, int N, int Hq, int Hkv, int d, int page,
                           int num_pages, int max_blocks, float scale, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return decode_common("attn_decode_paged_int8", kFmtInt8, q, k_pool, v_pool, k_scale, v_scale,
                       block_table, seq_lens, o, lse, N, Hq, Hkv, d, page, num_pages, max_blocks,
                       scale, ATTN_BF16, workspace, workspace_bytes, stream);
}

}  // extern "C"
