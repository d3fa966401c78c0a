// hbm_probe.hip -- read-only HBM bandwidth probe for the benchmark.
//
// Not part of the attention path and not linked into libattn.so: it is built
// into libattn_probe.so, which only the benchmark loads, to measure what a
// kernel that does nothing but read reaches on a given set of memory chunks.
// The paged decode must read the keys and values of every cached token once
// and paging does not change that byte count ("Fast attention kernels and
// operator fusion accelerate AI models", section on paged attention), so the
// probe reads exactly those chunks -- one key slab and one value slab per
// (page, KV head) of every sequence -- with the decode's grid shape (one-wave
// workgroups, equal contiguous ranges of units per wave), and reports how fast
// they can arrive with no compute, no block-table walk and no combine.  Given
// the chunks in ascending order of a contiguous buffer it measures plain
// sequential reading of the same byte count.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kUnroll = 4;   // units in flight per wave

// LPU 16-byte loads per lane per unit: a unit is LPU KiB of K and as much of V.
template <int LPU>
__global__ __launch_bounds__(64)
void probe_read_kernel(const u32x4* __restrict__ k, const u32x4* __restrict__ v,
                       const int32_t* __restrict__ units, int n, uint32_t* __restrict__ sink) {
  const int w = blockIdx.x, W = gridDim.x, lane = threadIdx.x;
  const int a = (int)((long long)w * n / W), b = (int)((long long)(w + 1) * n / W);
  uint32_t acc = 0;
  int u = a;
  for (; u + kUnroll <= b; u += kUnroll) {
    u32x4 r[kUnroll][2][LPU];
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) {
      const size_t base = (size_t)units[u + i] * (LPU * 64) + lane;
#pragma unroll
      for (int c = 0; c < LPU; ++c) {
        r[i][0][c] = k[base + (size_t)c * 64];
        r[i][1][c] = v[base + (size_t)c * 64];
      }
    }
#pragma unroll
    for (int i = 0; i < kUnroll; ++i)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int c = 0; c < LPU; ++c) acc ^= r[i][t][c][0] ^ r[i][t][c][1] ^ r[i][t][c][2] ^ r[i][t][c][3];
  }
  for (; u < b; ++u) {
    const size_t base = (size_t)units[u] * (LPU * 64) + lane;
#pragma unroll
    for (int c = 0; c < LPU; ++c) {
      const u32x4 x = k[base + (size_t)c * 64], y = v[base + (size_t)c * 64];
      acc ^= x[0] ^ x[1] ^ x[2] ^ x[3] ^ y[0] ^ y[1] ^ y[2] ^ y[3];
    }
  }
  sink[(size_t)w * 64 + lane] = acc;
}

}  // namespace

extern "C" {

// Reads, for every u < n_units, the unit_bytes at k_base + units[u] * unit_bytes
// and at v_base + units[u] * unit_bytes, with `waves` one-wave workgroups
// splitting the units into equal contiguous ranges; writes one word per lane
// to sink [waves * 64] uint32 (device memory).  unit_bytes must be 1, 2, 4 or
// 8 KiB; the caller guarantees every addressed unit lies inside its buffers.
// start_event / stop_event (hipEvent_t, both or neither): recorded as the
// kernel begins and ends, as the library's attn_time_next_call does.
// Returns 0, 1 on a bad argument, 3 on a launch error.
int attn_probe_read_units(const void* k_base, const void* v_base, const int32_t* units,
                          int n_units, int unit_bytes, uint32_t* sink, int waves, void* stream,
                          void* start_event, void* stop_event) {
  if (!k_base || !v_base || !units || !sink || n_units < 1 || waves < 1) return 1;
  if ((start_event == nullptr) != (stop_event == nullptr)) return 1;
  const u32x4* k = static_cast<const u32x4*>(k_base);
  const u32x4* v = static_cast<const u32x4*>(v_base);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipEvent_t e0 = static_cast<hipEvent_t>(start_event), e1 = static_cast<hipEvent_t>(stop_event);
  void (*kern)(const u32x4*, const u32x4*, const int32_t*, int, uint32_t*);
  switch (unit_bytes) {
    case 1024: kern = probe_read_kernel<1>; break;
    case 2048: kern = probe_read_kernel<2>; break;
    case 4096: kern = probe_read_kernel<4>; break;
    case 8192: kern = probe_read_kernel<8>; break;
    default: return 1;
  }
  if (e0 == nullptr) {
    hipLaunchKernelGGL(kern, dim3(waves), dim3(64), 0, st, k, v, units, n_units, sink);
  } else {
    hipExtLaunchKernelGGL(kern, dim3(waves), dim3(64), 0, st, e0, e1, 0u, k, v, units, n_units, sink);
  }
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

}  // extern "C"
