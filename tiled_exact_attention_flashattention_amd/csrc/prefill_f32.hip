// prefill_f32.hip -- tiled exact attention in float32 on the vector ALUs.
//
// Same method as the bf16 kernel ("Advanced Attention Mechanisms - II",
// section Tiling and the online-softmax section; the causal rule of
// "Accelerating Mamba-2 with high-performance forward-pass kernels in NVIDIA
// CUDA Tile"), kept in full float32 for callers that need fp32 results:
// one thread owns one query row (q and the output accumulator live in its
// registers), K/V tiles of BN keys are staged through LDS and read as
// broadcasts, and each tile updates the running max / normaliser with exp2.
#include "cdna4.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

constexpr int kRows = 128;   // query rows (= threads) per workgroup

template <int D> struct F32Tile;
template <> struct F32Tile<64> { static constexpr int BN = 32; };
template <> struct F32Tile<128> { static constexpr int BN = 16; };

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kRows)
void prefill_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                        const float* __restrict__ v, float* __restrict__ o,
                        float* __restrict__ lse, int B, int Hq, int Hkv, int T, int S,
                        float scale_log2, int window) {
  constexpr int BN = F32Tile<D>::BN;
  constexpr int V4 = BN * D / 4;             // float4 per tile
  __shared__ __attribute__((aligned(16))) float ks[BN * D];
  __shared__ __attribute__((aligned(16))) float vs[BN * D];

  const int ntq = (T + kRows - 1) / kRows;
  const int hpg = Hq / Hkv;
  int pid = blockIdx.x;
  const int h = pid % Hq;
  pid /= Hq;
  const int b = pid % B;
  const int rank = pid / B;
  const int qt = CAUSAL ? (ntq - 1 - rank) : rank;
  const int hk = h / hpg;
  const int q0 = qt * kRows;
  const int row = q0 + threadIdx.x;

  const size_t qbase = ((size_t)(b * Hq + h) * T) * D;
  const size_t kvbase = ((size_t)(b * Hkv + hk) * S) * D;

  float qv[D];
  if (row < T) {
#pragma unroll
    for (int c = 0; c < D; c += 4) {
      const float4 t = *reinterpret_cast<const float4*>(q + qbase + (size_t)row * D + c);
      qv[c] = t.x; qv[c + 1] = t.y; qv[c + 2] = t.z; qv[c + 3] = t.w;
    }
  } else {
#pragma unroll
    for (int c = 0; c < D; ++c) qv[c] = 0.f;
  }
  const int row_lim = CAUSAL ? min(row + (S - T), S - 1) : S - 1;
  // causal sliding window: keys <= row + (S - T) - window are hidden too
  const int row_lo = (CAUSAL && window > 0) ? row + (S - T) - window + 1 : 0;
  int kv_end = S, j0 = 0;
  if (CAUSAL) kv_end = min(S, min(q0 + kRows, T) + (S - T));
  if (CAUSAL && window > 0) j0 = max(0, q0 + (S - T) - window + 1) / BN;
  const int ntk = (kv_end + BN - 1) / BN;

  float m_run = -INFINITY, l_run = 0.f;
  float acc[D];
#pragma unroll
  for (int c = 0; c < D; ++c) acc[c] = 0.f;

  for (int j = j0; j < ntk; ++j) {
    __syncthreads();
    for (int i = threadIdx.x; i < V4; i += kRows) {
      const int key = j * BN + (i * 4) / D;
      float4 kk = make_float4(0.f, 0.f, 0.f, 0.f), vv = kk;
      if (key < S) {
        const size_t off = kvbase + (size_t)j * BN * D + (size_t)i * 4;
        kk = *reinterpret_cast<const float4*>(k + off);
        vv = *reinterpret_cast<const float4*>(v + off);
      }
      reinterpret_cast<float4*>(ks)[i] = kk;
      reinterpret_cast<float4*>(vs)[i] = vv;
    }
    __syncthreads();

    float sc[BN];
    float mx = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < BN; ++jj) {
      float dot = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) dot = __builtin_fmaf(qv[c], ks[jj * D + c], dot);
      sc[jj] = (j * BN + jj <= row_lim && j * BN + jj >= row_lo) ? dot : -INFINITY;
      mx = fmax2(mx, sc[jj]);
    }
    const float m_new = fmax2(m_run, mx * scale_log2);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2_hw(m_run - m_use);
    m_run = m_new;
    float rs = 0.f;
#pragma unroll
    for (int jj = 0; jj < BN; ++jj) {
      sc[jj] = exp2_hw(__builtin_fmaf(sc[jj], scale_log2, -m_use));
      rs += sc[jj];
    }
    l_run = __builtin_fmaf(l_run, alpha, rs);
#pragma unroll
    for (int c = 0; c < D; ++c) {
      float a = acc[c] * alpha;
#pragma unroll
      for (int jj = 0; jj < BN; ++jj) a = __builtin_fmaf(sc[jj], vs[jj * D + c], a);
      acc[c] = a;
    }
  }

  if (row < T) {
    float* op = o + qbase + (size_t)row * D;
#pragma unroll
    for (int c = 0; c < D; c += 4) {
      float4 t;
      t.x = acc[c] / l_run; t.y = acc[c + 1] / l_run;
      t.z = acc[c + 2] / l_run; t.w = acc[c + 3] / l_run;
      *reinterpret_cast<float4*>(op + c) = t;
    }
    if (lse != nullptr) lse[(size_t)(b * Hq + h) * T + row] = (m_run + log2f(l_run)) * kLn2;
  }
}

template <int D, bool CAUSAL>
hipError_t launch_one(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int Hq, int Hkv, int T, int S, float scale_log2, int window,
                      hipStream_t stream) {
  const long long ntq = (T + kRows - 1) / kRows;
  const long long grid = ntq * B * Hq;
  launch_kernel(prefill_f32_kernel<D, CAUSAL>, dim3((unsigned)grid), dim3(kRows), 0, stream,
                     static_cast<const float*>(q), static_cast<const float*>(k),
                     static_cast<const float*>(v), static_cast<float*>(o), lse, B, Hq, Hkv, T, S,
                     scale_log2, window);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_f32(const void* q, const void* k, const void* v, void* o, float* lse,
                              int B, int Hq, int Hkv, int T, int S, int d, float scale_log2,
                              bool causal, int window, hipStream_t stream) {
  if (d == 128)
    return causal ? launch_one<128, true>(q, k, v, o, lse, B, Hq, Hkv, T, S, scale_log2, window, stream)
                  : launch_one<128, false>(q, k, v, o, lse, B, Hq, Hkv, T, S, scale_log2, 0, stream);
  return causal ? launch_one<64, true>(q, k, v, o, lse, B, Hq, Hkv, T, S, scale_log2, window, stream)
                : launch_one<64, false>(q, k, v, o, lse, B, Hq, Hkv, T, S, scale_log2, 0, stream);
}

}  // namespace attn
