// decode_paged.hip -- one query token per sequence against a paged KV cache.
//
// The cache keeps keys and values in fixed-size pages and a block table maps
// each logical block of a sequence to its physical page; the kernel translates
// every position through that table ("Fast attention kernels and operator
// fusion accelerate AI models", section on FlashAttention-style and paged
// attention; 16-token pages as in its serving example).  The attention itself
// is the same online-softmax recurrence as the prefill kernel ("Advanced
// Attention Mechanisms - II", sections "Softmax stabiliser" and "Incremental /
// online softmax").
//
// A single query row cannot fill the machine, so the key range of each
// sequence is cut into splits of `split_pages` pages:
//   decode_split_kernel:  one workgroup per (split, KV head, sequence).  All
//     Hq/Hkv query heads that share the KV head are served from one read of
//     each K/V page (the query heads are the 16 columns of a 16x16x32 MFMA).
//     The 4 waves take page pairs round-robin, each with its own running
//     (m, l, acc); the waves are merged through LDS and the split writes its
//     normalised partial output and log-sum-exp to the workspace.
//   decode_combine_kernel: per (sequence, head) merges the splits by their
//     log-sum-exp: LSE = M + ln sum_s exp(lse_s - M), O = sum_s exp(lse_s - LSE) O_s.
// The combine is exact algebra of the same rescaling the online softmax uses.
//
// Memory: K of a page is read straight into MFMA A-operand registers (each
// lane one key row, 16 bytes per d-chunk); V of a page pair is copied
// row-major into the wave's LDS slice and read back transposed with the
// gfx950 LDS transpose read.  Positions at or past the sequence length, and
// pages outside [0, num_pages), are masked and never dereferenced.
#include "cdna4.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

constexpr int kPage = 16;
constexpr int kThreads = 256;
constexpr int kWaves = 4;

template <int D>
__global__ __launch_bounds__(kThreads)
void decode_split_kernel(const bf16* __restrict__ q, const bf16* __restrict__ kpool,
                         const bf16* __restrict__ vpool, const int32_t* __restrict__ block_table,
                         const int32_t* __restrict__ seq_lens, float* __restrict__ o_part,
                         float* __restrict__ lse_part, int Hq, int Hkv, int num_pages,
                         int max_blocks, int split_pages, int max_splits, float scale_log2) {
  constexpr int LDV = D + 8;                  // padded LDS row, bf16 elements
  constexpr int WAVE_LDS = 2 * kPage * LDV;   // one page pair, row-major [32][LDV]
  constexpr int NDC = D / 32;                 // k-chunks of the S^T MFMA
  constexpr int NDB = D / 16;                 // 16-row blocks of O^T
  constexpr int CPR = D / 8;                  // 16-byte chunks per row
  constexpr int VCH = 2 * kPage * CPR / 64;   // V chunks per lane per pair
  constexpr int RED_STRIDE = D + 4;           // fp32 row stride of the merge buffer

  extern __shared__ __attribute__((aligned(16))) bf16 smem[];

  const int split = blockIdx.x, hk = blockIdx.y, n = blockIdx.z;
  int len = seq_lens[n];
  len = max(0, min(len, max_blocks * kPage));
  const int blk0 = split * split_pages;
  if (blk0 * kPage >= len) return;            // whole workgroup: nothing in this split
  const int nblk = (len + kPage - 1) / kPage;
  const int blk_end = min(blk0 + split_pages, nblk);
  const int npairs = (blk_end - blk0 + 1) >> 1;

  const int G = Hq / Hkv;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g = lane >> 4;
  const int32_t* bt = block_table + (size_t)n * max_blocks;

  // Q operand (B of S^T = K Q^T): column l16 = query head hk*G + l16.
  bf16x8 qop[NDC];
  if (l16 < G) {
    const bf16* qp = q + ((size_t)n * Hq + hk * G + l16) * D + 8 * g;
#pragma unroll
    for (int c = 0; c < NDC; ++c) qop[c] = *reinterpret_cast<const bf16x8*>(qp + 32 * c);
  } else {
#pragma unroll
    for (int c = 0; c < NDC; ++c) qop[c] = bf16x8{};
  }

  float m_run = -INFINITY, l_part = 0.f;
  f32x4 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x4{};

  bf16* vl = smem + wave * WAVE_LDS;
  const size_t page_stride = (size_t)Hkv * kPage * D;     // elements per page
  const size_t head_off = (size_t)hk * kPage * D;

  for (int pi = wave; pi < npairs; pi += kWaves) {
    const int b0 = blk0 + 2 * pi;
    int pg[2];
    bool ok[2];
    pg[0] = bt[b0];
    ok[0] = pg[0] >= 0 && pg[0] < num_pages;
    const bool has1 = b0 + 1 < blk_end;
    pg[1] = has1 ? bt[b0 + 1] : 0;
    ok[1] = has1 && pg[1] >= 0 && pg[1] < num_pages;

    // K rows -> registers (A of S^T): lane key l16, d = 32c + 8g .. +7
    bf16x8 kop[2][NDC];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      if (ok[p]) {
        const bf16* kp = kpool + (size_t)pg[p] * page_stride + head_off + l16 * D + 8 * g;
#pragma unroll
        for (int c = 0; c < NDC; ++c) kop[p][c] = *reinterpret_cast<const bf16x8*>(kp + 32 * c);
      } else {
#pragma unroll
        for (int c = 0; c < NDC; ++c) kop[p][c] = bf16x8{};
      }
    }
    // V rows -> registers (coalesced 16-byte chunks), then row-major into LDS.
    // Rows at or past the length are zero: their weight is 0, and 0 * NaN
    // from a stale slot would otherwise poison the MFMA sum.
    u32x4 vreg[VCH];
#pragma unroll
    for (int r = 0; r < VCH; ++r) {
      const int c = lane + 64 * r;
      const int row = c / CPR, col = c % CPR;     // row 0..31: page row>>4, slot row&15
      const int p = row >> 4;
      if (ok[p] && (b0 + p) * kPage + (row & 15) < len) {
        vreg[r] = load16(vpool + (size_t)pg[p] * page_stride + head_off + (row & 15) * D + col * 8);
      } else {
        vreg[r] = u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int r = 0; r < VCH; ++r) {
      const int c = lane + 64 * r;
      const int row = c / CPR, col = c % CPR;
      *reinterpret_cast<u32x4*>(vl + row * LDV + col * 8) = vreg[r];
    }

    // S^T[key][head] for both pages
    f32x4 s[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      s[p] = f32x4{};
#pragma unroll
      for (int c = 0; c < NDC; ++c) s[p] = mfma_16x16x32(kop[p][c], qop[c], s[p]);
    }
    // mask positions past the length and blocks without a valid page
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = (b0 + p) * kPage + 4 * g + i;
        if (!ok[p] || tok >= len) s[p][i] = -INFINITY;
      }

    float mx = -INFINITY;
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmax2(mx, s[p][i]);
    mx = fmax2(mx, xor_lane(mx, 16));
    mx = fmax2(mx, xor_lane(mx, 32));
    const float m_new = fmax2(m_run, mx * scale_log2);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2_hw(m_run - m_use);
    m_run = m_new;
    float rs = 0.f;
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = exp2_hw(__builtin_fmaf(s[p][i], scale_log2, -m_use));
        s[p][i] = e;
        rs += e;
      }
    l_part = __builtin_fmaf(l_part, alpha, rs);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[db][i] *= alpha;

    // P operand (B of O^T = V^T P^T): slots 0-3 page 0 keys 4g+i, 4-7 page 1
    const bf16x8 pop = pack_bf16x8(s[0][0], s[0][1], s[0][2], s[0][3],
                                   s[1][0], s[1][1], s[1][2], s[1][3]);

    // the LDS writes above must land before other lanes of this wave read them
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // V^T operand: lane group g reads keys 4g..4g+3 of each page, d = 16db + l16
    const bf16* vp = vl + (4 * g + (l16 >> 2)) * LDV + 4 * (l16 & 3);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const i16x4 lo = lds_read_tr16(vp + 16 * db);
      const i16x4 hi4 = lds_read_tr16(vp + kPage * LDV + 16 * db);
      acc[db] = mfma_16x16x32(concat_tr(lo, hi4), pop, acc[db]);
    }

    // reads of this pair finish before the next pair overwrites the slice
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // ---- merge the 4 waves of this split through LDS ----
  float l_tot = l_part + xor_lane(l_part, 16);
  l_tot += xor_lane(l_tot, 32);
  __syncthreads();                                   // all V slices consumed
  float* red_o = reinterpret_cast<float*>(smem);     // [wave][16 heads][RED_STRIDE]
  float* red_m = red_o + kWaves * 16 * RED_STRIDE;   // [wave][16]
  float* red_l = red_m + kWaves * 16;                // [wave][16]
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      red_o[(wave * 16 + l16) * RED_STRIDE + 16 * db + 4 * g + i] = acc[db][i];
  if (g == 0) {
    red_m[wave * 16 + l16] = m_run;
    red_l[wave * 16 + l16] = l_tot;
  }
  __syncthreads();

  // thread -> (head, d-slice): 16 threads per head, D/16 values each
  const int hh = tid >> 4, part = tid & 15;
  if (hh < G) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmax2(M, red_m[w * 16 + hh]);
    float wgt[kWaves];
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      wgt[w] = (M == -INFINITY) ? 0.f : exp2f(red_m[w * 16 + hh] - M);
      L = __builtin_fmaf(red_l[w * 16 + hh], wgt[w], L);
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    const int head = hk * G + hh;
    const size_t slot = ((size_t)n * Hq + head) * max_splits + split;
    float* op = o_part + slot * D;
#pragma unroll
    for (int e = 0; e < D / 16; ++e) {
      const int d = part * (D / 16) + e;
      float x = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) x = __builtin_fmaf(red_o[(w * 16 + hh) * RED_STRIDE + d], wgt[w], x);
      op[d] = x * inv;
    }
    if (part == 0) lse_part[slot] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
  }
}

template <int D>
__global__ __launch_bounds__(64)
void decode_combine_kernel(const float* __restrict__ o_part, const float* __restrict__ lse_part,
                           const int32_t* __restrict__ seq_lens, bf16* __restrict__ o,
                           float* __restrict__ lse, int Hq, int max_blocks, int split_pages,
                           int max_splits) {
  constexpr int PER = D / 64;
  const int nh = blockIdx.x;
  const int n = nh / Hq;
  int len = seq_lens[n];
  len = max(0, min(len, max_blocks * kPage));
  const int nsplit = (len + split_pages * kPage - 1) / (split_pages * kPage);
  const float* lp = lse_part + (size_t)nh * max_splits;
  const float* op = o_part + (size_t)nh * max_splits * D;

  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmax2(M, lp[s]);
  float out[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) out[e] = 0.f;
  float W = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < nsplit; ++s) {
      const float w = expf(lp[s] - M);
      W += w;
#pragma unroll
      for (int e = 0; e < PER; ++e) out[e] = __builtin_fmaf(w, op[(size_t)s * D + threadIdx.x * PER + e], out[e]);
    }
  }
  const float inv = W > 0.f ? 1.f / W : 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) o[(size_t)nh * D + threadIdx.x * PER + e] = (bf16)(out[e] * inv);
  if (lse != nullptr && threadIdx.x == 0) lse[nh] = W > 0.f ? M + logf(W) : -INFINITY;
}

template <int D>
hipError_t launch_d(const void* q, const void* k_pool, const void* v_pool,
                    const int32_t* block_table, const int32_t* seq_lens, void* o, float* lse,
                    float* o_part, float* lse_part, int N, int Hq, int Hkv, int num_pages,
                    int max_blocks, int split_pages, int max_splits, float scale_log2,
                    hipStream_t stream) {
  constexpr size_t v_lds = (size_t)kWaves * 2 * kPage * (D + 8) * sizeof(bf16);
  constexpr size_t red_lds = ((size_t)kWaves * 16 * (D + 4) + 2 * kWaves * 16) * sizeof(float);
  constexpr size_t smem = v_lds > red_lds ? v_lds : red_lds;
  const int nsplit_grid = (max_blocks + split_pages - 1) / split_pages;
  hipLaunchKernelGGL((decode_split_kernel<D>), dim3(nsplit_grid, Hkv, N), dim3(kThreads), smem,
                     stream, static_cast<const bf16*>(q), static_cast<const bf16*>(k_pool),
                     static_cast<const bf16*>(v_pool), block_table, seq_lens, o_part, lse_part, Hq,
                     Hkv, num_pages, max_blocks, split_pages, max_splits, scale_log2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3(N * Hq), dim3(64), 0, stream, o_part,
                     lse_part, seq_lens, static_cast<bf16*>(o), lse, Hq, max_blocks, split_pages,
                     max_splits);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_paged(const void* q, const void* k_pool, const void* v_pool,
                               const int32_t* block_table, const int32_t* seq_lens, void* o,
                               float* lse, float* o_part, float* lse_part, int N, int Hq, int Hkv,
                               int d, int num_pages, int max_blocks, int split_pages,
                               int max_splits, float scale_log2, hipStream_t stream) {
  if (d == 128)
    return launch_d<128>(q, k_pool, v_pool, block_table, seq_lens, o, lse, o_part, lse_part, N, Hq,
                         Hkv, num_pages, max_blocks, split_pages, max_splits, scale_log2, stream);
  return launch_d<64>(q, k_pool, v_pool, block_table, seq_lens, o, lse, o_part, lse_part, N, Hq,
                      Hkv, num_pages, max_blocks, split_pages, max_splits, scale_log2, stream);
}

}  // namespace attn
