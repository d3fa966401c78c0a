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
constexpr int kMaxSplitPages = 256;   // page ids of one split staged in LDS

// 16-byte-chunk swizzle of V row `row` in a wave's LDS slice.  The transpose
// read takes 8 consecutive rows x 32 bytes per half-wave; XOR-ing the chunk
// pair index spreads those rows over distinct bank groups.  Rows r and r+16
// (the same slot of the two pages of a pair) share the swizzle.
template <int D>
__device__ __forceinline__ int dv_swz(int row) {
  return D == 128 ? 2 * (row & 7) : 2 * ((row >> 1) & 3);
}

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void decode_split_kernel(const bf16* __restrict__ q, const bf16* __restrict__ kpool,
                         const bf16* __restrict__ vpool, const int32_t* __restrict__ block_table,
                         const int32_t* __restrict__ seq_lens, float* __restrict__ o_part,
                         float* __restrict__ lse_part, int Hq, int Hkv, int num_pages,
                         int max_blocks, int split_pages, int max_splits, float scale_log2) {
  constexpr int WAVE_LDS = 2 * kPage * D;     // one page pair, [32 rows][D], swizzled
  constexpr int NDC = D / 32;                 // k-chunks of the S^T MFMA
  constexpr int NDB = D / 16;                 // 16-row blocks of O^T
  constexpr int CPR = D / 8;                  // 16-byte chunks per row
  constexpr int VCH = 2 * kPage * CPR / 64;   // V chunks per lane per pair
  constexpr int RED_STRIDE = D + 4;           // fp32 row stride of the merge buffer

  // LDS: [4 wave slices of V][page ids of this split]; the merge buffer of
  // the epilogue reuses the V slices.
  extern __shared__ __attribute__((aligned(16))) bf16 smem[];
  int32_t* pages = reinterpret_cast<int32_t*>(smem + kWaves * WAVE_LDS);

  const int split = blockIdx.x, hk = blockIdx.y, n = blockIdx.z;
  int len = seq_lens[n];
  len = max(0, min(len, max_blocks * kPage));
  const int blk0 = split * split_pages;
  if (blk0 * kPage >= len) return;            // whole workgroup: nothing in this split
  const int nblk = (len + kPage - 1) / kPage;
  const int blk_end = min(blk0 + split_pages, nblk);
  const int nb = blk_end - blk0;              // blocks of this split
  const int npairs = (nb + 1) >> 1;

  const int G = Hq / Hkv;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g = lane >> 4;

  // page ids of the whole split, once (-1 marks a block outside [0, num_pages))
  for (int i = tid; i < nb; i += kThreads) {
    const int p = block_table[(size_t)n * max_blocks + blk0 + i];
    pages[i] = (p >= 0 && p < num_pages) ? p : -1;
  }

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
  __syncthreads();

  float m_run = -INFINITY, l_part = 0.f;
  f32x4 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x4{};

  bf16* vl = smem + wave * WAVE_LDS;
  const size_t page_stride = (size_t)Hkv * kPage * D;     // elements per page
  const size_t head_off = (size_t)hk * kPage * D;

  // transpose-read address of this lane inside a slice (page 0; +16 rows for page 1)
  const int vrow = 4 * g + (l16 >> 2);
  const int vsw = dv_swz<D>(vrow);
  const bf16* vrd = vl + vrow * D + 4 * (l16 & 1);
  const int vchunk = (l16 & 3) >> 1;

  // Loads of one page pair into registers: K as MFMA A-operands (lane key
  // l16, d = 32c + 8g..+7), V as coalesced 16-byte row chunks.  The loads are
  // unconditional so that each page needs one base address: a block without a
  // valid page reads page 0 instead (in bounds), and its scores are masked and
  // its V rows zeroed before use, like the slots at or past the length.
  auto page_of = [&](int blk) { return blk < nb ? max(pages[blk], 0) : 0; };
  auto issue_k = [&](int pi, bf16x8 (&kop)[2][NDC]) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const bf16* kp = kpool + (size_t)page_of(2 * pi + p) * page_stride + head_off + l16 * D + 8 * g;
#pragma unroll
      for (int c = 0; c < NDC; ++c) kop[p][c] = *reinterpret_cast<const bf16x8*>(kp + 32 * c);
    }
  };
  auto issue_v = [&](int pi, u32x4 (&vreg)[VCH]) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const bf16* vp = vpool + (size_t)page_of(2 * pi + p) * page_stride + head_off + lane * 8;
#pragma unroll
      for (int r = 0; r < VCH / 2; ++r) vreg[p * (VCH / 2) + r] = load16(vp + 64 * 8 * r);
    }
  };
  auto block_ok = [&](int blk) { return blk < nb && pages[blk] >= 0; };
  // V chunk r of page p is row (lane + 64 r) / CPR of that page
  auto write_v = [&](int pi, const u32x4 (&vreg)[VCH]) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const bool ok = block_ok(2 * pi + p);
#pragma unroll
      for (int r = 0; r < VCH / 2; ++r) {
        const int c = lane + 64 * r;
        const int slot = c / CPR, col = c % CPR;
        const int row = 16 * p + slot;
        const bool live = ok && (blk0 + 2 * pi + p) * kPage + slot < len;
        const u32x4 zero = {0, 0, 0, 0};
        *reinterpret_cast<u32x4*>(vl + row * D + (col ^ dv_swz<D>(row)) * 8) =
            live ? vreg[p * (VCH / 2) + r] : zero;
      }
    }
  };

  auto compute = [&](int pi, const bf16x8 (&kop)[2][NDC]) {
    const int bl = 2 * pi;
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
    for (int p = 0; p < 2; ++p) {
      const bool ok = block_ok(bl + p);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = (blk0 + bl + p) * kPage + 4 * g + i;
        if (!ok || tok >= len) s[p][i] = -INFINITY;
      }
    }

    float mx = fmax2(fmax2(fmax2(s[0][0], s[0][1]), fmax2(s[0][2], s[0][3])),
                     fmax2(fmax2(s[1][0], s[1][1]), fmax2(s[1][2], s[1][3])));
    mx = pair_max32(pair_max16(mx));
    const float m_new = fmax2(m_run, mx * scale_log2);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2_hw(m_run - m_use);
    const bool rescale = wave_any(m_new != m_run);
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
    if (rescale) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[db][i] *= alpha;
    }

    // P operand (B of O^T = V^T P^T): slots 0-3 page 0 keys 4g+i, 4-7 page 1
    const bf16x8 pop = pack_bf16x8(s[0][0], s[0][1], s[0][2], s[0][3],
                                   s[1][0], s[1][1], s[1][2], s[1][3]);

    // the LDS writes of this pair must land before other lanes read them
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // V^T operand: lane group g reads keys 4g..4g+3 of each page, d = 16db + l16
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int off = ((2 * db + vchunk) ^ vsw) * 8;
      const i16x4 lo = lds_read_tr16(vrd + off);
      const i16x4 hi4 = lds_read_tr16(vrd + kPage * D + off);
      acc[db] = mfma_16x16x32(concat_tr(lo, hi4), pop, acc[db]);
    }

    // reads of this pair finish before the next pair overwrites the slice
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  // Software pipeline: K has two register sets, V one (it moves to LDS at the
  // top of each step, after which its registers take the next pair's V).
  // The loads of pair pi + 4 are in flight while pair pi is computed.  Every
  // load is issued unconditionally -- past the last pair the index is clamped,
  // re-reading that pair from L2 -- so the number of loads in flight is the
  // same on every path and the compiler's wait counts stay exact; a load
  // behind a branch would make it wait for the prefetched pair as well.
  bf16x8 ka[2][NDC], kb[2][NDC];
  u32x4 vreg[VCH];
  if (wave < npairs) {
    auto clampp = [&](int pi) { return min(pi, npairs - 1); };
    issue_k(wave, ka);
    issue_v(wave, vreg);
    for (int pi = wave;; pi += 2 * kWaves) {
      write_v(pi, vreg);
      issue_k(clampp(pi + kWaves), kb);
      issue_v(clampp(pi + kWaves), vreg);
      compute(pi, ka);
      if (pi + kWaves >= npairs) break;
      write_v(pi + kWaves, vreg);
      issue_k(clampp(pi + 2 * kWaves), ka);
      issue_v(clampp(pi + 2 * kWaves), vreg);
      compute(pi + kWaves, kb);
      if (pi + 2 * kWaves >= npairs) break;
    }
  }

  // ---- merge the 4 waves of this split through LDS ----
  const float l_tot = pair_sum32(pair_sum16(l_part));
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

// One wave per (sequence, head): lane s holds split s's log-sum-exp (splits
// beyond 64 are folded in a loop), the wave reduces max and sum, then each
// lane accumulates D/64 output elements over the splits.
template <int D>
__global__ __launch_bounds__(64)
void decode_combine_kernel(const float* __restrict__ o_part, const float* __restrict__ lse_part,
                           const int32_t* __restrict__ seq_lens, bf16* __restrict__ o,
                           float* __restrict__ lse, int Hq, int max_blocks, int split_pages,
                           int max_splits) {
  constexpr int PER = D / 64;
  const int nh = blockIdx.x;
  const int n = nh / Hq;
  const int lane = threadIdx.x;
  int len = seq_lens[n];
  len = max(0, min(len, max_blocks * kPage));
  const int nsplit = (len + split_pages * kPage - 1) / (split_pages * kPage);
  const float* lp = lse_part + (size_t)nh * max_splits;
  const float* op = o_part + (size_t)nh * max_splits * D;

  float M = -INFINITY;
  for (int s = lane; s < nsplit; s += 64) M = fmax2(M, lp[s]);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) M = fmax2(M, xor_lane(M, m));
  float W = 0.f;
  if (M != -INFINITY)
    for (int s = lane; s < nsplit; s += 64) W += expf(lp[s] - M);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) W += xor_lane(W, m);

  float out[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) out[e] = 0.f;
  if (W > 0.f) {
    int s = 0;
    for (; s + 4 <= nsplit; s += 4) {
      float w[4], x[4][PER];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        w[u] = expf(lp[s + u] - M);
#pragma unroll
        for (int e = 0; e < PER; ++e) x[u][e] = op[(size_t)(s + u) * D + lane * PER + e];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < PER; ++e) out[e] = __builtin_fmaf(w[u], x[u][e], out[e]);
    }
    for (; s < nsplit; ++s) {
      const float w = expf(lp[s] - M);
#pragma unroll
      for (int e = 0; e < PER; ++e) out[e] = __builtin_fmaf(w, op[(size_t)s * D + lane * PER + e], out[e]);
    }
  }
  const float inv = W > 0.f ? 1.f / W : 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) o[(size_t)nh * D + lane * PER + e] = (bf16)(out[e] * inv);
  if (lse != nullptr && lane == 0) lse[nh] = W > 0.f ? M + logf(W) : -INFINITY;
}

template <int D>
hipError_t launch_d(const void* q, const void* k_pool, const void* v_pool,
                    const int32_t* block_table, const int32_t* seq_lens, void* o, float* lse,
                    float* o_part, float* lse_part, int N, int Hq, int Hkv, int num_pages,
                    int max_blocks, int split_pages, int max_splits, float scale_log2,
                    hipStream_t stream) {
  constexpr size_t v_lds = (size_t)kWaves * 2 * kPage * D * sizeof(bf16) + kMaxSplitPages * 4;
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
