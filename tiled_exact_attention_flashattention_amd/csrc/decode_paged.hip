// decode_paged.hip -- one query token per sequence against a paged KV cache.
//
// The cache keeps keys and values in fixed-size pages and a block table maps
// each logical block of a sequence to its physical page; the kernel translates
// every position through that table ("Fast attention kernels and operator
// fusion accelerate AI models", section on FlashAttention-style and paged
// attention; 16-token pages as in its serving example).  The attention itself
// is the same online-softmax recurrence as the prefill kernel ("Advanced
// Attention Mechanisms - II", sections "Softmax stabiliser" and "Incremental /
// online softmax"); pieces of one sequence that are computed apart are merged
// by their log-sum-exp, LSE = M + ln sum_j exp(lse_j - M),
// O = sum_j exp(lse_j - LSE) O_j, the same rescaling the online softmax uses.
//
// Work distribution.  The unit of work is a page pair (32 keys) of one
// (sequence, KV head) segment; units are numbered sequence-major, then KV
// head, then pair.  A persistent grid of kDecodeWaves single-wave workgroups
// (3 per CU on 256 CUs) splits the U units into equal contiguous ranges, so
// every CU carries the same load: the kernel is bound by HBM and a CU's share
// of the bandwidth grows with the waves it holds, so an uneven spread of
// waves over CUs, not the bytes in flight, is what a fixed split size loses.
//   decode_stream_kernel: each wave finds its range from seq_lens (prefix
//     sums over 64 sequences at a time) and walks it.  A segment that lies
//     wholly inside the range is finished in place; a segment cut by a range
//     boundary leaves a normalised partial and its log-sum-exp in one of the
//     wave's two slots, and the wave holding the segment's first pair records
//     which waves hold its pieces.
//   decode_combine_kernel: one wave per (sequence, query head) merges the
//     pieces of cut segments and writes the output of empty sequences.  The
//     kernel boundary orders the partials' writes before their reads, which
//     a merge inside the first kernel would need device-wide fences for (on
//     this chip those write back and invalidate every XCD's L2).
//
// Inside a wave, page pairs (K and V, 16 KB at d = 128) are staged through a
// two-deep queue of registers: while one pair is consumed the next two are
// on their way, and the page ids of the pair after those travel with them.
// K of a pair is used straight from registers as MFMA A operands (each lane
// one key row, 16 bytes per d-chunk); V is copied row-major into the wave's
// LDS slice and read back transposed with the gfx950 LDS transpose read.
// All Hq/Hkv query heads of a KV head are the 16 columns of a 16x16x32 MFMA.
// Positions at or past the sequence length, and pages outside
// [0, num_pages), are masked and never dereferenced.
#include <mutex>
#include <type_traits>

#include "cdna4.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
constexpr int kPage = 16;
constexpr int kMinPairsPerWave = 4;   // fewer units than 4 per wave: use fewer waves
#ifndef DECODE_COMBINE_CH
#define DECODE_COMBINE_CH 16       // pieces whose partials one combine wave loads at a time
#endif

__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

__device__ __forceinline__ int wave_incl_scan(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const int y = __shfl_up(x, m);
    if (lane >= m) x += y;
  }
  return x;
}

// 16-byte-chunk swizzle of V row `row` in the wave's LDS slice.  The transpose
// read takes 8 consecutive rows x 32 bytes per half-wave; XOR-ing the chunk
// pair index spreads those rows over distinct bank groups.  Rows r and r+16
// (the same slot of the two pages of a pair) share the swizzle.
template <int D>
__device__ __forceinline__ int dv_swz(int row) {
  return D == 128 ? 2 * (row & 7) : 2 * ((row >> 1) & 3);
}

__device__ __forceinline__ int clamp_len(int len, int max_blocks) {
  return max(0, min(len, max_blocks * kPage));
}

// ---------------------------------------------------------------------------
// Stream kernel.

// Registers of one page pair in flight: K as A operands, V as row chunks.
// With fp8 pages each 16-byte load holds 16 codes: K two k-chunks of one key
// row, V half (D=64: all) of a row's 16-element chunk pair.
template <int D, bool FP8> struct PairRegs;
template <int D> struct PairRegs<D, false> {
  static constexpr int NDC = D / 32;                    // k-chunks of the S^T MFMA
  static constexpr int VCH = 2 * kPage * (D / 8) / 64;  // V chunks per lane
  bf16x8 k[2][NDC];
  u32x4 v[VCH];
};
template <int D> struct PairRegs<D, true> {
  static constexpr int NDC = D / 32;
  static constexpr int KLD = NDC / 2;                   // 16-byte K loads per page
  static constexpr int VCH = 2 * kPage * (D / 16) / 64; // 16-byte V loads per lane
  u32x4 k[2][KLD];
  u32x4 v[VCH];
};

// Page formats: bf16 values, or 8-bit codes with per-tensor scales.
constexpr int kFmtBf16 = 0, kFmtE4m3 = 1, kFmtInt8 = 2;

// Eight E4M3 codes (OCP "fn" format, as the conversion unit of this chip
// reads them) to bf16; every E4M3 value is exact in bf16.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
  const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(lo, false), b = __builtin_amdgcn_cvt_pk_f32_fp8(lo, true);
  const f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false), d = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
  return pack_bf16x8(a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]);
}

// Eight signed (two's-complement) bytes to bf16; every value -128 .. 127 is
// exact in bf16.
__device__ __forceinline__ float sbyte(uint32_t w, int i) {
  return (float)(int)(int8_t)(uint8_t)(w >> (8 * i));
}
__device__ __forceinline__ bf16x8 i8x8_to_bf16(uint32_t lo, uint32_t hi) {
  return pack_bf16x8(sbyte(lo, 0), sbyte(lo, 1), sbyte(lo, 2), sbyte(lo, 3), sbyte(hi, 0),
                     sbyte(hi, 1), sbyte(hi, 2), sbyte(hi, 3));
}

template <int FMT>
__device__ __forceinline__ bf16x8 codes8_to_bf16(uint32_t lo, uint32_t hi) {
  if constexpr (FMT == kFmtInt8) return i8x8_to_bf16(lo, hi);
  else return e4m3x8_to_bf16(lo, hi);
}

// One page pair, all fields wave-uniform.  n < 0 marks a padding pair.
struct PairMeta {
  int n, hk, p, np, len, u;   // sequence, KV head, pair in segment, pairs in segment, tokens, unit
  int tv0, tv1;               // tokens of page 0 / page 1 that take part (0: masked)
};

// FMT: bf16 pages, or E4M3 / int8 codes; with codes scale_log2 includes the
// key scale and v_scale multiplies the output (1 for bf16 pages).
template <int D, int FMT>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2)))
void decode_stream_kernel(const bf16* __restrict__ q, const void* __restrict__ kpool_v,
                          const void* __restrict__ vpool_v, const int32_t* __restrict__ block_table,
                          const int32_t* __restrict__ seq_lens, bf16* __restrict__ o,
                          float* __restrict__ lse, int2* __restrict__ seg_waves,
                          float* __restrict__ o_part, float* __restrict__ lse_part, int N, int Hq,
                          int Hkv, int num_pages, int max_blocks, float scale_log2, float v_scale) {
  constexpr bool FP8 = FMT != kFmtBf16;       // 8-bit codes (E4M3 or int8)
  using KV = typename std::conditional<FP8, uint8_t, bf16>::type;
  const KV* __restrict__ kpool = static_cast<const KV*>(kpool_v);
  const KV* __restrict__ vpool = static_cast<const KV*>(vpool_v);
  constexpr int NDC = PairRegs<D, FP8>::NDC;
  constexpr int VCH = PairRegs<D, FP8>::VCH;
  constexpr int NDB = D / 16;                 // 16-row blocks of O^T
  constexpr int CPR = D / 8;                  // 16-byte chunks per row

  __shared__ __attribute__((aligned(16))) bf16 vl[2 * kPage * D];   // one V pair, swizzled

  const int w = blockIdx.x;
  const int lane = threadIdx.x;
  auto pairs_of = [&](int n) {
    return n < N ? (clamp_len(seq_lens[n], max_blocks) + 2 * kPage - 1) / (2 * kPage) : 0;
  };

  // ---- this wave's unit range [a, b) and where it starts ----
  // (readfirstlane: the cross-lane sums are equal in every lane; saying so
  // keeps the whole walk in scalar registers and scalar branches)
  int pairs = 0;                              // page pairs of all sequences (< 2^31 / Hkv)
  for (int c0 = 0; c0 < N; c0 += 64)
    pairs += __builtin_amdgcn_readfirstlane(wave_sum(pairs_of(c0 + lane)));
  const int U = pairs * Hkv;
  const int W = U == 0 ? 0 : min(kDecodeWaves, max(1, U / kMinPairsPerWave));
  if (w >= W) return;
  const int a = (int)((long long)w * U / W), b = (int)((long long)(w + 1) * U / W);
  const int L = b - a;                        // >= 1 units
  int st_n = 0, st_np = 0, st_pairs_before = 0;
  for (int c0 = 0, base = 0;; c0 += 64) {     // sequence n whose units contain unit a
    const int np = pairs_of(c0 + lane);
    const int incl = wave_incl_scan(np);
    const unsigned long long hit = __builtin_amdgcn_ballot_w64((base + incl) * Hkv > a);
    if (hit != 0) {
      const int j = __builtin_ctzll(hit);
      st_n = c0 + j;
      st_np = __builtin_amdgcn_readlane(np, j);
      st_pairs_before = base + __builtin_amdgcn_readlane(incl, j) - st_np;
      break;
    }
    base += __builtin_amdgcn_readlane(incl, 63);
  }
  const int st_off = a - st_pairs_before * Hkv;
  const int4 st = make_int4(st_n, st_off / st_np, st_off % st_np, 0);

  const int G = Hq / Hkv;
  const int l16 = lane & 15, g = lane >> 4;
  const size_t page_stride = (size_t)Hkv * kPage * D;     // elements per page

  // wave holding unit u
  auto wave_of = [&](int u) { return (int)(((long long)(u + 1) * W - 1) / U); };

  // ---- cursor over this wave's units (wave-uniform) ----
  int c_k = 0, c_n = st.x, c_hk = st.y, c_p = st.z;
  int c_len = clamp_len(seq_lens[c_n], max_blocks);
  int c_np = (c_len + 2 * kPage - 1) / (2 * kPage);
  auto cur_meta = [&]() {
    PairMeta m;
    if (c_k < L) {
      m.n = c_n; m.hk = c_hk; m.p = c_p; m.np = c_np; m.len = c_len; m.u = a + c_k;
    } else {
      m.n = -1; m.hk = 0; m.p = 0; m.np = 1; m.len = 0; m.u = -1;
    }
    m.tv0 = m.tv1 = 0;
    return m;
  };
  auto advance = [&]() {
    if (++c_k >= L) return;
    if (++c_p < c_np) return;
    c_p = 0;
    if (++c_hk < Hkv) return;
    c_hk = 0;
    do {                                      // a later unit exists, so this ends before N
      ++c_n;
      c_len = clamp_len(seq_lens[c_n], max_blocks);
      c_np = (c_len + 2 * kPage - 1) / (2 * kPage);
    } while (c_np == 0);
  };
  // Page ids of the cursor's pair: lane 0 block 2p, lane 1 block 2p+1 (both
  // clamped to the last block), other lanes repeat them.  Padding reads entry 0.
  auto load_pid = [&]() {
    size_t idx = 0;
    if (c_k < L) {
      const int nblk = (c_len + kPage - 1) / kPage;
      idx = (size_t)c_n * max_blocks + min(2 * c_p + (lane & 1), nblk - 1);
    }
    return block_table[idx];
  };

  // ---- Q operand (B of S^T = K Q^T): column l16 = query head hk*G + l16 ----
  // k-slots of chunk c: d = 32 c + 8 g + (0..7); with fp8 pages the order
  // follows the 16-code K loads instead: chunk 2h + t takes d = 64 h + 16 g +
  // 8 t + (0..7) (any order of d serves, as long as K and Q share it)
  bf16x8 qop[NDC];
  int q_n = -1, q_hk = -1;
  auto load_q = [&](int n, int hk) {
    const bf16* qh = q + ((size_t)n * Hq + hk * G + min(l16, G - 1)) * D;
#pragma unroll
    for (int c = 0; c < NDC; ++c) {
      const int d0 = FP8 ? 64 * (c >> 1) + 16 * g + 8 * (c & 1) : 32 * c + 8 * g;
      qop[c] = *reinterpret_cast<const bf16x8*>(qh + d0);
    }
    if (l16 >= G) {
#pragma unroll
      for (int c = 0; c < NDC; ++c) qop[c] = bf16x8{};
    }
    q_n = n;
    q_hk = hk;
  };

  float m_run = -INFINITY, l_part = 0.f;
  f32x4 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x4{};

  // transpose-read address of this lane inside the slice (page 0; +16 rows for page 1)
  const int vrow = 4 * g + (l16 >> 2);
  const int vsw = dv_swz<D>(vrow);
  const bf16* vrd = vl + vrow * D + 4 * (l16 & 1);
  const int vchunk = (l16 & 3) >> 1;

  // K/V loads of pair m (page ids in pid): unconditional, so that the number
  // of loads in flight is the same on every path and the compiler's wait
  // counts stay exact.  A masked page (and a padding pair) reads page 0 of
  // KV head 0, which is in bounds and stays in L2.
  auto issue = [&](PairRegs<D, FP8>& r, int pid, PairMeta& m) {
    const int id0 = __builtin_amdgcn_readlane(pid, 0), id1 = __builtin_amdgcn_readlane(pid, 1);
    const bool ok0 = m.n >= 0 && id0 >= 0 && id0 < num_pages;
    const bool ok1 = m.n >= 0 && id1 >= 0 && id1 < num_pages;
    const int t0 = m.len - 2 * kPage * m.p;
    m.tv0 = ok0 ? max(0, min(t0, kPage)) : 0;
    m.tv1 = ok1 ? max(0, min(t0 - kPage, kPage)) : 0;
    const size_t head_off = (size_t)(m.n >= 0 ? m.hk : 0) * kPage * D;
    const size_t off0 = (ok0 ? (size_t)id0 * page_stride : 0) + head_off;
    const size_t off1 = (ok1 ? (size_t)id1 * page_stride : 0) + head_off;
    if constexpr (FP8) {
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const KV* kp = kpool + (p ? off1 : off0) + l16 * D + 16 * g;
#pragma unroll
        for (int h = 0; h < PairRegs<D, FP8>::KLD; ++h) r.k[p][h] = load16(kp + 64 * h);
      }
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const KV* vp = vpool + (p ? off1 : off0) + lane * 16;
#pragma unroll
        for (int c = 0; c < VCH / 2; ++c) r.v[p * (VCH / 2) + c] = load16(vp + 64 * 16 * c);
      }
    } else {
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const KV* kp = kpool + (p ? off1 : off0) + l16 * D + 8 * g;
#pragma unroll
        for (int c = 0; c < NDC; ++c) r.k[p][c] = *reinterpret_cast<const bf16x8*>(kp + 32 * c);
      }
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const KV* vp = vpool + (p ? off1 : off0) + lane * 8;
#pragma unroll
        for (int c = 0; c < VCH / 2; ++c) r.v[p * (VCH / 2) + c] = load16(vp + 64 * 8 * c);
      }
    }
  };

  // Writes the result of the piece that ends with pair m and resets the state.
  auto finish_piece = [&](const PairMeta& m) {
    const float l_tot = pair_sum32(pair_sum16(l_part));
    const float inv = l_tot > 0.f ? v_scale / l_tot : 0.f;
    const float lse_v = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
    const int s = m.u - m.p, e = s + m.np;
    if (s >= a && lane == 0)                  // this wave holds the segment's first pair
      seg_waves[(size_t)m.n * Hkv + m.hk] = make_int2(w, wave_of(e - 1));
    if (s >= a && e <= b) {                   // whole segment in this wave: final output
      if (l16 < G) {
        const size_t row = (size_t)m.n * Hq + m.hk * G + l16;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          bf16x4 x;
#pragma unroll
          for (int i = 0; i < 4; ++i) x[i] = (bf16)(acc[db][i] * inv);
          *reinterpret_cast<bf16x4*>(o + row * D + 16 * db + 4 * g) = x;
        }
        if (g == 0 && lse != nullptr) lse[row] = lse_v;
      }
    } else {                                  // cut segment: partial into slot (w, kind)
      const int kind = s < a ? 0 : 1;         // 1: the segment's first piece
      const size_t slot = 2 * (size_t)w + kind;
      if (l16 < G) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          *reinterpret_cast<f32x4*>(o_part + (slot * kDecodeMaxG + l16) * D + 16 * db + 4 * g) =
              acc[db] * inv;
        if (g == 0) lse_part[slot * kDecodeMaxG + l16] = lse_v;
      }
    }
    m_run = -INFINITY;
    l_part = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = f32x4{};
  };

  // One pair: V to LDS, S^T = K Q^T, the online-softmax update, then
  // O^T += V^T P^T.  As soon as S has consumed K, r takes the loads of pair
  // `mp` (page ids in pid), and pid takes the ids of the pair after that.
  auto step = [&](PairRegs<D, FP8>& r, PairMeta& mk, int& pid, PairMeta& mp) {
    const PairMeta m = mk;
    const u32x4 zero = {0, 0, 0, 0};
    if constexpr (FP8) {
      // V load c of page p holds codes 16 col .. +15 of row (lane + 64 c) / (D/16):
      // bf16 chunks 2 col and 2 col + 1 of that row
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int tv = p ? m.tv1 : m.tv0;
#pragma unroll
        for (int c = 0; c < VCH / 2; ++c) {
          const int ch = lane + 64 * c;
          const int slot = ch / (D / 16), col = ch % (D / 16);
          const int row = 16 * p + slot;
          const u32x4 raw = r.v[p * (VCH / 2) + c];
          const bf16x8 lo = codes8_to_bf16<FMT>(raw[0], raw[1]), hi = codes8_to_bf16<FMT>(raw[2], raw[3]);
          *reinterpret_cast<u32x4*>(vl + row * D + ((2 * col) ^ dv_swz<D>(row)) * 8) =
              slot < tv ? *reinterpret_cast<const u32x4*>(&lo) : zero;
          *reinterpret_cast<u32x4*>(vl + row * D + ((2 * col + 1) ^ dv_swz<D>(row)) * 8) =
              slot < tv ? *reinterpret_cast<const u32x4*>(&hi) : zero;
        }
      }
    } else {
      // V chunk c of page p is row (lane + 64 c) / CPR of that page
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int tv = p ? m.tv1 : m.tv0;
#pragma unroll
        for (int c = 0; c < VCH / 2; ++c) {
          const int ch = lane + 64 * c;
          const int slot = ch / CPR, col = ch % CPR;
          const int row = 16 * p + slot;
          *reinterpret_cast<u32x4*>(vl + row * D + (col ^ dv_swz<D>(row)) * 8) =
              slot < tv ? r.v[p * (VCH / 2) + c] : zero;
        }
      }
    }
    // A new segment needs its query rows.  The wait for them is taken inside
    // the branch (the empty asm consumes the registers), so the loop's other
    // paths keep their wait counts.
    if (m.n >= 0 && (m.n != q_n || m.hk != q_hk)) {
      load_q(m.n, m.hk);
#pragma unroll
      for (int c = 0; c < NDC; ++c) asm volatile("" ::"v"(qop[c]));
    }
    // S^T[key][head] for both pages
    f32x4 s[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      s[p] = f32x4{};
#pragma unroll
      for (int c = 0; c < NDC; ++c) {
        bf16x8 ka;
        if constexpr (FP8) {
          const u32x4 raw = r.k[p][c >> 1];
          ka = (c & 1) ? codes8_to_bf16<FMT>(raw[2], raw[3]) : codes8_to_bf16<FMT>(raw[0], raw[1]);
        } else {
          ka = r.k[p][c];
        }
        s[p] = mfma_16x16x32(ka, qop[c], s[p]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    issue(r, pid, mp);
    mk = mp;
    mp = cur_meta();
    pid = load_pid();
    advance();
    __builtin_amdgcn_sched_barrier(0);

    // mask positions past the length and masked pages (only a segment's last
    // pair, or a pair with a masked page, has any)
    if (m.tv0 < kPage || m.tv1 < kPage) {
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int tv = p ? m.tv1 : m.tv0;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (4 * g + i >= tv) s[p][i] = -INFINITY;
      }
    }

    float mx = max3_raw(max3_raw(s[0][0], s[0][1], s[0][2]), max3_raw(s[0][3], s[1][0], s[1][1]),
                        max3_raw(s[1][2], s[1][3], s[1][3]));
    mx = pair_max32_raw(pair_max16_raw(mx));
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

    if (m.n >= 0 && (m.p == m.np - 1 || m.u == b - 1)) finish_piece(m);
  };

  // ---- prologue: page ids of pairs 0 and 1, their K/V, then the ids of 2 and 3 ----
  load_q(st.x, st.y);
  PairMeta ma = cur_meta();
  int pida = load_pid();
  advance();
  PairMeta mb = cur_meta();
  int pidb = load_pid();
  advance();
  PairRegs<D, FP8> ra, rb;
  __builtin_amdgcn_sched_barrier(0);
  issue(ra, pida, ma);
  PairMeta mpa = cur_meta();
  pida = load_pid();
  advance();
  __builtin_amdgcn_sched_barrier(0);      // keep set a's loads ahead of set b's
  issue(rb, pidb, mb);
  PairMeta mpb = cur_meta();
  pidb = load_pid();
  advance();
  __builtin_amdgcn_sched_barrier(0);

  // Two register sets alternate and the loop always runs both steps (an odd
  // count gets one padding pair), so the loop has a single exit: with an exit
  // between the steps the compiler's wait counts would have to allow for
  // either order of the two sets and wait for both.
  int k = 0;                                  // L >= 1: no loop guard
  do {
    step(ra, ma, pida, mpa);
    step(rb, mb, pidb, mpb);
    k += 2;
  } while (k < L);
}

// One wave per (sequence, query head).  An empty sequence gets O = 0 and
// LSE = -inf; a segment finished by one wave is left alone; a cut segment's
// pieces (slot 2*w_first + 1, then slot 2*w for each later wave) are merged
// by their log-sum-exp.  Lane j keeps piece j's log-sum-exp (more than 64
// pieces are folded in a loop); each lane accumulates D/64 output elements,
// sixteen pieces' loads at a time.
template <int D>
__global__ __launch_bounds__(64)
void decode_combine_kernel(const int32_t* __restrict__ seq_lens, const int2* __restrict__ seg_waves,
                           const float* __restrict__ o_part, const float* __restrict__ lse_part,
                           bf16* __restrict__ o, float* __restrict__ lse, int Hq, int Hkv,
                           int max_blocks) {
  constexpr int PER = D / 64;
  constexpr int CH = DECODE_COMBINE_CH;
  const int nh = blockIdx.x;
  const int n = nh / Hq, h = nh - n * Hq;
  const int G = Hq / Hkv, hk = h / G, hh = h - hk * G;
  const int lane = threadIdx.x;
  bf16* orow = o + (size_t)nh * D + lane * PER;
  // both loads in one round trip (a segment's entry is only meaningful, and
  // only used, when the sequence is not empty)
  const int len = seq_lens[n];
  const int2 ws = seg_waves[(size_t)n * Hkv + hk];
  asm volatile("" ::"s"(len), "s"(ws.x), "s"(ws.y));   // (kept ahead of the branch)
  if (clamp_len(len, max_blocks) == 0) {
#pragma unroll
    for (int e = 0; e < PER; ++e) orow[e] = (bf16)0.f;
    if (lse != nullptr && lane == 0) lse[nh] = -INFINITY;
    return;
  }
  if (ws.x == ws.y) return;                   // finished in place
  if (ws.x < 0 || ws.y < ws.x || ws.y >= kDecodeWaves) return;   // never written: not ours
  const int npieces = ws.y - ws.x + 1;
  auto slot_of = [&](int j) { return (size_t)(2 * (ws.x + j) + (j == 0 ? 1 : 0)) * kDecodeMaxG + hh; };

  // loads of the first chunk of pieces (indices clamped to the last piece)
  float x[CH][PER];
#pragma unroll
  for (int u = 0; u < CH; ++u) {
    const float* op = o_part + slot_of(min(u, npieces - 1)) * D + lane * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) x[u][e] = op[e];
  }
  const float own = lane < npieces ? lse_part[slot_of(lane)] : -INFINITY;
  float M = own;
  for (int j = lane + 64; j < npieces; j += 64) M = fmax2(M, lse_part[slot_of(j)]);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) M = fmax2(M, xor_lane(M, m));
  float W = 0.f;
  if (M != -INFINITY) {
    W = lane < npieces ? expf(own - M) : 0.f;
    for (int j = lane + 64; j < npieces; j += 64) W += expf(lse_part[slot_of(j)] - M);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) W += xor_lane(W, m);

  float out[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) out[e] = 0.f;
  if (W > 0.f) {
    for (int j0 = 0;; j0 += CH) {
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        const int j = j0 + u;
        const float lj = j < 64 ? __shfl(own, j & 63) : lse_part[slot_of(min(j, npieces - 1))];
        const float wj = j < npieces ? expf(lj - M) : 0.f;
#pragma unroll
        for (int e = 0; e < PER; ++e) out[e] = __builtin_fmaf(wj, x[u][e], out[e]);
      }
      if (j0 + CH >= npieces) break;
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        const float* op = o_part + slot_of(min(j0 + CH + u, npieces - 1)) * D + lane * PER;
#pragma unroll
        for (int e = 0; e < PER; ++e) x[u][e] = op[e];
      }
    }
  }
  const float inv = W > 0.f ? 1.f / W : 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) orow[e] = (bf16)(out[e] * inv);
  if (lse != nullptr && lane == 0) lse[nh] = W > 0.f ? M + logf(W) : -INFINITY;
}

template <int D, int FMT>
hipError_t launch_d(const void* q, const void* k_pool, const void* v_pool,
                    const int32_t* block_table, const int32_t* seq_lens, void* o, float* lse,
                    const DecodeWorkspace& ws, int N, int Hq, int Hkv, int num_pages,
                    int max_blocks, float scale_log2, float v_scale, hipStream_t stream) {
  launch_kernel(decode_stream_kernel<D, FMT>, dim3(kDecodeWaves), dim3(64), 0, stream,
                     static_cast<const bf16*>(q), k_pool, v_pool, block_table, seq_lens,
                     static_cast<bf16*>(o), lse, ws.seg_waves, ws.o_part, ws.lse_part, N, Hq, Hkv,
                     num_pages, max_blocks, scale_log2, v_scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  launch_kernel(decode_combine_kernel<D>, dim3(N * Hq), dim3(64), 0, stream, seq_lens,
                     ws.seg_waves, ws.o_part, ws.lse_part, static_cast<bf16*>(o), lse, Hq, Hkv,
                     max_blocks);
  return hipGetLastError();
}

}  // namespace

// ---------------------------------------------------------------------------
// Scratch for callers that cannot allocate.  attn_decode_paged_noalloc runs
// the same two kernels with their workspace in this array instead of caller
// memory.  Each device holds its own copy until the process ends; in host
// code `scratch` names a host-side stand-in, so only the address that
// hipGetSymbolAddress returns for a device is ever handed to a kernel.  Calls
// that overlap in time on one device share the array and race.  Nothing in it
// needs clearing between calls: every entry the combine reads is written by
// the stream kernel of the same call.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

constexpr int kMaxScratchDevices = 64;

hipError_t decode_scratch(hipStream_t stream, void** ptr) {
  int dev = 0;
  hipError_t e = stream == nullptr ? hipGetDevice(&dev) : hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  static std::mutex mu;
  static void* table[kMaxScratchDevices] = {};
  std::lock_guard<std::mutex> lock(mu);
  if (table[dev] == nullptr) {
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    table[dev] = p;
  }
  *ptr = table[dev];
  return hipSuccess;
}

hipError_t launch_decode_paged(const void* q, const void* k_pool, const void* v_pool,
                               const int32_t* block_table, const int32_t* seq_lens, void* o,
                               float* lse, const DecodeWorkspace& ws, int N, int Hq, int Hkv,
                               int d, int num_pages, int max_blocks, float scale_log2,
                               int fmt, float v_scale, hipStream_t stream) {
#define ATTN_DECODE_LAUNCH(DD, FF)                                                           \
  launch_d<DD, FF>(q, k_pool, v_pool, block_table, seq_lens, o, lse, ws, N, Hq, Hkv, num_pages, \
                   max_blocks, scale_log2, FF == kFmtBf16 ? 1.f : v_scale, stream)
  if (fmt == kFmtE4m3) return d == 128 ? ATTN_DECODE_LAUNCH(128, kFmtE4m3) : ATTN_DECODE_LAUNCH(64, kFmtE4m3);
  if (fmt == kFmtInt8) return d == 128 ? ATTN_DECODE_LAUNCH(128, kFmtInt8) : ATTN_DECODE_LAUNCH(64, kFmtInt8);
  return d == 128 ? ATTN_DECODE_LAUNCH(128, kFmtBf16) : ATTN_DECODE_LAUNCH(64, kFmtBf16);
#undef ATTN_DECODE_LAUNCH
}

}  // namespace attn
