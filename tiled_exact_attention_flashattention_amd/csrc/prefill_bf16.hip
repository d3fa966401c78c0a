// prefill_bf16.hip -- tiled exact attention, bf16 inputs, fp32 accumulation.
//
// The method ("Advanced Attention Mechanisms - II", section Tiling, steps 1-3,
// and sections "Softmax stabiliser" / "Incremental / online softmax"):
// queries, keys and values are cut into tiles; each (Q tile, K/V tile) pair
// gives a tile of scaled scores that is folded into running row statistics
// (maximum m, normaliser l) and an output accumulator, so the full score
// matrix is never formed and only O and the row log-sum-exp leave the chip
// (same page, section "Flash Attention"; "Fast attention kernels and operator
// fusion accelerate AI models", section on FlashAttention-style attention).
// exp2 replaces exp with log2(e) folded into the scale ("Accelerating Mamba-2
// with high-performance forward-pass kernels in NVIDIA CUDA Tile", first
// kernel); since m is the running maximum every exponent is <= 0.
//
// gfx950 mapping:
//   * one workgroup = 4 waves = 128 query rows of one (batch, query head);
//     each wave owns 32 rows and keeps its Q rows in registers as MFMA
//     B-operands for the whole kernel;
//   * K and V tiles of BN keys are staged HBM -> registers -> LDS, double
//     buffered: the global loads of tile j+1 are in flight while tile j is
//     computed, and one barrier per tile separates the LDS phases;
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: lane l ends up holding 16 keys
//     of query row l%32 per 32-key block, so the row max needs one exchange
//     with lane l^32 and the row sum none until the end;
//   * the exponentiated scores are rounded to bf16 and used in place as the
//     B-operand of O^T = V^T P^T (same MFMA shape), with V^T read from the
//     row-major V tile by the gfx950 LDS transpose read; O^T's accumulator has
//     the same query-per-lane layout, so the rescale by exp2(m_old - m_new)
//     is a per-lane multiply;
//   * causal: K/V tiles past the workgroup's last visible key are never
//     loaded, a wave skips the MFMA work of tiles it cannot see, and only
//     tiles crossing the diagonal (or the ragged end) pay for the mask;
//   * heavy causal tiles are dispatched first, and when the number of
//     (batch, KV head) groups is a multiple of 8 every group stays on one XCD
//     so its K/V is re-read from that XCD's L2.
#include "cdna4.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

constexpr int kBM = 128;      // query rows per workgroup
constexpr int kThreads = 256; // 4 waves

// 16-byte-chunk swizzle of V row `row`: the transpose read touches 4
// consecutive rows x 64 bytes at once; XOR-ing the chunk index puts those rows
// in different bank groups (a row of D=128 spans all 64 banks, one of D=64
// half of them).  Depends on row bits 0-1 only, so it is the same for rows
// 16c + r and 16c + 8 + r.
template <int D>
__device__ __forceinline__ int v_swz_of(int row) {
  return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
}

template <int D> struct PrefillTile;
template <> struct PrefillTile<128> { static constexpr int BN = 64; };
template <> struct PrefillTile<64> { static constexpr int BN = 128; };

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_bf16_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                         const bf16* __restrict__ v, bf16* __restrict__ o,
                         float* __restrict__ lse, int B, int Hq, int Hkv, int T, int S,
                         float scale_log2) {
  constexpr int BN = PrefillTile<D>::BN;
  constexpr int LDK = D + 8;                 // padded K row in LDS, bf16 elements
  constexpr int KTILE = BN * LDK;            // one K tile in LDS
  constexpr int VTILE = BN * D;              // one V tile in LDS (unpadded, swizzled)
  constexpr int STAGE = KTILE + VTILE;
  constexpr int NKB = BN / 32;               // 32-key blocks of S^T
  constexpr int NDC = D / 16;                // k-chunks of the S^T MFMA
  constexpr int NDB = D / 32;                // 32-row blocks of O^T
  constexpr int NPC = BN / 16;               // k-chunks of the P.V MFMA
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int CPT = BN * CPR / kThreads;   // chunks per thread per tile
  static_assert(CPT * kThreads == BN * CPR, "tile must split evenly");
  auto v_swz = [](int row) { return v_swz_of<D>(row); };

  // LDS: 2 stages of [K tile (padded rows) | V tile (rows of D, 16-byte chunks
  // XOR-swizzled per row)].  K is read 16 rows x 16 bytes per bank cycle, which
  // the 16-byte row pad spreads over all banks; V is read by the transpose
  // read as 4 consecutive rows x 64 bytes, which the swizzle spreads instead.
  extern __shared__ __attribute__((aligned(16))) bf16 smem[];

  // ---- which (q tile, batch, head) this workgroup computes ----
  const int ntq = (T + kBM - 1) / kBM;
  const int hpg = Hq / Hkv;                  // query heads per KV head
  const int G = B * Hkv;                     // (batch, KV head) groups
  const int pid = blockIdx.x;
  int hgi, grp, rank;
  if ((G & 7) == 0) {
    // XCD pid%8 walks its own eighth of the groups: [tile rank][group][head].
    int s = pid >> 3;
    const int gpx = G >> 3;
    hgi = s % hpg;
    s /= hpg;
    grp = (pid & 7) * gpx + s % gpx;
    rank = s / gpx;
  } else {
    hgi = pid % hpg;
    const int s = pid / hpg;
    grp = s % G;
    rank = s / G;
  }
  const int b = grp / Hkv, hk = grp % Hkv, h = hk * hpg + hgi;
  const int qt = CAUSAL ? (ntq - 1 - rank) : rank;   // longest causal rows first
  const int q0 = qt * kBM;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hi = lane >> 5;

  const size_t qbase = ((size_t)(b * Hq + h) * T) * D;
  const size_t kvbase = ((size_t)(b * Hkv + hk) * S) * D;

  // ---- keys this workgroup / wave can see ----
  const int wrow0 = q0 + 32 * wave;                  // first row of this wave
  const bool wave_live = wrow0 < T;
  int wg_kv_end = S, wave_kv_end = S;                // exclusive
  if (CAUSAL) {
    wg_kv_end = min(S, min(q0 + kBM, T) + (S - T));
    wave_kv_end = min(S, min(wrow0 + 32, T) + (S - T));
  }
  const int ntk = (wg_kv_end + BN - 1) / BN;

  // ---- Q rows into registers (B operand of S^T = K Q^T) ----
  const int qrow = wrow0 + l32;
  bf16x8 qop[NDC];
  if (qrow < T) {
    const bf16* qp = q + qbase + (size_t)qrow * D + 8 * hi;
#pragma unroll
    for (int c = 0; c < NDC; ++c) qop[c] = *reinterpret_cast<const bf16x8*>(qp + 16 * c);
  } else {
#pragma unroll
    for (int c = 0; c < NDC; ++c) qop[c] = bf16x8{};
  }
  // last key visible to this lane's row (rows past T only feed discarded lanes)
  const int row_lim = CAUSAL ? min(qrow + (S - T), S - 1) : S - 1;

  // ---- tile staging ----
  u32x4 kr[CPT], vr[CPT];
  auto load_tile = [&](int j) {
#pragma unroll
    for (int r = 0; r < CPT; ++r) {
      const int c = tid + kThreads * r;
      const int row = c / CPR, col = c % CPR;
      const int key = j * BN + row;
      if (key < S) {
        const size_t off = kvbase + (size_t)key * D + col * 8;
        kr[r] = load16(k + off);
        vr[r] = load16(v + off);
      } else {
        kr[r] = u32x4{0, 0, 0, 0};
        vr[r] = u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&](int stage) {
    bf16* ks = smem + stage * STAGE;
    bf16* vs = ks + KTILE;
#pragma unroll
    for (int r = 0; r < CPT; ++r) {
      const int c = tid + kThreads * r;
      const int row = c / CPR, col = c % CPR;
      *reinterpret_cast<u32x4*>(ks + row * LDK + col * 8) = kr[r];
      *reinterpret_cast<u32x4*>(vs + row * D + (col ^ v_swz(row)) * 8) = vr[r];
    }
  };

  // ---- running softmax state of row qrow (replicated in lanes l, l^32) ----
  float m_run = -INFINITY;   // running max of scaled logits, log2 units
  float l_part = 0.f;        // sum over this lane's keys of exp2(s - m_run)
  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};

  // transpose-read addressing of V (see cdna4.hpp): lane group G = lane/16
  // covers rows d = 32*db + 16*(G&1) + lane%16 and key group hi = G>>1.  The
  // key row of this lane is 16*c + v_row_off (+8 for the second read); the
  // swizzle depends only on row bits that c and the +8 do not touch.
  const int g16 = lane >> 4, j16 = lane & 15;
  const int v_row_off = 4 * hi + (j16 >> 2);                  // key within a 16-key chunk
  // d of this lane's 8-byte row piece: 32*db + 16*(G&1) + 4*(j16&3), i.e.
  // 16-byte chunk 4*db + v_chunk, element v_in inside it
  const int v_chunk = 2 * (g16 & 1) + ((j16 & 3) >> 1);
  const int v_in = 4 * (j16 & 1);
  const int v_sw = v_swz(v_row_off);

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < ntk; ++j) {
    const int stage = j & 1;
    if (j + 1 < ntk) load_tile(j + 1);

    if (wave_live && j * BN < wave_kv_end) {
      const bf16* ks = smem + stage * STAGE;
      const bf16* vs = ks + KTILE;

      // S^T[key][row] for the BN keys of this tile.  The K operands of
      // d-chunk c+1 are read from LDS while the MFMAs of chunk c run, and the
      // NKB independent accumulators alternate so that dependent MFMAs are
      // not issued back to back.
      f32x16 s[NKB];
      const bf16* kp = ks + l32 * LDK + 8 * hi;
      bf16x8 kcur[NKB], knext[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        s[kb] = f32x16{};
        kcur[kb] = *reinterpret_cast<const bf16x8*>(kp + 32 * kb * LDK);
      }
#pragma unroll
      for (int c = 0; c < NDC; ++c) {
        if (c + 1 < NDC) {
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
            knext[kb] = *reinterpret_cast<const bf16x8*>(kp + 32 * kb * LDK + 16 * (c + 1));
        }
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) s[kb] = mfma_32x32x16(kcur[kb], qop[c], s[kb]);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) kcur[kb] = knext[kb];
      }

      // mask keys past the diagonal or past S (only tiles that need it)
      const bool need_mask = ((j + 1) * BN > S) || (CAUSAL && (j + 1) * BN - 1 > wrow0 + (S - T));
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = j * BN + 32 * kb + 8 * (i >> 2) + 4 * hi + (i & 3);
            if (key > row_lim) s[kb][i] = -INFINITY;
          }
      }

      // online softmax update (base 2)
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmax2(mx, s[kb][i]);
      mx = fmax2(mx, xor_lane(mx, 32));
      const float m_new = fmax2(m_run, mx * scale_log2);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = exp2_hw(m_run - m_use);
      m_run = m_new;
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = exp2_hw(__builtin_fmaf(s[kb][i], scale_log2, -m_use));
          s[kb][i] = p;
          rs += p;
        }
      l_part = __builtin_fmaf(l_part, alpha, rs);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;

      // O^T += V^T P^T, 16 keys at a time
#pragma unroll
      for (int c = 0; c < NPC; ++c) {
        const f32x16& sp = s[c >> 1];
        const int o8 = 8 * (c & 1);
        const bf16x8 pop = pack_bf16x8(sp[o8 + 0], sp[o8 + 1], sp[o8 + 2], sp[o8 + 3],
                                       sp[o8 + 4], sp[o8 + 5], sp[o8 + 6], sp[o8 + 7]);
        const bf16* vp = vs + (16 * c + v_row_off) * D + v_in;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int off = ((4 * db + v_chunk) ^ v_sw) * 8;
          const i16x4 lo = lds_read_tr16(vp + off);
          const i16x4 hi4 = lds_read_tr16(vp + 8 * D + off);
          acc[db] = mfma_32x32x16(concat_tr(lo, hi4), pop, acc[db]);
        }
      }
    }

    if (j + 1 < ntk) store_tile(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = acc / l (bf16, nearest even), LSE = ln2 * (m + log2 l) ----
  const float l_tot = l_part + xor_lane(l_part, 32);
  if (qrow < T) {
    const float inv = 1.f / l_tot;
    bf16* op = o + qbase + (size_t)qrow * D + 4 * hi;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        bf16x4 r;
        r[0] = (bf16)(acc[db][4 * jj + 0] * inv);
        r[1] = (bf16)(acc[db][4 * jj + 1] * inv);
        r[2] = (bf16)(acc[db][4 * jj + 2] * inv);
        r[3] = (bf16)(acc[db][4 * jj + 3] * inv);
        *reinterpret_cast<bf16x4*>(op + 32 * db + 8 * jj) = r;
      }
    if (lse != nullptr && hi == 0)
      lse[(size_t)(b * Hq + h) * T + qrow] = (m_run + log2f(l_tot)) * kLn2;
  }
}

template <int D, bool CAUSAL>
hipError_t launch_one(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int Hq, int Hkv, int T, int S, float scale_log2, hipStream_t stream) {
  constexpr int BN = PrefillTile<D>::BN;
  constexpr size_t smem = 2 * (size_t)BN * ((D + 8) + D) * sizeof(bf16);
  static bool attr_set = false;   // benign race: the attribute is idempotent
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)prefill_bf16_kernel<D, CAUSAL>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const long long ntq = (T + kBM - 1) / kBM;
  const long long grid = ntq * B * Hq;
  hipLaunchKernelGGL((prefill_bf16_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(kThreads), smem,
                     stream, static_cast<const bf16*>(q), static_cast<const bf16*>(k),
                     static_cast<const bf16*>(v), static_cast<bf16*>(o), lse, B, Hq, Hkv, T, S,
                     scale_log2);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                               int B, int Hq, int Hkv, int T, int S, int d, float scale_log2,
                               bool causal, hipStream_t stream) {
  if (d == 128)
    return causal ? launch_one<128, true>(q, k, v, o, lse, B, Hq, Hkv, T, S, scale_log2, stream)
                  : launch_one<128, false>(q, k, v, o, lse, B, Hq, Hkv, T, S, scale_log2, stream);
  return causal ? launch_one<64, true>(q, k, v, o, lse, B, Hq, Hkv, T, S, scale_log2, stream)
                : launch_one<64, false>(q, k, v, o, lse, B, Hq, Hkv, T, S, scale_log2, stream);
}

}  // namespace attn
