// backward_bf16.hip -- gradients of tiled exact attention: dQ, dK, dV for
// bf16 inputs with fp32 accumulation.
//
// The forward pass keeps only the row log-sum-exp, not the attention matrix
// ("Advanced Attention Mechanisms - II", section "Flash Attention": the
// matrix is not stored for the backward pass), so every tile of
// probabilities is rebuilt here from Q, K and the saved LSE:
//     P = exp(scale q.k - LSE),  dP = dO V^T,  D = rowsum(dO * O),
//     dS = P * (dP - D),  dV = P^T dO,  dQ = scale dS K,  dK = scale dS^T Q,
// the chain rule of the forward definition (the same scores, causal mask and
// grouped-query mapping as attn_fwd).
//
// Two kernels (three with head splits), no atomics, so results are
// bit-reproducible:
//   bwd_dq_kernel:    one workgroup per 128 query rows of one (batch, head),
//     shaped like the forward kernel: Q and dO stay in registers as MFMA B
//     operands, K and V tiles stream through two LDS stages by the
//     direct-to-LDS load; per tile S^T = K Q^T, dP^T = V dO^T, P, dS, and
//     dQ^T += K^T dS^T with K^T from the LDS transpose read.  Its prologue
//     forms each row's statistics (LSE * log2 e, D = rowsum(dO * O)) in fp32
//     and writes them to the workspace for the dK/dV kernel.
//   bwd_dkdv_kernel:  one workgroup of 8 waves per 128 keys of one (batch, KV
//     head); a pair of waves shares 32 keys (two 16-key blocks): one keeps
//     their K as MFMA B operands and accumulates dV, the other keeps V and
//     accumulates dK.  Both walk every query tile (32 rows) of every query
//     head of the group (or of its share of them, when the heads are split
//     between workgroups) that can see the keys.  Q and dO tiles and their
//     rows' statistics stream through a four-stage LDS ring by the
//     direct-to-LDS load.  Per tile the dV wave forms S = Q K^T and P, hands
//     P to its partner through LDS and adds P^T dO; the dK wave, one tile
//     behind, forms dP = dO V^T and dS = P (dP - D) and adds dS^T Q (dO and Q
//     from the transpose read).  Summing the group's heads in registers keeps
//     the grouped-query reduction exact in order.
// Tiles read both as MFMA row operands and through the transpose read use the
// dual swizzle of lds_stage.hpp, bank-conflict free for both.
#include "cdna4.hpp"
#include "kernels.hpp"
#include "lds_stage.hpp"

namespace attn {
namespace {

// ---------------------------------------------------------------------------
// dQ.  Workgroup = 4 waves x 32 query rows (two 16-row blocks per wave).
constexpr int kDqBN = 64;                    // keys per K/V tile

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_dq_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                   const bf16* __restrict__ v, const bf16* __restrict__ dout,
                   const bf16* __restrict__ o, const float* __restrict__ lse,
                   float* __restrict__ stats, bf16* __restrict__ dq, int B, int Hq,
                   int Hkv, int T, int S,
                   float scale_log2, float scale) {
  constexpr int BN = kDqBN;
  constexpr int kBM = 128;
  constexpr int CPR = D / 8;
  constexpr int NDC = D / 32;
  constexpr int NDB = D / 16;
  constexpr int NPC = BN / 32;
  constexpr int CPW = BN * CPR / 256;
  static_assert(CPW * 256 == BN * CPR, "tile must split evenly");

  __shared__ __attribute__((aligned(16))) bf16 k_st0[BN * D];
  __shared__ __attribute__((aligned(16))) bf16 k_st1[BN * D];
  __shared__ __attribute__((aligned(16))) bf16 v_st0[BN * D];
  __shared__ __attribute__((aligned(16))) bf16 v_st1[BN * D];

  // ---- (q tile, batch, head); longest causal rows first ----
  const int ntq = (T + kBM - 1) / kBM;
  const int hpg = Hq / Hkv;
  const int G = B * Hkv;
  const int pid = blockIdx.x;
  int hgi, grp, rank;
  if ((G & 7) == 0) {
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
  const int qt = CAUSAL ? (ntq - 1 - rank) : rank;
  const int q0 = qt * kBM;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g = lane >> 4;
  const size_t qbase = ((size_t)(b * Hq + h) * T) * D;
  const size_t kvbase = ((size_t)(b * Hkv + hk) * S) * D;

  const int wrow0 = q0 + 32 * wave;
  const bool wave_live = wrow0 < T;
  int wg_kv_end = S, wave_kv_end = S;
  if (CAUSAL) {
    wg_kv_end = min(S, min(q0 + kBM, T) + (S - T));
    wave_kv_end = min(S, min(wrow0 + 32, T) + (S - T));
  }
  const int ntk = (wg_kv_end + BN - 1) / BN;

  // ---- direct-to-LDS tile loads (see the forward kernel) ----
  const bf16* kg = k + kvbase;
  const bf16* vg = v + kvbase;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  uint32_t toff[CPW];
  int lrow[CPW];
#pragma unroll
  for (int r = 0; r < CPW; ++r) {
    const int p = 64 * (wave * CPW + r) + lane;
    const int row = p / CPR, cph = p % CPR;
    lrow[r] = row;
    toff[r] = (uint32_t)(row * D + (cph ^ dual_swz<D>(row)) * 8) * 2u;
  }
  auto load_tile = [&](int j, bf16* ks, bf16* vs) {
    const uint32_t kl = lds_addr(ks) + (uint32_t)(wave_s * CPW) * 1024u;
    const uint32_t vl = lds_addr(vs) + (uint32_t)(wave_s * CPW) * 1024u;
    const bool full = (j + 1) * BN <= S;
    if (full) {
      // the tile's offset goes into the scalar base: no per-lane arithmetic
      const void* kt = uniform_ptr(kg + (size_t)j * BN * D);
      const void* vt = uniform_ptr(vg + (size_t)j * BN * D);
#pragma unroll
      for (int r = 0; r < CPW; ++r) {
        lds_dma16(kt, toff[r], kl + 1024u * r);
        lds_dma16(vt, toff[r], vl + 1024u * r);
      }
    } else {
#pragma unroll
      for (int r = 0; r < CPW; ++r) {
        const int key = min(j * BN + lrow[r], S - 1);
        const uint32_t add = (uint32_t)((key - lrow[r]) * D) * 2u;
        lds_dma16(kg, toff[r] + add, kl + 1024u * r);
        lds_dma16(vg, toff[r] + add, vl + 1024u * r);
      }
    }
  };

  // ---- Q and dO rows (B operands), LSE (log2 units) and D of this lane's rows ----
  bf16x8 qop[2][NDC], dop[2][NDC];
  int row_lim[2];
  float lse2[2], dd[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = wrow0 + 16 * qb + l16;
    float dpart = 0.f;                       // this lane's share of rowsum(dO * O)
    if (row < T) {
      const bf16* qp = q + qbase + (size_t)row * D + 8 * g;
      const bf16* dp = dout + qbase + (size_t)row * D + 8 * g;
      const bf16* op = o + qbase + (size_t)row * D + 8 * g;
#pragma unroll
      for (int c = 0; c < NDC; ++c) {
        qop[qb][c] = *reinterpret_cast<const bf16x8*>(qp + 32 * c);
        dop[qb][c] = *reinterpret_cast<const bf16x8*>(dp + 32 * c);
        const bf16x8 ov = *reinterpret_cast<const bf16x8*>(op + 32 * c);
#pragma unroll
        for (int e = 0; e < 8; ++e) dpart = __builtin_fmaf((float)dop[qb][c][e], (float)ov[e], dpart);
      }
      lse2[qb] = lse[(size_t)(b * Hq + h) * T + row] * kLog2e;
    } else {
#pragma unroll
      for (int c = 0; c < NDC; ++c) qop[qb][c] = dop[qb][c] = bf16x8{};
      lse2[qb] = 0.f;
    }
    // the four lanes of a row (g = 0..3) hold its D / 4 chunks of 8 elements each
    dpart += __shfl_xor(dpart, 16);
    dpart += __shfl_xor(dpart, 32);
    dd[qb] = dpart;
    if (row < T && g == 0)
      *reinterpret_cast<float2*>(stats + 2 * ((size_t)(b * Hq + h) * T + row)) = make_float2(lse2[qb], dpart);
    row_lim[qb] = CAUSAL ? min(row + (S - T), S - 1) : S - 1;
  }

  f32x4 dqt[2][NDB];                          // dQ^T[d][row]
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < NDB; ++db) dqt[qb][db] = f32x4{};

  const int swz_l = dual_swz<D>(l16);                        // row 16 kb + l16
  const int t_row = 4 * g + (l16 >> 2);                      // transpose-read row in a 32-key chunk
  const int t_chunk = (l16 & 3) >> 1;
  const int t_in = 4 * (l16 & 1);

  auto compute_tile = [&](int j, const bf16* ks, const bf16* vs) {
    const bool need_mask = ((j + 1) * BN > S) || (CAUSAL && (j + 1) * BN - 1 > wrow0 + (S - T));
    // 32 keys at a time (keeps the score registers to one chunk)
#pragma unroll
    for (int c = 0; c < NPC; ++c) {
      // S^T[key][row] = K Q^T and dP^T[key][row] = V dO^T for keys 32 c + 16 kk + ...
      f32x4 s[2][2], dp[2][2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) s[0][kk] = s[1][kk] = dp[0][kk] = dp[1][kk] = f32x4{};
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int off = (32 * c + 16 * kk + l16) * D + (((4 * dc + g) ^ swz_l) * 8);
          const bf16x8 kop = *reinterpret_cast<const bf16x8*>(ks + off);
          const bf16x8 vop = *reinterpret_cast<const bf16x8*>(vs + off);
          s[0][kk] = mfma_16x16x32(kop, qop[0][dc], s[0][kk]);
          s[1][kk] = mfma_16x16x32(kop, qop[1][dc], s[1][kk]);
          dp[0][kk] = mfma_16x16x32(vop, dop[0][dc], dp[0][kk]);
          dp[1][kk] = mfma_16x16x32(vop, dop[1][dc], dp[1][kk]);
        }
      }
      // at d = 128 the K and V reads go four units ahead of their MFMAs, and
      // below the transpose reads four ahead of theirs (backward_3 856 -> 830
      // us, bit-identical; at d = 64 1-2 % slower, so left to the scheduler)
      if constexpr (D == 128) sched_reads_ahead<NDC * 2, 2, 4, 4>();
      // dS^T = P^T * (dP^T - D), P^T = exp2(scale_log2 s - LSE2), then zero
      // on keys a row cannot see (only tiles that need it: a select folded
      // into the loop above would cost two VALU instructions per score on
      // every tile; the hidden keys' dP is finite, so zeroing the product is
      // the same as zeroing P)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p = exp2_hw(__builtin_fmaf(s[qb][kk][i], scale_log2, -lse2[qb]));
            s[qb][kk][i] = p * (dp[qb][kk][i] - dd[qb]);
          }
      if (need_mask) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (j * BN + 32 * c + 16 * kk + 4 * g + i > row_lim[qb]) s[qb][kk][i] = 0.f;
      }
      // dQ^T[d][row] += K^T[d][key] dS^T[key][row] over these 32 keys
      bf16x8 dsop[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
        dsop[qb] = pack_bf16x8(s[qb][0][0], s[qb][0][1], s[qb][0][2], s[qb][0][3],
                               s[qb][1][0], s[qb][1][1], s[qb][1][2], s[qb][1][3]);
      const int r0 = 32 * c + t_row, r1 = r0 + 16;
      const int sw0 = dual_swz<D>(r0), sw1 = dual_swz<D>(r1);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int ch = 2 * db + t_chunk;
        const i16x4 lo = lds_read_tr16(ks + r0 * D + t_in + (ch ^ sw0) * 8);
        const i16x4 hi4 = lds_read_tr16(ks + r1 * D + t_in + (ch ^ sw1) * 8);
        const bf16x8 ktop = concat_tr(lo, hi4);
        dqt[0][db] = mfma_16x16x32(ktop, dsop[0], dqt[0][db]);
        dqt[1][db] = mfma_16x16x32(ktop, dsop[1], dqt[1][db]);
      }
      if constexpr (D == 128) sched_reads_ahead<NDB, 2, 2, 4>();
    }
  };

  auto step = [&](int j, const bf16* ks, const bf16* vs, bf16* kn, bf16* vn) {
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0 | vmcnt_bits(0));
    stage_barrier();
    if (j + 1 < ntk) load_tile(j + 1, kn, vn);
    if (wave_live && j * BN < wave_kv_end) compute_tile(j, ks, vs);
  };

  load_tile(0, k_st0, v_st0);
  // Settle the register loads above here, outside the loop: a wait the
  // compiler placed at their first use inside the loop would count the
  // untracked tile loads issued in between and stall on the next tile.
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int c = 0; c < NDC; ++c) asm volatile("" ::"v"(qop[qb][c]), "v"(dop[qb][c]));
  asm volatile("" ::"v"(lse2[0]), "v"(lse2[1]), "v"(dd[0]), "v"(dd[1]));
  for (int j = 0;;) {
    step(j, k_st0, v_st0, k_st1, v_st1);
    if (++j >= ntk) break;
    step(j, k_st1, v_st1, k_st0, v_st0);
    if (++j >= ntk) break;
  }

  // ---- dQ = scale * (dQ^T)^T, bf16 ----
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = wrow0 + 16 * qb + l16;
    if (row < T) {
      bf16* op = dq + qbase + (size_t)row * D + 4 * g;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        bf16x4 r;
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = (bf16)(dqt[qb][db][i] * scale);
        *reinterpret_cast<bf16x4*>(op + 16 * db) = r;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dK, dV.  Workgroup = 8 waves over 128 keys; wave pair (p, p + 4) shares the
// 32 keys k0 + 32 p .. + 31 and (waves being dealt to SIMDs in turn) SIMD p.
//   V side, wave p: the keys' K rows as MFMA B operands and the dV
//     accumulators; per streamed tile of 32 query rows S = Q K^T, then
//     P = exp2(scale_log2 S - LSE2) with the mask applied, P (fp32) to LDS for
//     the partner, dV += P^T dO.
//   K side, wave p + 4, one tile behind: the keys' V rows and the dK
//     accumulators; dP = dO V^T, P from LDS, dS = P (dP - D),
//     dK += dS^T Q.
// Both sides run the same instruction shape (row-operand MFMAs, an
// elementwise step, MFMAs on the transpose read), each with half of the
// operand and accumulator registers a wave needs for both gradients, so two
// waves fit per SIMD and one side's elementwise work runs beside the other's
// MFMAs.  The query heads of a group may be divided between workgroups (head
// splits) to fill the chip; their fp32 partial dK, dV are then summed in a
// fixed order by a second kernel.
constexpr int kKvKeysPerPair = 32;
constexpr int kKvBK = 4 * kKvKeysPerPair;    // keys per workgroup
constexpr int kKvBQ = 32;                    // query rows per streamed tile
constexpr int kKvStages = 4;                 // ring: the K side's tile, the V side's, 2 in flight
constexpr int kKvAhead = kKvStages - 2;      // tiles loaded ahead of the V side

// One ring stage: Q tile, dO tile (both [kKvBQ][D] bf16, dual-swizzled
// chunks) and the tile rows' statistics ([kKvBQ] x (LSE * log2 e, D)); after
// the ring, two buffers of P (4 pairs x 16 floats per lane, lane-major).
template <int D>
struct KvStage {
  static constexpr int kTile = kKvBQ * D * 2;
  static constexpr int kStats = kKvBQ * 8;
  static constexpr int kBytes = 2 * kTile + kStats;
  static constexpr int kRing = kKvStages * kBytes;
  static constexpr int kPBuf = 4 * 64 * 16 * 4;                 // one tile's P of all pairs
  static constexpr int kLds = kRing + 2 * kPBuf;
  // 16-byte loads per tile: Q and dO each kKvBQ * D / 8; at D = 128 every
  // wave loads one of each, at D = 64 waves 0-3 load Q and 4-7 dO
  static constexpr int kTileLoads = D == 128 ? 2 : 1;
  static constexpr int kDmaPerStep = kTileLoads + 1;            // + the statistics
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_dkdv_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                     const bf16* __restrict__ v, const bf16* __restrict__ dout,
                     const float* __restrict__ stats, bf16* __restrict__ dk,
                     bf16* __restrict__ dv, float* __restrict__ part, int B, int Hq, int Hkv,
                     int T, int S, float scale_log2, float scale, int nsplit) {
  using L = KvStage<D>;
  constexpr int BQ = kKvBQ;
  constexpr int CPR = D / 8;
  constexpr int NDC = D / 32;
  constexpr int NDB = D / 16;
  static_assert(L::kTileLoads * 512 == 2 * BQ * CPR, "tile loads must split evenly");
  extern __shared__ __attribute__((aligned(16))) char ring[];

  // ---- (key tile, batch, KV head, head split); head splits vary fastest so
  // that the longest causal key tiles (lowest index) start first ----
  const int G = B * Hkv;
  const int split = blockIdx.x % nsplit;
  const int rest = blockIdx.x / nsplit;
  const int grp = rest % G, kt = rest / G;
  const int b = grp / Hkv, hk = grp % Hkv;
  const int hpg = Hq / Hkv, hps = hpg / nsplit;
  const int h_first = hk * hpg + split * hps;
  const int k0 = kt * kKvBK;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g = lane >> 4;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const bool vside = wave_s < 4;             // V side (dV) or K side (dK)
  const int pair = wave_s & 3;
  const int kw0 = k0 + kKvKeysPerPair * pair;   // first key of this pair
  const size_t kvbase = ((size_t)(b * Hkv + hk) * S) * D;

  // query tiles that can see some key of this workgroup
  const int ntq = (T + BQ - 1) / BQ;
  const int qt0 = CAUSAL ? max(0, k0 - (S - T)) / BQ : 0;
  const int nq = max(0, ntq - qt0);
  const int ntiles = nq * hps;               // (head, q tile) pairs, head-major

  // ---- K (V side) or V (K side) rows of this lane's keys kw0 + 16 kb + l16 ----
  bf16x8 kv[2][NDC];
  {
    const bf16* src = vside ? k : v;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const size_t roff = kvbase + (size_t)min(kw0 + 16 * kb + l16, S - 1) * D + 8 * g;
#pragma unroll
      for (int c = 0; c < NDC; ++c) kv[kb][c] = *reinterpret_cast<const bf16x8*>(src + roff + 32 * c);
    }
  }

  // ---- direct-to-LDS loads of one ring stage ----
  // chunk p of the wave's share: row p / CPR, 16-byte chunk p % CPR of Q (and
  // of dO at D = 128; at D = 64 the K side's waves take dO)
  const int lp = 64 * (D == 128 ? wave : (wave & 3)) + lane;
  const int lrow = lp / CPR;
  const uint32_t toff = (uint32_t)(lrow * D + ((lp % CPR) ^ dual_swz<D>(lrow)) * 8) * 2u;
  const uint32_t ring_lds = lds_addr(ring);
  auto head_of = [&](int t) { return h_first + t / nq; };
  auto row0_of = [&](int t) { return (qt0 + t % nq) * BQ; };
  // Tile t into stage t % kKvStages.  Past the last tile the last tile is
  // loaded again (into a stage nobody reads), which keeps the number of loads
  // per step, and so the wait counts below, the same on every step.
  auto issue = [&](int t) {
    const int tc = min(t, ntiles - 1);
    const int h = head_of(tc), row0 = row0_of(tc);
    const size_t hbase = (size_t)(b * Hq + h) * T;
    const uint32_t sb = ring_lds + (uint32_t)((t % kKvStages) * L::kBytes);
    // a full tile's first row goes into the scalar base; rows past T re-read T-1
    const bool full = row0 + BQ <= T;
    const size_t rbase = hbase + (full ? (size_t)row0 : 0);
    const void* qg = uniform_ptr(q + rbase * D);
    const void* og = uniform_ptr(dout + rbase * D);
    const uint32_t off = full ? toff : toff + (uint32_t)(((row0 + lrow < T ? row0 + lrow : T - 1) - lrow) * D) * 2u;
    const uint32_t dst = (uint32_t)(64 * 16 * (D == 128 ? wave_s : (wave_s & 3)));
    if (D == 128) {
      lds_dma16(qg, off, sb + dst);
      lds_dma16(og, off, sb + (uint32_t)L::kTile + dst);
    } else {
      lds_dma16(vside ? qg : og, off, sb + (vside ? 0u : (uint32_t)L::kTile) + dst);
    }
    // statistics of rows row0 + 4 wave .. + 3: 8 dwords from this wave
    if (lane < 8) {
      const int row = min(row0 + 4 * wave + (lane >> 1), T - 1);
      lds_dma4(uniform_ptr(stats + 2 * hbase), (uint32_t)(row * 8 + (lane & 1) * 4),
               sb + (uint32_t)(2 * L::kTile + 32 * wave_s));
    }
  };

  f32x4 acc[2][NDB];                         // dV (V side) or dK (K side) [key][d] per 16-key block
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[kb][db] = f32x4{};

  const int t_row = 4 * g + (l16 >> 2);
  const int t_chunk = (l16 & 3) >> 1;
  const int t_in = 4 * (l16 & 1);
  const int sw_lo = dual_swz<D>(t_row), sw_hi = dual_swz<D>(t_row + 16);
  const int swz_l = dual_swz<D>(l16);
  const bool edge_keys = k0 + kKvBK > S;     // some key of the workgroup is past S
  f32x4* pbuf = reinterpret_cast<f32x4*>(ring + L::kRing);   // [2][4 pairs][4][64 lanes]

  // Tile t on this side: the V side's tile of step t, the K side's of step t + 1.
  auto compute_tile = [&](int t) {
    const char* sp = ring + (t % kKvStages) * L::kBytes;
    const bf16* qs = reinterpret_cast<const bf16*>(sp);
    const bf16* os = reinterpret_cast<const bf16*>(sp + L::kTile);
    const float4* st = reinterpret_cast<const float4*>(sp + 2 * L::kTile);
    const bf16* xs = vside ? qs : os;        // row operands of the first product
    const bf16* ys = vside ? os : qs;        // transpose-read operands of the second
    f32x4* pslot = pbuf + ((size_t)((t & 1) * 4 + pair) * 4) * 64 + lane;
    const int row0 = row0_of(t);
    // r[row][key] = X kv^T: S = Q K^T (V side) or dP = dO V^T (K side),
    // rows 16 qb + 4 g + i, column key 16 kb + l16
    f32x4 r[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) r[qb][0] = r[qb][1] = f32x4{};
    bf16x8 xa[NDC][2];
#pragma unroll
    for (int c = 0; c < NDC; ++c)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
        xa[c][qb] = *reinterpret_cast<const bf16x8*>(xs + (16 * qb + l16) * D + (((4 * c + g) ^ swz_l) * 8));
#pragma unroll
    for (int c = 0; c < NDC; ++c)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) r[qb][kb] = mfma_16x16x32(xa[c][qb], kv[kb][c], r[qb][kb]);
    // keep the reads of three d-chunks ahead of the MFMAs that use them
    sched_reads_ahead<NDC, 2, 4, 3>();
    // A operands of the second product: row = this lane's key, k-slots = rows
    // 4g..4g+3 then 16+4g..16+4g+3
    bf16x8 op[2];
    if (vside) {
      // P = exp2(scale_log2 s - LSE2), zero off the visible pairs
      float pv[2][2][4];                     // [kb][qb][i]
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const float4 ab = st[8 * qb + 2 * g], cd = st[8 * qb + 2 * g + 1];
        const float lse2[4] = {ab.x, ab.z, cd.x, cd.z};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            pv[kb][qb][i] = exp2_hw(__builtin_fmaf(r[qb][kb][i], scale_log2, -lse2[i]));
      }
      if (edge_keys || row0 + BQ > T || (CAUSAL && k0 + kKvBK - 1 > row0 + (S - T))) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int key = kw0 + 16 * kb + l16;
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int row = row0 + 16 * qb + 4 * g + i;
              const bool hide = key >= S || row >= T || (CAUSAL && key > row + (S - T));
              pv[kb][qb][i] = hide ? 0.f : pv[kb][qb][i];
            }
        }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          pslot[(2 * kb + qb) * 64] = f32x4{pv[kb][qb][0], pv[kb][qb][1], pv[kb][qb][2], pv[kb][qb][3]};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        op[kb] = pack_bf16x8(pv[kb][0][0], pv[kb][0][1], pv[kb][0][2], pv[kb][0][3],
                             pv[kb][1][0], pv[kb][1][1], pv[kb][1][2], pv[kb][1][3]);
    } else {
      // dS = P (dP - D), P as the partner wrote it (masked)
      float dsv[2][2][4];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const float4 ab = st[8 * qb + 2 * g], cd = st[8 * qb + 2 * g + 1];
        const float dd[4] = {ab.y, ab.w, cd.y, cd.w};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const f32x4 p4 = pslot[(2 * kb + qb) * 64];
#pragma unroll
          for (int i = 0; i < 4; ++i) dsv[kb][qb][i] = p4[i] * (r[qb][kb][i] - dd[i]);
        }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        op[kb] = pack_bf16x8(dsv[kb][0][0], dsv[kb][0][1], dsv[kb][0][2], dsv[kb][0][3],
                             dsv[kb][1][0], dsv[kb][1][1], dsv[kb][1][2], dsv[kb][1][3]);
    }
    // acc += op Y: dV += P^T dO (V side) or dK += dS^T Q (K side), Y from the
    // transpose read
    bf16x8 yb[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int ch = 2 * db + t_chunk;
      const int off_lo = t_row * D + t_in + (ch ^ sw_lo) * 8;
      const int off_hi = (t_row + 16) * D + t_in + (ch ^ sw_hi) * 8;
      yb[db] = concat_tr(lds_read_tr16(ys + off_lo), lds_read_tr16(ys + off_hi));
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) acc[kb][db] = mfma_16x16x32(op[kb], yb[db], acc[kb][db]);
    sched_reads_ahead<NDB, 2, 2, 3>();
  };

  if (ntiles > 0) {
#pragma unroll
    for (int t = 0; t < kKvAhead; ++t) issue(t);
    // K and V register loads settle here, not at a first use inside the loop
    // (see the dQ kernel)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int c = 0; c < NDC; ++c) asm volatile("" ::"v"(kv[kb][c]));
    // Step t: the V side computes tile t, the K side tile t - 1 (with the P
    // its partner wrote in step t - 1).  This wave's loads of tile t are done
    // once at most the two later tiles' loads are outstanding; the barrier
    // then publishes every wave's part of tile t and the P of tile t - 1, and
    // frees the stage of tile t - 2 for tile t + 3.
    for (int t = 0; t <= ntiles; ++t) {
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0 | vmcnt_bits((kKvAhead - 1) * L::kDmaPerStep));
      stage_barrier();
      issue(t + kKvAhead);
      if (vside ? t < ntiles : t >= 1) compute_tile(vside ? t : t - 1);
    }
    // the re-loads past the last tile land before the workgroup's LDS is released
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0 | vmcnt_bits(0));
  }

  // ---- rows key 16 kb + 4 g + i of the pair's 32, columns 16 db + l16 ----
  const float osc = vside ? 1.f : scale;     // dK = scale dS^T Q
  if (nsplit == 1) {
    bf16* dst = vside ? dv : dk;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kr = kw0 + 16 * kb + 4 * g + i;
        if (kr < S) {
          bf16* rp = dst + kvbase + (size_t)kr * D + l16;
#pragma unroll
          for (int db = 0; db < NDB; ++db) rp[16 * db] = (bf16)(acc[kb][db][i] * osc);
        }
      }
  } else {
    // fp32 partials of this head split: part[split][0: dK, 1: dV][B*Hkv*S*D]
    const size_t nkv = (size_t)B * Hkv * S * D;
    float* pp = part + (size_t)(2 * split + (vside ? 1 : 0)) * nkv + kvbase;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kr = kw0 + 16 * kb + 4 * g + i;
        if (kr < S) {
#pragma unroll
          for (int db = 0; db < NDB; ++db) pp[(size_t)kr * D + 16 * db + l16] = acc[kb][db][i];
        }
      }
  }
}

// dK = scale * sum over head splits, dV = sum, in split order; 4 elements per thread.
__global__ __launch_bounds__(256)
void bwd_kv_reduce_kernel(const float* __restrict__ part, bf16* __restrict__ dk,
                          bf16* __restrict__ dv, long long nkv, int nsplit, float scale) {
  const long long e = ((long long)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= nkv) return;                      // nkv is a multiple of 64
  float4 ak = *reinterpret_cast<const float4*>(part + e);
  float4 av = *reinterpret_cast<const float4*>(part + nkv + e);
  for (int sp = 1; sp < nsplit; ++sp) {
    const float4 bk = *reinterpret_cast<const float4*>(part + (size_t)(2 * sp) * nkv + e);
    const float4 bv = *reinterpret_cast<const float4*>(part + (size_t)(2 * sp + 1) * nkv + e);
    ak.x += bk.x; ak.y += bk.y; ak.z += bk.z; ak.w += bk.w;
    av.x += bv.x; av.y += bv.y; av.z += bv.z; av.w += bv.w;
  }
  bf16x4 rk, rv;
  rk[0] = (bf16)(ak.x * scale); rk[1] = (bf16)(ak.y * scale);
  rk[2] = (bf16)(ak.z * scale); rk[3] = (bf16)(ak.w * scale);
  rv[0] = (bf16)av.x; rv[1] = (bf16)av.y; rv[2] = (bf16)av.z; rv[3] = (bf16)av.w;
  *reinterpret_cast<bf16x4*>(dk + e) = rk;
  *reinterpret_cast<bf16x4*>(dv + e) = rv;
}

template <int D, bool CAUSAL>
hipError_t launch_bwd_d(const void* q, const void* k, const void* v, const void* o,
                        const float* lse, const void* dout, void* dq, void* dk, void* dv,
                        const BwdWorkspace& ws, int B, int Hq, int Hkv, int T, int S, float scale,
                        hipStream_t stream) {
  const float scale_log2 = scale * kLog2e;
  const long long gq = (long long)((T + 127) / 128) * B * Hq;
  launch_kernel(bwd_dq_kernel<D, CAUSAL>, dim3((unsigned)gq), dim3(256), 0, stream,
                     static_cast<const bf16*>(q), static_cast<const bf16*>(k),
                     static_cast<const bf16*>(v), static_cast<const bf16*>(dout),
                     static_cast<const bf16*>(o), lse, ws.stats,
                     static_cast<bf16*>(dq), B, Hq, Hkv, T, S, scale_log2, scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the ring is above the 64 KB of static LDS at d = 128
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_dkdv_kernel<D, CAUSAL>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, KvStage<D>::kLds);
  if (e != hipSuccess) return e;
  const int nsplit = bwd_kv_splits(B, Hq, Hkv, S);
  const long long gkv = (long long)((S + kKvBK - 1) / kKvBK) * B * Hkv * nsplit;
  launch_kernel(bwd_dkdv_kernel<D, CAUSAL>, dim3((unsigned)gkv), dim3(512),
                     KvStage<D>::kLds, stream,
                     static_cast<const bf16*>(q), static_cast<const bf16*>(k),
                     static_cast<const bf16*>(v), static_cast<const bf16*>(dout), ws.stats,
                     static_cast<bf16*>(dk), static_cast<bf16*>(dv), ws.kv_part, B, Hq, Hkv, T, S,
                     scale_log2, scale, nsplit);
  e = hipGetLastError();
  if (e != hipSuccess || nsplit == 1) return e;
  const long long nkv = (long long)B * Hkv * S * D;
  launch_kernel(bwd_kv_reduce_kernel, dim3((unsigned)((nkv / 4 + 255) / 256)), dim3(256), 0,
                     stream, ws.kv_part, static_cast<bf16*>(dk), static_cast<bf16*>(dv), nkv, nsplit,
                     scale);
  return hipGetLastError();
}

}  // namespace

int bwd_kv_splits(int B, int Hq, int Hkv, int S) {
  const long long base = (long long)((S + kKvBK - 1) / kKvBK) * B * Hkv;
  const int hpg = Hq / Hkv;
  int n = 1;
  while (base * n < kBwdTargetBlocks && n < hpg) {
    int m = n + 1;
    while (hpg % m != 0) ++m;
    n = m;
  }
  return n;
}

size_t bwd_kv_part_bytes(int B, int Hq, int Hkv, int S, int d) {
  const int n = bwd_kv_splits(B, Hq, Hkv, S);
  return n == 1 ? 0 : (size_t)2 * n * B * Hkv * S * d * 4;
}

hipError_t launch_backward_bf16(const void* q, const void* k, const void* v, const void* o,
                                const float* lse, const void* dout, void* dq, void* dk, void* dv,
                                const BwdWorkspace& ws, int B, int Hq, int Hkv, int T, int S,
                                int d, float scale, bool causal, hipStream_t stream) {
  if (d == 128)
    return causal ? launch_bwd_d<128, true>(q, k, v, o, lse, dout, dq, dk, dv, ws, B, Hq, Hkv, T, S, scale, stream)
                  : launch_bwd_d<128, false>(q, k, v, o, lse, dout, dq, dk, dv, ws, B, Hq, Hkv, T, S, scale, stream);
  return causal ? launch_bwd_d<64, true>(q, k, v, o, lse, dout, dq, dk, dv, ws, B, Hq, Hkv, T, S, scale, stream)
                : launch_bwd_d<64, false>(q, k, v, o, lse, dout, dq, dk, dv, ws, B, Hq, Hkv, T, S, scale, stream);
}

}  // namespace attn
