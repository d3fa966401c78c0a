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
// Three kernels, no atomics, so results are bit-reproducible:
//   bwd_prep_kernel:  D = rowsum(dO * O) per query row (fp32, workspace).
//   bwd_dq_kernel:    one workgroup per 128 query rows of one (batch, head),
//     shaped like the forward kernel: Q and dO stay in registers as MFMA B
//     operands, K and V tiles stream through two LDS stages by the
//     direct-to-LDS load; per tile S^T = K Q^T, dP^T = V dO^T, P, dS, and
//     dQ^T += K^T dS^T with K^T from the LDS transpose read.
//   bwd_dkdv_kernel:  one workgroup per 64 keys of one (batch, KV head); each
//     wave keeps its 16 keys' K and V in registers as MFMA B operands and
//     walks every query tile (32 rows) of every query head of the group that
//     can see them, Q and dO tiles streaming through LDS; per tile S = Q K^T,
//     dP = dO V^T, P, dS, then dV += P^T dO and dK += dS^T Q with dO and Q
//     from the transpose read.  Summing the group's heads in registers keeps
//     the grouped-query reduction exact in order.
// Tiles read both as MFMA row operands and through the transpose read use the
// dual swizzle of lds_stage.hpp, bank-conflict free for both.
#include "cdna4.hpp"
#include "kernels.hpp"
#include "lds_stage.hpp"

namespace attn {
namespace {

// ---------------------------------------------------------------------------
// D = rowsum(dO * O): 16 lanes per row, D/16 elements per lane.
template <int D>
__global__ __launch_bounds__(256)
void bwd_prep_kernel(const bf16* __restrict__ o, const bf16* __restrict__ dout,
                     float* __restrict__ dsum, long long rows) {
  constexpr int PER = D / 16;
  const long long row = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int j = threadIdx.x & 15;
  if (row >= rows) return;                   // whole 16-lane groups leave together
  const bf16* op = o + row * D + j * PER;
  const bf16* dp = dout + row * D + j * PER;
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) acc = __builtin_fmaf((float)op[e], (float)dp[e], acc);
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
  if (j == 0) dsum[row] = acc;
}

// ---------------------------------------------------------------------------
// dQ.  Workgroup = 4 waves x 32 query rows (two 16-row blocks per wave).
constexpr int kDqBN = 64;                    // keys per K/V tile

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_dq_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                   const bf16* __restrict__ v, const bf16* __restrict__ dout,
                   const float* __restrict__ lse, const float* __restrict__ dsum,
                   bf16* __restrict__ dq, int B, int Hq, int Hkv, int T, int S,
                   float scale_log2, float scale) {
  constexpr int BN = kDqBN;
  constexpr int kBM = 128;
  constexpr int CPR = D / 8;
  constexpr int NKB = BN / 16;
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
#pragma unroll
    for (int r = 0; r < CPW; ++r) {
      uint32_t add;
      if (full) {
        add = (uint32_t)(j * BN * D) * 2u;
      } else {
        const int key = min(j * BN + lrow[r], S - 1);
        add = (uint32_t)((key - lrow[r]) * D) * 2u;
      }
      lds_dma16(kg, toff[r] + add, kl + 1024u * r);
      lds_dma16(vg, toff[r] + add, vl + 1024u * r);
    }
  };

  // ---- Q and dO rows (B operands), LSE (log2 units) and D of this lane's rows ----
  bf16x8 qop[2][NDC], dop[2][NDC];
  int row_lim[2];
  float lse2[2], dd[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = wrow0 + 16 * qb + l16;
    if (row < T) {
      const bf16* qp = q + qbase + (size_t)row * D + 8 * g;
      const bf16* dp = dout + qbase + (size_t)row * D + 8 * g;
#pragma unroll
      for (int c = 0; c < NDC; ++c) {
        qop[qb][c] = *reinterpret_cast<const bf16x8*>(qp + 32 * c);
        dop[qb][c] = *reinterpret_cast<const bf16x8*>(dp + 32 * c);
      }
      lse2[qb] = lse[(size_t)(b * Hq + h) * T + row] * kLog2e;
      dd[qb] = dsum[(size_t)(b * Hq + h) * T + row];
    } else {
#pragma unroll
      for (int c = 0; c < NDC; ++c) qop[qb][c] = dop[qb][c] = bf16x8{};
      lse2[qb] = 0.f;
      dd[qb] = 0.f;
    }
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
    // S^T[key][row] = K Q^T and dP^T[key][row] = V dO^T
    f32x4 s[2][NKB], dp[2][NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[0][kb] = s[1][kb] = dp[0][kb] = dp[1][kb] = f32x4{};
#pragma unroll
    for (int c = 0; c < NDC; ++c) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int off = (16 * kb + l16) * D + (((4 * c + g) ^ swz_l) * 8);
        const bf16x8 kop = *reinterpret_cast<const bf16x8*>(ks + off);
        const bf16x8 vop = *reinterpret_cast<const bf16x8*>(vs + off);
        s[0][kb] = mfma_16x16x32(kop, qop[0][c], s[0][kb]);
        s[1][kb] = mfma_16x16x32(kop, qop[1][c], s[1][kb]);
        dp[0][kb] = mfma_16x16x32(vop, dop[0][c], dp[0][kb]);
        dp[1][kb] = mfma_16x16x32(vop, dop[1][c], dp[1][kb]);
      }
    }
    // dS^T = P^T * (dP^T - D), P^T = exp2(scale_log2 s - LSE2) on visible keys
    const bool need_mask = ((j + 1) * BN > S) || (CAUSAL && (j + 1) * BN - 1 > wrow0 + (S - T));
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float p = exp2_hw(__builtin_fmaf(s[qb][kb][i], scale_log2, -lse2[qb]));
          if (need_mask && j * BN + 16 * kb + 4 * g + i > row_lim[qb]) p = 0.f;
          s[qb][kb][i] = p * (dp[qb][kb][i] - dd[qb]);
        }
    // dQ^T[d][row] += K^T[d][key] dS^T[key][row], 32 keys at a time
#pragma unroll
    for (int c = 0; c < NPC; ++c) {
      bf16x8 dsop[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
        dsop[qb] = pack_bf16x8(s[qb][2 * c][0], s[qb][2 * c][1], s[qb][2 * c][2], s[qb][2 * c][3],
                               s[qb][2 * c + 1][0], s[qb][2 * c + 1][1], s[qb][2 * c + 1][2],
                               s[qb][2 * c + 1][3]);
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
    }
  };

  auto step = [&](int j, const bf16* ks, const bf16* vs, bf16* kn, bf16* vn) {
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0 | vmcnt_bits(0));
    stage_barrier();
    if (j + 1 < ntk) load_tile(j + 1, kn, vn);
    if (wave_live && j * BN < wave_kv_end) compute_tile(j, ks, vs);
  };

  load_tile(0, k_st0, v_st0);
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
// dK, dV.  Workgroup = 4 waves x 16 keys; query tiles of 32 rows.
constexpr int kKvBK = 64;                    // keys per workgroup
constexpr int kKvBQ = 32;                    // query rows per streamed tile

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_dkdv_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                     const bf16* __restrict__ v, const bf16* __restrict__ dout,
                     const float* __restrict__ lse, const float* __restrict__ dsum,
                     bf16* __restrict__ dk, bf16* __restrict__ dv, int B, int Hq, int Hkv,
                     int T, int S, float scale_log2, float scale) {
  constexpr int BQ = kKvBQ;
  constexpr int CPR = D / 8;
  constexpr int NDC = D / 32;
  constexpr int NDB = D / 16;
  constexpr int CPW = BQ * CPR / 256;        // loads per thread per Q (or dO) tile
  static_assert(CPW * 256 == BQ * CPR, "tile must split evenly");

  __shared__ __attribute__((aligned(16))) bf16 q_st0[BQ * D];
  __shared__ __attribute__((aligned(16))) bf16 q_st1[BQ * D];
  __shared__ __attribute__((aligned(16))) bf16 o_st0[BQ * D];   // dO
  __shared__ __attribute__((aligned(16))) bf16 o_st1[BQ * D];

  // ---- (key tile, batch, KV head); key tile 0 sees the most rows: first ----
  const int G = B * Hkv;
  const int kt = blockIdx.x / G, grp = blockIdx.x % G;
  const int b = grp / Hkv, hk = grp % Hkv;
  const int hpg = Hq / Hkv;
  const int k0 = kt * kKvBK;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g = lane >> 4;
  const int key = k0 + 16 * wave + l16;     // this lane's key (column of S)
  const bool key_ok = key < S;
  const size_t kvbase = ((size_t)(b * Hkv + hk) * S) * D;

  // query tiles that can see some key of this workgroup
  const int ntq = (T + BQ - 1) / BQ;
  const int qt0 = CAUSAL ? max(0, k0 - (S - T)) / BQ : 0;
  const int nq = max(0, ntq - qt0);
  const int ntiles = nq * hpg;               // (head, q tile) pairs, head-major

  // ---- this lane's K and V row as B operands (column key, k-group g) ----
  bf16x8 kop[NDC], vop[NDC];
  {
    const size_t roff = kvbase + (size_t)min(key, S - 1) * D + 8 * g;
#pragma unroll
    for (int c = 0; c < NDC; ++c) {
      kop[c] = *reinterpret_cast<const bf16x8*>(k + roff + 32 * c);
      vop[c] = *reinterpret_cast<const bf16x8*>(v + roff + 32 * c);
    }
  }

  // ---- direct-to-LDS loads of Q and dO tiles ----
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
  auto head_of = [&](int t) { return hk * hpg + t / nq; };
  auto row0_of = [&](int t) { return (qt0 + t % nq) * BQ; };
  auto load_tile = [&](int t, bf16* qs, bf16* os) {
    const int h = head_of(t), row0 = row0_of(t);
    const bf16* qg = q + ((size_t)(b * Hq + h) * T) * D;
    const bf16* og = dout + ((size_t)(b * Hq + h) * T) * D;
    const uint32_t ql = lds_addr(qs) + (uint32_t)(wave_s * CPW) * 1024u;
    const uint32_t ol = lds_addr(os) + (uint32_t)(wave_s * CPW) * 1024u;
    const bool full = row0 + BQ <= T;
#pragma unroll
    for (int r = 0; r < CPW; ++r) {
      const int rr = full ? row0 + lrow[r] : min(row0 + lrow[r], T - 1);   // rows past T re-read T-1
      const uint32_t add = (uint32_t)((rr - lrow[r]) * D) * 2u;
      lds_dma16(qg, toff[r] + add, ql + 1024u * r);
      lds_dma16(og, toff[r] + add, ol + 1024u * r);
    }
  };
  // LSE (log2 units) and D of rows row0 + 16 qb + 4 g + i (rows past T: 0)
  auto load_stats = [&](int t, f32x4 (&ls)[2], f32x4 (&ds)[2]) {
    const size_t base = (size_t)(b * Hq + head_of(t)) * T;
    const int row0 = row0_of(t);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = min(row0 + 16 * qb + 4 * g + i, T - 1);
        ls[qb][i] = lse[base + row] * kLog2e;
        ds[qb][i] = dsum[base + row];
      }
  };

  f32x4 dka[NDB], dva[NDB];                  // dK[key][d], dV[key][d] (rows key, cols d)
#pragma unroll
  for (int db = 0; db < NDB; ++db) dka[db] = dva[db] = f32x4{};

  const int t_row = 4 * g + (l16 >> 2);
  const int t_chunk = (l16 & 3) >> 1;
  const int t_in = 4 * (l16 & 1);
  const int sw_lo = dual_swz<D>(t_row), sw_hi = dual_swz<D>(t_row + 16);
  const int swz_l = dual_swz<D>(l16);

  auto compute_tile = [&](int t, const bf16* qs, const bf16* os, const f32x4 (&ls)[2],
                          const f32x4 (&dsv)[2]) {
    const int row0 = row0_of(t);
    // S[row][key] = Q K^T and dP[row][key] = dO V^T (rows 16 qb + 4 g + i, column key)
    f32x4 s[2], dp[2];
    s[0] = s[1] = dp[0] = dp[1] = f32x4{};
#pragma unroll
    for (int c = 0; c < NDC; ++c) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int off = (16 * qb + l16) * D + (((4 * c + g) ^ swz_l) * 8);
        const bf16x8 qa = *reinterpret_cast<const bf16x8*>(qs + off);
        const bf16x8 oa = *reinterpret_cast<const bf16x8*>(os + off);
        s[qb] = mfma_16x16x32(qa, kop[c], s[qb]);
        dp[qb] = mfma_16x16x32(oa, vop[c], dp[qb]);
      }
    }
    // P and dS on visible (row, key) pairs
    const bool need_mask = !key_ok || row0 + BQ > T || (CAUSAL && k0 + kKvBK - 1 > row0 + (S - T));
    float pv[2][4], dsw[2][4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = row0 + 16 * qb + 4 * g + i;
        float p = exp2_hw(__builtin_fmaf(s[qb][i], scale_log2, -ls[qb][i]));
        if (need_mask && (!key_ok || row >= T || (CAUSAL && key > row + (S - T)))) p = 0.f;
        pv[qb][i] = p;
        dsw[qb][i] = p * (dp[qb][i] - dsv[qb][i]);
      }
    // A operands: row = this lane's key, k-slots = rows 4g..4g+3 then 16+4g..16+4g+3
    const bf16x8 pta = pack_bf16x8(pv[0][0], pv[0][1], pv[0][2], pv[0][3],
                                   pv[1][0], pv[1][1], pv[1][2], pv[1][3]);
    const bf16x8 dsta = pack_bf16x8(dsw[0][0], dsw[0][1], dsw[0][2], dsw[0][3],
                                    dsw[1][0], dsw[1][1], dsw[1][2], dsw[1][3]);
    // dV += P^T dO and dK += dS^T Q, the B operands from the transpose read
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int ch = 2 * db + t_chunk;
      const int off_lo = t_row * D + t_in + (ch ^ sw_lo) * 8;
      const int off_hi = (t_row + 16) * D + t_in + (ch ^ sw_hi) * 8;
      const bf16x8 ob = concat_tr(lds_read_tr16(os + off_lo), lds_read_tr16(os + off_hi));
      const bf16x8 qbop = concat_tr(lds_read_tr16(qs + off_lo), lds_read_tr16(qs + off_hi));
      dva[db] = mfma_16x16x32(pta, ob, dva[db]);
      dka[db] = mfma_16x16x32(dsta, qbop, dka[db]);
    }
  };

  if (ntiles > 0) {
    f32x4 lsa[2], dsa[2], lsb[2], dsb[2];
    load_tile(0, q_st0, o_st0);
    load_stats(0, lsa, dsa);
    auto step = [&](int t, const bf16* qs, const bf16* os, bf16* qn, bf16* on, const f32x4 (&ls)[2],
                    const f32x4 (&dsv)[2], f32x4 (&lsn)[2], f32x4 (&dsn)[2]) {
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0 | vmcnt_bits(0));
      stage_barrier();
      if (t + 1 < ntiles) {
        load_tile(t + 1, qn, on);
        load_stats(t + 1, lsn, dsn);
      }
      compute_tile(t, qs, os, ls, dsv);
    };
    for (int t = 0;;) {
      step(t, q_st0, o_st0, q_st1, o_st1, lsa, dsa, lsb, dsb);
      if (++t >= ntiles) break;
      step(t, q_st1, o_st1, q_st0, o_st0, lsb, dsb, lsa, dsa);
      if (++t >= ntiles) break;
    }
  }

  // ---- dK = scale * dK, dV: rows key 4 g + i of the wave's 16, columns d ----
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int kr = k0 + 16 * wave + 4 * g + i;
    if (kr < S) {
      bf16* kp = dk + kvbase + (size_t)kr * D + l16;
      bf16* vp = dv + kvbase + (size_t)kr * D + l16;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        kp[16 * db] = (bf16)(dka[db][i] * scale);
        vp[16 * db] = (bf16)dva[db][i];
      }
    }
  }
}

template <int D, bool CAUSAL>
hipError_t launch_bwd_d(const void* q, const void* k, const void* v, const void* o,
                        const float* lse, const void* dout, void* dq, void* dk, void* dv,
                        float* dsum, int B, int Hq, int Hkv, int T, int S, float scale,
                        hipStream_t stream) {
  const long long rows = (long long)B * Hq * T;
  hipLaunchKernelGGL((bwd_prep_kernel<D>), dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, stream,
                     static_cast<const bf16*>(o), static_cast<const bf16*>(dout), dsum, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const float scale_log2 = scale * kLog2e;
  const long long gq = (long long)((T + 127) / 128) * B * Hq;
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)gq), dim3(256), 0, stream,
                     static_cast<const bf16*>(q), static_cast<const bf16*>(k),
                     static_cast<const bf16*>(v), static_cast<const bf16*>(dout), lse, dsum,
                     static_cast<bf16*>(dq), B, Hq, Hkv, T, S, scale_log2, scale);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long gkv = (long long)((S + kKvBK - 1) / kKvBK) * B * Hkv;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)gkv), dim3(256), 0, stream,
                     static_cast<const bf16*>(q), static_cast<const bf16*>(k),
                     static_cast<const bf16*>(v), static_cast<const bf16*>(dout), lse, dsum,
                     static_cast<bf16*>(dk), static_cast<bf16*>(dv), B, Hq, Hkv, T, S, scale_log2,
                     scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_backward_bf16(const void* q, const void* k, const void* v, const void* o,
                                const float* lse, const void* dout, void* dq, void* dk, void* dv,
                                float* dsum, int B, int Hq, int Hkv, int T, int S, int d,
                                float scale, bool causal, hipStream_t stream) {
  if (d == 128)
    return causal ? launch_bwd_d<128, true>(q, k, v, o, lse, dout, dq, dk, dv, dsum, B, Hq, Hkv, T, S, scale, stream)
                  : launch_bwd_d<128, false>(q, k, v, o, lse, dout, dq, dk, dv, dsum, B, Hq, Hkv, T, S, scale, stream);
  return causal ? launch_bwd_d<64, true>(q, k, v, o, lse, dout, dq, dk, dv, dsum, B, Hq, Hkv, T, S, scale, stream)
                : launch_bwd_d<64, false>(q, k, v, o, lse, dout, dq, dk, dv, dsum, B, Hq, Hkv, T, S, scale, stream);
}

}  // namespace attn
