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
// kernel).  The reference maximum is lazy: it moves only when a tile's
// maximum passes it by more than kLazyTau, so every exponent is at most
// kLazyTau (2^8 stays far inside bf16 and fp32 range).
//
// gfx950 mapping:
//   * one workgroup = 4 waves = 128 query rows of one (batch, query head);
//     each wave owns 32 rows as two 16-row blocks and keeps their Q in
//     registers as MFMA B-operands for the whole kernel (grids too small to
//     fill the chip take one 16-row block per wave, 64 rows a workgroup);
//   * K and V tiles of BN keys go HBM -> LDS by the gfx950 direct-to-LDS load
//     (no register staging), into two stages held in separate LDS objects:
//     the load of tile j+1 runs while tile j is computed, one barrier per
//     tile, with the vmcnt waits placed by hand;
//   * S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_16x16x32_bf16: a lane holds
//     4 keys of one query row per 16-key block, and the exponentiated scores
//     of two adjacent blocks are exactly the P operand of one P.V MFMA; V^T
//     comes from the row-major V tile through the LDS transpose read; every K
//     and V operand read from LDS feeds the MFMAs of both row blocks, and the
//     K reads run four operands ahead of their MFMAs;
//   * K and V tiles are stored unpadded with their 16-byte chunks XOR-swizzled
//     per row so that both operand read patterns are bank-conflict free;
//   * causal: K/V tiles past the workgroup's last visible key are never
//     loaded, a wave skips tiles it cannot see, and only tiles crossing the
//     diagonal (or the ragged end) pay for the mask;
//   * heavy causal tiles are dispatched first, and when the number of
//     (batch, KV head) groups is a multiple of 8 every group stays on one XCD
//     so its K/V is re-read from that XCD's L2; a grid resident all at once
//     pairs long and short query tiles on each CU instead.
#include "cdna4.hpp"
#include "kernels.hpp"
#include "lds_stage.hpp"

#ifndef PREFILL_SMALL_GRID
#define PREFILL_SMALL_GRID 256    // workgroups at two row blocks per wave
#endif
#ifndef PREFILL_D128_WAVES
#define PREFILL_D128_WAVES 4
#define PREFILL_D128_BN 64
#define PREFILL_D128_STAGES 2
#define PREFILL_D64_WAVES 4
#define PREFILL_D64_BN_QB1 128
#define PREFILL_D64_BN_QB2 64
#define PREFILL_D64_STAGES 2
#endif

namespace attn {
namespace {

// Tile configuration per head dimension and row blocks per wave (QB): waves
// per workgroup (16 QB query rows each), keys per K/V tile, and LDS stages in
// the load ring (the load of tile j + STAGES - 1 is in flight while tile j is
// computed).  At d = 64 one row block per wave serves the small grids, whose
// time is the longest workgroup's path, and takes 128-key tiles (half the
// steps on that path); two row blocks per wave serve full grids with 64-key
// tiles, which measured 5-8 % faster there than 128 (prefill_2, same-box A/B).
template <int D, int QB> struct PrefillCfg;
template <int QB> struct PrefillCfg<128, QB> {
  static constexpr int WAVES = PREFILL_D128_WAVES, BN = PREFILL_D128_BN, STAGES = PREFILL_D128_STAGES;
};
template <int QB> struct PrefillCfg<64, QB> {
  static constexpr int WAVES = PREFILL_D64_WAVES, STAGES = PREFILL_D64_STAGES;
  static constexpr int BN = QB == 1 ? PREFILL_D64_BN_QB1 : PREFILL_D64_BN_QB2;
};

// Chunk swizzles (16-byte chunks within a row of D bf16).
// K is read as 16 rows x one chunk per 16 lanes: spread the 16 rows over all
// banks.  V is read by the transpose read as 8 rows x 32 bytes per half-wave:
// spread those 8 rows.  A row of D=128 spans the 64 banks once, a row of D=64
// half of them, hence the different row bits.
template <int D>
__device__ __forceinline__ int k_swz(int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); }
template <int D>
__device__ __forceinline__ int v_swz(int row) { return D == 128 ? 2 * (row & 7) : 2 * ((row >> 1) & 3); }

// MI355X: 8 XCDs of 32 CUs; the dispatcher deals workgroups to XCDs in turn
// and, inside an XCD, to its CUs in turn.
constexpr int kXcdCount = 8;
constexpr int kCusPerXcd = 32;

// Chunked prefill: the index of the slot-th longest of the n sequences
// (lengths clamped to [0, lmax], ties by index), found by every thread of the
// workgroup.  The keys ~len of the first kSelCache sequences are staged in LDS
// by one coalesced pass.  Up to NT sequences, thread c counts the keys below
// its own (a rank, ties by index) and the thread whose rank is `slot` names
// itself.  Beyond that, radix selection on the key in four 8-bit digits, from
// the top: a histogram of the digit over the sequences that match the digits
// fixed so far locates the digit of the wanted rank and the rank left within
// it; the sequences with the selected length are then counted in index order
// to pick the remaining rank.  Each pass reads the n keys once, so the cost
// grows linearly with n.
constexpr int kSelCache = 1024;

template <int NT>
__device__ __forceinline__ int select_by_length(const int32_t* __restrict__ lens, int n, int lmax,
                                                int slot) {
  static_assert(NT % 64 == 0 && NT >= 256, "one wave scans 256 bins; a lane covers NT/64 counts");
  __shared__ unsigned cache[kSelCache];
  __shared__ unsigned hist[256];
  __shared__ unsigned sh_prefix, sh_rank;
  __shared__ unsigned sh_cnt[NT];
  const int tid = threadIdx.x, lane = tid & 63;
  auto load_key = [&](int c) { return ~(unsigned)min(max(lens[c], 0), lmax); };
  for (int c = tid; c < min(n, kSelCache); c += NT) cache[c] = load_key(c);
  __syncthreads();
  auto key = [&](int c) { return c < kSelCache ? cache[c] : load_key(c); };
  if (n <= NT) {
    if (tid < n) {
      const unsigned u = cache[tid];
      int rk = 0;
      for (int t = 0; t < n; ++t) {
        const unsigned x = cache[t];
        rk += (x < u) || (x == u && t < tid);
      }
      if (rk == slot) sh_prefix = (unsigned)tid;
    }
    __syncthreads();
    return (int)sh_prefix;
  }
  // Wave 0: of the counts v[0 .. per*64) (per consecutive ones a lane), the
  // position p where the running sum first exceeds `rank`, and the sum before it.
  auto find = [&](const unsigned* v, int per, unsigned rank, unsigned& before) {
    unsigned own = 0;
    for (int e = 0; e < per; ++e) own += v[per * lane + e];
    unsigned incl = own;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const unsigned y = __shfl_up(incl, m);
      if (lane >= m) incl += y;
    }
    const unsigned long long hit = __builtin_amdgcn_ballot_w64(incl > rank);
    const int L = hit ? __builtin_ctzll(hit) : 63;
    unsigned cum = __shfl(incl - own, L);
    int p = per * L;
    for (int e = 0; e < per - 1; ++e, ++p) {
      const unsigned x = v[p];
      if (cum + x > rank) break;
      cum += x;
    }
    before = cum;
    return p;
  };
  unsigned prefix = 0, mask = 0, rank = (unsigned)slot;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += NT) hist[i] = 0;
    __syncthreads();
    for (int c = tid; c < n; c += NT) {
      const unsigned u = key(c);
      if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      unsigned cum;
      const int d = find(hist, 4, rank, cum);
      if (lane == 0) {
        sh_prefix = prefix | ((unsigned)d << shift);
        sh_rank = rank - cum;
      }
    }
    __syncthreads();
    prefix = sh_prefix;
    rank = sh_rank;
    mask |= 255u << shift;
    __syncthreads();
  }
  // the rank-th (in index order) sequence whose key equals prefix
  const int chunk = (n + NT - 1) / NT, c0 = tid * chunk, c1 = min(n, c0 + chunk);
  unsigned cnt = 0;
  for (int c = c0; c < c1; ++c) cnt += key(c) == prefix;
  sh_cnt[tid] = cnt;
  __syncthreads();
  if (tid < 64) {
    unsigned before;
    const int t = find(sh_cnt, NT / 64, rank, before);
    if (lane == 0) {
      int c = t * chunk;
      for (unsigned seen = before;; ++c)
        if (key(c) == prefix && seen++ == rank) break;
      sh_prefix = (unsigned)c;
    }
  }
  __syncthreads();
  return (int)sh_prefix;
}

// Slack of the running maximum (log2 units): P = exp2(s - m) may reach
// 2^kLazyTau, far inside bf16 and fp32 range.
constexpr float kLazyTau = 8.f;

template <int D, bool CAUSAL, int QB, bool PAGED>
__global__ __launch_bounds__((64 * PrefillCfg<D, QB>::WAVES)) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_bf16_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                         const bf16* __restrict__ v, bf16* __restrict__ o,
                         float* __restrict__ lse, int B, int Hq, int Hkv, int T, int S,
                         float scale_log2, int window, const PagedKv pkv, int snake) {
  constexpr int BN = PrefillCfg<D, QB>::BN;
  constexpr int NST = PrefillCfg<D, QB>::STAGES;
  constexpr int kThreads = 64 * PrefillCfg<D, QB>::WAVES;
  constexpr int kWR = 16 * QB;               // query rows per wave (QB blocks of 16)
  constexpr int kBM = kWR * PrefillCfg<D, QB>::WAVES;  // query rows per workgroup
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int NKB = BN / 16;               // 16-key blocks of S^T
  constexpr int NDC = D / 32;                // k-chunks of the S^T MFMA
  constexpr int NDB = D / 16;                // 16-row blocks of O^T
  constexpr int NPC = BN / 32;               // 32-key chunks of the P.V MFMA
  constexpr int CPW = BN * CPR / kThreads;   // direct-to-LDS loads per thread per tile (K, and V)
  static_assert(CPW * kThreads == BN * CPR, "tile must split evenly");

  // the stages, each K and V in its own object so that the compiler can tell
  // the stage being read from the ones being loaded (a third stage exists
  // only when NST == 3)
  __shared__ __attribute__((aligned(16))) bf16 k_st0[BN * D];
  __shared__ __attribute__((aligned(16))) bf16 v_st0[BN * D];
  __shared__ __attribute__((aligned(16))) bf16 k_st1[BN * D];
  __shared__ __attribute__((aligned(16))) bf16 v_st1[BN * D];
  __shared__ __attribute__((aligned(16))) bf16 k_st2[NST == 3 ? BN * D : 8];
  __shared__ __attribute__((aligned(16))) bf16 v_st2[NST == 3 ? BN * D : 8];

  // ---- which (q tile, batch, head) this workgroup computes ----
  const int ntq = (T + kBM - 1) / kBM;
  const int hpg = Hq / Hkv;                  // query heads per KV head
  const int G = B * Hkv;                     // (batch, KV head) groups
  const int pid = blockIdx.x;
  int hgi, grp, rank;
  if (PAGED) {
    // Chunked prefill: a sequence's work grows with its cached length, so
    // sequences are dispatched longest first: workgroups [slot W, (slot+1) W)
    // take the slot-th longest (ties by index).  Every workgroup selects that
    // sequence itself from the same lengths, so all agree on the order.
    // The first two rounds of the dispatch put workgroups pid and pid + 256
    // on one CU (the first 512 ids fill two slots of each of the 256 CUs):
    // ids 256..511 take the lightest items, in reverse, so that each CU
    // starts with one long and one short query tile; later ids take the
    // middle of the order, longest first.
    const int G_all = (int)gridDim.x, nc = kXcdCount * kCusPerXcd;
    int item = pid;
    if (pid >= nc && pid < 2 * nc) item = G_all - 1 - (pid - nc);
    else if (pid >= 2 * nc) item = pid - nc;
    const int W = ntq * Hq, slot = item / W, w = item - slot * W;
    hgi = w % hpg;
    const int r = w / hpg;
    rank = r / Hkv;
    __shared__ int sel;
    const int chosen = select_by_length<kThreads>(pkv.seq_lens, B, pkv.max_blocks * 16, slot);
    if (threadIdx.x == 0) sel = chosen;
    __syncthreads();
    grp = sel * Hkv + r % Hkv;
  } else if ((G & 7) == 0) {
    // XCD pid%8 walks its own eighth of the groups: [tile rank][group][head].
    int s = pid >> 3;
    const int gpx = G >> 3;
    if (snake) {
      // The dispatcher deals an XCD's workgroups to its 32 CUs in turn, so
      // workgroups s, s+32, s+64, ... share a CU.  When the whole grid is
      // resident at once, taking every other run of 32 in reverse pairs the
      // heaviest causal tiles with the lightest on each CU.
      const int run = s >> 5, pos = s & 31;
      s = (run << 5) + ((run & 1) ? 31 - pos : pos);
    }
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
  // T is the row stride of q, o and lse.  On a paged cache sequence b has
  // its own lengths: S cached keys, of which the last T_n are this call's
  // queries (rows 0 .. T_n - 1 of its T); rows past T_n are not computed.
  const int Tst = T;
  if (PAGED) {
    S = min(max(pkv.seq_lens[b], 0), pkv.max_blocks * 16);
    T = min(max(pkv.q_lens[b], 0), min(Tst, S));
    if (q0 >= T) return;                             // whole workgroup: no barrier passed yet
  }

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g = lane >> 4;

  const size_t qbase = ((size_t)(b * Hq + h) * Tst) * D;
  const size_t kvbase = PAGED ? 0 : ((size_t)(b * Hkv + hk) * S) * D;

  // ---- keys this workgroup / wave can see ----
  const int wrow0 = q0 + kWR * wave;                 // first row of this wave
  const bool wave_live = wrow0 < T;
  int wg_kv_end = S, wave_kv_end = S;                // exclusive
  if (CAUSAL) {
    wg_kv_end = min(S, min(q0 + kBM, T) + (S - T));
    wave_kv_end = min(S, min(wrow0 + kWR, T) + (S - T));
  }
  const int ntk = (wg_kv_end + BN - 1) / BN;
  // Causal sliding window: row i also loses keys <= i + (S - T) - window.
  // Tiles wholly left of the first row's window are never loaded (j0), and a
  // wave skips those left of its own first row's window.
  const bool windowed = CAUSAL && window > 0;
  const int wave_kv_lo = windowed ? max(0, wrow0 + (S - T) - window + 1) : 0;
  const int j0 = windowed ? max(0, q0 + (S - T) - window + 1) / BN : 0;

  // ---- direct-to-LDS tile load ----
  // Instruction r of wave w fills LDS chunks [64 (w CPW + r), +64): lane l
  // writes chunk p = 64 (w CPW + r) + l, i.e. row p / CPR, physical chunk
  // p % CPR, which holds logical chunk (p % CPR) ^ swz(row).  The source is
  // the wave-uniform base of this (batch, KV head) plus a 32-bit per-lane
  // byte offset whose tile-independent part is kept per load (one VGPR each).
  // Rows past S re-read row S-1 (in bounds; their scores are masked and
  // their weights 0).
  const bf16* kg = k + kvbase;
  const bf16* vg = v + kvbase;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  uint32_t koff[CPW], voff[CPW];
  int lrow[CPW];
#pragma unroll
  for (int r = 0; r < CPW; ++r) {
    const int p = 64 * (wave * CPW + r) + lane;
    const int row = p / CPR, cph = p % CPR;
    lrow[r] = row;
    koff[r] = (uint32_t)(row * D + (cph ^ k_swz<D>(row)) * 8) * 2u;
    voff[r] = (uint32_t)(row * D + (cph ^ v_swz<D>(row)) * 8) * 2u;
  }
  // Paged cache: the rows of one load instruction (64 lanes x 16 bytes = 4
  // rows at D=128, 8 at D=64, aligned) lie in one 16-token page, so the page
  // is wave-uniform per instruction and its base a scalar address; the lane
  // adds its slot.  Each wave streams the BN/16 page ids of tile j into its
  // own LDS slot (j & 1) with a direct-to-LDS load two steps before tile j's
  // keys are loaded, so the per-step vector-memory wait covers them (a plain
  // load would be waited on, together with the tile loads in flight, where
  // it is used).  Rows past S re-read row S-1, in the same page as the
  // instruction's clamped first row.
  static_assert(!PAGED || NST == 2, "the page-id stream assumes a two-stage ring");
  constexpr int kRowsPerLoad = 64 / CPR;
  constexpr int kIds = BN / 16;
  __shared__ int32_t pg_ids[PAGED ? 2 * PrefillCfg<D, QB>::WAVES * 8 : 1];   // [slot][wave][id]
  const void* bt_row = PAGED ? uniform_ptr(pkv.block_table + (size_t)b * pkv.max_blocks) : nullptr;
  auto fetch_pages = [&](int j) {
    if (PAGED && lane < kIds) {
      const int blk = min(j * kIds + lane, ((S + 15) >> 4) - 1);
      lds_dma4(uniform_ptr(bt_row), (uint32_t)blk * 4u,
               lds_addr(pg_ids) + (uint32_t)(((j & 1) * PrefillCfg<D, QB>::WAVES + wave_s) * 32));
    }
  };
  auto load_tile = [&](int j, bf16* ks, bf16* vs) {
    const uint32_t kl = lds_addr(ks) + (uint32_t)(wave_s * CPW) * 1024u;
    const uint32_t vl = lds_addr(vs) + (uint32_t)(wave_s * CPW) * 1024u;
    const bool full = (j + 1) * BN <= S;
    if (PAGED) {
      const int32_t* ids = pg_ids + ((j & 1) * PrefillCfg<D, QB>::WAVES + wave) * 8;
#pragma unroll
      for (int r = 0; r < CPW; ++r) {
        const int key0 = min(j * BN + (wave_s * CPW + r) * kRowsPerLoad, S - 1);
        int pg = __builtin_amdgcn_readfirstlane(ids[(key0 >> 4) - j * kIds]);
        pg = min(max(pg, 0), pkv.num_pages - 1);     // never outside the pool
        const size_t pbase = ((size_t)pg * Hkv + hk) * 16 * D;
        const int key = full ? j * BN + lrow[r] : min(j * BN + lrow[r], S - 1);
        const uint32_t slot = (uint32_t)((key & 15) - (lrow[r] & 15)) * D * 2u;
        lds_dma16(k + pbase, koff[r] - (uint32_t)((lrow[r] & ~15) * D * 2) + slot, kl + 1024u * r);
        lds_dma16(v + pbase, voff[r] - (uint32_t)((lrow[r] & ~15) * D * 2) + slot, vl + 1024u * r);
      }
      return;
    }
    if (full) {
      // the tile's offset goes into the scalar base: no per-lane arithmetic
      const bf16* kt = kg + (size_t)j * BN * D;
      const bf16* vt = vg + (size_t)j * BN * D;
#pragma unroll
      for (int r = 0; r < CPW; ++r) {
        lds_dma16(kt, koff[r], kl + 1024u * r);
        lds_dma16(vt, voff[r], vl + 1024u * r);
      }
    } else {
#pragma unroll
      for (int r = 0; r < CPW; ++r) {
        const int key = min(j * BN + lrow[r], S - 1);
        const uint32_t add = (uint32_t)((key - lrow[r]) * D) * 2u;
        lds_dma16(kg, koff[r] + add, kl + 1024u * r);
        lds_dma16(vg, voff[r] + add, vl + 1024u * r);
      }
    }
  };

  // ---- Q rows into registers (B operand of S^T = K Q^T) ----
  bf16x8 qop[QB][NDC];
  int row_lim[QB], row_lo[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = wrow0 + 16 * qb + l16;
    if (row < T) {
      const bf16* qp = q + qbase + (size_t)row * D + 8 * g;
#pragma unroll
      for (int c = 0; c < NDC; ++c) qop[qb][c] = *reinterpret_cast<const bf16x8*>(qp + 32 * c);
    } else {
#pragma unroll
      for (int c = 0; c < NDC; ++c) qop[qb][c] = bf16x8{};
    }
    // last key visible to this row (rows past T only feed discarded lanes)
    row_lim[qb] = CAUSAL ? min(row + (S - T), S - 1) : S - 1;
    row_lo[qb] = windowed ? row + (S - T) - window + 1 : 0;
  }

  // ---- running softmax state of rows wrow0 + 16 qb + l16 ----
  float m_run[QB], l_part[QB];               // running max of scaled logits (log2 units);
  float m_use[QB];                           // m_run, or 0 while it is -inf (exponent offset)
  f32x4 acc[QB][NDB];                        // sum over this lane's keys of exp2(s - m_run)
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    m_use[qb] = 0.f;
    l_part[qb] = 0.f;
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[qb][db] = f32x4{};

  // per-lane operand addressing inside a stage
  const int kswz = k_swz<D>(l16);                             // same for row 16 kb + l16
  const int v_row = 4 * g + (l16 >> 2);                       // key within a 32-key chunk
  const int v_chunk = (l16 & 3) >> 1;                         // + 2 db
  const int v_sw = v_swz<D>(v_row);                           // same for v_row + 16, + 32 c
  const int v_in = 4 * (l16 & 1);

  auto compute_tile = [&](int j, const bf16* ks, const bf16* vs) {
    // S^T[key][row] for the BN keys of this tile; each K operand feeds both row blocks
    f32x4 s[QB][NKB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) s[qb][kb] = f32x4{};
#pragma unroll
    for (int c = 0; c < NDC; ++c) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const bf16x8 kop = *reinterpret_cast<const bf16x8*>(
            ks + (16 * kb + l16) * D + (((4 * c + g) ^ kswz) * 8));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb][kb] = mfma_16x16x32(kop, qop[qb][c], s[qb][kb]);
      }
    }
    // each K operand read four operands ahead of its MFMAs (the scheduler's
    // own choice, two ahead, left the MFMAs waiting on LDS; bit-identical,
    // prefill_3 and prefill_4 2-3 % faster)
    sched_reads_ahead<NDC * NKB, 1, QB, 4>();

    // mask keys past the diagonal or past S (only tiles that need it)
    const bool need_mask = ((j + 1) * BN > S) || (CAUSAL && (j + 1) * BN - 1 > wrow0 + (S - T));
    if (need_mask) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = j * BN + 16 * kb + 4 * g + i;
            if (key > row_lim[qb]) s[qb][kb][i] = -INFINITY;
          }
    }
    // and keys left of the window (tiles reaching past the last row's window start)
    if (windowed && j * BN < wrow0 + kWR + (S - T) - window) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = j * BN + 16 * kb + 4 * g + i;
            if (key < row_lo[qb]) s[qb][kb][i] = -INFINITY;
          }
    }

    // online softmax update (base 2)
    // row maximum of the tile per lane: a three-input max tree over its 4 NKB scores
    float mloc[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mk[4 * NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mk[4 * kb + i] = s[qb][kb][i];
#pragma unroll
      for (int w = 4 * NKB; w > 1; w = (w + 2) / 3)
#pragma unroll
        for (int i = 0; i < (w + 2) / 3; ++i) {
          if (3 * i + 1 == w) {                      // a lone last value moves up as is
            mk[i] = mk[3 * i];
          } else {
            const float a = mk[3 * i], b = mk[3 * i + 1], c = 3 * i + 2 < w ? mk[3 * i + 2] : b;
            mk[i] = max3_raw(a, b, c);
          }
        }
      mloc[qb] = mk[0];
    }
    // The reference maximum only moves when the tile's maximum exceeds it by
    // more than kLazyTau (log2 units), so exponents stay <= 2^kLazyTau and
    // the accumulator is rarely rescaled; any reference gives the same O and
    // LSE (it cancels between acc and l), only the rounding changes.  A row's
    // maximum can only pass that bar if one of its four lanes' own maxima does
    // (scale > 0), so the cross-lane maxima, the new references and the
    // rescale factors are only formed on tiles where some lane of the wave
    // passes it for some row block (one vote and one branch per tile);
    // elsewhere nothing moves and alpha is 1.
    float alpha[QB];
    bool pass = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      alpha[qb] = 1.f;
      pass |= mloc[qb] * scale_log2 > m_run[qb] + kLazyTau;   // always when m_run = -inf
    }
    if (wave_any(pass)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float m_tile = pair_max32_raw(pair_max16_raw(mloc[qb])) * scale_log2;
        const bool grow = m_tile > m_run[qb] + kLazyTau;
        const float m_new = grow ? m_tile : m_run[qb];
        const float m_off = (m_new == -INFINITY) ? 0.f : m_new;
        alpha[qb] = exp2_hw(m_run[qb] - m_off);
        m_run[qb] = m_new;
        m_use[qb] = m_off;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[qb][db][i] *= alpha[qb];
      }
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = exp2_hw(__builtin_fmaf(s[qb][kb][i], scale_log2, -m_use[qb]));
          s[qb][kb][i] = p;
          rs += p;
        }
      l_part[qb] = __builtin_fmaf(l_part[qb], alpha[qb], rs);
    }

    // O^T += V^T P^T, 32 keys at a time; each V operand feeds both row blocks
#pragma unroll
    for (int c = 0; c < NPC; ++c) {
      bf16x8 pop[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        pop[qb] = pack_bf16x8(s[qb][2 * c][0], s[qb][2 * c][1], s[qb][2 * c][2], s[qb][2 * c][3],
                              s[qb][2 * c + 1][0], s[qb][2 * c + 1][1], s[qb][2 * c + 1][2],
                              s[qb][2 * c + 1][3]);
      const bf16* vp = vs + (32 * c + v_row) * D + v_in;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int off = ((2 * db + v_chunk) ^ v_sw) * 8;
        const i16x4 lo = lds_read_tr16(vp + off);
        const i16x4 hi4 = lds_read_tr16(vp + 16 * D + off);
        const bf16x8 vop = concat_tr(lo, hi4);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) acc[qb][db] = mfma_16x16x32(vop, pop[qb], acc[qb][db]);
      }
    }
  };

  // One step: wait for this tile's loads, publish the tile to the workgroup
  // (which also proves every wave is done with the tile before, freeing its
  // stage), start loading tile j + NST - 1 into that freed stage, compute
  // tile j.  With three stages the load of tile j+1 may still be in flight at
  // the wait: it was issued after tile j's, so vmcnt(2 CPW) suffices.
  auto step = [&](int j, const bf16* ks, const bf16* vs, bf16* kn, bf16* vn) {
    if (NST == 3 && j + 1 < ntk) {
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0 | vmcnt_bits(2 * CPW));
    } else {
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0 | vmcnt_bits(0));
    }
    stage_barrier();
    if (j + NST - 1 < ntk) {
      load_tile(j + NST - 1, kn, vn);
      if (j + NST < ntk) fetch_pages(j + NST);
    }
    if (wave_live && j * BN < wave_kv_end && (j + 1) * BN > wave_kv_lo) compute_tile(j, ks, vs);
  };

  fetch_pages(j0);
  if (PAGED) __builtin_amdgcn_s_waitcnt(kWaitLgkm0 | vmcnt_bits(0));   // tile j0's page ids
  load_tile(j0, k_st0, v_st0);
  if (j0 + 1 < ntk) fetch_pages(j0 + 1);
  if (NST == 3) {
    if (j0 + 1 < ntk) {
      load_tile(j0 + 1, k_st1, v_st1);
      if (j0 + 2 < ntk) fetch_pages(j0 + 2);
    }
    for (int j = j0;;) {
      step(j, k_st0, v_st0, k_st2, v_st2);
      if (++j >= ntk) break;
      step(j, k_st1, v_st1, k_st0, v_st0);
      if (++j >= ntk) break;
      step(j, k_st2, v_st2, k_st1, v_st1);
      if (++j >= ntk) break;
    }
  } else {
    for (int j = j0;;) {
      step(j, k_st0, v_st0, k_st1, v_st1);
      if (++j >= ntk) break;
      step(j, k_st1, v_st1, k_st0, v_st0);
      if (++j >= ntk) break;
    }
  }

  // ---- epilogue: O = acc / l (bf16, nearest even), LSE = ln2 * (m + log2 l) ----
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = pair_sum32(pair_sum16(l_part[qb]));
    const int row = wrow0 + 16 * qb + l16;
    if (row < T) {
      const float inv = 1.f / l_tot;
      bf16* op = o + qbase + (size_t)row * D + 4 * g;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        bf16x4 r;
        r[0] = (bf16)(acc[qb][db][0] * inv);
        r[1] = (bf16)(acc[qb][db][1] * inv);
        r[2] = (bf16)(acc[qb][db][2] * inv);
        r[3] = (bf16)(acc[qb][db][3] * inv);
        *reinterpret_cast<bf16x4*>(op + 16 * db) = r;
      }
      if (lse != nullptr && g == 0)
        lse[(size_t)(b * Hq + h) * Tst + row] = (m_run[qb] + log2f(l_tot)) * kLn2;
    }
  }
}

template <int D, bool CAUSAL, int QB, bool PAGED>
hipError_t launch_one(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int Hq, int Hkv, int T, int S, float scale_log2, int window,
                      const PagedKv& pkv, hipStream_t stream) {
  constexpr int kThreads = 64 * PrefillCfg<D, QB>::WAVES;
  constexpr int kBM = 16 * QB * PrefillCfg<D, QB>::WAVES;
  const long long ntq = (T + kBM - 1) / kBM;
  const long long grid = ntq * B * Hq;
  // Snake order (see the kernel) when the grid is resident all at once and
  // every XCD's share is whole runs of 32 workgroups.
  static const int per_cu = [] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, reinterpret_cast<const void*>(prefill_bf16_kernel<D, CAUSAL, QB, PAGED>), kThreads,
            0) != hipSuccess)
      n = 0;
    return n;
  }();
  int snake = 0;
  if (CAUSAL && !PAGED && ((B * Hkv) & 7) == 0 && grid % 256 == 0 &&
      grid <= (long long)per_cu * kXcdCount * kCusPerXcd)
    snake = 1;
  launch_kernel(prefill_bf16_kernel<D, CAUSAL, QB, PAGED>, dim3((unsigned)grid),
                     dim3(kThreads), 0, stream, static_cast<const bf16*>(q),
                     static_cast<const bf16*>(k), static_cast<const bf16*>(v),
                     static_cast<bf16*>(o), lse, B, Hq, Hkv, T, S, scale_log2, window, pkv, snake);
  return hipGetLastError();
}

// Two 16-row blocks per wave share every K and V operand read; one block per
// wave halves the work on a workgroup's critical path (the longest causal
// query tile) at the price of twice the LDS reads per MFMA.  A grid of at
// most one workgroup per CU is bound by that path (B=1 at T=1024, d=64: 11 us
// instead of 16 us), so it gets one block per wave; a fuller grid is bound by
// the total work (B=8 at the same shape, 128-key tiles: 30 us instead of
// 28.5 us).
template <int D, bool CAUSAL, bool PAGED = false>
hipError_t launch_rows(const void* q, const void* k, const void* v, void* o, float* lse,
                       int B, int Hq, int Hkv, int T, int S, float scale_log2, int window,
                       hipStream_t stream, const PagedKv& pkv = PagedKv{}) {
  constexpr int kBM2 = 32 * PrefillCfg<D, 2>::WAVES;
  const long long wgs2 = (long long)((T + kBM2 - 1) / kBM2) * B * Hq;
  if (wgs2 < PREFILL_SMALL_GRID)
    return launch_one<D, CAUSAL, 1, PAGED>(q, k, v, o, lse, B, Hq, Hkv, T, S, scale_log2, window,
                                           pkv, stream);
  return launch_one<D, CAUSAL, 2, PAGED>(q, k, v, o, lse, B, Hq, Hkv, T, S, scale_log2, window,
                                         pkv, stream);
}

}  // namespace

hipError_t launch_prefill_paged_bf16(const void* q, const void* k_pool, const void* v_pool,
                                     void* o, float* lse, const PagedKv& pkv, int N, int Hq,
                                     int Hkv, int T, int d, float scale_log2, int window,
                                     hipStream_t stream) {
  if (d == 128)
    return launch_rows<128, true, true>(q, k_pool, v_pool, o, lse, N, Hq, Hkv, T, 0, scale_log2,
                                        window, stream, pkv);
  return launch_rows<64, true, true>(q, k_pool, v_pool, o, lse, N, Hq, Hkv, T, 0, scale_log2,
                                     window, stream, pkv);
}

hipError_t launch_prefill_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                               int B, int Hq, int Hkv, int T, int S, int d, float scale_log2,
                               bool causal, int window, hipStream_t stream) {
  if (d == 128)
    return causal ? launch_rows<128, true>(q, k, v, o, lse, B, Hq, Hkv, T, S, scale_log2, window, stream)
                  : launch_rows<128, false>(q, k, v, o, lse, B, Hq, Hkv, T, S, scale_log2, 0, stream);
  return causal ? launch_rows<64, true>(q, k, v, o, lse, B, Hq, Hkv, T, S, scale_log2, window, stream)
                : launch_rows<64, false>(q, k, v, o, lse, B, Hq, Hkv, T, S, scale_log2, 0, stream);
}

}  // namespace attn
