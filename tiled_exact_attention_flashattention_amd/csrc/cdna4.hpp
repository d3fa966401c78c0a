// cdna4.hpp -- small device helpers for gfx950 (CDNA4): vector types, the two
// bf16 MFMA shapes the kernels use, exp2/log2, bf16 packing and cross-lane
// reductions.  Everything here is wave64.
//
// MFMA operand layouts (checked on the device against a host matmul):
//   32x32x16 bf16: A[32][16]: lane l holds row l%32, 8 k-values of group l/32;
//                  B[16][32]: lane l holds column l%32, the same 8 k-values;
//                  D[32][32]: lane l, register i holds
//                             row 8*(i/4) + 4*(l/32) + i%4, column l%32.
//   16x16x32 bf16: A[16][32]: lane l holds row l%16, 8 k-values of group l/16;
//                  B[32][16]: lane l holds column l%16, the same 8 k-values;
//                  D[16][16]: lane l, register i holds row 4*(l/16) + i,
//                             column l%16.
// Only the pairing of A and B k-slots matters for a dot product, so the
// kernels are free to decide which logical k each (lane group, slot) carries.
//
// ds_read_b64_tr_b16 (gfx950 LDS transpose read), checked on the device:
// inside each 16-lane group, lane 4a+b receives element b of the 8-byte rows
// addressed by lanes 4i+a, for i = 0..3 (a 4x4 transpose of 16-bit values
// across lanes).  Pointing lane j of a group at row (base_key + j/4), column
// (base_d + 4*(j%4)) of a row-major [key][d] tile hands lane 4a+b the four
// keys base_key..base_key+3 of column base_d + 4a + b.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ f32x16 mfma_32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Hardware base-2 exponential (v_exp_f32).  exp2(-inf) == 0.  Its arguments
// are at most 0 (decode, fp32 prefill, backward) or at most the bf16
// prefill's lazy slack of 8, so results lie in [0, 1] or [0, 2^8].
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Transposed 4 x 16-bit read from LDS (see the header comment).
__device__ __forceinline__ i16x4 lds_read_tr16(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

__device__ __forceinline__ bf16x8 pack_bf16x8(float a0, float a1, float a2, float a3,
                                              float a4, float a5, float a6, float a7) {
  bf16x8 r;
  r[0] = (bf16)a0; r[1] = (bf16)a1; r[2] = (bf16)a2; r[3] = (bf16)a3;
  r[4] = (bf16)a4; r[5] = (bf16)a5; r[6] = (bf16)a6; r[7] = (bf16)a7;
  return r;
}

__device__ __forceinline__ bf16x8 concat_tr(i16x4 lo, i16x4 hi) {
  union { i16x4 s[2]; bf16x8 b; } u;
  u.s[0] = lo;
  u.s[1] = hi;
  return u.b;
}

__device__ __forceinline__ float xor_lane(float x, int mask) { return __shfl_xor(x, mask); }

// Pair reductions across lanes l and l^16 (resp. l^32) with the gfx950
// v_permlane16_swap / v_permlane32_swap VALU ops (no LDS round trip).  Called
// with the same value in both operands, the swap returns, in every lane, the
// pair (x[l & ~m], x[l | m]) in that order (checked on the device), so both
// lanes of a pair compute the same max / sum bit for bit.
__device__ __forceinline__ float pair_max16(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_max32(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum16(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair_sum32(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Maximum of three floats, one v_max3_f32.  Written out because fmaxf first
// quiets signalling NaNs in every operand that the compiler cannot prove
// canonical (one v_max per operand, twice the work); the operands here are
// MFMA results or their maxima, finite or -inf.
__device__ __forceinline__ float max3_raw(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// pair_max16 / pair_max32 on max3_raw.
__device__ __forceinline__ float pair_max16_raw(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return max3_raw(__uint_as_float(r[0]), __uint_as_float(r[1]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_max32_raw(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return max3_raw(__uint_as_float(r[0]), __uint_as_float(r[1]), __uint_as_float(r[1]));
}

// True in every lane if the predicate holds in any lane of the wave.
__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// Exact-rounding-independent max: both operands are finite or -inf.
__device__ __forceinline__ float fmax2(float a, float b) { return __builtin_fmaxf(a, b); }

// 16-byte global load / store helpers (addresses must be 16-byte aligned).
__device__ __forceinline__ u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void store16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }

// Instruction order for a run of N steps that each take R LDS reads and M
// MFMAs: the reads of the first A steps, then per step its M MFMAs followed
// by the reads of the step A ahead.  With few waves per SIMD the main cover
// for LDS latency is reads in flight; left alone the scheduler pulls each
// read next to its first use.  Place it in the block that holds the run.
template <int N, int R, int M, int A>
__device__ __forceinline__ void sched_reads_ahead() {
  constexpr int kDsRead = 0x100, kMfma = 0x008;
  __builtin_amdgcn_sched_group_barrier(kDsRead, R * (N < A ? N : A), 0);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_group_barrier(kMfma, M, 0);
    if (i + A < N) __builtin_amdgcn_sched_group_barrier(kDsRead, R, 0);
  }
}

// Workgroup-id remap that keeps the workgroups of one logical group on one
// XCD.  The dispatcher hands workgroup ids to the 8 XCDs round-robin, so id
// `pid` runs on XCD pid % 8 as that XCD's (pid / 8)-th workgroup.  Returns the
// logical index such that each XCD walks one contiguous eighth of the logical
// range in order.  Requires total % 8 == 0.
__device__ __forceinline__ int xcd_contiguous(int pid, int total) {
  return (pid & 7) * (total >> 3) + (pid >> 3);
}

}  // namespace attn
