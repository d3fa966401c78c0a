// lds_stage.hpp -- staging of tiles HBM -> LDS with the gfx950 direct-to-LDS
// load, shared by the kernels that stream tiles through LDS stages.
//
// The load is issued through asm so that the compiler does not track it: its
// own wait insertion would otherwise stall the LDS reads of the stage being
// computed until a load aimed at another stage completed.  Completion is
// awaited explicitly (s_waitcnt vmcnt) before the barrier that publishes a
// stage.  The asm sets M0; a kernel that uses these helpers must not rely on
// M0 otherwise (no compiler-issued LDS DMA, no indirect register indexing,
// no messages).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// s_waitcnt encodings (gfx9): vmcnt in bits [3:0] and [15:14], expcnt in
// [6:4], lgkmcnt in [11:8].  kWaitLgkm0 | vmcnt_bits(n) waits for lgkmcnt(0)
// and vmcnt(n) with expcnt unconstrained.
constexpr unsigned kWaitLgkm0 = 0x0070;
constexpr unsigned vmcnt_bits(int n) { return (unsigned)(n & 15) | ((unsigned)(n >> 4) << 14); }

// One 16-byte-per-lane direct-to-LDS load: lane i's 16 bytes from `sbase` +
// `voff` (a wave-uniform base and a 32-bit per-lane byte offset) land at LDS
// byte address `lds_base` + 16 i (lds_base wave-uniform, in M0).
__device__ __forceinline__ void lds_dma16(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(sbase), "s"(lds_base) : "memory");
}

// The 4-byte form: lane i's dword from `sbase` + `voff` lands at `lds_base` +
// 4 i.  Lanes switched off by the execution mask load nothing.
__device__ __forceinline__ void lds_dma4(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1"
               :: "v"(voff), "s"(sbase), "s"(lds_base) : "memory");
}

// A pointer every lane holds the same value of, moved to scalar registers
// (the base operand of the loads above must be scalar; inside a divergent
// branch the compiler may otherwise keep it in vector registers).
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Workgroup barrier without a memory fence: the LDS stages are filled by the
// direct-to-LDS loads, whose completion is awaited explicitly with vmcnt, and
// a fence here would make the compiler wait for the load in flight as well.
// The empty asm statements keep the optimiser from moving LDS accesses across.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 16-byte-chunk swizzle for a row-major [rows][D] bf16 tile that is read both
// ways: as MFMA row operands (16 consecutive rows, one chunk each, by
// ds_read_b128) and through the LDS transpose read (8 consecutive rows, one
// 32-byte chunk pair each).  Measured on gfx950 with SQ_LDS_BANK_CONFLICT
// for both read patterns of the kernels that use it: this form (the chunk
// pair index from the row, D = 64 rows being half a bank line) reads both
// ways without conflicts; adding row bit 3 into chunk bit 0 made every
// ds_read_b128 of the pattern pay about four conflict cycles.
template <int D>
__device__ __forceinline__ int dual_swz(int row) {
  return D == 128 ? 2 * (row & 7) : 2 * ((row >> 1) & 3);
}

}  // namespace attn
