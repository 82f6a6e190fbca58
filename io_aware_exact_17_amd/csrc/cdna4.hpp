// cdna4.hpp — small device helpers for gfx950 (CDNA4): vector types, the bf16
// matrix-core product, wave64 cross-lane exchanges and fast exp2/log2.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLn2 = 0.693147180559945309417f;
constexpr float kLog2e = 1.442695040888963407360f;

// D[32x32] += A[32x16] * B[16x32], bf16 operands, fp32 accumulate.
// Operand layout (wave64): lane l holds A[l%32][8*(l/32) + 0..7] and
// B[8*(l/32) + 0..7][l%32].  Accumulator register r of lane l holds
// D[8*(r/4) + 4*(l/32) + r%4][l%32].
__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Two fp32 -> packed bf16x2 with round-to-nearest-even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  bf16x2 r = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 2^x on the transcendental unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }

// Lanes l and l^32 exchange halves in one v_permlane32_swap; the pair's
// maximum / sum is then available in both lanes.
__device__ __forceinline__ float max_across_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_across_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// All-reduce over each aligned group of 16 lanes with DPP row operations:
// xor-1 and xor-2 inside quads, then the half-row mirror (lane i <-> 7-i)
// and the row mirror (lane i <-> 15-i).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float sum_row16(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror
  x += dpp<0x140>(x);  // row_mirror
  return x;
}
// Same over aligned groups of 8 lanes.
__device__ __forceinline__ float sum_row8(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  return x;
}

// s_waitcnt immediate for "at most n vector-memory operations outstanding"
// (expcnt and lgkmcnt left at their maxima).
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// One 16-byte-per-lane copy from global memory straight into LDS
// (global_load_lds_dwordx4): lane l's 16 bytes at gbase + voff land at LDS
// byte lds_addr + 16 l.  Issued from inline assembly so that the compiler
// does not tie later LDS reads to it with waits of its own: the kernel waits
// for these copies explicitly (vmcnt, then a barrier) before reading a tile.
__device__ __forceinline__ void copy_to_lds(const char* gbase, uint32_t voff, uint32_t lds_addr) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(gbase), "s"(lds_addr)
               : "memory", "m0");
#pragma clang diagnostic pop
}

// Race-check build (compiled with FA_PARANOID_SYNC): at every point where a
// kernel moves from one LDS stage to the next, every memory operation of the
// wave completes (vmcnt, expcnt and lgkmcnt all zero) and the workgroup meets
// at a barrier.  Nothing is then in flight across a stage boundary, so a
// missing or miscounted wait in the normal build shows up as a difference
// between the two builds' results.  A no-op in the normal build.
__device__ __forceinline__ void paranoid_sync() {
#ifdef FA_PARANOID_SYNC
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
#endif
}

__device__ __forceinline__ bool wave_any(bool p) {
  return __builtin_amdgcn_ballot_w64(p) != 0;
}

}  // namespace fa
