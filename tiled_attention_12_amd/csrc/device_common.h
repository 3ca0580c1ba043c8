// Device helpers shared by the gfx950 attention kernels.
//
// Lane layouts used throughout (wave64, checked on the hardware):
//  * v_mfma_f32_32x32x16_bf16: A (32x16) lane l holds row l%32, k = 8*(l/32)+j
//    for j = 0..7; B (16x32) lane l holds column l%32, k = 8*(l/32)+j;
//    C/D (32x32 fp32) lane l holds column l%32, rows 8*(i/4) + 4*(l/32) + i%4
//    for i = 0..15.
//  * ds_read_b64_tr_b16: inside each group of 16 lanes, lane i receives, as
//    its element r (r = 0..3), element i%4 of the 8-byte block addressed by
//    lane 4*r + i/4 of the same group.
//  * global_load_lds_dwordx4: lane l's 16 bytes land at LDS base + 16*l, the
//    base being wave-uniform.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace tattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Compile-time loop: f(std::integral_constant<int, i>{}) for i = 0..N-1, so
// the body can use i as a constant expression (template arguments, asm
// immediates).
template <int... Is, class F>
__device__ __forceinline__ void static_for_impl(std::integer_sequence<int, Is...>, F&& f) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(std::make_integer_sequence<int, N>{}, f);
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Position of 16-byte chunk `c` of row `r` inside a tile whose rows hold
// `CPR` chunks. The XOR on the low chunk bits makes the two LDS read
// patterns conflict-free: 16 consecutive rows at one chunk (MFMA operand
// reads along a row) and 4 aligned rows x 4 aligned chunks (the transposing
// reads of the value operand).
template <int CPR>
__device__ __forceinline__ int swz(int r, int c) {
  if constexpr (CPR >= 16) {
    return c ^ (((r & 3) << 2) | ((r >> 2) & 3));
  } else {
    static_assert(CPR == 8, "rows of 8 or >= 16 chunks");
    return c ^ ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
  }
}

// 16-byte direct global -> LDS load through inline asm (M0 <- LDS base, then
// the load); lane l writes LDS base + 16*l.
// The compiler does not see this write to LDS, so its LDS reads (including
// the transposing-read builtin) are not made to wait for it; callers order
// LDS reuse with wait_vmcnt() and barrier(). M0 is written here and by no
// compiler-generated code in the kernels that use this (checked in their
// assembly), so the clobber of the reserved register is safe there.
__device__ __forceinline__ void load_lds16_asm(const void* gptr, uint32_t lds_base_uniform) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(gptr), "s"(lds_base_uniform) : "memory", "m0");
}

// The same load in the instruction's scalar-base form: a wave-uniform 64-bit
// base address in SGPRs plus a 32-bit unsigned per-lane byte offset, so each
// load needs one VGPR for its offset and no per-lane 64-bit address add.
__device__ __forceinline__ void load_lds16_sbase(const void* base_uniform, uint32_t voff,
                                                 uint32_t lds_base_uniform) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(base_uniform), "s"(lds_base_uniform) : "memory", "m0");
}

// ds_read_b64_tr_b16 through the compiler builtin (it tracks lgkmcnt and can
// place the result directly in an MFMA operand tuple).
template <int OFF>
__device__ __forceinline__ u32x2 lds_read_tr16(uint32_t lds_addr) {
  const auto r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(uintptr_t)(lds_addr + OFF));
  return __builtin_bit_cast(u32x2, r);
}

__device__ __forceinline__ u32x4 lds_read128(const void* p) {
  return *(const __attribute__((address_space(3))) u32x4*)((__attribute__((address_space(3))) const char*)(uintptr_t)p);
}

// ds_read_b64_tr_b16 issued through inline asm. The compiler does not see it
// as an LDS access, so it neither counts it for lgkmcnt nor makes it wait for
// in-flight global->LDS loads into other buffers; the caller waits with
// wait_lds_tied_n() before using the result. `byte_off` is the instruction's
// immediate offset.
template <int OFF>
__device__ __forceinline__ u32x2 lds_read_tr16_async(uint32_t lds_addr) {
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(lds_addr), "i"(OFF));
  return r;
}

// s_waitcnt lgkmcnt(N) tied to two values: they are complete once at most N
// later LDS operations are still outstanding (LDS operations complete in
// order; the caller must have no scalar-memory loads in flight).
template <int N>
__device__ __forceinline__ void wait_lds_tied_n(u32x2& a, u32x2& b) {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "i"(N));
}

// ds_read_b128 through inline asm (not counted by the compiler; wait with
// wait_lds_tied_n4 before use).
template <int OFF>
__device__ __forceinline__ u32x4 lds_read128_async(uint32_t lds_addr) {
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(lds_addr), "i"(OFF));
  return r;
}
template <int N>
__device__ __forceinline__ void wait_lds_tied_n4(u32x4& a) {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(a) : "i"(N));
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)(p);
}

// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
}

// Workgroup barrier that orders LDS traffic only: callers wait for the
// counters they need first. The asm memory clobber keeps the compiler from
// moving memory operations across it.
__device__ __forceinline__ void barrier() {
  asm volatile("s_barrier" ::: "memory");
}

// v_permlane32_swap with both operands = x returns, in every lane l, the pair
// {x(l), x(l ^ 32)} (in lane-dependent order), so these reductions across the
// two wave halves give identical bits in lanes l and l ^ 32.
__device__ __forceinline__ float max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Sum of x over the 8 lanes of an aligned lane octet (every lane gets it):
// xor 1 and xor 2 inside each quad (DPP quad permutes), then the mirror
// inside each half-row pairs every lane of one quad with a lane of the other.
__device__ __forceinline__ float octet_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
  return x;
}

// x *= alpha for an MFMA accumulator that lives in AGPRs, element by element
// through one temporary VGPR (VALU cannot read AGPRs directly), so a rare
// rescale of a large accumulator never needs a block of VGPRs.
__device__ __forceinline__ void scale_acc16(f32x16& x, float alpha) {
  float e[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) e[i] = x[i];
  float t;
#define TATTN_SCALE4(i0, i1, i2, i3)                                                        \
  asm volatile(                                                                            \
      "v_accvgpr_read_b32 %4, %0\n\tv_mul_f32 %4, %4, %5\n\tv_accvgpr_write_b32 %0, %4\n\t" \
      "v_accvgpr_read_b32 %4, %1\n\tv_mul_f32 %4, %4, %5\n\tv_accvgpr_write_b32 %1, %4\n\t" \
      "v_accvgpr_read_b32 %4, %2\n\tv_mul_f32 %4, %4, %5\n\tv_accvgpr_write_b32 %2, %4\n\t" \
      "v_accvgpr_read_b32 %4, %3\n\tv_mul_f32 %4, %4, %5\n\tv_accvgpr_write_b32 %3, %4"       \
      : "+a"(e[i0]), "+a"(e[i1]), "+a"(e[i2]), "+a"(e[i3]), "=&v"(t)                           \
      : "v"(alpha))
  TATTN_SCALE4(0, 1, 2, 3);
  TATTN_SCALE4(4, 5, 6, 7);
  TATTN_SCALE4(8, 9, 10, 11);
  TATTN_SCALE4(12, 13, 14, 15);
#undef TATTN_SCALE4
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = e[i];
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Round two floats to bf16 (nearest-even) and pack them, lo in bits 15:0.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 v = __builtin_convertvector(f32x2{lo, hi}, bf16x2);
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ bf16x8 cat_tr(u32x2 a, u32x2 b) {
  u32x4 r = {a[0], a[1], b[0], b[1]};
  return __builtin_bit_cast(bf16x8, r);
}

}  // namespace tattn
