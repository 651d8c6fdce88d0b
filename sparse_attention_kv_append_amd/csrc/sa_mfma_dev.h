// Device helpers shared by the matrix-core forward kernels: vector types,
// compile-time loops, LDS reads/writes issued as inline asm with immediate
// offsets and counted waits, the gfx950 cross-lane permutes used for row
// reductions, and bf16 packing.
#pragma once

#include <utility>

#include "sa_internal.h"

namespace sa {

typedef __bf16 bf16x8_l __attribute__((ext_vector_type(8)));
typedef float f32x4_l __attribute__((ext_vector_type(4)));
typedef short s16x4_l __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_l __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_l __attribute__((ext_vector_type(2)));
typedef float f32x2_l __attribute__((ext_vector_type(2)));
typedef unsigned u32x2_l __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) u32x4_l lds_u32x4;

constexpr float kLog2eL = 1.4426950408889634f;

// compile-time loop: f(std::integral_constant<int, I>) for I = 0 .. N-1
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// two fp32 -> bf16 (round to nearest even) packed in one word, low = a
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_l){a, b}, bf16x2_l));
}

// cache policy of a buffer store written through the XCD's L2 (sc1): a
// launch's end then has no dirty lines of it to write back
constexpr int kWriteThrough = 16;

// vmcnt-only wait (gfx9 encoding: expcnt and lgkmcnt left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// LDS atomic minimum issued as inline asm. The compiler treats a visible LDS
// atomic as possibly touching what the direct-to-LDS gathers in flight write
// and waits for all of them first; this one does not. LDS operations complete
// in order, so the compiler's own later LDS waits still cover it.
__device__ __forceinline__ void ds_min_i32_at(uint32_t addr, int v) {
  asm volatile("ds_min_i32 %0, %1" : : "v"(addr), "v"(v) : "memory");
}

__device__ __forceinline__ void ds_min_u64_at(uint32_t addr, unsigned long long v) {
  asm volatile("ds_min_u64 %0, %1" : : "v"(addr), "v"(v) : "memory");
}

// LDS reads issued as inline asm with an immediate offset. The compiler
// would wait for every outstanding LDS DMA before its own LDS reads, and
// drains all reads at each of its waits; these are waited for explicitly.
template <int OFF>
__device__ __forceinline__ u32x4_l ds_read_b128_at(uint32_t addr) {
  u32x4_l r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF) : "memory");
  return r;
}
template <int OFF>
__device__ __forceinline__ s16x4_l ds_read_tr16_at(uint32_t addr) {
  s16x4_l r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF) : "memory");
  return r;
}
template <int OFF>
__device__ __forceinline__ void ds_write_b128_off(uint32_t addr, u32x4_l v) {
  asm volatile("ds_write_b128 %0, %1 offset:%2" : : "v"(addr), "v"(v), "n"(OFF) : "memory");
}
__device__ __forceinline__ void ds_write_b128_at(uint32_t addr, u32x4_l v) {
  asm volatile("ds_write_b128 %0, %1" : : "v"(addr), "v"(v) : "memory");
}
__device__ __forceinline__ void ds_write_b64_at(uint32_t addr, u32x2_l v) {
  asm volatile("ds_write_b64 %0, %1" : : "v"(addr), "v"(v) : "memory");
}

// Wait until at most N LDS/scalar-memory operations are outstanding and make
// the values depend on the wait. LDS operations complete in issue order, so
// every LDS read issued more than N LDS operations ago has landed.
template <int N, typename T>
__device__ __forceinline__ void lgkm_wait_tied(T& a, T& b) {
  static_assert(N >= 0 && N <= 15, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "n"(N) : "memory");
}
template <int N, typename T>
__device__ __forceinline__ void lgkm_wait_tied1(T& a) {
  static_assert(N >= 0 && N <= 15, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(a) : "n"(N) : "memory");
}
template <int N, typename A, typename B>
__device__ __forceinline__ void lgkm_wait6(A& a0, A& a1, B& b0, B& b1, B& b2, B& b3) {
  static_assert(N >= 0 && N <= 15, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%6)" : "+v"(a0), "+v"(a1), "+v"(b0), "+v"(b1), "+v"(b2), "+v"(b3) : "n"(N) : "memory");
}
template <int N, typename A, typename B>
__device__ __forceinline__ void lgkm_wait4(A& a0, A& a1, B& b0, B& b1) {
  static_assert(N >= 0 && N <= 15, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(a0), "+v"(a1), "+v"(b0), "+v"(b1) : "n"(N) : "memory");
}
template <int N, typename A, typename B>
__device__ __forceinline__ void lgkm_wait3(A& a0, B& b0, B& b1) {
  static_assert(N >= 0 && N <= 15, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%3)" : "+v"(a0), "+v"(b0), "+v"(b1) : "n"(N) : "memory");
}

// Reductions over the lanes l, l ^ 16 and l ^ 32 with the gfx950 permlane
// swaps (plain VALU ops; a shuffle would be an LDS round trip).
__device__ __forceinline__ float max_x16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_x32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_x16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_x32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Maximum of a non-negative int over the 64 lanes of the wave (uniform result).
__device__ __forceinline__ int wave_max_nonneg(int x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x = max(x, __shfl_xor(x, m));
  return __builtin_amdgcn_readfirstlane(x);
}

// Workgroup barrier for the tile pipelines: this wave's LDS operations have
// completed, global loads stay in flight. (__syncthreads() also waits for
// every outstanding global load, which would drain the gathers in flight.)
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace sa
