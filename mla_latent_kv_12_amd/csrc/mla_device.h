// Device-side helpers shared by the decode kernels of libmla (gfx950):
// vector types, direct HBM -> LDS copies with counted waits, score-operand
// LDS reads, MFMA wrappers for accumulators kept in ordinary registers,
// cross-lane reductions and the XCD-aware workgroup order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace mla {
namespace kern {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
#define LDS_AS __attribute__((address_space(3)))

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.693147180559945309f;
// The running maximum is only moved (and O rescaled) when a tile's maximum
// exceeds it by more than this (log2 units); exp2 values stay below 2^8.
constexpr float kRescaleSlack = 8.0f;

// Load of data that no kernel of the launch writes (sizes, schedule): through
// the constant address space the compiler may use scalar loads, whose waits
// do not also wait for the vector memory queue.
template <typename T>
__device__ __forceinline__ T ldc(const T* p) {
  return *(const __attribute__((address_space(4))) T*)reinterpret_cast<uintptr_t>(p);
}

__device__ __forceinline__ bf16x8 cvt8_fp8(u32x2 v) {
  bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], 1.0f, false);
  bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], 1.0f, true);
  bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], 1.0f, false);
  bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], 1.0f, true);
  bf16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// op(x[l], x[l ^ 32]) in every lane: the two halves of a query row's tokens.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The O accumulator lives in accumulation registers next to the MFMA unit.
// VALU work on it goes through explicit moves so the register allocator keeps
// it there instead of splitting it into ordinary VGPRs (which do not fit
// beside the 144 registers of query).
__device__ __forceinline__ void acc_scale(f32x16& v, float s) {
#pragma unroll
  for (int i = 0; i < 16; i++) {
    float t;
    asm("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
        : "+a"(v[i]), "=&v"(t)
        : "v"(s));
  }
}
__device__ __forceinline__ float acc_get(const f32x16& v, int i) {
  float t;
  asm("v_accvgpr_read_b32 %0, %1" : "=v"(t) : "a"(v[i]));
  return t;
}
// Workgroup i is dispatched to XCD i % 8; give each XCD a contiguous range
// of logical workgroups so neighbours (which share sequences and their
// query rows) share an L2.
__device__ __forceinline__ int xcd_logical(int i, int G) {
  int q = G >> 3, r = G & 7, x = i & 7, k = i >> 3;
  return x * q + min(x, r) + k;
}

// ---------------------------------------------------------------------------
// Direct HBM -> LDS copies, written as inline assembly: the kernel counts
// them itself (s_waitcnt vmcnt with the exact number of younger copies), so
// the compiler must neither wait for them on its own nor move them across
// the explicit waits.  M0 holds the LDS destination (every active lane
// writes M0 + size*lane); it is an input operand, so the compiler sets it
// and knows the assembly leaves it unchanged.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>(p);
}
// 16 bytes per lane from a wave-uniform base plus a per-lane byte offset.
__device__ __forceinline__ void copy16_s(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile(
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(base), "{m0}"(lds));
}
// 16 bytes per lane through a raw buffer resource (stride 0): a lane whose
// offset is at or past the resource's size reads zeros (the hardware range
// check), so rows past a sequence's end need no address of their own.
__device__ __forceinline__ void copy16_b(i32x4 rsrc, uint32_t voff, uint32_t lds) {
  asm volatile(
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, 0 offen lds"
      :
      : "v"(voff), "s"(rsrc), "{m0}"(lds));
}
// The same with a wave-uniform byte offset added to every lane's (the range
// check applies to the sum).
__device__ __forceinline__ void copy16_bs(i32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile(
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, %2 offen lds"
      :
      : "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds));
}
// Raw buffer resource over `bytes` bytes from `base` (gfx9 word 3: untyped
// 32-bit data, no swizzle); every word is wave-uniform.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(b >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;
  return r;
}
// 16 bytes per lane from a per-lane address.
__device__ __forceinline__ void copy16_v(const void* addr, uint32_t lds) {
  asm volatile(
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(addr), "{m0}"(lds));
}
// 4 bytes per lane from a per-lane address.
__device__ __forceinline__ void copy4_v(const void* addr, uint32_t lds) {
  asm volatile(
      "s_nop 0\n\t"
      "global_load_lds_dword %0, off"
      :
      : "v"(addr), "{m0}"(lds));
}
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// Score-operand LDS reads issued from assembly with explicit counted waits:
// left to itself the compiler keeps only one or two of them in flight, and
// each MFMA then waits out a full LDS round trip.
template <int OFF>
__device__ __forceinline__ void lds_rd16(bf16x8& dst, uint32_t addr) {
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(dst) : "v"(addr), "n"(OFF));
}
template <int OFF>
__device__ __forceinline__ void lds_rd8(u32x2& dst, uint32_t addr) {
  asm volatile("ds_read_b64 %0, %1 offset:%2" : "=v"(dst) : "v"(addr), "n"(OFF));
}
// Wait until at most N LDS operations are outstanding; `v` (the register
// the caller is about to use) is tied to the wait so its use cannot move
// above it.
template <int N, typename V>
__device__ __forceinline__ void lds_ready(V& v) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(v) : "n"(N));
}
// Score MFMAs with the accumulator in ordinary registers (the accumulation
// registers all hold O).  Back-to-back MFMAs accumulating into exactly the
// same registers need no wait states; the first of a chain starts from 0;
// mfma_settle() supplies the wait states a VALU read of the result needs
// after the last one (more than the 8-pass 32x32x16 MFMA requires).
__device__ __forceinline__ void mfma_first(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_acc(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_settle(f32x16& acc) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(acc));
}
// The same for two registers about to be used.
template <int N, typename V>
__device__ __forceinline__ void lds_ready2(V& v, V& w) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(v), "+v"(w) : "n"(N));
}
template <typename F, int... I>
__device__ __forceinline__ void unroll_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
// f(std::integral_constant<int, i>) for i = 0 .. N-1, in order.
template <int N, typename F>
__device__ __forceinline__ void unroll(F&& f) {
  unroll_impl(f, std::make_integer_sequence<int, N>{});
}

}  // namespace kern
}  // namespace mla
