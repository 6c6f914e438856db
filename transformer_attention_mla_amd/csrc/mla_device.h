// Device helpers for the gfx950 kernels: vector types, bf16 packing, MFMA and
// cross-lane wrappers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// bf16 bit pattern -> float (exact).
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16, round to nearest even (gfx950: v_cvt_pk_bf16_f32).
__device__ __forceinline__ __bf16 f32_to_bf16(float x) { return (__bf16)x; }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ u32x4 ld_global_16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x2 ld_global_8(const void* p) {
  return *reinterpret_cast<const u32x2*>(p);
}

// A 16-byte load of data read once per call (a cache or weight stream), with
// the non-temporal policy so the stream does not displace reusable lines.
__device__ __forceinline__ u32x4 ld_stream_16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// a / s rounded as the e4m3 quantizer needs it, from y = 1/s (correctly
// rounded, computed once per block): q = a*y, the residual a - q*s exact by
// FMA, one correction q + r*y (Markstein's iteration).  For every block scale
// s = max(amax, 1e-4)/448 and every bf16 value |a| <= amax this equals the
// correctly rounded a / s bit for bit wherever |a/s| > 2^-11, and elsewhere has
// its sign and magnitude <= 2^-10 -- both round to the same e4m3 code (checked
// exhaustively on the host over all bf16 amax and a).  An exact quotient (r = 0,
// a = +-0 included) is returned as q, which keeps the sign of zero.
__device__ __forceinline__ float div_by_scale(float a, float s, float y) {
  const float q = __fmul_rn(a, y);
  const float r = __fmaf_rn(-q, s, a);
  return r == 0.0f ? q : __fmaf_rn(r, y, q);
}

// gfx950 transposing LDS read (ds_read_b64_tr_b16), per 16-lane group: each
// lane addresses 8 bytes (four 16-bit elements); lane i receives element i%4
// of the pieces that lanes i/4, i/4+4, i/4+8 and i/4+12 address, in that order.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ s16x4 ds_read_tr(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
}
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 v) { return __builtin_bit_cast(u32x4, v); }

// D = A(32x16) * B(16x32) + C, bf16 inputs, fp32 accumulate.
// Lane l supplies row (l % 32) of A and column (l % 32) of B, k-elements
// (l / 32) * 8 .. +7; it receives column (l % 32) of D, rows
// (r / 4) * 8 + (l / 32) * 4 + (r % 4) in register r.
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D = A(16x32) * B(32x16) + C.  Lane l supplies row (l % 16) of A and column
// (l % 16) of B, k-elements (l / 16) * 8 .. +7; it receives column (l % 16),
// rows (l / 16) * 4 + r in register r.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Combine the values of lanes l and l ^ 32 (v_permlane32_swap exchanges one
// half-wave of the first register with the other half-wave of the second; with
// both registers holding x, the two results hold x[l] and x[l ^ 32] in some
// order, so a commutative operation on them gives the same value in both lanes).
__device__ __forceinline__ float max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ------------------------------------------------------------------------
// Asynchronous buffer -> LDS copies (gfx950).

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// One wave-instruction copying 64 x 16 B from a buffer into LDS at
// lds_wave_base + 16 * lane.  Written as inline assembly so that the compiler
// does not treat it as a store that may alias every later LDS read (it would
// then wait for all outstanding copies before each read); completion is
// ordered explicitly with vmcnt waits before the barriers instead.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint8_t* lds_wave_base, uint32_t voff) {
  const uint32_t lds = (uint32_t)(uintptr_t)(lds_ptr_t)lds_wave_base;
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(lds), "v"(voff), "s"(r)
      : "memory", "m0");
}

// dma16 with the non-temporal policy, for bytes read once per call.
__device__ __forceinline__ void dma16_stream(__amdgpu_buffer_rsrc_t r, uint8_t* lds_wave_base, uint32_t voff) {
  const uint32_t lds = (uint32_t)(uintptr_t)(lds_ptr_t)lds_wave_base;
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen nt lds"
      :
      : "s"(lds), "v"(voff), "s"(r)
      : "memory", "m0");
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// The waitcnt and barrier builtins touch no memory as far as the compiler is
// concerned, so it may move loads and stores across them; the empty asm
// statements with a memory clobber pin every memory access of the wave to its
// side of the wait (compiler ordering only: no instruction is emitted).
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// s_waitcnt vmcnt(n) (lgkmcnt and expcnt untouched); n is a compile-time constant.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  compiler_fence();
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
  compiler_fence();
}

// Workgroup barrier without the implicit full memory fence of __syncthreads:
// LDS reads of this wave are complete (lgkmcnt(0)); outstanding copies are
// accounted for explicitly by the caller.
__device__ __forceinline__ void barrier_lds() {
  compiler_fence();
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  compiler_fence();
}

}  // namespace mla
