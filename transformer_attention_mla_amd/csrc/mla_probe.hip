// Matrix-core rate probe: back-to-back MFMA instructions on register operands,
// every compute unit busy (two workgroups of four waves each, so two waves per
// SIMD), four independent accumulator chains per wave, no memory traffic
// inside the loop.  It measures what the matrix cores of this GPU sustain
// under full load (clock and power limits included) for the two instruction
// kinds the path uses -- v_mfma_f32_32x32x16_bf16 and the e4m3 form of
// v_mfma_f32_32x32x64_f8f6f4 -- the figures beside which the kernels' rates
// are read; it computes nothing the attention path uses.
#include "mla_device.h"
#include "mla_probe.h"

namespace mla {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(kProbeThreads) void mfma_probe_kernel(float* __restrict__ out, int iters) {
  const int tid = threadIdx.x;
  // Operands depend on the thread id and the iteration count, so the compiler
  // can neither fold the products nor hoist them out of the loop.
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = f32_to_bf16(1.0f + 0x1p-7f * (float)((5 * tid + 3 * e) & 127));
    b[e] = f32_to_bf16(0x1p-20f * (float)((iters + e + 3 * tid) & 3));
  }
  f32x16 acc[kProbeChains] = {};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c) acc[c] = mfma32x32x16(a, b, acc[c]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[(size_t)blockIdx.x * kProbeThreads + tid] = s;
}

// e4m3 operands (0x38 = 1.0, 0x30 = 0.5): every 4-byte group of a lane's A
// operand is (a, a, a, 0) with a set by the lane's parity, of its B operand
// (0, b, b, b) with b set by the parity of iters; A and B bytes at the same
// position meet the same k, so each group adds 2ab.
__global__ __launch_bounds__(kProbeThreads) void mfma_probe_fp8_kernel(float* __restrict__ out, int iters) {
  const int tid = threadIdx.x;
  const uint32_t aw = (uint32_t)((tid & 1) ? 0x30 : 0x38) * 0x00010101u;    // a a a 0
  const uint32_t bw = (uint32_t)((iters & 1) ? 0x30 : 0x38) * 0x01010100u;  // 0 b b b
  i32x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (int)aw;
    b[e] = (int)bw;
  }
  f32x16 acc[kProbeChains] = {};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[c], 0, 0, 0, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[(size_t)blockIdx.x * kProbeThreads + tid] = s;
}

// Kinds 2 and 3: the same loop with operands that change from one instruction
// to the next -- eight random operand sets per lane, cycled (chain c at step v
// takes A set (v + c) mod 8 and B set (v + 3c) mod 8) -- so the matrix cores
// switch bits as they do on real data.  The data-dependent switching power
// lowers the clock the chip holds under load: this is the rate to read a
// kernel on random inputs against.  Sets come from xorshift32 (shifts 13, 17,
// 5) seeded with 0x9e3779b9 * (thread + 1) xor iters, two draws per element
// (A then B): bf16 A = ±(1 + (h & 0xffff) 2^-16), B = ±(0.5 + (h & 0xffff)
// 2^-17), the sign bit 16 of the draw, rounded to nearest even; e4m3 bytes
// (sign bit 7 of the draw) | (5 + (h >> 3) % 5) << 3 | (h & 7), i.e. normal
// values of magnitude 1/4 .. 4.
__device__ __forceinline__ uint32_t xorshift32(uint32_t h) {
  h ^= h << 13;
  h ^= h >> 17;
  h ^= h << 5;
  return h;
}

__global__ __launch_bounds__(kProbeThreads) void mfma_probe_rand_kernel(float* __restrict__ out, int iters) {
  const int tid = threadIdx.x;
  bf16x8 a[8], b[8];
  uint32_t h = (0x9e3779b9u * (uint32_t)(tid + 1)) ^ (uint32_t)iters;
#pragma unroll
  for (int v = 0; v < 8; ++v)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      h = xorshift32(h);
      const float fa = (1.0f + (float)(h & 0xffff) * 0x1p-16f) * (((h >> 16) & 1) ? -1.f : 1.f);
      h = xorshift32(h);
      const float fb = (0.5f + (float)(h & 0xffff) * 0x1p-17f) * (((h >> 16) & 1) ? -1.f : 1.f);
      a[v][e] = f32_to_bf16(fa);
      b[v][e] = f32_to_bf16(fb);
    }
  f32x16 acc[kProbeChains] = {};
  for (int i = 0; i < iters; i += 8) {
#pragma unroll
    for (int v = 0; v < 8; ++v)
#pragma unroll
      for (int c = 0; c < kProbeChains; ++c)
        acc[c] = mfma32x32x16(a[(v + c) & 7], b[(v + 3 * c) & 7], acc[c]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[(size_t)blockIdx.x * kProbeThreads + tid] = s;
}

__global__ __launch_bounds__(kProbeThreads) void mfma_probe_fp8_rand_kernel(float* __restrict__ out, int iters) {
  const int tid = threadIdx.x;
  i32x8 a[8], b[8];
  uint32_t h = (0x9e3779b9u * (uint32_t)(tid + 1)) ^ (uint32_t)iters;
#pragma unroll
  for (int v = 0; v < 8; ++v)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t wa = 0, wb = 0;
#pragma unroll
      for (int byte = 0; byte < 4; ++byte) {
        h = xorshift32(h);
        wa |= (((h >> 7) & 0x80u) | ((5u + (h >> 3) % 5u) << 3) | (h & 7u)) << (8 * byte);
        h = xorshift32(h);
        wb |= (((h >> 7) & 0x80u) | ((5u + (h >> 3) % 5u) << 3) | (h & 7u)) << (8 * byte);
      }
      a[v][e] = (int)wa;
      b[v][e] = (int)wb;
    }
  f32x16 acc[kProbeChains] = {};
  for (int i = 0; i < iters; i += 8) {
#pragma unroll
    for (int v = 0; v < 8; ++v)
#pragma unroll
      for (int c = 0; c < kProbeChains; ++c)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[(v + c) & 7], b[(v + 3 * c) & 7], acc[c],
                                                                 0, 0, 0, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[(size_t)blockIdx.x * kProbeThreads + tid] = s;
}

}  // namespace

hipError_t launch_mfma_probe(float* out, int iters, int kind, hipStream_t stream) {
  const dim3 g(kProbeBlocks), t(kProbeThreads);
  switch (kind) {
    case 0: hipLaunchKernelGGL(mfma_probe_kernel, g, t, 0, stream, out, iters); break;
    case 1: hipLaunchKernelGGL(mfma_probe_fp8_kernel, g, t, 0, stream, out, iters); break;
    case 2: hipLaunchKernelGGL(mfma_probe_rand_kernel, g, t, 0, stream, out, iters); break;
    case 3: hipLaunchKernelGGL(mfma_probe_fp8_rand_kernel, g, t, 0, stream, out, iters); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mla
