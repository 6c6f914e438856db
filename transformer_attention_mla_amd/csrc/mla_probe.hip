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

}  // namespace

hipError_t launch_mfma_probe(float* out, int iters, int kind, hipStream_t stream) {
  if (kind == 1)
    hipLaunchKernelGGL(mfma_probe_fp8_kernel, dim3(kProbeBlocks), dim3(kProbeThreads), 0, stream, out, iters);
  else
    hipLaunchKernelGGL(mfma_probe_kernel, dim3(kProbeBlocks), dim3(kProbeThreads), 0, stream, out, iters);
  return hipGetLastError();
}

}  // namespace mla
