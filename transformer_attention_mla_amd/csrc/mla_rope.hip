// Rotary prologue of the prefill: cos/sin of the angle table and the rotated
// shared rotary key.
//
// Page "Kimi K2 · Mix and project", code excerpt "mla-prefill": cos and sin
// come from the rotary embedding and rotate q_pe and k_pe; the key's rotated
// part is a single tensor shared by every head.  Page "Kimi K2 · Transformer
// blocks", I/O header: the angles arrive as R [T positions, 32 pairs].
//
// One thread per (t, pair): sincosf (the accurate, range-reduced libm routine,
// not the hardware approximation: angles reach 1.6e4 radians) gives the
// float32 (cos, sin) table that the prefill kernel uses to rotate q_pe in
// registers, then the thread rotates pair i of k_pe at position t for every
// sequence b and stores it as bf16 (round to nearest even).  Rotating the
// shared key once here, instead of once per key tile in each attention block,
// removes (heads - 1)/heads of that work and keeps the attention loop free of
// it.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

__global__ __launch_bounds__(256) void rope_prep_kernel(const float* __restrict__ R,
                                                        const uint16_t* __restrict__ k_pe,
                                                        float2* __restrict__ cs,
                                                        uint16_t* __restrict__ kpe_rot, int B,
                                                        int T) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= T * kPairs) return;
  const int t = idx / kPairs;
  const int i = idx % kPairs;
  float s, c;
  sincosf(R[idx], &s, &c);
  cs[idx] = make_float2(c, s);
  for (int b = 0; b < B; ++b) {
    const size_t row = ((size_t)b * T + t) * kRope;
    const float lo = bf16_to_f32(k_pe[row + i]);
    const float hi = bf16_to_f32(k_pe[row + i + kPairs]);
    const float ylo = fmaf(lo, c, -(hi * s));
    const float yhi = fmaf(hi, c, lo * s);
    kpe_rot[row + i] = __builtin_bit_cast(uint16_t, f32_to_bf16(ylo));
    kpe_rot[row + i + kPairs] = __builtin_bit_cast(uint16_t, f32_to_bf16(yhi));
  }
}

hipError_t launch_rope_prep(const PrefillParams& p, hipStream_t stream) {
  const int n = p.T * kPairs;
  const int threads = 256;
  const int blocks = (n + threads - 1) / threads;
  hipLaunchKernelGGL(rope_prep_kernel, dim3(blocks), dim3(threads), 0, stream, p.R, p.k_pe, p.cs,
                     p.kpe_rot, p.B, p.T);
  return hipGetLastError();
}

}  // namespace mla
