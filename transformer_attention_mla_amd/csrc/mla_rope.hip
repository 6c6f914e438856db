// Rotary prologue of the prefill: cos/sin of the angle table and the rotated
// shared rotary key; the same kernel writes the rotated key of a new chunk
// into the cache (position ids start after the cached tokens: page "Kimi K2 ·
// Transformer blocks", model-body excerpt), next to a plain row copy for the
// chunk's nope keys and values.
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

__global__ __launch_bounds__(256) void rope_prep_kernel(const float* __restrict__ R, int r_off,
                                                        const uint16_t* __restrict__ k_pe,
                                                        float2* __restrict__ cs,
                                                        uint16_t* __restrict__ dst, int dst_rows,
                                                        int dst_off, int B, int T) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= T * kPairs) return;
  const int t = idx / kPairs;
  const int i = idx % kPairs;
  float s, c;
  sincosf(R[(size_t)r_off * kPairs + idx], &s, &c);
  if (cs) cs[idx] = make_float2(c, s);
  if (!k_pe) return;
  for (int b = 0; b < B; ++b) {
    const size_t row = ((size_t)b * T + t) * kRope;
    const size_t out = ((size_t)b * dst_rows + dst_off + t) * kRope;
    const float lo = bf16_to_f32(k_pe[row + i]);
    const float hi = bf16_to_f32(k_pe[row + i + kPairs]);
    const float ylo = fmaf(lo, c, -(hi * s));
    const float yhi = fmaf(hi, c, lo * s);
    dst[out + i] = __builtin_bit_cast(uint16_t, f32_to_bf16(ylo));
    dst[out + i + kPairs] = __builtin_bit_cast(uint16_t, f32_to_bf16(yhi));
  }
}

// Cache append of 256-byte rows: 16 threads per row, one 16-byte piece each.
__global__ __launch_bounds__(256) void append_rows_kernel(const uint16_t* __restrict__ src,
                                                          uint16_t* __restrict__ dst, int T,
                                                          int dst_rows, int dst_off, long n) {
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  const long row = idx >> 4;  // (bh, t)
  const int piece = (int)(idx & 15);
  const long bh = row / T;
  const int t = (int)(row % T);
  const u32x4 v = ld_global_16(src + row * 128 + piece * 8);
  *reinterpret_cast<u32x4*>(dst + (bh * dst_rows + dst_off + t) * 128 + piece * 8) = v;
}

hipError_t launch_rope(const float* R, int r_off, const uint16_t* k_pe, float2* cs, uint16_t* dst,
                       int dst_rows, int dst_off, int B, int T, hipStream_t stream) {
  const int n = T * kPairs;
  const int threads = 256;
  const int blocks = (n + threads - 1) / threads;
  hipLaunchKernelGGL(rope_prep_kernel, dim3(blocks), dim3(threads), 0, stream, R, r_off, k_pe, cs,
                     dst, dst_rows, dst_off, B, T);
  return hipGetLastError();
}

hipError_t launch_rope_prep(const PrefillParams& p, hipStream_t stream) {
  return launch_rope(p.R, p.past, p.k_pe, p.cs, p.kpe_rot, p.LK, 0, p.B, p.T, stream);
}

// The last key tile of key-blocked V per head, its slots of positions T..
// zeroed (the caller's padding may hold any bits): 8 KiB per (b, h), one
// 16-byte piece (8 positions of one feature) per thread.
__global__ __launch_bounds__(512) void v_tail_kernel(const uint16_t* __restrict__ v,
                                                     uint16_t* __restrict__ tail, int T) {
  const int bh = blockIdx.x, u = threadIdx.x;  // u = blk*256 + d*2 + half
  const int NB = (T + 15) >> 4;
  const int gb = 2 * ((T - 1) / 32) + (u >> 8);  // global block
  const int key = gb * 16 + (u & 1) * 8;
  u32x4 x = {0, 0, 0, 0};
  if (gb < NB) x = *reinterpret_cast<const u32x4*>(v + ((size_t)bh * NB + gb) * 2048 + (u & 255) * 8);
#pragma unroll
  for (int e = 0; e < 4; ++e)
    x[e] &= (key + 2 * e < T ? 0xffffu : 0u) | (key + 2 * e + 1 < T ? 0xffff0000u : 0u);
  *reinterpret_cast<u32x4*>(tail + (size_t)bh * kVTileElems + u * 8) = x;
}

hipError_t launch_v_tail(const PrefillParams& p, hipStream_t stream) {
  const long blocks = (long)p.B * p.H;
  if (!p.v_blocked || !p.v_tail || p.T % 16 == 0 || blocks > 0x7fffffffL)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(v_tail_kernel, dim3((unsigned)blocks), dim3(512), 0, stream, p.v, p.v_tail, p.T);
  return hipGetLastError();
}

hipError_t launch_append_rows(const uint16_t* src, uint16_t* dst, int BH, int T, int dst_rows,
                              int dst_off, hipStream_t stream) {
  const long n = (long)BH * T * 16;
  const long blocks = (n + 255) / 256;
  if (blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(append_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, src, dst, T,
                     dst_rows, dst_off, n);
  return hipGetLastError();
}

}  // namespace mla
