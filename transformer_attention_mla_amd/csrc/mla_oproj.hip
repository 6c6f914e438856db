// Output projection o_proj for gfx950: y[M][N] = x[M][K] · w[N][K]ᵀ, bf16
// inputs, float32 accumulation, no bias.
//
// Page "Kimi K2 · Mix and project": parameter table (8,192 × 7,168 output
// projection), explanation (the only step that mixes heads) and code excerpt
// "mla-output" (o_proj applied to the head-major [B, T, 64·128] output);
// page "Block input", config.json: attention_bias false.
//
// Design: both operands are K-contiguous (the linear layer's weight is stored
// one row per output feature), so each MFMA operand fragment is one 16-byte
// LDS read.  The kernel computes the transposed tile Yᵀ = W·Xᵀ with
// v_mfma_f32_32x32x16_bf16 so that each lane ends with 4 consecutive output
// features of one row (one 8- or 16-byte store).  Tiles of 128 (n) × 128 (m)
// per workgroup of 4 waves; k is staged 64 at a time through registers into
// XOR-swizzled LDS, the next slab's global loads being issued before the
// current slab is multiplied.  For small M the K range is split over
// workgroups (float32 partials in the caller's workspace, then a reduction
// kernel) so the weight stream is spread over every compute unit.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int OBN = 128;  // rows of w (output features) per tile
constexpr int OBM = 128;  // rows of x per tile
constexpr int OBK = 64;   // k per LDS slab
constexpr int OWN = 2;    // waves along n
constexpr int OWM = 2;    // waves along m
constexpr int ONT = 64 * OWN * OWM;
constexpr int OTN = OBN / OWN / 32;  // 32x32 blocks per wave along n
constexpr int OTM = OBM / OWM / 32;  // along m

// Chunk swizzle for 128-byte LDS rows (8 chunks of 16 B): distinct for any 8
// consecutive rows and for same-parity rows among 16 consecutive ones.
__device__ __forceinline__ int rswz(int row) { return (row ^ (row >> 3)) & 7; }

__global__ __launch_bounds__(ONT) void oproj_kernel(OprojParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t sW[OBN * OBK];
  __shared__ __attribute__((aligned(16))) uint16_t sX[OBM * OBK];

  const int M = p.M, N = p.N, K = p.K;
  const int tiles_n = (N + OBN - 1) / OBN;
  const int tile = blockIdx.x;
  const int split = blockIdx.y;
  const int tn = tile % tiles_n;
  const int tm = tile / tiles_n;
  const int n0 = tn * OBN, m0 = tm * OBM;
  const int kslabs = K / OBK / p.splits;
  const int kbeg = split * kslabs * OBK;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int ln = lane & 31, hf = lane >> 5;
  const int wn = wave % OWN, wm = wave / OWN;

  constexpr int WCH = OBN * 8 / ONT;  // 16-byte chunks per thread per slab
  constexpr int XCH = OBM * 8 / ONT;
  u32x4 rw[WCH], rx[XCH];

  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      const int c = tid + i * ONT;
      const int row = c >> 3, ch = c & 7;
      const int n = min(n0 + row, N - 1);
      rw[i] = ld_global_16(p.w + (size_t)n * K + k0 + ch * 8);
    }
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int c = tid + i * ONT;
      const int row = c >> 3, ch = c & 7;
      const int m = min(m0 + row, M - 1);
      rx[i] = ld_global_16(p.x + (size_t)m * K + k0 + ch * 8);
    }
  };

  f32x16 acc[OTN][OTM] = {};
  load(kbeg);
  for (int ks = 0; ks < kslabs; ++ks) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      const int c = tid + i * ONT;
      const int row = c >> 3, ch = c & 7;
      *reinterpret_cast<u32x4*>(sW + row * OBK + ((ch ^ rswz(row)) * 8)) = rw[i];
    }
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int c = tid + i * ONT;
      const int row = c >> 3, ch = c & 7;
      *reinterpret_cast<u32x4*>(sX + row * OBK + ((ch ^ rswz(row)) * 8)) = rx[i];
    }
    __syncthreads();
    if (ks + 1 < kslabs) load(kbeg + (ks + 1) * OBK);
#pragma unroll
    for (int kk = 0; kk < OBK / 16; ++kk) {
      bf16x8 a[OTN], bb[OTM];
#pragma unroll
      for (int i = 0; i < OTN; ++i) {
        const int row = wn * (OTN * 32) + i * 32 + ln;
        a[i] = *reinterpret_cast<const bf16x8*>(sW + row * OBK + (((kk * 2 + hf) ^ rswz(row)) * 8));
      }
#pragma unroll
      for (int jm = 0; jm < OTM; ++jm) {
        const int row = wm * (OTM * 32) + jm * 32 + ln;
        bb[jm] = *reinterpret_cast<const bf16x8*>(sX + row * OBK + (((kk * 2 + hf) ^ rswz(row)) * 8));
      }
#pragma unroll
      for (int i = 0; i < OTN; ++i)
#pragma unroll
        for (int jm = 0; jm < OTM; ++jm) acc[i][jm] = mfma32x32x16(a[i], bb[jm], acc[i][jm]);
    }
  }

  // ---- epilogue: lane holds y[m][n..n+3] for m = m-block + ln
#pragma unroll
  for (int jm = 0; jm < OTM; ++jm) {
    const int m = m0 + wm * (OTM * 32) + jm * 32 + ln;
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < OTN; ++i)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int n = n0 + wn * (OTN * 32) + i * 32 + gq * 8 + hf * 4;
        const float v0 = acc[i][jm][gq * 4 + 0], v1 = acc[i][jm][gq * 4 + 1];
        const float v2 = acc[i][jm][gq * 4 + 2], v3 = acc[i][jm][gq * 4 + 3];
        if (p.splits > 1) {
          float* dst = p.part + ((size_t)split * M + m) * N + n;
          if (n + 3 < N && (N & 3) == 0) {
            *reinterpret_cast<f32x4*>(dst) = f32x4{v0, v1, v2, v3};
          } else {
            if (n < N) dst[0] = v0;
            if (n + 1 < N) dst[1] = v1;
            if (n + 2 < N) dst[2] = v2;
            if (n + 3 < N) dst[3] = v3;
          }
        } else if (p.out_f32) {
          float* dst = static_cast<float*>(p.y) + (size_t)m * N + n;
          if (n + 3 < N && (N & 3) == 0) {
            *reinterpret_cast<f32x4*>(dst) = f32x4{v0, v1, v2, v3};
          } else {
            if (n < N) dst[0] = v0;
            if (n + 1 < N) dst[1] = v1;
            if (n + 2 < N) dst[2] = v2;
            if (n + 3 < N) dst[3] = v3;
          }
        } else {
          __bf16* dst = static_cast<__bf16*>(p.y) + (size_t)m * N + n;
          if (n + 3 < N && (N & 3) == 0) {
            *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
          } else {
            if (n < N) dst[0] = f32_to_bf16(v0);
            if (n + 1 < N) dst[1] = f32_to_bf16(v1);
            if (n + 2 < N) dst[2] = f32_to_bf16(v2);
            if (n + 3 < N) dst[3] = f32_to_bf16(v3);
          }
        }
      }
  }
}

// y = sum over splits of the float32 partials, in split order.
__global__ __launch_bounds__(256) void oproj_reduce_kernel(OprojParams p) {
  const size_t total = (size_t)p.M * p.N;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    float acc = 0.f;
    for (int s = 0; s < p.splits; ++s) acc += p.part[(size_t)s * total + i];
    if (p.out_f32)
      static_cast<float*>(p.y)[i] = acc;
    else
      static_cast<__bf16*>(p.y)[i] = f32_to_bf16(acc);
  }
}

}  // namespace

int oproj_choose_splits(int M, int K, int N) {
  const long tiles = (long)((M + OBM - 1) / OBM) * ((N + OBN - 1) / OBN);
  const int slabs = K / OBK;
  if (tiles >= 256 || slabs <= 1) return 1;
  // Spread the weight stream over the chip: aim for >= 512 workgroups, keep
  // >= 4 slabs (256 k) per split, and split K into equal whole slabs.
  int best = 1;
  for (int s = 2; s <= slabs / 4; ++s) {
    if (slabs % s) continue;
    best = s;
    if (tiles * s >= 512) break;
  }
  return best;
}

hipError_t launch_oproj(const OprojParams& p, hipStream_t stream) {
  const long tiles = (long)((p.M + OBM - 1) / OBM) * ((p.N + OBN - 1) / OBN);
  if (tiles <= 0 || tiles > 0x7fffffffL || p.splits < 1 || p.splits > 65535)
    return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(oproj_kernel, dim3((unsigned)tiles, (unsigned)p.splits), dim3(ONT), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  const size_t total = (size_t)p.M * p.N;
  size_t blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(oproj_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
