// Output projection o_proj for gfx950: y[M][N] = x[M][K] · w[N][K]ᵀ, bf16
// inputs, float32 accumulation, no bias.
//
// Page "Kimi K2 · Mix and project": parameter table (8,192 × 7,168 output
// projection), explanation (no earlier step combines heads) and code excerpt
// "mla-output" (o_proj applied to the head-major [B, T, 64·128] output);
// page "Block input", config.json: attention_bias false.
//
// Design: both operands are K-contiguous (the linear layer's weight is stored
// one row per output feature), so each MFMA operand fragment is one 16-byte
// LDS read.  The kernel computes the transposed tile Yᵀ = W·Xᵀ with
// v_mfma_f32_32x32x16_bf16 so that each lane ends with 4 consecutive output
// features of one row (one 8- or 16-byte store).  Tiles of 128 (n) × 128 (m)
// (× 64 when M <= 64) per workgroup of 4 waves; k is staged 64 at a time
// through registers into XOR-swizzled LDS, the next slab's global loads being
// issued before the current slab is multiplied.  For small M the K range is split over
// workgroups (float32 partials in the caller's workspace, then a reduction
// kernel) so the weight stream is spread over every compute unit.
//
// Large M (enough 256 x 256 tiles to fill the chip) takes a second kernel:
// 256 (n) × 256 (m) tiles per workgroup of 8 waves, k staged 64 at a time in
// two LDS stages filled by asynchronous buffer→LDS copies (details at the
// kernel).  Tiles are handed to
// the XCDs (workgroup ids are dealt round-robin over the 8 XCDs) as
// contiguous runs of a grouped order — a few m-tiles against every n-tile —
// so the workgroups resident on one XCD share x rows and weight rows through
// that XCD's L2, and all XCDs sweep the weight in step.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int OBN = 128;  // rows of w (output features) per tile
constexpr int OBM = 128;  // rows of x per tile (64 when M <= 64: no idle half tile)
constexpr int OBK = 64;   // k per LDS slab (128 for the FP8 weight at M <= 64)
constexpr int OWN = 2;    // waves along n
constexpr int OWM = 2;    // waves along m
constexpr int ONT = 64 * OWN * OWM;
constexpr int OTN = OBN / OWN / 32;  // 32x32 blocks per wave along n

// Chunk swizzle for 128-byte LDS rows (8 chunks of 16 B): distinct for any 8
// consecutive rows and for same-parity rows among 16 consecutive ones.
__device__ __forceinline__ int rswz(int row) { return (row ^ (row >> 3)) & 7; }
// The same for 256-byte rows (16 chunks): distinct for any 16 consecutive rows.
__device__ __forceinline__ int rswz16(int row) { return (row ^ (row >> 4)) & 15; }

// FP8 weights (e4m3, OCP "fn" variant, as the checkpoint stores them with one
// float32 scale per 128 x 128 block): 8 values, the float32 product with the
// block scale rounded to bf16 -- the bf16 weight the projection multiplies.
__device__ __forceinline__ u32x4 dequant8(u32x2 raw, float s) {
  u32x4 r;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int w = (int)(uint32_t)raw[h];
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);  // bytes 0, 1
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);   // bytes 2, 3
    r[2 * h] = pack_bf16x2(lo[0] * s, lo[1] * s);
    r[2 * h + 1] = pack_bf16x2(hi[0] * s, hi[1] * s);
  }
  return r;
}

// Output features n .. n+3 (n a multiple of 4) of row m, unless they are past
// N: row-major y [M][N] in float32 or bf16.
__device__ __forceinline__ void store_y4(const OprojParams& p, int m, int n, float v0, float v1,
                                         float v2, float v3) {
  const int N = p.N;
  if (p.out_f32) {
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

// Head-major split store.  Row m = b*T + t maps to split_row(m) = b*H*T + t;
// a block of 32 output features from nb (a multiple of 32; hd, d0 and N are
// multiples of 32, so the block lies in one part of one head) to split_col.
struct SplitCol {
  void* base;       // y or y1
  size_t head_off;  // h*T rows
  int width, d;     // the part's row width and the block's first feature in it
  int h;            // head
  bool blk;         // the key-blocked second part
};
__device__ __forceinline__ size_t split_row(const OprojParams& p, int m) {
  const int b = m / p.T;
  return (size_t)b * (p.N / p.hd) * p.T + (m - b * p.T);
}
__device__ __forceinline__ SplitCol split_col(const OprojParams& p, int nb) {
  const int h = nb / p.hd, d = nb - h * p.hd;
  const bool first = d < p.d0;
  return SplitCol{first ? p.y : p.y1, (size_t)h * p.T, first ? p.d0 : p.hd - p.d0,
                  first ? d : d - p.d0, h, !first && p.y1_blocked};
}
// Element offset of feature d of head h, row m = b*T + t, in the key-blocked part.
__device__ __forceinline__ size_t blocked_off(const OprojParams& p, int m, int h, int d) {
  const int b = m / p.T, t = m - b * p.T;
  const int H = p.N / p.hd, NB = (p.T + 15) >> 4, w = p.hd - p.d0;
  return ((size_t)(b * H + h) * NB + (t >> 4)) * (16 * w) + d * 16 + (t & 15);
}
// Features c.d + dn .. +3 of the block for row m (at split_row r).
__device__ __forceinline__ void store_split4(const OprojParams& p, const SplitCol& c, size_t r, int m,
                                             int dn, float v0, float v1, float v2, float v3) {
  if (c.blk) {
    const float v[4] = {v0, v1, v2, v3};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const size_t off = blocked_off(p, m, c.h, c.d + dn + e);
      if (p.out_f32)
        static_cast<float*>(c.base)[off] = v[e];
      else
        static_cast<__bf16*>(c.base)[off] = f32_to_bf16(v[e]);
    }
    return;
  }
  const size_t off = (r + c.head_off) * c.width + c.d + dn;
  if (p.out_f32)
    *reinterpret_cast<f32x4*>(static_cast<float*>(c.base) + off) = f32x4{v0, v1, v2, v3};
  else
    *reinterpret_cast<u32x2*>(static_cast<__bf16*>(c.base) + off) =
        u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
}

template <bool FP8, int BM, int BK>
__global__ __launch_bounds__(ONT) void oproj_kernel(OprojParams p) {
  constexpr int OTM = BM / OWM / 32;  // 32x32 blocks per wave along m
  constexpr int CH = BK / 8;          // 16-byte chunks per LDS row
  static_assert(OTM >= 1 && BM % (OWM * 32) == 0, "x tile");
  static_assert(CH == 8 || CH == 16, "slab depth");
  auto swz = [](int row) { return CH == 16 ? rswz16(row) : rswz(row); };
  __shared__ __attribute__((aligned(16))) uint16_t sW[OBN * BK];
  __shared__ __attribute__((aligned(16))) uint16_t sX[BM * BK];

  const int M = p.M, N = p.N, K = p.K;
  const int tiles_n = (N + OBN - 1) / OBN;
  const int tile = blockIdx.x;
  const int split = blockIdx.y;
  const int tn = tile % tiles_n;
  const int tm = tile / tiles_n;
  const int n0 = tn * OBN, m0 = tm * BM;
  const int kslabs = K / BK / p.splits;
  const int kbeg = split * kslabs * BK;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int ln = lane & 31, hf = lane >> 5;
  const int wn = wave % OWN, wm = wave / OWN;

  constexpr int WCH = OBN * CH / ONT;  // 16-byte chunks per thread per slab
  constexpr int XCH = BM * CH / ONT;
  u32x4 rw[WCH], rx[XCH];
  u32x2 rw8[FP8 ? WCH : 1];
  float rs[FP8 ? WCH : 1];
  const int KB = (K + 127) / 128;

  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      const int c = tid + i * ONT;
      const int row = c / CH, ch = c % CH;
      const int n = min(n0 + row, N - 1);
      if constexpr (FP8) {
        rw8[i] = ld_global_8(p.w8 + (size_t)n * K + k0 + ch * 8);
        rs[i] = p.w_scale[(n >> 7) * KB + ((k0 + ch * 8) >> 7)];
      } else {
        rw[i] = ld_global_16(p.w + (size_t)n * K + k0 + ch * 8);
      }
    }
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int c = tid + i * ONT;
      const int row = c / CH, ch = c % CH;
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
      const int row = c / CH, ch = c % CH;
      if constexpr (FP8) rw[i] = dequant8(rw8[i], rs[i]);
      *reinterpret_cast<u32x4*>(sW + row * BK + ((ch ^ swz(row)) * 8)) = rw[i];
    }
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int c = tid + i * ONT;
      const int row = c / CH, ch = c % CH;
      *reinterpret_cast<u32x4*>(sX + row * BK + ((ch ^ swz(row)) * 8)) = rx[i];
    }
    __syncthreads();
    if (ks + 1 < kslabs) load(kbeg + (ks + 1) * BK);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 a[OTN], bb[OTM];
#pragma unroll
      for (int i = 0; i < OTN; ++i) {
        const int row = wn * (OTN * 32) + i * 32 + ln;
        a[i] = *reinterpret_cast<const bf16x8*>(sW + row * BK + (((kk * 2 + hf) ^ swz(row)) * 8));
      }
#pragma unroll
      for (int jm = 0; jm < OTM; ++jm) {
        const int row = wm * (OTM * 32) + jm * 32 + ln;
        bb[jm] = *reinterpret_cast<const bf16x8*>(sX + row * BK + (((kk * 2 + hf) ^ swz(row)) * 8));
      }
#pragma unroll
      for (int i = 0; i < OTN; ++i)
#pragma unroll
        for (int jm = 0; jm < OTM; ++jm) acc[i][jm] = mfma32x32x16(a[i], bb[jm], acc[i][jm]);
    }
  }

  // ---- epilogue: lane holds y[m][n..n+3] for m = m-block + ln
  if (p.hd > 0) {
#pragma unroll
    for (int jm = 0; jm < OTM; ++jm) {
      const int m = m0 + wm * (OTM * 32) + jm * 32 + ln;
      if (m >= M) continue;
      const size_t r = split_row(p, m);
#pragma unroll
      for (int i = 0; i < OTN; ++i) {
        const int nb = n0 + wn * (OTN * 32) + i * 32;
        if (nb >= N) continue;
        const SplitCol c = split_col(p, nb);
#pragma unroll
        for (int gq = 0; gq < 4; ++gq)
          store_split4(p, c, r, m, gq * 8 + hf * 4, acc[i][jm][gq * 4 + 0], acc[i][jm][gq * 4 + 1],
                       acc[i][jm][gq * 4 + 2], acc[i][jm][gq * 4 + 3]);
      }
    }
    return;
  }
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
        } else {
          store_y4(p, m, n, v0, v1, v2, v3);
        }
      }
  }
}

// ---------------------------------------------------------------- wide tiles --
// 256 (n) × 256 (m) tiles per workgroup of 8 waves (two per SIMD; wave w
// computes n rows 128(w%2).. and m rows 64(w/2).. of the tile).  k is staged
// 64 at a time: 128-byte LDS rows, so every 8 lanes of a copy fetch one whole
// 128-byte line, in two LDS stages of 64 KiB.  Each slab is multiplied in two
// 32-k halves so the fragment reads of one half overlap the MFMAs of the
// other; the copy of slab kt+2 is issued as soon as every wave has read slab
// kt.  The buffer→LDS copy rate per CU, not the MFMA rate, bounds this kernel
// (a copy-only run of it takes about 80% of its time).
constexpr int WBN = 256;  // w rows (n) per tile
constexpr int WBM = 256;  // x rows (m) per tile
constexpr int WBK = 64;   // k per slab
constexpr int WNW = 8;    // waves: 2 along n × 4 along m
constexpr int WNT = 64 * WNW;
constexpr int WTN = WBN / 2 / 32;          // 32-row w blocks per wave (4)
constexpr int WTM = WBM / (WNW / 2) / 32;  // 32-row x blocks per wave (2)
constexpr int WGROUP_M = 4;                // m-tiles per group of the tile order
constexpr int WPART = WBN * WBK * 2;       // 32 KiB: one operand's slab
constexpr int WSTAGE_B = 2 * WPART;        // 64 KiB per stage
constexpr int WCPW = WSTAGE_B / 1024 / WNW;  // copies (1 KiB = 8 rows) per wave per slab
static_assert(WBN == WBM, "one copy plan for both operands");
static_assert(2 * WSTAGE_B <= 160 * 1024, "LDS budget");

// Slot of 16-byte chunk c (of 8) in 128-byte row r: c ^ wswz(r).  Any 8
// consecutive rows read at one chunk hit 8 distinct slots mod 128 B, any 16
// (from a multiple of 16) 16 distinct slots mod 256 B; depends on r mod 32 only.
__device__ __forceinline__ int wswz(int row) { return (row & 7) ^ ((row >> 3) & 3); }

__shared__ __attribute__((aligned(1024))) uint8_t wlds[2 * WSTAGE_B];

__global__ __launch_bounds__(WNT) void oproj_wide_kernel(OprojParams p) {
  const int M = p.M, N = p.N, K = p.K;
  const int tiles_n = (N + WBN - 1) / WBN;
  const int tiles_m = (M + WBM - 1) / WBM;
  const int ntiles = tiles_m * tiles_n;

  const int b = blockIdx.x;
  const int xcd = b & 7, seq = b >> 3;
  const int t = xcd * (ntiles >> 3) + min(xcd, ntiles & 7) + seq;
  const int gm = p.group_m;
  const int group = t / (gm * tiles_n);
  const int first_m = group * gm;
  const int rows_m = min(gm, tiles_m - first_m);
  const int within = t - group * gm * tiles_n;
  const int tm = first_m + within % rows_m;
  const int tn = within / rows_m;
  const int n0 = tn * WBN, m0 = tm * WBM;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 31, hf = lane >> 5;
  const int wn = wave & 1, wm = wave >> 1;

  // Copy plan: wave w copies 1 KiB chunks j = w + WNW i (8 rows each); chunks
  // 0..31 are w rows, 32..63 x rows.  Lane l writes bytes 16l.. of its chunk:
  // row 8(j%32) + l/8, slot l%8, which holds source chunk slot ^ wswz(row).
  uint32_t voff[WCPW];
#pragma unroll
  for (int i = 0; i < WCPW; ++i) {
    const int j = wave + WNW * i;
    const int row = (j & 31) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ wswz(row);
    voff[i] = (uint32_t)row * (uint32_t)K * 2u + (uint32_t)c * 16u;
  }
  const uint16_t* wbase = p.w + (size_t)n0 * K;
  const uint16_t* xbase = p.x + (size_t)m0 * K;
  const size_t wbytes = (size_t)(N - n0) * K * 2;
  const size_t xbytes = (size_t)(M - m0) * K * 2;
  const int nk = K / WBK;

  auto issue = [&](int stage, int kt) {
    const int k0 = kt * WBK;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(wbase + k0, (uint32_t)min(wbytes - (size_t)k0 * 2, (size_t)0x7fffffff));
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(xbase + k0, (uint32_t)min(xbytes - (size_t)k0 * 2, (size_t)0x7fffffff));
    uint8_t* sb = wlds + stage * WSTAGE_B;
#pragma unroll
    for (int i = 0; i < WCPW; ++i)  // i < WCPW/2: w rows
      dma16(i < WCPW / 2 ? rw : rx, sb + (wave + WNW * i) * 1024, voff[i]);
  };

  // Fragment of k16 step kk (0..3) for row ln of a 32-row block: chunk 2kk + hf.
  const int swz = wswz(ln);
  int foff[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) foff[kk] = ln * 128 + ((2 * kk + hf) ^ swz) * 16;

  struct Frags {
    bf16x8 a[WTN][2], bx[WTM][2];
  };
  auto load_frags = [&](Frags& f, int stage, int half) {
    const uint8_t* sw = wlds + stage * WSTAGE_B + wn * (WTN * 32) * 128;
    const uint8_t* sx = wlds + stage * WSTAGE_B + WPART + wm * (WTM * 32) * 128;
    const int o0 = half ? foff[2] : foff[0];
    const int o1 = half ? foff[3] : foff[1];
#pragma unroll
    for (int i = 0; i < WTN; ++i) {
      f.a[i][0] = *reinterpret_cast<const bf16x8*>(sw + i * 32 * 128 + o0);
      f.a[i][1] = *reinterpret_cast<const bf16x8*>(sw + i * 32 * 128 + o1);
    }
#pragma unroll
    for (int jm = 0; jm < WTM; ++jm) {
      f.bx[jm][0] = *reinterpret_cast<const bf16x8*>(sx + jm * 32 * 128 + o0);
      f.bx[jm][1] = *reinterpret_cast<const bf16x8*>(sx + jm * 32 * 128 + o1);
    }
  };
  f32x16 acc[WTN][WTM] = {};
  auto mma = [&](const Frags& f) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int i = 0; i < WTN; ++i)
#pragma unroll
        for (int jm = 0; jm < WTM; ++jm) acc[i][jm] = mfma32x32x16(f.a[i][kk], f.bx[jm][kk], acc[i][jm]);
  };

  issue(0, 0);
  issue(1, 1);  // nk >= 2 (K % 128 == 0)
  wait_vm<WCPW>();
  barrier_lds();
  Frags f0, f1;
  load_frags(f0, 0, 0);
  // Slab kt (stage kt & 1), first half's fragments in f0:
  //   read the second half (f1), multiply the first;
  //   wait for slab kt+1 (its copies are the only ones in flight), barrier:
  //   slab kt+1 visible, and every wave has read all of slab kt;
  //   refill slab kt's stage with slab kt+2; read slab kt+1's first half
  //   (f0); multiply slab kt's second half.
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    load_frags(f1, st, 1);
    __builtin_amdgcn_sched_barrier(0);
    mma(f0);
    if (kt + 1 < nk) {
      wait_vm<0>();  // slab kt+1's copies are the only ones in flight
      barrier_lds();
      if (kt + 2 < nk) issue(st, kt + 2);
      load_frags(f0, st ^ 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    mma(f1);
  }

  // bf16 output: the tile goes through LDS (both stages are free now, 256
  // rows x 512 B = 128 KiB), so that each global store writes whole 128-byte
  // lines of a row -- a lane's own results are 8-byte pieces of 32 different
  // rows, which the memory system absorbs far more slowly (the stores then
  // cost a fifth of the time at K = 1536 and almost half at K = 512).
  // Row r keeps its 16-byte chunk c at c ^ (r % 32).
  if (!p.out_f32 && (p.hd > 0 || (N & 7) == 0)) {
    barrier_lds();  // every wave has read its last fragments
#pragma unroll
    for (int jm = 0; jm < WTM; ++jm) {
      const int r = wm * (WTM * 32) + jm * 32 + ln;
#pragma unroll
      for (int i = 0; i < WTN; ++i)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int c = wn * (WTN * 4) + i * 4 + gq;
          *reinterpret_cast<u32x2*>(wlds + r * 512 + ((c ^ (r & 31)) * 16) + hf * 8) =
              u32x2{pack_bf16x2(acc[i][jm][gq * 4 + 0], acc[i][jm][gq * 4 + 1]),
                    pack_bf16x2(acc[i][jm][gq * 4 + 2], acc[i][jm][gq * 4 + 3])};
        }
    }
    barrier_lds();
    if (p.y1_blocked) {
      // The tile is one head (hd = 256, d0 = 128): chunks 0..15 are its first
      // part, stored as row pieces, four rows per wave instruction; the second
      // part goes key-blocked, each wave instruction writing one 16-row block
      // of 32 features (1 KiB), a lane's 8 rows of one feature gathered by
      // two transposing LDS reads (lane i of a 16-lane group receives element
      // i%4 of the 8-byte pieces that lanes i/4, i/4+4, i/4+8, i/4+12 address).
      const int h = n0 / p.hd;
      {
        const int c = lane & 15;
        const SplitCol sc = split_col(p, n0 + (c >> 2) * 32);
#pragma unroll 4
        for (int rr = 0; rr < WBM / (4 * WNW); ++rr) {
          const int r = (rr * WNW + wave) * 4 + (lane >> 4);
          const int m = m0 + r;
          if (m >= M) continue;
          const u32x4 v = *reinterpret_cast<const u32x4*>(wlds + r * 512 + ((c ^ (r & 31)) * 16));
          const size_t off = (split_row(p, m) + sc.head_off) * sc.width + sc.d + (c & 3) * 8;
          *reinterpret_cast<u32x4*>(static_cast<__bf16*>(sc.base) + off) = v;
        }
      }
      uint16_t* y1 = static_cast<uint16_t*>(p.y1);
      if ((p.T & 15) == 0) {  // every 16-row block lies in one sequence (M % 16 == 0 too)
        const int g = lane >> 4, i = lane & 15, half = g >> 1, q = i & 3;
        const int H = N / p.hd, NB = p.T >> 4;
#pragma unroll 2
        for (int it = 0; it < (WBM / 16) * 4 / WNW; ++it) {
          const int w = it * WNW + wave;
          const int j = w >> 2, fg = w & 3;  // 16-row block, 32-feature group
          const int m = m0 + j * 16;
          if (m >= M) continue;
          const int b = m / p.T, t = m - b * p.T;
          // as a source, lane (g, i) addresses features 16(g&1) + 4q .. +3 of the
          // group in row i/4 (+4) of the block's half `half`
          const int cc = 16 + fg * 4 + 2 * (g & 1) + (q >> 1);
          const int rA = j * 16 + half * 8 + (i >> 2), rB = rA + 4;
          const s16x4 lo = ds_read_tr(wlds + rA * 512 + ((cc ^ (rA & 31)) * 16) + (q & 1) * 8);
          const s16x4 hi = ds_read_tr(wlds + rB * 512 + ((cc ^ (rB & 31)) * 16) + (q & 1) * 8);
          const int d = fg * 32 + 16 * (g & 1) + i;  // received: feature d, rows half*8 .. +7
          *reinterpret_cast<u32x4*>(y1 + ((size_t)(b * H + h) * NB + (t >> 4)) * 2048 + d * 16 + half * 8) =
              __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
      } else {  // a 16-row block may span two sequences: element stores
        const int c = 16 + (lane & 15);
        for (int rr = 0; rr < WBM / (4 * WNW); ++rr) {
          const int r = (rr * WNW + wave) * 4 + (lane >> 4);
          const int m = m0 + r;
          if (m >= M) continue;
          const u32x4 v = *reinterpret_cast<const u32x4*>(wlds + r * 512 + ((c ^ (r & 31)) * 16));
#pragma unroll
          for (int e = 0; e < 8; ++e)
            y1[blocked_off(p, m, h, (c - 16) * 8 + e)] = (uint16_t)(v[e >> 1] >> ((e & 1) * 16));
        }
      }
      return;
    }
    const int c = lane & 31;  // chunk: columns n0 + 8c .. +7
    const int n = n0 + c * 8;
    SplitCol sc;
    if (p.hd > 0 && n < N) sc = split_col(p, n0 + (c >> 2) * 32);
#pragma unroll 4
    for (int rr = 0; rr < WBM / (2 * WNW); ++rr) {
      const int r = (rr * WNW + wave) * 2 + (lane >> 5);
      const int m = m0 + r;
      if (m >= M || n >= N) continue;
      const u32x4 v = *reinterpret_cast<const u32x4*>(wlds + r * 512 + ((c ^ (r & 31)) * 16));
      if (p.hd > 0) {
        const size_t off = (split_row(p, m) + sc.head_off) * sc.width + sc.d + (c & 3) * 8;
        *reinterpret_cast<u32x4*>(static_cast<__bf16*>(sc.base) + off) = v;
      } else {
        *reinterpret_cast<u32x4*>(static_cast<__bf16*>(p.y) + (size_t)m * N + n) = v;
      }
    }
    return;
  }
  if (p.hd > 0) {
#pragma unroll
    for (int jm = 0; jm < WTM; ++jm) {
      const int m = m0 + wm * (WTM * 32) + jm * 32 + ln;
      if (m >= M) continue;
      const size_t r = split_row(p, m);
#pragma unroll
      for (int i = 0; i < WTN; ++i) {
        const int nb = n0 + wn * (WTN * 32) + i * 32;
        if (nb >= N) continue;
        const SplitCol c = split_col(p, nb);
#pragma unroll
        for (int gq = 0; gq < 4; ++gq)
          store_split4(p, c, r, m, gq * 8 + hf * 4, acc[i][jm][gq * 4 + 0], acc[i][jm][gq * 4 + 1],
                       acc[i][jm][gq * 4 + 2], acc[i][jm][gq * 4 + 3]);
      }
    }
    return;
  }
#pragma unroll
  for (int jm = 0; jm < WTM; ++jm) {
    const int m = m0 + wm * (WTM * 32) + jm * 32 + ln;
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < WTN; ++i)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int n = n0 + wn * (WTN * 32) + i * 32 + gq * 8 + hf * 4;
        const float v0 = acc[i][jm][gq * 4 + 0], v1 = acc[i][jm][gq * 4 + 1];
        const float v2 = acc[i][jm][gq * 4 + 2], v3 = acc[i][jm][gq * 4 + 3];
        store_y4(p, m, n, v0, v1, v2, v3);
      }
  }
}

// y = sum over splits of the float32 partials, in split order.
// Sum of the split-K partials, in split order: four consecutive outputs per
// thread with 16-byte loads (all splits' loads issued before the sums) when
// M*N is a multiple of 4, one per thread otherwise.
__global__ __launch_bounds__(256) void oproj_reduce_kernel(OprojParams p) {
  const size_t total = (size_t)p.M * p.N;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  if ((total & 3) == 0) {
    const f32x4* part = reinterpret_cast<const f32x4*>(p.part);
    const size_t total4 = total >> 2;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total4; i += stride) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      int s = 0;
      for (; s + 4 <= p.splits; s += 4) {
        f32x4 v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = part[(size_t)(s + j) * total4 + i];
#pragma unroll
        for (int j = 0; j < 4; ++j) acc += v[j];
      }
      for (; s < p.splits; ++s) acc += part[(size_t)s * total4 + i];
      if (p.out_f32) {
        reinterpret_cast<f32x4*>(p.y)[i] = acc;
      } else {
        reinterpret_cast<u32x2*>(p.y)[i] = u32x2{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
      }
    }
    return;
  }
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    float acc = 0.f;
    for (int s = 0; s < p.splits; ++s) acc += p.part[(size_t)s * total + i];
    if (p.out_f32)
      static_cast<float*>(p.y)[i] = acc;
    else
      static_cast<__bf16*>(p.y)[i] = f32_to_bf16(acc);
  }
}

// FP8 weight -> bf16 weight (the same arithmetic as dequant8 in the load
// path of the small-tile kernel), 8 values per thread: used at large M, where
// the weight is dequantized once into the workspace and the wide bf16 kernel
// (which copies raw bytes into LDS and cannot dequantize) does the product.
__global__ __launch_bounds__(256) void dequant_fp8_kernel(const uint8_t* __restrict__ w8,
                                                          const float* __restrict__ w_scale,
                                                          uint16_t* __restrict__ w, int N, int K) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;  // 8-value group
  if (i >= (long)N * K / 8) return;
  const long e = i * 8;
  const int n = (int)(e / K), k = (int)(e - (long)n * K);
  const float sc = w_scale[(size_t)(n >> 7) * ((K + 127) / 128) + (k >> 7)];
  *reinterpret_cast<u32x4*>(w + e) = dequant8(ld_global_8(w8 + e), sc);
}

// ------------------------------------------------------ FP8 activations --
// Page "Block input", config.json quantization_config: e4m3 with the
// activation scheme "dynamic".  One 128-column block per 16 lanes (8 values
// per lane): block maximum by a 16-lane butterfly, scale = max(amax, 1e-4) /
// 448 and codes e4m3(x / scale), the quotients those of correctly rounded
// float32 divisions (one division per block for the reciprocal, then
// div_by_scale per value) and v_cvt_pk_fp8_f32 rounding to nearest even.  The scales are stored
// transposed, [K/128][M], so that one slab's scales for a tile of rows are
// contiguous (the GEMM copies them into LDS with its tiles), row stride
// act_scale_stride(M).
__global__ __launch_bounds__(256) void act_quant_kernel(const uint16_t* __restrict__ x,
                                                        uint8_t* __restrict__ x8,
                                                        float* __restrict__ sxT, int M, int K) {
  const int KB = K / 128;
  const long g = (long)blockIdx.x * 256 + threadIdx.x;
  const long blk = g >> 4;  // (m, kb): the 16 lanes of a group share it
  const int sub = (int)(g & 15);
  if (blk >= (long)M * KB) return;
  const int m = (int)(blk / KB), kb = (int)(blk - (long)m * KB);
  const size_t off = (size_t)m * K + (size_t)kb * 128 + sub * 8;
  const u32x4 raw = ld_global_16(x + off);
  float v[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = bf16lo(raw[e]);
    v[2 * e + 1] = bf16hi(raw[e]);
  }
  float a = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(v[e]));
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) a = fmaxf(a, __shfl_xor(a, o, 16));
  a = fmaxf(a, 1e-4f);
  const float sc = a / 448.0f;
  const float ry = 1.0f / sc;
  u32x2 q;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    int w = 0;
    w = __builtin_amdgcn_cvt_pk_fp8_f32(div_by_scale(v[4 * h], sc, ry), div_by_scale(v[4 * h + 1], sc, ry),
                                        w, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(div_by_scale(v[4 * h + 2], sc, ry),
                                        div_by_scale(v[4 * h + 3], sc, ry), w, true);
    q[h] = (uint32_t)w;
  }
  *reinterpret_cast<u32x2*>(x8 + off) = q;
  if (sub == 0) sxT[(size_t)kb * act_scale_stride(M) + m] = sc;
}

// ------------------------------------------------------------ FP8 x FP8 --
// Yᵀ = W8·X8ᵀ with v_mfma_f32_32x32x64_f8f6f4 (both operands e4m3).  A k slab
// is 128 deep -- one 128-byte LDS row per operand row, the same copy plan as
// the wide bf16 kernel (8 lanes fetch one whole line; chunk slots swizzled by
// wswz) -- plus the slab's activation scales (1 KiB chunk).  Each 32x32 tile's
// slab product (two MFMAs) goes to a float32 temporary and is added to the
// accumulator times w_scale[block of n][slab] · x_scale[m][slab]: the two
// block scales change with every 128-deep slab, so the sum over k is taken
// slab by slab in float32 (the order the format implies).  A wave computes
// WTN x WTM tiles of 32x32; the workgroup WN x WM waves; NSTG LDS stages,
// the copies of slab kt+NSTG-1 issued once every wave has finished slab kt-1.
// Both MFMA operands take their 32 bytes per lane of a 64-deep k step from
// the same byte range of the row, so A and B agree on which k each operand
// slot holds.
template <int WN, int WM, int WTN, int WTM, int NSTG>
__global__ __launch_bounds__(64 * WN * WM) void oproj_fp8_kernel(OprojParams p) {
  typedef int i32x8 __attribute__((ext_vector_type(8)));
  constexpr int NWAVE = WN * WM;
  constexpr int BN = WN * WTN * 32, BM = WM * WTM * 32;
  constexpr int APART = BN * 128, BPART = BM * 128;
  constexpr int SXOFF = APART + BPART;
  constexpr int STG = SXOFF + 1024;         // + activation scales (BM floats, padded)
  constexpr int NCH = STG / 1024;           // 1 KiB copies per slab
  constexpr int CPW = (NCH + NWAVE - 1) / NWAVE;
  static_assert(BM <= 256, "one 1 KiB chunk of activation scales per slab");
  static_assert(WTN * 32 <= 128 && 128 % (WTN * 32) == 0, "a wave's rows lie in one 128-row weight block");
  static_assert(NSTG * STG <= 160 * 1024, "LDS budget");
  static_assert((NSTG - 1) * CPW < 64, "vmcnt range");
  constexpr int NBLK = BN / 128;   // 128-row weight blocks of a tile
  constexpr int MAXS = 256;        // slabs per split (launch checks)
  __shared__ __attribute__((aligned(1024))) uint8_t fl[NSTG * STG];
  __shared__ float wsl[NBLK * MAXS];  // the tile's weight scales, [block][slab]

  const int M = p.M, N = p.N, K = p.K, KB = K / 128;
  const int tiles_n = (N + BN - 1) / BN;
  const int tiles_m = (M + BM - 1) / BM;
  const int ntiles = tiles_m * tiles_n;
  // grouped tile order dealt to the XCDs as in the wide kernel
  const int bid = blockIdx.x;
  const int xcd = bid & 7, seq = bid >> 3;
  const int t = xcd * (ntiles >> 3) + min(xcd, ntiles & 7) + seq;
  const int gm = p.group_m;
  const int group = t / (gm * tiles_n);
  const int first_m = group * gm;
  const int rows_m = min(gm, tiles_m - first_m);
  const int within = t - group * gm * tiles_n;
  const int tm = first_m + within % rows_m;
  const int tn = within / rows_m;
  const int n0 = tn * BN, m0 = tm * BM;
  const int nks = KB / p.splits;  // slabs of this split
  const int kb0 = blockIdx.y * nks;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 31, hf = lane >> 5;
  const int wn = wave % WN, wm = wave / WN;

  // Copy plan: chunk j < APART/1024 holds weight rows 8j..8j+7, then x rows,
  // then the scales; lane l writes bytes 16l.. of its chunk: row 8j' + l/8,
  // slot l%8, which holds source chunk slot ^ wswz(row).  Copy i of a wave is
  // chunk wave + NWAVE*i, so with both operand parts a whole number of
  // NWAVE-chunk rounds its kind (weight, x or scales) depends on i alone and
  // is known at compile time.  Copies past the last chunk repeat the scale
  // chunk (identical bytes).
  static_assert((APART / 1024) % NWAVE == 0 && (BPART / 1024) % NWAVE == 0, "copy rounds");
  auto kind_of = [](int i) { return NWAVE * i < APART / 1024 ? 0 : (NWAVE * i < SXOFF / 1024 ? 1 : 2); };
  uint32_t voff[CPW];
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int j = wave + NWAVE * i;
    if (kind_of(i) == 0) {
      const int row = j * 8 + (lane >> 3);
      voff[i] = (uint32_t)row * (uint32_t)K + (uint32_t)(((lane & 7) ^ wswz(row)) * 16);
    } else if (kind_of(i) == 1) {
      const int row = (j - APART / 1024) * 8 + (lane >> 3);
      voff[i] = (uint32_t)row * (uint32_t)K + (uint32_t)(((lane & 7) ^ wswz(row)) * 16);
    } else {
      voff[i] = (uint32_t)lane * 16u;  // scales of rows m0 + 4 lane ..
    }
  }
  const size_t wbytes = (size_t)(N - n0) * K;
  const size_t xbytes = (size_t)(M - m0) * K;
  // scale rows copied: rounded up to 4 so that no 16-byte copy straddles the
  // extent (the row stride of the transposed scales is M rounded up to 4)
  const int srows = (min(BM, M - m0) + 3) & ~3;

  auto issue = [&](int stage, int ks) {
    const int kb = kb0 + ks;
    const size_t k0 = (size_t)kb * 128;
    // extents clamped to 31 bits: a tile's rows lie within 256 K < 2^31 bytes
    const __amdgpu_buffer_rsrc_t rw =
        make_rsrc(p.w8 + (size_t)n0 * K + k0, (uint32_t)min(wbytes - k0, (size_t)0x7fffffff));
    const __amdgpu_buffer_rsrc_t rx =
        make_rsrc(p.x8 + (size_t)m0 * K + k0, (uint32_t)min(xbytes - k0, (size_t)0x7fffffff));
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(p.x_scaleT + (size_t)kb * act_scale_stride(M) + m0, (uint32_t)srows * 4u);
    uint8_t* sb = fl + stage * STG;
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int j = min(wave + NWAVE * i, NCH - 1);
      dma16(kind_of(i) == 0 ? rw : (kind_of(i) == 1 ? rx : rs), sb + j * 1024, voff[i]);
    }
  };

  // Fragment (32 bytes) of k step kk for LDS row `row`: chunks 4kk+2hf, +1.
  auto frag = [&](const uint8_t* part, int row, int kk) {
    const int sw = wswz(row);
    const uint8_t* r = part + row * 128;
    const u32x4 lo = *reinterpret_cast<const u32x4*>(r + (((4 * kk + 2 * hf) ^ sw) * 16));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(r + (((4 * kk + 2 * hf + 1) ^ sw) * 16));
    return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  f32x16 acc[WTN][WTM] = {};
  // The tile's weight scales go to LDS before any copy is issued (a vector
  // load inside the loop would make the compiler wait for the copies too).
  // Rows past N use the last block, whose products are zero and never stored.
  const int NB = (N + 127) >> 7;
  for (int i = tid; i < NBLK * nks; i += 64 * NWAVE) {
    const int blk = min((n0 >> 7) + i / nks, NB - 1);
    wsl[i] = p.w_scale[(size_t)blk * KB + kb0 + i % nks];
  }
  const int wblk = (wn * WTN * 32) >> 7;  // this wave's rows lie in one block

#pragma unroll
  for (int s = 0; s < NSTG - 1; ++s)
    if (s < nks) issue(s, s);
  // Tile t = i*WTM + jm of a slab: its two MFMAs go to tq[t&1]; the scale
  // FMAs of tile t-1 are issued while the matrix core computes tile t (one
  // temporary would serialize every tile on the MFMA result latency).  The
  // last tile's FMAs wait for the next slab, where they cover the latency of
  // its first fragment reads.
  constexpr int TL = WTN * WTM - 1;
  f32x16 tq[2];
  float scp = 0.f;  // scale of the last tile of the previous slab
  for (int ks = 0; ks < nks; ++ks) {
    // this wave's copies of slab ks are done (those of ks+1 .. ks+NSTG-2 may
    // not be; fewer are in flight near the end); after the barrier every
    // wave's are, and every wave has finished slab ks-1, whose stage the next
    // copies refill
    if (ks + NSTG - 2 < nks)
      wait_vm<(NSTG - 2) * CPW>();
    else
      wait_vm<0>();
    barrier_lds();
    if (ks + NSTG - 1 < nks) issue((ks + NSTG - 1) % NSTG, ks + NSTG - 1);
    const uint8_t* sb = fl + (ks % NSTG) * STG;
    const float swv = wsl[wblk * nks + ks];  // (visible: the barrier above)
    i32x8 bfr[WTM][2];
    float sc[WTM];
#pragma unroll
    for (int jm = 0; jm < WTM; ++jm) {
      const int row = wm * (WTM * 32) + jm * 32 + ln;
      bfr[jm][0] = frag(sb + APART, row, 0);
      bfr[jm][1] = frag(sb + APART, row, 1);
      sc[jm] = swv * *reinterpret_cast<const float*>(sb + SXOFF + row * 4);
    }
    if (ks > 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        acc[TL / WTM][TL % WTM][r] = fmaf(tq[TL & 1][r], scp, acc[TL / WTM][TL % WTM][r]);
    }
#pragma unroll
    for (int i = 0; i < WTN; ++i) {
      const int row = wn * (WTN * 32) + i * 32 + ln;
      const i32x8 a0 = frag(sb, row, 0), a1 = frag(sb, row, 1);
#pragma unroll
      for (int jm = 0; jm < WTM; ++jm) {
        const int t = i * WTM + jm;
        tq[t & 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, bfr[jm][0], f32x16{}, 0, 0, 0, 0, 0, 0);
        tq[t & 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, bfr[jm][1], tq[t & 1], 0, 0, 0, 0, 0, 0);
        if (t > 0) {
          const int pi = (t - 1) / WTM, pj = (t - 1) % WTM;
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[pi][pj][r] = fmaf(tq[(t - 1) & 1][r], sc[pj], acc[pi][pj][r]);
        }
      }
    }
    scp = sc[TL % WTM];
  }
  if (nks > 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      acc[TL / WTM][TL % WTM][r] = fmaf(tq[TL & 1][r], scp, acc[TL / WTM][TL % WTM][r]);
  }

  // bf16 output of the 256 x 256 tile: staged through the free LDS stages
  // and stored as whole lines, as in the wide bf16 kernel.
  if constexpr (BN == 256 && BM * BN * 2 <= NSTG * STG) {
    if (p.splits == 1 && !p.out_f32 && (N & 7) == 0) {
      barrier_lds();  // every wave has read its last fragments
#pragma unroll
      for (int jm = 0; jm < WTM; ++jm) {
        const int r = wm * (WTM * 32) + jm * 32 + ln;
#pragma unroll
        for (int i = 0; i < WTN; ++i)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const int c = wn * (WTN * 4) + i * 4 + gq;
            *reinterpret_cast<u32x2*>(fl + r * 512 + ((c ^ (r & 31)) * 16) + hf * 8) =
                u32x2{pack_bf16x2(acc[i][jm][gq * 4 + 0], acc[i][jm][gq * 4 + 1]),
                      pack_bf16x2(acc[i][jm][gq * 4 + 2], acc[i][jm][gq * 4 + 3])};
          }
      }
      barrier_lds();
      const int c = lane & 31;
      const int n = n0 + c * 8;
#pragma unroll 4
      for (int rr = 0; rr < BM / (2 * NWAVE); ++rr) {
        const int r = (rr * NWAVE + wave) * 2 + (lane >> 5);
        const int m = m0 + r;
        if (m >= M || n >= N) continue;
        *reinterpret_cast<u32x4*>(static_cast<__bf16*>(p.y) + (size_t)m * N + n) =
            *reinterpret_cast<const u32x4*>(fl + r * 512 + ((c ^ (r & 31)) * 16));
      }
      return;
    }
  }

#pragma unroll
  for (int jm = 0; jm < WTM; ++jm) {
    const int m = m0 + wm * (WTM * 32) + jm * 32 + ln;
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < WTN; ++i)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int n = n0 + wn * (WTN * 32) + i * 32 + gq * 8 + hf * 4;
        const float v0 = acc[i][jm][gq * 4 + 0], v1 = acc[i][jm][gq * 4 + 1];
        const float v2 = acc[i][jm][gq * 4 + 2], v3 = acc[i][jm][gq * 4 + 3];
        if (p.splits > 1) {
          float* dst = p.part + ((size_t)blockIdx.y * M + m) * N + n;
          if (n + 3 < N && (N & 3) == 0) {
            *reinterpret_cast<f32x4*>(dst) = f32x4{v0, v1, v2, v3};
          } else {
            if (n < N) dst[0] = v0;
            if (n + 1 < N) dst[1] = v1;
            if (n + 2 < N) dst[2] = v2;
            if (n + 3 < N) dst[3] = v3;
          }
        } else {
          store_y4(p, m, n, v0, v1, v2, v3);
        }
      }
  }
}

}  // namespace

// The wide kernel needs enough 256 x 256 tiles to fill the chip, and 32-bit
// buffer offsets for 256 rows of x or w.
static bool oproj_use_wide(int M, int K, int N) {
  const long wide_tiles = (long)((M + WBM - 1) / WBM) * ((N + WBN - 1) / WBN);
  return wide_tiles >= 256 && (long long)K * 2 * WBM < 0x7fffffffLL;
}

// k per LDS slab of the small-tile kernel: 128 for the FP8 weight at M <= 64
// (16 KiB of weight per slab, as for the bf16 weight at 64; 29 us against 33
// us at M = 64, K = 8192, N = 7168), 64 otherwise (at M = 16384 the deeper
// slab measured 2.49 ms against 2.35).
static int oproj_slab_k(int M, bool fp8) { return fp8 && M <= 64 ? 2 * OBK : OBK; }

int oproj_choose_splits(int M, int K, int N, bool fp8) {
  if (!fp8 && oproj_use_wide(M, K, N)) return 1;
  const long tiles = (long)((M + OBM - 1) / OBM) * ((N + OBN - 1) / OBN);
  const int slabs = K / oproj_slab_k(M, fp8);
  if (tiles >= 256 || slabs <= 1) return 1;
  // Spread the weight stream over the chip: aim for >= 256 workgroups (at
  // M = 64, N = 7168, K = 8192: 8 splits, 448 workgroups, 33 us against
  // 48 us for 16 splits, whose float32 partials cost more than they spread),
  // keep >= 4 slabs per split, and split K into equal whole slabs.
  int best = 1;
  for (int s = 2; s <= slabs / 4; ++s) {
    if (slabs % s) continue;
    best = s;
    if (tiles * s >= 256) break;
  }
  return best;
}

static unsigned reduce_blocks(const OprojParams& p) {
  const size_t total = (size_t)p.M * p.N;
  const size_t items = (total & 3) == 0 ? total >> 2 : total;
  size_t blocks = (items + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  return (unsigned)blocks;
}

hipError_t launch_oproj(const OprojParams& p_in, hipStream_t stream) {
  OprojParams p = p_in;
  if (p.hd > 0 && (p.splits != 1 || p.w8 || p.T <= 0 || p.M % p.T != 0 || p.N % p.hd != 0 ||
                   p.hd % 32 != 0 || p.d0 % 32 != 0 || p.d0 <= 0 || p.d0 >= p.hd || !p.y1))
    return hipErrorInvalidConfiguration;
  if (!p.w8 && p.splits == 1 && oproj_use_wide(p.M, p.K, p.N)) {
    if (p.y1_blocked && (p.hd != WBN || p.d0 != WBN / 2)) return hipErrorInvalidConfiguration;
    const long wide_tiles = (long)((p.M + WBM - 1) / WBM) * ((p.N + WBN - 1) / WBN);
    if (wide_tiles > 0x7fffffffL) return hipErrorInvalidConfiguration;
    if (p.group_m <= 0) p.group_m = WGROUP_M;
    hipLaunchKernelGGL(oproj_wide_kernel, dim3((unsigned)wide_tiles), dim3(WNT), 0, stream, p);
    return hipGetLastError();
  }
  const long tiles = (long)((p.M + OBM - 1) / OBM) * ((p.N + OBN - 1) / OBN);
  const int bk = oproj_slab_k(p.M, p.w8 != nullptr);
  if (tiles <= 0 || tiles > 0x7fffffffL || p.splits < 1 || p.splits > 65535 || p.K % (bk * p.splits) != 0)
    return hipErrorInvalidConfiguration;
  // M <= 64 is one m-tile at either height; the 64-row tile loads and
  // multiplies no rows past M.
  const dim3 grid((unsigned)tiles, (unsigned)p.splits);
  const bool m64 = p.M <= 64;
  if (p.w8 && m64)
    hipLaunchKernelGGL((oproj_kernel<true, 64, 2 * OBK>), grid, dim3(ONT), 0, stream, p);
  else if (p.w8)
    hipLaunchKernelGGL((oproj_kernel<true, OBM, OBK>), grid, dim3(ONT), 0, stream, p);
  else if (m64)
    hipLaunchKernelGGL((oproj_kernel<false, 64, OBK>), grid, dim3(ONT), 0, stream, p);
  else
    hipLaunchKernelGGL((oproj_kernel<false, OBM, OBK>), grid, dim3(ONT), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  hipLaunchKernelGGL(oproj_reduce_kernel, dim3(reduce_blocks(p)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

bool oproj_fp8_wide(int M, int K, int N) { return oproj_use_wide(M, K, N) && K % 8 == 0; }

hipError_t launch_dequant_fp8(const uint8_t* w8, const float* w_scale, uint16_t* w, int N, int K,
                              hipStream_t stream) {
  const long groups = (long)N * K / 8;
  const long blocks = (groups + 255) / 256;
  if (K % 8 != 0 || blocks <= 0 || blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(dequant_fp8_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, w8, w_scale, w,
                     N, K);
  return hipGetLastError();
}

hipError_t launch_act_quant(const uint16_t* x, uint8_t* x8, float* x_scaleT, int M, int K,
                            hipStream_t stream) {
  const long threads = (long)M * (K / 128) * 16;
  const long blocks = (threads + 255) / 256;
  if (K % 128 != 0 || blocks <= 0 || blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(act_quant_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, x8, x_scaleT,
                     M, K);
  return hipGetLastError();
}

// Large M: 256 x 256 tiles, 8 waves of 4 x 2 tiles, two stages.  Small M
// (M <= 64): 128 (n) x 64 (m) tiles, 4 waves of 2 x 1 tiles, three stages of
// 25 KiB (two workgroups fit a compute unit), K split into equal whole slabs
// until >= 192 workgroups run.  At M = 64, K = 8192, N = 7168 (56 tiles, 4
// splits) the GEMM takes 15.7 us warm against 16.5 with 8 splits and 22.0 for
// 256 x 64 tiles with 16 splits (448 workgroups of four slabs, one per
// compute unit), and the float32 partials halve.
static bool fp8dyn_small(int M) { return M <= 64; }

int oproj_fp8dyn_splits(int M, int K, int N) {
  if (!fp8dyn_small(M)) return 1;
  const int tiles = (N + 127) / 128;
  const int slabs = K / 128;
  int best = 1;
  for (int s = 2; s <= slabs / 2; ++s) {
    if (slabs % s) continue;
    best = s;
    if (tiles * s >= 3 * kComputeUnits / 4) break;
  }
  return best;
}

hipError_t launch_oproj_fp8dyn(const OprojParams& p_in, hipStream_t stream) {
  OprojParams p = p_in;
  if (!p.w8 || !p.w_scale || !p.x8 || !p.x_scaleT || p.K % 128 != 0 || p.splits < 1 ||
      (p.K / 128) % p.splits != 0 || p.hd > 0)
    return hipErrorInvalidConfiguration;
  if ((long long)p.K * 256 >= 0x7fffffffLL || p.K / 128 / p.splits > 256)
    return hipErrorInvalidConfiguration;
  p.group_m = p.group_m > 0 ? p.group_m : WGROUP_M;
  if (fp8dyn_small(p.M)) {
    const long tiles = (p.N + 127) / 128;
    p.group_m = 1;
    hipLaunchKernelGGL((oproj_fp8_kernel<2, 2, 2, 1, 3>), dim3((unsigned)tiles, (unsigned)p.splits),
                       dim3(256), 0, stream, p);
  } else {
    const long tiles = (long)((p.M + 255) / 256) * ((p.N + 255) / 256);
    if (tiles > 0x7fffffffL || p.splits != 1) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((oproj_fp8_kernel<2, 4, 4, 2, 2>), dim3((unsigned)tiles, 1), dim3(512), 0,
                       stream, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  hipLaunchKernelGGL(oproj_reduce_kernel, dim3(reduce_blocks(p)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
