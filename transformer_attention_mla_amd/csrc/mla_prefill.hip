// Causal MLA prefill attention for gfx950 (CDNA4), flash-style.
//
// Page "Kimi K2 · Mix and project", code excerpt "mla-prefill": per head,
// query = [q_nope | rot(q_pe)] and key = [k_nope | rot(k_pe)] (192 wide; the
// key's rotated part is one tensor shared by all heads), scores are
// Q·Kᵀ·softmax_scale plus the causal mask, softmax runs in float32 over keys,
// and the weights mix the 128-wide values.  Excerpt "mla-output": the output
// is stored transposed to [B, T, heads·128], head-major.  Page "Kimi K2 ·
// Transformer blocks": causal mask M [T queries, T keys], positions 0..T-1.
//
// Work decomposition
//   * A workgroup (8 waves) owns 2 heads × 128 queries of one sequence; each
//     wave owns 32 queries of one head.  It processes a pair of query tiles,
//     i and NQ-1-i, one after the other, so every workgroup does the same
//     amount of causal work.  Workgroups of the same (sequence, head pair) are
//     placed on the same XCD and issued together, so that XCD's L2 serves
//     their shared key/value stream.
//   * Per key tile (64 keys) the workgroup stages k_nope of both heads, the
//     rotated shared rotary key (once for both heads) and V of both heads in
//     LDS, with asynchronous buffer→LDS copies into a second buffer while the
//     current tile is multiplied.
//
// Per wave and key tile
//   * Sᵀ = K·Qᵀ with v_mfma_f32_32x32x16_bf16: the key tile is the A operand
//     (LDS), the query the B operand (registers for the whole pass; q_pe is
//     rotated on load).  In the transposed product every lane holds scores of
//     ONE query, so the softmax statistics are per-lane values plus one
//     exchange between half-waves.  192 = 8 k-steps over k_nope + 4 over the
//     shared rotated key.
//   * Key rows are stored in LDS in the order the A lanes read them, chosen so
//     that the Sᵀ accumulator registers are directly the B-operand layout of
//     Pᵀ in Oᵀ += Vᵀ·Pᵀ (no data movement between the two products).
//   * Vᵀ fragments come from V's natural [key][dim] layout with the gfx950
//     transposing LDS read ds_read_b64_tr_b16.
//   * Online softmax in base 2, softmax_scale·log2(e) folded into one FMA.  The
//     reference maximum is only raised when a tile's maximum exceeds it by
//     more than 8 (weights then stay <= 2^8); the result is the same softmax.
//     The row sum is accumulated (v_dot2_f32_bf16 against ones) from the same
//     bf16-rounded weights that enter the PV product.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int G = 2;          // heads per workgroup
constexpr int WPH = 4;        // waves per head
constexpr int NW = G * WPH;   // 8 waves
constexpr int NT = 64 * NW;   // 512 threads
constexpr int BQ = 32 * WPH;  // 128 queries per head per tile
constexpr int BK = 64;        // keys per tile
constexpr float TAU = 8.0f;   // lazy-rescale threshold (log2 units)

// LDS stage layout (bytes)
constexpr int K_ROW = 272;                  // 256 B of k_nope + 16 B pad (17 slots)
constexpr int K_HEAD = BK * K_ROW;          // 17408
constexpr int KP_ROW = 144;                 // 128 B of rotated key + 16 B pad (9 slots)
constexpr int V_ROW = 256;                  // natural layout, 64 B blocks XOR-swizzled
constexpr int V_HEAD = BK * V_ROW;          // 16384
constexpr int KOFF = 0;
constexpr int KPOFF = KOFF + G * K_HEAD;    // 34816
constexpr int VOFF = KPOFF + BK * KP_ROW;   // 44032
constexpr int STAGE = VOFF + G * V_HEAD;    // 76800

// DMA work per stage, in 1 KiB chunks (one wave-instruction of 64 x 16 B each).
constexpr int DK = (BK * 17) / 64;           // 17 per head
constexpr int DKP = (BK * 9) / 64;           // 9
constexpr int DV = (BK * 16) / 64;           // 16 per head

static_assert(BK * 17 % 64 == 0 && BK * 9 % 64 == 0, "slot counts must fill whole wave loads");

// Tile-local key held in LDS row R of a 32-key block: the key that A-operand
// lane R fetches.  Accumulator register r of lane (n, h) is row
// (r/4)*8 + h*4 + r%4; with this order it holds key (r/4 >> 1)*16 + h*8 +
// (r/4 & 1)*4 + r%4, so lane half h owns keys h*8..h*8+7 of every 16-key
// chunk in 8 consecutive registers -- the B-operand layout of the PV product.
__device__ __forceinline__ int akey(int R) {
  const int g4 = R >> 3, h = (R >> 2) & 1, i = R & 3;
  return (g4 >> 1) * 16 + h * 8 + (g4 & 1) * 4 + i;
}

__shared__ __attribute__((aligned(16))) uint8_t lds_a[STAGE];
__shared__ __attribute__((aligned(16))) uint8_t lds_b[STAGE];

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint8_t* lds_wave_base, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds_wave_base, 16, (int)voff, 0, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ s16x4 ds_read_tr(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
}

__global__ __launch_bounds__(NT) void prefill_kernel(PrefillParams p) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int ln = lane & 31;
  const int hf = lane >> 5;

  const int H = p.H, T = p.T;
  const int HG = (H + G - 1) / G;
  const int NQ = (T + BQ - 1) / BQ;
  const int NP = (NQ + 1) / 2;  // query-tile pairs
  const int U = p.B * HG;       // (sequence, head pair) units

  // ---- XCD-aware placement: workgroup P runs on XCD P % 8; give each XCD whole
  // units, and issue a unit's pairs back to back.
  int unit, pair;
  {
    const int P = blockIdx.x;
    if (U % 8 == 0) {
      const int x = P % 8, o = P / 8;
      unit = x + 8 * (o / NP);
      pair = o % NP;
    } else {
      unit = P / NP;
      pair = P % NP;
    }
  }
  const int b = unit / HG;
  const int hg = unit % HG;
  const int g = wave / WPH;
  const int qb = wave % WPH;
  const int head = hg * G + g;
  const bool head_ok = head < H;

  // ---- asynchronous tile copies.  The stage buffer is a sequence of 1 KiB
  // chunks (k_nope head 0 | head 1 | rotated key | V head 0 | head 1); wave w
  // copies chunks w, w+8, ... of each region.  Every lane's byte offset inside
  // its sequence's tensor is fixed up to the tile start, added per tile.  One
  // buffer descriptor per tensor and sequence: rows past the end of the tensor
  // read as zero; rows past T inside it belong to the next head and are masked.
  constexpr int NCK = G * DK, NCKP = DKP, NCV = G * DV;  // 34, 9, 32 chunks
  constexpr int IK = (NCK + NW - 1) / NW, IKP = (NCKP + NW - 1) / NW, IV = (NCV + NW - 1) / NW;
  uint32_t voffK[IK], voffKP[IKP], voffV[IV];
#pragma unroll
  for (int i = 0; i < IK; ++i) {
    const int j = wave + NW * i;
    const int gg = j / DK;
    const int hh = min(hg * G + gg, H - 1);
    const int s = (j % DK) * 64 + lane;
    const int R = s / 17;
    int c = s % 17;
    if (c == 16) c = 15;  // pad slot: harmless duplicate
    voffK[i] = ((uint32_t)hh * (uint32_t)T + (uint32_t)((R >> 5) * 32 + akey(R & 31))) * 256u + c * 16;
  }
#pragma unroll
  for (int i = 0; i < IKP; ++i) {
    const int s = (wave + NW * i) * 64 + lane;
    const int R = s / 9;
    int c = s % 9;
    if (c == 8) c = 7;
    voffKP[i] = (uint32_t)(((R >> 5) * 32 + akey(R & 31)) * 128 + c * 16);
  }
#pragma unroll
  for (int i = 0; i < IV; ++i) {
    const int j = wave + NW * i;
    const int gg = j / DV;
    const int hh = min(hg * G + gg, H - 1);
    const int s = (j % DV) * 64 + lane;
    const int row = s / 16;
    const int c = (s % 16) ^ ((row & 3) << 2);
    voffV[i] = ((uint32_t)hh * (uint32_t)T + (uint32_t)row) * 256u + c * 16;
  }
  const uint32_t seq_bytes = (uint32_t)((size_t)H * T * 256);
  const __amdgpu_buffer_rsrc_t rK = make_rsrc(p.k_nope + (size_t)b * H * T * kNope, seq_bytes);
  const __amdgpu_buffer_rsrc_t rV = make_rsrc(p.v + (size_t)b * H * T * kV, seq_bytes);
  const __amdgpu_buffer_rsrc_t rKP = make_rsrc(p.kpe_rot + (size_t)b * T * kRope, (uint32_t)T * 128u);

  auto issue_tile = [&](uint8_t* buf, int kt) {
    const uint32_t k0 = (uint32_t)(kt * BK);
#pragma unroll
    for (int i = 0; i < IK; ++i) {
      const int j = wave + NW * i;
      if (j < NCK) dma16(rK, buf + KOFF + j * 1024, voffK[i] + k0 * 256u);
    }
#pragma unroll
    for (int i = 0; i < IKP; ++i) {
      const int j = wave + NW * i;
      if (j < NCKP) dma16(rKP, buf + KPOFF + j * 1024, voffKP[i] + k0 * 128u);
    }
#pragma unroll
    for (int i = 0; i < IV; ++i) {
      const int j = wave + NW * i;
      if (j < NCV) dma16(rV, buf + VOFF + j * 1024, voffV[i] + k0 * 256u);
    }
  };

  // Zero both stages once, so rows that a copy leaves unwritten hold finite values.
  for (int o = tid * 16; o < STAGE; o += NT * 16) {
    *reinterpret_cast<u32x4*>(lds_a + o) = u32x4{0, 0, 0, 0};
    *reinterpret_cast<u32x4*>(lds_b + o) = u32x4{0, 0, 0, 0};
  }
  __syncthreads();

  // Per-lane LDS addresses for the products.
  const int k_lane = g * K_HEAD + ln * K_ROW + hf * 16;         // + j*32*K_ROW + kb*32
  const int kp_lane = ln * KP_ROW + hf * 16;                     // + j*32*KP_ROW + kb*32
  const int q16 = lane >> 4, s16 = lane & 15;
  // ds_read_b64_tr_b16: lane s of a 16-lane group addresses key row
  // (q16/2)*8 + t*4 + s/4 of a 16-key chunk, dims (q16%2)*16 + (s%4)*4 .. +3 of a
  // 32-dim block; lane i of the group then receives dim (q16%2)*16 + i of the
  // block for those four keys.
  const int v_row = (q16 >> 1) * 8 + (s16 >> 2);
  int v_lane[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
    v_lane[db] = g * V_HEAD + v_row * V_ROW +
                 (((db ^ (s16 >> 2)) * 4 + (q16 & 1) * 2 + ((s16 & 3) >> 1)) * 16) + (s16 & 1) * 8;

  const float cl2 = p.scale_log2;
  const uint32_t ones = 0x3f803f80u;  // bf16 pair (1, 1)
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

  const int npass = (pair == NQ - 1 - pair) ? 1 : 2;
  for (int pass = 0; pass < npass; ++pass) {
    const int qt = pass == 0 ? NQ - 1 - pair : pair;  // longer tile first
    const int q0 = qt * BQ + qb * 32;
    const int myq = q0 + ln;
    const int myqc = myq < T ? myq : T - 1;
    const int headc = head_ok ? head : H - 1;

    // ---- query fragments (B operand), rotary part rotated in registers
    bf16x8 qf[12];
    {
      const size_t qrow = ((size_t)b * H + headc) * T + myqc;
      const uint16_t* qn = p.q_nope + qrow * kNope;
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) qf[kb] = as_bf16x8(ld_global_16(qn + kb * 16 + hf * 8));
      const uint16_t* qp = p.q_pe + qrow * kRope;
      u32x4 x[4];
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) x[pp] = ld_global_16(qp + pp * 16 + hf * 8);
      const float2* csr = p.cs + (size_t)myqc * kPairs;
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        bf16x8 ylo, yhi;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float2 c = csr[pp * 16 + hf * 8 + e];
          const uint32_t wl = x[pp][e >> 1], wh = x[pp + 2][e >> 1];
          const float lo = (e & 1) ? bf16hi(wl) : bf16lo(wl);
          const float hi = (e & 1) ? bf16hi(wh) : bf16lo(wh);
          ylo[e] = f32_to_bf16(fmaf(lo, c.x, -(hi * c.y)));
          yhi[e] = f32_to_bf16(fmaf(hi, c.x, lo * c.y));
        }
        qf[8 + pp] = ylo;
        qf[10 + pp] = yhi;
      }
    }

    float m_run = -INFINITY;  // reference maximum of scaled scores (base 2)
    float l_run = 0.f;        // this lane's share of the row sum
    f32x16 acc[4] = {};       // Oᵀ: dims db*32 + (r/4)*8 + hf*4 + r%4, query ln

    auto compute_tile = [&](const uint8_t* buf, int kt) {
      const int k0 = kt * BK;
      if (!head_ok || k0 > q0 + 31) return;  // every key after this wave's queries
      f32x16 s[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        s[j] = f32x16{};
        const uint8_t* kr = buf + KOFF + k_lane + j * 32 * K_ROW;
#pragma unroll
        for (int kb = 0; kb < 8; ++kb)
          s[j] = mfma32x32x16(*reinterpret_cast<const bf16x8*>(kr + kb * 32), qf[kb], s[j]);
        const uint8_t* pr = buf + KPOFF + kp_lane + j * 32 * KP_ROW;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          s[j] = mfma32x32x16(*reinterpret_cast<const bf16x8*>(pr + kb * 32), qf[8 + kb], s[j]);
      }
      if (k0 + BK - 1 > q0) {  // tile straddles this wave's diagonal
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + j * 32 + ((r >> 3) * 16) + hf * 8 + ((r >> 2) & 1) * 4 + (r & 3);
            if (key > myq) s[j][r] = -INFINITY;
          }
      }
      float mx = fmaxf(s[0][0], s[1][0]);
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(s[0][r], s[1][r]));
      mx = max_halves(mx) * cl2;
      const bool need = mx > m_run + TAU;
      if (__builtin_amdgcn_ballot_w64(need) != 0) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = fast_exp2(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db) acc[db] *= alpha;
        m_run = m_new;
      }
      bf16x8 pf[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float p0 = fast_exp2(fmaf(s[c >> 1][(c & 1) * 8 + e], cl2, -m_run));
          const float p1 = fast_exp2(fmaf(s[c >> 1][(c & 1) * 8 + e + 1], cl2, -m_run));
          const uint32_t pk = pack_bf16x2(p0, p1);
          l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk),
                                                  __builtin_bit_cast(bf16x2, ones), l_run, false);
          const bf16x2 pb = __builtin_bit_cast(bf16x2, pk);
          pf[c][e] = pb[0];
          pf[c][e + 1] = pb[1];
        }
      }
      // Oᵀ += Vᵀ·Pᵀ
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const uint8_t* vr = buf + VOFF + v_lane[db];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const s16x4 lo = ds_read_tr(vr + c * 16 * V_ROW);
          const s16x4 hi = ds_read_tr(vr + c * 16 * V_ROW + 4 * V_ROW);
          const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          acc[db] = mfma32x32x16(a, pf[c], acc[db]);
        }
      }
    };

    const int kend = min(T, qt * BQ + BQ);
    const int nkt = (kend + BK - 1) / BK;
    issue_tile(lds_a, 0);
    wait_vmem();
    __syncthreads();
    for (int kt = 0; kt < nkt; kt += 2) {
      if (kt + 1 < nkt) issue_tile(lds_b, kt + 1);
      compute_tile(lds_a, kt);
      wait_vmem();
      __syncthreads();
      if (kt + 1 >= nkt) break;
      if (kt + 2 < nkt) issue_tile(lds_a, kt + 2);
      compute_tile(lds_b, kt + 1);
      wait_vmem();
      __syncthreads();
    }

    // ---- epilogue
    if (head_ok) {
      const float l_tot = sum_halves(l_run);
      const float inv = 1.0f / l_tot;
      if (myq < T) {
        const size_t obase = ((size_t)b * T + myq) * ((size_t)H * kV) + (size_t)head * kV;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const int d0 = db * 32 + gq * 8 + hf * 4;
            const float o0 = acc[db][gq * 4 + 0] * inv, o1 = acc[db][gq * 4 + 1] * inv;
            const float o2 = acc[db][gq * 4 + 2] * inv, o3 = acc[db][gq * 4 + 3] * inv;
            if (p.out_f32) {
              *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + obase + d0) = f32x4{o0, o1, o2, o3};
            } else {
              *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.out) + obase + d0) =
                  u32x2{pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
            }
          }
        if (p.lse && hf == 0)
          p.lse[((size_t)b * H + head) * T + myq] = (m_run + log2f(l_tot)) * 0.69314718055994530942f;
      }
    }
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
  const int HG = (p.H + G - 1) / G;
  const int NQ = (p.T + BQ - 1) / BQ;
  const int NP = (NQ + 1) / 2;
  const long blocks = (long)p.B * HG * NP;
  if (blocks <= 0 || blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(prefill_kernel, dim3((unsigned)blocks), dim3(NT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
