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
// Design (one workgroup = G heads × BQ queries of one sequence):
//   * Each wave owns 32 queries of one head.  It computes Sᵀ = K·Qᵀ with
//     v_mfma_f32_32x32x16_bf16: the key tile is the A operand (from LDS) and
//     the query the B operand (kept in registers for the whole key loop, with
//     q_pe rotated in registers on load).  In the transposed product every lane
//     holds 16 scores of ONE query, so the row max/sum of the online softmax
//     are per-lane values plus one exchange between the two half-waves.
//   * The 192-long contraction is 8 MFMA k-steps over k_nope and 4 over the
//     rotated shared key; the rotated key tile is staged into LDS once per
//     workgroup and read by every head of the workgroup.
//   * Oᵀ += Vᵀ·Pᵀ: the bf16-rounded weights stay in registers as the B operand;
//     the order in which the A lanes fetch key rows is permuted so that the
//     accumulator layout of Sᵀ is exactly the B-operand layout of Pᵀ (no data
//     movement).  V is stored transposed in LDS ([dim][key]).
//   * Online softmax in base 2 with softmax_scale·log2(e) folded into one FMA;
//     the running sum is accumulated from the same bf16-rounded weights that
//     enter the PV product, so the weights that multiply V sum exactly to the
//     normaliser up to float32 summation order.
//   * Causal tiles: a workgroup loads only key tiles up to its last query;
//     a wave skips tiles entirely after its queries and masks (j > i) only on
//     tiles that straddle its diagonal.  The longest query tiles are issued
//     first so the causal triangle does not leave an idle tail.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int BK = 64;             // keys per tile
constexpr int VT_STRIDE = BK + 8;  // Vᵀ LDS row stride in elements (144 B: conflict-free reads)

// XOR swizzle of the 16-byte chunks of a key row in LDS.  Lanes that read the
// same logical chunk of different key rows land on distinct bank groups.
__device__ __forceinline__ int kswz(int key) {
  return (key & 3) | (((key >> 3) & 1) << 2) | (((key >> 2) & 1) << 3);
}

// Tile-local key fetched by A-operand lane R (0..31) of a 32-key block.  The
// accumulator register r of lane (n, h) holds row (r/4)*8 + h*4 + r%4; with
// this order that row is key (r/4 >> 1)*16 + h*8 + (r/4 & 1)*4 + r%4, so lane
// half h holds keys h*8..h*8+7 of each 16-key chunk in 8 consecutive
// registers -- the B-operand layout of the PV product.
__device__ __forceinline__ int akey(int R) {
  const int g4 = R >> 3, h = (R >> 2) & 1, i = R & 3;
  return (g4 >> 1) * 16 + h * 8 + (g4 & 1) * 4 + i;
}

template <int G, int WPH>
struct Cfg {
  static constexpr int NW = G * WPH;
  static constexpr int NT = 64 * NW;
  static constexpr int BQ = 32 * WPH;
  static constexpr int SK = G * BK * kNope;   // k_nope tiles, per head
  static constexpr int SKP = BK * kRope;      // shared rotated key tile
  static constexpr int SVT = G * kV * VT_STRIDE;
  static constexpr int LDS_BYTES = 2 * (SK + SKP + SVT);
};

template <int G, int WPH>
__global__ __launch_bounds__(64 * G * WPH) void prefill_kernel(PrefillParams p) {
  using C = Cfg<G, WPH>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[C::SK + C::SKP + C::SVT];
  uint16_t* sK = smem;
  uint16_t* sKP = sK + C::SK;
  uint16_t* sVt = sKP + C::SKP;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int ln = lane & 31;
  const int hf = lane >> 5;

  const int H = p.H, T = p.T;
  const int HG = (H + G - 1) / G;
  const int NQ = (T + C::BQ - 1) / C::BQ;
  const int per_q = p.B * HG;
  const int id = blockIdx.x;
  const int qt = NQ - 1 - id / per_q;  // longest query tiles first
  const int rem = id % per_q;
  const int b = rem / HG;
  const int hg = rem % HG;

  const int g = wave / WPH;
  const int qb = wave % WPH;
  const int head = hg * G + g;
  const bool head_ok = head < H;
  const int headc = head_ok ? head : H - 1;
  const int q0 = qt * C::BQ + qb * 32;  // first query of this wave
  const int myq = q0 + ln;
  const int myqc = myq < T ? myq : T - 1;

  // ---- query fragments: B operand of Sᵀ = K·Qᵀ, k-step kb covers dims
  // kb*16 + hf*8 .. +7 of the 192-wide query (0..7 nope, 8..11 rotary).
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
    // Rotary dims pp*16 + hf*8 + e (pp = 0, 1) pair with the dims 32 higher
    // (pp + 2): rotate in float32 and round to bf16.
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

  const int kend = min(T, qt * C::BQ + C::BQ);  // keys visible to this workgroup
  const int nkt = (kend + BK - 1) / BK;
  const float cl2 = p.scale_log2;
  const int r_key = akey(ln);

  float m_run = -INFINITY;  // running max of scaled scores (base-2 units)
  float l_run = 0.f;        // this lane's share of the running sum
  f32x16 acc[4] = {};       // Oᵀ: dims db*32 + (r/4)*8 + hf*4 + r%4, query ln

  for (int kt = 0; kt < nkt; ++kt) {
    const int k0 = kt * BK;
    __syncthreads();
    // ---- stage the key tile: k_nope of each head, shared rotated key, Vᵀ.
    // Rows past T repeat row T-1 (finite values); they are causally masked.
    for (int it = tid; it < G * BK * 16; it += C::NT) {
      const int gg = it / (BK * 16);
      const int r = (it / 16) % BK;
      const int ch = it % 16;
      const int hh = min(hg * G + gg, H - 1);
      const int key = min(k0 + r, T - 1);
      const u32x4 v = ld_global_16(p.k_nope + (((size_t)b * H + hh) * T + key) * kNope + ch * 8);
      *reinterpret_cast<u32x4*>(sK + (gg * BK + r) * kNope + ((ch ^ kswz(r)) * 8)) = v;
    }
    for (int it = tid; it < BK * 8; it += C::NT) {
      const int r = it / 8, ch = it % 8;
      const int key = min(k0 + r, T - 1);
      const u32x4 v = ld_global_16(p.kpe_rot + ((size_t)b * T + key) * kRope + ch * 8);
      *reinterpret_cast<u32x4*>(sKP + r * kRope + ((ch ^ (kswz(r) & 7)) * 8)) = v;
    }
    for (int it = tid; it < G * (BK / 8) * 32; it += C::NT) {
      // 8 keys x 4 dims per item: load rows, transpose in registers.
      const int gg = it / ((BK / 8) * 32);
      const int r2 = it % ((BK / 8) * 32);
      const int kg = r2 / 32, dg = r2 % 32;
      const int hh = min(hg * G + gg, H - 1);
      const uint16_t* vb = p.v + ((size_t)b * H + hh) * T * kV + dg * 4;
      u32x2 w[8];
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int key = min(k0 + kg * 8 + kk, T - 1);
        w[kk] = ld_global_8(vb + (size_t)key * kV);
      }
      uint16_t* dst = sVt + (gg * kV + dg * 4) * VT_STRIDE + kg * 8;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t a0 = w[2 * e][j >> 1], a1 = w[2 * e + 1][j >> 1];
          o[e] = (j & 1) ? ((a0 >> 16) | (a1 & 0xffff0000u)) : ((a0 & 0xffffu) | (a1 << 16));
        }
        *reinterpret_cast<u32x4*>(dst + j * VT_STRIDE) = o;
      }
    }
    __syncthreads();
    if (!head_ok || k0 > q0 + 31) continue;  // every key of the tile is after this wave's queries

    // ---- Sᵀ = K·Qᵀ for two 32-key blocks
    f32x16 s[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      s[j] = f32x16{};
      const int r = j * 32 + r_key;
      const int sw = kswz(r);
      const uint16_t* krow = sK + (g * BK + r) * kNope;
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + (((kb * 2 + hf) ^ sw) * 8));
        s[j] = mfma32x32x16(a, qf[kb], s[j]);
      }
      const uint16_t* prow = sKP + r * kRope;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(prow + (((kb * 2 + hf) ^ (sw & 7)) * 8));
        s[j] = mfma32x32x16(a, qf[8 + kb], s[j]);
      }
    }
    // ---- causal mask where the tile straddles this wave's diagonal
    if (k0 + BK - 1 > q0) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + j * 32 + ((r >> 2) >> 1) * 16 + hf * 8 + ((r >> 2) & 1) * 4 + (r & 3);
          if (key > myq) s[j][r] = -INFINITY;
        }
    }
    // ---- online softmax (base 2)
    float mx = s[0][0];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[j][r]);
    mx = max_halves(mx);
    const float m_new = fmaxf(m_run, mx * cl2);
    const float alpha = fast_exp2(m_run - m_new);
    bf16x8 pf[4];
    float ls = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pv = fast_exp2(fmaf(s[c >> 1][(c & 1) * 8 + e], cl2, -m_new));
        const __bf16 pb = f32_to_bf16(pv);
        pf[c][e] = pb;
        ls += (float)pb;
      }
    l_run = l_run * alpha + ls;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < 4; ++db) acc[db] *= alpha;
    // ---- Oᵀ += Vᵀ·Pᵀ
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const uint16_t* vrow = sVt + (g * kV + db * 32 + ln) * VT_STRIDE + hf * 8;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(vrow + c * 16);
        acc[db] = mfma32x32x16(a, pf[c], acc[db]);
      }
    }
  }

  if (!head_ok) return;
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

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
  constexpr int G = 2, WPH = 2;
  using C = Cfg<G, WPH>;
  const int HG = (p.H + G - 1) / G;
  const int NQ = (p.T + C::BQ - 1) / C::BQ;
  const long blocks = (long)NQ * p.B * HG;
  if (blocks <= 0 || blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((prefill_kernel<G, WPH>), dim3((unsigned)blocks), dim3(C::NT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
