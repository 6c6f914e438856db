// MLA decode attention for gfx950: one new query per (sequence, head)
// against L cached keys, bound by the HBM stream of the cache.
//
// Page "Kimi K2 · Mix and project", code excerpt "mla-prefill": the cache is
// updated with keys that are already rotated and joined ([k_nope | rot(k_pe)],
// 192 wide) and with the values; scores are Q·Kᵀ·softmax_scale, the softmax
// runs in float32 and mixes the 128-wide values.  The new query is rotated at
// its own position (page "Kimi K2 · Transformer blocks": position ids start
// after the tokens already cached).
//
// Two cache layouts: joined key rows [nope 128 | rotated rope 64] per head,
// or nope rows per head plus one rotated rope key per position shared by all
// heads (page "Kimi K2 · Mix and project": the key's rotated part is one tensor
// for every head), which reads 1/3 fewer key bytes per head.
//
// Design:
//   * Workgroup = one (b, h, split) of 4 waves; a split is a contiguous key
//     range [L·s/S, L·(s+1)/S).  Inside a wave, 8 lanes share one key: each
//     lane reads 16-byte pieces of the key row (384 B) and value row (256 B),
//     so every load instruction moves contiguous 128-byte segments and each
//     cache byte is read exactly once, with non-temporal loads (the streamed
//     rows are not kept in the caches; measured 3.03 ms against 3.42 with
//     ordinary loads at B=64, L=8192, H=64).  A wave step covers 32 keys (8 groups ×
//     4 keys); the next step's rows are loaded before the current step is
//     consumed so two steps of loads are in flight per wave.
//   * Scores: v_dot2_f32_bf16 on packed bf16 pairs (no unpacking of the key),
//     then a 3-step butterfly over the 8 lanes of the group.
//   * Each lane group runs its own online softmax (base 2, one rescale per
//     4 keys); the 32 group states of the workgroup are merged in LDS by the
//     log-sum-exp rule.  With one split the result is normalised and stored;
//     otherwise (max, sum, unnormalised output) go to the workspace and a
//     merge kernel combines the splits the same way.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int DWAVES = 4;
constexpr int KPG = 4;                  // keys per lane group per step
constexpr int WSTEP = 8 * KPG;          // keys per wave step
constexpr int NGROUPS = DWAVES * 8;     // lane groups per workgroup

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

// Sum over the 8 lanes of a group (lanes 8k..8k+7); every lane gets the same
// bits because each step adds the same two operands in both partner lanes.
__device__ __forceinline__ float group8_sum(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 4);
  return x;
}

template <bool SHARED_KPE>
__global__ __launch_bounds__(64 * DWAVES) void decode_split_kernel(DecodeParams p) {
  __shared__ float s_m[NGROUPS], s_l[NGROUPS];
  __shared__ float s_o[NGROUPS][kV];

  const int S = p.splits;
  int bh, split;
  {
    const int bid = blockIdx.x;
    if (SHARED_KPE && p.B % 8 == 0) {
      // Workgroup ids are dealt round-robin to the 8 XCDs: give every (head,
      // split) of a sequence to one XCD, issued back to back, so that XCD's L2
      // serves the sequence's shared rope rows to all its heads.
      const int x = bid % 8, o = bid / 8;
      const int per_seq = p.H * S;
      const int b = x + 8 * (o / per_seq);
      const int r = o % per_seq;
      bh = b * p.H + r / S;
      split = r % S;
    } else {
      split = bid % S;
      bh = bid / S;
    }
  }
  const int L = p.L;
  const int ks = (int)((long long)L * split / S);
  const int ke = (int)((long long)L * (split + 1) / S);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kq = lane >> 3;  // key slot of this lane's group within a step
  const int j = lane & 7;    // 16-byte piece index within the group

  // ---- query pieces: nope dims j*8.. and 64+j*8.., rotary dims j*8.. (rotated
  // at q_pos: dim r pairs with r ± 32, angle R[q_pos][r mod 32]).
  const uint16_t* qn = p.q_nope + (size_t)bh * kNope;
  const u32x4 qa = ld_global_16(qn + j * 8);
  const u32x4 qb = ld_global_16(qn + 64 + j * 8);
  u32x4 qr;
  {
    const uint16_t* qp = p.q_pe + (size_t)bh * kRope;
    const u32x4 xo = ld_global_16(qp + j * 8);
    const u32x4 xp = ld_global_16(qp + ((j * 8 + 32) & 63));
    const bool lo_half = j < 4;  // dims j*8.. are < 32
    const float* Rrow = p.R + (size_t)p.q_pos * kPairs;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float y[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int pair = (j * 8 + 2 * w + e) & 31;
        float sn, cs;
        sincosf(Rrow[pair], &sn, &cs);
        const float own = e ? bf16hi(xo[w]) : bf16lo(xo[w]);
        const float oth = e ? bf16hi(xp[w]) : bf16lo(xp[w]);
        // lo dim: own·cos − partner·sin ; hi dim: own·cos + partner·sin
        y[e] = lo_half ? fmaf(own, cs, -(oth * sn)) : fmaf(own, cs, oth * sn);
      }
      qr[w] = pack_bf16x2(y[0], y[1]);
    }
  }

  const float cl2 = p.scale_log2;
  constexpr int KROW = SHARED_KPE ? kNope : kQK;  // elements per cached key row
  const uint16_t* kbase = p.k_cache + (size_t)bh * L * KROW;
  const uint16_t* vbase = p.v_cache + (size_t)bh * L * kV;
  const uint16_t* pbase = SHARED_KPE ? p.kpe_cache + (size_t)(bh / p.H) * L * kRope : nullptr;

  float m_run = -INFINITY, l_run = 0.f;
  float o[16];
#pragma unroll
  for (int d = 0; d < 16; ++d) o[d] = 0.f;

  u32x4 kr[KPG][3], vr[KPG][2];
  auto load_step = [&](int base) {
#pragma unroll
    for (int u = 0; u < KPG; ++u) {
      const int key = min(base + u * 8 + kq, ke - 1);
      const uint16_t* krow = kbase + (size_t)key * KROW;
      const uint16_t* vrow = vbase + (size_t)key * kV;
      kr[u][0] = ld_stream_16(krow + j * 8);
      kr[u][1] = ld_stream_16(krow + 64 + j * 8);
      if constexpr (SHARED_KPE)
        kr[u][2] = ld_global_16(pbase + (size_t)key * kRope + j * 8);  // shared by the heads: cached
      else
        kr[u][2] = ld_stream_16(krow + 128 + j * 8);
      vr[u][0] = ld_stream_16(vrow + j * 8);
      vr[u][1] = ld_stream_16(vrow + 64 + j * 8);
    }
  };

  int base = ks + wave * WSTEP;
  if (base < ke) load_step(base);
  for (; base < ke; base += DWAVES * WSTEP) {
    u32x4 ck[KPG][3], cv[KPG][2];
#pragma unroll
    for (int u = 0; u < KPG; ++u) {
      ck[u][0] = kr[u][0]; ck[u][1] = kr[u][1]; ck[u][2] = kr[u][2];
      cv[u][0] = vr[u][0]; cv[u][1] = vr[u][1];
    }
    const int next = base + DWAVES * WSTEP;
    if (next < ke) load_step(next);

    float sc[KPG];
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < KPG; ++u) {
      float a = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        a = dot2(ck[u][0][w], qa[w], a);
        a = dot2(ck[u][1][w], qb[w], a);
        a = dot2(ck[u][2][w], qr[w], a);
      }
      a = group8_sum(a);
      const int key = base + u * 8 + kq;
      sc[u] = key < ke ? a * cl2 : -INFINITY;
      mx = fmaxf(mx, sc[u]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float pw[KPG];
    float ls = 0.f;
#pragma unroll
    for (int u = 0; u < KPG; ++u) {
      pw[u] = fast_exp2(sc[u] - m_use);
      ls += pw[u];
    }
    l_run = l_run * alpha + ls;
    m_run = m_new;
#pragma unroll
    for (int d = 0; d < 16; ++d) o[d] *= alpha;
#pragma unroll
    for (int u = 0; u < KPG; ++u) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        o[2 * w] = fmaf(pw[u], bf16lo(cv[u][0][w]), o[2 * w]);
        o[2 * w + 1] = fmaf(pw[u], bf16hi(cv[u][0][w]), o[2 * w + 1]);
        o[8 + 2 * w] = fmaf(pw[u], bf16lo(cv[u][1][w]), o[8 + 2 * w]);
        o[8 + 2 * w + 1] = fmaf(pw[u], bf16hi(cv[u][1][w]), o[8 + 2 * w + 1]);
      }
    }
  }

  // ---- merge the 32 lane-group states of the workgroup
  const int grp = wave * 8 + kq;
  if (j == 0) {
    s_m[grp] = m_run;
    s_l[grp] = l_run;
  }
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    s_o[grp][j * 8 + d] = o[d];
    s_o[grp][64 + j * 8 + d] = o[8 + d];
  }
  __syncthreads();
  if (tid < kV) {
    float M = -INFINITY;
    for (int g2 = 0; g2 < NGROUPS; ++g2) M = fmaxf(M, s_m[g2]);
    float lt = 0.f, od = 0.f;
    for (int g2 = 0; g2 < NGROUPS; ++g2) {
      const float w = s_m[g2] == -INFINITY ? 0.f : fast_exp2(s_m[g2] - M);
      lt = fmaf(s_l[g2], w, lt);
      od = fmaf(s_o[g2][tid], w, od);
    }
    if (S == 1) {
      const float val = od / lt;
      if (p.out_f32)
        static_cast<float*>(p.out)[(size_t)bh * kV + tid] = val;
      else
        static_cast<__bf16*>(p.out)[(size_t)bh * kV + tid] = f32_to_bf16(val);
      if (p.lse && tid == 0) p.lse[bh] = (M + log2f(lt)) * 0.69314718055994530942f;
    } else {
      float* part = p.part + ((size_t)bh * S + split) * kDecodePart;
      if (tid == 0) {
        part[0] = M;
        part[1] = lt;
      }
      part[8 + tid] = od;
    }
  }
}

// Combine the split partials of one (b, h): one thread per output dim.
__global__ __launch_bounds__(kV) void decode_merge_kernel(DecodeParams p) {
  const int bh = blockIdx.x;
  const int d = threadIdx.x;
  const int S = p.splits;
  const float* part = p.part + (size_t)bh * S * kDecodePart;
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, part[s * kDecodePart]);
  float lt = 0.f, od = 0.f;
  for (int s = 0; s < S; ++s) {
    const float ms = part[s * kDecodePart];
    const float w = ms == -INFINITY ? 0.f : fast_exp2(ms - M);
    lt = fmaf(part[s * kDecodePart + 1], w, lt);
    od = fmaf(part[s * kDecodePart + 8 + d], w, od);
  }
  const float val = od / lt;
  if (p.out_f32)
    static_cast<float*>(p.out)[(size_t)bh * kV + d] = val;
  else
    static_cast<__bf16*>(p.out)[(size_t)bh * kV + d] = f32_to_bf16(val);
  if (p.lse && d == 0) p.lse[bh] = (M + log2f(lt)) * 0.69314718055994530942f;
}

}  // namespace

int decode_choose_splits(int B, int H, int L, int requested) {
  if (requested > 0) return requested < L ? requested : L;
  const long units = (long)B * H;
  const long target = 1024;  // workgroups: four per compute unit
  long s = (target + units - 1) / units;
  long cap = L / 256;        // keep at least 256 keys per split
  if (cap < 1) cap = 1;
  if (s > cap) s = cap;
  if (s < 1) s = 1;
  return (int)s;
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  const long blocks = (long)p.B * p.H * p.splits;
  if (blocks <= 0 || blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
  if (p.kpe_cache)
    hipLaunchKernelGGL(decode_split_kernel<true>, dim3((unsigned)blocks), dim3(64 * DWAVES), 0, stream, p);
  else
    hipLaunchKernelGGL(decode_split_kernel<false>, dim3((unsigned)blocks), dim3(64 * DWAVES), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  hipLaunchKernelGGL(decode_merge_kernel, dim3((unsigned)((long)p.B * p.H)), dim3(kV), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
