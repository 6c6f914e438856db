// MLA decode against a latent cache, for gfx950.
//
// Page "Block input" (config.json): kv_lora_rank 512, 64 heads of 128 nope +
// 64 rope query/key dims and 128 value dims; the dense-block parameter total
// fixes kv_b_proj as one 512 -> 64·(128+128) linear map.  Page "Kimi K2 · Mix
// and project", code excerpt "mla-prefill": keys join each head's nope part with
// the rotated rope part that all heads share; the softmax runs in float32 and
// mixes the values.  A cache that keeps only the latent c (512) and the rotated
// rope key (64) per position holds everything the keys and values are made of:
// head h's nope key is W_uk,h·c and its value W_uv,h·c (rows h·256.. and
// h·256+128.. of kv_b_proj).
//
// Because both maps are linear, the products regroup exactly:
//   q_nope·(W_uk c) = (W_ukᵀ q_nope)·c        (absorb the query once)
//   Σ_j p_j (W_uv c_j) = W_uv (Σ_j p_j c_j)   (apply W_uv once, after the mix)
// so every head attends over the same 576-wide cache rows [c | rope key], and
// the cache is read once per sequence for all heads: 1152 bytes per position
// instead of 64·640 for per-head keys and values.
//
// Kernels (one stream, in order):
//   latent_q_kernel       q_lat[b,h] = bf16(q_nope[b,h] · W_uk,h)   (MFMA 16x16x32)
//   latent_decode_kernel  one workgroup per (sequence, split): 4 waves of 16
//                         heads each; Sᵀ = K·Qᵀ over 576 dims and Oᵀ += Cᵀ·Pᵀ over
//                         the 512 latent dims with 16x16x32 bf16 MFMA; cache
//                         tiles of 32 positions staged in LDS by buffer->LDS
//                         copies three tiles ahead
//   latent_out_kernel     log-sum-exp merge of the split partials into bf16
//                         latent rows in LDS, then out[b,h] = W_uv,h · o_lat[b,h]
//                         (MFMA 16x16x32)
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int LW = 4;                     // waves per decode workgroup
constexpr int LHW = 16;                   // heads per wave
constexpr int LBK = 32;                   // positions per tile
constexpr int LNST = 4;                   // LDS stages (copies run LNST-1 tiles ahead)
constexpr int L_CROW = kLatent * 2;       // 1024 B latent row
constexpr int L_PROW = kRope * 2;         // 128 B rope-key row
constexpr int L_POFF = LBK * L_CROW;      // rope-key region of a stage
constexpr int L_STAGE = L_POFF + LBK * L_PROW;  // 36864
constexpr int L_CHUNKS = L_STAGE / 1024;  // 36 copies of 1 KiB per tile
constexpr int L_CPW = L_CHUNKS / LW;      // 9 per wave
constexpr float L_TAU = 8.0f;             // lazy-rescale threshold (log2 units)
static_assert(L_STAGE % 1024 == 0 && L_CHUNKS % LW == 0, "copy layout");
static_assert(LNST * L_STAGE <= 160 * 1024, "LDS budget");
static_assert((LNST - 2) * L_CPW < 64, "vmcnt range");

// 16-byte chunk swizzle of latent row r (chunk x stored at x ^ lsw(r)); rows
// are 1 KiB, so a chunk's bank group is its physical index mod 16 (64 banks),
// or mod 8 within a 128-byte half.  Score reads take one chunk from 16
// consecutive rows: lsw is a bijection on r mod 16, and on r mod 8 over any 8
// aligned rows.  Transposed value reads: the 32 lanes of a half-wave take two
// neighbouring chunks (one pair) from each of 8 aligned rows, and the pair
// indices lsw(r) >> 1 are distinct mod 8 over those rows.
__device__ __forceinline__ int lsw(int r) { return (r & 7) | (((r ^ (r >> 3)) & 1) << 3); }
// Rope-key rows (8 chunks): distinct for any 8 consecutive rows and for
// same-parity rows among 16 consecutive ones.
__device__ __forceinline__ int psw(int r) { return (r ^ (r >> 3)) & 7; }

typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ s16x4 ds_read_tr(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
}
__device__ __forceinline__ u32x4 ds_read_16(const uint8_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Lanes l and l ^ 16 (v_permlane16_swap, same pattern as max_halves).
__device__ __forceinline__ float max_xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bf16x8 pack8(const float* y) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = pack_bf16x2(y[2 * i], y[2 * i + 1]);
  return as_bf16x8(r);
}

// ------------------------------------------------------------------ absorb --
// q_lat[b][h][c] = bf16(Σ_d q_nope[b][h][d] · W[h·256 + d][c]).  One workgroup
// per (head h, 64 latent columns), 4 waves of 16 columns, looping over the
// sequences 16 at a time; K = 128 in 4 MFMA steps.  The weight's reduction
// index d is its row, so the 128 x 64 weight block is staged in LDS with
// 16-byte loads and its B fragments (8 consecutive rows of one column) come
// from ds_read_b64_tr_b16.  LDS row d (128 B) keeps chunk x at x ^ qsw(d): the
// 32 lanes of a half-wave read two chunks from each of rows 8g..8g+3 and
// 8g+8..8g+11 (+4 for the second read), which qsw spreads over 16 bank groups.
__device__ __forceinline__ int qsw(int d) { return ((((d >> 1) & 1) | (((d >> 3) & 1) << 1)) << 1); }

__global__ __launch_bounds__(256) void latent_q_kernel(LatentParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t wt[kNope * 128];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.x, cb = blockIdx.y * 64;
  const int q = lane >> 4, i = lane & 15;
  const int H = p.H;
  // Stage W[h·256 + d][cb .. cb+63], d < 128: 1024 chunks of 16 B, 4 per thread.
  const uint16_t* wsrc = p.w_kv_b + (size_t)h * 256 * kLatent + cb;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int item = tid + it * 256;
    const int d = item >> 3, x = item & 7;
    const u32x4 v = ld_global_16(wsrc + (size_t)d * kLatent + x * 8);
    *reinterpret_cast<u32x4*>(wt + d * 128 + ((x ^ qsw(d)) * 16)) = v;
  }
  __syncthreads();
  // B fragments of this wave's 16 columns for the 4 k-steps: lane s of group q
  // addresses row ks*32 + 8q + s/4 (+4), columns 16*wave + (s%4)*4 .. +3.
  bf16x8 bf[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int d = ks * 32 + q * 8 + (i >> 2);
    const int colb = wave * 32 + (i & 3) * 8;  // byte offset of the column group in the row
    const s16x4 lo = ds_read_tr(wt + d * 128 + ((((colb >> 4) ^ qsw(d)) * 16)) + (colb & 15));
    const s16x4 hi = ds_read_tr(wt + (d + 4) * 128 + ((((colb >> 4) ^ qsw(d + 4)) * 16)) + (colb & 15));
    bf[ks] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
  const int c = cb + wave * 16 + i;
  for (int b0 = 0; b0 < p.B; b0 += 16) {
    const int brow = b0 + i;
    const uint16_t* qn = p.q_nope + ((size_t)(brow < p.B ? brow : 0) * H + h) * kNope + q * 8;
    u32x4 a[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) a[ks] = brow < p.B ? ld_global_16(qn + ks * 32) : (u32x4){0u, 0u, 0u, 0u};
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) acc = mfma16x16x32(as_bf16x8(a[ks]), bf[ks], acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int b = b0 + q * 4 + r;
      if (b < p.B)
        reinterpret_cast<__bf16*>(p.q_lat)[((size_t)b * H + h) * kLatent + c] = f32_to_bf16(acc[r]);
    }
  }
}

// ------------------------------------------------------------------ decode --
__shared__ __attribute__((aligned(1024))) uint8_t llds[LNST * L_STAGE];

__global__ __launch_bounds__(64 * LW) __attribute__((amdgpu_waves_per_eu(1, 1)))
void latent_decode_kernel(LatentParams p) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4, i16 = lane & 15;
  const int H = p.H, L = p.L, S = p.splits;
  const int b = blockIdx.x / S, split = blockIdx.x % S;
  const int ks = (int)((long long)L * split / S);
  const int ke = (int)((long long)L * (split + 1) / S);
  const int ntiles = (ke - ks + LBK - 1) / LBK;
  const int hh = wave * LHW + i16;  // this lane's head (column of Sᵀ and Oᵀ)
  const bool hv = hh < H;

  // ---- copies: wave w moves chunks w*9 .. w*9+8 of every tile.  Chunk j < 32
  // is latent row j (lane x fetches its logical chunk x ^ lsw(j)); chunk 32+k
  // holds rope rows 8k..8k+7 (lane x: row 8k + x/8, logical chunk (x%8) ^ psw).
  const uint16_t* cbase = p.ckv + (size_t)b * L * kLatent;
  const uint16_t* pbase = p.kpe + (size_t)b * L * kRope;
  const __amdgpu_buffer_rsrc_t crs = make_rsrc(cbase, (uint32_t)L * L_CROW);
  const __amdgpu_buffer_rsrc_t prs = make_rsrc(pbase, (uint32_t)L * L_PROW);
  const __amdgpu_buffer_rsrc_t none = make_rsrc(cbase, 0);
  uint32_t voff[L_CPW];
#pragma unroll
  for (int u = 0; u < L_CPW; ++u) {
    const int j = wave * L_CPW + u;
    if (j < LBK) {
      voff[u] = (uint32_t)(j * L_CROW + ((lane ^ lsw(j)) * 16));
    } else {
      const int r = (j - LBK) * 8 + (lane >> 3);
      voff[u] = (uint32_t)(r * L_PROW + (((lane & 7) ^ psw(r)) * 16));
    }
  }
  auto copy_tile = [&](int t) {
    uint8_t* st = llds + (t % LNST) * L_STAGE;
    const bool live = t < ntiles;
    const uint32_t k0 = (uint32_t)(ks + t * LBK);
#pragma unroll
    for (int u = 0; u < L_CPW; ++u) {
      const int j = wave * L_CPW + u;
      if (j < LBK)  // every cached byte is read once per call: non-temporal
        dma16_stream(live ? crs : none, st + j * 1024, voff[u] + k0 * L_CROW);
      else
        dma16_stream(live ? prs : none, st + j * 1024, voff[u] + k0 * L_PROW);
    }
  };

  // ---- query fragments (B operand of Sᵀ = K·Qᵀ): lane (q, i16) holds head hh,
  // dims c*32 + 8q .. +7; c < 16 the absorbed query, c = 16, 17 the rotated
  // q_pe (dim r pairs with r + 32: both halves sit in this lane).
  bf16x8 qf[18];
  {
    const u32x4 z = {0u, 0u, 0u, 0u};
    const uint16_t* ql = p.q_lat + ((size_t)b * H + (hv ? hh : 0)) * kLatent + q * 8;
#pragma unroll
    for (int c = 0; c < 16; ++c) qf[c] = as_bf16x8(hv ? ld_global_16(ql + c * 32) : z);
    const uint16_t* qp = p.q_pe + ((size_t)b * H + (hv ? hh : 0)) * kRope + q * 8;
    const u32x4 xa = hv ? ld_global_16(qp) : z;
    const u32x4 xb = hv ? ld_global_16(qp + 32) : z;
    const float* Rrow = p.R + (size_t)p.q_pos * kPairs + q * 8;
    float ya[8], yb[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float sn, cs;
      sincosf(Rrow[e], &sn, &cs);
      const float a = (e & 1) ? bf16hi(xa[e >> 1]) : bf16lo(xa[e >> 1]);
      const float c = (e & 1) ? bf16hi(xb[e >> 1]) : bf16lo(xb[e >> 1]);
      ya[e] = fmaf(a, cs, -(c * sn));
      yb[e] = fmaf(c, cs, a * sn);
    }
    qf[16] = pack8(ya);
    qf[17] = pack8(yb);
  }

  // Per-lane LDS offsets.  Score reads (A = key tile, 16 rows x 32 dims): row
  // kb*16 + i16, logical chunk c*4 + q.  Value reads (ds_read_b64_tr_b16, A =
  // Cᵀ: 16 dims x 32 positions): lane s of group q addresses row 4q + s/4 (and
  // 16 + that), bytes db*32 + (s%4)*8, i.e. chunk 2db + (s%4)/2, half s%2; lane
  // i then receives dim db*16 + i of those four positions.  The position order
  // (4q..4q+3, 16+4q..16+4q+3) is the order in which the Sᵀ accumulators hold
  // them, so the weights are the B operand without any exchange.
  // The swizzle only permutes the low 4 bits of a chunk index, so a read's
  // address splits into a lane part (kept in a register) and a constant part
  // (the instruction's offset): score reads of chunk 4m + j use k_lane[j] +
  // 256m; value reads of dim block 8m + j use v_lane[j] + 256m.
  const int srow_sw = lsw(i16);  // rows i16 and 16 + i16 share the swizzle
  int k_lane[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) k_lane[j] = i16 * L_CROW + (((j * 4 + q) ^ srow_sw) * 16);
  int p_lane[2][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int c = 0; c < 2; ++c)
      p_lane[kb][c] = L_POFF + (kb * 16 + i16) * L_PROW + (((c * 4 + q) ^ psw(kb * 16 + i16)) * 16);
  const int vrow = q * 4 + (i16 >> 2);
  const int vrow_sw = lsw(vrow);
  int v_lane[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    v_lane[j] = vrow * L_CROW + (((2 * j + ((i16 & 3) >> 1)) ^ vrow_sw) * 16) + (i16 & 1) * 8;

  const float cl2 = p.scale_log2;
  const uint32_t ones = 0x3f803f80u;
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc[32];
#pragma unroll
  for (int db = 0; db < 32; ++db) acc[db] = (f32x4){0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int t = 0; t < LNST - 1; ++t) copy_tile(t);

  for (int t = 0; t < ntiles; ++t) {
    wait_vm<(LNST - 2) * L_CPW>();
    barrier_lds();
    const uint8_t* st = llds + (t % LNST) * L_STAGE;

    // Sᵀ for the two 16-position halves of the tile.  With one wave per SIMD
    // nothing hides an LDS read's latency, so reads run ahead of the products:
    // the first half's 18 key fragments are requested up front, the second
    // half's one by one behind the first half's products.
    auto kread = [&](int kb, int c) {
      return c < 16 ? ds_read_16(st + k_lane[c & 3] + kb * 16 * L_CROW + (c >> 2) * 256)
                    : ds_read_16(st + p_lane[kb][c - 16]);
    };
    u32x4 k0f[18], k1f[18];
#pragma unroll
    for (int c = 0; c < 18; ++c) k0f[c] = kread(0, c);
    __builtin_amdgcn_sched_barrier(0);
    f32x4 s[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int c = 0; c < 18; ++c) {
      s[0] = mfma16x16x32(as_bf16x8(k0f[c]), qf[c], s[0]);
      k1f[c] = kread(1, c);
    }
    // Pin the order product, read, product, read, ...: each second-half
    // fragment takes the registers of a first-half one already consumed.
#pragma unroll
    for (int c = 0; c < 18; ++c) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < 18; ++c) s[1] = mfma16x16x32(as_bf16x8(k1f[c]), qf[c], s[1]);

    // Value fragments, 8 dim blocks per group; the first group is requested
    // before the softmax so its reads overlap that work.
    bf16x8 vf[8];
    auto vload = [&](int g) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int off = v_lane[u] + g * 256;
        const s16x4 lo = ds_read_tr(st + off);
        const s16x4 hi = ds_read_tr(st + off + 16 * L_CROW);
        vf[u] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    };
    vload(0);

    // Online softmax (base 2) over this tile: lane holds positions
    // kb*16 + 4q + r of head hh; the other 24 are in lanes q' != q.
    const int k0 = ks + t * LBK;
    float x[8];
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = k0 + kb * 16 + q * 4 + r;
        const float v = key < ke ? s[kb][r] * cl2 : -INFINITY;
        x[kb * 4 + r] = v;
        mx = fmaxf(mx, v);
      }
    mx = max_halves(max_xor16(mx));
    const float m_new = fmaxf(m_run, mx);
    if (__builtin_amdgcn_ballot_w64(m_new > m_run + L_TAU) != 0) {
      const float alpha = m_run == -INFINITY ? 0.f : fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 32; ++db) acc[db] *= alpha;
      m_run = m_new;
    }
    float pw[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pw[e] = fast_exp2(x[e] - m_run);
    u32x4 pk;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // A scalar copy: bit-casting the vector element pk[e] would read element 0.
      const uint32_t pe = pack_bf16x2(pw[2 * e], pw[2 * e + 1]);
      pk[e] = pe;
      l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pe),
                                              __builtin_bit_cast(bf16x2, ones), l_run, false);
    }
    const bf16x8 pf = as_bf16x8(pk);
    // The next copies go out here, not at the top of the step: a wave stalls
    // until the copy engine accepts each copy, and with one wave per SIMD a
    // stall before the score products idles the matrix core (16% slower).
    copy_tile(t + LNST - 1);

    // Oᵀ += Cᵀ·Pᵀ over the 512 latent dims, 16 at a time; each group's reads
    // are issued right behind the previous group's products.
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < 8; ++u) acc[g * 8 + u] = mfma16x16x32(vf[u], pf, acc[g * 8 + u]);
      if (g + 1 < 4) vload(g + 1);
    }
  }
  wait_vm<0>();

  // ---- results of head hh: every lane of the head holds dims db*16 + 4q + r.
  const float l_tot = sum_halves(sum_xor16(l_run));
  if (!hv) return;
  if (S == 1) {
    const float inv = 1.f / l_tot;
    float* dst = p.o_lat + ((size_t)b * H + hh) * kLatent + q * 4;
#pragma unroll
    for (int db = 0; db < 32; ++db) *reinterpret_cast<f32x4*>(dst + db * 16) = acc[db] * inv;
    if (p.lse && q == 0) p.lse[(size_t)b * H + hh] = (m_run + log2f(l_tot)) * 0.69314718055994530942f;
  } else {
    float* part = p.part + (((size_t)b * H + hh) * S + split) * kLatentPart;
    if (q == 0) {
      part[0] = m_run;
      part[1] = l_tot;
    }
#pragma unroll
    for (int db = 0; db < 32; ++db) *reinterpret_cast<f32x4*>(part + 8 + db * 16 + q * 4) = acc[db];
  }
}

// ----------------------------------------------------------- merge+expand --
// One workgroup per (head h, 16 sequences), 8 waves.  First the 16 latent
// output rows are formed in LDS as bf16 (RNE): with splits, by the
// log-sum-exp merge of the partials (max, sum, unnormalised output), else
// from the normalised rows the decode kernel stored.  Then wave w computes
// out[b][h·128 + 16w .. +15] = Σ_c W[h·256 + 128 + e][c] · o[b][c] over the
// 512 latent dims in 16 MFMA steps; the weight rows are K-contiguous and all
// 16 of a lane's fragments are requested before the first product.  LDS row r
// keeps chunk x (8 dims) at x ^ r.
__global__ __launch_bounds__(512) void latent_out_kernel(LatentParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t tile[16 * L_CROW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.x, b0 = blockIdx.y * 16;
  const int H = p.H, S = p.splits;
  const int q = lane >> 4, i = lane & 15;
  const int e0 = wave * 16;

  // Weight fragments first: their latency overlaps the merge below.
  const uint16_t* w = p.w_kv_b + ((size_t)h * 256 + kNope + e0 + i) * kLatent + q * 8;
  u32x4 wf[16];
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) wf[ks] = ld_global_16(w + ks * 32);

#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int item = tid + it * 512;  // 16 rows x 64 chunks of 8 dims
    const int r = item >> 6, ch = item & 63;
    const int b = b0 + r;
    float y[8];
    if (b >= p.B) {
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = 0.f;
    } else if (S == 1) {
      const float* o = p.o_lat + ((size_t)b * H + h) * kLatent + ch * 8;
      const f32x4 lo = *reinterpret_cast<const f32x4*>(o);
      const f32x4 hi = *reinterpret_cast<const f32x4*>(o + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        y[e] = lo[e];
        y[4 + e] = hi[e];
      }
    } else {
      const float* part = p.part + ((size_t)b * H + h) * S * kLatentPart;
      float M = -INFINITY;
      for (int sp = 0; sp < S; ++sp) M = fmaxf(M, part[sp * kLatentPart]);
      float lt = 0.f;
      f32x4 lo = {0.f, 0.f, 0.f, 0.f}, hi = {0.f, 0.f, 0.f, 0.f};
      for (int sp = 0; sp < S; ++sp) {
        const float* ps = part + sp * kLatentPart;
        const float ms = ps[0];
        const float wt = ms == -INFINITY ? 0.f : fast_exp2(ms - M);
        lt = fmaf(ps[1], wt, lt);
        lo += *reinterpret_cast<const f32x4*>(ps + 8 + ch * 8) * wt;
        hi += *reinterpret_cast<const f32x4*>(ps + 12 + ch * 8) * wt;
      }
      const float inv = 1.f / lt;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        y[e] = lo[e] * inv;
        y[4 + e] = hi[e] * inv;
      }
      if (p.lse && ch == 0) p.lse[(size_t)b * H + h] = (M + log2f(lt)) * 0.69314718055994530942f;
    }
    *reinterpret_cast<u32x4*>(tile + r * L_CROW + ((ch ^ r) * 16)) = as_u32x4(pack8(y));
  }
  __syncthreads();

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(tile + i * L_CROW + (((ks * 4 + q) ^ i) * 16));
    acc = mfma16x16x32(as_bf16x8(a), as_bf16x8(wf[ks]), acc);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int b = b0 + q * 4 + r;
    if (b >= p.B) continue;
    const size_t idx = (size_t)b * H * kV + (size_t)h * kV + e0 + i;
    if (p.out_f32)
      static_cast<float*>(p.out)[idx] = acc[r];
    else
      static_cast<__bf16*>(p.out)[idx] = f32_to_bf16(acc[r]);
  }
}

}  // namespace

LatentWorkspace latent_workspace_layout(int B, int H, int splits) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  LatentWorkspace w;
  w.q_off = 0;
  w.o_off = up((size_t)B * H * kLatent * 2);
  w.part_off = w.o_off + up((size_t)B * H * kLatent * 4);
  w.total = w.part_off + (splits > 1 ? up((size_t)B * H * splits * kLatentPart * 4) : 0);
  return w;
}

int latent_choose_splits(int B, int L, int requested) {
  if (requested > 0) return requested < L ? requested : L;
  long s = (kComputeUnits + B - 1) / B;  // one workgroup per compute unit
  long cap = L / (2 * LBK);              // at least two tiles per split
  if (cap < 1) cap = 1;
  if (s > cap) s = cap;
  if (s < 1) s = 1;
  return (int)s;
}

hipError_t launch_decode_latent(const LatentParams& p, hipStream_t stream) {
  const long bblocks = (p.B + 15) / 16;
  const long dblocks = (long)p.B * p.splits;
  if (dblocks <= 0 || dblocks > 0x7fffffffL || bblocks > 65535 || p.H > LW * LHW)
    return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(latent_q_kernel, dim3(p.H, kLatent / 64), dim3(256), 0, stream, p);
  hipLaunchKernelGGL(latent_decode_kernel, dim3((unsigned)dblocks), dim3(64 * LW), 0, stream, p);
  hipLaunchKernelGGL(latent_out_kernel, dim3(p.H, (unsigned)bblocks), dim3(512), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
