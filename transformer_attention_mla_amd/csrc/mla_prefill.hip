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
//   * A workgroup (8 waves) owns one head × 256 queries of one sequence; each
//     wave owns 32 queries.  It processes a pair of query tiles, i and NQ-1-i,
//     one after the other, so every workgroup does the same amount of causal
//     work -- unless that leaves fewer than two workgroups per compute unit
//     (short sequences), when each workgroup takes one query tile, the
//     longest first.  Workgroups of the same (sequence, head) are placed on the same
//     XCD and issued together, so that XCD's L2 serves their key/value stream.
//     (The head count per workgroup, G, is a constant: two heads per
//     workgroup share one staged copy of the rotated key tile, but one head
//     with twice the queries copies 43% fewer key/value bytes per query-head,
//     which measured faster.  The rotated key is computed once per position
//     for all heads either way.)
//   * Key tiles are 32 keys.  A tile (k_nope, the rotated shared rotary key and
//     V) lives in one of four LDS stages.  Asynchronous buffer→LDS copies run
//     three tiles ahead of the tile being multiplied; the workgroup barrier
//     between tiles waits only for the next tile's copies (explicit, in-order
//     vmcnt counts), never for the ones still in flight behind it.  A wave
//     issuing copies stalls until the copy engine takes them, so the copies
//     are issued by the two waves that finish each step first (the SIMD gives
//     the older of its two waves the matrix core first), at the end of the
//     step, where they would otherwise idle at the barrier.  Past the last
//     tile the copies are empty (zero-length descriptors), keeping the counts
//     uniform.
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
//   * Vᵀ fragments (8 consecutive keys of one feature per lane) come from V's
//     natural [key][dim] layout with the gfx950 transposing LDS read
//     ds_read_b64_tr_b16, or, when V is given key-blocked (16-key blocks
//     stored feature by feature), with one plain 16-byte read each: the
//     transposing read moves about 90 B per clock per compute unit against
//     about 236 for ds_read_b128.
//   * Online softmax in base 2, softmax_scale·log2(e) folded into one FMA.  The
//     reference maximum is only raised when a tile's maximum exceeds it by
//     more than 8 (weights then stay <= 2^8); the result is the same softmax.
//     The row sum is accumulated (v_dot2_f32_bf16 against ones) from the same
//     bf16-rounded weights that enter the PV product.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int G = 1;          // heads per workgroup
constexpr int WPH = 8;        // waves per head
constexpr int NW = G * WPH;   // 8 waves
constexpr int NT = 64 * NW;   // 512 threads
constexpr int BQ = 32 * WPH;  // 256 queries per tile
constexpr int BK = 32;        // keys per tile
constexpr int NSTAGE = 4;     // LDS stages; copies run NSTAGE-1 tiles ahead
constexpr float TAU = 8.0f;   // lazy-rescale threshold (log2 units)

// LDS stage layout (bytes): k_nope head 0 | head 1 | rotated key | V head 0 | head 1.
constexpr int K_ROW = 272;                  // 256 B of k_nope + 16 B pad (17 slots)
constexpr int K_HEAD = BK * K_ROW;          // 8704
constexpr int KPOFF = (G * K_HEAD + 1023) / 1024 * 1024;  // k_nope region in whole 1 KiB chunks
constexpr int KP_ROW = 128;                 // rotated key, 16 B chunks XOR-swizzled
constexpr int VOFF = KPOFF + BK * KP_ROW;   // 13312
constexpr int V_ROW = 256;                  // natural layout, 64 B blocks XOR-swizzled
constexpr int V_HEAD = BK * V_ROW;          // 8192
constexpr int STAGE = VOFF + G * V_HEAD;    // 21504

// Copies per tile in 1 KiB chunks (one wave-instruction of 64 x 16 B each):
// chunks [0, CK) k_nope (padded to whole chunks), [CK, CKP) rotated key,
// [CKP, NCHUNK) V.  Only the first
// NCW waves copy (the SIMD gives them its matrix core first, so they reach
// the end of a step early and issue the copies while the other waves still
// compute); each issues the same number (the spare ones repeat a chunk another
// wave also copies, writing identical bytes), so one vmcnt count fits all.
constexpr int NCHUNK = STAGE / 1024;           // 21
constexpr int CK = KPOFF / 1024;               // 9
constexpr int CKP = VOFF / 1024;               // 13
constexpr int NCW = 2;                         // waves that copy
constexpr int DPW = (NCHUNK + NCW - 1) / NCW;  // 11 copies per copying wave per tile
static_assert(STAGE % 1024 == 0 && KPOFF % 1024 == 0 && VOFF % 1024 == 0, "chunk layout");
static_assert(NSTAGE * STAGE <= 160 * 1024, "LDS budget");
static_assert(BQ * kV * 2 <= NSTAGE * STAGE, "the staged output tile fits the stages");
static_assert((NSTAGE - 2) * DPW < 64, "vmcnt range");
static_assert(NCHUNK - NCW >= CKP, "spare copies repeat V chunks");

// Tile-local key held in LDS row R of a 32-key block: the key that A-operand
// lane R fetches.  Accumulator register r of lane (n, h) is row
// (r/4)*8 + h*4 + r%4; with this order it holds key (r/4 >> 1)*16 + h*8 +
// (r/4 & 1)*4 + r%4, so lane half h owns keys h*8..h*8+7 of every 16-key
// chunk in 8 consecutive registers -- the B-operand layout of the PV product.
__device__ __forceinline__ int akey(int R) {
  const int g4 = R >> 3, h = (R >> 2) & 1, i = R & 3;
  return (g4 >> 1) * 16 + h * 8 + (g4 & 1) * 4 + i;
}

// XOR swizzle of the 16 B chunks of a 128 B rotated-key row: distinct for any
// 8 consecutive rows and for same-parity rows among 16 consecutive ones.
__device__ __forceinline__ int kpswz(int R) { return (R ^ (R >> 3)) & 7; }

__shared__ __attribute__((aligned(1024))) uint8_t lds[NSTAGE * STAGE];


__device__ __forceinline__ float max3(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// VB: V key-blocked, [B][H][ceil(LK/16)][128][16] (past = 0 only).
template <bool VB>
__global__ __launch_bounds__(NT) void prefill_kernel(PrefillParams p) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int ln = lane & 31;
  const int hf = lane >> 5;

  const int H = p.H, T = p.T;
  const int past = p.past, LK = p.LK;  // key positions 0 .. past+T-1, LK rows per head
  const int HG = (H + G - 1) / G;
  const int NQ = (T + BQ - 1) / BQ;
  const int NP = p.paired ? (NQ + 1) / 2 : NQ;  // query-tile pairs (or single tiles)
  const int U = p.B * HG;       // (sequence, head group) units

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

  // ---- asynchronous tile copies.  Copy i of copying wave w moves chunk
  // j = (w + NCW i) (a spare copy repeats chunk j - NCW).  Lane offsets inside the
  // head's rows are fixed; the buffer descriptor's base advances with the tile.
  // One descriptor per tensor and (sequence, head), whose extent ends at the
  // last row that holds data (position past+T-1): rows beyond it read as zero,
  // so cache rows the caller never wrote (any bit pattern, NaN included) reach
  // neither the scores nor the value product.
  static_assert(G == 1, "per-head copy descriptors assume one head per workgroup");
  uint32_t voff[DPW];
  int kind[DPW];  // 0 k_nope, 1 rotated key, 2 V (wave-uniform)
#pragma unroll
  for (int i = 0; i < DPW; ++i) {
    int j = (wave % NCW) + NCW * i;
    if (j >= NCHUNK) j -= NCW;
    uint32_t v;
    if (j < CK) {
      const int s = j * 64 + lane;  // slot in the k_nope region (17 per row)
      const int gg = s / (BK * 17);
      const int s2 = s % (BK * 17);
      int R = s2 / 17;
      int c = s2 % 17;
      if (c == 16) c = 15;  // pad slot: harmless duplicate
      if (gg >= G) {        // slot in the padding after the last head: duplicate too
        R = BK - 1;
        c = 15;
      }
      v = (uint32_t)akey(R) * 256u + c * 16;
      kind[i] = 0;
    } else if (j < CKP) {
      const int s = (j - CK) * 64 + lane;  // slot in the rotated-key region (8 per row)
      const int R = s / 8;
      const int c = (s % 8) ^ kpswz(R);
      v = (uint32_t)(akey(R) * 128 + c * 16);
      kind[i] = 1;
    } else if (!VB) {
      const int s = (j - CKP) * 64 + lane;  // slot in the V region (16 per row)
      const int row = s / 16;
      const int c = (s % 16) ^ ((row & 3) << 2);
      v = (uint32_t)row * 256u + c * 16;
      kind[i] = 2;
    } else {
      // Key-blocked V: the tile is two 4 KiB blocks [128 features][16 keys];
      // feature d's 32-byte row keeps its key halves swapped when d & 8, so
      // that 16 lanes reading 16 consecutive features hit 64 distinct banks.
      const int s = (j - CKP) * 64 + lane;
      const int blk = s >> 8, d = (s >> 1) & 127, half = (s & 1) ^ ((d >> 3) & 1);
      v = (uint32_t)(blk * 4096 + d * 32 + half * 16);
      kind[i] = 2;
    }
    voff[i] = v;
  }
  const int headc = head_ok ? head : H - 1;
  const uint16_t* khead = p.k_nope + ((size_t)b * H + headc) * LK * kNope;
  const int LKV = VB ? (LK + 15) / 16 * 16 : LK;  // V rows per head (whole blocks when blocked)
  const uint16_t* vhead = p.v + ((size_t)b * H + headc) * LKV * kV;
  const uint16_t* pseq = p.kpe_rot + (size_t)b * LK * kRope;
  const uint32_t nvis = (uint32_t)(past + p.T);  // rows 0 .. past+T-1 hold data
  // Blocked V: the extent covers whole 16-key blocks.  When the last block is
  // partial, its slots past the data may hold any bits, so the tile holding
  // it is read from the zero-padded copy in the workspace instead.
  const uint32_t nvis_v = VB ? (nvis + 15u) / 16u * 16u : nvis;
  const int kt_tail = (VB && (nvis & 15u)) ? (int)((nvis - 1) / BK) : -1;
  const uint16_t* vtail = VB && p.v_tail ? p.v_tail + ((size_t)b * H + headc) * kVTileElems : nullptr;

  // Copies of one tile: descriptors whose base advances with the tile, and the
  // stage they fill.  Past the last tile the descriptors are empty (nothing is
  // read; the copies write zeros into a stage no later tile of the pass uses),
  // so every step issues the same number of copies.
  struct Copies {
    __amdgpu_buffer_rsrc_t rK, rP, rV;
    uint8_t* buf;
  };
  auto plan = [&](uint8_t* buf, int kt, int nkt) {
    const bool live = kt < nkt;
    const uint32_t k0 = live ? (uint32_t)(kt * BK) : 0u;
    Copies c;
    // live tiles start below kend <= nvis, so the extents are positive
    c.rK = make_rsrc(khead + (size_t)k0 * kNope, live ? (nvis - k0) * 256u : 0u);
    c.rP = make_rsrc(pseq + (size_t)k0 * kRope, live ? (nvis - k0) * 128u : 0u);
    const bool tail = live && kt == kt_tail;
    c.rV = make_rsrc(tail ? vtail : vhead + (size_t)k0 * kV,
                     tail ? (uint32_t)kVTileElems * 2u : live ? (nvis_v - k0) * 256u : 0u);
    c.buf = buf;
    return c;
  };
  auto copy_one = [&](const Copies& c, int i) {
    int j = (wave % NCW) + NCW * i;
    if (j >= NCHUNK) j -= NCW;
    uint8_t* dst = c.buf + j * 1024;
    if (kind[i] == 0)
      dma16(c.rK, dst, voff[i]);
    else if (kind[i] == 1)
      dma16(c.rP, dst, voff[i]);
    else
      dma16(c.rV, dst, voff[i]);
  };
  auto copy_all = [&](const Copies& c) {
    if (wave >= NCW) return;
#pragma unroll
    for (int i = 0; i < DPW; ++i) copy_one(c, i);
  };

  // Zero the stages once, so rows that a copy leaves unwritten hold finite values.
  for (int o = tid * 16; o < NSTAGE * STAGE; o += NT * 16)
    *reinterpret_cast<u32x4*>(lds + o) = u32x4{0, 0, 0, 0};
  __syncthreads();

  // Per-lane LDS addresses for the products.
  const int k_lane = g * K_HEAD + ln * K_ROW + hf * 16;  // + kb*32
  int kp_lane[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) kp_lane[kb] = KPOFF + ln * KP_ROW + (((kb * 2 + hf) ^ kpswz(ln)) * 16);
  const int q16 = lane >> 4, s16 = lane & 15;
  // ds_read_b64_tr_b16: lane s of a 16-lane group addresses key row
  // (q16/2)*8 + t*4 + s/4 of a 16-key chunk, dims (q16%2)*16 + (s%4)*4 .. +3 of a
  // 32-dim block; lane i of the group then receives dim (q16%2)*16 + i of the
  // block for those four keys.
  const int v_row = (q16 >> 1) * 8 + (s16 >> 2);
  int v_lane[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
    v_lane[db] = VOFF + g * V_HEAD + v_row * V_ROW +
                 (((db ^ (s16 >> 2)) * 4 + (q16 & 1) * 2 + ((s16 & 3) >> 1)) * 16) + (s16 & 1) * 8;
  // blocked V: lane (ln, hf) reads feature db*32 + ln, keys c*16 + hf*8 .. +7
  const int vb_lane = VOFF + ln * 32 + ((hf ^ ((ln >> 3) & 1)) * 16);  // + c*4096 + db*1024

  const float cl2 = p.scale_log2;
  const uint32_t ones = 0x3f803f80u;  // bf16 pair (1, 1)
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

  const int npass = (!p.paired || pair == NQ - 1 - pair) ? 1 : 2;
  for (int pass = 0; pass < npass; ++pass) {
    const int qt = pass == 0 ? NQ - 1 - pair : pair;  // longer tile first
    const int q0 = qt * BQ + qb * 32;
    const int myq = q0 + ln;
    const int myqc = myq < T ? myq : T - 1;
    const int kend = past + min(T, qt * BQ + BQ);  // keys of the tile's last query, plus one
    const int nkt = (kend + BK - 1) / BK;

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

    // ---- first copies of the pass, issued after the query loads so that
    // waiting for those does not wait for the copies (the previous pass ended
    // with all waves past their last LDS read and no copy outstanding)
    auto stage = [&](int kt) { return lds + (kt % NSTAGE) * STAGE; };

#pragma unroll
    for (int st = 0; st < NSTAGE - 1; ++st) copy_all(plan(stage(st), st, nkt));

    float m_run = -INFINITY;  // reference maximum of scaled scores (base 2)
    float l_run = 0.f;        // this lane's share of the row sum
    f32x16 acc[4] = {};       // Oᵀ: dims db*32 + (r/4)*8 + hf*4 + r%4, query ln

    // Scores, softmax and PV of key tile kt held in stage `buf`.
    auto compute = [&](const uint8_t* buf, int kt) {
      const int k0 = kt * BK;
      bf16x8 kf[12];
      const uint8_t* kr = buf + k_lane;
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) kf[kb] = *reinterpret_cast<const bf16x8*>(kr + kb * 32);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) kf[8 + kb] = *reinterpret_cast<const bf16x8*>(buf + kp_lane[kb]);
      __builtin_amdgcn_sched_barrier(0);
      f32x16 s = {};
#pragma unroll
      for (int kb = 0; kb < 12; ++kb) s = mfma32x32x16(kf[kb], qf[kb], s);
      if (k0 + BK - 1 > past + q0) {  // the tile on this wave's diagonal
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + ((r >> 3) * 16) + hf * 8 + ((r >> 2) & 1) * 4 + (r & 3);
          if (key > past + myq) s[r] = -INFINITY;
        }
      }
      float mx = max3(s[0], s[1], s[2]);
#pragma unroll
      for (int r = 3; r < 15; r += 2) mx = max3(mx, s[r], s[r + 1]);
      mx = fmaxf(mx, s[15]);
      mx = max_halves(mx) * cl2;
      if (__builtin_amdgcn_ballot_w64(mx > m_run + TAU) != 0) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = fast_exp2(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db) acc[db] *= alpha;
        m_run = m_new;
      }
      bf16x8 pf[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = fast_exp2(fmaf(s[c * 8 + 2 * e], cl2, -m_run));
          const float p1 = fast_exp2(fmaf(s[c * 8 + 2 * e + 1], cl2, -m_run));
          // (a scalar: __builtin_bit_cast of a vector element reads element 0)
          const uint32_t pk = pack_bf16x2(p0, p1);
          w[e] = pk;
          l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk),
                                                  __builtin_bit_cast(bf16x2, ones), l_run, false);
        }
        pf[c] = as_bf16x8(w);
      }
      bf16x8 vf[4][2];
      if constexpr (VB) {
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int c = 0; c < 2; ++c)
            vf[db][c] = *reinterpret_cast<const bf16x8*>(buf + vb_lane + c * 4096 + db * 1024);
      } else {
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const uint8_t* vr = buf + v_lane[db];
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const s16x4 lo = ds_read_tr(vr + c * 16 * V_ROW);
            const s16x4 hi = ds_read_tr(vr + c * 16 * V_ROW + 4 * V_ROW);
            vf[db][c] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int db = 0; db < 4; ++db) acc[db] = mfma32x32x16(vf[db][c], pf[c], acc[db]);
    };

    // Wait until this wave's copies of tile kt are done (copies of tiles
    // kt+1 and kt+2, when issued, may still be in flight), then barrier: after
    // it every wave's copies of tile kt have landed and every wave has left
    // the stage that the next copy overwrites.
    auto wait_tile = [&](int kt) {
      (void)kt;
      wait_vm<(NSTAGE - 2) * DPW>();  // later tiles' (possibly empty) copies may still be in flight
      barrier_lds();
    };

    wait_tile(0);
    // Iteration kt: multiply tile kt, then copy tile kt+3 into the stage tile
    // kt-1 used (every wave left it before the barrier that opened this
    // iteration) just before waiting at the barrier for tile kt+1.
    auto step = [&](uint8_t* cur, uint8_t* ahead, int kt) {
      if (head_ok && kt * BK <= past + q0 + 31) compute(cur, kt);
      copy_all(plan(ahead, kt + NSTAGE - 1, nkt));
      if (kt + 1 < nkt) wait_tile(kt + 1);
    };
    for (int kt = 0; kt < nkt; ++kt) step(stage(kt), stage(kt + NSTAGE - 1), kt);
    wait_vm<0>();   // the empty copies past the last tile are done too
    barrier_lds();  // every wave is done with the stages before the next pass refills them

    // ---- epilogue
    if (head_ok && p.out8) {
      // FP8 output: the bf16-rounded outputs of this query and head (64 per
      // lane, the other 64 in lane ^ 32) are one 128-column block of the
      // o_proj input; scale = max(block amax, 1e-4) / 448, codes e4m3(x /
      // scale) with the quotients those of correctly rounded divisions (via
      // div_by_scale) -- the arithmetic of the activation quantizer, so the
      // codes equal its codes of the bf16 output.
      const float l_tot = sum_halves(l_run);
      const float inv = 1.0f / l_tot;
      float amax = 0.f;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          acc[db][r] = (float)f32_to_bf16(acc[db][r] * inv);
          amax = fmaxf(amax, fabsf(acc[db][r]));
        }
      const float sc = fmaxf(max_halves(amax), 1e-4f) / 448.0f;
      const float ry = 1.0f / sc;
      if (myq < T) {
        const size_t row = (size_t)b * T + myq;
        uint8_t* dst = p.out8 + row * ((size_t)H * kV) + (size_t)head * kV;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            int w = 0;
            w = __builtin_amdgcn_cvt_pk_fp8_f32(div_by_scale(acc[db][gq * 4 + 0], sc, ry),
                                                div_by_scale(acc[db][gq * 4 + 1], sc, ry), w, false);
            w = __builtin_amdgcn_cvt_pk_fp8_f32(div_by_scale(acc[db][gq * 4 + 2], sc, ry),
                                                div_by_scale(acc[db][gq * 4 + 3], sc, ry), w, true);
            *reinterpret_cast<uint32_t*>(dst + db * 32 + gq * 8 + hf * 4) = (uint32_t)w;
          }
        if (hf == 0) {
          p.out_sT[(size_t)head * act_scale_stride(p.B * T) + row] = sc;
          if (p.lse)
            p.lse[((size_t)b * H + head) * T + myq] = (m_run + log2f(l_tot)) * 0.69314718055994530942f;
        }
      }
    } else if (head_ok && !p.out_f32) {
      // bf16 output: the workgroup's 256 query rows x 256 B go through LDS
      // (free: every wave is past its last tile) so that each global store
      // writes whole lines of a row; a lane's own results are 8-byte pieces
      // of 32 rows.  Row q keeps its 16-byte chunk c at c ^ (q mod 16).
      const float l_tot = sum_halves(l_run);
      const float inv = 1.0f / l_tot;
      const int q = qb * 32 + ln;  // tile-local row
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int c = db * 4 + gq;
          *reinterpret_cast<u32x2*>(lds + q * 256 + ((c ^ (q & 15)) * 16) + hf * 8) =
              u32x2{pack_bf16x2(acc[db][gq * 4 + 0] * inv, acc[db][gq * 4 + 1] * inv),
                    pack_bf16x2(acc[db][gq * 4 + 2] * inv, acc[db][gq * 4 + 3] * inv)};
        }
      if (p.lse && hf == 0 && myq < T)
        p.lse[((size_t)b * H + head) * T + myq] = (m_run + log2f(l_tot)) * 0.69314718055994530942f;
      barrier_lds();
      const int c = lane & 15;
#pragma unroll
      for (int rr = 0; rr < BQ / (4 * NW); ++rr) {
        const int r = (rr * NW + wave) * 4 + (lane >> 4);
        const int t = qt * BQ + r;
        if (t >= T) continue;
        *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p.out) + ((size_t)b * T + t) * ((size_t)H * kV) +
                                  (size_t)head * kV + c * 8) =
            *reinterpret_cast<const u32x4*>(lds + r * 256 + ((c ^ (r & 15)) * 16));
      }
      barrier_lds();  // every wave has read the staged rows before the next pass's copies
    } else if (head_ok) {
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
  PrefillParams q = p;
  // Pairs balance causal work; single tiles double the workgroups, which
  // matters when pairs would leave compute units idle.
  const long paired_blocks = (long)p.B * HG * ((NQ + 1) / 2);
  q.paired = paired_blocks >= 2 * kComputeUnits ? 1 : 0;
  const long blocks = (long)p.B * HG * (q.paired ? (NQ + 1) / 2 : NQ);
  if (blocks <= 0 || blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
  if (p.v_blocked) {
    if (p.past != 0 || p.LK != p.T || (p.T % 16 != 0 && !p.v_tail)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(prefill_kernel<true>, dim3((unsigned)blocks), dim3(NT), 0, stream, q);
  } else {
    hipLaunchKernelGGL(prefill_kernel<false>, dim3((unsigned)blocks), dim3(NT), 0, stream, q);
  }
  return hipGetLastError();
}

}  // namespace mla
