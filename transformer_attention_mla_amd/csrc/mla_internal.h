// Internal declarations shared by the HIP kernels and the C-ABI layer of the
// MLA library.  Not installed; the public interface is include/mla.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

// Head widths of Kimi K2's latent attention (config.json on the page "Block
// input": qk_nope_head_dim, qk_rope_head_dim, v_head_dim).
constexpr int kNope = 128;
constexpr int kRope = 64;
constexpr int kPairs = 32;
constexpr int kQK = kNope + kRope;  // 192
constexpr int kV = 128;
constexpr int kComputeUnits = 256;  // MI355X (gfx950): 8 XCDs x 32 CUs

constexpr size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ---------------------------------------------------------------- prefill --
struct PrefillWorkspace {
  size_t cs_off, cs_bytes;    // float2 [T][32]: (cos, sin) of R[t][i]
  size_t kpe_off, kpe_bytes;  // bf16 [B][T][64]: rotated shared key
  // When T % 16 != 0: bf16 [B][H][2][128][16], per head the key-blocked value
  // tile (blocks 2*((T-1)/32) and the next) with the slots of positions T..
  // zeroed, read instead of v's own last tile (used with key-blocked v only).
  size_t vtail_off, vtail_bytes;
  size_t total;
};

constexpr int kVTileElems = 2 * 16 * 128;  // one 32-key tile of key-blocked V

inline PrefillWorkspace prefill_workspace_layout(int B, int H, int T) {
  PrefillWorkspace w;
  w.cs_off = 0;
  w.cs_bytes = align_up((size_t)T * kPairs * 8, 256);
  w.kpe_off = w.cs_off + w.cs_bytes;
  w.kpe_bytes = align_up((size_t)B * T * kRope * 2, 256);
  w.vtail_off = w.kpe_off + w.kpe_bytes;
  w.vtail_bytes = (T % 16) ? align_up((size_t)B * H * kVTileElems * 2, 256) : 0;
  w.total = w.vtail_off + w.vtail_bytes;
  return w;
}

struct PrefillParams {
  const uint16_t* q_nope;  // [B][H][T][128]
  const uint16_t* q_pe;    // [B][H][T][64], unrotated
  const uint16_t* k_nope;  // [B][H][LK][128]
  const uint16_t* k_pe;    // [B][T][64] unrotated (rotated by the prologue), or null
  const uint16_t* v;       // [B][H][LK][128]
  const float* R;
  float2* cs;          // workspace: (cos, sin) of the queries' positions, [T][32]
  uint16_t* kpe_rot;   // rotated shared key [B][LK][64]: workspace, or the caller's cache
  void* out;
  float* lse;
  int B, H, T;
  int past;            // queries sit at positions past .. past+T-1 and see keys 0 .. past+t
  int LK;              // rows per (sequence, head) of k_nope / v and per sequence of kpe_rot
  float scale_log2;    // softmax_scale * log2(e)
  int out_f32;
  int paired;          // set by launch_prefill: 1 = a workgroup takes query tiles i and NQ-1-i
  // FP8 output instead of `out` (when out8 is set): the bf16-rounded outputs
  // quantized as launch_act_quant quantizes the o_proj input, one 128-column
  // block per (row b*T + t, head): codes out8 [B*T][H*128] e4m3, scales
  // out_sT [H][act_scale_stride(B*T)].
  uint8_t* out8 = nullptr;
  float* out_sT = nullptr;
  // V key-blocked (plain prefill only: past = 0, LK = T): v [B][H][ceil(T/16)][128][16],
  // element (b, h, t, d) at ((b*H + h)*ceil(T/16) + t/16)*2048 + d*16 + t%16.
  int v_blocked = 0;
  // With v_blocked and T % 16 != 0: per head the last key tile of v with its
  // slots past T zeroed ([B][H][kVTileElems], workspace; written by
  // launch_v_tail), which the kernel reads in place of that tile.
  uint16_t* v_tail = nullptr;
};

hipError_t launch_rope_prep(const PrefillParams& p, hipStream_t stream);
// p.v_tail from p.v (key-blocked; p.T % 16 != 0).
hipError_t launch_v_tail(const PrefillParams& p, hipStream_t stream);

// Rotary table and rotated shared key at positions r_off + t, t < T: cs[t]
// (when cs is set) and dst[b][dst_off + t] (rows of dst_rows) from k_pe[b][t]
// (when k_pe is set).
hipError_t launch_rope(const float* R, int r_off, const uint16_t* k_pe, float2* cs, uint16_t* dst,
                       int dst_rows, int dst_off, int B, int T, hipStream_t stream);
// Copy rows [B*H][T][128] to rows dst_off .. of [B*H][dst_rows][128] (bf16).
hipError_t launch_append_rows(const uint16_t* src, uint16_t* dst, int BH, int T, int dst_rows,
                              int dst_off, hipStream_t stream);
hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream);

// ----------------------------------------------------------------- decode --
struct DecodeParams {
  const uint16_t* q_nope;
  const uint16_t* q_pe;
  const uint16_t* k_cache;    // [B][H][L][192] joined keys, or [B][H][L][128] nope keys
  const uint16_t* kpe_cache;  // null (joined layout) or [B][L][64] rotated keys shared by heads
  const uint16_t* v_cache;
  const float* R;
  int q_pos;
  float scale_log2;
  int B, H, L;
  int splits;
  float* part;  // workspace [B][H][splits][kDecodePart] when splits > 1
  void* out;
  float* lse;
  int out_f32;
};

// One split partial: running max (base-2 scaled units), sum, 128 outputs,
// padded to 136 floats (544 bytes, a multiple of 16).
constexpr int kDecodePart = 136;

int decode_choose_splits(int B, int H, int L, int requested);
hipError_t launch_decode(const DecodeParams& p, hipStream_t stream);

// ---------------------------------------------------------- latent decode --
constexpr int kLatent = 512;      // kv_lora_rank
constexpr int kLatentPart = 520;  // split partial: max, sum, 6 pad, 512 outputs

struct LatentParams {
  const uint16_t* q_nope;  // [B][H][128]
  const uint16_t* q_pe;    // [B][H][64], unrotated
  const uint16_t* ckv;     // [B][L][512] cached latent
  const uint16_t* kpe;     // [B][L][64] rotated rope keys shared by heads
  const uint16_t* w_kv_b;  // [H*256][512]: per head 128 key rows, 128 value rows
  const float* R;
  int q_pos;
  float scale_log2;
  int B, H, L;
  int splits;
  uint16_t* q_lat;  // workspace [B][H][512] bf16: q_nope·W_uk
  float* o_lat;     // workspace [B][H][512]: normalised latent output
  float* part;      // workspace [B][H][splits][kLatentPart] when splits > 1
  float* lse;
  void* out;        // [B][H*128]
  int out_f32;
};

struct LatentWorkspace {
  size_t q_off, o_off, part_off, total;
};
LatentWorkspace latent_workspace_layout(int B, int H, int splits);
int latent_choose_splits(int B, int L, int requested);
hipError_t launch_decode_latent(const LatentParams& p, hipStream_t stream);

// ---------------------------------------------------------- up-projection --
constexpr int kQRank = 1536;  // q_lora_rank

// ----------------------------------------------------------------- o_proj --
struct OprojParams {
  const uint16_t* x;  // [M][K]
  const uint16_t* w;  // [N][K]
  void* y;            // [M][N]
  float* part;        // [splits][M][N] when splits > 1
  int M, K, N;
  int splits;
  int out_f32;
  int group_m;        // wide kernel: m-tiles per group of the tile order
  const uint8_t* w8;      // FP8 weight [N][K] (e4m3) instead of w, or null
  const float* w_scale;   // its float32 scales, [ceil(N/128)][ceil(K/128)]
  // FP8 activations (with w8): x8 [M][K] e4m3 codes and their scales
  // transposed, x_scaleT [K/128][act_scale_stride(M)] (set by act_quant); x is
  // then unused.
  const uint8_t* x8 = nullptr;
  const float* x_scaleT = nullptr;
  // Head-major split store (hd > 0; splits 1, bf16 weight): row m = b*T + t,
  // column n = h*hd + d goes to y [B][H][T][d0] at d < d0, else to y1
  // [B][H][T][hd-d0] at d - d0 (H = N / hd; hd and d0 multiples of 32).
  int hd = 0, d0 = 0, T = 0;
  void* y1 = nullptr;
  // y1 key-blocked (hd > 0): column h*hd + d (d >= d0) of row b*T + t goes to
  // y1 [B][H][ceil(T/16)][hd-d0][16] at ((b*H + h)*ceil(T/16) + t/16)*16*(hd-d0)
  // + (d-d0)*16 + t%16.
  int y1_blocked = 0;
};

int oproj_choose_splits(int M, int K, int N, bool fp8 = false);
// FP8 weight at large M: dequantize it once (bf16 [N][K] into the workspace)
// and run the wide bf16 kernel when this holds.
bool oproj_fp8_wide(int M, int K, int N);
hipError_t launch_dequant_fp8(const uint8_t* w8, const float* w_scale, uint16_t* w, int N, int K,
                              hipStream_t stream);
hipError_t launch_oproj(const OprojParams& p, hipStream_t stream);

// Row stride of the transposed activation scales: M rounded up to 4 floats,
// so every slab's row of scales starts 16-byte aligned.
constexpr int act_scale_stride(int M) { return (M + 3) & ~3; }

// FP8 activations: x [M][K] bf16 -> x8 [M][K] e4m3 and x_scaleT [K/128][stride]
// (per row and 128-column block: scale = max(amax, 1e-4) / 448, codes
// e4m3(x / scale) rounded to nearest even).  K % 128 == 0.
hipError_t launch_act_quant(const uint16_t* x, uint8_t* x8, float* x_scaleT, int M, int K,
                            hipStream_t stream);
// y = (x8, x_scaleT) · (w8, w_scale)ᵀ with FP8 MFMA; splits > 1: float32
// partials in p.part, then a reduction.
int oproj_fp8dyn_splits(int M, int K, int N);
hipError_t launch_oproj_fp8dyn(const OprojParams& p, hipStream_t stream);

}  // namespace mla
