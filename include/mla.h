/*
 * mla.h — C ABI of the MI355X (gfx950) library for Kimi K2's latent-attention
 * (MLA) attend-and-combine step.
 *
 * What the calls compute (the pages' notation):
 *   page "Kimi K2 · Mix and project", code excerpt "mla-prefill": the 64-wide
 *   rotary parts of query and key are rotated; each head's 192-wide query and
 *   key are the 128-wide non-rotated part followed by the rotated part, the
 *   key's rotated part being one tensor shared by every head; scores
 *   Q·Kᵀ·softmax_scale get the additive causal mask, a float32 softmax over
 *   keys, and mix the 128-wide values.  Excerpt "mla-output": head outputs are
 *   transposed to [B, T, 64·128] (head-major) and go through o_proj, an
 *   8,192 → 7,168 linear map without bias (the parameter table of that page;
 *   per the page's explanation, no earlier step combines different heads).
 *   page "Kimi K2 · Transformer blocks", I/O header: R [T positions, 32 pairs]
 *   and the causal mask M [T queries, T keys]; in the model-body excerpt the
 *   position ids start right after the tokens already cached (at 0 for a
 *   prefill without cache).
 *   page "Block input", config.json: 64 heads, qk_nope_head_dim 128,
 *   qk_rope_head_dim 64, v_head_dim 128, attention_bias false, bfloat16.
 *
 * Conventions shared by every call
 *   - Tensors are contiguous, row-major.  "bf16" arguments point at IEEE
 *     bfloat16 values (their 16-bit patterns; mla_bf16 below).
 *   - Every pointer argument is DEVICE memory owned by the caller; the library
 *     allocates nothing, keeps no pointer after the call returns and has no
 *     global state besides a per-device architecture check.
 *   - Pointers must be 16-byte aligned.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     runs asynchronously; the library never synchronises.
 *   - All validation happens before anything is enqueued.  On any error
 *     nothing is enqueued and no output byte is written.  The library never
 *     aborts or throws across this boundary.
 *   - Outputs are fully overwritten; inputs are read only.  Outputs may not
 *     overlap inputs or each other (MLA_ERR_ALIAS).
 *   - Rotary reading: pair i (0..31) couples elements i and i+32 of the
 *     64-wide rotary part; at position t it turns by angle R[t][i]:
 *       y_i = x_i·cos − x_{i+32}·sin,  y_{i+32} = x_{i+32}·cos + x_i·sin.
 *     Rotated parts are rounded to bf16 (they are bf16 query/key tensors).
 *   - Rounding of every float → bf16 store is round-to-nearest-even.
 *   - Thread safety: calls are reentrant; concurrent calls on different
 *     streams are independent.
 */
#ifndef MLA_H
#define MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 16-bit pattern of an IEEE bfloat16 value. */
typedef uint16_t mla_bf16;

typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULL = 1,      /* a required pointer is NULL */
  MLA_ERR_DIM = 2,       /* a size is <= 0, inconsistent, or exceeds the angle table */
  MLA_ERR_ALIGN = 3,     /* a pointer is not 16-byte aligned */
  MLA_ERR_ALIAS = 4,     /* an output overlaps an input or another output */
  MLA_ERR_WORKSPACE = 5, /* workspace missing or smaller than required */
  MLA_ERR_SCALE = 6,     /* softmax_scale is not finite or not > 0 */
  MLA_ERR_DEVICE = 7,    /* the current device is not gfx950 (or none) */
  MLA_ERR_LAUNCH = 8,    /* the runtime reported an error when enqueueing */
  MLA_ERR_FLAGS = 9      /* unknown bits in `flags` */
} mla_status;

#define MLA_ABI_VERSION 1

/* flags bit: store `out` / `y` as float32 instead of bf16.  The arithmetic is
 * identical; only the final store differs, so a bf16 result equals the
 * round-to-nearest-even of its float32 twin. */
#define MLA_OUT_F32 0x1u

/* flags bit for mla_attend_prefill (and its _fp8 and _noalloc forms) and
 * mla_up_project: `v` is held key-blocked instead of [B, H, T, 128]:
 *
 *   v  [B, H, NB, 128, 16] bf16, NB = ceil(T/16); value feature d of position
 *      t at element ((b*H + h)*NB + t/16)*2048 + d*16 + t%16
 *
 * i.e. each block of 16 consecutive positions is stored feature by feature.
 * The value product takes 8 consecutive keys of one feature per lane, which
 * in this layout are 16 contiguous bytes; from the natural layout the
 * attention kernel transposes them on every LDS read.  The slots of
 * positions T .. NB*16-1 in the last block of each head never reach a result
 * (any contents, NaN included) and mla_up_project leaves them unwritten.
 * Everything else (the results bit for bit included) is as without the bit. */
#define MLA_V_BLOCKED 0x2u

/* Version of this ABI (MLA_ABI_VERSION). */
int mla_abi_version(void);

/* Static, NUL-terminated name of a status code ("MLA_OK", ...); "unknown
 * status" for other values.  Never NULL. */
const char *mla_status_string(int status);

/* -------------------------------------------------------------- prefill --
 * Causal prefill attention over positions 0..T-1 (no cache), all heads.
 *
 *   q_nope  [B, H, T, 128] bf16   non-rotated query part
 *   q_pe    [B, H, T, 64]  bf16   rotary query part, NOT yet rotated
 *   k_nope  [B, H, T, 128] bf16   non-rotated key part
 *   k_pe    [B, 1, T, 64]  bf16   rotary key part, NOT yet rotated, shared by all heads
 *   v       [B, H, T, 128] bf16   values (key-blocked with MLA_V_BLOCKED)
 *   R       [r_rows, 32]   float  angle table in radians, row t = position t; T <= r_rows
 *   softmax_scale                 score multiplier (Kimi K2: 192^-0.5), finite and > 0
 *   workspace                     device scratch of >= mla_prefill_workspace_bytes(B,H,T)
 *                                 bytes (cos/sin table, the rotated shared key and,
 *                                 when T % 16 != 0, a zero-padded copy of each
 *                                 head's last key-blocked value tile)
 *   out     [B, T, H*128]  bf16, or float32 with MLA_OUT_F32; element
 *                          [b][t][h*128+d] is head h's output (head-major flatten)
 *   lse     [B, H, T] float natural-log sum of exp of the scaled, masked scores
 *                     per row, or NULL
 *
 * Row t of head h is softmax_j≤t(scale·(q_nope·k_noperᵀ + rot(q_pe)·rot(k_pe)ᵀ))·V.
 * flags: MLA_OUT_F32, MLA_V_BLOCKED (others MLA_ERR_FLAGS).
 * B, H, T >= 1 with any tails.  The softmax is evaluated online in float32 in
 * base 2; the weights that multiply V are rounded to bf16 and the row sum is
 * accumulated from those same rounded weights.
 */
size_t mla_prefill_workspace_bytes(int B, int H, int T);

int mla_attend_prefill(const mla_bf16 *q_nope, const mla_bf16 *q_pe, const mla_bf16 *k_nope,
                       const mla_bf16 *k_pe, const mla_bf16 *v, const float *R, int r_rows,
                       float softmax_scale, int B, int H, int T, void *workspace,
                       size_t workspace_bytes, void *out, float *lse, uint32_t flags,
                       void *stream);

/* mla_attend_prefill with the output already quantized for the FP8 o_proj
 * (page "Block input", config.json quantization_config: e4m3, activation
 * scheme "dynamic"): the kernel rounds each output to bf16, as
 * mla_attend_prefill stores it, and quantizes it in its epilogue exactly as
 * mla_act_quant would quantize that bf16 output -- head h's 128 values of
 * row b*T + t are one 128-column block of the o_proj input, so the block
 * maximum is taken across the lanes that hold them.  The separate
 * quantization pass (a read of the bf16 output, a write of the codes) is
 * thereby folded into the attention's own store.
 *
 *   out8        [B, T, H*128] uint8 e4m3 codes: the [M = B*T, K = H*128]
 *               input of mla_out_proj_fp8_q
 *   out_scaleT  [H, mla_act_scale_stride(B*T)] float32 scales (row m of
 *               block h at h * stride + m; columns B*T .. stride-1 are not
 *               written)
 *   lse         as for mla_attend_prefill (optional)
 * Other arguments and the errors as for mla_attend_prefill; out8 or
 * out_scaleT NULL is MLA_ERR_NULL, a flag bit other than MLA_V_BLOCKED
 * MLA_ERR_FLAGS, B*T >= 2^31
 * MLA_ERR_DIM, an output overlapping an input or another output
 * MLA_ERR_ALIAS.
 */
int mla_attend_prefill_fp8(const mla_bf16 *q_nope, const mla_bf16 *q_pe, const mla_bf16 *k_nope,
                           const mla_bf16 *k_pe, const mla_bf16 *v, const float *R, int r_rows,
                           float softmax_scale, int B, int H, int T, void *workspace,
                           size_t workspace_bytes, uint8_t *out8, float *out_scaleT, float *lse,
                           uint32_t flags, void *stream);

/* Allocation-free variant of mla_attend_prefill, for callers that cannot
 * allocate device memory or pass a workspace: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments,
 * computation and results (bit for bit) as mla_attend_prefill, without
 * `workspace` / `workspace_bytes`: the cos/sin table and the rotated shared key
 * (and, when T % 16 != 0, the zero-padded last value tile of each head) go to
 * a static buffer of MLA_PREFILL_NOALLOC_SCRATCH_BYTES that each GPU holds for
 * the life of the process.  The call needs mla_prefill_workspace_bytes(B, H, T)
 * = T·256 + B·T·128 (+ B·H·8192 when T % 16 != 0) bytes (each part rounded up
 * to 256); sizes beyond MLA_PREFILL_NOALLOC_SCRATCH_BYTES (16 MiB:
 * e.g. B·T up to 98,304 positions at T = 16384, 129,024 at T = 1024) return
 * MLA_ERR_WORKSPACE before anything is enqueued.  No device memory is
 * allocated or freed by this call.  Every call on one GPU uses that GPU's
 * single buffer, so calls that overlap in time on one GPU (other streams,
 * other host threads) race and must be serialised by the caller; the buffer
 * needs no clearing (each call writes what it reads).  Other errors as for
 * mla_attend_prefill. */
#define MLA_PREFILL_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

int mla_attend_prefill_noalloc(const mla_bf16 *q_nope, const mla_bf16 *q_pe,
                               const mla_bf16 *k_nope, const mla_bf16 *k_pe, const mla_bf16 *v,
                               const float *R, int r_rows, float softmax_scale, int B, int H,
                               int T, void *out, float *lse, uint32_t flags, void *stream);

/* KV-cache append (page "Kimi K2 · Mix and project", excerpt "mla-prefill": the
 * cache is updated with the keys after the rotary step; page "Kimi K2 ·
 * Transformer blocks": position ids start after the cached tokens): a chunk
 * of T positions goes to rows past .. past+T-1 of a cache in the shared-rotary
 * layout, the rope key rotated at its position (R row past + t) and rounded to
 * bf16 with the same arithmetic as the prefill's own rotation.
 *
 *   k_nope [B, H, T, 128], k_pe [B, 1, T, 64] (unrotated), v [B, H, T, 128]
 *   k_nope_cache [B, H, L_cap, 128], kpe_cache [B, L_cap, 64], v_cache
 *   [B, H, L_cap, 128]   caller-owned, written at rows past .. past+T-1 only
 *   R [r_rows, 32]; past >= 0, past + T <= L_cap and <= r_rows (else MLA_ERR_DIM)
 *   flags must be 0.
 */
int mla_append_kv(const mla_bf16 *k_nope, const mla_bf16 *k_pe, const mla_bf16 *v, const float *R,
                  int r_rows, int past, int B, int H, int T, int L_cap, mla_bf16 *k_nope_cache,
                  mla_bf16 *kpe_cache, mla_bf16 *v_cache, uint32_t flags, void *stream);

/* Chunked prefill over the cache (same pages): the T queries sit at positions
 * past .. past+T-1 (q_pe rotated with R rows past + t) and query t sees cache
 * rows 0 .. past+t (the chunk's own keys appended first, with mla_append_kv).
 * With past = 0 and the chunk appended at 0 this is mla_attend_prefill.
 *
 *   q_nope [B, H, T, 128], q_pe [B, H, T, 64] (unrotated); caches as for
 *   mla_append_kv, holding rows 0 .. past+T-1; out [B, T, H*128], lse [B, H, T]
 *   workspace >= mla_prefill_chunk_workspace_bytes(T) bytes (cos/sin table)
 *   H * L_cap * 256 must fit in 32 bits (else MLA_ERR_DIM); other arguments
 *   and errors as for mla_attend_prefill.
 */
size_t mla_prefill_chunk_workspace_bytes(int T);

int mla_attend_prefill_chunk(const mla_bf16 *q_nope, const mla_bf16 *q_pe,
                             const mla_bf16 *k_nope_cache, const mla_bf16 *kpe_cache,
                             const mla_bf16 *v_cache, const float *R, int r_rows, int past,
                             float softmax_scale, int B, int H, int T, int L_cap, void *workspace,
                             size_t workspace_bytes, void *out, float *lse, uint32_t flags,
                             void *stream);

/* --------------------------------------------------------------- decode --
 * One new query per sequence against L cached keys (page "Kimi K2 · Mix and
 * project", excerpt "mla-prefill": the cache stores keys after the rotary step,
 * as [non-rotated 128 | rotated 64], and values).
 *
 *   q_nope  [B, H, 128]     bf16   non-rotated query part
 *   q_pe    [B, H, 64]      bf16   rotary query part, NOT yet rotated; rotated at q_pos
 *   k_cache [B, H, L, 192]  bf16   cached keys, already rotated
 *   v_cache [B, H, L, 128]  bf16   cached values
 *   R       [r_rows, 32]    float  angle table; 0 <= q_pos < r_rows
 *   num_splits                     key-range splits per (b, h); 0 = library's choice,
 *                                  otherwise 1..L (larger values are clamped to L)
 *   workspace                      >= mla_decode_workspace_bytes(B, H, L, num_splits)
 *                                  bytes (0 bytes, NULL allowed, when one split is used)
 *   out     [B, H*128]      bf16, or float32 with MLA_OUT_F32 (head-major)
 *   lse     [B, H]          float natural-log row lse, or NULL
 *
 * Every one of the L keys is visible.  Split partials (running max, sum and
 * unnormalised output in float32) are merged by the log-sum-exp rule.
 */
size_t mla_decode_workspace_bytes(int B, int H, int L, int num_splits);

/* Number of splits the library uses for (B, H, L, num_splits). */
int mla_decode_splits(int B, int H, int L, int num_splits);

int mla_attend_decode(const mla_bf16 *q_nope, const mla_bf16 *q_pe, const mla_bf16 *k_cache,
                      const mla_bf16 *v_cache, const float *R, int r_rows, int q_pos,
                      float softmax_scale, int B, int H, int L, int num_splits, void *workspace,
                      size_t workspace_bytes, void *out, float *lse, uint32_t flags,
                      void *stream);

/* Decode against a cache that keeps the rotated rope key once per position
 * for all heads (page "Kimi K2 · Mix and project": the key's rotated part is
 * one shared tensor for every head; the cache stores keys after the rotary
 * step).  Same computation as mla_attend_decode with the joined key row
 * [k_nope_cache[b,h,j] | kpe_cache[b,j]]; each head reads 256 + 256 bytes of its own
 * per key instead of 384 + 256; the shared rope rows (128 bytes per key) serve
 * every head of the sequence.
 *
 *   k_nope_cache [B, H, L, 128]  bf16   non-rotated key parts
 *   kpe_cache    [B, L, 64]      bf16   rotated rope keys, one per position
 *   (all other arguments, the workspace size -- mla_decode_workspace_bytes --
 *   and the error behaviour as for mla_attend_decode; kpe_cache NULL is
 *   MLA_ERR_NULL, misaligned MLA_ERR_ALIGN, overlapping an output MLA_ERR_ALIAS)
 */
int mla_attend_decode_shared_kpe(const mla_bf16 *q_nope, const mla_bf16 *q_pe,
                                 const mla_bf16 *k_nope_cache, const mla_bf16 *kpe_cache,
                                 const mla_bf16 *v_cache, const float *R, int r_rows, int q_pos,
                                 float softmax_scale, int B, int H, int L, int num_splits,
                                 void *workspace, size_t workspace_bytes, void *out, float *lse,
                                 uint32_t flags, void *stream);

/* Decode against a latent cache.  Page "Block input" (config.json):
 * kv_lora_rank 512, and the dense-block parameter total fixes kv_b_proj as one
 * 512 -> H·(128+128) linear map; page "Kimi K2 · Mix and project": keys join a
 * per-head nope part with the rotated rope part shared by all heads.  The cache
 * keeps per position the 512-wide latent c (after its normalisation) and the
 * rotated rope key; head h's nope key is W[h·256 .. h·256+127]·c and its value
 * W[h·256+128 .. h·256+255]·c (W = kv_b_proj as the linear layer stores it,
 * [out, in]).  The result equals the shared-rotary decode on those up-projected
 * keys and values; the library computes it without forming them (query
 * absorbed into the latent, W_uv applied after the value mix), reading 1,152
 * bytes per position for all heads.
 *
 *   q_nope    [B, H, 128]     bf16   non-rotated query part
 *   q_pe      [B, H, 64]      bf16   rotary query part, rotated at q_pos
 *   ckv_cache [B, L, 512]     bf16   cached latent
 *   kpe_cache [B, L, 64]      bf16   rotated rope keys, one per position
 *   w_kv_b    [H*256, 512]    bf16   kv_b_proj weight
 *   R, r_rows, q_pos, softmax_scale, out [B, H*128], lse [B, H], flags, stream
 *                                    as for mla_attend_decode
 *   num_splits                       position-range splits per sequence; 0 =
 *                                    library's choice, else 1..L (clamped to L)
 *   workspace  >= mla_decode_latent_workspace_bytes(B, H, L, num_splits) bytes,
 *              always required (absorbed queries and latent outputs live there)
 *
 * Limits: 1 <= H <= 64 (all heads of a sequence share one workgroup),
 * 1 <= L < 2^21, 1 <= B <= 2^20; otherwise MLA_ERR_DIM.  Other errors as for
 * mla_attend_decode.
 */
size_t mla_decode_latent_workspace_bytes(int B, int H, int L, int num_splits);

int mla_attend_decode_latent(const mla_bf16 *q_nope, const mla_bf16 *q_pe,
                             const mla_bf16 *ckv_cache, const mla_bf16 *kpe_cache,
                             const mla_bf16 *w_kv_b, const float *R, int r_rows, int q_pos,
                             float softmax_scale, int B, int H, int L, int num_splits,
                             void *workspace, size_t workspace_bytes, void *out, float *lse,
                             uint32_t flags, void *stream);

/* --------------------------------------------------------------- o_proj --
 * y = x · w_oᵀ, the 8,192 → 7,168 output projection without bias (page "Kimi
 * K2 · Mix and project", parameter table and excerpt "mla-output").
 *
 *   x     [M, K]  bf16   flattened attention output (K = heads·128)
 *   w_o   [N, K]  bf16   the linear layer's weight as the layer stores it:
 *                        row n holds the K input weights of output feature n
 *   y     [M, N]  bf16, or float32 with MLA_OUT_F32
 *   workspace     >= mla_out_proj_workspace_bytes(M, K, N) bytes; the library
 *                 splits K for small M and keeps float32 partials there
 *
 * M, N >= 1, K >= 1 and a multiple of 128.  Accumulation is float32.
 */
size_t mla_out_proj_workspace_bytes(int M, int K, int N);

int mla_out_proj(const mla_bf16 *x, const mla_bf16 *w_o, void *y, int M, int K, int N,
                 void *workspace, size_t workspace_bytes, uint32_t flags, void *stream);

/* The same projection with the weight as the checkpoint stores it: FP8 values
 * with one float32 scale per 128 x 128 block (pages "Kimi K2 · Transformer
 * blocks" and "Kimi K2 · Mix and project": the parameter counts exclude the
 * FP8 block scales).  Each weight element is dequantized as the float32
 * product of its e4m3 value and its block's scale, rounded to bf16; then
 * y = x · w_oᵀ as in mla_out_proj.  The weight stream is half as large, which is
 * what bounds the projection at decode sizes.
 *
 *   w8       [N, K]                       uint8  e4m3 (OCP "fn": bias 7, no
 *                                                infinities, 0x7f/0xff NaN)
 *   w_scale  [ceil(N/128), K/128]         float  block scales, row-major
 *   workspace >= mla_out_proj_fp8_workspace_bytes(M, K, N) bytes.  At
 *            decode sizes it holds the float32 partials of split K; when
 *            y spans at least 256 tiles of 256 x 256 (M = 16384, N = 7168
 *            among them) it holds the whole dequantized weight, N*K*2
 *            bytes: the weight is converted once per call and the product
 *            then runs as mla_out_proj's, with identical results.  The
 *            workspace must not overlap x, w8, w_scale or y.
 *   (x, y, M, K, N, flags, stream and the errors as for mla_out_proj; w8 or
 *   w_scale NULL is MLA_ERR_NULL, misaligned MLA_ERR_ALIGN)
 */
size_t mla_out_proj_fp8_workspace_bytes(int M, int K, int N);

int mla_out_proj_fp8(const mla_bf16 *x, const uint8_t *w8, const float *w_scale, void *y, int M,
                     int K, int N, void *workspace, size_t workspace_bytes, uint32_t flags,
                     void *stream);

/* FP8 activations, the config's "dynamic" scheme (page "Block input",
 * config.json quantization_config: fmt e4m3, activation_scheme dynamic).  The
 * pages give no recipe for the run-time scales; this is the public recipe of
 * the model family's FP8 format (DeepSeek-V3 technical report, fine-grained
 * quantization, 1 x 128 activation tiles): per row m and 128-column block b,
 * scale = max(max |x[m, 128b .. 128b+127]|, 1e-4) / 448 and codes
 * e4m3(x / scale) (float32, the division correctly rounded, round to nearest
 * even).
 *
 *   x         [M, K] bf16, K a multiple of 128
 *   x8        [M, K] uint8 e4m3 codes (output)
 *   x_scaleT  [K/128, mla_act_scale_stride(M)] float scales, transposed
 *             (output; columns M .. stride-1 are not written)
 * All device pointers, 16-byte aligned, caller-owned.  Returns MLA_ERR_NULL,
 * MLA_ERR_DIM (M < 1, K not a multiple of 128, M*K >= 2^31), MLA_ERR_ALIGN,
 * MLA_ERR_ALIAS (an output overlapping x or the other output) before
 * enqueueing anything.  mla_out_proj_fp8_dyn runs the same quantizer.
 * mla_act_scale_stride returns M rounded up to 4 (0 for M out of range).
 */
int mla_act_scale_stride(int M);

int mla_act_quant(const mla_bf16 *x, int M, int K, uint8_t *x8, float *x_scaleT, void *stream);

/* o_proj in FP8 throughout: y = dequant(act_quant(x)) · dequant(w8, w_scale)ᵀ,
 * where a dequantized value is its e4m3 code times its block's scale (x: 1 x
 * 128 blocks from mla_act_quant, weight: 128 x 128 blocks as the checkpoint
 * stores them).  The products run on the FP8 matrix cores; each 128-deep slab
 * of the sum is scaled by its two block scales and accumulated in float32.
 *
 *   x, w8, w_scale, y, M, N, flags, stream as for mla_out_proj_fp8 (K a
 *   multiple of 128, at most 2^31 / 256 - 1)
 *   workspace >= mla_out_proj_fp8_dyn_workspace_bytes(M, K, N) bytes: the
 *   quantized activations and their scales (and float32 partials when the
 *   library splits K for M <= 64)
 */
size_t mla_out_proj_fp8_dyn_workspace_bytes(int M, int K, int N);

int mla_out_proj_fp8_dyn(const mla_bf16 *x, const uint8_t *w8, const float *w_scale, void *y,
                         int M, int K, int N, void *workspace, size_t workspace_bytes,
                         uint32_t flags, void *stream);

/* The product of mla_out_proj_fp8_dyn on activations already quantized (by
 * mla_act_quant, or by mla_attend_prefill_fp8 in its epilogue): y =
 * dequant(x8, x_scaleT) · dequant(w8, w_scale)ᵀ, the same kernels and results
 * as mla_out_proj_fp8_dyn on the input those codes came from.
 *
 *   x8        [M, K] uint8 e4m3 codes, K a multiple of 128
 *   x_scaleT  [K/128, mla_act_scale_stride(M)] float32 scales, transposed
 *   w8, w_scale, y, M, N, flags, stream as for mla_out_proj_fp8_dyn
 *   workspace >= mla_out_proj_fp8_q_workspace_bytes(M, K, N) bytes (float32
 *             partials when the library splits K for M <= 64; 0 otherwise,
 *             and then workspace may be NULL)
 * Errors as for mla_out_proj_fp8_dyn.
 */
size_t mla_out_proj_fp8_q_workspace_bytes(int M, int K, int N);

int mla_out_proj_fp8_q(const uint8_t *x8, const float *x_scaleT, const uint8_t *w8,
                       const float *w_scale, void *y, int M, int K, int N, void *workspace,
                       size_t workspace_bytes, uint32_t flags, void *stream);

/* ------------------------------------------------------- up-projection --
 * The MLA up-projection in front of the attention: the query from its
 * rank-1536 latent and the nope key and value from the rank-512 latent
 * (page "Block input", config.json: q_lora_rank 1536, kv_lora_rank 512, 64
 * heads of 128 nope + 64 rope query features and 128 value features; page
 * "Kimi K2 · Mix and project", excerpt "mla-prefill": each head's query is
 * its nope part then its rope part, and the key's nope part and the value
 * are read per head).  Two linear maps without bias, each weight held as the
 * linear layer holds it (row n = the input weights of output feature n):
 *
 *   q_lat   [B, T, 1536]  bf16   the query latent (after its normalisation)
 *   ckv     [B, T, 512]   bf16   the key/value latent (after its normalisation)
 *   w_q_b   [H*192, 1536] bf16   rows h*192 .. +127: head h's q_nope features,
 *                                rows h*192+128 .. +63: its q_pe features
 *   w_kv_b  [H*256, 512]  bf16   rows h*256 .. +127: head h's nope key,
 *                                rows h*256+128 .. +127: its value
 *   q_nope  [B, H, T, 128], q_pe [B, H, T, 64] (unrotated: the rotary step is
 *   the attention's), k_nope [B, H, T, 128], v [B, H, T, 128]: outputs in the
 *   layouts mla_attend_prefill takes; bf16, or float32 with MLA_OUT_F32; v
 *   key-blocked ([B, H, ceil(T/16), 128, 16], the slots past T unwritten)
 *   with MLA_V_BLOCKED.
 *
 * Float32 accumulation over the latent, one rounding per output.  No
 * workspace.  Errors: a NULL pointer MLA_ERR_NULL; B, T, H < 1 or too large
 * MLA_ERR_DIM; a pointer not 16-byte aligned MLA_ERR_ALIGN; an output
 * overlapping an input or another output MLA_ERR_ALIAS; unknown flag bits
 * MLA_ERR_FLAGS.  Asynchronous on `stream`.
 */
int mla_up_project(const mla_bf16 *q_lat, const mla_bf16 *ckv, const mla_bf16 *w_q_b,
                   const mla_bf16 *w_kv_b, int B, int T, int H, void *q_nope, void *q_pe,
                   void *k_nope, void *v, uint32_t flags, void *stream);

/* ------------------------------------------------------------------------
 * Measurement helper (not a step of the attention path): the rate the matrix
 * cores of this GPU sustain with every compute unit busy, clock and power
 * limits included -- the measured figures beside which the published peaks
 * and the kernels' rates are read.  One launch of 512 workgroups of 4 waves
 * (two waves per SIMD), each wave running `iters` rounds of four independent
 * MFMA chains on register operands, with no memory traffic in the loop:
 * kind 0 v_mfma_f32_32x32x16_bf16 (the attention and bf16 GEMM products),
 * kind 1 v_mfma_f32_32x32x64_f8f6f4 on e4m3 operands (the FP8 o_proj), each
 * on operands that stay the same from one instruction to the next; kinds 2
 * (bf16) and 3 (e4m3) cycle every chain through eight random operand sets,
 * so the matrix cores switch bits as on real data -- the switching power
 * then lowers the clock the chip holds, and these are the rates to read a
 * kernel on random inputs against.  Operand sets: xorshift32 (shifts 13, 17,
 * 5) seeded with 0x9e3779b9 * (thread + 1) xor iters, for each set and
 * element one draw for A then one for B (four per 4-byte group for e4m3):
 * bf16 A = ±(1 + (h & 0xffff)·2^-16), B = ±(0.5 + (h & 0xffff)·2^-17), the
 * sign from bit 16, rounded to nearest even; e4m3 byte = bit 7 of h>>7 (sign)
 * | (5 + (h>>3) mod 5) << 3 | (h & 7); chain c at step v (iteration 8j + v)
 * multiplies A set (v + c) mod 8 by B set (v + 3c) mod 8.  It performs
 * mla_mfma_probe_flops(iters, kind) floating-point operations (0 when iters
 * or kind is out of range).
 *
 *   out    device, float32, MLA_MFMA_PROBE_OUT elements, 16-byte aligned,
 *          caller-owned; receives per-thread sums of the products
 *   iters  1 .. 2^24 (a multiple of 8 for kinds 2 and 3), kind 0 .. 3 (else
 *          MLA_ERR_DIM)
 *
 * Errors: out NULL MLA_ERR_NULL, misaligned MLA_ERR_ALIGN, not gfx950
 * MLA_ERR_DEVICE.  Asynchronous on `stream`; time it with events on it.
 */
#define MLA_MFMA_PROBE_OUT (512 * 256)
double mla_mfma_probe_flops(int iters, int kind);
int mla_mfma_probe(float *out, int iters, int kind, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H */
