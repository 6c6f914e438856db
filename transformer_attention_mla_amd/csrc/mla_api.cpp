// C ABI of the MLA library (declared in include/mla.h): argument validation,
// workspace layout and kernel launches on the caller's stream.
//
// Error convention: the page "Kimi K2 · Mix and project" (code excerpt
// "mla-prefill") raises ValueError when the score or mask shapes are not
// (bsz, heads, q_len, kv_len) / (bsz, 1, q_len, kv_len) and asserts that a mask
// exists.  Here every such check becomes a status code returned before any
// work is enqueued; nothing is thrown or aborted across the boundary.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>

#include "mla.h"
#include "mla_internal.h"
#include "mla_probe.h"

namespace {

using mla::kNope;
using mla::kQK;
using mla::kRope;
using mla::kV;

constexpr long long kMaxDim = 1LL << 24;      // any single size
constexpr long long kMaxElems = 1LL << 40;    // any tensor

bool aligned16(const void* p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
  const void* p;
  size_t bytes;
};

bool overlap(Range a, Range b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Outputs may not overlap inputs or each other.
bool any_alias(const Range* in, int n_in, const Range* out, int n_out) {
  for (int i = 0; i < n_out; ++i) {
    for (int j = 0; j < n_in; ++j)
      if (overlap(out[i], in[j])) return true;
    for (int j = i + 1; j < n_out; ++j)
      if (overlap(out[i], out[j])) return true;
  }
  return false;
}

bool dims_ok(long long a, long long b, long long c, long long d) {
  if (a <= 0 || b <= 0 || c <= 0 || d <= 0) return false;
  if (a > kMaxDim || b > kMaxDim || c > kMaxDim || d > kMaxDim) return false;
  return a * b <= kMaxElems && a * b * c <= kMaxElems && a * b * c * d <= kMaxElems;
}

// The kernels are built for gfx950 only; check the current device once.
int check_device() {
  static std::atomic<int> cache[64];  // 0 unknown, 1 gfx950, 2 other
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MLA_ERR_DEVICE;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c == 1) return MLA_OK;
    if (c == 2) return MLA_ERR_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MLA_ERR_DEVICE;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) cache[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? MLA_OK : MLA_ERR_DEVICE;
}

size_t decode_ws_bytes(int B, int H, int splits) {
  if (splits <= 1) return 0;
  return (size_t)B * H * splits * mla::kDecodePart * sizeof(float);
}

size_t oproj_ws_bytes(int M, int N, int splits) {
  if (splits <= 1) return 0;
  return (size_t)splits * M * N * sizeof(float);
}

}  // namespace

extern "C" {

int mla_abi_version(void) { return MLA_ABI_VERSION; }

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_NULL: return "MLA_ERR_NULL: a required pointer is NULL";
    case MLA_ERR_DIM: return "MLA_ERR_DIM: invalid or inconsistent size";
    case MLA_ERR_ALIGN: return "MLA_ERR_ALIGN: pointer not 16-byte aligned";
    case MLA_ERR_ALIAS: return "MLA_ERR_ALIAS: an output overlaps an input or another output";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE: workspace missing or too small";
    case MLA_ERR_SCALE: return "MLA_ERR_SCALE: softmax_scale must be finite and > 0";
    case MLA_ERR_DEVICE: return "MLA_ERR_DEVICE: current device is not gfx950";
    case MLA_ERR_LAUNCH: return "MLA_ERR_LAUNCH: kernel launch failed";
    case MLA_ERR_FLAGS: return "MLA_ERR_FLAGS: unknown flag bits";
    default: return "unknown status";
  }
}

// ------------------------------------------------------------------ prefill

size_t mla_prefill_workspace_bytes(int B, int H, int T) {
  if (!dims_ok(B, H, T, kQK)) return 0;
  return mla::prefill_workspace_layout(B, H, T).total;
}

}  // extern "C"

namespace {

// Shared by mla_attend_prefill and mla_attend_prefill_noalloc.  `scratch` is
// null for the caller-workspace entry point; otherwise it resolves the static
// buffer once the arguments are validated (it needs the current device).
// With out8 set (FP8 output), `out` is unused and out_sT receives the scales.
int attend_prefill(const mla_bf16* q_nope, const mla_bf16* q_pe, const mla_bf16* k_nope,
                   const mla_bf16* k_pe, const mla_bf16* v, const float* R, int r_rows,
                   float softmax_scale, int B, int H, int T, void* workspace,
                   size_t workspace_bytes, void* out, float* lse, uint32_t flags, void* stream,
                   void* (*scratch)(int* status), uint8_t* out8 = nullptr,
                   float* out_sT = nullptr) {
  const bool fp8 = out8 != nullptr || out_sT != nullptr;
  if (!q_nope || !q_pe || !k_nope || !k_pe || !v || !R || (!fp8 && !out) || (fp8 && (!out8 || !out_sT)))
    return MLA_ERR_NULL;
  if (flags & ~(MLA_V_BLOCKED | (fp8 ? 0u : MLA_OUT_F32))) return MLA_ERR_FLAGS;
  const bool vblk = (flags & MLA_V_BLOCKED) != 0;
  if (!dims_ok(B, H, T, kQK) || r_rows <= 0 || r_rows > kMaxDim || T > r_rows ||
      (size_t)H * T * 256 > 0xffffffffu)
    return MLA_ERR_DIM;
  if (fp8 && (long long)B * T > 0x7ffffff0LL) return MLA_ERR_DIM;
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f)) return MLA_ERR_SCALE;
  const mla::PrefillWorkspace ws = mla::prefill_workspace_layout(B, H, T);
  if (!scratch && !workspace) return MLA_ERR_WORKSPACE;
  if (workspace_bytes < ws.total) return MLA_ERR_WORKSPACE;
  if (!aligned16(q_nope) || !aligned16(q_pe) || !aligned16(k_nope) || !aligned16(k_pe) ||
      !aligned16(v) || !aligned16(R) || !aligned16(out) || !aligned16(lse) || !aligned16(workspace) ||
      !aligned16(out8) || !aligned16(out_sT))
    return MLA_ERR_ALIGN;
  const size_t bht = (size_t)B * H * T;
  const size_t v_rows = vblk ? (size_t)B * H * ((T + 15) / 16 * 16) : bht;
  const size_t out_elt = (flags & MLA_OUT_F32) ? 4 : 2;
  const Range in[] = {{q_nope, bht * kNope * 2}, {q_pe, bht * kRope * 2}, {k_nope, bht * kNope * 2},
                      {k_pe, (size_t)B * T * kRope * 2}, {v, v_rows * kV * 2},
                      {R, (size_t)r_rows * mla::kPairs * 4}};
  const Range outs[] = {{fp8 ? nullptr : out, bht * kV * out_elt}, {lse, lse ? bht * 4 : 0},
                        {workspace, scratch ? 0 : ws.total}, {out8, fp8 ? bht * kV : 0},
                        {out_sT, fp8 ? (size_t)H * mla::act_scale_stride(B * T) * 4 : 0}};
  if (any_alias(in, 6, outs, 5)) return MLA_ERR_ALIAS;
  const int dev = check_device();
  if (dev != MLA_OK) return dev;
  if (scratch) {
    int st = MLA_OK;
    workspace = scratch(&st);
    if (st != MLA_OK) return st;
  }

  mla::PrefillParams p;
  p.q_nope = q_nope;
  p.q_pe = q_pe;
  p.k_nope = k_nope;
  p.k_pe = k_pe;
  p.v = v;
  p.R = R;
  p.cs = reinterpret_cast<float2*>(static_cast<char*>(workspace) + ws.cs_off);
  p.kpe_rot = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + ws.kpe_off);
  p.out = fp8 ? nullptr : out;
  p.out8 = out8;
  p.out_sT = out_sT;
  p.lse = lse;
  p.B = B;
  p.H = H;
  p.T = T;
  p.past = 0;
  p.LK = T;
  p.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634074);
  p.out_f32 = (flags & MLA_OUT_F32) ? 1 : 0;
  p.v_blocked = vblk ? 1 : 0;
  if (vblk && ws.vtail_bytes)
    p.v_tail = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + ws.vtail_off);
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // start from a clean error state
  if (mla::launch_rope_prep(p, s) != hipSuccess) return MLA_ERR_LAUNCH;
  if (p.v_tail && mla::launch_v_tail(p, s) != hipSuccess) return MLA_ERR_LAUNCH;
  if (mla::launch_prefill(p, s) != hipSuccess) return MLA_ERR_LAUNCH;
  return MLA_OK;
}

}  // namespace

// Static workspace of mla_attend_prefill_noalloc: the cos/sin table and the
// rotated shared key of one call.  Each device holds its own copy for the
// life of the process.  In host code `scratch` names a host-side stand-in, not
// device memory: its device address is taken once per device with
// hipGetSymbolAddress and only that address is passed to kernels.
static __device__ __align__(256) uint8_t scratch[MLA_PREFILL_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of this device's `scratch` (the current device, already
// checked to be gfx950).  Resolved on the first call on each device.
void* device_scratch(int* status) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *status = MLA_ERR_DEVICE;
    return nullptr;
  }
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr) return ptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (!ptr) {
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      *status = MLA_ERR_DEVICE;
      return nullptr;
    }
    g_scratch_ptr[dev].store(ptr, std::memory_order_release);
  }
  return ptr;
}

}  // namespace

extern "C" {

int mla_attend_prefill(const mla_bf16* q_nope, const mla_bf16* q_pe, const mla_bf16* k_nope,
                       const mla_bf16* k_pe, const mla_bf16* v, const float* R, int r_rows,
                       float softmax_scale, int B, int H, int T, void* workspace,
                       size_t workspace_bytes, void* out, float* lse, uint32_t flags,
                       void* stream) {
  return attend_prefill(q_nope, q_pe, k_nope, k_pe, v, R, r_rows, softmax_scale, B, H, T,
                        workspace, workspace_bytes, out, lse, flags, stream, nullptr);
}

int mla_attend_prefill_fp8(const mla_bf16* q_nope, const mla_bf16* q_pe, const mla_bf16* k_nope,
                           const mla_bf16* k_pe, const mla_bf16* v, const float* R, int r_rows,
                           float softmax_scale, int B, int H, int T, void* workspace,
                           size_t workspace_bytes, uint8_t* out8, float* out_scaleT, float* lse,
                           uint32_t flags, void* stream) {
  return attend_prefill(q_nope, q_pe, k_nope, k_pe, v, R, r_rows, softmax_scale, B, H, T,
                        workspace, workspace_bytes, nullptr, lse, flags, stream, nullptr, out8,
                        out_scaleT);
}

int mla_attend_prefill_noalloc(const mla_bf16* q_nope, const mla_bf16* q_pe,
                               const mla_bf16* k_nope, const mla_bf16* k_pe, const mla_bf16* v,
                               const float* R, int r_rows, float softmax_scale, int B, int H,
                               int T, void* out, float* lse, uint32_t flags, void* stream) {
  return attend_prefill(q_nope, q_pe, k_nope, k_pe, v, R, r_rows, softmax_scale, B, H, T, nullptr,
                        MLA_PREFILL_NOALLOC_SCRATCH_BYTES, out, lse, flags, stream,
                        device_scratch);
}

// ------------------------------------------------ chunked prefill, append

size_t mla_prefill_chunk_workspace_bytes(int T) {
  if (T <= 0 || T > kMaxDim) return 0;
  return mla::align_up((size_t)T * mla::kPairs * 8, 256);
}

int mla_append_kv(const mla_bf16* k_nope, const mla_bf16* k_pe, const mla_bf16* v, const float* R,
                  int r_rows, int past, int B, int H, int T, int L_cap, mla_bf16* k_nope_cache,
                  mla_bf16* kpe_cache, mla_bf16* v_cache, uint32_t flags, void* stream) {
  if (!k_nope || !k_pe || !v || !R || !k_nope_cache || !kpe_cache || !v_cache) return MLA_ERR_NULL;
  if (flags) return MLA_ERR_FLAGS;
  if (!dims_ok(B, H, T, kQK) || !dims_ok(B, H, L_cap, kQK) || past < 0 || r_rows <= 0 ||
      r_rows > kMaxDim || (long long)past + T > L_cap || (long long)past + T > r_rows)
    return MLA_ERR_DIM;
  if (!aligned16(k_nope) || !aligned16(k_pe) || !aligned16(v) || !aligned16(R) ||
      !aligned16(k_nope_cache) || !aligned16(kpe_cache) || !aligned16(v_cache))
    return MLA_ERR_ALIGN;
  const size_t bht = (size_t)B * H * T, bhl = (size_t)B * H * L_cap;
  const Range in[] = {{k_nope, bht * kNope * 2}, {k_pe, (size_t)B * T * kRope * 2},
                      {v, bht * kV * 2}, {R, (size_t)r_rows * mla::kPairs * 4}};
  const Range outs[] = {{k_nope_cache, bhl * kNope * 2}, {kpe_cache, (size_t)B * L_cap * kRope * 2},
                        {v_cache, bhl * kV * 2}};
  if (any_alias(in, 4, outs, 3)) return MLA_ERR_ALIAS;
  const int dev = check_device();
  if (dev != MLA_OK) return dev;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (mla::launch_append_rows(k_nope, k_nope_cache, B * H, T, L_cap, past, s) != hipSuccess ||
      mla::launch_append_rows(v, v_cache, B * H, T, L_cap, past, s) != hipSuccess ||
      mla::launch_rope(R, past, k_pe, nullptr, kpe_cache, L_cap, past, B, T, s) != hipSuccess)
    return MLA_ERR_LAUNCH;
  return MLA_OK;
}

int mla_attend_prefill_chunk(const mla_bf16* q_nope, const mla_bf16* q_pe,
                             const mla_bf16* k_nope_cache, const mla_bf16* kpe_cache,
                             const mla_bf16* v_cache, const float* R, int r_rows, int past,
                             float softmax_scale, int B, int H, int T, int L_cap, void* workspace,
                             size_t workspace_bytes, void* out, float* lse, uint32_t flags,
                             void* stream) {
  if (!q_nope || !q_pe || !k_nope_cache || !kpe_cache || !v_cache || !R || !out) return MLA_ERR_NULL;
  if (flags & ~MLA_OUT_F32) return MLA_ERR_FLAGS;
  if (!dims_ok(B, H, T, kQK) || !dims_ok(B, H, L_cap, kQK) || past < 0 || r_rows <= 0 ||
      r_rows > kMaxDim || (long long)past + T > L_cap || (long long)past + T > r_rows ||
      (size_t)H * L_cap * 256 > 0xffffffffu)
    return MLA_ERR_DIM;
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f)) return MLA_ERR_SCALE;
  const size_t need = mla_prefill_chunk_workspace_bytes(T);
  if (!workspace || workspace_bytes < need) return MLA_ERR_WORKSPACE;
  if (!aligned16(q_nope) || !aligned16(q_pe) || !aligned16(k_nope_cache) || !aligned16(kpe_cache) ||
      !aligned16(v_cache) || !aligned16(R) || !aligned16(out) || !aligned16(lse) ||
      !aligned16(workspace))
    return MLA_ERR_ALIGN;
  const size_t bht = (size_t)B * H * T, bhl = (size_t)B * H * L_cap;
  const size_t out_elt = (flags & MLA_OUT_F32) ? 4 : 2;
  const Range in[] = {{q_nope, bht * kNope * 2}, {q_pe, bht * kRope * 2},
                      {k_nope_cache, bhl * kNope * 2}, {kpe_cache, (size_t)B * L_cap * kRope * 2},
                      {v_cache, bhl * kV * 2}, {R, (size_t)r_rows * mla::kPairs * 4}};
  const Range outs[] = {{out, bht * kV * out_elt}, {lse, lse ? bht * 4 : 0}, {workspace, need}};
  if (any_alias(in, 6, outs, 3)) return MLA_ERR_ALIAS;
  const int dev = check_device();
  if (dev != MLA_OK) return dev;

  mla::PrefillParams p;
  p.q_nope = q_nope;
  p.q_pe = q_pe;
  p.k_nope = k_nope_cache;
  p.k_pe = nullptr;  // the cache holds rotated keys
  p.v = v_cache;
  p.R = R;
  p.cs = static_cast<float2*>(workspace);
  p.kpe_rot = const_cast<uint16_t*>(kpe_cache);
  p.out = out;
  p.lse = lse;
  p.B = B;
  p.H = H;
  p.T = T;
  p.past = past;
  p.LK = L_cap;
  p.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634074);
  p.out_f32 = (flags & MLA_OUT_F32) ? 1 : 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (mla::launch_rope_prep(p, s) != hipSuccess) return MLA_ERR_LAUNCH;
  if (mla::launch_prefill(p, s) != hipSuccess) return MLA_ERR_LAUNCH;
  return MLA_OK;
}

// ------------------------------------------------------------------- decode

int mla_decode_splits(int B, int H, int L, int num_splits) {
  if (!dims_ok(B, H, L, kQK) || num_splits < 0) return 0;
  return mla::decode_choose_splits(B, H, L, num_splits);
}

size_t mla_decode_workspace_bytes(int B, int H, int L, int num_splits) {
  const int s = mla_decode_splits(B, H, L, num_splits);
  if (s <= 0) return 0;
  return decode_ws_bytes(B, H, s);
}

}  // extern "C"

namespace {

// Both decode entry points: kpe_cache null selects the joined key layout.
int decode_common(const mla_bf16* q_nope, const mla_bf16* q_pe, const mla_bf16* k_cache,
                  const mla_bf16* kpe_cache, bool shared_kpe, const mla_bf16* v_cache,
                  const float* R, int r_rows, int q_pos, float softmax_scale, int B, int H, int L,
                  int num_splits, void* workspace, size_t workspace_bytes, void* out, float* lse,
                  uint32_t flags, void* stream) {
  if (!q_nope || !q_pe || !k_cache || !v_cache || !R || !out || (shared_kpe && !kpe_cache))
    return MLA_ERR_NULL;
  if (flags & ~MLA_OUT_F32) return MLA_ERR_FLAGS;
  if (!dims_ok(B, H, L, kQK) || r_rows <= 0 || r_rows > kMaxDim || q_pos < 0 || q_pos >= r_rows ||
      num_splits < 0)
    return MLA_ERR_DIM;
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f)) return MLA_ERR_SCALE;
  const int splits = mla::decode_choose_splits(B, H, L, num_splits);
  const size_t need = decode_ws_bytes(B, H, splits);
  if (need > 0 && (!workspace || workspace_bytes < need)) return MLA_ERR_WORKSPACE;
  if (!aligned16(q_nope) || !aligned16(q_pe) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned16(R) || !aligned16(out) || !aligned16(lse) || !aligned16(workspace) ||
      !aligned16(kpe_cache))
    return MLA_ERR_ALIGN;
  const size_t bh = (size_t)B * H;
  const size_t out_elt = (flags & MLA_OUT_F32) ? 4 : 2;
  const size_t krow = shared_kpe ? kNope : kQK;
  const Range in[] = {{q_nope, bh * kNope * 2}, {q_pe, bh * kRope * 2},
                      {k_cache, bh * L * krow * 2}, {v_cache, bh * L * kV * 2},
                      {R, (size_t)r_rows * mla::kPairs * 4},
                      {shared_kpe ? kpe_cache : nullptr, shared_kpe ? (size_t)B * L * kRope * 2 : 0}};
  const Range outs[] = {{out, bh * kV * out_elt}, {lse, lse ? bh * 4 : 0},
                        {need ? workspace : nullptr, need}};
  if (any_alias(in, 6, outs, 3)) return MLA_ERR_ALIAS;
  const int dev = check_device();
  if (dev != MLA_OK) return dev;

  mla::DecodeParams p;
  p.q_nope = q_nope;
  p.q_pe = q_pe;
  p.k_cache = k_cache;
  p.kpe_cache = shared_kpe ? kpe_cache : nullptr;
  p.v_cache = v_cache;
  p.R = R;
  p.q_pos = q_pos;
  p.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634074);
  p.B = B;
  p.H = H;
  p.L = L;
  p.splits = splits;
  p.part = static_cast<float*>(need ? workspace : nullptr);
  p.out = out;
  p.lse = lse;
  p.out_f32 = (flags & MLA_OUT_F32) ? 1 : 0;
  (void)hipGetLastError();
  if (mla::launch_decode(p, static_cast<hipStream_t>(stream)) != hipSuccess) return MLA_ERR_LAUNCH;
  return MLA_OK;
}

}  // namespace

extern "C" {

int mla_attend_decode(const mla_bf16* q_nope, const mla_bf16* q_pe, const mla_bf16* k_cache,
                      const mla_bf16* v_cache, const float* R, int r_rows, int q_pos,
                      float softmax_scale, int B, int H, int L, int num_splits, void* workspace,
                      size_t workspace_bytes, void* out, float* lse, uint32_t flags,
                      void* stream) {
  return decode_common(q_nope, q_pe, k_cache, nullptr, false, v_cache, R, r_rows, q_pos,
                       softmax_scale, B, H, L, num_splits, workspace, workspace_bytes, out, lse,
                       flags, stream);
}

int mla_attend_decode_shared_kpe(const mla_bf16* q_nope, const mla_bf16* q_pe,
                                 const mla_bf16* k_nope_cache, const mla_bf16* kpe_cache,
                                 const mla_bf16* v_cache, const float* R, int r_rows, int q_pos,
                                 float softmax_scale, int B, int H, int L, int num_splits,
                                 void* workspace, size_t workspace_bytes, void* out, float* lse,
                                 uint32_t flags, void* stream) {
  return decode_common(q_nope, q_pe, k_nope_cache, kpe_cache, true, v_cache, R, r_rows, q_pos,
                       softmax_scale, B, H, L, num_splits, workspace, workspace_bytes, out, lse,
                       flags, stream);
}

// ------------------------------------------------------------ latent decode

}  // extern "C"

namespace {

constexpr int kLatentMaxL = (1 << 21) - 1;  // L·1024 bytes must fit a buffer record count
constexpr int kLatentMaxB = 1 << 20;        // ceil(B/16) grid rows

bool latent_dims_ok(int B, int H, int L) {
  return dims_ok(B, H, L, mla::kLatent + kRope) && H <= 64 && L <= kLatentMaxL && B <= kLatentMaxB;
}

}  // namespace

extern "C" {

size_t mla_decode_latent_workspace_bytes(int B, int H, int L, int num_splits) {
  if (!latent_dims_ok(B, H, L) || num_splits < 0) return 0;
  return mla::latent_workspace_layout(B, H, mla::latent_choose_splits(B, L, num_splits)).total;
}

int mla_attend_decode_latent(const mla_bf16* q_nope, const mla_bf16* q_pe, const mla_bf16* ckv_cache,
                             const mla_bf16* kpe_cache, const mla_bf16* w_kv_b, const float* R,
                             int r_rows, int q_pos, float softmax_scale, int B, int H, int L,
                             int num_splits, void* workspace, size_t workspace_bytes, void* out,
                             float* lse, uint32_t flags, void* stream) {
  if (!q_nope || !q_pe || !ckv_cache || !kpe_cache || !w_kv_b || !R || !out) return MLA_ERR_NULL;
  if (flags & ~MLA_OUT_F32) return MLA_ERR_FLAGS;
  if (!latent_dims_ok(B, H, L) || r_rows <= 0 || r_rows > kMaxDim || q_pos < 0 || q_pos >= r_rows ||
      num_splits < 0)
    return MLA_ERR_DIM;
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f)) return MLA_ERR_SCALE;
  const int splits = mla::latent_choose_splits(B, L, num_splits);
  const mla::LatentWorkspace ws = mla::latent_workspace_layout(B, H, splits);
  if (!workspace || workspace_bytes < ws.total) return MLA_ERR_WORKSPACE;
  if (!aligned16(q_nope) || !aligned16(q_pe) || !aligned16(ckv_cache) || !aligned16(kpe_cache) ||
      !aligned16(w_kv_b) || !aligned16(R) || !aligned16(out) || !aligned16(lse) ||
      !aligned16(workspace))
    return MLA_ERR_ALIGN;
  const size_t bh = (size_t)B * H;
  const size_t out_elt = (flags & MLA_OUT_F32) ? 4 : 2;
  const Range in[] = {{q_nope, bh * kNope * 2},
                      {q_pe, bh * kRope * 2},
                      {ckv_cache, (size_t)B * L * mla::kLatent * 2},
                      {kpe_cache, (size_t)B * L * kRope * 2},
                      {w_kv_b, (size_t)H * 256 * mla::kLatent * 2},
                      {R, (size_t)r_rows * mla::kPairs * 4}};
  const Range outs[] = {{out, bh * kV * out_elt}, {lse, lse ? bh * 4 : 0}, {workspace, ws.total}};
  if (any_alias(in, 6, outs, 3)) return MLA_ERR_ALIAS;
  const int dev = check_device();
  if (dev != MLA_OK) return dev;

  char* w = static_cast<char*>(workspace);
  mla::LatentParams p;
  p.q_nope = q_nope;
  p.q_pe = q_pe;
  p.ckv = ckv_cache;
  p.kpe = kpe_cache;
  p.w_kv_b = w_kv_b;
  p.R = R;
  p.q_pos = q_pos;
  p.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634074);
  p.B = B;
  p.H = H;
  p.L = L;
  p.splits = splits;
  p.q_lat = reinterpret_cast<uint16_t*>(w + ws.q_off);
  p.o_lat = reinterpret_cast<float*>(w + ws.o_off);
  p.part = splits > 1 ? reinterpret_cast<float*>(w + ws.part_off) : nullptr;
  p.lse = lse;
  p.out = out;
  p.out_f32 = (flags & MLA_OUT_F32) ? 1 : 0;
  (void)hipGetLastError();
  if (mla::launch_decode_latent(p, static_cast<hipStream_t>(stream)) != hipSuccess)
    return MLA_ERR_LAUNCH;
  return MLA_OK;
}

// ------------------------------------------------------------------- o_proj

size_t mla_out_proj_workspace_bytes(int M, int K, int N) {
  if (!dims_ok(M, K, N, 1) || K % 128 != 0) return 0;
  return oproj_ws_bytes(M, N, mla::oproj_choose_splits(M, K, N));
}

int mla_out_proj(const mla_bf16* x, const mla_bf16* w_o, void* y, int M, int K, int N,
                 void* workspace, size_t workspace_bytes, uint32_t flags, void* stream) {
  if (!x || !w_o || !y) return MLA_ERR_NULL;
  if (flags & ~MLA_OUT_F32) return MLA_ERR_FLAGS;
  if (!dims_ok(M, K, N, 1) || K % 128 != 0 || (long long)M * N > kMaxElems) return MLA_ERR_DIM;
  const int splits = mla::oproj_choose_splits(M, K, N);
  const size_t need = oproj_ws_bytes(M, N, splits);
  if (need > 0 && (!workspace || workspace_bytes < need)) return MLA_ERR_WORKSPACE;
  if (!aligned16(x) || !aligned16(w_o) || !aligned16(y) || !aligned16(workspace)) return MLA_ERR_ALIGN;
  const size_t out_elt = (flags & MLA_OUT_F32) ? 4 : 2;
  const Range in[] = {{x, (size_t)M * K * 2}, {w_o, (size_t)N * K * 2}};
  const Range outs[] = {{y, (size_t)M * N * out_elt}, {need ? workspace : nullptr, need}};
  if (any_alias(in, 2, outs, 2)) return MLA_ERR_ALIAS;
  const int dev = check_device();
  if (dev != MLA_OK) return dev;

  mla::OprojParams p;
  p.x = x;
  p.w = w_o;
  p.y = y;
  p.part = static_cast<float*>(need ? workspace : nullptr);
  p.M = M;
  p.K = K;
  p.N = N;
  p.splits = splits;
  p.out_f32 = (flags & MLA_OUT_F32) ? 1 : 0;
  p.group_m = 0;  // kernel default
  p.w8 = nullptr;
  p.w_scale = nullptr;
  (void)hipGetLastError();
  if (mla::launch_oproj(p, static_cast<hipStream_t>(stream)) != hipSuccess) return MLA_ERR_LAUNCH;
  return MLA_OK;
}

int mla_up_project(const mla_bf16* q_lat, const mla_bf16* ckv, const mla_bf16* w_q_b,
                   const mla_bf16* w_kv_b, int B, int T, int H, void* q_nope, void* q_pe,
                   void* k_nope, void* v, uint32_t flags, void* stream) {
  if (!q_lat || !ckv || !w_q_b || !w_kv_b || !q_nope || !q_pe || !k_nope || !v) return MLA_ERR_NULL;
  if (flags & ~(MLA_OUT_F32 | MLA_V_BLOCKED)) return MLA_ERR_FLAGS;
  const bool vblk = (flags & MLA_V_BLOCKED) != 0;
  if (!dims_ok(B, T, H, mla::kQK + kV) || (long long)B * T > 0x7fffffffLL ||
      (long long)H * (kNope + kV) > 0x7fffffffLL)
    return MLA_ERR_DIM;
  if (!aligned16(q_lat) || !aligned16(ckv) || !aligned16(w_q_b) || !aligned16(w_kv_b) ||
      !aligned16(q_nope) || !aligned16(q_pe) || !aligned16(k_nope) || !aligned16(v))
    return MLA_ERR_ALIGN;
  const size_t M = (size_t)B * T, rows = (size_t)B * H * T;
  const size_t v_rows = vblk ? (size_t)B * H * ((T + 15) / 16 * 16) : rows;
  const size_t elt = (flags & MLA_OUT_F32) ? 4 : 2;
  const Range in[] = {{q_lat, M * mla::kQRank * 2},
                      {ckv, M * mla::kLatent * 2},
                      {w_q_b, (size_t)H * kQK * mla::kQRank * 2},
                      {w_kv_b, (size_t)H * (kNope + kV) * mla::kLatent * 2}};
  const Range outs[] = {{q_nope, rows * kNope * elt},
                        {q_pe, rows * kRope * elt},
                        {k_nope, rows * kNope * elt},
                        {v, v_rows * kV * elt}};
  if (any_alias(in, 4, outs, 4)) return MLA_ERR_ALIAS;
  const int dev = check_device();
  if (dev != MLA_OK) return dev;

  const hipStream_t s = static_cast<hipStream_t>(stream);
  mla::OprojParams p;
  p.part = nullptr;
  p.M = (int)M;
  p.splits = 1;
  p.out_f32 = (flags & MLA_OUT_F32) ? 1 : 0;
  p.group_m = 0;
  p.w8 = nullptr;
  p.w_scale = nullptr;
  p.T = T;
  p.d0 = kNope;
  // q = q_lat · w_q_bᵀ: per head 128 q_nope then 64 q_pe features
  p.x = q_lat;
  p.w = w_q_b;
  p.K = mla::kQRank;
  p.N = H * kQK;
  p.hd = kQK;
  p.y = q_nope;
  p.y1 = q_pe;
  (void)hipGetLastError();
  if (mla::launch_oproj(p, s) != hipSuccess) return MLA_ERR_LAUNCH;
  // kv = ckv · w_kv_bᵀ: per head 128 nope key then 128 value features
  p.x = ckv;
  p.w = w_kv_b;
  p.K = mla::kLatent;
  p.N = H * (kNope + kV);
  p.hd = kNope + kV;
  p.y = k_nope;
  p.y1 = v;
  p.y1_blocked = vblk ? 1 : 0;
  if (mla::launch_oproj(p, s) != hipSuccess) return MLA_ERR_LAUNCH;
  return MLA_OK;
}

size_t mla_out_proj_fp8_workspace_bytes(int M, int K, int N) {
  if (!dims_ok(M, K, N, 1) || K % 128 != 0) return 0;
  if (mla::oproj_fp8_wide(M, K, N)) return mla::align_up((size_t)N * K * 2, 256);
  return oproj_ws_bytes(M, N, mla::oproj_choose_splits(M, K, N, true));
}

int mla_out_proj_fp8(const mla_bf16* x, const uint8_t* w8, const float* w_scale, void* y, int M,
                     int K, int N, void* workspace, size_t workspace_bytes, uint32_t flags,
                     void* stream) {
  if (!x || !w8 || !w_scale || !y) return MLA_ERR_NULL;
  if (flags & ~MLA_OUT_F32) return MLA_ERR_FLAGS;
  if (!dims_ok(M, K, N, 1) || K % 128 != 0 || (long long)M * N > kMaxElems) return MLA_ERR_DIM;
  const bool wide = mla::oproj_fp8_wide(M, K, N);
  const int splits = wide ? 1 : mla::oproj_choose_splits(M, K, N, true);
  const size_t need = wide ? mla::align_up((size_t)N * K * 2, 256) : oproj_ws_bytes(M, N, splits);
  if (need > 0 && (!workspace || workspace_bytes < need)) return MLA_ERR_WORKSPACE;
  if (!aligned16(x) || !aligned16(w8) || !aligned16(w_scale) || !aligned16(y) ||
      !aligned16(workspace))
    return MLA_ERR_ALIGN;
  const size_t out_elt = (flags & MLA_OUT_F32) ? 4 : 2;
  const size_t nb = (size_t)(N + 127) / 128, kb = (size_t)K / 128;
  const Range in[] = {{x, (size_t)M * K * 2}, {w8, (size_t)N * K}, {w_scale, nb * kb * 4}};
  const Range outs[] = {{y, (size_t)M * N * out_elt}, {need ? workspace : nullptr, need}};
  if (any_alias(in, 3, outs, 2)) return MLA_ERR_ALIAS;
  const int dev = check_device();
  if (dev != MLA_OK) return dev;

  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  mla::OprojParams p;
  p.x = x;
  p.w = nullptr;
  p.w8 = w8;
  p.w_scale = w_scale;
  p.y = y;
  p.part = static_cast<float*>(need && !wide ? workspace : nullptr);
  if (wide) {
    // the bf16 weight the small-tile kernel would form in its load path,
    // formed once, then the wide bf16 kernel
    uint16_t* wbf = static_cast<uint16_t*>(workspace);
    if (mla::launch_dequant_fp8(w8, w_scale, wbf, N, K, s) != hipSuccess) return MLA_ERR_LAUNCH;
    p.w = wbf;
    p.w8 = nullptr;
    p.w_scale = nullptr;
  }
  p.M = M;
  p.K = K;
  p.N = N;
  p.splits = splits;
  p.out_f32 = (flags & MLA_OUT_F32) ? 1 : 0;
  p.group_m = 0;
  if (mla::launch_oproj(p, s) != hipSuccess) return MLA_ERR_LAUNCH;
  return MLA_OK;
}

// -------------------------------------------------------- FP8 activations

int mla_act_scale_stride(int M) { return M > 0 && M <= kMaxDim ? mla::act_scale_stride(M) : 0; }

int mla_act_quant(const mla_bf16* x, int M, int K, uint8_t* x8, float* x_scaleT, void* stream) {
  if (!x || !x8 || !x_scaleT) return MLA_ERR_NULL;
  if (!dims_ok(M, K, 1, 1) || K % 128 != 0 || (long long)M * K > 0x7fffffffLL) return MLA_ERR_DIM;
  if (!aligned16(x) || !aligned16(x8) || !aligned16(x_scaleT)) return MLA_ERR_ALIGN;
  const size_t ms = (size_t)mla::act_scale_stride(M);
  const Range in[] = {{x, (size_t)M * K * 2}};
  const Range outs[] = {{x8, (size_t)M * K}, {x_scaleT, (size_t)(K / 128) * ms * 4}};
  if (any_alias(in, 1, outs, 2)) return MLA_ERR_ALIAS;
  const int dev = check_device();
  if (dev != MLA_OK) return dev;
  (void)hipGetLastError();
  if (mla::launch_act_quant(x, x8, x_scaleT, M, K, static_cast<hipStream_t>(stream)) != hipSuccess)
    return MLA_ERR_LAUNCH;
  return MLA_OK;
}

namespace {
struct Fp8DynWorkspace {
  size_t x8_off, xs_off, part_off, total;
  int splits;
};
Fp8DynWorkspace fp8dyn_layout(int M, int K, int N) {
  Fp8DynWorkspace w;
  w.splits = mla::oproj_fp8dyn_splits(M, K, N);
  w.x8_off = 0;
  w.xs_off = mla::align_up((size_t)M * K, 256);
  w.part_off = w.xs_off + mla::align_up((size_t)(K / 128) * mla::act_scale_stride(M) * 4, 256);
  w.total = w.part_off + (w.splits > 1 ? (size_t)w.splits * M * N * 4 : 0);
  return w;
}
bool fp8dyn_dims_ok(int M, int K, int N) {
  return dims_ok(M, K, N, 1) && K % 128 == 0 && (long long)K * 256 < 0x7fffffffLL &&
         (long long)M * K <= 0x7fffffffLL && (long long)M * N <= kMaxElems;
}
}  // namespace

size_t mla_out_proj_fp8_q_workspace_bytes(int M, int K, int N) {
  if (!fp8dyn_dims_ok(M, K, N)) return 0;
  const Fp8DynWorkspace ws = fp8dyn_layout(M, K, N);
  return ws.total - ws.part_off;
}

int mla_out_proj_fp8_q(const uint8_t* x8, const float* x_scaleT, const uint8_t* w8,
                       const float* w_scale, void* y, int M, int K, int N, void* workspace,
                       size_t workspace_bytes, uint32_t flags, void* stream) {
  if (!x8 || !x_scaleT || !w8 || !w_scale || !y) return MLA_ERR_NULL;
  if (flags & ~MLA_OUT_F32) return MLA_ERR_FLAGS;
  if (!fp8dyn_dims_ok(M, K, N)) return MLA_ERR_DIM;
  const Fp8DynWorkspace ws = fp8dyn_layout(M, K, N);
  const size_t need = ws.total - ws.part_off;  // the split partials only
  if (need > 0 && (!workspace || workspace_bytes < need)) return MLA_ERR_WORKSPACE;
  if (!aligned16(x8) || !aligned16(x_scaleT) || !aligned16(w8) || !aligned16(w_scale) ||
      !aligned16(y) || !aligned16(workspace))
    return MLA_ERR_ALIGN;
  const size_t out_elt = (flags & MLA_OUT_F32) ? 4 : 2;
  const size_t nb = (size_t)(N + 127) / 128, kb = (size_t)K / 128;
  const Range in[] = {{x8, (size_t)M * K}, {x_scaleT, kb * mla::act_scale_stride(M) * 4},
                      {w8, (size_t)N * K}, {w_scale, nb * kb * 4}};
  const Range outs[] = {{y, (size_t)M * N * out_elt}, {need ? workspace : nullptr, need}};
  if (any_alias(in, 4, outs, 2)) return MLA_ERR_ALIAS;
  const int dev = check_device();
  if (dev != MLA_OK) return dev;
  (void)hipGetLastError();
  mla::OprojParams p;
  p.x = nullptr;
  p.w = nullptr;
  p.w8 = w8;
  p.w_scale = w_scale;
  p.x8 = x8;
  p.x_scaleT = x_scaleT;
  p.y = y;
  p.part = ws.splits > 1 ? static_cast<float*>(workspace) : nullptr;
  p.M = M;
  p.K = K;
  p.N = N;
  p.splits = ws.splits;
  p.out_f32 = (flags & MLA_OUT_F32) ? 1 : 0;
  p.group_m = 0;
  if (mla::launch_oproj_fp8dyn(p, static_cast<hipStream_t>(stream)) != hipSuccess) return MLA_ERR_LAUNCH;
  return MLA_OK;
}

size_t mla_out_proj_fp8_dyn_workspace_bytes(int M, int K, int N) {
  if (!fp8dyn_dims_ok(M, K, N)) return 0;
  return fp8dyn_layout(M, K, N).total;
}

int mla_out_proj_fp8_dyn(const mla_bf16* x, const uint8_t* w8, const float* w_scale, void* y,
                         int M, int K, int N, void* workspace, size_t workspace_bytes,
                         uint32_t flags, void* stream) {
  if (!x || !w8 || !w_scale || !y) return MLA_ERR_NULL;
  if (flags & ~MLA_OUT_F32) return MLA_ERR_FLAGS;
  if (!fp8dyn_dims_ok(M, K, N)) return MLA_ERR_DIM;
  const Fp8DynWorkspace ws = fp8dyn_layout(M, K, N);
  if (!workspace || workspace_bytes < ws.total) return MLA_ERR_WORKSPACE;
  if (!aligned16(x) || !aligned16(w8) || !aligned16(w_scale) || !aligned16(y) ||
      !aligned16(workspace))
    return MLA_ERR_ALIGN;
  const size_t out_elt = (flags & MLA_OUT_F32) ? 4 : 2;
  const size_t nb = (size_t)(N + 127) / 128, kb = (size_t)K / 128;
  const Range in[] = {{x, (size_t)M * K * 2}, {w8, (size_t)N * K}, {w_scale, nb * kb * 4}};
  const Range outs[] = {{y, (size_t)M * N * out_elt}, {workspace, ws.total}};
  if (any_alias(in, 3, outs, 2)) return MLA_ERR_ALIAS;
  const int dev = check_device();
  if (dev != MLA_OK) return dev;

  char* wsb = static_cast<char*>(workspace);
  uint8_t* x8 = reinterpret_cast<uint8_t*>(wsb + ws.x8_off);
  float* xs = reinterpret_cast<float*>(wsb + ws.xs_off);
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (mla::launch_act_quant(x, x8, xs, M, K, s) != hipSuccess) return MLA_ERR_LAUNCH;
  mla::OprojParams p;
  p.x = nullptr;
  p.w = nullptr;
  p.w8 = w8;
  p.w_scale = w_scale;
  p.x8 = x8;
  p.x_scaleT = xs;
  p.y = y;
  p.part = ws.splits > 1 ? reinterpret_cast<float*>(wsb + ws.part_off) : nullptr;
  p.M = M;
  p.K = K;
  p.N = N;
  p.splits = ws.splits;
  p.out_f32 = (flags & MLA_OUT_F32) ? 1 : 0;
  p.group_m = 0;
  if (mla::launch_oproj_fp8dyn(p, s) != hipSuccess) return MLA_ERR_LAUNCH;
  return MLA_OK;
}

}  // extern "C"

// ------------------------------------------------------ matrix-core probe
double mla_mfma_probe_flops(int iters, int kind) {
  if (!mla::probe_args_ok(iters, kind)) return 0.0;
  return (double)mla::kProbeBlocks * (mla::kProbeThreads / 64) * mla::kProbeChains * (double)iters *
         mla::kProbeFlopsPerMfma[kind];
}

int mla_mfma_probe(float* out, int iters, int kind, void* stream) {
  if (!out) return MLA_ERR_NULL;
  if (!mla::probe_args_ok(iters, kind)) return MLA_ERR_DIM;
  if (!aligned16(out)) return MLA_ERR_ALIGN;
  const int dev = check_device();
  if (dev != MLA_OK) return dev;
  (void)hipGetLastError();
  if (mla::launch_mfma_probe(out, iters, kind, static_cast<hipStream_t>(stream)) != hipSuccess)
    return MLA_ERR_LAUNCH;
  return MLA_OK;
}
