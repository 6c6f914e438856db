// Internal declaration of the matrix-core rate probe (a measurement helper,
// not a step of the attention path).
#pragma once

#include <hip/hip_runtime.h>

namespace mla {

constexpr int kProbeBlocks = 512;   // two workgroups of 4 waves per compute unit
constexpr int kProbeThreads = 256;
constexpr int kProbeChains = 4;     // independent accumulators per wave
// flops of one instruction: kinds 0 and 2 v_mfma_f32_32x32x16_bf16, kinds 1
// and 3 v_mfma_f32_32x32x64_f8f6f4 (e4m3 operands); kinds 2 and 3 take
// changing random operands and need iters % 8 == 0
constexpr int kProbeKinds = 4;
constexpr double kProbeFlopsPerMfma[kProbeKinds] = {2.0 * 32 * 32 * 16, 2.0 * 32 * 32 * 64,
                                                    2.0 * 32 * 32 * 16, 2.0 * 32 * 32 * 64};
constexpr bool probe_args_ok(int iters, int kind) {
  return iters >= 1 && iters <= (1 << 24) && kind >= 0 && kind < kProbeKinds && (kind < 2 || iters % 8 == 0);
}

hipError_t launch_mfma_probe(float* out, int iters, int kind, hipStream_t stream);

}  // namespace mla
