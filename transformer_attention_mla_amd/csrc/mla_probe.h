// Internal declaration of the matrix-core rate probe (a measurement helper,
// not a step of the attention path).
#pragma once

#include <hip/hip_runtime.h>

namespace mla {

constexpr int kProbeBlocks = 512;   // two workgroups of 4 waves per compute unit
constexpr int kProbeThreads = 256;
constexpr int kProbeChains = 4;     // independent accumulators per wave
// flops of one instruction: kind 0 v_mfma_f32_32x32x16_bf16, kind 1
// v_mfma_f32_32x32x64_f8f6f4 (e4m3 operands)
constexpr double kProbeFlopsPerMfma[2] = {2.0 * 32 * 32 * 16, 2.0 * 32 * 32 * 64};

hipError_t launch_mfma_probe(float* out, int iters, int kind, hipStream_t stream);

}  // namespace mla
