// Measurement aid, not part of the block: a matrix-core loop on register
// operands only (no memory traffic), to measure the rate the MFMA units sustain
// on this part, clock under load included, beside the published peak.
#include "kernels.hpp"
#include "llama_block.h"

namespace lb {

// Eight independent accumulator chains per wavefront, so that every MFMA can
// issue as soon as the unit is free (a chain's next MFMA comes seven
// instructions later).  Operands are lane-dependent non-trivial bf16 values.
__global__ __launch_bounds__(256) void k_probe_mfma_bf16(int iters, float* sink) {
  const uint32_t t = threadIdx.x * 2654435761u + blockIdx.x * 40503u;
  uint32_t wa[4], wb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // bf16 pairs with exponents near 1.0 and varied mantissas
    const uint32_t h = (t >> (3 * j)) ^ (t << (5 * j + 1));
    wa[j] = 0x3f803f80u | (h & 0x007f007fu);
    wb[j] = 0x3f003f00u | ((h >> 7) & 0x007f007fu);
  }
  bf16x8 a, b;
  __builtin_memcpy(&a, wa, 16);
  __builtin_memcpy(&b, wb, 16);
  f32x16 acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = (f32x16){};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace lb

using namespace lb;

extern "C" llama_status llama_probe_mfma_bf16(int32_t blocks, int32_t iters, float* sink, void* stream) {
  if (blocks <= 0 || iters <= 0 || !sink) return LLAMA_ERR_INVALID_ARG;
  hipLaunchKernelGGL(k_probe_mfma_bf16, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, sink);
  return hipGetLastError() == hipSuccess ? LLAMA_OK : LLAMA_ERR_HIP;
}
