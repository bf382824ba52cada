// W8A8 projection path: per-token E4M3 activation quantisation and the
// fp8 x fp8 GEMM (launchers in gemm8.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace quail {

struct W8A8Params {
  const uint8_t* A;        // activation codes [M][K]
  const float* a_scale;    // one fp32 scale per token [M]
  const uint8_t* B;        // weight codes [N][K]
  const uint16_t* b_scale; // one bf16 scale per output row [N]
  uint16_t* Y;             // bf16 [M][N]
  int32_t M, N, K;
};

// codes[m][k] = E4M3(x[m][k] * (448 / amax_m)), scale[m] = amax_m / 448
// (x bf16 [M][K], K a multiple of 8)
hipError_t launch_act_quant_e4m3(int32_t M, int32_t K, const uint16_t* x, uint8_t* codes, float* scale,
                                 hipStream_t s);
// N a multiple of 256, K a multiple of 128
hipError_t launch_gemm_w8a8(const W8A8Params& p, hipStream_t s);

}  // namespace quail
