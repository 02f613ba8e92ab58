// Internal interface between the C ABI (q4g128_api.cpp) and the kernels
// (q4g128_kernels.hip).  Arguments reaching these launchers are validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace q4g128 {

constexpr int kMaxM = 8;

struct GemvArgs {
    const uint16_t *x;       // bf16 [M][K]
    int M, K;
    const uint32_t *W;       // [N][K/8]
    const uint16_t *scale;   // bf16 [N][K/128]
    const uint16_t *mn;      // bf16 [N][K/128]
    int N;
    float *out;              // S == 1: y [M][N]; S > 1: partials [S][M][N]
    int S;                   // K splits (group-aligned), 1..K/128
};

// Output columns one workgroup covers for a given tiles-per-wave setting.
int columns_per_block(int tpw);

hipError_t launch_gemv(const GemvArgs &a, int tpw, hipStream_t stream);
hipError_t launch_splitk_sum(const float *P, int S, size_t MN, float *y, hipStream_t stream);
hipError_t launch_dequant(const uint32_t *W, const uint16_t *scale, const uint16_t *mn, int K, int N,
                          float *w, hipStream_t stream);

}  // namespace q4g128
